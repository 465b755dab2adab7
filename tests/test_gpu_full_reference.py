"""GPU: every output element of the launches the benchmark times, against a
plain band attention written with torch on the GPU: score blocks of 512
queries against the keys of their band, the band predicate 0 <= i - j < W as
a mask, softmax, weighted sum ("27. Sliding-Window Attention", Step-by-Step
Approach), and its gradients block by block.  Covered: the three full-size
bf16 prefill workloads, the backward of two of them, the chunk continuation
at the benchmark's shapes, the module of one layer, a full fp32 layer and
the fp32 decode at the decode benchmark's shape (those two against fp64).  The fp64
oracle stays the authority (it checks sampled rows of the same launches in
test_gpu_parity.py and the others); this supplementary check covers all
outputs, which the oracle cannot do in seconds at these sizes.  It shares
nothing with the library: torch's own matrix products (contiguous operands)
and elementwise operations.

Bars: the bf16 one, |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise, against an
fp32 reference (fp32 against fp64 differs by about 1e-6 here, far inside
it); the fp32 one, max |gpu - ref| <= 1e-5, against an fp64 reference.
"""

import math

import pytest
import torch

import sliding_window_causal_amd as swa
import swa_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF_ATOL, BF_RTOL = 2e-2, 1e-2
BQ = 512


@torch.no_grad()
def band_attention_block(q, k, v, i0, i1, W):
    """fp32 band attention of queries [i0, i1) of one batch entry (q, k, v:
    [H, T, D] float32): keys [max(0, i0 - W + 1), i1), masked to the band."""
    lo = max(0, i0 - W + 1)
    kt = k[:, lo:i1].transpose(1, 2).contiguous()
    s = torch.matmul(q[:, i0:i1].contiguous(), kt) * (1.0 / math.sqrt(q.shape[-1]))
    i = torch.arange(i0, i1, device=q.device).view(-1, 1)
    j = torch.arange(lo, i1, device=q.device).view(1, -1)
    visible = (i - j >= 0) & (i - j < W)
    s = s.masked_fill(~visible, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v[:, lo:i1].contiguous())


@pytest.mark.parametrize("name", ["prefill_bf16_b1_h32_t8192_d128_w4096",
                                  "prefill_bf16_b8_h32_t4096_d128_w1024",
                                  "prefill_bf16_b1_h32_t65536_d128_w4096"])
def test_full_size_prefill_every_element_against_fp32_band_attention(name):
    w = si.WORKLOADS[name]
    q, k, v = si.workload_qkv(w, DEV)
    out = torch.empty_like(q)
    swa.swa_forward(q, k, v, out, w.W)
    torch.cuda.synchronize()
    W = min(w.W, w.T)
    worst = 0.0
    for b in range(w.B):
        qf, kf, vf = q[b].float(), k[b].float(), v[b].float()
        for i0 in range(0, w.T, BQ):
            i1 = min(w.T, i0 + BQ)
            ref = band_attention_block(qf, kf, vf, i0, i1, W)
            got = out[b, :, i0:i1].float()
            ratio = ((got - ref).abs() / (BF_ATOL + BF_RTOL * ref.abs())).max().item()
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"{name} b={b} rows [{i0}, {i1}): {ratio:.3f} of the bar"
        del qf, kf, vf
    print(f"{name}: worst error {worst:.3f} of the bf16 bar")


@torch.no_grad()
def band_attention_backward(q, k, v, do, W, scale):
    """fp32 gradients of band attention for one batch entry (q, k, v, do:
    [H, T, D] float32), block by block over the queries: P and dP over each
    block's band, delta from the block's own fp32 output, dS = P (dP - delta),
    dq = dS k scale, and dk += dS^T q scale, dv += P^T do over the band."""
    H, T, D = q.shape
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    for i0 in range(0, T, BQ):
        i1 = min(T, i0 + BQ)
        lo = max(0, i0 - W + 1)
        kb, vb = k[:, lo:i1].contiguous(), v[:, lo:i1].contiguous()
        qb, dob = q[:, i0:i1].contiguous(), do[:, i0:i1].contiguous()
        s = torch.matmul(qb, kb.transpose(1, 2).contiguous()) * scale
        i = torch.arange(i0, i1, device=q.device).view(-1, 1)
        j = torch.arange(lo, i1, device=q.device).view(1, -1)
        s = s.masked_fill(~((i - j >= 0) & (i - j < W)), float("-inf"))
        p = torch.softmax(s, dim=-1)
        o = torch.matmul(p, vb)
        dp = torch.matmul(dob, vb.transpose(1, 2).contiguous())
        delta = (dob * o).sum(-1, keepdim=True)
        ds = p * (dp - delta)
        dq[:, i0:i1] = torch.matmul(ds, kb) * scale
        dk[:, lo:i1] += torch.matmul(ds.transpose(1, 2).contiguous(), qb) * scale
        dv[:, lo:i1] += torch.matmul(p.transpose(1, 2).contiguous(), dob)
    return dq, dk, dv


@pytest.mark.parametrize("name", ["prefill_bf16_b1_h32_t8192_d128_w4096",
                                  "prefill_bf16_b8_h32_t4096_d128_w1024"])
def test_full_size_backward_every_element_against_fp32_band_attention(name):
    """The bf16 backward of the prefill workloads as the benchmark launches it
    (given the forward's log-sum-exp): every element of dq, dk and dv against
    the fp32 gradients above, at the bf16 bar."""
    w = si.WORKLOADS[name]
    q, k, v = si.workload_qkv(w, DEV)
    do = si.normal(tuple(q.shape), si.generator(w.seed + 11, DEV), torch.bfloat16, DEV)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out, lse, w.W)
    grads = [torch.empty_like(q) for _ in range(3)]
    swa.swa_backward(q, k, v, out, do, *grads, w.W, lse=lse)
    torch.cuda.synchronize()
    W = min(w.W, w.T)
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in range(w.B):
        refs = band_attention_backward(q[b].float(), k[b].float(), v[b].float(), do[b].float(),
                                       W, 1.0 / math.sqrt(w.D))
        for nm, g, r in zip(("dq", "dk", "dv"), grads, refs):
            ratio = ((g[b].float() - r).abs() / (BF_ATOL + BF_RTOL * r.abs())).max().item()
            worst[nm] = max(worst[nm], ratio)
            assert ratio <= 1.0, f"{name} b={b} {nm}: {ratio:.3f} of the bar"
        del refs
    print(f"{name}: worst error of the bf16 bar {worst}")


@pytest.mark.parametrize("S,C", [(1, 2048), (4, 512), (1, 128)])
def test_chunk_benchmark_shapes_every_element(S, C):
    """The chunk continuation at the shapes the benchmark times (32 heads, D
    128, full 4096-slot rings, first position 5W + 123, inputs drawn as it
    draws them), plain and split: every element against the fp32 band
    attention over the sequence the ring and the chunk hold (the W - 1
    positions before the chunk from ring slot position mod W, then the
    chunk's keys)."""
    w = si.WORKLOADS["prefill_bf16_b1_h32_t8192_d128_w4096"]
    H, D, W = w.H, w.D, w.W
    g = si.generator(w.seed, DEV)
    qc, kc, vc = (si.normal((S, H, C, D), g, torch.bfloat16, DEV) for _ in range(3))
    kr = si.normal((S, H, W, D), g, torch.bfloat16, DEV)
    vr = si.normal((S, H, W, D), g, torch.bfloat16, DEV)
    p0 = 5 * W + 123
    pos0 = torch.tensor([p0] * S, dtype=torch.int64, device=DEV)
    plain = torch.empty_like(qc)
    swa.swa_chunk_forward(qc, kc, vc, kr, vr, pos0, plain)
    ws = torch.empty(max(swa.swa_chunk_workspace_bytes(S, H, C, D, W, torch.bfloat16), 1),
                     dtype=torch.uint8, device=DEV)
    split = torch.empty_like(qc)
    swa.swa_chunk_forward_split(qc, kc, vc, kr, vr, pos0, split, ws)
    torch.cuda.synchronize()
    slots = (p0 - W + 1 + torch.arange(W - 1, device=DEV)) % W
    for s in range(S):
        kf = torch.cat([kr[s][:, slots], kc[s]], dim=1).float()
        vf = torch.cat([vr[s][:, slots], vc[s]], dim=1).float()
        qf = torch.cat([torch.zeros((H, W - 1, D), device=DEV), qc[s].float()], dim=1)
        for i0 in range(W - 1, W - 1 + C, BQ):
            i1 = min(W - 1 + C, i0 + BQ)
            ref = band_attention_block(qf, kf, vf, i0, i1, W)
            for tag, o in (("plain", plain), ("split", split)):
                got = o[s, :, i0 - (W - 1):i1 - (W - 1)].float()
                ratio = ((got - ref).abs() / (BF_ATOL + BF_RTOL * ref.abs())).max().item()
                assert ratio <= 1.0, f"{tag} S={S} C={C} s={s} rows {i0 - W + 1}..: {ratio:.3f}"


def test_fp32_full_layer_every_element_against_fp64_band_attention():
    """The fp32 matrix-core prefill of a full [1, 32, 8192, 128] layer, W 4096:
    every element against the same band attention computed in fp64 with torch
    on the GPU, at the fp32 bar max |gpu - ref| <= 1e-5."""
    B, H, T, D, W = 1, 32, 8192, 128, 4096
    g = si.generator(7300, DEV)
    q, k, v = (si.normal((B, H, T, D), g, torch.float32, DEV) for _ in range(3))
    out = torch.empty_like(q)
    swa.swa_forward(q, k, v, out, W)
    torch.cuda.synchronize()
    qd, kd, vd = q[0].double(), k[0].double(), v[0].double()
    worst = 0.0
    for i0 in range(0, T, BQ):
        i1 = min(T, i0 + BQ)
        ref = band_attention_block(qd, kd, vd, i0, i1, W)
        err = (out[0, :, i0:i1].double() - ref).abs().max().item()
        worst = max(worst, err)
        assert err <= 1e-5, f"rows [{i0}, {i1}): max abs err {err:.3e}"
    print(f"fp32 layer: worst abs error {worst:.3e}")


def test_fp32_decode_full_size_every_element_against_fp64():
    """The fp32 instantiation of the decode kernel at the decode benchmark's
    shape (256 streams, 32 heads, D 128, full 4096-slot rings): every element
    against softmax(q k^T / sqrt(D)) v over each ring's occupied slots (all of
    them: every position is past W), in fp64 with torch, at the fp32 bar."""
    S, H, D, W = 256, 32, 128, 4096
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.float32, 8100, DEV)
    assert bool((pos >= W).all())
    out = swa.decode(q, kr, vr, pos)
    torch.cuda.synchronize()
    worst = 0.0
    for s0 in range(0, S, 16):
        qd = q[s0:s0 + 16].double().reshape(-1, 1, D)
        kd = kr[s0:s0 + 16].double().reshape(-1, W, D)
        vd = vr[s0:s0 + 16].double().reshape(-1, W, D)
        sc = torch.matmul(qd, kd.transpose(1, 2).contiguous()) / math.sqrt(D)
        ref = torch.matmul(torch.softmax(sc, dim=-1), vd).reshape(-1, H, D)
        err = (out[s0:s0 + 16].double() - ref).abs().max().item()
        worst = max(worst, err)
        assert err <= 1e-5, f"streams [{s0}, {s0 + 16}): max abs err {err:.3e}"
        del qd, kd, vd, sc, ref
    print(f"fp32 decode: worst abs error {worst:.3e}")


def test_module_full_size_every_element():
    """The module of one 32-head layer as the benchmark launches it (d_model
    4096 = 32 x 128, T 8192, W 4096, inputs and weights drawn as it draws
    them): every output element against the same module in fp32 with torch
    (x @ w projections with the biases, 32 heads of band attention, output
    projection), at the bf16 bar."""
    w = si.WORKLOADS["prefill_bf16_b1_h32_t8192_d128_w4096"]
    dm, H, D, T, W = w.H * w.D, w.H, w.D, w.T, w.W
    g = si.generator(w.seed + 7, DEV)
    x = si.normal((w.B, T, dm), g, torch.bfloat16, DEV)
    wts = [si.normal((dm, dm), g, torch.float32, DEV).mul_(dm ** -0.5).to(torch.bfloat16)
           for _ in range(4)]
    bss = [torch.zeros(dm, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    out = torch.empty_like(x)
    ws = torch.empty(swa.swa_mha_workspace_bytes(w.B, T, dm, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    swa.swa_mha_forward(x, wts[0], bss[0], wts[1], bss[1], wts[2], bss[2], wts[3], bss[3], out,
                        H, W, workspace=ws)
    torch.cuda.synchronize()
    xf = x[0].float()
    wf = [t.float() for t in wts]
    bf = [t.float() for t in bss]
    # [T, dm] -> [H, T, D]
    heads = [(torch.matmul(xf, wf[i]) + bf[i]).view(T, H, D).transpose(0, 1).contiguous()
             for i in range(3)]
    o = torch.empty((H, T, D), dtype=torch.float32, device=DEV)
    for i0 in range(0, T, BQ):
        o[:, i0:i0 + BQ] = band_attention_block(heads[0], heads[1], heads[2], i0,
                                                min(T, i0 + BQ), W)
    ref = torch.matmul(o.transpose(0, 1).reshape(T, dm), wf[3]) + bf[3]
    ratio = ((out[0].float() - ref).abs() / (BF_ATOL + BF_RTOL * ref.abs())).max().item()
    print(f"module: worst error {ratio:.3f} of the bf16 bar")
    assert ratio <= 1.0, f"{ratio:.3f} of the bar"
