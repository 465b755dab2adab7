"""GPU: every element of the three full-size bf16 prefill workloads, launched
as the benchmark launches them (and of the backward of two of them), against
a plain fp32 band attention (and its gradients) written with torch on the GPU (score blocks of 512 queries against the keys of their
band, the band predicate 0 <= i - j < W as a mask, softmax, weighted sum:
"27. Sliding-Window Attention", Step-by-Step Approach).  The fp64 oracle
stays the authority (it checks sampled rows of the same launches in
test_gpu_parity.py); this supplementary check covers all B*H*T*D outputs,
which the oracle cannot do in seconds at these sizes.  It shares nothing with
the library: torch's own matrix products (fp32, contiguous operands) and
elementwise operations.

Bar: the bf16 one, |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise; fp32
against fp64 differs by about 1e-6 here, far inside it.
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
