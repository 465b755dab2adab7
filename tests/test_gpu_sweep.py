"""GPU: a seeded random sweep over the argument space of the entry points,
each case against the fp64 oracle.

The cases are drawn once from a fixed seed (so every run checks the same
ones): sequence lengths from 1 to 700 (tile-aligned and ragged), windows from
1 past 2T, head sizes, batch and head counts, explicit scales of either sign,
the (batch, seq, heads, head_dim) layout through the strided entry, partly
filled and wrapped rings, chunks shorter and longer than the window.

Bars: fp32 max |gpu - oracle| <= 1e-5 (gradients: 1e-5 * max(1, max |oracle|));
bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise.
"""

import numpy as np
import pytest
import torch

import sliding_window_causal_amd as swa
import swa_inputs as si
from oracle import swa_oracle as so

pytestmark = pytest.mark.gpu

DEV = "cuda"
F32_ATOL = 1e-5
BF_ATOL, BF_RTOL = 2e-2, 1e-2


def npy(t):
    return t.detach().float().cpu().numpy()


def check(gpu, ref, dtype, what, grad=False):
    g = npy(gpu).astype(np.float64)
    assert np.all(np.isfinite(g)), f"non-finite output {what}"
    err = np.abs(g - ref)
    if dtype == torch.float32:
        bound = F32_ATOL * (max(1.0, float(np.abs(ref).max())) if grad else 1.0)
        assert err.max() <= bound, f"{what}: max abs err {err.max():.3e} > {bound:.3e}"
    else:
        b = BF_ATOL + BF_RTOL * np.abs(ref)
        worst = np.argmax(err - b)
        assert np.all(err <= b), f"{what}: err {err.flat[worst]:.3e} > {b.flat[worst]:.3e}"


def _window(rng, T):
    kind = rng.integers(6)
    return int([1, 2, rng.integers(1, T + 1), T, T + rng.integers(1, 50), 2 * T][kind])


def _scale(rng):
    if rng.random() < 0.5:
        return None
    s = float(rng.uniform(0.02, 0.4))
    return -s if rng.random() < 0.3 else s


def _dtype_d(rng):
    if rng.random() < 0.7:
        return torch.bfloat16, int(rng.choice([64, 128]))
    return torch.float32, int(rng.integers(1, 257))


def _prefill_cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, D = _dtype_d(rng)
        T = int(rng.choice([1, 31, 32, 33, 127, 128, 129, 256]) if rng.random() < 0.3
                else rng.integers(1, 701))
        out.append(dict(i=i, dtype=dtype, D=D, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                        T=T, W=_window(rng, T), scale=_scale(rng),
                        layout="bshd" if rng.random() < 0.3 else None))
    return out


def _ids(cases):
    return [f"{c['i']}-{'bf16' if c['dtype'] == torch.bfloat16 else 'f32'}-D{c['D']}-T{c['T']}"
            f"-W{c['W']}" for c in cases]


PREFILL = _prefill_cases()


@pytest.mark.parametrize("c", PREFILL, ids=_ids(PREFILL))
def test_prefill_sweep(c):
    dtype, B, H, T, D, W, scale = c["dtype"], c["B"], c["H"], c["T"], c["D"], c["W"], c["scale"]
    g = si.generator(3000 + c["i"], DEV)
    if c["layout"] == "bshd":
        q, k, v = (si.normal((B, T, H, D), g, dtype, DEV) for _ in range(3))
        out = swa.sliding_window_attention(q, k, v, W, scale=scale, layout="bshd")
        torch.cuda.synchronize()
        to = lambda x: np.ascontiguousarray(np.swapaxes(npy(x), 1, 2))
        ref = so.swa_dense(to(q), to(k), to(v), W, scale=scale)
        check(out.transpose(1, 2), ref, dtype, "bshd")
        return
    q, k, v = (si.normal((B, H, T, D), g, dtype, DEV) for _ in range(3))
    out = swa.sliding_window_attention(q, k, v, W, scale=scale)
    out2 = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out2, lse, W, scale=scale)
    torch.cuda.synchronize()
    ref = so.swa_dense(npy(q), npy(k), npy(v), W, scale=scale)
    check(out, ref, dtype, "out")
    assert torch.equal(out, out2)
    lref = so.swa_lse(npy(q), npy(k), W, scale=scale)
    err = np.abs(npy(lse).astype(np.float64) - lref).max()
    tol = 1e-5 * max(1.0, np.abs(lref).max()) if dtype == torch.float32 else 2e-2
    assert err <= tol, f"lse max err {err:.3e}"


def _backward_cases(n=16, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, D = _dtype_d(rng)
        T = int(rng.integers(1, 400))
        out.append(dict(i=i, dtype=dtype, D=D, B=1, H=int(rng.integers(1, 3)), T=T,
                        W=_window(rng, T), scale=_scale(rng)))
    return out


BACKWARD = _backward_cases()


@pytest.mark.parametrize("c", BACKWARD, ids=_ids(BACKWARD))
def test_backward_sweep(c):
    dtype, B, H, T, D, W, scale = c["dtype"], c["B"], c["H"], c["T"], c["D"], c["W"], c["scale"]
    g = si.generator(4000 + c["i"], DEV)
    q, k, v, do = (si.normal((B, H, T, D), g, dtype, DEV) for _ in range(4))
    out = swa.sliding_window_attention(q, k, v, W, scale=scale)
    grads = [torch.empty_like(q) for _ in range(3)]
    swa.swa_backward(q, k, v, out, do, *grads, W, scale=scale)
    torch.cuda.synchronize()
    refs = so.swa_backward(npy(q), npy(k), npy(v), W, npy(do), scale=scale)
    for name, gg, r in zip(("dq", "dk", "dv"), grads, refs):
        check(gg, r, dtype, name, grad=True)


def _chunk_cases(n=12, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, D = _dtype_d(rng)
        W = int(rng.integers(1, 300))
        S = int(rng.integers(1, 4))
        pos0 = [int(rng.choice([0, rng.integers(0, W + 1), rng.integers(W, 4 * W + 2)])) for _ in range(S)]
        out.append(dict(i=i, dtype=dtype, D=D, H=int(rng.integers(1, 3)), W=W,
                        C=int(rng.integers(1, 300)), pos0=pos0, split=bool(rng.random() < 0.5)))
    return out


CHUNK = _chunk_cases()


@pytest.mark.parametrize("c", CHUNK, ids=[f"{c['i']}-D{c['D']}-W{c['W']}-C{c['C']}" for c in CHUNK])
def test_chunk_sweep(c):
    dtype, D, H, W, C, pos0 = c["dtype"], c["D"], c["H"], c["W"], c["C"], c["pos0"]
    S = len(pos0)
    T = max(pos0) + C
    g = si.generator(5000 + c["i"], DEV)
    q, k, v = (si.normal((S, H, T, D), g, dtype, DEV) for _ in range(3))
    take = lambda x: torch.stack([x[s, :, pos0[s]:pos0[s] + C] for s in range(S)]).contiguous()
    qc, kc, vc = take(q), take(k), take(v)
    kr = np.full((S, H, W, D), np.nan)
    vr = np.full((S, H, W, D), np.nan)
    for s in range(S):
        if pos0[s] > 0:
            a, b = so.ring_fill(npy(k[s:s + 1]), npy(v[s:s + 1]), [pos0[s] - 1], W)
            kr[s], vr[s] = a[0], b[0]
    to = lambda x: torch.from_numpy(x).to(dtype).to(DEV)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, to(kr), to(vr), p0, split=c["split"])
    torch.cuda.synchronize()
    for s in range(S):
        ref = so.swa_rows(npy(q[s]), npy(k[s]), npy(v[s]), W, range(pos0[s], pos0[s] + C))
        check(out[s], ref, dtype, f"stream {s}")


def _decode_cases(n=12, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, D = _dtype_d(rng)
        W = int(rng.integers(1, 500))
        S = int(rng.integers(1, 7))
        pos = [int(rng.choice([rng.integers(0, W), W - 1, rng.integers(W, 3 * W + 1)])) for _ in range(S)]
        out.append(dict(i=i, dtype=dtype, D=D, H=int(rng.integers(1, 4)), W=W, pos=pos))
    return out


DECODE = _decode_cases()


@pytest.mark.parametrize("c", DECODE, ids=[f"{c['i']}-D{c['D']}-W{c['W']}-S{len(c['pos'])}" for c in DECODE])
def test_decode_sweep(c):
    dtype, D, H, W, pos = c["dtype"], c["D"], c["H"], c["W"], c["pos"]
    S = len(pos)
    T = max(pos) + 1
    g = si.generator(6000 + c["i"], DEV)
    q, k, v = (si.normal((S, H, T, D), g, dtype, DEV) for _ in range(3))
    kr, vr = so.ring_fill(npy(k), npy(v), pos, W)
    to = lambda x: torch.from_numpy(x).to(dtype).to(DEV)
    kr, vr = to(kr), to(vr)
    qs = torch.stack([q[s, :, pos[s]] for s in range(S)]).contiguous()
    pt = torch.tensor(pos, dtype=torch.int64, device=DEV)
    ref = np.stack([so.swa_rows(npy(q[s]), npy(k[s]), npy(v[s]), W, [pos[s]])[:, 0]
                    for s in range(S)])
    out = swa.decode(qs, kr, vr, pt)
    outs = swa.decode(qs, kr, vr, pt, split=True)
    outn = torch.empty_like(qs)
    swa.swa_decode_split_noalloc(qs, kr, vr, pt, outn)
    torch.cuda.synchronize()
    check(out, ref, dtype, "decode")
    check(outs, ref, dtype, "split decode")
    assert torch.equal(outn, outs)
