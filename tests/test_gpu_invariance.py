"""GPU: bitwise out-of-window invariance on data chosen to put it at risk.

The pages' independence check ("25. Sliding-Window Causal Attention for
Streaming Inference", Step-by-Step Approach step 6 and the corrupt-and-compare
check; "NNX Sliding-Window Attention", the moving-average example's assertion
on the later rows) says a query's output depends on its own window only.
Here that holds bit for bit for finite corruption, on inputs where a kernel
that shares work between rows could break it:

  * a row whose in-window scores jump far above its first tiles' scores,
    next to rows whose corrupted windows overflow (any recomputation with a
    different running reference would change its rounding);
  * keys near the bf16 maximum (finite, but their fp32 dot products overflow
    to inf or NaN) in tiles that a wavefront computes without needing them:
    future keys of its rows, and keys older than their windows;
  * values near the bf16 maximum, so that p * v overflows in rows that see
    them.

Rows outside [j0, j0 + W - 1] of a corrupted position j0 must be
bit-identical to the clean run (compared as integers, so NaN never hides a
difference); where the oracle can compute the corrupted rows it is checked
too, at the bf16 bar |gpu - oracle| <= 2e-2 + 1e-2 |oracle|.
"""

import numpy as np
import pytest
import torch

import sliding_window_causal_amd as swa
import swa_inputs as si
from oracle import swa_oracle as so

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF_ATOL, BF_RTOL = 2e-2, 1e-2
LOG2E = 1.4426950408889634
BIG = 3.0e38          # finite in bf16 (largest finite bf16 is about 3.39e38)


def npy(t):
    return t.detach().float().cpu().numpy()


def same_rows(a, b):
    """Per query row (last-but-one axis), True where every element of every
    leading index is bit-identical."""
    it = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    eq = a.contiguous().view(it) == b.contiguous().view(it)
    eq = eq.all(dim=-1)
    while eq.dim() > 1:
        eq = eq.all(dim=0)
    return eq.cpu().numpy()


def assert_close(gpu, ref, what=""):
    g = npy(gpu).astype(np.float64)
    assert np.all(np.isfinite(g)), f"non-finite output {what}"
    err = np.abs(g - ref)
    bound = BF_ATOL + BF_RTOL * np.abs(ref)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (
        f"{what}: err {err.flat[worst]:.3e} > bound {bound.flat[worst]:.3e}")


def fwd(q, k, v, W):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out, lse, W)
    torch.cuda.synchronize()
    return out, lse


def outside(T, j0, W):
    i = np.arange(T)
    return (i < j0) | (i > j0 + W - 1)


# ----------------------------------------------------------------------------
# A sharp row beside rows whose corrupted windows overflow
# ----------------------------------------------------------------------------

def _sharp_case(D=128, T=2048, W=256, i_sharp=1151, j_sharp=1000, seed=61):
    """N(0, 1) q, k, v with q[i_sharp] = a k[j_sharp], a = 1.6 sqrt(128 / D):
    that row's score on key j_sharp stands about a |k|^2 / sqrt(D) above its
    other scores (10 to 30 log2 units over 200 seeds of a CPU draw)."""
    q, k, v = si.prefill_qkv(1, 2, T, D, dtype=torch.bfloat16, seed=seed, device=DEV)
    q[:, :, i_sharp] = (k[:, :, j_sharp].float() * 1.6 * (128 / D) ** 0.5).bfloat16()
    # the jump really is there: above every key of the row's window before
    # j_sharp's tile by more than 8 log2 units, and far inside the fp32 range
    qs, ks = npy(q)[0], npy(k)[0]
    lo = i_sharp - W + 1
    for h in range(2):
        s = ks[h, lo:i_sharp + 1] @ qs[h, i_sharp] / np.sqrt(D)
        before = s[: (j_sharp // 32) * 32 - lo]
        jump = (s[j_sharp - lo] - before.max()) * LOG2E
        assert 8.5 < jump < 100, f"h={h}: jump {jump:.1f} log2 units"
    return q, k, v


@pytest.mark.parametrize("D", [128, 64])
def test_sharp_row_keeps_its_bits_when_neighbours_overflow(D):
    """Corrupting k[850] makes the rows that see it overflow; row 1151 (in
    the same 128-query block, window starting at 896) has a key more than 8
    log2 units above its first tiles and must keep every bit, as must every other
    row outside [850, 1105]; the output's log-sum-exp likewise."""
    T, W, j0 = 2048, 256, 850
    q, k, v = _sharp_case(D=D, T=T, W=W)
    base, lbase = fwd(q, k, v, W)
    k2 = k.clone()
    k2[:, :, j0] = 2000.0
    out, lse = fwd(q, k2, v, W)
    keep = outside(T, j0, W)
    same = same_rows(out, base)
    assert np.all(same[keep]), f"rows changed outside the window: {np.where(~same & keep)[0][:10]}"
    lsame = (lse.view(torch.int32) == lbase.view(torch.int32)).all(dim=0).all(dim=0).cpu().numpy()
    assert np.all(lsame[keep])
    assert not np.all(same[~keep]), "the corruption must reach the rows that see it"
    # the corrupted run is still the attention of the corrupted inputs
    ref = so.swa_dense(npy(q), npy(k2), npy(v), W)
    assert_close(out, ref, "corrupted run vs oracle")
    assert_close(base, so.swa_dense(npy(q), npy(k), npy(v), W), "clean run vs oracle")


def test_ramped_rows_keep_their_bits_when_huge_values_overflow():
    """Scores rising about 50 log2 units across each window (so any redo with
    the max taken on every tile would rescale) and v[j0] near the bf16
    maximum (p * v overflows in the rows that see it): every row outside
    [j0, j0 + W - 1] keeps its bits."""
    T, W, D = 2048, 256, 128
    g = si.generator(63, DEV)
    q = torch.full((1, 2, T, D), 0.25, device=DEV)
    slope = 50.0 / (0.25 * D ** 0.5 * W * LOG2E)
    ramp = slope * torch.arange(T, device=DEV, dtype=torch.float32).view(1, 1, T, 1)
    k = ramp + 0.1 * si.normal((1, 2, T, D), g, torch.float32, DEV)
    v = si.normal((1, 2, T, D), g, torch.float32, DEV)
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    base, _ = fwd(q, k, v, W)
    assert_close(base, so.swa_dense(npy(q), npy(k), npy(v), W), "clean ramp vs oracle")
    for j0 in (850, 1000, 1023, 1500):
        v2 = v.clone()
        v2[:, :, j0] = BIG
        v2[:, :, j0 + 1] = BIG
        out, _ = fwd(q, k, v2, W)
        keep = outside(T, j0, W) & outside(T, j0 + 1, W)
        same = same_rows(out, base)
        assert np.all(same[keep]), f"j0={j0}: rows changed {np.where(~same & keep)[0][:10]}"


# ----------------------------------------------------------------------------
# Keys and values near the bf16 maximum where a wavefront does not need them
# ----------------------------------------------------------------------------

def _huge_key(k, v, j0, sign_flip):
    k2, v2 = k.clone(), v.clone()
    D = k.shape[-1]
    pat = torch.ones(D, device=DEV)
    if sign_flip:
        pat[1::2] = -1.0            # partial sums overflow both ways: NaN scores
    k2[:, :, j0] = (BIG * pat).to(k.dtype)
    v2[:, :, j0] = (-BIG * pat).to(v.dtype)
    return k2, v2


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("sign_flip", [False, True])
def test_huge_finite_keys_outside_the_window_are_invisible(D, sign_flip):
    """k[j0] and v[j0] near the bf16 maximum.  j0 runs over future keys in a
    block's last tiles (computed, not needed, by its first wavefronts), keys
    in a block's first tile older than its later wavefronts' windows, the
    key at i - W for tile-aligned rows i, and tile edges.  Every row outside
    [j0, j0 + W - 1] is bit-identical to the clean run."""
    T, W = 700, 100
    q, k, v = si.prefill_qkv(1, 2, T, D, dtype=torch.bfloat16, seed=65 + D, device=DEV)
    base, lbase = fwd(q, k, v, W)
    # block of 128 queries at i0 = 256: its key range starts at 157 (tile 4,
    # keys 128..159); wavefront 0 holds rows 256..287
    j0s = [0, 31, 32, 127, 128, 157, 158, 159,     # first tile of the block at 256
           290, 300, 356, 383,                      # future keys of wavefronts 0..2 there
           256 - W, 288 - W, 320 - W, 384 - W,      # i - W for block / wave starts i
           T - W - 1, T - 2, T - 1]
    for j0 in j0s:
        k2, v2 = _huge_key(k, v, j0, sign_flip)
        out, lse = fwd(q, k2, v2, W)
        keep = outside(T, j0, W)
        same = same_rows(out, base)
        assert np.all(same[keep]), f"j0={j0}: rows changed {np.where(~same & keep)[0][:10]}"
        lsame = (lse.view(torch.int32) == lbase.view(torch.int32)).all(dim=0).all(dim=0).cpu().numpy()
        assert np.all(lsame[keep]), f"j0={j0}: lse changed"


@pytest.mark.parametrize("W,T", [(4096, 4500), (1024, 3000), (33, 300)])
def test_huge_finite_keys_at_the_edges_of_large_windows(W, T):
    """The same at the benchmark windows and a window just over one tile."""
    D = 128
    q, k, v = si.prefill_qkv(1, 1, T, D, dtype=torch.bfloat16, seed=W + T, device=DEV)
    base, _ = fwd(q, k, v, W)
    rng = np.random.default_rng(W)
    j0s = sorted({0, 1, 127, 128, T - W - 1, T - W, T - 1, T - 130,
                  *(int(x) for x in rng.integers(0, T, 6))})
    for j0 in j0s:
        if j0 < 0:
            continue
        k2, v2 = _huge_key(k, v, j0, True)
        out, _ = fwd(q, k2, v2, W)
        keep = outside(T, j0, W)
        same = same_rows(out, base)
        assert np.all(same[keep]), f"W={W} j0={j0}: rows changed {np.where(~same & keep)[0][:10]}"


# ----------------------------------------------------------------------------
# The chunk continuation of a ring
# ----------------------------------------------------------------------------

def _chunk_inputs(q, k, v, pos0, C, W):
    """The chunk [pos0, pos0 + C) of one sequence and rings holding the W
    tokens before it (slot = position mod W), as device tensors."""
    qc, kc, vc = (x[:, :, pos0:pos0 + C].contiguous() for x in (q, k, v))
    H, D = q.shape[1], q.shape[3]
    kr = torch.zeros((1, H, W, D), dtype=q.dtype, device=DEV)
    vr = torch.zeros_like(kr)
    for p in range(max(0, pos0 - W), pos0):
        kr[0, :, p % W] = k[0, :, p]
        vr[0, :, p % W] = v[0, :, p]
    return qc, kc, vc, kr, vr


def _chunk_run(qc, kc, vc, kr, vr, pos0, split):
    p0 = torch.tensor([pos0], dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, kr, vr, p0, split=split)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("split", [False, True])
def test_chunk_sharp_row_keeps_its_bits(split):
    """The sharp-row case through the chunk continuation: positions 768 ..
    2047 as one chunk over a ring holding 512 .. 767."""
    T, W, j0, pos0 = 2048, 256, 850, 768
    q, k, v = _sharp_case(D=128, T=T, W=W)
    C = T - pos0
    base = _chunk_run(*_chunk_inputs(q, k, v, pos0, C, W), pos0, split)
    k2 = k.clone()
    k2[:, :, j0] = 2000.0
    out = _chunk_run(*_chunk_inputs(q, k2, v, pos0, C, W), pos0, split)
    keep = outside(T, j0, W)[pos0:]
    same = same_rows(out, base)
    assert np.all(same[keep]), f"rows changed {pos0 + np.where(~same & keep)[0][:10]}"
    ref = so.swa_rows(npy(q[0]), npy(k2[0]), npy(v[0]), W, list(range(pos0, T)))
    assert_close(out[0], ref, "corrupted chunk vs oracle rows")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("D", [128, 64])
def test_chunk_huge_finite_keys_outside_the_window_are_invisible(D, split):
    """Huge finite k, v in the chunk (future keys of a block's first
    wavefronts, tile edges) and in the ring (the token at p - W): rows whose
    windows exclude the corrupted position keep every bit."""
    T, W, pos0 = 900, 100, 300
    C = T - pos0
    q, k, v = si.prefill_qkv(1, 2, T, D, dtype=torch.bfloat16, seed=67 + D, device=DEV)
    base = _chunk_run(*_chunk_inputs(q, k, v, pos0, C, W), pos0, split)
    for j0 in (pos0 - W, pos0 - W + 1, pos0 - 1, pos0, pos0 + 40, pos0 + 100, pos0 + 127,
               pos0 + 128, T - W - 1, T - 1):
        k2, v2 = _huge_key(k, v, j0, True)
        out = _chunk_run(*_chunk_inputs(q, k2, v2, pos0, C, W), pos0, split)
        keep = outside(T, j0, W)[pos0:]
        same = same_rows(out, base)
        assert np.all(same[keep]), f"j0={j0}: rows changed {pos0 + np.where(~same & keep)[0][:10]}"
