"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars (written in each test):
  fp32 inputs  max |gpu - oracle| <= 1e-5
  bf16 inputs  |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise
  bitwise      out-of-window corruption (finite values), W = 1 (out == v),
               the integer worked example, determinism across runs
The oracle always receives exactly the values the GPU received (bf16 inputs
upcast exactly).
"""

import numpy as np
import pytest
import torch

import sliding_window_causal_amd as swa
import swa_inputs as si
from conftest import read_golden
from oracle import swa_oracle as so

pytestmark = pytest.mark.gpu

DEV = "cuda"
F32_ATOL = 1e-5
BF_ATOL, BF_RTOL = 2e-2, 1e-2


def npy(t):
    return t.detach().float().cpu().numpy()


def assert_close(gpu, ref, dtype, what=""):
    g = npy(gpu).astype(np.float64)
    assert np.all(np.isfinite(g)), f"non-finite output {what}"
    err = np.abs(g - ref)
    if dtype == torch.float32:
        assert err.max() <= F32_ATOL, f"{what}: max abs err {err.max():.3e}"
    else:
        bound = BF_ATOL + BF_RTOL * np.abs(ref)
        worst = np.argmax(err - bound)
        assert np.all(err <= bound), (
            f"{what}: err {err.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} "
            f"(max abs err {err.max():.3e})")


def run_fwd(q, k, v, W):
    out = swa.sliding_window_attention(q, k, v, W)
    torch.cuda.synchronize()
    return out


def _masks():
    res = []
    for name in ("mask_8tok_w4.txt", "mask_5tok_w3.txt"):
        lines = read_golden(name)
        hdr = dict(t.split("=") for t in lines[0].split())
        grid = lines[1:]
        m = np.array([[c in ".1" for c in row] for row in grid])
        res.append((int(hdr["T"]), int(hdr["W"]), m))
    return res


# ----------------------------------------------------------------------------
# fp32 path: the small workload, its window sweep, the pages' examples
# ----------------------------------------------------------------------------

TINY = si.WORKLOADS["prefill_f32_b1_h2_t128_d64_w32"]


@pytest.mark.parametrize("W", [TINY.W, *TINY.sweep])
def test_f32_tiny_workload_and_window_sweep(W):
    q, k, v = si.workload_qkv(TINY, DEV)
    out = run_fwd(q, k, v, W)
    ref = so.swa_dense(npy(q), npy(k), npy(v), W)
    assert_close(out, ref, torch.float32, f"W={W}")


@pytest.mark.parametrize("shape,W", [((1, 2, 6, 4), 3), ((1, 1, 5, 3), 2), ((1, 4, 16, 32), 4),
                                     ((2, 3, 37, 1), 5), ((1, 2, 200, 256), 70),
                                     ((3, 1, 65, 17), 64), ((1, 1, 1, 8), 1)])
def test_f32_page_shapes_and_odd_head_sizes(shape, W):
    q, k, v = si.prefill_qkv(*shape, dtype=torch.float32, seed=7, device=DEV)
    out = run_fwd(q, k, v, W)
    assert out.shape == q.shape
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), W), torch.float32, str(shape))


def test_f32_three_dim_input_is_one_head():
    """P2's (batch, seq, dim) layout through the binding."""
    g = si.generator(8, DEV)
    q, k, v = (si.normal((1, 5, 3), g, torch.float32, DEV) for _ in range(3))
    out = run_fwd(q, k, v, 2)
    assert out.shape == (1, 5, 3)
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), 2), torch.float32)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 8), (torch.bfloat16, 64)])
def test_mask_probe_reproduces_printed_masks(dtype, D):
    """q = k = 0, v = one-hot rows: out[i, j] > 0 exactly on visible keys."""
    for T, W, m in _masks():
        z = torch.zeros(1, 1, T, D, dtype=dtype, device=DEV)
        v = torch.zeros(1, 1, T, D, dtype=dtype, device=DEV)
        v[0, 0, torch.arange(T), torch.arange(T)] = 1
        out = npy(run_fwd(z, z, v, W))[0, 0, :, :T]
        assert np.array_equal(out > 0, m), f"T={T} W={W}"


@pytest.mark.parametrize("dtype,D", [(torch.float32, 7), (torch.float32, 64),
                                     (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_window_one_returns_v_exactly(dtype, D):
    q, k, v = si.prefill_qkv(2, 3, 150, D, dtype=dtype, seed=9, device=DEV)
    out = run_fwd(q, k, v, 1)
    assert torch.equal(out, v)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 1), (torch.bfloat16, 64)])
def test_p5_worked_example(dtype, D):
    lines = read_golden("p5_moving_average.txt")
    W = int(lines[0].split("=")[1])
    x = np.array([[float(t) for t in ln.split()] for ln in lines[lines.index("x") + 1:lines.index("out")]])
    exp = np.array([[float(t) for t in ln.split()]
                    for ln in lines[lines.index("out") + 1:lines.index("corrupt_row0")]])
    T = x.shape[0]
    z = torch.zeros(1, 2, T, D, dtype=dtype, device=DEV)
    v = torch.zeros(1, 2, T, D, dtype=dtype, device=DEV)
    v[0, :, :, 0] = torch.tensor(x.T, dtype=dtype)
    out = npy(run_fwd(z, z, v, W))[0, :, :, 0].T
    assert np.array_equal(out, exp)
    v2 = v.clone()
    v2[0, :, 0, 0] = torch.tensor([100.0, 200.0], dtype=dtype)
    out2 = npy(run_fwd(z, z, v2, W))[0, :, :, 0].T
    assert np.array_equal(out2[3:], out[3:])


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_zero_qk_is_trailing_moving_average(dtype, D):
    g = si.generator(10, DEV)
    T, W = 300, 37
    v = si.normal((1, 2, T, D), g, dtype, DEV)
    z = torch.zeros_like(v)
    out = run_fwd(z, z, v, W)
    vv = npy(v).astype(np.float64)
    C = np.concatenate([np.zeros((1, 2, 1, D)), np.cumsum(vv, axis=2)], axis=2)
    lo = np.maximum(0, np.arange(T) - W + 1)
    n = (np.arange(T) - lo + 1)[None, None, :, None]
    ref = (C[:, :, np.arange(T) + 1] - C[:, :, lo]) / n
    assert_close(out, ref, dtype)


# ----------------------------------------------------------------------------
# bf16 MFMA path at oracle-friendly sizes: tiles, ragged tails, windows
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,W", [(1, 1), (2, 5), (63, 7), (65, 64), (127, 3), (129, 128),
                                 (333, 17), (333, 100), (333, 333), (333, 1000), (520, 129),
                                 (700, 256), (1000, 1)])
def test_bf16_prefill_vs_dense_oracle(T, W, D):
    q, k, v = si.prefill_qkv(2, 3, T, D, dtype=torch.bfloat16, seed=T * 31 + W, device=DEV)
    out = run_fwd(q, k, v, W)
    ref = so.swa_dense(npy(q), npy(k), npy(v), W)
    assert_close(out, ref, torch.bfloat16, f"T={T} W={W} D={D}")


def test_bf16_tile_boundary_sweep():
    """Sequence lengths on either side of the 128-query workgroup tile and
    windows on either side of the 32-key tile (and of W = 64, where an edge
    tile becomes one-sided): the kernel's band, interior and fast-pass tile
    ranges and the end of its tile loads all move by one here."""
    bad = []
    for T in (127, 128, 129, 255, 256, 257):
        for W in (31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129):
            q, k, v = si.prefill_qkv(1, 2, T, 64, dtype=torch.bfloat16, seed=7 * T + W, device=DEV)
            out = npy(run_fwd(q, k, v, W)).astype(np.float64)
            ref = so.swa_dense(npy(q), npy(k), npy(v), W)
            over = np.abs(out - ref) - (BF_ATOL + BF_RTOL * np.abs(ref))
            if not (np.isfinite(out).all() and (over <= 0).all()):
                bad.append((T, W, float(np.nanmax(over))))
    assert not bad, bad


def test_bf16_scaled_inputs_stay_within_tolerance():
    """Larger logits (q, k ~ N(0, 3^2)) exercise the running-max rescale."""
    q, k, v = si.prefill_qkv(1, 4, 600, 128, dtype=torch.float32, seed=12, device=DEV)
    q, k, v = (3 * q).bfloat16(), (3 * k).bfloat16(), v.bfloat16()
    out = run_fwd(q, k, v, 200)
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), 200), torch.bfloat16)


def _ramp_qkv(T, D, slope, seed):
    """Scores that grow along the sequence: q = 1/4, k_j = slope * j plus a
    little noise, v ~ N(0, 1); q . k_j / sqrt(D) rises by about
    8 * slope * sqrt(D) / 4 per key."""
    g = si.generator(seed, DEV)
    q = torch.full((1, 2, T, D), 0.25, device=DEV)
    ramp = slope * torch.arange(T, device=DEV, dtype=torch.float32).view(1, 1, T, 1)
    k = ramp + 0.1 * si.normal((1, 2, T, D), g, torch.float32, DEV)
    v = si.normal((1, 2, T, D), g, torch.float32, DEV)
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_negative_scale_with_scores_growing_beyond_fp32_range(D):
    """A negative scale is applied as -q times |scale|; q is flipped once,
    after the prologue's wait.  Keys ramping the other way make the scaled
    scores climb hundreds of log2 units within a window, so workgroups redo
    their rows in the careful pass, which must not flip q again."""
    T, W = 1024, 512
    q, k, v = _ramp_qkv(T, D, -1.0, seed=77 + D)
    scale = -1.0 / D ** 0.5
    s = (q.float()[0, 0, 0] @ k.float()[0, 0].T) * scale
    assert (s[W - 1] - s[0]).item() * 1.4427 > 200        # the growth is really there
    out = swa.sliding_window_attention(q, k, v, W, scale=scale)
    ref = so.swa_dense(npy(q), npy(k), npy(v), W, scale=scale)
    assert_close(out, ref, torch.bfloat16, f"D={D} scale {scale}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,W", [(1024, 1024), (2048, 256), (700, 100)])
def test_bf16_scores_growing_beyond_fp32_range(T, W, D):
    """Within a window the scores rise by hundreds of log2 units above those
    of its first key tile, far past the fp32 exponent range: probabilities
    taken against an early reference would overflow.  The output (and the
    row log-sum-exp) must still be finite and match the oracle."""
    q, k, v = _ramp_qkv(T, D, 1.0, seed=T + W + D)
    s = q.float()[0, 0, 0] @ k.float()[0, 0].T / D ** 0.5
    assert (s[W - 1] - s[0]).item() * 1.4427 > 200        # the growth is really there
    out = run_fwd(q, k, v, W)
    ref = so.swa_dense(npy(q), npy(k), npy(v), W)
    assert_close(out, ref, torch.bfloat16, f"T={T} W={W} D={D}")
    out2 = torch.empty_like(q)
    lse = torch.empty(1, 2, T, dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out2, lse, W)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    lref = so.swa_lse(npy(q), npy(k), W)
    assert np.all(np.abs(npy(lse) - lref) <= 1e-2 + 1e-3 * np.abs(lref))


@pytest.mark.parametrize("D,W,T", [(128, 128, 700), (128, 4096, 5000), (64, 96, 400)])
def test_bf16_equal_scores_far_below_zero(D, W, T):
    """Every score equal to about -130 in log2 units (q = -a, k = 1): the
    weights are uniform and each row is the mean of v over its window, but
    exponentials taken against a zero reference would land in the fp32 and
    bf16 subnormal range.  Rows whose first keys lie in a tile that is
    interior to every row's band must still get a reference from a row
    max."""
    a = 130.0 / (D ** 0.5 * 1.4426950408889634)
    a = float(torch.tensor(a).bfloat16())
    q = torch.full((1, 2, T, D), -a, dtype=torch.bfloat16, device=DEV)
    k = torch.ones_like(q)
    v = si.normal((1, 2, T, D), si.generator(T + W, DEV), torch.bfloat16, DEV)
    out = run_fwd(q, k, v, W)
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), W), torch.bfloat16, f"T={T} W={W}")


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_one_huge_key_matches_oracle_and_stays_local(D):
    """One key with an enormous dot product against half of the queries:
    rows whose window holds it follow it (and overflow any early reference);
    every other row is bit-identical to the run without it."""
    T, W = 900, 200
    q, k, v = si.prefill_qkv(1, 2, T, D, dtype=torch.bfloat16, seed=15, device=DEV)
    base = run_fwd(q, k, v, W)
    j0 = 300
    k2, v2 = k.clone(), v.clone()
    k2[:, :, j0] = 2000.0
    v2[:, :, j0] = -1000.0
    out = run_fwd(q, k2, v2, W)
    assert_close(out, so.swa_dense(npy(q), npy(k2), npy(v2), W), torch.bfloat16, "huge key")
    for i in range(T):
        if not (j0 <= i <= j0 + W - 1):
            assert torch.equal(out[:, :, i], base[:, :, i]), f"row {i}"


# ----------------------------------------------------------------------------
# Bitwise invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,T,W", [(torch.float32, 64, 300, 50),
                                         (torch.bfloat16, 128, 700, 100),
                                         (torch.bfloat16, 128, 700, 64),
                                         (torch.bfloat16, 64, 520, 129)])
def test_out_of_window_corruption_is_bitwise_invisible(dtype, D, T, W):
    """Corrupt k and v at j0 with large finite values: every row outside
    [j0, j0 + W - 1] is bit-identical, including row j0 + W (the sharp lower
    edge) and row j0 - 1 (the causal edge); rows inside change."""
    q, k, v = si.prefill_qkv(1, 2, T, D, dtype=dtype, seed=13, device=DEV)
    base = run_fwd(q, k, v, W)
    for j0 in (0, 63, 64, 127, 128, 200, T - W - 1):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j0] = 30.0
        v2[:, :, j0] = -1000.0
        out = run_fwd(q, k2, v2, W)
        for i in range(T):
            same = torch.equal(out[:, :, i], base[:, :, i])
            inside = j0 <= i <= j0 + W - 1
            assert same != inside, f"j0={j0} row={i} inside={inside} same={same}"


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_lower_edge_is_w_keys_not_w_plus_one(dtype, D):
    """q = k = 0 and one large value at i - W: a window of W + 1 keys would
    move row i by about 1e3 / (W + 1)."""
    T = 600
    for W in (64, 100, 256):
        v = torch.zeros(1, 1, T, D, dtype=dtype, device=DEV)
        z = torch.zeros_like(v)
        i = T - 1
        v[0, 0, i - W] = 1000.0
        out = npy(run_fwd(z, z, v, W))
        assert np.all(out[0, 0, i] == 0.0)
        assert np.all(out[0, 0, i - 1] > 1000.0 / (W + 1) * 0.9)


def test_determinism_bitwise():
    q, k, v = si.prefill_qkv(2, 8, 1000, 128, dtype=torch.bfloat16, seed=14, device=DEV)
    a = run_fwd(q, k, v, 300)
    b = run_fwd(q, k, v, 300)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_output_guard_canaries(dtype, D):
    """Writes stay inside out: canary regions on both sides are untouched."""
    B, H, T, W = 1, 3, 200, 50
    q, k, v = si.prefill_qkv(B, H, T, D, dtype=dtype, seed=15, device=DEV)
    n = B * H * T * D
    pad = 4096
    buf = torch.full((n + 2 * pad,), 123.0, dtype=dtype, device=DEV)
    out = buf[pad:pad + n].view(B, H, T, D)
    swa.swa_forward(q, k, v, out, W)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 123.0) and torch.all(buf[pad + n:] == 123.0)
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), W), dtype)


# ----------------------------------------------------------------------------
# Full-size workloads, sampled rows
# ----------------------------------------------------------------------------

def host64(x):
    """Exact fp64 host copy of a device tensor (through pinned memory)."""
    buf = torch.empty(tuple(x.shape), dtype=torch.float64, pin_memory=True)
    buf.copy_(x)
    return buf.numpy()


def _seeded_rows(T, W, n, seed):
    """n distinct rows: the window and tile edges of sample_rows, then seeded
    random rows."""
    rows = set(int(r) for r in si.sample_rows(T, W, n_random=0, seed=seed))
    rng = np.random.default_rng(seed)
    while len(rows) < min(n, T):
        rows.add(int(rng.integers(0, T)))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["prefill_bf16_b1_h32_t8192_d128_w4096",
                                  "prefill_bf16_b8_h32_t4096_d128_w1024",
                                  "prefill_bf16_b1_h32_t65536_d128_w4096"])
def test_full_size_prefill(name):
    """The benchmark workloads in the launch the benchmark times
    (swa_forward on contiguous [B, H, T, D]): every row of 4 seeded (b, h)
    pairs (the first, the last and two random ones) against the oracle's
    band-blocked tier, and 512 seeded rows (window and tile edges included)
    in every (b, h) against its per-row tier."""
    w = si.WORKLOADS[name]
    q, k, v = si.workload_qkv(w, DEV)
    out = run_fwd(q, k, v, w.W)
    qh, kh, vh = host64(q), host64(k), host64(v)
    del q, k, v
    oh = npy(out).astype(np.float64)
    rng = np.random.default_rng(w.seed + 3)
    pairs = [(0, 0), (w.B - 1, w.H - 1)]
    while len(pairs) < 4:
        p = (int(rng.integers(w.B)), int(rng.integers(w.H)))
        if p not in pairs:
            pairs.append(p)
    bound = lambda ref: BF_ATOL + BF_RTOL * np.abs(ref)
    for b, h in pairs:
        ref = so.swa_blocked(qh[b, h], kh[b, h], vh[b, h], w.W)
        err = np.abs(oh[b, h] - ref)
        bad = np.argwhere(err > bound(ref))
        assert bad.size == 0, f"{name} b={b} h={h}: {len(bad)} elements over the bar, first {bad[0]}"
    rows = _seeded_rows(w.T, w.W, 512, w.seed)
    assert len(rows) == 512
    for b in range(w.B):
        ref = so.swa_rows(qh[b], kh[b], vh[b], w.W, rows)
        got = oh[b][:, rows]
        assert np.all(np.abs(got - ref) <= bound(ref)), f"{name} b={b}: 512 rows x all heads"


@pytest.mark.parametrize("T", [(1 << 23) - 1, 1 << 23])
def test_bf16_longest_sequences_either_side_of_the_slab_limit(T):
    """The matrix-core kernel addresses a (b, h) slab of k and v with 32-bit
    byte offsets: with D = 128, T = 2^23 - 1 is the longest sequence it
    takes and T = 2^23 runs on the row kernel.  Rows at the start, the middle
    and the very end match the oracle on either side."""
    D, W = 128, 4096
    g = si.generator(T % 997, DEV)
    q, k, v = (si.normal((1, 1, T, D), g, torch.bfloat16, DEV) for _ in range(3))
    out = run_fwd(q, k, v, W)
    for i in (0, W - 1, T // 2 + 17, T - 2, T - 1):
        lo = max(0, i - W + 1)
        qs, ks, vs = (npy(x[0, :, lo:i + 1]) for x in (q, k, v))
        ref = so.swa_rows(qs, ks, vs, W, [i - lo])
        assert_close(out[0][:, i:i + 1], ref, torch.bfloat16, f"T={T} row {i}")
    del q, k, v, out


# ----------------------------------------------------------------------------
# Decode against the ring
# ----------------------------------------------------------------------------

def _ring_from_appends(kseq, vseq, pos, W):
    """Fill rings with the GPU append kernel, token by token, leaving NaN in
    the slots no token reaches (they must never be read)."""
    S, H, T, D = kseq.shape
    kr = torch.full((S, H, W, D), float("nan"), dtype=kseq.dtype, device=DEV)
    vr = torch.full_like(kr, float("nan"))
    for s in range(S):
        for t in range(max(0, pos[s] - W + 1), pos[s] + 1):
            tt = torch.tensor([t], dtype=torch.int64, device=DEV)
            swa.swa_ring_append(kseq[s:s + 1, :, t].contiguous(), vseq[s:s + 1, :, t].contiguous(),
                                kr[s:s + 1], vr[s:s + 1], tt)
    torch.cuda.synchronize()
    return kr, vr


@pytest.mark.parametrize("dtype,D,W", [(torch.bfloat16, 128, 37), (torch.bfloat16, 64, 64),
                                       (torch.float32, 128, 37), (torch.float32, 5, 9),
                                       (torch.bfloat16, 128, 300)])
def test_decode_matches_oracle_and_prefill_row(dtype, D, W):
    S, H = 5, 3
    T = 2 * W + 10
    g = si.generator(16, DEV)
    q, k, v = (si.normal((S, H, T, D), g, dtype, DEV) for _ in range(3))
    pos = [0, W - 2, W - 1, W + 3, T - 1]     # empty-ish, partly filled, just full, wrapped
    kr, vr = _ring_from_appends(k, v, pos, W)
    qs = torch.stack([q[s, :, pos[s]] for s in range(S)]).contiguous()
    out = swa.decode(qs, kr, vr, torch.as_tensor(pos, device=DEV))
    torch.cuda.synchronize()
    ref = np.stack([so.swa_rows(npy(q[s]), npy(k[s]), npy(v[s]), W, [pos[s]])[:, 0]
                    for s in range(S)])
    assert_close(out, ref, dtype, "decode vs oracle prefill row")
    # oracle decode on the very ring contents the GPU wrote
    ref2 = so.swa_decode(npy(qs), npy(kr), npy(vr), pos, W)
    assert_close(out, ref2, dtype, "decode vs oracle decode")
    # the GPU prefill row of the same sequence
    pre = swa.sliding_window_attention(q, k, v, W)
    torch.cuda.synchronize()
    rows = torch.stack([pre[s, :, pos[s]] for s in range(S)])
    assert_close(out, npy(rows).astype(np.float64), dtype, "decode vs gpu prefill row")


def test_decode_window_one_returns_current_value():
    S, H, D, W = 4, 2, 128, 1
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, seed=17, device=DEV)
    out = swa.decode(q, kr, vr, pos)
    torch.cuda.synchronize()
    assert torch.equal(out, vr[:, :, 0])


def test_decode_large_window_fallback_path():
    """W above the LDS-resident score limit goes through the row kernel."""
    S, H, D, W = 2, 2, 128, 20000
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, seed=18, device=DEV)
    out = swa.decode(q, kr, vr, pos)
    torch.cuda.synchronize()
    ref = so.swa_decode(npy(q), npy(kr), npy(vr), pos.cpu().numpy(), W)
    assert_close(out, ref, torch.bfloat16)


def test_decode_negative_position_writes_zeros():
    S, H, D, W = 2, 2, 128, 16
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, seed=19, device=DEV)
    pos = torch.tensor([-1, 3], dtype=torch.int64, device=DEV)
    out = swa.decode(q, kr, vr, pos)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    ref = so.swa_decode(npy(q[1:]), npy(kr[1:]), npy(vr[1:]), [3], W)
    assert_close(out[1:], ref, torch.bfloat16)


def test_full_size_decode_all_streams():
    """The 256-stream decode workload as the benchmark launches it: all 8192
    (stream, head) pairs against the oracle's decode, each stream's ring
    slabs copied to the host one at a time; and the launch is deterministic."""
    w = si.WORKLOADS["decode_bf16_s256_h32_d128_w4096"]
    q, kr, vr, pos = si.decode_inputs(w.S, w.H, w.D, w.W, torch.bfloat16, w.seed, DEV)
    out = swa.decode(q, kr, vr, pos)
    torch.cuda.synchronize()
    pos_h = pos.cpu().numpy()
    assert np.all(pos_h > w.W)
    qh, oh = host64(q), npy(out).astype(np.float64)
    hk = torch.empty((1, w.H, w.W, w.D), dtype=torch.float32, pin_memory=True)
    hv = torch.empty((1, w.H, w.W, w.D), dtype=torch.float32, pin_memory=True)
    worst = 0.0
    for s in range(w.S):
        hk.copy_(kr[s:s + 1])
        hv.copy_(vr[s:s + 1])
        ref = so.swa_decode(qh[s:s + 1], hk.numpy(), hv.numpy(), pos_h[s:s + 1], w.W)
        err = np.abs(oh[s:s + 1] - ref)
        worst = max(worst, float((err / (BF_ATOL + BF_RTOL * np.abs(ref))).max()))
        assert np.all(err <= BF_ATOL + BF_RTOL * np.abs(ref)), f"stream {s}"
    assert worst <= 1.0
    out2 = swa.decode(q, kr, vr, pos)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
