"""Pins of the CPU oracle to what the pages and the mathematics fix.

Runs on the CPU only.  Every oracle function is checked against something
other than itself: the two printed masks, P5's printed worked example, the
reduction of W >= T to a library causal-attention routine
(``torch.nn.functional.scaled_dot_product_attention`` in float64), W = 1
returning v, the trailing moving average for zero Q/K (prefix-sum closed form),
out-of-window corruption invariance, convexity, time-shift invariance and brute
force on tiny inputs.  The mutation tests at the end plant mistakes in the
oracle and check that at least one pin fails for each.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import swa_oracle as so

TIERS = {
    "dense": lambda q, k, v, W: so.swa_dense(q, k, v, W),
    "rows": lambda q, k, v, W: so.swa_rows(q, k, v, W, range(q.shape[-2])),
    # small blocks, so the pins' short sequences span several of them
    "blocked": lambda q, k, v, W: so.swa_blocked(q, k, v, W, block=3),
    "loop": lambda q, k, v, W: so.swa_loop(q, k, v, W),
}


def _rng(seed):
    return np.random.default_rng(seed)


def _load_mask(name):
    lines = read_golden(name)
    header = dict(tok.split("=") for tok in lines[0].split())
    T, W = int(header["T"]), int(header["W"])
    grid = lines[1:]
    assert len(grid) == T
    if "." in "".join(grid):
        m = np.array([[c == "." for c in row] for row in grid])
    else:
        m = np.array([[c == "1" for c in row] for row in grid])
    assert m.shape == (T, T)
    return T, W, m


PRINTED_MASKS = ["mask_8tok_w4.txt", "mask_5tok_w3.txt"]


def _load_p5():
    lines = read_golden("p5_moving_average.txt")
    W = int(lines[0].split("=")[1])
    i_x = lines.index("x")
    i_out = lines.index("out")
    i_c = lines.index("corrupt_row0")
    i_u = lines.index("unchanged_from_row")
    x = np.array([[float(t) for t in ln.split()] for ln in lines[i_x + 1:i_out]])
    out = np.array([[float(t) for t in ln.split()] for ln in lines[i_out + 1:i_c]])
    corrupt = np.array([float(t) for t in lines[i_c + 1].split()])
    unchanged_from = int(lines[i_u + 1])
    return W, x, out, corrupt, unchanged_from


def _sdpa(q, k, v, mask=None, causal=False):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    attn_mask = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=attn_mask, is_causal=causal).numpy()


# ----------------------------------------------------------------------------
# Pin checks, each returning True when the pin holds for an oracle callable
# fn(q, k, v, W) -> (..., T, D).
# ----------------------------------------------------------------------------

def pin_mask_probe(fn):
    """q = k = 0 and v = one-hot rows: out[i, j] = 1/n_i on visible keys, 0
    elsewhere, so out > 0 reproduces the band.  Compared with both printed
    masks."""
    for name in PRINTED_MASKS:
        T, W, m = _load_mask(name)
        z = np.zeros((1, T, T))
        out = fn(z, z, np.eye(T)[None], W)[0]
        if not np.array_equal(out > 0, m):
            return False
        n = m.sum(axis=1, keepdims=True)
        if not np.allclose(out, m / n, rtol=0, atol=1e-15):
            return False
    return True


def pin_causal_sdpa(fn):
    """W >= T reduces to ordinary causal attention [P1 step 6; P2 step 6;
    P5 first section]; compared with torch's SDPA in float64."""
    r = _rng(11)
    T, D = 12, 5
    q, k, v = (r.standard_normal((2, 3, T, D)) for _ in range(3))
    ref = _sdpa(q, k, v, causal=True)
    return all(np.max(np.abs(fn(q, k, v, W) - ref)) <= 1e-12 for W in (T, T + 1, 2 * T))


def pin_band_sdpa(fn):
    """Any W: torch's SDPA given the (printed-mask-pinned) band as a boolean
    attention mask."""
    r = _rng(12)
    T, D = 20, 6
    q, k, v = (r.standard_normal((2, T, D)) for _ in range(3))
    for W in (1, 2, 3, 7, 19):
        ref = _sdpa(q, k, v, mask=so.band_mask(T, W))
        if np.max(np.abs(fn(q, k, v, W) - ref)) > 1e-12:
            return False
    return True


def pin_w1(fn):
    """W = 1 is self-attention only [P5 first section]: the output is v,
    exactly (one weight exp(0) = 1, divided by 1)."""
    r = _rng(13)
    q, k, v = (r.standard_normal((3, 10, 4)) for _ in range(3))
    return np.array_equal(fn(q, k, v, 1), v)


def pin_moving_average(fn):
    """Zero Q and K give uniform weights over the window [P5 worked-example
    discussion], so out_i = (C[i+1] - C[lo_i]) / n_i with prefix sums C."""
    r = _rng(14)
    T, D = 17, 3
    v = r.standard_normal((2, T, D))
    z = np.zeros((2, T, D))
    for W in (1, 2, 5, 16, 17, 40):
        C = np.concatenate([np.zeros((2, 1, D)), np.cumsum(v, axis=1)], axis=1)
        lo = np.maximum(0, np.arange(T) - W + 1)
        n = (np.arange(T) - lo + 1)[None, :, None]
        ref = (C[:, np.arange(T) + 1] - C[:, lo]) / n
        if np.max(np.abs(fn(z, z, v, W) - ref)) > 1e-12:
            return False
    return True


def pin_p5_example(fn):
    """P5's printed worked example: two heads of width 1, Q = K = 0, V = x.
    The page's values are integers; the oracle reaches them up to the fp64
    rounding of the 1/3 weights (1e-12).  Replacing row 0 leaves rows 3
    onward unchanged, exactly."""
    W, x, expected, corrupt, unchanged_from = _load_p5()
    T = x.shape[0]
    z = np.zeros((2, T, 1))
    heads = x.T[:, :, None]                         # (H=2, T, Dh=1)
    out = fn(z, z, heads, W)[:, :, 0].T             # back to (T, 2)
    if np.max(np.abs(out - expected)) > 1e-12:
        return False
    x2 = x.copy()
    x2[0] = corrupt
    out2 = fn(z, z, x2.T[:, :, None], W)[:, :, 0].T
    return np.array_equal(out2[unchanged_from:], out[unchanged_from:]) and \
        not np.array_equal(out2[:unchanged_from], out[:unchanged_from])


def pin_corruption(fn):
    """Corrupting k and v of one position j0 with large finite values leaves
    every query outside [j0, j0 + W - 1] bit-for-bit unchanged and changes
    every query inside it [P2 step 6 and its corrupt-and-compare note; P5
    worked example assertion]."""
    r = _rng(15)
    T, D = 24, 4
    q, k, v = (r.standard_normal((1, T, D)) for _ in range(3))
    for W in (1, 3, 8):
        base = fn(q, k, v, W)
        for j0 in (0, 5, 11, T - 1):
            k2, v2 = k.copy(), v.copy()
            k2[0, j0] = 1e6
            v2[0, j0] = -3e5
            out = fn(q, k2, v2, W)
            for i in range(T):
                same = np.array_equal(out[0, i], base[0, i])
                inside = j0 <= i <= j0 + W - 1
                if inside == same:
                    return False
    return True


PINS = [pin_mask_probe, pin_causal_sdpa, pin_band_sdpa, pin_w1, pin_moving_average,
        pin_p5_example, pin_corruption]


# ----------------------------------------------------------------------------
# The pins hold for every tier
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("tier", sorted(TIERS))
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(tier, pin):
    assert pin(TIERS[tier])


@pytest.mark.parametrize("name", PRINTED_MASKS)
def test_band_mask_equals_printed(name):
    T, W, m = _load_mask(name)
    assert np.array_equal(so.band_mask(T, W), m)


def test_printed_mask_reading():
    """P3's reading of its mask: row 0 sees only itself, row 3 sees 0..3,
    row 4 drops position 0, every later row sees exactly W positions."""
    T, W, m = _load_mask("mask_8tok_w4.txt")
    assert list(np.flatnonzero(m[0])) == [0]
    assert list(np.flatnonzero(m[3])) == [0, 1, 2, 3]
    assert list(np.flatnonzero(m[4])) == [1, 2, 3, 4]
    assert all(m[i].sum() == W for i in range(W - 1, T))


@pytest.mark.parametrize("T,W", [(8, 4), (5, 3), (10, 1), (10, 9), (6, 6), (6, 20)])
def test_page4_form_is_the_off_by_one(T, W):
    """P4's max(0, i-W) <= j <= i admits W + 1 keys: it equals the band of
    width W + 1 and not the band of width W (unless W >= T)."""
    p4 = so.band_mask_max_form(T, W)
    assert np.array_equal(p4, so.band_mask(T, W + 1))
    assert np.array_equal(p4, so.band_mask(T, W)) == (W >= T)


@pytest.mark.parametrize("name", PRINTED_MASKS)
def test_page4_form_differs_from_printed(name):
    T, W, m = _load_mask(name)
    p4 = so.band_mask_max_form(T, W)
    assert not np.array_equal(p4, m)
    assert p4[W, 0] and not m[W, 0]


def test_tiers_agree_random():
    r = _rng(21)
    for T, D, W in [(1, 1, 1), (7, 3, 2), (9, 5, 4), (16, 8, 5), (11, 2, 30)]:
        q, k, v = (r.standard_normal((2, T, D)) for _ in range(3))
        ref = so.swa_dense(q, k, v, W)
        assert np.max(np.abs(so.swa_rows(q, k, v, W, range(T)) - ref)) <= 1e-12
        assert np.max(np.abs(so.swa_loop(q, k, v, W) - ref)) <= 1e-12
        for block in (1, 2, 5, T, 256):
            assert np.max(np.abs(so.swa_blocked(q, k, v, W, block=block) - ref)) <= 1e-12


@pytest.mark.parametrize("T,W,block,scale", [(300, 64, 64, None), (300, 64, 37, None),
                                             (257, 300, 50, 0.3), (200, 1, 16, None),
                                             (129, 128, 128, -0.2)])
def test_blocked_tier_matches_dense_across_blocks(T, W, block, scale):
    """Blocks aligned and not aligned with W, W > T, W = 1, a ragged last
    block and explicit (also negative) scales: the band-blocked tier is the
    dense recipe to 1e-12."""
    r = _rng(T + W + block)
    q, k, v = (r.standard_normal((2, T, 16)) for _ in range(3))
    ref = so.swa_dense(q, k, v, W, scale=scale)
    got = so.swa_blocked(q, k, v, W, block=block, scale=scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_blocked_tier_row_ranges_are_rows_of_the_whole():
    r = _rng(31)
    T, W = 300, 70
    q, k, v = (r.standard_normal((3, T, 8)) for _ in range(3))
    ref = so.swa_dense(q, k, v, W)
    for a, b, block in ((0, T, 64), (69, 69 + 64, 64), (100, 101, 16), (250, T, 7), (5, 5, 4)):
        got = so.swa_blocked(q, k, v, W, block=block, start=a, stop=b)
        assert got.shape == (3, b - a, 8)
        assert np.max(np.abs(got - ref[:, a:b]), initial=0.0) <= 1e-12


def test_blocked_tier_rejects_bad_arguments():
    x = np.zeros((4, 2))
    with pytest.raises(IndexError):
        so.swa_blocked(x, x, x, 2, start=3, stop=2)
    with pytest.raises(IndexError):
        so.swa_blocked(x, x, x, 2, stop=5)
    with pytest.raises(ValueError):
        so.swa_blocked(x, x, x, 2, block=0)
    with pytest.raises(ValueError):
        so.swa_blocked(x, x, x, 0)
    with pytest.raises(ValueError):
        so.swa_blocked(x, np.zeros((5, 2)), x, 2)


def test_convexity():
    """Softmax weights are non-negative and sum to 1 [P3 closing remarks], so
    each output coordinate lies inside the range of the window's values."""
    r = _rng(22)
    T, D, W = 30, 6, 7
    q, k, v = (3.0 * r.standard_normal((T, D)) for _ in range(3))
    out, wts = so.swa_dense(q, k, v, W, return_weights=True)
    assert np.all(wts >= 0) and np.allclose(wts.sum(-1), 1.0, atol=1e-14)
    for i in range(T):
        lo = max(0, i - W + 1)
        win = v[lo:i + 1]
        assert np.all(out[i] >= win.min(0) - 1e-12) and np.all(out[i] <= win.max(0) + 1e-12)


def test_time_shift():
    """Only the window matters: dropping a prefix of s tokens leaves row i
    unchanged whenever its whole window lies after the prefix."""
    r = _rng(23)
    T, D, W, s = 40, 4, 6, 9
    q, k, v = (r.standard_normal((T, D)) for _ in range(3))
    full = so.swa_dense(q, k, v, W)
    tail = so.swa_dense(q[s:], k[s:], v[s:], W)
    for i in range(s + W - 1, T):
        assert np.max(np.abs(full[i] - tail[i - s])) <= 1e-12


def test_page_shapes():
    """Doctest shapes of P1 and P2 and the printed shapes of P3's demo."""
    r = _rng(24)
    x = r.standard_normal((1, 2, 6, 4))
    assert so.swa_dense(x, x, x, 3).shape == (1, 2, 6, 4)
    y = r.standard_normal((1, 5, 3))
    assert so.swa_dense(y, y, y, 2).shape == (1, 5, 3)
    assert np.max(np.abs(so.swa_dense(y, y, y, 5) - _sdpa(y, y, y, causal=True))) <= 1e-12
    # P3 works in (batch, seq, heads, dim) and transposes to heads-first.
    bshd = r.standard_normal((1, 16, 4, 32))
    t = bshd.transpose(0, 2, 1, 3)
    out, w = so.swa_dense(t, t, t, 4, return_weights=True)
    assert out.transpose(0, 2, 1, 3).shape == (1, 16, 4, 32)
    assert w.shape == (1, 4, 16, 16)
    assert np.all(w[..., ~so.band_mask(16, 4)] == 0)


def test_page3_demo_qualitative():
    """P3's demo (unseeded on the page, seeded here): head 0 with q_i = 6 k_i
    puts most weight on the diagonal, head 1 with tiny queries is close to
    uniform inside the window.  Qualitative only: the page prints no values."""
    r = np.random.default_rng(25)
    B, T, H, D, W = 1, 16, 4, 32, 4
    q = r.standard_normal((B, T, H, D)).astype(np.float32)
    k = r.standard_normal((B, T, H, D)).astype(np.float32)
    v = r.standard_normal((B, T, H, D)).astype(np.float32)
    for i in range(1, T):
        q[0, i, 0] = k[0, i, 0] * 6.0
    q[0, :, 1] = r.standard_normal((T, D)).astype(np.float32) * 0.05
    tr = lambda a: a.transpose(0, 2, 1, 3)
    out, w = so.swa_dense(tr(q), tr(k), tr(v), W, return_weights=True)
    diag = np.array([w[0, 0, i, i] for i in range(1, T)])
    assert diag.mean() >= 0.95
    for i in range(T):
        n = min(i + 1, W)
        band = w[0, 1, i, max(0, i - W + 1):i + 1]
        assert np.all(np.abs(band - 1.0 / n) <= 0.25 / n)


@pytest.mark.parametrize("W", [0, -1])
def test_nonpositive_window_rejected(W):
    x = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        so.swa_dense(x, x, x, W)
    with pytest.raises(ValueError):
        so.swa_rows(x, x, x, W, [0])
    with pytest.raises(ValueError):
        so.band_mask(4, W)


# ----------------------------------------------------------------------------
# Decode and chunked prefill over the W-slot ring
# ----------------------------------------------------------------------------

def test_ring_slot_layout():
    """Ring of W = 4 slots after position 10: tokens 7, 8, 9, 10 sit in slots
    3, 0, 1, 2 (p mod W); slots no token reached stay at the fill value."""
    T, W = 12, 4
    seq = np.arange(T, dtype=np.float64).reshape(1, 1, T, 1)
    kr, vr = so.ring_fill(seq, seq, [10], W)
    assert kr[0, 0, :, 0].tolist() == [8.0, 9.0, 10.0, 7.0]
    kr, _ = so.ring_fill(seq, seq, [1], W)
    assert kr[0, 0, :2, 0].tolist() == [0.0, 1.0] and np.all(np.isnan(kr[0, 0, 2:, 0]))


def _decode_case(S, H, T, D, W, seed):
    r = _rng(seed)
    q, k, v = (r.standard_normal((S, H, T, D)) for _ in range(3))
    pos = r.integers(0, T, size=S)
    return q, k, v, pos


def test_decode_equals_prefill_row():
    S, H, T, D, W = 4, 3, 50, 5, 7
    q, k, v, pos = _decode_case(S, H, T, D, W, 31)
    pos[0], pos[1] = 0, W - 2          # partly filled rings
    kr, vr = so.ring_fill(k, v, pos, W)
    qs = np.stack([q[s, :, pos[s]] for s in range(S)])
    out = so.swa_decode(qs, kr, vr, pos, W)
    for s in range(S):
        ref = so.swa_rows(q[s], k[s], v[s], W, [pos[s]])[:, 0]
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


def test_decode_partial_fill_matches_causal_and_ignores_empty_slots():
    """While fewer than W tokens exist the ring's empty slots (NaN here) are
    never read and the result is plain causal attention over the prefix."""
    H, T, D, W = 2, 9, 3, 16
    r = _rng(32)
    q, k, v = (r.standard_normal((1, H, T, D)) for _ in range(3))
    p = T - 1
    kr, vr = so.ring_fill(k, v, [p], W)
    assert np.isnan(kr).any()
    out = so.swa_decode(q[:, :, p], kr, vr, [p], W)
    ref = _sdpa(q[0], k[0], v[0], causal=True)[:, p]
    assert np.all(np.isfinite(out)) and np.max(np.abs(out[0] - ref)) <= 1e-12


def test_decode_rotation_invariance_and_w1():
    S, H, T, D, W = 2, 2, 30, 4, 6
    q, k, v, pos = _decode_case(S, H, T, D, W, 33)
    pos[:] = [20, 25]
    kr, vr = so.ring_fill(k, v, pos, W)
    qs = np.stack([q[s, :, pos[s]] for s in range(S)])
    base = so.swa_decode(qs, kr, vr, pos, W)
    # the same tokens with the write head shifted by W keep their slots
    shifted = so.swa_decode(qs, kr, vr, pos + W, W)
    assert np.max(np.abs(base - shifted)) <= 1e-12
    # W = 1: a one-slot ring returns the current value exactly
    kr1, vr1 = so.ring_fill(k, v, pos, 1)
    out1 = so.swa_decode(qs, kr1, vr1, pos, 1)
    assert np.array_equal(out1, np.stack([v[s, :, pos[s]] for s in range(S)]))


def test_decode_zero_qk_is_window_mean():
    S, H, T, D, W = 3, 2, 40, 3, 5
    q, k, v, pos = _decode_case(S, H, T, D, W, 34)
    pos[:] = [2, 4, 33]
    z = np.zeros_like(k)
    kr, vr = so.ring_fill(z, v, pos, W)
    out = so.swa_decode(np.zeros((S, H, D)), kr, vr, pos, W)
    for s in range(S):
        lo = max(0, pos[s] - W + 1)
        assert np.max(np.abs(out[s] - v[s, :, lo:pos[s] + 1].mean(axis=1))) <= 1e-12


def test_chunk_continues_ring():
    """Chunked prefill over (ring of earlier tokens + chunk) equals prefill
    rows of the whole sequence."""
    S, H, T, D, W, C = 3, 2, 60, 4, 9, 7
    r = _rng(35)
    q, k, v = (r.standard_normal((S, H, T, D)) for _ in range(3))
    pos0 = np.array([0, 5, 40])
    kr, vr = np.full((S, H, W, D), np.nan), np.full((S, H, W, D), np.nan)
    for s in range(S):
        if pos0[s] > 0:
            a, b = so.ring_fill(k[s:s + 1], v[s:s + 1], [pos0[s] - 1], W)
            kr[s], vr[s] = a[0], b[0]
    qc = np.stack([q[s, :, pos0[s]:pos0[s] + C] for s in range(S)])
    kc = np.stack([k[s, :, pos0[s]:pos0[s] + C] for s in range(S)])
    vc = np.stack([v[s, :, pos0[s]:pos0[s] + C] for s in range(S)])
    out = so.swa_chunk(qc, kc, vc, kr, vr, pos0, W)
    for s in range(S):
        ref = so.swa_rows(q[s], k[s], v[s], W, range(pos0[s], pos0[s] + C))
        assert np.all(np.isfinite(out[s]))
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


# ----------------------------------------------------------------------------
# Explicit score scale [P3 Step 2: scores = q k^T * scale, default 1/sqrt(D)]
# ----------------------------------------------------------------------------

def _sdpa_scaled(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("scale", [0.05, 0.7, 2.0])
def test_scale_reduces_to_library_causal_attention(scale):
    """W >= T with an explicit scale equals torch's SDPA given that scale
    (torch's math path mishandles negative scales under its causal mask, so
    those are pinned by the sign symmetry below)."""
    r = _rng(21)
    T, D = 13, 6
    q, k, v = (r.standard_normal((2, 2, T, D)) for _ in range(3))
    ref = _sdpa_scaled(q, k, v, scale, causal=True)
    for fn in (lambda W: so.swa_dense(q, k, v, W, scale=scale),
               lambda W: so.swa_rows(q, k, v, W, range(T), scale=scale)):
        for W in (T, 2 * T):
            assert np.max(np.abs(fn(W) - ref)) <= 1e-12


def test_scale_default_is_inverse_sqrt_d_and_band_matches_library():
    r = _rng(22)
    T, D = 16, 8
    q, k, v = (r.standard_normal((3, T, D)) for _ in range(3))
    for W in (1, 4, 9):
        a = so.swa_dense(q, k, v, W)
        b = so.swa_dense(q, k, v, W, scale=1 / math.sqrt(D))
        assert np.max(np.abs(a - b)) <= 1e-12
        t = lambda x: torch.from_numpy(x)
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(q), t(k), t(v), attn_mask=t(so.band_mask(T, W)), scale=0.37).numpy()
        assert np.max(np.abs(so.swa_dense(q, k, v, W, scale=0.37) - ref)) <= 1e-12
        rows = so.swa_rows(q, k, v, W, [0, 3, T - 1], scale=0.37)
        assert np.max(np.abs(rows - ref[:, [0, 3, T - 1]])) <= 1e-12


def test_negative_scale_is_negated_queries():
    """scale = -s scores q . k * (-s) = (-q) . k * s; negating q is exact."""
    r = _rng(24)
    T, D = 10, 4
    q, k, v = (r.standard_normal((2, T, D)) for _ in range(3))
    for W in (2, 5, 10):
        a = so.swa_dense(q, k, v, W, scale=-0.4)
        b = so.swa_dense(-q, k, v, W, scale=0.4)
        assert np.array_equal(a, b)
        assert np.max(np.abs(so.swa_rows(q, k, v, W, range(T), scale=-0.4) - a)) <= 1e-12


def test_scale_zero_is_trailing_moving_average():
    """scale = 0 zeroes every score: uniform weights over the window, the
    closed-form trailing mean of v."""
    r = _rng(23)
    T, D = 11, 3
    q, k, v = (r.standard_normal((1, T, D)) for _ in range(3))
    C = np.concatenate([np.zeros((1, 1, D)), np.cumsum(v, axis=1)], axis=1)
    for W in (1, 3, 11):
        lo = np.maximum(np.arange(T) - W + 1, 0)
        n = (np.arange(T) - lo + 1)[None, :, None]
        ref = (C[:, 1:] - C[:, lo]) / n
        assert np.max(np.abs(so.swa_dense(q, k, v, W, scale=0.0) - ref)) <= 1e-12


def test_nonfinite_scale_rejected():
    x = np.zeros((1, 4, 2))
    for bad in (float("nan"), float("inf")):
        with pytest.raises(ValueError):
            so.swa_dense(x, x, x, 2, scale=bad)


# ----------------------------------------------------------------------------
# Backward (gradients of the band attention)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("W", [1, 3, 8, 30])
@pytest.mark.parametrize("scale", [None, 0.4])
def test_backward_matches_library_autograd(W, scale):
    """torch autograd through its own scaled dot-product attention (band as a
    boolean mask), float64 on the CPU."""
    r = _rng(41 + W)
    T, D = 19, 6
    q, k, v, do = (r.standard_normal((2, T, D)) for _ in range(4))
    dq, dk, dv = so.swa_backward(q, k, v, W, do, scale=scale)
    t = lambda a: torch.from_numpy(a.copy()).requires_grad_(True)
    qt, kt, vt = t(q), t(k), t(v)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(so.band_mask(T, W)), scale=scale)
    out.backward(torch.from_numpy(do))
    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-12


@pytest.mark.parametrize("W,scale", [(1, None), (4, None), (11, 0.3), (40, None)])
def test_lse_matches_library_logsumexp(W, scale):
    """torch.logsumexp over the masked scores, and weights = exp(s - lse)."""
    r = _rng(45 + W)
    T, D = 15, 5
    q, k, v = (r.standard_normal((2, T, D)) for _ in range(3))
    lse = so.swa_lse(q, k, W, scale=scale)
    sc = 1 / math.sqrt(D) if scale is None else scale
    s = torch.from_numpy(q @ np.swapaxes(k, -1, -2) * sc)
    s = s.masked_fill(~torch.from_numpy(so.band_mask(T, W)), -math.inf)
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12
    _, P = so.swa_dense(q, k, v, W, return_weights=True, scale=scale)
    band = so.band_mask(T, W)
    assert np.max(np.abs(np.where(band, np.exp(s.numpy() - lse[..., None]), 0.0) - P)) <= 1e-12


def test_backward_matches_finite_differences():
    """Central differences of sum(dout * out) on a tiny case (step 1e-6)."""
    r = _rng(42)
    T, D, W = 6, 3, 3
    q, k, v, do = (r.standard_normal((T, D)) for _ in range(4))
    grads = so.swa_backward(q, k, v, W, do)
    f = lambda a, b, c: float(np.sum(do * so.swa_dense(a, b, c, W)))
    h = 1e-6
    for which in range(3):
        args = [q, k, v]
        num = np.zeros_like(args[which])
        for idx in np.ndindex(num.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            num[idx] = (f(*plus) - f(*minus)) / (2 * h)
        assert np.max(np.abs(num - grads[which])) <= 1e-7


def test_backward_window_one_closed_form():
    """W = 1: out = v, so dv = dout and dq = dk = 0 exactly."""
    r = _rng(43)
    q, k, v, do = (r.standard_normal((4, 7, 5)) for _ in range(4))
    dq, dk, dv = so.swa_backward(q, k, v, 1, do)
    assert np.array_equal(dv, do)
    assert not np.any(dq) and not np.any(dk)


def test_backward_gradient_support_is_the_window():
    """dk_j and dv_j come only from queries i in [j, j + W - 1]: zeroing dout
    there zeroes them."""
    r = _rng(44)
    T, D, W, j = 20, 4, 5, 7
    q, k, v, do = (r.standard_normal((T, D)) for _ in range(4))
    do2 = do.copy()
    do2[j:j + W] = 0.0
    _, dk, dv = so.swa_backward(q, k, v, W, do2)
    assert not np.any(dk[j]) and not np.any(dv[j])
    _, dk, dv = so.swa_backward(q, k, v, W, do)
    assert np.any(dk[j]) and np.any(dv[j])


# ----------------------------------------------------------------------------
# Module forward [P5 "A complete example with moving averages"]
# ----------------------------------------------------------------------------

def test_mha_forward_reproduces_p5_printed_example():
    """d_model 2, two heads, zero Q/K kernels, identity V and output kernels,
    zero biases: the page's printed output, and rows from 3 on unchanged when
    row 0 is replaced."""
    W, x, expected, corrupt, unchanged_from = _load_p5()
    z, eye = np.zeros((2, 2)), np.eye(2)
    out = so.mha_forward(x, z, None, z, None, eye, None, eye, None, 2, W)
    assert np.max(np.abs(out - expected)) <= 1e-12
    x2 = x.copy()
    x2[0] = corrupt
    out2 = so.mha_forward(x2, z, None, z, None, eye, None, eye, None, 2, W)
    assert np.array_equal(out2[unchanged_from:], out[unchanged_from:])
    assert not np.array_equal(out2[:unchanged_from], out[:unchanged_from])


@pytest.mark.parametrize("H,W", [(1, 3), (2, 5), (4, 1), (4, 40)])
def test_mha_forward_matches_library_multihead_attention(H, W):
    """torch's multi-head attention (its own projections, head split and
    output projection) with the band as a boolean mask, in float64."""
    r = _rng(31 + H + W)
    T, dm = 17, 8
    x = r.standard_normal((2, T, dm))
    ws = [r.standard_normal((dm, dm)) / math.sqrt(dm) for _ in range(4)]
    bs = [r.standard_normal(dm) for _ in range(4)]
    out = so.mha_forward(x, ws[0], bs[0], ws[1], bs[1], ws[2], bs[2], ws[3], bs[3], H, W)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    xt = t(np.swapaxes(x, 0, 1))                      # (T, B, dm), torch's default layout
    in_w = t(np.concatenate([w.T for w in ws[:3]], axis=0))   # torch applies x @ w^T
    in_b = t(np.concatenate(bs[:3]))
    masked = t(~so.band_mask(T, W))                   # True = not allowed, in torch's convention
    ref, _ = torch.nn.functional.multi_head_attention_forward(
        xt, xt, xt, dm, H, in_w, in_b, None, None, False, 0.0, t(ws[3].T), t(bs[3]),
        training=False, need_weights=False, attn_mask=masked)
    ref = np.swapaxes(ref.numpy(), 0, 1)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_mha_forward_one_head_identity_is_self_attention():
    """One head with identity kernels and zero biases is the attention of x
    with itself."""
    x = _rng(35).standard_normal((9, 4))
    eye = np.eye(4)
    out = so.mha_forward(x, eye, None, eye, None, eye, None, eye, None, 1, 4)
    assert np.max(np.abs(out - so.swa_dense(x, x, x, 4))) <= 1e-12


def test_mha_forward_rejects_bad_heads():
    x = np.zeros((3, 6))
    w = np.zeros((6, 6))
    with pytest.raises(ValueError):
        so.mha_forward(x, w, None, w, None, w, None, w, None, 4, 2)


# ----------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

MUTANTS = {
    # W + 1 keys (P4's form)
    "window_plus_one": lambda q, k, v, W: so.swa_dense(q, k, v, W + 1),
    # W - 1 keys (strict bound on the wrong side); W = 1 degenerates, keep >= 1
    "window_minus_one": lambda q, k, v, W: so.swa_dense(q, k, v, max(W - 1, 1)) if W > 1
    else so.swa_dense(q, k, v, W) * 0.5,
    # k and v swapped
    "k_v_swapped": lambda q, k, v, W: so.swa_dense(q, v, k, W) if k.shape == v.shape
    else so.swa_dense(q, k, v, W) + 1.0,
    # scale 1/D instead of 1/sqrt(D)
    "scale_one_over_d": lambda q, k, v, W: so.swa_dense(q / math.sqrt(q.shape[-1]), k, v, W),
    # no scale at all
    "no_scale": lambda q, k, v, W: so.swa_dense(q * math.sqrt(q.shape[-1]), k, v, W),
    # q and k swapped: transposes the score matrix
    "scores_transposed": lambda q, k, v, W: so.swa_dense(k, q, v, W),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    fn = MUTANTS[name]
    assert not all(p(fn) for p in PINS)


def test_planted_mask_mistake_is_caught(monkeypatch):
    """Plant P4's off-by-one inside the oracle's own mask; the printed-mask
    probe and the corruption pin must fail."""
    monkeypatch.setattr(so, "band_mask", so.band_mask_max_form)
    fn = TIERS["dense"]
    assert not pin_mask_probe(fn)
    assert not pin_corruption(fn)


def test_planted_noncausal_mistake_is_caught(monkeypatch):
    def symmetric(T, W):
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        return np.abs(i - j) < W
    monkeypatch.setattr(so, "band_mask", symmetric)
    assert not pin_mask_probe(TIERS["dense"])
    assert not pin_causal_sdpa(TIERS["dense"])


@pytest.mark.parametrize("T,W,scale", [(23, 1, None), (23, 5, None), (23, 9, 0.35),
                                       (23, 23, None), (23, 40, -0.2), (64, 17, None)])
def test_backward_rows_match_full_backward(T, W, scale):
    """The sampled-row gradients equal the full chain-rule gradients (which the
    tests above pin to torch autograd and central differences) on every row,
    including rows whose band is cut by the sequence start or end."""
    r = _rng(60 + T + W)
    D, Dv = 6, 4
    q, k = r.standard_normal((T, D)), r.standard_normal((T, D))
    v, do = r.standard_normal((T, Dv)), r.standard_normal((T, Dv))
    dq, dk, dv = so.swa_backward(q, k, v, W, do, scale=scale)
    rows = range(T)
    sq, sk, sv = so.swa_backward_rows(q, k, v, W, do, rows, rows, scale=scale)
    for mine, ref in ((sq, dq), (sk, dk), (sv, dv)):
        assert np.max(np.abs(mine - ref)) <= 1e-12
    # an arbitrary sample, in any order, gives those rows
    qs, ks = [T - 1, 0, T // 2], [3, T - 1, 0]
    sq, sk, sv = so.swa_backward_rows(q, k, v, W, do, qs, ks, scale=scale)
    assert np.max(np.abs(sq - dq[qs])) <= 1e-12
    assert np.max(np.abs(sk - dk[ks])) <= 1e-12
    assert np.max(np.abs(sv - dv[ks])) <= 1e-12


def test_backward_rows_rejects_rows_outside_the_sequence():
    x = np.zeros((4, 2))
    with pytest.raises(IndexError):
        so.swa_backward_rows(x, x, x, 2, x, [4], [])
    with pytest.raises(IndexError):
        so.swa_backward_rows(x, x, x, 2, x, [], [-1])


@pytest.mark.parametrize("H,W,bias", [(1, 3, True), (2, 5, False), (4, 40, True), (3, 1, True)])
def test_mha_rows_match_the_module_forward(H, W, bias):
    """Sampled rows of the module equal the pinned mha_forward's rows, in any
    order and with repeats."""
    r = _rng(70 + H + W)
    T, dm = 21, 12
    x = r.standard_normal((T, dm))
    ws = [r.standard_normal((dm, dm)) / math.sqrt(dm) for _ in range(4)]
    bs = [r.standard_normal(dm) if bias else None for _ in range(4)]
    args = (ws[0], bs[0], ws[1], bs[1], ws[2], bs[2], ws[3], bs[3], H, W)
    ref = so.mha_forward(x, *args)
    assert np.max(np.abs(so.mha_rows(x, *args, range(T)) - ref)) <= 1e-12
    rows = [T - 1, 0, 7, 7, W]
    rows = [i for i in rows if i < T]
    assert np.max(np.abs(so.mha_rows(x, *args, rows) - ref[rows])) <= 1e-12
