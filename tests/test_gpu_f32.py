"""GPU: the fp32 matrix-core prefill and backward (head sizes 32, 64, 128)
against the fp64 oracle, at sizes that span several 32-row tiles with ragged
tails, windows from 1 past T, scales of both signs; W = 1 bit for bit; and
sampled rows of a full [1, 32, 8192, 128] layer, forward and backward.

Bars: max |gpu - oracle| <= 1e-5 (outputs); 1e-5 * max(1, max |oracle|)
(gradients, log-sum-exp).
"""

import numpy as np
import pytest
import torch

import sliding_window_causal_amd as swa
import swa_inputs as si
from oracle import swa_oracle as so

pytestmark = pytest.mark.gpu

DEV = "cuda"
ATOL = 1e-5


def npy(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def close(gpu, ref, what, rel=False):
    bound = ATOL * (max(1.0, float(np.abs(ref).max())) if rel else 1.0)
    err = np.abs(npy(gpu) - ref).max()
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"


CASES = [(D, T, W, scale) for D in (32, 64, 128)
         for (T, W) in ((1, 1), (31, 5), (33, 32), (97, 33), (300, 64), (300, 300), (129, 400))
         for scale in (None, -0.2)]


@pytest.mark.parametrize("D,T,W,scale", CASES)
def test_f32_prefill_and_lse(D, T, W, scale):
    g = si.generator(7000 + D + T + W, DEV)
    q, k, v = (si.normal((2, 3, T, D), g, torch.float32, DEV) for _ in range(3))
    out = torch.empty_like(q)
    lse = torch.empty((2, 3, T), dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out, lse, W, scale=scale)
    plain = swa.sliding_window_attention(q, k, v, W, scale=scale)
    torch.cuda.synchronize()
    close(out, so.swa_dense(npy(q), npy(k), npy(v), W, scale=scale), "out")
    close(lse, so.swa_lse(npy(q), npy(k), W, scale=scale), "lse", rel=True)
    assert torch.equal(out, plain)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_f32_window_one_returns_v(D):
    g = si.generator(7100 + D, DEV)
    q, k, v = (si.normal((1, 2, 77, D), g, torch.float32, DEV) for _ in range(3))
    assert torch.equal(swa.sliding_window_attention(q, k, v, 1), v)
    assert torch.equal(swa.sliding_window_attention(q, k, v, 1, scale=-0.7), v)


BWD = [(D, T, W, scale) for D in (32, 64, 128)
       for (T, W) in ((31, 5), (97, 33), (200, 64), (130, 300))
       for scale in (None, -0.2)]


@pytest.mark.parametrize("D,T,W,scale", BWD)
def test_f32_backward(D, T, W, scale):
    g = si.generator(7200 + D + T + W, DEV)
    q, k, v, do = (si.normal((1, 2, T, D), g, torch.float32, DEV) for _ in range(4))
    out = torch.empty_like(q)
    lse = torch.empty((1, 2, T), dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out, lse, W, scale=scale)
    a = [torch.empty_like(q) for _ in range(3)]
    b = [torch.empty_like(q) for _ in range(3)]
    swa.swa_backward(q, k, v, out, do, *a, W, scale=scale)
    swa.swa_backward(q, k, v, out, do, *b, W, scale=scale, lse=lse)
    torch.cuda.synchronize()
    refs = so.swa_backward(npy(q), npy(k), npy(v), W, npy(do), scale=scale)
    for name, x, y, r in zip(("dq", "dk", "dv"), a, b, refs):
        close(x, r, name, rel=True)
        assert torch.equal(x, y), f"{name}: kept lse and forward rerun differ"


def test_f32_full_size_sampled_rows():
    B, H, T, D, W = 1, 32, 8192, 128, 4096
    g = si.generator(7300, DEV)
    q, k, v = (si.normal((B, H, T, D), g, torch.float32, DEV) for _ in range(3))
    out = swa.sliding_window_attention(q, k, v, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7301)
    for h in rng.choice(H, 4, replace=False):
        rows = np.sort(np.concatenate([rng.choice(T, 60, replace=False), [0, 31, 32, W - 1, W, T - 1]]))
        qh, kh, vh = (npy(x[0, h]) for x in (q, k, v))
        ref = so.swa_rows(qh[None], kh[None], vh[None], W, rows)[0]
        close(out[0, h, rows], ref, f"head {h}")


def test_f32_full_size_backward_sampled_rows():
    """The fp32 backward of a full [1, 32, 8192, 128] layer, W = 4096, on the
    matrix cores with the forward's log-sum-exp kept and with the forward
    rerun (bit for bit the same): dq of sampled query rows and dk, dv of
    sampled key rows (window and tile edges, sequence ends, random rows) in
    three heads against the oracle's band-only gradients."""
    B, H, T, D, W = 1, 32, 8192, 128, 4096
    g = si.generator(7400, DEV)
    q, k, v, do = (si.normal((B, H, T, D), g, torch.float32, DEV) for _ in range(4))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(q, k, v, out, lse, W)
    kept = [torch.empty_like(q) for _ in range(3)]
    rerun = [torch.empty_like(q) for _ in range(3)]
    swa.swa_backward(q, k, v, out, do, *kept, W, lse=lse)
    swa.swa_backward(q, k, v, out, do, *rerun, W)
    torch.cuda.synchronize()
    for x, y in zip(kept, rerun):
        assert torch.equal(x, y), "kept lse and forward rerun differ"
    q_rows = si.sample_rows(T, W, n_random=8, seed=7401)
    k_rows = [0, 32, W - 1, W, T - W, T - 1, 5000]
    for h in (0, 17, H - 1):
        rq, rk, rv = so.swa_backward_rows(npy(q[0, h]), npy(k[0, h]), npy(v[0, h]), W,
                                          npy(do[0, h]), q_rows, k_rows)
        dq, dk, dv = kept
        close(dq[0, h][torch.as_tensor(q_rows, device=DEV)], rq, f"dq head {h}", rel=True)
        close(dk[0, h][torch.as_tensor(k_rows, device=DEV)], rk, f"dk head {h}", rel=True)
        close(dv[0, h][torch.as_tensor(k_rows, device=DEV)], rv, f"dv head {h}", rel=True)


@pytest.mark.parametrize("D,W,S,H", [(32, 50, 2, 3), (64, 97, 16, 16), (128, 64, 2, 2), (128, 40, 32, 8)])
def test_f32_decode(D, W, S, H):
    """fp32 decode on the bf16 decode kernel's two lane mappings (quads of
    lanes below 256 workgroups, D / 4 lanes per slot row from 256 up), rings
    fresh, partly filled, full and wrapped."""
    pos = [[0, 1, W // 2, W - 1, W, 2 * W + 3, 3 * W - 1, 3 * W + 7][s % 8] for s in range(S)]
    T = max(pos) + 1
    g = si.generator(7400 + D + W, DEV)
    q, k, v = (si.normal((S, H, T, D), g, torch.float32, DEV) for _ in range(3))
    kr, vr = so.ring_fill(npy(k), npy(v), pos, W)
    to = lambda x: torch.from_numpy(x).float().to(DEV)
    kr, vr = to(kr), to(vr)
    qs = torch.stack([q[s, :, pos[s]] for s in range(S)]).contiguous()
    p = torch.tensor(pos, dtype=torch.int64, device=DEV)
    out = swa.decode(qs, kr, vr, p)
    torch.cuda.synchronize()
    ref = so.swa_decode(npy(qs), npy(kr), npy(vr), pos, W)
    close(out, ref, "decode")
    rows = np.stack([so.swa_rows(npy(q[s]), npy(k[s]), npy(v[s]), W, [pos[s]])[:, 0] for s in range(S)])
    close(out, rows, "decode vs prefill row")


@pytest.mark.parametrize("D,W,C,pos0", [(32, 45, 70, [0, 44, 45, 3 * 45 + 7]),
                                        (128, 64, 100, [5, 63, 64, 1000]),
                                        (64, 100, 33, [2 ** 31 + 77, 99, 7, 0])])
def test_f32_chunk(D, W, C, pos0):
    """fp32 chunk continuation on the matrix cores: tiles that straddle the
    ring and the chunk, rings fresh, partly filled, full and wrapped, and a
    stream position past 2^31 (positions taken relative to an origin)."""
    S, H = len(pos0), 2
    g = si.generator(7500 + D + W, DEV)
    qc, kc, vc = (si.normal((S, H, C, D), g, torch.float32, DEV) for _ in range(3))
    # ring contents: tokens p0 - W .. p0 - 1 of each stream at slot (t mod W)
    kprev, vprev = (si.normal((S, H, W, D), g, torch.float32, DEV) for _ in range(2))
    kr = torch.full((S, H, W, D), float("nan"), device=DEV)
    vr = torch.full_like(kr, float("nan"))
    for s, p0 in enumerate(pos0):
        for j in range(W):
            t = p0 - W + j
            if t >= 0:
                kr[s, :, t % W] = kprev[s, :, j]
                vr[s, :, t % W] = vprev[s, :, j]
    p = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, kr, vr, p)
    torch.cuda.synchronize()
    # the oracle on the explicit sequence: the W ring tokens (those that
    # exist), then the chunk
    for s, p0 in enumerate(pos0):
        nprev = min(p0, W)
        keys = torch.cat([kprev[s, :, W - nprev:], kc[s]], dim=1)
        vals = torch.cat([vprev[s, :, W - nprev:], vc[s]], dim=1)
        qs = torch.cat([torch.zeros((H, nprev, D), device=DEV), qc[s]], dim=1)
        ref = so.swa_rows(npy(qs), npy(keys), npy(vals), W, range(nprev, nprev + C))
        close(out[s], ref, f"stream {s} (p0 {p0})")


@pytest.mark.parametrize("D,W,S,H,pos", [(128, 4096, 1, 4, [4095 + 777]), (32, 300, 3, 2, [5, 298, 1201]),
                                         (64, 1000, 2, 3, [0, 999 * 3 + 5])])
def test_f32_split_and_fused_decode(D, W, S, H, pos):
    """fp32 split decode (partials merged by the combine kernel, which also
    handles D = 32 with half its lanes idle) and the fused append + decode,
    against the oracle; the fused launch bitwise equal to append then split
    decode."""
    T = max(pos) + 1
    g = si.generator(7600 + D + W, DEV)
    q, k, v = (si.normal((S, H, T, D), g, torch.float32, DEV) for _ in range(3))
    assert swa.swa_decode_workspace_bytes(S, H, D, W, torch.float32) > 0
    to = lambda x: torch.from_numpy(x).float().to(DEV)
    kr, vr = (to(x) for x in so.ring_fill(npy(k), npy(v), pos, W))
    qs = torch.stack([q[s, :, pos[s]] for s in range(S)]).contiguous()
    p = torch.tensor(pos, dtype=torch.int64, device=DEV)
    split = swa.decode(qs, kr, vr, p, split=True)
    noalloc = torch.empty_like(qs)
    swa.swa_decode_split_noalloc(qs, kr, vr, p, noalloc)
    prev = [max(x - 1, 0) for x in pos]
    kr2, vr2 = (to(x) for x in so.ring_fill(npy(k), npy(v), prev, W))
    for s in range(S):
        if pos[s] == 0:
            kr2[s].fill_(float("nan"))
            vr2[s].fill_(float("nan"))
    kr3, vr3 = kr2.clone(), vr2.clone()
    take = lambda x: torch.stack([x[s, :, pos[s]] for s in range(S)]).contiguous()
    fused = swa.decode_append(qs, take(k), take(v), kr2, vr2, p)
    swa.swa_ring_append(take(k), take(v), kr3, vr3, p)
    unfused = swa.decode(qs, kr3, vr3, p, split=True)
    torch.cuda.synchronize()
    ref = so.swa_decode(npy(qs), npy(kr), npy(vr), pos, W)
    close(split, ref, "split decode")
    close(fused, ref, "fused append + decode")
    assert torch.equal(noalloc, split)
    assert torch.equal(fused, unfused)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_f32_out_of_window_corruption_is_bitwise_invisible(D):
    """k[j0] and v[j0] set to +-3e38 (finite fp32; the dot products with q
    overflow): every row outside [j0, j0 + W - 1] keeps its output and its
    log-sum-exp bit for bit.  j0 runs over tile edges, keys at i - W for
    tile-aligned rows i, and keys a wavefront walks but does not need."""
    T, W = 300, 100
    g = si.generator(7700 + D, DEV)
    q, k, v = (si.normal((1, 2, T, D), g, torch.float32, DEV) for _ in range(3))

    def fwd(kk, vv):
        out = torch.empty_like(q)
        lse = torch.empty((1, 2, T), dtype=torch.float32, device=DEV)
        swa.swa_forward_lse(q, kk, vv, out, lse, W)
        torch.cuda.synchronize()
        return out, lse

    base, lbase = fwd(k, v)
    sign = torch.where(torch.arange(D, device=DEV) % 2 == 0, 1.0, -1.0)
    for j0 in (0, 31, 32, 63, 64 - W + 100, 95, 96, 127, 128, 159, 160 - W + 100, 191, 250, T - W - 1, T - 1):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j0] = 3e38 * sign
        v2[:, :, j0] = -3e38 * sign
        out, lse = fwd(k2, v2)
        rows = np.array([i for i in range(T) if not (j0 <= i <= j0 + W - 1)])
        if len(rows) == 0:
            continue
        assert torch.equal(out[:, :, rows], base[:, :, rows]), f"j0={j0}: rows changed"
        assert torch.equal(lse[:, :, rows], lbase[:, :, rows]), f"j0={j0}: lse changed"
