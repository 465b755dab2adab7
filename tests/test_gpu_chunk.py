"""GPU parity of the chunked prefill that continues a ring (swa_chunk_forward)
and of the chunk append (swa_ring_append_chunk), through the C ABI, against
the fp64 oracle.

Bars: fp32 max |gpu - oracle| <= 1e-5; bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|;
the append is a copy and is checked bitwise; causality inside a chunk and
unread (NaN) ring slots are checked bitwise.
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
            f"{what}: err {err.flat[worst]:.3e} > bound {bound.flat[worst]:.3e}")


def _rings_before(kseq, vseq, pos0, W, dtype):
    """Device rings holding each stream's tokens before pos0[s] (oracle
    ring_fill), NaN in every slot no such token reaches."""
    S, H, T, D = kseq.shape
    kr = np.full((S, H, W, D), np.nan)
    vr = np.full((S, H, W, D), np.nan)
    for s in range(S):
        if pos0[s] > 0:
            a, b = so.ring_fill(npy(kseq[s:s + 1]), npy(vseq[s:s + 1]), [pos0[s] - 1], W)
            kr[s], vr[s] = a[0], b[0]
    to = lambda x: torch.from_numpy(x).to(dtype).to(DEV)
    return to(kr), to(vr)


def _chunk_case(S, H, C, D, W, pos0, dtype, seed):
    T = max(pos0) + C
    g = si.generator(seed, DEV)
    q, k, v = (si.normal((S, H, T, D), g, dtype, DEV) for _ in range(3))
    idx = torch.stack([torch.arange(p, p + C, device=DEV) for p in pos0])     # (S, C)
    take = lambda x: torch.stack([x[s, :, idx[s]] for s in range(S)]).contiguous()
    qc, kc, vc = take(q), take(k), take(v)
    kr, vr = _rings_before(k, v, pos0, W, dtype)
    return q, k, v, qc, kc, vc, kr, vr


CASES = [
    # dtype, D, W, C, pos0 per stream (fresh, partly filled, exactly full, wrapped)
    (torch.float32, 64, 37, 20, [0, 15, 37, 3 * 37 + 5]),
    (torch.float32, 7, 9, 30, [0, 4, 9, 50]),              # C > W, odd head size
    (torch.bfloat16, 128, 37, 20, [0, 15, 37, 3 * 37 + 5]),
    (torch.bfloat16, 64, 64, 100, [0, 63, 64, 200]),       # C > W
    (torch.bfloat16, 128, 300, 1, [0, 150, 299, 1000]),    # one token: a decode step
    (torch.bfloat16, 256, 16, 70, [3, 17, 80, 0]),         # largest row head size
    (torch.float32, 128, 1, 5, [0, 1, 2, 9]),              # W = 1: out == vc
]


@pytest.mark.parametrize("dtype,D,W,C,pos0", CASES)
def test_chunk_matches_oracle(dtype, D, W, C, pos0):
    S, H = len(pos0), 3
    q, k, v, qc, kc, vc, kr, vr = _chunk_case(S, H, C, D, W, pos0, dtype, seed=40 + D + C)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, kr, vr, p0)
    torch.cuda.synchronize()
    ref = so.swa_chunk(npy(qc), npy(kc), npy(vc), npy(kr), npy(vr), pos0, W)
    assert_close(out, ref, dtype, "chunk vs oracle chunk")
    # the same rows of the whole sequence, from the oracle's row tier
    for s in range(S):
        rows = so.swa_rows(npy(q[s]), npy(k[s]), npy(v[s]), W, list(range(pos0[s], pos0[s] + C)))
        assert_close(out[s], rows, dtype, f"chunk vs whole-sequence rows, stream {s}")
    if W == 1:
        assert torch.equal(out, vc)


@pytest.mark.parametrize("dtype,D,W,C", [(torch.bfloat16, 128, 37, 20), (torch.float32, 5, 8, 30),
                                         (torch.bfloat16, 64, 16, 16)])
def test_append_chunk_writes_the_window_bitwise(dtype, D, W, C):
    S, H = 3, 2
    pos0 = [0, W - 3, 5 * W + 2]
    _, k, v, _, kc, vc, kr, vr = _chunk_case(S, H, C, D, W, pos0, dtype, seed=7)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    swa.swa_ring_append_chunk(kc, vc, kr, vr, p0)
    torch.cuda.synchronize()
    for s in range(S):
        last = pos0[s] + C - 1
        ek, ev = so.ring_fill(npy(k[s:s + 1]), npy(v[s:s + 1]), [last], W)
        occ = [w for w, _ in so._ring_tokens(last, W)]
        assert np.array_equal(npy(kr[s])[:, occ], ek[0][:, occ]), f"k ring, stream {s}"
        assert np.array_equal(npy(vr[s])[:, occ], ev[0][:, occ]), f"v ring, stream {s}"


@pytest.mark.parametrize("dtype,D,W", [(torch.bfloat16, 128, 37), (torch.float32, 64, 50),
                                       (torch.bfloat16, 64, 128)])
def test_streaming_chunks_reproduce_prefill(dtype, D, W):
    """A sequence fed chunk by chunk (forward, then append) gives the rows of
    one prefill over the whole sequence; chunk sizes mix 1, < W and > W."""
    H = 2
    sizes = [1, 20, W + 13, 7, 1, 2 * W, 33]
    T = sum(sizes)
    g = si.generator(99, DEV)
    q, k, v = (si.normal((1, H, T, D), g, dtype, DEV) for _ in range(3))
    kr = torch.full((1, H, W, D), float("nan"), dtype=dtype, device=DEV)
    vr = torch.full_like(kr, float("nan"))
    outs, p = [], 0
    for C in sizes:
        sl = slice(p, p + C)
        qc, kc, vc = (x[:, :, sl].contiguous() for x in (q, k, v))
        p0 = torch.tensor([p], dtype=torch.int64, device=DEV)
        outs.append(swa.chunk_attention(qc, kc, vc, kr, vr, p0))
        swa.swa_ring_append_chunk(kc, vc, kr, vr, p0)
        p += C
    out = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    ref = so.swa_dense(npy(q[0]), npy(k[0]), npy(v[0]), W)
    assert_close(out[0], ref, dtype, "streamed chunks vs oracle prefill")
    pre = swa.sliding_window_attention(q, k, v, W)
    torch.cuda.synchronize()
    assert_close(out, npy(pre).astype(np.float64), dtype, "streamed chunks vs gpu prefill")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_is_causal_bitwise(dtype):
    """Changing chunk tokens after c never changes row c."""
    S, H, C, D, W = 2, 2, 40, 64, 24
    pos0 = [10, 100]
    _, _, _, qc, kc, vc, kr, vr = _chunk_case(S, H, C, D, W, pos0, dtype, seed=3)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    base = swa.chunk_attention(qc, kc, vc, kr, vr, p0)
    cut = 17
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, :, cut:] = 1e3
    vc2[:, :, cut:] = -7.0
    out = swa.chunk_attention(qc, kc2, vc2, kr, vr, p0)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, :cut], base[:, :, :cut])
    assert not torch.equal(out[:, :, cut:], base[:, :, cut:])


def test_chunk_full_size_sampled():
    """Mistral-7B-shaped chunk (32 heads, head size 128, window 4096) over
    full random rings at wrapped write heads; every row against the oracle."""
    S, H, C, D, W = 2, 32, 16, 128, 4096
    g = si.generator(1234, DEV)
    qc, kc, vc = (si.normal((S, H, C, D), g, torch.bfloat16, DEV) for _ in range(3))
    kr = si.normal((S, H, W, D), g, torch.bfloat16, DEV)
    vr = si.normal((S, H, W, D), g, torch.bfloat16, DEV)
    pos0 = [W + 777, 9 * W + 5]
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, kr, vr, p0)
    torch.cuda.synchronize()
    ref = so.swa_chunk(npy(qc), npy(kc), npy(vc), npy(kr), npy(vr), pos0, W)
    assert_close(out, ref, torch.bfloat16, "full-size chunk")


def test_negative_pos0_is_treated_as_zero():
    S, H, C, D, W = 1, 2, 12, 64, 8
    _, _, _, qc, kc, vc, kr, vr = _chunk_case(S, H, C, D, W, [0], torch.bfloat16, seed=5)
    a = swa.chunk_attention(qc, kc, vc, kr, vr, torch.tensor([0], device=DEV))
    b = swa.chunk_attention(qc, kc, vc, kr, vr, torch.tensor([-5], device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- the matrix-core chunk kernel (bf16, D in {64, 128}) at larger chunks ----

MFMA_CASES = [
    # D, W, C, pos0 per stream
    (128, 256, 300, [0, 100, 256, 1_000_017]),      # W a multiple of the 32-key tile
    (128, 300, 257, [7, 299, 300, 5 * 300 + 13]),   # ring wraps inside a tile
    (64, 1000, 700, [0, 999, 4321, 2_000_003]),
    (128, 40, 200, [0, 3, 41, 999]),                # W < 64
]


@pytest.mark.parametrize("D,W,C,pos0", MFMA_CASES)
def test_mfma_chunk_matches_oracle(D, W, C, pos0):
    S, H = len(pos0), 2
    dtype = torch.bfloat16
    g = si.generator(90 + W, DEV)
    qc, kc, vc = (si.normal((S, H, C, D), g, dtype, DEV) for _ in range(3))
    # rings as the stream left them: full rings of random tokens, except a
    # stream younger than W, whose slots at and above pos0 are never written
    kr = si.normal((S, H, W, D), g, dtype, DEV)
    vr = si.normal((S, H, W, D), g, dtype, DEV)
    for s in range(S):
        if pos0[s] < W:
            kr[s, :, pos0[s]:] = float("nan")
            vr[s, :, pos0[s]:] = float("nan")
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, kr, vr, p0)
    torch.cuda.synchronize()
    ref = so.swa_chunk(npy(qc), npy(kc), npy(vc), npy(kr), npy(vr), pos0, W)
    assert_close(out, ref, dtype, "mfma chunk vs oracle")


def test_mfma_chunk_stream_matches_mfma_prefill():
    """Prefill of a 2500-token sequence in chunks of 512 / 1000 / 988 through
    the matrix-core chunk kernel against one matrix-core prefill."""
    H, D, W, T = 4, 128, 640, 2500
    dtype = torch.bfloat16
    g = si.generator(97, DEV)
    q, k, v = (si.normal((1, H, T, D), g, dtype, DEV) for _ in range(3))
    kr = torch.full((1, H, W, D), float("nan"), dtype=dtype, device=DEV)
    vr = torch.full_like(kr, float("nan"))
    outs, p = [], 0
    for C in (512, 1000, 988):
        sl = slice(p, p + C)
        qc, kc, vc = (x[:, :, sl].contiguous() for x in (q, k, v))
        p0 = torch.tensor([p], dtype=torch.int64, device=DEV)
        outs.append(swa.chunk_attention(qc, kc, vc, kr, vr, p0))
        swa.swa_ring_append_chunk(kc, vc, kr, vr, p0)
        p += C
    out = torch.cat(outs, dim=2)
    pre = swa.sliding_window_attention(q, k, v, W)
    torch.cuda.synchronize()
    assert_close(out, npy(pre).astype(np.float64), dtype, "chunks vs prefill")
    rows = [0, 511, 512, 513, 1511, 1512, T - 1]
    ref = so.swa_rows(npy(q[0]), npy(k[0]), npy(v[0]), W, rows)
    assert_close(out[0][:, rows], ref, dtype, "chunks vs oracle rows")


# ---- key-range split for few streams (swa_chunk_forward_split) ----

SPLIT_CASES = [
    # D, W, C, pos0 per stream
    (128, 4096, 128, [4096 * 3 + 77]),             # one stream, one query tile: 16 splits
    (128, 1000, 300, [0, 5000]),                   # a young and a wrapped stream
    (64, 640, 200, [300, 640, 100_003]),
]


@pytest.mark.parametrize("D,W,C,pos0", SPLIT_CASES)
def test_split_chunk_matches_oracle_and_unsplit(D, W, C, pos0):
    S, H = len(pos0), 4
    dtype = torch.bfloat16
    assert swa.swa_chunk_workspace_bytes(S, H, C, D, W, dtype) > 0
    g = si.generator(200 + W, DEV)
    qc, kc, vc = (si.normal((S, H, C, D), g, dtype, DEV) for _ in range(3))
    kr = si.normal((S, H, W, D), g, dtype, DEV)
    vr = si.normal((S, H, W, D), g, dtype, DEV)
    for s in range(S):
        if pos0[s] < W:
            kr[s, :, pos0[s]:] = float("nan")
            vr[s, :, pos0[s]:] = float("nan")
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    out = swa.chunk_attention(qc, kc, vc, kr, vr, p0, split=True)
    base = swa.chunk_attention(qc, kc, vc, kr, vr, p0)
    torch.cuda.synchronize()
    ref = so.swa_chunk(npy(qc), npy(kc), npy(vc), npy(kr), npy(vr), pos0, W)
    assert_close(out, ref, dtype, "split chunk vs oracle")
    assert_close(out, npy(base).astype(np.float64), dtype, "split chunk vs unsplit")


def test_split_chunk_stream_matches_prefill():
    """A 1100-token sequence fed in chunks of 128 (the last ragged) through
    the split path, against one prefill."""
    H, D, W, T = 4, 128, 512, 1100
    dtype = torch.bfloat16
    g = si.generator(210, DEV)
    q, k, v = (si.normal((1, H, T, D), g, dtype, DEV) for _ in range(3))
    kr = torch.full((1, H, W, D), float("nan"), dtype=dtype, device=DEV)
    vr = torch.full_like(kr, float("nan"))
    outs, p = [], 0
    while p < T:
        C = min(128, T - p)
        sl = slice(p, p + C)
        qc, kc, vc = (x[:, :, sl].contiguous() for x in (q, k, v))
        p0 = torch.tensor([p], dtype=torch.int64, device=DEV)
        outs.append(swa.chunk_attention(qc, kc, vc, kr, vr, p0, split=True))
        swa.swa_ring_append_chunk(kc, vc, kr, vr, p0)
        p += C
    out = torch.cat(outs, dim=2)
    pre = swa.sliding_window_attention(q, k, v, W)
    torch.cuda.synchronize()
    assert_close(out, npy(pre).astype(np.float64), dtype, "split chunks vs prefill")


@pytest.mark.parametrize("S,C", [(1, 2048), (4, 512), (1, 128)])
def test_chunk_benchmark_shapes(S, C):
    """The chunk shapes the benchmark times (32 heads, D 128, full 4096-slot
    rings at write head 5W + 123, inputs drawn as it draws them), through both
    the plain and the split launch: every row of three (stream, head) pairs
    against the oracle (two pairs at C 2048)."""
    w = si.WORKLOADS["prefill_bf16_b1_h32_t8192_d128_w4096"]
    H, D, W = w.H, w.D, w.W
    g = si.generator(w.seed, DEV)
    qc, kc, vc = (si.normal((S, H, C, D), g, torch.bfloat16, DEV) for _ in range(3))
    kr = si.normal((S, H, W, D), g, torch.bfloat16, DEV)
    vr = si.normal((S, H, W, D), g, torch.bfloat16, DEV)
    pos0 = [5 * W + 123] * S
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    plain = torch.empty_like(qc)
    swa.swa_chunk_forward(qc, kc, vc, kr, vr, p0, plain)
    nws = swa.swa_chunk_workspace_bytes(S, H, C, D, W, torch.bfloat16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    split = torch.empty_like(qc)
    swa.swa_chunk_forward_split(qc, kc, vc, kr, vr, p0, split, ws)
    torch.cuda.synchronize()
    pairs = [(0, 0), (S - 1, H - 1), (S // 2, 13)]
    for s, h in pairs[:2] if C > 512 else pairs:
        sl = (slice(s, s + 1), slice(h, h + 1))
        ref = so.swa_chunk(npy(qc[sl]), npy(kc[sl]), npy(vc[sl]), npy(kr[sl]), npy(vr[sl]),
                           pos0[s:s + 1], W)
        assert_close(plain[sl], ref, torch.bfloat16, f"plain S={S} C={C} s={s} h={h}")
        assert_close(split[sl], ref, torch.bfloat16, f"split S={S} C={C} s={s} h={h}")
