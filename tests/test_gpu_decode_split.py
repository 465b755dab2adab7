"""GPU parity of the split-window decode (swa_decode_split) and the fused
append + decode (swa_decode_append), through the C ABI, against the fp64
oracle.

Bars: fp32 max |gpu - oracle| <= 1e-5; bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|;
ring contents bitwise; the fused launch bitwise equal to append-then-split-decode
(the same kernel reads the same values).
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


def _rings(kseq, vseq, pos, W, dtype):
    """Device rings of every stream up to and including position pos[s]
    (oracle ring_fill), NaN in slots no token reaches."""
    kr, vr = so.ring_fill(npy(kseq), npy(vseq), pos, W)
    to = lambda x: torch.from_numpy(x).to(dtype).to(DEV)
    return to(kr), to(vr)


def _case(S, H, D, W, pos, dtype, seed):
    T = max(pos) + 2
    g = si.generator(seed, DEV)
    q, k, v = (si.normal((S, H, T, D), g, dtype, DEV) for _ in range(3))
    return q, k, v


SPLIT_CASES = [
    # S, H, D, W, positions (fresh, partial, just full, wrapped)
    (1, 4, 128, 4096, [4095 + 777]),
    (2, 3, 128, 1000, [0, 999 * 3 + 5]),
    (3, 4, 64, 300, [5, 298, 1201]),
    (1, 2, 64, 37, [100]),                 # too short to split: one workgroup
    (2, 8, 128, 513, [511, 512]),
]


@pytest.mark.parametrize("S,H,D,W,pos", SPLIT_CASES)
def test_split_decode_matches_oracle(S, H, D, W, pos):
    dtype = torch.bfloat16
    q, k, v = _case(S, H, D, W, pos, dtype, seed=50 + W)
    kr, vr = _rings(k, v, pos, W, dtype)
    qs = torch.stack([q[s, :, pos[s]] for s in range(S)]).contiguous()
    p = torch.tensor(pos, dtype=torch.int64, device=DEV)
    out = swa.decode(qs, kr, vr, p, split=True)
    base = swa.decode(qs, kr, vr, p)
    torch.cuda.synchronize()
    ref = so.swa_decode(npy(qs), npy(kr), npy(vr), pos, W)
    assert_close(out, ref, dtype, "split decode vs oracle")
    assert_close(base, ref, dtype, "decode vs oracle")
    rows = np.stack([so.swa_rows(npy(q[s]), npy(k[s]), npy(v[s]), W, [pos[s]])[:, 0]
                     for s in range(S)])
    assert_close(out, rows, dtype, "split decode vs prefill row")


def test_small_batch_uses_a_workspace():
    assert swa.swa_decode_workspace_bytes(1, 32, 128, 4096, torch.bfloat16) > 0
    assert swa.swa_decode_workspace_bytes(256, 32, 128, 4096, torch.bfloat16) == 0
    assert swa.swa_decode_workspace_bytes(1, 32, 128, 4096, torch.float32) > 0
    assert swa.swa_decode_workspace_bytes(1, 32, 48, 4096, torch.float32) == 0


@pytest.mark.parametrize("dtype,D,W", [(torch.bfloat16, 128, 600), (torch.bfloat16, 64, 37),
                                       (torch.float32, 48, 50)])
def test_fused_append_writes_ring_and_attends(dtype, D, W):
    S, H = 3, 4
    pos = [0, W - 1, 3 * W + 11]
    q, k, v = _case(S, H, D, W, pos, dtype, seed=60 + D)
    prev = [max(p - 1, 0) for p in pos]
    kr, vr = _rings(k, v, prev, W, dtype)
    for s in range(S):
        if pos[s] == 0:                     # nothing before the first token
            kr[s].fill_(float("nan"))
            vr[s].fill_(float("nan"))
    kr2, vr2 = kr.clone(), vr.clone()
    take = lambda x: torch.stack([x[s, :, pos[s]] for s in range(S)]).contiguous()
    qs, kn, vn = take(q), take(k), take(v)
    p = torch.tensor(pos, dtype=torch.int64, device=DEV)
    out = swa.decode_append(qs, kn, vn, kr, vr, p)
    # the unfused order: append, then the split decode
    swa.swa_ring_append(kn, vn, kr2, vr2, p)
    out2 = swa.decode(qs, kr2, vr2, p, split=True)
    torch.cuda.synchronize()
    ek, ev = so.ring_fill(npy(k), npy(v), pos, W)
    for s in range(S):
        occ = [w for w, _ in so._ring_tokens(pos[s], W)]
        assert np.array_equal(npy(kr[s])[:, occ], ek[s][:, occ])
        assert np.array_equal(npy(vr[s])[:, occ], ev[s][:, occ])
    assert torch.equal(out, out2)
    ref = so.swa_decode(npy(qs), ek, ev, pos, W)
    assert_close(out, ref, dtype, "fused append + decode")


@pytest.mark.parametrize("D,W", [(128, 64), (64, 300)])
def test_token_by_token_stream_reproduces_prefill(D, W):
    """A whole sequence decoded token by token with the fused launch (ring
    starts empty) gives the rows of one prefill over the sequence."""
    S, H, T = 2, 2, 400
    dtype = torch.bfloat16
    g = si.generator(70 + D, DEV)
    q, k, v = (si.normal((S, H, T, D), g, dtype, DEV) for _ in range(3))
    kr = torch.full((S, H, W, D), float("nan"), dtype=dtype, device=DEV)
    vr = torch.full_like(kr, float("nan"))
    outs = []
    for t in range(T):
        p = torch.full((S,), t, dtype=torch.int64, device=DEV)
        outs.append(swa.decode_append(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                      v[:, :, t].contiguous(), kr, vr, p))
    out = torch.stack(outs, dim=2)
    torch.cuda.synchronize()
    for s in range(S):
        assert_close(out[s], so.swa_dense(npy(q[s]), npy(k[s]), npy(v[s]), W), dtype,
                     f"stream {s}")


def test_fused_negative_position():
    S, H, D, W = 2, 2, 128, 40
    dtype = torch.bfloat16
    g = si.generator(80, DEV)
    qs, kn, vn = (si.normal((S, H, D), g, dtype, DEV) for _ in range(3))
    kr = torch.zeros((S, H, W, D), dtype=dtype, device=DEV)
    vr = torch.zeros_like(kr)
    p = torch.tensor([-3, 5], dtype=torch.int64, device=DEV)
    out = swa.decode_append(qs, kn, vn, kr, vr, p)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    assert torch.equal(kr[0, :, W - 3], kn[0]) and torch.equal(vr[0, :, W - 3], vn[0])
    assert torch.equal(kr[1, :, 5], kn[1])


@pytest.mark.parametrize("pos", [16383 + 5000, 9000])
def test_sixty_four_way_split_merge(pos):
    """One head against a 16384-slot ring takes the most splits, 64: the
    merge's lanes cover them all, in eight batches of partial rows.  Also a
    ring only partly filled (position 9000), where the last splits are empty
    (their max is -inf) and must not contribute."""
    S, H, D, W = 1, 1, 128, 16384
    assert swa.swa_decode_workspace_bytes(S, H, D, W, torch.bfloat16) == 64 * (D + 2) * 4
    q, k, v = _case(S, H, D, W, [pos], torch.bfloat16, seed=pos)
    kr, vr = _rings(k, v, [pos], W, torch.bfloat16)
    qs = q[:, :, pos].contiguous()
    p = torch.tensor([pos], dtype=torch.int64, device=DEV)
    out = swa.decode(qs, kr, vr, p, split=True)
    whole = swa.decode(qs, kr, vr, p)
    torch.cuda.synchronize()
    ek, ev = so.ring_fill(npy(k), npy(v), [pos], W)
    ref = so.swa_decode(npy(qs), ek, ev, [pos], W)
    assert_close(out, ref, torch.bfloat16, f"64-way split, pos {pos}")
    assert_close(whole, ref, torch.bfloat16, f"one workgroup, pos {pos}")


def test_full_size_single_stream_split():
    """One stream, 32 heads, D = 128, a full 4096-slot ring at a wrapped head."""
    S, H, D, W = 1, 32, 128, 4096
    qs, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, 1234, DEV)
    out = swa.decode(qs, kr, vr, pos, split=True)
    torch.cuda.synchronize()
    ref = so.swa_decode(npy(qs), npy(kr), npy(vr), pos.cpu().tolist(), W)
    assert_close(out, ref, torch.bfloat16, "full-size split decode")


@pytest.mark.parametrize("D,W", [(128, 97), (64, 64)])
def test_both_lane_mappings(D, W):
    """Launches of at least 256 workgroups read each slot row with D / 8
    lanes and non-temporal loads; smaller ones with quads of lanes.  Both,
    plain, split and fused with the append, against the oracle, on rings
    fresh, partly filled, just full and wrapped."""
    S, H = 16, 16                      # 256 workgroups: the row mapping
    dtype = torch.bfloat16
    pos = [[0, 1, W // 2, W - 1, W, 2 * W + 3, 3 * W - 1, 3 * W + 7][s % 8] for s in range(S)]
    q, k, v = _case(S, H, D, W, pos, dtype, seed=90 + D)
    kr, vr = _rings(k, v, pos, W, dtype)
    qs = torch.stack([q[s, :, pos[s]] for s in range(S)]).contiguous()
    p = torch.tensor(pos, dtype=torch.int64, device=DEV)
    ref = so.swa_decode(npy(qs), npy(kr), npy(vr), pos, W)
    rows_map = swa.decode(qs, kr, vr, p)
    split = swa.decode(qs, kr, vr, p, split=True)
    # two streams alone: 32 workgroups, the quad mapping
    quad_map = swa.decode(qs[:2].contiguous(), kr[:2].contiguous(), vr[:2].contiguous(), p[:2])
    torch.cuda.synchronize()
    assert_close(rows_map, ref, dtype, "row mapping")
    assert_close(split, ref, dtype, "split")
    assert_close(quad_map, ref[:2], dtype, "quad mapping")
    # fused append in the row mapping: the rings up to pos - 1 plus the token
    prev = [max(x - 1, 0) for x in pos]
    kr2, vr2 = _rings(k, v, prev, W, dtype)
    for s in range(S):
        if pos[s] == 0:
            kr2[s].fill_(float("nan"))
            vr2[s].fill_(float("nan"))
    take = lambda x: torch.stack([x[s, :, pos[s]] for s in range(S)]).contiguous()
    fused = swa.decode_append(qs, take(k), take(v), kr2, vr2, p)
    torch.cuda.synchronize()
    assert_close(fused, ref, dtype, "fused append, row mapping")


def test_workspace_on_another_device_is_rejected_before_any_launch():
    """A caller workspace that is not a contiguous tensor on the inputs' device
    raises in the binding (split decode, fused append, chunk split, backward),
    before the library is called."""
    q, kr, vr, pos = si.decode_inputs(1, 4, 128, 256, torch.bfloat16, 3, DEV)
    out = torch.empty_like(q)
    host_ws = torch.empty(1 << 20, dtype=torch.uint8)
    strided_ws = torch.empty(2 << 20, dtype=torch.uint8, device=DEV)[::2]
    for ws in (host_ws, strided_ws):
        with pytest.raises(ValueError, match="workspace"):
            swa.swa_decode_split(q, kr, vr, pos, out, workspace=ws)
        with pytest.raises(ValueError, match="workspace"):
            swa.swa_decode_append(q, q, q, kr, vr, pos, out, workspace=ws)
    qc = torch.zeros((1, 4, 64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="workspace"):
        swa.swa_chunk_forward_split(qc, qc, qc, kr, vr, pos, torch.empty_like(qc),
                                    workspace=host_ws)
    t = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=DEV)
    g = [torch.empty_like(t) for _ in range(3)]
    with pytest.raises(ValueError, match="workspace"):
        swa.swa_backward(t, t, t, t, t, *g, 16, workspace=host_ws)
