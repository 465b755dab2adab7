"""The allocation-free split decode (swa_decode_split_noalloc) against the
split decode with a caller workspace (swa_decode_split), through the C ABI.

Both run the same kernels, so the outputs must be bit-identical; each is
also checked against the fp64 oracle at the bf16 bar
|gpu - oracle| <= 2e-2 + 1e-2 |oracle|.  Two calls in a row, the second with
smaller sizes, show that what the first call left in the library's static
scratch does not leak into the second.  A last case captures the call in a
HIP graph and replays it with new inputs placed in the captured buffers.
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


def npy(t):
    return t.detach().float().cpu().numpy()


def _case(S, H, D, W, seed, full):
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, seed, DEV, full=full)
    need = swa.swa_decode_workspace_bytes(S, H, D, W, torch.bfloat16)
    assert 0 < need <= swa.NOALLOC_SCRATCH_BYTES     # the split (and the scratch) is used
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref = torch.empty_like(q)
    swa.swa_decode_split(q, kr, vr, pos, ref, workspace=ws)
    got = torch.full_like(q, float("nan"))
    swa.swa_decode_split_noalloc(q, kr, vr, pos, got)
    torch.cuda.synchronize()
    return q, kr, vr, pos, ref, got


def test_noalloc_split_decode_matches_the_workspace_entry_point():
    # the second call is smaller: fewer (stream, head) pairs, a shorter ring
    # and partly filled rings, so it reads only what it writes itself
    for S, H, D, W, full in ((4, 32, 128, 4096, True), (1, 8, 64, 1000, False)):
        q, kr, vr, pos, ref, got = _case(S, H, D, W, seed=S * 100 + W, full=full)
        assert torch.equal(got, ref), f"S={S} H={H} D={D} W={W}"
        oref = so.swa_decode(npy(q), npy(kr), npy(vr), pos.cpu().numpy(), W)
        err = np.abs(npy(got).astype(np.float64) - oref)
        assert np.all(err <= BF_ATOL + BF_RTOL * np.abs(oref)), f"max err {err.max():.3e}"
        del q, kr, vr, pos, ref, got


def test_noalloc_without_a_split_runs_the_plain_decode():
    """Sizes with no split (S * H >= 512) take no scratch and give
    swa_decode's result."""
    S, H, D, W = 32, 16, 128, 256
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, 7, DEV)
    assert swa.swa_decode_workspace_bytes(S, H, D, W, torch.bfloat16) == 0
    ref = torch.empty_like(q)
    swa.swa_decode(q, kr, vr, pos, ref)
    got = torch.full_like(q, float("nan"))
    swa.swa_decode_split_noalloc(q, kr, vr, pos, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_noalloc_decode_replays_in_a_hip_graph():
    """What the entry point is for: a decode step captured in a HIP graph
    (no allocation, no workspace, no memset in the captured work) and
    replayed with new queries and write positions placed in the captured
    buffers between replays; each replay equals an eager call on the same
    inputs, bit for bit."""
    S, H, D, W = 2, 8, 128, 1024
    q, kr, vr, pos = si.decode_inputs(S, H, D, W, torch.bfloat16, 11, DEV)
    assert 0 < swa.swa_decode_workspace_bytes(S, H, D, W, torch.bfloat16) <= swa.NOALLOC_SCRATCH_BYTES
    out = torch.empty_like(q)
    # an eager call first: the library looks up its scratch address and sets
    # kernel attributes outside the capture
    swa.swa_decode_split_noalloc(q, kr, vr, pos, out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swa.swa_decode_split_noalloc(q, kr, vr, pos, out)
    torch.cuda.synchronize()
    gen = si.generator(12, DEV)
    rng = np.random.default_rng(13)
    for r in range(3):
        q.copy_(si.normal(tuple(q.shape), gen, torch.bfloat16, DEV))
        pos.copy_(torch.tensor(rng.integers(0, 3 * W, S), dtype=torch.int64, device=DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(q)
        swa.swa_decode_split_noalloc(q, kr, vr, pos, ref)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}"
    del graph
