"""The allocation-free split decode (swa_decode_split_noalloc) against the
split decode with a caller workspace (swa_decode_split), through the C ABI.

Both run the same kernels, so the outputs must be bit-identical; each is
also checked against the fp64 oracle at the bf16 bar
|gpu - oracle| <= 2e-2 + 1e-2 |oracle|.  Two calls in a row, the second with
smaller sizes, show that what the first call left in the library's static
scratch does not leak into the second.
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
