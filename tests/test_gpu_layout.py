"""GPU parity of the strided prefill entry (swa_forward_strided) through the
C ABI: the (batch, seq, heads, head_dim) layout and its scale argument of
"Implementation: Sliding Window Attention" Step 2, the one-head (batch, seq,
d_model) layout of "25. Sliding-Window Causal Attention for Streaming
Inference", packed qkv views, padded rows, a key/value head shared by all
query heads, and explicit scales, against the fp64 oracle.

Bars: fp32 max |gpu - oracle| <= 1e-5; bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|;
bitwise where the same kernel reads the same values through other strides.
"""

import math

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


def bhtd(x):
    """(B, T, H, D) array -> (B, H, T, D)."""
    return np.ascontiguousarray(np.swapaxes(npy(x), 1, 2))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 48)])
def test_bshd_matches_oracle_and_bhtd_bitwise(dtype, D):
    B, T, H, W = 2, 300, 3, 77
    g = si.generator(31, DEV)
    q, k, v = (si.normal((B, T, H, D), g, dtype, DEV) for _ in range(3))
    out = swa.sliding_window_attention(q, k, v, W, layout="bshd")
    torch.cuda.synchronize()
    assert out.shape == (B, T, H, D)
    ref = so.swa_dense(bhtd(q), bhtd(k), bhtd(v), W)
    assert_close(out.transpose(1, 2), ref, dtype, "bshd vs oracle")
    # the same values laid out [B, H, T, D] through the contiguous entry
    c = [x.transpose(1, 2).contiguous() for x in (q, k, v)]
    base = swa.sliding_window_attention(*c, W)
    torch.cuda.synchronize()
    assert torch.equal(out.transpose(1, 2), base)


def test_packed_qkv_views_read_in_place():
    """q, k, v as views of one (B, T, 3, H, D) projection output, written
    into a view of a (B, T, H, D + 8) buffer."""
    B, T, H, D, W = 1, 700, 4, 128, 200
    g = si.generator(32, DEV)
    x = si.normal((B, T, 3, H, D), g, torch.bfloat16, DEV)
    q, k, v = x[:, :, 0], x[:, :, 1], x[:, :, 2]
    obuf = torch.full((B, T, H, D + 8), 7.0, dtype=torch.bfloat16, device=DEV)
    out = obuf[..., :D]
    swa.swa_forward_strided(*(t.permute(0, 2, 1, 3) for t in (q, k, v, out)), W)
    torch.cuda.synchronize()
    ref = so.swa_dense(bhtd(q), bhtd(k), bhtd(v), W)
    assert_close(out.transpose(1, 2), ref, torch.bfloat16, "packed qkv")
    assert torch.all(obuf[..., D:] == 7.0), "padding columns were written"
    base = swa.sliding_window_attention(*(t.transpose(1, 2).contiguous() for t in (q, k, v)), W)
    torch.cuda.synchronize()
    assert torch.equal(out.transpose(1, 2), base)


@pytest.mark.parametrize("pad", [4, 1])
def test_padded_rows_take_the_row_kernel(pad):
    """Row strides that are not a multiple of 8 elements leave the matrix-core
    kernel's alignment; the row-wise kernel must give the same attention."""
    B, H, T, D, W = 1, 2, 257, 128, 64
    g = si.generator(33, DEV)
    bufs = [si.normal((B, H, T, D + pad), g, torch.bfloat16, DEV) for _ in range(3)]
    q, k, v = (b[..., :D] for b in bufs)
    out = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=DEV)
    swa.swa_forward_strided(q, k, v, out, W)
    torch.cuda.synchronize()
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), W), torch.bfloat16, "padded rows")


def test_btd_single_head_layout():
    B, T, D, W = 3, 129, 64, 16
    g = si.generator(34, DEV)
    q, k, v = (si.normal((B, T, D), g, torch.bfloat16, DEV) for _ in range(3))
    out = swa.sliding_window_attention(q, k, v, W, layout="btd")
    torch.cuda.synchronize()
    assert out.shape == (B, T, D)
    assert_close(out, so.swa_dense(npy(q), npy(k), npy(v), W), torch.bfloat16, "btd")


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 32)])
def test_shared_kv_head_through_zero_stride(dtype, D):
    """One key/value head broadcast to every query head (head stride 0)."""
    B, H, T, W = 2, 4, 200, 50
    g = si.generator(35, DEV)
    q = si.normal((B, H, T, D), g, dtype, DEV)
    k1, v1 = (si.normal((B, 1, T, D), g, dtype, DEV) for _ in range(2))
    k, v = k1.expand(B, H, T, D), v1.expand(B, H, T, D)
    assert k.stride(1) == 0
    out = torch.empty_like(q)
    swa.swa_forward_strided(q, k, v, out, W)
    torch.cuda.synchronize()
    ref = so.swa_dense(npy(q), np.broadcast_to(npy(k1), (B, H, T, D)),
                       np.broadcast_to(npy(v1), (B, H, T, D)), W)
    assert_close(out, ref, dtype, "shared kv head")


@pytest.mark.parametrize("dtype,D,scale", [(torch.bfloat16, 128, 0.02), (torch.bfloat16, 128, 0.3),
                                           (torch.bfloat16, 64, -0.1), (torch.float32, 40, 0.5),
                                           (torch.float32, 40, -1.5)])
def test_explicit_scale(dtype, D, scale):
    B, H, T, W = 1, 3, 333, 90
    g = si.generator(36, DEV)
    q, k, v = (si.normal((B, H, T, D), g, dtype, DEV) for _ in range(3))
    out = swa.sliding_window_attention(q, k, v, W, scale=scale)
    torch.cuda.synchronize()
    ref = so.swa_dense(npy(q), npy(k), npy(v), W, scale=scale)
    assert_close(out, ref, dtype, f"scale {scale}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_explicit_default_scale_and_window_one(dtype):
    D = 64
    g = si.generator(37, DEV)
    q, k, v = (si.normal((1, 2, 150, D), g, dtype, DEV) for _ in range(3))
    a = swa.sliding_window_attention(q, k, v, 30)
    b = swa.sliding_window_attention(q, k, v, 30, scale=1 / math.sqrt(D))
    w1 = swa.sliding_window_attention(q, k, v, 1, scale=0.77)
    torch.cuda.synchronize()
    assert torch.equal(a, b)          # 1/8 is exact: the same arithmetic
    assert torch.equal(w1, v)


def test_bshd_mid_size_sampled_rows():
    """Mistral-like head layout straight from a (B, T, H, D) projection:
    T = 4096, 8 heads, W = 1024; rows at tile edges and the window edge."""
    B, T, H, D, W = 1, 4096, 8, 128, 1024
    g = si.generator(38, DEV)
    q, k, v = (si.normal((B, T, H, D), g, torch.bfloat16, DEV) for _ in range(3))
    out = swa.sliding_window_attention(q, k, v, W, layout="bshd")
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, W - 2, W - 1, W, W + 1, 2047, 2048, T - 1]
    ref = so.swa_rows(bhtd(q)[0], bhtd(k)[0], bhtd(v)[0], W, rows)
    assert_close(out[0, rows].transpose(0, 1), ref, torch.bfloat16, "bshd sampled rows")
