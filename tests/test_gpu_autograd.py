"""GPU parity of the differentiable sliding_window_attention: with inputs
that require grad, the forward runs swa_forward_lse and torch's autograd
calls swa_backward with that log-sum-exp.  Gradients are checked against the
fp64 oracle's swa_backward (the chain rule through the dense recipe, pinned
to torch autograd and central differences) and bitwise against the explicit
C-ABI calls they stand for.

Bars as in the backward tests: fp32 max |gpu - oracle| <= 1e-5 * max(1,
max |oracle|); bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|.
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


def _check(gpu, ref, dtype, what):
    g = npy(gpu).astype(np.float64)
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - ref)
    if dtype == torch.float32:
        bound = 1e-5 * max(1.0, np.abs(ref).max())
        assert err.max() <= bound, f"{what}: max err {err.max():.3e} > {bound:.3e}"
    else:
        b = BF_ATOL + BF_RTOL * np.abs(ref)
        worst = np.argmax(err - b)
        assert np.all(err <= b), f"{what}: err {err.flat[worst]:.3e} > {b.flat[worst]:.3e}"


def _leaves(shape, dtype, seed, n=3):
    g = si.generator(seed, DEV)
    return [si.normal(shape, g, dtype, DEV).requires_grad_() for _ in range(n)]


@pytest.mark.parametrize("dtype,D,T,W", [(torch.float32, 64, 150, 37),
                                         (torch.bfloat16, 128, 300, 64),
                                         (torch.bfloat16, 64, 257, 300)])
def test_autograd_matches_oracle(dtype, D, T, W):
    q, k, v = _leaves((1, 2, T, D), dtype, 500 + D + W)
    do = si.normal((1, 2, T, D), si.generator(600 + W, DEV), dtype, DEV)
    out = swa.sliding_window_attention(q, k, v, W)
    out.backward(do)
    torch.cuda.synchronize()
    _check(out, so.swa_dense(npy(q), npy(k), npy(v), W), dtype, "out")
    rq, rk, rv = so.swa_backward(npy(q), npy(k), npy(v), W, npy(do))
    _check(q.grad, rq, dtype, "dq")
    _check(k.grad, rk, dtype, "dk")
    _check(v.grad, rv, dtype, "dv")


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_autograd_is_the_explicit_calls_bitwise(dtype, D):
    """Output equal to swa_forward's, gradients equal to swa_backward's given
    the lse of swa_forward_lse, bit for bit."""
    T, W = 200, 50
    q, k, v = _leaves((2, 2, T, D), dtype, 700 + D)
    do = si.normal((2, 2, T, D), si.generator(701, DEV), dtype, DEV)
    out = swa.sliding_window_attention(q, k, v, W)
    out.backward(do)
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    plain = torch.empty_like(qd)
    swa.swa_forward(qd, kd, vd, plain, W)
    o2, lse = torch.empty_like(qd), torch.empty((2, 2, T), dtype=torch.float32, device=DEV)
    swa.swa_forward_lse(qd, kd, vd, o2, lse, W)
    grads = [torch.empty_like(qd) for _ in range(3)]
    swa.swa_backward(qd, kd, vd, o2, do, *grads, W, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), plain)
    for name, a, b in zip("qkv", (q.grad, k.grad, v.grad), grads):
        assert torch.equal(a, b), f"d{name}"


@pytest.mark.parametrize("scale", [0.3, -0.2])
def test_autograd_at_a_sharp_explicit_scale(scale):
    """D = 128 with an explicit scale well above 1/sqrt(D) (and a negative
    one) through autograd, against the oracle at the bf16 bar."""
    T, D, W = 300, 128, 100
    q, k, v = _leaves((1, 2, T, D), torch.bfloat16, 960)
    do = si.normal((1, 2, T, D), si.generator(961, DEV), torch.bfloat16, DEV)
    out = swa.sliding_window_attention(q, k, v, W, scale=scale)
    out.backward(do)
    torch.cuda.synchronize()
    _check(out, so.swa_dense(npy(q), npy(k), npy(v), W, scale=scale), torch.bfloat16, "out")
    rq, rk, rv = so.swa_backward(npy(q), npy(k), npy(v), W, npy(do), scale=scale)
    _check(q.grad, rq, torch.bfloat16, "dq")
    _check(k.grad, rk, torch.bfloat16, "dk")
    _check(v.grad, rv, torch.bfloat16, "dv")


def test_autograd_layouts_and_scale_match_bhtd():
    """[B, T, H, D] and [B, T, D] inputs, with an explicit scale, give the
    [B, H, T, D] path's output and gradients, moved back to their layout."""
    T, D, W, scale = 180, 64, 40, 0.2
    q, k, v = _leaves((1, 3, T, D), torch.bfloat16, 800)
    do = si.normal((1, 3, T, D), si.generator(801, DEV), torch.bfloat16, DEV)
    out = swa.sliding_window_attention(q, k, v, W, scale=scale)
    out.backward(do)
    # BSHD leaves holding the same values
    qs, ks, vs = (t.detach().transpose(1, 2).contiguous().requires_grad_() for t in (q, k, v))
    out_s = swa.sliding_window_attention(qs, ks, vs, W, scale=scale, layout="bshd")
    out_s.backward(do.transpose(1, 2))
    assert torch.equal(out_s.detach().transpose(1, 2), out.detach())
    for a, b in zip((qs.grad, ks.grad, vs.grad), (q.grad, k.grad, v.grad)):
        assert torch.equal(a.transpose(1, 2), b)
    # one head as [B, T, D]
    q1, k1, v1 = (t.detach()[:, 0].clone().requires_grad_() for t in (q, k, v))
    out1 = swa.sliding_window_attention(q1, k1, v1, W, scale=scale)
    out1.backward(do[:, 0])
    assert torch.equal(out1.detach(), out.detach()[:, 0])
    for a, b in zip((q1.grad, k1.grad, v1.grad), (q.grad, k.grad, v.grad)):
        assert torch.equal(a, b[:, 0])


def test_autograd_through_a_shared_kv_head():
    """K and V of one head expanded over four query heads: autograd sums the
    four heads' key and value gradients into the shared head, which must
    match the oracle's per-head gradients summed."""
    T, D, W, H = 160, 64, 48, 4
    g = si.generator(900, DEV)
    q = si.normal((1, H, T, D), g, torch.float32, DEV).requires_grad_()
    k1 = si.normal((1, 1, T, D), g, torch.float32, DEV).requires_grad_()
    v1 = si.normal((1, 1, T, D), g, torch.float32, DEV).requires_grad_()
    do = si.normal((1, H, T, D), g, torch.float32, DEV)
    out = swa.sliding_window_attention(q, k1.expand(1, H, T, D), v1.expand(1, H, T, D), W)
    out.backward(do)
    torch.cuda.synchronize()
    kk, vv = np.repeat(npy(k1), H, axis=1), np.repeat(npy(v1), H, axis=1)
    rq, rk, rv = so.swa_backward(npy(q), kk, vv, W, npy(do))
    _check(q.grad, rq, torch.float32, "dq")
    _check(k1.grad, rk.sum(axis=1, keepdims=True), torch.float32, "dk (summed)")
    _check(v1.grad, rv.sum(axis=1, keepdims=True), torch.float32, "dv (summed)")


def test_no_grad_path_is_unchanged():
    """Under torch.no_grad (or without inputs that require grad) the call is
    the plain forward: no log-sum-exp, no graph."""
    q, k, v = _leaves((1, 2, 100, 64), torch.bfloat16, 950)
    with torch.no_grad():
        out = swa.sliding_window_attention(q, k, v, 30)
    assert out.grad_fn is None and not out.requires_grad
    out2 = swa.sliding_window_attention(q.detach(), k.detach(), v.detach(), 30)
    assert out2.grad_fn is None
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
