"""GPU: every output element of the three full-size bf16 prefill workloads,
launched as the benchmark launches them, against a property that holds at any
size: softmax weights are non-negative and sum to one, so each output
coordinate is a convex combination of that coordinate of the values in the
row's window and lies within their minimum and maximum ("27. Sliding-Window
Attention", Step-by-Step Approach: a softmax over the allowed keys, then the
weighted sum of their values).  The window extremes come from a sliding
minimum / maximum in O(T D) per head (prefix and suffix extremes inside
blocks of W rows), in torch on the GPU; no kernel of the library is involved
in them.  This catches any row, head or batch mapped to the wrong data, a
stale or unwritten row, and any NaN, on all B*H*T*D elements; the exact
values are checked on sampled rows against the oracle elsewhere.  q and k are
the workload's; v is a ramp along the sequence with a little noise, its sign
alternating over the (b, h) pairs, so that every row's window has its own
range and a row, tile or head read from the wrong place falls outside it.

Bar: min - tol <= out <= max + tol with tol = 2^-8 max(|min|, |max|): the
output is rounded once to bf16 (half an ulp is at most 2^-9 of it) after an
fp32 weighted average of the same values.
"""

import pytest
import torch

import sliding_window_causal_amd as swa
import swa_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda"


def window_extremes(v, W):
    """Per row i and column d, the minimum and maximum of v[j, d] over
    j in [max(0, i - W + 1), i], for v of shape [N, T, D] (float32)."""
    N, T, D = v.shape
    L = T + W - 1                                   # W - 1 rows of padding in front
    nb = (L + W - 1) // W
    out = []
    for fill, op in ((float("inf"), torch.cummin), (float("-inf"), torch.cummax)):
        x = torch.full((N, nb * W, D), fill, dtype=torch.float32, device=v.device)
        x[:, W - 1:W - 1 + T] = v
        xb = x.view(N, nb, W, D)
        pre = op(xb, dim=2).values.view(N, nb * W, D)
        suf = op(xb.flip(2), dim=2).values.flip(2).reshape(N, nb * W, D)
        # output row i covers padded rows [i, i + W - 1]: the suffix extreme
        # from i to its block's end and the prefix extreme up to i + W - 1
        a, b = suf[:, 0:T], pre[:, W - 1:W - 1 + T]
        out.append(torch.minimum(a, b) if fill > 0 else torch.maximum(a, b))
        del x, xb, pre, suf
    return out[0], out[1]


def test_window_extremes_helper_on_a_small_case():
    g = torch.Generator(device="cpu").manual_seed(5)
    v = torch.randn(2, 37, 3, generator=g).to(DEV)
    for W in (1, 4, 7, 37, 50):
        mn, mx = window_extremes(v, W)
        for i in range(37):
            lo = max(0, i - W + 1)
            assert torch.equal(mn[:, i], v[:, lo:i + 1].amin(1))
            assert torch.equal(mx[:, i], v[:, lo:i + 1].amax(1))


@pytest.mark.parametrize("name", ["prefill_bf16_b1_h32_t8192_d128_w4096",
                                  "prefill_bf16_b8_h32_t4096_d128_w1024",
                                  "prefill_bf16_b1_h32_t65536_d128_w4096"])
def test_full_size_prefill_every_element_within_its_window_range(name):
    w = si.WORKLOADS[name]
    q, k, _ = si.workload_qkv(w, DEV)
    ramp = torch.arange(w.T, dtype=torch.float32, device=DEV).view(1, 1, w.T, 1)
    sign = 1.0 - 2.0 * (torch.arange(w.B * w.H, device=DEV) % 2).float().view(w.B, w.H, 1, 1)
    noise = si.normal(tuple(q.shape), si.generator(w.seed + 21, DEV), torch.float32, DEV)
    v = (sign * (ramp + 0.25 * noise)).to(torch.bfloat16)
    del noise
    out = torch.empty_like(q)
    swa.swa_forward(q, k, v, out, w.W)
    torch.cuda.synchronize()
    W = min(w.W, w.T)
    for b in range(w.B):
        vf = v[b].float()
        mn, mx = window_extremes(vf, W)
        o = out[b].float()
        tol = torch.maximum(mn.abs(), mx.abs()) * 2.0 ** -8
        assert torch.isfinite(o).all(), f"{name} b={b}: non-finite output"
        low = (o < mn - tol).nonzero()
        high = (o > mx + tol).nonzero()
        assert low.numel() == 0, f"{name} b={b}: below the window minimum at {low[:4].tolist()}"
        assert high.numel() == 0, f"{name} b={b}: above the window maximum at {high[:4].tolist()}"
        del vf, mn, mx, o, tol
