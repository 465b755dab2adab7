"""GPU parity of the multi-head module forward (swa_mha_forward: q, k, v and
output projections around the banded attention, the module of "NNX
Sliding-Window Attention") through the C ABI, against the fp64 oracle's
mha_forward on the same (rounded) inputs and weights.

Bars: the page's printed example exactly (fp32); fp32 max |gpu - oracle|
<= 1e-5 x the output scale; bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|; rows
outside a corrupted row's window bitwise unchanged.
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
BF_ATOL, BF_RTOL = 2e-2, 1e-2


def npy(t):
    return None if t is None else t.detach().float().cpu().numpy()


def _load_p5():
    lines = read_golden("p5_moving_average.txt")
    W = int(lines[0].split("=")[1])
    i_x, i_out, i_c = lines.index("x"), lines.index("out"), lines.index("corrupt_row0")
    x = np.array([[float(t) for t in ln.split()] for ln in lines[i_x + 1:i_out]])
    out = np.array([[float(t) for t in ln.split()] for ln in lines[i_out + 1:i_c]])
    corrupt = np.array([float(t) for t in lines[i_c + 1].split()])
    unchanged_from = int(lines[lines.index("unchanged_from_row") + 1])
    return W, x, out, corrupt, unchanged_from


def test_p5_printed_example_exact():
    W, x, expected, corrupt, unchanged_from = _load_p5()
    m = swa.SlidingWindowMHA(2, 2, dtype=torch.float32, device=DEV)
    m.wq.zero_()
    m.wk.zero_()
    m.wv.copy_(torch.eye(2))
    m.wo.copy_(torch.eye(2))
    xt = torch.tensor(x, dtype=torch.float32, device=DEV)
    out = m(xt, W)
    x2 = xt.clone()
    x2[0] = torch.tensor(corrupt, dtype=torch.float32, device=DEV)
    out2 = m(x2, W)
    torch.cuda.synchronize()
    assert np.array_equal(npy(out), expected)
    assert torch.equal(out2[unchanged_from:], out[unchanged_from:])
    assert not torch.equal(out2[:unchanged_from], out[:unchanged_from])


def _weights(dm, dtype, g, bias=True):
    w = [si.normal((dm, dm), g, torch.float32, DEV).mul_(dm ** -0.5).to(dtype) for _ in range(4)]
    b = [si.normal((dm,), g, dtype, DEV) if bias else None for _ in range(4)]
    return w, b


@pytest.mark.parametrize("B,T,dm,H,W", [(2, 300, 256, 2, 64), (1, 513, 512, 8, 100),
                                        (1, 200, 128, 1, 1000)])
def test_bf16_module_matches_oracle(B, T, dm, H, W):
    g = si.generator(110 + dm, DEV)
    x = si.normal((B, T, dm), g, torch.bfloat16, DEV)
    (wq, wk, wv, wo), (bq, bk, bv, bo) = _weights(dm, torch.bfloat16, g)
    out = torch.empty_like(x)
    swa.swa_mha_forward(x, wq, bq, wk, bk, wv, bv, wo, bo, out, H, W)
    torch.cuda.synchronize()
    ref = so.mha_forward(npy(x), npy(wq), npy(bq), npy(wk), npy(bk), npy(wv), npy(bv), npy(wo),
                         npy(bo), H, W)
    g64 = npy(out).astype(np.float64)
    assert np.all(np.isfinite(g64))
    err, bound = np.abs(g64 - ref), BF_ATOL + BF_RTOL * np.abs(ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}"


@pytest.mark.parametrize("bias", [True, False])
def test_fp32_module_matches_oracle(bias):
    B, T, dm, H, W = 2, 150, 48, 3, 20
    g = si.generator(120, DEV)
    x = si.normal((B, T, dm), g, torch.float32, DEV)
    (wq, wk, wv, wo), (bq, bk, bv, bo) = _weights(dm, torch.float32, g, bias)
    out = torch.empty_like(x)
    swa.swa_mha_forward(x, wq, bq, wk, bk, wv, bv, wo, bo, out, H, W)
    torch.cuda.synchronize()
    ref = so.mha_forward(npy(x), npy(wq), npy(bq), npy(wk), npy(bk), npy(wv), npy(bv), npy(wo),
                         npy(bo), H, W)
    err = np.abs(npy(out).astype(np.float64) - ref).max()
    # fp32 projections of width 48 carry ~1e-6 relative error into O(1) outputs
    assert err <= 1e-5 * max(1.0, np.abs(ref).max()), f"max err {err:.3e}"


def test_module_corruption_outside_window_is_bitwise_invisible():
    B, T, dm, H, W = 1, 260, 256, 2, 50
    g = si.generator(130, DEV)
    x = si.normal((B, T, dm), g, torch.bfloat16, DEV)
    (wq, wk, wv, wo), (bq, bk, bv, bo) = _weights(dm, torch.bfloat16, g)
    m = swa.SlidingWindowMHA(dm, H, device=DEV)
    m.wq, m.wk, m.wv, m.wo, m.bq, m.bk, m.bv, m.bo = wq, wk, wv, wo, bq, bk, bv, bo
    base = m(x, W)
    j0 = 100
    x2 = x.clone()
    x2[0, j0] = 50.0
    out = m(x2, W)
    torch.cuda.synchronize()
    assert torch.equal(out[0, :j0], base[0, :j0])
    assert torch.equal(out[0, j0 + W:], base[0, j0 + W:])
    assert not torch.equal(out[0, j0:j0 + W], base[0, j0:j0 + W])


def test_module_calls_from_two_threads_on_two_streams():
    """Two host threads run the module at the same time, each on a stream of
    its own (ctypes releases the GIL during the call): every result equals
    the same call made alone.  The library's rocBLAS handle carries a stream,
    so each call holds it from setting the stream to its last product."""
    import threading
    B, T, dm, H, W, N = 1, 1024, 1024, 8, 256, 20
    g = si.generator(130, DEV)
    xs = [si.normal((B, T, dm), g, torch.bfloat16, DEV) for _ in range(2)]
    (wq, wk, wv, wo), (bq, bk, bv, bo) = _weights(dm, torch.bfloat16, g)
    refs = []
    for x in xs:
        o = torch.empty_like(x)
        swa.swa_mha_forward(x, wq, bq, wk, bk, wv, bv, wo, bo, o, H, W)
        refs.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [[], []]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(N):
                    o = torch.empty_like(xs[i])
                    swa.swa_mha_forward(xs[i], wq, bq, wk, bk, wv, bv, wo, bo, o, H, W)
                    outs[i].append(o)
        except Exception as e:          # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(outs[i]) == N
        for n, o in enumerate(outs[i]):
            assert torch.equal(o, refs[i]), f"thread {i}, call {n}"



def test_full_size_module_sampled_rows():
    """The module of one 32-head layer (d_model 4096 = 32 x 128, T 8192,
    W 4096, inputs and weights drawn as the benchmark draws them, workspace
    allocated once): sampled output rows (window and tile edges, both ends,
    random rows) against the oracle's row-by-row module forward."""
    w = si.WORKLOADS["prefill_bf16_b1_h32_t8192_d128_w4096"]
    dm = w.H * w.D
    g = si.generator(w.seed + 7, DEV)
    x = si.normal((w.B, w.T, dm), g, torch.bfloat16, DEV)
    wts = [si.normal((dm, dm), g, torch.float32, DEV).mul_(dm ** -0.5).to(torch.bfloat16)
           for _ in range(4)]
    bss = [torch.zeros(dm, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    out = torch.empty_like(x)
    ws = torch.empty(swa.swa_mha_workspace_bytes(w.B, w.T, dm, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    swa.swa_mha_forward(x, wts[0], bss[0], wts[1], bss[1], wts[2], bss[2], wts[3], bss[3], out,
                        w.H, w.W, workspace=ws)
    torch.cuda.synchronize()
    rows = si.sample_rows(w.T, w.W, n_random=12, seed=w.seed + 7)
    ref = so.mha_rows(npy(x[0]), npy(wts[0]), npy(bss[0]), npy(wts[1]), npy(bss[1]),
                      npy(wts[2]), npy(bss[2]), npy(wts[3]), npy(bss[3]), w.H, w.W, rows)
    g64 = npy(out[0][torch.as_tensor(rows, device=DEV)]).astype(np.float64)
    assert np.all(np.isfinite(g64))
    err, bound = np.abs(g64 - ref), BF_ATOL + BF_RTOL * np.abs(ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"
