#!/usr/bin/env python3
"""Throughput of the causal sliding-window attention hot path on one GPU.

One step is one pass of the whole path over resident synthetic inputs:
  * prefill of one Mistral-7B-shaped attention layer, bf16 [1, 32, 8192, 128],
    window 4096 (swa_forward), and
  * one decode token for 256 independent streams, 32 heads, head size 128,
    against full 4096-slot bf16 rings (swa_decode).

    python bench.py [--gpus 1] [--steps 50] [--warmup 20]

Prints one JSON line.  ``value`` is the prefill's useful band TFLOP/s,
4 * B * H * D * sum_i min(i + 1, W) flops per launch; the decode's KV GB/s
(bytes of the valid slots' k and v plus q and out) is reported beside it.
Kernel times come from HIP events recorded on the stream the kernels are
launched on; ms_per_step is the wall time of the K timed steps between two
device synchronisations.  The two other prefill workloads (a batched
narrow band, B=8 T=4096 W=1024, and a long context, T=65536 W=4096) are
timed after the steps, each with its own roofline fraction.  The
``cpu_baseline`` leg times the fp64 CPU oracle's band-blocked tier on a
bounded sample of the T=8192 layer's query blocks, on all the host cores the
process may use (multithreaded BLAS for the matmuls).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("band attention TFLOP/s & % MFMA peak (prefill); KV GB/s & % HBM peak (decode)")
PREFILL = "prefill_bf16_b1_h32_t8192_d128_w4096"
DECODE = "decode_bf16_s256_h32_d128_w4096"
# the other prefill workloads, timed after the steps
PREFILL_MORE = {"prefill_narrow": "prefill_bf16_b8_h32_t4096_d128_w1024",
                "prefill_long": "prefill_bf16_b1_h32_t65536_d128_w4096"}
# MI355X: 256 compute units; dense bf16 matrix work per CU and clock
CUS = 256
BF16_FLOP_PER_CLK_CU = 4096
# MI355X published peaks: dense bf16 matrix throughput and HBM3E bandwidth.
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
PREFILL_SOURCES = ["sliding_window_causal_amd/csrc/swa_prefill_bf16.hip",
                   "sliding_window_causal_amd/csrc/swa_mfma.h",
                   "sliding_window_causal_amd/csrc/swa_internal.h"]
DECODE_SOURCES = ["sliding_window_causal_amd/csrc/swa_decode_bf16.hip",
                  "sliding_window_causal_amd/csrc/swa_internal.h"]


def band_pairs(T: int, W: int) -> int:
    """sum_{i<T} min(i + 1, W): (query, key) pairs inside the band."""
    if W >= T:
        return T * (T + 1) // 2
    return W * T - W * (W - 1) // 2


def prefill_flops(B, H, T, D, W) -> int:
    return 4 * B * H * D * band_pairs(T, W)


def decode_bytes(S, H, D, n, elem=2) -> int:
    """k and v of the n valid slots, plus q and out, per launch."""
    return 2 * S * H * n * D * elem + 2 * S * H * D * elem


def stats_ms(ms):
    """mean, median and min of a list of per-launch milliseconds."""
    xs = sorted(ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"kernel_ms_mean": sum(xs) / n, "kernel_ms_median": med, "kernel_ms_min": xs[0]}


def time_each(fn, stream, reps: int, warmup: int = 5):
    """Per-call milliseconds of reps back-to-back fn() calls, each bracketed
    by HIP events on the launching stream."""
    import torch
    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_launches(fn, stream, reps: int, warmup: int = 10) -> float:
    """Mean ms of one fn() call over reps back-to-back calls (HIP events on
    the launching stream)."""
    import torch
    for _ in range(warmup):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile_value(name: str, sha: str, key: str):
    """A figure from a committed PMC summary, if it was taken on this exact
    kernel source (else None)."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            k, val = ln.split(":", 1)
            kv[k.strip()] = val.strip()
    if kv.get("kernel_source_sha") != sha or key not in kv:
        return None
    return float(kv[key])


def read_traffic(name: str, sha: str):
    """HBM bytes per launch from a committed PMC summary, if it was taken on
    this exact kernel source (else None)."""
    return read_profile_value(name, sha, "hbm_bytes_per_launch")


def clock_fields(tflops: float, kernel_ms: float, name: str, sha: str):
    """The shader clock of this run and the dense bf16 peak at it.  A
    committed counter summary of the same kernel source gives the busy
    clock cycles per launch (GRBM_GUI_ACTIVE over the 8 XCDs); over this
    run's kernel time they give the clock it sustained, which under this
    load sits well below the 2.4 GHz the published peak assumes."""
    cyc = read_profile_value(name, sha, "busy_cycles_per_launch")
    if cyc is None:
        return {"clock_mhz": None, "peak_at_clock": None, "frac_at_clock": None}
    mhz = cyc / (kernel_ms * 1e-3) / 1e6
    peak = CUS * BF16_FLOP_PER_CLK_CU * mhz * 1e6 / 1e12
    return {"clock_mhz": mhz, "peak_at_clock": peak, "frac_at_clock": tflops / peak,
            "busy_cycles_per_launch": cyc}


def host_info():
    """Cores this process may run on, the BLAS library's thread count and the
    CPU model."""
    from threadpoolctl import threadpool_info
    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        cores = min(cores, int(env))
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [f"{d.get('internal_api')}:{d.get('num_threads')}" for d in threadpool_info()
            if d.get("user_api") == "blas"]
    return cores, model, blas


def cpu_baseline_prefill(q, k, v, W, seconds: float, block: int = 256):
    """Time the fp64 oracle's band-blocked tier on the prefill workload's
    query blocks, in random order, until all are done or about ``seconds``
    have passed; returns useful TFLOP/s (each block's band pairs)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import swa_oracle as so

    # exact fp64 copies of the inputs, staged before the timed region
    qh, kh, vh = (x[0].double().cpu().numpy() for x in (q, k, v))
    H, T, D = qh.shape
    cores, model, _ = host_info()
    rng = np.random.default_rng(0)
    starts = rng.permutation(np.arange(0, T, block))
    flops = 0
    done = 0
    with threadpool_limits(limits=cores, user_api="blas"):
        _, _, blas = host_info()
        t0 = time.perf_counter()
        for i0 in starts:
            i1 = min(T, int(i0) + block)
            so.swa_blocked(qh, kh, vh, W, block=block, start=int(i0), stop=i1)
            flops += 4 * H * D * (band_pairs(i1, W) - band_pairs(int(i0), W))
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"the whole {PREFILL} layer" if done == len(starts) else
                   f"{done} of the {len(starts)} blocks of {block} queries (all {H} heads, "
                   f"random order) of the {PREFILL} layer") +
                  f", fp64 band-blocked oracle tier, {dt:.1f} s",
        "blas_threads": blas,
        "cpu_model": model,
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The GPU's clocks ramp up over the first ~50 ms of sustained matrix work;
    # 20 steps (~70 ms) reach the plateau before timing starts.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward", "copy"], default="all",
                    help="profiling aid: run one kernel only (the JSON line is then partial)")
    ap.add_argument("--workload", default=PREFILL,
                    help="prefill workload for --only prefill (the default step always uses the "
                         "T=8192/W=4096 layer)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-more-prefill", action="store_true",
                    help="skip the narrow-band and long-context prefill lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the path shards by heads, batch or streams with no communication, and bench.py "
              "times one GPU's share; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import sliding_window_causal_amd as swa
    import swa_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only == "copy":
        # Plain copy of a known size, the reference for PMC byte counters.
        n = 1 << 28                              # 256 Mi floats = 1 GiB read + 1 GiB written
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                          "launches": args.warmup + args.steps}))
        return 0

    if args.workload != PREFILL and args.only != "prefill":
        print("--workload applies to --only prefill", file=sys.stderr)
        return 2
    wp = si.WORKLOADS[args.workload]
    wd = si.WORKLOADS[DECODE]
    do_p = args.only in ("all", "prefill")
    do_d = args.only in ("all", "decode")
    do_b = args.only in ("all", "backward")
    print(f"# device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}",
          file=sys.stderr, flush=True)
    if do_p or do_b:
        q, k, v = si.workload_qkv(wp, dev)
        out = torch.empty_like(q)
    if do_d:
        qd, kr, vr, pos = si.decode_inputs(wd.S, wd.H, wd.D, wd.W, torch.bfloat16, wd.seed, dev)
        od = torch.empty_like(qd)
        n_valid = min(int(pos.min().item()) + 1, wd.W)
        assert n_valid == wd.W
    torch.cuda.synchronize()
    print("# inputs resident", file=sys.stderr, flush=True)

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if do_p:
            swa.swa_forward(q, k, v, out, wp.W, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        if do_d:
            swa.swa_decode(qd, kr, vr, pos, od, stream=stream)
        if evs is not None:
            evs[2].record(stream)

    n_steps = 0 if args.only == "backward" else args.steps
    for _ in range(args.warmup if n_steps else 0):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_steps)]
    t0 = time.perf_counter()
    for i in range(n_steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = [e[0].elapsed_time(e[1]) for e in evs]
    d_ms = [e[1].elapsed_time(e[2]) for e in evs]
    print("# timed steps done", file=sys.stderr, flush=True)

    res = {
        "metric": METRIC,
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / n_steps * 1e3 if n_steps else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{PREFILL} + {DECODE}" if args.only == "all" else
                   (wp.name if do_p or do_b else DECODE)},
    }
    if do_p:
        flops = prefill_flops(wp.B, wp.H, wp.T, wp.D, wp.W)
        pst = stats_ms(p_ms)
        pm = pst["kernel_ms_mean"]
        tflops = flops / (pm * 1e-3) / 1e12
        sha = source_sha(PREFILL_SOURCES)
        res["value"] = tflops
        res["config"]["prefill"] = {"B": wp.B, "H": wp.H, "T": wp.T, "D": wp.D, "W": wp.W,
                                    "useful_flop_per_launch": flops, **pst,
                                    "TFLOPs_median": flops / (pst["kernel_ms_median"] * 1e-3) / 1e12}
        if do_d:
            # context: in the step each prefill follows a decode that streams
            # 16 GiB through the caches; launched back to back it starts warm
            pb = time_launches(lambda: swa.swa_forward(q, k, v, out, wp.W, stream=stream),
                               stream, 20, 5)
            res["config"]["prefill"]["kernel_ms_back_to_back"] = pb
            res["config"]["prefill"]["TFLOPs_back_to_back"] = flops / (pb * 1e-3) / 1e12
            # context: what the vendor library's bf16 GEMM (torch.mm ->
            # hipBLASLt) reaches on this device, 8192^3, fp32 accumulate
            gg = si.generator(wp.seed + 13, dev)
            ga = si.normal((8192, 8192), gg, torch.bfloat16, dev)
            gb = si.normal((8192, 8192), gg, torch.bfloat16, dev)
            tg = time_launches(lambda: torch.mm(ga, gb), stream, 20, 30)
            vendor_ref = {"TFLOPs": 2 * 8192 ** 3 / (tg * 1e-3) / 1e12,
                          "how": "torch.mm bf16 8192 x 8192 x 8192 on this device, 30 warm-up "
                                 "launches then 20 timed"}
            del ga, gb
        res["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                           "traffic": read_traffic("prefill_bf16_t8192_w4096_traffic.txt", sha),
                           "kernel": "prefill_bf16_kernel<128,4>", "kernel_source_sha": sha,
                           **clock_fields(tflops, pm, "prefill_bf16_t8192_w4096_counters.txt", sha)}
        if do_d:
            res["roofline"]["vendor_gemm_reference"] = vendor_ref
    if do_d:
        nbytes = decode_bytes(wd.S, wd.H, wd.D, wd.W)
        dst = stats_ms(d_ms)
        dm = dst["kernel_ms_mean"]
        gbs = nbytes / (dm * 1e-3) / 1e9
        sha = source_sha(DECODE_SOURCES)
        res["decode"] = {
            "value": gbs, "unit": "GB/s", **dst,
            "GBs_median": nbytes / (dst["kernel_ms_median"] * 1e-3) / 1e9,
            "S": wd.S, "H": wd.H, "D": wd.D, "W": wd.W, "bytes_per_launch": nbytes,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": read_traffic("decode_bf16_s256_w4096_traffic.txt", sha),
                         "kernel": "decode_bf16_kernel<bf16,128,rows>", "kernel_source_sha": sha},
        }
        if not do_p:
            res["value"], res["unit"] = gbs, "GB/s"
        # Latency of one decode token for a single stream (32 heads, full
        # 4096-slot rings): one workgroup per head, the window split over
        # workgroups, and the fused append + split decode.
        q1, kr1, vr1, pos1 = si.decode_inputs(1, wd.H, wd.D, wd.W, torch.bfloat16, wd.seed, dev)
        o1 = torch.empty_like(q1)
        kn1, vn1 = q1.clone(), q1.clone()
        nws = swa.swa_decode_workspace_bytes(1, wd.H, wd.D, wd.W, torch.bfloat16)
        ws1 = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        b1 = decode_bytes(1, wd.H, wd.D, wd.W)
        t_plain = time_launches(lambda: swa.swa_decode(q1, kr1, vr1, pos1, o1, stream=stream),
                                stream, 100)
        t_split = time_launches(lambda: swa.swa_decode_split(q1, kr1, vr1, pos1, o1, ws1,
                                                             stream=stream), stream, 100)
        t_fused = time_launches(lambda: swa.swa_decode_append(q1, kn1, vn1, kr1, vr1, pos1, o1,
                                                              ws1, stream=stream), stream, 100)
        res["decode"]["single_stream"] = {
            "S": 1, "H": wd.H, "D": wd.D, "W": wd.W, "workspace_bytes": nws,
            "us_one_wg_per_head": t_plain * 1e3, "us_split": t_split * 1e3,
            "us_fused_append_split": t_fused * 1e3,
            "GBs_split": b1 / (t_split * 1e-3) / 1e9}
    if do_p and args.only == "all":
        # Chunked prefill continuing full 4096-slot rings (the streaming
        # path): 2048 new tokens of one stream, and 512 of four, 32 heads,
        # D = 128; every query sees W keys.
        res["chunk"] = []
        for S, Cn in ((1, 2048), (4, 512), (1, 128)):
            gc = si.generator(wp.seed, dev)
            qc, kc, vc = (si.normal((S, wp.H, Cn, wp.D), gc, torch.bfloat16, dev) for _ in range(3))
            krc = si.normal((S, wp.H, wp.W, wp.D), gc, torch.bfloat16, dev)
            vrc = si.normal((S, wp.H, wp.W, wp.D), gc, torch.bfloat16, dev)
            p0c = torch.full((S,), 5 * wp.W + 123, dtype=torch.int64, device=dev)
            oc = torch.empty_like(qc)
            tc = time_launches(lambda: swa.swa_chunk_forward(qc, kc, vc, krc, vrc, p0c, oc,
                                                             stream=stream), stream, 50, 20)
            nws = swa.swa_chunk_workspace_bytes(S, wp.H, Cn, wp.D, wp.W, torch.bfloat16)
            wsc = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
            ts = time_launches(lambda: swa.swa_chunk_forward_split(
                qc, kc, vc, krc, vrc, p0c, oc, wsc, stream=stream), stream, 50, 20)
            fl = 4 * S * wp.H * wp.D * Cn * wp.W
            res["chunk"].append({"S": S, "C": Cn, "H": wp.H, "D": wp.D, "W": wp.W,
                                 "kernel_ms_mean": tc, "useful_flop_per_launch": fl,
                                 "TFLOPs": fl / (tc * 1e-3) / 1e12,
                                 "split_workspace_bytes": nws, "split_ms_mean": ts,
                                 "split_TFLOPs": fl / (ts * 1e-3) / 1e12})
            del qc, kc, vc, krc, vrc, oc, wsc
    if do_p and args.only == "all":
        # The whole attention module of one such layer (d_model 4096 = 32
        # heads x 128): q, k, v, output projections (rocBLAS) around the band.
        dm = wp.H * wp.D
        gm = si.generator(wp.seed + 7, dev)
        xm = si.normal((wp.B, wp.T, dm), gm, torch.bfloat16, dev)
        wts = [si.normal((dm, dm), gm, torch.float32, dev).mul_(dm ** -0.5).to(torch.bfloat16)
               for _ in range(4)]
        bss = [torch.zeros(dm, dtype=torch.bfloat16, device=dev) for _ in range(4)]
        om = torch.empty_like(xm)
        wsm = torch.empty(swa.swa_mha_workspace_bytes(wp.B, wp.T, dm, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        tm = time_launches(lambda: swa.swa_mha_forward(
            xm, wts[0], bss[0], wts[1], bss[1], wts[2], bss[2], wts[3], bss[3], om, wp.H, wp.W,
            workspace=wsm, stream=stream), stream, 20, 5)
        proj = 4 * 2 * wp.B * wp.T * dm * dm
        att = prefill_flops(wp.B, wp.H, wp.T, wp.D, wp.W)
        res["module"] = {"B": wp.B, "T": wp.T, "d_model": dm, "H": wp.H, "W": wp.W,
                         "ms_mean": tm, "projection_flop": proj, "attention_flop": att,
                         "TFLOPs": (proj + att) / (tm * 1e-3) / 1e12}
        del xm, wts, om, wsm
    if do_b:
        # Backward of the same layer: dq, dk, dv given dout (includes the
        # forward rerun that rebuilds the per-row softmax normalisers).
        gb = si.generator(wp.seed + 11, dev)
        dob = si.normal(tuple(q.shape), gb, torch.bfloat16, dev)
        gq, gk, gv = (torch.empty_like(q) for _ in range(3))
        wsb = torch.empty(int(swa.lib().swa_backward_workspace_bytes(wp.B, wp.H, wp.T)),
                          dtype=torch.uint8, device=dev)
        # 30 warm-up launches: run alone (--only backward) the clocks start cold
        tb = time_launches(lambda: swa.swa_backward(q, k, v, out, dob, gq, gk, gv, wp.W,
                                                    workspace=wsb, stream=stream), stream, 10, 30)
        # training order: the forward keeps its row log-sum-exp for the backward
        lse = torch.empty((wp.B, wp.H, wp.T), dtype=torch.float32, device=dev)
        swa.swa_forward_lse(q, k, v, out, lse, wp.W, stream=stream)
        tl = time_launches(lambda: swa.swa_backward(q, k, v, out, dob, gq, gk, gv, wp.W, lse=lse,
                                                    workspace=wsb, stream=stream), stream, 10, 3)
        bf = 10 * wp.B * wp.H * wp.D * band_pairs(wp.T, wp.W)
        res["backward"] = {"ms_mean": tb, "ms_mean_given_lse": tl, "band_product_flop": bf,
                           "TFLOPs": bf / (tb * 1e-3) / 1e12,
                           "TFLOPs_given_lse": bf / (tl * 1e-3) / 1e12,
                           "note": "five band products (S, dP, dV, dK, dQ) counted; the "
                                   "forward rerun (absent given lse) and the recomputed S "
                                   "products are not"}
        if not do_p:
            res["value"] = res["backward"]["TFLOPs_given_lse"]
        del dob, gq, gk, gv, wsb, lse
    if do_p and args.only == "all" and not args.no_more_prefill:
        # The other prefill workloads, each timed launch by launch (HIP events
        # on the stream) after 5 warm-up launches.
        sha = source_sha(PREFILL_SOURCES)
        for key, name in PREFILL_MORE.items():
            w = si.WORKLOADS[name]
            qm, km, vm = si.workload_qkv(w, dev)
            om = torch.empty_like(qm)
            ms = time_each(lambda: swa.swa_forward(qm, km, vm, om, w.W, stream=stream), stream,
                           20, 5)
            st = stats_ms(ms)
            fl = prefill_flops(w.B, w.H, w.T, w.D, w.W)
            tf = fl / (st["kernel_ms_mean"] * 1e-3) / 1e12
            res[key] = {"workload": name, "B": w.B, "H": w.H, "T": w.T, "D": w.D, "W": w.W,
                        "useful_flop_per_launch": fl, **st, "TFLOPs": tf,
                        "TFLOPs_median": fl / (st["kernel_ms_median"] * 1e-3) / 1e12,
                        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                                     "traffic": read_traffic(f"{name}_traffic.txt", sha),
                                     "kernel": "prefill_bf16_kernel<128,4>",
                                     "kernel_source_sha": sha,
                                     **clock_fields(tf, st["kernel_ms_mean"], f"{name}_counters.txt",
                                                    sha)}}
            del qm, km, vm, om
        print("# more prefill workloads done", file=sys.stderr, flush=True)
    if do_p and args.only == "all" and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(q, k, v, wp.W, args.cpu_seconds)
    res["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "compute_units": props.multi_processor_count,
                     "torch": torch.__version__, "hip": torch.version.hip}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
