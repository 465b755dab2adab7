"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws N(0, 1) tensors from
seeded generators and rounds them to the storage dtype, so that the HIP path
and the CPU oracle receive bit-identical values.  The pages run their examples
on i.i.d. standard-normal tensors (``torch.randn`` / ``np.random.randn``); the
workloads below keep that distribution at the shapes being measured.

Draw order within one workload is fixed: q, then k, then v (then the ring
contents stream by stream for decode).  Rounding to bf16 is round-to-nearest-
even (``Tensor.to``), and the oracle receives the rounded values.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                    # "prefill" or "decode"
    dtype: str                   # "f32" or "bf16"
    seed: int
    D: int
    W: int
    B: int = 1
    H: int = 1
    T: int = 0                   # prefill sequence length
    S: int = 0                   # decode: number of independent streams
    sweep: Tuple[int, ...] = field(default_factory=tuple)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    # fp32, small enough for the dense oracle; window sweep on the same tensors
    "prefill_f32_b1_h2_t128_d64_w32": Workload(
        "prefill_f32_b1_h2_t128_d64_w32", "prefill", "f32", 1001,
        B=1, H=2, T=128, D=64, W=32, sweep=(1, 3, 127, 128, 256)),
    # one Mistral-7B-shaped attention layer
    "prefill_bf16_b1_h32_t8192_d128_w4096": Workload(
        "prefill_bf16_b1_h32_t8192_d128_w4096", "prefill", "bf16", 1002,
        B=1, H=32, T=8192, D=128, W=4096),
    # batched, narrow band: most K/V tiles lie outside every band
    "prefill_bf16_b8_h32_t4096_d128_w1024": Workload(
        "prefill_bf16_b8_h32_t4096_d128_w1024", "prefill", "bf16", 1003,
        B=8, H=32, T=4096, D=128, W=1024),
    # long context: O(T*W) scaling against the T=8192 layer
    "prefill_bf16_b1_h32_t65536_d128_w4096": Workload(
        "prefill_bf16_b1_h32_t65536_d128_w4096", "prefill", "bf16", 1004,
        B=1, H=32, T=65536, D=128, W=4096),
    # streaming decode: 256 streams, one query each, full 4096-slot rings
    "decode_bf16_s256_h32_d128_w4096": Workload(
        "decode_bf16_s256_h32_d128_w4096", "decode", "bf16", 1005,
        S=256, H=32, D=128, W=4096),
}


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, g: torch.Generator, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """i.i.d. N(0, 1) drawn in fp32 from ``g``, then rounded to ``dtype``."""
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def prefill_qkv(B: int, H: int, T: int, D: int, dtype=torch.float32, seed: int = 0,
                device="cpu"):
    """q, k, v of shape [B, H, T, D], drawn in that order from one generator."""
    g = generator(seed, device)
    q = normal((B, H, T, D), g, dtype, device)
    k = normal((B, H, T, D), g, dtype, device)
    v = normal((B, H, T, D), g, dtype, device)
    return q, k, v


def workload_qkv(w: Workload, device="cpu"):
    assert w.kind == "prefill"
    return prefill_qkv(w.B, w.H, w.T, w.D, w.torch_dtype, w.seed, device)


def decode_positions(S: int, W: int, seed: int, full: bool = True) -> np.ndarray:
    """Absolute positions of the current query per stream.

    ``full``: every ring is full, pos = W + 1 + U[0, 2^20) (write head at a
    random offset); otherwise pos = U[0, W) (a partly filled ring).
    """
    rng = np.random.default_rng(int(seed))
    if full:
        return (W + 1 + rng.integers(0, 1 << 20, size=S)).astype(np.int64)
    return rng.integers(0, W, size=S).astype(np.int64)


def decode_inputs(S: int, H: int, D: int, W: int, dtype=torch.bfloat16, seed: int = 0,
                  device="cpu", full: bool = True):
    """q [S, H, D], kring/vring [S, H, W, D] and pos [S] (int64).

    The rings are filled stream by stream (k slab then v slab), so a device
    generator never needs the whole ring in fp32 at once.
    """
    g = generator(seed, device)
    q = normal((S, H, D), g, dtype, device)
    kring = torch.empty((S, H, W, D), dtype=dtype, device=device)
    vring = torch.empty((S, H, W, D), dtype=dtype, device=device)
    for s in range(S):
        kring[s].copy_(normal((H, W, D), g, dtype, device))
        vring[s].copy_(normal((H, W, D), g, dtype, device))
    pos = torch.from_numpy(decode_positions(S, W, seed, full)).to(device)
    return q, kring, vring, pos


def sample_rows(T: int, W: int, n_random: int, seed: int, tile: int = 64) -> np.ndarray:
    """Rows to check at full size: the window and tile edges plus random rows.

    Always includes 0, W-2, W-1, W, T-1 and the rows on either side of every
    ``tile``-aligned boundary near the start, the window edge and the end.
    """
    fixed = {0, 1, T - 1, T - 2}
    for r in (W - 2, W - 1, W, W + 1):
        if 0 <= r < T:
            fixed.add(r)
    for base in (tile, 2 * tile, W, T - tile):
        for r in (base - 1, base, base + 1):
            if 0 <= r < T:
                fixed.add(r)
    rng = np.random.default_rng(int(seed))
    rand = rng.integers(0, T, size=n_random)
    return np.array(sorted(fixed | {int(r) for r in rand}), dtype=np.int64)
