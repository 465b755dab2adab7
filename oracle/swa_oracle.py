"""Plain fp64 CPU definition of causal sliding-window attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It
shares no code with the HIP library and never imports it.

Sources (the five pages on the subject; cited by title and section):
  [P1] "27. Sliding-Window Attention" (ai-labs PyTorch problem set)
  [P2] "25. Sliding-Window Causal Attention for Streaming Inference"
       (cartesia PyTorch problem set)
  [P3] "Implementation: Sliding Window Attention" (Mistral Architecture
       chapter of the Language AI Handbook)
  [P4] "Sliding Window Attention" (bembew.net article)
  [P5] "NNX Sliding-Window Attention" (crackedaicode exercise)

What is computed.  Attention is the ordinary scaled dot-product attention
softmax(q k^T / sqrt(D)) v with a band mask applied before the softmax
[P1 Step-by-Step Approach, steps 1-5; P2 steps 1-5; P3 Step 2; P5 "Mask before
softmax"].

Window convention.  W counts keys *including the query itself*: key j is
visible to query i iff j <= i and i - j < W [P1 step 2; P2 step 3 and its note
that the lower bound is strict; P3 Step 1, the blocking rule and the printed
8-token mask; P5 "Build the band by index difference" and its printed 5-token
mask].  P4 ("Mathematical Formulation and Attention Masking") states
max(0, i - W) <= j <= i, which admits W + 1 keys once i >= W; P5 names exactly
that form as including one key too many.  The oracle takes the four-page
reading; ``band_mask_max_form`` keeps P4's form only so that the tests can show
that it is the off-by-one.

Masking is a *select* to -inf (P1 ``masked_fill``, P5 ``where``), not P3's
additive 0/-inf matrix: the two agree for finite scores, and the select form
stays defined when an out-of-window score is itself infinite.

Precision.  Inputs are upcast exactly to float64 (fp32 and bf16 values are
exactly representable), and everything is computed in float64.

Pins: every function here is checked in ``tests/test_oracle.py`` against the
masks the pages print, P5's worked example, W >= T reducing to a library
causal-attention routine, W = 1 returning v, the trailing moving average for
zero Q/K, out-of-window corruption invariance, and brute force on tiny inputs.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# Window predicate
# ----------------------------------------------------------------------------

def _check_window(W) -> int:
    """Positive integer window.  [P5 "Mask before softmax": a positive W keeps
    the diagonal, so no row is entirely masked; a fully masked row is outside
    the contract.]  W < 1 is rejected rather than producing NaN rows."""
    if isinstance(W, bool) or not isinstance(W, (int, np.integer)):
        raise TypeError(f"window size must be an integer, got {type(W).__name__}")
    W = int(W)
    if W < 1:
        raise ValueError(f"window size must be >= 1, got {W}")
    return W


def band_mask(T: int, W: int, rows=None, keys=None) -> np.ndarray:
    """Boolean (T, T) band: ``[i, j]`` is True iff key j is visible to query i.

    [P1 step 2: keep (j <= i) & ((i - j) < window_size).  P5 "Build the band by
    index difference": diff = i - j, keep (diff >= 0) & (diff < W).]
    With ``rows`` and ``keys`` (index sequences) only that (rows, keys) block
    of it.
    """
    W = _check_window(W)
    i = (np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = (np.arange(T) if keys is None else np.asarray(keys, dtype=np.int64))[None, :]
    diff = i - j
    return (diff >= 0) & (diff < W)


def band_mask_max_form(T: int, W: int) -> np.ndarray:
    """P4's printed visibility rule, max(0, i - W) <= j <= i.

    [P4 "Mathematical Formulation and Attention Masking".]  Kept only so that
    tests can show it equals ``band_mask(T, W + 1)`` (one extra key, as P5's
    "Build the band by index difference" warns) and differs from both printed
    masks.  Not used by any attention function here.
    """
    W = _check_window(W)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j >= np.maximum(0, i - W)) & (j <= i)


# ----------------------------------------------------------------------------
# Prefill: four independent tiers of the same definition
# ----------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _scores(qk, D: int, scale):
    """Raw dot products to scores: divided by sqrt(D) [P1 step 1; P2 step 1;
    P5 code], or multiplied by an explicit ``scale`` [P3 Step 2, whose
    ``scale`` argument defaults to 1 / sqrt(head_dim)]."""
    if scale is None:
        return qk / math.sqrt(D)
    scale = float(scale)
    if not math.isfinite(scale):
        raise ValueError("scale must be finite")
    return qk * scale


def swa_dense(q, k, v, W: int, return_weights: bool = False, scale=None):
    """The pages' dense recipe in float64.

    q, k: (..., T, D); v: (..., T, Dv); any leading dims (P1 and P4 use
    (B, H, T, D), P2 uses (B, T, D), P5 uses (H, T, Dh)).

    1. scores = q @ k^T / sqrt(D)          [P1 step 1; P2 step 1; P5 code]
       (or q @ k^T * scale                 [P3 Step 2])
    2. band mask, select -inf outside it   [P1 steps 2-3; P5 "Mask before softmax"]
    3. stable softmax over keys            [P3 Step 2: subtract the row max,
                                            exponentiate, divide by the sum]
    4. weights @ v                         [P1 step 5]

    Returns (..., T, Dv) float64, and the (..., T, T) weights when asked
    (P3's function returns both).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, D = q.shape[-2], q.shape[-1]
    if k.shape[-2] != T or v.shape[-2] != T or k.shape[-1] != D:
        raise ValueError("q, k, v must share T, and q, k must share D")
    scores = _scores(np.matmul(q, np.swapaxes(k, -1, -2)), D, scale)
    mask = band_mask(T, W)
    scores = np.where(mask, scores, -np.inf)
    row_max = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - row_max)
    weights = e / e.sum(axis=-1, keepdims=True)
    out = np.matmul(weights, v)
    if return_weights:
        return out, weights
    return out


def swa_rows(q, k, v, W: int, rows: Iterable[int], scale=None):
    """Output rows ``rows`` computed one by one from the definition.

    For query i the visible keys are j in [max(0, i - W + 1), i] (the same set
    as ``band_mask``: j <= i and i - j < W, P1 step 2, P5 "Build the band by
    index difference").  Over that set: s_j = q_i . k_j / sqrt(D) (or times
    ``scale``, P3 Step 2), then a stable softmax and the weighted sum of v_j
    (P3 Step 2).  Only the band is
    touched, so this works at full size for a sample of rows.

    q, k: (..., T, D); v: (..., T, Dv) (float arrays of any float dtype).
    Returns (..., len(rows), Dv) float64.
    """
    W = _check_window(W)
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    T, D = q.shape[-2], q.shape[-1]
    Dv = v.shape[-1]
    lead = q.shape[:-2]
    Q = q.reshape(-1, T, D)
    K = k.reshape(-1, T, D)
    V = v.reshape(-1, T, Dv)
    rows = [int(r) for r in rows]
    out = np.empty((Q.shape[0], len(rows), Dv), dtype=np.float64)
    for r, i in enumerate(rows):
        if not 0 <= i < T:
            raise IndexError(f"row {i} outside [0, {T})")
        lo = max(0, i - W + 1)
        kk = _f64(K[:, lo:i + 1, :])                           # (N, n, D)
        vv = _f64(V[:, lo:i + 1, :])                           # (N, n, Dv)
        qi = _f64(Q[:, i, :])                                  # (N, D)
        s = _scores(np.matmul(kk, qi[:, :, None])[:, :, 0], D, scale)   # (N, n)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        w = e / e.sum(axis=1, keepdims=True)
        out[:, r, :] = np.matmul(w[:, None, :], vv)[:, 0, :]
    return out.reshape(lead + (len(rows), Dv))


def swa_blocked(q, k, v, W: int, block: int = 256, scale=None, start: int = 0, stop=None):
    """The dense recipe of ``swa_dense``, a block of queries at a time.

    Queries [i0, i1) can only see keys [max(0, i0 - W + 1), i1) (the band of
    ``band_mask``: j <= i and i - j < W), so each block takes that slab of
    keys only: scores by matmul, the band mask by select, the stable softmax
    and the weighted sum of v [P1 steps 1-5; P3 Step 2; P5 "Mask before
    softmax"].  Keys outside the slab are masked for every query of the
    block, and masked entries add exact zeros, so this is ``swa_dense`` up to
    summation order, with memory O(block * (W + block)) instead of O(T^2)
    (P5 "A local mask is not a sparse implementation" names that gap).

    q, k: (..., T, D); v: (..., T, Dv) (any float dtype, upcast exactly).
    Returns the rows [start, stop) (default: all), (..., stop - start, Dv)
    float64.
    """
    W = _check_window(W)
    if block < 1:
        raise ValueError("block must be >= 1")
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    T, D = q.shape[-2], q.shape[-1]
    if k.shape[-2] != T or v.shape[-2] != T or k.shape[-1] != D:
        raise ValueError("q, k, v must share T, and q, k must share D")
    stop = T if stop is None else int(stop)
    start = int(start)
    if not 0 <= start <= stop <= T:
        raise IndexError(f"rows [{start}, {stop}) outside [0, {T}]")
    out = np.empty(q.shape[:-2] + (stop - start, v.shape[-1]), dtype=np.float64)
    for i0 in range(start, stop, block):
        i1 = min(stop, i0 + block)
        lo = max(0, i0 - W + 1)
        qb = _f64(q[..., i0:i1, :])
        kb = _f64(k[..., lo:i1, :])
        vb = _f64(v[..., lo:i1, :])
        scores = _scores(np.matmul(qb, np.swapaxes(kb, -1, -2)), D, scale)
        mask = band_mask(T, W, rows=range(i0, i1), keys=range(lo, i1))
        scores = np.where(mask, scores, -np.inf)
        row_max = scores.max(axis=-1, keepdims=True)
        e = np.exp(scores - row_max)
        out[..., i0 - start:i1 - start, :] = np.matmul(e / e.sum(axis=-1, keepdims=True), vb)
    return out


def swa_loop(q, k, v, W: int):
    """Pure-Python triple loop (tiny inputs only, T * W * D small).

    Same definition as ``swa_dense``, written with scalar arithmetic so that no
    library routine is involved.  q, k: (..., T, D); v: (..., T, Dv).
    """
    W = _check_window(W)
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    T, D = q.shape[-2], q.shape[-1]
    Dv = v.shape[-1]
    lead = q.shape[:-2]
    Q = q.reshape(-1, T, D)
    K = k.reshape(-1, T, D)
    V = v.reshape(-1, T, Dv)
    out = np.zeros((Q.shape[0], T, Dv), dtype=np.float64)
    root_d = math.sqrt(D)
    for n in range(Q.shape[0]):
        for i in range(T):
            keys = [j for j in range(T) if j <= i and i - j < W]
            s = []
            for j in keys:
                acc = 0.0
                for d in range(D):
                    acc += float(Q[n, i, d]) * float(K[n, j, d])
                s.append(acc / root_d)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            total = sum(e)
            for d in range(Dv):
                acc = 0.0
                for j, ej in zip(keys, e):
                    acc += (ej / total) * float(V[n, j, d])
                out[n, i, d] = acc
    return out.reshape(lead + (T, Dv))


# ----------------------------------------------------------------------------
# Row log-sum-exp and the backward (the chain rule through the definition)
# ----------------------------------------------------------------------------

def swa_lse(q, k, W: int, scale=None):
    """Each row's log-sum-exp of its scaled in-band scores, ln(sum_j exp(s_ij))
    over j in the band of i, in float64: the normaliser of the stable
    softmax of P3 Step 2 (weights = exp(s - lse)).  q, k: (..., T, D);
    returns (..., T)."""
    q, k = _f64(q), _f64(k)
    T, D = q.shape[-2], q.shape[-1]
    s = _scores(np.matmul(q, np.swapaxes(k, -1, -2)), D, scale)
    s = np.where(band_mask(T, W), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True)))[..., 0]


def swa_backward(q, k, v, W: int, dout, scale=None):
    """Gradients of the band attention output with respect to q, k and v,
    in float64, by the chain rule through the dense recipe of ``swa_dense``
    (the pages define the forward only; gradients are named by P5, "Mask
    before softmax": masked weights are zero and gradients stay defined for
    finite allowed scores).

    With S = q k^T * scale (scale = 1/sqrt(D) by default), P = softmax of S
    over the band (0 outside it) and out = P v:
      dV = P^T dout
      dP = dout v^T
      dS = P * (dP - rowsum(P * dP))        (softmax Jacobian, per row)
      dQ = dS k * scale,  dK = dS^T q * scale
    Entries outside the band have P = 0 and hence dS = 0.

    q, k: (..., T, D); v, dout: (..., T, Dv).  Returns (dq, dk, dv) float64.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    T, D = q.shape[-2], q.shape[-1]
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _, P = swa_dense(q, k, v, W, return_weights=True, scale=scale)
    tr = lambda a: np.swapaxes(a, -1, -2)
    dv = np.matmul(tr(P), dout)
    dP = np.matmul(dout, tr(v))
    dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
    dq = np.matmul(dS, k) * sc
    dk = np.matmul(tr(dS), q) * sc
    return dq, dk, dv


def _band_weights_and_ds(q, k, v, dout, rows, keys_lo: int, keys_hi: int, W: int, sc: float):
    """For query rows ``rows`` (consecutive, ascending) of one head: the softmax
    weights P over keys [keys_lo, keys_hi) (zero outside each row's band) and
    dS = P * (dP - rowsum(P * dP)) with dP = dout v^T, as in ``swa_backward``.
    Every row's band must lie inside [keys_lo, keys_hi)."""
    i = np.asarray(rows)[:, None]
    j = np.arange(keys_lo, keys_hi)[None, :]
    band = (j <= i) & (i - j < W)                           # P1 step 2, P5 band rule
    s = np.matmul(q[rows], k[keys_lo:keys_hi].T) * sc
    s = np.where(band, s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    P = e / e.sum(axis=1, keepdims=True)                    # P3 Step 2
    dP = np.matmul(dout[rows], v[keys_lo:keys_hi].T)
    return P, P * (dP - np.sum(P * dP, axis=1, keepdims=True))


def swa_backward_rows(q, k, v, W: int, dout, q_rows: Iterable[int], k_rows: Iterable[int],
                      scale=None):
    """``swa_backward`` restricted to sampled rows, from the band alone, so that
    it runs at full size: dq for query rows ``q_rows``, dk and dv for key rows
    ``k_rows``.  Same formulas as ``swa_backward``:
      dq_i = scale * sum over j in band(i) of dS_ij k_j,  band(i) = [i-W+1, i]
      dk_j = scale * sum over i in rows(j) of dS_ij q_i,  rows(j) = [j, j+W-1]
      dv_j =         sum over i in rows(j) of P_ij dout_i
    where row i's P and dS need all of band(i), so a key row reads the keys
    [j-W+1, j+W-1].

    q, k: (T, D); v, dout: (T, Dv), one head.  Returns (dq (len(q_rows), D),
    dk (len(k_rows), D), dv (len(k_rows), Dv)) float64.
    """
    W = _check_window(W)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    T, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    q_rows, k_rows = [int(r) for r in q_rows], [int(r) for r in k_rows]
    for r in q_rows + k_rows:
        if not 0 <= r < T:
            raise IndexError(f"row {r} outside [0, {T})")
    dq = np.empty((len(q_rows), D))
    for n, i in enumerate(q_rows):
        lo = max(0, i - W + 1)
        _, dS = _band_weights_and_ds(q, k, v, dout, [i], lo, i + 1, W, sc)
        dq[n] = np.matmul(dS, k[lo:i + 1])[0] * sc
    dk = np.empty((len(k_rows), D))
    dv = np.empty((len(k_rows), v.shape[1]))
    for n, j in enumerate(k_rows):
        rows = np.arange(j, min(T, j + W))
        P, dS = _band_weights_and_ds(q, k, v, dout, rows, max(0, j - W + 1), min(T, j + W), W, sc)
        col = j - max(0, j - W + 1)
        dk[n] = np.matmul(dS[:, col], q[rows]) * sc
        dv[n] = np.matmul(P[:, col], dout[rows])
    return dq, dk, dv


# ----------------------------------------------------------------------------
# The multi-head module forward (projections around the attention)
# ----------------------------------------------------------------------------

def mha_forward(x, wq, bq, wk, bk, wv, bv, wo, bo, H: int, W: int):
    """Multi-head sliding-window self-attention module forward in float64
    [P5 "A complete example with moving averages", the module's __call__].

    x: (..., T, d_model); w*: (d_model, d_model) kernels applied as x @ w
    (input features by output features); b*: (d_model,) biases or None (zero).
    1. q, k, v = x @ wq + bq, x @ wk + bk, x @ wv + bv
    2. split the feature axis into H heads of width d_model / H
    3. per head: swa_dense (scores / sqrt(head width), band, softmax, @ v)
    4. heads concatenated back along the feature axis, then @ wo + bo
    Returns (..., T, d_model) float64.
    """
    x = _f64(x)
    T, dm = x.shape[-2], x.shape[-1]
    H = int(H)
    if H < 1 or dm % H != 0:
        raise ValueError("d_model must be a positive multiple of the head count")
    dh = dm // H

    def proj(a, w, b):
        y = np.matmul(a, _f64(w))
        return y if b is None else y + _f64(b)

    def heads(y):                                     # (..., T, dm) -> (..., H, T, dh)
        return np.swapaxes(y.reshape(y.shape[:-1] + (H, dh)), -2, -3)

    q, k, v = (heads(proj(x, w, b)) for w, b in ((wq, bq), (wk, bk), (wv, bv)))
    o = swa_dense(q, k, v, W)                         # (..., H, T, dh)
    concat = np.swapaxes(o, -2, -3).reshape(x.shape[:-1] + (dm,))
    return proj(concat, wo, bo)


def mha_rows(x, wq, bq, wk, bk, wv, bv, wo, bo, H: int, W: int, rows: Iterable[int]):
    """Rows ``rows`` of ``mha_forward`` for one sequence, without the T x T
    scores, so that it runs at full size: the same steps 1-4, with step 3 done
    by ``swa_rows`` over each row's band, and the query projection taken only
    for the sampled rows.

    x: (T, d_model); weights and biases as in ``mha_forward``.
    Returns (len(rows), d_model) float64.
    """
    x = _f64(x)
    T, dm = x.shape
    H = int(H)
    if H < 1 or dm % H != 0:
        raise ValueError("d_model must be a positive multiple of the head count")
    dh = dm // H
    rows = [int(r) for r in rows]

    def proj(a, w, b):
        y = np.matmul(a, _f64(w))
        return y if b is None else y + _f64(b)

    k, v = proj(x, wk, bk), proj(x, wv, bv)           # (T, dm): every row may be a key
    o = np.empty((len(rows), dm))
    for h in range(H):
        cols = slice(h * dh, (h + 1) * dh)
        qh = np.zeros((T, dh))
        qh[rows] = proj(x[rows], wq, bq)[:, cols]       # only sampled rows act as queries
        o[:, cols] = swa_rows(qh, k[:, cols], v[:, cols], W, rows)
    return proj(o, wo, bo)


# ----------------------------------------------------------------------------
# Decode against a bounded W-slot ring, and the chunk continuation
# ----------------------------------------------------------------------------

def ring_slot(p: int, W: int) -> int:
    """Slot of absolute position p in a W-slot ring.

    Reading of the bounded cache that keeps only the window and drops anything
    older [P2 Problem; P4 Key Advantages, "KV cache of size W"]: W slots, and a
    token overwrites the one exactly W positions older, so position p lives in
    slot p mod W.
    """
    W = _check_window(W)
    if p < 0:
        raise ValueError("position must be >= 0")
    return int(p) % W


def ring_fill(kseq, vseq, pos: Sequence[int], W: int, fill: float = np.nan):
    """Build ring contents from whole token sequences.

    kseq, vseq: (S, H, T, D) per-stream token sequences; pos: (S,) current
    absolute position per stream (pos[s] < T).  Every token t in
    (pos - W, pos] is written to slot ``ring_slot(t, W)``; slots no token has
    reached yet hold ``fill``.  Returns float64 rings (S, H, W, D).
    """
    W = _check_window(W)
    kseq = np.asarray(kseq)
    vseq = np.asarray(vseq)
    S, H, T, D = kseq.shape
    Dv = vseq.shape[-1]
    kring = np.full((S, H, W, D), fill, dtype=np.float64)
    vring = np.full((S, H, W, Dv), fill, dtype=np.float64)
    for s in range(S):
        p = int(pos[s])
        if not 0 <= p < T:
            raise ValueError("pos must lie in [0, T)")
        for t in range(max(0, p - W + 1), p + 1):
            w = ring_slot(t, W)
            kring[s, :, w, :] = kseq[s, :, t, :]
            vring[s, :, w, :] = vseq[s, :, t, :]
    return kring, vring


def _ring_tokens(p: int, W: int) -> list:
    """(slot, token) pairs held by a ring whose newest token is at position p.

    Slot w holds the token t in (p - W, p] with t mod W == w, i.e.
    t = p - ((p - w) mod W); slots whose token would be negative are empty.
    """
    pairs = []
    for w in range(W):
        t = p - ((p - w) % W)
        if t >= 0:
            pairs.append((w, t))
    return pairs


def swa_decode(q, kring, vring, pos: Sequence[int], W: int):
    """One decode step per stream against its ring.

    q: (S, H, D) query of each stream at absolute position pos[s], whose own
    K/V are already in the ring; kring, vring: (S, H, W, D).  The visible keys
    are exactly the ring's occupied slots, which hold the tokens
    (pos - W, pos] (the same window as prefill row pos).  Softmax over them and
    the weighted sum of their values (P3 Step 2).  Empty slots are never read,
    so they may hold anything.  Returns (S, H, Dv) float64.
    """
    W = _check_window(W)
    q = np.asarray(q)
    kring = np.asarray(kring)
    vring = np.asarray(vring)
    S, H, D = q.shape
    Dv = vring.shape[-1]
    if kring.shape[:3] != (S, H, W) or vring.shape[:3] != (S, H, W):
        raise ValueError("rings must be (S, H, W, D)")
    out = np.empty((S, H, Dv), dtype=np.float64)
    root_d = math.sqrt(D)
    for s in range(S):
        p = int(pos[s])
        if p < 0:
            raise ValueError("pos must be >= 0")
        slots = [w for w, _ in _ring_tokens(p, W)]
        for h in range(H):
            kk = _f64(kring[s, h])[slots]                       # (n, D)
            vv = _f64(vring[s, h])[slots]                       # (n, Dv)
            sc = (kk @ _f64(q[s, h])) / root_d                  # (n,)
            e = np.exp(sc - sc.max())
            out[s, h] = (e / e.sum()) @ vv
    return out


def swa_chunk(q, kc, vc, kring, vring, pos0: Sequence[int], W: int):
    """Chunked prefill that continues a stream held in a W-slot ring.

    A chunk of C new tokens at absolute positions pos0[s] .. pos0[s] + C - 1
    arrives for every stream; the ring holds the stream's tokens before pos0
    (positions (pos0 - W, pos0), see ``ring_fill``).  Query p of the chunk sees
    the tokens (p - W, p]: those older than pos0 come from the ring, the rest
    from the chunk itself.  This is the definition of prefill row p over the
    stream's whole history [P1 Problem, the rolling-buffer follow-up; P2
    Problem, bounded cache].

    q, kc, vc: (S, H, C, D); kring, vring: (S, H, W, D).  Returns
    (S, H, C, Dv) float64.
    """
    W = _check_window(W)
    q = np.asarray(q)
    kc = np.asarray(kc)
    vc = np.asarray(vc)
    kring = np.asarray(kring)
    vring = np.asarray(vring)
    S, H, C, D = q.shape
    Dv = vc.shape[-1]
    out = np.empty((S, H, C, Dv), dtype=np.float64)
    root_d = math.sqrt(D)
    for s in range(S):
        p0 = int(pos0[s])
        if p0 < 0:
            raise ValueError("pos0 must be >= 0")
        for c in range(C):
            p = p0 + c
            ks, vs = [], []
            for t in range(max(0, p - W + 1), p + 1):
                if t < p0:
                    w = t % W
                    ks.append(kring[s, :, w, :])
                    vs.append(vring[s, :, w, :])
                else:
                    ks.append(kc[s, :, t - p0, :])
                    vs.append(vc[s, :, t - p0, :])
            kk = np.stack(ks, axis=1).astype(np.float64)        # (H, n, D)
            vv = np.stack(vs, axis=1).astype(np.float64)        # (H, n, Dv)
            qs = q[s, :, c, :].astype(np.float64)               # (H, D)
            sc = np.matmul(kk, qs[:, :, None])[:, :, 0] / root_d
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            w = e / e.sum(axis=1, keepdims=True)
            out[s, :, c, :] = np.matmul(w[:, None, :], vv)[:, 0, :]
    return out
