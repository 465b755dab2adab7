"""Python binding of libswa, causal sliding-window attention on gfx950.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/swa.h``.  PyTorch provides the
device memory and the stream; nothing here computes attention, and there is
no CPU fallback: if ``libswa.so`` is missing every entry point raises.

Entry points (same names as the C ABI):
  swa_forward(q, k, v, out, window_size)        prefill, [B, H, T, D]
  swa_forward_strided(q, k, v, out, window_size, scale=None)
                                                 prefill over strided [B, H, T, D] views
  swa_decode(q, kring, vring, pos, out)          decode against a W-slot ring
  swa_ring_append(knew, vnew, kring, vring, pos) write position pos into slot pos mod W
  swa_decode_workspace_bytes(S, H, D, W, dtype)  workspace of the two entries below
  swa_decode_split(q, kring, vring, pos, out)    decode, window split over workgroups
  swa_decode_append(q, knew, vnew, kring, vring, pos, out)
                                                 append + decode in one launch
  swa_decode_split_noalloc(q, kring, vring, pos, out)
                                                 split decode with the library's static
                                                 scratch (allocates nothing)
  swa_chunk_forward(q, kc, vc, kring, vring, pos0, out)
                                                 chunk of new tokens continuing a ring
  swa_chunk_forward_split(q, kc, vc, kring, vring, pos0, out)
                                                 the same, key range split for few streams
  swa_ring_append_chunk(kc, vc, kring, vring, pos0)
                                                 write a chunk's tokens into the ring
  swa_forward_lse(q, k, v, out, lse, window_size, scale=None)
                                                 prefill that also writes the row log-sum-exp
  swa_backward(q, k, v, out, dout, dq, dk, dv, window_size, scale=None, lse=None)
                                                 gradients of the prefill
  swa_mha_forward(x, wq, bq, wk, bk, wv, bv, wo, bo, out, num_heads, window)
                                                 module forward with projections
Conveniences that allocate the output with torch:
  sliding_window_attention(q, k, v, window_size, scale=None, layout=None) -> out
                                                 differentiable: with an input that
                                                 requires grad, the forward keeps its row
                                                 log-sum-exp and backward calls swa_backward
  decode(q, kring, vring, pos, split=False) -> out
  decode_append(q, knew, vnew, kring, vring, pos) -> out
  chunk_attention(q, kc, vc, kring, vring, pos0, split=False) -> out
  SlidingWindowMHA(d_model, num_heads)(x, window) -> out
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "SWA_F32", "SWA_BF16", "SWA_OK", "SWA_ERR_INVALID_ARG",
    "SWA_ERR_UNSUPPORTED", "SWA_ERR_LAUNCH", "SWAError", "lib", "abi_version",
    "status_string", "swa_forward", "swa_forward_strided", "swa_decode", "swa_ring_append", "swa_chunk_forward",
    "swa_ring_append_chunk", "swa_chunk_workspace_bytes", "swa_chunk_forward_split",
    "swa_decode_workspace_bytes", "swa_decode_split", "swa_decode_split_noalloc",
    "SWA_ERR_SCRATCH_LIMIT", "NOALLOC_SCRATCH_BYTES",
    "swa_decode_append", "swa_forward_lse", "swa_backward", "swa_mha_workspace_bytes", "swa_mha_forward", "SlidingWindowMHA",
    "sliding_window_attention", "decode", "decode_append", "chunk_attention",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswa.so")

SWA_F32, SWA_BF16 = 0, 1
SWA_OK, SWA_ERR_INVALID_ARG, SWA_ERR_UNSUPPORTED, SWA_ERR_LAUNCH = 0, 1, 2, 3
SWA_ERR_SCRATCH_LIMIT = 4
NOALLOC_SCRATCH_BYTES = 2 * 1024 * 1024     # SWA_NOALLOC_SCRATCH_BYTES of include/swa.h

_DTYPES = {torch.float32: SWA_F32, torch.bfloat16: SWA_BF16}
_lib = None


class SWAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libswa error {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libswa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m sliding_window_causal_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.swa_abi_version.argtypes = []
    L.swa_abi_version.restype = i32
    L.swa_status_string.argtypes = [i32]
    L.swa_status_string.restype = ctypes.c_char_p
    L.swa_forward.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i32, p]
    L.swa_forward.restype = i32
    L.swa_forward_strided.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, p, ctypes.c_double,
                                      i32, p]
    L.swa_forward_strided.restype = i32
    L.swa_decode.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, p]
    L.swa_decode.restype = i32
    L.swa_ring_append.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, p]
    L.swa_ring_append.restype = i32
    L.swa_backward_workspace_bytes.argtypes = [i64, i64, i64]
    L.swa_backward_workspace_bytes.restype = i64
    L.swa_backward.argtypes = [p] * 9 + [i64, i64, i64, i64, i64, ctypes.c_double, i32, p, i64, p]
    L.swa_forward_lse.argtypes = [p] * 5 + [i64, i64, i64, i64, i64, ctypes.c_double, i32, p]
    L.swa_forward_lse.restype = i32
    L.swa_backward.restype = i32
    L.swa_mha_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.swa_mha_workspace_bytes.restype = i64
    L.swa_mha_forward.argtypes = [p] * 10 + [i64, i64, i64, i64, i64, i32, p, i64, p]
    L.swa_mha_forward.restype = i32
    L.swa_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    L.swa_decode_workspace_bytes.restype = i64
    L.swa_decode_split.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, p, i64, p]
    L.swa_decode_split.restype = i32
    L.swa_decode_split_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, p]
    L.swa_decode_split_noalloc.restype = i32
    L.swa_decode_append.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i32, p, i64, p]
    L.swa_decode_append.restype = i32
    L.swa_chunk_forward.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i32, p]
    L.swa_chunk_forward.restype = i32
    L.swa_chunk_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.swa_chunk_workspace_bytes.restype = i64
    L.swa_chunk_forward_split.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i32, p,
                                          i64, p]
    L.swa_chunk_forward_split.restype = i32
    L.swa_ring_append_chunk.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, p]
    L.swa_ring_append_chunk.restype = i32
    _lib = L
    return L


def abi_version() -> int:
    return int(lib().swa_abi_version())


def status_string(status: int) -> str:
    return lib().swa_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != SWA_OK:
        raise SWAError(status, status_string(status))


def _stream(t: torch.Tensor, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _dtype_code(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    if any(t.dtype != dt for t in ts):
        raise TypeError("all tensors must share one dtype")
    if dt not in _DTYPES:
        raise TypeError(f"dtype {dt} not supported (float32 or bfloat16)")
    return _DTYPES[dt]


def _check_device(*ts: torch.Tensor, contiguous: bool = True) -> None:
    dev = ts[0].device
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU device (no CPU fallback)")
        if t.device != dev:
            raise ValueError("tensors must be on one device")
        if contiguous and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _window(window_size) -> int:
    if isinstance(window_size, bool) or not isinstance(window_size, int):
        raise TypeError("window_size must be an int")
    if window_size < 1:
        raise ValueError("window_size must be >= 1")
    return window_size


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def swa_forward(q, k, v, out, window_size: int, stream=None) -> None:
    """Prefill into ``out``; q, k, v, out are contiguous [B, H, T, D]."""
    W = _window(window_size)
    _check_device(q, k, v, out)
    code = _dtype_code(q, k, v, out)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, k, v, out must all be [B, H, T, D] of one shape")
    B, H, T, D = q.shape
    _check(lib().swa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, D, W, code,
                             _stream(q, stream)))


def swa_forward_strided(q, k, v, out, window_size: int, scale=None, stream=None) -> None:
    """Prefill into ``out`` for [B, H, T, D] views of any strides whose last
    axis is contiguous (e.g. a (B, T, H, D) tensor seen through
    ``permute(0, 2, 1, 3)``); ``scale`` multiplies the scores (None: 1/sqrt(D))."""
    W = _window(window_size)
    _check_device(q, k, v, out, contiguous=False)
    code = _dtype_code(q, k, v, out)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, k, v, out must all be [B, H, T, D] views of one shape")
    if any(t.stride(3) != 1 for t in (q, k, v, out)):
        raise ValueError("the head-size axis must be contiguous")
    if scale is None:
        scale = 0.0                       # the library's code for 1 / sqrt(D)
    elif isinstance(scale, bool) or not isinstance(scale, (int, float)):
        raise TypeError("scale must be a number")
    elif scale == 0 or scale != scale or abs(scale) == float("inf"):
        raise ValueError("scale must be finite and non-zero")
    B, H, T, D = q.shape
    st = (ctypes.c_int64 * 12)(*[x for t in (q, k, v, out) for x in t.stride()[:3]])
    _check(lib().swa_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, D, W, st,
                                     float(scale), code, _stream(q, stream)))


def _scale_code(scale) -> float:
    if scale is None:
        return 0.0                        # the library's code for 1 / sqrt(D)
    if isinstance(scale, bool) or not isinstance(scale, (int, float)):
        raise TypeError("scale must be a number")
    if scale == 0 or scale != scale or abs(scale) == float("inf"):
        raise ValueError("scale must be finite and non-zero")
    return float(scale)


def _check_lse(lse, q):
    B, H, T, _ = q.shape
    if lse.dtype != torch.float32 or lse.shape != (B, H, T):
        raise ValueError("lse must be float32 [B, H, T]")
    _check_device(q, lse)


def swa_forward_lse(q, k, v, out, lse, window_size: int, scale=None, stream=None) -> None:
    """Prefill into ``out`` ([B, H, T, D], contiguous) and each row's
    log-sum-exp of its scaled scores into ``lse`` (float32 [B, H, T])."""
    W = _window(window_size)
    _check_device(q, k, v, out)
    code = _dtype_code(q, k, v, out)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, k, v, out must all be [B, H, T, D] of one shape")
    _check_lse(lse, q)
    B, H, T, D = q.shape
    _check(lib().swa_forward_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, T, D, W,
                                 _scale_code(scale), code, _stream(q, stream)))


def swa_backward(q, k, v, out, dout, dq, dk, dv, window_size: int, scale=None, lse=None,
                 workspace=None, stream=None) -> None:
    """Gradients dq, dk, dv ([B, H, T, D]) of the prefill given its output
    ``out`` and dout; ``scale`` None means 1/sqrt(D); ``lse`` optionally the
    forward's log-sum-exp (swa_forward_lse)."""
    W = _window(window_size)
    ts = (q, k, v, out, dout, dq, dk, dv)
    _check_device(*ts)
    code = _dtype_code(*ts)
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("all tensors must be [B, H, T, D] of one shape")
    scale = _scale_code(scale)
    if lse is not None:
        _check_lse(lse, q)
    B, H, T, D = q.shape
    need = int(lib().swa_backward_workspace_bytes(B, H, T))
    if need < 0:
        raise SWAError(-need, status_string(-need))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    else:
        _given_workspace(workspace, q.device)
    _check(lib().swa_backward(*[_ptr(t) for t in ts[:5]], None if lse is None else _ptr(lse),
                              *[_ptr(t) for t in ts[5:]], B, H, T, D, W, scale, code,
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(q, stream)))


def swa_decode(q, kring, vring, pos, out, stream=None) -> None:
    """Decode into ``out``; q, out [S, H, D]; rings [S, H, W, D]; pos int64 [S]."""
    _check_device(q, kring, vring, pos, out)
    code = _dtype_code(q, kring, vring, out)
    if q.dim() != 3 or kring.dim() != 4 or vring.shape != kring.shape or out.shape != q.shape:
        raise ValueError("q/out must be [S, H, D] and rings [S, H, W, D]")
    S, H, D = q.shape
    if kring.shape[0] != S or kring.shape[1] != H or kring.shape[3] != D:
        raise ValueError("ring shape does not match q")
    if pos.dtype != torch.int64 or pos.shape != (S,):
        raise ValueError("pos must be int64 [S]")
    W = kring.shape[2]
    _check(lib().swa_decode(_ptr(q), _ptr(kring), _ptr(vring), _ptr(pos), _ptr(out), S, H, D, W,
                            code, _stream(q, stream)))


def swa_decode_workspace_bytes(S: int, H: int, D: int, W: int, dtype) -> int:
    """Device workspace bytes swa_decode_split / swa_decode_append need (0: none)."""
    code = _DTYPES.get(dtype, dtype) if not isinstance(dtype, int) else dtype
    n = int(lib().swa_decode_workspace_bytes(S, H, D, W, code))
    if n < 0:
        raise SWAError(-n, status_string(-n))
    return n


def _decode_dims(q, kring, vring, pos, out):
    if q.dim() != 3 or kring.dim() != 4 or vring.shape != kring.shape or out.shape != q.shape:
        raise ValueError("q/out must be [S, H, D] and rings [S, H, W, D]")
    S, H, D = q.shape
    if kring.shape[0] != S or kring.shape[1] != H or kring.shape[3] != D:
        raise ValueError("ring shape does not match q")
    if pos.dtype != torch.int64 or pos.shape != (S,):
        raise ValueError("pos must be int64 [S]")
    return S, H, D, kring.shape[2]


def _given_workspace(workspace, device):
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace


def _workspace(q, S, H, D, W, workspace):
    need = swa_decode_workspace_bytes(S, H, D, W, _DTYPES[q.dtype])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _given_workspace(workspace, q.device)
    return workspace, workspace.numel() * workspace.element_size()


def swa_decode_split(q, kring, vring, pos, out, workspace=None, stream=None) -> None:
    """swa_decode with the window split over several workgroups when S * H is
    small; ``workspace`` (bytes from swa_decode_workspace_bytes) is allocated
    here when not given."""
    _check_device(q, kring, vring, pos, out)
    code = _dtype_code(q, kring, vring, out)
    S, H, D, W = _decode_dims(q, kring, vring, pos, out)
    ws, nb = _workspace(q, S, H, D, W, workspace)
    _check(lib().swa_decode_split(_ptr(q), _ptr(kring), _ptr(vring), _ptr(pos), _ptr(out), S, H,
                                  D, W, code, _ptr(ws), nb, _stream(q, stream)))


def swa_decode_split_noalloc(q, kring, vring, pos, out, stream=None) -> None:
    """swa_decode_split with the split's partials in the library's static
    device scratch: no allocation, no workspace; overlapping calls on one GPU
    race."""
    _check_device(q, kring, vring, pos, out)
    code = _dtype_code(q, kring, vring, out)
    S, H, D, W = _decode_dims(q, kring, vring, pos, out)
    _check(lib().swa_decode_split_noalloc(_ptr(q), _ptr(kring), _ptr(vring), _ptr(pos),
                                          _ptr(out), S, H, D, W, code, _stream(q, stream)))


def swa_decode_append(q, knew, vnew, kring, vring, pos, out, workspace=None, stream=None) -> None:
    """Write knew, vnew ([S, H, D]) into slot pos mod W and decode q against
    the ring including them, in one launch."""
    _check_device(q, knew, vnew, kring, vring, pos, out)
    code = _dtype_code(q, knew, vnew, kring, vring, out)
    S, H, D, W = _decode_dims(q, kring, vring, pos, out)
    if knew.shape != q.shape or vnew.shape != q.shape:
        raise ValueError("knew, vnew must be [S, H, D] like q")
    ws, nb = _workspace(q, S, H, D, W, workspace)
    _check(lib().swa_decode_append(_ptr(q), _ptr(knew), _ptr(vnew), _ptr(kring), _ptr(vring),
                                   _ptr(pos), _ptr(out), S, H, D, W, code, _ptr(ws), nb,
                                   _stream(q, stream)))


def swa_ring_append(knew, vnew, kring, vring, pos, stream=None) -> None:
    """kring[s, h, pos[s] mod W] = knew[s, h] (and v); knew [S, H, D]."""
    _check_device(knew, vnew, kring, vring, pos)
    code = _dtype_code(knew, vnew, kring, vring)
    if knew.dim() != 3 or vnew.shape != knew.shape or kring.dim() != 4 or vring.shape != kring.shape:
        raise ValueError("knew/vnew must be [S, H, D] and rings [S, H, W, D]")
    S, H, D = knew.shape
    if kring.shape[0] != S or kring.shape[1] != H or kring.shape[3] != D:
        raise ValueError("ring shape does not match knew")
    if pos.dtype != torch.int64 or pos.shape != (S,):
        raise ValueError("pos must be int64 [S]")
    W = kring.shape[2]
    _check(lib().swa_ring_append(_ptr(knew), _ptr(vnew), _ptr(kring), _ptr(vring), _ptr(pos),
                                 S, H, D, W, code, _stream(knew, stream)))


def _check_chunk(q, kc, vc, kring, vring, pos0):
    if q.dim() != 4 or kc.shape != q.shape or vc.shape != q.shape:
        raise ValueError("q, kc, vc must be [S, H, C, D] of one shape")
    S, H, C, D = q.shape
    if kring.dim() != 4 or vring.shape != kring.shape or kring.shape[0] != S or \
            kring.shape[1] != H or kring.shape[3] != D:
        raise ValueError("rings must be [S, H, W, D] matching the chunk")
    if pos0.dtype != torch.int64 or pos0.shape != (S,):
        raise ValueError("pos0 must be int64 [S]")
    return S, H, C, D, kring.shape[2]


def swa_chunk_forward(q, kc, vc, kring, vring, pos0, out, stream=None) -> None:
    """Chunk continuation of a ring into ``out`` [S, H, C, D]; the ring is read only."""
    _check_device(q, kc, vc, kring, vring, pos0, out)
    code = _dtype_code(q, kc, vc, kring, vring, out)
    S, H, C, D, W = _check_chunk(q, kc, vc, kring, vring, pos0)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    _check(lib().swa_chunk_forward(_ptr(q), _ptr(kc), _ptr(vc), _ptr(kring), _ptr(vring),
                                   _ptr(pos0), _ptr(out), S, H, C, D, W, code, _stream(q, stream)))


def swa_chunk_workspace_bytes(S: int, H: int, C: int, D: int, W: int, dtype) -> int:
    code = _DTYPES.get(dtype, dtype) if not isinstance(dtype, int) else dtype
    n = int(lib().swa_chunk_workspace_bytes(S, H, C, D, W, code))
    if n < 0:
        raise SWAError(-n, status_string(-n))
    return n


def swa_chunk_forward_split(q, kc, vc, kring, vring, pos0, out, workspace=None,
                            stream=None) -> None:
    """swa_chunk_forward with the key range split over workgroups for few
    streams; ``workspace`` is allocated here when not given."""
    _check_device(q, kc, vc, kring, vring, pos0, out)
    code = _dtype_code(q, kc, vc, kring, vring, out)
    S, H, C, D, W = _check_chunk(q, kc, vc, kring, vring, pos0)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    need = swa_chunk_workspace_bytes(S, H, C, D, W, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _given_workspace(workspace, q.device)
    _check(lib().swa_chunk_forward_split(_ptr(q), _ptr(kc), _ptr(vc), _ptr(kring), _ptr(vring),
                                         _ptr(pos0), _ptr(out), S, H, C, D, W, code,
                                         _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(q, stream)))


def swa_ring_append_chunk(kc, vc, kring, vring, pos0, stream=None) -> None:
    """Write the chunk's last min(C, W) tokens into ring slots (pos0 + c) mod W."""
    _check_device(kc, vc, kring, vring, pos0)
    code = _dtype_code(kc, vc, kring, vring)
    S, H, C, D, W = _check_chunk(kc, kc, vc, kring, vring, pos0)
    _check(lib().swa_ring_append_chunk(_ptr(kc), _ptr(vc), _ptr(kring), _ptr(vring), _ptr(pos0),
                                       S, H, C, D, W, code, _stream(kc, stream)))


def chunk_attention(q, kc, vc, kring, vring, pos0, split: bool = False):
    """Chunk continuation returning a new [S, H, C, D] tensor (split:
    swa_chunk_forward_split)."""
    out = torch.empty_like(q)
    if split:
        swa_chunk_forward_split(q, kc, vc, kring, vring, pos0, out)
    else:
        swa_chunk_forward(q, kc, vc, kring, vring, pos0, out)
    return out


def swa_mha_workspace_bytes(B: int, T: int, d_model: int, dtype) -> int:
    code = _DTYPES.get(dtype, dtype) if not isinstance(dtype, int) else dtype
    n = int(lib().swa_mha_workspace_bytes(B, T, d_model, code))
    if n < 0:
        raise SWAError(-n, status_string(-n))
    return n


def swa_mha_forward(x, wq, bq, wk, bk, wv, bv, wo, bo, out, num_heads: int, window_size: int,
                    workspace=None, stream=None) -> None:
    """Module forward into ``out``: x, out [B, T, d_model]; w* [d_model, d_model]
    applied as x @ w; b* [d_model] or None (zero)."""
    W = _window(window_size)
    ws = [t for t in (x, wq, wk, wv, wo, out, bq, bk, bv, bo) if t is not None]
    _check_device(*ws)
    code = _dtype_code(*ws)
    if x.dim() != 3 or out.shape != x.shape:
        raise ValueError("x and out must be [B, T, d_model]")
    B, T, dm = x.shape
    for w in (wq, wk, wv, wo):
        if w.shape != (dm, dm):
            raise ValueError("projection kernels must be [d_model, d_model]")
    for b in (bq, bk, bv, bo):
        if b is not None and b.shape != (dm,):
            raise ValueError("biases must be [d_model]")
    need = swa_mha_workspace_bytes(B, T, dm, x.dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    else:
        _given_workspace(workspace, x.device)
    ptr = lambda t: None if t is None else _ptr(t)
    _check(lib().swa_mha_forward(_ptr(x), _ptr(wq), ptr(bq), _ptr(wk), ptr(bk), _ptr(wv), ptr(bv),
                                 _ptr(wo), ptr(bo), _ptr(out), B, T, dm, int(num_heads), W, code,
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(x, stream)))


class SlidingWindowMHA:
    """Multi-head sliding-window self-attention with q, k, v and output
    projections (the module of the NNX exercise), forward only.  Weights are
    plain tensors: kernels [d_model, d_model] applied as x @ w, biases
    [d_model]; by default kernels ~ N(0, 1/d_model) and zero biases."""

    def __init__(self, d_model: int, num_heads: int, dtype=torch.bfloat16, device="cuda",
                 generator=None):
        if num_heads < 1 or d_model % num_heads:
            raise ValueError("d_model must be a positive multiple of num_heads")
        self.d_model, self.num_heads = d_model, num_heads
        std = d_model ** -0.5
        mk = lambda: (torch.randn(d_model, d_model, generator=generator, device=device) * std
                      ).to(dtype)
        self.wq, self.wk, self.wv, self.wo = mk(), mk(), mk(), mk()
        z = lambda: torch.zeros(d_model, dtype=dtype, device=device)
        self.bq, self.bk, self.bv, self.bo = z(), z(), z(), z()

    def __call__(self, x, window: int):
        squeeze = x.dim() == 2                        # the exercise's (T, d_model)
        xb = x.unsqueeze(0) if squeeze else x
        out = torch.empty_like(xb)
        swa_mha_forward(xb, self.wq, self.bq, self.wk, self.bk, self.wv, self.bv, self.wo,
                        self.bo, out, self.num_heads, window)
        return out[0] if squeeze else out


_LAYOUTS = ("bhtd", "bshd", "btd")


class _SlidingWindowAttention(torch.autograd.Function):
    """swa_forward_lse forward, swa_backward backward, on contiguous
    [B, H, T, D] tensors; the row log-sum-exp saved by the forward spares the
    backward its own forward pass."""

    @staticmethod
    def forward(ctx, q, k, v, window_size, scale):
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        swa_forward_lse(q, k, v, out, lse, window_size, scale=scale)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.window_size, ctx.scale = window_size, scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        swa_backward(q, k, v, out, dout.contiguous(), dq, dk, dv, ctx.window_size,
                     scale=ctx.scale, lse=lse)
        return dq, dk, dv, None, None


def sliding_window_attention(q, k, v, window_size: int, scale=None, layout: str = None):
    """Prefill returning a new tensor in the layout of ``q``.

    layout "bhtd": [B, H, T, D];  "bshd": [B, T, H, D];  "btd": [B, T, D], one
    head.  Default: "bhtd" for 4-D inputs, "btd" for 3-D.  ``scale`` multiplies
    the scores (None: 1/sqrt(D)).  Contiguous [B, H, T, D] inputs with the
    default scale go through swa_forward; everything else through
    swa_forward_strided, reading the tensors in place.

    When autograd is on and q, k or v requires grad, the result is
    differentiable: the inputs are brought to contiguous [B, H, T, D] (views,
    or copies where the layout needs them), the forward runs swa_forward_lse
    and the backward swa_backward with that log-sum-exp; the result is then a
    view in the layout of ``q``.
    """
    if layout is None:
        layout = "btd" if q.dim() == 3 else "bhtd"
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {_LAYOUTS}")
    if q.dim() != (3 if layout == "btd" else 4):
        raise ValueError(f"layout {layout!r} needs {3 if layout == 'btd' else 4}-D tensors")
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v)):
        if layout == "btd":
            to4, back = (lambda t: t.unsqueeze(1)), (lambda t: t.squeeze(1))
        elif layout == "bshd":
            to4, back = (lambda t: t.transpose(1, 2)), (lambda t: t.transpose(1, 2))
        else:
            to4, back = (lambda t: t), (lambda t: t)
        qb, kb, vb = (to4(t).contiguous() for t in (q, k, v))
        return back(_SlidingWindowAttention.apply(qb, kb, vb, window_size, scale))
    out = torch.empty_like(q)
    if layout == "btd":
        views = [t.unsqueeze(1) for t in (q, k, v, out)]
    elif layout == "bshd":
        views = [t.permute(0, 2, 1, 3) for t in (q, k, v, out)]
    else:
        views = [q, k, v, out]
    if scale is None and all(t.is_contiguous() for t in views):
        swa_forward(*views, window_size)
    else:
        swa_forward_strided(*views, window_size, scale=scale)
    return out


def decode(q, kring, vring, pos, split: bool = False):
    """Decode returning a new [S, H, D] tensor (split: swa_decode_split)."""
    out = torch.empty_like(q)
    if split:
        swa_decode_split(q, kring, vring, pos, out)
    else:
        swa_decode(q, kring, vring, pos, out)
    return out


def decode_append(q, knew, vnew, kring, vring, pos):
    """Fused append + decode returning a new [S, H, D] tensor."""
    out = torch.empty_like(q)
    swa_decode_append(q, knew, vnew, kring, vring, pos, out)
    return out
