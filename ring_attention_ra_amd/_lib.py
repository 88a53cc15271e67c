"""ctypes binding of libra.so: one Python function per C entry point, same names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are passed
to the C ABI. Every computation happens in the library's HIP kernels. If the
library has not been built this module raises; there is no fallback.
bind() does the checking and marshalling of one call once and returns a
function that repeats the call, for loops that issue the same calls again.
"""

from __future__ import annotations

import contextvars
import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# RA_LIB may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("RA_LIB") or os.path.join(PKG, "libra.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ra.h")

RA_OK, RA_ERR_INVALID_ARGUMENT, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_NONFINITE = 0, 1, 2, 3, 4
RA_BF16, RA_FP32 = 0, 1
RA_CONTIGUOUS, RA_ZIGZAG = 0, 1

_DTYPE_CODE = {torch.bfloat16: RA_BF16, torch.float32: RA_FP32}
LAYOUTS = {"contiguous": RA_CONTIGUOUS, "zigzag": RA_ZIGZAG}


class RaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class RaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("len_q", ctypes.c_int32), ("len_kv", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_DIMS = ctypes.POINTER(RaDims)

_SIGNATURES = {
    "ra_positions": [_I64, _I32, _I32, _I32, _P, _P],
    "ra_layout_permute": [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P],
    "ra_rope": [_P, _P, _P, _I64, _I64, _I32, _I32, _F32, _P],
    "ra_state_init": [_DIMS, _P, _P, _P, _P],
    "ra_step_fwd": [_DIMS, _P, _P, _P, _P, _P, _I32, _F32, _P, _P, _P, _P, _P],
    "ra_finalize": [_DIMS, _P, _P, _P, _P, _P, _P],
    "ra_bwd_delta": [_DIMS, _P, _P, _P, _P],
    "ra_step_bwd": [_DIMS, _P, _P, _P, _P, _P, _I32, _F32, _P, _P, _P, _P, _P, _P, _P, _P],
    "ra_count_nonfinite": [_P, _I64, _I32, ctypes.POINTER(ctypes.c_int64), _P],
    "ra_count_nonfinite_noalloc": [_P, _I64, _I32, ctypes.POINTER(ctypes.c_int64), _P],
    "ra_last_error": [],
    "ra_abi_version": [],
}


def lib() -> ctypes.CDLL:
    """The loaded libra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m ring_attention_ra_amd.build`")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        cdll.ra_last_error.restype = ctypes.c_char_p
        _lib = cdll
    return _lib


def header_symbols() -> list[str]:
    """Names of the entry points declared in include/ra.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:ra_status|const char\*|int32_t)\s+(ra_\w+)\s*\(", text, re.M)))


def _check(status: int, name: str) -> None:
    if status != RA_OK:
        raise RaError(status, f"{name}: {lib().ra_last_error().decode()}")


# While bind() records a call, the entry points hand their marshalled
# arguments to it instead of calling the library.
_RECORDING: contextvars.ContextVar = contextvars.ContextVar("ra_recording", default=None)


def _invoke(name: str, *cargs) -> None:
    rec = _RECORDING.get()
    if rec is not None:
        rec.append((name, cargs))
        return
    _check(getattr(lib(), name)(*cargs), name)


def bind(entry, *args, **kwargs):
    """Check and marshal the arguments of one call of `entry` (one of the
    entry-point functions below that return nothing) once, without calling
    the library; returns a function of no arguments that makes exactly that
    call (same pointers, sizes and stream) and raises RaError on a non-OK
    status. The caller keeps the tensors alive and in place. For loops that
    issue the same calls many times (a ring of steps), where checking the
    tensors on every call would cost more host time than the GPU spends."""
    rec: list = []
    token = _RECORDING.set(rec)
    try:
        entry(*args, **kwargs)
    finally:
        _RECORDING.reset(token)
    if len(rec) != 1:
        raise ValueError(f"{getattr(entry, '__name__', entry)} cannot be bound")
    name, cargs = rec[0]
    fn = getattr(lib(), name)

    def call() -> None:
        status = fn(*cargs)
        if status != RA_OK:
            _check(status, name)

    call.__name__ = f"bound_{name}"
    return call


def _ptr(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def dtype_code(dt: torch.dtype) -> int:
    try:
        return _DTYPE_CODE[dt]
    except KeyError:
        raise ValueError(f"unsupported dtype {dt}") from None


def make_dims(batch, heads_q, heads_kv, head_dim, len_q, len_kv, dtype) -> RaDims:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return RaDims(batch, heads_q, heads_kv, head_dim, len_q, len_kv, code)


def dims_of(q: torch.Tensor, k_blk: torch.Tensor) -> RaDims:
    """Dims of a step from q [B,Hq,Lq,D] and a K chunk [B,Hkv,Lkv,D]."""
    b, hq, lq, d = q.shape
    _, hkv, lkv, _ = k_blk.shape
    return make_dims(b, hq, hkv, d, lq, lkv, q.dtype)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def ra_positions(seq_len, n_ranks, rank, layout, pos_out, stream=None):
    lay = LAYOUTS.get(layout, layout)
    _invoke("ra_positions", seq_len, n_ranks, rank, lay, _ptr(pos_out, "pos_out", torch.int32),
                              _stream(stream))


def ra_layout_permute(src, dst, pos, outer, seq_len, row_elems, n_ranks, layout, rank=-1, inverse=0,
                      stream=None):
    if src.dtype != dst.dtype:
        raise ValueError("src and dst must have the same dtype")
    lay = LAYOUTS.get(layout, layout)
    _invoke("ra_layout_permute", _ptr(src, "src"), _ptr(dst, "dst"),
                                   _ptr(pos, "pos", torch.int32, allow_none=True), outer, seq_len,
                                   row_elems, dtype_code(src.dtype), n_ranks, lay, rank, int(inverse),
                                   _stream(stream))


def ra_rope(x, y, pos, base=10000.0, stream=None):
    """RoPE of x ``[..., L, D]`` into y (may be x) at the int32 positions ``[L]``."""
    if x.dtype != y.dtype or x.shape != y.shape:
        raise ValueError("x and y must have the same dtype and shape")
    if x.dim() < 2:
        raise ValueError("x must be [..., L, D]")
    length, d = x.shape[-2], x.shape[-1]
    outer = x.numel() // max(length * d, 1)
    _invoke("ra_rope", _ptr(x, "x"), _ptr(y, "y"), _ptr(pos, "pos", torch.int32, length), outer, length, d,
                         dtype_code(x.dtype), float(base), _stream(stream))


def ra_state_init(dims, o_acc, m, l, stream=None):
    rows = dims.batch * dims.heads_q * dims.len_q
    _invoke("ra_state_init", ctypes.byref(dims), _ptr(o_acc, "o_acc", torch.float32, rows * dims.head_dim),
                               _ptr(m, "m", torch.float32, rows), _ptr(l, "l", torch.float32, rows),
                               _stream(stream))


def ra_step_fwd(dims, q, k_blk, v_blk, q_pos, k_pos, causal, scale, alibi_slopes, o_acc, m, l, stream=None):
    dt = q.dtype
    rows = dims.batch * dims.heads_q * dims.len_q
    kv = dims.batch * dims.heads_kv * dims.len_kv * dims.head_dim
    _invoke("ra_step_fwd",
        ctypes.byref(dims), _ptr(q, "q", dt, rows * dims.head_dim), _ptr(k_blk, "k_blk", dt, kv),
        _ptr(v_blk, "v_blk", dt, kv), _ptr(q_pos, "q_pos", torch.int32, dims.len_q),
        _ptr(k_pos, "k_pos", torch.int32, dims.len_kv), int(bool(causal)), float(scale),
        _ptr(alibi_slopes, "alibi_slopes", torch.float32, dims.heads_q, allow_none=True),
        _ptr(o_acc, "o_acc", torch.float32, rows * dims.head_dim), _ptr(m, "m", torch.float32, rows),
        _ptr(l, "l", torch.float32, rows), _stream(stream))


def ra_finalize(dims, o_acc, m, l, o, lse, stream=None):
    rows = dims.batch * dims.heads_q * dims.len_q
    odt = torch.bfloat16 if dims.dtype == RA_BF16 else torch.float32
    _invoke("ra_finalize",
        ctypes.byref(dims), _ptr(o_acc, "o_acc", torch.float32, rows * dims.head_dim),
        _ptr(m, "m", torch.float32, rows), _ptr(l, "l", torch.float32, rows),
        _ptr(o, "o", odt, rows * dims.head_dim, allow_none=True),
        _ptr(lse, "lse", torch.float32, rows, allow_none=True), _stream(stream))


def ra_bwd_delta(dims, o, d_o, delta, stream=None):
    rows = dims.batch * dims.heads_q * dims.len_q
    odt = torch.bfloat16 if dims.dtype == RA_BF16 else torch.float32
    _invoke("ra_bwd_delta", ctypes.byref(dims), _ptr(o, "o", odt, rows * dims.head_dim),
                              _ptr(d_o, "d_o", odt, rows * dims.head_dim),
                              _ptr(delta, "delta", torch.float32, rows), _stream(stream))


def ra_step_bwd(dims, q, k_blk, v_blk, q_pos, k_pos, causal, scale, alibi_slopes, d_o, lse, delta,
                dq_acc, dk_blk, dv_blk, stream=None):
    dt = q.dtype
    rows = dims.batch * dims.heads_q * dims.len_q
    kv = dims.batch * dims.heads_kv * dims.len_kv * dims.head_dim
    _invoke("ra_step_bwd",
        ctypes.byref(dims), _ptr(q, "q", dt, rows * dims.head_dim), _ptr(k_blk, "k_blk", dt, kv),
        _ptr(v_blk, "v_blk", dt, kv), _ptr(q_pos, "q_pos", torch.int32, dims.len_q),
        _ptr(k_pos, "k_pos", torch.int32, dims.len_kv), int(bool(causal)), float(scale),
        _ptr(alibi_slopes, "alibi_slopes", torch.float32, dims.heads_q, allow_none=True),
        _ptr(d_o, "d_o", dt, rows * dims.head_dim), _ptr(lse, "lse", torch.float32, rows),
        _ptr(delta, "delta", torch.float32, rows), _ptr(dq_acc, "dq_acc", torch.float32, rows * dims.head_dim),
        _ptr(dk_blk, "dk_blk", torch.float32, kv), _ptr(dv_blk, "dv_blk", torch.float32, kv),
        _stream(stream))


def ra_count_nonfinite(x, stream=None) -> int:
    """Number of NaN / Inf elements of the bf16 or fp32 GPU tensor x (waits
    for the stream)."""
    n = ctypes.c_int64(-1)
    _check(lib().ra_count_nonfinite(_ptr(x, "x"), x.numel(), dtype_code(x.dtype), ctypes.byref(n),
                                    _stream(stream)), "ra_count_nonfinite")
    return int(n.value)


def ra_count_nonfinite_noalloc(x, stream=None) -> int:
    """ra_count_nonfinite through the library's static scratch counter (no
    device allocation; calls that overlap on one GPU race)."""
    n = ctypes.c_int64(-1)
    _check(lib().ra_count_nonfinite_noalloc(_ptr(x, "x"), x.numel(), dtype_code(x.dtype), ctypes.byref(n),
                                            _stream(stream)), "ra_count_nonfinite_noalloc")
    return int(n.value)


def ra_last_error() -> str:
    return lib().ra_last_error().decode()


def ra_abi_version() -> int:
    return int(lib().ra_abi_version())
