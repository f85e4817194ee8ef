"""ctypes binding of libtp_linear.so (include/tp_linear.h).

Argument marshalling only: torch tensors are used for their device pointers,
strides and the current stream, outputs are allocated with ``torch.empty``
when the caller passes none, and every step of the computation runs in the
HIP kernels behind the C ABI.  There is no CPU path: a missing library or a
tensor that is not on the GPU is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtp_linear.so")

TP_OK = 0
TP_ERR_INVALID_ARG = -1
TP_ERR_NOT_DIVISIBLE = -2
TP_ERR_UNSUPPORTED = -3
TP_ERR_HIP = -4
TP_ERR_IO = -5

TP_BF16 = 0
TP_F32 = 1
TP_ACT_NONE = 0
TP_ACT_GELU_TANH = 1
TP_ACT_SWIGLU = 2
TP_COLWISE = 0
TP_ROWWISE = 1
TP_ROWWISE_SPLIT_INPUT = 2
TP_COMBINE_SUM = 0
TP_COMBINE_CONCAT = 1

# Every symbol the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
SIGNATURES = {
    "tp_linear_colwise": (_I, [_P, _I64, _P, _I64, _P, _P, _I64, _I, _I, _I64, _I64, _I64, _P]),
    "tp_linear_rowwise": (_I, [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P]),
    "tp_linear_tile_shape": (_I, [_I64, _I64, _I64, _I, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "tp_linear_rowwise_split_input": (_I, [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _I64, _I, _I, _P]),
    "tp_fused_qkv_split": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _P]),
    "tp_partial_combine": (_I, [ctypes.POINTER(_P), _I, _I64, _P, _I64, _I, _I, _I, _P,
                                ctypes.POINTER(_I64), _I, _I64, _I64, _P]),
    "tp_plan_shard_slice": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, ctypes.POINTER(_I64), _I, _I,
                                 _I, ctypes.POINTER(_I64), ctypes.POINTER(_I64), _P]),
    "tp_load_shard": (_I, [ctypes.c_char_p, ctypes.c_char_p, _I, ctypes.POINTER(_I64), _I, _I, _I, _P, _I64,
                           ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I), _P]),
    "tp_last_error": (ctypes.c_char_p, []),
}

_lib = None


class TPError(Exception):
    """Base class of errors reported by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class TPValueError(TPError, ValueError):
    """Invalid argument, plan-divisibility violation or unsupported request."""


class TPRuntimeError(TPError, RuntimeError):
    """The HIP runtime reported an error."""


class TPIOError(TPError, OSError):
    """A checkpoint file could not be read or is malformed."""


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (built by ``tensor_sharded_linear_amd.build``); fail loudly if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def tp_last_error() -> str:
    msg = load_library().tp_last_error()
    return msg.decode() if msg else ""


def _check(status: int) -> None:
    if status == TP_OK:
        return
    msg = tp_last_error()
    if status == TP_ERR_HIP:
        raise TPRuntimeError(status, msg)
    if status == TP_ERR_IO:
        raise TPIOError(status, msg)
    raise TPValueError(status, msg)


# --------------------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------------------

_DT = {torch.bfloat16: TP_BF16, torch.float32: TP_F32}


def _stream(stream, t: torch.Tensor) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev2d(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (there is no CPU path)")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major, possibly padded rows)")
    return t


def _ld(t: torch.Tensor) -> int:
    """Row stride in elements; a single row has no meaningful stride, so report its width."""
    if t.shape[0] > 1:
        return t.stride(0)
    return max(t.stride(0), t.shape[1])


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _vec(t: Optional[torch.Tensor], name: str, n: int) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 1 or t.shape[0] != n or \
            (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous bf16 GPU vector of length {n}")
    return t


# --------------------------------------------------------------------------------------
# the five entry points
# --------------------------------------------------------------------------------------

def tp_linear_colwise(x: torch.Tensor, w_shard: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      *, act: str = "none", out: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """Colwise shard: ``out = act(x @ w_shard.T + bias)`` (bf16 in, fp32 accumulate).

    ``act="swiglu"``: ``w_shard`` is a packed [gate; up] shard of 2 n rows (and ``bias``
    2 n entries); ``out`` [M, n] = silu(x @ gate.T + b_gate) * (x @ up.T + b_up)."""
    lib = load_library()
    x = _dev2d(x, "x", torch.bfloat16)
    w_shard = _dev2d(w_shard, "w_shard", torch.bfloat16)
    m, k = x.shape
    try:
        a = {"none": TP_ACT_NONE, "gelu_tanh": TP_ACT_GELU_TANH, "swiglu": TP_ACT_SWIGLU}[act]
    except KeyError:
        raise ValueError("act must be 'none', 'gelu_tanh' or 'swiglu'") from None
    rows = w_shard.shape[0]
    if a == TP_ACT_SWIGLU and rows % 2:
        raise ValueError(f"a SwiGLU shard has an even number of rows [gate; up], got {rows}")
    n = rows // 2 if a == TP_ACT_SWIGLU else rows
    if w_shard.shape[1] != k:
        raise ValueError(f"x is [M, {k}] but w_shard is {tuple(w_shard.shape)}")
    bias = _vec(bias, "bias", rows)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    out = _dev2d(out, "out")
    if tuple(out.shape) != (m, n) or out.dtype not in _DT:
        raise ValueError(f"out must be [{m}, {n}] bf16 or fp32")
    _check(lib.tp_linear_colwise(_ptr(x), _ld(x), _ptr(w_shard), _ld(w_shard), _ptr(bias), _ptr(out),
                                 _ld(out), _DT[out.dtype], a, m, n, k, _stream(stream, x)))
    return out


def tp_linear_tile_shape(m: int, n: int, k: int, act: str = "none") -> tuple:
    """(rows, cols) of the output tile the tiled kernel uses for an [m, k] x [n, k]^T problem
    on the current device (rows 256, 224, 192, 128 or 64; cols 256 or 192, 128 with SwiGLU); for the
    split-K kernel (up to 128 rows) (its row blocks x 16, its run of 4 to 48 output columns per
    workgroup, at most 16 with SwiGLU); or (0, 0)
    where the weight-streaming kernel runs.  For ``act="swiglu"`` n counts the outputs.
    Host-only query: no device work."""
    lib = load_library()
    try:
        a = {"none": TP_ACT_NONE, "gelu_tanh": TP_ACT_GELU_TANH, "swiglu": TP_ACT_SWIGLU}[act]
    except KeyError:
        raise ValueError("act must be 'none', 'gelu_tanh' or 'swiglu'") from None
    rows, cols = _I64(), _I64()
    _check(lib.tp_linear_tile_shape(m, n, k, a, ctypes.byref(rows), ctypes.byref(cols)))
    return rows.value, cols.value


def tp_linear_rowwise(x_shard: torch.Tensor, w_shard: torch.Tensor, *,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Rowwise shard: fp32 partial ``out = x_shard @ w_shard.T`` (no bias)."""
    lib = load_library()
    x_shard = _dev2d(x_shard, "x_shard", torch.bfloat16)
    w_shard = _dev2d(w_shard, "w_shard", torch.bfloat16)
    m, k = x_shard.shape
    n = w_shard.shape[0]
    if w_shard.shape[1] != k:
        raise ValueError(f"x_shard is [M, {k}] but w_shard is {tuple(w_shard.shape)}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x_shard.device)
    out = _dev2d(out, "out", torch.float32)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    _check(lib.tp_linear_rowwise(_ptr(x_shard), _ld(x_shard), _ptr(w_shard), _ld(w_shard), _ptr(out),
                                 _ld(out), m, n, k, _stream(stream, x_shard)))
    return out


def tp_linear_rowwise_split_input(x_full: torch.Tensor, w_shard: torch.Tensor, tp_degree: int, rank: int, *,
                                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rowwise_split_input shard: fp32 partial ``out = x_full[:, slice_r] @ w_shard.T``.

    ``x_full`` is the replicated input [M, K]; the library cuts rank ``rank``'s
    slice of its K columns (K / tp_degree of them) itself.  ``w_shard`` is the
    rank's column block [N, K / tp_degree] of the weight."""
    lib = load_library()
    x_full = _dev2d(x_full, "x_full", torch.bfloat16)
    w_shard = _dev2d(w_shard, "w_shard", torch.bfloat16)
    m, k_full = x_full.shape
    n = w_shard.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x_full.device)
    out = _dev2d(out, "out", torch.float32)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    if tp_degree >= 1 and k_full % tp_degree == 0 and w_shard.shape[1] != k_full // tp_degree:
        raise ValueError(f"w_shard is {tuple(w_shard.shape)} but the input slice has {k_full // tp_degree} columns")
    _check(lib.tp_linear_rowwise_split_input(_ptr(x_full), _ld(x_full), k_full, _ptr(w_shard), _ld(w_shard),
                                             _ptr(out), _ld(out), m, n, tp_degree, rank,
                                             _stream(stream, x_full)))
    return out


def tp_fused_qkv_split(w_qkv: torch.Tensor, b_qkv: Optional[torch.Tensor], num_heads: int,
                       head_dim: int, tp_degree: int, rank: int, *,
                       w_out: Optional[torch.Tensor] = None, b_out: Optional[torch.Tensor] = None,
                       stream=None):
    """Head-aligned shard ``[Q_r; K_r; V_r]`` of a fused QKV weight (and bias)."""
    lib = load_library()
    if not w_qkv.is_cuda or w_qkv.dim() != 2 or not w_qkv.is_contiguous() or w_qkv.dtype not in _DT:
        raise ValueError("w_qkv must be a contiguous 2-D bf16/fp32 GPU tensor")
    k = w_qkv.shape[1]
    rows = 3 * (num_heads // tp_degree) * head_dim if tp_degree > 0 else 0
    if w_out is None:
        w_out = torch.empty((rows, k), dtype=w_qkv.dtype, device=w_qkv.device)
    if b_qkv is not None and b_out is None:
        b_out = torch.empty((rows,), dtype=b_qkv.dtype, device=w_qkv.device)
    for t, name in ((w_out, "w_out"), (b_qkv, "b_qkv"), (b_out, "b_out")):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != w_qkv.dtype):
            raise ValueError(f"{name} must be a contiguous GPU tensor of the weight's dtype")
    if w_qkv.shape[0] != 3 * num_heads * head_dim:
        raise ValueError("w_qkv must have 3 * num_heads * head_dim rows")
    _check(lib.tp_fused_qkv_split(_ptr(w_qkv), _ptr(b_qkv), _ptr(w_out), _ptr(b_out), num_heads,
                                  head_dim, k, _DT[w_qkv.dtype], tp_degree, rank,
                                  _stream(stream, w_qkv)))
    return w_out, b_out


def tp_partial_combine(parts: Sequence[torch.Tensor], mode: str = "sum", *,
                       bias: Optional[torch.Tensor] = None, blocks: Optional[Sequence[int]] = None,
                       out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                       stream=None) -> torch.Tensor:
    """Layer-boundary combine on one device: ``"sum"`` of fp32 partials (+ bias once) or
    ``"concat"`` of colwise output slices (``blocks`` for a packed output)."""
    lib = load_library()
    parts = list(parts)
    if not parts:
        raise ValueError("no parts")
    p0 = _dev2d(parts[0], "parts[0]")
    m, n_part = p0.shape
    ld = _ld(p0)
    for i, p in enumerate(parts):
        _dev2d(p, f"parts[{i}]", p0.dtype)
        if tuple(p.shape) != (m, n_part) or _ld(p) != ld:
            raise ValueError("all parts must share shape and row stride")
    if mode == "sum":
        mode_c, n_out = TP_COMBINE_SUM, n_part
        out_dtype = out_dtype or torch.float32
        bias = _vec(bias, "bias", n_part)
    elif mode == "concat":
        mode_c, n_out = TP_COMBINE_CONCAT, n_part * len(parts)
        out_dtype = out_dtype or p0.dtype
    else:
        raise ValueError("mode must be 'sum' or 'concat'")
    if out is None:
        out = torch.empty((m, n_out), dtype=out_dtype, device=p0.device)
    out = _dev2d(out, "out")
    if tuple(out.shape) != (m, n_out) or out.dtype not in _DT:
        raise ValueError(f"out must be [{m}, {n_out}]")
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    bl = None
    nb = 0
    if blocks is not None:
        nb = len(blocks)
        bl = (ctypes.c_int64 * max(nb, 1))(*[int(b) for b in blocks])
    _check(lib.tp_partial_combine(arr, len(parts), ld, _ptr(out), _ld(out), _DT[p0.dtype],
                                  _DT[out.dtype], mode_c, _ptr(bias), bl, nb, m, n_part,
                                  _stream(stream, p0)))
    return out


def tp_plan_shard_shape(out_features: int, in_features: int, style: str, tp_degree: int, rank: int,
                        blocks: Optional[Sequence[int]] = None):
    """Shape query of :func:`tp_plan_shard_slice` (validation only, no device work)."""
    lib = load_library()
    rows, cols = ctypes.c_int64(0), ctypes.c_int64(0)
    bl, nb = _blocks(blocks)
    _check(lib.tp_plan_shard_slice(None, None, None, None, out_features, in_features, TP_BF16,
                                   _style(style), bl, nb, tp_degree, rank, ctypes.byref(rows),
                                   ctypes.byref(cols), None))
    return rows.value, cols.value


def _style(style: str) -> int:
    try:
        return {"colwise": TP_COLWISE, "rowwise": TP_ROWWISE, "rowwise_split_input": TP_ROWWISE_SPLIT_INPUT}[style]
    except KeyError:
        raise ValueError("style must be 'colwise', 'rowwise' or 'rowwise_split_input'") from None


def _blocks(blocks):
    if blocks is None:
        return None, 0
    nb = len(blocks)
    return (ctypes.c_int64 * max(nb, 1))(*[int(b) for b in blocks]), nb


def tp_plan_shard_slice(w_full: torch.Tensor, b_full: Optional[torch.Tensor], style: str,
                        tp_degree: int, rank: int, *, blocks: Optional[Sequence[int]] = None,
                        w_out: Optional[torch.Tensor] = None, b_out: Optional[torch.Tensor] = None,
                        stream=None):
    """Rank ``rank``'s shard of a full nn.Linear weight (and, colwise, its bias)."""
    lib = load_library()
    if not w_full.is_cuda or w_full.dim() != 2 or not w_full.is_contiguous() or w_full.dtype not in _DT:
        raise ValueError("w_full must be a contiguous 2-D bf16/fp32 GPU tensor")
    o, i = w_full.shape
    rows, cols = tp_plan_shard_shape(o, i, style, tp_degree, rank, blocks)
    if w_out is None:
        w_out = torch.empty((rows, cols), dtype=w_full.dtype, device=w_full.device)
    if b_full is not None and b_out is None:
        b_out = torch.empty((rows,), dtype=b_full.dtype, device=w_full.device)
    for t, name in ((w_out, "w_out"), (b_full, "b_full"), (b_out, "b_out")):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != w_full.dtype):
            raise ValueError(f"{name} must be a contiguous GPU tensor of the weight's dtype")
    if tuple(w_out.shape) != (rows, cols):
        raise ValueError(f"w_out must be [{rows}, {cols}]")
    bl, nb = _blocks(blocks)
    r_, c_ = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.tp_plan_shard_slice(_ptr(w_full), _ptr(b_full), _ptr(w_out), _ptr(b_out), o, i,
                                   _DT[w_full.dtype], _style(style), bl, nb, tp_degree, rank,
                                   ctypes.byref(r_), ctypes.byref(c_), _stream(stream, w_full)))
    return w_out, b_out


_DT_OF = {TP_BF16: torch.bfloat16, TP_F32: torch.float32}


def tp_load_shard_shape(path: str, name: str, style: str = "colwise", tp_degree: int = 1, rank: int = 0, *,
                        blocks: Optional[Sequence[int]] = None):
    """Shape query of :func:`tp_load_shard`: reads the file's header only.

    Returns ``(shard_rows, shard_cols, dtype)``; a 1-D tensor reports one row."""
    lib = load_library()
    rows, cols, dt = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int(0)
    bl, nb = _blocks(blocks)
    _check(lib.tp_load_shard(os.fsencode(path), name.encode(), _style(style), bl, nb, tp_degree, rank, None, 0,
                             ctypes.byref(rows), ctypes.byref(cols), ctypes.byref(dt), None))
    return rows.value, cols.value, _DT_OF[dt.value]


def tp_load_shard(path: str, name: str, style: str = "colwise", tp_degree: int = 1, rank: int = 0, *,
                  blocks: Optional[Sequence[int]] = None, out: Optional[torch.Tensor] = None,
                  device=None, stream=None) -> torch.Tensor:
    """Rank ``rank``'s shard of tensor ``name`` read from the safetensors file ``path``
    straight into GPU memory (only the slice's bytes are read).

    A 2-D weight is cut by ``style`` (and packed ``blocks``) like
    :func:`tp_plan_shard_slice`; a 1-D bias only colwise.  Returns a contiguous
    GPU tensor of the file's dtype: ``[rows, cols]``, or ``[cols]`` for a bias."""
    lib = load_library()
    rows, cols, dt = tp_load_shard_shape(path, name, style, tp_degree, rank, blocks=blocks)
    if out is None:
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        if dev.type != "cuda":
            raise TypeError("tp_load_shard writes GPU memory (there is no CPU path)")
        one_d = _header_ndim(path, name) == 1   # a 1-D tensor comes back 1-D
        out = torch.empty((cols,) if one_d else (rows, cols), dtype=dt, device=dev)
    if not isinstance(out, torch.Tensor) or not out.is_cuda or not out.is_contiguous() or out.dtype != dt:
        raise ValueError(f"out must be a contiguous {dt} GPU tensor")
    if out.numel() != rows * cols:
        raise ValueError(f"out must hold {rows} x {cols} elements, got shape {tuple(out.shape)}")
    bl, nb = _blocks(blocks)
    r_, c_, d_ = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int(0)
    _check(lib.tp_load_shard(os.fsencode(path), name.encode(), _style(style), bl, nb, tp_degree, rank,
                             out.data_ptr(), out.numel() * out.element_size(), ctypes.byref(r_), ctypes.byref(c_),
                             ctypes.byref(d_), _stream(stream, out)))
    return out


def _header_ndim(path: str, name: str) -> int:
    """Number of dimensions (1 or 2) of tensor ``name``, from two shape queries: a 1-D tensor
    and a [1, n] weight both report one row, but only the weight accepts a rowwise cut."""
    rows, _, _ = tp_load_shard_shape(path, name, "colwise", 1, 0)
    if rows != 1:
        return 2
    try:
        tp_load_shard_shape(path, name, "rowwise", 1, 0)
        return 2
    except TPValueError:
        return 1
