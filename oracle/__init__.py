"""CPU oracle for one rank's share of tensor-parallel linear layers.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library and never imports it; the two meet only through the
seeded inputs of ``synth_inputs``.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation, explicit
slicing); this module is argument marshalling with numpy plus the plan
validation rules, which are integer checks written out in Python.

Source pages (Hugging Face Diffusers documentation):
  [TP] "Tensor parallelism": opening definition; "Colwise and rowwise";
       "Fused projections"; "Constraints and verification".
  [DI] "Distributed inference": section "Tensor parallelism".

bf16 tensors are numpy ``uint16`` arrays holding the bit patterns.  Weights
are nn.Linear ``W[out_features, in_features]``.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (brute force, closed forms, library routines,
invariants, and the page-derived fixtures under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ACT_NONE = 0
ACT_GELU_TANH = 1


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I = ctypes.c_int
            lib.orc_bf16_from_double.restype = ctypes.c_uint16
            lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
            lib.orc_bf16_to_double.restype = ctypes.c_double
            lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.orc_round_bf16.argtypes = [P, P, I64]
            lib.orc_widen_bf16.argtypes = [P, P, I64]
            lib.orc_gelu_tanh.restype = ctypes.c_double
            lib.orc_gelu_tanh.argtypes = [ctypes.c_double]
            lib.orc_linear_rows.argtypes = [P, I64, P, I64, P, I, P, I64, I64, I64, P, I]
            lib.orc_shard_colwise.argtypes = [P, P, I64, I64, I, I, P, P]
            lib.orc_shard_rowwise.argtypes = [P, I64, I64, I, I, P]
            lib.orc_shard_packed_colwise.argtypes = [P, P, I64, I64, P, I, I, I, P, P]
            lib.orc_qkv_split.restype = I
            lib.orc_qkv_split.argtypes = [P, P, I64, I64, I64, I, I, P, P]
            lib.orc_combine_sum_f32.argtypes = [P, I, I64, I64, I64, P, P, I64]
            lib.orc_combine_concat.argtypes = [P, I, I64, I64, I64, P, I, I, P, I64]
            _lib = lib
    return _lib


def default_threads() -> int:
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(a, name):
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected uint16 bf16 bit patterns, got {a.dtype}")
    return np.ascontiguousarray(a)


# --------------------------------------------------------------------------------------
# bf16 and GELU
# --------------------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even), returning uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def bf16_widen(h) -> np.ndarray:
    """Exact bf16 -> float64 widening."""
    h = _u16(h, "h")
    out = np.empty(h.shape, dtype=np.float64)
    _load().orc_widen_bf16(_ptr(h), _ptr(out), h.size)
    return out


def gelu_tanh(v: float) -> float:
    """GELU, tanh approximation, evaluated in double."""
    return _load().orc_gelu_tanh(float(v))


# --------------------------------------------------------------------------------------
# Linear layers
# --------------------------------------------------------------------------------------

def linear(x, w, bias=None, act=ACT_NONE, rows=None, threads=None) -> np.ndarray:
    """``act(x . w^T + bias)`` in float64 for the listed rows of x (all rows by default).

    x: uint16 [M, K] (a strided view is copied; use :func:`linear_strided` to keep strides),
    w: uint16 [N, K], bias: uint16 [N] or None.  Returns float64 [len(rows), N].
    """
    x = _u16(x, "x")
    return linear_strided(x, x.shape[1], x.shape[1], w, bias, act, rows, threads, m=x.shape[0])


def linear_strided(xbuf, ldx, k, w, bias=None, act=ACT_NONE, rows=None, threads=None,
                   m=None, col0=0) -> np.ndarray:
    """Like :func:`linear` but x is columns ``[col0, col0 + k)`` of a row-major buffer of stride ldx."""
    xbuf = _u16(xbuf, "x").reshape(-1)
    w = _u16(w, "w")
    n, kw = w.shape
    if kw != k:
        raise ValueError("w inner dim mismatch")
    if m is None:
        m = (xbuf.size - col0 - k) // ldx + 1 if xbuf.size else 0
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if rows.size and (rows.min() < 0 or rows.max() >= m):
        raise ValueError("row index out of range")
    if bias is not None:
        bias = _u16(bias, "bias")
        if bias.shape != (n,):
            raise ValueError("bias shape mismatch")
    out = np.empty((rows.size, n), dtype=np.float64)
    if rows.size and n:
        base = xbuf[col0:]
        _load().orc_linear_rows(_ptr(base), ldx, _ptr(w), k, _ptr(bias), int(act), _ptr(rows),
                                rows.size, n, k, _ptr(out),
                                int(threads or default_threads()))
    return out


def colwise(x, w_shard, b_shard=None, act=ACT_NONE, rows=None, threads=None) -> np.ndarray:
    """[TP] "Colwise and rowwise": a colwise rank computes its output slice
    ``act(x . W_r^T + b_r)``; float64 before the output rounding."""
    return linear(x, w_shard, b_shard, act, rows, threads)


def rowwise(x_full, rank: int, tp_degree: int, w_shard, rows=None, threads=None) -> np.ndarray:
    """[TP] "Colwise and rowwise": a rowwise rank computes a partial sum from its slice of
    the input features, ``x[:, r*K/P:(r+1)*K/P] . W_r^T`` (no bias); float64."""
    x_full = _u16(x_full, "x")
    m, k_full = x_full.shape
    k_loc = k_full // tp_degree
    return linear_strided(x_full, k_full, k_loc, w_shard, None, ACT_NONE, rows, threads,
                          m=m, col0=rank * k_loc)


def colwise_swiglu(x, w_shard, b_shard=None, rows=None, threads=None) -> np.ndarray:
    """[TP] "Fused projections": a SwiGLU gate and up projection packed with blocks
    [1, 1]; a rank's shard holds its gate rows then its up rows (2 n rows).  Output
    ``silu(g) * u`` with ``g = x . gate^T + b_gate`` and ``u = x . up^T + b_up`` in
    float64, ``silu(v) = v / (1 + e^-v)`` (the Swish gate of SwiGLU); float64 before
    the output rounding."""
    w = _u16(w_shard, "w")
    if w.shape[0] % 2:
        raise ValueError("a SwiGLU shard has an even number of rows [gate; up]")
    n = w.shape[0] // 2
    bg = bu = None
    if b_shard is not None:
        b = _u16(b_shard, "b")
        bg, bu = b[:n], b[n:]
    g = linear(x, np.ascontiguousarray(w[:n]), bg, ACT_NONE, rows, threads)
    u = linear(x, np.ascontiguousarray(w[n:]), bu, ACT_NONE, rows, threads)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def rowwise_split_input(x_full, rank: int, tp_degree: int, w_shard, rows=None, threads=None) -> np.ndarray:
    """[TP] "Colwise and rowwise" (the rowwise_split_input style): the input is the
    same on every rank and each rank cuts its own slice of the input features, then
    computes the rowwise partial ``x[:, r*K/P:(r+1)*K/P] . W_r^T`` (no bias); float64.
    The P partials summed, plus the bias once, are the unsharded layer."""
    x_full = _u16(x_full, "x")
    check_plan("rowwise", tp_degree, rank, _u16(w_shard, "w").shape[0], x_full.shape[1])
    return rowwise(x_full, rank, tp_degree, w_shard, rows, threads)


# --------------------------------------------------------------------------------------
# Slicing
# --------------------------------------------------------------------------------------

def shard_colwise(w, b, tp_degree: int, rank: int):
    """[TP] "Colwise and rowwise": rows ``[r*N/P, (r+1)*N/P)`` of W and of b."""
    w = _u16(w, "w")
    n, k = w.shape
    check_plan("colwise", tp_degree, rank, n, k)
    ws = np.empty((n // tp_degree, k), dtype=np.uint16)
    bs = None
    if b is not None:
        b = _u16(b, "b")
        bs = np.empty(n // tp_degree, dtype=np.uint16)
    _load().orc_shard_colwise(_ptr(w), _ptr(b), n, k, tp_degree, rank, _ptr(ws), _ptr(bs))
    return ws, bs


def shard_rowwise(w, tp_degree: int, rank: int):
    """[TP] "Colwise and rowwise": columns ``[r*K/P, (r+1)*K/P)`` of W; the bias is not cut."""
    w = _u16(w, "w")
    n, k = w.shape
    check_plan("rowwise", tp_degree, rank, n, k)
    ws = np.empty((n, k // tp_degree), dtype=np.uint16)
    _load().orc_shard_rowwise(_ptr(w), n, k, tp_degree, rank, _ptr(ws))
    return ws


def shard_packed_colwise(w, b, blocks, tp_degree: int, rank: int):
    """[TP] "Fused projections": shard each packed block independently (blocks proportional)."""
    w = _u16(w, "w")
    n, k = w.shape
    check_plan("colwise", tp_degree, rank, n, k, blocks=blocks)
    bl = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    ws = np.empty((n // tp_degree, k), dtype=np.uint16)
    bs = None
    if b is not None:
        b = _u16(b, "b")
        bs = np.empty(n // tp_degree, dtype=np.uint16)
    _load().orc_shard_packed_colwise(_ptr(w), _ptr(b), n, k, _ptr(bl), bl.size, tp_degree,
                                     rank, _ptr(ws), _ptr(bs))
    return ws, bs


def qkv_split(w, b, num_heads: int, head_dim: int, tp_degree: int, rank: int):
    """[TP] "Colwise and rowwise" (attention): rank r's whole heads of each of Q, K, V."""
    w = _u16(w, "w")
    n, k = w.shape
    if n != 3 * num_heads * head_dim:
        raise ValueError("fused QKV weight must have 3*num_heads*head_dim rows")
    check_plan("qkv", tp_degree, rank, n, k, num_heads=num_heads)
    n_loc = n // tp_degree
    ws = np.empty((n_loc, k), dtype=np.uint16)
    bs = None
    if b is not None:
        b = _u16(b, "b")
        bs = np.empty(n_loc, dtype=np.uint16)
    rc = _load().orc_qkv_split(_ptr(w), _ptr(b), num_heads, head_dim, k, tp_degree, rank,
                               _ptr(ws), _ptr(bs))
    if rc != 0:
        raise ValueError("qkv split rejected")
    return ws, bs


# --------------------------------------------------------------------------------------
# Checkpoint reading
# --------------------------------------------------------------------------------------

_ST_DTYPES = {"BF16": np.dtype("<u2"), "F32": np.dtype("<f4")}


def read_safetensors(path: str, name: str):
    """[TP] "Load a sharded model" / "Limitations": the sharded load reads safetensors
    files.  Tensor ``name`` read whole, from the format's published definition: an 8-byte
    little-endian header length H, H bytes of JSON mapping each name to its dtype, shape and
    ``data_offsets`` [begin, end) into the byte buffer that follows the header, and row-major
    data.  Returns ``(array, dtype_name)``; BF16 comes back as uint16 bit patterns."""
    import json
    with open(path, "rb") as f:
        h = int.from_bytes(f.read(8), "little")
        header = json.loads(f.read(h).decode("utf-8"))
        entry = header[name]
        begin, end = entry["data_offsets"]
        f.seek(8 + h + begin)
        raw = f.read(end - begin)
    dt = _ST_DTYPES[entry["dtype"]]
    shape = tuple(entry["shape"])
    if len(raw) != int(np.prod(shape)) * dt.itemsize:
        raise ValueError("data_offsets do not match the shape")
    return np.frombuffer(raw, dtype=dt).reshape(shape).astype(dt.newbyteorder("="), copy=True), entry["dtype"]


def load_shard(path: str, name: str, style: str, tp_degree: int, rank: int, blocks=None):
    """[TP] "Load a sharded model": rank ``rank``'s shard of tensor ``name`` -- the whole
    tensor read by :func:`read_safetensors`, then cut by this module's slicers (a colwise cut
    of a 1-D bias takes its rows; a rowwise cut takes the columns of W, i.e. the rows of
    W^T, so packed rowwise blocks reuse the packed colwise slicer on W^T).  fp32 tensors are
    sliced as pairs of uint16 halves, which leaves every cut bit-exact."""
    t, dt = read_safetensors(path, name)
    u = t.view(np.uint16) if dt == "F32" else t   # [.., 2 * cols] for fp32
    per = 2 if dt == "F32" else 1
    if t.ndim == 1:
        if style != "colwise":
            raise PlanError("a 1-D tensor is sharded colwise only")
        col = u.reshape(t.shape[0], per)
        ws = shard_packed_colwise(col, None, blocks or [1], tp_degree, rank)[0]
        out = ws.reshape(-1)
    elif style == "colwise":
        out = shard_packed_colwise(u, None, blocks or [1], tp_degree, rank)[0]
    elif style in ("rowwise", "rowwise_split_input"):
        n, k = t.shape
        # columns of W (in units of whole elements): slice W^T's rows, then transpose back
        wt = np.ascontiguousarray(u.reshape(n, k, per).transpose(1, 0, 2).reshape(k, n * per))
        s_t = shard_packed_colwise(wt, None, blocks or [1], tp_degree, rank)[0]
        out = np.ascontiguousarray(s_t.reshape(k // tp_degree, n, per).transpose(1, 0, 2).reshape(n, -1))
    else:
        raise ValueError("style must be colwise, rowwise or rowwise_split_input")
    return (out.view(np.float32) if dt == "F32" else out), dt


# --------------------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------------------

def combine_sum(parts, bias=None) -> np.ndarray:
    """[TP] AllReduce of rowwise partials, one GPU: ``((p0 + p1) + ...) + b`` in fp32,
    ascending rank, bias (bf16 bits) once.  parts: list of float32 [M, N]."""
    parts = [np.ascontiguousarray(np.asarray(p, dtype=np.float32)) for p in parts]
    if not parts:
        raise ValueError("no parts")
    m, n = parts[0].shape
    for p in parts:
        if p.shape != (m, n):
            raise ValueError("part shape mismatch")
    if bias is not None:
        bias = _u16(bias, "bias")
        if bias.shape != (n,):
            raise ValueError("bias shape mismatch")
    out = np.empty((m, n), dtype=np.float32)
    arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
    _load().orc_combine_sum_f32(arr, len(parts), n, m, n, _ptr(bias), _ptr(out), n)
    return out


def combine_concat(parts, blocks=None) -> np.ndarray:
    """[TP] AllGather of colwise outputs, one GPU: the inverse of the (packed) colwise
    slicing of output columns.  parts: list of [M, n_part] uint16 or float32 arrays."""
    parts = [np.ascontiguousarray(p) for p in parts]
    if not parts:
        raise ValueError("no parts")
    dt = parts[0].dtype
    if dt not in (np.uint16, np.float32):
        raise TypeError("concat parts must be uint16 (bf16) or float32")
    m, n_part = parts[0].shape
    for p in parts:
        if p.shape != (m, n_part) or p.dtype != dt:
            raise ValueError("part shape/dtype mismatch")
    tp = len(parts)
    check_plan("colwise", tp, 0, n_part * tp, 1, blocks=blocks)
    out = np.empty((m, n_part * tp), dtype=dt)
    arr = (ctypes.c_void_p * tp)(*[p.ctypes.data for p in parts])
    bl = None if blocks is None else np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    _load().orc_combine_concat(arr, tp, n_part, m, n_part, _ptr(bl), 0 if bl is None else bl.size,
                               dt.itemsize, _ptr(out), n_part * tp)
    return out


# --------------------------------------------------------------------------------------
# Plan validation (integer rules)
# --------------------------------------------------------------------------------------

class PlanError(ValueError):
    """A plan that the pages' constraints reject."""


def check_plan(style: str, tp_degree: int, rank: int, out_features: int, in_features: int,
               blocks=None, num_heads=None) -> None:
    """[TP] "Constraints and verification": tp_degree divides the head count; every packed
    block (not only their sum) is divisible by tp_degree; checked before any slicing.
    [TP] "Fused projections": block proportions must sum to a divisor of the packed dim.
    Plain colwise needs P | out_features, rowwise P | in_features."""
    if tp_degree < 1:
        raise PlanError("tp_degree must be >= 1")
    if not (0 <= rank < tp_degree):
        raise PlanError("rank out of range")
    if out_features < 0 or in_features < 0:
        raise PlanError("negative dims")
    if style == "qkv":
        if num_heads is None or num_heads < 1:
            raise PlanError("num_heads required")
        if num_heads % tp_degree:
            raise PlanError("tp_degree must divide the number of attention heads")
        blocks = [1, 1, 1]
        style = "colwise"
    dim = out_features if style == "colwise" else in_features
    if style not in ("colwise", "rowwise"):
        raise PlanError(f"unknown style {style}")
    if blocks is None:
        if dim % tp_degree:
            raise PlanError("tp_degree must divide the sharded dim")
        return
    blocks = [int(b) for b in blocks]
    if not blocks or any(b < 1 for b in blocks):
        raise PlanError("blocks must be positive integers")
    s = sum(blocks)
    if dim % s:
        raise PlanError("sum(blocks) must divide the packed dim")
    unit = dim // s
    for b in blocks:
        if (b * unit) % tp_degree:
            raise PlanError("each packed block must be divisible by tp_degree")
