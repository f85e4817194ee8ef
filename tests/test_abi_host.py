"""Host-side tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before any device work.  CPU only: no call here
reaches a kernel launch (every call fails validation, is a shape query, or is
an M == 0 no-op).
"""
import ctypes
import os
import re

import pytest

import oracle
import tensor_sharded_linear_amd as tsl
from tensor_sharded_linear_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_linear.h")

# Fake, well-aligned device addresses: validation never dereferences them.
A = 0x7F0000000000
A2 = 0x7F0000100000
A3 = 0x7F0000200000


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(tp_[a-z_]+)\s*\(", text))


def test_library_loads_and_exports_every_declared_symbol():
    lib = tsl.load_library()
    syms = declared_symbols()
    assert syms == {"tp_linear_colwise", "tp_linear_rowwise", "tp_linear_rowwise_split_input",
                    "tp_fused_qkv_split", "tp_partial_combine", "tp_plan_shard_slice", "tp_load_shard",
                    "tp_linear_tile_shape", "tp_last_error"}
    for s in syms:
        assert hasattr(lib, s), s
    assert set(B.SIGNATURES) == syms


def test_nm_shows_extern_c_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", tsl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for s in declared_symbols():
        assert s in names, s


def _call(name, *args):
    lib = tsl.load_library()
    return getattr(lib, name)(*args)


def colwise(**kw):
    a = dict(x=A, ldx=256, w=A2, ldw=256, bias=None, y=A3, ldy=512, y_dtype=B.TP_BF16,
             act=B.TP_ACT_NONE, M=64, N=512, K=256, stream=None)
    a.update(kw)
    return _call("tp_linear_colwise", *a.values())


def rowwise(**kw):
    a = dict(x=A, ldx=512, w=A2, ldw=512, p=A3, ldp=256, M=64, N=256, K=512, stream=None)
    a.update(kw)
    return _call("tp_linear_rowwise", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), B.TP_ERR_UNSUPPORTED),
    (dict(N=500), B.TP_ERR_UNSUPPORTED),
    (dict(M=-1), B.TP_ERR_INVALID_ARG),
    (dict(N=0), B.TP_ERR_INVALID_ARG),
    (dict(ldx=128), B.TP_ERR_INVALID_ARG),
    (dict(ldx=260), B.TP_ERR_INVALID_ARG),
    (dict(ldw=200), B.TP_ERR_INVALID_ARG),
    (dict(ldy=500), B.TP_ERR_INVALID_ARG),
    (dict(x=None), B.TP_ERR_INVALID_ARG),
    (dict(w=None), B.TP_ERR_INVALID_ARG),
    (dict(y=None), B.TP_ERR_INVALID_ARG),
    (dict(x=A + 2), B.TP_ERR_INVALID_ARG),
    (dict(bias=A + 4), B.TP_ERR_INVALID_ARG),
    (dict(y_dtype=7), B.TP_ERR_INVALID_ARG),
    (dict(act=3), B.TP_ERR_INVALID_ARG),
    (dict(K=(1 << 31)), B.TP_ERR_UNSUPPORTED),
    # operand views of 2 GiB or more: the kernels use 32-bit byte offsets
    (dict(M=1 << 20, ldx=1 << 10, ldw=1 << 10, K=1 << 10), B.TP_ERR_UNSUPPORTED),
    (dict(N=1 << 20, ldy=1 << 20, ldx=1 << 10, ldw=1 << 10, K=1 << 10), B.TP_ERR_UNSUPPORTED),
    # strides whose products with a row count would overflow 64 bits
    (dict(ldw=1 << 62), B.TP_ERR_UNSUPPORTED),
    (dict(ldx=1 << 62), B.TP_ERR_UNSUPPORTED),
    (dict(ldy=(1 << 61) + 512), B.TP_ERR_UNSUPPORTED),
    # more output tiles than one launch can hold (2^22): 2^21 x 2^21 with one-row operands
    (dict(M=1 << 21, N=1 << 21, ldy=1 << 21, ldx=64, ldw=64, K=64), B.TP_ERR_UNSUPPORTED),
])
def test_colwise_validation(kw, status):
    assert colwise(**kw) == status
    assert tsl.tp_last_error().startswith("tp_linear_colwise")


def test_swiglu_weight_extent_counts_both_halves():
    """A SwiGLU shard reads 2 n_shard weight rows: n rows fit under 2 GiB, 2 n do not."""
    n, k = 1 << 18, 1 << 11
    st = colwise(N=n, ldy=n, K=k, ldx=k, ldw=k, act=B.TP_ACT_SWIGLU)
    assert st == B.TP_ERR_UNSUPPORTED
    assert "2 GiB" in tsl.tp_last_error()


def test_colwise_and_rowwise_empty_is_noop():
    assert colwise(M=0, x=None, y=None) == B.TP_OK
    assert rowwise(M=0, x=None, p=None) == B.TP_OK
    assert tsl.tp_last_error() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), B.TP_ERR_UNSUPPORTED),
    (dict(N=250), B.TP_ERR_UNSUPPORTED),
    (dict(ldp=258), B.TP_ERR_INVALID_ARG),
    (dict(ldp=128), B.TP_ERR_INVALID_ARG),
    (dict(ldx=500), B.TP_ERR_INVALID_ARG),
    (dict(p=A3 + 8), B.TP_ERR_INVALID_ARG),
    (dict(M=(1 << 20) + 1, ldx=1 << 10, ldw=1 << 10, K=1 << 10), B.TP_ERR_UNSUPPORTED),
])
def test_rowwise_validation(kw, status):
    assert rowwise(**kw) == status


def split_input(**kw):
    a = dict(x=A, ldx=1024, k_full=1024, w=A2, ldw=256, p=A3, ldp=256, M=4, N=256, P=4, r=1, stream=None)
    a.update(kw)
    return _call("tp_linear_rowwise_split_input", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), B.TP_ERR_INVALID_ARG),
    (dict(r=4), B.TP_ERR_INVALID_ARG),
    (dict(r=-1), B.TP_ERR_INVALID_ARG),
    (dict(k_full=1002, ldx=1008), B.TP_ERR_NOT_DIVISIBLE),  # 4 does not divide 1002
    (dict(k_full=384, ldx=384), B.TP_ERR_UNSUPPORTED),      # slice of 96 columns: not a multiple of 64
    (dict(ldx=1000), B.TP_ERR_INVALID_ARG),                  # ldx < k_full
    (dict(ldw=100), B.TP_ERR_INVALID_ARG),                   # ldw < slice width
    (dict(x=None), B.TP_ERR_INVALID_ARG),
    (dict(p=A3 + 4), B.TP_ERR_INVALID_ARG),
])
def test_split_input_validation(kw, status):
    assert split_input(**kw) == status
    assert tsl.tp_last_error().startswith("tp_linear_rowwise_split_input")


def qkv(**kw):
    a = dict(w=A, b=None, ws=A2, bs=None, H=24, hd=128, K=3072, dtype=B.TP_BF16, P=4, r=0,
             stream=None)
    a.update(kw)
    return _call("tp_fused_qkv_split", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(P=5), B.TP_ERR_NOT_DIVISIBLE),      # 5 does not divide 24 heads
    (dict(P=0), B.TP_ERR_INVALID_ARG),
    (dict(r=4), B.TP_ERR_INVALID_ARG),
    (dict(r=-1), B.TP_ERR_INVALID_ARG),
    (dict(H=0), B.TP_ERR_INVALID_ARG),
    (dict(b=A3), B.TP_ERR_INVALID_ARG),       # bias in without bias out
    (dict(w=None), B.TP_ERR_INVALID_ARG),
    (dict(dtype=9), B.TP_ERR_INVALID_ARG),
    (dict(H=1 << 20, hd=1 << 10, P=1), B.TP_ERR_UNSUPPORTED),  # 3 * 2^30 fused rows
])
def test_qkv_split_validation(kw, status):
    assert qkv(**kw) == status


def test_qkv_divisibility_matches_oracle():
    for heads in (1, 5, 6, 24, 48):
        for P in range(1, 10):
            st = qkv(H=heads, P=P, hd=2, K=8, w=None)  # null weight: only divisibility can pass first
            try:
                oracle.check_plan("qkv", P, 0, 3 * heads * 2, 8, num_heads=heads)
                want = B.TP_ERR_INVALID_ARG   # plan fine, then the null pointer is rejected
            except oracle.PlanError:
                want = B.TP_ERR_NOT_DIVISIBLE
            assert st == want, (heads, P)


def shape_query(o, i, style, P, r, blocks=None):
    return tsl.tp_plan_shard_shape(o, i, style, P, r, blocks)


def test_split_input_shard_shape_is_the_rowwise_shape():
    """[TP]: a rowwise_split_input weight is cut along the input features, like rowwise."""
    for o, i, P in [(36864, 6144, 4), (256, 1024, 2), (8, 12, 3)]:
        assert shape_query(o, i, "rowwise_split_input", P, P - 1) == shape_query(o, i, "rowwise", P, P - 1) \
            == (o, i // P)


@pytest.mark.parametrize("o,i,style,P,blocks", [
    (1024, 256, "colwise", 2, None), (256, 1024, "rowwise", 2, None),
    (9216, 3072, "colwise", 4, [1, 1, 1]), (18432, 6144, "colwise", 8, [1, 1, 1]),
    (6144, 18432, "rowwise", 8, None), (36864, 6144, "colwise", 4, None),
    (18, 4, "colwise", 2, [1, 1, 1, 3, 3]), (8, 4, "colwise", 4, [1, 3]),
    (8, 4, "colwise", 3, None), (4, 9, "rowwise", 2, None), (8, 4, "colwise", 1, [1, 1, 1]),
    (8, 6, "rowwise", 2, [1, 2]), (24, 8, "rowwise", 2, [1, 1, 1, 3, 3]),
])
def test_shard_shape_query_agrees_with_oracle_plan_rules(o, i, style, P, blocks):
    try:
        oracle.check_plan(style, P, 0, o, i, blocks=blocks)
        ok = True
    except oracle.PlanError:
        ok = False
    if ok:
        rows, cols = shape_query(o, i, style, P, 0, blocks)
        assert (rows, cols) == ((o // P, i) if style == "colwise" else (o, i // P))
    else:
        with pytest.raises(ValueError) as e:
            shape_query(o, i, style, P, 0, blocks)
        assert e.value.status == B.TP_ERR_NOT_DIVISIBLE


@pytest.mark.parametrize("args,status", [
    (dict(P=0), B.TP_ERR_INVALID_ARG), (dict(r=2), B.TP_ERR_INVALID_ARG),
    (dict(style=5), B.TP_ERR_INVALID_ARG), (dict(dtype=3), B.TP_ERR_INVALID_ARG),
    (dict(o=0), B.TP_ERR_INVALID_ARG), (dict(blocks=[0, 1]), B.TP_ERR_INVALID_ARG),
    (dict(blocks=[1] * 17), B.TP_ERR_INVALID_ARG),
    (dict(style=B.TP_ROWWISE, b=A3, bs=A3 + 64), B.TP_ERR_INVALID_ARG),
    (dict(style=B.TP_ROWWISE_SPLIT_INPUT, b=A3, bs=A3 + 64), B.TP_ERR_INVALID_ARG),
    (dict(style=B.TP_ROWWISE_SPLIT_INPUT, i=33), B.TP_ERR_NOT_DIVISIBLE),
    (dict(b=A3), B.TP_ERR_INVALID_ARG), (dict(w=None), B.TP_ERR_INVALID_ARG),
])
def test_shard_slice_validation(args, status):
    a = dict(w=A, b=None, ws=A2, bs=None, o=64, i=32, dtype=B.TP_BF16, style=B.TP_COLWISE,
             blocks=None, P=2, r=0)
    a.update(args)
    bl = a.pop("blocks")
    arr = None if bl is None else (ctypes.c_int64 * len(bl))(*bl)
    r_, c_ = ctypes.c_int64(), ctypes.c_int64()
    st = _call("tp_plan_shard_slice", a["w"], a["b"], a["ws"], a["bs"], a["o"], a["i"], a["dtype"],
               a["style"], arr, 0 if bl is None else len(bl), a["P"], a["r"], ctypes.byref(r_),
               ctypes.byref(c_), None)
    assert st == status


def combine(parts, mode=B.TP_COMBINE_SUM, **kw):
    a = dict(ld_part=256, out=A3, ld_out=256, in_dtype=B.TP_F32, out_dtype=B.TP_F32, mode=mode,
             bias=None, blocks=None, nb=0, M=64, n=256, stream=None)
    a.update(kw)
    arr = (ctypes.c_void_p * max(len(parts), 1))(*parts) if parts is not None else None
    bl = a.pop("blocks")
    blarr = None if bl is None else (ctypes.c_int64 * len(bl))(*bl)
    return _call("tp_partial_combine", arr, len(parts or []), a["ld_part"], a["out"], a["ld_out"],
                 a["in_dtype"], a["out_dtype"], a["mode"], a["bias"], blarr, a["nb"], a["M"], a["n"],
                 a["stream"])


def test_combine_validation():
    two = [A, A2]
    assert combine([]) == B.TP_ERR_INVALID_ARG
    assert combine([A] * 17) == B.TP_ERR_INVALID_ARG
    assert combine(two, in_dtype=B.TP_BF16) == B.TP_ERR_INVALID_ARG
    assert combine(two, ld_part=100) == B.TP_ERR_INVALID_ARG
    assert combine(two, ld_out=100) == B.TP_ERR_INVALID_ARG
    assert combine(two, blocks=[1], nb=1) == B.TP_ERR_INVALID_ARG
    assert combine([A, A2 + 4]) == B.TP_ERR_INVALID_ARG
    assert combine(two, out=A2) == B.TP_ERR_INVALID_ARG          # out aliases parts[1]
    assert combine(two, out=A, out_dtype=B.TP_BF16) == B.TP_ERR_INVALID_ARG  # bf16 in place
    assert combine(two, mode=9) == B.TP_ERR_INVALID_ARG
    assert combine(two, M=0) == B.TP_OK
    assert combine(two, ld_part=1 << 62) == B.TP_ERR_UNSUPPORTED
    assert combine(two, ld_out=1 << 62) == B.TP_ERR_UNSUPPORTED
    # concat
    cc = dict(mode=B.TP_COMBINE_CONCAT, in_dtype=B.TP_BF16, out_dtype=B.TP_BF16, ld_out=512)
    assert combine(two, **cc, M=0) == B.TP_OK
    assert combine(two, **dict(cc, out_dtype=B.TP_F32)) == B.TP_ERR_INVALID_ARG
    assert combine(two, **dict(cc, ld_out=500)) == B.TP_ERR_INVALID_ARG
    assert combine(two, **cc, bias=A3) == B.TP_ERR_INVALID_ARG
    # packed blocks: [1,3] over 512 columns with 2 parts -> 128 and 384, each divisible by 2: ok
    assert combine(two, **cc, blocks=[1, 3], nb=2, M=0) == B.TP_OK
    # [1,1,1] does not divide 512
    assert combine(two, **cc, blocks=[1, 1, 1], nb=3) == B.TP_ERR_NOT_DIVISIBLE
    # 4 parts of 2 columns: blocks [1,3] -> sizes 2 and 6, not divisible by 4
    assert combine([A] * 4, **dict(cc, ld_part=8, ld_out=8, n=2), blocks=[1, 3], nb=2) == \
        B.TP_ERR_NOT_DIVISIBLE


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        tsl.tp_linear_colwise(x, x)


def test_tile_shape_query():
    """The query names the kernel and tile each workload shape runs with.  Without a GPU the
    library assumes 256 compute units, MI355X's count."""
    q = tsl.tp_linear_tile_shape
    assert q(4, 9216, 6144) == (0, 0)                     # adaLN rows: weight-streaming kernel
    assert q(4, 9216, 6144, "swiglu") == (16, 12)         # no gated epilogue there: split-K kernel
    assert q(5, 9216, 6144) == (0, 0) and q(6, 9216, 6144) == (16, 36)   # skinny row limit: 5
    assert q(5, 9216, 4096) == (0, 0) and q(8, 9216, 4096) == (16, 36)
    assert q(2, 9216, 8192) == (0, 0) and q(3, 9216, 8192) == (16, 36)   # 16 chunks: 2 rows
    # split-K kernel: rows per workgroup balance the weight over the 256 CUs
    assert q(64, 9216, 6144) == (64, 36)                  # 256 workgroups of 36 rows
    assert q(64, 18432, 6144) == (64, 36)                 # 512: two per CU
    assert q(64, 4608, 6144) == (64, 20)                  # 231 workgroups
    assert q(64, 512, 256, "gelu_tanh") == (64, 4)        # the tiny MLP's colwise GEMM
    assert q(33, 2080, 128, "swiglu") == (48, 12)
    assert q(65, 9216, 6144) == (96, 36) and q(128, 9216, 6144) == (128, 36)
    assert q(129, 9216, 6144) == (64, 192)                # past 128 rows: tiled kernel, 64- and
    assert q(384, 9216, 6144) == (64, 256)                # 128-row tiles while they fill the CUs
    assert q(512, 9216, 6144) == (128, 192)               # better
    assert q(768, 9216, 6144) == (128, 256) and q(1024, 9216, 6144) == (224, 192)
    # launch sizes: a split-K launch has at most 2^23 workgroups of 256 threads, a tiled one at
    # most 2^22 tiles of 512 threads; past that the next kernel that fits takes the problem
    assert q(8, 48 << 23, 64) == (16, 48)
    assert q(8, (48 << 23) + 48, 64) == (64, 256) and q(8, 1 << 30, 64) == (64, 256)
    assert q(300, 3072, 128, "swiglu") == (192, 128)      # no 64-row SwiGLU tile
    assert q(4608, 2304, 6144) == (224, 192)              # 252 tiles, one round
    assert q(4608, 4608, 6144, "gelu_tanh") == (224, 192)  # 504 tiles, 1.97 rounds
    assert q(4608, 9216, 6144, "gelu_tanh") == (224, 256)  # 756 tiles in three rounds of 256
    assert q(4608, 6144, 768) == (224, 256)               # 504 tiles, 1.97 rounds
    assert q(4608, 6144, 128, "gelu_tanh") == (224, 256)
    assert q(2048, 6656, 128, "gelu_tanh") == (256, 256)  # 208 tiles, one round
    assert q(4608, 3072, 128, "swiglu") == (224, 128)     # 128 outputs per SwiGLU tile
    assert q(960, 6656, 128, "swiglu") == (256, 128)
    assert q(0, 16, 64)[0] in (0, 192, 224, 256)
    with pytest.raises(ValueError):
        q(-1, 16, 64)
    with pytest.raises(ValueError):
        q(16, 16, 64, "relu")
