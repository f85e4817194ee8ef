"""GPU parity of the colwise / rowwise GEMMs (tiled MFMA kernel, the split-K
kernel for up to 128 rows and the skinny weight-streaming kernel) against the
oracle, through the C ABI.

Ragged shapes span several tiles with partial tiles on both edges.  The
kernel picks its tile shape per problem (64, 128, 192, 224 or 256 rows by 192
or 256 columns, whichever needs the least time in rounds of tiles over the CUs;
tp_linear_tile_shape reports the choice); the 192- to 256-row tiles (SwiGLU
always) run on four waves, the 64- and 128-row tiles on eight.  On a 256-CU device the RAGGED shapes
with more than 128 rows and the first LARGE one run 64 x 192 tiles, the second
LARGE one 224 x 192; the RAGGED shapes with 16 to 64 rows take the split-K
kernel, those with 1 and 5 rows the weight-streaming kernel.  TALL runs
224 x 256 tiles (504 in two rounds), so its last tile row is ragged.  WIDE
runs 256 x 256 tiles (256 in one round).  test_gpu_tiles.py reaches every tile
shape with every epilogue.
Integer-valued inputs make every summation order exact, so there the GPU must
equal the oracle bit for bit, which pins operand layout and indexing; random
inputs are held to the stated tolerance and to the derived per-element bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import abs_dot, bits_to_dev, check_close, check_swiglu, dev_to_f64, sample_rows

pytestmark = pytest.mark.gpu

RAGGED = [(1, 16, 64), (17, 48, 128), (255, 272, 320), (257, 512, 256), (300, 784, 576),
          (64, 512, 256), (513, 256, 1024), (16, 1024, 192), (5, 80, 6144)]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_colwise_integer_inputs_exact(M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = si.int_bf16(rng, (M, K), -4, 4)
    w = si.int_bf16(rng, (N, K), -4, 4)
    b = si.int_bf16(rng, (N,), -8, 8)
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), out_dtype=torch.float32)
    ref = oracle.colwise(x, w, b)
    assert np.array_equal(dev_to_f64(y), ref)


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_rowwise_integer_inputs_exact(M, N, K):
    rng = np.random.default_rng(7 * M + N + K)
    P = 2
    x = si.int_bf16(rng, (M, 2 * K), -4, 4)
    w = si.int_bf16(rng, (N, 2 * K), -4, 4)
    xd, wd = bits_to_dev(x), bits_to_dev(w)
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise", P, r)
        p = tsl.tp_linear_rowwise(xd[:, r * K:(r + 1) * K], ws)  # strided input slice, ldx = 2K
        ref = oracle.rowwise(x, r, P, oracle.shard_rowwise(w, P, r))
        assert np.array_equal(dev_to_f64(p), ref)


@pytest.mark.parametrize("M,N,K", RAGGED)
@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
def test_colwise_random_bf16_out(M, N, K, act):
    rng = np.random.default_rng(3 * M + N + 5 * K)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act=act)
    a = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    ref = oracle.colwise(x, w, b, act=a)
    check_close(dev_to_f64(y), ref, K, True, S=abs_dot(x, w, b), what=f"colwise {M}x{N}x{K} {act}")


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_rowwise_random_f32_partial(M, N, K):
    rng = np.random.default_rng(11 * M + N + K)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    p = tsl.tp_linear_rowwise(bits_to_dev(x), bits_to_dev(w))
    ref = oracle.linear(x, w)
    check_close(dev_to_f64(p), ref, K, False, S=abs_dot(x, w), what=f"rowwise {M}x{N}x{K}")


def test_colwise_f32_out_with_gelu_and_padded_strides():
    rng = np.random.default_rng(99)
    M, N, K = 200, 96, 128
    xb = si.normal_bf16(rng, (M, K + 64))
    wb = si.normal_bf16(rng, (N, K + 32), 1 / np.sqrt(K))
    x = bits_to_dev(xb)[:, 64:]          # ldx = K + 64, offset 128 bytes
    w = bits_to_dev(wb)[:, :K]           # ldw = K + 32
    out_big = torch.full((M, N + 16), 7.0, dtype=torch.float32, device="cuda")
    out = out_big[:, :N]
    tsl.tp_linear_colwise(x, w, act="gelu_tanh", out=out)
    ref = oracle.colwise(np.ascontiguousarray(xb[:, 64:]), np.ascontiguousarray(wb[:, :K]),
                         act=oracle.ACT_GELU_TANH)
    check_close(dev_to_f64(out), ref, K, False, what="colwise f32 gelu strided")
    assert torch.all(out_big[:, N:] == 7.0)


def test_empty_m_is_noop():
    w = torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(0, 128, dtype=torch.bfloat16, device="cuda")
    y = tsl.tp_linear_colwise(x, w)
    assert y.shape == (0, 64)
    p = tsl.tp_linear_rowwise(x, w)
    assert p.shape == (0, 64)


@pytest.mark.parametrize("P", [2, 4])
def test_concat_of_colwise_shards_equals_unsharded_gpu(P):
    """[TP] opening definition, on the GPU alone: the colwise shards' outputs, gathered,
    equal the unsharded layer bit for bit (each output element's arithmetic does not
    depend on the sharding)."""
    rng = np.random.default_rng(P)
    M, N, K = 600, 1024, 512
    x = bits_to_dev(si.normal_bf16(rng, (M, K)))
    w = bits_to_dev(si.normal_bf16(rng, (N, K), 1 / np.sqrt(K)))
    b = bits_to_dev(si.normal_bf16(rng, (N,)))
    full = tsl.tp_linear_colwise(x, w, b, act="gelu_tanh")
    outs = []
    for r in range(P):
        ws, bs = tsl.tp_plan_shard_slice(w, b, "colwise", P, r)
        outs.append(tsl.tp_linear_colwise(x, ws, bs, act="gelu_tanh"))
    cat = tsl.tp_partial_combine(outs, "concat")
    assert torch.equal(cat.view(torch.int16), full.view(torch.int16))


def test_repeat_runs_are_bitwise_identical():
    rng = np.random.default_rng(5)
    M, N, K = 700, 512, 768
    x = bits_to_dev(si.normal_bf16(rng, (M, K)))
    w = bits_to_dev(si.normal_bf16(rng, (N, K), 1 / np.sqrt(K)))
    a = tsl.tp_linear_rowwise(x, w)
    b = tsl.tp_linear_rowwise(x, w)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 7, 8, 16])
@pytest.mark.parametrize("act,bias", [("none", False), ("gelu_tanh", True)])
def test_skinny_path_random(B, act, bias):
    rng = np.random.default_rng(B)
    N, K = 528, 1536
    c = si.normal_bf16(rng, (B, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    bb = si.normal_bf16(rng, (N,)) if bias else None
    y = tsl.tp_linear_colwise(bits_to_dev(c), bits_to_dev(w), bits_to_dev(bb) if bias else None, act=act)
    a = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    ref = oracle.colwise(c, w, bb, act=a)
    check_close(dev_to_f64(y), ref, K, True, S=abs_dot(c, w, bb), what=f"skinny B={B}")


@pytest.mark.parametrize("B", [1, 4, 16])
def test_skinny_path_integer_exact(B):
    rng = np.random.default_rng(40 + B)
    N, K = 272, 2048
    c = si.int_bf16(rng, (B, K), -4, 4)
    w = si.int_bf16(rng, (N, K), -4, 4)
    y = tsl.tp_linear_colwise(bits_to_dev(c), bits_to_dev(w), out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.colwise(c, w))
    p = tsl.tp_linear_rowwise(bits_to_dev(c), bits_to_dev(w))
    assert np.array_equal(dev_to_f64(p), oracle.linear(c, w))


@pytest.mark.parametrize("K", [6144, 5696])
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_skinny_adaln_width_exact(B, K):
    """The adaLN width: K in (4096, 6144] is 12 chunks per lane, and K = 5696
    leaves lanes past the row end.  Integer inputs: exact, with bias."""
    rng = np.random.default_rng(60 + B + K)
    N = 400
    c = si.int_bf16(rng, (B, K), -2, 2)
    w = si.int_bf16(rng, (N, K), -2, 2)
    b = si.int_bf16(rng, (N,), -8, 8)
    y = tsl.tp_linear_colwise(bits_to_dev(c), bits_to_dev(w), bits_to_dev(b), out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.colwise(c, w, b))


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_skinny_adaln_width_random_gelu(B):
    rng = np.random.default_rng(70 + B)
    N, K = 528, 6144
    c = si.normal_bf16(rng, (B, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    bb = si.normal_bf16(rng, (N,))
    y = tsl.tp_linear_colwise(bits_to_dev(c), bits_to_dev(w), bits_to_dev(bb), act="gelu_tanh")
    ref = oracle.colwise(c, w, bb, act=oracle.ACT_GELU_TANH)
    check_close(dev_to_f64(y), ref, K, True, S=abs_dot(c, w, bb), what=f"skinny adaLN width B={B}")


# Larger shapes: 1100 x 1040 x 2048 is ragged on both edges of a 5 x 5 tile
# grid with 32 k-tiles; 4608 x 2304 x 3072 is a full-size rowwise shard.
LARGE_SHAPES = [(1100, 1040, 2048), (4608, 2304, 3072)]


@pytest.mark.parametrize("M,N,K", LARGE_SHAPES)
def test_large_integer_inputs_exact(M, N, K):
    rng = np.random.default_rng(M + K)
    x = si.int_bf16(rng, (M, K), -4, 4)
    w = si.int_bf16(rng, (N, K), -4, 4)
    p = tsl.tp_linear_rowwise(bits_to_dev(x), bits_to_dev(w))
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    ref = oracle.linear(x, w, rows=rows)
    assert np.array_equal(dev_to_f64(p)[rows], ref)
    # every output element, against an exact integer product on the host
    xi = torch.from_numpy(oracle.bf16_widen(x)).to(torch.float64)
    wi = torch.from_numpy(oracle.bf16_widen(w)).to(torch.float64)
    assert torch.equal(p.cpu().to(torch.float64), xi @ wi.T)


@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
def test_large_random_vs_oracle(act):
    M, N, K = LARGE_SHAPES[0]
    rng = np.random.default_rng(17)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act=act)
    rows = np.unique(np.concatenate([np.arange(0, M, 37), [M - 1, 255, 256, 511, 512]]))
    a = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    ref = oracle.colwise(x, w, b, act=a, rows=rows)
    check_close(dev_to_f64(y)[rows], ref, K, True, S=abs_dot(x[rows], w, b), what=f"large colwise {act}")


def test_large_repeat_runs_and_output_dtypes_agree():
    M, N, K = LARGE_SHAPES[1]
    rng = np.random.default_rng(23)
    x = bits_to_dev(si.normal_bf16(rng, (M, K)))
    w = bits_to_dev(si.normal_bf16(rng, (N, K), 1 / np.sqrt(K)))
    a = tsl.tp_linear_rowwise(x, w)
    b = tsl.tp_linear_rowwise(x, w)
    c = tsl.tp_linear_colwise(x, w, out_dtype=torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


TALL = (4600, 6128, 3072)


def test_tall_integer_inputs_exact():
    M, N, K = TALL
    rng = np.random.default_rng(31)
    x = si.int_bf16(rng, (M, K), -4, 4)
    w = si.int_bf16(rng, (N, K), -4, 4)
    b = si.int_bf16(rng, (N,), -8, 8)
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), out_dtype=torch.float32)
    rows = np.unique(np.concatenate([np.arange(0, M, 211), [223, 224, 255, 256, 4479, 4480, M - 1]]))
    assert np.array_equal(dev_to_f64(y)[rows], oracle.colwise(x, w, b, rows=rows))
    xi = torch.from_numpy(oracle.bf16_widen(x)).to(torch.float64)
    wi = torch.from_numpy(oracle.bf16_widen(w)).to(torch.float64)
    bi = torch.from_numpy(oracle.bf16_widen(b)).to(torch.float64)
    assert torch.equal(y.cpu().to(torch.float64), xi @ wi.T + bi)


WIDE = (2040, 8176, 128)


def test_wide_integer_inputs_exact():
    M, N, K = WIDE
    rng = np.random.default_rng(41)
    x = si.int_bf16(rng, (M, K), -4, 4)
    w = si.int_bf16(rng, (N, K), -4, 4)
    p = tsl.tp_linear_rowwise(bits_to_dev(x), bits_to_dev(w))
    xi = torch.from_numpy(oracle.bf16_widen(x)).to(torch.float64)
    wi = torch.from_numpy(oracle.bf16_widen(w)).to(torch.float64)
    assert torch.equal(p.cpu().to(torch.float64), xi @ wi.T)
    rows = np.unique(np.concatenate([np.arange(0, M, 173), [255, 256, 1791, 1792, M - 1]]))
    assert np.array_equal(dev_to_f64(p)[rows], oracle.linear(x, w, rows=rows))


def test_wide_random_gelu_vs_oracle():
    M, N, K = WIDE
    rng = np.random.default_rng(43)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act="gelu_tanh")
    rows = np.unique(np.concatenate([np.arange(0, M, 131), [255, 256, 1791, 1792, M - 1]]))
    ref = oracle.colwise(x, w, b, act=oracle.ACT_GELU_TANH, rows=rows)
    check_close(dev_to_f64(y)[rows], ref, K, True, S=abs_dot(x[rows], w, b), what="wide colwise gelu")


def test_tall_random_gelu_vs_oracle():
    M, N, K = TALL
    rng = np.random.default_rng(37)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act="gelu_tanh")
    rows = np.unique(np.concatenate([np.arange(0, M, 149), [223, 224, 255, 256, 4351, 4352, 4479, 4480, M - 1]]))
    ref = oracle.colwise(x, w, b, act=oracle.ACT_GELU_TANH, rows=rows)
    check_close(dev_to_f64(y)[rows], ref, K, True, S=abs_dot(x[rows], w, b), what="tall colwise gelu")


@pytest.mark.parametrize("K", [512, 576, 1600, 4160])
def test_skinny_path_reads_only_its_staged_rows(K):
    """Lanes past the end of a row pair the weight's last chunk with their
    activation row's zero chunk.  A tiled GEMM on 1e30-valued operands runs first
    so that LDS holds huge stale values on every CU: a read outside the staged
    rows would turn into inf or a wrong sum.  K is chosen so that every case has
    lanes past the row end (K not a multiple of 512, or fewer chunks than the
    kernel's chunk count)."""
    big = torch.full((4096, 128), 1e30, dtype=torch.bfloat16, device="cuda")
    tsl.tp_linear_colwise(big, big, out_dtype=torch.float32)
    rng = np.random.default_rng(K)
    N = 272
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    wd = bits_to_dev(w)
    for B in range(1, 9):
        c = si.normal_bf16(rng, (B, K))
        y = tsl.tp_linear_colwise(bits_to_dev(c), wd, out_dtype=torch.float32)
        check_close(dev_to_f64(y), oracle.colwise(c, w), K, False, S=abs_dot(c, w), what=f"skinny K={K} B={B}")


@pytest.mark.parametrize("K", [448, 768, 1536, 2560, 3072, 3584, 4096, 6656, 8192])
def test_skinny_every_chunk_count_exact(K):
    """One K per chunk-count instance of the skinny kernel (1, 2, 3, 6, 8, 16 chunks per lane,
    full and partial), every row count the kernel takes at that K, integer inputs with bias:
    exact.  N = 2 x 2048 + 16 leaves each wave two or three rows (the peeled last rows)."""
    rng = np.random.default_rng(90 + K)
    N = 2 * 2048 + 16
    w = si.int_bf16(rng, (N, K), -2, 2)
    b = si.int_bf16(rng, (N,), -8, 8)
    wd, bd = bits_to_dev(w), bits_to_dev(b)
    for B in range(1, 9):
        if tsl.tp_linear_tile_shape(B, N, K) != (0, 0):
            break                                  # past the kernel's row limit at this K
        c = si.int_bf16(rng, (B, K), -2, 2)
        y = tsl.tp_linear_colwise(bits_to_dev(c), wd, bd, out_dtype=torch.float32)
        assert np.array_equal(dev_to_f64(y), oracle.colwise(c, w, b)), (K, B)
    assert B >= 2


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_skinny_adaln_shard_gelu_bias(B):
    """The adaLN shard at tp 4 (9216 x 6144: 4.5 weight rows per wave, so rows are dealt
    wave-major), random operands, bias and GELU, bf16 output, against the oracle on a sample
    of weight rows: every 7th, the rows around 8192 where some waves' fifth rows begin, and
    the last."""
    rng = np.random.default_rng(80 + B)
    N, K = 9216, 6144
    c = si.normal_bf16(rng, (B, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    bb = si.normal_bf16(rng, (N,))
    y = dev_to_f64(tsl.tp_linear_colwise(bits_to_dev(c), bits_to_dev(w), bits_to_dev(bb), act="gelu_tanh"))
    cols = np.unique(np.concatenate([np.arange(0, N, 7), np.arange(8 * 1024 - 8, 8 * 1024 + 8), [N - 1]]))
    ref = oracle.colwise(c, w[cols], bb[cols], act=oracle.ACT_GELU_TANH)
    check_close(y[:, cols], ref, K, True, S=abs_dot(c, w[cols], bb[cols]), what=f"adaLN shard B={B}")


@pytest.mark.parametrize("N", [16, 304, 2048, 2064, 3 * 2048 - 16, 5 * 2048 + 1008])
def test_skinny_rows_per_wave(N):
    """Rows per wave from one (a grid smaller than the chip) to six, so that every peeled ending
    of the row loop runs (2048 waves for N >= 2048)."""
    rng = np.random.default_rng(N)
    K = 1024
    w = si.int_bf16(rng, (N, K), -2, 2)
    b = si.int_bf16(rng, (N,), -8, 8)
    for B in (1, 4):
        c = si.int_bf16(rng, (B, K), -2, 2)
        y = tsl.tp_linear_colwise(bits_to_dev(c), bits_to_dev(w), bits_to_dev(b), out_dtype=torch.float32)
        assert np.array_equal(dev_to_f64(y), oracle.colwise(c, w, b)), (N, B)


# 256-row tiles: the no-bias GELU and SwiGLU epilogues at the largest register footprint of
# the four-wave kernel.  Sampled rows
# against the oracle include every tile edge; the whole tensor must equal the same call with
# an all-zero bias (another kernel instance, the same arithmetic per element).
TALL256 = (2048, 6656, 128)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gelu_no_bias_256_row_tiles(out):
    M, N, K = TALL256
    assert tsl.tp_linear_tile_shape(M, N, K, "gelu_tanh") == (256, 256)
    rng = np.random.default_rng(41)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    xd, wd = bits_to_dev(x), bits_to_dev(w)
    y = tsl.tp_linear_colwise(xd, wd, act="gelu_tanh", out_dtype=dt)
    rows = sample_rows(M, 32, seed=41, tile=256)
    ref = oracle.colwise(x, w, None, act=oracle.ACT_GELU_TANH, rows=rows)
    check_close(dev_to_f64(y[torch.from_numpy(rows).cuda()]), ref, K, out == "bf16",
                S=abs_dot(x[rows], w), what=f"gelu no bias 256-row tiles {out}")
    y0 = tsl.tp_linear_colwise(xd, wd, torch.zeros(N, dtype=torch.bfloat16, device="cuda"),
                               act="gelu_tanh", out_dtype=dt)
    assert torch.equal(y, y0)


def test_swiglu_no_bias_256_row_tiles():
    M, n, K = 960, 6656, 128
    assert tsl.tp_linear_tile_shape(M, n, K, "swiglu") == (256, 128)
    rng = np.random.default_rng(42)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (2 * n, K), 1 / np.sqrt(K))
    xd, wd = bits_to_dev(x), bits_to_dev(w)
    y = tsl.tp_linear_colwise(xd, wd, act="swiglu")
    rows = sample_rows(M, 32, seed=42, tile=256)
    check_swiglu(dev_to_f64(y[torch.from_numpy(rows).cuda()]), x, w, None, True, rows=rows,
                 what="swiglu no bias 256-row tiles")
    y0 = tsl.tp_linear_colwise(xd, wd, torch.zeros(2 * n, dtype=torch.bfloat16, device="cuda"), act="swiglu")
    assert torch.equal(y, y0)
