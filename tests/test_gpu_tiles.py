"""Every tile shape of the tiled GEMM with every epilogue, through the C ABI.

The tiled kernel has one instance per tile shape (192, 224 or 256 rows by 192
or 256 columns, and 64 or 128 rows by 192 or 256 columns for the plain
epilogues;
SwiGLU always 256 weight rows = 128 outputs), output dtype,
bias or not, and epilogue.  For each shape the library can choose, a problem
that gets it is found with tp_linear_tile_shape (on the device that runs the
test, whose compute-unit count the choice depends on), and every instance of
that shape is checked:

* against the oracle on sampled rows: rows 0, 1, M - 1, both rows at every
  tile edge, seeded random rows, all columns (so every column tile edge);
* on the whole tensor's first 160 rows, bit for bit, against the same call on
  those rows alone, which usually runs another tile shape: each output element
  sees the same products in the same order whatever the tile (no split-K).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import abs_dot, bits_to_dev, check_close, check_swiglu, dev_to_f64, sample_rows

pytestmark = pytest.mark.gpu

SHAPES = [(r, c) for r in (256, 224, 192, 128, 64) for c in (256, 192)]
SUB_ROWS = 160


def find_problem(rows, cols, act):
    """The cheapest (M, N, K) of a small grid that runs a rows x cols tile, with at least
    two tiles each way (so the problem has inner tile edges)."""
    best = None
    for K in (64, 3072):
        for M in (192, 224, 256, 300, 448, 672, 1000, 1344, 2048, 3072, 4608):
            for N in (192, 256, 384, 576, 768, 1152, 1536, 2304, 3072, 4608, 4864, 6144, 6656):
                if M >= 2 * rows and N >= 2 * cols and tsl.tp_linear_tile_shape(M, N, K, act) == (rows, cols):
                    cost = M * N * K
                    if best is None or cost < best[0]:
                        best = (cost, (M, N, K))
    return None if best is None else best[1]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_every_tile_shape_every_epilogue(rows, cols):
    prob = find_problem(rows, cols, "none")
    assert prob is not None, f"no problem in the search grid runs a {rows} x {cols} tile"
    M, N, K = prob
    rng = np.random.default_rng(rows * 1000 + cols)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    xd, wd, bd = bits_to_dev(x), bits_to_dev(w), bits_to_dev(b)
    srows = sample_rows(M, 8, seed=rows + cols, tile=rows)
    idx = torch.from_numpy(srows).cuda()
    for act, out, bias in itertools.product(("none", "gelu_tanh"), (torch.bfloat16, torch.float32), (False, True)):
        assert tsl.tp_linear_tile_shape(M, N, K, act) == (rows, cols)
        what = f"{rows}x{cols} tile, {M}x{N}x{K} {act} {out} bias={bias}"
        y = tsl.tp_linear_colwise(xd, wd, bd if bias else None, act=act, out_dtype=out)
        a = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
        ref = oracle.colwise(x, w, b if bias else None, act=a, rows=srows)
        check_close(dev_to_f64(y[idx]), ref, K, out == torch.bfloat16,
                    S=abs_dot(x[srows], w, b if bias else None), what=what)
        y_sub = tsl.tp_linear_colwise(xd[:SUB_ROWS], wd, bd if bias else None, act=act, out_dtype=out)
        assert torch.equal(y[:SUB_ROWS], y_sub), what + ": differs from the same rows computed alone"


@pytest.mark.parametrize("rows", [256, 224, 192])
def test_every_swiglu_tile_height(rows):
    prob = find_problem(rows, 128, "swiglu")
    assert prob is not None, f"no problem in the search grid runs a {rows}-row SwiGLU tile"
    M, n, K = prob
    rng = np.random.default_rng(rows + 7)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (2 * n, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (2 * n,))
    xd, wd, bd = bits_to_dev(x), bits_to_dev(w), bits_to_dev(b)
    srows = sample_rows(M, 8, seed=rows, tile=rows)
    idx = torch.from_numpy(srows).cuda()
    for out, bias in itertools.product((torch.bfloat16, torch.float32), (False, True)):
        what = f"SwiGLU {rows}-row tile, {M}x{n}x{K} {out} bias={bias}"
        y = tsl.tp_linear_colwise(xd, wd, bd if bias else None, act="swiglu", out_dtype=out)
        check_swiglu(dev_to_f64(y[idx]), x, w, b if bias else None, out == torch.bfloat16, rows=srows, what=what)
        y_sub = tsl.tp_linear_colwise(xd[:SUB_ROWS], wd, bd if bias else None, act="swiglu", out_dtype=out)
        assert torch.equal(y[:SUB_ROWS], y_sub), what + ": differs from the same rows computed alone"


# The 64- and 128-row tiles keep several k-tiles in flight (4 stages for 64 x 192, 3 for the
# others) when K has at least that many k-tiles, and double buffer below that.  These
# problems run each of them at 3, 4, 5 and 25 k-tiles: the double-buffered path, exactly the
# stage count (every load issued before the loop), one more, and a long loop whose last
# iterations wait for everything.
MULTISTAGE = [((64, 192), 136, 1024), ((64, 256), 328, 8192), ((128, 192), 648, 6144), ((128, 256), 648, 8192)]


@pytest.mark.parametrize("tile,M,N", MULTISTAGE)
@pytest.mark.parametrize("K", [192, 256, 320, 1600])
def test_multistage_tiles_integer_exact(tile, M, N, K):
    if tsl.tp_linear_tile_shape(M, N, K) != tile:
        pytest.skip(f"{M}x{N}x{K} takes another tile on this device's CU count")
    rng = np.random.default_rng(tile[0] + tile[1] + K)
    x = si.int_bf16(rng, (M, K), -3, 3)
    w = si.int_bf16(rng, (N, K), -3, 3)
    b = si.int_bf16(rng, (N,), -8, 8)
    xd, wd, bd = bits_to_dev(x), bits_to_dev(w), bits_to_dev(b)
    y = tsl.tp_linear_colwise(xd, wd, bd, out_dtype=torch.float32)
    srows = sample_rows(M, 8, seed=K, tile=tile[0])
    idx = torch.from_numpy(srows).cuda()
    assert np.array_equal(dev_to_f64(y[idx]), oracle.colwise(x, w, b, rows=srows))
    y_sub = tsl.tp_linear_colwise(xd[:SUB_ROWS], wd, bd, out_dtype=torch.float32)
    assert torch.equal(y[:SUB_ROWS], y_sub)
    p = tsl.tp_linear_rowwise(xd, wd)
    assert np.array_equal(dev_to_f64(p[idx]), oracle.colwise(x, w, rows=srows))


FOUR_WAVE = [(256, 256), (224, 256), (192, 256), (256, 192), (224, 192), (192, 192)]


@pytest.mark.parametrize("rows,cols", FOUR_WAVE)
def test_four_wave_tiles_every_k_tile_count(rows, cols):
    """The 192- to 256-row tiles of the plain, bias and GELU epilogues run on four waves, one
    per SIMD, whose pipeline has a prologue, a steady loop that loads the k-tile after next,
    a loop for the last k-tiles and a final k32 step.  1, 2, 3, 5 and 20 k-tiles reach every
    part.  Integer-valued operands make every summation order exact, so the output equals
    the oracle bit for bit (bf16 output: the exact value rounded once), with and without
    bias, on sampled rows (both rows of every tile edge) and all columns; M and N are ragged,
    so the last tile row and column are partial.  GELU is checked on random normal operands
    (where the stated tolerance applies) at 20 k-tiles."""
    M, N, _ = find_problem(rows, cols, "none")
    M, N = M - 3, N - 16
    rng = np.random.default_rng(rows * 7 + cols)
    srows = sample_rows(M, 8, seed=rows * cols, tile=rows)
    idx = torch.from_numpy(srows).cuda()
    for K in (64, 128, 192, 320, 1280):
        assert tsl.tp_linear_tile_shape(M, N, K) == (rows, cols)
        x = si.int_bf16(rng, (M, K), -4, 4)
        w = si.int_bf16(rng, (N, K), -4, 4)
        b = si.int_bf16(rng, (N,), -8, 8)
        xd, wd, bd = bits_to_dev(x), bits_to_dev(w), bits_to_dev(b)
        for bias in (False, True):
            ref = oracle.colwise(x, w, b if bias else None, rows=srows)
            what = f"{rows}x{cols} tile, {M}x{N}x{K} bias={bias}"
            y32 = tsl.tp_linear_colwise(xd, wd, bd if bias else None, out_dtype=torch.float32)
            assert np.array_equal(dev_to_f64(y32[idx]), ref), what + " fp32 out"
            y16 = tsl.tp_linear_colwise(xd, wd, bd if bias else None)
            assert np.array_equal(dev_to_f64(y16[idx]), oracle.bf16_widen(oracle.bf16_round(ref))), what + " bf16 out"
        if K == 1280:
            x = si.normal_bf16(rng, (M, K))
            w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
            b = si.normal_bf16(rng, (N,))
            yg = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act="gelu_tanh")
            refg = oracle.colwise(x, w, b, act=oracle.ACT_GELU_TANH, rows=srows)
            check_close(dev_to_f64(yg[idx]), refg, K, True, S=abs_dot(x[srows], w, b),
                        what=f"{rows}x{cols} tile, {M}x{N}x{K} GELU")
