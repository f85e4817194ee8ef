"""GPU parity of the split-K MFMA kernel that runs linear layers with few rows
(up to 128, beyond the weight-streaming kernel's row limit) against the oracle,
through the C ABI.

The kernel gives each workgroup all M rows (16-row MFMA blocks, the last one
partial) and a run of output columns (weight rows) that the host sizes to
balance the CUs: a multiple of 4, at most 48 (one to three 16-row weight blocks,
the last one partial) or 16 with SwiGLU, the last workgroup's run shorter when
it does not divide N.  K is dealt over the 4 waves in 64-element steps
(unevenly when 4 does not divide them, none at all for some waves when K = 64),
and the 4 partial sums are added in wave order.  The shapes below reach every
row-block count with full and partial last blocks, runs of one, two and three
weight blocks with and without a shorter last run, all three epilogues, both
output types and strided operands.  Integer-valued inputs make every summation order exact:
the GPU must equal the oracle bit for bit, which pins operand layout and
indexing.  Random inputs are held to the stated tolerance and the derived
per-element bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import abs_dot, bits_to_dev, check_close, check_swiglu, dev_to_f64

pytestmark = pytest.mark.gpu

ROWS = [9, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 80, 96, 97, 112, 127, 128]
SHAPES = [(16, 64), (48, 192), (2064, 448), (304, 6144)]


def _row_blocks(M):
    """16-row blocks of the kernel instance for M rows: 1-4, then 6 and 8."""
    mb = (M + 15) // 16
    return {5: 6, 7: 8}.get(mb, mb)


def _narrow(M, N, K, act="none"):
    rows, cols = tsl.tp_linear_tile_shape(M, N, K, act=act)
    return rows == 16 * _row_blocks(M) and cols % 4 == 0 and 4 <= cols <= (16 if act == "swiglu" else 48)


# (N, weight rows per workgroup on 256 CUs at K = 128): one, two and three 16-row weight
# blocks per workgroup, each with N a multiple of the run and not.
RUNS = [(2080, 12), (4160, 20), (4112, 20), (8208, 36), (8224, 36)]


@pytest.mark.parametrize("M", [9, 40, 64, 80, 100, 128])
@pytest.mark.parametrize("N,run", RUNS)
def test_narrow_balanced_runs_integer_exact(M, N, run):
    rng = np.random.default_rng(1500 + M + N)
    K = 128
    x = si.int_bf16(rng, (M, K), -3, 3)
    w = si.int_bf16(rng, (N, K), -3, 3)
    b = si.int_bf16(rng, (N,), -8, 8)
    rows, cols = tsl.tp_linear_tile_shape(M, N, K)
    assert rows == 16 * _row_blocks(M)
    if tsl.tp_linear_tile_shape(4608, 2304, 6144) == (224, 192):   # 256 CUs: the runs listed
        assert cols == run
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act="gelu_tanh",
                              out_dtype=torch.float32)
    check_close(dev_to_f64(y), oracle.colwise(x, w, b, act=oracle.ACT_GELU_TANH), K, False,
                S=abs_dot(x, w, b), what=f"narrow run {M}x{N}")
    p = tsl.tp_linear_rowwise(bits_to_dev(x), bits_to_dev(w))
    assert np.array_equal(dev_to_f64(p), oracle.linear(x, w))


@pytest.mark.parametrize("M", ROWS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_narrow_integer_inputs_exact(M, N, K):
    rng = np.random.default_rng(1000 + M + N + K)
    x = si.int_bf16(rng, (M, K), -3, 3)
    w = si.int_bf16(rng, (N, K), -3, 3)
    b = si.int_bf16(rng, (N,), -8, 8)
    assert _narrow(M, N, K)
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.colwise(x, w, b))


@pytest.mark.parametrize("M", [6, 7, 8, 20, 64])
def test_narrow_rows_past_the_weight_streaming_limit(M):
    """K = 6144: the weight-streaming kernel takes at most 5 rows; from 6 rows on the
    split-K kernel runs (integer inputs, bf16 output: exact after rounding)."""
    rng = np.random.default_rng(2000 + M)
    N, K = 2064, 6144
    x = si.int_bf16(rng, (M, K), -2, 2)
    w = si.int_bf16(rng, (N, K), -2, 2)
    assert _narrow(M, N, K)
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w))
    ref = oracle.colwise(x, w)
    assert np.array_equal(dev_to_f64(y), oracle.bf16_widen(oracle.bf16_round(ref)))


@pytest.mark.parametrize("M", [9, 33, 64, 90, 128])
@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
def test_narrow_random_bf16_out(M, act):
    rng = np.random.default_rng(3000 + M)
    N, K = 2064, 1536
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act=act)
    a = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    check_close(dev_to_f64(y), oracle.colwise(x, w, b, act=a), K, True, S=abs_dot(x, w, b),
                what=f"narrow {M}x{N}x{K} {act}")


@pytest.mark.parametrize("M", [17, 64])
def test_narrow_gelu_f32_out_no_bias(M):
    rng = np.random.default_rng(3500 + M)
    N, K = 304, 448
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), act="gelu_tanh", out_dtype=torch.float32)
    check_close(dev_to_f64(y), oracle.colwise(x, w, act=oracle.ACT_GELU_TANH), K, False, S=abs_dot(x, w),
                what=f"narrow gelu f32 {M}")


@pytest.mark.parametrize("M", [9, 40, 64, 111])
def test_narrow_rowwise_strided_slices_exact(M):
    """Rowwise partials from column slices of the activation (ldx = 2 K) on
    integer inputs: exact."""
    rng = np.random.default_rng(4000 + M)
    N, K, P = 784, 576, 2
    x = si.int_bf16(rng, (M, P * K), -4, 4)
    w = si.int_bf16(rng, (N, P * K), -4, 4)
    xd, wd = bits_to_dev(x), bits_to_dev(w)
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise", P, r)
        assert _narrow(M, N, K)
        p = tsl.tp_linear_rowwise(xd[:, r * K:(r + 1) * K], ws)
        assert np.array_equal(dev_to_f64(p), oracle.rowwise(x, r, P, oracle.shard_rowwise(w, P, r)))


@pytest.mark.parametrize("M", [9, 33, 64, 128])
@pytest.mark.parametrize("bias,out", [(False, "bf16"), (True, "bf16"), (True, "f32")])
def test_narrow_swiglu_vs_oracle(M, bias, out):
    rng = np.random.default_rng(5000 + M)
    n, K = 272, 1024
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (2 * n, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (2 * n,)) if bias else None
    assert _narrow(M, n, K, act="swiglu")
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b) if bias else None,
                              act="swiglu", out_dtype=dt)
    assert tuple(y.shape) == (M, n)
    check_swiglu(dev_to_f64(y), x, w, b, out == "bf16", what=f"narrow swiglu {M} bias={bias} {out}")


@pytest.mark.parametrize("M", [9, 64, 81])
def test_narrow_swiglu_ragged_runs(M):
    """2080 outputs: 12 gate rows and 12 up rows per workgroup, the last run shorter."""
    rng = np.random.default_rng(5200 + M)
    n, K = 2080, 192
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (2 * n, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (2 * n,))
    assert _narrow(M, n, K, act="swiglu")
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), act="swiglu")
    check_swiglu(dev_to_f64(y), x, w, b, True, what=f"narrow swiglu runs {M}")


def test_narrow_swiglu_saturated_gate_exact():
    """Gate pre-activations >= 64: silu(g) = g in fp32, so the fp32 output is exactly
    g * u; the gate and up rows must not be swapped or misaligned."""
    rng = np.random.default_rng(5500)
    M, n, K = 33, 272, 64
    x = si.int_bf16(rng, (M, K), 1, 3)
    g = si.int_bf16(rng, (n, K), 1, 4)
    u = si.int_bf16(rng, (n, K), -4, 4)
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(np.concatenate([g, u])), act="swiglu",
                              out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.linear(x, g) * oracle.linear(x, u))


@pytest.mark.parametrize("P,M", [(2, 48), (4, 48), (4, 120)])
def test_narrow_concat_of_shards_equals_unsharded(P, M):
    """Each output is the same sum whatever N and the run length are: the shards' outputs
    placed side by side equal the unsharded product bit for bit (random inputs)."""
    rng = np.random.default_rng(6000 + P + M)
    N, K = 1024, 768
    x = bits_to_dev(si.normal_bf16(rng, (M, K)))
    w = bits_to_dev(si.normal_bf16(rng, (N, K), 1 / np.sqrt(K)))
    b = bits_to_dev(si.normal_bf16(rng, (N,)))
    full = tsl.tp_linear_colwise(x, w, b, act="gelu_tanh")
    parts = []
    for r in range(P):
        ws, bs = tsl.tp_plan_shard_slice(w, b, "colwise", P, r)
        parts.append(tsl.tp_linear_colwise(x, ws, bs, act="gelu_tanh"))
    assert torch.equal(torch.cat(parts, dim=1), full)


def test_narrow_output_view_and_padded_strides():
    """Operands and output with row strides wider than their rows: the columns
    around the output view keep their values."""
    rng = np.random.default_rng(6500)
    M, N, K = 40, 208, 320
    xb = si.int_bf16(rng, (M, K + 64), -3, 3)
    wb = si.int_bf16(rng, (N, K + 32), -3, 3)
    x = bits_to_dev(xb)[:, 64:]
    w = bits_to_dev(wb)[:, :K]
    big = torch.full((M, N + 48), 7.0, dtype=torch.float32, device="cuda")
    tsl.tp_linear_colwise(x, w, out=big[:, 16:16 + N])
    ref = oracle.linear(xb[:, 64:], wb[:, :K])
    got = dev_to_f64(big)
    assert np.array_equal(got[:, 16:16 + N], ref)
    assert np.all(got[:, :16] == 7.0) and np.all(got[:, 16 + N:] == 7.0)


@pytest.mark.parametrize("M", [64, 128])
def test_narrow_adaln_width_random_vs_oracle(M):
    """64 and 128 rows against the adaLN shard's width (9216 x 6144, 113 MB of weight):
    every output against the oracle."""
    rng = np.random.default_rng(7000 + M)
    N, K = 9216, 6144
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    assert _narrow(M, N, K)
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b))
    check_close(dev_to_f64(y), oracle.colwise(x, w, b), K, True, S=abs_dot(x, w, b), what="narrow adaLN width")


def test_narrow_repeat_runs_are_bitwise_identical():
    rng = np.random.default_rng(7500)
    M, N, K = 33, 2064, 2048
    x = bits_to_dev(si.normal_bf16(rng, (M, K)))
    w = bits_to_dev(si.normal_bf16(rng, (N, K), 1 / np.sqrt(K)))
    y0 = tsl.tp_linear_rowwise(x, w)
    for _ in range(3):
        assert torch.equal(tsl.tp_linear_rowwise(x, w), y0)


@pytest.mark.parametrize("M", [5, 6, 128, 129])
def test_kernel_boundaries_integer_exact(M):
    """Both sides of each boundary between the three GEMM kernels: 5 rows take the
    weight-streaming kernel and 6 the split-K kernel (K = 1024), 128 rows the split-K kernel
    and 129 the tiled one; integer inputs with bias and GELU-free fp32 output: exact."""
    rng = np.random.default_rng(8000 + M)
    N, K = 2064, 1024
    x = si.int_bf16(rng, (M, K), -3, 3)
    w = si.int_bf16(rng, (N, K), -3, 3)
    b = si.int_bf16(rng, (N,), -8, 8)
    rows, cols = tsl.tp_linear_tile_shape(M, N, K)
    kernel = "weight-streaming" if (rows, cols) == (0, 0) else ("split-K" if cols <= 48 else "tiled")
    assert kernel == {5: "weight-streaming", 6: "split-K", 128: "split-K", 129: "tiled"}[M]
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b), out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.colwise(x, w, b))
