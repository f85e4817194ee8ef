"""GPU parity of the fused SwiGLU epilogue through the C ABI.

[TP] "Fused projections": a SwiGLU gate and up projection packed with blocks
[1, 1] is sharded block by block, so each rank's shard is its gate rows followed
by the matching up rows, and the rank computes silu(x . gate^T + b_gate) *
(x . up^T + b_up) for its slice of the hidden features.  The tiled kernel pairs
gate and up columns inside a tile, so the output is written once, already
gated.  Ragged shapes span several 128-column output tiles with partial tiles
on both edges; up to 128 rows the split-K kernel pairs the 16 gate rows and 16
up rows of each 16-column block in one workgroup instead (test_gpu_narrow.py).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import bits_to_dev, check_swiglu, dev_to_bits, dev_to_f64, sample_rows

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16, 64), (5, 144, 512), (300, 272, 320), (257, 528, 1024), (513, 1040, 192), (1100, 1040, 2048)]


@pytest.mark.parametrize("M,n,K", SHAPES)
@pytest.mark.parametrize("bias,out", [(False, "bf16"), (True, "bf16"), (True, "f32")])
def test_swiglu_random_vs_oracle(M, n, K, bias, out):
    rng = np.random.default_rng(M + 3 * n + K)
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (2 * n, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (2 * n,)) if bias else None
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), bits_to_dev(b) if bias else None,
                              act="swiglu", out_dtype=dt)
    assert tuple(y.shape) == (M, n)
    check_swiglu(dev_to_f64(y), x, w, b, out == "bf16", what=f"swiglu {M}x{n}x{K} bias={bias} {out}")


def test_swiglu_saturated_gate_exact():
    """Gate pre-activations >= 64 (integer inputs): silu(g) = g in fp32 too, so the
    fp32 output is exactly g * u; the halves must not be swapped."""
    rng = np.random.default_rng(7)
    M, n, K = 300, 272, 64
    x = si.int_bf16(rng, (M, K), 1, 3)
    g = si.int_bf16(rng, (n, K), 1, 4)
    u = si.int_bf16(rng, (n, K), -4, 4)
    w = np.concatenate([g, u])
    y = tsl.tp_linear_colwise(bits_to_dev(x), bits_to_dev(w), act="swiglu", out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.linear(x, g) * oracle.linear(x, u))


def test_swiglu_strided_and_output_view():
    rng = np.random.default_rng(8)
    M, n, K = 200, 144, 256
    xb = si.normal_bf16(rng, (M, K + 64))
    wb = si.normal_bf16(rng, (2 * n, K + 32), 1 / 16)
    x = bits_to_dev(xb)[:, 64:]
    w = bits_to_dev(wb)[:, :K]
    big = torch.full((M, n + 32), 5.0, dtype=torch.float32, device="cuda")
    tsl.tp_linear_colwise(x, w, act="swiglu", out=big[:, :n])
    check_swiglu(dev_to_f64(big[:, :n]), np.ascontiguousarray(xb[:, 64:]), np.ascontiguousarray(wb[:, :K]), None,
                 False, what="swiglu strided")
    assert torch.all(big[:, n:] == 5.0)


@pytest.mark.parametrize("P", [2, 4])
def test_swiglu_packed_shards_full_size(P):
    """A FLUX.2-style fused gate/up projection (hidden 6144 -> 2 x 18432) sharded with
    blocks [1, 1]: the GPU slice equals the oracle's, each rank's gated output matches
    the oracle on sampled rows, and the ranks' outputs side by side match the
    unsharded fused output."""
    rng = np.random.default_rng(120 + P)
    M, hidden, ffn = 4608, 6144, 18432
    x = si.normal_bf16(rng, (M, hidden))
    w = si.normal_bf16(rng, (2 * ffn, hidden), 1 / np.sqrt(hidden))
    b = si.normal_bf16(rng, (2 * ffn,))
    xd, wd, bd = bits_to_dev(x), bits_to_dev(w), bits_to_dev(b)
    rows = sample_rows(M, 6, seed=P)
    outs = []
    for r in range(P):
        ws, bs = tsl.tp_plan_shard_slice(wd, bd, "colwise", P, r, blocks=[1, 1])
        ow, ob = oracle.shard_packed_colwise(w, b, [1, 1], P, r)
        assert np.array_equal(dev_to_bits(ws), ow) and np.array_equal(dev_to_bits(bs), ob)
        y = tsl.tp_linear_colwise(xd, ws, bs, act="swiglu")
        check_swiglu(dev_to_f64(y[torch.from_numpy(rows).cuda()]), x, ow, ob, True, rows=rows,
                     what=f"flux2 ffn-up P{P} r{r}")
        outs.append(y)
    full = tsl.tp_linear_colwise(xd, wd, bd, act="swiglu")
    cat = tsl.tp_partial_combine(outs, "concat")
    # every output element sees the same gate and up products in the same order, sharded or
    # not (no split-K), so the gather equals the unsharded fused output bit for bit
    assert torch.equal(cat, full), f"P{P}: concat of the SwiGLU shards differs from the unsharded output"
