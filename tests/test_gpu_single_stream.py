"""GPU parity of a FLUX.2-style single-stream block's linear layers, sharded and combined.

[TP] "Fused projections": the single-stream block packs Q, K, V and the SwiGLU
gate and up projections in one weight, sharded colwise with blocks
[1, 1, 1, 3, 3]; its output projection takes the attention output and the MLP
hidden features side by side and is sharded rowwise with the packed row
blocks [inner_dim, mlp_hidden_dim] ([1, 3] here).  Each rank's slices of the two
weights line up (its heads, its hidden features), so the rank's partial needs
no data from other ranks, and the SUM of the partials equals the unsharded
layer.

Attention itself is not on this path: the rank's V heads stand in for its
attention output (attention is rank-local per head, so any per-head function
keeps the layout argument intact).  Every intermediate is written by the
library into column views of one input buffer; nothing is concatenated on the
host or by torch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import bits_to_dev, check_close, dev_to_f64

pytestmark = pytest.mark.gpu

D = 128          # hidden size (8 heads of 16)
HEAD_DIM = 16
M = 300          # tokens: one full 256-row tile and a ragged one


def _inputs(seed):
    rng = np.random.default_rng(seed)
    x = si.normal_bf16(rng, (M, D))
    w_f = si.normal_bf16(rng, (9 * D, D), 1 / np.sqrt(D))        # [Q; K; V; gate; up] = [1, 1, 1, 3, 3]
    w_o = si.normal_bf16(rng, (D, 4 * D), 1 / np.sqrt(4 * D))    # input [attn | mlp hidden] = [1, 3]
    b_o = si.normal_bf16(rng, (D,))
    return x, w_f, w_o, b_o


def _sharded(P, x, w_f, w_o, b_o):
    xd, wfd, wod = bits_to_dev(x), bits_to_dev(w_f), bits_to_dev(w_o)
    a, h = D // P, 3 * D // P                  # the rank's attention width and MLP hidden width
    parts = []
    for r in range(P):
        sf, _ = tsl.tp_plan_shard_slice(wfd, None, "colwise", P, r, blocks=[1, 1, 1, 3, 3])  # [Q;K;V;G;U]_r
        so, _ = tsl.tp_plan_shard_slice(wod, None, "rowwise", P, r, blocks=[1, 3])            # [D, a + h]
        assert tuple(sf.shape) == (9 * D // P, D) and tuple(so.shape) == (D, a + h)
        inp = torch.empty((M, a + h), dtype=torch.bfloat16, device="cuda")
        # the rank's V heads (rows 2a .. 3a of its fused shard) -> columns [0, a)
        tsl.tp_linear_colwise(xd, sf[2 * a:3 * a], out=inp[:, :a])
        # its SwiGLU hidden features from its [gate; up] rows -> columns [a, a + h)
        tsl.tp_linear_colwise(xd, sf[3 * a:], act="swiglu", out=inp[:, a:])
        parts.append(tsl.tp_linear_rowwise(inp, so))
    return tsl.tp_partial_combine(parts, "sum", bias=bits_to_dev(b_o))


def _reference(x, w_f, w_o, b_o):
    v = oracle.bf16_round(oracle.linear(x, w_f[2 * D:3 * D]))          # all heads' V, bf16 as stored
    mlp = oracle.bf16_round(oracle.colwise_swiglu(x, w_f[3 * D:]))     # [gate; up] of the whole layer
    return oracle.linear(np.concatenate([v, mlp], axis=1), w_o, b_o)


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_single_stream_block_sharded_equals_unsharded(P):
    x, w_f, w_o, b_o = _inputs(50 + P)
    y = _sharded(P, x, w_f, w_o, b_o)
    torch.cuda.synchronize()
    check_close(dev_to_f64(y), _reference(x, w_f, w_o, b_o), 4 * D, out_bf16=False,
                what=f"single-stream block P={P}")


def test_single_stream_partials_sum_to_the_one_rank_result():
    """GPU against GPU: the tp 4 result equals the tp 1 result up to fp32 reassociation of
    the rowwise sum (the colwise intermediates are the same values at any tp degree)."""
    x, w_f, w_o, b_o = _inputs(60)
    y1 = dev_to_f64(_sharded(1, x, w_f, w_o, b_o))
    y4 = dev_to_f64(_sharded(4, x, w_f, w_o, b_o))
    # |x . w| summed in four pieces instead of one: a few fp32 ulps of the sum of magnitudes
    v = oracle.bf16_widen(oracle.bf16_round(oracle.linear(x, w_f[2 * D:3 * D])))
    mlp = oracle.bf16_widen(oracle.bf16_round(oracle.colwise_swiglu(x, w_f[3 * D:])))
    s = np.abs(np.concatenate([v, mlp], axis=1)) @ np.abs(oracle.bf16_widen(w_o)).T
    assert np.all(np.abs(y4 - y1) <= 8 * 4 * D * 2.0 ** -24 * s + 1e-6)
