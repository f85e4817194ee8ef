"""GPU parity of the rowwise_split_input style through the C ABI.

[TP] "Colwise and rowwise" (rowwise_split_input) and "What to leave out" (a
large AdaLN modulation projection is sharded this way): the input is the same
on every rank, each rank cuts its own slice of the input features, computes an
fp32 partial with its column block of the weight, and the SUM combine (bias
added once) rebuilds the unsharded layer.  Skinny inputs (up to 5 rows) run the
weight-streaming kernel, up to 128 rows the split-K kernel, taller ones the tiled
MFMA kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import abs_dot, bits_to_dev, check_close, dev_to_bits, dev_to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 3, 8, 300])
def test_split_input_integer_inputs_exact(M):
    """Integer-valued inputs: every partial and the combined sum are exact."""
    rng = np.random.default_rng(60 + M)
    P, N, K = 4, 272, 2048
    x = si.int_bf16(rng, (M, K), -4, 4)
    w = si.int_bf16(rng, (N, K), -4, 4)
    b = si.int_bf16(rng, (N,), -8, 8)
    xd, wd = bits_to_dev(x), bits_to_dev(w)
    parts = []
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise_split_input", P, r)
        ow = oracle.shard_rowwise(w, P, r)
        assert np.array_equal(dev_to_bits(ws), ow)
        p = tsl.tp_linear_rowwise_split_input(xd, ws, P, r)
        assert np.array_equal(dev_to_f64(p), oracle.rowwise_split_input(x, r, P, ow))
        parts.append(p)
    y = tsl.tp_partial_combine(parts, "sum", bias=bits_to_dev(b), out_dtype=torch.float32)
    assert np.array_equal(dev_to_f64(y), oracle.linear(x, w, b))


@pytest.mark.parametrize("M,P", [(2, 2), (5, 8), (257, 2)])
def test_split_input_random_vs_oracle(M, P):
    rng = np.random.default_rng(70 + M + P)
    N, K = 528, 4096
    x = si.normal_bf16(rng, (M, K))
    w = si.normal_bf16(rng, (N, K), 1 / np.sqrt(K))
    b = si.normal_bf16(rng, (N,))
    xd, wd = bits_to_dev(x), bits_to_dev(w)
    kl = K // P
    parts = []
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise_split_input", P, r)
        ow = oracle.shard_rowwise(w, P, r)
        p = tsl.tp_linear_rowwise_split_input(xd, ws, P, r)
        check_close(dev_to_f64(p), oracle.rowwise_split_input(x, r, P, ow), kl, False,
                    S=abs_dot(np.ascontiguousarray(x[:, r * kl:(r + 1) * kl]), ow), what=f"split r{r}")
        parts.append(p)
    y = tsl.tp_partial_combine(parts, "sum", bias=bits_to_dev(b), out_dtype=torch.bfloat16)
    check_close(dev_to_f64(y), oracle.linear(x, w, b), K + P, True, S=abs_dot(x, w, b), what="split sum")


def test_split_input_equals_rowwise_on_the_input_slice():
    """The entry point cuts the same slice a caller would pass to tp_linear_rowwise."""
    rng = np.random.default_rng(80)
    P, N, K = 4, 512, 6144
    for M in (4, 96):
        xd = bits_to_dev(si.normal_bf16(rng, (M, K)))
        wd = bits_to_dev(si.normal_bf16(rng, (N, K), 1 / np.sqrt(K)))
        kl = K // P
        for r in range(P):
            ws, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise", P, r)
            a = tsl.tp_linear_rowwise_split_input(xd, ws, P, r)
            b = tsl.tp_linear_rowwise(xd[:, r * kl:(r + 1) * kl], ws)
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_split_input_adaln_full_size_p4():
    """The adaLN modulation workload (c [4, 6144], W [36864, 6144]) sharded with
    rowwise_split_input at tp 4: every rank's partial and the combined output."""
    wl = si.workload("adaln")
    a = wl.arrays
    P, K = 4, 6144
    kl = K // P
    c = a["c"]
    b = si.normal_bf16(np.random.default_rng(90), (a["w_ada"].shape[0],))
    cd, wd = bits_to_dev(c), bits_to_dev(a["w_ada"])
    parts = []
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise_split_input", P, r)
        ow = oracle.shard_rowwise(a["w_ada"], P, r)
        assert np.array_equal(dev_to_bits(ws), ow)
        p = tsl.tp_linear_rowwise_split_input(cd, ws, P, r)
        check_close(dev_to_f64(p), oracle.rowwise_split_input(c, r, P, ow), kl, False,
                    S=abs_dot(np.ascontiguousarray(c[:, r * kl:(r + 1) * kl]), ow), what=f"adaln split r{r}")
        parts.append(p)
    y = tsl.tp_partial_combine(parts, "sum", bias=bits_to_dev(b), out_dtype=torch.bfloat16)
    check_close(dev_to_f64(y), oracle.linear(c, a["w_ada"], b), K + P, True, S=abs_dot(c, a["w_ada"], b),
                what="adaln split sum")
