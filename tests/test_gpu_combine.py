"""GPU parity of the SUM combine (the one-device AllReduce of rowwise partials).

The reading that fixes the result: fp32 adds in ascending part order, the bias
added once at the end, one rounding to the output dtype.  With the order fixed
the result is unique, so the GPU must equal the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import bits_to_dev, dev_to_bits, f32_to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("M,N", [(64, 256), (129, 1000), (3, 6), (2, 4100)])
@pytest.mark.parametrize("bias", [False, True])
def test_sum_bit_exact(P, M, N, bias):
    rng = np.random.default_rng(P * 1000 + M + N)
    parts = [si.normal_f32(rng, (M, N), 3.0) for _ in range(P)]
    b = si.normal_bf16(rng, (N,)) if bias else None
    # N not a multiple of 4 needs a padded row stride (16-byte rows)
    ld = (N + 3) // 4 * 4
    dev = []
    for p in parts:
        t = torch.zeros(M, ld, dtype=torch.float32, device="cuda")
        t[:, :N] = f32_to_dev(p)
        dev.append(t[:, :N])
    ref = oracle.combine_sum(parts, b)
    out_big = torch.zeros(M, ld, dtype=torch.float32, device="cuda")
    out = tsl.tp_partial_combine(dev, "sum", bias=bits_to_dev(b) if bias else None, out=out_big[:, :N])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    ld16 = (N + 7) // 8 * 8
    outb_big = torch.zeros(M, ld16, dtype=torch.bfloat16, device="cuda")
    outb = tsl.tp_partial_combine(dev, "sum", bias=bits_to_dev(b) if bias else None,
                                  out=outb_big[:, :N])
    assert np.array_equal(dev_to_bits(outb), oracle.bf16_round(ref.astype(np.float64)))


def test_sum_order_is_ascending_rank():
    vals = [1e8, 1.0, -1e8]
    dev = [torch.full((1, 4), v, dtype=torch.float32, device="cuda") for v in vals]
    out = tsl.tp_partial_combine(dev, "sum")
    assert torch.all(out == 0.0)
    dev = [dev[0], dev[2], dev[1]]
    assert torch.all(tsl.tp_partial_combine(dev, "sum") == 1.0)


def test_sum_in_place_into_first_part():
    rng = np.random.default_rng(3)
    parts = [si.normal_f32(rng, (50, 96)) for _ in range(4)]
    dev = [f32_to_dev(p) for p in parts]
    ref = oracle.combine_sum(parts)
    tsl.tp_partial_combine(dev, "sum", out=dev[0])
    assert np.array_equal(dev[0].cpu().numpy(), ref)


def test_mlp_pair_tiny_all_on_gpu_matches_oracle_chain():
    """[TP] pairing rule end to end on the tiny MLP (P=2): colwise + GELU, rowwise partials,
    one SUM with the bias added once."""
    from helpers import check_close, dev_to_f64
    wl = si.workload("tiny_mlp")
    a = wl.arrays
    P = 2
    x = bits_to_dev(a["x"])
    partials = []
    ref_parts = []
    for r in range(P):
        w1s, b1s = tsl.tp_plan_shard_slice(bits_to_dev(a["w1"]), bits_to_dev(a["b1"]), "colwise", P, r)
        w2s, _ = tsl.tp_plan_shard_slice(bits_to_dev(a["w2"]), None, "rowwise", P, r)
        h = tsl.tp_linear_colwise(x, w1s, b1s, act="gelu_tanh")
        partials.append(tsl.tp_linear_rowwise(h, w2s))
        ow1, ob1 = oracle.shard_colwise(a["w1"], a["b1"], P, r)
        oh = oracle.bf16_round(oracle.colwise(a["x"], ow1, ob1, act=oracle.ACT_GELU_TANH))
        ref_parts.append(oracle.linear(oh, oracle.shard_rowwise(a["w2"], P, r)))
    y = tsl.tp_partial_combine(partials, "sum", bias=bits_to_dev(a["b2"]))
    ref = np.sum(ref_parts, axis=0) + oracle.bf16_widen(a["b2"])[None, :]
    check_close(dev_to_f64(y), ref, 1024, False, what="tiny MLP pair")
    # and against the unsharded MLP
    hid = oracle.bf16_round(oracle.linear(a["x"], a["w1"], a["b1"], act=oracle.ACT_GELU_TANH))
    full = oracle.linear(hid, a["w2"], a["b2"])
    check_close(dev_to_f64(y), full, 1024, False, what="tiny MLP vs unsharded")
