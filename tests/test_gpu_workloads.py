"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, through the C ABI.

Index work (slices, QKV split, CONCAT) and the SUM combine are checked bit for
bit on whole tensors.  GEMM outputs are checked against the oracle on sampled
rows, all columns, every rank: rows 0, 1 and M - 1, both rows at every edge of
the output tiles that the library picks for that GEMM's shape (192, 224 or 256
rows at these sizes, from tp_linear_tile_shape), and seeded random rows.  Whole tensors are
checked through GPU-side invariants of the method: the colwise shards' outputs
gather bit for bit to the unsharded output (the tiled kernel has no split-K, so
each output element sees the same products in the same order whatever the tile
height or column offset), and the rowwise partials sum to it (to rounding: the
sum of P partials and one K-long accumulation add in different orders).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import (abs_dot, bits_to_dev, check_close, dev_to_bits, dev_to_f64,
                     sample_rows)

pytestmark = pytest.mark.gpu


def _rows_of(t: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    return t[torch.from_numpy(rows).to(t.device)]


def _edge_rows(m, n, k, act, n_random, seed):
    """Sample rows at the real tile edges of an [m, k] x [n, k]^T GEMM."""
    tile, _ = tsl.tp_linear_tile_shape(m, n, k, act)
    assert tile in (192, 224, 256), tile
    return sample_rows(m, n_random, seed, tile=tile)


def _check_colwise(y, x_bits, w_bits, rows, act, what, bias_bits=None):
    a = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    ref = oracle.colwise(x_bits, w_bits, bias_bits, act=a, rows=rows)
    S = abs_dot(x_bits[rows], w_bits, bias_bits)
    return check_close(dev_to_f64(_rows_of(y, rows)), ref, w_bits.shape[1], y.dtype == torch.bfloat16,
                       S=S, what=what)


def _check_rowwise(p, x_rows_bits, w_bits, what):
    ref = oracle.linear(x_rows_bits, w_bits)
    return check_close(dev_to_f64(p), ref, w_bits.shape[1], False, S=abs_dot(x_rows_bits, w_bits),
                       what=what)


def test_tiny_mlp_full_parity():
    wl = si.workload("tiny_mlp")
    a = wl.arrays
    P = 2
    rows = np.arange(64)
    x = bits_to_dev(a["x"])
    parts, hs = [], []
    for r in range(P):
        w1s, b1s = tsl.tp_plan_shard_slice(bits_to_dev(a["w1"]), bits_to_dev(a["b1"]), "colwise", P, r)
        ow1, ob1 = oracle.shard_colwise(a["w1"], a["b1"], P, r)
        assert np.array_equal(dev_to_bits(w1s), ow1) and np.array_equal(dev_to_bits(b1s), ob1)
        w2s, _ = tsl.tp_plan_shard_slice(bits_to_dev(a["w2"]), None, "rowwise", P, r)
        ow2 = oracle.shard_rowwise(a["w2"], P, r)
        assert np.array_equal(dev_to_bits(w2s), ow2)
        h = tsl.tp_linear_colwise(x, w1s, b1s, act="gelu_tanh")
        _check_colwise(h, a["x"], ow1, rows, "gelu_tanh", f"tiny colwise r{r}", ob1)
        p = tsl.tp_linear_rowwise(h, w2s)
        _check_rowwise(p, dev_to_bits(h), ow2, f"tiny rowwise r{r}")
        parts.append(p)
        hs.append(h)
    y = tsl.tp_partial_combine(parts, "sum", bias=bits_to_dev(a["b2"]))
    ref = oracle.combine_sum([p.cpu().numpy() for p in parts], a["b2"])
    assert np.array_equal(y.cpu().numpy(), ref)
    hcat = tsl.tp_partial_combine(hs, "concat")
    assert np.array_equal(dev_to_bits(hcat), oracle.combine_concat([dev_to_bits(h) for h in hs]))


def test_attention_projections_p4():
    wl = si.workload("attention_proj")
    a, m = wl.arrays, wl.meta
    P, H, hd = 4, m["heads"], m["head_dim"]
    k_loc = m["hidden"] // P
    rows_q = _edge_rows(m["M"], 3 * H // P * hd, m["hidden"], "none", 16, seed=1)
    rows_o = _edge_rows(m["M"], m["hidden"], k_loc, "none", 16, seed=11)
    x, A = bits_to_dev(a["x"]), bits_to_dev(a["a"])
    wqkv, wo = bits_to_dev(a["w_qkv"]), bits_to_dev(a["w_o"])
    qkv_out, parts = [], []
    for r in range(P):
        ws, _ = tsl.tp_fused_qkv_split(wqkv, None, H, hd, P, r)
        ow, _ = oracle.qkv_split(a["w_qkv"], None, H, hd, P, r)
        assert np.array_equal(dev_to_bits(ws), ow), f"qkv split r{r}"
        y = tsl.tp_linear_colwise(x, ws)
        _check_colwise(y, a["x"], ow, rows_q, "none", f"attn qkv r{r}")
        qkv_out.append(y)
        wos, _ = tsl.tp_plan_shard_slice(wo, None, "rowwise", P, r)
        oo = oracle.shard_rowwise(a["w_o"], P, r)
        assert np.array_equal(dev_to_bits(wos), oo)
        p = tsl.tp_linear_rowwise(A[:, r * k_loc:(r + 1) * k_loc], wos)
        _check_rowwise(_rows_of(p, rows_o), np.ascontiguousarray(a["a"][rows_o, r * k_loc:(r + 1) * k_loc]),
                       oo, f"attn out-proj r{r}")
        parts.append(p)
    total = tsl.tp_partial_combine(parts, "sum")
    assert np.array_equal(total.cpu().numpy(), oracle.combine_sum([p.cpu().numpy() for p in parts]))
    check_close(dev_to_f64(_rows_of(total, rows_o)), oracle.linear(a["a"], a["w_o"], rows=rows_o), 3072,
                False, S=abs_dot(a["a"][rows_o], a["w_o"]), what="attn out-proj sum vs unsharded")
    # head-aligned shards gather back into the unsharded fused projection, bit for bit
    full = tsl.tp_linear_colwise(x, wqkv)
    cat = tsl.tp_partial_combine(qkv_out, "concat", blocks=[1, 1, 1])
    assert torch.equal(cat, full), "attn concat(qkv) differs from the unsharded projection"


def test_mlp_p4():
    wl = si.workload("mlp_large")
    a, m = wl.arrays, wl.meta
    P = 4
    rows_up = _edge_rows(m["M"], m["ffn"] // P, m["hidden"], "gelu_tanh", 6, seed=2)
    rows_dn = _edge_rows(m["M"], m["hidden"], m["ffn"] // P, "none", 6, seed=12)
    x = bits_to_dev(a["x"])
    w1, w2 = bits_to_dev(a["w1"]), bits_to_dev(a["w2"])
    parts = []
    for r in range(P):
        w1s, _ = tsl.tp_plan_shard_slice(w1, None, "colwise", P, r)
        ow1, _ = oracle.shard_colwise(a["w1"], None, P, r)
        assert np.array_equal(dev_to_bits(w1s), ow1)
        w2s, _ = tsl.tp_plan_shard_slice(w2, None, "rowwise", P, r)
        ow2 = oracle.shard_rowwise(a["w2"], P, r)
        assert np.array_equal(dev_to_bits(w2s), ow2)
        h = tsl.tp_linear_colwise(x, w1s, act="gelu_tanh")
        _check_colwise(h, a["x"], ow1, rows_up, "gelu_tanh", f"mlp up r{r}")
        p = tsl.tp_linear_rowwise(h, w2s)
        _check_rowwise(_rows_of(p, rows_dn), dev_to_bits(_rows_of(h, rows_dn)), ow2, f"mlp down r{r}")
        parts.append(p)
        del h
    total = tsl.tp_partial_combine(parts, "sum", out_dtype=torch.bfloat16)
    ref = oracle.combine_sum([p.cpu().numpy() for p in parts])
    assert np.array_equal(dev_to_bits(total), oracle.bf16_round(ref.astype(np.float64)))


@pytest.mark.parametrize("P", [2, 4, 8])
def test_full_block(P):
    wl = si.workload("full_block")
    a, m = wl.arrays, wl.meta
    H, hd, hidden, ffn, M = m["heads"], m["head_dim"], m["hidden"], m["ffn"], m["M"]
    kq, k_loc, f_loc = 3 * H // P * hd, hidden // P, ffn // P
    rows_q = _edge_rows(M, kq, hidden, "none", 2, seed=3 + P)
    rows_o = _edge_rows(M, hidden, k_loc, "none", 2, seed=13 + P)
    rows_up = _edge_rows(M, f_loc, hidden, "gelu_tanh", 2, seed=23 + P)
    rows_dn = _edge_rows(M, hidden, f_loc, "none", 2, seed=33 + P)
    x, A = bits_to_dev(a["x"]), bits_to_dev(a["a"])
    wqkv, wo = bits_to_dev(a["w_qkv"]), bits_to_dev(a["w_o"])
    w1, w2 = bits_to_dev(a["w1"]), bits_to_dev(a["w2"])
    qkv_out, up_out, out_parts, down_parts = [], [], [], []
    for r in range(P):
        ws, _ = tsl.tp_fused_qkv_split(wqkv, None, H, hd, P, r)
        oq, _ = oracle.qkv_split(a["w_qkv"], None, H, hd, P, r)
        assert np.array_equal(dev_to_bits(ws), oq)
        wos, _ = tsl.tp_plan_shard_slice(wo, None, "rowwise", P, r)
        oo = oracle.shard_rowwise(a["w_o"], P, r)
        assert np.array_equal(dev_to_bits(wos), oo)
        w1s, _ = tsl.tp_plan_shard_slice(w1, None, "colwise", P, r)
        o1, _ = oracle.shard_colwise(a["w1"], None, P, r)
        assert np.array_equal(dev_to_bits(w1s), o1)
        w2s, _ = tsl.tp_plan_shard_slice(w2, None, "rowwise", P, r)
        o2 = oracle.shard_rowwise(a["w2"], P, r)
        assert np.array_equal(dev_to_bits(w2s), o2)

        q = tsl.tp_linear_colwise(x, ws)
        _check_colwise(q, a["x"], oq, rows_q, "none", f"block P{P} qkv r{r}")
        po = tsl.tp_linear_rowwise(A[:, r * k_loc:(r + 1) * k_loc], wos)
        _check_rowwise(_rows_of(po, rows_o), np.ascontiguousarray(a["a"][rows_o, r * k_loc:(r + 1) * k_loc]),
                       oo, f"block P{P} out-proj r{r}")
        h = tsl.tp_linear_colwise(x, w1s, act="gelu_tanh")
        _check_colwise(h, a["x"], o1, rows_up, "gelu_tanh", f"block P{P} up r{r}")
        pd = tsl.tp_linear_rowwise(h, w2s)
        _check_rowwise(_rows_of(pd, rows_dn), dev_to_bits(_rows_of(h, rows_dn)), o2, f"block P{P} down r{r}")
        qkv_out.append(q)
        up_out.append(h)
        out_parts.append(po)
        down_parts.append(pd)

    # SUM x2 and CONCAT x2, bit-exact on whole tensors
    s_out = tsl.tp_partial_combine(out_parts, "sum")
    assert np.array_equal(s_out.cpu().numpy(), oracle.combine_sum([p.cpu().numpy() for p in out_parts]))
    s_down = tsl.tp_partial_combine(down_parts, "sum", out_dtype=torch.bfloat16)
    ref_down = oracle.combine_sum([p.cpu().numpy() for p in down_parts])
    assert np.array_equal(dev_to_bits(s_down), oracle.bf16_round(ref_down.astype(np.float64)))
    c_qkv = tsl.tp_partial_combine(qkv_out, "concat", blocks=[1, 1, 1])
    assert np.array_equal(dev_to_bits(c_qkv), oracle.combine_concat([dev_to_bits(t) for t in qkv_out],
                                                                      [1, 1, 1]))
    c_up = tsl.tp_partial_combine(up_out, "concat")
    assert np.array_equal(dev_to_bits(c_up), oracle.combine_concat([dev_to_bits(t) for t in up_out]))

    # whole-tensor invariants against the unsharded layers on the GPU: the colwise gathers
    # bit for bit, the rowwise sum to rounding
    full_qkv = tsl.tp_linear_colwise(x, wqkv)
    assert torch.equal(c_qkv, full_qkv), f"P{P} concat(qkv) differs from the unsharded projection"
    del full_qkv
    full_up = tsl.tp_linear_colwise(x, w1, act="gelu_tanh")
    assert torch.equal(c_up, full_up), f"P{P} concat(up) differs from the unsharded projection"
    del full_up
    full_out = tsl.tp_linear_rowwise(A, wo)
    check_close(dev_to_f64(s_out), dev_to_f64(full_out), hidden, False, what=f"P{P} sum(out) vs unsharded")
    del full_out
    # sampled rows of the combined results against the oracle's unsharded layers
    check_close(dev_to_f64(_rows_of(s_out, rows_o)), oracle.linear(a["a"], a["w_o"], rows=rows_o), hidden,
                False, S=abs_dot(a["a"][rows_o], a["w_o"]), what=f"P{P} sum(out) vs oracle")
    hid_rows = dev_to_bits(_rows_of(c_up, rows_dn))
    check_close(dev_to_f64(_rows_of(s_down, rows_dn)), oracle.linear(hid_rows, a["w2"]), ffn, True,
                S=abs_dot(hid_rows, a["w2"]), what=f"P{P} sum(down) vs oracle")


def test_adaln_skinny_p4():
    wl = si.workload("adaln")
    a = wl.arrays
    P = 4
    wd = bits_to_dev(a["w_ada"])
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(wd, None, "colwise", P, r)
        ow, _ = oracle.shard_colwise(a["w_ada"], None, P, r)
        assert np.array_equal(dev_to_bits(ws), ow)
        for B in (1, 2, 3, 4):
            c = np.ascontiguousarray(a["c"][:B])
            y = tsl.tp_linear_colwise(bits_to_dev(c), ws)
            check_close(dev_to_f64(y), oracle.colwise(c, ow), 6144, True, S=abs_dot(c, ow),
                        what=f"adaln r{r} B{B}")
