"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties an oracle function to brute force in exact arithmetic, a closed
form, a library routine, an invariant the tensor-parallel pages state, or a
page-derived fixture, so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -53  # unit roundoff of double


def _gamma(n, u=U):
    return n * u / (1 - n * u)


def _index_weight(n, k):
    """W[row, col] = row * k + col as uint16 bits: every element names its own position."""
    assert n * k < 65536
    return np.arange(n * k, dtype=np.uint16).reshape(n, k)


# --------------------------------------------------------------------------------------
# bf16 conversion
# --------------------------------------------------------------------------------------

def test_bf16_widen_known_patterns():
    assert oracle.bf16_widen(np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.bf16_widen(np.array([0xC000], np.uint16))[0] == -2.0
    assert oracle.bf16_widen(np.array([0x3E80], np.uint16))[0] == 0.25
    assert oracle.bf16_widen(np.array([0x7F80], np.uint16))[0] == math.inf
    assert oracle.bf16_widen(np.array([0x0001], np.uint16))[0] == 2.0 ** -133
    assert oracle.bf16_widen(np.array([0x7F7F], np.uint16))[0] == (2 - 2 ** -7) * 2.0 ** 127


def test_bf16_round_ties_and_edges_by_hand():
    cases = [
        (1.0 + 2 ** -8, 0x3F80),              # tie -> even (1.0)
        (1.0 + 3 * 2 ** -8, 0x3F82),          # tie between 1+2^-7 (odd) and 1+2^-6 (even)
        (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),   # just above a tie: up (double rounding via fp32 would give 1.0)
        (-(1.0 + 2 ** -8 - 2 ** -40), 0xBF80),
        (2.0 ** -133, 0x0001),                # smallest subnormal
        (2.0 ** -134, 0x0000),                # tie between 0 and 2^-133 -> even (0)
        (1.5 * 2.0 ** -133, 0x0002),          # tie between 1 and 2 quanta -> 2
        ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80), # tie between max (odd) and 2^128 -> inf
        ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F), # max finite
        (-0.0, 0x8000),
        (1e300, 0x7F80),
        (-1e-300, 0x8000),
    ]
    got = oracle.bf16_round(np.array([c[0] for c in cases]))
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_bf16_round_matches_torch_on_float32_values():
    """Library routine: torch's fp32 -> bf16 conversion (round to nearest even).  On values that
    are exact in fp32 the double path cannot double-round, so both must agree bit for bit."""
    rng = np.random.default_rng(123)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e30).astype(np.float32),
        (rng.standard_normal(50000) * 1e-38).astype(np.float32),
        # every bf16 tie point in [1, 2): x.5 ulp
        (1.0 + (np.arange(128) + 0.5) * 2.0 ** -7).astype(np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_roundtrip_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = oracle.bf16_widen(pats)
    back = oracle.bf16_round(w)
    finite_or_inf = ~np.isnan(w)
    assert np.array_equal(back[finite_or_inf], pats[finite_or_inf])


# --------------------------------------------------------------------------------------
# GELU-tanh
# --------------------------------------------------------------------------------------

def test_gelu_identities():
    assert oracle.gelu_tanh(0.0) == 0.0
    for v in np.linspace(-9, 9, 181):
        g, gm = oracle.gelu_tanh(v), oracle.gelu_tanh(-v)
        # tanh is odd, so g(v) - g(-v) = v exactly in real arithmetic
        assert abs((g - gm) - v) <= 4e-16 * max(1.0, abs(v))
    for v in (10.0, 20.0, 40.0):
        assert abs(oracle.gelu_tanh(v) / v - 1.0) < 1e-15
        assert abs(oracle.gelu_tanh(-v)) < 1e-15


def test_gelu_matches_torch_tanh_gelu_float64():
    v = np.linspace(-12, 12, 4801)
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh(x) for x in v])
    assert np.max(np.abs(got - ref)) <= 1e-14


def test_gelu_close_to_erf_gelu():
    """The tanh form approximates x*Phi(x) to < 5e-4 (a wrong cubic constant exceeds that)."""
    v = np.linspace(-10, 10, 20001)
    erf_gelu = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in v])
    got = np.array([oracle.gelu_tanh(x) for x in v])
    assert np.max(np.abs(got - erf_gelu)) < 5e-4


# --------------------------------------------------------------------------------------
# linear (the GEMM definition)
# --------------------------------------------------------------------------------------

def _exact_linear(x, w, b):
    xf = oracle.bf16_widen(x)
    wf = oracle.bf16_widen(w)
    bf = oracle.bf16_widen(b) if b is not None else None
    m, k = xf.shape
    n = wf.shape[0]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            s = sum((Fraction(float(xf[i, t])) * Fraction(float(wf[j, t])) for t in range(k)),
                    Fraction(0))
            if bf is not None:
                s += Fraction(float(bf[j]))
            out[i, j] = s
    return out


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (5, 3, 16)])
def test_linear_exact_rational_brute_force(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    x = si.normal_bf16(rng, (m, k))
    w = si.normal_bf16(rng, (n, k), 0.3)
    b = si.normal_bf16(rng, (n,))
    exact = _exact_linear(x, w, b)
    got = oracle.linear(x, w, b)
    absx = np.abs(oracle.bf16_widen(x))
    absw = np.abs(oracle.bf16_widen(w))
    bound = _gamma(k + 1) * (absx @ absw.T + np.abs(oracle.bf16_widen(b))[None, :])
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(got[i, j])) - exact[i, j]) <= Fraction(float(bound[i, j])) + \
                Fraction(1, 2 ** 1074)


def test_linear_closed_form_ones_and_ramp():
    """x = 1, W[n, k] = n + 1, b[n] = -n  =>  y[i, n] = K (n + 1) - n."""
    m, n, k = 6, 10, 96
    x = si.to_bf16_bits(np.ones((m, k), np.float32))
    w = si.to_bf16_bits(np.repeat(np.arange(1, n + 1, dtype=np.float32)[:, None], k, axis=1))
    b = si.to_bf16_bits(-np.arange(n, dtype=np.float32))
    y = oracle.linear(x, w, b)
    want = k * (np.arange(n) + 1.0) - np.arange(n)
    assert np.array_equal(y, np.broadcast_to(want, (m, n)))


def test_linear_one_hot_selects_weight_column():
    """x row i = e_{c_i}  =>  y[i, n] = W[n, c_i] (catches a transposed or mis-strided W)."""
    rng = np.random.default_rng(7)
    n, k = 12, 20
    w = si.normal_bf16(rng, (n, k))
    cols = np.array([0, 5, 19, 7, 13])
    xf = np.zeros((cols.size, k), np.float32)
    xf[np.arange(cols.size), cols] = 1.0
    y = oracle.linear(si.to_bf16_bits(xf), w)
    wf = oracle.bf16_widen(w)
    assert np.array_equal(y, wf[:, cols].T)


def test_linear_matches_numpy_float64_matmul():
    rng = np.random.default_rng(11)
    m, n, k = 33, 47, 320
    x = si.normal_bf16(rng, (m, k))
    w = si.normal_bf16(rng, (n, k), 1 / math.sqrt(k))
    b = si.normal_bf16(rng, (n,))
    xf, wf, bf = oracle.bf16_widen(x), oracle.bf16_widen(w), oracle.bf16_widen(b)
    ref = xf @ wf.T + bf
    got = oracle.linear(x, w, b)
    bound = 2 * _gamma(k + 1) * (np.abs(xf) @ np.abs(wf).T + np.abs(bf))
    assert np.all(np.abs(got - ref) <= bound)


def test_linear_gelu_is_gelu_of_linear_and_matches_torch():
    rng = np.random.default_rng(5)
    x = si.normal_bf16(rng, (9, 64))
    w = si.normal_bf16(rng, (17, 64), 0.125)
    b = si.normal_bf16(rng, (17,))
    pre = oracle.linear(x, w, b)
    post = oracle.linear(x, w, b, act=oracle.ACT_GELU_TANH)
    assert np.array_equal(post, np.vectorize(oracle.gelu_tanh)(pre))
    ref = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    assert np.max(np.abs(post - ref)) < 1e-14


def test_linear_row_subset_and_threads_do_not_change_results():
    rng = np.random.default_rng(9)
    x = si.normal_bf16(rng, (40, 128))
    w = si.normal_bf16(rng, (24, 128), 0.1)
    full1 = oracle.linear(x, w, threads=1)
    full7 = oracle.linear(x, w, threads=7)
    assert np.array_equal(full1, full7)
    rows = [39, 0, 17, 17, 3]
    assert np.array_equal(oracle.linear(x, w, rows=rows), full1[rows])


def test_integer_valued_inputs_are_exact():
    """Integers in [-8, 8]: every product and partial sum is an exact small integer."""
    rng = np.random.default_rng(3)
    x = si.int_bf16(rng, (16, 256))
    w = si.int_bf16(rng, (32, 256))
    xi = oracle.bf16_widen(x).astype(np.int64)
    wi = oracle.bf16_widen(w).astype(np.int64)
    assert np.array_equal(oracle.linear(x, w), (xi @ wi.T).astype(np.float64))


# --------------------------------------------------------------------------------------
# the pages' invariants for colwise / rowwise
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_concat_of_colwise_outputs_equals_unsharded_bit_exact(P):
    """[TP] opening definition: gathering the colwise output slices rebuilds the full output."""
    rng = np.random.default_rng(P)
    m, n, k = 13, 64, 96
    x = si.normal_bf16(rng, (m, k))
    w = si.normal_bf16(rng, (n, k), 0.1)
    b = si.normal_bf16(rng, (n,))
    full = oracle.linear(x, w, b, act=oracle.ACT_GELU_TANH)
    outs = []
    for r in range(P):
        ws, bs = oracle.shard_colwise(w, b, P, r)
        outs.append(oracle.colwise(x, ws, bs, act=oracle.ACT_GELU_TANH))
    assert np.array_equal(np.concatenate(outs, axis=1), full)


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_sum_of_rowwise_partials_equals_unsharded(P):
    """[TP] pairing rule: the AllReduce of rowwise partial sums rebuilds the full output."""
    rng = np.random.default_rng(10 + P)
    m, n, k = 11, 24, 256
    x = si.normal_bf16(rng, (m, k))
    w = si.normal_bf16(rng, (n, k), 1 / 16)
    full = oracle.linear(x, w)
    parts = [oracle.rowwise(x, r, P, oracle.shard_rowwise(w, P, r)) for r in range(P)]
    tot = np.sum(parts, axis=0)
    bound = 2 * _gamma(k + P) * (np.abs(oracle.bf16_widen(x)) @ np.abs(oracle.bf16_widen(w)).T)
    assert np.all(np.abs(tot - full) <= bound)
    # integer inputs: exact
    xi = si.int_bf16(rng, (m, k))
    wi = si.int_bf16(rng, (n, k))
    parts = [oracle.rowwise(xi, r, P, oracle.shard_rowwise(wi, P, r)) for r in range(P)]
    assert np.array_equal(np.sum(parts, axis=0), oracle.linear(xi, wi))


def test_mlp_pair_equals_unsharded_mlp():
    """[TP] pairing: colwise -> activation -> rowwise -> one sum equals the unsharded MLP."""
    rng = np.random.default_rng(21)
    m, h, f, P = 7, 64, 256, 4
    x = si.normal_bf16(rng, (m, h))
    w1 = si.normal_bf16(rng, (f, h), 1 / 8)
    b1 = si.normal_bf16(rng, (f,))
    w2 = si.normal_bf16(rng, (h, f), 1 / 16)
    hid = oracle.bf16_round(oracle.linear(x, w1, b1, act=oracle.ACT_GELU_TANH))
    full = oracle.linear(hid, w2)
    parts = []
    for r in range(P):
        w1s, b1s = oracle.shard_colwise(w1, b1, P, r)
        h_r = oracle.bf16_round(oracle.colwise(x, w1s, b1s, act=oracle.ACT_GELU_TANH))
        w2s = oracle.shard_rowwise(w2, P, r)
        parts.append(oracle.linear(h_r, w2s))
    bound = 2 * _gamma(f + P) * (np.abs(oracle.bf16_widen(hid)) @ np.abs(oracle.bf16_widen(w2)).T)
    assert np.all(np.abs(np.sum(parts, axis=0) - full) <= bound)


def test_rowwise_strided_input_matches_copied_slice():
    rng = np.random.default_rng(2)
    x = si.normal_bf16(rng, (9, 96))
    w = si.normal_bf16(rng, (5, 24))
    for r in range(4):
        got = oracle.rowwise(x, r, 4, w)
        ref = oracle.linear(np.ascontiguousarray(x[:, r * 24:(r + 1) * 24]), w)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("P", [1, 2, 4])
def test_rowwise_split_input_brute_force_and_allreduce(P):
    """[TP] rowwise_split_input: rank r computes from columns [r*K/P, (r+1)*K/P) of the
    replicated input; adding the bias once to the sum of the P partials is the
    unsharded layer (a skinny AdaLN-like shape: 3 conditioning rows)."""
    rng = np.random.default_rng(50 + P)
    b_rows, n, k = 3, 10, 32
    x = si.normal_bf16(rng, (b_rows, k))
    w = si.normal_bf16(rng, (n, k))
    xf = [[Fraction(float(v)) for v in row] for row in oracle.bf16_widen(x)]
    wf = [[Fraction(float(v)) for v in row] for row in oracle.bf16_widen(w)]
    kl = k // P
    parts = []
    for r in range(P):
        got = oracle.rowwise_split_input(x, r, P, oracle.shard_rowwise(w, P, r))
        for i in range(b_rows):
            for o in range(n):
                terms = [xf[i][r * kl + j] * wf[o][r * kl + j] for j in range(kl)]
                exact = sum(terms)  # bf16 products are exact rationals
                assert abs(Fraction(got[i, o]) - exact) <= sum(abs(t) for t in terms) * Fraction(_gamma(kl))
        parts.append(got)
    b = si.normal_bf16(rng, (n,))
    tot = np.sum(parts, axis=0) + oracle.bf16_widen(b)[None, :]
    full = oracle.linear(x, w, b)
    bound = 2 * _gamma(k + P + 1) * (np.abs(oracle.bf16_widen(x)) @ np.abs(oracle.bf16_widen(w)).T
                                     + np.abs(oracle.bf16_widen(b))[None, :])
    assert np.all(np.abs(tot - full) <= bound)


def test_rowwise_split_input_checks_the_plan():
    x = np.zeros((2, 30), np.uint16)
    with pytest.raises(oracle.PlanError):
        oracle.rowwise_split_input(x, 0, 4, np.zeros((3, 7), np.uint16))   # 4 does not divide 30
    with pytest.raises(oracle.PlanError):
        oracle.rowwise_split_input(x, 3, 3, np.zeros((3, 10), np.uint16))  # rank out of range


# --------------------------------------------------------------------------------------
# SwiGLU of a packed [gate; up] projection
# --------------------------------------------------------------------------------------

def _gate_up(rng, m, n, k, gate_lo, gate_hi):
    """Integer inputs with every gate pre-activation in k*[gate_lo, gate_hi]*[1, 3]."""
    x = si.int_bf16(rng, (m, k), 1, 3)
    g = si.int_bf16(rng, (n, k), gate_lo, gate_hi)
    u = si.int_bf16(rng, (n, k), -4, 4)
    return x, np.concatenate([g, u])


def test_swiglu_zero_gate_is_zero():
    """silu(0) = 0: a zero gate half gives exactly 0 whatever the up half."""
    rng = np.random.default_rng(100)
    x = si.normal_bf16(rng, (5, 64))
    w = np.concatenate([np.zeros((7, 64), np.uint16), si.normal_bf16(rng, (7, 64))])
    assert np.all(oracle.colwise_swiglu(x, w) == 0.0)


def test_swiglu_saturated_gate_is_gate_times_up():
    """A gate pre-activation >= 64 has silu(g) = g to double precision (e^-64 < 2^-53), so
    the output is exactly g * u.  Gate first, up second: swapping the halves, or a missing
    product, fails this."""
    rng = np.random.default_rng(101)
    m, n, k = 6, 9, 64
    x, w = _gate_up(rng, m, n, k, 1, 4)
    g = oracle.linear(x, w[:n])
    u = oracle.linear(x, w[n:])
    assert g.min() >= 64
    assert np.array_equal(oracle.colwise_swiglu(x, w), g * u)


def test_swiglu_saturated_negative_gate_vanishes():
    rng = np.random.default_rng(102)
    m, n, k = 4, 5, 64
    x, w = _gate_up(rng, m, n, k, -4, -1)
    assert oracle.linear(x, w[:n]).max() <= -64
    assert np.all(np.abs(oracle.colwise_swiglu(x, w)) < 1e-20)


def test_swiglu_unit_gate_is_sigmoid_of_one():
    """g = 1 exactly (one-hot input, unit gate weight): output = sigma(1) * u,
    sigma(1) = 0.7310585786300049."""
    k = 64
    x = np.zeros((1, k), np.uint16)
    x[0, 3] = 0x3F80                      # 1.0
    gate = np.zeros((1, k), np.uint16)
    gate[0, 3] = 0x3F80
    up = np.zeros((1, k), np.uint16)
    up[0, 3] = 0x4040                     # 3.0
    out = oracle.colwise_swiglu(x, np.concatenate([gate, up]))
    assert abs(out[0, 0] - 3 * 0.7310585786300049) < 1e-15


@pytest.mark.parametrize("P", [1, 2, 4])
def test_swiglu_packed_shards_concat_equals_unsharded(P):
    """[TP] "Fused projections": blocks [1, 1] shard the gate and the up halves
    independently, so rank r's shard pairs its gate rows with the matching up rows and
    the ranks' outputs, side by side, are the unsharded output.  Plain colwise slicing
    of the packed weight misaligns gate and up."""
    rng = np.random.default_rng(110 + P)
    m, n, k = 7, 16, 64
    x = si.normal_bf16(rng, (m, k))
    w = si.normal_bf16(rng, (2 * n, k), 1 / 8)
    b = si.normal_bf16(rng, (2 * n,))
    full = oracle.colwise_swiglu(x, w, b)
    outs = []
    for r in range(P):
        ws, bs = oracle.shard_packed_colwise(w, b, [1, 1], P, r)
        outs.append(oracle.colwise_swiglu(x, ws, bs))
    assert np.array_equal(np.concatenate(outs, axis=1), full)
    if P > 1:
        ws, bs = oracle.shard_colwise(w, b, P, 0)
        assert not np.allclose(oracle.colwise_swiglu(x, ws, bs), full[:, :n // P])


# --------------------------------------------------------------------------------------
# slicing
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 2, 4])
def test_shard_colwise_rowwise_brute_force(P):
    n, k = 16, 24
    w = _index_weight(n, k)
    b = np.arange(n, dtype=np.uint16) + 1000
    for r in range(P):
        ws, bs = oracle.shard_colwise(w, b, P, r)
        rows = list(range(r * n // P, (r + 1) * n // P))
        assert np.array_equal(ws, w[rows])
        assert np.array_equal(bs, b[rows])
        wr = oracle.shard_rowwise(w, P, r)
        cols = list(range(r * k // P, (r + 1) * k // P))
        assert np.array_equal(wr, w[:, cols])
    if P == 1:
        assert np.array_equal(oracle.shard_colwise(w, b, 1, 0)[0], w)


def test_packed_slicing_golden_page_examples():
    with open(os.path.join(GOLDEN, "packed_colwise_index.json")) as f:
        g = json.load(f)
    k = 3
    for case in g["cases"]:
        d, P = case["D"], case["P"]
        w = _index_weight(d, k)
        b = np.arange(d, dtype=np.uint16)
        for r, rows in enumerate(case["shards"]):
            if case["blocks"] is None:
                ws, bs = oracle.shard_colwise(w, b, P, r)
            else:
                ws, bs = oracle.shard_packed_colwise(w, b, case["blocks"], P, r)
            assert np.array_equal(ws, w[rows]), case["what"]
            assert np.array_equal(bs, b[rows]), case["what"]
            if "heads" in case:
                wq, bq = oracle.qkv_split(w, b, case["heads"], case["head_dim"], P, r)
                assert np.array_equal(wq, w[rows]) and np.array_equal(bq, b[rows])
    for case in g["rejected"]:
        with pytest.raises(ValueError):
            if "qkv_heads" in case:
                d = 3 * case["qkv_heads"] * case["head_dim"]
                oracle.qkv_split(_index_weight(d, 2), None, case["qkv_heads"], case["head_dim"],
                                 case["P"], 0)
            else:
                oracle.shard_packed_colwise(_index_weight(case["D"], 2), None, case["blocks"],
                                            case["P"], 0)


@pytest.mark.parametrize("H,hd,P", [(24, 4, 4), (48, 2, 8), (6, 3, 2), (5, 2, 1)])
def test_qkv_split_owns_whole_heads_and_equals_packed_111(H, hd, P):
    d, k = 3 * H * hd, 2
    w = np.arange(d * k, dtype=np.uint32).astype(np.uint16).reshape(d, k)
    for r in range(P):
        ws, _ = oracle.qkv_split(w, None, H, hd, P, r)
        wp, _ = oracle.shard_packed_colwise(w, None, [1, 1, 1], P, r)
        assert np.array_equal(ws, wp)
        src_rows = ws[:, 0].astype(np.int64) // k
        which, rem = np.divmod(src_rows, H * hd)
        heads = rem // hd
        assert np.array_equal(which, np.repeat([0, 1, 2], H // P * hd))
        assert heads.min() >= r * H // P and heads.max() < (r + 1) * H // P


def test_naive_colwise_on_fused_qkv_misaligns():
    """[TP] "Fused projections": a plain slice cuts across the packed blocks."""
    H, hd, P = 4, 2, 2
    w = _index_weight(3 * H * hd, 2)
    naive, _ = oracle.shard_colwise(w, None, P, 0)
    head_aligned, _ = oracle.qkv_split(w, None, H, hd, P, 0)
    assert not np.array_equal(naive, head_aligned)


@pytest.mark.parametrize("blocks,P", [(None, 4), ([1, 1, 1], 4), ([1, 1], 2), ([1, 1, 1, 3, 3], 2)])
def test_concat_inverts_packed_colwise_slicing(blocks, P):
    """Head-aligned / packed slices reconstruct the fused weight exactly: gather the per-rank
    row slices back through the concat map (rows of W are output columns of y)."""
    unit = 4 * P
    d = unit * (3 if blocks is None else sum(blocks))
    k = 5
    w = _index_weight(d, k)
    shards = []
    for r in range(P):
        if blocks is None:
            ws, _ = oracle.shard_colwise(w, None, P, r)
        else:
            ws, _ = oracle.shard_packed_colwise(w, None, blocks, P, r)
        shards.append(np.ascontiguousarray(ws.T))
    back = oracle.combine_concat(shards, blocks)
    assert np.array_equal(back.T, w)


def test_plan_validation_rules():
    ok = [("colwise", 4, 3, 8, 2, None, None), ("rowwise", 2, 1, 3, 4, None, None),
          ("qkv", 8, 7, 3 * 48 * 128, 6144, None, 48), ("colwise", 2, 0, 18, 1, [1, 1, 1, 3, 3], None)]
    for style, P, r, n, k, bl, h in ok:
        oracle.check_plan(style, P, r, n, k, blocks=bl, num_heads=h)
    bad = [("colwise", 0, 0, 8, 8, None, None), ("colwise", 4, 4, 8, 8, None, None),
           ("colwise", 3, 0, 8, 8, None, None), ("rowwise", 3, 0, 9, 8, None, None),
           ("qkv", 5, 0, 3 * 48 * 2, 4, None, 48), ("colwise", 4, 0, 8, 1, [1, 3], None),
           ("colwise", 2, 0, 8, 1, [1, 0, 1], None), ("colwise", -1, 0, 8, 8, None, None)]
    for style, P, r, n, k, bl, h in bad:
        with pytest.raises(oracle.PlanError):
            oracle.check_plan(style, P, r, n, k, blocks=bl, num_heads=h)


# --------------------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------------------

def test_combine_sum_integer_closed_form():
    m, n, P = 5, 7, 6
    i = np.arange(m, dtype=np.float32)[:, None]
    j = np.arange(n, dtype=np.float32)[None, :]
    parts = [(r + 1) * i + (r - 2) * j + r for r in range(P)]
    b = si.to_bf16_bits(np.arange(n, dtype=np.float32) - 3)
    got = oracle.combine_sum(parts, b)
    # sum_r (r+1) = 21, sum_r (r-2) = 3, sum_r r = 15
    want = 21 * i + 3 * j + 15 + (np.arange(n) - 3)[None, :]
    assert np.array_equal(got, want.astype(np.float32))


def test_combine_sum_fixed_order_by_hand():
    """Ascending-rank fp32 order decides: (1e8 + 1) - 1e8 = 0 in fp32 (ulp(1e8) = 8)."""
    p = [np.full((1, 1), v, np.float32) for v in (1e8, 1.0, -1e8)]
    assert oracle.combine_sum(p)[0, 0] == 0.0
    p = [np.full((1, 1), v, np.float32) for v in (1e8, -1e8, 1.0)]
    assert oracle.combine_sum(p)[0, 0] == 1.0


def test_combine_sum_close_to_exact_and_p1_identity():
    rng = np.random.default_rng(4)
    parts = [si.normal_f32(rng, (33, 65)) for _ in range(8)]
    b = si.normal_bf16(rng, (65,))
    got = oracle.combine_sum(parts, b).astype(np.float64)
    exact = np.sum([p.astype(np.float64) for p in parts], axis=0) + oracle.bf16_widen(b)
    mag = np.sum([np.abs(p.astype(np.float64)) for p in parts], axis=0) + np.abs(oracle.bf16_widen(b))
    assert np.all(np.abs(got - exact) <= _gamma(9, 2.0 ** -24) * mag)
    one = oracle.combine_sum(parts[:1], b)
    assert np.array_equal(one, parts[0] + oracle.bf16_widen(b).astype(np.float32))
    assert np.array_equal(oracle.combine_sum(parts[:1]), parts[0])


@pytest.mark.parametrize("dt", [np.uint16, np.float32])
def test_combine_concat_brute_force(dt):
    m, n_part, P = 3, 4, 3
    parts = [(np.arange(m * n_part).reshape(m, n_part) + 100 * r).astype(dt) for r in range(P)]
    got = oracle.combine_concat(parts)
    assert np.array_equal(got, np.concatenate(parts, axis=1))
    # packed [1,1] with P=2: shard r holds [gate_r | up_r]
    parts2 = [np.array([[10 * r + 0, 10 * r + 1, 10 * r + 2, 10 * r + 3]], dtype=dt) for r in range(2)]
    got2 = oracle.combine_concat(parts2, [1, 1])
    assert got2.tolist() == [[0, 1, 10, 11, 2, 3, 12, 13]]
