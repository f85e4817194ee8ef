"""GPU parity of the index work: shard slicing, head-aligned fused-QKV split and
the CONCAT combine.  Bit-exact against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import bits_to_dev, dev_to_bits

pytestmark = pytest.mark.gpu


def _rand_bits(seed, shape):
    return si.random_bits(np.random.default_rng(seed), shape)


@pytest.mark.parametrize("o,i,P", [(1024, 256, 2), (64, 40, 4), (48, 24, 8), (16, 8, 1), (18, 10, 2)])
def test_shard_slice_colwise_rowwise_bit_exact(o, i, P):
    w = _rand_bits(o + i, (o, i))
    b = _rand_bits(o, (o,))
    wd, bd = bits_to_dev(w), bits_to_dev(b)
    for r in range(P):
        ws, bs = tsl.tp_plan_shard_slice(wd, bd, "colwise", P, r)
        rw, rb = oracle.shard_colwise(w, b, P, r)
        assert np.array_equal(dev_to_bits(ws), rw) and np.array_equal(dev_to_bits(bs), rb)
        if i % P == 0:
            wr, _ = tsl.tp_plan_shard_slice(wd, None, "rowwise", P, r)
            assert np.array_equal(dev_to_bits(wr), oracle.shard_rowwise(w, P, r))


@pytest.mark.parametrize("blocks,d,P", [([1, 1], 64, 2), ([1, 1], 64, 4), ([1, 1, 1, 3, 3], 36, 2),
                                        ([1, 1, 1], 48, 8), ([2, 1], 12, 2)])
def test_packed_colwise_slice_bit_exact(blocks, d, P):
    k = 24
    w = _rand_bits(d, (d, k))
    b = _rand_bits(d + 1, (d,))
    for r in range(P):
        ws, bs = tsl.tp_plan_shard_slice(bits_to_dev(w), bits_to_dev(b), "colwise", P, r, blocks=blocks)
        rw, rb = oracle.shard_packed_colwise(w, b, blocks, P, r)
        assert np.array_equal(dev_to_bits(ws), rw) and np.array_equal(dev_to_bits(bs), rb)


def test_packed_rowwise_slice_matches_column_view_of_packed_colwise():
    """Packed rowwise (blocks along in-features) is packed colwise on W^T."""
    o, i, P, blocks = 10, 24, 2, [1, 2]
    w = _rand_bits(5, (o, i))
    for r in range(P):
        ws, _ = tsl.tp_plan_shard_slice(bits_to_dev(w), None, "rowwise", P, r, blocks=blocks)
        ref, _ = oracle.shard_packed_colwise(np.ascontiguousarray(w.T), None, blocks, P, r)
        assert np.array_equal(dev_to_bits(ws), ref.T)


# (4, 2, 8, 4): one head per rank (P = H); (24, 128, 64, 1): P = 1 is the identity
@pytest.mark.parametrize("H,hd,K,P", [(24, 128, 3072, 4), (4, 2, 8, 2), (6, 8, 16, 3), (48, 128, 64, 8),
                                      (4, 2, 8, 4), (24, 128, 64, 1), (48, 128, 6144, 16)])
def test_qkv_split_bit_exact_and_roundtrip(H, hd, K, P):
    w = _rand_bits(H * hd + K, (3 * H * hd, K))
    b = _rand_bits(H, (3 * H * hd,))
    wd, bd = bits_to_dev(w), bits_to_dev(b)
    shards_t = []
    for r in range(P):
        ws, bs = tsl.tp_fused_qkv_split(wd, bd, H, hd, P, r)
        rw, rb = oracle.qkv_split(w, b, H, hd, P, r)
        assert np.array_equal(dev_to_bits(ws), rw)
        assert np.array_equal(dev_to_bits(bs), rb)
        shards_t.append(ws.t().contiguous())
    # rows of W are output features: concat (blocks [1,1,1]) of the shards' transposes
    # rebuilds the fused weight exactly
    back = tsl.tp_partial_combine(shards_t, "concat", blocks=[1, 1, 1])
    assert np.array_equal(dev_to_bits(back.t().contiguous()), w)


def test_qkv_split_rejects_head_count_not_divisible():
    w = torch.zeros(3 * 6 * 4, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        tsl.tp_fused_qkv_split(w, None, 6, 4, 4, 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,n_part,P,blocks", [(64, 512, 2, None), (7, 48, 4, [1, 1, 1]),
                                               (33, 8, 2, [1, 1]), (5, 18, 2, [1, 1, 1, 3, 3]),
                                               (300, 2304, 8, [1, 1, 1]), (1, 4, 16, None),
                                               (16, 64, 1, None), (9, 6, 1, [1, 1, 1])])
def test_concat_bit_exact(dtype, M, n_part, P, blocks):
    rng = np.random.default_rng(M * n_part + P)
    if dtype == torch.bfloat16:
        parts = [si.random_bits(rng, (M, n_part)) for _ in range(P)]
        dev = [bits_to_dev(p) for p in parts]
    else:
        parts = [si.normal_f32(rng, (M, n_part)) for _ in range(P)]
        dev = [torch.from_numpy(p).cuda() for p in parts]
    out = tsl.tp_partial_combine(dev, "concat", blocks=blocks)
    ref = oracle.combine_concat(parts, blocks)
    got = dev_to_bits(out) if dtype == torch.bfloat16 else out.cpu().numpy()
    assert got.dtype == ref.dtype and np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def test_concat_strided_parts_and_padded_output():
    M, n_part, P = 9, 24, 3
    rng = np.random.default_rng(1)
    big = [si.random_bits(rng, (M, 40)) for _ in range(P)]
    dev = [bits_to_dev(b)[:, 8:8 + n_part] for b in big]
    out_big = torch.zeros(M, 80, dtype=torch.bfloat16, device="cuda")
    out = out_big[:, :P * n_part]
    tsl.tp_partial_combine(dev, "concat", out=out)
    ref = oracle.combine_concat([np.ascontiguousarray(b[:, 8:8 + n_part]) for b in big])
    assert np.array_equal(dev_to_bits(out), ref)
    assert torch.count_nonzero(out_big[:, P * n_part:].float()) == 0
