"""GPU parity of the sharded checkpoint load (tp_load_shard), bit-exact against the oracle.

[TP] "Load a sharded model": each rank reads only its own slice of each weight,
straight onto its GPU.  The checkpoints are written by the ``safetensors``
library; the oracle reads the whole tensor (``oracle.read_safetensors``) and cuts
it with its slicers (``oracle.load_shard``).
"""
import numpy as np
import pytest
import torch
from safetensors.torch import save_file

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl

pytestmark = pytest.mark.gpu


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _same(gpu: torch.Tensor, ref: np.ndarray) -> bool:
    got = _bits(gpu)
    if ref.dtype == np.float32:  # compare fp32 by bit pattern (NaN payloads included)
        return got.shape == ref.shape and np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    return got.shape == ref.shape and np.array_equal(got, ref)


@pytest.fixture(scope="module")
def small_ckpt(tmp_path_factory):
    rng = np.random.default_rng(21)
    t = {
        "w_bf16": _bf16(si.random_bits(rng, (96, 80))),
        "w_f32": torch.from_numpy(rng.integers(0, 1 << 32, size=(48, 24), dtype=np.uint32).view(np.float32)),
        "b_bf16": _bf16(si.random_bits(rng, (96,))),
        "b_f32": torch.from_numpy(si.normal_f32(rng, (48,))),
        "qkv": _bf16(si.random_bits(rng, (3 * 8 * 16, 64))),
        "fused": _bf16(si.random_bits(rng, (9 * 8, 32))),   # [1, 1, 1, 3, 3] of 8-row units
    }
    path = str(tmp_path_factory.mktemp("ckpt") / "small.safetensors")
    save_file(t, path)
    return path


SMALL = [("w_bf16", "colwise", None, (1, 2, 4, 8)), ("w_bf16", "rowwise", None, (1, 2, 4, 8)),
         ("w_bf16", "rowwise_split_input", None, (2, 4)), ("w_bf16", "colwise", [1, 1, 1], (2, 4)),
         ("w_bf16", "rowwise", [1, 3], (2, 4)), ("w_f32", "colwise", None, (1, 2, 4, 8)),
         ("w_f32", "rowwise", None, (2, 4, 8)), ("w_f32", "rowwise", [1, 2], (2, 4)),
         ("b_bf16", "colwise", None, (1, 2, 4)), ("b_bf16", "colwise", [1, 1, 1], (2, 4)),
         ("b_f32", "colwise", [1, 2], (2, 4, 8)), ("qkv", "colwise", [1, 1, 1], (1, 2, 4, 8)),
         ("fused", "colwise", [1, 1, 1, 3, 3], (2, 4, 8))]


@pytest.mark.parametrize("name,style,blocks,tps", SMALL)
def test_small_shards_bit_exact(small_ckpt, name, style, blocks, tps):
    for P in tps:
        for r in range(P):
            got = tsl.tp_load_shard(small_ckpt, name, style, P, r, blocks=blocks)
            ref, _ = oracle.load_shard(small_ckpt, name, style, P, r, blocks=blocks)
            assert _same(got, ref), (name, style, blocks, P, r)


def test_qkv_shard_owns_whole_heads(small_ckpt):
    """The packed [1, 1, 1] load of a fused QKV weight is the head-aligned split."""
    full, _ = oracle.read_safetensors(small_ckpt, "qkv")
    for P in (2, 4, 8):
        for r in range(P):
            got = tsl.tp_load_shard(small_ckpt, "qkv", "colwise", P, r, blocks=[1, 1, 1])
            assert _same(got, oracle.qkv_split(full, None, 8, 16, P, r)[0])


def test_given_output_and_stream(small_ckpt):
    s = torch.cuda.Stream()
    out = torch.full((24, 80), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    got = tsl.tp_load_shard(small_ckpt, "w_bf16", "colwise", 4, 3, out=out, stream=s)
    assert got.data_ptr() == out.data_ptr()
    # the call returns once the shard is on the device: no synchronisation needed before use
    ref, _ = oracle.load_shard(small_ckpt, "w_bf16", "colwise", 4, 3)
    assert _same(out, ref)


def test_short_destination_is_rejected_and_untouched(small_ckpt):
    from tensor_sharded_linear_amd import _binding as B
    lib = tsl.load_library()
    dst = torch.full((10,), 7, dtype=torch.int32, device="cuda")
    rows, cols, dt = tsl.tp_load_shard_shape(small_ckpt, "w_bf16", "colwise", 2, 0)
    st = lib.tp_load_shard(small_ckpt.encode(), b"w_bf16", B.TP_COLWISE, None, 0, 2, 0, dst.data_ptr(),
                           dst.numel() * 4, None, None, None, None)
    assert st == B.TP_ERR_INVALID_ARG and rows * cols * 2 > 40
    assert torch.equal(dst.cpu(), torch.full((10,), 7, dtype=torch.int32))
    with pytest.raises(ValueError):
        tsl.tp_load_shard(small_ckpt, "w_bf16", "colwise", 2, 0, out=torch.empty(48, 80, device="cuda"))


@pytest.fixture(scope="module")
def big_ckpt(tmp_path_factory):
    """A full-size FFN weight, [18432, 6144] bf16 (226 MB): every shard spans several
    32 MiB staging buffers, and a rowwise shard is 18432 separate byte ranges."""
    rng = np.random.default_rng(22)
    w = _bf16(si.random_bits(rng, (18432, 6144)))
    path = str(tmp_path_factory.mktemp("ckpt_big") / "ffn.safetensors")
    save_file({"ff.w1": w, "ff.b1": _bf16(si.random_bits(rng, (18432,)))}, path)
    return path


@pytest.mark.parametrize("style,blocks,P,r", [("colwise", None, 4, 1), ("rowwise", None, 4, 3),
                                              ("colwise", [1, 1], 8, 5), ("rowwise", None, 1, 0)])
def test_full_size_shard_bit_exact(big_ckpt, style, blocks, P, r):
    got = tsl.tp_load_shard(big_ckpt, "ff.w1", style, P, r, blocks=blocks)
    ref, _ = oracle.load_shard(big_ckpt, "ff.w1", style, P, r, blocks=blocks)
    assert _same(got, ref)
    b = tsl.tp_load_shard(big_ckpt, "ff.b1", "colwise", P, r, blocks=blocks)
    rb, _ = oracle.load_shard(big_ckpt, "ff.b1", "colwise", P, r, blocks=blocks)
    assert _same(b, rb)


@pytest.fixture(scope="module")
def tall_ckpt(tmp_path_factory):
    """A tall, narrow tensor: its rowwise shard at tp 8 is 150000 pieces of 4 bytes, more
    than one staging chunk takes, so the load cuts chunks by piece count as well as bytes."""
    rng = np.random.default_rng(23)
    path = str(tmp_path_factory.mktemp("ckpt_tall") / "tall.safetensors")
    save_file({"tall": _bf16(si.random_bits(rng, (150000, 16)))}, path)
    return path


@pytest.mark.parametrize("style,blocks,P,r", [("rowwise", None, 8, 0), ("rowwise", None, 8, 7),
                                              ("rowwise", [1, 3], 4, 2), ("colwise", None, 3, 1)])
def test_tall_tensor_many_pieces_bit_exact(tall_ckpt, style, blocks, P, r):
    got = tsl.tp_load_shard(tall_ckpt, "tall", style, P, r, blocks=blocks)
    ref, _ = oracle.load_shard(tall_ckpt, "tall", style, P, r, blocks=blocks)
    assert _same(got, ref)
