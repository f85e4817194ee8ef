"""Sharded checkpoint loading, host side (CPU only).

[TP] "Load a sharded model": the checkpoint is cut as it is read, each rank
reading only its own slice of each weight.  [TP] "Limitations": the sharded
load takes safetensors files only.

Pins of the oracle's reader and slicer, and the library's header parsing,
shape queries and error paths.  No call here reaches the device: every
``tp_load_shard`` call is a shape query (no destination) or fails validation.
The checkpoints are written by the ``safetensors`` library itself, so the
oracle's reader (written from the format's definition) is checked against an
independent implementation of the format.
"""
import json
import os
import struct

import numpy as np
import pytest
import torch
from safetensors.torch import load_file, save_file

import oracle
import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from tensor_sharded_linear_amd import _binding as B


def _bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _write(path, tensors):
    save_file(tensors, str(path))
    return str(path)


@pytest.fixture
def ckpt(tmp_path):
    rng = np.random.default_rng(11)
    t = {
        "w_bf16": _bf16(si.random_bits(rng, (48, 40))),
        "w_f32": torch.from_numpy(rng.integers(0, 1 << 32, size=(24, 16), dtype=np.uint32).view(np.float32)),
        "bias": _bf16(si.random_bits(rng, (48,))),
        "bias_f32": torch.from_numpy(si.normal_f32(rng, (24,))),
        "qkv": _bf16(si.random_bits(rng, (3 * 8 * 4, 12))),
        "row1": _bf16(si.random_bits(rng, (1, 32))),
    }
    return _write(tmp_path / "ckpt.safetensors", t), t


def _index_f32(shape):
    """Element value = its flat index (exact in fp32 below 2^24)."""
    return np.arange(int(np.prod(shape)), dtype=np.float32).reshape(shape)


# ---------------------------------------------------------------------------------------
# oracle pins
# ---------------------------------------------------------------------------------------

def test_oracle_reader_matches_the_safetensors_library(ckpt):
    path, t = ckpt
    lib = load_file(path)
    for name in t:
        arr, dt = oracle.read_safetensors(path, name)
        ref = lib[name]
        assert dt == {torch.bfloat16: "BF16", torch.float32: "F32"}[ref.dtype]
        got = torch.from_numpy(arr.view(np.int16) if dt == "BF16" else arr.view(np.int32))
        want = ref.view(torch.int16) if dt == "BF16" else ref.view(torch.int32)
        assert tuple(arr.shape) == tuple(ref.shape) and torch.equal(got, want), name


def test_oracle_load_shard_is_numpy_slicing_of_index_tensors(tmp_path):
    """Index-valued tensors: every shard element names its source position, checked
    against plain numpy slicing of the full tensor (the definition of each cut)."""
    w = _index_f32((24, 36))
    b = _index_f32((24,))
    path = _write(tmp_path / "idx.safetensors", {"w": torch.from_numpy(w), "b": torch.from_numpy(b),
                                                  "wb": torch.from_numpy(w).to(torch.bfloat16)})
    for P in (1, 2, 3, 4, 6):
        for r in range(P):
            s, _ = oracle.load_shard(path, "w", "colwise", P, r)
            assert np.array_equal(s, w[r * 24 // P:(r + 1) * 24 // P])
            s, _ = oracle.load_shard(path, "w", "rowwise", P, r)
            assert np.array_equal(s, w[:, r * 36 // P:(r + 1) * 36 // P])
            s, _ = oracle.load_shard(path, "w", "rowwise_split_input", P, r)
            assert np.array_equal(s, w[:, r * 36 // P:(r + 1) * 36 // P])
            s, _ = oracle.load_shard(path, "b", "colwise", P, r)
            assert np.array_equal(s, b[r * 24 // P:(r + 1) * 24 // P])
    # packed [1, 1, 1] (Q, K, V of 8 rows each) at P = 2: rank 1 takes rows 4-7 of each block
    s, _ = oracle.load_shard(path, "w", "colwise", 2, 1, blocks=[1, 1, 1])
    assert np.array_equal(s, np.concatenate([w[4:8], w[12:16], w[20:24]]))
    # packed [1, 2] along in-features (rowwise): blocks of 12 and 24 columns, P = 2, rank 0
    s, _ = oracle.load_shard(path, "w", "rowwise", 2, 0, blocks=[1, 2])
    assert np.array_equal(s, np.concatenate([w[:, 0:6], w[:, 12:24]], axis=1))
    # a packed bias is cut like the rows of its weight
    s, _ = oracle.load_shard(path, "b", "colwise", 2, 1, blocks=[1, 1, 1])
    assert np.array_equal(s, np.concatenate([b[4:8], b[12:16], b[20:24]]))
    # bf16 bit patterns follow the same map
    s, dt = oracle.load_shard(path, "wb", "rowwise", 4, 2)
    wb = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert dt == "BF16" and np.array_equal(s, wb[:, 18:27])


def test_oracle_shards_reassemble_the_tensor(ckpt):
    path, t = ckpt
    full, _ = oracle.read_safetensors(path, "w_bf16")
    for P in (1, 2, 4, 8):
        assert np.array_equal(np.concatenate([oracle.load_shard(path, "w_bf16", "colwise", P, r)[0]
                                              for r in range(P)]), full)
        assert np.array_equal(np.concatenate([oracle.load_shard(path, "w_bf16", "rowwise", P, r)[0]
                                              for r in range(P)], axis=1), full)
    # the head-aligned QKV shard equals the oracle's QKV split
    qkv, _ = oracle.read_safetensors(path, "qkv")
    for r in range(4):
        s, _ = oracle.load_shard(path, "qkv", "colwise", 4, r, blocks=[1, 1, 1])
        assert np.array_equal(s, oracle.qkv_split(qkv, None, 8, 4, 4, r)[0])


# ---------------------------------------------------------------------------------------
# library: shape queries (header parsing only)
# ---------------------------------------------------------------------------------------

CASES = [("w_bf16", "colwise", 4, None), ("w_bf16", "rowwise", 8, None), ("w_bf16", "rowwise_split_input", 2, None),
         ("w_bf16", "colwise", 2, [1, 1, 1]), ("w_bf16", "rowwise", 2, [1, 1]), ("w_f32", "colwise", 8, None),
         ("w_f32", "rowwise", 4, None), ("bias", "colwise", 4, [1, 2]), ("bias_f32", "colwise", 1, None),
         ("qkv", "colwise", 8, [1, 1, 1]), ("row1", "rowwise", 4, None)]


@pytest.mark.parametrize("name,style,P,blocks", CASES)
def test_shape_query_matches_the_oracle(ckpt, name, style, P, blocks):
    path, t = ckpt
    for r in range(P):
        rows, cols, dt = tsl.tp_load_shard_shape(path, name, style, P, r, blocks=blocks)
        ref, rdt = oracle.load_shard(path, name, style, P, r, blocks=blocks)
        shape = (1, ref.shape[0]) if ref.ndim == 1 else ref.shape
        assert (rows, cols) == shape
        assert dt == {"BF16": torch.bfloat16, "F32": torch.float32}[rdt]


def test_query_reads_unicode_names_and_padded_headers(tmp_path):
    # a hand-built file: escaped and raw UTF-8 names, metadata, numbers with exponents in an
    # unrelated entry, and the trailing-space padding that writers use for alignment
    data = np.arange(12, dtype=np.float32).tobytes()
    header = {
        "__metadata__": {"format": "pt", "note": "café \"quoted\" \\ slash"},
        "blocks.0.wéight": {"dtype": "F32", "shape": [3, 4], "data_offsets": [0, 48]},
        "other": {"dtype": "F32", "shape": [0], "data_offsets": [48, 48], "extra": [1.5e3, -2, True, None]},
    }
    text = json.dumps(header, ensure_ascii=True).encode()  # non-ASCII as \\u escapes
    text += b" " * (-len(text) % 8)
    path = tmp_path / "hand.safetensors"
    path.write_bytes(struct.pack("<Q", len(text)) + text + data)
    assert tsl.tp_load_shard_shape(str(path), "blocks.0.wéight", "colwise", 3, 1) == (1, 4, torch.float32)
    # the same header with raw UTF-8 instead of escapes
    text = json.dumps(header, ensure_ascii=False).encode()
    path.write_bytes(struct.pack("<Q", len(text)) + text + data)
    assert tsl.tp_load_shard_shape(str(path), "blocks.0.wéight", "rowwise", 2, 0) == (3, 2, torch.float32)
    arr, _ = oracle.read_safetensors(str(path), "blocks.0.wéight")
    assert np.array_equal(arr, np.arange(12, dtype=np.float32).reshape(3, 4))


# ---------------------------------------------------------------------------------------
# library: errors (raised before any device work)
# ---------------------------------------------------------------------------------------

def _expect(path, name, style, P, r, status, **kw):
    with pytest.raises(tsl.TPError) as e:
        tsl.tp_load_shard_shape(path, name, style, P, r, **kw)
    assert e.value.status == status, (name, style, P, r, kw, str(e.value))
    return e.value


def test_rejects_bad_plans(ckpt):
    """[TP] "Constraints and verification": tp_degree divides the sharded dimension and
    every packed block, not only their sum; checked before any read of weight data."""
    path, _ = ckpt                      # w_bf16 is [48, 40], bias [48], qkv [96, 12]
    _expect(path, "w_bf16", "colwise", 0, 0, B.TP_ERR_INVALID_ARG)          # tp_degree 0
    _expect(path, "w_bf16", "colwise", 4, 4, B.TP_ERR_INVALID_ARG)          # rank outside [0, 4)
    _expect(path, "w_bf16", "colwise", 4, -1, B.TP_ERR_INVALID_ARG)
    _expect(path, "w_bf16", "colwise", 5, 0, B.TP_ERR_NOT_DIVISIBLE)        # 5 does not divide 48 rows
    _expect(path, "w_bf16", "rowwise", 3, 0, B.TP_ERR_NOT_DIVISIBLE)        # 3 does not divide 40 columns
    _expect(path, "w_bf16", "colwise", 2, 0, B.TP_ERR_NOT_DIVISIBLE, blocks=[1, 1, 1, 1, 1])  # 5 does not divide 48
    # blocks [1, 3] of 48 rows are 12 and 36 rows: 8 divides 48 but not the block of 12
    _expect(path, "w_bf16", "colwise", 8, 0, B.TP_ERR_NOT_DIVISIBLE, blocks=[1, 3])
    _expect(path, "w_bf16", "colwise", 2, 0, B.TP_ERR_INVALID_ARG, blocks=[0, 1])
    _expect(path, "w_bf16", "colwise", 2, 0, B.TP_ERR_INVALID_ARG, blocks=[1] * 17)  # at most 16 blocks
    _expect(path, "bias", "rowwise", 2, 0, B.TP_ERR_INVALID_ARG)            # a bias is cut colwise only
    _expect(path, "bias", "rowwise_split_input", 1, 0, B.TP_ERR_INVALID_ARG)
    _expect(path, "__metadata__", "colwise", 1, 0, B.TP_ERR_INVALID_ARG)
    with pytest.raises(ValueError):
        tsl.tp_load_shard_shape(path, "w_bf16", "diagonal", 1, 0)
    # the same plans that pass here pass the oracle's rules, and vice versa
    with pytest.raises(oracle.PlanError):
        oracle.load_shard(path, "w_bf16", "colwise", 8, 0, blocks=[1, 3])


def _raw(tmp_path, header_bytes: bytes, data: bytes = b"", length=None):
    path = tmp_path / "raw.safetensors"
    n = len(header_bytes) if length is None else length
    path.write_bytes(struct.pack("<Q", n) + header_bytes + data)
    return str(path)


def test_rejects_unreadable_and_malformed_files(tmp_path, ckpt):
    path, _ = ckpt
    io = B.TP_ERR_IO
    _expect(str(tmp_path / "missing.safetensors"), "w", "colwise", 1, 0, io)
    _expect(str(tmp_path), "w", "colwise", 1, 0, io)                          # a directory
    _expect(path, "no_such_tensor", "colwise", 1, 0, io)
    (tmp_path / "short").write_bytes(b"\x10\x00\x00")
    _expect(str(tmp_path / "short"), "w", "colwise", 1, 0, io)                # shorter than the length field
    good = json.dumps({"w": {"dtype": "F32", "shape": [2, 2], "data_offsets": [0, 16]}}).encode()
    data = bytes(16)
    _expect(_raw(tmp_path, good, data, length=len(good) + 17), "w", "colwise", 1, 0, io)  # header past the end
    _expect(_raw(tmp_path, good, data, length=0), "w", "colwise", 1, 0, io)   # empty header
    _expect(_raw(tmp_path, good[:-1], data), "w", "colwise", 1, 0, io)        # truncated JSON
    _expect(_raw(tmp_path, b"[1, 2]", data), "w", "colwise", 1, 0, io)        # not an object
    _expect(_raw(tmp_path, good + b"x", data), "w", "colwise", 1, 0, io)      # trailing garbage
    _expect(_raw(tmp_path, good, data[:8]), "w", "colwise", 1, 0, io)         # data shorter than the offsets
    for entry in ({"dtype": "F32", "shape": [2, 2], "data_offsets": [0, 12]},     # size does not match the shape
                  {"dtype": "F32", "shape": [2, 2], "data_offsets": [4, 0]},      # end before begin
                  {"dtype": "F32", "shape": [2, 2], "data_offsets": [0]},
                  {"dtype": "F32", "shape": [2, -2], "data_offsets": [0, 16]},
                  {"dtype": "F32", "shape": [2, 2.5], "data_offsets": [0, 16]},
                  {"dtype": 7, "shape": [2, 2], "data_offsets": [0, 16]},
                  {"shape": [2, 2], "data_offsets": [0, 16]}):
        _expect(_raw(tmp_path, json.dumps({"w": entry}).encode(), data), "w", "colwise", 1, 0, io)


def test_rejects_unsupported_tensors(tmp_path):
    t = {"h": torch.zeros(4, 4, dtype=torch.float16), "i": torch.zeros(4, 4, dtype=torch.int32),
         "cube": torch.zeros(2, 2, 2, dtype=torch.bfloat16), "s": torch.zeros((), dtype=torch.float32)}
    path = _write(tmp_path / "other.safetensors", t)
    for name in t:
        _expect(path, name, "colwise", 1, 0, B.TP_ERR_UNSUPPORTED)
    empty = json.dumps({"e": {"dtype": "BF16", "shape": [0, 4], "data_offsets": [0, 0]}}).encode()
    _expect(_raw(tmp_path, empty), "e", "colwise", 1, 0, B.TP_ERR_UNSUPPORTED)


def test_message_names_the_problem(ckpt):
    path, _ = ckpt
    e = _expect(path, "no_such_tensor", "colwise", 1, 0, B.TP_ERR_IO)
    assert "no_such_tensor" in str(e) and isinstance(e, OSError)
    e = _expect(path, "w_bf16", "colwise", 5, 0, B.TP_ERR_NOT_DIVISIBLE)
    assert "tp_degree=5" in str(e) and isinstance(e, ValueError)
