"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers: it holds none of the method's arithmetic (no
slicing, no products, no combine, no activation).  Both the CPU oracle and the
HIP library are fed from it; neither is imported here.

Recipe (the workloads are diffusion-transformer linear layers at the shapes
the tensor-parallel pages discuss; no dataset or checkpoint is involved):
  * ``numpy.random.default_rng(seed).standard_normal(shape, dtype=float32)``,
    arrays drawn in the order listed per workload;
  * weights are nn.Linear ``W[out, in]`` scaled by ``1/sqrt(in)`` of the
    *unsharded* layer (full weights are drawn, then sliced);
  * activations and biases are N(0, 1);
  * every array is then rounded to bf16 by torch's CPU conversion (round to
    nearest even) and returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import functools
import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

# --------------------------------------------------------------------------------------
# primitive draws
# --------------------------------------------------------------------------------------


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) via torch's CPU conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return to_bf16_bits(a)


def int_bf16(rng: np.random.Generator, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers in [lo, hi], exactly representable in bf16."""
    return to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


def random_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """Arbitrary uint16 patterns (for bit-exact copy tests)."""
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def normal_f32(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def checksum(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


# --------------------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------------------


@dataclass
class Workload:
    name: str
    seed: int
    tp: tuple            # tp degrees exercised
    arrays: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)


def _draw(seed, spec):
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape, scale in spec:
        out[name] = normal_bf16(rng, shape, scale)
    return out


def tiny_mlp() -> Workload:
    """Tiny MLP pair at P=2: x[64,256]; W1[1024,256], b1[1024]; W2[256,1024], b2[256]. Seed 0."""
    spec = [("x", (64, 256), 1.0),
            ("w1", (1024, 256), 1.0 / np.sqrt(256.0)),
            ("b1", (1024,), 1.0),
            ("w2", (256, 1024), 1.0 / np.sqrt(1024.0)),
            ("b2", (256,), 1.0)]
    return Workload("tiny_mlp_p2", 0, (2,), _draw(0, spec),
                    dict(M=64, hidden=256, ffn=1024))


def attention_proj() -> Workload:
    """Attention projections at P=4: hidden 3072, 24 heads x 128, 4608 tokens. Seed 1.
    x[4608,3072]; W_qkv[9216,3072]; A[4608,3072] (attention output); W_o[3072,3072]."""
    s = 1.0 / np.sqrt(3072.0)
    spec = [("x", (4608, 3072), 1.0), ("w_qkv", (9216, 3072), s),
            ("a", (4608, 3072), 1.0), ("w_o", (3072, 3072), s)]
    return Workload("attn_proj_h3072_p4", 1, (4,), _draw(1, spec),
                    dict(M=4608, hidden=3072, heads=24, head_dim=128))


def mlp_large() -> Workload:
    """MLP at P=4: hidden 6144, FFN 18432, 4608 tokens. Seed 2. x; W1[18432,6144]; W2[6144,18432]."""
    spec = [("x", (4608, 6144), 1.0),
            ("w1", (18432, 6144), 1.0 / np.sqrt(6144.0)),
            ("w2", (6144, 18432), 1.0 / np.sqrt(18432.0))]
    return Workload("mlp_h6144_f18432_p4", 2, (4,), _draw(2, spec),
                    dict(M=4608, hidden=6144, ffn=18432))


def full_block() -> Workload:
    """Full-block linear set, P in {2,4,8}: hidden 6144, 48 heads x 128, FFN 18432, 4608 tokens.
    Seed 3.  x; A; W_qkv[18432,6144]; W_o[6144,6144]; W1[18432,6144]; W2[6144,18432]."""
    s_h = 1.0 / np.sqrt(6144.0)
    spec = [("x", (4608, 6144), 1.0), ("a", (4608, 6144), 1.0),
            ("w_qkv", (18432, 6144), s_h), ("w_o", (6144, 6144), s_h),
            ("w1", (18432, 6144), s_h), ("w2", (6144, 18432), 1.0 / np.sqrt(18432.0))]
    return Workload("dit_block_h6144_p2_4_8", 3, (2, 4, 8), _draw(3, spec),
                    dict(M=4608, hidden=6144, heads=48, head_dim=128, ffn=18432))


def adaln() -> Workload:
    """Skinny adaLN modulation at P=4: c[4,6144]; W_ada[36864,6144]. Seed 4."""
    spec = [("c", (4, 6144), 1.0), ("w_ada", (36864, 6144), 1.0 / np.sqrt(6144.0))]
    return Workload("adaln_6144x36864_p4", 4, (4,), _draw(4, spec),
                    dict(hidden=6144, out=36864))


def swiglu_ffn() -> Workload:
    """FLUX.2-style fused gate/up projection of the FFN, packed with blocks [1, 1]:
    hidden 6144 -> 2 x 18432 (gate then up), 4608 tokens, P=4.  Seed 5.
    x; W_gu[36864,6144]; b_gu[36864]."""
    spec = [("x", (4608, 6144), 1.0), ("w_gu", (36864, 6144), 1.0 / np.sqrt(6144.0)),
            ("b_gu", (36864,), 1.0)]
    return Workload("swiglu_ffn_h6144_f18432_p4", 5, (4,), _draw(5, spec),
                    dict(M=4608, hidden=6144, ffn=18432))


WORKLOADS = {
    "tiny_mlp": tiny_mlp,
    "attention_proj": attention_proj,
    "mlp_large": mlp_large,
    "full_block": full_block,
    "adaln": adaln,
    "swiglu_ffn": swiglu_ffn,
}


@functools.lru_cache(maxsize=2)
def workload(name: str) -> Workload:
    return WORKLOADS[name]()
