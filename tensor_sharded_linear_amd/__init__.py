"""tensor_sharded_linear_amd -- one rank's share of tensor-parallel linear layers on MI355X.

The compute lives in ``libtp_linear.so`` (hand-written HIP for gfx950, C ABI in
``include/tp_linear.h``); this package is its ctypes binding, with the same
entry-point names.  See the Hugging Face Diffusers "Tensor parallelism" page
for the method: colwise / rowwise sharding, head-aligned fused projections,
and the AllReduce / AllGather combine at the layer boundary.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    SIGNATURES,
    TPError,
    TPIOError,
    TPRuntimeError,
    TPValueError,
    load_library,
    tp_fused_qkv_split,
    tp_last_error,
    tp_linear_colwise,
    tp_linear_rowwise,
    tp_linear_rowwise_split_input,
    tp_linear_tile_shape,
    tp_load_shard,
    tp_load_shard_shape,
    tp_partial_combine,
    tp_plan_shard_shape,
    tp_plan_shard_slice,
)

__all__ = [
    "tp_linear_colwise", "tp_linear_rowwise", "tp_linear_rowwise_split_input", "tp_linear_tile_shape",
    "tp_fused_qkv_split", "tp_partial_combine",
    "tp_plan_shard_slice", "tp_plan_shard_shape", "tp_load_shard", "tp_load_shard_shape", "tp_last_error",
    "load_library", "TPError", "TPValueError", "TPRuntimeError", "TPIOError",
]
