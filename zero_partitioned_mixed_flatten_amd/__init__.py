"""MI355X-native ZeRO partitioned mixed-precision Adam shard step.

The computation is HIP kernels for gfx950 behind the C ABI declared in
include/zero_mi355x.h (libzero_mi355x.so, built in-tree); this package is the
ctypes binding with the same entry-point names plus a small helper that wires
them to torch-owned device buffers.  Importing it loads the library and fails
loudly if it has not been built -- there is no CPU fallback.
"""
from ._lib import (EXPORTS, NORM_PARTIAL_BYTES, ONEBIT_STATE_BYTES, STATE_BYTES, ZERO_F16, ZERO_F32, BucketPlan,
                   HParams, OneBitState, Segment, StepState, read_onebit_state, zero_onebit_state_init,
                   zero_onebit_step, zero_onebit_workspace_bytes,
                   ZeroError, lib, make_segments, read_state, zero_bucket_segments, zero_decide_workspace_bytes,
                   zero_flatten_bucket, zero_flatten_buckets, zero_flatten_norm_bucket,
                   zero_flatten_norm_bucket_f32, zero_flatten_norm_partials, zero_norm_workspace_bytes, zero_shard_adam_step,
                   zero_shard_adam_step_f32, zero_shard_decide, zero_shard_decide_f32, zero_shard_norm_overflow,
                   zero_shard_norm_overflow_f32, zero_shard_norm_overflow_noalloc, zero_state_bytes,
                   zero_status_string, zero_step_state_init,
                   zero_stream_copy, zero_host_create, zero_host_destroy, zero_host_threads, zero_host_state_init,
                   zero_host_norm_overflow, zero_host_adam_step, zero_offload_step, zero_host_stream_copy)
from .stepper import AccumStep, HostContext, OffloadStep, OneBitStep, ShardStep, hparams

lib()

__all__ = ["EXPORTS", "NORM_PARTIAL_BYTES", "STATE_BYTES", "ZERO_F16", "ZERO_F32", "AccumStep", "BucketPlan", "HParams",
           "Segment", "ShardStep", "StepState", "ZeroError", "hparams", "lib", "make_segments", "read_state",
           "zero_bucket_segments", "zero_decide_workspace_bytes", "zero_flatten_bucket", "zero_flatten_buckets",
           "zero_flatten_norm_bucket", "zero_flatten_norm_bucket_f32", "zero_flatten_norm_partials",
           "zero_norm_workspace_bytes", "zero_shard_adam_step", "zero_shard_adam_step_f32", "zero_shard_decide", "zero_shard_decide_f32",
           "zero_shard_norm_overflow", "zero_shard_norm_overflow_f32", "zero_shard_norm_overflow_noalloc",
           "zero_state_bytes", "zero_status_string",
           "zero_step_state_init", "zero_stream_copy", "HostContext", "OffloadStep", "zero_host_create",
           "zero_host_destroy", "zero_host_threads", "zero_host_state_init", "zero_host_norm_overflow",
           "zero_host_adam_step", "zero_offload_step", "zero_host_stream_copy", "ONEBIT_STATE_BYTES", "OneBitState",
           "OneBitStep", "read_onebit_state", "zero_onebit_state_init", "zero_onebit_step",
           "zero_onebit_workspace_bytes"]
