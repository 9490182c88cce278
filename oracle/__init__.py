"""Reference oracle for the ZeRO partitioned mixed-precision Adam shard step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import, call or link anything here;
the HIP library and its Python binding never do, and this package imports
nothing from them.  The arithmetic is plain single-threaded C in
zero_oracle.c; zero_oracle.py only marshals numpy arrays.
"""
from .zero_oracle import (OracleHParams, OracleState, adam_update, adam_update_f32, decide,
                          f16_from_f32, f32_from_f16, flatten, hparams, lib, new_state,
                          norm_overflow, norm_overflow_f32, onebit_pack, onebit_scale, onebit_step,
                          state_bytes, step)

__all__ = ["OracleHParams", "OracleState", "adam_update", "adam_update_f32", "decide",
           "f16_from_f32", "f32_from_f16", "flatten", "hparams", "lib", "new_state",
           "norm_overflow", "norm_overflow_f32", "onebit_pack", "onebit_scale", "onebit_step", "state_bytes",
           "step"]
