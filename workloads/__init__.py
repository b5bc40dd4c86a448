"""Seeded synthetic inputs for block-sparse video attention (shared by the tests, the bench
and the oracle's calibration).  This package holds no arithmetic of the attention method:
no token reorder, pooling, scoring, routing or attention.  It only draws Q/K/V."""

from .gen import (CONFIGS, Config, get_config, gen_qkv, gen_qkv_steps, bf16_bits_from_f64,
                  f64_from_bf16_bits)

__all__ = ["CONFIGS", "Config", "get_config", "gen_qkv", "gen_qkv_steps", "bf16_bits_from_f64",
           "f64_from_bf16_bits"]
