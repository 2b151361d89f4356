"""Seeded synthetic inputs shared by the oracle and the HIP path (no delta-rule arithmetic)."""
from .gen import (DeltaInputs, make_case, make_config, CONFIG_NAMES, make_epilogue_inputs,  # noqa: F401
                  f32_to_bf16_bits, bf16_bits_to_f32, to_f64)
