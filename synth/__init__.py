"""Seeded synthetic inputs (no operator arithmetic) shared by tests, bench and smoke."""
from .configs import WORKLOADS, Workload, SEED_BASE  # noqa: F401
from .planted import (prefill_inputs, decode_inputs, round_to, to_f64,  # noqa: F401
                      f64_to_bf16_bits, bf16_bits_to_f64, sharpness)
