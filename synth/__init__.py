"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests
and the benchmark.  Holds workload sizes, random draws and storage encoders
only -- no step of the DFlash2 method is computed here."""
from .configs import Workload, WORKLOADS, TEST_WORKLOADS, get  # noqa: F401
from .generate import (Tensor, Layer, Weights, StepInputs, make_weights,  # noqa: F401
                       make_step_inputs, make_target_logits, make_verified_taps, make_selector_inputs,
                       make_integer_tables, make_selector_tables, accepted_draws, normal, encode,
                       make_sampling_inputs, make_uniforms)
