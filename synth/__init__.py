"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package only draws random numbers and describes workload shapes; it holds
none of the backward pass's arithmetic.  Both sides of every parity test take
their inputs from here (directly, or after the oracle's float64 forward turns
the draws into consistent saved activations).
"""
from .configs import CONFIGS, LayerConfig, LmHeadConfig, get_config  # noqa: F401
from .gen import draw_layer, draw_lm_head, draw_timing_layer, stream, TENSOR_IDS  # noqa: F401
