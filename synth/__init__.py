"""Seeded synthetic inputs shared by the HIP library's tests/bench and the oracle."""
from .moe_inputs import (LayerSpec, LayerWeights, Matrix, WORKLOADS, WORKLOAD_TOKENS,  # noqa: F401
                         make_attention_residual, make_tokens, make_weights, quantize_u4_g64)
