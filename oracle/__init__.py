"""CPU oracle of the sparse-MoE FFN layer: test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
import this package. It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import LayerWeights, layer_forward, layer_rows  # noqa: F401
