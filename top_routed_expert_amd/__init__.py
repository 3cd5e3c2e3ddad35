"""MI355X-native sparse Mixture-of-Experts FFN layer (Step 3.5 Flash style).

The compute path is libmoe.so: hand-written HIP kernels for gfx950 behind
the C ABI of include/moe.h (moe_route[_dynamic], moe_permute, moe_expert_gate_up,
moe_expert_down, moe_grouped_ffn, moe_combine, moe_layer_forward[_dynamic],
moe_pack_weights, moe_quantize_fp8, moe_route_group_stats, moe_ep_receive_plan,
moe_gather_rows, moe_layer_forward_noalloc).
This package is its Python binding.
"""
from .moe import (BF16, F32, LAYOUT_FP8, LAYOUT_PACKED, LAYOUT_ROWS, Config, MoeError, Workspace,  # noqa: F401
                  combine, ep_receive_plan, expert_down, expert_gate_up, fp8_weights_bytes, gather_rows, grouped_ffn,
                  layer_forward, layer_forward_noalloc, lib, noalloc_scratch_bytes, pack_layer, pack_weights, packed_weights_bytes, permute, quantize_fp8,
                  quantize_layer, route, route_group_stats, status_string, weights_struct)


def config_for(spec, packed: bool = False, fp8: bool = False) -> Config:
    """Config of a layer workload description with fields D, E, K, F, Fs and torch_dtype."""
    return Config(spec.D, spec.E, spec.K, spec.F, spec.Fs, spec.torch_dtype, spec.out_dtype, packed, fp8)
