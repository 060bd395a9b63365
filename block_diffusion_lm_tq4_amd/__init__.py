"""TQ4_1S ("Config-I") dequantize-and-multiply library for AMD MI355X (gfx950).

The kernels live in ``libtq4.so`` (C ABI in ``include/tq4.h``), built in-tree
by ``block_diffusion_lm_tq4_amd.build``.  ``ops`` is the torch-facing binding;
``inputs`` holds the seeded synthetic workloads.
"""

from .ops import (act_mxfp8, act_rht, codebook, fp8_cache, fp8_cache_experts,  # noqa: F401
                  linear, linear_epilogue, linear_epilogue_bf16, linear_fp8,
                  linear_fp8_quantized, linear_rotated, linear_workspace_size, moe_block,
                  moe_grouped, moe_grouped_fp8, moe_grouped_fp8_workspace_size, moe_route,
                  moe_router, moe_workspace_size, pack, packed_size)
