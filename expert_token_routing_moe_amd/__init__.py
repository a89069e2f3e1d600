"""MI355X-native MoE layer forward: route -> count/capacity -> dispatch
permute -> SwiGLU grouped GEMM -> combine, as hand-written HIP kernels for
gfx950 behind a C ABI (``include/moe.h``).  The Python side only marshals
arguments; import ``expert_token_routing_moe_amd.api`` for the calls.
"""
