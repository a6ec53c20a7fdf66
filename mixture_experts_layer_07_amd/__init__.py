"""MI355X (gfx950) MoE layer forward: route -> permute -> grouped GEMM FC1+SwiGLU ->
grouped GEMM FC2 -> weighted finalize, as hand-written HIP kernels behind the C
ABI in include/moe.h.  This package holds the in-tree library (libmoe.so), its
ctypes binding, a preallocating layer wrapper and the seeded workloads."""
from .binding import (BF16, F32, FP8_E4M3, ROUTE_DEEPSEEKV3, ROUTE_DEFAULT,  # noqa: F401
                      ROUTE_RENORMALIZE, ROUTE_RENORMALIZE_NAIVE, MoeError, alloc_workspace,
                      expert_ffn, expert_ffn_fp8, expert_ffn_fp8_fused, expert_ffn_fused,
                      expert_ffn_noalloc,
                      finalize, kernel_times, lib, permute,
                      quantize_fp8, route, timing_enable, workspace_size)
from .layer import MoELayer, layer_for_workload  # noqa: F401
