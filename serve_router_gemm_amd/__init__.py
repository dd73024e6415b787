"""Batch-invariant Mixture-of-Experts layer forward for AMD MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP, C ABI in include/moe.h);
`serve_router_gemm_amd.moe` is its thin torch binding and
`serve_router_gemm_amd.inputs` the seeded synthetic input generator.
"""
