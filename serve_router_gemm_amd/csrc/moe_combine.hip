// moe_combine.hip -- fixed-order fp32 weighted combine of the top-k expert
// outputs.
//
// Both the precision and the execution order of weighting and summing the
// expert outputs must be pinned (Fireworks page on numerical alignment and MoE
// routing, section "混合专家模型更难对齐").  Here: acc starts at +0, one fp32
// fused multiply-add per slot in slot order j = 0..k-1, one bf16
// round-to-nearest-even at the end.  A token's k expert rows are adjacent in
// y (assignment order a = t*k + j), so each thread streams k float4 rows.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// All k loads of a thread are issued before its fma chain (KMAX >= k slots,
// unrolled), so each thread keeps k 16-byte loads in flight.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(int T, int H4, int k,
                                                      const float4* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      uint2* __restrict__ out) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)T * H4) return;
    const int t = (int)(idx / H4);
    const int h4 = (int)(idx - (long)t * H4);
    const float4* yt = y + (size_t)t * k * H4 + h4;
    const float* wt = w + (size_t)t * k;
    float4 v[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v r = __builtin_nontemporal_load(
                reinterpret_cast<const f4v*>(yt + (size_t)j * H4));
            v[j] = make_float4(r.x, r.y, r.z, r.w);
            wj[j] = wt[j];
        }
    }
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            a0 = __builtin_fmaf(wj[j], v[j].x, a0);
            a1 = __builtin_fmaf(wj[j], v[j].y, a1);
            a2 = __builtin_fmaf(wj[j], v[j].z, a2);
            a3 = __builtin_fmaf(wj[j], v[j].w, a3);
        }
    }
    uint2 o;
    o.x = f32_to_bf16_rne(a0) | (f32_to_bf16_rne(a1) << 16);
    o.y = f32_to_bf16_rne(a2) | (f32_to_bf16_rne(a3) << 16);
    out[idx] = o;
}

// Router replay may hand in expert ids outside [0,E); permute leaves those
// assignments unplaced (inv_perm = -1) and no GEMM writes their y rows.  They
// contribute nothing: their rows are set to 0 here (one block per row).
__global__ __launch_bounds__(256) void zero_unplaced_kernel(int H4, const int32_t* __restrict__ inv_perm,
                                                            float4* __restrict__ y) {
    const int a = blockIdx.x;
    if (inv_perm[a] >= 0) return;
    float4* row = y + (size_t)a * H4;
    for (int i = threadIdx.x; i < H4; i += 256) row[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_zero_unplaced(int A, int H, const int32_t* inv_perm, float* y, hipStream_t s) {
    zero_unplaced_kernel<<<A, 256, 0, s>>>(H / 4, inv_perm, reinterpret_cast<float4*>(y));
    return hipGetLastError();
}

hipError_t launch_combine(int T, int H, int k, const float* y, const float* w, uint16_t* out,
                          hipStream_t s) {
    const int H4 = H / 4;
    const long n = (long)T * H4;
    const int blocks = (int)((n + 255) / 256);
    const float4* y4 = reinterpret_cast<const float4*>(y);
    uint2* o2 = reinterpret_cast<uint2*>(out);
    if (k <= 8)
        combine_kernel<8><<<blocks, 256, 0, s>>>(T, H4, k, y4, w, o2);
    else
        combine_kernel<16><<<blocks, 256, 0, s>>>(T, H4, k, y4, w, o2);
    return hipGetLastError();
}

}  // namespace moe
