// moe_device.h -- device-side helpers shared by the HIP kernels of libmoe.
// (gfx950 / CDNA4: 64-lane wavefronts.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even.  NaN stays a
// quiet NaN with its sign; overflow rounds to +-inf.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x0040u;
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

// Order-preserving 32-bit code of a selection key: larger code = ahead.
// -0 and +0 share a code; every NaN maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t key_code(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0u;     // NaN
    if ((b & 0x7FFFFFFFu) == 0u) b = 0u;                 // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// 64-bit selection rank: key code, then lower expert index ahead.  Never 0
// for a real expert (the low word ~e is nonzero for e < 2^32 - 1), so 0 marks
// "taken" or "absent".
__device__ __forceinline__ uint64_t sel_rank(float key, int e) {
    return ((uint64_t)key_code(key) << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, m, kWave);
    hi = __shfl_xor(hi, m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace moe
