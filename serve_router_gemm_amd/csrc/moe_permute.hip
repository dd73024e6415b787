// moe_permute.hip -- expert histogram, offsets and the stable permutation.
//
// How many tokens each expert receives depends on every other token in the
// batch (Fireworks page "位级一致：前沿训练的差异化关键", section
// "为什么比特级一致是一个复杂的问题").  That count may change launch work but
// must never change a token's arithmetic; the permutation itself is pure
// integer work and deterministic: assignments a = t*k + j are grouped by
// expert and kept in ascending a inside each expert (a stable counting sort).
//
// Three launches (one for small batches, below), no atomics whose winner
// decides a position:
//   hist    one block per chunk of assignments: per-chunk expert counts
//           (LDS integer atomics: the count does not depend on their order)
//   scan    one block: per expert, exclusive prefix over chunks; counts;
//           exclusive prefix over experts -> offsets; chunk bases
//   scatter one wave per chunk, 64 assignments per step in order: lanes with
//           the same expert find each other by ballots over the expert-id
//           bits, the rank inside the step is a popcount of the lower lanes
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kHistThreads = 256;
constexpr int kMaxExperts = 512;
constexpr int kExpertBits = 9;   // ids < 512
constexpr int kScanBatch = 64;   // chunk counts loaded together in the scan (against 16:
                                 // A = 131072 permute 39.8 -> 38.6 us, A = 2^21 142 -> 128 us)

__global__ __launch_bounds__(kHistThreads) void permute_hist_kernel(
    int A, int E, int chunk, const int32_t* __restrict__ ids, int32_t* __restrict__ bh) {
    __shared__ int hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kHistThreads) hist[e] = 0;
    __syncthreads();
    const int a0 = blockIdx.x * chunk;
    const int a1 = min(A, a0 + chunk);
    for (int a = a0 + threadIdx.x; a < a1; a += kHistThreads) {
        const int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kHistThreads) bh[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of kMaxExperts threads.  bh[b][e] becomes the first permuted
// position of chunk b's assignments to expert e.
__global__ __launch_bounds__(kMaxExperts) void permute_scan_kernel(
    int E, int nchunks, int32_t* __restrict__ bh, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets) {
    __shared__ int sc[kMaxExperts];
    const int e = threadIdx.x;
    // The chunk counts of an expert are read kScanBatch at a time, so that
    // their loads are in flight together rather than one after another.
    int run = 0;
    if (e < E)
        for (int b0 = 0; b0 < nchunks; b0 += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u)
                v[u] = (b0 + u < nchunks) ? bh[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u)
                if (b0 + u < nchunks) {
                    bh[(size_t)(b0 + u) * E + e] = run;
                    run += v[u];
                }
        }
    sc[e] = (e < E) ? run : 0;
    __syncthreads();
    // inclusive scan over experts (Hillis-Steele on integers: exact)
    for (int d = 1; d < kMaxExperts; d <<= 1) {
        const int v = (e >= d) ? sc[e - d] : 0;
        __syncthreads();
        sc[e] += v;
        __syncthreads();
    }
    const int excl = sc[e] - ((e < E) ? run : 0);
    if (e < E) {
        counts[e] = run;
        offsets[e] = excl;
        for (int b0 = 0; b0 < nchunks; b0 += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u)
                v[u] = (b0 + u < nchunks) ? bh[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u)
                if (b0 + u < nchunks) bh[(size_t)(b0 + u) * E + e] = v[u] + excl;
        }
    }
    if (e == E - 1) offsets[E] = sc[e];
}

__global__ __launch_bounds__(kWave) void permute_scatter_kernel(
    int A, int E, int chunk, const int32_t* __restrict__ ids, const int32_t* __restrict__ bh,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
    __shared__ int base[kMaxExperts];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) base[e] = bh[(size_t)blockIdx.x * E + e];
    __syncthreads();
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int a0 = blockIdx.x * chunk;
    const int a1 = min(A, a0 + chunk);
    for (int s = a0; s < a1; s += kWave) {
        const int a = s + lane;
        const int e = (a < a1) ? ids[a] : -1;
        const bool valid = (e >= 0) && (e < E);
        uint64_t same = __ballot(valid);
        if (!valid) same = 0;
#pragma unroll
        for (int b = 0; b < kExpertBits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        const int rank = __popcll(same & lower);
        const int cnt = __popcll(same);
        int pos = -1;
        if (valid) pos = base[e] + rank;
        __syncthreads();
        if (valid && rank == cnt - 1) base[e] = pos + 1;
        __syncthreads();
        if (valid) perm[pos] = a;
        if (a < a1) inv_perm[a] = pos;
    }
}

// Small batches (A <= kSmallA assignments): the three steps above in one
// block of 16 waves, so a small step pays one launch for them.  Wave w takes
// the w-th chunk of `chunk` assignments (A / 16 rounded up to whole waves):
// per-wave histograms in LDS, then per expert the prefix over waves (the
// chunk bases) and the exclusive prefix over experts (offsets), then each
// wave places its chunk in order with the same ballot ranking.  Same
// permutation as the three launches.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;   // 16
constexpr int kSmallMaxChunk = 1024;
constexpr int kSmallA = kSmallWaves * kSmallMaxChunk;   // 16384

int small_chunk(int A) {
    const int per_wave = (A + kSmallWaves - 1) / kSmallWaves;
    return std::max(kWave, (per_wave + kWave - 1) / kWave * kWave);
}

__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    int A, int E, int chunk, const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
    __shared__ int hw[kSmallWaves][kMaxExperts];   // per-wave counts, then per-wave bases
    __shared__ int sc[kMaxExperts];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int i = tid; i < kSmallWaves * kMaxExperts; i += kSmallThreads) (&hw[0][0])[i] = 0;
    __syncthreads();
    const int a0 = wave * chunk;
    const int a1 = min(A, a0 + chunk);
    for (int a = a0 + lane; a < a1; a += kWave) {
        const int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&hw[wave][e], 1);
    }
    __syncthreads();
    // per expert: chunk bases relative to the expert's segment, and its count
    int run = 0;
    if (tid < kMaxExperts) {
        for (int w = 0; w < kSmallWaves; ++w) {
            const int v = hw[w][tid];
            hw[w][tid] = run;
            run += v;
        }
        sc[tid] = (tid < E) ? run : 0;
    }
    __syncthreads();
    for (int d = 1; d < kMaxExperts; d <<= 1) {
        int v = 0;
        if (tid < kMaxExperts && tid >= d) v = sc[tid - d];
        __syncthreads();
        if (tid < kMaxExperts) sc[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        const int excl = sc[tid] - run;
        counts[tid] = run;
        offsets[tid] = excl;
        for (int w = 0; w < kSmallWaves; ++w) hw[w][tid] += excl;
        if (tid == E - 1) offsets[E] = sc[tid];
    }
    __syncthreads();
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int s = a0; s < a1; s += kWave) {
        const int a = s + lane;
        const int e = (a < a1) ? ids[a] : -1;
        const bool valid = (e >= 0) && (e < E);
        uint64_t same = __ballot(valid);
        if (!valid) same = 0;
#pragma unroll
        for (int b = 0; b < kExpertBits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        const int rank = __popcll(same & lower);
        const int cnt = __popcll(same);
        int pos = -1;
        if (valid) pos = hw[wave][e] + rank;
        // the wave's own row of bases: lanes of one wave, no block barrier
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == cnt - 1) hw[wave][e] = pos + 1;
        __builtin_amdgcn_wave_barrier();
        if (valid) perm[pos] = a;
        if (a < a1) inv_perm[a] = pos;
    }
}

}  // namespace

int permute_chunk(int A) {
    // at most 1024 chunks, each a multiple of the wave width
    int c = 1024;
    while ((long)c * 1024 < (long)A) c *= 2;
    return c;
}

size_t permute_ws_bytes(int A, int E) {
    if (A <= kSmallA) return 0;
    const int chunk = permute_chunk(A);
    const int nchunks = (A + chunk - 1) / chunk;
    return (size_t)nchunks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute(int A, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv_perm, int32_t* ws, hipStream_t s) {
    if (A <= kSmallA) {
        permute_small_kernel<<<1, kSmallThreads, 0, s>>>(A, E, small_chunk(A), ids, counts,
                                                         offsets, perm, inv_perm);
        return hipGetLastError();
    }
    const int chunk = permute_chunk(A);
    const int nchunks = (A + chunk - 1) / chunk;
    permute_hist_kernel<<<nchunks, kHistThreads, 0, s>>>(A, E, chunk, ids, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    permute_scan_kernel<<<1, kMaxExperts, 0, s>>>(E, nchunks, ws, counts, offsets);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    permute_scatter_kernel<<<nchunks, kWave, 0, s>>>(A, E, chunk, ids, ws, perm, inv_perm);
    return hipGetLastError();
}

}  // namespace moe
