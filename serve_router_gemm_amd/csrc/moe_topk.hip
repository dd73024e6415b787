// moe_topk.hip -- the large-k top-k of a sparse attention indexer: the top
// k (2048 on the pages) of every row of scores, exactly and in one order.
//
// A non-deterministic indexer top-k made the trainer attend to other tokens
// than the rollout did; the selected set depends on ties at the boundary,
// sort stability, NaN handling and the index dtype ("GLM Post-Training Beyond
// SFT", sections "DSA 的确定性为什么是 RL 问题" and "迁移到 NPU 时", and the
// sparse/version contract).  The order is the router top-k's: score
// descending, index ascending, -0 == +0, NaN below everything (NaNs by
// index).  It is a total order on (score, index), so the result is one
// well-defined list whatever the thread schedule.
//
// One 1024-thread block per row; each thread loads 16 scores of a batch
// before using them.  With n > k valid scores and k at most half of 4096:
// up to 4096 scores, sampled in 64-score chunks spread over the row, give by
// a two-level radix select on their codes a threshold that about 2k scores
// of the row should reach (fewer than 4096).  One read collects every score
// at or above it; when that is between k and 4096 scores (they hold the top
// k, since every score left out is below all of them), one sort of their
// ranks gives the list.  When the guess misses, or for larger k, a
// histogram of the top 11 code bits finds the bin that holds the k-th
// element; when that bin and the ones above it hold at most 4096 elements (no
// heavy ties), a second read collects them and the same sort follows.
// Otherwise:
//   1. radix select on the 32-bit order-preserving code, 8 bits per pass from
//      the top (LDS histograms, integer counts): the code c* of the k-th
//      element and kk, how many elements equal to c* are taken;
//   2. every element above c* is taken (LDS atomic slot; the slots are
//      sorted next, so their order does not matter), and the kk lowest
//      indices equal to c*, found by a block-wide scan in index order;
//   3. a bitonic sort of the k 64-bit ranks (code << 32 | ~index) in LDS,
//      descending.
// With n <= k every valid element is taken and sorted; the rest is -1.
// Which of these routes a row takes changes the work, never the list.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkU = 16;   // scores per thread per batch: element base + u * 1024 + tid
constexpr int kTkBatch = kTkThreads * kTkU;

constexpr int kTkTopBits = 11;                 // first pass: histogram of the top 11 code bits
constexpr int kTkTopBins = 1 << kTkTopBits;
constexpr int kTkTopShift = 32 - kTkTopBits;
constexpr int kTkSubShift = kTkTopShift - 8;    // second level: the next 8 code bits

constexpr int kTkSampleU = 4;                            // sample chunks per wave
constexpr int kTkSampleChunks = kTkWaves * kTkSampleU;   // 64 chunks of 64 scores

// wave 0 only: the highest bin b of h[0..NB) whose count from the top,
// sum over j >= b of h[j], reaches need (the total must reach it); writes
// *bin = b and *above = the sum over j > b.  Lane l sums bins [P l, P l + P)
// and a suffix scan over the lanes finds the group L; then lane j < P takes
// bin P L + j and a second suffix scan finds the bin inside the group.
__device__ __forceinline__ int suffix_sum_lanes(int x, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_down(x, d, kWave);
        if (lane + d < kWave) x += t;
    }
    return x;
}

template <int NB>
__device__ __forceinline__ void find_bin_from_top(const int* h, int need, int lane, int* bin,
                                                  int* above_out) {
    constexpr int P = NB / kWave;
    static_assert(P >= 1 && P <= kWave, "bins per lane");
    int g = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) g += h[lane * P + j];
    const int suf = suffix_sum_lanes(g, lane);
    const uint64_t reach = __ballot(suf >= need);            // non-increasing in lane
    const int L = 63 - __clzll((long long)reach);
    const int above_groups = __shfl(suf - g, L, kWave);      // elements in groups > L
    const int x = lane < P ? h[L * P + lane] : 0;
    const int suf2 = suffix_sum_lanes(x, lane);
    const uint64_t reach2 = __ballot(lane < P && above_groups + suf2 >= need);
    const int j = 63 - __clzll((long long)reach2);           // lane 0 always qualifies
    const int above = above_groups + __shfl(suf2 - x, j, kWave);
    if (lane == 0) {
        *bin = L * P + j;
        *above_out = above;
    }
}

// v[4 u + c] <- score base + 4 (u * 1024 + tid) + c of the row (0 past n):
// one 16-byte load where the row is 16-byte aligned and the four are inside
// it, four 4-byte loads otherwise.  For passes whose result does not depend
// on the order in which the scores are seen.
__device__ __forceinline__ int vec_index(int base, int w, int tid) {
    return base + 4 * ((w >> 2) * kTkThreads + tid) + (w & 3);
}

__device__ __forceinline__ void load_batch_vec(const float* __restrict__ row, int n, int base, int tid,
                                               bool aligned, float (&v)[kTkU]) {
#pragma unroll
    for (int u = 0; u < kTkU / 4; ++u) {
        const int i0 = base + 4 * (u * kTkThreads + tid);
        if (aligned && i0 + 3 < n) {
            const float4 f = *reinterpret_cast<const float4*>(row + i0);
            v[4 * u] = f.x;
            v[4 * u + 1] = f.y;
            v[4 * u + 2] = f.z;
            v[4 * u + 3] = f.w;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[4 * u + c] = i0 + c < n ? row[i0 + c] : 0.0f;
        }
    }
}

// The float whose order code is c (codes of NaN patterns give NaN).
__device__ __forceinline__ float code_to_float(uint32_t c) {
    return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

// Order code of -inf: a threshold above it is met exactly by the scores
// x >= code_to_float(thr) in IEEE order (denormals are kept, -0 == +0, NaN
// never passes); at or below it the code itself is compared.
constexpr uint32_t kCodeNegInf = 0x007FFFFFu;

// Loads of one collect batch: KFULL, the batch lies inside the row and the
// row is 16-byte aligned (no per-score bounds test).
template <bool KFULL>
__device__ __forceinline__ void collect_load(const float* __restrict__ row, int n, int base, int tid,
                                             bool aligned, float (&v)[kTkU]) {
    if (KFULL) {
#pragma unroll
        for (int u = 0; u < kTkU / 4; ++u) {
            const float4 f = *reinterpret_cast<const float4*>(row + base + 4 * (u * kTkThreads + tid));
            v[4 * u] = f.x;
            v[4 * u + 1] = f.y;
            v[4 * u + 2] = f.z;
            v[4 * u + 3] = f.w;
        }
    } else {
        load_batch_vec(row, n, base, tid, aligned, v);
    }
}

// The first batch of a collect, loaded ahead of it.
__device__ __forceinline__ void collect_preload(const float* __restrict__ row, int n, int tid,
                                                float (&v)[kTkU]) {
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    if (aligned && kTkBatch <= n) collect_load<true>(row, n, 0, tid, aligned, v);
    else collect_load<false>(row, n, 0, tid, aligned, v);
}

// One batch of collect_at_least, its scores already in v.
template <bool KFLOAT, bool KFULL>
__device__ __forceinline__ void collect_batch(const float (&v)[kTkU], int n, int base, uint32_t thr,
                                              float t, uint64_t* rk, int cap, int* fill, int tid,
                                              int lane) {
    bool c[kTkU];
    uint64_t m[kTkU];
    int tot = 0;
#pragma unroll
    for (int u = 0; u < kTkU; ++u) {
        c[u] = (KFLOAT ? (v[u] >= t) : (key_code(v[u]) >= thr)) &&
               (KFULL || vec_index(base, u, tid) < n);
        m[u] = __ballot(c[u]);
        tot += __popcll(m[u]);
    }
    if (tot == 0) return;
    int slot = 0;
    if (lane == 0) slot = atomicAdd(fill, tot);
    slot = __builtin_amdgcn_readfirstlane(slot);
    // ~index of v[u]: ~(base + 4 tid) minus the offset of slice u
    const uint32_t nbase = ~(uint32_t)(base + 4 * tid);
#pragma unroll
    for (int u = 0; u < kTkU; ++u) {
        if (m[u] == 0) continue;
        if (c[u]) {
            // slot + the number of lanes below this one that take slice u
            const int p = (int)__builtin_amdgcn_mbcnt_hi(
                (uint32_t)(m[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[u], (uint32_t)slot));
            const uint32_t ni = nbase - (uint32_t)(4 * (u >> 2) * kTkThreads + (u & 3));
            if (p < cap) rk[p] = ((uint64_t)__float_as_uint(v[u]) << 32) | ni;
        }
        slot += __popcll(m[u]);
    }
}

// Every valid score of the row whose code is at least thr gets a slot of rk,
// as (float bits << 32 | ~index) (the sort turns the bits into the code):
// one slot claim per wave per batch, slots at or past cap counted in *fill
// but not written.  The slot order depends on the schedule; the sort that
// follows removes it.  v0 holds the first batch (collect_preload).
__device__ __forceinline__ void collect_at_least(const float* __restrict__ row, int n, uint32_t thr,
                                                 uint64_t* rk, int cap, int* fill, int tid, int lane,
                                                 const float (&v0)[kTkU]) {
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    const float t = code_to_float(thr);
    for (int base = 0; base < n; base += kTkBatch) {
        const bool full = aligned && base + kTkBatch <= n;
        float v[kTkU];
        if (base == 0) {
#pragma unroll
            for (int u = 0; u < kTkU; ++u) v[u] = v0[u];
        } else if (full) {
            collect_load<true>(row, n, base, tid, aligned, v);
        } else {
            collect_load<false>(row, n, base, tid, aligned, v);
        }
        if (thr > kCodeNegInf) {
            if (full) collect_batch<true, true>(v, n, base, thr, t, rk, cap, fill, tid, lane);
            else collect_batch<true, false>(v, n, base, thr, t, rk, cap, fill, tid, lane);
        } else {
            collect_batch<false, false>(v, n, base, thr, t, rk, cap, fill, tid, lane);
        }
    }
}

// Lane l of the wave receives v from lane l ^ M (M a power of two below 64):
// DPP quad permutes for M = 1 and 2, ds_swizzle's bit mode (within 32 lanes)
// for 4 to 16, ds_bpermute for 32.  The whole wave must be active.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    static_assert(M >= 1 && M < kWave && (M & (M - 1)) == 0, "lane distance");
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    } else if constexpr (M < 32) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));
    } else {
        const int lane = (int)(threadIdx.x & (kWave - 1));
        return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ M) << 2, (int)v);
    }
}

template <int M>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v) {
    const uint32_t lo = lane_xor<M>((uint32_t)v), hi = lane_xor<M>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// One bitonic compare-exchange stage (block size, STRIDE) on the four ranks
// a thread holds: element j = 4 tid + e.  The pair (j, j ^ STRIDE) ends with
// the larger rank at the lower index inside blocks whose bit `size` of j is
// 0 (descending) and the other way round inside the others.  Strides 1 and 2
// pair a thread's own registers, strides 4 to 128 pair lanes of one wave.
// Then the stages of the strides below, down to 1.
template <int STRIDE>
__device__ __forceinline__ void bitonic_stages_regs(uint64_t (&a)[4], int size, int tid) {
    if constexpr (STRIDE >= 4) {
        constexpr int m = STRIDE >> 2;
        const bool keep_max = ((tid & m) == 0) == (((4 * tid) & size) == 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t b = lane_xor_u64<m>(a[e]);
            a[e] = ((a[e] < b) == keep_max) ? b : a[e];    // equal ranks: either
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e & STRIDE) continue;
            const int p = e | STRIDE;
            const bool desc = ((4 * tid + e) & size) == 0;
            const uint64_t lo = a[e], hi = a[p];
            const bool sw = (lo < hi) == desc;               // equal ranks: either
            a[e] = sw ? hi : lo;
            a[p] = sw ? lo : hi;
        }
    }
    if constexpr (STRIDE > 1) bitonic_stages_regs<STRIDE / 2>(a, size, tid);
}

// Bitonic sort of rk[0..P) descending, P a power of two in [256, 4096]
// (zeros, the padding, sink).  Entries come in as (float bits << 32 |
// ~index) and are sorted, and left, as (code << 32 | ~index).  Thread tid holds elements 4 tid .. 4 tid + 3
// in registers while the strides are below 256 (no barriers: those stages
// stay inside one wave); the stages of stride 256 and up pair elements of
// different waves and run on rk in LDS, one barrier each.  Waves whose
// elements are all at or past P skip the register stages (P is a multiple of
// the 256 elements a wave holds).
__device__ __forceinline__ void sort_ranks_desc(uint64_t* rk, int P, int tid) {
    const bool act = 4 * tid < P;
    uint64_t a[4] = {0, 0, 0, 0};
    if (act) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t r = rk[4 * tid + e];
            a[e] = r ? (((uint64_t)key_code(__uint_as_float((uint32_t)(r >> 32))) << 32) |
                        (r & 0xFFFFFFFFull))
                     : 0ull;
        }
        bitonic_stages_regs<1>(a, 2, tid);
        bitonic_stages_regs<2>(a, 4, tid);
        bitonic_stages_regs<4>(a, 8, tid);
        bitonic_stages_regs<8>(a, 16, tid);
        bitonic_stages_regs<16>(a, 32, tid);
        bitonic_stages_regs<32>(a, 64, tid);
        bitonic_stages_regs<64>(a, 128, tid);
        bitonic_stages_regs<128>(a, 256, tid);
#pragma unroll
        for (int e = 0; e < 4; ++e) rk[4 * tid + e] = a[e];
    }
    for (int size = 512; size <= P; size <<= 1) {
        __syncthreads();
        for (int stride = size >> 1; stride >= 256; stride >>= 1) {
            for (int t = tid; t < P / 2; t += kTkThreads) {
                const int i = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
                const int j = i + stride;
                const uint64_t x = rk[i], y = rk[j];
                if ((x < y) == ((i & size) == 0)) { rk[i] = y; rk[j] = x; }
            }
            __syncthreads();
        }
        if (act) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = rk[4 * tid + e];
            bitonic_stages_regs<128>(a, size, tid);
#pragma unroll
            for (int e = 0; e < 4; ++e) rk[4 * tid + e] = a[e];
        }
    }
    __syncthreads();
}

// Eight waves per SIMD: two blocks per CU, so one block's barriers and
// sort overlap the other's loads (the SGPRs this costs spill to VGPR lanes).
__global__ __launch_bounds__(kTkThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_large_kernel(
    int N, int k, const float* __restrict__ scores, const int32_t* __restrict__ lengths,
    int32_t* __restrict__ idx, float* __restrict__ vals) {
    __shared__ uint64_t rk[kMaxTopkLarge];
    __shared__ int hist[256];
    __shared__ int ucnt[kTkU * kTkWaves];   // equal-to-c* counts per (u, wave), then their prefix
    __shared__ int s_bin, s_above, s_fill, s_run, s_done, s_tot, s_nsamp;
    __shared__ int thist[kTkTopBins];

    const int q = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const float* row = scores + (size_t)q * N;
    int n = lengths ? lengths[q] : N;
    n = n < 0 ? 0 : (n > N ? N : n);
    const int take = min(k, n);
    int kp = 1;

    bool fast = false;
    int ncand = 0;
    if (n > k && 2 * k <= kMaxTopkLarge) {
        float v0[kTkU];
        // Sampled threshold.  Sample chunk c (c < nsc) is the 64 scores of
        // row chunk c * stride + rot, stride = nch / nsc and rot a hash of
        // the row index mod stride: the chunks spread evenly over the row
        // (all of it when nch <= 64), and rows whose starts are a power of
        // two apart do not all read the same offsets at once.
        for (int b = tid; b < kTkTopBins; b += kTkThreads) thist[b] = 0;
        for (int b = tid; b < 256; b += kTkThreads) hist[b] = 0;
        if (tid == 0) {
            s_fill = 0;
            s_nsamp = 0;
        }
        const int nch = (n + kWave - 1) / kWave;
        const int nsc = min(nch, kTkSampleChunks);
        const int stride = nch / nsc;
        const int rot = (int)((((uint32_t)q * 0x9E3779B1u) >> 16) % (uint32_t)stride);
        uint32_t sc[kTkSampleU];
        uint32_t sval = 0;
#pragma unroll
        for (int u = 0; u < kTkSampleU; ++u) {
            const int c = wave + kTkWaves * u;
            const int i = (c * stride + rot) * kWave + lane;
            const bool ok = c < nsc && i < n;
            sc[u] = ok ? key_code(row[i]) : 0u;
            sval |= (ok ? 1u : 0u) << u;
        }
        // the first batch of the collect is loaded while the sample is used
        collect_preload(row, n, tid, v0);
        __syncthreads();
        int ns = 0;
#pragma unroll
        for (int u = 0; u < kTkSampleU; ++u) {
            if (sval & (1u << u)) atomicAdd(&thist[sc[u] >> kTkTopShift], 1);
            ns += __popcll(__ballot((sval >> u) & 1u));
        }
        if (lane == 0) atomicAdd(&s_nsamp, ns);
        __syncthreads();
        // The sample rank r whose code should leave about T scores of the
        // row at or above it: T = 2k, but at least 64 samples' worth (the
        // relative spread of the count is about 1 / sqrt(r)) and at most
        // (k + 4096) / 2.  S, T <= 4096 and n <= 2^24: no overflow.
        const int S = s_nsamp;
        const int T = min(k + (kMaxTopkLarge - k) / 2, max(2 * k, (64 * n + S - 1) / S));
        const int r = max(1, min(S, (T * S + n - 1) / n));
        if (wave == 0) find_bin_from_top<kTkTopBins>(thist, r, lane, &s_bin, &s_above);
        __syncthreads();
        const uint32_t b1 = (uint32_t)s_bin;
        const int need2 = r - s_above;
#pragma unroll
        for (int u = 0; u < kTkSampleU; ++u)
            if ((sval & (1u << u)) && (sc[u] >> kTkTopShift) == b1)
                atomicAdd(&hist[(sc[u] >> kTkSubShift) & 255u], 1);
        __syncthreads();
        if (wave == 0) find_bin_from_top<256>(hist, need2, lane, &s_bin, &s_above);
        __syncthreads();
        const uint32_t thr = (b1 << kTkTopShift) | ((uint32_t)s_bin << kTkSubShift);
        collect_at_least(row, n, thr, rk, kMaxTopkLarge, &s_fill, tid, lane, v0);
        __syncthreads();
        ncand = s_fill;
        fast = ncand >= k && ncand <= kMaxTopkLarge;
        __syncthreads();   // every thread has read s_fill
    }
    if (n > k && !fast) {
        // Exact: a histogram of the top 11 code bits finds the bin b1 where
        // the count from the top reaches k; every element in b1 or above is
        // a candidate (at least k of them, the top k among them), and when
        // they fit in rk a second read collects them.
        for (int b = tid; b < kTkTopBins; b += kTkThreads) thist[b] = 0;
        __syncthreads();
        const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
        for (int base = 0; base < n; base += kTkBatch) {
            float v[kTkU];
            load_batch_vec(row, n, base, tid, aligned, v);
#pragma unroll
            for (int u = 0; u < kTkU; ++u)
                if (vec_index(base, u, tid) < n) atomicAdd(&thist[key_code(v[u]) >> kTkTopShift], 1);
        }
        __syncthreads();
        if (wave == 0) find_bin_from_top<kTkTopBins>(thist, k, lane, &s_bin, &s_above);
        __syncthreads();
        if (s_above + thist[s_bin] <= kMaxTopkLarge) {
            const uint32_t thr = (uint32_t)s_bin << kTkTopShift;
            __syncthreads();   // every thread has read s_bin
            if (tid == 0) s_fill = 0;
            __syncthreads();
            float v0[kTkU];
            collect_preload(row, n, tid, v0);
            collect_at_least(row, n, thr, rk, kMaxTopkLarge, &s_fill, tid, lane, v0);
            __syncthreads();
            ncand = s_fill;    // = the histogram's count
            fast = ncand >= k && ncand <= kMaxTopkLarge;
        }
    }
    __syncthreads();
    const int nrank = fast ? ncand : take;     // entries sorted
    kp = 256;                                  // the sort's size: at least 256
    while (kp < nrank) kp <<= 1;
    if (fast) {
        for (int i = ncand + tid; i < kp; i += kTkThreads) rk[i] = 0;
    } else {
        for (int i = tid; i < kp; i += kTkThreads) rk[i] = 0;
        if (tid == 0) s_fill = 0;
    }
    __syncthreads();

    if (!fast && n <= k) {
        for (int i = tid; i < n; i += kTkThreads) {
            const int pos = atomicAdd(&s_fill, 1);
            rk[pos] = ((uint64_t)__float_as_uint(row[i]) << 32) | (uint32_t)(~(uint32_t)i);
        }
    } else if (!fast) {
        // 1. radix select: prefix/mask describe the code bits fixed so far,
        //    need = how many of the elements matching them are still wanted.
        //    Each thread loads its kTkU scores of a batch before using them.
        uint32_t prefix = 0, mask = 0;
        int need = k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int b = tid; b < 256; b += kTkThreads) hist[b] = 0;
            __syncthreads();
            for (int base = 0; base < n; base += kTkBatch) {
                float v[kTkU];
#pragma unroll
                for (int u = 0; u < kTkU; ++u) {
                    const int i = base + u * kTkThreads + tid;
                    v[u] = i < n ? row[i] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < kTkU; ++u) {
                    const int i = base + u * kTkThreads + tid;
                    const uint32_t c = key_code(v[u]);
                    if (i < n && (c & mask) == prefix) atomicAdd(&hist[(c >> shift) & 255u], 1);
                }
            }
            __syncthreads();
            if (wave == 0) find_bin_from_top<256>(hist, need, lane, &s_bin, &s_above);
            __syncthreads();
            prefix |= (uint32_t)s_bin << shift;
            mask |= 255u << shift;
            need -= s_above;
            __syncthreads();
        }
        const uint32_t cstar = prefix;   // the k-th element's code; take `need` of them
        // 2. elements above c* (any slot order), then the `need` lowest
        //    indices equal to c*, in index order, after them.  Index order in
        //    a batch is (u, wave, lane): an element's rank among the equal ones
        //    is the prefix of the per-(u, wave) counts plus its lane prefix.
        if (tid == 0) s_run = 0;
        __syncthreads();
        const int base_eq = k - need;
        for (int base = 0; base < n; base += kTkBatch) {
            float v[kTkU];
#pragma unroll
            for (int u = 0; u < kTkU; ++u) {
                const int i = base + u * kTkThreads + tid;
                v[u] = i < n ? row[i] : 0.0f;
            }
            uint32_t eqbits = 0;
            int lpre[kTkU];
#pragma unroll
            for (int u = 0; u < kTkU; ++u) {
                const int i = base + u * kTkThreads + tid;
                const uint32_t c = key_code(v[u]);
                const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
                // elements above c*: one slot claim per wave
                const bool up = (i < n) && (c > cstar);
                const uint64_t ubal = __ballot(up);
                if (ubal) {
                    int slot0 = 0;
                    if (lane == 0) slot0 = atomicAdd(&s_fill, __popcll(ubal));
                    slot0 = __shfl(slot0, 0, kWave);
                    if (up) rk[slot0 + __popcll(ubal & below)] =
                        ((uint64_t)__float_as_uint(v[u]) << 32) | (uint32_t)(~(uint32_t)i);
                }
                const bool eq = (i < n) && (c == cstar);
                const uint64_t bal = __ballot(eq);
                lpre[u] = __popcll(bal & below);
                if (lane == 0) ucnt[u * kTkWaves + wave] = __popcll(bal);
                eqbits |= (eq ? 1u : 0u) << u;
            }
            __syncthreads();
            if (wave == 0) {
                // exclusive prefix of the 256 counts in (u, wave) order: lane
                // l holds entries 4l .. 4l + 3
                const int c0 = ucnt[4 * lane], c1 = ucnt[4 * lane + 1];
                const int c2 = ucnt[4 * lane + 2], c3 = ucnt[4 * lane + 3];
                const int sum = c0 + c1 + c2 + c3;
                int incl = sum;
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) {
                    const int t = __shfl_up(incl, d, kWave);
                    if (lane >= d) incl += t;
                }
                const int ex = incl - sum;
                ucnt[4 * lane] = ex;
                ucnt[4 * lane + 1] = ex + c0;
                ucnt[4 * lane + 2] = ex + c0 + c1;
                ucnt[4 * lane + 3] = ex + c0 + c1 + c2;
                if (lane == kWave - 1) s_tot = incl;
            }
            __syncthreads();
            const int run = s_run;
#pragma unroll
            for (int u = 0; u < kTkU; ++u) {
                if (eqbits & (1u << u)) {
                    const int r = run + ucnt[u * kTkWaves + wave] + lpre[u];
                    const int i = base + u * kTkThreads + tid;
                    if (r < need)
                        rk[base_eq + r] = ((uint64_t)__float_as_uint(v[u]) << 32) |
                                          (uint32_t)(~(uint32_t)i);
                }
            }
            __syncthreads();
            // One thread decides whether both parts are complete: s_fill and
            // s_tot are final for this batch here (their writes came before
            // the barriers above), and the decision is read by all after the
            // next barrier, before anyone can change it again.
            if (tid == 0) {
                s_run = run + s_tot;
                s_done = (s_run >= need && s_fill >= base_eq) ? 1 : 0;
            }
            __syncthreads();
            if (s_done) break;
        }
    }
    __syncthreads();

    // 3. sort rk[0..kp) descending (zeros, the padding, sink)
    sort_ranks_desc(rk, kp, tid);

    for (int j = tid; j < k; j += kTkThreads) {
        int v = -1;
        if (j < take) v = (int)(~(uint32_t)(rk[j] & 0xFFFFFFFFull));
        idx[(size_t)q * k + j] = v;
        if (vals) vals[(size_t)q * k + j] = v >= 0 ? row[v] : __int_as_float(0x7FC00000);
    }
}

}  // namespace

hipError_t launch_topk_large(int Q, int N, int k, const float* scores, const int32_t* lengths,
                             int32_t* idx, float* vals, hipStream_t s) {
    topk_large_kernel<<<Q, kTkThreads, 0, s>>>(N, k, scores, lengths, idx, vals);
    return hipGetLastError();
}

}  // namespace moe
