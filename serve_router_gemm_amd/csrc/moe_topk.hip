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
// before using them.  With n > k valid scores, a histogram of the top 11
// code bits first finds the bin that holds the k-th element; when that bin
// and the ones above it hold at most 4096 elements (no heavy ties), a second
// read collects them and one sort of their ranks gives the list (two reads
// of the row).  Otherwise:
//   1. radix select on the 32-bit order-preserving code, 8 bits per pass from
//      the top (LDS histograms, integer counts): the code c* of the k-th
//      element and kk, how many elements equal to c* are taken;
//   2. every element above c* is taken (LDS atomic slot; the slots are
//      sorted next, so their order does not matter), and the kk lowest
//      indices equal to c*, found by a block-wide scan in index order;
//   3. a bitonic sort of the k 64-bit ranks (code << 32 | ~index) in LDS,
//      descending.
// With n <= k every valid element is taken and sorted; the rest is -1.
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

// bitonic sort of rk[0..kp) descending (kp a power of two; zeros sink)
__device__ __forceinline__ void sort_ranks_desc(uint64_t* rk, int kp, int tid) {
    for (int size = 2; size <= kp; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < kp / 2; t += kTkThreads) {
                const int i = 2 * stride * (t / stride) + (t % stride);
                const int j = i + stride;
                const uint64_t a = rk[i], b = rk[j];
                const bool desc = (i & size) == 0;
                if (desc ? (a < b) : (a > b)) { rk[i] = b; rk[j] = a; }
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(kTkThreads) void topk_large_kernel(
    int N, int k, const float* __restrict__ scores, const int32_t* __restrict__ lengths,
    int32_t* __restrict__ idx, float* __restrict__ vals) {
    __shared__ uint64_t rk[kMaxTopkLarge];
    __shared__ int hist[256];
    __shared__ int ucnt[kTkU * kTkWaves];   // equal-to-c* counts per (u, wave), then their prefix
    __shared__ int s_bin, s_above, s_fill, s_run, s_done, s_tot, s_cand;
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

    // Two reads of the row when they suffice: a histogram of the top 11 code
    // bits finds the bin b1 where the count from the top reaches k; every
    // element in b1 or above is a candidate (at least k of them, the top k
    // among them), and when they fit in rk one sort of their 64-bit ranks
    // gives the list.  Otherwise (heavy ties) the radix select below runs.
    bool fast = false;
    if (n > k) {
        for (int b = tid; b < kTkTopBins; b += kTkThreads) thist[b] = 0;
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
                if (i < n) atomicAdd(&thist[key_code(v[u]) >> kTkTopShift], 1);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane l: bins [32l, 32l + 32); suffix sums over lanes find the
            // group holding the k-th element, one lane scans inside it
            int g = 0;
            for (int j = 0; j < kTkTopBins / kWave; ++j) g += thist[lane * (kTkTopBins / kWave) + j];
            int suf = g;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int t = __shfl_down(suf, d, kWave);
                if (lane + d < kWave) suf += t;
            }
            const uint64_t reach = __ballot(suf >= k);          // non-increasing in lane
            const int L = 63 - __clzll((long long)reach);
            const int above_groups = __shfl(suf - g, L, kWave);  // elements in groups > L
            if (lane == L) {
                int above = above_groups, b = L * (kTkTopBins / kWave) + (kTkTopBins / kWave) - 1;
                for (; b > L * (kTkTopBins / kWave); --b) {
                    if (above + thist[b] >= k) break;
                    above += thist[b];
                }
                s_bin = b;
                s_cand = above + thist[b];
            }
        }
        __syncthreads();
        fast = s_cand <= kMaxTopkLarge;
    }
    const int nrank = fast ? s_cand : take;     // entries sorted
    kp = 1;
    while (kp < nrank) kp <<= 1;
    for (int i = tid; i < kp; i += kTkThreads) rk[i] = 0;
    if (tid == 0) s_fill = 0;
    __syncthreads();

    if (fast) {
        const uint32_t b1 = (uint32_t)s_bin;
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
                const bool cand = i < n && (c >> kTkTopShift) >= b1;
                const uint64_t bal = __ballot(cand);
                if (bal) {
                    int slot0 = 0;
                    if (lane == 0) slot0 = atomicAdd(&s_fill, __popcll(bal));
                    slot0 = __shfl(slot0, 0, kWave);
                    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
                    if (cand) rk[slot0 + __popcll(bal & below)] =
                        ((uint64_t)c << 32) | (uint32_t)(~(uint32_t)i);
                }
            }
        }
    } else if (n <= k) {
        for (int i = tid; i < n; i += kTkThreads) {
            const int pos = atomicAdd(&s_fill, 1);
            rk[pos] = sel_rank(row[i], i);
        }
    } else {
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
            if (tid == 0) {
                int above = 0, b = 255;
                for (; b > 0; --b) {
                    if (above + hist[b] >= need) break;
                    above += hist[b];
                }
                s_bin = b;
                s_above = above;
            }
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
                        ((uint64_t)c << 32) | (uint32_t)(~(uint32_t)i);
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
                        rk[base_eq + r] = ((uint64_t)cstar << 32) | (uint32_t)(~(uint32_t)i);
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
