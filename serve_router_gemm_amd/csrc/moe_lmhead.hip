// moe_lmhead.hip -- the measurement downstream of a decode step: an fp32
// log-softmax over the vocabulary projection of the layer's output, and
// Schulman's k3 estimator between two such distributions.
//
// What training and serving compare in the end is the probability a model
// gives the next token, and the KL estimate k3 between two runs, against a
// 0.001 threshold (best2ai.com page on numerical alignment and MoE routing,
// sections "数值差异如何扰乱学习" and "混合专家模型更难对齐").  The pages fix
// neither the projection's order nor the sums; both are pinned here:
//   z      the router's chunked fp32 chain (moe_route.hip);
//   S      chunks of 256 consecutive v, each an ascending fp32 sum of
//          exp32(z_v - m) from +0, chunk sums added in ascending order;
//   logp_v = z_v - (m + log32(S)), m = max_v z_v;
//   exp32, log32: the fp32 exponential and logarithm correctly rounded,
//          taken as the fp64 function rounded once to fp32 (correct unless
//          the exact value is within an fp64 ulp of an fp32 rounding
//          boundary), so that any two implementations of S agree bit for
//          bit instead of depending on a single-precision expf's last bit;
//   k3     d_v = logp_ref - logp_test (fp64), term_v = exp(logp_test) *
//          (expm1(d_v) - d_v), summed in fp64 in the same chunked order;
//          greedy = the lowest v of largest logp_test, with its (unweighted)
//          term.  Identical inputs give exactly 0.
// Each row is cut into segments of kSegChunks whole chunks, one block per
// (row, segment), so a decode batch of 64 rows fills the GPU.  A block's
// coalesced pass computes its chunks' terms (exp32(z - m), or the k3 term)
// into LDS, one thread per chunk runs the chunk's ascending chain from LDS,
// and the chunk sums go to the workspace; a later launch adds a row's chunk
// sums in ascending order.  Log-softmax: segment maxima, then chunk sums, then
// S, lse and logp (three launches); k3: chunk sums and the segment's greedy
// candidate, then the ordered fold (two launches).  The row never depends on
// the batch, and every sum is taken in the order above.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kSegThreads = 256;
// chunks per block (2048 values: 8 values per thread; T = 64 on V = 65536 gives
// 2048 blocks.  Against 8192-value segments: log-softmax 24.6 -> 17.7 us at
// T = 1 and 30.0 -> 26.8 us at T = 64, k3 30.7 -> 20.7 and 37.2 -> 34.3 us;
// 1024-value segments, or reading each chain's next 8 values ahead, measured
// slower)
constexpr int kSegChunks = 8;
constexpr int kSegLen = kSegChunks * kSumChunk;
constexpr int kSegU = kSegLen / kSegThreads;          // 32 values per thread
constexpr int kPad = kSumChunk + 1;   // LDS stride of a chunk: chains of neighbouring
                                      // chunks fall on different banks

__device__ __forceinline__ float exp32(float a) { return (float)exp((double)a); }
__device__ __forceinline__ float log32(float a) { return (float)log((double)a); }

__device__ __forceinline__ double k3_term(float ref, float test) {
    const double d = (double)ref - (double)test;
    return expm1(d) - d;
}

// Segment (row blockIdx.x, segment blockIdx.y) of a row of V values:
// [v0, v1).  A thread loads its kSegU values before using any.
__device__ __forceinline__ void seg_range(int V, int& v0, int& v1) {
    v0 = blockIdx.y * kSegLen;
    v1 = min(V, v0 + kSegLen);
}

__device__ __forceinline__ float block_max256(float v, float* red) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float m = red[0];
    for (int i = 1; i < kSegThreads / 64; ++i) m = fmaxf(m, red[i]);
    return m;
}

// 1: the segment's maximum (NaN ignored, as the row maximum ignores it)
__global__ __launch_bounds__(kSegThreads) void ls_max_kernel(int V, int nseg,
                                                             const float* __restrict__ z,
                                                             float* __restrict__ segmax) {
    __shared__ float red[kSegThreads / 64];
    int v0, v1;
    seg_range(V, v0, v1);
    const float* zr = z + (size_t)blockIdx.x * V;
    float t[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int v = v0 + u * kSegThreads + threadIdx.x;
        t[u] = v < v1 ? zr[v] : -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSegU; ++u) m = fmaxf(m, t[u]);
    m = block_max256(m, red);
    if (threadIdx.x == 0) segmax[(size_t)blockIdx.x * nseg + blockIdx.y] = m;
}

constexpr int kMaxSeg = (kMaxVocab + kSegLen - 1) / kSegLen;      // 512
constexpr int kMaxChunks = (kMaxVocab + kSumChunk - 1) / kSumChunk;  // 4096

// The row's maximum from its segment maxima, loaded by the block's threads
// together (one memory latency) and reduced from LDS.
__device__ __forceinline__ float row_max(int nseg, const float* segmax, float* sm_l) {
    const float* sm = segmax + (size_t)blockIdx.x * nseg;
    for (int i = threadIdx.x; i < nseg; i += kSegThreads) sm_l[i] = sm[i];
    __syncthreads();
    float m = -INFINITY;
    for (int i = 0; i < nseg; ++i) m = fmaxf(m, sm_l[i]);
    return m;
}

// 2: the segment's chunk sums of exp32(z - m), each an ascending fp32 chain
__global__ __launch_bounds__(kSegThreads) void ls_chunk_kernel(int V, int nseg, int nch,
                                                               const float* __restrict__ z,
                                                               const float* __restrict__ segmax,
                                                               float* __restrict__ csum) {
    __shared__ float seg[kSegChunks * kPad];
    __shared__ float sm_l[kMaxSeg];
    int v0, v1;
    seg_range(V, v0, v1);
    const float* zr = z + (size_t)blockIdx.x * V;
    // the segment's values are loaded before the row maximum, so the two
    // memory round trips overlap
    float t[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int v = v0 + u * kSegThreads + threadIdx.x;
        t[u] = v < v1 ? zr[v] : 0.0f;
    }
    const float m = row_max(nseg, segmax, sm_l);
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int i = u * kSegThreads + threadIdx.x;
        if (v0 + i < v1) seg[(i / kSumChunk) * kPad + (i % kSumChunk)] = exp32(t[u] - m);
    }
    __syncthreads();
    const int c0 = blockIdx.y * kSegChunks;
    const int nc = min(kSegChunks, nch - c0);
    if (threadIdx.x < nc) {
        const int c = threadIdx.x;
        const int len = min(kSumChunk, V - (c0 + c) * kSumChunk);
        float s = 0.0f;
        int i = 0;
        for (; i + 8 <= len; i += 8) {
            float w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = seg[c * kPad + i + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) s = s + w[j];
        }
        for (; i < len; ++i) s = s + seg[c * kPad + i];
        csum[(size_t)blockIdx.x * nch + c0 + c] = s;
    }
}

// 3: S = the chunk sums added in ascending order, lse = m + log32(S), and
// logp = z - lse for the segment (logp may be z: each value is read before
// it is written, by the same thread)
__global__ __launch_bounds__(kSegThreads) void ls_write_kernel(int V, int nseg, int nch,
                                                               const float* __restrict__ z,
                                                               const float* __restrict__ segmax,
                                                               const float* __restrict__ csum,
                                                               float* logp) {
    __shared__ float s_lse;
    __shared__ float sm_l[kMaxSeg];
    __shared__ float cs_l[kMaxChunks];
    int v0, v1;
    seg_range(V, v0, v1);
    const float* zr = z + (size_t)blockIdx.x * V;
    float* lr = logp + (size_t)blockIdx.x * V;
    // the segment's values first: their loads overlap the fold below
    float t[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int v = v0 + u * kSegThreads + threadIdx.x;
        t[u] = v < v1 ? zr[v] : 0.0f;
    }
    // the row's chunk sums, loaded together, then added in ascending order
    const float* cs = csum + (size_t)blockIdx.x * nch;
    for (int i = threadIdx.x; i < nch; i += kSegThreads) cs_l[i] = cs[i];
    const float m = row_max(nseg, segmax, sm_l);   // (its barrier publishes cs_l too)
    if (threadIdx.x == 0) {
        float S = 0.0f;
        for (int c = 0; c < nch; ++c) S = S + cs_l[c];
        s_lse = m + log32(S);
    }
    __syncthreads();
    const float lse = s_lse;
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int v = v0 + u * kSegThreads + threadIdx.x;
        if (v < v1) lr[v] = t[u] - lse;
    }
}

// k3, 1: the segment's chunk sums of exp(logp_test) * (expm1(d) - d) (fp64
// ascending chains) and its greedy candidate: the first index of its largest
// non-NaN logp_test (index V if it has none)
__global__ __launch_bounds__(kSegThreads) void k3_chunk_kernel(int V, int nseg, int nch,
                                                               const float* __restrict__ ref,
                                                               const float* __restrict__ test,
                                                               double* __restrict__ csum,
                                                               float* __restrict__ gval,
                                                               int32_t* __restrict__ gidx,
                                                               double* __restrict__ gterm) {
    __shared__ double seg[kSegChunks * kPad];
    __shared__ float best_v[kSegThreads / 64];
    __shared__ float best_r[kSegThreads / 64];
    __shared__ int best_i[kSegThreads / 64];
    int v0, v1;
    seg_range(V, v0, v1);
    const float* rr = ref + (size_t)blockIdx.x * V;
    const float* qr = test + (size_t)blockIdx.x * V;
    float tq[kSegU], tr[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int v = v0 + u * kSegThreads + threadIdx.x;
        tq[u] = v < v1 ? qr[v] : 0.0f;
        tr[u] = v < v1 ? rr[v] : 0.0f;
    }
    // the candidate carries its logp_ref value, so the segment can give the
    // candidate's own term and the fold needs no further loads
    float bv = -INFINITY, br = 0.0f;
    int bi = V;
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int i = u * kSegThreads + threadIdx.x;
        const int v = v0 + i;
        if (v < v1) {
            seg[(i / kSumChunk) * kPad + (i % kSumChunk)] = exp((double)tq[u]) * k3_term(tr[u], tq[u]);
            if (!isnan(tq[u]) && (bi == V || tq[u] > bv)) { bv = tq[u]; br = tr[u]; bi = v; }
        }
    }
    // (value descending, index ascending, no element last) is a total order,
    // so a tree reduction finds the same first largest element
    for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const float orr = __shfl_xor(br, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (oi < V && (bi == V || ov > bv || (ov == bv && oi < bi))) { bv = ov; br = orr; bi = oi; }
    }
    if ((threadIdx.x & 63) == 0) {
        best_v[threadIdx.x >> 6] = bv;
        best_r[threadIdx.x >> 6] = br;
        best_i[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    const int c0 = blockIdx.y * kSegChunks;
    const int nc = min(kSegChunks, nch - c0);
    if (threadIdx.x < nc) {
        const int c = threadIdx.x;
        const int len = min(kSumChunk, V - (c0 + c) * kSumChunk);
        double s = 0.0;
        int i = 0;
        for (; i + 8 <= len; i += 8) {
            double w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = seg[c * kPad + i + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) s = s + w[j];
        }
        for (; i < len; ++i) s = s + seg[c * kPad + i];
        csum[(size_t)blockIdx.x * nch + c0 + c] = s;
    }
    if (threadIdx.x == 0) {
        float gv = -INFINITY, gr = 0.0f;
        int gi = V;
        for (int j = 0; j < kSegThreads / 64; ++j) {
            const int i = best_i[j];
            if (i >= V) continue;
            const float w = best_v[j];
            if (gi == V || w > gv || (w == gv && i < gi)) { gv = w; gr = best_r[j]; gi = i; }
        }
        const size_t o = (size_t)blockIdx.x * nseg + blockIdx.y;
        gval[o] = gv;
        gidx[o] = gi;
        gterm[o] = gi < V ? k3_term(gr, gv) : 0.0;
    }
}

// k3, 2: one block per row: the chunk sums (loaded together into LDS) added
// in ascending order, the greedy token over the segments' candidates (0 if
// logp_test[0] is NaN, the rule of a running "strictly greater" scan from
// index 0), and its term (the winning segment's, or index 0's)
__global__ __launch_bounds__(kSegThreads) void k3_fold_kernel(int V, int nseg, int nch,
                                                              const float* __restrict__ ref,
                                                              const float* __restrict__ test,
                                                              const double* __restrict__ csum,
                                                              const float* __restrict__ gval,
                                                              const int32_t* __restrict__ gidx,
                                                              const double* __restrict__ gterm,
                                                              double* __restrict__ mean,
                                                              double* __restrict__ greedy_k3,
                                                              int32_t* __restrict__ greedy) {
    __shared__ double cs_l[kMaxChunks];
    __shared__ double gt_l[kMaxSeg];
    __shared__ float gv_l[kMaxSeg];
    __shared__ int gi_l[kMaxSeg];
    const int t = blockIdx.x;
    // index 0's values, loaded with the rest (one memory round trip)
    const float q0 = test[(size_t)t * V];
    const float r0 = ref[(size_t)t * V];
    const double* cs = csum + (size_t)t * nch;
    for (int i = threadIdx.x; i < nch; i += kSegThreads) cs_l[i] = cs[i];
    for (int i = threadIdx.x; i < nseg; i += kSegThreads) {
        gv_l[i] = gval[(size_t)t * nseg + i];
        gi_l[i] = gidx[(size_t)t * nseg + i];
        gt_l[i] = gterm[(size_t)t * nseg + i];
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    double S = 0.0;
    for (int c = 0; c < nch; ++c) S = S + cs_l[c];
    float gv = -INFINITY;
    int gi = V, gj = -1;
    for (int j = 0; j < nseg; ++j) {
        const int i = gi_l[j];
        if (i >= V) continue;
        const float w = gv_l[j];
        if (gi == V || w > gv || (w == gv && i < gi)) { gv = w; gi = i; gj = j; }
    }
    double term;
    if (gi == V || isnan(q0)) {
        gi = 0;
        term = k3_term(r0, q0);
    } else {
        term = gt_l[gj];
    }
    mean[t] = S;
    greedy[t] = gi;
    greedy_k3[t] = term;
}

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

int measure_segments(int V) { return (V + kSegLen - 1) / kSegLen; }

size_t log_softmax_ws_bytes(int T, int V) {
    const int nseg = measure_segments(V), nch = (V + kSumChunk - 1) / kSumChunk;
    return up256((size_t)T * nseg * 4) + up256((size_t)T * nch * 4);
}

size_t k3_ws_bytes(int T, int V) {
    const int nseg = measure_segments(V), nch = (V + kSumChunk - 1) / kSumChunk;
    return up256((size_t)T * nch * 8) + up256((size_t)T * nseg * 4) + up256((size_t)T * nseg * 4) +
           up256((size_t)T * nseg * 8);
}

hipError_t launch_log_softmax(int T, int V, const float* z, float* logp, void* ws,
                              hipStream_t s) {
    const int nseg = measure_segments(V), nch = (V + kSumChunk - 1) / kSumChunk;
    float* segmax = static_cast<float*>(ws);
    float* csum = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) +
                                           up256((size_t)T * nseg * 4));
    const dim3 grid(T, nseg);
    ls_max_kernel<<<grid, kSegThreads, 0, s>>>(V, nseg, z, segmax);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ls_chunk_kernel<<<grid, kSegThreads, 0, s>>>(V, nseg, nch, z, segmax, csum);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    ls_write_kernel<<<grid, kSegThreads, 0, s>>>(V, nseg, nch, z, segmax, csum, logp);
    return hipGetLastError();
}

hipError_t launch_k3(int T, int V, const float* logp_ref, const float* logp_test, double* mean,
                     double* greedy_k3, int32_t* greedy, void* ws, hipStream_t s) {
    const int nseg = measure_segments(V), nch = (V + kSumChunk - 1) / kSumChunk;
    unsigned char* w = static_cast<unsigned char*>(ws);
    double* csum = reinterpret_cast<double*>(w);
    w += up256((size_t)T * nch * 8);
    float* gval = reinterpret_cast<float*>(w);
    w += up256((size_t)T * nseg * 4);
    int32_t* gidx = reinterpret_cast<int32_t*>(w);
    w += up256((size_t)T * nseg * 4);
    double* gterm = reinterpret_cast<double*>(w);
    k3_chunk_kernel<<<dim3(T, nseg), kSegThreads, 0, s>>>(V, nseg, nch, logp_ref, logp_test,
                                                           csum, gval, gidx, gterm);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    k3_fold_kernel<<<T, kSegThreads, 0, s>>>(V, nseg, nch, logp_ref, logp_test, csum, gval, gidx,
                                              gterm, mean, greedy_k3, greedy);
    return hipGetLastError();
}

}  // namespace moe
