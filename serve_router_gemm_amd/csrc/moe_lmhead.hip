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
// One block per row.  The row is taken in segments of whole chunks: a
// coalesced pass computes the chunk's terms (expf(z - m), or the k3 term) into
// LDS, one thread per chunk then runs the chunk's ascending chain from LDS,
// and one thread adds the segment's chunk sums to S in ascending order.  The
// row never depends on the batch.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kRowThreads = 1024;
constexpr int kRowU = 16;             // loads in flight per thread in the row passes
constexpr int kPad = kSumChunk + 1;   // LDS stride of a chunk: chains of neighbouring
                                      // chunks fall on different banks
constexpr int kSegF = 128;            // chunks per segment, fp32 terms (128.5 KB)
constexpr int kSegD = 64;             // chunks per segment, fp64 terms (128.5 KB)

__device__ __forceinline__ float exp32(float a) { return (float)exp((double)a); }
__device__ __forceinline__ float log32(float a) { return (float)log((double)a); }

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float m = red[0];
    for (int i = 1; i < kRowThreads / 64; ++i) m = fmaxf(m, red[i]);
    return m;
}

__global__ __launch_bounds__(kRowThreads) void log_softmax_kernel(int V, const float* __restrict__ z,
                                                                  float* __restrict__ logp) {
    __shared__ float seg[kSegF * kPad];
    __shared__ float seg_sum[kSegF];
    __shared__ float red[kRowThreads / 64];
    __shared__ float s_S;
    const float* zr = z + (size_t)blockIdx.x * V;
    float* lr = logp + (size_t)blockIdx.x * V;
    const int nch = (V + kSumChunk - 1) / kSumChunk;

    float m = -INFINITY;
    for (int b = 0; b < V; b += kRowThreads * kRowU) {
        float t[kRowU];
#pragma unroll
        for (int u = 0; u < kRowU; ++u) {
            const int v = b + u * kRowThreads + threadIdx.x;
            t[u] = v < V ? zr[v] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < kRowU; ++u) m = fmaxf(m, t[u]);
    }
    m = block_max(m, red);

    if (threadIdx.x == 0) s_S = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += kSegF) {
        const int nc = min(kSegF, nch - c0);
        const int v0 = c0 * kSumChunk, v1 = min(V, v0 + nc * kSumChunk);
        for (int b = v0; b < v1; b += kRowThreads * kRowU) {
            float t[kRowU];
#pragma unroll
            for (int u = 0; u < kRowU; ++u) {
                const int v = b + u * kRowThreads + threadIdx.x;
                t[u] = v < v1 ? zr[v] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kRowU; ++u) {
                const int v = b + u * kRowThreads + threadIdx.x;
                if (v < v1) seg[(v / kSumChunk - c0) * kPad + (v % kSumChunk)] = exp32(t[u] - m);
            }
        }
        __syncthreads();
        if (threadIdx.x < nc) {
            const int c = threadIdx.x;
            const int len = min(kSumChunk, V - (c0 + c) * kSumChunk);
            float s = 0.0f;
            int i = 0;
            for (; i + 8 <= len; i += 8) {
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = seg[c * kPad + i + j];
#pragma unroll
                for (int j = 0; j < 8; ++j) s = s + t[j];
            }
            for (; i < len; ++i) s = s + seg[c * kPad + i];
            seg_sum[c] = s;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float S = s_S;
            int c = 0;
            for (; c + 8 <= nc; c += 8) {
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = seg_sum[c + j];
#pragma unroll
                for (int j = 0; j < 8; ++j) S = S + t[j];
            }
            for (; c < nc; ++c) S = S + seg_sum[c];
            s_S = S;
        }
        __syncthreads();
    }
    const float lse = m + log32(s_S);
    for (int b = 0; b < V; b += kRowThreads * kRowU) {
        float t[kRowU];
#pragma unroll
        for (int u = 0; u < kRowU; ++u) {
            const int v = b + u * kRowThreads + threadIdx.x;
            t[u] = v < V ? zr[v] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kRowU; ++u) {
            const int v = b + u * kRowThreads + threadIdx.x;
            if (v < V) lr[v] = t[u] - lse;
        }
    }
}

__device__ __forceinline__ double k3_term(float ref, float test) {
    const double d = (double)ref - (double)test;
    return expm1(d) - d;
}

__global__ __launch_bounds__(kRowThreads) void k3_kernel(int V, const float* __restrict__ ref,
                                                         const float* __restrict__ test,
                                                         double* __restrict__ mean,
                                                         double* __restrict__ greedy_k3,
                                                         int32_t* __restrict__ greedy) {
    __shared__ double seg[kSegD * kPad];
    __shared__ double seg_sum[kSegD];
    __shared__ double s_S;
    __shared__ float best_v[kRowThreads / 64];
    __shared__ int best_i[kRowThreads / 64];
    const float* rr = ref + (size_t)blockIdx.x * V;
    const float* qr = test + (size_t)blockIdx.x * V;
    const int nch = (V + kSumChunk - 1) / kSumChunk;

    // greedy token: the first index of the largest non-NaN logp_test (and 0
    // if logp_test[0] is NaN, the rule of a running "strictly greater" scan
    // from index 0).  Per thread the first largest of its elements, then the
    // largest overall, the lowest index among equals.
    float bv = -INFINITY;
    int bi = V;
    for (int b = 0; b < V; b += kRowThreads * kRowU) {
        float t[kRowU];
#pragma unroll
        for (int u = 0; u < kRowU; ++u) {
            const int v = b + u * kRowThreads + threadIdx.x;
            t[u] = v < V ? qr[v] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kRowU; ++u) {
            const int v = b + u * kRowThreads + threadIdx.x;
            if (v < V && !isnan(t[u]) && (bi == V || t[u] > bv)) { bv = t[u]; bi = v; }
        }
    }
    // (value descending, index ascending, no element last) is a total order,
    // so a tree reduction finds the same first largest element
    for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (oi < V && (bi == V || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
    }
    if ((threadIdx.x & 63) == 0) {
        best_v[threadIdx.x >> 6] = bv;
        best_i[threadIdx.x >> 6] = bi;
    }

    if (threadIdx.x == 0) s_S = 0.0;
    for (int c0 = 0; c0 < nch; c0 += kSegD) {
        const int nc = min(kSegD, nch - c0);
        const int v0 = c0 * kSumChunk, v1 = min(V, v0 + nc * kSumChunk);
        for (int b = v0; b < v1; b += kRowThreads * kRowU) {
            float tq[kRowU], tr[kRowU];
#pragma unroll
            for (int u = 0; u < kRowU; ++u) {
                const int v = b + u * kRowThreads + threadIdx.x;
                tq[u] = v < v1 ? qr[v] : 0.0f;
                tr[u] = v < v1 ? rr[v] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kRowU; ++u) {
                const int v = b + u * kRowThreads + threadIdx.x;
                if (v < v1)
                    seg[(v / kSumChunk - c0) * kPad + (v % kSumChunk)] =
                        exp((double)tq[u]) * k3_term(tr[u], tq[u]);
            }
        }
        __syncthreads();
        if (threadIdx.x < nc) {
            const int c = threadIdx.x;
            const int len = min(kSumChunk, V - (c0 + c) * kSumChunk);
            double s = 0.0;
            int i = 0;
            for (; i + 8 <= len; i += 8) {
                double t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = seg[c * kPad + i + j];
#pragma unroll
                for (int j = 0; j < 8; ++j) s = s + t[j];
            }
            for (; i < len; ++i) s = s + seg[c * kPad + i];
            seg_sum[c] = s;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double S = s_S;
            int c = 0;
            for (; c + 8 <= nc; c += 8) {
                double t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = seg_sum[c + j];
#pragma unroll
                for (int j = 0; j < 8; ++j) S = S + t[j];
            }
            for (; c < nc; ++c) S = S + seg_sum[c];
            s_S = S;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        float gv = -INFINITY;
        int gi = V;
        for (int j = 0; j < kRowThreads / 64; ++j) {
            const int i = best_i[j];
            if (i >= V) continue;
            const float v = best_v[j];
            if (gi == V || v > gv || (v == gv && i < gi)) { gv = v; gi = i; }
        }
        if (gi == V || isnan(qr[0])) gi = 0;
        mean[blockIdx.x] = s_S;
        greedy[blockIdx.x] = gi;
        greedy_k3[blockIdx.x] = k3_term(rr[gi], qr[gi]);
    }
}

}  // namespace

hipError_t launch_log_softmax(int T, int V, const float* z, float* logp, hipStream_t s) {
    log_softmax_kernel<<<T, kRowThreads, 0, s>>>(V, z, logp);
    return hipGetLastError();
}

hipError_t launch_k3(int T, int V, const float* logp_ref, const float* logp_test, double* mean,
                     double* greedy_k3, int32_t* greedy, hipStream_t s) {
    k3_kernel<<<T, kRowThreads, 0, s>>>(V, logp_ref, logp_test, mean, greedy_k3, greedy);
    return hipGetLastError();
}

}  // namespace moe
