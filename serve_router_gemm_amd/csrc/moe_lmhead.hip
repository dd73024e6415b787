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
//          expf(z_v - m) from +0, chunk sums added in ascending order;
//   logp_v = z_v - (m + logf(S)), m = max_v z_v;
//   k3     d_v = logp_ref - logp_test (fp64), term_v = exp(logp_test) *
//          (expm1(d_v) - d_v), summed in fp64 in the same chunked order;
//          greedy = the lowest v of largest logp_test, with its (unweighted)
//          term.  Identical inputs give exactly 0.
// One block per row; thread j owns chunks j, j+256, ...; chunk sums meet in
// LDS and one thread adds them in order.  The row never depends on the batch.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxChunks = kMaxVocab / kSumChunk;   // 4096

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
    __shared__ float chunk_sum[kMaxChunks];
    __shared__ float red[kRowThreads / 64];
    __shared__ float s_lse;
    const float* zr = z + (size_t)blockIdx.x * V;
    float* lr = logp + (size_t)blockIdx.x * V;
    const int nch = (V + kSumChunk - 1) / kSumChunk;

    float m = -INFINITY;
    for (int v = threadIdx.x; v < V; v += kRowThreads) m = fmaxf(m, zr[v]);
    m = block_max(m, red);

    for (int c = threadIdx.x; c < nch; c += kRowThreads) {
        const int v0 = c * kSumChunk, v1 = min(V, v0 + kSumChunk);
        float s = 0.0f;
        for (int v = v0; v < v1; ++v) s = s + expf(zr[v] - m);
        chunk_sum[c] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float S = 0.0f;
        for (int c = 0; c < nch; ++c) S = S + chunk_sum[c];
        s_lse = m + logf(S);
    }
    __syncthreads();
    const float lse = s_lse;
    for (int v = threadIdx.x; v < V; v += kRowThreads) lr[v] = zr[v] - lse;
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
    __shared__ double chunk_sum[kMaxChunks];
    __shared__ float best_v[kRowThreads];
    __shared__ int best_i[kRowThreads];
    const float* rr = ref + (size_t)blockIdx.x * V;
    const float* qr = test + (size_t)blockIdx.x * V;
    const int nch = (V + kSumChunk - 1) / kSumChunk;

    // greedy token: the first index of the largest non-NaN logp_test (and 0
    // if logp_test[0] is NaN, the rule of a running "strictly greater" scan
    // from index 0).  Per thread the first largest of its elements, then the
    // largest overall, the lowest index among equals.
    float bv = -INFINITY;
    int bi = V;
    for (int v = threadIdx.x; v < V; v += kRowThreads) {
        const float q = qr[v];
        if (!isnan(q) && (bi == V || q > bv)) { bv = q; bi = v; }
    }
    best_v[threadIdx.x] = bv;
    best_i[threadIdx.x] = bi;

    for (int c = threadIdx.x; c < nch; c += kRowThreads) {
        const int v0 = c * kSumChunk, v1 = min(V, v0 + kSumChunk);
        double s = 0.0;
        for (int v = v0; v < v1; ++v) s = s + exp((double)qr[v]) * k3_term(rr[v], qr[v]);
        chunk_sum[c] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double S = 0.0;
        for (int c = 0; c < nch; ++c) S = S + chunk_sum[c];
        float gv = -INFINITY;
        int gi = V;
        for (int j = 0; j < kRowThreads; ++j) {
            const int i = best_i[j];
            if (i >= V) continue;
            const float v = best_v[j];
            if (gi == V || v > gv || (v == gv && i < gi)) { gv = v; gi = i; }
        }
        if (gi == V || isnan(qr[0])) gi = 0;
        mean[blockIdx.x] = S;
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
