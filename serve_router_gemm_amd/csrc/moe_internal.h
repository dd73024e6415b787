// moe_internal.h -- launchers shared between the translation units of libmoe.
// Host-side declarations only; every launcher enqueues on `stream` and
// returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Router logit order: chunks of this many consecutive hidden indices, each an
// ascending fp32 fma chain, chunk sums added in ascending order.
constexpr int kLogitChunk = 256;

// router -------------------------------------------------------------------
struct RoutePlan {
    int split;     // 0: logits kernel folds every chunk; 1: one block per chunk
    int nparts;    // partial-logit planes the select kernel folds
    int tt, te;    // token / expert register tile of the VALU logits kernel
    int mfma;      // 1: the matrix-core logits kernel, its waves wt x we (4 or 8)
    int wt, we;
};
RoutePlan route_plan(int T, int H, int E);
size_t route_ws_bytes(int T, int H, int E);
// replay != nullptr: router replay -- the experts are read from replay [T,k]
// (ids is not written) and only the weights w are computed.
hipError_t launch_route(int T, int H, int E, int k, int score, int renorm,
                        const uint16_t* x, const uint16_t* wr, const float* bias,
                        int32_t* ids, float* w, float* part_ws, hipStream_t s,
                        const int32_t* replay = nullptr);

// permute ------------------------------------------------------------------
int permute_chunk(int A);
size_t permute_ws_bytes(int A, int E);
hipError_t launch_permute(int A, int E, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                          int32_t* ws, hipStream_t s);

// expert GEMMs ---------------------------------------------------------------
size_t gemm_sched_ws_bytes(int E);  // tile_start [E+1] + short-tile list [1+E]
// Extra workspace of the load-dependent variant (variant = 1) of either GEMM:
// the split experts' partial sums and their row map.
size_t gemm_variant_ws_bytes(int T, int H, int E, int F, int k);
// variant = 1: the load-dependent variant, with vws holding
// gemm_variant_ws_bytes() bytes; variant = 0: the invariant kernels.
hipError_t launch_gate_up(int T, int H, int E, int F, int k, const uint16_t* x,
                          const int32_t* perm, const int32_t* offsets,
                          const uint16_t* wg, const uint16_t* wu, uint16_t* h_act,
                          int32_t* sched_ws, hipStream_t s, int variant = 0,
                          void* vws = nullptr);
hipError_t launch_down(int T, int H, int E, int F, int k, const uint16_t* h_act,
                       const int32_t* perm, const int32_t* offsets, const uint16_t* wd,
                       float* y, int variant, int32_t* sched_ws, hipStream_t s,
                       void* vws = nullptr);
// the tile list of the grouped GEMMs into sched_ws (gemm_sched_ws_bytes(E));
// experts with at most skip_upto tokens get no tile
hipError_t launch_tile_schedule(int E, int skip_upto, int reorder, const int32_t* offsets,
                                int32_t* sched_ws, hipStream_t s);

// FP8 rollout path ------------------------------------------------------------
constexpr int kFp8Block = 128;     // scale block: 128 K (x 128 rows for weights)
constexpr int kFp8MaxKB = 64;      // K blocks a GEMM holds (K <= 8192)
hipError_t launch_quantize_fp8(int R, int K, int block_rows, const uint16_t* src, uint8_t* q,
                               int8_t* exps, hipStream_t s);
hipError_t launch_gate_up_fp8(int T, int H, int E, int F, int k, const uint8_t* xq,
                              const int8_t* xe, const int32_t* perm, const int32_t* offsets,
                              const uint8_t* wgq, const int8_t* wge, const uint8_t* wuq,
                              const int8_t* wue, uint8_t* aq, int8_t* ae, uint16_t* act_bf16,
                              int32_t* sched_ws, hipStream_t s);
hipError_t launch_down_fp8(int T, int H, int E, int F, int k, const uint8_t* aq,
                           const int8_t* ae, const int32_t* perm, const int32_t* offsets,
                           const uint8_t* wdq, const int8_t* wde, float* y, int32_t* sched_ws,
                           hipStream_t s);

// decode-step measurement: vocabulary projection, log-softmax, k3 ------------
constexpr int kSumChunk = 256;     // fixed chunk of the vocabulary sums
constexpr int kMaxVocab = 1 << 20;
hipError_t launch_lm_logits(int T, int H, int V, const uint16_t* h, const uint16_t* proj,
                            float* z, hipStream_t s);
size_t log_softmax_ws_bytes(int T, int V);
size_t k3_ws_bytes(int T, int V);
hipError_t launch_log_softmax(int T, int V, const float* z, float* logp, void* ws,
                              hipStream_t s);
hipError_t launch_k3(int T, int V, const float* logp_ref, const float* logp_test,
                     double* mean, double* greedy_k3, int32_t* greedy, void* ws, hipStream_t s);

// large-k top-k (sparse attention indexer) ------------------------------------
constexpr int kMaxTopkLarge = 4096;
hipError_t launch_topk_large(int Q, int N, int k, const float* scores, const int32_t* lengths,
                             int32_t* idx, float* vals, hipStream_t s);

// combine ------------------------------------------------------------------
// y rows of assignments that permute skipped (inv_perm = -1) are set to 0.
hipError_t launch_zero_unplaced(int A, int H, const int32_t* inv_perm, float* y, hipStream_t s);
hipError_t launch_combine(int T, int H, int k, const float* y, const float* w,
                          uint16_t* out, hipStream_t s);

int device_cu_count();

}  // namespace moe
