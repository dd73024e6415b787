/*
 * moe.h -- C ABI of the batch-invariant Mixture-of-Experts layer forward for
 * AMD Instinct MI355X (gfx950).  Library: libmoe.so.
 *
 * What the library guarantees.  For one layer shape (H, E, F, top_k, score,
 * renormalize) and the invariant GEMM variant, every token's rows of
 * `topk_ids`, `topk_w` and `out` are bit-identical whatever the number of
 * tokens in the call, whichever other tokens share it, and wherever the
 * token sits in it.  Sources on the pages:
 *   - Fireworks page "位级一致：前沿训练的差异化关键" (bit-level agreement),
 *     section "曾经只有前沿实验室才有的功能": batch invariance is a request
 *     getting the same result whatever else shares its batch; the MoE router
 *     and the expert GEMMs are reductions that must stay consistent; split-K
 *     breaks invariance.
 *   - Same page, section "为什么比特级一致是一个复杂的问题": per-expert matmul
 *     kernels that change with the expert's token count, and router near-ties,
 *     both move bits; the fix is one expert-matmul kernel choice whatever the
 *     token count and a deterministic router tie-break.
 *   - Fireworks page on numerical alignment and MoE routing, section
 *     "混合专家模型更难对齐": the precision and the order of the weighted sum of
 *     the expert outputs must both be fixed.
 *   - "GLM Post-Training Beyond SFT", section "迁移到 NPU 时": a top-k must fix
 *     boundary ties, stability, NaN handling and the index dtype.
 *
 * The layer (the pages give no formula; this is the reading the library
 * implements):
 *   logits  l[t,e] = sum_i x[t,i] * w_router[e,i] in fp32 and in one fixed
 *           order: i in chunks of 256, each chunk an ascending chain of fp32
 *           fmas from +0 (bf16*bf16 products are exact), chunk sums added to
 *           +0 in ascending chunk order.
 *   select  softmax: key = l;  sigmoid: key = fp32(1/(1+exp(-l))) + bias[e].
 *           top_k experts by key descending, ties to the lower expert index,
 *           -0 == +0, NaN keys last (NaNs by index).  Slot j = j-th selected.
 *   weights softmax p = exp(l - max l) / sum exp(...) over all E experts;
 *           sigmoid p = 1/(1+exp(-l)) (bias excluded); renormalize: w_j =
 *           p_j / sum_j p_j, else w_j = p_j.  fp32.
 *   permute a = t*top_k + j is an assignment; perm lists assignments grouped
 *           by expert ascending and, inside an expert, by a ascending.
 *   experts act = bf16(silu(x W_gate[e]^T) * (x W_up[e]^T)),
 *           y[a] = act W_down[e]^T in fp32 (not rounded).  bf16 MFMA, fp32
 *           accumulate, one MFMA instruction and one ascending K order for
 *           every tile of every expert, no split-K (invariant variant).
 *   combine acc = 0; for j = 0..top_k-1: acc = fmaf(w[t,j], y[t*top_k+j,h], acc);
 *           out[t,h] = bf16(acc) (round to nearest even).
 *
 * Conventions for every entry point.
 *   - Pointers marked [device] are device pointers (hipMalloc'd or equivalent
 *     coarse-grained memory) and must be 16-byte aligned.  [host] pointers
 *     are host memory.  bf16 tensors are passed as uint16_t bit patterns.
 *   - Row-major layouts, K contiguous:
 *       x [T,H], w_router [E,H], w_gate [E,F,H], w_up [E,F,H], w_down [E,H,F],
 *       bias [E] fp32, topk_ids [T,k] int32, topk_w [T,k] fp32,
 *       expert_counts [E], expert_offsets [E+1], perm [T*k], inv_perm [T*k]
 *       (int32), h_act [T*k,F] bf16 (rows in perm order), y [T*k,H] fp32
 *       (rows in assignment order a = t*k + j), out [T,H] bf16.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on that stream and returns; it never synchronizes,
 *     allocates, frees, prints or aborts, and keeps no state between calls.
 *     The caller owns every buffer; outputs are fully overwritten.
 *   - `ws` is caller-owned device scratch of at least moe_workspace_bytes()
 *     bytes for the same op and sizes; it may be NULL when that size is 0.
 *     Its contents on entry do not matter.  Calls that overlap in time on
 *     different streams must use different workspaces.
 *   - Every argument is checked on the host before anything is enqueued; a
 *     failed check enqueues nothing and returns a negative moe_status.  T == 0
 *     is valid and enqueues nothing.  A launch failure returns MOE_ERR_HIP.
 *   - Limits: 1 <= E <= 512; 1 <= top_k <= min(E, 16); H and F multiples of
 *     64 in [64, 65536]; 0 <= T; T*top_k <= 2^24 and T*top_k*max(H,F) < 2^31.
 *   - Thread-safe and reentrant (no global mutable state), except
 *     moe_forward_static, whose calls share one scratch array per GPU.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* a size is out of range (see Limits) */
    MOE_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned */
    MOE_ERR_UNSUPPORTED = -4, /* H or F not a multiple of 64, bad enum value */
    MOE_ERR_WORKSPACE = -5,   /* ws_bytes smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = -6,         /* the HIP runtime reported a launch error */
    MOE_ERR_SCRATCH = -7      /* moe_forward_static: the sizes need more than
                                 the library's static scratch */
} moe_status;

typedef enum moe_score_fn {
    MOE_SCORE_SOFTMAX = 0,
    MOE_SCORE_SIGMOID = 1
} moe_score_fn;

typedef enum moe_gemm_variant {
    /* fixed tile, one MFMA instruction, ascending K, no split-K */
    MOE_GEMM_INVARIANT = 0,
    /* deliberately NOT batch-invariant, as load-dependent kernels are (the
     * per-expert kernel and tiling that change with the expert's token
     * count: Fireworks page "位级一致：前沿训练的差异化关键", section
     * "为什么比特级一致是一个复杂的问题"): in both expert GEMMs, an expert
     * with at most 32 tokens has its K range split into parts chosen from its
     * token count (4 parts up to 4 tokens, else 2; fewer where K does not
     * divide), each part summed on its own and the parts added in a second
     * pass; larger experts take the invariant kernel.  Deterministic from run
     * to run, but a token's bits depend on how many tokens its experts got.
     * Exists to show that drift and to measure what invariance costs. */
    MOE_GEMM_SPLITK_VARIANT = 1
} moe_gemm_variant;

typedef enum moe_op {
    MOE_OP_ROUTE = 0,
    MOE_OP_PERMUTE = 1,
    MOE_OP_GATE_UP = 2,
    MOE_OP_DOWN = 3,
    MOE_OP_GROUPED_SWIGLU = 4,
    MOE_OP_COMBINE = 5,
    MOE_OP_FORWARD = 6,
    MOE_OP_GATE_UP_FP8 = 7,
    MOE_OP_DOWN_FP8 = 8,
    MOE_OP_FORWARD_FP8 = 9,
    MOE_OP_LOG_SOFTMAX = 10,  /* moe_workspace_bytes: pass the vocabulary V as H */
    MOE_OP_K3 = 11            /* moe_workspace_bytes: pass the vocabulary V as H */
} moe_op;

/* Bytes of device scratch the entry point `op` needs for these sizes
 * (0 when it needs none).  Host only; never touches the GPU.  Returns 0 for
 * sizes that the entry point would reject. */
size_t moe_workspace_bytes(int op, int T, int H, int E, int F, int top_k, int variant);

/* Static description of a status code.  Host only. */
const char* moe_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int moe_version(void);

/* Router: logits, selection and weights (the "route" step).  The router is
 * one of the reductions whose order must not depend on the batch, and near
 * ties between experts must break deterministically (Fireworks page
 * "位级一致：前沿训练的差异化关键", sections "曾经只有前沿实验室才有的功能" and
 * "为什么比特级一致是一个复杂的问题"); hence the fixed logit order and the
 * lowest-index tie-break described at the top of this file.
 *   x [device] [T,H] bf16; w_router [device] [E,H] bf16;
 *   bias [device] [E] fp32 or NULL (sigmoid only: NULL means all zero; a
 *   non-NULL bias with softmax is rejected with MOE_ERR_UNSUPPORTED);
 *   topk_ids [device] out [T,k] int32; topk_w [device] out [T,k] fp32.
 * score: moe_score_fn.  renormalize: 0 or 1.  ws [device] holds the logits,
 * or one plane of partial logits per 256-wide chunk where the library splits
 * the hidden dimension over blocks (moe_workspace_bytes(MOE_OP_ROUTE, ...)
 * gives the size the library will use; its content on entry is ignored).
 * Whether the chains run on the VALU or on the matrix cores (the K = 1 fp32
 * MFMA) is the library's choice from T, H and E; both give the same bits. */
int moe_route(int T, int H, int E, int top_k, int score, int renormalize,
              const uint16_t* x, const uint16_t* w_router, const float* bias,
              int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Expert histogram, offsets and the stable permutation (the "permute" step).
 * How many tokens each expert receives depends on the whole batch (same
 * page, section "为什么比特级一致是一个复杂的问题"); this step is integer-only
 * and stable, so the counts change launch work but never a token's values.
 *   topk_ids [device] [T,k] int32 with values in [0,E) (other values are
 *   skipped: not counted and not placed, and the tail of perm is then left
 *   unwritten);
 *   expert_counts [device] out [E]; expert_offsets [device] out [E+1]
 *   (exclusive prefix sum, offsets[E] = number of placed assignments);
 *   perm [device] out [T*k]: perm[p] = assignment id at permuted position p;
 *   inv_perm [device] out [T*k]: inv_perm[perm[p]] = p (-1 if skipped). */
int moe_permute(int T, int E, int top_k, const int32_t* topk_ids,
                int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Gate/up projections with the SwiGLU epilogue, grouped by expert (the
 * first expert GEMM).  One kernel choice, tile and K order for every expert
 * whatever its token count, and no split-K (same page, sections
 * "为什么比特级一致是一个复杂的问题" and "曾经只有前沿实验室才有的功能").
 * For every permuted row p of expert e:
 *   h_act[p, f] = bf16(silu(g) * u), g = x[perm[p]/k] . w_gate[e,f,:],
 *   u = x[perm[p]/k] . w_up[e,f,:], fp32 accumulation.
 *   x [device] [T,H]; perm, expert_offsets [device] from moe_permute;
 *   w_gate, w_up [device] [E,F,H]; h_act [device] out [T*k,F] bf16.
 * Always the invariant kernels (the load-dependent variant of this GEMM is
 * reached through moe_grouped_swiglu, moe_forward and moe_forward_replay). */
int moe_expert_gate_up(int T, int H, int E, int F, int top_k, const uint16_t* x,
                       const int32_t* perm, const int32_t* expert_offsets,
                       const uint16_t* w_gate, const uint16_t* w_up, uint16_t* h_act,
                       void* ws, size_t ws_bytes, void* stream);

/* Down projection grouped by expert (the second expert GEMM), under the same
 * fixed-kernel rule as the gate/up GEMM (same page and sections): for every
 * permuted row p of expert e, y[perm[p], h] = h_act[p,:] . w_down[e,h,:] in
 * fp32, written to assignment order.
 *   h_act [device] [T*k,F] bf16; w_down [device] [E,H,F]; y [device] out
 *   [T*k,H] fp32.  variant: moe_gemm_variant (the variant's partial sums live
 *   in the workspace, which is then larger: moe_workspace_bytes with the
 *   same variant). */
int moe_expert_down(int T, int H, int E, int F, int top_k, const uint16_t* h_act,
                    const int32_t* perm, const int32_t* expert_offsets,
                    const uint16_t* w_down, float* y, int variant,
                    void* ws, size_t ws_bytes, void* stream);

/* Both expert GEMMs (the grouped SwiGLU expert FFN; same page and sections
 * as moe_expert_gate_up): moe_expert_gate_up then moe_expert_down, with
 * h_act kept in the workspace. */
int moe_grouped_swiglu(int T, int H, int E, int F, int top_k, const uint16_t* x,
                       const int32_t* perm, const int32_t* expert_offsets,
                       const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, float* y, int variant,
                       void* ws, size_t ws_bytes, void* stream);

/* Fixed-order fp32 weighted combine (the "combine" step).  Both the
 * precision and the order of the weighted sum of the expert outputs must be
 * fixed (Fireworks page on numerical alignment and MoE routing, section
 * "混合专家模型更难对齐"):
 *   out[t,h] = bf16(fma chain over j = 0..k-1 of topk_w[t,j] * y[t*k+j,h]).
 *   y [device] [T*k,H] fp32; topk_w [device] [T,k]; out [device] out [T,H]. */
int moe_combine(int T, int H, int top_k, const float* y, const float* topk_w,
                uint16_t* out, void* stream);

/* The whole layer: route, permute, both expert GEMMs, combine, enqueued in
 * that order on `stream`.  Each token's out is bit-identical whatever else
 * shares the call (Fireworks page "位级一致：前沿训练的差异化关键", sections
 * "曾经只有前沿实验室才有的功能" and "端到端零 KLD").  topk_ids / topk_w may be NULL (then they live in
 * the workspace); when given they receive the routing. */
int moe_forward(int T, int H, int E, int F, int top_k, int score, int renormalize,
                const uint16_t* x, const uint16_t* w_router, const float* bias,
                const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                uint16_t* out, int32_t* topk_ids, float* topk_w, int variant,
                void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  Arguments and results are those of
 * moe_forward (same kernels, bit-identical out, topk_ids and topk_w); the
 * workspace is a static array inside the library, 32 MiB per GPU, which each
 * GPU the library runs on holds until the process ends.  The call allocates
 * and frees nothing.  Sizes whose moe_forward workspace
 * (moe_workspace_bytes(MOE_OP_FORWARD, ...)) exceeds 32 MiB are rejected
 * with MOE_ERR_SCRATCH before anything is enqueued (e.g. H = 6144, F = 2048,
 * E = 256, top_k = 8 fits up to T = 132 tokens).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be ordered by
 * the caller.  The array keeps the last call's contents; nothing in the
 * layer reads scratch it has not written in the same call. */
int moe_forward_static(int T, int H, int E, int F, int top_k, int score, int renormalize,
                       const uint16_t* x, const uint16_t* w_router, const float* bias,
                       const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                       uint16_t* out, int32_t* topk_ids, float* topk_w, int variant,
                       void* stream);

/* Router replay: the whole layer with each token's experts given instead of
 * selected.  The pages describe recording the routing decisions taken while
 * generating a rollout and reusing them in the trainer, so that both use the
 * same experts (best2ai.com page on numerical alignment and MoE routing,
 * sections "MoE 路由会放大这种不匹配" and "Fireworks 保持训练循环一致";
 * Fireworks page "位级一致：前沿训练的差异化关键", section
 * "曾经只有前沿实验室才有的功能", names it the popular MoE fix).
 *   topk_ids [device] [T,k] int32: the recorded experts, in recorded slot
 *     order.  An id outside [0,E) contributes nothing: its expert output is
 *     0 and, when weights are recomputed, its weight is 0 and it is left out
 *     of the renormalisation.
 *   topk_w [device] [T,k] fp32, or NULL: the recorded weights.  When NULL,
 *     the weights are recomputed from w_router for the given experts exactly
 *     as moe_route computes them (score, renormalize; the bias only shapes
 *     selection, so it is not an argument), and w_out [device] [T,k] (may be
 *     NULL) receives them.  w_router may be NULL when topk_w is given.
 *   Everything else as moe_forward; the workspace is moe_forward's
 *   (moe_workspace_bytes(MOE_OP_FORWARD, ...)).
 * Replaying the ids (and weights) that moe_forward returned for the same
 * inputs gives an out bit-identical to moe_forward's. */
int moe_forward_replay(int T, int H, int E, int F, int top_k, int score, int renormalize,
                       const uint16_t* x, const uint16_t* w_router, const int32_t* topk_ids,
                       const float* topk_w, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, uint16_t* out, float* w_out, int variant,
                       void* ws, size_t ws_bytes, void* stream);

/* Large-k top-k of a sparse attention indexer: for every query row, the top
 * k (2048 on the pages) of its scores.  A non-deterministic indexer top-k
 * made the trainer see other tokens than the rollout, and ties at the
 * boundary, sort stability, NaN handling and the index dtype all change the
 * chosen set ("GLM Post-Training Beyond SFT", sections
 * "DSA 的确定性为什么是 RL 问题" and "迁移到 NPU 时", and its sparse/version
 * contract).  Order: score descending, then index ascending; -0 == +0; a
 * NaN ranks below every other score (-inf included), NaNs by index.
 *   scores [device] [Q,N] fp32;
 *   lengths [device] [Q] int32 or NULL: row q considers scores[q, 0..len)
 *     (clamped to [0,N]); NULL = all N (a causal indexer passes the prefix);
 *   idx [device] out [Q,k] int32: slot j = the j-th selected index, slots
 *     past min(k, len) = -1;
 *   vals [device] out [Q,k] fp32 or NULL: the selected scores (NaN in
 *     the -1 slots).
 * Limits: 0 <= Q; 1 <= N <= 2^24; 1 <= k <= 4096; Q*N < 2^31.  Each row's
 * result depends on that row only.  Per-shard lists merged under the same
 * order give the same list as one call over the whole row. */
int moe_topk_large(int Q, int N, int k, const float* scores, const int32_t* lengths,
                   int32_t* idx, float* vals, void* stream);

/* ------------------------------------------------------------------------
 * The measurement downstream of a decode step.  What training and serving
 * finally compare is the log-probability of the next token and a KL estimate
 * (k3) between two runs, judged against a 0.001 threshold (best2ai.com page
 * on numerical alignment and MoE routing, sections "数值差异如何扰乱学习" and
 * "混合专家模型更难对齐").  The pages fix neither the projection's order nor
 * the sums; these entry points pin both, so a token's results never depend
 * on what else is in the call.  Limits: H a multiple of 64 in [64, 65536];
 * 1 <= V <= 2^20; 0 <= T; T*V < 2^31.  moe_log_softmax and moe_k3 take a
 * workspace of moe_workspace_bytes(MOE_OP_LOG_SOFTMAX / MOE_OP_K3, T, V, ...)
 * bytes (the per-row segment maxima and chunk sums, about 4 KB per row at
 * V = 65536); the vocabulary projection takes none.
 * ------------------------------------------------------------------------ */

/* Vocabulary projection (LM head) of layer outputs:
 *   z[t,v] = sum_i h[t,i] * proj[v,i] in fp32, in the logits' order (i in
 *   chunks of 256, each an ascending fp32 fma chain from +0, chunk sums added
 *   in ascending order).
 *   h [device] [T,H] bf16; proj [device] [V,H] bf16; z [device] out [T,V]. */
int moe_lm_head_logits(int T, int H, int V, const uint16_t* h, const uint16_t* proj,
                       float* z, void* stream);

/* fp32 log-softmax over v with fixed sums:
 *   m = max_v z; S = +0, for each chunk of 256 consecutive v (ascending):
 *   s = +0, s = s + exp32(z_v - m) for v ascending, S = S + s;
 *   logp[t,v] = z[t,v] - (m + log32(S)), every operation in fp32, where
 *   exp32 and log32 are the exponential and logarithm correctly rounded to
 *   fp32 (evaluated as the fp64 function rounded once).
 *   z [device] [T,V] fp32; logp [device] out [T,V] fp32; logp == z allowed
 *   (in place).  NaN inputs give NaN rows.  ws [device]: the workspace. */
int moe_log_softmax(int T, int V, const float* z, float* logp, void* ws, size_t ws_bytes,
                    void* stream);

/* Schulman's k3 estimator, r = p_ref / p_test, per row t:
 *   d_v = logp_ref[t,v] - logp_test[t,v] (fp64),
 *   k3_mean[t]   = sum_v exp(logp_test[t,v]) * (expm1(d_v) - d_v) in fp64,
 *                  summed in the log-softmax's chunked order (this is the
 *                  KL divergence of p_test from p_ref; identical rows give
 *                  exactly 0);
 *   greedy[t]    = the lowest v with the largest logp_test[t,v] (0 if
 *                  logp_test[t,0] is NaN; other NaNs are skipped);
 *   k3_greedy[t] = expm1(d) - d at v = greedy[t] (unweighted).
 *   logp_ref, logp_test [device] [T,V] fp32; k3_mean, k3_greedy [device] out
 *   [T] fp64; greedy [device] out [T] int32; ws [device]: the workspace. */
int moe_k3(int T, int V, const float* logp_ref, const float* logp_test, double* k3_mean,
           double* k3_greedy, int32_t* greedy, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FP8 rollout path.  The pages' large-MoE recipe trains in BF16, samples
 * rollouts with FP8 expert weights converted from the BF16 ones, and keeps
 * measuring the gap between the two ("GLM Post-Training Beyond SFT",
 * quantisation section).  They fix no format; the reading taken:
 *   codes     OCP E4M3FN bytes (uint8): bias 7, 3 mantissa bits,
 *             subnormals, largest 448, 0x7F/0xFF NaN; fp32 -> e4m3 rounds to
 *             nearest, ties to even.
 *   exponents one signed byte e per block, value ~ code * 2^e, e = the
 *             smallest integer with max|v| <= 448 * 2^e over the block,
 *             clamped to [-127, 127] (0 for an all-zero block, 127 if the
 *             block holds an infinity).  Weight blocks are 128 output rows x
 *             128 K, activation blocks 1 row x 128 K.
 *   GEMM      out = fp32 sum over K blocks, ascending, of 2^(ea + ew) x the
 *             block's sum of 128 code products; the matrix unit forms each
 *             block sum in groups of 8 products aligned to the group's
 *             largest (products more than 13 binades below it are cut
 *             toward zero), so an output is within 7 * 2^-13 * sum over
 *             groups of the largest |product| (times 2^(ea+ew)) plus fp32
 *             roundings of the exact-block-sum value.
 *   expert    g, u by the GEMM; act = bf16(silu(g) * u); act is quantised
 *             by rows for the down GEMM.  Routing and combine are those of
 *             the bf16 layer (the router stays bf16).
 * Layouts: weights as the bf16 ones (w_gate/w_up codes [E,F,H] with
 * exponents [E,F/128,H/128]; w_down codes [E,H,F] with [E,H/128,F/128]).
 * Limits: those of the bf16 layer, and H, F multiples of 128 with the K side
 * of each GEMM (H for gate/up, F for down) at most 8192 (else
 * MOE_ERR_UNSUPPORTED / MOE_ERR_SHAPE).  Batch invariance holds as in the
 * bf16 GEMMs: one tile, one instruction, ascending K blocks, no split.
 * ------------------------------------------------------------------------ */

/* Block quantiser: src [device] [R,K] bf16 -> q [device] out [R,K] e4m3 codes
 * and exps [device] out [R/block_rows, K/128] int8.  Rows r*block_rows ..
 * (r+1)*block_rows - 1 and 128 consecutive columns form a block (weights
 * [E,N,K] pass R = E*N rows with block_rows = 128; activations pass
 * block_rows = 1).  Limits: 0 <= R, 1 <= block_rows, R % block_rows == 0,
 * K % 128 == 0, 128 <= K <= 65536, R*K <= 2^40 (a whole expert weight
 * tensor in one call).  No workspace. */
int moe_quantize_fp8(int R, int K, int block_rows, const uint16_t* src, uint8_t* q,
                     int8_t* exps, void* stream);

/* FP8 gate/up GEMM with the SwiGLU epilogue, quantising its output:
 *   xq [device] [T,H] codes, xe [device] [T,H/128] exps (x quantised by
 *   rows); perm, expert_offsets as moe_expert_gate_up; wg_q, wu_q [device]
 *   [E,F,H] codes with wg_e, wu_e [device] [E,F/128,H/128];
 *   act_q [device] out [T*k,F] codes and act_e [device] out [T*k,F/128]
 *   exps of act = bf16(silu(g)*u), rows in permuted order;
 *   act_bf16 [device] out [T*k,F] bf16 or NULL: act itself.
 *   ws: moe_workspace_bytes(MOE_OP_GATE_UP_FP8, ...); a call of at most 32
 *   tokens streams the weights (same bits) and keeps act there when
 *   act_bf16 is NULL.  Rows outside every expert segment are not written. */
int moe_expert_gate_up_fp8(int T, int H, int E, int F, int top_k, const uint8_t* xq,
                           const int8_t* xe, const int32_t* perm, const int32_t* expert_offsets,
                           const uint8_t* wg_q, const int8_t* wg_e, const uint8_t* wu_q,
                           const int8_t* wu_e, uint8_t* act_q, int8_t* act_e, uint16_t* act_bf16,
                           void* ws, size_t ws_bytes, void* stream);

/* FP8 down GEMM: act_q [device] [T*k,F] codes with act_e [T*k,F/128] (rows
 * in permuted order, as moe_expert_gate_up_fp8 writes them); wd_q [device]
 * [E,H,F] codes with wd_e [E,H/128,F/128]; y [device] out [T*k,H] fp32 in
 * assignment order.  ws: moe_workspace_bytes(MOE_OP_DOWN_FP8, ...). */
int moe_expert_down_fp8(int T, int H, int E, int F, int top_k, const uint8_t* act_q,
                        const int8_t* act_e, const int32_t* perm, const int32_t* expert_offsets,
                        const uint8_t* wd_q, const int8_t* wd_e, float* y, void* ws,
                        size_t ws_bytes, void* stream);

/* The FP8 layer: bf16 routing (as moe_forward), x quantised by rows,
 * permute, the two FP8 GEMMs, the fixed-order combine.  Weights are passed
 * quantised (moe_quantize_fp8 once, at load time).  topk_ids / topk_w as in
 * moe_forward.  ws: moe_workspace_bytes(MOE_OP_FORWARD_FP8, ...). */
int moe_forward_fp8(int T, int H, int E, int F, int top_k, int score, int renormalize,
                    const uint16_t* x, const uint16_t* w_router, const float* bias,
                    const uint8_t* wg_q, const int8_t* wg_e, const uint8_t* wu_q,
                    const int8_t* wu_e, const uint8_t* wd_q, const int8_t* wd_e, uint16_t* out,
                    int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
