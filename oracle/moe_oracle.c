/*
 * moe_oracle.c -- plain, slow CPU oracle of the batch-invariant MoE layer
 * forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library) never calls it and shares no code with it.
 *
 * What the layer computes, and where the pages ask for it:
 *   - Fireworks page "位级一致：前沿训练的差异化关键" (bit-level agreement),
 *     section "为什么比特级一致是一个复杂的问题" (why bit-level agreement is
 *     hard): float addition is not associative; the router can nearly tie
 *     between experts; per-expert matmul kernels change with the per-expert
 *     token count.  The fix named there: one fixed kernel choice for the expert
 *     matmuls whatever the token count, and a deterministic router tie-break.
 *   - Same page, section "曾经只有前沿实验室才有的功能" (capabilities once
 *     exclusive to frontier labs): batch invariance means a request's result
 *     does not depend on what else shares its batch; the MoE router and the
 *     expert GEMMs are among the reductions that must stay consistent; split-K
 *     breaks invariance.
 *   - Fireworks page on numerical alignment and MoE routing (best2ai.com),
 *     section "混合专家模型更难对齐" (MoE models are harder to align): the
 *     precision and the order used to weight and sum the expert outputs must
 *     both be fixed.
 *   - "GLM Post-Training Beyond SFT", section "迁移到 NPU 时" (when moving to
 *     NPU) and the sparse/version contract: a top-k must fix ties at the
 *     boundary, sort stability, NaN handling and the index dtype, and is
 *     compared by index set and order.
 *
 * The pages never write the layer's formula.  The definition implemented here
 * (steps D1..D7) is the plainest reading consistent with them:
 *   D1 l[t,e]:  i = 0..H-1 is cut into chunks of 256 consecutive indices
 *               (the last may be shorter).  Each chunk is an fp32 chain in
 *               ascending i from +0: s = fma(x_i, w_i, s) (bf16 x bf16
 *               products are exact in fp32, so this equals multiply-then-add);
 *               then l = +0, l = l + s_c for c ascending, in fp32.  The logit
 *               decides an integer (the expert set), so it is taken in the
 *               kernel's precision and in one fixed order.  The pages fix no
 *               order; the chunked one lets the many short chains of a small
 *               batch run in parallel.
 *   D2 keys:   softmax -> key_e = l_e (softmax is strictly increasing, so the
 *               top-k of the logits is the top-k of the exact probabilities);
 *               sigmoid -> key_e = fp32(1/(1+expf(-l_e))) + bias_e in fp32.
 *   D3 top-k:  order by key descending, then expert index ascending; -0 equals
 *               +0; a NaN key ranks below every other key (also below -inf),
 *               NaNs among themselves by index.  Slot j holds the j-th.
 *   D4 weights (fp64, rounded to fp32 once): softmax p_e = exp(l_e-m)/sum_e
 *               exp(l_e-m) with m = max_e l_e; sigmoid p_e = 1/(1+exp(-l_e));
 *               renormalised w_j = p_{e_j} / sum_j p_{e_j}, else w_j = p_{e_j}.
 *               The bias never enters the weights.
 *   D5 permute: counts[e], offsets = exclusive prefix sum, perm lists the
 *               assignment ids a = t*k + j routed to e in ascending a,
 *               inv_perm[perm[p]] = p.
 *   D6 expert:  g_f = sum_i x_i Wg[e,f,i], u_f = sum_i x_i Wu[e,f,i] (fp64);
 *               act_f = bf16_rne(fp32(silu(g_f) * u_f)), silu(g) = g/(1+e^-g);
 *               Y[a,h] = fp32(sum_f act_f Wd[e,h,f]) (fp64 sum, one rounding).
 *               act is a stored bf16 code, so it is rounded from fp32, the
 *               precision the kernel decides it in.
 *   D7 combine: acc = +0.0f; for j = 0..k-1: acc = fmaf(w[t,j], Y[t*k+j,h], acc);
 *               out[t,h] = bf16_rne(acc).  The precision (fp32) and the order
 *               (slot order) are both part of the definition.
 *
 * Everything is plain loops.  Tokens are independent, so the token loop may
 * run on several threads; every per-token result is the same at any thread
 * count.  Built with -ffp-contract=off: every fma below is an explicit call.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

float orc_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even.  NaN stays a (quiet) NaN with
 * its sign; overflow rounds to +-inf as IEEE rounding does. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t b = bits_from_f32(f);
    if (isnan(f))
        return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t upper = b >> 16;
    uint32_t lower = b & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;  /* carries into the exponent where needed, up to inf */
    return (uint16_t)upper;
}

void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int orc_max_threads(void) { return set_threads(0); }

/* ------------------------------------------------------------------------ */
/* D1: router logits                                                         */
/* ------------------------------------------------------------------------ */

#define ORC_LOGIT_CHUNK 256

static float logit_one(const uint16_t* xrow, const uint16_t* wrow, int H)
{
    float total = 0.0f;
    for (int c0 = 0; c0 < H; c0 += ORC_LOGIT_CHUNK) {
        int c1 = c0 + ORC_LOGIT_CHUNK < H ? c0 + ORC_LOGIT_CHUNK : H;
        float s = 0.0f;
        for (int i = c0; i < c1; ++i)
            s = fmaf(orc_bf16_to_f32(xrow[i]), orc_bf16_to_f32(wrow[i]), s);
        total = total + s;
    }
    return total;
}

void orc_router_logits(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                       float* logits, int nthreads)
{
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 4)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e)
            logits[(int64_t)t * E + e] = logit_one(x + (int64_t)t * H, wr + (int64_t)e * H, H);
}

/* ------------------------------------------------------------------------ */
/* D2 + D3: selection keys and top-k                                         */
/* ------------------------------------------------------------------------ */

/* Is expert a (key ka) ahead of expert b (key kb) in selection order? */
static int ranks_before(float ka, int a, float kb, int b)
{
    int na = isnan(ka), nb = isnan(kb);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb;  /* the non-NaN one is ahead */
    }
    if (ka > kb) return 1;
    if (ka < kb) return 0;
    return a < b;   /* equal by value (covers -0 == +0): lower index first */
}

/* Select k of E keys: repeated scans for the best key not yet taken. */
static void select_topk(const float* key, int E, int k, int32_t* ids, unsigned char* taken)
{
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || ranks_before(key[e], e, key[best], best)) best = e;
        }
        taken[best] = 1;
        ids[j] = best;
    }
}

/* Top-k over given keys (exported for the tie/NaN pin tests). */
void orc_topk_keys(int n, int E, int k, const float* keys, int32_t* ids)
{
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int r = 0; r < n; ++r)
        select_topk(keys + (int64_t)r * E, E, k, ids + (int64_t)r * k, taken);
    free(taken);
}

static float sigmoid_key_f32(float l, float b)
{
    float s = 1.0f / (1.0f + expf(-l));
    return s + b;
}

/* D4: the weights of the experts ids[0..k-1] from one token's logits, in
 * fp64, rounded to fp32 once.  An id outside [0,E) (router replay only) gets
 * weight 0 and is left out of the renormalisation; a zero sum gives zeros. */
static void weights_for(const float* logits, int E, int k, int score, int renorm,
                        const int32_t* ids, float* w)
{
    double p[16];
    if (score == ORC_SOFTMAX) {
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if ((double)logits[e] > m) m = (double)logits[e];
        double S = 0.0;
        for (int e = 0; e < E; ++e) S += exp((double)logits[e] - m);
        for (int j = 0; j < k; ++j)
            p[j] = (ids[j] >= 0 && ids[j] < E) ? exp((double)logits[ids[j]] - m) / S : 0.0;
    } else {
        for (int j = 0; j < k; ++j)
            p[j] = (ids[j] >= 0 && ids[j] < E) ? 1.0 / (1.0 + exp(-(double)logits[ids[j]])) : 0.0;
    }
    if (renorm) {
        double D = 0.0;
        for (int j = 0; j < k; ++j) D += p[j];
        for (int j = 0; j < k; ++j) w[j] = D > 0.0 ? (float)(p[j] / D) : 0.0f;
    } else {
        for (int j = 0; j < k; ++j) w[j] = (float)p[j];
    }
}

/* D1..D4 for one token. scratch: 2*E floats + E bytes. */
static void route_one(const uint16_t* xrow, const uint16_t* wr, const float* bias,
                      int H, int E, int k, int score, int renorm,
                      int32_t* ids, float* w, double* gap, float* keys, float* logits,
                      unsigned char* taken)
{
    for (int e = 0; e < E; ++e) logits[e] = logit_one(xrow, wr + (int64_t)e * H, H);
    for (int e = 0; e < E; ++e)
        keys[e] = (score == ORC_SOFTMAX) ? logits[e]
                                         : sigmoid_key_f32(logits[e], bias ? bias[e] : 0.0f);
    select_topk(keys, E, k, ids, taken);

    /* gap between the k-th and (k+1)-th key, in fp64 (diagnostic for the
     * near-tie exemption); +inf when k == E */
    if (gap) {
        if (k >= E) {
            *gap = INFINITY;
        } else {
            int next = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (next < 0 || ranks_before(keys[e], e, keys[next], next)) next = e;
            }
            *gap = (double)keys[ids[k - 1]] - (double)keys[next];
        }
    }

    weights_for(logits, E, k, score, renorm, ids, w);
}

/* Route T tokens.  ids [T,k] int32, w [T,k] fp32, gap [T] fp64 (or NULL). */
int orc_route(int T, int H, int E, int k, int score, int renorm,
              const uint16_t* x, const uint16_t* wr, const float* bias,
              int32_t* ids, float* w, double* gap, int nthreads)
{
    if (k < 1 || k > E || k > 16) return -2;
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        float* keys = (float*)malloc(sizeof(float) * (size_t)E * 2);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(dynamic, 4)
        for (int t = 0; t < T; ++t)
            route_one(x + (int64_t)t * H, wr, bias, H, E, k, score, renorm,
                      ids + (int64_t)t * k, w + (int64_t)t * k, gap ? gap + t : NULL,
                      keys, keys + E, taken);
        free(keys);
        free(taken);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* D5: histogram, offsets and the stable permutation                         */
/* ------------------------------------------------------------------------ */

int orc_permute(int A, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* inv_perm)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int a = 0; a < A; ++a) {
        if (ids[a] < 0 || ids[a] >= E) return -2;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    /* walk assignments in ascending id; each lands after the earlier ones of
     * its expert (a stable counting sort) */
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int a = 0; a < A; ++a) {
        int p = fill[ids[a]]++;
        perm[p] = a;
        inv_perm[a] = p;
    }
    free(fill);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* D6: one expert's SwiGLU FFN for one token                                 */
/* ------------------------------------------------------------------------ */

static double silu_d(double g) { return g / (1.0 + exp(-g)); }

/* act_out [F] bf16 (may be NULL), y_out [H] fp32.  scratch [F] doubles. */
static void expert_one(const uint16_t* xrow, int e, int H, int F,
                       const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                       uint16_t* act_out, float* y_out, double* act_d)
{
    const uint16_t* G = wg + (int64_t)e * F * H;
    const uint16_t* U = wu + (int64_t)e * F * H;
    const uint16_t* D = wd + (int64_t)e * H * F;
    for (int f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        const uint16_t* gr = G + (int64_t)f * H;
        const uint16_t* ur = U + (int64_t)f * H;
        for (int i = 0; i < H; ++i) {
            double xi = (double)orc_bf16_to_f32(xrow[i]);
            g += xi * (double)orc_bf16_to_f32(gr[i]);
            u += xi * (double)orc_bf16_to_f32(ur[i]);
        }
        uint16_t a = orc_f32_to_bf16((float)(silu_d(g) * u));
        if (act_out) act_out[f] = a;
        act_d[f] = (double)orc_bf16_to_f32(a);
    }
    for (int h = 0; h < H; ++h) {
        const uint16_t* dr = D + (int64_t)h * F;
        double y = 0.0;
        for (int f = 0; f < F; ++f) y += act_d[f] * (double)orc_bf16_to_f32(dr[f]);
        y_out[h] = (float)y;
    }
}

/* n (token, expert) pairs -> act [n,F] bf16 (or NULL) and y [n,H] fp32. */
int orc_expert_ffn(int n, const int32_t* tokens, const int32_t* experts,
                   int H, int E, int F, const uint16_t* x,
                   const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                   uint16_t* act, float* y, int nthreads)
{
    for (int r = 0; r < n; ++r)
        if (experts[r] < 0 || experts[r] >= E) return -2;
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        double* act_d = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n; ++r)
            expert_one(x + (int64_t)tokens[r] * H, experts[r], H, F, wg, wu, wd,
                       act ? act + (int64_t)r * F : NULL, y + (int64_t)r * H, act_d);
        free(act_d);
    }
    return 0;
}

/* The down projection of D6 alone, on given act codes: n rows, row r uses
 * expert experts[r] and act[r, :] (bf16 bits); y[r,h] = fp32(sum_f act Wd)
 * with an fp64 sum.  Lets a test check the second expert GEMM on the first
 * one's output. */
int orc_expert_down(int n, const int32_t* experts, int H, int E, int F,
                    const uint16_t* act, const uint16_t* wd, float* y, int nthreads)
{
    for (int r = 0; r < n; ++r)
        if (experts[r] < 0 || experts[r] >= E) return -2;
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int r = 0; r < n; ++r) {
        const uint16_t* D = wd + (int64_t)experts[r] * H * F;
        const uint16_t* a = act + (int64_t)r * F;
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int f = 0; f < F; ++f)
                acc += (double)orc_bf16_to_f32(a[f]) * (double)orc_bf16_to_f32(D[(int64_t)h * F + f]);
            y[(int64_t)r * H + h] = (float)acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* D7: fixed-order fp32 combine                                              */
/* ------------------------------------------------------------------------ */

static void combine_one(const float* y_tok /* [k,H] */, const float* w, int H, int k,
                        uint16_t* out_row)
{
    for (int h = 0; h < H; ++h) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) acc = fmaf(w[j], y_tok[(int64_t)j * H + h], acc);
        out_row[h] = orc_f32_to_bf16(acc);
    }
}

void orc_combine(int T, int H, int k, const float* y, const float* w, uint16_t* out)
{
    for (int t = 0; t < T; ++t)
        combine_one(y + (int64_t)t * k * H, w + (int64_t)t * k, H, k, out + (int64_t)t * H);
}

/* ------------------------------------------------------------------------ */
/* whole layer                                                               */
/* ------------------------------------------------------------------------ */

/* The layer in the method's order: route all tokens, permute, run each
 * expert over its segment of the permutation, combine.  Optional outputs
 * (NULL to skip): ids [T,k], w [T,k], gap [T], counts [E], offsets [E+1],
 * perm [A], inv_perm [A], y [A,H] (assignment order). */
int orc_forward(int T, int H, int E, int F, int k, int score, int renorm,
                const uint16_t* x, const uint16_t* wr, const float* bias,
                const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                uint16_t* out, int32_t* ids_o, float* w_o, double* gap_o,
                int32_t* counts_o, int32_t* offsets_o, int32_t* perm_o,
                int32_t* inv_perm_o, float* y_o, int nthreads)
{
    if (k < 1 || k > E || k > 16) return -2;
    int64_t A = (int64_t)T * k;
    int32_t* ids = ids_o ? ids_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
    float* w = w_o ? w_o : (float*)malloc(sizeof(float) * (size_t)(A + 1));
    int32_t* counts = counts_o ? counts_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = offsets_o ? offsets_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* perm = perm_o ? perm_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
    int32_t* inv = inv_perm_o ? inv_perm_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
    float* y = y_o ? y_o : (float*)malloc(sizeof(float) * (size_t)(A * H + 1));
    int rc = orc_route(T, H, E, k, score, renorm, x, wr, bias, ids, w, gap_o, nthreads);
    if (rc == 0) rc = orc_permute((int)A, E, ids, counts, offsets, perm, inv);
    if (rc == 0) {
        /* expert by expert over its contiguous segment of the permutation */
        int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
        int32_t* exp_ = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
        float* yp = (float*)malloc(sizeof(float) * (size_t)(A * H + 1));
        for (int e = 0; e < E; ++e)
            for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
                tok[p] = perm[p] / k;
                exp_[p] = e;
            }
        rc = orc_expert_ffn((int)A, tok, exp_, H, E, F, x, wg, wu, wd, NULL, yp, nthreads);
        /* scatter expert outputs back to assignment order */
        for (int64_t p = 0; p < A; ++p)
            memcpy(y + (int64_t)perm[p] * H, yp + p * H, sizeof(float) * (size_t)H);
        free(tok); free(exp_); free(yp);
    }
    if (rc == 0) orc_combine(T, H, k, y, w, out);
    if (!ids_o) free(ids);
    if (!w_o) free(w);
    if (!counts_o) free(counts);
    if (!offsets_o) free(offsets);
    if (!perm_o) free(perm);
    if (!inv_perm_o) free(inv);
    if (!y_o) free(y);
    return rc;
}

/* Per-token evaluation of a chosen subset of tokens (no permutation): route
 * token t, run its k experts, combine.  Each token's result does not depend on
 * any other token, so this equals orc_forward on those rows.  out [n,H],
 * ids [n,k], w [n,k], gap [n] (optional). */
int orc_forward_tokens(int n, const int32_t* tokens, int H, int E, int F, int k,
                       int score, int renorm, const uint16_t* x, const uint16_t* wr,
                       const float* bias, const uint16_t* wg, const uint16_t* wu,
                       const uint16_t* wd, uint16_t* out, int32_t* ids_o, float* w_o,
                       double* gap_o, int nthreads)
{
    if (k < 1 || k > E || k > 16) return -2;
    int nt = set_threads(nthreads);
    (void)nt;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)n * k + 4);
    float* w = (float*)malloc(sizeof(float) * (size_t)n * k + 4);
    float* y = (float*)malloc(sizeof(float) * ((size_t)n * k * H + 1));
#pragma omp parallel num_threads(nt)
    {
        float* keys = (float*)malloc(sizeof(float) * (size_t)E * 2);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        double* act_d = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n * k; ++r) {
            int i = r / k, j = r % k;
            const uint16_t* xrow = x + (int64_t)tokens[i] * H;
            int32_t sel[16];
            float wsel[16];
            route_one(xrow, wr, bias, H, E, k, score, renorm, sel, wsel,
                      (j == 0 && gap_o) ? gap_o + i : NULL, keys, keys + E, taken);
            if (j == 0)
                for (int q = 0; q < k; ++q) {
                    ids[(int64_t)i * k + q] = sel[q];
                    w[(int64_t)i * k + q] = wsel[q];
                }
            expert_one(xrow, sel[j], H, F, wg, wu, wd, NULL, y + (int64_t)r * H, act_d);
        }
        free(keys); free(taken); free(act_d);
    }
    orc_combine(n, H, k, y, w, out);
    if (ids_o) memcpy(ids_o, ids, sizeof(int32_t) * (size_t)n * k);
    if (w_o) memcpy(w_o, w, sizeof(float) * (size_t)n * k);
    free(ids); free(w); free(y);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* D8: the downstream measurement of a decode step                           */
/* ------------------------------------------------------------------------ */
/*
 * Bit-identical layer outputs are a means; what training and serving compare
 * is the log-probability a model assigns to the next token, and a KL
 * estimate ("k3") between two runs, compared with a small threshold (the
 * best2ai.com page on numerical alignment and MoE routing, sections
 * "数值差异如何扰乱学习" and "混合专家模型更难对齐").  The pages fix neither
 * the projection's order nor the sums.  Reading taken here: the same pinned
 * order as D1, and fixed chunked sums.
 *   z[t,v]    = the D1 chain of out[t,:] against proj[v,:] (bf16 x bf16, fp32);
 *   m         = max_v z[t,v];
 *   S         = +0; for each chunk of 256 consecutive v (ascending): s = +0,
 *               s = s + exp32(z_v - m) for v ascending; S = S + s   (fp32);
 *   logp[t,v] = z[t,v] - (m + log32(S))                              (fp32);
 *   exp32(a), log32(a): the fp32 exponential and logarithm, correctly rounded
 *               (the exact value rounded to nearest fp32, ties to even).  They
 *               are evaluated as the fp64 library function rounded once to
 *               fp32, which is the correctly rounded value unless the exact
 *               value lies within an fp64 ulp of an fp32 rounding boundary.
 *               Fixing the transcendental's rounding (rather than taking
 *               whatever a platform's single-precision expf returns) is what
 *               lets two implementations of S agree bit for bit.
 *   k3        (Schulman's estimator, r = p_ref / p_test):
 *               d_v = logp_ref[v] - logp_test[v] (fp64), r - 1 = expm1(d_v),
 *               ln r = d_v; mean = sum_v exp(logp_test[v]) * (expm1(d_v) - d_v)
 *               in fp64, summed in the same chunked order as S; greedy = the
 *               lowest v with the largest logp_test, and the k3 term there
 *               (unweighted).  The mean is the KL divergence of p_test from
 *               p_ref; identical inputs give exactly 0.
 */

#define ORC_SUM_CHUNK 256

void orc_lm_head_logits(int T, int H, int V, const uint16_t* h, const uint16_t* proj,
                        float* z, int nthreads)
{
    orc_router_logits(T, H, V, h, proj, z, nthreads);
}

/* exp32 / log32 of the definition above */
float orc_exp32(float a) { return (float)exp((double)a); }
float orc_log32(float a) { return (float)log((double)a); }

static void log_softmax_row(const float* z, int V, float* logp)
{
    float m = -INFINITY;
    for (int v = 0; v < V; ++v) m = z[v] > m ? z[v] : m;
    float S = 0.0f;
    for (int c0 = 0; c0 < V; c0 += ORC_SUM_CHUNK) {
        int c1 = c0 + ORC_SUM_CHUNK < V ? c0 + ORC_SUM_CHUNK : V;
        float s = 0.0f;
        for (int v = c0; v < c1; ++v) s = s + orc_exp32(z[v] - m);
        S = S + s;
    }
    float lse = m + orc_log32(S);
    for (int v = 0; v < V; ++v) logp[v] = z[v] - lse;
}

void orc_log_softmax(int T, int V, const float* z, float* logp, int nthreads)
{
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int t = 0; t < T; ++t)
        log_softmax_row(z + (int64_t)t * V, V, logp + (int64_t)t * V);
}

static double k3_term(float ref, float test)
{
    double d = (double)ref - (double)test;
    return expm1(d) - d;
}

void orc_k3(int T, int V, const float* logp_ref, const float* logp_test, double* mean,
            double* greedy_k3, int32_t* greedy)
{
    for (int t = 0; t < T; ++t) {
        const float* r = logp_ref + (int64_t)t * V;
        const float* q = logp_test + (int64_t)t * V;
        double S = 0.0;
        for (int c0 = 0; c0 < V; c0 += ORC_SUM_CHUNK) {
            int c1 = c0 + ORC_SUM_CHUNK < V ? c0 + ORC_SUM_CHUNK : V;
            double s = 0.0;
            for (int v = c0; v < c1; ++v) s = s + exp((double)q[v]) * k3_term(r[v], q[v]);
            S = S + s;
        }
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (q[v] > q[best]) best = v;
        mean[t] = S;
        greedy[t] = best;
        greedy_k3[t] = k3_term(r[best], q[best]);
    }
}

/* ------------------------------------------------------------------------ */
/* Router replay                                                             */
/* ------------------------------------------------------------------------ */
/*
 * The pages describe router replay as recording the expert choices made
 * while generating a rollout and reusing them in the trainer (best2ai.com
 * page on numerical alignment and MoE routing, sections
 * "MoE 路由会放大这种不匹配" and "Fireworks 保持训练循环一致").  Reading
 * taken: the layer of D5..D7 with the experts of each slot given (ids
 * [T,k], recorded slot order); the weights either given too, or those of D4
 * for the given experts.  An id outside [0,E) contributes nothing (expert
 * output 0; weight 0 when recomputed, and left out of the renormalisation).
 * Evaluated token by token (no permutation), like orc_forward_tokens.
 */
int orc_replay_weights(int T, int H, int E, int k, int score, int renorm, const uint16_t* x,
                       const uint16_t* wr, const int32_t* ids, float* w, int nthreads)
{
    if (k < 1 || k > 16) return -2;
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        float* logits = (float*)malloc(sizeof(float) * (size_t)E);
#pragma omp for schedule(dynamic, 4)
        for (int t = 0; t < T; ++t) {
            const uint16_t* xrow = x + (int64_t)t * H;
            for (int e = 0; e < E; ++e) logits[e] = logit_one(xrow, wr + (int64_t)e * H, H);
            weights_for(logits, E, k, score, renorm, ids + (int64_t)t * k, w + (int64_t)t * k);
        }
        free(logits);
    }
    return 0;
}

int orc_forward_replay(int T, int H, int E, int F, int k, int score, int renorm,
                       const uint16_t* x, const uint16_t* wr, const int32_t* ids,
                       const float* w_in, const uint16_t* wg, const uint16_t* wu,
                       const uint16_t* wd, uint16_t* out, float* w_out, int nthreads)
{
    if (k < 1 || k > 16) return -2;
    int nt = set_threads(nthreads);
    (void)nt;
    float* w = (float*)malloc(sizeof(float) * (size_t)T * k + 4);
    float* y = (float*)malloc(sizeof(float) * ((size_t)T * k * H + 1));
    if (w_in)
        memcpy(w, w_in, sizeof(float) * (size_t)T * k);
    else
        orc_replay_weights(T, H, E, k, score, renorm, x, wr, ids, w, nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* act_d = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < T * k; ++r) {
            const int t = r / k;
            const int e = ids[r];
            if (e < 0 || e >= E) {
                memset(y + (int64_t)r * H, 0, sizeof(float) * (size_t)H);
                continue;
            }
            expert_one(x + (int64_t)t * H, e, H, F, wg, wu, wd, NULL, y + (int64_t)r * H, act_d);
        }
        free(act_d);
    }
    orc_combine(T, H, k, y, w, out);
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)T * k);
    free(w);
    free(y);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Large-k top-k (the sparse attention indexer's selection)                  */
/* ------------------------------------------------------------------------ */
/*
 * A sparse attention indexer picks, for every query, the top 2048 keys; a
 * top-k that is not deterministic changed what the trainer saw from what the
 * rollout saw, and ties, sort stability, NaN handling and the index dtype
 * all change the chosen set ("GLM Post-Training Beyond SFT", sections
 * "DSA 的确定性为什么是 RL 问题", "迁移到 NPU 时" and the sparse/version
 * contract; the Fireworks bit-level page, section
 * "为什么比特级一致是一个复杂的问题", on the indexer returning one set in
 * different orders).  Reading taken: the order of D3 (score descending,
 * index ascending; -0 == +0; NaN below everything, NaNs by index) over the
 * first lengths[q] scores of row q (all N when lengths is NULL); slot j holds
 * the j-th; slots past min(k, lengths[q]) hold -1 (value NaN).  int32 ids.
 * Plain comparison sort of the row's indices under that total order.
 */
static const float* g_topk_row;   /* comparator context (sort is per thread) */
#ifdef _OPENMP
#pragma omp threadprivate(g_topk_row)
#endif

static int topk_cmp(const void* pa, const void* pb)
{
    int a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    if (a == b) return 0;
    return ranks_before(g_topk_row[a], a, g_topk_row[b], b) ? -1 : 1;
}

void orc_topk_large(int Q, int N, int k, const float* scores, const int32_t* lengths,
                    int32_t* idx, float* vals, int nthreads)
{
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int q = 0; q < Q; ++q) {
            int n = lengths ? lengths[q] : N;
            if (n < 0) n = 0;
            if (n > N) n = N;
            const float* row = scores + (int64_t)q * N;
            for (int i = 0; i < n; ++i) order[i] = i;
            g_topk_row = row;
            qsort(order, (size_t)n, sizeof(int32_t), topk_cmp);
            for (int j = 0; j < k; ++j) {
                int v = j < n ? order[j] : -1;
                idx[(int64_t)q * k + j] = v;
                if (vals) vals[(int64_t)q * k + j] = v >= 0 ? row[v] : NAN;
            }
        }
        free(order);
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 rollout path: e4m3 experts with block scales                          */
/* ------------------------------------------------------------------------ */
/*
 * The pages' large-MoE recipe trains in BF16 and samples rollouts with FP8
 * weights converted from the BF16 ones by the rollout's quantisation config,
 * and asks that the gap between the two policies' log-probabilities keep
 * being measured ("GLM Post-Training Beyond SFT", section on quantisation,
 * "量化：三件事不要混为一谈").  The pages give no format or block shape.
 * Reading taken:
 *   e4m3      OCP E4M3FN: bias 7, 3 mantissa bits, subnormals, max 448, no
 *             infinities; fp32 -> e4m3 rounds to nearest, ties to even; a
 *             NaN stays NaN.  Values beyond 448 never occur (the scales keep
 *             every value within range); they saturate to +-448 here.
 *   scales    powers of two, per block: e = the smallest integer with
 *             amax <= 448 * 2^e (amax = max |v| over the block; e = 0 for an
 *             all-zero block; clamped to [-127, 127], the range of a biased
 *             scale byte), q = e4m3(v * 2^-e), v ~ q * 2^e.  Weight blocks
 *             are 128 output rows x 128 K; activation blocks 1 row x 128 K.
 *   GEMM      out = sum over K blocks kb ascending, in fp32, of
 *             fp32(exact sum_{k in kb} qa*qw) * 2^(ea + ew); the products of
 *             two e4m3 codes and their 128-term sum are exact in fp64.
 *   expert    g, u by that GEMM (fp32); act = bf16(fp32(silu(g)*u)) with
 *             silu in fp64; act is quantised by rows (1 x 128 blocks) for
 *             the down GEMM; y = that GEMM, fp32.  Routing and combine are
 *             those of D1..D7 (the router stays bf16).
 */

#define ORC_FP8_MAX 448.0f
#define ORC_FP8_BLOCK 128

/* e4m3 code -> value */
float orc_e4m3_to_f32(uint8_t c)
{
    int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    float v;
    if (ex == 15 && m == 7) return s ? -NAN : NAN;
    if (ex == 0)
        v = ldexpf((float)m, -9);                 /* subnormal: m/8 * 2^-6 */
    else
        v = ldexpf(1.0f + (float)m / 8.0f, ex - 7);
    return s ? -v : v;
}

/* value -> e4m3 code: nearest, ties to even, saturating at +-448 */
uint8_t orc_f32_to_e4m3(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t s = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return s | 0x7E;
    /* the grid spacing at a: 2^(max(exponent, -6) - 3) */
    int e;
    if (a < ldexp(1.0, -6)) {
        e = -6;
    } else {
        frexp(a, &e);
        e -= 1;                                     /* a in [2^e, 2^(e+1)) */
    }
    double q = ldexp(1.0, e - 3);
    double n = floor(a / q);
    double r = a / q - n;                           /* exact: q is a power of two */
    if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) == 1.0)) n += 1.0;
    double val = n * q;                             /* the rounded magnitude */
    if (val >= 448.0) return s | 0x7E;
    if (val == 0.0) return s;
    int ve;
    frexp(val, &ve);
    ve -= 1;
    if (ve < -6) {                                  /* subnormal code */
        return s | (uint8_t)(int)(val / ldexp(1.0, -9));
    }
    int m = (int)((val / ldexp(1.0, ve) - 1.0) * 8.0);
    return s | (uint8_t)(((ve + 7) << 3) | m);
}

/* smallest integer e with amax <= 448 * 2^e (0 for amax == 0), clamped to
 * [-127, 127]: the exponent is stored in a signed byte and carried as a
 * biased scale byte (127 + e), whose range ends there.  A block whose amax is
 * below 448 * 2^-127 takes e = -127 (its codes are then not full-range); an
 * infinite amax takes 127. */
int orc_fp8_block_exp(float amax)
{
    if (!(amax > 0.0f)) return 0;
    if (isinf(amax)) return 127;
    int e = (int)floor(log2((double)amax / 448.0));
    while ((double)amax > 448.0 * ldexp(1.0, e)) ++e;
    while ((double)amax <= 448.0 * ldexp(1.0, e - 1)) --e;
    if (e < -127) e = -127;
    return e;
}

/* Quantise bf16 rows [R,K] in blocks of block_rows x 128: q [R,K] codes,
 * exps [R/block_rows, K/128] int8. */
void orc_quantize_fp8(int R, int K, int block_rows, const uint16_t* src, uint8_t* q,
                      int8_t* exps)
{
    int nkb = K / ORC_FP8_BLOCK;
    for (int rb = 0; rb < R / block_rows; ++rb)
        for (int kb = 0; kb < nkb; ++kb) {
            float amax = 0.0f;
            for (int r = rb * block_rows; r < (rb + 1) * block_rows; ++r)
                for (int k = kb * ORC_FP8_BLOCK; k < (kb + 1) * ORC_FP8_BLOCK; ++k) {
                    float a = fabsf(orc_bf16_to_f32(src[(int64_t)r * K + k]));
                    if (a > amax) amax = a;
                }
            int e = orc_fp8_block_exp(amax);
            exps[(int64_t)rb * nkb + kb] = (int8_t)e;
            for (int r = rb * block_rows; r < (rb + 1) * block_rows; ++r)
                for (int k = kb * ORC_FP8_BLOCK; k < (kb + 1) * ORC_FP8_BLOCK; ++k)
                    q[(int64_t)r * K + k] =
                        orc_f32_to_e4m3(ldexpf(orc_bf16_to_f32(src[(int64_t)r * K + k]), -e));
        }
}

/* One output of the block-scaled GEMM: a row of codes (with its per-block
 * exponents) against a weight row (with its block row's exponents). */
static float fp8_dot(const uint8_t* aq, const int8_t* ae, const uint8_t* wq, const int8_t* we,
                     int K)
{
    float acc = 0.0f;
    for (int kb = 0; kb < K / ORC_FP8_BLOCK; ++kb) {
        double s = 0.0;
        for (int k = kb * ORC_FP8_BLOCK; k < (kb + 1) * ORC_FP8_BLOCK; ++k)
            s += (double)orc_e4m3_to_f32(aq[k]) * (double)orc_e4m3_to_f32(wq[k]);
        acc = acc + ldexpf((float)s, ae[kb] + we[kb]);
    }
    return acc;
}

/* The block-scaled GEMM alone: row i of codes aq [n,K] (exponents ae
 * [n,K/128]) against the N weight rows of expert experts[i], wq [E,N,K] codes
 * with we [E,N/128,K/128]: y [n,N] fp32. */
int orc_fp8_gemm(int n, int K, int N, const uint8_t* aq, const int8_t* ae,
                 const int32_t* experts, const uint8_t* wq, const int8_t* we, float* y,
                 int nthreads)
{
    if (K % ORC_FP8_BLOCK || N % ORC_FP8_BLOCK) return -4;
    int nt = set_threads(nthreads);
    (void)nt;
    int nkb = K / ORC_FP8_BLOCK, nnb = N / ORC_FP8_BLOCK;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        int e = experts[i];
        for (int o = 0; o < N; ++o)
            y[(int64_t)i * N + o] =
                fp8_dot(aq + (int64_t)i * K, ae + (int64_t)i * nkb, wq + ((int64_t)e * N + o) * K,
                        we + ((int64_t)e * nnb + o / ORC_FP8_BLOCK) * nkb, K);
    }
    return 0;
}

/* FP8 expert FFN of n (token, expert) pairs.  xq [T,H] codes with xe
 * [T,H/128]; wgq, wuq [E,F,H] codes with wge, wue [E,F/128,H/128]; wdq
 * [E,H,F] codes with wde [E,H/128,F/128].  y [n,H] fp32; act [n,F] bf16 (or
 * NULL). */
int orc_expert_ffn_fp8(int n, const int32_t* tokens, const int32_t* experts, int H, int F,
                       const uint8_t* xq, const int8_t* xe, const uint8_t* wgq,
                       const int8_t* wge, const uint8_t* wuq, const int8_t* wue,
                       const uint8_t* wdq, const int8_t* wde, float* y, uint16_t* act_o,
                       int nthreads)
{
    if (H % ORC_FP8_BLOCK || F % ORC_FP8_BLOCK) return -4;
    int nt = set_threads(nthreads);
    (void)nt;
    int nhb = H / ORC_FP8_BLOCK, nfb = F / ORC_FP8_BLOCK;
#pragma omp parallel num_threads(nt)
    {
        uint16_t* act = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)F);
        uint8_t* aq = (uint8_t*)malloc((size_t)F);
        int8_t* ae = (int8_t*)malloc((size_t)nfb);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            int t = tokens[i], e = experts[i];
            const uint8_t* xr = xq + (int64_t)t * H;
            const int8_t* xer = xe + (int64_t)t * nhb;
            for (int f = 0; f < F; ++f) {
                int64_t row = (int64_t)e * F + f;
                const int8_t* geb = wge + ((int64_t)e * nfb + f / ORC_FP8_BLOCK) * nhb;
                const int8_t* ueb = wue + ((int64_t)e * nfb + f / ORC_FP8_BLOCK) * nhb;
                float g = fp8_dot(xr, xer, wgq + row * H, geb, H);
                float u = fp8_dot(xr, xer, wuq + row * H, ueb, H);
                double gd = (double)g;
                act[f] = orc_f32_to_bf16((float)(gd / (1.0 + exp(-gd)) * (double)u));
            }
            if (act_o) memcpy(act_o + (int64_t)i * F, act, sizeof(uint16_t) * (size_t)F);
            orc_quantize_fp8(1, F, 1, act, aq, ae);
            for (int h = 0; h < H; ++h) {
                int64_t row = (int64_t)e * H + h;
                const int8_t* deb = wde + ((int64_t)e * nhb + h / ORC_FP8_BLOCK) * nfb;
                y[(int64_t)i * H + h] = fp8_dot(aq, ae, wdq + row * F, deb, F);
            }
        }
        free(act); free(aq); free(ae);
    }
    return 0;
}

/* The FP8 layer for chosen tokens (per token, no permutation): routing of
 * D1..D4 on the bf16 router, experts by orc_expert_ffn_fp8, combine D7.
 * x [T,H] bf16 (routing) with xq/xe its quantised rows (experts). */
int orc_forward_tokens_fp8(int n, const int32_t* tokens, int H, int E, int F, int k,
                           int score, int renorm, const uint16_t* x, const uint16_t* wr,
                           const float* bias, const uint8_t* xq, const int8_t* xe,
                           const uint8_t* wgq, const int8_t* wge, const uint8_t* wuq,
                           const int8_t* wue, const uint8_t* wdq, const int8_t* wde,
                           uint16_t* out, int32_t* ids_o, float* w_o, int nthreads)
{
    if (k < 1 || k > E || k > 16) return -2;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)n * k + 4);
    float* w = (float*)malloc(sizeof(float) * (size_t)n * k + 4);
    int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)n * k + 4);
    float* y = (float*)malloc(sizeof(float) * ((size_t)n * k * H + 1));
    float* keys = (float*)malloc(sizeof(float) * (size_t)E * 2);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int i = 0; i < n; ++i) {
        route_one(x + (int64_t)tokens[i] * H, wr, bias, H, E, k, score, renorm,
                  ids + (int64_t)i * k, w + (int64_t)i * k, NULL, keys, keys + E, taken);
        for (int j = 0; j < k; ++j) tok[i * k + j] = tokens[i];
    }
    int rc = orc_expert_ffn_fp8(n * k, tok, ids, H, F, xq, xe, wgq, wge, wuq, wue, wdq, wde, y,
                                NULL, nthreads);
    if (rc == 0) orc_combine(n, H, k, y, w, out);
    if (ids_o) memcpy(ids_o, ids, sizeof(int32_t) * (size_t)n * k);
    if (w_o) memcpy(w_o, w, sizeof(float) * (size_t)n * k);
    free(ids); free(w); free(tok); free(y); free(keys); free(taken);
    return rc;
}

void orc_f32_to_e4m3_array(const float* in, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_e4m3(in[i]);
}
