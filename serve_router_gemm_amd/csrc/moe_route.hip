// moe_route.hip -- router logits, selection keys, top-k and weights.
//
// The router's near-ties are what flips experts between runs (Fireworks page
// "位级一致：前沿训练的差异化关键", section "为什么比特级一致是一个复杂的问题");
// a deterministic tie-break is the fix named there.  A top-k must also fix
// boundary ties, stability, NaN handling and the index dtype ("GLM
// Post-Training Beyond SFT", section "迁移到 NPU 时").
//
// Logits are taken in one fixed order, independent of the batch: hidden
// indices in chunks of 256, each chunk an ascending fp32 fma chain from +0,
// chunk sums added in ascending order.  The logits kernels either fold all
// chunks of their tile themselves or write each chunk's sum to its own plane
// for the select kernel to fold (where the chunks give the parallelism).
// Both produce the same bits.
//
// A matrix instruction that sums several products (K > 1) adds them in an
// order of the hardware's that no plain CPU program reproduces, so the chains
// run either on the VALU or on the matrix cores through the K = 1 fp32 MFMA,
// which adds exactly one product per accumulator and instruction, rounded as
// the VALU's fma rounds: the same chain either way.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kStageK = 32;   // hidden indices staged in LDS per step

typedef float floatx32 __attribute__((ext_vector_type(32)));

// part[c][t][e] = fp32 logit (SPLIT=false: all chunks folded, c = 0) or the
// chunk-c partial sum (SPLIT=true: blockIdx.z = c).  With PF the next step's
// x and w pieces are loaded into registers while the current step's chains
// run from LDS: the vocabulary projection streams its rows from HBM and gains
// (T = 64: 0.89 -> 0.85 ms, T = 1: 0.47 -> 0.38 ms); the router, whose
// operands sit in L2, loses 4% with it and runs without.  The chains, and so
// the bits, are the same either way.
// Thread (ty, tx): tokens t0 + ty*TT + i, experts e0 + tx*TE + j (contiguous,
// so a thread reads its TE expert values of a step as 16-byte LDS reads).
template <int TT, int TE, bool SPLIT, bool PF>
__global__ __launch_bounds__(kRouteThreads) void router_logits_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    float* __restrict__ part) {
    constexpr int BT = 8 * TT;
    constexpr int BE = 32 * TE;
    __shared__ __attribute__((aligned(16))) float xs[kStageK][BT];
    __shared__ __attribute__((aligned(16))) float ws[kStageK][BE];

    const int tid = threadIdx.x;
    const int tx = tid & 31, ty = tid >> 5;
    const int t0 = blockIdx.x * BT;
    const int e0 = blockIdx.y * BE;

    int k_begin = 0, k_end = H;
    if (SPLIT) {
        k_begin = blockIdx.z * kLogitChunk;
        k_end = min(H, k_begin + kLogitChunk);
    }

    float total[TT][TE];
    float acc[TT][TE];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) { total[i][j] = 0.0f; acc[i][j] = 0.0f; }

    if constexpr (PF) {
        // piece c of a step: row c / 4, hidden indices k0 + 8 * (c % 4) .. + 7.
        // The next step's pieces are loaded into registers while the current
        // step's chains run from LDS; the chains are unchanged by this.
        constexpr int NX = (BT * 4 + kRouteThreads - 1) / kRouteThreads;
        constexpr int NW = (BE * 4 + kRouteThreads - 1) / kRouteThreads;
        uint4 xr[NX], wg[NW];
        auto fetch = [&](int k0) {
#pragma unroll
            for (int i = 0; i < NX; ++i) {
                const int c = tid + i * kRouteThreads;
                const int t = t0 + (c >> 2);
                xr[i] = make_uint4(0, 0, 0, 0);
                if (c < BT * 4 && t < T)
                    xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + k0 + (c & 3) * 8);
            }
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const int c = tid + i * kRouteThreads;
                const int e = e0 + (c >> 2);
                wg[i] = make_uint4(0, 0, 0, 0);
                if (c < BE * 4 && e < E)
                    wg[i] = *reinterpret_cast<const uint4*>(wr + (size_t)e * H + k0 + (c & 3) * 8);
            }
        };
        if (k_begin < k_end) fetch(k_begin);
        for (int k0 = k_begin; k0 < k_end; k0 += kStageK) {
            __syncthreads();
            // stage x[t0:t0+BT, k0:k0+32] and wr[e0:e0+BE, k0:k0+32] as fp32, k-major
#pragma unroll
            for (int i = 0; i < NX; ++i) {
                const int c = tid + i * kRouteThreads;
                if (c >= BT * 4) continue;
                const int row = c >> 2, q = c & 3;
                const uint32_t w4[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    xs[q * 8 + 2 * u][row] = bf16_to_f32(w4[u] & 0xFFFFu);
                    xs[q * 8 + 2 * u + 1][row] = bf16_to_f32(w4[u] >> 16);
                }
            }
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const int c = tid + i * kRouteThreads;
                if (c >= BE * 4) continue;
                const int row = c >> 2, q = c & 3;
                const uint32_t w4[4] = {wg[i].x, wg[i].y, wg[i].z, wg[i].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ws[q * 8 + 2 * u][row] = bf16_to_f32(w4[u] & 0xFFFFu);
                    ws[q * 8 + 2 * u + 1][row] = bf16_to_f32(w4[u] >> 16);
                }
            }
            __syncthreads();
            if (k0 + kStageK < k_end) fetch(k0 + kStageK);
#pragma unroll 4
            for (int kk = 0; kk < kStageK; ++kk) {
                float xv[TT], wv[TE];
#pragma unroll
                for (int i = 0; i < TT; ++i) xv[i] = xs[kk][ty * TT + i];
#pragma unroll
                for (int j = 0; j < TE; ++j) wv[j] = ws[kk][tx * TE + j];
#pragma unroll
                for (int i = 0; i < TT; ++i)
#pragma unroll
                    for (int j = 0; j < TE; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
            }
            // end of a 256-wide chunk (or of H): fold the chunk sum in order
            const int kn = k0 + kStageK;
            if (!SPLIT && ((kn % kLogitChunk) == 0 || kn == k_end)) {
#pragma unroll
                for (int i = 0; i < TT; ++i)
#pragma unroll
                    for (int j = 0; j < TE; ++j) {
                        total[i][j] = total[i][j] + acc[i][j];
                        acc[i][j] = 0.0f;
                    }
            }
        }
    } else {
        for (int k0 = k_begin; k0 < k_end; k0 += kStageK) {
            __syncthreads();
            // stage x[t0:t0+BT, k0:k0+32] and wr[e0:e0+BE, k0:k0+32] as fp32, k-major
            for (int c = tid; c < BT * 4; c += kRouteThreads) {
                const int row = c >> 2, q = c & 3;
                const int t = t0 + row;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (t < T) v = *reinterpret_cast<const uint4*>(x + (size_t)t * H + k0 + q * 8);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    xs[q * 8 + 2 * u][row] = bf16_to_f32(w4[u] & 0xFFFFu);
                    xs[q * 8 + 2 * u + 1][row] = bf16_to_f32(w4[u] >> 16);
                }
            }
            for (int c = tid; c < BE * 4; c += kRouteThreads) {
                const int row = c >> 2, q = c & 3;
                const int e = e0 + row;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (e < E) v = *reinterpret_cast<const uint4*>(wr + (size_t)e * H + k0 + q * 8);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ws[q * 8 + 2 * u][row] = bf16_to_f32(w4[u] & 0xFFFFu);
                    ws[q * 8 + 2 * u + 1][row] = bf16_to_f32(w4[u] >> 16);
                }
            }
            __syncthreads();
#pragma unroll 4
            for (int kk = 0; kk < kStageK; ++kk) {
                float xv[TT], wv[TE];
#pragma unroll
                for (int i = 0; i < TT; ++i) xv[i] = xs[kk][ty * TT + i];
#pragma unroll
                for (int j = 0; j < TE; ++j) wv[j] = ws[kk][tx * TE + j];
#pragma unroll
                for (int i = 0; i < TT; ++i)
#pragma unroll
                    for (int j = 0; j < TE; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
            }
            // end of a 256-wide chunk (or of H): fold the chunk sum in order
            const int kn = k0 + kStageK;
            if (!SPLIT && ((kn % kLogitChunk) == 0 || kn == k_end)) {
#pragma unroll
                for (int i = 0; i < TT; ++i)
#pragma unroll
                    for (int j = 0; j < TE; ++j) {
                        total[i][j] = total[i][j] + acc[i][j];
                        acc[i][j] = 0.0f;
                    }
            }
        }
    }

    float* plane = part + (SPLIT ? (size_t)blockIdx.z * T * E : 0);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int t = t0 + ty * TT + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < TE; ++j) {
            const int e = e0 + tx * TE + j;
            if (e < E) plane[(size_t)t * E + e] = SPLIT ? acc[i][j] : total[i][j];
        }
    }
}

// Router logits on the matrix cores, in the same order.  v_mfma_f32_32x32x1_2b_f32
// adds one product to each of its accumulators per instruction, and on gfx950
// that add rounds exactly as the VALU's fused multiply-add does (checked on
// normals, wide exponents, denormal products and sums, signed zeros,
// infinities and NaN: chains of either are bit-identical).  A chain of these
// instructions over k ascending is thus the chain of the kernel above, bit
// for bit, at the matrix cores' fp32 rate (twice the non-packed VALU rate).
// Block: 4 or 8 waves, WT x WE of them along tokens x experts (the first 4
// issue the loads); a wave computes 32
// tokens x 64 experts, one instruction per k (two 32 x 32 blocks, its two
// expert halves): lane L supplies token L % 32 and expert L of the wave's 64.
// The stages of x and w come as loaded (bf16 rows of 32 k) by direct-to-LDS
// loads into a ring of four (55 KB at 2 x 2 waves, 90 KB at 2 x 4), three
// steps of loads in flight, and each group of 8 k's operands is read from LDS
// one group ahead of its MFMAs, as one 16-byte read per operand widened to
// fp32 in registers.
// (Measured on the large layer's route, same bits throughout: 0.540 ms with
// k-major fp32 stages written from registers (8 conversions and 8 4-byte
// writes per piece, 4-byte operand reads), 0.518 with bf16 rows written
// from registers and 8-byte reads of 4 k, 0.511 / 0.497 with this ring and
// 8- / 16-byte reads, 0.504 with a ring of three.  A wave tile of 64 x 64 as
// two chains, one block per CU, measured 10% slower.)
template <int WT, int WE, bool SPLIT>
__global__ __launch_bounds__(WT * WE * kWave) void router_logits_mfma_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    float* __restrict__ part) {
    static_assert(WT * WE == 4 || WT * WE == 8, "4 or 8 waves; the first 4 issue the loads");
    constexpr int BT = 32 * WT;
    constexpr int BE = 64 * WE;
    // Stages arrive by direct-to-LDS loads, NB of them in a ring (the loads
    // of NB - 1 steps in flight).  A stage is NG groups of 16 rows x 64 bytes
    // (token rows, then expert rows), each group 1 KB written by one wave
    // instruction and padded to 1152 bytes; in a group, lane l fills row l/4
    // at chunk position l%4 with the row's chunk (l%4) ^ ((l/16) & 3), so the
    // 16 rows of a group read at one k offset (16 bytes a lane) cover the 64
    // banks once: a wave's 32 token rows take the two passes 512 bytes need.
    constexpr int GX = BT / 16, GW = BE / 16, NG = GX + GW;
    static_assert(NG % 4 == 0, "each issuing wave loads NG / 4 groups");
    constexpr int kPerWave = NG / 4;
    constexpr int kGroupBytes = 1024 + 128;
    constexpr int kStageBytes = NG * kGroupBytes;
    constexpr int NB = 4;
    __shared__ __attribute__((aligned(1024))) unsigned char sm[NB * kStageBytes];
    const uint32_t lds0 =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)sm);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / WE, we = wave % WE;
    const int t0 = blockIdx.x * BT;
    const int e0 = blockIdx.y * BE;

    int k_begin = 0, k_end = H;
    if (SPLIT) {
        k_begin = blockIdx.z * kLogitChunk;
        k_end = min(H, k_begin + kLogitChunk);
    }

    // source rows of this wave's groups (rows past T or E load the last row;
    // their results are dropped at the store)
    const int rl = lane >> 2;
    const int lchunk = (lane & 3) ^ ((rl >> 2) & 3);
    const uint16_t* src[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int gi = min(wave, 3) * kPerWave + i;
        if (gi < GX) {
            const int t = min(t0 + gi * 16 + rl, T - 1);
            src[i] = x + (size_t)t * H + lchunk * 8;
        } else {
            const int e = min(e0 + (gi - GX) * 16 + rl, E - 1);
            src[i] = wr + (size_t)e * H + lchunk * 8;
        }
    }
    auto issue = [&](int st) {
        if (wave >= 4) return;
        const uint32_t sb = lds0 + (uint32_t)((st % NB) * kStageBytes);
        const int k0 = k_begin + st * kStageK;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int gi = wave * kPerWave + i;
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                         :: "v"(src[i] + k0), "s"(sb + (uint32_t)(gi * kGroupBytes)) : "memory");
        }
    };
    // this lane's token row and expert row: group, row in group, swizzle
    const int tr = wt * 32 + (lane & 31), er = we * 64 + lane;
    const int xoff = (tr >> 4) * kGroupBytes + (tr & 15) * 64, xsw = ((tr & 15) >> 2) & 3;
    const int woff = (GX + (er >> 4)) * kGroupBytes + (er & 15) * 64, wsw = ((er & 15) >> 2) & 3;

    floatx32 acc, total;
#pragma unroll
    for (int r = 0; r < 32; ++r) { acc[r] = 0.0f; total[r] = 0.0f; }

    const int nsteps = (k_end - k_begin) / kStageK;
    for (int j = 0; j < NB - 1; ++j)
        if (j < nsteps) issue(j);
    for (int st = 0; st < nsteps; ++st) {
        const int k0 = k_begin + st * kStageK;
        // this wave's loads of stage st landed (those of the later stages
        // already issued may stay in flight; loads complete in order), then
        // every wave's
        static_assert(NB == 4, "the waits below count two later stages at most");
        const int later = min(NB - 2, nsteps - 1 - st);
        if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kPerWave) : "memory");
        else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kPerWave) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // the buffer of step st-1 is free: every wave read it before this barrier
        if (st + NB - 1 < nsteps) issue(st + NB - 1);
        const unsigned char* sb = sm + (st % NB) * kStageBytes;
        constexpr int G = 8;
        float oa[2][G], ob[2][G];
        auto rd = [&](int slot, int gk) {
            const uint4 a = *reinterpret_cast<const uint4*>(sb + xoff + ((gk ^ xsw) << 4));
            const uint4 w = *reinterpret_cast<const uint4*>(sb + woff + ((gk ^ wsw) << 4));
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                oa[slot][2 * j] = __uint_as_float(av[j] << 16);
                oa[slot][2 * j + 1] = __uint_as_float(av[j] & 0xFFFF0000u);
                ob[slot][2 * j] = __uint_as_float(wv[j] << 16);
                ob[slot][2 * j + 1] = __uint_as_float(wv[j] & 0xFFFF0000u);
            }
        };
        rd(0, 0);
#pragma unroll
        for (int gk = 0; gk < kStageK / G; ++gk) {
            if (gk + 1 < kStageK / G) rd((gk + 1) & 1, gk + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < G; ++u)
                acc = __builtin_amdgcn_mfma_f32_32x32x1f32(oa[gk & 1][u], ob[gk & 1][u], acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // end of a 256-wide chunk (or of H): fold the chunk sum in order
        const int kn = k0 + kStageK;
        if (!SPLIT && ((kn % kLogitChunk) == 0 || kn == k_end)) {
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                total[r] = total[r] + acc[r];
                acc[r] = 0.0f;
            }
        }
    }

    // accumulator r: 32 x 32 block r / 16 (the expert half), token
    // 8 * ((r % 16) / 4) + 4 * (L / 32) + r % 4 of the wave's 32, expert L % 32
    float* plane = part + (SPLIT ? (size_t)blockIdx.z * T * E : 0);
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        const int rr = r & 15;
        const int t = t0 + wt * 32 + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
        const int e = e0 + we * 64 + 32 * (r >> 4) + (lane & 31);
        if (t < T && e < E) plane[(size_t)t * E + e] = SPLIT ? acc[r] : total[r];
    }
}

// Router logits of a few tokens (T <= TT <= 8), one partial plane per
// 256-wide chunk: one wave per (chunk, 64 experts), one thread per expert.
// A thread loads its expert's 512-byte piece of the chunk at once (32 loads
// in flight) and runs the chunk's ascending fp32 fma chain from +0 for every
// token from registers; the tokens' pieces sit in LDS as fp32.  The select
// kernel folds the planes in ascending order: the same chains and the same
// bits as the tiled kernel above, with one memory latency per block instead
// of one per 32 hidden indices.
template <int TT>
__global__ __launch_bounds__(kWave) void router_logits_few_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) float xs[TT][kLogitChunk];
    const int lane = threadIdx.x;
    const int c = blockIdx.y;
    const int k0 = c * kLogitChunk;
    const int n = min(kLogitChunk, H - k0);           // a multiple of 64
    const int e = blockIdx.x * kWave + lane;
    const uint16_t* row = wr + (size_t)min(e, E - 1) * H + k0;
    uint4 w[kLogitChunk / 8];
#pragma unroll
    for (int u = 0; u < kLogitChunk / 8; ++u)
        if (8 * u < n) w[u] = *reinterpret_cast<const uint4*>(row + 8 * u);
    // the tokens' pieces: 16-byte loads, all issued before any is used
    constexpr int kPieces = kLogitChunk / 8;                  // per token
    constexpr int NX = (TT * kPieces + kWave - 1) / kWave;
    uint4 xr[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int c = lane + i * kWave;
        const int t = c / kPieces, kk = 8 * (c % kPieces);
        xr[i] = make_uint4(0, 0, 0, 0);
        if (t < TT && t < T && kk < n)
            xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + k0 + kk);
    }
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int c = lane + i * kWave;
        const int t = c / kPieces, kk = 8 * (c % kPieces);
        if (t >= TT) continue;
        const uint32_t q[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            xs[t][kk + j] = bf16_to_f32((j & 1) ? (q[j >> 1] >> 16) : (q[j >> 1] & 0xFFFFu));
    }
    __syncthreads();
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int u = 0; u < kLogitChunk / 8; ++u) {
        if (8 * u >= n) break;
        const uint32_t q[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
        float wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wv[j] = bf16_to_f32((j & 1) ? (q[j >> 1] >> 16) : (q[j >> 1] & 0xFFFFu));
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            // the token's 8 hidden values: two 16-byte LDS reads (a broadcast)
            const float4 xa = *reinterpret_cast<const float4*>(&xs[t][8 * u]);
            const float4 xb = *reinterpret_cast<const float4*>(&xs[t][8 * u + 4]);
            const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[t] = __builtin_fmaf(xv[j], wv[j], acc[t]);
        }
    }
    if (e < E) {
        float* plane = part + (size_t)c * T * E;
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (t < T) plane[(size_t)t * E + e] = acc[t];
    }
}

template <int TT>
hipError_t launch_logits_few(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                             float* part, hipStream_t s) {
    const int nchunks = (H + kLogitChunk - 1) / kLogitChunk;
    dim3 grid((E + kWave - 1) / kWave, nchunks);
    router_logits_few_kernel<TT><<<grid, kWave, 0, s>>>(T, H, E, x, wr, part);
    return hipGetLastError();
}

// Vocabulary projection for 5 to 8 tokens: one thread per
// vocabulary row streams the row in 16-byte loads (two groups of 8 in flight
// per lane) and runs the same chains as the folded router kernel: within
// each 256-wide chunk an ascending fp32 fma chain from +0 for every token,
// chunk sums added in ascending order.  The tokens' hidden states sit in LDS
// as fp32, 2048 indices at a time.  Rows past V read row V-1 and drop it.
constexpr int kStreamThreads = 256;
constexpr int kStreamCh = 2048;   // hidden indices of the tokens staged in LDS

template <int TT>
__global__ __launch_bounds__(kStreamThreads) void lm_logits_stream_kernel(
    int T, int H, int V, const uint16_t* __restrict__ h, const uint16_t* __restrict__ proj,
    float* __restrict__ z) {
    static_assert(kStreamCh % kLogitChunk == 0, "staged span is whole chunks");
    __shared__ __attribute__((aligned(16))) float xs[TT][kStreamCh];
    const int v = blockIdx.x * kStreamThreads + threadIdx.x;
    const uint16_t* row = proj + (size_t)min(v, V - 1) * H;

    float total[TT], acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) { total[t] = 0.0f; acc[t] = 0.0f; }

    for (int c0 = 0; c0 < H; c0 += kStreamCh) {
        const int n = min(kStreamCh, H - c0);   // a multiple of 64
        __syncthreads();   // every thread done with the previous span
        // the tokens' span in 16-byte loads, issued before any is used
        constexpr int kPieces = kStreamCh / 8;                     // per token
        constexpr int NX = (TT * kPieces + kStreamThreads - 1) / kStreamThreads;
        uint4 hr[NX];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int c = threadIdx.x + i * kStreamThreads;
            const int t = c / kPieces, kk = 8 * (c % kPieces);
            hr[i] = make_uint4(0, 0, 0, 0);
            if (t < TT && t < T && kk < n)
                hr[i] = *reinterpret_cast<const uint4*>(h + (size_t)t * H + c0 + kk);
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int c = threadIdx.x + i * kStreamThreads;
            const int t = c / kPieces, kk = 8 * (c % kPieces);
            if (t >= TT) continue;
            const uint32_t q[4] = {hr[i].x, hr[i].y, hr[i].z, hr[i].w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                xs[t][kk + j] = bf16_to_f32((j & 1) ? (q[j >> 1] >> 16) : (q[j >> 1] & 0xFFFFu));
        }
        __syncthreads();
#pragma unroll 2
        for (int i0 = 0; i0 < n; i0 += 64) {
            uint4 w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                w[u] = *reinterpret_cast<const uint4*>(row + c0 + i0 + 8 * u);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t q[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float wv = bf16_to_f32((e & 1) ? (q[e >> 1] >> 16) : (q[e >> 1] & 0xFFFFu));
#pragma unroll
                    for (int t = 0; t < TT; ++t)
                        acc[t] = __builtin_fmaf(xs[t][i0 + 8 * u + e], wv, acc[t]);
                }
            }
            // end of a 256-wide chunk (or of H): fold the chunk sum in order
            const int kn = c0 + i0 + 64;
            if ((kn % kLogitChunk) == 0 || kn == H) {
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    total[t] = total[t] + acc[t];
                    acc[t] = 0.0f;
                }
            }
        }
    }
    if (v < V) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (t < T) z[(size_t)t * V + v] = total[t];
    }
}

// Vocabulary projection for one or two tokens, the same chains as the kernel
// above.  A wave takes 64 vocabulary rows (lane = row) and runs them through
// the whole hidden state.  Each step of 64 hidden indices is 8 KB of rows
// loaded as whole 128-byte lines (lane l of load i: row 8i + l/8, chunk l%8), kLmRing
// steps in flight, and passed through 8 KB of the wave's own LDS (chunks
// XOR-swizzled by row; one wave's LDS operations run in order) so that each
// lane reads its own row's 128 bytes.  The tokens' hidden values are the same
// for every lane (scalar loads; with more than two tokens they no longer fit
// the scalar registers, and the kernel above is faster).  Against the kernel
// above at one token (H = 6144, V = 65536): 0.172 -> 0.152 ms, two tokens
// 0.228 -> 0.200, bit-identical.  Rows past V read row V-1 and drop it.
constexpr int kLmRows = 64;
constexpr int kLmRing = 4;
typedef unsigned int lm_u32x4 __attribute__((ext_vector_type(4)));

template <int TT>
__global__ __launch_bounds__(256) void lm_logits_lines_kernel(
    int T, int H, int V, const uint16_t* __restrict__ h, const uint16_t* __restrict__ proj,
    float* __restrict__ z) {
    __shared__ lm_u32x4 tr[4][kLmRows * 8];             // a wave's step: 64 rows x 128 B
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * 4 + wave) * kLmRows;
    if (r0 >= V) return;                             // whole wave leaves
    lm_u32x4* const my = tr[wave];
    const uint16_t* src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        src[i] = proj + (size_t)min(r0 + 8 * i + (lane >> 3), V - 1) * H + (lane & 7) * 8;
    const int nst = H / 64;                          // H is a multiple of 64

    float total[TT], acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) { total[t] = 0.0f; acc[t] = 0.0f; }
    lm_u32x4 ring[kLmRing][8];
#pragma unroll
    for (int u = 0; u < kLmRing; ++u) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ring[u][i] = *reinterpret_cast<const lm_u32x4*>(src[i] + 64 * min(u, nst - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = 0; s0 < nst; s0 += kLmRing) {
#pragma unroll
        for (int u = 0; u < kLmRing; ++u) {
            const int s = s0 + u;
            if (s < nst) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int row = 8 * i + (lane >> 3);
                    my[row * 8 + ((lane & 7) ^ (row & 7))] = ring[u][i];
                }
                lm_u32x4 w[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) w[j] = my[lane * 8 + (j ^ (lane & 7))];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    lm_u32x4 xq[TT];
#pragma unroll
                    for (int t = 0; t < TT; ++t)
                        xq[t] = *reinterpret_cast<const lm_u32x4*>(h + (size_t)(t < T ? t : 0) * H +
                                                                64 * s + 8 * j);
                    const uint32_t q[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float wv = bf16_to_f32((e & 1) ? (q[e >> 1] >> 16)
                                                             : (q[e >> 1] & 0xFFFFu));
#pragma unroll
                        for (int t = 0; t < TT; ++t) {
                            const uint32_t xw = (e >> 1) == 0 ? xq[t].x : (e >> 1) == 1 ? xq[t].y
                                              : (e >> 1) == 2 ? xq[t].z : xq[t].w;
                            const float xv = bf16_to_f32((e & 1) ? (xw >> 16) : (xw & 0xFFFFu));
                            acc[t] = __builtin_fmaf(xv, wv, acc[t]);
                        }
                    }
                }
                // end of a 256-wide chunk (or of H): fold the chunk sum in order
                const int kn = 64 * (s + 1);
                if ((kn % kLogitChunk) == 0 || kn == H) {
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        total[t] = total[t] + acc[t];
                        acc[t] = 0.0f;
                    }
                }
            }
            const int sn = min(s + kLmRing, nst - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ring[u][i] = *reinterpret_cast<const lm_u32x4*>(src[i] + 64 * sn);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (r0 + lane < V) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (t < T) z[(size_t)t * V + r0 + lane] = total[t];
    }
}

// Vocabulary projection for 3-4 and 9-16 tokens: the kernel above with the
// tokens' hidden values staged in LDS as fp32, kLmSpan indices at a time (the
// block's four waves step through a span together; the stage is published by
// a barrier that leaves the row loads of later steps in flight).  Against one
// thread per row (4 tokens) and the matrix-core kernel (16 tokens), H = 6144,
// V = 65536: 0.201 -> 0.169 ms and 0.519 -> 0.383 ms, bit-identical; at 8
// tokens it ties with one thread per row, at 32 the matrix cores are faster
// (0.52 vs 0.68 ms), and with few vocabulary rows (V = 1000: 4 blocks) it
// loses to both.
constexpr int kLmSpan = 512;

template <int TT, int RING>
__global__ __launch_bounds__(256) void lm_logits_lines_lds_kernel(
    int T, int H, int V, const uint16_t* __restrict__ h, const uint16_t* __restrict__ proj,
    float* __restrict__ z) {
    __shared__ lm_u32x4 tr[4][kLmRows * 8];
    __shared__ __attribute__((aligned(16))) float xs[TT][kLmSpan];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * 4 + wave) * kLmRows;   // may pass V: rows clamp, none stored
    lm_u32x4* const my = tr[wave];
    const uint16_t* src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        src[i] = proj + (size_t)min(r0 + 8 * i + (lane >> 3), V - 1) * H + (lane & 7) * 8;
    const int nst = H / 64;
    constexpr int kSpanSteps = kLmSpan / 64;
    static_assert(kSpanSteps % RING == 0, "ring rounds inside a span");

    float total[TT], acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) { total[t] = 0.0f; acc[t] = 0.0f; }
    lm_u32x4 ring[RING][8];
#pragma unroll
    for (int u = 0; u < RING; ++u) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ring[u][i] = *reinterpret_cast<const lm_u32x4*>(src[i] + 64 * min(u, nst - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int sp = 0; sp < nst; sp += kSpanSteps) {
        // every wave done with the previous span's values
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        {
            const int k0 = 64 * sp;
            const int n = min(kLmSpan, H - k0);
            for (int c = threadIdx.x; c < TT * (kLmSpan / 8); c += 256) {
                const int t = c / (kLmSpan / 8), kk = 8 * (c % (kLmSpan / 8));
                if (kk >= n) continue;
                const lm_u32x4 q =
                    *reinterpret_cast<const lm_u32x4*>(h + (size_t)(t < T ? t : 0) * H + k0 + kk);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    xs[t][kk + j] = bf16_to_f32((j & 1) ? (q[j >> 1] >> 16) : (q[j >> 1] & 0xFFFFu));
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int s0 = sp; s0 < sp + kSpanSteps; s0 += RING) {
#pragma unroll
            for (int u = 0; u < RING; ++u) {
                const int s = s0 + u;
                if (s < nst) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int row = 8 * i + (lane >> 3);
                        my[row * 8 + ((lane & 7) ^ (row & 7))] = ring[u][i];
                    }
                    lm_u32x4 w[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) w[j] = my[lane * 8 + (j ^ (lane & 7))];
                    const int kx = 64 * (s - sp);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t qw = w[j][e >> 1];
                            const float wv = bf16_to_f32((e & 1) ? (qw >> 16) : (qw & 0xFFFFu));
#pragma unroll
                            for (int t = 0; t < TT; ++t)
                                acc[t] = __builtin_fmaf(xs[t][kx + 8 * j + e], wv, acc[t]);
                        }
                    }
                    const int kn = 64 * (s + 1);
                    if ((kn % kLogitChunk) == 0 || kn == H) {
#pragma unroll
                        for (int t = 0; t < TT; ++t) {
                            total[t] = total[t] + acc[t];
                            acc[t] = 0.0f;
                        }
                    }
                }
                const int sn = min(s + RING, nst - 1);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    ring[u][i] = *reinterpret_cast<const lm_u32x4*>(src[i] + 64 * sn);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (r0 + lane < V) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (t < T) z[(size_t)t * V + r0 + lane] = total[t];
    }
}

template <int TT>
hipError_t launch_lm_stream(int T, int H, int V, const uint16_t* h, const uint16_t* proj,
                            float* z, hipStream_t s) {
    if constexpr (TT <= 2) {
        const int blocks = (V + 4 * kLmRows - 1) / (4 * kLmRows);
        lm_logits_lines_kernel<TT><<<blocks, 256, 0, s>>>(T, H, V, h, proj, z);
    } else if constexpr (TT == 4 || TT == 16) {
        const int blocks = (V + 4 * kLmRows - 1) / (4 * kLmRows);
        lm_logits_lines_lds_kernel<TT, (TT <= 8 ? 4 : 2)><<<blocks, 256, 0, s>>>(T, H, V, h,
                                                                                 proj, z);
    } else {
        const int blocks = (V + kStreamThreads - 1) / kStreamThreads;
        lm_logits_stream_kernel<TT><<<blocks, kStreamThreads, 0, s>>>(T, H, V, h, proj, z);
    }
    return hipGetLastError();
}

// Wave-uniform maximum of a 64-bit value: DPP exchanges inside each 16-lane
// row (quad neighbours, then the mirrored half row, then the mirrored row), so
// that every lane holds its row's maximum, then the four rows' maxima read
// into scalars.  No LDS crossbar traffic (the 64-bit xor-shuffle butterfly it
// replaces took 12 crossbar shuffles per maximum); the maximum of distinct
// keys is the same in any order.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, 0xF, 0xF, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, 0xF, 0xF, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_u64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_max_u64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_max_u64<0x141>(v);   // row_half_mirror
    v = dpp_max_u64<0x140>(v);   // row_mirror
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < kWave / 16; ++r) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
        const uint64_t x = ((uint64_t)hi << 32) | lo;
        m = x > m ? x : m;
    }
    return m;
}

// The permutation outputs of a batch of at most 4 tokens, filled by the
// select kernel itself (kPermute): one launch fewer for a decode-sized step.
struct SmallPermute {
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv_perm;
};

// The expert histogram, offsets and stable permutation of A <= 64
// assignments (a = t*k + j), as the permute kernels compute them: counts[e];
// offsets = their exclusive prefix in expert order, offsets[E] = A;
// perm lists the assignments grouped by expert, ascending a inside each;
// inv_perm[perm[p]] = p.  Each wave (one per token) leaves its k ids in LDS;
// after the block barrier wave 0 holds assignment a in lane a.
template <int kSelMaxQ>
__device__ __forceinline__ void permute_tiny(int A, int E, int t, int k, int my_sel,
                                             const SmallPermute& sp) {
    __shared__ int s_ids[64];
    __shared__ int s_cnt[64 * kSelMaxQ];
    __shared__ int s_off[64 * kSelMaxQ];
    const int lane = threadIdx.x & 63;
    if (lane < k) s_ids[t * k + lane] = my_sel;
    __syncthreads();
    if (t != 0) return;
    const int ea = lane < A ? s_ids[lane] : -1;
    const bool valid = ea >= 0 && ea < E;
    // lanes holding the same expert: one ballot per bit of the id (E <= 512)
    uint64_t same = __ballot(valid);
    if (!valid) same = 0;
#pragma unroll
    for (int bt = 0; bt < 9; ++bt) {
        const bool bit = valid && ((ea >> bt) & 1);
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & lower);   // lower lanes with this expert
    const int cnt = __popcll(same);
    // counts: zero, then the last lane of each expert's group writes the count
#pragma unroll
    for (int q = 0; q < kSelMaxQ; ++q) s_cnt[lane + 64 * q] = 0;
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == cnt - 1) s_cnt[ea] = cnt;
    __builtin_amdgcn_wave_barrier();
    // exclusive prefix in expert order (q major, lane minor)
    int carry = 0;
#pragma unroll
    for (int q = 0; q < kSelMaxQ; ++q) {
        const int e = lane + 64 * q;
        const int c = s_cnt[e];
        int incl = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const int excl = carry + incl - c;
        if (e < E) {
            sp.counts[e] = c;
            sp.offsets[e] = excl;
        }
        s_off[e] = excl;
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) sp.offsets[E] = carry;
    __builtin_amdgcn_wave_barrier();
    const int pos = valid ? s_off[ea] + rank : -1;
    if (valid) sp.perm[pos] = lane;
    if (lane < A) sp.inv_perm[lane] = pos;
}

// One wave per token: fold partial logits, keys, top-k, weights.  With
// `replay` set (router replay), the experts of each slot are read from it
// instead of selected, and only the weights are computed, by the same code:
// replaying the ids this kernel chose reproduces its weights bit for bit.  A
// replayed id outside [0,E) gets weight 0 and is left out of the sum.
// kSelMaxQ = experts per lane (E <= 64 * kSelMaxQ); kSelBatch partial planes
// are loaded together in the fold (one memory latency per batch: a decode
// step's 24 planes of a 6144-wide hidden state come in one batch).  The
// bias is loaded before the fold, and each selected logit is read from its
// owner lane into a scalar register (no LDS crossbar round trip per slot).
template <int kSelMaxQ, int kSelBatch, bool kPermute>
__global__ __launch_bounds__(256) void router_select_kernel(
    int T, int E, int k, int nparts, int score, int renorm, const float* __restrict__ part,
    const float* __restrict__ bias, const int32_t* __restrict__ replay,
    int32_t* __restrict__ ids, float* __restrict__ wout, SmallPermute sp) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    // (with kPermute the block is one wave per token: none leaves here)
    if (t >= T) return;  // whole wave leaves together
    // the experts of this lane: with 4 a lane, 4 consecutive ones (one
    // 16-byte load per plane: decode route 0.0149 -> 0.0139 ms on the large
    // layer, same bits); else lane, lane + 64, ...  (Which lane holds an
    // expert changes only the softmax denominator's summation order, the
    // same at every batch size.)
    constexpr bool kVec = kSelMaxQ == 4;
    auto eof = [&](int q) { return kVec ? lane * kSelMaxQ + q : lane + 64 * q; };

    float bz[kSelMaxQ];
#pragma unroll
    for (int q = 0; q < kSelMaxQ; ++q) {
        const int e = eof(q);
        bz[q] = (score != 0 && bias && e < E) ? bias[e] : 0.0f;
    }
    float lg[kSelMaxQ];
    uint64_t rk[kSelMaxQ];
    // fold the partial planes in ascending order
#pragma unroll
    for (int q = 0; q < kSelMaxQ; ++q) lg[q] = 0.0f;
    for (int c0 = 0; c0 < nparts; c0 += kSelBatch) {
        float pv[kSelBatch][kSelMaxQ];
        if (kVec && (E & 3) == 0) {
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u) {
                float4 f4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (4 * lane < E && c0 + u < nparts)
                    f4 = *reinterpret_cast<const float4*>(
                        part + ((size_t)(c0 + u) * T + t) * E + 4 * lane);
                pv[u][0] = f4.x;
                pv[u][1 % kSelMaxQ] = f4.y;
                pv[u][2 % kSelMaxQ] = f4.z;
                pv[u][3 % kSelMaxQ] = f4.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u)
#pragma unroll
                for (int q = 0; q < kSelMaxQ; ++q) {
                    const int e = eof(q);
                    pv[u][q] = (e < E && c0 + u < nparts)
                                   ? part[((size_t)(c0 + u) * T + t) * E + e] : 0.0f;
                }
        }
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u)
#pragma unroll
            for (int q = 0; q < kSelMaxQ; ++q)
                if (c0 + u < nparts) lg[q] = lg[q] + pv[u][q];
    }
#pragma unroll
    for (int q = 0; q < kSelMaxQ; ++q) {
        const int e = eof(q);
        rk[q] = 0;
        if (e < E) {
            const float v = lg[q];
            float key;
            if (score == 0) {
                key = v;
            } else {
                const float sg = 1.0f / (1.0f + expf(-v));
                key = sg + bz[q];
            }
            rk[q] = sel_rank(key, e);
        }
    }

    // the logit of expert e (uniform), read from its owner lane
    auto logit_of = [&](int e) -> float {
        const int qs = kVec ? e % kSelMaxQ : e >> 6, owner = kVec ? e / kSelMaxQ : e & 63;
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kSelMaxQ; ++q)
            if (q == qs) v = lg[q];
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), owner));
    };

    // slot j's expert and logit end up in lane j, which computes that slot's
    // weight (the same expression for every slot as a wave-wide loop would
    // evaluate; the renormalising sum still runs over j in order)
    int my_sel = -1;
    float my_l = 0.0f;
    for (int j = 0; j < k; ++j) {
        int e;
        float l;
        if (replay) {
            e = replay[(size_t)t * k + j];
            l = (e >= 0 && e < E) ? logit_of(e) : 0.0f;
        } else {
            uint64_t best = rk[0];
#pragma unroll
            for (int q = 1; q < kSelMaxQ; ++q) best = rk[q] > best ? rk[q] : best;
            best = wave_max_u64(best);
            e = (int)(~(uint32_t)best);
            const int qs = kVec ? e % kSelMaxQ : e >> 6, owner = kVec ? e / kSelMaxQ : e & 63;
#pragma unroll
            for (int q = 0; q < kSelMaxQ; ++q)
                if (q == qs && lane == owner) rk[q] = 0;  // taken
            l = logit_of(e);
        }
        if (lane == j) {
            my_sel = e;
            my_l = l;
        }
    }

    float p;
    if (score == 0) {
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < kSelMaxQ; ++q)
            if (eof(q) < E) m = fmaxf(m, lg[q]);
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
        float S = 0.0f;
#pragma unroll
        for (int q = 0; q < kSelMaxQ; ++q)
            if (eof(q) < E) S = S + expf(lg[q] - m);
        // (the butterfly gives every lane the same sum: each step adds the
        // same two values on both lanes of a pair)
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) S = S + __shfl_xor(S, s, 64);
        p = expf(my_l - m) / S;
    } else {
        p = 1.0f / (1.0f + expf(-my_l));
    }
    if (replay && (my_sel < 0 || my_sel >= E)) p = 0.0f;
    if (renorm) {
        float D = 0.0f;
        for (int j = 0; j < k; ++j)
            D = D + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j));
        p = D > 0.0f ? p / D : 0.0f;
    }
    if (lane < k) {
        if (!replay) ids[(size_t)t * k + lane] = my_sel;
        wout[(size_t)t * k + lane] = p;
    }
    if constexpr (kPermute) permute_tiny<kSelMaxQ>(T * k, E, t, k, my_sel, sp);
}

template <int TT, int TE, bool SPLIT, bool PF = false>
hipError_t launch_logits(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                         float* part, hipStream_t s) {
    constexpr int BT = 8 * TT, BE = 32 * TE;
    const int nchunks = (H + kLogitChunk - 1) / kLogitChunk;
    dim3 grid((T + BT - 1) / BT, (E + BE - 1) / BE, SPLIT ? nchunks : 1);
    router_logits_kernel<TT, TE, SPLIT, PF><<<grid, kRouteThreads, 0, s>>>(T, H, E, x, wr, part);
    return hipGetLastError();
}

template <int WT, int WE, bool SPLIT>
hipError_t launch_logits_mfma(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                              float* part, hipStream_t s) {
    constexpr int BT = 32 * WT, BE = 64 * WE;
    const int nchunks = (H + kLogitChunk - 1) / kLogitChunk;
    dim3 grid((T + BT - 1) / BT, (E + BE - 1) / BE, SPLIT ? nchunks : 1);
    router_logits_mfma_kernel<WT, WE, SPLIT><<<grid, WT * WE * kWave, 0, s>>>(T, H, E, x, wr,
                                                                             part);
    return hipGetLastError();
}

template <bool SPLIT>
hipError_t launch_logits_mfma_plan(const RoutePlan& p, int T, int H, int E, const uint16_t* x,
                                   const uint16_t* wr, float* part, hipStream_t s) {
    if (p.we == 4) return launch_logits_mfma<2, 4, SPLIT>(T, H, E, x, wr, part, s);
    if (p.we == 2) return launch_logits_mfma<2, 2, SPLIT>(T, H, E, x, wr, part, s);
    return launch_logits_mfma<4, 1, SPLIT>(T, H, E, x, wr, part, s);
}

}  // namespace

// 8 tokens x 8 contiguous experts per thread for E > 128: 64 fmas per four
// 16-byte LDS reads (large layer 0.90 -> 0.86 ms alone, same bits; 4 tokens
// x 8 experts, for twice the blocks, measured 1.00 ms)
constexpr int kBigTT = 8;

RoutePlan route_plan(int T, int H, int E) {
    RoutePlan p;
    p.mfma = 0;
    p.wt = 1;
    p.we = 4;
    const int nchunks = (H + kLogitChunk - 1) / kLogitChunk;
    // More than 128 experts and tokens enough for a block of 8 waves per CU:
    // 64 tokens x 256 experts per block, so each token row is staged once
    // (large layer: route 0.58 -> 0.55 ms in the step; with a block per chunk
    // the 4-wave blocks below stay faster)
    if (E > 128) {
        const long mb8 = (long)((T + 63) / 64) * ((E + 255) / 256);
        if (mb8 >= 256) {
            p.mfma = 1; p.wt = 2; p.we = 4; p.tt = 8; p.te = 8;
            p.split = 0; p.nparts = 1;
            return p;
        }
    }
    // else matrix cores where they fill the chip: 32 x 64 per wave, the block's 4
    // waves 2 x 2 (E > 64: 64 tokens x 128 experts) or 4 x 1 (128 x 64) along
    // tokens x experts; every chunk folded in the kernel when that alone gives
    // two blocks per CU (16384 tokens: one plane instead of one per chunk),
    // else one block per chunk for batches of 512 tokens or more with a block
    // per CU (mid T = 4096: 0.048 -> 0.037 ms against the VALU plan)
    {
        const int we = E > 64 ? 2 : 1, wt = 4 / we;
        const long mb = (long)((T + 32 * wt - 1) / (32 * wt)) * ((E + 64 * we - 1) / (64 * we));
        if (mb >= 512 || (T >= 512 && mb * nchunks >= 256)) {
            p.mfma = 1; p.wt = wt; p.we = we; p.tt = 8; p.te = 8;
            p.split = mb >= 512 ? 0 : 1;
            p.nparts = p.split ? nchunks : 1;
            return p;
        }
    }
    // folded tiles: 64 tokens x up to 256 experts per block
    const int te = E <= 32 ? 1 : (E <= 64 ? 2 : (E <= 128 ? 4 : 8));
    const long blocks = (long)((T + 63) / 64) * ((E + 32 * te - 1) / (32 * te));
    if (blocks >= 512 || nchunks == 1) {
        p.split = 0; p.nparts = 1; p.tt = 8; p.te = te;
    } else if (T >= 512) {
        // mid-sized batch: 32 tokens x up to 256 experts per block, one block
        // per chunk (mid layer, T = 600 / 1024 / 2048: route 0.034 / 0.033 /
        // 0.036 ms with 64-token blocks, 0.025 / 0.025 / 0.027 with these)
        p.split = 1; p.nparts = nchunks; p.tt = 4; p.te = te;
    } else {
        // small batch: one logit per thread, one block per chunk
        p.split = 1; p.nparts = nchunks; p.tt = 1; p.te = 1;
    }
    return p;
}

size_t route_ws_bytes(int T, int H, int E) {
    const RoutePlan p = route_plan(T, H, E);
    return (size_t)p.nparts * (size_t)T * (size_t)E * sizeof(float);
}

// Vocabulary projection of a decode step (z = h . proj^T) in the router's
// pinned order: 1-4 tokens, and 9-16 over a large vocabulary, by the VALU
// kernels with whole-line row loads; 5-8 by one vocabulary row per thread;
// more by the matrix-core router kernel (64 tokens x 128 vocabulary rows per
// block, every chunk folded).  Each z depends only on its own row pair and is
// the same chain in all of them, so the choice never changes its bits.
hipError_t launch_lm_logits(int T, int H, int V, const uint16_t* h, const uint16_t* proj,
                            float* z, hipStream_t s) {
    if (T <= 1) return launch_lm_stream<1>(T, H, V, h, proj, z, s);
    if (T <= 2) return launch_lm_stream<2>(T, H, V, h, proj, z, s);
    if (T <= 4) return launch_lm_stream<4>(T, H, V, h, proj, z, s);
    if (T <= 8) return launch_lm_stream<8>(T, H, V, h, proj, z, s);
    // 9-16 tokens over a large vocabulary: the VALU kernel with whole-line
    // loads; else (and above 16 tokens) the matrix cores
    if (T <= 16 && V >= 16384) return launch_lm_stream<16>(T, H, V, h, proj, z, s);
    return launch_logits_mfma<2, 2, false>(T, H, V, h, proj, z, s);
}

// Select for E <= 64 * Q experts per token.  The partial planes are folded
// from batches of loads: the smallest batch of 8, 16 or 32 planes that holds
// them all (at most 128 values per lane), since unused slots of a batch still
// take registers and so waves per SIMD (8 planes in the tie layer's 8192
// tokens with a 32-plane batch: 0.117 -> 0.123 ms).
template <int Q, int B, bool P>
hipError_t launch_select_qb(int T, int E, int k, int nparts, int score, int renorm,
                            const float* part, const float* bias, const int32_t* replay,
                            int32_t* ids, float* w, const SmallPermute& sp, hipStream_t s) {
    // with the permutation: one block of one wave per token (T <= 4)
    const int blocks = P ? 1 : (T + 3) / 4;
    const int threads = P ? 64 * T : 256;
    router_select_kernel<Q, B, P><<<blocks, threads, 0, s>>>(T, E, k, nparts, score, renorm,
                                                             part, bias, replay, ids, w, sp);
    return hipGetLastError();
}

template <int Q, bool P>
hipError_t launch_select_q(int T, int E, int k, int nparts, int score, int renorm,
                           const float* part, const float* bias, const int32_t* replay,
                           int32_t* ids, float* w, const SmallPermute& sp, hipStream_t s) {
    constexpr int kMaxBatch = 128 / Q;
    if (nparts <= 1)
        return launch_select_qb<Q, 1, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids,
                                         w, sp, s);
    if (nparts <= 8 || kMaxBatch < 16)
        return launch_select_qb<Q, 8, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids,
                                         w, sp, s);
    if (nparts <= 16 || kMaxBatch < 32)
        return launch_select_qb<Q, 16, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids,
                                          w, sp, s);
    return launch_select_qb<Q, 32, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids, w,
                                      sp, s);
}

template <bool P>
hipError_t launch_select(int T, int E, int k, int nparts, int score, int renorm,
                         const float* part, const float* bias, const int32_t* replay,
                         int32_t* ids, float* w, const SmallPermute& sp, hipStream_t s) {
    if (E <= 64)
        return launch_select_q<1, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids, w, sp, s);
    if (E <= 128)
        return launch_select_q<2, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids, w, sp, s);
    if (E <= 256)
        return launch_select_q<4, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids, w, sp, s);
    return launch_select_q<8, P>(T, E, k, nparts, score, renorm, part, bias, replay, ids, w, sp, s);
}

namespace {

hipError_t launch_route_logits(const RoutePlan& p, int T, int H, int E, const uint16_t* x,
                               const uint16_t* wr, float* part_ws, hipStream_t s) {
    hipError_t err;
    if (p.mfma) {
        err = p.split ? launch_logits_mfma_plan<true>(p, T, H, E, x, wr, part_ws, s)
                      : launch_logits_mfma_plan<false>(p, T, H, E, x, wr, part_ws, s);
    } else if (p.split && T <= 8) {
        if (T <= 1) err = launch_logits_few<1>(T, H, E, x, wr, part_ws, s);
        else if (T <= 2) err = launch_logits_few<2>(T, H, E, x, wr, part_ws, s);
        else if (T <= 4) err = launch_logits_few<4>(T, H, E, x, wr, part_ws, s);
        else err = launch_logits_few<8>(T, H, E, x, wr, part_ws, s);
    } else if (p.split && p.tt == 1) {
        err = launch_logits<1, 1, true>(T, H, E, x, wr, part_ws, s);
    } else if (p.split) {
        if (p.te == 1) err = launch_logits<4, 1, true>(T, H, E, x, wr, part_ws, s);
        else if (p.te == 2) err = launch_logits<4, 2, true>(T, H, E, x, wr, part_ws, s);
        else if (p.te == 4) err = launch_logits<4, 4, true>(T, H, E, x, wr, part_ws, s);
        else err = launch_logits<4, 8, true>(T, H, E, x, wr, part_ws, s);
    } else if (p.te == 1) {
        err = launch_logits<8, 1, false>(T, H, E, x, wr, part_ws, s);
    } else if (p.te == 2) {
        err = launch_logits<8, 2, false>(T, H, E, x, wr, part_ws, s);
    } else if (p.te == 4) {
        err = launch_logits<8, 4, false>(T, H, E, x, wr, part_ws, s);
    } else {
        err = launch_logits<kBigTT, 8, false>(T, H, E, x, wr, part_ws, s);
    }
    return err;
}

}  // namespace

hipError_t launch_route(int T, int H, int E, int k, int score, int renorm, const uint16_t* x,
                        const uint16_t* wr, const float* bias, int32_t* ids, float* w,
                        float* part_ws, hipStream_t s, const int32_t* replay) {
    const RoutePlan p = route_plan(T, H, E);
    const hipError_t err = launch_route_logits(p, T, H, E, x, wr, part_ws, s);
    if (err != hipSuccess) return err;
    return launch_select<false>(T, E, k, p.nparts, score, renorm, part_ws, bias, replay, ids, w,
                                SmallPermute{}, s);
}

// Route and permute in one call: for batches of at most kRoutePermuteMaxT
// tokens (one wave each in the select kernel's single block, at most 64
// assignments) the select kernel also writes counts, offsets, perm and
// inv_perm; larger batches run launch_route, then launch_permute.
constexpr int kRoutePermuteMaxT = 4;

hipError_t launch_route_permute(int T, int H, int E, int k, int score, int renorm,
                                const uint16_t* x, const uint16_t* wr, const float* bias,
                                int32_t* ids, float* w, float* part_ws, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* permute_ws, hipStream_t s) {
    if (T < 1 || T > kRoutePermuteMaxT) {
        const hipError_t err = launch_route(T, H, E, k, score, renorm, x, wr, bias, ids, w,
                                            part_ws, s);
        if (err != hipSuccess) return err;
        return launch_permute(T * k, E, ids, counts, offsets, perm, inv_perm, permute_ws, s);
    }
    const RoutePlan p = route_plan(T, H, E);
    const hipError_t err = launch_route_logits(p, T, H, E, x, wr, part_ws, s);
    if (err != hipSuccess) return err;
    return launch_select<true>(T, E, k, p.nparts, score, renorm, part_ws, bias, nullptr, ids, w,
                               SmallPermute{counts, offsets, perm, inv_perm}, s);
}

}  // namespace moe
