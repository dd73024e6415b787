// moe_fp8.hip -- the FP8 rollout path of the expert FFN: e4m3 codes with
// power-of-two block scales, the block quantiser, and the two grouped GEMMs.
//
// The pages' large-MoE recipe trains in BF16 and samples rollouts with FP8
// weights, and keeps measuring the gap between the two policies ("GLM
// Post-Training Beyond SFT", quantisation section).  They fix no format or
// block shape.  Reading taken (the same as the CPU definition):
//   e4m3    OCP E4M3FN, fp32 -> e4m3 round to nearest, ties to even;
//   scale   2^e per block, e = the smallest integer with amax <= 448 * 2^e,
//           clamped to [-127, 127] (0 for an all-zero block); weight blocks
//           128 output rows x 128 K, activation blocks 1 row x 128 K;
//   GEMM    fp32 accumulation over the K blocks in ascending order of
//           2^(ea + ew) * sum of the block's 128 code products;
//   expert  act = bf16(silu(g) * u), quantised by rows for the down GEMM.
//
// Matrix instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 on both
// sides.  Lane l supplies 32 codes of row l%16 of each operand (the same 32 K
// positions on both sides) and a biased exponent byte (127 + e) per operand,
// which the instruction applies to its 128-term block sum: one instruction is
// one 16 x 16 block of one 128-wide K block, scales included.  Measured on
// gfx950: the instruction adds its products in groups of 8 K positions; in a
// group, products more than 13 binades below the group's largest are cut
// (toward zero) to that grid, and the group sums and the accumulator are
// added at fp32 precision.  Every output therefore lies within
// 7 * 2^-13 * sum over groups (largest |product|) plus a few fp32 roundings
// of the block sum -- the bound the GPU tests hold it to.
//
// Batch invariance is kept as in the bf16 GEMMs: one tile shape (256 weight
// rows x 256 token rows), one instruction, K blocks in ascending order, no
// split, whatever the expert's token count; padding rows only feed dropped
// results.
#include <algorithm>

#include "moe_device.h"
#include "moe_gemm_tiles.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 for amax = 0
// (and for NaN, which the block maximum never holds), 127 for +inf
__device__ __forceinline__ int fp8_block_exp(float amax) {
    if (!(amax > 0.0f)) return 0;
    if (amax > 3.40282347e38f) return 127;
    int ex;
    const float f = frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
    // 448 * 2^e = 0.875 * 2^(e + 9)
    const int e = ex - 9 + (f > 0.875f ? 1 : 0);
    return e < -127 ? -127 : e;
}

// e4m3 code of a value already scaled into [-448, 448] (or non-finite):
// the hardware conversion rounds to nearest even; NaN -> 0x7F and +-inf ->
// +-448 as in the CPU definition.
__device__ __forceinline__ uint32_t fix_nonfinite(uint32_t w, float v, int byte) {
    const uint32_t b = __float_as_uint(v);
    if ((b & 0x7FFFFFFFu) >= 0x7F800000u) {
        const uint32_t c = ((b & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7Fu : (((b >> 24) & 0x80u) | 0x7Eu);
        w = (w & ~(0xFFu << (8 * byte))) | (c << (8 * byte));
    }
    return w;
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
    w = fix_nonfinite(w, a, 0);
    w = fix_nonfinite(w, b, 1);
    w = fix_nonfinite(w, c, 2);
    return fix_nonfinite(w, d, 3);
}

// 8 bf16 (one 16-byte load) -> largest magnitude (NaN ignored)
__device__ __forceinline__ float absmax8(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fabsf(bf16_to_f32(w[i] & 0xFFFFu)));
        m = fmaxf(m, fabsf(bf16_to_f32(w[i] >> 16)));
    }
    return m;
}

// ---------------------------------------------------------------------------
// Block quantiser: bf16 [R, K] -> codes [R, K] and exponents
// [R / block_rows, K / 128].  One 16-lane group per (row block, K block);
// lane i of the group holds columns [8i, 8i + 8) of each row of the block:
// one pass for the block maximum, one for the codes (exact scaling by 2^-e,
// then the hardware conversion).
// ---------------------------------------------------------------------------
// (rows != null: only the rows in [rows[0], rows[nseg]), bounds the device
// holds, e.g. the expert offsets of a permuted matrix.)
__global__ __launch_bounds__(256) void quantize_fp8_kernel(int R, int K, int block_rows,
                                                           const uint16_t* __restrict__ src,
                                                           uint8_t* __restrict__ q,
                                                           int8_t* __restrict__ exps,
                                                           const int32_t* __restrict__ rows,
                                                           int nseg) {
    const int nkb = K / kFp8Block;
    const long units = (long)(R / block_rows) * nkb;
    const long unit = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
    if (unit >= units) return;   // a 16-lane group leaves as a whole
    const int li = threadIdx.x & 15;
    const int rb = (int)(unit / nkb), kb = (int)(unit % nkb);
    if (rows && (rb * block_rows < rows[0] || rb * block_rows >= rows[nseg])) return;
    const size_t col = (size_t)kb * kFp8Block + li * 8;
    const int r0 = rb * block_rows, r1 = r0 + block_rows;
    float amax = 0.0f;
    for (int r = r0; r < r1; ++r)
        amax = fmaxf(amax, absmax8(*reinterpret_cast<const uint4*>(src + (size_t)r * K + col)));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    const int e = fp8_block_exp(amax);
    if (li == 0) exps[unit] = (int8_t)e;
    for (int r = r0; r < r1; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * K + col);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = ldexpf(bf16_to_f32(w[i] & 0xFFFFu), -e);
            f[2 * i + 1] = ldexpf(bf16_to_f32(w[i] >> 16), -e);
        }
        uint2 out;
        out.x = e4m3x4(f[0], f[1], f[2], f[3]);
        out.y = e4m3x4(f[4], f[5], f[6], f[7]);
        *reinterpret_cast<uint2*>(q + (size_t)r * K + col) = out;
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMMs.  8 waves, tile = 256 weight rows x 256 token rows; K staged
// 128 codes (one scale block, 128 bytes per row) at a time through two 64 KB
// LDS stages filled by direct-to-LDS loads, with the byte layout, XOR swizzle
// and load issue of the bf16 pipelined kernel (8 rows x 128 bytes per
// instruction, waves 0-3 issue).  Each wave computes 128 weight rows x 64
// token rows.  The tile's exponents are staged in LDS at tile start as
// biased scale bytes.  A lane's 32 codes of a 16-row group are 16-byte
// chunks c and c + 4 (c = lane / 16) of its row: the same K positions on the
// weight and the token side.
// ---------------------------------------------------------------------------
constexpr int kQ_Threads = 512;
constexpr int kQ_Tok = kTileTok;
constexpr int kQ_W = 256;
constexpr int kQ_BK = kFp8Block;                    // 128 codes = 128 bytes
constexpr int kQ_StageBytes = (kQ_W + kQ_Tok) * kQ_BK;
constexpr int kQ_Blocks = (kQ_W + kQ_Tok) / 8;      // 64 blocks of 8 rows
constexpr int kQ_WBlocks = kQ_W / 8;                // 32
constexpr int kQ_Issuers = 4;
constexpr int kQ_Dma = kQ_Blocks / kQ_Issuers;      // 16
constexpr int kQ_WDma = kQ_WBlocks / kQ_Issuers;    // 8
constexpr int kQ_GateUpF = kQ_W / 2;                // 128: one gate block + one up block
constexpr int kMB = 8;
constexpr int kNB = 4;

constexpr int MODE_GATE_UP = 0;
constexpr int MODE_DOWN = 1;

struct Fp8Params {
    int K;                     // H (gate/up) or F (down)
    int N;                     // F (gate/up) or H (down)
    int n_tiles;
    int top_k;
    int E;
    const uint8_t* act;        // gate/up: x codes [T,H]; down: act codes [A,F] (permuted rows)
    const int8_t* act_e;       // their exponents [rows, K/128]
    const int32_t* perm;
    const int32_t* offsets;    // [E+1]
    const int32_t* tile_start;
    const int32_t* tail;
    const uint8_t* w0;         // w_gate or w_down codes [E,N,K]
    const int8_t* we0;         // [E,N/128,K/128]
    const uint8_t* w1;         // w_up codes (gate/up)
    const int8_t* we1;
    void* out;                 // gate/up: act codes u8 [A,F]; down: y fp32 [A,H]
    int8_t* out_e;             // gate/up: act exponents [A,F/128]
    uint16_t* out_bf16;        // gate/up: bf16 act [A,F], or null
};

__device__ __forceinline__ int8v frag(const unsigned char* blk, int off0, int off1) {
    const int4v lo = *reinterpret_cast<const int4v*>(blk + off0);
    const int4v hi = *reinterpret_cast<const int4v*>(blk + off1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Direct-to-LDS load with a wave-uniform base (SGPR pair) and a 32-bit lane
// offset: half the address registers of the 64-bit form.
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}

// A tile with at most 64 valid token rows needs 32 KB of weight rows and
// 8 KB of token rows per step: three such stages fit where two full stages
// do, and keep the loads of two steps in flight.
constexpr int kQ_DeepTok = 64;
constexpr int kQ_DeepStageBytes = kQ_WBlocks * 1024 + (kQ_DeepTok / 8) * 1024;   // 40960
static_assert(3 * kQ_DeepStageBytes <= 2 * kQ_StageBytes, "three deep stages fit");

template <int MODE, bool DEEP>
__device__ __forceinline__ void expert_gemm_fp8_body(const Fp8Params& P, unsigned char* smem,
                                                     uint8_t* s_tsc, uint8_t* s_wsc,
                                                     float* s_amax) {
    const uint32_t lds0 =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;   // weight half: 128 rows (gate/up: 64 gate + 64 up)
    const int wt = wave >> 1;  // token quarter: 64 rows

    const int fr = lane & 7;
    const int fblk = (lane >> 3) & 1;
    const int off0 = fblk * 1024 + fr * 128 + (((lane >> 4) ^ fr) << 4);
    const int off1 = fblk * 1024 + fr * 128 + (((4 + (lane >> 4)) ^ fr) << 4);
    const int drow = lane >> 3;
    const int dchunk = (lane & 7) ^ drow;

    const int E = P.E;
    const int total_long = P.tile_start[E];
    const int total_m = total_long + P.tail[0];
    const int total = total_m * P.n_tiles;
    const int nblk = gridDim.x;
    const int slot = tile_slot();
    const int nkb = P.K / kQ_BK;
    const int nwb = P.N / kFp8Block;   // weight blocks along N

    auto wgrp = [&](int mb) {
        if (MODE == MODE_GATE_UP)
            return (mb < 4) ? (wm * 8 + mb * 2) : (kQ_WBlocks / 2 + wm * 8 + (mb - 4) * 2);
        return wm * 16 + mb * 2;
    };

    for (int base = 0; base < total; base += nblk) {
        const int lt = base + slot;
        if (lt >= total) break;
        const TileRef tr = tile_at(lt, total_m, total_long, P.n_tiles, E, P.tile_start, P.tail,
                                   P.offsets);
        const int e = tr.e, nt = tr.nt;
        const int seg1 = P.offsets[e + 1];
        const int p0 = P.offsets[e] + tr.local * kQ_Tok;
        const int valid = seg1 - p0;
        const int ntb = (valid + 7) >> 3;
        const bool active = wt * 64 < valid;

        // direct-to-LDS sources: slot i of issuing wave iw fills block
        // i * 4 + iw; slots 0-3 are weight blocks 0-15 (gate rows in gate/up),
        // 4-7 blocks 16-31 (up rows), 8-15 token blocks.  Base per slot group
        // (uniform) + 32-bit row offset per lane (< 2^31: one expert's weight
        // matrix, or the code matrix of all rows).
        const int iw = wave % kQ_Issuers;
        const uint8_t* wb0 = P.w0 + (size_t)e * P.N * P.K;
        const uint8_t* wb1 = (MODE == MODE_GATE_UP) ? P.w1 + (size_t)e * P.N * P.K : wb0;
        uint32_t voff[kQ_Dma];
#pragma unroll
        for (int i = 0; i < kQ_Dma; ++i) {
            const int b = i * kQ_Issuers + iw;
            int row;
            if (i < kQ_WDma) {
                const int rr = b * 8 + drow;
                if (MODE == MODE_GATE_UP)
                    row = nt * kQ_GateUpF + (rr & (kQ_GateUpF - 1));
                else
                    row = min(nt * kQ_W + rr, P.N - 1);
            } else {
                const int p = min(p0 + (b - kQ_WBlocks) * 8 + drow, seg1 - 1);
                row = (MODE == MODE_GATE_UP) ? P.perm[p] / P.top_k : p;
            }
            voff[i] = (uint32_t)row * (uint32_t)P.K + (uint32_t)(dchunk * 16);
        }

        floatx4 acc[kMB][kNB];
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

        // previous tile: stores drained, every wave done with the stages and
        // the exponent tables
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        block_barrier();

        // this tile's exponents -> LDS (published by the first stage barrier)
        {
            const int r = tid & (kQ_Tok - 1);
            const int p = min(p0 + r, seg1 - 1);
            const int ar = (MODE == MODE_GATE_UP) ? P.perm[p] / P.top_k : p;
            const int8_t* er = P.act_e + (size_t)ar * nkb;
            for (int kb = tid >> 8; kb < nkb; kb += kQ_Threads / kQ_Tok)
                s_tsc[kb * kQ_Tok + r] = (uint8_t)(127 + er[kb]);
            if (tid < 2 * nkb) {
                const int kb = tid >> 1, j = tid & 1;
                const int8_t* we;
                if (MODE == MODE_GATE_UP)
                    we = (j ? P.we1 : P.we0) + ((size_t)e * nwb + nt) * nkb;
                else
                    we = P.we0 + ((size_t)e * nwb + min(nt * 2 + j, nwb - 1)) * nkb;
                s_wsc[kb * 2 + j] = (uint8_t)(127 + we[kb]);
            }
        }

        // In a launch that only streams weights (DEEP), a tile with at most
        // 64 valid rows ("deep") cycles through three 40 KB stages with the
        // loads of two steps in flight; every other tile alternates two 64 KB
        // stages, one step ahead.  Either way a stage is refilled only after
        // the barrier that follows every wave's reads of it, and the MFMA
        // sequence of an output element is the same.
        const bool deep = DEEP && valid <= kQ_DeepTok;
        auto stage_off = [&](int kt) {
            return deep ? (kt % 3) * kQ_DeepStageBytes : (kt & 1) * kQ_StageBytes;
        };
        auto issue = [&](int kt) {
            const uint32_t sbase = lds0 + (uint32_t)stage_off(kt);
            if (wave >= kQ_Issuers) return;
            const size_t ko = (size_t)kt * kQ_BK;
#pragma unroll
            for (int i = 0; i < kQ_Dma; ++i) {
                if (i >= kQ_WDma && (i - kQ_WDma) * kQ_Issuers + iw >= ntb) continue;
                const uint8_t* bse = (i < kQ_WDma / 2) ? wb0 : (i < kQ_WDma ? wb1 : P.act);
                dma16_sbase(bse + ko, voff[i], sbase + (uint32_t)((i * kQ_Issuers + iw) * 1024));
            }
        };
        const int ahead = deep ? 2 : 1;
        // loads per step of this thread in a deep tile: 8 weight blocks and
        // its token blocks below ntb (at most 8 in all)
        const int nload =
            wave < kQ_Issuers ? kQ_WDma + (ntb > iw ? 1 : 0) + (ntb > iw + 4 ? 1 : 0) : 0;
        for (int j = 0; j < ahead; ++j)
            if (j < nkb) issue(j);

        for (int kt = 0; kt < nkb; ++kt) {
            // this step's loads landed; a deep tile leaves the next step's
            // nload loads of this thread in flight (loads complete in order)
            if (deep && kt + 1 < nkb && nload == 8)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else if (deep && kt + 1 < nkb && nload == 9)
                asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
            else if (deep && kt + 1 < nkb && nload == 10)
                asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            block_barrier();
            if (kt + ahead < nkb) issue(kt + ahead);
            if (!active) continue;
            const unsigned char* sb = smem + stage_off(kt);
            const int sa0 = s_wsc[kt * 2 + (MODE == MODE_GATE_UP ? 0 : wm)];
            const int sa1 = (MODE == MODE_GATE_UP) ? (int)s_wsc[kt * 2 + 1] : sa0;
            int sbv[kNB];
            int8v fb[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                sbv[nb] = s_tsc[kt * kQ_Tok + wt * 64 + nb * 16 + (lane & 15)];
                fb[nb] = frag(sb + (kQ_WBlocks + wt * 8 + nb * 2) * 1024, off0, off1);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int8v fa[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) fa[mb] = frag(sb + wgrp(h * 4 + mb) * 1024, off0, off1);
                const int sa = h ? sa1 : sa0;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb)
                        acc[h * 4 + mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            fa[mb], fb[nb], acc[h * 4 + mb][nb], 0, 0, 0, sa, 0, sbv[nb]);
            }
        }

        // epilogue: lane holds weight rows 4*(lane>>4)+q of token column lane&15
        const int colq = 4 * (lane >> 4);
        if (MODE == MODE_GATE_UP) {
            // act = bf16(silu(g) * u) of this wave's 64 columns; the 1 x 128
            // block of a token row spans both column halves (wm = 0, 1)
            uint32_t hb[kNB][4][2];
            float am[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                am[nb] = 0.0f;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    uint32_t h[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h[q] = f32_to_bf16_rne(silu_f(acc[mb][nb][q]) * acc[mb + 4][nb][q]);
                        am[nb] = fmaxf(am[nb], fabsf(bf16_to_f32(h[q])));
                    }
                    hb[nb][mb][0] = h[0] | (h[1] << 16);
                    hb[nb][mb][1] = h[2] | (h[3] << 16);
                }
                am[nb] = fmaxf(am[nb], __shfl_xor(am[nb], 16, kWave));
                am[nb] = fmaxf(am[nb], __shfl_xor(am[nb], 32, kWave));
            }
            if (lane < 16) {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) s_amax[wm * kQ_Tok + wt * 64 + nb * 16 + lane] = am[nb];
            }
            __syncthreads();
            uint8_t* qout = reinterpret_cast<uint8_t*>(P.out);
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const int r = wt * 64 + nb * 16 + (lane & 15);
                const int p = p0 + r;
                if (p >= seg1) continue;
                const int ex = fp8_block_exp(fmaxf(s_amax[r], s_amax[kQ_Tok + r]));
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const int f = nt * kQ_GateUpF + wm * 64 + mb * 16 + colq;
                    const uint32_t h0 = hb[nb][mb][0], h1 = hb[nb][mb][1];
                    const uint32_t c = e4m3x4(ldexpf(bf16_to_f32(h0 & 0xFFFFu), -ex),
                                              ldexpf(bf16_to_f32(h0 >> 16), -ex),
                                              ldexpf(bf16_to_f32(h1 & 0xFFFFu), -ex),
                                              ldexpf(bf16_to_f32(h1 >> 16), -ex));
                    *reinterpret_cast<uint32_t*>(qout + (size_t)p * P.N + f) = c;
                    if (P.out_bf16) {
                        uint2 pk;
                        pk.x = h0;
                        pk.y = h1;
                        *reinterpret_cast<uint2*>(P.out_bf16 + (size_t)p * P.N + f) = pk;
                    }
                }
                if (wm == 0 && lane < 16) P.out_e[(size_t)p * nwb + nt] = (int8_t)ex;
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const int p = p0 + wt * 64 + nb * 16 + (lane & 15);
                if (p >= seg1) continue;
                const int a = P.perm[p];
                float* yout = reinterpret_cast<float*>(P.out) + (size_t)a * P.N;
#pragma unroll
                for (int mb = 0; mb < kMB; ++mb) {
                    const int h = nt * kQ_W + wm * 128 + mb * 16 + colq;
                    if (h >= P.N) continue;
                    *reinterpret_cast<floatx4*>(yout + h) = acc[mb][nb];
                }
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// A gate/up launch whose tile list holds no long tile (every expert has at
// most 128 tokens: decode-sized batches) only streams expert weights and runs
// the body that keeps two steps of loads in flight; the choice is made once
// per launch from the tile list and never changes the MFMA sequence.
template <int MODE>
__global__ __launch_bounds__(kQ_Threads) void expert_gemm_fp8_kernel(Fp8Params P) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kQ_StageBytes];
    __shared__ uint8_t s_tsc[kFp8MaxKB * kQ_Tok];   // [kb][token row] 127 + e
    __shared__ uint8_t s_wsc[kFp8MaxKB * 2];        // [kb][gate|up, or weight half] 127 + e
    __shared__ float s_amax[2 * kQ_Tok];            // gate/up: |act| max per column half
    if (MODE == MODE_GATE_UP && P.tile_start[P.E] == 0)
        expert_gemm_fp8_body<MODE, MODE == MODE_GATE_UP>(P, smem, s_tsc, s_wsc, s_amax);
    else
        expert_gemm_fp8_body<MODE, false>(P, smem, s_tsc, s_wsc, s_amax);
}

// ---------------------------------------------------------------------------
// Weight-streaming FP8 GEMMs, for calls of at most 32 tokens.  Such a call
// only streams the active experts' weights, and the 256-row tiles above would
// leave most CUs idle (8 active experts x F/128 tiles).  A work item is one
// active expert x 64 weight rows (gate/up: 32 gate + 32 up rows of the same
// features; down: 64 output rows); each of the block's 4 waves multiplies 16
// weight rows by the expert's token rows (16 or 32 at a time).  A wave's
// weight rows arrive as whole 128-byte lines, one K block (128 codes a row)
// per pair of loads (lane l: rows l/8 and 8 + l/8, chunk (l%8) ^ (l/8)), four
// K blocks in flight, and pass through 2 KB of the wave's own LDS into the
// fragment layout (one wave's LDS operations run in order: no barrier).  The
// token fragments and both exponents come straight from global memory.
//
// The MFMA sequence of an output element is the tiled kernel's: one
// v_mfma_scale_f32_16x16x128_f8f6f4 per K block, K blocks ascending, lane l
// holding row l%16 and chunks l/16 and 4 + l/16 of the block on both sides,
// with the same scale bytes, accumulators from 0.  So the bits are equal.
// gate/up writes act = bf16(silu(g) * u) and leaves its quantisation to the
// block quantiser (the same exponent and codes the tiled epilogue computes
// from the same bf16 values), since a 128-feature scale block spans four
// work items.
// ---------------------------------------------------------------------------
constexpr int kQS_MaxE = 512;
constexpr int kQS_Ring = 4;            // K blocks in flight per wave
constexpr int kQS_GateUpF = 32;        // gate/up features per work item
constexpr int kQS_DownH = 64;          // down output rows per work item

template <int MODE, int NB>
__global__ __launch_bounds__(256) void expert_gemm_fp8_stream_kernel(Fp8Params P,
                                                                     uint16_t* act16) {
    __shared__ int act_list[kQS_MaxE];
    __shared__ int4v wscr[4][128];                  // a wave's K block of weight rows
    __shared__ floatx4 xch[2][NB][kWave];           // up waves' sums, for the gate waves
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int E = P.E;
    const int nkb = P.K / kFp8Block;
    const int nwb = P.N / kFp8Block;

    // the active experts, ascending (wave 0 builds the list; counts <= 32)
    __shared__ int s_nact;
    if (wave == 0) {
        int n = 0;
        for (int e0 = 0; e0 < E; e0 += kWave) {
            const int e = e0 + lane;
            const bool a = e < E && P.offsets[e + 1] > P.offsets[e];
            const uint64_t m = __ballot(a);
            if (a) act_list[n + __popcll(m & ((1ull << lane) - 1))] = e;
            n += __popcll(m);
        }
        if (lane == 0) s_nact = n;
    }
    __syncthreads();
    const int n_act = s_nact;
    const int total = n_act * P.n_tiles;

    const int r = lane & 15, rr = r & 7;
    const int rd0 = (r >> 3) * 64 + rr * 8 + ((lane >> 4) ^ rr);         // int4v units
    const int rd1 = (r >> 3) * 64 + rr * 8 + ((4 + (lane >> 4)) ^ rr);
    int4v* const scr = wscr[wave];
    const int colq = 4 * (lane >> 4);

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int li = item / P.n_tiles;
        const int nt = item - li * P.n_tiles;
        const int e = act_list[li];
        const int seg0 = P.offsets[e], seg1 = P.offsets[e + 1];

        // this wave's 16 weight rows and their exponent row
        const int r0 = (MODE == MODE_GATE_UP) ? nt * kQS_GateUpF + (wave & 1) * 16
                                              : nt * kQS_DownH + wave * 16;
        const uint8_t* wb = (MODE == MODE_GATE_UP && wave >= 2) ? P.w1 : P.w0;
        const int8_t* web = (MODE == MODE_GATE_UP && wave >= 2) ? P.we1 : P.we0;
        const uint8_t* pw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            pw[h] = wb + ((size_t)e * P.N + r0 + (lane >> 3) + 8 * h) * P.K +
                    ((lane & 7) ^ (lane >> 3)) * 16;
        const int8_t* pwe = web + ((size_t)e * nwb + r0 / kFp8Block) * nkb;

        for (int tb = seg0; tb < seg1; tb += NB * 16) {
            const uint8_t* pt[NB];
            const int8_t* pte[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int p = min(tb + nb * 16 + (lane & 15), seg1 - 1);
                const int ar = (MODE == MODE_GATE_UP) ? P.perm[p] / P.top_k : p;
                pt[nb] = P.act + (size_t)ar * P.K + (lane >> 4) * 16;
                pte[nb] = P.act_e + (size_t)ar * nkb;
            }
            // a ring of kQS_Ring K blocks: slot u holds block kb0 + u and is
            // refilled with block kb0 + u + kQS_Ring after its MFMAs (the last
            // block again past the end: cache hits whose values are unused)
            int4v wf[kQS_Ring][2], tf[kQS_Ring][NB][2];
            int wsc[kQS_Ring], tsc[kQS_Ring][NB];
            auto load = [&](int u, int kb) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wf[u][h] = *reinterpret_cast<const int4v*>(pw[h] + (size_t)kb * kFp8Block);
                wsc[u] = 127 + pwe[kb];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    tf[u][nb][0] = *reinterpret_cast<const int4v*>(pt[nb] + (size_t)kb * kFp8Block);
                    tf[u][nb][1] =
                        *reinterpret_cast<const int4v*>(pt[nb] + (size_t)kb * kFp8Block + 64);
                    tsc[u][nb] = 127 + pte[nb][kb];
                }
            };
#pragma unroll
            for (int u = 0; u < kQS_Ring; ++u) {
                load(u, min(u, nkb - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
            floatx4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int kb0 = 0; kb0 < nkb; kb0 += kQS_Ring) {
#pragma unroll
                for (int u = 0; u < kQS_Ring; ++u) {
                    if (kb0 + u < nkb) {
                        scr[lane] = wf[u][0];
                        scr[64 + lane] = wf[u][1];
                        const int8v fa = __builtin_shufflevector(scr[rd0], scr[rd1], 0, 1, 2, 3,
                                                                 4, 5, 6, 7);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const int8v fb = __builtin_shufflevector(tf[u][nb][0], tf[u][nb][1],
                                                                     0, 1, 2, 3, 4, 5, 6, 7);
                            acc[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                fa, fb, acc[nb], 0, 0, 0, wsc[u], 0, tsc[u][nb]);
                        }
                    }
                    load(u, min(kb0 + u + kQS_Ring, nkb - 1));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // epilogue: lane holds weight rows r0 + colq + q of token column lane&15
            if (MODE == MODE_GATE_UP) {
                if (wave >= 2) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) xch[wave - 2][nb][lane] = acc[nb];
                }
                __syncthreads();
                if (wave < 2) {
                    const int f = r0 + colq;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int p = tb + nb * 16 + (lane & 15);
                        if (p >= seg1) continue;
                        const floatx4 up = xch[wave][nb][lane];
                        uint32_t h[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            h[q] = f32_to_bf16_rne(silu_f(acc[nb][q]) * up[q]);
                        uint2 pk;
                        pk.x = h[0] | (h[1] << 16);
                        pk.y = h[2] | (h[3] << 16);
                        *reinterpret_cast<uint2*>(act16 + (size_t)p * P.N + f) = pk;
                    }
                }
                __syncthreads();
            } else {
                const int hrow = r0 + colq;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int p = tb + nb * 16 + (lane & 15);
                    if (p >= seg1) continue;
                    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(P.out) +
                                                (size_t)P.perm[p] * P.N + hrow) = acc[nb];
                }
            }
        }
    }
}

template <int MODE>
hipError_t launch_fp8_stream(const Fp8Params& P, int T, uint16_t* act16, hipStream_t s) {
    // at most min(E, T*k) experts are active: no more work items than that
    const long items = (long)std::min(P.E, T * P.top_k) * P.n_tiles;
    const int grid = (int)std::max(1L, std::min(items, (long)device_cu_count() * 8));
    if (T <= 16)
        expert_gemm_fp8_stream_kernel<MODE, 1><<<grid, 256, 0, s>>>(P, act16);
    else
        expert_gemm_fp8_stream_kernel<MODE, 2><<<grid, 256, 0, s>>>(P, act16);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_fp8_gemm(const Fp8Params& P, hipStream_t s) {
    const int cu = device_cu_count();
    const int b = (cu + kXcds - 1) / kXcds * kXcds;
    expert_gemm_fp8_kernel<MODE><<<b, kQ_Threads, 0, s>>>(P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(int R, int K, int block_rows, const uint16_t* src, uint8_t* q,
                               int8_t* exps, hipStream_t s) {
    const long units = (long)(R / block_rows) * (K / kFp8Block);
    if (units == 0) return hipSuccess;
    const long blocks = (units + 15) / 16;
    quantize_fp8_kernel<<<(unsigned)blocks, 256, 0, s>>>(R, K, block_rows, src, q, exps, nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_gate_up_fp8(int T, int H, int E, int F, int k, const uint8_t* xq,
                              const int8_t* xe, const int32_t* perm, const int32_t* offsets,
                              const uint8_t* wgq, const int8_t* wge, const uint8_t* wuq,
                              const int8_t* wue, uint8_t* aq, int8_t* ae, uint16_t* act_bf16,
                              int32_t* sched_ws, hipStream_t s) {
    (void)T;
    hipError_t err = launch_tile_schedule(E, 0, 1, offsets, sched_ws, s);
    if (err != hipSuccess) return err;
    Fp8Params P;
    P.K = H; P.N = F; P.n_tiles = F / kQ_GateUpF; P.top_k = k; P.E = E;
    P.act = xq; P.act_e = xe; P.perm = perm; P.offsets = offsets;
    P.tile_start = sched_ws; P.tail = sched_ws + E + 1;
    P.w0 = wgq; P.we0 = wge; P.w1 = wuq; P.we1 = wue;
    P.out = aq; P.out_e = ae; P.out_bf16 = act_bf16;
    return launch_fp8_gemm<MODE_GATE_UP>(P, s);
}

hipError_t launch_down_fp8(int T, int H, int E, int F, int k, const uint8_t* aq,
                           const int8_t* ae, const int32_t* perm, const int32_t* offsets,
                           const uint8_t* wdq, const int8_t* wde, float* y, int32_t* sched_ws,
                           hipStream_t s) {
    (void)T;
    hipError_t err = launch_tile_schedule(E, 0, 0, offsets, sched_ws, s);
    if (err != hipSuccess) return err;
    Fp8Params P;
    P.K = F; P.N = H; P.n_tiles = (H + kQ_W - 1) / kQ_W; P.top_k = k; P.E = E;
    P.act = aq; P.act_e = ae; P.perm = perm; P.offsets = offsets;
    P.tile_start = sched_ws; P.tail = sched_ws + E + 1;
    P.w0 = wdq; P.we0 = wde; P.w1 = nullptr; P.we1 = nullptr;
    P.out = y; P.out_e = nullptr; P.out_bf16 = nullptr;
    return launch_fp8_gemm<MODE_DOWN>(P, s);
}

// The weight-streaming forms (calls of at most kFp8StreamMaxTok tokens; the
// caller checks).  gate/up writes the bf16 act to act16 ([A, F], permuted
// rows) and quantises the placed rows from it.
hipError_t launch_gate_up_fp8_stream(int T, int H, int E, int F, int k, const uint8_t* xq,
                                     const int8_t* xe, const int32_t* perm,
                                     const int32_t* offsets, const uint8_t* wgq,
                                     const int8_t* wge, const uint8_t* wuq, const int8_t* wue,
                                     uint8_t* aq, int8_t* ae, uint16_t* act16, hipStream_t s) {
    Fp8Params P;
    P.K = H; P.N = F; P.n_tiles = F / kQS_GateUpF; P.top_k = k; P.E = E;
    P.act = xq; P.act_e = xe; P.perm = perm; P.offsets = offsets;
    P.tile_start = nullptr; P.tail = nullptr;
    P.w0 = wgq; P.we0 = wge; P.w1 = wuq; P.we1 = wue;
    P.out = nullptr; P.out_e = nullptr; P.out_bf16 = nullptr;
    hipError_t err = launch_fp8_stream<MODE_GATE_UP>(P, T, act16, s);
    if (err != hipSuccess) return err;
    const int A = T * k;
    const long blocks = ((long)A * (F / kFp8Block) + 15) / 16;
    quantize_fp8_kernel<<<(unsigned)blocks, 256, 0, s>>>(A, F, 1, act16, aq, ae, offsets, E);
    return hipGetLastError();
}

hipError_t launch_down_fp8_stream(int T, int H, int E, int F, int k, const uint8_t* aq,
                                  const int8_t* ae, const int32_t* perm, const int32_t* offsets,
                                  const uint8_t* wdq, const int8_t* wde, float* y, hipStream_t s) {
    Fp8Params P;
    P.K = F; P.N = H; P.n_tiles = H / kQS_DownH; P.top_k = k; P.E = E;
    P.act = aq; P.act_e = ae; P.perm = perm; P.offsets = offsets;
    P.tile_start = nullptr; P.tail = nullptr;
    P.w0 = wdq; P.we0 = wde; P.w1 = nullptr; P.we1 = nullptr;
    P.out = y; P.out_e = nullptr; P.out_bf16 = nullptr;
    return launch_fp8_stream<MODE_DOWN>(P, T, nullptr, s);
}

}  // namespace moe
