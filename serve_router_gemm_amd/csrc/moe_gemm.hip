// moe_gemm.hip -- grouped expert GEMMs: gate/up with the SwiGLU epilogue, and
// the down projection.
//
// Batch invariance of the expert matmuls: a per-expert kernel or tiling that
// changes with the expert's token count moves bits, so one kernel choice
// must serve every token count (Fireworks page "位级一致：前沿训练的差异化关键",
// section "为什么比特级一致是一个复杂的问题"), and split-K is out because it
// breaks invariance (same page, section "曾经只有前沿实验室才有的功能").
//
// Invariant kernel, for every tile of every expert at every batch size:
//   * one tile shape: 256 weight rows (gate/up: 128 gate + 128 up) x 256
//     token rows, K staged 64 at a time;
//   * one instruction: v_mfma_f32_16x16x32_bf16, fp32 accumulators from 0;
//   * one K order: k = 0, 32, 64, ... ascending, no split;
// so an output element is the same sequence of MFMAs over the same operands
// whatever other rows share its tile.  Rows past an expert's segment are
// loaded from its last valid row and their results dropped.  (The bits of an
// element depend on that MFMA sequence only: 256 x 128 and 512 x 128 tilings
// of this kernel produced identical outputs on the large layer.)
//
// Operand roles: the weight rows are the MFMA "A" (M) side and the token rows
// the "B" (N) side, so each lane's four accumulators run along the output
// feature dimension and store as one contiguous vector.
//
// Scheduling: one persistent workgroup per CU walks the device-side tile
// list; tile ids go to XCDs in contiguous blocks and are rastered in groups of
// 8 token tiles so the workgroups of one XCD share weight and token rows in
// its L2.  Only the launch work depends on the per-expert counts, never the
// arithmetic.
//
// The load-dependent variant exists to measure what invariance costs and to
// show what breaking it does: experts with at most 32 tokens have the K range
// of both GEMMs cut into parts chosen from their token count, each part
// summed on its own into a workspace and the parts added by a separate pass
// (deterministic run to run, but an expert's arithmetic then depends on how
// many tokens the batch sent it); larger experts take the tiled kernel.
#include <algorithm>
#include <atomic>

#include "moe_device.h"
#include "moe_gemm_tiles.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMB = 8;                   // MFMA blocks of 16 weight rows per wave
constexpr int kNB = 4;                   // MFMA blocks of 16 token rows per wave

constexpr int MODE_GATE_UP = 0;
constexpr int MODE_DOWN = 1;

struct GemmParams {
    int K;            // reduction length: H (gate/up) or F (down)
    int N;            // output features: F (gate/up) or H (down)
    int n_tiles;      // output tiles along N
    int top_k;
    int E;
    const uint16_t* act;       // gate/up: x [T,H]; down: h_act [A,F]
    const int32_t* perm;
    const int32_t* offsets;    // [E+1]
    const int32_t* tile_start; // [E+1] prefix of long token tiles
    const int32_t* tail;       // [1+E] count, then experts whose last tile is short
    const uint16_t* w0;        // w_gate or w_down [E, N, K]
    const uint16_t* w1;        // w_up (gate/up only)
    void* out;                 // h_act bf16 [A,F] or y fp32 [A,H]
    // streaming kernel: experts with 0 < count <= max_count; in the split
    // (variant) mode their partial sums go to part [parts_max][R][NW] fp32
    // (NW = 2F: g then u, or H), rowmap [R][2] (permuted row, parts) and
    // nrows [1] (rows used)
    int max_count;
    int parts_max;
    int R;
    float* part;
    int32_t* rowmap;
    int32_t* nrows;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ---------------------------------------------------------------------------
// Pipelined kernel: 8 waves, tile = 256 weight rows x 256 token rows, K staged
// 64 at a time through a ring of five 32 KB LDS units (the whole 160 KB) filled
// by direct-to-LDS loads: the weight rows of a step fill one unit, its token
// rows another.  Each wave computes 128 weight rows x 64 token rows.
//
// A unit holds 256 rows x 128 bytes as 32 blocks of 8 rows (1 KB).  A
// direct-to-LDS load (global_load_lds_dwordx4) writes lane l's 16 bytes at
// M0 + 16*l, so one wave instruction fills one block: lane l lands at row
// l/8, physical chunk l%8, and loads logical chunk (l%8) ^ (l/8) of that row.
// Each instruction thus reads 8 whole 128-byte lines (measured on gfx950:
// ~1.7x the rate of 16 half lines).  Fragment reads use the same XOR
// swizzle, which keeps every 8-lane group of a ds_read_b128 (the unit the
// LDS serves per cycle) on 8 different 16-byte bank groups.
//
// The loads are issued from inline assembly so the compiler does not drain
// them at barriers; each wave waits for its own loads before the barrier
// that publishes a step's units.  A wave stalls at a load instruction until
// the CU's address unit accepts it (about 16 cycles per 1 KB instruction on
// gfx950), so only one wave per SIMD issues loads, and it issues them in two
// halves per step: the other wave of the SIMD keeps the matrix core busy
// meanwhile (measured: 5% faster than every wave issuing an eighth of the
// loads; eight issuing waves with the same split measured no better).  After
// each barrier the MFMAs of the previous step's last quarter run from
// registers while the new step's fragment reads are in flight.  The MFMA
// sequence of an output element: 16x16x32 bf16 steps over k = 0, 32, 64, ...
// ascending, accumulators from 0.
// ---------------------------------------------------------------------------
constexpr int kP_Threads = 512;
constexpr int kP_Tok = kTileTok;
constexpr int kP_W = 256;
constexpr int kP_BK = 64;
constexpr int kP_Rows = kP_W + kP_Tok;          // 512
constexpr int kP_Blocks = kP_Rows / 8;          // 64 blocks of 8 rows of kP_BK bf16 (128 B)
constexpr int kP_WBlocks = kP_W / 8;            // 32
#ifndef MOE_ISSUERS
#define MOE_ISSUERS 4
#endif
constexpr int kP_Issuers = MOE_ISSUERS;         // waves that issue the loads
constexpr int kP_Dma = kP_Blocks / kP_Issuers;  // loads per issuing thread per K step
constexpr int kP_WDma = kP_WBlocks / kP_Issuers;   // the first of them: weight blocks
constexpr int kP_GateUpF = kP_W / 2;            // 128
// A tile with at most 64 valid token rows needs 32 KB of weight rows and
// 8 KB of token rows per step: three such stages fit in the ring's space and
// keep the loads of two steps in flight.
constexpr int kP_DeepTok = 64;
constexpr int kP_DeepStageBytes = kP_WBlocks * 1024 + (kP_DeepTok / 8) * 1024;   // 40960
constexpr int kP_Unit = kP_WBlocks * 1024;     // 32 KB: one operand of one K step
constexpr int kP_Ring = 5;                      // units in the 160 KB ring
static_assert(kP_Unit == (kP_Tok / 8) * 1024, "token rows of a step fill one unit");
static_assert(kP_WDma == 8, "a weight unit is 8 loads per issuing thread");
static_assert(3 * kP_DeepStageBytes <= kP_Ring * kP_Unit, "three deep stages fit");

template <int MODE, bool DEEP>
__device__ __forceinline__ void expert_gemm_body(const GemmParams& P, unsigned char* smem) {
    const uint32_t lds0 =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
    const int wm = wave & 1;   // weight half: 128 rows (gate/up: 64 gate + 64 up)
    const int wt = wave >> 1;  // token quarter: 64 rows

    // fragment read of a 16-row group (two 8-row blocks): row lane&15,
    // 16-byte chunk kk*4 + lane>>4 for the kk-th 32-wide half of the stage
    const int fr = lane & 7;
    const int fblk = (lane >> 3) & 1;
    int frag_off[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        frag_off[kk] = fblk * 1024 + fr * 128 + (((kk * 4 + (lane >> 4)) ^ fr) << 4);
    // direct-to-LDS slot of this lane inside a block
    const int drow = lane >> 3;
    const int dchunk = (lane & 7) ^ drow;

    const int E = P.E;
    const int total_long = P.tile_start[E];
    const int total_m = total_long + P.tail[0];
    const int total = total_m * P.n_tiles;
    const int nblk = gridDim.x;
    const int slot = tile_slot();
    const int KT = P.K / kP_BK;

    // 16-row weight group mb (0..7) of this wave -> first 8-row block
    auto wgrp = [&](int mb) {
        if (MODE == MODE_GATE_UP)
            return (mb < 4) ? (wm * 8 + mb * 2) : (kP_WBlocks / 2 + wm * 8 + (mb - 4) * 2);
        return wm * 16 + mb * 2;
    };

    for (int base = 0; base < total; base += nblk) {
        const int lt = base + slot;
        if (lt >= total) break;

        const TileRef tr = tile_at(lt, total_m, total_long, P.n_tiles, E, P.tile_start, P.tail,
                                   P.offsets);
        const int e = tr.e, local = tr.local, nt = tr.nt;
        const int seg1 = P.offsets[e + 1];
        const int p0 = P.offsets[e] + local * kP_Tok;
        const int kt0 = 0, kt1 = KT;

        // Rows of the token tile that hold tokens of this expert (>= 1); the
        // rest is padding.  An 8-row token block with no valid row is not
        // loaded (its LDS rows keep stale data that only reaches dropped
        // results), and a wave whose 64 token rows are all padding skips its
        // MFMAs.  A valid row's MFMA sequence is the same either way.
        const int valid = seg1 - p0;
        const int ntb = (valid + 7) >> 3;                 // token blocks to load
        const bool active = wt * 64 < valid;              // uniform in the wave

        // source row of each of this thread's direct-to-LDS slots: slot i of
        // issuing wave w fills block i*kP_Issuers + w (weight blocks first)
        const int iw = wave % kP_Issuers;
        const uint16_t* src[kP_Dma];
#pragma unroll
        for (int i = 0; i < kP_Dma; ++i) {
            const int b = i * kP_Issuers + iw;
            const uint16_t* row;
            if (b < kP_WBlocks) {
                const int rr = b * 8 + drow;
                if (MODE == MODE_GATE_UP) {
                    const int f = min(nt * kP_GateUpF + (rr & (kP_GateUpF - 1)), P.N - 1);
                    row = ((rr < kP_GateUpF) ? P.w0 : P.w1) + ((size_t)e * P.N + f) * P.K;
                } else {
                    const int h = min(nt * kP_W + rr, P.N - 1);
                    row = P.w0 + ((size_t)e * P.N + h) * P.K;
                }
            } else {
                const int p = min(p0 + (b - kP_WBlocks) * 8 + drow, seg1 - 1);
                const int ar = (MODE == MODE_GATE_UP) ? P.perm[p] / P.top_k : p;
                row = P.act + (size_t)ar * P.K;
            }
            src[i] = row + dchunk * 8;
        }

        floatx4 acc[kMB][kNB];
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

        // previous tile: its stores drained, every wave done reading its stages
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        block_barrier();

        // LDS layout.  In a launch that only streams weights (DEEP), a tile
        // with at most 64 valid token rows ("deep") cycles through three 40 KB
        // stages (32 KB of weight rows, then its token blocks) with the loads
        // of two steps in flight.  Every other tile keeps a ring of five 32 KB
        // units: unit 2kt holds the weight rows of step kt, unit 2kt+1 its
        // token rows.  After the barrier that opens step kt the units of step
        // kt-1 are free: the token rows of step kt+1 are loaded into one at
        // once, the weight rows of step kt+2 into the other after the first
        // group of this step's MFMAs.  Weight rows, the operand with the least
        // reuse between workgroups (an expert's weight tile serves only its
        // own token tiles), so get about 1.5 steps to arrive, and an issuing
        // wave stalls on half as many loads at a time.  (Measured on gfx950
        // against two 64 KB stages loaded one step ahead: -4% on the large
        // layer's gate/up, -11% with 256 experts of 512 tokens, +1% with a
        // single expert; issuing both operands at the barrier was slower than
        // two stages.)  Either way a unit is refilled only after the barrier
        // that follows every wave's reads of it, and the MFMA sequence of an
        // output element is the same.
        const bool deep = DEEP && valid <= kP_DeepTok;
        auto w_off = [&](int kt) -> uint32_t {
            return deep ? (uint32_t)((kt % 3) * kP_DeepStageBytes)
                        : (uint32_t)(((2 * kt) % kP_Ring) * kP_Unit);
        };
        auto x_off = [&](int kt) -> uint32_t {
            return deep ? (uint32_t)((kt % 3) * kP_DeepStageBytes + kP_Unit)
                        : (uint32_t)(((2 * kt + 1) % kP_Ring) * kP_Unit);
        };
        auto issue_w = [&](int kt) {
            if (wave >= kP_Issuers) return;
            const uint32_t sb = lds0 + w_off(kt);
#pragma unroll
            for (int i = 0; i < kP_WDma; ++i)
                dma16(src[i] + (size_t)kt * kP_BK, sb + (uint32_t)((i * kP_Issuers + iw) * 1024));
        };
        auto issue_x = [&](int kt) {
            if (wave >= kP_Issuers) return;
            const uint32_t sb = lds0 + x_off(kt);
#pragma unroll
            for (int i = kP_WDma; i < kP_Dma; ++i) {
                const int bx = (i - kP_WDma) * kP_Issuers + iw;
                if (bx >= ntb) continue;
                dma16(src[i] + (size_t)kt * kP_BK, sb + (uint32_t)(bx * 1024));
            }
        };
        // loads per step of this thread in a deep tile: 8 weight blocks and
        // its token blocks below ntb (at most 8 in all)
        const int nload =
            wave < kP_Issuers ? kP_WDma + (ntb > iw ? 1 : 0) + (ntb > iw + 4 ? 1 : 0) : 0;
        if (deep) {
            for (int j = 0; j < 2; ++j)
                if (kt0 + j < kt1) { issue_w(kt0 + j); issue_x(kt0 + j); }
        } else {
            issue_w(kt0);
            issue_x(kt0);
            if (kt0 + 1 < kt1) issue_w(kt0 + 1);
        }

        bf16x8 fbP[kNB], faP[4];
        for (int kt = kt0; kt < kt1; ++kt) {
            // this step's loads landed.  A deep tile leaves the next step's
            // nload loads of this thread in flight, a ring tile the weight
            // rows of the next step, issued after this step's token rows
            // (loads complete in order).
            if (deep && kt + 1 < kt1 && nload == 8)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else if (deep && kt + 1 < kt1 && nload == 9)
                asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
            else if (deep && kt + 1 < kt1 && nload == 10)
                asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
            else if (!deep && kt + 1 < kt1)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            block_barrier();
            if (deep) {
                if (kt + 2 < kt1) { issue_w(kt + 2); issue_x(kt + 2); }
            } else if (kt + 1 < kt1) {
                issue_x(kt + 1);
            }
            // a ring tile's weight rows of step kt+2: issued after the first
            // group of this step's MFMAs (by a wave without MFMAs at once)
            const bool late_w = !deep && kt + 2 < kt1;
            if (!active) {
                if (late_w) issue_w(kt + 2);
                continue;
            }
            const unsigned char* sw = smem + w_off(kt);
            const unsigned char* sx = smem + x_off(kt);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 fb[kNB], fa[4];
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb)
                    fb[nb] = *reinterpret_cast<const bf16x8*>(sx + frag_off[kk] +
                                                              (wt * 8 + nb * 2) * 1024);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    fa[mb] = *reinterpret_cast<const bf16x8*>(sw + frag_off[kk] + wgrp(mb) * 1024);
                // second half of the previous 32-wide step (from registers)
                if (kk == 1 || kt > kt0) {
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int nb = 0; nb < kNB; ++nb)
                            acc[mb + 4][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                faP[mb], fbP[nb], acc[mb + 4][nb], 0, 0, 0);
                }
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    faP[mb] = *reinterpret_cast<const bf16x8*>(sw + frag_off[kk] +
                                                               wgrp(mb + 4) * 1024);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) fbP[nb] = fb[nb];
                if (kk == 0 && late_w) issue_w(kt + 2);
            }
        }
        if (kt1 > kt0 && active) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb)
                    acc[mb + 4][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        faP[mb], fbP[nb], acc[mb + 4][nb], 0, 0, 0);
        }

        // epilogue: lane holds weight rows 4*(lane>>4)+q of token column lane&15
        const int colq = 4 * (lane >> 4);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const int p = p0 + wt * 64 + nb * 16 + (lane & 15);
            if (p >= seg1) continue;
            if (MODE == MODE_GATE_UP) {
                uint16_t* hout = reinterpret_cast<uint16_t*>(P.out) + (size_t)p * P.N;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const int f = nt * kP_GateUpF + wm * 64 + mb * 16 + colq;
                    if (f >= P.N) continue;
                    uint32_t h[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        h[q] = f32_to_bf16_rne(silu_f(acc[mb][nb][q]) * acc[mb + 4][nb][q]);
                    uint2 pk;
                    pk.x = h[0] | (h[1] << 16);
                    pk.y = h[2] | (h[3] << 16);
                    *reinterpret_cast<uint2*>(hout + f) = pk;
                }
            } else {
                const int a = P.perm[p];
                float* yout = reinterpret_cast<float*>(P.out) + (size_t)a * P.N;
#pragma unroll
                for (int mb = 0; mb < kMB; ++mb) {
                    const int h = nt * kP_W + wm * 128 + mb * 16 + colq;
                    if (h >= P.N) continue;
                    *reinterpret_cast<floatx4*>(yout + h) = acc[mb][nb];
                }
            }
        }
    }
    // leave no load in flight
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One kernel per GEMM.  A gate/up launch whose tile list holds no long tile
// (every expert has at most 128 tokens: decode-sized batches) only streams
// expert weights, and runs the body that keeps two steps of loads in flight
// for its tiles of at most 64 rows.  Which body runs is decided from the tile
// list once per launch and changes the load pipeline only, never the MFMA
// sequence of an output element.  (Three stages for the short tails of a
// large batch, or for the down projection's short tiles, which run between
// long tiles, measured slower; so did deciding per tile inside one loop.)
template <int MODE>
__global__ __launch_bounds__(kP_Threads) void expert_gemm_pipe_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kP_Ring * kP_Unit];
    if (MODE == MODE_GATE_UP && P.tile_start[P.E] == 0)
        expert_gemm_body<MODE, MODE == MODE_GATE_UP>(P, smem);
    else
        expert_gemm_body<MODE, false>(P, smem);
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel.  The host picks it for calls of at most 32 tokens
// (so an expert rarely has more; any count is still handled, in chunks of
// NB*16 rows).  Such a launch only streams the active experts' weights, and
// the 256-row tiles above would leave most CUs idle (8 active experts x F/128
// output tiles).  Here a work item is one expert x 64 weight rows (gate/up:
// 32 gate + 32 up rows of the same features), so the same launch spreads over
// every CU.  4 waves; wave w multiplies 16 weight rows (gate/up: waves 0-1
// gate, 2-3 up) by the expert's token rows.  Its weight rows arrive as whole
// 128-byte lines, two K steps per pair of loads, four pairs in flight, and
// each pair passes through 2 KB of LDS into the fragment layout (against
// loads of 16 half lines straight into the fragment registers, one K step
// each: gate/up 0.367 -> 0.344 ms at 16 tokens on the large layer, 0.095 ->
// 0.085 ms at 7 on the mid layer, bit-identical; eight pairs in flight
// measured no faster).  The token fragments still come straight from
// global memory (cache hits).  A gate/up launch with fewer
// such items than two per CU (one token on the mid layer: 8 experts x 44
// items) takes items of 16 features instead, one gate and one up wave each:
// a CU streams about 25 GB/s whatever it runs, so the time is set by the CUs
// given the most bytes (mid, one token: 0.029 -> 0.025 ms; with more items the
// 4-wave blocks measured faster).  The list of experts it
// serves (0 < count <= max_count) is built in LDS from the offsets at kernel
// start, so no separate schedule launch is needed.
//
// The MFMA sequence of an output element is the one of the 256 x 256 kernel:
// v_mfma_f32_16x16x32_bf16, lane l holding row l%16 and K positions
// 32s + 8(l/16) .. +7 of step s on both operands, accumulators from 0, steps
// ascending, no split.  So the bits equal those of the tiled kernel.
//
// SPLIT (the load-dependent variant only): an expert's K steps are cut into
// variant_parts(count) parts, one work item each; a part's fp32 sums go to a
// workspace row of its own and variant_reduce_kernel adds the parts.  The
// summation order of an element then depends on its expert's token count:
// this mode is deliberately not batch-invariant.
// ---------------------------------------------------------------------------
constexpr int kS_MaxE = 512;
constexpr int kS_DownH = 64;           // output rows per down work item (4 waves)
// features per gate/up work item of a block of TH threads: half its waves
// hold gate rows, the other half up rows of the same features
constexpr int stream_gate_up_f(int TH) { return TH / kWave / 2 * 16; }
constexpr int kS_MaxTok = 32;          // invariant path: tokens per call for this kernel
constexpr int kS_Ring = 4;             // pairs of K steps in flight per wave
constexpr int kV_MaxTok = 32;          // variant: experts up to this count are split

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

// K parts of a split expert: the fewer tokens, the more parts
__device__ __forceinline__ int variant_parts(int m, int parts_max) {
    return min(parts_max, m <= 4 ? 4 : 2);
}

template <int MODE, int NB, bool SPLIT, int kS_Threads>
__global__ __launch_bounds__(kS_Threads) void expert_gemm_stream_kernel(GemmParams P) {
    constexpr int kHalf = kS_Threads / kWave / 2;   // gate/up: gate waves, then as many up waves
    constexpr int kS_GateUpF = stream_gate_up_f(kS_Threads);
    static_assert(MODE == MODE_GATE_UP || kS_Threads == 4 * kWave, "down: 4 waves of 16 rows");
    __shared__ int act_list[kS_MaxE];
    __shared__ int item_start[kS_MaxE + 1];    // SPLIT: first work item of a list entry
    __shared__ int row_start[kS_MaxE + 1];     // SPLIT: first workspace row of an entry
    __shared__ int wsum[3][kS_Threads / kWave];
    __shared__ floatx4 xch[kHalf][NB][kWave];  // up waves' accumulators, for the gate waves
    __shared__ bf16x8 wscr[kS_Threads / kWave][128];   // a wave's pair of weight steps

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int E = P.E;
    const int n_tiles = P.n_tiles;
    const int KS = P.K / 32;

    // the experts served, ascending, with (SPLIT) the prefix of their work
    // items (n_tiles x parts) and of their rows
    int n_act = 0, items_tot = 0, rows_tot = 0;
    for (int e0 = 0; e0 < E; e0 += kS_Threads) {
        const int e = e0 + tid;
        const int m = (e < E) ? P.offsets[e + 1] - P.offsets[e] : 0;
        const bool a = m > 0 && m <= P.max_count;
        const int c_items = a ? n_tiles * (SPLIT ? variant_parts(m, P.parts_max) : 1) : 0;
        const int c_rows = a ? m : 0;
        const int s_act = wave_incl_scan(a ? 1 : 0, lane);
        const int s_items = wave_incl_scan(c_items, lane);
        const int s_rows = wave_incl_scan(c_rows, lane);
        if (lane == kWave - 1) {
            wsum[0][wave] = s_act;
            wsum[1][wave] = s_items;
            wsum[2][wave] = s_rows;
        }
        __syncthreads();
        int o_act = n_act, o_items = items_tot, o_rows = rows_tot;
#pragma unroll
        for (int w = 0; w < kS_Threads / kWave; ++w) {
            if (w < wave) {
                o_act += wsum[0][w];
                o_items += wsum[1][w];
                o_rows += wsum[2][w];
            }
            n_act += wsum[0][w];
            items_tot += wsum[1][w];
            rows_tot += wsum[2][w];
        }
        if (a) {
            const int idx = o_act + s_act - 1;
            act_list[idx] = e;
            if (SPLIT) {
                item_start[idx] = o_items + s_items - c_items;
                row_start[idx] = o_rows + s_rows - c_rows;
            }
        }
        __syncthreads();
    }
    if (SPLIT && tid == 0) {
        item_start[n_act] = items_tot;
        row_start[n_act] = rows_tot;
        if (blockIdx.x == 0) P.nrows[0] = rows_tot;
    }
    __syncthreads();

    const int total = SPLIT ? items_tot : n_act * n_tiles;
    const int koff = (lane >> 4) * 8;          // this lane's K offset inside a step
    const int colq = 4 * (lane >> 4);          // epilogue: this lane's first output row
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int li, nt, part = 0, parts = 1;
        if (SPLIT) {
            int lo = 0, hi = n_act - 1;        // the list entry holding this item
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (item_start[mid] <= item) lo = mid; else hi = mid - 1;
            }
            li = lo;
            const int ee = act_list[li];
            parts = variant_parts(P.offsets[ee + 1] - P.offsets[ee], P.parts_max);
            const int r = item - item_start[li];
            nt = r / parts;
            part = r - nt * parts;
        } else {
            li = item / n_tiles;
            nt = item - li * n_tiles;
        }
        const int e = act_list[li];
        const int seg0 = P.offsets[e], seg1 = P.offsets[e + 1];
        const int ks_part = KS / parts;        // even (the host's choice of parts_max)
        const int s_begin = part * ks_part, s_end = s_begin + ks_part;

        // this wave's 16 weight rows, read as whole 128-byte lines: a pair of
        // K steps (64 k) is two loads, lane l taking rows l/8 and 8 + l/8 and
        // the 16-byte chunk (l%8) ^ (l/8) of each; the pair passes through
        // LDS (2 KB per wave) into the fragment layout of its two steps
        const uint16_t* pw[2];
        {
            const int r0 = (MODE == MODE_GATE_UP) ? nt * kS_GateUpF + (wave % kHalf) * 16
                                                  : nt * kS_DownH + wave * 16;
            const uint16_t* wb = (MODE == MODE_GATE_UP && wave >= kHalf) ? P.w1 : P.w0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int f = min(r0 + (lane >> 3) + 8 * h, P.N - 1);
                pw[h] = wb + ((size_t)e * P.N + f) * P.K + ((lane & 7) ^ (lane >> 3)) * 8;
            }
        }
        int rd_off[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = lane & 15, c = 4 * j + (lane >> 4);
            rd_off[j] = (r >> 3) * 64 + (r & 7) * 8 + (c ^ (r & 7));
        }
        bf16x8* const scr = wscr[wave];
        const int p_begin = s_begin / 2, p_end = s_end / 2;

        for (int tb = seg0; tb < seg1; tb += NB * 16) {
            const uint16_t* pb[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int p = min(tb + nb * 16 + (lane & 15), seg1 - 1);
                const int ar = (MODE == MODE_GATE_UP) ? P.perm[p] / P.top_k : p;
                pb[nb] = P.act + (size_t)ar * P.K + koff;
            }
            // a ring of kS_Ring pairs: slot u holds pair pp0 + u; after its MFMAs
            // it is refilled with pair pp0 + u + kS_Ring (the last pair again past
            // the end: a cache hit whose value is unused)
            bf16x8 wf[kS_Ring][2], rb[kS_Ring][2][NB];
#pragma unroll
            for (int u = 0; u < kS_Ring; ++u) {
                const int pr = min(p_begin + u, p_end - 1);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wf[u][h] = *reinterpret_cast<const bf16x8*>(pw[h] + (size_t)pr * 64);
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        rb[u][j][nb] =
                            *reinterpret_cast<const bf16x8*>(pb[nb] + (size_t)(2 * pr + j) * 32);
                __builtin_amdgcn_sched_barrier(0);
            }
            floatx4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int pp0 = p_begin; pp0 < p_end; pp0 += kS_Ring) {
#pragma unroll
                for (int u = 0; u < kS_Ring; ++u) {
                    if (pp0 + u < p_end) {
                        scr[lane] = wf[u][0];
                        scr[64 + lane] = wf[u][1];
                        const bf16x8 a0 = scr[rd_off[0]];
                        const bf16x8 a1 = scr[rd_off[1]];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, rb[u][0][nb],
                                                                               acc[nb], 0, 0, 0);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, rb[u][1][nb],
                                                                               acc[nb], 0, 0, 0);
                    }
                    const int pn = min(pp0 + u + kS_Ring, p_end - 1);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        wf[u][h] = *reinterpret_cast<const bf16x8*>(pw[h] + (size_t)pn * 64);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            rb[u][j][nb] = *reinterpret_cast<const bf16x8*>(
                                pb[nb] + (size_t)(2 * pn + j) * 32);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // epilogue: lane holds weight rows colq + q of token column lane&15
            if (SPLIT) {
                const int NW = (MODE == MODE_GATE_UP) ? 2 * P.N : P.N;
                const int col = (MODE == MODE_GATE_UP)
                                    ? (wave >= kHalf ? P.N : 0) + nt * kS_GateUpF +
                                          (wave % kHalf) * 16 + colq
                                    : nt * kS_DownH + wave * 16 + colq;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int p = tb + nb * 16 + (lane & 15);
                    if (p >= seg1) continue;
                    const int q = row_start[li] + (p - seg0);
                    *reinterpret_cast<floatx4*>(P.part + ((size_t)part * P.R + q) * NW + col) =
                        acc[nb];
                    if (nt == 0 && part == 0 && wave == 0 && lane < 16) {
                        P.rowmap[2 * q] = p;
                        P.rowmap[2 * q + 1] = parts;
                    }
                }
            } else if (MODE == MODE_GATE_UP) {
                if (wave >= kHalf) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) xch[wave - kHalf][nb][lane] = acc[nb];
                }
                __syncthreads();
                if (wave < kHalf) {
                    const int f = nt * kS_GateUpF + wave * 16 + colq;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int p = tb + nb * 16 + (lane & 15);
                        if (p >= seg1 || f >= P.N) continue;
                        const floatx4 up = xch[wave][nb][lane];
                        uint32_t h[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            h[q] = f32_to_bf16_rne(silu_f(acc[nb][q]) * up[q]);
                        uint2 pk;
                        pk.x = h[0] | (h[1] << 16);
                        pk.y = h[2] | (h[3] << 16);
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) +
                                                  (size_t)p * P.N + f) = pk;
                    }
                }
                __syncthreads();
            } else {
                const int h = nt * kS_DownH + wave * 16 + colq;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int p = tb + nb * 16 + (lane & 15);
                    if (p >= seg1 || h >= P.N) continue;
                    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(P.out) +
                                                (size_t)P.perm[p] * P.N + h) = acc[nb];
                }
            }
        }
    }
}

// Variant: add the K parts of every split row in ascending part order, then
// finish the row: act = bf16(silu(g) * u) (gate/up) or y (down).  One block
// per workspace row; rows past the count the streaming kernel recorded skip.
template <int MODE>
__global__ __launch_bounds__(256) void variant_reduce_kernel(GemmParams P) {
    const int r = blockIdx.x;
    if (r >= P.nrows[0]) return;
    const int p = P.rowmap[2 * r], parts = P.rowmap[2 * r + 1];
    const int N = P.N;
    const int NW = (MODE == MODE_GATE_UP) ? 2 * N : N;
    for (int c = threadIdx.x * 4; c < N; c += 256 * 4) {
        const float* base = P.part + (size_t)r * NW + c;
        const size_t plane = (size_t)P.R * NW;
        floatx4 a = *reinterpret_cast<const floatx4*>(base);
        for (int pp = 1; pp < parts; ++pp)
            a = a + *reinterpret_cast<const floatx4*>(base + pp * plane);
        if (MODE == MODE_GATE_UP) {
            floatx4 u = *reinterpret_cast<const floatx4*>(base + N);
            for (int pp = 1; pp < parts; ++pp)
                u = u + *reinterpret_cast<const floatx4*>(base + N + pp * plane);
            uint32_t h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16_rne(silu_f(a[q]) * u[q]);
            uint2 pk;
            pk.x = h[0] | (h[1] << 16);
            pk.y = h[2] | (h[3] << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + (size_t)p * N + c) = pk;
        } else {
            *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(P.out) +
                                        (size_t)P.perm[p] * N + c) = a;
        }
    }
}


template <int MODE, bool SPLIT, int TH>
hipError_t launch_stream_th(GemmParams P, int T, int max_rows, hipStream_t s) {
    P.n_tiles = (MODE == MODE_GATE_UP) ? P.N / stream_gate_up_f(TH) : P.N / kS_DownH;
    // at most min(E, T*k) experts are active: no more work items than that
    const long items = (long)std::min(P.E, T * P.top_k) * P.n_tiles * (SPLIT ? P.parts_max : 1);
    const int grid = (int)std::max(1L, std::min(items, (long)device_cu_count() * 8));
    if (max_rows <= 16)
        expert_gemm_stream_kernel<MODE, 1, SPLIT, TH><<<grid, TH, 0, s>>>(P);
    else
        expert_gemm_stream_kernel<MODE, 2, SPLIT, TH><<<grid, TH, 0, s>>>(P);
    return hipGetLastError();
}

// max_rows: the most token rows an expert served by this launch can have
// (16 or fewer: one 16-row chunk per pass; else 32-row chunks).
template <int MODE, bool SPLIT>
hipError_t launch_stream(const GemmParams& P, int T, int max_rows, hipStream_t s) {
    if constexpr (MODE == MODE_GATE_UP && !SPLIT) {
        // fewer 32-feature items than two per CU: 16-feature items
        const long items32 = (long)std::min(P.E, T * P.top_k) * (P.N / stream_gate_up_f(256));
        if (items32 < 2L * device_cu_count())
            return launch_stream_th<MODE, SPLIT, 128>(P, T, max_rows, s);
    }
    return launch_stream_th<MODE, SPLIT, 256>(P, T, max_rows, s);
}

// The token-tile list.  A tile whose valid rows fill at most half of it
// (<= 128 of 256) runs with half of its waves and takes about half as long.
// Such short tiles (the last tile of an expert, at most one per expert) are
// listed after every long tile, so that the 32 workgroups of an XCD, which
// start a round of tiles together, finish it together too and stay in step
// through K: that is what lets them share weight and token rows in L2.
// (Measured on the large layer: L2 hit rate 48% -> 62% and gate/up 3%
// faster.  The down projection keeps expert order: there a short tile moved
// away from its expert's long tiles no longer shares their weights, which
// cost more than the lockstep gained.)
//   tile_start[e] = number of long tiles of experts e' < e;
//   tail[0] = number of short tiles, tail[1..] = their experts, ascending.
// With reorder = 0 every tile is listed as long, in expert order.  Experts
// with at most skip_upto tokens get no tile (the load-dependent variant hands
// them to the split streaming kernel).  One block.
__device__ __forceinline__ void block_scan_512(int* sc, int e) {
    for (int d = 1; d < 512; d <<= 1) {
        const int v = (e >= d) ? sc[e - d] : 0;
        __syncthreads();
        sc[e] += v;
        __syncthreads();
    }
}

__global__ __launch_bounds__(512) void tile_schedule_kernel(int E, int skip_upto, int reorder,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ tile_start,
                                                            int32_t* __restrict__ tail) {
    __shared__ int sl[512], ss[512];
    const int e = threadIdx.x;
    int nlong = 0, nshort = 0;
    if (e < E) {
        int m = offsets[e + 1] - offsets[e];
        if (m <= skip_upto) m = 0;
        const int ntile = (m + kP_Tok - 1) / kP_Tok;
        const int rem = m % kP_Tok;
        nshort = (reorder && rem != 0 && rem <= kP_Tok / 2) ? 1 : 0;
        nlong = ntile - nshort;
    }
    sl[e] = nlong;
    ss[e] = nshort;
    __syncthreads();
    block_scan_512(sl, e);
    block_scan_512(ss, e);
    if (e < E) {
        tile_start[e] = sl[e] - nlong;
        if (nshort) tail[1 + ss[e] - 1] = e;
    }
    if (e == E - 1) {
        tile_start[E] = sl[e];
        tail[0] = ss[e];
    }
}

template <int MODE>
hipError_t launch_gemm(const GemmParams& P, hipStream_t s) {
    // one persistent workgroup per CU (its 160 KB LDS ring fills the CU),
    // rounded up to whole XCD rows
    const int cu = device_cu_count();
    const int b = (cu + kXcds - 1) / kXcds * kXcds;
    expert_gemm_pipe_kernel<MODE><<<b, kP_Threads, 0, s>>>(P);
    return hipGetLastError();
}

}  // namespace

// CU count of the current device, queried once per device and kept (a launch
// only reads the cache; the attribute query is not repeated per launch).
int device_cu_count() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDev) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
        return 256;
    if (dev >= 0 && dev < kMaxDev) cache[dev].store(cu, std::memory_order_relaxed);
    return cu;
}

size_t gemm_sched_ws_bytes(int E) { return (size_t)(2 * E + 2) * sizeof(int32_t); }

namespace {

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// Variant: K parts of the GEMM with reduction length K (a part's K steps
// stay even), and rows of the split experts (each has at most kV_MaxTok).
int variant_parts_max(int K) {
    const int ks = K / 32;
    return ks % 8 == 0 ? 4 : (ks % 4 == 0 ? 2 : 1);
}
int variant_rows(int T, int k, int E) {
    return (int)std::min((long)T * k, (long)kV_MaxTok * E);
}
size_t variant_gemm_ws(int T, int k, int E, int K, int NW) {
    const size_t R = (size_t)variant_rows(T, k, E);
    return up256((size_t)variant_parts_max(K) * R * NW * 4) + up256(R * 8) + 256;
}

// The variant's split streaming launch and its reduce, on workspace vws.
template <int MODE>
hipError_t launch_variant_small(GemmParams P, int T, int k, void* vws, hipStream_t s) {
    const int NW = (MODE == MODE_GATE_UP) ? 2 * P.N : P.N;
    P.max_count = kV_MaxTok;
    P.parts_max = variant_parts_max(P.K);
    P.R = variant_rows(T, k, P.E);
    unsigned char* w = static_cast<unsigned char*>(vws);
    P.part = reinterpret_cast<float*>(w);
    w += up256((size_t)P.parts_max * P.R * NW * 4);
    P.rowmap = reinterpret_cast<int32_t*>(w);
    w += up256((size_t)P.R * 8);
    P.nrows = reinterpret_cast<int32_t*>(w);
    hipError_t err = launch_stream<MODE, true>(P, T, std::min(T, kV_MaxTok), s);
    if (err != hipSuccess) return err;
    variant_reduce_kernel<MODE><<<P.R, 256, 0, s>>>(P);
    return hipGetLastError();
}

}  // namespace

size_t gemm_variant_ws_bytes(int T, int H, int E, int F, int k) {
    return std::max(variant_gemm_ws(T, k, E, H, 2 * F), variant_gemm_ws(T, k, E, F, H));
}

hipError_t launch_tile_schedule(int E, int skip_upto, int reorder, const int32_t* offsets,
                                int32_t* sched_ws, hipStream_t s) {
    tile_schedule_kernel<<<1, 512, 0, s>>>(E, skip_upto, reorder, offsets, sched_ws,
                                           sched_ws + E + 1);
    return hipGetLastError();
}

hipError_t launch_gate_up(int T, int H, int E, int F, int k, const uint16_t* x,
                          const int32_t* perm, const int32_t* offsets, const uint16_t* wg,
                          const uint16_t* wu, uint16_t* h_act, int32_t* sched_ws,
                          hipStream_t s, int variant, void* vws) {
    GemmParams P{};
    P.K = H; P.N = F; P.top_k = k; P.E = E;
    P.act = x; P.perm = perm; P.offsets = offsets; P.w0 = wg; P.w1 = wu; P.out = h_act;
    if (variant == 0 && T <= kS_MaxTok) {
        P.max_count = T * k;   // every active expert
        return launch_stream<MODE_GATE_UP, false>(P, T, T, s);
    }
    if (variant == 0 || T > kV_MaxTok) {
        // the tiled kernel: every expert, or (variant) those above kV_MaxTok
        int32_t* tile_start = sched_ws;
        int32_t* tail = sched_ws + E + 1;
        tile_schedule_kernel<<<1, 512, 0, s>>>(E, variant ? kV_MaxTok : 0, 1, offsets, tile_start,
                                               tail);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        GemmParams Q = P;
        Q.n_tiles = (F + kP_GateUpF - 1) / kP_GateUpF;
        Q.tile_start = tile_start;
        Q.tail = tail;
        err = launch_gemm<MODE_GATE_UP>(Q, s);
        if (err != hipSuccess || variant == 0) return err;
    }
    return launch_variant_small<MODE_GATE_UP>(P, T, k, vws, s);
}

hipError_t launch_down(int T, int H, int E, int F, int k, const uint16_t* h_act,
                       const int32_t* perm, const int32_t* offsets, const uint16_t* wd,
                       float* y, int variant, int32_t* sched_ws, hipStream_t s, void* vws) {
    GemmParams P{};
    P.K = F; P.N = H; P.top_k = k; P.E = E;
    P.act = h_act; P.perm = perm; P.offsets = offsets; P.w0 = wd; P.w1 = nullptr; P.out = y;
    if (variant == 0 && T <= kS_MaxTok) {
        P.max_count = T * k;
        return launch_stream<MODE_DOWN, false>(P, T, T, s);
    }
    if (variant == 0 || T > kV_MaxTok) {
        int32_t* tile_start = sched_ws;
        int32_t* tail = sched_ws + E + 1;
        tile_schedule_kernel<<<1, 512, 0, s>>>(E, variant ? kV_MaxTok : 0, 0, offsets, tile_start,
                                               tail);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        GemmParams Q = P;
        Q.n_tiles = (H + kP_W - 1) / kP_W;
        Q.tile_start = tile_start;
        Q.tail = tail;
        err = launch_gemm<MODE_DOWN>(Q, s);
        if (err != hipSuccess || variant == 0) return err;
    }
    return launch_variant_small<MODE_DOWN>(P, T, k, vws, s);
}

}  // namespace moe
