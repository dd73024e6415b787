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
//   * one tile shape: 256 weight rows x 128 token rows, K staged 64 at a time;
//   * one instruction: v_mfma_f32_16x16x32_bf16, fp32 accumulators from 0;
//   * one K order: k = 0, 32, 64, ... ascending, no split;
// so an output element is the same sequence of MFMAs over the same operands
// whatever other rows share its tile.  Rows past an expert's segment are
// loaded from its last valid row and their results dropped.
//
// Operand roles: the weight rows are the MFMA "A" (M) side and the token rows
// the "B" (N) side, so each lane's four accumulators run along the output
// feature dimension and store as one contiguous vector.
//
// Scheduling: a persistent grid walks the device-side tile list; tile ids go
// to XCDs in contiguous blocks and are rastered in groups of 8 token tiles so
// the workgroups of one XCD share weight and token rows in its L2.  Only the
// launch work depends on the per-expert counts, never the arithmetic.
//
// The split-K variant (down projection only) exists to show what invariance
// costs and what breaking it does: experts with few tokens have their K range
// cut into 2..8 parts, each summed on its own and added with fp32 atomics.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 4 waves: 2 (weight halves) x 2 (token halves)
constexpr int kWaveW = kTileW / 2;       // 128 weight rows per wave
constexpr int kWaveT = kTileTok / 2;     // 64 token rows per wave
constexpr int kMB = kWaveW / 16;         // 8 MFMA blocks along weights
constexpr int kNB = kWaveT / 16;         // 4 MFMA blocks along tokens
constexpr int kRowBytes = kTileK * 2;    // 128 bytes per staged row
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
#ifndef MOE_XCD_REMAP
#define MOE_XCD_REMAP 1
#endif
#ifndef MOE_BLOCKS_PER_CU
#define MOE_BLOCKS_PER_CU 2
#endif
constexpr int kGroupM = MOE_GROUP_M;     // token tiles per raster group
constexpr int kXcds = 8;

constexpr int MODE_GATE_UP = 0;
constexpr int MODE_DOWN = 1;
constexpr int MODE_DOWN_SPLITK = 2;

// byte offset of 16-byte chunk c of staged row r (XOR swizzle: the 8 rows a
// quarter-wave reads at one chunk index land in 8 different chunk slots)
__device__ __forceinline__ int swz(int r, int c) {
    return r * kRowBytes + ((c ^ (r & 7)) << 4);
}

struct GemmParams {
    int K;            // reduction length: H (gate/up) or F (down)
    int N;            // output features: F (gate/up) or H (down)
    int n_tiles;      // output tiles along N
    int top_k;
    int E;
    const uint16_t* act;       // gate/up: x [T,H]; down: h_act [A,F]
    const int32_t* perm;
    const int32_t* offsets;    // [E+1]
    const int32_t* tile_start; // [E+1] prefix of token tiles (x split parts)
    const int32_t* split;      // [E] K parts per expert (split-K variant)
    const uint16_t* w0;        // w_gate or w_down [E, N, K]
    const uint16_t* w1;        // w_up (gate/up only)
    void* out;                 // h_act bf16 [A,F] or y fp32 [A,H]
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void expert_gemm_kernel(GemmParams P) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* sW = smem;                              // 256 rows x 128 B
    unsigned char* sT = smem + kTileW * kRowBytes;         // 128 rows x 128 B

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // weight half
    const int wt = wave >> 1;  // token half
    const int lrow = tid >> 3; // 0..31: staging row within a 32-row slab
    const int lchk = tid & 7;  // staging chunk (16 B) within the 128-B row

    const int E = P.E;
    const int total_m = P.tile_start[E];
    const int total = total_m * P.n_tiles;
    const int nblk = gridDim.x;
    const int per_xcd = nblk / kXcds;
    const int slot = MOE_XCD_REMAP ? (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds
                                   : (int)blockIdx.x;
    const int KT = P.K / kTileK;

    for (int base = 0; base < total; base += nblk) {
        const int lt = base + slot;
        if (lt >= total) break;

        // grouped raster: kGroupM token tiles x all n tiles per group
        const int gsize = kGroupM * P.n_tiles;
        const int g = lt / gsize;
        const int first_m = g * kGroupM;
        const int gm = min(total_m - first_m, kGroupM);
        const int r = lt - g * gsize;
        const int mt = first_m + r % gm;
        const int nt = r / gm;

        // expert of token tile mt: the largest e with tile_start[e] <= mt
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (P.tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int local = mt - P.tile_start[e];
        int parts = 1, part = 0, mloc = local;
        if (MODE == MODE_DOWN_SPLITK) {
            parts = P.split[e];
            mloc = local / parts;
            part = local - mloc * parts;
        }
        const int seg0 = P.offsets[e], seg1 = P.offsets[e + 1];
        const int p0 = seg0 + mloc * kTileTok;

        // K range of this tile (all of K unless split)
        int kt0 = 0, kt1 = KT;
        if (MODE == MODE_DOWN_SPLITK && parts > 1) {
            const int per = (KT + parts - 1) / parts;
            kt0 = min(KT, part * per);
            kt1 = min(KT, kt0 + per);
        }

        // --- staging addresses ----------------------------------------------
        // Thread (lrow, lchk) stages 16-byte chunk lchk of weight rows
        // lrow + 32*i (i < 8) and token rows lrow + 32*i (i < 4).  Row
        // offsets are 32-bit element offsets from per-tile uniform bases
        // (T*k*max(H,F) < 2^31 and one expert's N*K < 2^31).
        const uint16_t* wbase0;
        const uint16_t* wbase1;
        uint32_t woff[4];
        if (MODE == MODE_GATE_UP) {
            wbase0 = P.w0 + (size_t)e * P.N * P.K;   // gate rows
            wbase1 = P.w1 + (size_t)e * P.N * P.K;   // up rows
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = min(nt * kGateUpF + lrow + 32 * i, P.N - 1);
                woff[i] = (uint32_t)f * (uint32_t)P.K;
            }
        } else {
            wbase0 = P.w0 + (size_t)e * P.N * P.K;   // rows h of this tile, first half
            wbase1 = wbase0;                         // second half: same base, +128 rows
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = min(nt * kTileW + lrow + 32 * i, P.N - 1);
                woff[i] = (uint32_t)h * (uint32_t)P.K;
            }
        }
        uint32_t woff_hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (MODE == MODE_GATE_UP) {
                woff_hi[i] = woff[i];
            } else {
                const int h = min(nt * kTileW + kTileW / 2 + lrow + 32 * i, P.N - 1);
                woff_hi[i] = (uint32_t)h * (uint32_t)P.K;
            }
        }
        uint32_t toff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = min(p0 + lrow + 32 * i, seg1 - 1);
            const int row = (MODE == MODE_GATE_UP) ? P.perm[p] / P.top_k : p;
            toff[i] = (uint32_t)row * (uint32_t)P.K;
        }

        floatx4 acc[kMB][kNB];
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

        u32x4 rw[8], rt[4];
#define MOE_LOAD_STAGE(KT_)                                                              \
        {                                                                                \
            const uint32_t koff = (uint32_t)(KT_) * kTileK + lchk * 8;                   \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                \
                rw[i] = *reinterpret_cast<const u32x4*>(wbase0 + woff[i] + koff);        \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                \
                rw[4 + i] = *reinterpret_cast<const u32x4*>(wbase1 + woff_hi[i] + koff); \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                \
                rt[i] = *reinterpret_cast<const u32x4*>(P.act + toff[i] + koff);         \
        }

        if (kt0 < kt1) MOE_LOAD_STAGE(kt0);
        for (int kt = kt0; kt < kt1; ++kt) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<u32x4*>(sW + swz(lrow + 32 * i, lchk)) = rw[i];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(sT + swz(lrow + 32 * i, lchk)) = rt[i];
            __syncthreads();
            if (kt + 1 < kt1) MOE_LOAD_STAGE(kt + 1);

#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c = kk * 4 + (lane >> 4);
                bf16x8 fb[kNB];
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    const int tr0 = wt * kWaveT + nb * 16;
                    fb[nb] = *reinterpret_cast<const bf16x8*>(sT + swz(tr0 + (lane & 15), c));
                }
#pragma unroll
                for (int mb = 0; mb < kMB; ++mb) {
                    int wr0;
                    if (MODE == MODE_GATE_UP)
                        wr0 = (mb < 4) ? (wm * 64 + mb * 16) : (kGateUpF + wm * 64 + (mb - 4) * 16);
                    else
                        wr0 = wm * kWaveW + mb * 16;
                    const bf16x8 fa =
                        *reinterpret_cast<const bf16x8*>(sW + swz(wr0 + (lane & 15), c));
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            fa, fb[nb], acc[mb][nb], 0, 0, 0);
                }
            }
        }
#undef MOE_LOAD_STAGE

        // --- epilogue ------------------------------------------------------------
        // lane holds rows 4*(lane>>4)+q (weight side) of column lane&15 (token side)
        const int colq = 4 * (lane >> 4);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const int p = p0 + wt * kWaveT + nb * 16 + (lane & 15);
            if (p >= seg1) continue;
            if (MODE == MODE_GATE_UP) {
                uint16_t* hout = reinterpret_cast<uint16_t*>(P.out) + (size_t)p * P.N;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const int f = nt * kGateUpF + wm * 64 + mb * 16 + colq;
                    if (f >= P.N) continue;
                    uint32_t h[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float gv = acc[mb][nb][q];
                        const float uv = acc[mb + 4][nb][q];
                        h[q] = f32_to_bf16_rne(silu_f(gv) * uv);
                    }
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
                    const int h = nt * kTileW + wm * kWaveW + mb * 16 + colq;
                    if (h >= P.N) continue;
                    if (MODE == MODE_DOWN_SPLITK && parts > 1) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) unsafeAtomicAdd(yout + h + q, acc[mb][nb][q]);
                    } else {
                        *reinterpret_cast<floatx4*>(yout + h) = acc[mb][nb];
                    }
                }
            }
        }
    }
}

// K parts for the split-K variant: more parts the fewer tokens an expert has.
__device__ __forceinline__ int splitk_parts(int m) {
    return m <= 1 ? 8 : (m <= 4 ? 4 : (m <= 32 ? 2 : 1));
}

// tile_start[e] = sum over e' < e of parts(e') * ceil(M_e' / kTileTok); one block.
__global__ __launch_bounds__(512) void tile_schedule_kernel(int E, int variant,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ tile_start,
                                                            int32_t* __restrict__ split) {
    __shared__ int sc[512];
    const int e = threadIdx.x;
    int tiles = 0;
    if (e < E) {
        const int m = offsets[e + 1] - offsets[e];
        const int parts = (variant == 1) ? splitk_parts(m) : 1;
        tiles = parts * ((m + kTileTok - 1) / kTileTok);
        split[e] = parts;
    }
    sc[e] = tiles;
    __syncthreads();
    for (int d = 1; d < 512; d <<= 1) {
        const int v = (e >= d) ? sc[e - d] : 0;
        __syncthreads();
        sc[e] += v;
        __syncthreads();
    }
    if (e < E) tile_start[e] = sc[e] - tiles;
    if (e == E - 1) tile_start[E] = sc[e];
}

// Zero the y rows of experts whose down projection is split (they are summed
// with atomics).  One block per permuted row; rows of unsplit experts skip.
__global__ __launch_bounds__(256) void zero_split_rows_kernel(int A, int E, int H,
                                                              const int32_t* __restrict__ perm,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ split,
                                                              float* __restrict__ y) {
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
    }
    if (split[lo] <= 1) return;
    float4* row = reinterpret_cast<float4*>(y + (size_t)perm[p] * H);
    for (int i = threadIdx.x; i < H / 4; i += 256) row[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

constexpr size_t kSmemBytes = (size_t)(kTileW + kTileTok) * kRowBytes;  // 48 KB

int persistent_blocks() {
    int cu = device_cu_count();
    int b = cu * MOE_BLOCKS_PER_CU;
    b = (b + kXcds - 1) / kXcds * kXcds;
    return b < kXcds ? kXcds : b;
}

template <int MODE>
hipError_t launch_gemm(const GemmParams& P, hipStream_t s) {
    expert_gemm_kernel<MODE><<<persistent_blocks(), kThreads, kSmemBytes, s>>>(P);
    return hipGetLastError();
}

}  // namespace

int device_cu_count() {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
        return 256;
    return cu;
}

size_t gemm_sched_ws_bytes(int E) { return (size_t)(2 * E + 1) * sizeof(int32_t); }

hipError_t launch_gate_up(int T, int H, int E, int F, int k, const uint16_t* x,
                          const int32_t* perm, const int32_t* offsets, const uint16_t* wg,
                          const uint16_t* wu, uint16_t* h_act, int32_t* sched_ws,
                          hipStream_t s) {
    (void)T;
    int32_t* tile_start = sched_ws;
    int32_t* split = sched_ws + E + 1;
    tile_schedule_kernel<<<1, 512, 0, s>>>(E, 0, offsets, tile_start, split);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    GemmParams P;
    P.K = H; P.N = F; P.n_tiles = (F + kGateUpF - 1) / kGateUpF; P.top_k = k; P.E = E;
    P.act = x; P.perm = perm; P.offsets = offsets; P.tile_start = tile_start; P.split = split;
    P.w0 = wg; P.w1 = wu; P.out = h_act;
    return launch_gemm<MODE_GATE_UP>(P, s);
}

hipError_t launch_down(int T, int H, int E, int F, int k, const uint16_t* h_act,
                       const int32_t* perm, const int32_t* offsets, const uint16_t* wd,
                       float* y, int variant, int32_t* sched_ws, hipStream_t s) {
    int32_t* tile_start = sched_ws;
    int32_t* split = sched_ws + E + 1;
    tile_schedule_kernel<<<1, 512, 0, s>>>(E, variant, offsets, tile_start, split);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    GemmParams P;
    P.K = F; P.N = H; P.n_tiles = (H + kTileW - 1) / kTileW; P.top_k = k; P.E = E;
    P.act = h_act; P.perm = perm; P.offsets = offsets; P.tile_start = tile_start;
    P.split = split; P.w0 = wd; P.w1 = nullptr; P.out = y;
    if (variant == 1) {
        const int A = T * k;
        zero_split_rows_kernel<<<A, 256, 0, s>>>(A, E, H, perm, offsets, split, y);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        return launch_gemm<MODE_DOWN_SPLITK>(P, s);
    }
    return launch_gemm<MODE_DOWN>(P, s);
}

}  // namespace moe
