// moe_gemm_tiles.h -- pieces shared by the grouped expert GEMMs (bf16 and
// fp8): the direct-to-LDS load, the stage barrier, and the walk over the
// device-side tile list.
//
// Tile list: token tiles of 256 permuted rows per expert, in expert order;
// tile_start[e] counts the long tiles of experts before e, and the short last
// tiles (at most one per expert) listed in tail[1..tail[0]] come after every
// long tile.  Each token tile pairs with n_tiles output tiles.  Persistent
// workgroups walk the (token tile, output tile) pairs in rounds of gridDim.x;
// consecutive slots of one XCD get consecutive list entries, rastered in
// groups of kGroupM token tiles so an XCD's workgroups share weight and token
// rows in its L2.  Only the order in which tiles run depends on the per-expert
// counts, never the arithmetic of an output element.
#pragma once

#include "moe_device.h"

namespace moe {

#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
#ifndef MOE_XCD_REMAP
#define MOE_XCD_REMAP 1
#endif
constexpr int kGroupM = MOE_GROUP_M;     // token tiles per raster group
constexpr int kXcds = 8;
constexpr int kTileTok = 256;            // permuted token rows per tile

// One 16-byte direct-to-LDS load: lane l's 16 bytes land at M0 + 16*l.
// Issued from inline assembly so the compiler does not drain it at barriers;
// the caller waits for it (s_waitcnt vmcnt) before the barrier that
// publishes the stage.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory");
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// This workgroup's slot: XCD x (= blockIdx % 8) owns slots
// [x * per_xcd, (x + 1) * per_xcd).
__device__ __forceinline__ int tile_slot() {
    const int per_xcd = gridDim.x / kXcds;
    return MOE_XCD_REMAP ? (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds)
                         : (int)blockIdx.x;
}

struct TileRef {
    int e;       // expert
    int local;   // token tile inside the expert (x split parts in split-K)
    int nt;      // output tile
};

// List entry lt -> (expert, its token tile, output tile).
__device__ __forceinline__ TileRef tile_at(int lt, int total_m, int total_long, int n_tiles,
                                           int E, const int32_t* tile_start,
                                           const int32_t* tail, const int32_t* offsets) {
    const int gsize = kGroupM * n_tiles;
    const int g = lt / gsize;
    const int first_m = g * kGroupM;
    const int gm = min(total_m - first_m, kGroupM);
    const int r = lt - g * gsize;
    const int mt = first_m + r % gm;
    TileRef t;
    t.nt = r / gm;
    if (mt < total_long) {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
        }
        t.e = lo;
        t.local = mt - tile_start[lo];
    } else {
        // a short last tile: the list holds them after all long tiles
        t.e = tail[1 + mt - total_long];
        t.local = (offsets[t.e + 1] - offsets[t.e] - 1) / kTileTok;
    }
    return t;
}

}  // namespace moe
