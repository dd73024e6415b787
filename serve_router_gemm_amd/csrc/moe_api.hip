// moe_api.hip -- the C ABI of libmoe (declared in include/moe.h): argument
// checks, workspace layout and the order of launches.  Every check runs on
// the host before anything is enqueued; nothing here allocates or
// synchronizes.  The only state is moe_forward_static's per-GPU scratch array
// and the device address of it that is looked up once per GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
// Route and permute in one call (moe_route.hip): for batches of at most 4
// tokens the select kernel also writes counts, offsets, perm and inv_perm
// (one launch fewer); larger batches run launch_route, then launch_permute.
// The outputs are those of the two calls.  (Declared here, its only caller,
// rather than among the shared declarations the expert GEMMs build against.)
hipError_t launch_route_permute(int T, int H, int E, int k, int score, int renorm,
                                const uint16_t* x, const uint16_t* wr, const float* bias,
                                int32_t* ids, float* w, float* part_ws, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* permute_ws, hipStream_t s);
// FP8 expert GEMMs of calls of at most kFp8StreamMaxTok tokens: the
// weight-streaming forms (same bits as the tiled kernel).  gate/up writes the
// bf16 act to act16 ([T*k, F]) and quantises it from there.
constexpr int kFp8StreamMaxTok = 32;
hipError_t launch_gate_up_fp8_stream(int T, int H, int E, int F, int k, const uint8_t* xq,
                                     const int8_t* xe, const int32_t* perm,
                                     const int32_t* offsets, const uint8_t* wgq,
                                     const int8_t* wge, const uint8_t* wuq, const int8_t* wue,
                                     uint8_t* aq, int8_t* ae, uint16_t* act16, hipStream_t s);
hipError_t launch_down_fp8_stream(int T, int H, int E, int F, int k, const uint8_t* aq,
                                  const int8_t* ae, const int32_t* perm, const int32_t* offsets,
                                  const uint8_t* wdq, const int8_t* wde, float* y, hipStream_t s);
}  // namespace moe

namespace {

using moe::launch_combine;

constexpr int kMaxE = 512;
constexpr int kMaxK = 16;
constexpr long kMaxA = 1L << 24;
constexpr long kMaxElems = (1L << 31) - 1;
constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dim(int v) { return (v >= 64 && v <= 65536) ? ((v % 64 == 0) ? 0 : MOE_ERR_UNSUPPORTED) : MOE_ERR_SHAPE; }

int check_tk(int T, int top_k) {
    if (T < 0 || top_k < 1 || top_k > kMaxK) return MOE_ERR_SHAPE;
    if ((long)T * top_k > kMaxA) return MOE_ERR_SHAPE;
    return 0;
}

int check_e(int E, int top_k) {
    if (E < 1 || E > kMaxE || top_k > E) return MOE_ERR_SHAPE;
    return 0;
}

int check_elems(int T, int top_k, int D) {
    return ((long)T * top_k * (long)D > kMaxElems) ? MOE_ERR_SHAPE : 0;
}

#define MOE_TRY(expr)          \
    do {                       \
        const int rc_ = (expr); \
        if (rc_ != 0) return rc_; \
    } while (0)

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Shape checks shared by the expert GEMM entry points.
int check_layer(int T, int H, int E, int F, int top_k) {
    MOE_TRY(check_tk(T, top_k));
    MOE_TRY(check_e(E, top_k));
    MOE_TRY(check_dim(H));
    MOE_TRY(check_dim(F));
    MOE_TRY(check_elems(T, top_k, H > F ? H : F));
    return 0;
}

// Workspace layout of moe_forward (every piece 256-byte aligned).
struct FwdLayout {
    size_t ids, w, counts, offsets, perm, inv_perm, route, permute, sched, hact, y, var, total;
};

FwdLayout fwd_layout(int T, int H, int E, int F, int top_k, int variant = 0) {
    const size_t A = (size_t)T * top_k;
    FwdLayout L;
    size_t o = 0;
    L.ids = o; o += up(A * 4);
    L.w = o; o += up(A * 4);
    L.counts = o; o += up((size_t)E * 4);
    L.offsets = o; o += up((size_t)(E + 1) * 4);
    L.perm = o; o += up(A * 4);
    L.inv_perm = o; o += up(A * 4);
    L.route = o; o += up(moe::route_ws_bytes(T, H, E));
    L.permute = o; o += up(moe::permute_ws_bytes((int)A, E));
    L.sched = o; o += up(moe::gemm_sched_ws_bytes(E));
    L.hact = o; o += up(A * (size_t)F * 2);
    L.y = o; o += up(A * (size_t)H * 4);
    L.var = o; o += variant ? up(moe::gemm_variant_ws_bytes(T, H, E, F, top_k)) : 0;
    L.total = o;
    return L;
}

// FP8 path: H and F in 128-wide blocks, a GEMM's K side at most 8192.
int check_layer_fp8(int T, int H, int E, int F, int top_k) {
    MOE_TRY(check_layer(T, H, E, F, top_k));
    if (H % moe::kFp8Block || F % moe::kFp8Block) return MOE_ERR_UNSUPPORTED;
    if (H > moe::kFp8MaxKB * moe::kFp8Block || F > moe::kFp8MaxKB * moe::kFp8Block)
        return MOE_ERR_SHAPE;
    return 0;
}

// gate/up FP8 workspace: the tile schedule, or for a weight-streaming call
// the bf16 act it quantises from (used when the caller passes no act_bf16).
size_t gate_up_fp8_ws(int T, int E, int F, int top_k) {
    const size_t sched = moe::gemm_sched_ws_bytes(E);
    if (T > moe::kFp8StreamMaxTok) return sched;
    return std::max(sched, up((size_t)T * top_k * F * 2));
}

// Workspace layout of moe_forward_fp8.
struct Fwd8Layout {
    size_t ids, w, counts, offsets, perm, inv_perm, route, permute, sched, xq, xe, aq, ae, y,
        abf, total;
};

Fwd8Layout fwd8_layout(int T, int H, int E, int F, int top_k) {
    const size_t A = (size_t)T * top_k;
    Fwd8Layout L;
    size_t o = 0;
    L.ids = o; o += up(A * 4);
    L.w = o; o += up(A * 4);
    L.counts = o; o += up((size_t)E * 4);
    L.offsets = o; o += up((size_t)(E + 1) * 4);
    L.perm = o; o += up(A * 4);
    L.inv_perm = o; o += up(A * 4);
    L.route = o; o += up(moe::route_ws_bytes(T, H, E));
    L.permute = o; o += up(moe::permute_ws_bytes((int)A, E));
    L.sched = o; o += up(moe::gemm_sched_ws_bytes(E));
    L.xq = o; o += up((size_t)T * H);
    L.xe = o; o += up((size_t)T * (H / moe::kFp8Block));
    L.aq = o; o += up(A * (size_t)F);
    L.ae = o; o += up(A * (size_t)(F / moe::kFp8Block));
    L.y = o; o += up(A * (size_t)H * 4);
    L.abf = o; o += T <= moe::kFp8StreamMaxTok ? up(A * (size_t)F * 2) : 0;
    L.total = o;
    return L;
}

size_t swiglu_ws(int T, int H, int E, int F, int top_k, int variant) {
    return up(moe::gemm_sched_ws_bytes(E)) + up((size_t)T * top_k * (size_t)F * 2) +
           (variant ? up(moe::gemm_variant_ws_bytes(T, H, E, F, top_k)) : 0);
}

size_t down_ws(int T, int H, int E, int F, int top_k, int variant) {
    return up(moe::gemm_sched_ws_bytes(E)) +
           (variant ? up(moe::gemm_variant_ws_bytes(T, H, E, F, top_k)) : 0);
}

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_vocab(int T, int V) {
    if (T < 0 || V < 1 || V > moe::kMaxVocab) return MOE_ERR_SHAPE;
    return ((long)T * (long)V > kMaxElems) ? MOE_ERR_SHAPE : 0;
}


template <typename P>
unsigned char* at(P* base, size_t off) {
    return reinterpret_cast<unsigned char*>(base) + off;
}

// Checks of moe_forward's arguments other than the workspace (shared with
// moe_forward_static).
int check_forward(int T, int H, int E, int F, int top_k, int score, int renormalize,
                  const uint16_t* x, const uint16_t* w_router, const float* bias,
                  const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                  const uint16_t* out, const int32_t* topk_ids, const float* topk_w,
                  int variant) {
    MOE_TRY(check_layer(T, H, E, F, top_k));
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_UNSUPPORTED;
    if (score == MOE_SCORE_SOFTMAX && bias) return MOE_ERR_UNSUPPORTED;
    if (variant != MOE_GEMM_INVARIANT && variant != MOE_GEMM_SPLITK_VARIANT)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !w_gate || !w_up || !w_down || !out) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
        !aligned16(w_down) || !aligned16(out) || (bias && !aligned16(bias)) ||
        (topk_ids && !aligned16(topk_ids)) || (topk_w && !aligned16(topk_w)))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

// The five steps of the layer on stream s, with the workspace laid out by
// fwd_layout (at least that many bytes at ws, 256-byte aligned).
int enqueue_forward(int T, int H, int E, int F, int top_k, int score, int renormalize,
                    const uint16_t* x, const uint16_t* w_router, const float* bias,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    uint16_t* out, int32_t* topk_ids, float* topk_w, int variant, void* ws,
                    hipStream_t s) {
    const FwdLayout L = fwd_layout(T, H, E, F, top_k, variant);
    int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(at(ws, L.ids));
    float* w = topk_w ? topk_w : reinterpret_cast<float*>(at(ws, L.w));
    int32_t* counts = reinterpret_cast<int32_t*>(at(ws, L.counts));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(ws, L.offsets));
    int32_t* perm = reinterpret_cast<int32_t*>(at(ws, L.perm));
    int32_t* inv = reinterpret_cast<int32_t*>(at(ws, L.inv_perm));
    float* part = reinterpret_cast<float*>(at(ws, L.route));
    int32_t* pws = reinterpret_cast<int32_t*>(at(ws, L.permute));
    int32_t* sched = reinterpret_cast<int32_t*>(at(ws, L.sched));
    uint16_t* hact = reinterpret_cast<uint16_t*>(at(ws, L.hact));
    float* y = reinterpret_cast<float*>(at(ws, L.y));
    MOE_TRY(hip_rc(moe::launch_route_permute(T, H, E, top_k, score, renormalize, x, w_router,
                                             bias, ids, w, part, counts, offsets, perm, inv, pws,
                                             s)));
    void* vws = variant ? at(ws, L.var) : nullptr;
    MOE_TRY(hip_rc(moe::launch_gate_up(T, H, E, F, top_k, x, perm, offsets, w_gate, w_up, hact,
                                       sched, s, variant, vws)));
    MOE_TRY(hip_rc(moe::launch_down(T, H, E, F, top_k, hact, perm, offsets, w_down, y, variant,
                                    sched, s, vws)));
    return hip_rc(launch_combine(T, H, top_k, y, w, out, s));
}

// ---------------------------------------------------------------------------
// Static scratch of moe_forward_static: the workspace of moe_forward for
// callers that cannot allocate device memory.  Every GPU the library runs on
// holds its own copy of this array until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the device address
// of the current GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept, and only that address is handed to kernels.
// Nothing in the forward path needs the scratch zeroed on entry (every piece
// is written before it is read), so the contents a previous call left are
// harmless; calls that overlap in time on one GPU share the array and race.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

int static_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_version(void) { return 10000; }

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of the supported range";
        case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case MOE_ERR_UNSUPPORTED: return "unsupported argument (H/F not a multiple of 64, or bad enum)";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
        case MOE_ERR_HIP: return "the HIP runtime reported a launch error";
        case MOE_ERR_SCRATCH:
            return "the call needs more than the library's static scratch (32 MiB per GPU)";
        default: return "unknown status";
    }
}

size_t moe_workspace_bytes(int op, int T, int H, int E, int F, int top_k, int variant) {
    if (variant != MOE_GEMM_INVARIANT && variant != MOE_GEMM_SPLITK_VARIANT) return 0;
    switch (op) {
        case MOE_OP_ROUTE:
            if (check_tk(T, top_k) || check_e(E, top_k) || check_dim(H) || check_elems(T, 1, H))
                return 0;
            return moe::route_ws_bytes(T, H, E);
        case MOE_OP_PERMUTE:
            if (check_tk(T, top_k) || check_e(E, top_k)) return 0;
            return moe::permute_ws_bytes(T * top_k, E);
        case MOE_OP_GATE_UP:
            if (check_layer(T, H, E, F, top_k)) return 0;
            return moe::gemm_sched_ws_bytes(E);
        case MOE_OP_DOWN:
            if (check_layer(T, H, E, F, top_k)) return 0;
            return down_ws(T, H, E, F, top_k, variant);
        case MOE_OP_GROUPED_SWIGLU:
            if (check_layer(T, H, E, F, top_k)) return 0;
            return swiglu_ws(T, H, E, F, top_k, variant);
        case MOE_OP_COMBINE:
            return 0;
        case MOE_OP_FORWARD:
            if (check_layer(T, H, E, F, top_k)) return 0;
            return fwd_layout(T, H, E, F, top_k, variant).total;
        case MOE_OP_GATE_UP_FP8:
            if (variant != MOE_GEMM_INVARIANT || check_layer_fp8(T, H, E, F, top_k)) return 0;
            return gate_up_fp8_ws(T, E, F, top_k);
        case MOE_OP_DOWN_FP8:
            if (variant != MOE_GEMM_INVARIANT || check_layer_fp8(T, H, E, F, top_k)) return 0;
            return moe::gemm_sched_ws_bytes(E);
        case MOE_OP_FORWARD_FP8:
            if (variant != MOE_GEMM_INVARIANT || check_layer_fp8(T, H, E, F, top_k)) return 0;
            return fwd8_layout(T, H, E, F, top_k).total;
        case MOE_OP_LOG_SOFTMAX:   // H is the vocabulary size V
            if (check_vocab(T, H)) return 0;
            return moe::log_softmax_ws_bytes(T, H);
        case MOE_OP_K3:            // H is the vocabulary size V
            if (check_vocab(T, H)) return 0;
            return moe::k3_ws_bytes(T, H);
        default:
            return 0;
    }
}

int moe_route(int T, int H, int E, int top_k, int score, int renormalize, const uint16_t* x,
              const uint16_t* w_router, const float* bias, int32_t* topk_ids, float* topk_w,
              void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_tk(T, top_k));
    MOE_TRY(check_e(E, top_k));
    MOE_TRY(check_dim(H));
    MOE_TRY(check_elems(T, 1, H));
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_UNSUPPORTED;
    if (score == MOE_SCORE_SOFTMAX && bias) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w || !ws) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_ids) || !aligned16(topk_w) ||
        !aligned16(ws) || (bias && !aligned16(bias)))
        return MOE_ERR_ALIGN;
    if (ws_bytes < moe::route_ws_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
    return hip_rc(moe::launch_route(T, H, E, top_k, score, renormalize, x, w_router, bias,
                                    topk_ids, topk_w, static_cast<float*>(ws), S(stream)));
}

int moe_permute(int T, int E, int top_k, const int32_t* topk_ids, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                size_t ws_bytes, void* stream) {
    MOE_TRY(check_tk(T, top_k));
    MOE_TRY(check_e(E, top_k));
    if (T == 0) return MOE_OK;
    const size_t need = moe::permute_ws_bytes(T * top_k, E);   // 0 for small batches
    if (!topk_ids || !expert_counts || !expert_offsets || !perm || !inv_perm || (need && !ws))
        return MOE_ERR_NULL;
    if (!aligned16(topk_ids) || !aligned16(expert_counts) || !aligned16(expert_offsets) ||
        !aligned16(perm) || !aligned16(inv_perm) || (ws && !aligned16(ws)))
        return MOE_ERR_ALIGN;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    return hip_rc(moe::launch_permute(T * top_k, E, topk_ids, expert_counts, expert_offsets, perm,
                                      inv_perm, static_cast<int32_t*>(ws), S(stream)));
}

int moe_expert_gate_up(int T, int H, int E, int F, int top_k, const uint16_t* x,
                       const int32_t* perm, const int32_t* expert_offsets, const uint16_t* w_gate,
                       const uint16_t* w_up, uint16_t* h_act, void* ws, size_t ws_bytes,
                       void* stream) {
    MOE_TRY(check_layer(T, H, E, F, top_k));
    if (T == 0) return MOE_OK;
    if (!x || !perm || !expert_offsets || !w_gate || !w_up || !h_act || !ws) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(perm) || !aligned16(expert_offsets) || !aligned16(w_gate) ||
        !aligned16(w_up) || !aligned16(h_act) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (ws_bytes < moe::gemm_sched_ws_bytes(E)) return MOE_ERR_WORKSPACE;
    return hip_rc(moe::launch_gate_up(T, H, E, F, top_k, x, perm, expert_offsets, w_gate, w_up,
                                      h_act, static_cast<int32_t*>(ws), S(stream)));
}

int moe_expert_down(int T, int H, int E, int F, int top_k, const uint16_t* h_act,
                    const int32_t* perm, const int32_t* expert_offsets, const uint16_t* w_down,
                    float* y, int variant, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer(T, H, E, F, top_k));
    if (variant != MOE_GEMM_INVARIANT && variant != MOE_GEMM_SPLITK_VARIANT)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!h_act || !perm || !expert_offsets || !w_down || !y || !ws) return MOE_ERR_NULL;
    if (!aligned16(h_act) || !aligned16(perm) || !aligned16(expert_offsets) ||
        !aligned16(w_down) || !aligned16(y) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (ws_bytes < down_ws(T, H, E, F, top_k, variant)) return MOE_ERR_WORKSPACE;
    return hip_rc(moe::launch_down(T, H, E, F, top_k, h_act, perm, expert_offsets, w_down, y,
                                   variant, static_cast<int32_t*>(ws), S(stream),
                                   at(ws, up(moe::gemm_sched_ws_bytes(E)))));
}

int moe_grouped_swiglu(int T, int H, int E, int F, int top_k, const uint16_t* x,
                       const int32_t* perm, const int32_t* expert_offsets, const uint16_t* w_gate,
                       const uint16_t* w_up, const uint16_t* w_down, float* y, int variant,
                       void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer(T, H, E, F, top_k));
    if (variant != MOE_GEMM_INVARIANT && variant != MOE_GEMM_SPLITK_VARIANT)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !perm || !expert_offsets || !w_gate || !w_up || !w_down || !y || !ws)
        return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(perm) || !aligned16(expert_offsets) || !aligned16(w_gate) ||
        !aligned16(w_up) || !aligned16(w_down) || !aligned16(y) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (ws_bytes < swiglu_ws(T, H, E, F, top_k, variant)) return MOE_ERR_WORKSPACE;
    int32_t* sched = static_cast<int32_t*>(ws);
    const size_t o_hact = up(moe::gemm_sched_ws_bytes(E));
    uint16_t* hact = reinterpret_cast<uint16_t*>(at(ws, o_hact));
    void* vws = variant ? at(ws, o_hact + up((size_t)T * top_k * (size_t)F * 2)) : nullptr;
    MOE_TRY(hip_rc(moe::launch_gate_up(T, H, E, F, top_k, x, perm, expert_offsets, w_gate, w_up,
                                       hact, sched, S(stream), variant, vws)));
    return hip_rc(moe::launch_down(T, H, E, F, top_k, hact, perm, expert_offsets, w_down, y,
                                   variant, sched, S(stream), vws));
}

int moe_combine(int T, int H, int top_k, const float* y, const float* topk_w, uint16_t* out,
                void* stream) {
    MOE_TRY(check_tk(T, top_k));
    MOE_TRY(check_dim(H));
    MOE_TRY(check_elems(T, top_k, H));
    if (T == 0) return MOE_OK;
    if (!y || !topk_w || !out) return MOE_ERR_NULL;
    if (!aligned16(y) || !aligned16(topk_w) || !aligned16(out)) return MOE_ERR_ALIGN;
    return hip_rc(launch_combine(T, H, top_k, y, topk_w, out, S(stream)));
}

int moe_forward(int T, int H, int E, int F, int top_k, int score, int renormalize,
                const uint16_t* x, const uint16_t* w_router, const float* bias,
                const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                uint16_t* out, int32_t* topk_ids, float* topk_w, int variant, void* ws,
                size_t ws_bytes, void* stream) {
    MOE_TRY(check_forward(T, H, E, F, top_k, score, renormalize, x, w_router, bias, w_gate, w_up,
                          w_down, out, topk_ids, topk_w, variant));
    if (T == 0) return MOE_OK;
    if (!ws) return MOE_ERR_NULL;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    if (ws_bytes < fwd_layout(T, H, E, F, top_k, variant).total) return MOE_ERR_WORKSPACE;
    return enqueue_forward(T, H, E, F, top_k, score, renormalize, x, w_router, bias, w_gate, w_up,
                           w_down, out, topk_ids, topk_w, variant, ws, S(stream));
}

int moe_forward_static(int T, int H, int E, int F, int top_k, int score, int renormalize,
                       const uint16_t* x, const uint16_t* w_router, const float* bias,
                       const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                       uint16_t* out, int32_t* topk_ids, float* topk_w, int variant,
                       void* stream) {
    MOE_TRY(check_forward(T, H, E, F, top_k, score, renormalize, x, w_router, bias, w_gate, w_up,
                          w_down, out, topk_ids, topk_w, variant));
    if (T == 0) return MOE_OK;
    if (fwd_layout(T, H, E, F, top_k, variant).total > kStaticScratchBytes)
        return MOE_ERR_SCRATCH;
    void* ws = nullptr;
    MOE_TRY(static_scratch(&ws));
    return enqueue_forward(T, H, E, F, top_k, score, renormalize, x, w_router, bias, w_gate, w_up,
                           w_down, out, topk_ids, topk_w, variant, ws, S(stream));
}

int moe_forward_replay(int T, int H, int E, int F, int top_k, int score, int renormalize,
                       const uint16_t* x, const uint16_t* w_router, const int32_t* topk_ids,
                       const float* topk_w, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, uint16_t* out, float* w_out, int variant,
                       void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer(T, H, E, F, top_k));
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_UNSUPPORTED;
    if (variant != MOE_GEMM_INVARIANT && variant != MOE_GEMM_SPLITK_VARIANT)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !topk_ids || !w_gate || !w_up || !w_down || !out || !ws) return MOE_ERR_NULL;
    if (!topk_w && !w_router) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(w_gate) || !aligned16(w_up) ||
        !aligned16(w_down) || !aligned16(out) || !aligned16(ws) ||
        (w_router && !aligned16(w_router)) || (topk_w && !aligned16(topk_w)) ||
        (w_out && !aligned16(w_out)))
        return MOE_ERR_ALIGN;
    const FwdLayout L = fwd_layout(T, H, E, F, top_k, variant);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    const int A = T * top_k;
    void* vws = variant ? at(ws, L.var) : nullptr;
    int32_t* counts = reinterpret_cast<int32_t*>(at(ws, L.counts));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(ws, L.offsets));
    int32_t* perm = reinterpret_cast<int32_t*>(at(ws, L.perm));
    int32_t* inv = reinterpret_cast<int32_t*>(at(ws, L.inv_perm));
    float* part = reinterpret_cast<float*>(at(ws, L.route));
    int32_t* pws = reinterpret_cast<int32_t*>(at(ws, L.permute));
    int32_t* sched = reinterpret_cast<int32_t*>(at(ws, L.sched));
    uint16_t* hact = reinterpret_cast<uint16_t*>(at(ws, L.hact));
    float* y = reinterpret_cast<float*>(at(ws, L.y));
    hipStream_t s = S(stream);
    const float* w = topk_w;
    if (!topk_w) {
        float* wr = w_out ? w_out : reinterpret_cast<float*>(at(ws, L.w));
        MOE_TRY(hip_rc(moe::launch_route(T, H, E, top_k, score, renormalize, x, w_router,
                                         nullptr, nullptr, wr, part, s, topk_ids)));
        w = wr;
    }
    MOE_TRY(hip_rc(moe::launch_permute(A, E, topk_ids, counts, offsets, perm, inv, pws, s)));
    MOE_TRY(hip_rc(moe::launch_gate_up(T, H, E, F, top_k, x, perm, offsets, w_gate, w_up, hact,
                                       sched, s, variant, vws)));
    MOE_TRY(hip_rc(moe::launch_down(T, H, E, F, top_k, hact, perm, offsets, w_down, y, variant,
                                    sched, s, vws)));
    MOE_TRY(hip_rc(moe::launch_zero_unplaced(A, H, inv, y, s)));
    return hip_rc(launch_combine(T, H, top_k, y, w, out, s));
}

int moe_topk_large(int Q, int N, int k, const float* scores, const int32_t* lengths,
                   int32_t* idx, float* vals, void* stream) {
    if (Q < 0 || N < 1 || N > (1 << 24) || k < 1 || k > moe::kMaxTopkLarge) return MOE_ERR_SHAPE;
    if ((long)Q * N > kMaxElems || (long)Q * k > kMaxElems) return MOE_ERR_SHAPE;
    if (Q == 0) return MOE_OK;
    if (!scores || !idx) return MOE_ERR_NULL;
    if (!aligned16(scores) || !aligned16(idx) || (lengths && !aligned16(lengths)) ||
        (vals && !aligned16(vals)))
        return MOE_ERR_ALIGN;
    return hip_rc(moe::launch_topk_large(Q, N, k, scores, lengths, idx, vals, S(stream)));
}

// ---------------------------------------------------------------------------
// decode-step measurement
// ---------------------------------------------------------------------------

int moe_lm_head_logits(int T, int H, int V, const uint16_t* h, const uint16_t* proj, float* z,
                       void* stream) {
    MOE_TRY(check_vocab(T, V));
    MOE_TRY(check_dim(H));
    if ((long)T * H > kMaxElems || (long)V * H > kMaxElems) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!h || !proj || !z) return MOE_ERR_NULL;
    if (!aligned16(h) || !aligned16(proj) || !aligned16(z)) return MOE_ERR_ALIGN;
    return hip_rc(moe::launch_lm_logits(T, H, V, h, proj, z, S(stream)));
}

int moe_log_softmax(int T, int V, const float* z, float* logp, void* ws, size_t ws_bytes,
                    void* stream) {
    MOE_TRY(check_vocab(T, V));
    if (T == 0) return MOE_OK;
    if (!z || !logp || !ws) return MOE_ERR_NULL;
    if (!aligned16(z) || !aligned16(logp) || !aligned16(ws)) return MOE_ERR_ALIGN;
    if (ws_bytes < moe::log_softmax_ws_bytes(T, V)) return MOE_ERR_WORKSPACE;
    return hip_rc(moe::launch_log_softmax(T, V, z, logp, ws, S(stream)));
}

int moe_k3(int T, int V, const float* logp_ref, const float* logp_test, double* k3_mean,
           double* k3_greedy, int32_t* greedy, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_vocab(T, V));
    if (T == 0) return MOE_OK;
    if (!logp_ref || !logp_test || !k3_mean || !k3_greedy || !greedy || !ws) return MOE_ERR_NULL;
    if (!aligned16(logp_ref) || !aligned16(logp_test) || !aligned16(k3_mean) ||
        !aligned16(k3_greedy) || !aligned16(greedy) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (ws_bytes < moe::k3_ws_bytes(T, V)) return MOE_ERR_WORKSPACE;
    return hip_rc(moe::launch_k3(T, V, logp_ref, logp_test, k3_mean, k3_greedy, greedy, ws,
                                 S(stream)));
}

// ---------------------------------------------------------------------------
// FP8 rollout path
// ---------------------------------------------------------------------------

int moe_quantize_fp8(int R, int K, int block_rows, const uint16_t* src, uint8_t* q,
                     int8_t* exps, void* stream) {
    if (R < 0 || block_rows < 1 || K < moe::kFp8Block || K > 65536) return MOE_ERR_SHAPE;
    if (K % moe::kFp8Block || R % block_rows) return MOE_ERR_SHAPE;
    if ((long)R * K > (1L << 40)) return MOE_ERR_SHAPE;   // 64-bit offsets inside
    if (R == 0) return MOE_OK;
    if (!src || !q || !exps) return MOE_ERR_NULL;
    if (!aligned16(src) || !aligned16(q) || !aligned16(exps)) return MOE_ERR_ALIGN;
    return hip_rc(moe::launch_quantize_fp8(R, K, block_rows, src, q, exps, S(stream)));
}

int moe_expert_gate_up_fp8(int T, int H, int E, int F, int top_k, const uint8_t* xq,
                           const int8_t* xe, const int32_t* perm, const int32_t* expert_offsets,
                           const uint8_t* wg_q, const int8_t* wg_e, const uint8_t* wu_q,
                           const int8_t* wu_e, uint8_t* act_q, int8_t* act_e, uint16_t* act_bf16,
                           void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer_fp8(T, H, E, F, top_k));
    if (T == 0) return MOE_OK;
    if (!xq || !xe || !perm || !expert_offsets || !wg_q || !wg_e || !wu_q || !wu_e || !act_q ||
        !act_e || !ws)
        return MOE_ERR_NULL;
    if (!aligned16(xq) || !aligned16(xe) || !aligned16(perm) || !aligned16(expert_offsets) ||
        !aligned16(wg_q) || !aligned16(wg_e) || !aligned16(wu_q) || !aligned16(wu_e) ||
        !aligned16(act_q) || !aligned16(act_e) || !aligned16(ws) ||
        (act_bf16 && !aligned16(act_bf16)))
        return MOE_ERR_ALIGN;
    if (ws_bytes < gate_up_fp8_ws(T, E, F, top_k)) return MOE_ERR_WORKSPACE;
    if (T <= moe::kFp8StreamMaxTok)
        return hip_rc(moe::launch_gate_up_fp8_stream(
            T, H, E, F, top_k, xq, xe, perm, expert_offsets, wg_q, wg_e, wu_q, wu_e, act_q, act_e,
            act_bf16 ? act_bf16 : static_cast<uint16_t*>(ws), S(stream)));
    return hip_rc(moe::launch_gate_up_fp8(T, H, E, F, top_k, xq, xe, perm, expert_offsets, wg_q,
                                          wg_e, wu_q, wu_e, act_q, act_e, act_bf16,
                                          static_cast<int32_t*>(ws), S(stream)));
}

int moe_expert_down_fp8(int T, int H, int E, int F, int top_k, const uint8_t* act_q,
                        const int8_t* act_e, const int32_t* perm, const int32_t* expert_offsets,
                        const uint8_t* wd_q, const int8_t* wd_e, float* y, void* ws,
                        size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer_fp8(T, H, E, F, top_k));
    if (T == 0) return MOE_OK;
    if (!act_q || !act_e || !perm || !expert_offsets || !wd_q || !wd_e || !y || !ws)
        return MOE_ERR_NULL;
    if (!aligned16(act_q) || !aligned16(act_e) || !aligned16(perm) ||
        !aligned16(expert_offsets) || !aligned16(wd_q) || !aligned16(wd_e) || !aligned16(y) ||
        !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (ws_bytes < moe::gemm_sched_ws_bytes(E)) return MOE_ERR_WORKSPACE;
    if (T <= moe::kFp8StreamMaxTok)
        return hip_rc(moe::launch_down_fp8_stream(T, H, E, F, top_k, act_q, act_e, perm,
                                                  expert_offsets, wd_q, wd_e, y, S(stream)));
    return hip_rc(moe::launch_down_fp8(T, H, E, F, top_k, act_q, act_e, perm, expert_offsets,
                                       wd_q, wd_e, y, static_cast<int32_t*>(ws), S(stream)));
}

int moe_forward_fp8(int T, int H, int E, int F, int top_k, int score, int renormalize,
                    const uint16_t* x, const uint16_t* w_router, const float* bias,
                    const uint8_t* wg_q, const int8_t* wg_e, const uint8_t* wu_q,
                    const int8_t* wu_e, const uint8_t* wd_q, const int8_t* wd_e, uint16_t* out,
                    int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer_fp8(T, H, E, F, top_k));
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_UNSUPPORTED;
    if (score == MOE_SCORE_SOFTMAX && bias) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !wg_q || !wg_e || !wu_q || !wu_e || !wd_q || !wd_e || !out || !ws)
        return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(wg_q) || !aligned16(wg_e) ||
        !aligned16(wu_q) || !aligned16(wu_e) || !aligned16(wd_q) || !aligned16(wd_e) ||
        !aligned16(out) || !aligned16(ws) || (bias && !aligned16(bias)) ||
        (topk_ids && !aligned16(topk_ids)) || (topk_w && !aligned16(topk_w)))
        return MOE_ERR_ALIGN;
    const Fwd8Layout L = fwd8_layout(T, H, E, F, top_k);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(at(ws, L.ids));
    float* w = topk_w ? topk_w : reinterpret_cast<float*>(at(ws, L.w));
    int32_t* counts = reinterpret_cast<int32_t*>(at(ws, L.counts));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(ws, L.offsets));
    int32_t* perm = reinterpret_cast<int32_t*>(at(ws, L.perm));
    int32_t* inv = reinterpret_cast<int32_t*>(at(ws, L.inv_perm));
    float* part = reinterpret_cast<float*>(at(ws, L.route));
    int32_t* pws = reinterpret_cast<int32_t*>(at(ws, L.permute));
    int32_t* sched = reinterpret_cast<int32_t*>(at(ws, L.sched));
    uint8_t* xq = reinterpret_cast<uint8_t*>(at(ws, L.xq));
    int8_t* xe = reinterpret_cast<int8_t*>(at(ws, L.xe));
    uint8_t* aq = reinterpret_cast<uint8_t*>(at(ws, L.aq));
    int8_t* ae = reinterpret_cast<int8_t*>(at(ws, L.ae));
    float* y = reinterpret_cast<float*>(at(ws, L.y));
    hipStream_t s = S(stream);
    MOE_TRY(hip_rc(moe::launch_route_permute(T, H, E, top_k, score, renormalize, x, w_router,
                                             bias, ids, w, part, counts, offsets, perm, inv, pws,
                                             s)));
    MOE_TRY(hip_rc(moe::launch_quantize_fp8(T, H, 1, x, xq, xe, s)));
    if (T <= moe::kFp8StreamMaxTok) {
        uint16_t* abf = reinterpret_cast<uint16_t*>(at(ws, L.abf));
        MOE_TRY(hip_rc(moe::launch_gate_up_fp8_stream(T, H, E, F, top_k, xq, xe, perm, offsets,
                                                      wg_q, wg_e, wu_q, wu_e, aq, ae, abf, s)));
        MOE_TRY(hip_rc(moe::launch_down_fp8_stream(T, H, E, F, top_k, aq, ae, perm, offsets,
                                                   wd_q, wd_e, y, s)));
    } else {
        MOE_TRY(hip_rc(moe::launch_gate_up_fp8(T, H, E, F, top_k, xq, xe, perm, offsets, wg_q,
                                               wg_e, wu_q, wu_e, aq, ae, nullptr, sched, s)));
        MOE_TRY(hip_rc(moe::launch_down_fp8(T, H, E, F, top_k, aq, ae, perm, offsets, wd_q,
                                            wd_e, y, sched, s)));
    }
    return hip_rc(launch_combine(T, H, top_k, y, w, out, s));
}

}  // extern "C"
