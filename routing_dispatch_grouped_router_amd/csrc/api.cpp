// C ABI of the routed MoE block (declarations and contracts in include/moe.h).
// Host-side only: validates arguments, carves the caller's workspace and
// enqueues the gfx950 kernels on the caller's stream.  Nothing here allocates
// device memory, copies to the host or synchronises, except moe_kernel_times
// and the host-synchronising comparison path moe_forward_host_sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
    size_t hist, base, psum, ppart, rwt, h, h_scale, sync, route_end, gemm_end;
    size_t idx, gate, counts, offsets, pos, row_token, xe, xe_scale, xst, ye, ab, total;
};

size_t act_bytes(int act) { return act == MOE_F32 ? 4 : (act == MOE_BF16 ? 2 : 1); }

// bf16 experts run both projections in one launch when each contraction has
// at least two 64-wide K-tiles (the fused kernel streams a tile's first two
// K-tiles ahead)
bool use_ffn(const moe_problem& p) {
    return p.act_dtype == MOE_BF16 && p.d_model >= 128 && p.d_hidden >= 128;
}

// moe_forward's fused bf16 FFN reads each expert-major row from x through
// row_token, so that forward writes no dispatched copy xe
bool forward_gathers(const moe_problem& p) { return use_ffn(p) && !(p.flags & MOE_IDENTITY_EXPERTS); }

// MOE_KEEP_GATE_UP: moe_forward's GEMM1 (the fused bf16 FFN's, or the MXFP8
// one) also stores its pre-activations a | b as bf16, and moe_backward's chain
// reads them instead of recomputing xe W1
bool keeps_gate_up(const moe_problem& p) { return (p.flags & MOE_KEEP_GATE_UP) != 0; }

// moe_forward of an MXFP8 block with d_model >= 256 quantises each token row
// once (codes [T][d], per-token scales) and GEMM1 reads the code rows through
// row_token; only the scales are laid out per expert-major row.  (GEMM1's row
// tables run one tile ahead, which needs at least two 128-wide K-tiles.)
bool forward_quantises_tokens(const moe_problem& p) { return p.act_dtype == MOE_MXFP8 && p.d_model >= 256; }

Layout layout(const moe_problem& p) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t T = p.T, E = p.n_experts, k = p.top_k, d = p.d_model, H = p.d_hidden;
    const size_t R = T * k, nblk = route_blocks(p.T);
    const bool mx = p.act_dtype == MOE_MXFP8;
    L.hist = take(nblk * E * 4);
    L.base = take(nblk * E * 4);
    L.psum = take(nblk * E * 4);
    L.ppart = take(nblk * route_lanes(p.n_experts) * E * 4);
    L.rwt = take(p.act_dtype != MOE_F32 && !(p.flags & MOE_LOGITS_GIVEN) ? E * d * 2 : 0);   // router W^T
    L.route_end = off;
    L.h = take(R * H * act_bytes(p.act_dtype));
    L.h_scale = take(mx ? R * H / 32 : 0);
    L.sync = take(use_ffn(p) ? (size_t)ffn_sync_ints((int)R, (int)E) * 4 : 0);   // fused FFN counters
    L.gemm_end = off;
    L.idx = take(R * 4);
    L.gate = take(R * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.pos = take(R * 4);
    L.row_token = take(R * 4);
    const bool tok = forward_quantises_tokens(p);
    L.xe = take(forward_gathers(p) ? 0 : (tok ? T : R) * d * act_bytes(p.act_dtype));   // MXFP8: codes per token
    L.xe_scale = take(mx ? R * d / 32 : 0);
    L.xst = take(tok ? T * d / 32 : 0);   // per-token scale dwords [T][d/128]
    L.ye = take(R * d * (p.act_dtype == MOE_F32 ? 4 : 2));
    L.ab = take(keeps_gate_up(p) ? R * 2 * H * 2 : 0);   // a | b [R][2H] bf16, packed column order
    L.total = off;
    return L;
}

struct Packed {
    size_t w1, w2, s1, s2, total;
};

Packed packed_layout(const moe_problem& p) {
    Packed P{};
    const size_t E = p.n_experts, d = p.d_model, H = p.d_hidden, b = act_bytes(p.act_dtype);
    const bool mx = p.act_dtype == MOE_MXFP8;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    P.w1 = take(E * 2 * H * d * b);
    P.w2 = take(E * d * H * b);
    P.s1 = take(mx ? E * 2 * H * d / 32 : 0);
    P.s2 = take(mx ? E * d * H / 32 : 0);
    P.total = off;
    return P;
}

// Backward workspace: a | b (then da | db) [R][2H], dye (then dxe) [R][d],
// dh [R][H], dsel [T][k] (router gradient at the selected experts); for the
// learned router W_r^T [E][d], the router gradient per routed row and the
// per-tile partials of dW_r; for MXFP8 blocks the dequantised xe [R][d] and h
// [R][H] (bfloat16).
struct BwdLayout {
    size_t ab, dye, dh, dsel, wrt, srow, rpart, xe16, h16, sync, total;
};

// The backward runs in the activation type, bfloat16 for MXFP8 blocks (their
// saved activations are dequantised first).
int bwd_act(int act) { return act == MOE_MXFP8 ? MOE_BF16 : act; }

// bf16 backward data-gradient GEMMs (dh, da | db, dxe) as one fused launch when
// every phase has at least four 32-wide K-tiles
bool use_bwd_chain(const moe_problem& p) {
    return bwd_act(p.act_dtype) == MOE_BF16 && p.d_model >= 128 && p.d_hidden >= 128;
}

BwdLayout bwd_layout(const moe_problem& p) {
    BwdLayout B{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const int ba = bwd_act(p.act_dtype);
    const size_t R = (size_t)p.T * p.top_k, d = p.d_model, H = p.d_hidden, b = act_bytes(ba);
    B.ab = take(R * 2 * H * b);
    B.dye = take(R * d * b);
    B.dh = take(R * H * b);
    B.dsel = take((size_t)p.T * p.top_k * 4);
    const bool learned = !(p.flags & MOE_LOGITS_GIVEN);
    B.wrt = take(learned ? (size_t)p.n_experts * d * b : 0);
    B.srow = take(learned ? R * 4 : 0);
    B.rpart = take(learned ? router_wgrad_part_bytes((int)R, p.n_experts, p.d_model) : 0);
    const bool mx = p.act_dtype == MOE_MXFP8;
    B.xe16 = take(mx || forward_gathers(p) ? R * d * 2 : 0);   // xe dequantised, or gathered again from x
    B.h16 = take(mx ? R * H * 2 : 0);
    B.sync = take(use_bwd_chain(p) ? (size_t)fused_sync_ints((int)R, p.n_experts, 3) * 4 : 0);
    B.total = off;
    return B;
}

// Backward weight cache: W1T [E][d][2H], W_down [E][H][d] and, for MXFP8
// blocks, the packed W1 [E][2H][d] the gate/up recompute multiplies with; in
// the backward's activation type (MXFP8: bfloat16 of the quantised values).
struct BwdPacked {
    size_t w1t, wd, w1, total;
};

BwdPacked bwd_packed_layout(const moe_problem& p) {
    BwdPacked P{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t E = p.n_experts, d = p.d_model, H = p.d_hidden, b = act_bytes(bwd_act(p.act_dtype));
    P.w1t = take(E * d * 2 * H * b);
    P.wd = take(E * H * d * b);
    P.w1 = take(p.act_dtype == MOE_MXFP8 ? E * 2 * H * d * b : 0);
    P.total = off;
    return P;
}

int32_t check_problem(const moe_problem* p) {
    if (p == nullptr) return MOE_ERR_NULL;
    if (p->act_dtype != MOE_F32 && p->act_dtype != MOE_BF16 && p->act_dtype != MOE_MXFP8)
        return MOE_ERR_DTYPE;
    if (p->flags & ~(MOE_LOGITS_GIVEN | MOE_IDENTITY_EXPERTS | MOE_KEEP_GATE_UP)) return MOE_ERR_DTYPE;
    if ((p->flags & MOE_IDENTITY_EXPERTS) && p->act_dtype == MOE_MXFP8) return MOE_ERR_DTYPE;
    // a | b are kept by the fused bf16 FFN (bf16 with d_model, d_hidden >= 128) and the MXFP8 GEMM1
    if ((p->flags & MOE_KEEP_GATE_UP) &&
        (p->act_dtype == MOE_F32 || (p->flags & MOE_IDENTITY_EXPERTS) ||
         (p->act_dtype == MOE_BF16 && (p->d_model < 128 || p->d_hidden < 128))))
        return MOE_ERR_DTYPE;
    if (p->T < 1 || p->n_experts < 1 || p->n_experts > kMaxExperts || p->top_k < 1 ||
        p->top_k > std::min(p->n_experts, kMaxTopK) || p->d_model < 1 || p->d_hidden < 1)
        return MOE_ERR_SHAPE;
    const int mult = p->act_dtype == MOE_MXFP8 ? 128 : 64;
    if (p->d_model % mult || p->d_hidden % mult) return MOE_ERR_SHAPE;
    // row indices are int32 and element offsets of one row-block must stay in range
    const long long R = (long long)p->T * p->top_k;
    if (R > INT_MAX / 2 || (long long)p->d_model > INT_MAX / 8 || (long long)p->d_hidden > INT_MAX / 8)
        return MOE_ERR_SHAPE;
    // the pipelined GEMMs address an activation buffer, and one expert's packed
    // weights, with 32-bit byte offsets
    const long long eb = p->act_dtype == MOE_F32 ? 4 : (p->act_dtype == MOE_BF16 ? 2 : 1);
    const long long wide = std::max<long long>(p->d_model, p->d_hidden);
    if (R * wide * eb >= (1LL << 32) || 2LL * p->d_hidden * p->d_model * eb >= (1LL << 32)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int32_t launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

// ------------------------------------------------------------------ profiling (moe_forward only)
// Events are recorded on the forward's own stream before the first kernel and
// after each kernel.  Up to kMaxCalls consecutive calls keep their own event
// sets, so the per-stage durations of a whole timed loop can be averaged
// without synchronising inside it.
constexpr int kMaxStages = 10;
constexpr int kMaxCalls = 128;
struct Profiler {
    bool enabled = false;
    int calls = 0;          // profiled calls since enabling
    int n = 0;              // stages recorded in the current call
    int stages = 0;         // stages of a complete call
    hipEvent_t ev[kMaxCalls][kMaxStages + 1] = {};
    const char* names[kMaxStages] = {};
    int device = -1;
} g_prof;

int32_t prof_begin(hipStream_t s) {
    if (!g_prof.enabled) return MOE_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
    if (g_prof.device != dev) {
        for (auto& row : g_prof.ev)
            for (auto& e : row) {
                if (e) (void)hipEventDestroy(e);   // events of the previous device: nothing to do on failure
                e = nullptr;
            }
        for (auto& row : g_prof.ev)
            for (auto& e : row)
                if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_LAUNCH;
        g_prof.device = dev;
    }
    g_prof.n = 0;
    return launched(hipEventRecord(g_prof.ev[g_prof.calls % kMaxCalls][0], s));
}

int32_t prof_mark(const char* name, hipStream_t s) {
    if (!g_prof.enabled || g_prof.n >= kMaxStages) return MOE_OK;
    g_prof.names[g_prof.n] = name;
    ++g_prof.n;
    return launched(hipEventRecord(g_prof.ev[g_prof.calls % kMaxCalls][g_prof.n], s));
}

void prof_end() {
    if (!g_prof.enabled) return;
    g_prof.stages = g_prof.n;
    ++g_prof.calls;
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

const char* moe_status_string(int32_t status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "null pointer argument";
        case MOE_ERR_SHAPE: return "unsupported problem shape";
        case MOE_ERR_DTYPE: return "unsupported dtype or flag";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_LAUNCH: return "kernel launch or HIP runtime call failed";
        case MOE_ERR_STATE: return "no profiled forward, or inconsistent host counts";
        case MOE_ERR_ARG: return "setting out of range";
        default: return "unknown status";
    }
}

int32_t moe_workspace_bytes(const moe_problem* p, size_t* bytes) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (!bytes) return MOE_ERR_NULL;
    *bytes = layout(*p).total;
    return MOE_OK;
}

int32_t moe_packed_weight_bytes(const moe_problem* p, size_t* bytes) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (!bytes) return MOE_ERR_NULL;
    *bytes = packed_layout(*p).total;
    return MOE_OK;
}

int32_t moe_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up,
                         const void* w_down, void* packed, void* stream) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (!w_gate || !w_up || !w_down || !packed) return MOE_ERR_NULL;
    const Packed P = packed_layout(*p);
    return launched(launch_pack(p->act_dtype, w_gate, w_up, w_down, at(packed, P.w1), at(packed, P.w2),
                                reinterpret_cast<uint8_t*>(at(packed, P.s1)),
                                reinterpret_cast<uint8_t*>(at(packed, P.s2)), p->n_experts, p->d_model,
                                p->d_hidden, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int32_t check_route_args(const moe_problem* p, const void* x, const void* w_router, float* logits,
                         int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* pos,
                         int32_t* row_token) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (!logits || !topk_idx || !topk_gate || !counts || !offsets || !pos || !row_token) return MOE_ERR_NULL;
    if (!(p->flags & MOE_LOGITS_GIVEN) && (!x || !w_router)) return MOE_ERR_NULL;
    return MOE_OK;
}

// The routing kernels on arguments already validated; ws holds at least
// layout(*p).route_end bytes (histograms, block bases, probability partials
// and the bf16 router's transposed weights), every byte of which the kernels
// write before they read it.
int32_t route_impl(const moe_problem* p, const void* x, const void* w_router, float* logits, int32_t* topk_idx,
                   float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_token,
                   float* router_stats, void* ws, hipStream_t s) {
    int32_t st = MOE_OK;
    const bool given = p->flags & MOE_LOGITS_GIVEN;
    const Layout L = layout(*p);
    int32_t* hist = reinterpret_cast<int32_t*>(at(ws, L.hist));
    int32_t* base = reinterpret_cast<int32_t*>(at(ws, L.base));
    float* psum = router_stats ? reinterpret_cast<float*>(at(ws, L.psum)) : nullptr;
    const int T = p->T, E = p->n_experts, k = p->top_k, d = p->d_model;
    if (!given && (st = launched(launch_router_logits(p->act_dtype, x, w_router, logits, T, d, E,
                                                       reinterpret_cast<uint16_t*>(at(ws, L.rwt)), s))))
        return st;
    if ((st = launched(launch_route_topk(logits, T, E, k, topk_idx, topk_gate, pos, hist, psum,
                                                  reinterpret_cast<float*>(at(ws, L.ppart)), s)))) return st;
    if ((st = launched(launch_route_scan(hist, route_blocks(T), E, base, counts, offsets, psum, router_stats, T,
                                         k, s))))
        return st;
    return launched(launch_route_finalize(topk_idx, base, T, E, k, pos, row_token, s));
}

}  // namespace

// Scratch of moe_route_noalloc: one array per device, which holds it until the
// process ends.  In host code the name `scratch` is a host-side stand-in, not
// a device address; the device address of each device's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[MOE_ROUTE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array.
int32_t route_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MOE_ERR_LAUNCH;
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_route(const moe_problem* p, const void* x, const void* w_router, float* logits,
                  int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                  int32_t* pos, int32_t* row_token, float* router_stats, void* ws, size_t ws_bytes,
                  void* stream) {
    int32_t st = check_route_args(p, x, w_router, logits, topk_idx, topk_gate, counts, offsets, pos, row_token);
    if (st) return st;
    if (!ws) return MOE_ERR_NULL;
    if (ws_bytes < layout(*p).route_end) return MOE_ERR_WORKSPACE;
    return route_impl(p, x, w_router, logits, topk_idx, topk_gate, counts, offsets, pos, row_token, router_stats,
                      ws, static_cast<hipStream_t>(stream));
}

int32_t moe_route_noalloc(const moe_problem* p, const void* x, const void* w_router, float* logits,
                          int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* pos,
                          int32_t* row_token, float* router_stats, void* stream) {
    int32_t st = check_route_args(p, x, w_router, logits, topk_idx, topk_gate, counts, offsets, pos, row_token);
    if (st) return st;
    if (layout(*p).route_end > (size_t)MOE_ROUTE_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = route_scratch(&ws))) return st;
    return route_impl(p, x, w_router, logits, topk_idx, topk_gate, counts, offsets, pos, row_token, router_stats,
                      ws, static_cast<hipStream_t>(stream));
}

int32_t moe_dispatch(const moe_problem* p, const void* x, const int32_t* pos, void* xe,
                     uint8_t* xe_scale, void* stream) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (!x || !pos || !xe || (p->act_dtype == MOE_MXFP8 && !xe_scale)) return MOE_ERR_NULL;
    return launched(launch_dispatch(p->act_dtype, x, const_cast<int32_t*>(pos), nullptr, nullptr,
                                    nullptr, xe, xe_scale, p->T, p->d_model, p->n_experts, p->top_k,
                                    static_cast<hipStream_t>(stream)));
}

int32_t moe_grouped_swiglu(const moe_problem* p, const void* xe, const uint8_t* xe_scale,
                           const void* packed_w, const int32_t* offsets, void* ye, void* ws,
                           size_t ws_bytes, void* stream) {
    int32_t st = check_problem(p);
    if (st) return st;
    const bool mx = p->act_dtype == MOE_MXFP8;
    if (!xe || !packed_w || !offsets || !ye || !ws || (mx && !xe_scale)) return MOE_ERR_NULL;
    const Layout L = layout(*p);
    if (ws_bytes < L.gemm_end) return MOE_ERR_WORKSPACE;
    const Packed P = packed_layout(*p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int R = p->T * p->top_k, E = p->n_experts, d = p->d_model, H = p->d_hidden;
    const void* pw = packed_w;
    const uint8_t* s1 = reinterpret_cast<const uint8_t*>(static_cast<const char*>(pw) + P.s1);
    const uint8_t* s2 = reinterpret_cast<const uint8_t*>(static_cast<const char*>(pw) + P.s2);
    void* h = at(ws, L.h);
    uint8_t* hs = reinterpret_cast<uint8_t*>(at(ws, L.h_scale));
    if (use_ffn(*p)) {
        int32_t* ffn_sync = reinterpret_cast<int32_t*>(at(ws, L.sync));
        if ((st = launched(launch_zero_i32(ffn_sync, ffn_sync_ints(R, E), s)))) return st;
        return launched(launch_bf16_ffn(static_cast<const uint16_t*>(xe), nullptr, nullptr,
                                        reinterpret_cast<const uint16_t*>(static_cast<const char*>(pw) + P.w1),
                                        static_cast<uint16_t*>(h),
                                        reinterpret_cast<const uint16_t*>(static_cast<const char*>(pw) + P.w2),
                                        static_cast<uint16_t*>(ye), offsets, ffn_sync, R, E, d, H, nullptr, s));
    }
    if ((st = launched(launch_gemm1(p->act_dtype, xe, xe_scale, static_cast<const char*>(pw) + P.w1, s1,
                                    offsets, h, hs, R, E, d, H, nullptr, s))))
        return st;
    return launched(launch_gemm2(p->act_dtype, h, hs, static_cast<const char*>(pw) + P.w2, s2, offsets,
                                 ye, R, E, d, H, nullptr, s));
}

int32_t moe_combine(const moe_problem* p, const void* ye, const float* topk_gate, const int32_t* pos,
                    void* y, void* stream) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (!ye || !topk_gate || !pos || !y) return MOE_ERR_NULL;
    return launched(launch_combine(p->act_dtype, ye, topk_gate, pos, y, p->T, p->d_model, p->top_k,
                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The block on one stream.  With host_counts == NULL nothing waits for the
// host.  Otherwise the per-expert counts are copied to host_counts right after
// routing and the host waits for them before sizing and launching the grouped
// GEMMs, as the original MoE path did (routing counts on the CPU before the
// group sizes are known); everything the kernels compute is the same.
int32_t forward_impl(const moe_problem* p, const void* x, const void* w_router, float* logits,
                     const void* packed_w, void* y, int32_t* topk_idx, float* topk_gate,
                     int32_t* counts, int32_t* offsets, int32_t* pos, float* router_stats, void* ws,
                     size_t ws_bytes, void* stream, int32_t* host_counts) {
    int32_t st = check_problem(p);
    if (st) return st;
    const bool given = p->flags & MOE_LOGITS_GIVEN;
    const bool identity = p->flags & MOE_IDENTITY_EXPERTS;
    if (!x || !logits || !y || !ws || (!identity && !packed_w)) return MOE_ERR_NULL;
    if (!given && !w_router) return MOE_ERR_NULL;
    const Layout L = layout(*p);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int T = p->T, E = p->n_experts, k = p->top_k, d = p->d_model, H = p->d_hidden;
    const int R = T * k, act = p->act_dtype;
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(at(ws, L.idx));
    float* gate = topk_gate ? topk_gate : reinterpret_cast<float*>(at(ws, L.gate));
    int32_t* cnt = counts ? counts : reinterpret_cast<int32_t*>(at(ws, L.counts));
    int32_t* off = offsets ? offsets : reinterpret_cast<int32_t*>(at(ws, L.offsets));
    int32_t* ps = pos ? pos : reinterpret_cast<int32_t*>(at(ws, L.pos));
    int32_t* row_token = reinterpret_cast<int32_t*>(at(ws, L.row_token));
    int32_t* hist = reinterpret_cast<int32_t*>(at(ws, L.hist));
    int32_t* base = reinterpret_cast<int32_t*>(at(ws, L.base));
    float* psum = router_stats ? reinterpret_cast<float*>(at(ws, L.psum)) : nullptr;
    void* xe = at(ws, L.xe);
    uint8_t* xs = reinterpret_cast<uint8_t*>(at(ws, L.xe_scale));
    void* ye = identity ? xe : at(ws, L.ye);

    if ((st = prof_begin(s))) return st;
    if (!given) {
        if ((st = launched(launch_router_logits(act, x, w_router, logits, T, d, E,
                                                reinterpret_cast<uint16_t*>(at(ws, L.rwt)), s))))
            return st;
        if ((st = prof_mark("router_logits", s))) return st;
    }
    if ((st = launched(launch_route_topk(logits, T, E, k, idx, gate, ps, hist, psum,
                                                  reinterpret_cast<float*>(at(ws, L.ppart)), s)))) return st;
    if ((st = prof_mark("route_topk", s))) return st;
    const bool ffn = !identity && use_ffn(*p);
    int32_t* ffn_sync = reinterpret_cast<int32_t*>(at(ws, L.sync));
    if ((st = launched(launch_route_scan(hist, route_blocks(T), E, base, cnt, off, psum, router_stats, T, k, s,
                                         ffn ? ffn_sync : nullptr, ffn ? ffn_sync_ints(R, E) : 0))))
        return st;
    if ((st = prof_mark("route_scan", s))) return st;
    if (host_counts) {
        if ((st = launched(hipMemcpyAsync(host_counts, cnt, (size_t)E * 4, hipMemcpyDeviceToHost, s)))) return st;
        if ((st = launched(hipStreamSynchronize(s)))) return st;
        long rows = 0;
        for (int e = 0; e < E; ++e) rows += host_counts[e];
        if (rows != (long)R) return MOE_ERR_STATE;
        // GPU time from the end of routing until work resumes after the host wait
        if ((st = prof_mark("host_count_wait", s))) return st;
    }
    if (ffn) {
        // the fused bf16 FFN reads each expert-major row straight from x
        // through row_token, so only the positions are finalised here
        if ((st = launched(launch_route_finalize(idx, base, T, E, k, ps, row_token, s)))) return st;
        if ((st = prof_mark("route_finalize", s))) return st;
    } else if (forward_quantises_tokens(*p)) {
        // each token quantised once (positions finalised in the same pass);
        // GEMM1 reads its code rows through row_token, and only the scales are
        // laid out per expert-major row
        uint32_t* xst = reinterpret_cast<uint32_t*>(at(ws, L.xst));
        if ((st = launched(launch_quantize_mxfp8(x, ps, idx, base, row_token, xe, xst, T, d, E, k, s)))) return st;
        if ((st = prof_mark("quantize", s))) return st;
        if ((st = launched(launch_scale_gather(xst, row_token, xs, R, d, s)))) return st;
        if ((st = prof_mark("scale_gather", s))) return st;
    } else {
        if ((st = launched(launch_dispatch(act, x, ps, idx, base, row_token, xe, xs, T, d, E, k, s))))
            return st;
        if ((st = prof_mark("dispatch", s))) return st;
    }
    if (!identity) {
        const Packed P = packed_layout(*p);
        const char* pw = static_cast<const char*>(packed_w);
        void* h = at(ws, L.h);
        uint8_t* hs = reinterpret_cast<uint8_t*>(at(ws, L.h_scale));
        if (ffn) {
            uint16_t* ab = keeps_gate_up(*p) ? reinterpret_cast<uint16_t*>(at(ws, L.ab)) : nullptr;
            if ((st = launched(launch_bf16_ffn(nullptr, static_cast<const uint16_t*>(x), row_token,
                                               reinterpret_cast<const uint16_t*>(pw + P.w1), static_cast<uint16_t*>(h),
                                               reinterpret_cast<const uint16_t*>(pw + P.w2),
                                               static_cast<uint16_t*>(ye), off, ffn_sync, R, E, d, H, host_counts, s,
                                               ab))))
                return st;
            if ((st = prof_mark("grouped_ffn", s))) return st;
        } else {
            uint16_t* ab = keeps_gate_up(*p) ? reinterpret_cast<uint16_t*>(at(ws, L.ab)) : nullptr;
            if ((st = launched(launch_gemm1(act, xe, xs, pw + P.w1, reinterpret_cast<const uint8_t*>(pw + P.s1),
                                            off, h, hs, R, E, d, H, host_counts, s,
                                            forward_quantises_tokens(*p) ? row_token : nullptr, ab))))
                return st;
            if ((st = prof_mark("gemm1_gate_up_swiglu", s))) return st;
            if ((st = launched(launch_gemm2(act, h, hs, pw + P.w2, reinterpret_cast<const uint8_t*>(pw + P.s2),
                                            off, ye, R, E, d, H, host_counts, s))))
                return st;
            if ((st = prof_mark("gemm2_down", s))) return st;
        }
    }
    if ((st = launched(launch_combine(act, ye, gate, ps, y, T, d, k, s)))) return st;
    if ((st = prof_mark("combine", s))) return st;
    prof_end();
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_forward(const moe_problem* p, const void* x, const void* w_router, float* logits,
                    const void* packed_w, void* y, int32_t* topk_idx, float* topk_gate,
                    int32_t* counts, int32_t* offsets, int32_t* pos, float* router_stats, void* ws,
                    size_t ws_bytes, void* stream) {
    return forward_impl(p, x, w_router, logits, packed_w, y, topk_idx, topk_gate, counts, offsets, pos,
                        router_stats, ws, ws_bytes, stream, nullptr);
}

int32_t moe_forward_host_sync(const moe_problem* p, const void* x, const void* w_router, float* logits,
                              const void* packed_w, void* y, int32_t* topk_idx, float* topk_gate,
                              int32_t* counts, int32_t* offsets, int32_t* pos, float* router_stats, void* ws,
                              size_t ws_bytes, void* stream, int32_t* host_counts) {
    if (!host_counts) return MOE_ERR_NULL;
    return forward_impl(p, x, w_router, logits, packed_w, y, topk_idx, topk_gate, counts, offsets, pos,
                        router_stats, ws, ws_bytes, stream, host_counts);
}

int32_t moe_set_profiling(int32_t enable) {
    g_prof.enabled = enable != 0;
    g_prof.calls = 0;
    return MOE_OK;
}

int32_t moe_set_gemm_grid_cap(int32_t cap) {
    if (cap != 0 && cap < 8) return MOE_ERR_ARG;
    return set_pipe_grid_cap(cap) ? MOE_ERR_ARG : MOE_OK;
}

static int32_t check_backward(const moe_problem* p);

int32_t moe_set_test_flags(int32_t flags) {
    if (flags & ~(MOE_TEST_FFN_WAIT | MOE_TEST_FFN_GIVE_UP)) return MOE_ERR_ARG;
    set_ffn_force_wait(flags & MOE_TEST_FFN_WAIT);
    set_ffn_give_up(flags & MOE_TEST_FFN_GIVE_UP);
    return MOE_OK;
}

int32_t moe_fused_status(const moe_problem* p, const void* ws, size_t ws_bytes, int32_t which, int32_t* status,
                         void* stream) {
    int32_t st = which == MOE_STATUS_BACKWARD ? check_backward(p) : check_problem(p);
    if (st) return st;
    if (which != MOE_STATUS_FORWARD && which != MOE_STATUS_BACKWARD) return MOE_ERR_ARG;
    if (!ws || !status) return MOE_ERR_NULL;
    size_t sync = 0, need = 0;
    bool fused = false;
    if (which == MOE_STATUS_FORWARD) {
        const Layout L = layout(*p);
        sync = L.sync;
        need = L.gemm_end;
        fused = use_ffn(*p);
    } else {
        const BwdLayout B = bwd_layout(*p);
        sync = B.sync;
        need = B.total;
        fused = use_bwd_chain(*p);
    }
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    *status = MOE_OK;
    if (!fused) return MOE_OK;   // no fused launch, nothing waits
    int32_t word = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = launched(hipMemcpyAsync(&word, static_cast<const char*>(ws) + sync + 4 * (size_t)kSyncErrWord, 4,
                                      hipMemcpyDeviceToHost, s))))
        return st;
    if ((st = launched(hipStreamSynchronize(s)))) return st;
    *status = word ? MOE_ERR_STATE : MOE_OK;
    return MOE_OK;
}

int32_t moe_kernel_times(const char** names, float* ms, int32_t max_n, int32_t* n) {
    if (!n) return MOE_ERR_NULL;
    if (g_prof.calls == 0) return MOE_ERR_STATE;
    const int calls = std::min(g_prof.calls, kMaxCalls);
    if (hipEventSynchronize(g_prof.ev[(g_prof.calls - 1) % kMaxCalls][g_prof.stages]) != hipSuccess)
        return MOE_ERR_LAUNCH;
    *n = g_prof.stages;
    for (int i = 0; i < g_prof.stages && i < max_n; ++i) {
        double sum = 0.0;
        for (int c = 0; c < calls; ++c) {
            const int slot = (g_prof.calls - 1 - c) % kMaxCalls;
            float t = 0.f;
            if (hipEventElapsedTime(&t, g_prof.ev[slot][i], g_prof.ev[slot][i + 1]) != hipSuccess)
                return MOE_ERR_LAUNCH;
            sum += t;
        }
        if (ms) ms[i] = (float)(sum / calls);
        if (names) names[i] = g_prof.names[i];
    }
    return MOE_OK;
}

// ----------------------------------------------------------------------------- backward

static int32_t check_backward(const moe_problem* p) {
    int32_t st = check_problem(p);
    if (st) return st;
    if (p->flags & MOE_IDENTITY_EXPERTS) return MOE_ERR_DTYPE;
    // the data-gradient GEMM over 2H reads rows of 2H activations with 32-bit offsets
    const long long eb = act_bytes(bwd_act(p->act_dtype));
    if ((long long)p->T * p->top_k * 2 * p->d_hidden * eb >= (1LL << 32)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int32_t moe_backward_workspace_bytes(const moe_problem* p, size_t* bytes) {
    int32_t st = check_backward(p);
    if (st) return st;
    if (!bytes) return MOE_ERR_NULL;
    *bytes = bwd_layout(*p).total;
    return MOE_OK;
}

int32_t moe_backward_weight_bytes(const moe_problem* p, size_t* bytes) {
    int32_t st = check_backward(p);
    if (st) return st;
    if (!bytes) return MOE_ERR_NULL;
    *bytes = bwd_packed_layout(*p).total;
    return MOE_OK;
}

int32_t moe_pack_weights_backward(const moe_problem* p, const void* w_gate, const void* w_up, const void* w_down,
                                  void* packed_bwd, void* stream) {
    int32_t st = check_backward(p);
    if (st) return st;
    if (!w_gate || !w_up || !w_down || !packed_bwd) return MOE_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const BwdPacked P = bwd_packed_layout(*p);
    const int E = p->n_experts, d = p->d_model, H = p->d_hidden;
    if (p->act_dtype == MOE_MXFP8)
        return launched(launch_pack_bwd_mx(w_gate, w_up, w_down, at(packed_bwd, P.w1t), at(packed_bwd, P.w1),
                                           at(packed_bwd, P.wd), E, d, H, s));
    if ((st = launched(launch_pack_w1t(p->act_dtype, w_gate, w_up, at(packed_bwd, P.w1t), E, d, H, s)))) return st;
    return launched(launch_copy_bytes(w_down, at(packed_bwd, P.wd), (size_t)E * H * d * act_bytes(p->act_dtype), s));
}

int32_t moe_backward(const moe_problem* p, const void* dy, const void* x, const void* w_router, const void* packed_w,
                     const void* packed_bwd, const int32_t* topk_idx, const float* topk_gate, const int32_t* offsets,
                     const int32_t* pos, const void* fwd_ws, size_t fwd_ws_bytes, void* dx, float* dlogits,
                     float* dw_gate, float* dw_up, float* dw_down, float* dw_router, void* ws, size_t ws_bytes,
                     void* stream) {
    int32_t st = check_backward(p);
    if (st) return st;
    const bool given = p->flags & MOE_LOGITS_GIVEN;
    const bool mx = p->act_dtype == MOE_MXFP8;
    if (!dy || !packed_bwd || !fwd_ws || !dx || !dlogits || !dw_gate || !dw_up || !dw_down || !ws ||
        (!mx && !packed_w))
        return MOE_ERR_NULL;
    if (!given && (!x || !w_router || !dw_router)) return MOE_ERR_NULL;
    const bool regather = forward_gathers(*p);   // the forward kept no xe: rebuilt from x
    if (regather && !x) return MOE_ERR_NULL;
    const Layout L = layout(*p);
    const BwdLayout BL = bwd_layout(*p);
    if (fwd_ws_bytes < L.total || ws_bytes < BL.total) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int T = p->T, E = p->n_experts, k = p->top_k, d = p->d_model, H = p->d_hidden;
    const int R = T * k, act = bwd_act(p->act_dtype);
    // forward state: the caller's arrays, or the workspace copies moe_forward wrote
    void* fw = const_cast<void*>(fwd_ws);
    const int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<const int32_t*>(at(fw, L.idx));
    const float* gate = topk_gate ? topk_gate : reinterpret_cast<const float*>(at(fw, L.gate));
    const int32_t* off = offsets ? offsets : reinterpret_cast<const int32_t*>(at(fw, L.offsets));
    const int32_t* ps = pos ? pos : reinterpret_cast<const int32_t*>(at(fw, L.pos));
    const void* xe = at(fw, L.xe);
    const void* h = at(fw, L.h);
    const void* ye = at(fw, L.ye);
    const BwdPacked BP = bwd_packed_layout(*p);
    const char* pb = static_cast<const char*>(packed_bwd);
    const void* w1 = mx ? static_cast<const void*>(pb + BP.w1)
                        : static_cast<const void*>(static_cast<const char*>(packed_w) + packed_layout(*p).w1);
    if (mx) {   // dequantise the saved MXFP8 activations; the rest runs in bf16
        uint16_t* xe16 = reinterpret_cast<uint16_t*>(at(ws, BL.xe16));
        uint16_t* h16 = reinterpret_cast<uint16_t*>(at(ws, BL.h16));
        // the forward kept one code row per token when it quantised tokens: gathered through row_token
        const int32_t* rows = forward_quantises_tokens(*p) ? reinterpret_cast<const int32_t*>(at(fw, L.row_token))
                                                           : nullptr;
        if ((st = launched(launch_dq_mxfp8(static_cast<const uint8_t*>(xe),
                                           reinterpret_cast<const uint8_t*>(at(fw, L.xe_scale)), R, d, xe16, s,
                                           rows))))
            return st;
        if ((st = launched(launch_dq_mxfp8(static_cast<const uint8_t*>(h),
                                           reinterpret_cast<const uint8_t*>(at(fw, L.h_scale)), R, H, h16, s))))
            return st;
        xe = xe16;
        h = h16;
    } else if (regather) {
        uint16_t* xe16 = reinterpret_cast<uint16_t*>(at(ws, BL.xe16));
        if ((st = launched(launch_dispatch(MOE_BF16, x, const_cast<int32_t*>(ps), idx, nullptr, nullptr, xe16,
                                           nullptr, T, d, E, k, s))))
            return st;
        xe = xe16;
    }
    void* ab = at(ws, BL.ab);
    void* dye = at(ws, BL.dye);   // later dxe
    void* dh = at(ws, BL.dh);
    float* dsel = reinterpret_cast<float*>(at(ws, BL.dsel));

    float* srow = given ? nullptr : reinterpret_cast<float*>(at(ws, BL.srow));
    if ((st = launched(launch_combine_bwd(act, dy, ye, gate, ps, idx, dye, dlogits, dsel, srow, T, d, E, k, s))))
        return st;
    const bool bf = act == MOE_BF16;
    const bool chain = use_bwd_chain(*p);
    if (bf) {
        // dW_down = h^T dye per expert (before dxe overwrites dye)
        if ((st = launched(launch_wgrad_rows(0, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(dye), off,
                                             E, H, d, dw_down, nullptr, s))))
            return st;
        if (chain && keeps_gate_up(*p)) {
            // dh = dye W_down^T with da | db from the forward's a | b in its
            // epilogue, then dxe = (da | db) W1^T (into dye), in one launch
            int32_t* sync = reinterpret_cast<int32_t*>(at(ws, BL.sync));
            if ((st = launched(launch_zero_i32(sync, fused_sync_ints(R, E, 3), s)))) return st;
            if ((st = launched(launch_bf16_bwd_chain_kept(
                     static_cast<const uint16_t*>(dye), reinterpret_cast<const uint16_t*>(pb + BP.wd),
                     reinterpret_cast<const uint16_t*>(at(fw, L.ab)), static_cast<uint16_t*>(ab),
                     reinterpret_cast<const uint16_t*>(pb + BP.w1t), static_cast<uint16_t*>(dye), off, sync, R, E, d,
                     H, s))))
                return st;
        } else if (chain) {
            // dh = dye W_down^T, da | db from the gate/up recompute and dh, and
            // dxe = (da | db) W1^T (into dye) in one launch
            int32_t* sync = reinterpret_cast<int32_t*>(at(ws, BL.sync));
            if ((st = launched(launch_zero_i32(sync, fused_sync_ints(R, E, 3), s)))) return st;
            if ((st = launched(launch_bf16_bwd_chain(
                     static_cast<const uint16_t*>(dye), reinterpret_cast<const uint16_t*>(pb + BP.wd),
                     static_cast<uint16_t*>(dh), static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(w1),
                     static_cast<uint16_t*>(ab), reinterpret_cast<const uint16_t*>(pb + BP.w1t),
                     static_cast<uint16_t*>(dye), off, sync, R, E, d, H, s))))
                return st;
        } else {
            // dh = dye W_down^T, then the gate/up recompute with the SwiGLU
            // backward in its epilogue: da | db straight into ab
            if ((st = launched(launch_gemm_plain(act, dye, pb + BP.wd, dh, off, R, E, H, d, H, s)))) return st;
            if ((st = launched(launch_gemm_dswiglu(xe, w1, dh, ab, off, R, E, d, H, s)))) return st;
        }
        // dW_gate | dW_up = xe^T (da | db) per expert
        if ((st = launched(launch_wgrad_rows(1, static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(ab), off,
                                             E, d, 2 * H, dw_gate, dw_up, s))))
            return st;
    } else {
        if ((st = launched(launch_gemm_plain(act, xe, w1, ab, off, R, E, 2 * H, d, 2 * H, s)))) return st;
        if ((st = launched(launch_gemm_plain(act, dye, pb + BP.wd, dh, off, R, E, H, d, H, s)))) return st;
        if ((st = launched(launch_wgrad_down(act, h, dye, off, E, R, H, d, dw_down, s)))) return st;
        if ((st = launched(launch_swiglu_bwd(act, dh, ab, R, H, s)))) return st;   // da | db over a | b in place
        if ((st = launched(launch_wgrad_w1(act, xe, ab, off, E, R, d, H, dw_gate, dw_up, s)))) return st;
    }
    if (!(bf && chain) && (st = launched(launch_gemm_plain(act, ab, pb + BP.w1t, dye, off, R, E, d, 2 * H, d, s))))
        return st;
    void* wrt = given ? nullptr : at(ws, BL.wrt);
    if (!given && (st = launched(launch_router_transpose(act, w_router, d, E, wrt, s)))) return st;
    if ((st = launched(launch_dx(act, dye, ps, idx, dsel, wrt, dx, T, d, E, k, s)))) return st;
    const int32_t* row_token = reinterpret_cast<const int32_t*>(at(fw, L.row_token));
    if (!given && (st = launched(launch_wgrad_router(act, x, row_token, srow, off, T, k, d, E,
                                                      reinterpret_cast<float*>(at(ws, BL.rpart)), dw_router, s))))
        return st;
    return MOE_OK;
}

}  // extern "C"
