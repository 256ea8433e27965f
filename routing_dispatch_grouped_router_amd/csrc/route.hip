// Routing kernels for gfx950: router logits, top-k with gates, per-block
// expert histograms / ranks, the count-offset scan and position finalisation.
//
// Routing metadata never leaves the device ("Supercharging Olmo-core ...",
// Abstract; "Section 24: Conclusion", 24.1 and Evidence 3 / Figure 74: the
// original path copied route counts to the host, which stalled submission).
// Positions are a stable counting sort by expert computed without global
// atomics: each block of kRouteBlock tokens records, per expert, a bitmask of
// its tokens; a token's rank is a popcount of the bits below it, and a single
// scan over (block, expert) histograms turns ranks into global positions.
// Results are therefore identical from run to run.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ----------------------------------------------------------------------------- router logits

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <typename TIn>
__device__ __forceinline__ float load1(const TIn* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename TIn>
__device__ __forceinline__ void load8w(const TIn* p, float (&v)[8]);   // 8 consecutive weights
template <>
__device__ __forceinline__ void load8w<float>(const float* p, float (&v)[8]) { load8<float>(p, v); }
template <>
__device__ __forceinline__ void load8w<uint16_t>(const uint16_t* p, float (&v)[8]) { load8<uint16_t>(p, v); }

// float32 router logits.  One workgroup of 4 waves computes 8 tokens x 8 experts at a time; wave w
// takes the w-th quarter of d, its lanes runs of 8 elements of it (so 4x as
// many waves share the load of x as with one wave per token group).  The 64
// partial sums of a lane are reduce-scattered across the wave (halving the
// value set at each of the 6 butterfly steps: 63 shuffles instead of 6 per
// value), after which lane l holds its wave's sum for token l / 8, expert
// l % 8; the four waves' sums are added in wave order through LDS.
constexpr int kRtTok = 8;

template <typename TIn>
__global__ __launch_bounds__(256) void router_logits_kernel(const TIn* __restrict__ x,
                                                            const TIn* __restrict__ w,
                                                            float* __restrict__ logits, int T,
                                                            int d, int E) {
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kRtTok;
    const bool vec_w = (E & 7) == 0;
    const int quarter = (d / 8 + 3) / 4 * 8;      // elements per wave, a multiple of 8 (d % 64 == 0)
    const int k_lo = wave * quarter, k_hi = min(d, k_lo + quarter);
    for (int e0 = 0; e0 < E; e0 += 8) {
        float acc[64];
#pragma unroll
        for (int i = 0; i < 64; ++i) acc[i] = 0.f;
        for (int kb = k_lo + lane * 8; kb < k_hi; kb += 64 * 8) {
            float xv[kRtTok][8];
#pragma unroll
            for (int a = 0; a < kRtTok; ++a) {
                const int t = min(t0 + a, T - 1);
                load8<TIn>(x + (size_t)t * d + kb, xv[a]);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const TIn* wr = w + (size_t)(kb + q) * E + e0;
                float wv[8];
                if (vec_w) {
                    load8w<TIn>(wr, wv);
                } else {
#pragma unroll
                    for (int b = 0; b < 8; ++b) wv[b] = (e0 + b < E) ? load1<TIn>(wr + b) : 0.f;
                }
#pragma unroll
                for (int a = 0; a < kRtTok; ++a)
#pragma unroll
                    for (int b = 0; b < 8; ++b) acc[a * 8 + b] = fmaf(xv[a][q], wv[b], acc[a * 8 + b]);
            }
        }
        // reduce-scatter: at mask m the lane keeps the upper half of its current
        // values if (lane & m) else the lower half, adding the partner's copy
#pragma unroll
        for (int m = 32, n = 64; m >= 1; m >>= 1, n >>= 1) {
            const bool up = (lane & m) != 0;
#pragma unroll
            for (int i = 0; i < n / 2; ++i) {
                const float keep = up ? acc[i + n / 2] : acc[i];
                const float send = up ? acc[i] : acc[i + n / 2];
                acc[i] = keep + __shfl_xor(send, m);
            }
        }
        red[wave][lane] = acc[0];
        __syncthreads();
        if (wave == 0) {
            const float sum = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
            const int a = lane >> 3, b = lane & 7;
            if (t0 + a < T && e0 + b < E) logits[(size_t)(t0 + a) * E + e0 + b] = sum;
        }
        __syncthreads();   // red is rewritten for the next group of experts
    }
}

// W^T [E][d] from the router weight W [d][E] (bfloat16), so that each
// expert's weights are contiguous along d for the MFMA operand loads.
__global__ __launch_bounds__(256) void router_wt_kernel(const uint16_t* __restrict__ w, int d, int E,
                                                        uint16_t* __restrict__ wt) {
    const int n = d * E;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
        const int e = i / d, c = i - e * d;
        wt[i] = w[(size_t)c * E + e];
    }
}

typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef float f32x4_r __attribute__((ext_vector_type(4)));

// bf16 router logits on MFMA: L = x W as 16 x 16 output blocks of
// v_mfma_f32_16x16x32_bf16 (lane l holds row l % 16 and k 8 (l / 16) .. +8 of
// each operand; output element i of lane l is token row 4 (l / 16) + i and
// expert column l % 16).  A workgroup owns 16 tokens and 16 experts; its four
// waves take the four quarters of d, walking them in steps of 32 with both
// operands loaded straight from global memory (x rows and rows of W^T, 16
// bytes per lane, eight steps in flight), and the quarters' float32 sums are
// added in wave order through LDS.  Rows past T and experts past E are
// clamped in the loads and not stored.
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wt,
                                                                 float* __restrict__ logits, int T, int d, int E) {
    __shared__ f32x4_r red[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
    const int ta = min(t0 + (lane & 15), T - 1), eb = min(e0 + (lane & 15), E - 1);
    const int ns = d / 32, s_lo = wave * ns / 4, s_hi = (wave + 1) * ns / 4;   // this wave's 32-wide steps
    const int kq = 8 * (lane >> 4);
    const uint16_t* xa = x + (size_t)ta * d + kq;
    const uint16_t* wb = wt + (size_t)eb * d + kq;
    f32x4_r acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_lo; s0 < s_hi; s0 += 8) {
        bf16x8_r a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = 32 * min(s0 + u, s_hi - 1);   // a clamped step is loaded but not accumulated
            a[u] = *reinterpret_cast<const bf16x8_r*>(xa + k);
            b[u] = *reinterpret_cast<const bf16x8_r*>(wb + k);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < s_hi) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        const f32x4_r s = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        const int e = e0 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * (lane >> 4) + i;
            if (t < T && e < E) logits[(size_t)t * E + e] = s[i];
        }
    }
}

// The same logits with W read in its stored [d][E] layout, for E a multiple
// of 8, so no transposed copy is made first: per batch of eight 32-wide steps
// each wave stages the 256 rows of its 16 expert columns (8 KB, columns past E
// zero) in its own LDS slab, row-major with 32 bytes per row, and builds each
// B operand (8 consecutive k of one expert column per lane) from two
// transposing LDS reads (ds_read_b64_tr_b16: 16 lanes addressing rows
// r0 + L / 4 and columns 4 (L % 4) .. + 3 receive rows r0 .. r0 + 3 of column
// L).  The x loads of the batch are issued together with the slab's, and the
// MFMA operands are the same bf16 values in the same order as above, so the
// logits are bitwise those of the transposed path.
__global__ __launch_bounds__(256) void router_logits_mfma_wr_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ w,
                                                                    float* __restrict__ logits, int T, int d, int E) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lp;
    __shared__ f32x4_r red[4][64];
    __shared__ u32x4 slab[4][512];   // per wave: 256 rows x 2 halves of 8 columns
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
    const int ta = min(t0 + (lane & 15), T - 1);
    const int ns = d / 32, s_lo = wave * ns / 4, s_hi = (wave + 1) * ns / 4;   // this wave's 32-wide steps
    const uint16_t* xa = x + (size_t)ta * d + 8 * (lane >> 4);
    u32x4* const sw = slab[wave];
    const __attribute__((address_space(3))) char* const sb =
        (const __attribute__((address_space(3))) char*)(const __attribute__((address_space(3))) void*)sw;
    const int L = lane & 15, g = lane >> 4;
    const uint32_t tr0 = (uint32_t)(8 * g + L / 4) * 32u + (uint32_t)(L % 4) * 8u;   // step 0, first read
    f32x4_r acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_lo; s0 < s_hi; s0 += 8) {
        bf16x8_r a[8];
        u32x4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = 32 * min(s0 + u, s_hi - 1);   // a clamped step is loaded but not accumulated
            a[u] = *reinterpret_cast<const bf16x8_r*>(xa + k);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = lane + 64 * i, row = q >> 1, half = q & 1;
            const int k = min(32 * s0 + row, d - 1);   // rows of clamped steps are never read
            wv[i] = e0 + 8 * half + 8 <= E ? *reinterpret_cast<const u32x4*>(w + (size_t)k * E + e0 + 8 * half)
                                           : (u32x4){0u, 0u, 0u, 0u};
        }
        // the previous batch's reads of the slab are complete before it is overwritten
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < 8; ++i) sw[lane + 64 * i] = wv[i];
        // the slab is private to the wave: its own writes complete, then any lane reads any row
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (s0 + u < s_hi) {
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(sb + tr0 + 1024u * u));
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(sb + tr0 + 1024u * u + 128u));
                const bf16x8_r b = __builtin_bit_cast(bf16x8_r, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b, acc, 0, 0, 0);
            }
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        const f32x4_r sum = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        const int e = e0 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * (lane >> 4) + i;
            if (t < T && e < E) logits[(size_t)t * E + e] = sum[i];
        }
    }
}

hipError_t launch_router_logits(int act, const void* x, const void* w, float* logits, int T, int d,
                                int E, uint16_t* wt, hipStream_t s) {
    if (act == kF32) {
        dim3 grid((T + kRtTok - 1) / kRtTok), block(256);
        hipLaunchKernelGGL(router_logits_kernel<float>, grid, block, 0, s,
                           static_cast<const float*>(x), static_cast<const float*>(w), logits, T, d, E);
    } else {
        dim3 grid((T + 15) / 16, (E + 15) / 16), block(256);
        if (E % 8 == 0) {
            hipLaunchKernelGGL(router_logits_mfma_wr_kernel, grid, block, 0, s, static_cast<const uint16_t*>(x),
                               static_cast<const uint16_t*>(w), logits, T, d, E);
            return hipGetLastError();
        }
        const int n = d * E;
        hipLaunchKernelGGL(router_wt_kernel, dim3(std::min((n + 255) / 256, 1024)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(w), d, E, wt);
        hipLaunchKernelGGL(router_logits_mfma_kernel, grid, block, 0, s, static_cast<const uint16_t*>(x), wt, logits,
                           T, d, E);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- top-k

// Top-k.  route_select_kernel gives every token G lanes (each holding V of
// its logits, experts r*V .. r*V+V-1 for lane r of the group).  For G > 4 a
// workgroup of 256 threads holds 256 / G tokens, so there are as many
// workgroups as the tokens need and the whole chip works on the selection;
// route_rank_kernel then turns each routing block's selected experts into
// within-block ranks and the block's expert histogram.  For G <= 4 one
// workgroup of 256 G threads holds a whole routing block and ranks it itself.

// Orderable 32-bit image of a float32 logit: larger logits give larger values,
// -0.0 maps like +0.0, and 0 stays free to mark an expert already taken (the
// one pattern that would map there, the all-ones NaN, is moved up by one).
__device__ __forceinline__ uint32_t logit_ord(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return o > 1u ? o : 1u;
}
__device__ __forceinline__ float ord_logit(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Cross-lane steps inside aligned groups of G lanes (G a power of two <= 64):
// quad permutations and the row mirrors are DPP operand modifiers (no LDS
// round trip); only groups wider than a 16-lane row use ds_bpermute.  Every
// lane of a group ends with the same value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int G, typename Op>
__device__ __forceinline__ uint32_t group_reduce(uint32_t v, Op op) {
    if constexpr (G >= 2) v = op(v, dpp_u32<0xB1>(v));     // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v = op(v, dpp_u32<0x4E>(v));     // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v = op(v, dpp_u32<0x141>(v));    // row_half_mirror: the other quad of 8
    if constexpr (G >= 16) v = op(v, dpp_u32<0x140>(v));   // row_mirror: the other half of 16
    if constexpr (G >= 32) v = op(v, (uint32_t)__shfl_xor((int)v, 16));
    if constexpr (G >= 64) v = op(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}
struct MaxU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
struct MinU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct AddF32 {   // a + b == b + a bitwise, so both lanes of a pair agree
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }
};

constexpr int kSelThreads = 256;

// One token per group of G lanes.  k rounds each take the group's largest
// remaining key and, among the lanes holding it, the lowest expert index, so
// slot j holds the j-th largest logit with ties to the lower index.
//
// FUSE (G <= 4): the workgroup is one routing block of kRouteBlock tokens and
// also writes the ranks and the block histogram: each selected (token, slot)
// sets its token's bit in its expert's LDS bitmask, a token's rank is the
// popcount of the bits below it, the block's count of expert e the popcount
// of e's mask.
//
// With psum non-NULL the workgroup also sums, per expert, the full-softmax
// probability over its tokens (in token order, through a fixed two-level
// tree) into psum[blockIdx.x][E]; without FUSE these are partial rows that the
// rank kernel adds G at a time in order, so the statistics do not depend on
// scheduling.
template <int G, int V, bool FUSE>
__global__ __launch_bounds__(FUSE ? kRouteBlock * G : kSelThreads) void route_select_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, int32_t* __restrict__ rank, int32_t* __restrict__ hist,
    float* __restrict__ psum) {
    constexpr int NTHR = FUSE ? kRouteBlock * G : kSelThreads;
    constexpr int TA = NTHR / G;                 // tokens per workgroup
    constexpr int kWords = kRouteBlock / 32;
    static_assert(!FUSE || G <= 4, "a fused workgroup holds 256 G threads");
    __shared__ float s_p[NTHR * V + NTHR];
    __shared__ uint32_t mask[FUSE ? G * V * kWords : 1];
    if (FUSE) {
        for (int i = threadIdx.x; i < E * kWords; i += NTHR) mask[i] = 0u;
        __syncthreads();
    }
    const int tid = threadIdx.x, r = tid % G, grp = tid / G;
    const int t = blockIdx.x * TA + grp;
    const bool live = t < T;
    const int e0 = r * V;                        // this lane's first expert
    float lv[V];
#pragma unroll
    for (int v = 0; v < V; ++v) lv[v] = 0.f;
    if (live) {
        const float* row = logits + (size_t)t * E + e0;
        if ((E & 3) == 0 && e0 + V <= E) {       // whole run in range and 16-byte aligned
#pragma unroll
            for (int v = 0; v < V; v += 4) {
                const float4 q = *reinterpret_cast<const float4*>(row + v);
                lv[v] = q.x; lv[v + 1] = q.y; lv[v + 2] = q.z; lv[v + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (e0 + v < E) lv[v] = row[v];
        }
    }
    uint32_t o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) o[v] = (live && e0 + v < E) ? logit_ord(lv[v]) : 0u;

    uint32_t so[kMaxTopK];
    int se[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
            uint32_t m = o[0];
#pragma unroll
            for (int v = 1; v < V; ++v) m = o[v] > m ? o[v] : m;
            m = group_reduce<G>(m, MaxU32{});
            int cv = V;
#pragma unroll
            for (int v = V - 1; v >= 0; --v) cv = (o[v] == m) ? v : cv;
            const uint32_t e = group_reduce<G>(cv < V ? (uint32_t)(e0 + cv) : 0xFFFFFFFFu, MinU32{});
            so[j] = m;
            se[j] = (int)e;
            const int q = (int)e - e0;           // in [0, V) only on the lane holding e
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = (q == v) ? 0u : o[v];
        }
    }
    // gates: softmax over all E renormalised over the selected k equals the
    // softmax over the k selected logits
    const float l0 = ord_logit(so[0]);
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) den += expf(ord_logit(so[j]) - l0);
    const float inv = 1.0f / den;
    if (live) {
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < k && (j % G) == r) {
                topk_idx[(size_t)t * k + j] = se[j];
                topk_gate[(size_t)t * k + j] = expf(ord_logit(so[j]) - l0) * inv;
                if (FUSE) atomicOr(&mask[se[j] * kWords + (grp >> 5)], 1u << (grp & 31));
            }
        }
    }
    if (FUSE) {
        __syncthreads();
        if (live) {
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j < k && (j % G) == r) {
                    const uint32_t* me = mask + se[j] * kWords;
                    int c = __popc(me[grp >> 5] & ((1u << (grp & 31)) - 1u));
                    for (int w = 0; w < (grp >> 5); ++w) c += __popc(me[w]);
                    rank[(size_t)t * k + j] = c;
                }
            }
        }
        for (int e = tid; e < E; e += NTHR) {
            int c = 0;
#pragma unroll
            for (int w = 0; w < kWords; ++w) c += __popc(mask[e * kWords + w]);
            hist[(size_t)blockIdx.x * E + e] = c;
        }
    }
    if (psum == nullptr) return;
    // full softmax over the E logits, l0 being their maximum
    float z[V], zs = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        z[v] = (live && e0 + v < E) ? expf(lv[v] - l0) : 0.f;
        zs += z[v];
    }
    zs = __uint_as_float(group_reduce<G>(__float_as_uint(zs), AddF32{}));
    const float iz = live ? 1.0f / zs : 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
        if (e0 + v < E) s_p[grp * E + e0 + v] = z[v] * iz;
    __syncthreads();
    if (E <= NTHR) {
        int C = 1;                               // chunks of TA / C tokens, summed first
        while (2 * C * E <= NTHR && 2 * C <= TA) C *= 2;
        float* s_c = s_p + TA * E;
        const int e = tid % E, c = tid / E, cs = TA / C;
        if (c < C) {
            float sum = 0.f;
            for (int g = c * cs; g < (c + 1) * cs; ++g) sum += s_p[g * E + e];
            s_c[c * E + e] = sum;
        }
        __syncthreads();
        if (tid < E) {
            float sum = 0.f;
            for (int cc = 0; cc < C; ++cc) sum += s_c[cc * E + tid];
            psum[(size_t)blockIdx.x * E + tid] = sum;
        }
    } else {
        for (int e = tid; e < E; e += NTHR) {
            float sum = 0.f;
            for (int g = 0; g < TA; ++g) sum += s_p[g * E + e];
            psum[(size_t)blockIdx.x * E + e] = sum;
        }
    }
}

// One workgroup per routing block: each selected (token, slot) sets its
// token's bit in its expert's bitmask; a token's rank is the popcount of the
// bits below it, the block's count of expert e the popcount of e's mask.
// With psum non-NULL it adds the block's G partial probability rows in order.
__global__ __launch_bounds__(256) void route_rank_kernel(const int32_t* __restrict__ topk_idx, int T, int E,
                                                         int k, int32_t* __restrict__ rank,
                                                         int32_t* __restrict__ hist,
                                                         const float* __restrict__ ppart, int G,
                                                         float* __restrict__ psum) {
    constexpr int kWords = kRouteBlock / 32;
    __shared__ uint32_t mask[kMaxExperts * kWords];
    const int tid = threadIdx.x, blk = blockIdx.x;
    const int t0 = blk * kRouteBlock, n = min(kRouteBlock, T - t0) * k;
    for (int i = tid; i < E * kWords; i += 256) mask[i] = 0u;
    __syncthreads();
    const int32_t* bidx = topk_idx + (size_t)t0 * k;
    int ev[kMaxTopK];
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q) {
        const int i = tid + 256 * q;             // entry (i / k, i % k) of the block
        ev[q] = -1;
        if (q < k && i < n) {
            ev[q] = bidx[i];
            const int lt = i / k;
            atomicOr(&mask[ev[q] * kWords + (lt >> 5)], 1u << (lt & 31));
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q) {
        if (q < k && ev[q] >= 0) {
            const int i = tid + 256 * q, lt = i / k;
            const uint32_t* me = mask + ev[q] * kWords;
            int c = __popc(me[lt >> 5] & ((1u << (lt & 31)) - 1u));
            for (int w = 0; w < (lt >> 5); ++w) c += __popc(me[w]);
            rank[(size_t)t0 * k + i] = c;
        }
    }
    for (int e = tid; e < E; e += 256) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w) c += __popc(mask[e * kWords + w]);
        hist[(size_t)blk * E + e] = c;
    }
    if (psum != nullptr) {
        const int TA = kSelThreads / G;
        for (int e = tid; e < E; e += 256) {
            float sum = 0.f;
            for (int g = 0; g < G; ++g) {
                const int a = blk * G + g;       // selection workgroup a covers tokens [a TA, a TA + TA)
                if (a * TA < T) sum += ppart[(size_t)a * E + e];
            }
            psum[(size_t)blk * E + e] = sum;
        }
    }
}

template <int G, int V>
static void launch_select(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_gate,
                          int32_t* rank, int32_t* hist, float* psum, float* ppart, hipStream_t s) {
    if constexpr (G <= 4) {
        hipLaunchKernelGGL((route_select_kernel<G, V, true>), dim3(route_blocks(T)), dim3(kRouteBlock * G), 0, s,
                           logits, T, E, k, topk_idx, topk_gate, rank, hist, psum);
    } else {
        constexpr int TA = kSelThreads / G;
        float* pp = psum != nullptr ? ppart : nullptr;
        hipLaunchKernelGGL((route_select_kernel<G, V, false>), dim3((T + TA - 1) / TA), dim3(kSelThreads), 0, s,
                           logits, T, E, k, topk_idx, topk_gate, nullptr, nullptr, pp);
        hipLaunchKernelGGL(route_rank_kernel, dim3(route_blocks(T)), dim3(256), 0, s, topk_idx, T, E, k, rank, hist,
                           pp, G, psum);
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                             float* topk_gate, int32_t* rank, int32_t* hist, float* psum, float* ppart,
                             hipStream_t s) {
    switch (route_lanes(E)) {
        case 1: launch_select<1, 8>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
        case 2: launch_select<2, 8>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
        case 4: launch_select<4, 8>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
        case 8: launch_select<8, 8>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
        case 16: launch_select<16, 8>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
        case 32: launch_select<32, 8>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
        default: launch_select<64, 16>(logits, T, E, k, topk_idx, topk_gate, rank, hist, psum, ppart, s); break;
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- scan

// One workgroup of 1024 threads.  Thread (e, c) sums expert e's counts over a
// contiguous chunk c of routing blocks; chunk partials are scanned per expert,
// expert totals are scanned into offsets, and each thread then writes the
// global base position of expert e for every block of its chunk.
//
// With psum non-NULL it also finishes the router statistics into stats[E + 2]:
// stats[e] = P_e = (sum over blocks of psum[b][e]) / T, the mean full-softmax
// probability of expert e; stats[E] = E * sum_e (counts[e] / (T k)) * P_e, the
// Switch-style load-balancing scalar; stats[E + 1] = max_e counts[e] / (T k / E),
// the worst-case load over the mean load.  Sums run in a fixed order.
constexpr int kScanBatch = 8;

__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ hist,
                                                          int nblk, int E,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          const float* __restrict__ psum,
                                                          float* __restrict__ stats, int T, int k,
                                                          int32_t* __restrict__ zero, int nzero) {
    __shared__ int32_t part[1024];
    __shared__ int32_t tot[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i < nzero; i += 1024) zero[i] = 0;
    const int NC = max(1, min(1024 / E, nblk));    // chunks per expert (E <= 1024), at most one block each when few
    const int CS = (nblk + NC - 1) / NC;           // blocks per chunk
    const int e = tid % E, c = tid / E;
    const bool act = c < NC;
    const int b0 = c * CS, b1 = min(nblk, b0 + CS);
    // hist is read kScanBatch blocks at a time: the loads of a batch are
    // independent, so one memory latency covers the batch
    int s = 0;
    if (act) {
        for (int b = b0; b < b1; b += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) v[u] = b + u < b1 ? hist[(size_t)(b + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) s += v[u];
        }
    }
    part[tid] = s;
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int cc = 0; cc < NC; ++cc) {
            int v = part[cc * E + tid];
            part[cc * E + tid] = run;
            run += v;
        }
        tot[tid] = run;
    } else {
        tot[tid] = 0;
    }
    __syncthreads();
    // inclusive Hillis-Steele scan of tot[0..E) (entries past E are zero)
    for (int off = 1; off < E; off <<= 1) {
        int v = tid >= off ? tot[tid - off] : 0;
        __syncthreads();
        tot[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        int excl = tid == 0 ? 0 : tot[tid - 1];
        offsets[tid] = excl;
        counts[tid] = tot[tid] - excl;
    }
    if (tid == 0) offsets[E] = tot[E - 1];
    if (psum != nullptr) {
        __shared__ float s_fp[1024];
        __shared__ int s_cnt[1024];
        if (tid < E) {
            float sum = 0.f;
            for (int b = 0; b < nblk; b += kScanBatch) {
                float v[kScanBatch];
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u) v[u] = b + u < nblk ? psum[(size_t)(b + u) * E + tid] : 0.f;
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u)
                    if (b + u < nblk) sum += v[u];
            }
            const float P = sum / (float)T;
            const int c = tot[tid] - (tid == 0 ? 0 : tot[tid - 1]);
            stats[tid] = P;
            s_fp[tid] = (float)c / ((float)T * (float)k) * P;
            s_cnt[tid] = c;
        }
        __syncthreads();
        if (tid == 0) {
            float acc = 0.f;
            int mx = 0;
            for (int e = 0; e < E; ++e) {
                acc += s_fp[e];
                mx = max(mx, s_cnt[e]);
            }
            stats[E] = (float)E * acc;
            stats[E + 1] = (float)mx * (float)E / ((float)T * (float)k);
        }
    }
    if (act) {
        int run = (e == 0 ? 0 : tot[e - 1]) + part[c * E + e];
        for (int b = b0; b < b1; b += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) v[u] = b + u < b1 ? hist[(size_t)(b + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) {
                if (b + u < b1) base[(size_t)(b + u) * E + e] = run;
                run += v[u];
            }
        }
    }
}

hipError_t launch_route_scan(const int32_t* hist, int nblk, int E, int32_t* base, int32_t* counts,
                             int32_t* offsets, const float* psum, float* stats, int T, int k, hipStream_t s,
                             int32_t* zero, int nzero) {
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nblk, E, base, counts,
                       offsets, psum, stats, T, k, zero, nzero);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- finalize

__global__ __launch_bounds__(256) void route_finalize_kernel(const int32_t* __restrict__ topk_idx,
                                                             const int32_t* __restrict__ base,
                                                             int T, int E, int k,
                                                             int32_t* __restrict__ pos,
                                                             int32_t* __restrict__ row_token) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * k) return;
    const int t = (int)(i / k);
    const int e = topk_idx[i];
    const int p = base[(size_t)(t / kRouteBlock) * E + e] + pos[i];
    pos[i] = p;
    row_token[p] = t;
}

hipError_t launch_route_finalize(const int32_t* topk_idx, const int32_t* base, int T, int E, int k,
                                 int32_t* pos, int32_t* row_token, hipStream_t s) {
    const size_t n = (size_t)T * k;
    hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       topk_idx, base, T, E, k, pos, row_token);
    return hipGetLastError();
}

}  // namespace moe
