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

hipError_t launch_router_logits(int act, const void* x, const void* w, float* logits, int T, int d,
                                int E, uint16_t* wt, hipStream_t s) {
    if (act == kF32) {
        dim3 grid((T + kRtTok - 1) / kRtTok), block(256);
        hipLaunchKernelGGL(router_logits_kernel<float>, grid, block, 0, s,
                           static_cast<const float*>(x), static_cast<const float*>(w), logits, T, d, E);
    } else {
        const int n = d * E;
        hipLaunchKernelGGL(router_wt_kernel, dim3(std::min((n + 255) / 256, 1024)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(w), d, E, wt);
        dim3 grid((T + 15) / 16, (E + 15) / 16), block(256);
        hipLaunchKernelGGL(router_logits_mfma_kernel, grid, block, 0, s, static_cast<const uint16_t*>(x), wt, logits,
                           T, d, E);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- top-k

// G lanes cooperate on one token, each holding V of its E logits (expert
// r + G*v for lane r of the group).  k rounds of a group-wide max over
// orderable 64-bit keys select the experts in (logit desc, index asc) order.
//
// With psum non-NULL the kernel also sums, per expert, the full-softmax router
// probability over the block's tokens (the soft half of the load-balancing
// statistics): each lane accumulates its experts over the tokens of its group
// in token order, and the groups' partial sums are added in group order, so
// the result does not depend on scheduling.  psum[blk][e] receives the sum.
template <int V>
__global__ __launch_bounds__(1024) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int G,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_gate,
                                                          int32_t* __restrict__ rank,
                                                          int32_t* __restrict__ hist,
                                                          float* __restrict__ psum) {
    constexpr int kWords = kRouteBlock / 32;
    __shared__ uint32_t mask[kMaxExperts * kWords];
    __shared__ int32_t s_idx[kRouteBlock * kMaxTopK];   // selected experts of this block
    __shared__ float s_ps[1024 * V];                    // [group][expert] probability partials
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int blk = blockIdx.x;
    for (int i = tid; i < E * kWords; i += nthr) mask[i] = 0u;
    __syncthreads();

    const int r = tid % G;
    const int grp = tid / G;
    const int per_pass = nthr / G;
    float pacc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) pacc[v] = 0.f;
    for (int lt = grp; lt < kRouteBlock; lt += per_pass) {
        const int t = blk * kRouteBlock + lt;
        if (t >= T) break;       // uniform within a group: G divides 64
        uint64_t key[V];
        float lv[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            int e = r + G * v;
            lv[v] = (e < E) ? logits[(size_t)t * E + e] : 0.f;
            key[v] = (e < E) ? route_key(lv[v], e) : 0ull;
        }
        uint64_t sel[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < k) {
                uint64_t best = 0ull;
#pragma unroll
                for (int v = 0; v < V; ++v) best = key[v] > best ? key[v] : best;
                for (int m = 1; m < G; m <<= 1) {
                    uint64_t o = shfl_xor_u64(best, m);
                    best = o > best ? o : best;
                }
                sel[j] = best;
#pragma unroll
                for (int v = 0; v < V; ++v)
                    if (key[v] == best) key[v] = 0ull;
            }
        }
        // gates: softmax over all E renormalised over the selected k equals the
        // softmax over the k selected logits
        const float l0 = key_logit(sel[0]);
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if (j < k) den += expf(key_logit(sel[j]) - l0);
        const float inv = 1.0f / den;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < k && (j % G) == r) {
                int e = key_expert(sel[j]);
                topk_idx[(size_t)t * k + j] = e;
                s_idx[lt * k + j] = e;
                topk_gate[(size_t)t * k + j] = expf(key_logit(sel[j]) - l0) * inv;
                atomicOr(&mask[e * kWords + (lt >> 5)], 1u << (lt & 31));
            }
        }
        if (psum != nullptr) {
            // full softmax over the E logits, l0 being their maximum
            float z[V], zs = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                z[v] = (r + G * v < E) ? expf(lv[v] - l0) : 0.f;
                zs += z[v];
            }
            for (int m = 1; m < G; m <<= 1) zs += __shfl_xor(zs, m);
            const float iz = 1.0f / zs;
#pragma unroll
            for (int v = 0; v < V; ++v) pacc[v] += z[v] * iz;
        }
    }
    if (psum != nullptr) {
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (r + G * v < E) s_ps[grp * E + r + G * v] = pacc[v];
    }
    __syncthreads();
    if (psum != nullptr) {
        for (int e = tid; e < E; e += nthr) {
            float sum = 0.f;
            for (int g = 0; g < per_pass; ++g) sum += s_ps[g * E + e];
            psum[(size_t)blk * E + e] = sum;
        }
    }
    // within-block rank of every (token, slot): popcount of earlier tokens of the same expert
    for (int i = tid; i < kRouteBlock * k; i += nthr) {
        const int lt = i / k, j = i % k;
        const int t = blk * kRouteBlock + lt;
        if (t >= T) continue;
        const int e = s_idx[lt * k + j];
        const uint32_t* me = mask + e * kWords;
        int c = __popc(me[lt >> 5] & ((1u << (lt & 31)) - 1u));
        for (int w = 0; w < (lt >> 5); ++w) c += __popc(me[w]);
        rank[(size_t)t * k + j] = c;
    }
    for (int e = tid; e < E; e += nthr) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w) c += __popc(mask[e * kWords + w]);
        hist[(size_t)blk * E + e] = c;
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                             float* topk_gate, int32_t* rank, int32_t* hist, float* psum, hipStream_t s) {
    // lanes per token: smallest power of two G <= 64 with E / G <= 8 (or 16 at G = 64)
    int G = 1;
    while (G < 64 && (E + G - 1) / G > 8) G <<= 1;
    const int V = (E + G - 1) / G;
    const int threads = min(1024, kRouteBlock * G);
    dim3 grid(route_blocks(T)), block(threads);
    if (V <= 8)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, G, topk_idx,
                           topk_gate, rank, hist, psum);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, G, topk_idx,
                           topk_gate, rank, hist, psum);
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
__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ hist,
                                                          int nblk, int E,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          const float* __restrict__ psum,
                                                          float* __restrict__ stats, int T, int k) {
    __shared__ int32_t part[1024];
    __shared__ int32_t tot[1024];
    const int tid = threadIdx.x;
    const int NC = max(1, min(1024 / E, nblk));    // chunks per expert (E <= 1024), at most one block each when few
    const int CS = (nblk + NC - 1) / NC;           // blocks per chunk
    const int e = tid % E, c = tid / E;
    const bool act = c < NC;
    const int b0 = c * CS, b1 = min(nblk, b0 + CS);
    int s = 0;
    if (act)
        for (int b = b0; b < b1; ++b) s += hist[(size_t)b * E + e];
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
            for (int b = 0; b < nblk; ++b) sum += psum[(size_t)b * E + tid];
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
        for (int b = b0; b < b1; ++b) {
            base[(size_t)b * E + e] = run;
            run += hist[(size_t)b * E + e];
        }
    }
}

hipError_t launch_route_scan(const int32_t* hist, int nblk, int E, int32_t* base, int32_t* counts,
                             int32_t* offsets, const float* psum, float* stats, int T, int k, hipStream_t s) {
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nblk, E, base, counts,
                       offsets, psum, stats, T, k);
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
