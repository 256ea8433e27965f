// Rowwise dispatch and combine for gfx950.
//
// Dispatch writes every token row straight into its expert's segment of the
// expert-major buffer at the position routing computed, with no separate
// permutation pass ("Supercharging Olmo-core ...", Abstract: rowwise EP writes
// each token directly into its expert's buffer; explainer "Olmo-core 3 ...",
// section "Olmo-core 3's answer").  For MXFP8 the quantiser runs inside the
// dispatch, producing the codes and scales the grouped GEMM reads directly
// ("Section 24: Conclusion", 24.3: a quantiser must produce a layout the
// transport and GEMM consume without conversion; Evidence 6 counted separate
// quantise / swizzle kernels as overhead).
//
// Both kernels are HBM-bound streaming copies: one wavefront per token row,
// 16-byte loads and stores, each source row read once and written k times
// (dispatch) or k rows read and one written (combine).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kRowsPerBlock = 4;   // one wave per token, 4 waves per workgroup
constexpr int kGroup = 4;          // 16-byte chunks per lane loaded before they are stored

// Final positions of token t's k slots: with `base` non-NULL, pos holds the
// within-block ranks and is rewritten here (rank + the block's base for the
// expert), and row_token[p] = t.  Every lane computes the values (slots past k
// repeat slot k - 1, so the loads are unconditional and issued together);
// lane j writes slot j.
template <int KMAX>
__device__ __forceinline__ void final_positions(int32_t* pos, const int32_t* topk_idx, const int32_t* base,
                                                int32_t* row_token, int t, int k, int E, int lane, int (&p)[KMAX]) {
    int ex[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const size_t i = (size_t)t * k + min(j, k - 1);
        p[j] = pos[i];
        ex[j] = topk_idx[i];
    }
    if (base == nullptr) return;
    const int32_t* b = base + (size_t)(t / kRouteBlock) * E;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) p[j] += b[ex[j]];
    // all lanes have read the ranks before any lane overwrites them
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k && lane == j) {
            pos[(size_t)t * k + j] = p[j];
            row_token[p[j]] = t;
        }
    }
}

template <int KMAX>
__global__ __launch_bounds__(256) void dispatch_copy_kernel(const uint4* __restrict__ x,
                                                            int32_t* __restrict__ pos,
                                                            const int32_t* __restrict__ topk_idx,
                                                            const int32_t* __restrict__ base,
                                                            int32_t* __restrict__ row_token,
                                                            uint4* __restrict__ xe, int T,
                                                            int row_chunks, int E, int k) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    // the row's first chunks are requested before the positions, which they do
    // not depend on; a lane's loads of a group are issued before any store
    // (chunks past the row end are loaded clamped and not stored)
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + (size_t)t * row_chunks;
    u32x4* dst = reinterpret_cast<u32x4*>(xe);
    u32x4 v[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) v[g] = src[min(lane + 64 * g, row_chunks - 1)];
    int p[KMAX];
    final_positions<KMAX>(pos, topk_idx, base, row_token, t, k, E, lane, p);
    for (int c0 = lane; c0 < row_chunks; c0 += 64 * kGroup) {
        if (c0 != lane) {
#pragma unroll
            for (int g = 0; g < kGroup; ++g) v[g] = src[min(c0 + 64 * g, row_chunks - 1)];
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
#pragma unroll
                for (int g = 0; g < kGroup; ++g)
                    if (c0 + 64 * g < row_chunks) dst[(size_t)p[j] * row_chunks + c0 + 64 * g] = v[g];
            }
        }
    }
}

// MXFP8: each lane quantises 16 bf16 values (two 16-byte loads, one 16-byte
// store of codes); lanes 2b and 2b + 1 form block b of 32 and agree on its
// maximum with one shuffle.  Scales are stored [d/128][R][4] (the four scales
// of a 128-wide slice of a row in one dword, rows adjacent), the layout the
// MXFP8 GEMM loads directly; the even lane of each group of 8 lanes gathers
// the slice's four scale bytes and writes the dword.
template <int KMAX>
__global__ __launch_bounds__(256) void dispatch_mxfp8_kernel(const uint4* __restrict__ x,
                                                             int32_t* __restrict__ pos,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ row_token,
                                                             uint4* __restrict__ xq,
                                                             uint32_t* __restrict__ xs, int T, int d,
                                                             int E, int k) {
    const size_t R = (size_t)T * k;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    // d % 128 == 0: a row is d / 16 lane-slices of 16 values; a group of 8
    // lanes covers one 128-wide slice, so groups never straddle a row's end.
    // The first slices are requested before the positions (slices past the
    // row end are loaded clamped and not stored).
    const int slices = d / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + (size_t)t * (d / 8);
    constexpr int kG = 2;   // lane-slices per lane loaded before any is stored
    u32x4 v[kG][2];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        const int c = min(lane + 64 * g, slices - 1);
        v[g][0] = src[2 * c];
        v[g][1] = src[2 * c + 1];
    }
    int p[KMAX];
    final_positions<KMAX>(pos, topk_idx, base, row_token, t, k, E, lane, p);
    for (int c0 = lane; c0 < slices; c0 += 64 * kG) {
        if (c0 != lane) {
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const int c = min(c0 + 64 * g, slices - 1);
                v[g][0] = src[2 * c];
                v[g][1] = src[2 * c + 1];
            }
        }
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int c = c0 + 64 * g;
            if (c >= slices) continue;   // uniform per group of 8 lanes
            float f[16];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f[8 * h + 2 * i] = __uint_as_float(v[g][h][i] << 16);
                    f[8 * h + 2 * i + 1] = __uint_as_float(v[g][h][i] & 0xFFFF0000u);
                }
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            const int se = mx_shared_exp(amax);
            const float inv = mx_inv_scale(se);
            const u32x4 q = {e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                             e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv),
                             e4m3x4(f[8] * inv, f[9] * inv, f[10] * inv, f[11] * inv),
                             e4m3x4(f[12] * inv, f[13] * inv, f[14] * inv, f[15] * inv)};
            // scale byte of block c / 2 at position (c / 2) % 4 of slice c / 8's dword
            uint32_t sw = (uint32_t)(se + 127) << (8 * ((c >> 1) & 3));
            sw |= __shfl_xor(sw, 2);
            sw |= __shfl_xor(sw, 4);
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j < k) {
                    reinterpret_cast<u32x4*>(xq)[(size_t)p[j] * (d / 16) + c] = q;
                    if ((lane & 7) == 0) xs[(size_t)(c >> 3) * R + p[j]] = sw;
                }
            }
        }
    }
}

// The per-slot arrays of the kernels are sized by KMAX >= k (a small bound
// keeps them, and the loops over slots, short).
template <int KMAX>
static void launch_dispatch_k(int act, const void* x, int32_t* pos, const int32_t* topk_idx, const int32_t* base,
                              int32_t* row_token, void* xe, uint8_t* xe_scale, int T, int d, int E, int k,
                              hipStream_t s) {
    dim3 grid((T + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
    if (act == kMXFP8) {
        hipLaunchKernelGGL(dispatch_mxfp8_kernel<KMAX>, grid, block, 0, s, static_cast<const uint4*>(x), pos,
                           topk_idx, base, row_token, static_cast<uint4*>(xe),
                           reinterpret_cast<uint32_t*>(xe_scale), T, d, E, k);
    } else {
        const int row_chunks = d * (act == kF32 ? 4 : 2) / 16;
        hipLaunchKernelGGL(dispatch_copy_kernel<KMAX>, grid, block, 0, s, static_cast<const uint4*>(x), pos,
                           topk_idx, base, row_token, static_cast<uint4*>(xe), T, row_chunks, E, k);
    }
}

hipError_t launch_dispatch(int act, const void* x, int32_t* pos, const int32_t* topk_idx,
                           const int32_t* base, int32_t* row_token, void* xe, uint8_t* xe_scale,
                           int T, int d, int E, int k, hipStream_t s) {
    if (k <= 2) launch_dispatch_k<2>(act, x, pos, topk_idx, base, row_token, xe, xe_scale, T, d, E, k, s);
    else if (k <= 4) launch_dispatch_k<4>(act, x, pos, topk_idx, base, row_token, xe, xe_scale, T, d, E, k, s);
    else if (k <= 8) launch_dispatch_k<8>(act, x, pos, topk_idx, base, row_token, xe, xe_scale, T, d, E, k, s);
    else launch_dispatch_k<kMaxTopK>(act, x, pos, topk_idx, base, row_token, xe, xe_scale, T, d, E, k, s);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- MXFP8 rows in place
//
// The MXFP8 forward quantises each token row once instead of once per slot:
// codes xq [T][d] and, per token, the four E8M0 scales of each 128-wide slice
// as one dword, xst [T][d/128] (both written in whole lines), with the same
// arithmetic as the dispatch; the wave also finalises the token's positions
// and row_token, as the dispatch does.  GEMM1 then reads the code rows of x
// through row_token, and only the scales are laid out per expert-major row
// (scale_gather_kernel), in the slice-major [d/128][R] dwords the GEMM loads.
template <int KMAX>
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const uint4* __restrict__ x, int32_t* __restrict__ pos,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ row_token, uint4* __restrict__ xq,
                                                             uint32_t* __restrict__ xst, int T, int d, int E, int k) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int p[KMAX];
    final_positions<KMAX>(pos, topk_idx, base, row_token, t, k, E, lane, p);
    const int slices = d / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + (size_t)t * (d / 8);
    for (int c = lane; c < slices; c += 64) {   // a group of 8 lanes covers one 128-wide slice
        const u32x4 v0 = src[2 * c], v1 = src[2 * c + 1];
        float f[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v0[i] << 16);
            f[2 * i + 1] = __uint_as_float(v0[i] & 0xFFFF0000u);
            f[8 + 2 * i] = __uint_as_float(v1[i] << 16);
            f[8 + 2 * i + 1] = __uint_as_float(v1[i] & 0xFFFF0000u);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        const int se = mx_shared_exp(amax);
        const float inv = mx_inv_scale(se);
        const u32x4 q = {e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                         e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv),
                         e4m3x4(f[8] * inv, f[9] * inv, f[10] * inv, f[11] * inv),
                         e4m3x4(f[12] * inv, f[13] * inv, f[14] * inv, f[15] * inv)};
        uint32_t sw = (uint32_t)(se + 127) << (8 * ((c >> 1) & 3));
        sw |= __shfl_xor(sw, 2);
        sw |= __shfl_xor(sw, 4);
        reinterpret_cast<u32x4*>(xq)[(size_t)t * slices + c] = q;
        if ((lane & 7) == 0) xst[(size_t)t * (d / 128) + (c >> 3)] = sw;
    }
}

// xs[s][r] = xst[row_token[r]][s]: the scale dwords of expert-major row r,
// one thread per (slice, row) with rows fastest, so the stores are contiguous
// (the reads are scattered but stay in the L2: xst is T * d / 32 bytes).
__global__ __launch_bounds__(256) void scale_gather_kernel(const uint32_t* __restrict__ xst,
                                                           const int32_t* __restrict__ row_token,
                                                           uint32_t* __restrict__ xs, int R, int S) {
    const int r = blockIdx.x * 256 + threadIdx.x, sl = blockIdx.y;
    if (r >= R) return;
    xs[(size_t)sl * R + r] = xst[(size_t)row_token[r] * S + sl];
}

template <int KMAX>
static void launch_quantize_k(const void* x, int32_t* pos, const int32_t* topk_idx, const int32_t* base,
                              int32_t* row_token, void* xq, uint32_t* xst, int T, int d, int E, int k, hipStream_t s) {
    hipLaunchKernelGGL(quantize_mxfp8_kernel<KMAX>, dim3((T + kRowsPerBlock - 1) / kRowsPerBlock),
                       dim3(64 * kRowsPerBlock), 0, s, static_cast<const uint4*>(x), pos, topk_idx, base, row_token,
                       static_cast<uint4*>(xq), xst, T, d, E, k);
}

hipError_t launch_quantize_mxfp8(const void* x, int32_t* pos, const int32_t* topk_idx, const int32_t* base,
                                 int32_t* row_token, void* xq, uint32_t* xst, int T, int d, int E, int k,
                                 hipStream_t s) {
    if (k <= 2) launch_quantize_k<2>(x, pos, topk_idx, base, row_token, xq, xst, T, d, E, k, s);
    else if (k <= 4) launch_quantize_k<4>(x, pos, topk_idx, base, row_token, xq, xst, T, d, E, k, s);
    else if (k <= 8) launch_quantize_k<8>(x, pos, topk_idx, base, row_token, xq, xst, T, d, E, k, s);
    else launch_quantize_k<kMaxTopK>(x, pos, topk_idx, base, row_token, xq, xst, T, d, E, k, s);
    return hipGetLastError();
}

hipError_t launch_scale_gather(const uint32_t* xst, const int32_t* row_token, uint8_t* xs, int R, int d,
                               hipStream_t s) {
    const int S = d / 128;
    hipLaunchKernelGGL(scale_gather_kernel, dim3((unsigned)((R + 255) / 256), (unsigned)S), dim3(256), 0, s, xst,
                       row_token, reinterpret_cast<uint32_t*>(xs), R, S);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- combine

template <bool kBf16, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ ye,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ pos,
                                                      uint4* __restrict__ y, int T, int row_chunks,
                                                      int k) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    // slots past k repeat slot k - 1 (loaded, never used) so that every load
    // is unconditional: all KMAX x CG loads of a chunk group are in flight
    // together, then accumulated in slot order.  ye is read once, so its loads
    // are non-temporal: on blocks whose ye exceeds the caches this took the
    // combine from 0.62 to 0.71 of the HBM peak (T=16384, d=4096, k=8) and
    // from 0.61 to 0.79 (T=32768, d=2048, k=4)
    constexpr int CG = KMAX <= 4 ? kGroup : (KMAX <= 8 ? 2 : 1);
    int p[KMAX];
    float gt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const size_t i = (size_t)t * k + min(j, k - 1);
        p[j] = pos[i];
        gt[j] = gate[i];
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(ye);
    u32x4* dst = reinterpret_cast<u32x4*>(y);
    constexpr int kN = kBf16 ? 8 : 4;
    for (int c0 = lane; c0 < row_chunks; c0 += 64 * CG) {
        float acc[CG][kN];
#pragma unroll
        for (int g = 0; g < CG; ++g)
#pragma unroll
            for (int i = 0; i < kN; ++i) acc[g][i] = 0.f;
        u32x4 vv[KMAX][CG];
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
#pragma unroll
            for (int g = 0; g < CG; ++g)
                vv[j][g] = __builtin_nontemporal_load(&src[(size_t)p[j] * row_chunks + min(c0 + 64 * g, row_chunks - 1)]);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
                const u32x4 (&v)[CG] = vv[j];
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    if (c0 + 64 * g >= row_chunks) continue;
                    if (kBf16) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[g][2 * i] = fmaf(gt[j], __uint_as_float(v[g][i] << 16), acc[g][2 * i]);
                            acc[g][2 * i + 1] = fmaf(gt[j], __uint_as_float(v[g][i] & 0xFFFF0000u), acc[g][2 * i + 1]);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[g][i] = fmaf(gt[j], __uint_as_float(v[g][i]), acc[g][i]);
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            if (c0 + 64 * g >= row_chunks) continue;
            u32x4 o;
            if (kBf16) {
                o = (u32x4){pack_bf16x2(acc[g][0], acc[g][1]), pack_bf16x2(acc[g][2], acc[g][3]),
                            pack_bf16x2(acc[g][4], acc[g][5]), pack_bf16x2(acc[g][6], acc[g][7])};
            } else {
                o = (u32x4){__float_as_uint(acc[g][0]), __float_as_uint(acc[g][1]), __float_as_uint(acc[g][2]),
                            __float_as_uint(acc[g][3])};
            }
            dst[(size_t)t * row_chunks + c0 + 64 * g] = o;
        }
    }
}

template <int KMAX>
static void launch_combine_k(int act, const void* ye, const float* gate, const int32_t* pos, void* y, int T,
                             int d, int k, hipStream_t s) {
    dim3 grid((T + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
    const bool bf = act != kF32;
    const int row_chunks = d * (bf ? 2 : 4) / 16;
    if (bf)
        hipLaunchKernelGGL((combine_kernel<true, KMAX>), grid, block, 0, s, static_cast<const uint4*>(ye), gate,
                           pos, static_cast<uint4*>(y), T, row_chunks, k);
    else
        hipLaunchKernelGGL((combine_kernel<false, KMAX>), grid, block, 0, s, static_cast<const uint4*>(ye), gate,
                           pos, static_cast<uint4*>(y), T, row_chunks, k);
}

hipError_t launch_combine(int act, const void* ye, const float* gate, const int32_t* pos, void* y,
                          int T, int d, int k, hipStream_t s) {
    if (k <= 2) launch_combine_k<2>(act, ye, gate, pos, y, T, d, k, s);
    else if (k <= 4) launch_combine_k<4>(act, ye, gate, pos, y, T, d, k, s);
    else if (k <= 8) launch_combine_k<8>(act, ye, gate, pos, y, T, d, k, s);
    else launch_combine_k<kMaxTopK>(act, ye, gate, pos, y, T, d, k, s);
    return hipGetLastError();
}

}  // namespace moe
