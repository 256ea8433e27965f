// Expert weight packing (setup, outside the timed path).
//
// W1 [E][2H][d]: row n is gate column 32*(n/64) + n%32 when (n/32) is even,
// else the up column with the same formula.  W2 [E][d][H] is W_down
// transposed.  For MXFP8 the packed rows are quantised in blocks of 32 along
// K with one E8M0 scale each (OCP MX v1.0), the forward weight cache of the
// report ("Section 24: Conclusion", 24.3, two MXFP8 weight caches; only the
// K-major forward one is needed here).  Scales are stored [E][K/128][N][4]:
// the four scales of a 128-wide K slice of row n form one dword, and the
// dwords of consecutive rows are adjacent, so the GEMM loads a slice's scales
// for a block of rows as one contiguous run.
//
// One workgroup moves a 32 (K) x 64 (N) tile through LDS: reads are
// coalesced along the source rows (N), writes along the packed rows (K).
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <typename TIn>
__device__ __forceinline__ float ld(const TIn* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

// which == 1: W1 from (w_gate, w_up) [E][d][H];  which == 2: W2 from w_down [E][H][d].
template <typename TIn, int OUT>   // OUT: 0 float32, 1 bfloat16, 2 MXFP8
__global__ __launch_bounds__(256) void pack_kernel(const TIn* __restrict__ wg, const TIn* __restrict__ wu,
                                                   const TIn* __restrict__ wd, void* __restrict__ out,
                                                   uint8_t* __restrict__ scales, int which, int E, int d,
                                                   int H) {
    __shared__ float tile[32][65];
    const int N = which == 1 ? 2 * H : d;
    const int K = which == 1 ? d : H;
    const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 32, e = blockIdx.z;
    const int tid = threadIdx.x;
    for (int i = tid; i < 32 * 64; i += 256) {
        const int kk = i >> 6, nn = i & 63;
        const int n = n0 + nn, k = k0 + kk;
        float v;
        if (which == 1) {
            const int h = 32 * (n >> 6) + (n & 31);
            const TIn* src = ((n >> 5) & 1) ? wu : wg;
            v = ld<TIn>(src, ((size_t)e * d + k) * H + h);
        } else {
            v = ld<TIn>(wd, ((size_t)e * H + k) * d + n);
        }
        tile[kk][nn] = v;
    }
    __syncthreads();
    const size_t row_base = (size_t)e * N;
    if (OUT == 2) {
        if (tid < 64) {
            const int nn = tid;
            float amax = 0.f;
            for (int kk = 0; kk < 32; ++kk) amax = fmaxf(amax, fabsf(tile[kk][nn]));
            const int se = mx_shared_exp(amax);
            const float inv = mx_inv_scale(se);
            uint8_t* q = static_cast<uint8_t*>(out) + (row_base + n0 + nn) * K + k0;
            for (int w = 0; w < 8; ++w) {
                uint32_t word = 0;
                for (int b = 0; b < 4; ++b) word |= e4m3_encode(tile[4 * w + b][nn] * inv) << (8 * b);
                reinterpret_cast<uint32_t*>(q)[w] = word;
            }
            scales[(((size_t)e * (K / 128) + k0 / 128) * N + n0 + nn) * 4 + (k0 / 32) % 4] = (uint8_t)(se + 127);
        }
    } else {
        for (int i = tid; i < 32 * 64; i += 256) {
            const int nn = i >> 5, kk = i & 31;
            const size_t o = (row_base + n0 + nn) * K + k0 + kk;
            if (OUT == 0) static_cast<float*>(out)[o] = tile[kk][nn];
            else static_cast<uint16_t*>(out)[o] = f32_to_bf16(tile[kk][nn]);   // exact: input is bf16
        }
    }
}

// Backward weight cache W1T [E][d][2H]: row c holds, for every column n of
// the packed W1 (32 gate, then 32 up columns per 64), W1[e][n][c], i.e. the
// gate or up weight of input c and hidden unit 32 (n / 64) + n % 32: the B
// operand of the grouped GEMM dxe = (da | db) W1T, contraction axis 2H
// contiguous.  Both the source rows (over h) and the packed rows (over n) are
// contiguous in runs of 32, so this is a strided copy without a transpose.
template <typename T>
__global__ __launch_bounds__(256) void pack_w1t_kernel(const T* __restrict__ wg, const T* __restrict__ wu,
                                                       T* __restrict__ out, int E, int d, int H) {
    const size_t n_all = (size_t)E * d * 2 * H;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all; i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i % (2 * H));
        const size_t ec = i / (2 * H);      // e * d + c
        const int h = 32 * (n >> 6) + (n & 31);
        out[i] = (((n >> 5) & 1) ? wu : wg)[ec * H + h];
    }
}

hipError_t launch_pack_w1t(int act, const void* w_gate, const void* w_up, void* out, int E, int d, int H,
                           hipStream_t s) {
    const size_t n_all = (size_t)E * d * 2 * H;
    const int grid = (int)std::min<size_t>((n_all + 255) / 256, 256 * 64);
    if (act == kF32)
        hipLaunchKernelGGL((pack_w1t_kernel<float>), dim3(grid), dim3(256), 0, s, static_cast<const float*>(w_gate),
                           static_cast<const float*>(w_up), static_cast<float*>(out), E, d, H);
    else
        hipLaunchKernelGGL((pack_w1t_kernel<uint16_t>), dim3(grid), dim3(256), 0, s,
                           static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
                           static_cast<uint16_t*>(out), E, d, H);
    return hipGetLastError();
}

// E4M3 "FN" code to float (sign, 4-bit exponent with bias 7, 3-bit mantissa;
// exponent 0 is subnormal with step 2^-9).  Codes 0x7F / 0xFF (NaN) are never
// produced by the saturating encoder.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float a = e ? ldexpf(1.0f + (float)m * 0.125f, (int)e - 7) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -a : a;
}

// Backward weight caches of an MXFP8 block, in bfloat16, holding the values the
// forward multiplied with (quantise then dequantise in the forward's blocks).
// which == 1: a 32 (d) x 64 (packed W1 column n) tile of w_gate / w_up, blocks
// of 32 along d, written both as W1T [E][d][2H] and as packed W1 [E][2H][d].
// which == 2: a 32 (H) x 64 (d) tile of w_down [E][H][d], blocks of 32 along H,
// written back in the same layout.
__global__ __launch_bounds__(256) void fq_pack_kernel(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                      const uint16_t* __restrict__ wd, uint16_t* __restrict__ w1t,
                                                      uint16_t* __restrict__ w1, uint16_t* __restrict__ wdq, int which,
                                                      int E, int d, int H) {
    __shared__ float tile[32][65];
    const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 32, e = blockIdx.z;
    const int tid = threadIdx.x;
    for (int i = tid; i < 32 * 64; i += 256) {
        const int kk = i >> 6, nn = i & 63;
        const int n = n0 + nn, k = k0 + kk;
        float v;
        if (which == 1) {
            const int h = 32 * (n >> 6) + (n & 31);
            v = bf16_to_f32((((n >> 5) & 1) ? wu : wg)[((size_t)e * d + k) * H + h]);
        } else {
            v = bf16_to_f32(wd[((size_t)e * H + k) * d + n]);
        }
        tile[kk][nn] = v;
    }
    __syncthreads();
    if (tid < 64) {
        float amax = 0.f;
        for (int kk = 0; kk < 32; ++kk) amax = fmaxf(amax, fabsf(tile[kk][tid]));
        const int se = mx_shared_exp(amax);
        const float inv = mx_inv_scale(se);
        for (int kk = 0; kk < 32; ++kk) tile[kk][tid] = ldexpf(e4m3_value(e4m3_encode(tile[kk][tid] * inv)), se);
    }
    __syncthreads();
    if (which == 1) {
        const int N = 2 * H;
        for (int i = tid; i < 32 * 64; i += 256) {   // W1T rows k (d), contiguous n
            const int kk = i >> 6, nn = i & 63;
            w1t[((size_t)e * d + k0 + kk) * N + n0 + nn] = f32_to_bf16(tile[kk][nn]);
        }
        for (int i = tid; i < 32 * 64; i += 256) {   // packed W1 rows n, contiguous k
            const int nn = i >> 5, kk = i & 31;
            w1[((size_t)e * N + n0 + nn) * d + k0 + kk] = f32_to_bf16(tile[kk][nn]);
        }
    } else {
        for (int i = tid; i < 32 * 64; i += 256) {
            const int kk = i >> 6, nn = i & 63;
            wdq[((size_t)e * H + k0 + kk) * d + n0 + nn] = f32_to_bf16(tile[kk][nn]);
        }
    }
}

hipError_t launch_pack_bwd_mx(const void* w_gate, const void* w_up, const void* w_down, void* w1t, void* w1,
                              void* wdq, int E, int d, int H, hipStream_t s) {
    auto wg = static_cast<const uint16_t*>(w_gate), wu = static_cast<const uint16_t*>(w_up),
         wd = static_cast<const uint16_t*>(w_down);
    auto o1 = static_cast<uint16_t*>(w1t), o2 = static_cast<uint16_t*>(w1), o3 = static_cast<uint16_t*>(wdq);
    hipLaunchKernelGGL(fq_pack_kernel, dim3((2 * H) / 64, d / 32, E), dim3(256), 0, s, wg, wu, wd, o1, o2, o3, 1, E, d,
                       H);
    hipLaunchKernelGGL(fq_pack_kernel, dim3(d / 64, H / 32, E), dim3(256), 0, s, wg, wu, wd, o1, o2, o3, 2, E, d, H);
    return hipGetLastError();
}

hipError_t launch_copy_bytes(const void* src, void* dst, size_t bytes, hipStream_t s) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
}

hipError_t launch_pack(int act, const void* w_gate, const void* w_up, const void* w_down, void* w1,
                       void* w2, uint8_t* s1, uint8_t* s2, int E, int d, int H, hipStream_t s) {
    dim3 block(256);
    dim3 g1((2 * H) / 64, d / 32, E), g2(d / 64, H / 32, E);
    if (act == kF32) {
        auto wg = static_cast<const float*>(w_gate), wu = static_cast<const float*>(w_up),
             wd = static_cast<const float*>(w_down);
        hipLaunchKernelGGL((pack_kernel<float, 0>), g1, block, 0, s, wg, wu, wd, w1, nullptr, 1, E, d, H);
        hipLaunchKernelGGL((pack_kernel<float, 0>), g2, block, 0, s, wg, wu, wd, w2, nullptr, 2, E, d, H);
    } else {
        auto wg = static_cast<const uint16_t*>(w_gate), wu = static_cast<const uint16_t*>(w_up),
             wd = static_cast<const uint16_t*>(w_down);
        if (act == kBF16) {
            hipLaunchKernelGGL((pack_kernel<uint16_t, 1>), g1, block, 0, s, wg, wu, wd, w1, nullptr, 1, E, d, H);
            hipLaunchKernelGGL((pack_kernel<uint16_t, 1>), g2, block, 0, s, wg, wu, wd, w2, nullptr, 2, E, d, H);
        } else {
            hipLaunchKernelGGL((pack_kernel<uint16_t, 2>), g1, block, 0, s, wg, wu, wd, w1, s1, 1, E, d, H);
            hipLaunchKernelGGL((pack_kernel<uint16_t, 2>), g2, block, 0, s, wg, wu, wd, w2, s2, 2, E, d, H);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
