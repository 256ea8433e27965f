// Grouped expert GEMMs for gfx950: the float32 kernel and the launchers that
// route each activation type to its kernel (bf16: gemm_pipe.hip), each as
// GEMM1 (gate and up fused, SwiGLU epilogue) and GEMM2 (down projection).
//
// The group of rows of expert e is [offsets[e], offsets[e+1]) of the
// expert-major buffer written by dispatch; the tile schedule is derived on
// the device from those offsets (grouped_sched.h), so no host round trip and
// no padding of experts to a common capacity ("Supercharging Olmo-core ...",
// Abstract; explainer "Olmo-core 3 ...", section "Olmo-core 3's answer").
//
// Packed weights are [E][N][K] with the contraction axis K contiguous, so A
// rows and B rows are both loaded as 16-byte runs of K.  GEMM1's N axis
// interleaves 32 gate columns with the matching 32 up columns, so the
// accumulators for gate and up of one (row, h) land in the same lane and the
// SwiGLU is applied in registers before h is stored.
#include <mutex>

#include "grouped_sched.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

// ----------------------------------------------------------------------------- float32

// Plain LDS-tiled FMA kernel for the float32 block: workgroup tile 64 x 64 x 16,
// each of 256 threads computes rows ty + 16 i and columns tx + 16 j.  With the
// 32-column gate/up interleave, columns tx, tx + 16 are gate and tx + 32,
// tx + 48 the matching up columns.
namespace f32g {
constexpr int BM = 64, BN = 64, BK = 16, NTHR = 256;
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ C,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       int N, int K, int ldc) {
    using namespace f32g;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];
    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

    for (int tile = xcd_slot(blockIdx.x, G); tile < total; tile += G) {
        const int mt = tile / NT, nt = tile - mt * NT;
        const int e = tile_expert(s_tstart, E, mt);
        const int row0 = offsets[e] + (mt - s_tstart[e]) * BM;
        const int rows = min(BM, offsets[e + 1] - row0);
        const int n0 = nt * BN;
        const float* Be = B + (size_t)e * N * K;
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        const float* ga = A + (size_t)(row0 + min(lr, rows - 1)) * K + lk;
        const float* gb = Be + (size_t)min(n0 + lr, N - 1) * K + lk;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
        for (int k0 = 0; k0 < K; k0 += BK) {
            const float4 va = *reinterpret_cast<const float4*>(ga + k0);
            const float4 vb = *reinterpret_cast<const float4*>(gb + k0);
            __syncthreads();
            As[lk + 0][lr] = va.x; As[lk + 1][lr] = va.y; As[lk + 2][lr] = va.z; As[lk + 3][lr] = va.w;
            Bs[lk + 0][lr] = vb.x; Bs[lk + 1][lr] = vb.y; Bs[lk + 2][lr] = vb.z; Bs[lk + 3][lr] = vb.w;
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < BK; ++kk) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ty + 16 * i;
            if (r >= rows) continue;
            if (EPI == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + tx + 16 * j;
                    if (col < N) C[(size_t)(row0 + r) * ldc + col] = acc[i][j];
                }
            } else if (n0 < N) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    C[(size_t)(row0 + r) * ldc + n0 / 2 + tx + 16 * j] = silu_mul(acc[i][j], acc[i][j + 2]);
            }
        }
    }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// ----------------------------------------------------------------------------- launchers

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(std::max(1, std::min((n + 255) / 256, 64))), dim3(256), 0, s, p, n);
    return hipGetLastError();
}


static int g_pipe_grid_cap = 0;   // 0: no cap

int set_pipe_grid_cap(int cap) {
    if (cap < 0 || cap > 256 || cap % kXcds) return -1;
    g_pipe_grid_cap = cap;
    return 0;
}

int device_compute_units() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cus[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

int persistent_grid(int R, int E, int N, int BM, int BN, int per_cu, const int32_t* host_counts) {
    long mt = (long)R / BM + (long)min(E, R);
    if (host_counts) {
        mt = 0;
        for (int e = 0; e < E; ++e) mt += (host_counts[e] + BM - 1) / BM;
    }
    const long tiles = mt * ((N + BN - 1) / BN);
    // at most one workgroup per compute unit for the pipelined kernels (their
    // LDS allows no more), as a multiple of the 8 XCDs: every workgroup is
    // resident at once, which the fused launches' dependency waits rely on
    const long cus = max(device_compute_units(), kXcds);
    const long cap = per_cu == 1 ? cus / kXcds * kXcds : cus * per_cu;
    long g = min(tiles, cap);
    g = (g + kXcds - 1) / kXcds * kXcds;
    g = max(g, (long)kXcds);
    if (per_cu == 1 && g_pipe_grid_cap) g = min(g, (long)g_pipe_grid_cap);
    return (int)g;
}

hipError_t launch_gemm1(int act, const void* xe, const uint8_t* xe_scale, const void* w1,
                        const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                        int R, int E, int d, int H, const int32_t* host_counts, hipStream_t s,
                        const int32_t* row_token, uint16_t* ab) {
    const int N = 2 * H, K = d;
    if (ab && act != kMXFP8) return hipErrorInvalidValue;   // a | b are kept by the MXFP8 kernel only
    if (act == kBF16) {
        return launch_bf16_pipe(1, static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(w1),
                                static_cast<uint16_t*>(h), offsets, R, E, N, K, H, host_counts, s);
    } else if (act == kF32) {
        dim3 grid(persistent_grid(R, E, N, f32g::BM, f32g::BN, 4, host_counts)), block(f32g::NTHR);
        hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, block, 0, s, static_cast<const float*>(xe),
                           static_cast<const float*>(w1), static_cast<float*>(h), offsets, E, N, K, H);
    } else {
        if (row_token && K / 128 < 2) return hipErrorInvalidValue;   // the row tables run one tile ahead
        return launch_fp8_pipe(1, static_cast<const uint8_t*>(xe), xe_scale, static_cast<const uint8_t*>(w1), w1_scale,
                               h, h_scale, offsets, R, E, N, K, H, host_counts, s, row_token, ab);
    }
    return hipGetLastError();
}

hipError_t launch_gemm2(int act, const void* h, const uint8_t* h_scale, const void* w2,
                        const uint8_t* w2_scale, const int32_t* offsets, void* ye, int R, int E,
                        int d, int H, const int32_t* host_counts, hipStream_t s) {
    const int N = d, K = H;
    if (act == kBF16) {
        return launch_bf16_pipe(0, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w2),
                                static_cast<uint16_t*>(ye), offsets, R, E, N, K, d, host_counts, s);
    } else if (act == kF32) {
        dim3 grid(persistent_grid(R, E, N, f32g::BM, f32g::BN, 4, host_counts)), block(f32g::NTHR);
        hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, block, 0, s, static_cast<const float*>(h),
                           static_cast<const float*>(w2), static_cast<float*>(ye), offsets, E, N, K, d);
    } else {
        return launch_fp8_pipe(0, static_cast<const uint8_t*>(h), h_scale, static_cast<const uint8_t*>(w2), w2_scale,
                               ye, nullptr, offsets, R, E, N, K, d, host_counts, s);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_dswiglu(const void* xe, const void* w1, const void* dh, void* dab, const int32_t* offsets,
                               int R, int E, int d, int H, hipStream_t s) {
    return launch_bf16_pipe(2, static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(w1),
                            static_cast<uint16_t*>(dab), offsets, R, E, 2 * H, d, 2 * H, nullptr, s,
                            static_cast<const uint16_t*>(dh));
}

hipError_t launch_gemm_plain(int act, const void* A, const void* B, void* C, const int32_t* offsets, int R, int E,
                             int N, int K, int ldc, hipStream_t s) {
    if (act == kBF16)
        return launch_bf16_pipe(0, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B),
                                static_cast<uint16_t*>(C), offsets, R, E, N, K, ldc, nullptr, s);
    dim3 grid(persistent_grid(R, E, N, f32g::BM, f32g::BN, 4, nullptr)), block(f32g::NTHR);
    hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, block, 0, s, static_cast<const float*>(A),
                       static_cast<const float*>(B), static_cast<float*>(C), offsets, E, N, K, ldc);
    return hipGetLastError();
}

}  // namespace moe
