// Grouped expert GEMMs for gfx950: bf16 on MFMA (v_mfma_f32_32x32x16_bf16) and
// a float32 variant, each as GEMM1 (gate and up fused, SwiGLU epilogue) and
// GEMM2 (down projection).
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
#include "grouped_sched.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

// ----------------------------------------------------------------------------- bf16 MFMA

// Workgroup tile 128 x 128 x 64, four waves in a 2 x 2 grid, each wave a
// 64 x 64 block of 2 x 2 MFMA 32x32 tiles.  LDS holds two K-slices of A and
// B (double buffer); 16-byte chunks of each 128-byte row are XOR-swizzled by
// the row index so that the fragment reads of 8 consecutive rows hit
// distinct banks.  Global loads of slice k+1 are issued before the MFMAs of
// slice k.
namespace bf16g {
constexpr int BM = 128, BN = 128, BK = 64, NTHR = 256;
constexpr int CHUNKS = BM * BK / 8;          // 16-byte chunks per operand slice
constexpr int PER_THR = CHUNKS / NTHR;       // 4
}  // namespace bf16g

template <int EPI>   // 0: C = A B (bf16);  1: C = silu(A Bgate) * (A Bup) (bf16, N/2 columns)
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ B,
                                                           uint16_t* __restrict__ C,
                                                           const int32_t* __restrict__ offsets,
                                                           int E, int N, int K, int ldc) {
    using namespace bf16g;
    __shared__ u32x4 sA[2][CHUNKS];
    __shared__ u32x4 sB[2][CHUNKS];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];

    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = K / BK;
    const int kchunks = K / 8;

    for (int tile = xcd_slot(blockIdx.x, G); tile < total; tile += G) {
        const int mt = tile / NT, nt = tile - mt * NT;
        const int e = tile_expert(s_tstart, E, mt);
        const int row0 = offsets[e] + (mt - s_tstart[e]) * BM;
        const int rows = min(BM, offsets[e + 1] - row0);
        const int n0 = nt * BN;
        const u32x4* Bq = reinterpret_cast<const u32x4*>(B) + (size_t)e * N * kchunks;
        const u32x4* gA[PER_THR];
        const u32x4* gB[PER_THR];
        int lds[PER_THR];
#pragma unroll
        for (int i = 0; i < PER_THR; ++i) {
            const int q = tid + NTHR * i, r = q >> 3, c = q & 7;
            const int ar = row0 + min(r, rows - 1);              // clamp ragged rows in-bounds
            const int br = min(n0 + r, N - 1);
            gA[i] = reinterpret_cast<const u32x4*>(A) + (size_t)ar * kchunks + c;
            gB[i] = Bq + (size_t)br * kchunks + c;
            lds[i] = r * 8 + (c ^ (r & 7));
        }
        f32x16 acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        u32x4 ra[PER_THR], rb[PER_THR];
#pragma unroll
        for (int i = 0; i < PER_THR; ++i) { ra[i] = gA[i][0]; rb[i] = gB[i][0]; }
        __syncthreads();   // the previous tile's last reads of buffer 0 are done
#pragma unroll
        for (int i = 0; i < PER_THR; ++i) { sA[0][lds[i]] = ra[i]; sB[0][lds[i]] = rb[i]; }
        __syncthreads();

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) {
#pragma unroll
                for (int i = 0; i < PER_THR; ++i) {
                    ra[i] = gA[i][(kt + 1) * 8];
                    rb[i] = gB[i][(kt + 1) * 8];
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 2 * s + (lane >> 5);
                bf16x8 a[2], b[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) {
                    const int r = wm * 64 + mi * 32 + (lane & 31);
                    a[mi] = __builtin_bit_cast(bf16x8, sA[cur][r * 8 + (c ^ (r & 7))]);
                }
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int r = wn * 64 + ni * 32 + (lane & 31);
                    b[ni] = __builtin_bit_cast(bf16x8, sB[cur][r * 8 + (c ^ (r & 7))]);
                }
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
            }
            if (kt + 1 < nk) {
#pragma unroll
                for (int i = 0; i < PER_THR; ++i) { sA[cur ^ 1][lds[i]] = ra[i]; sB[cur ^ 1][lds[i]] = rb[i]; }
            }
            __syncthreads();
        }

        // accumulator (mi, ni)[v] holds row wm*64 + mi*32 + 8*(v/4) + 4*(lane/32) + v%4,
        // column wn*64 + ni*32 + lane%32 of the tile
        if (EPI == 0) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                        if (r < rows && col < N)
                            C[(size_t)(row0 + r) * ldc + col] = f32_to_bf16(acc[mi][ni][v]);
                    }
                }
        } else {
            // ni = 0: gate columns h0 .. h0+31, ni = 1: the matching up columns
            const int hcol = (n0 + wn * 64) / 2 + (lane & 31);
            if (n0 + wn * 64 < N) {
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                        if (r < rows)
                            C[(size_t)(row0 + r) * ldc + hcol] =
                                f32_to_bf16(silu_mul(acc[mi][0][v], acc[mi][1][v]));
                    }
            }
        }
    }
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

// ----------------------------------------------------------------------------- launchers

static int persistent_grid(int R, int E, int N, int BM, int BN, int per_cu) {
    const long mt_bound = (long)R / BM + (long)min(E, R);
    const long tiles = mt_bound * ((N + BN - 1) / BN);
    long g = min(tiles, (long)256 * per_cu);
    g = (g + kXcds - 1) / kXcds * kXcds;
    return (int)max(g, (long)kXcds);
}

hipError_t launch_gemm1(int act, const void* xe, const uint8_t* xe_scale, const void* w1,
                        const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                        int R, int E, int d, int H, hipStream_t s) {
    (void)xe_scale; (void)w1_scale; (void)h_scale;
    const int N = 2 * H, K = d;
    if (act == kBF16) {
        dim3 grid(persistent_grid(R, E, N, bf16g::BM, bf16g::BN, 2)), block(bf16g::NTHR);
        hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, block, 0, s, static_cast<const uint16_t*>(xe),
                           static_cast<const uint16_t*>(w1), static_cast<uint16_t*>(h), offsets, E, N,
                           K, H);
    } else if (act == kF32) {
        dim3 grid(persistent_grid(R, E, N, f32g::BM, f32g::BN, 4)), block(f32g::NTHR);
        hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, block, 0, s, static_cast<const float*>(xe),
                           static_cast<const float*>(w1), static_cast<float*>(h), offsets, E, N, K, H);
    } else {
        return hipErrorNotSupported;
    }
    return hipGetLastError();
}

hipError_t launch_gemm2(int act, const void* h, const uint8_t* h_scale, const void* w2,
                        const uint8_t* w2_scale, const int32_t* offsets, void* ye, int R, int E,
                        int d, int H, hipStream_t s) {
    (void)h_scale; (void)w2_scale;
    const int N = d, K = H;
    if (act == kBF16) {
        dim3 grid(persistent_grid(R, E, N, bf16g::BM, bf16g::BN, 2)), block(bf16g::NTHR);
        hipLaunchKernelGGL(gemm_bf16_kernel<0>, grid, block, 0, s, static_cast<const uint16_t*>(h),
                           static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(ye), offsets, E, N,
                           K, d);
    } else if (act == kF32) {
        dim3 grid(persistent_grid(R, E, N, f32g::BM, f32g::BN, 4)), block(f32g::NTHR);
        hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, block, 0, s, static_cast<const float*>(h),
                           static_cast<const float*>(w2), static_cast<float*>(ye), offsets, E, N, K, d);
    } else {
        return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace moe
