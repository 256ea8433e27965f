// Backward pass of the routed block on gfx950 (float32 and bf16 activations).
//
// The report treats dispatch and combine as each other's transposes and runs
// the expert FFN as grouped GEMMs in both directions, with data gradients
// grouped by expert rows and weight gradients contracting over each expert's
// rows ("Supercharging Olmo-core ...", "Section 24: Conclusion", Evidence 7
// and Evidence 11).  The steps and their storage points:
//
//   combine backward   dgate[t, j] = dy[t] . ye[pos[t, j]],  dye[pos[t, j]] = g[t, j] dy[t]
//   router backward    dL[t, e_j] = g_j (dgate_j - sum_i g_i dgate_i), 0 elsewhere
//                      (the gates are the softmax of the k selected logits)
//   recompute          a | b = xe W1 (gate/up interleaved as packed), stored
//   down dgrad         dh = dye W_down^T  (B operand: W_down [E][H][d] as given)
//   SwiGLU backward    da = dh b silu'(a), db = dh silu(a), written over a | b
//   up/gate dgrad      dxe = (da | db) W1T  (W1T [E][d][2H], the backward weight cache)
//   weight gradients   dW_down[e] = h^T dye, dW_gate[e] | dW_up[e] = xe^T (da | db),
//                      dW_r = x^T dL   (K-grouped: contraction over an expert's rows)
//   dispatch backward  dx[t] = sum_j dxe[pos[t, j]] + sum_j dL[t, e_j] W_r[:, e_j]
//
// Every reduction runs in a fixed order, so results are bitwise reproducible.
#include <algorithm>

#include "grouped_sched.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTokPerBlock = 4;   // one wave per token

struct bf16raw {
    uint16_t v;
};
__device__ __forceinline__ float ldv(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldv(const bf16raw* p, size_t i) { return bf16_to_f32(p[i].v); }

// E4M3 "FN" code to float (bias 7; exponent 0 is subnormal with step 2^-9).
__device__ __forceinline__ float e4m3_val(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float a = e ? ldexpf(1.0f + (float)m * 0.125f, (int)e - 7) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -a : a;
}

// A 16-byte chunk of a row as float32 values.  Streams read exactly once per
// step (dy, ye, dxe) are loaded non-temporal, so they do not displace what the
// caches hold for later kernels.
template <bool BF>
__device__ __forceinline__ void load_chunk(const void* base, size_t chunk, float (&v)[8]) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + chunk);
    if (BF) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    }
}

template <bool BF>
__device__ __forceinline__ void store_chunk(void* base, size_t chunk, const float (&v)[8]) {
    u32x4 w;
    if (BF) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
    }
    reinterpret_cast<u32x4*>(base)[chunk] = w;
}

// Fixed-pattern butterfly: every lane ends with the same sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

}  // namespace

// One wave per token: the k dot products dy . ye[pos] (each lane sums its
// 16-byte chunks in order, then one butterfly), dye rows, the router
// gradient row dL[t][:] and dsel[t][j] = dL[t][idx[t][j]].
template <bool BF, int KMAX>
__global__ __launch_bounds__(64 * kTokPerBlock) void combine_bwd_kernel(
    const void* __restrict__ dy, const void* __restrict__ ye, const float* __restrict__ gate,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ idx, void* __restrict__ dye,
    float* __restrict__ dL, float* __restrict__ dsel, float* __restrict__ srow, int T, int row_chunks, int E, int k) {
    constexpr int NV = BF ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int p[KMAX], ex[KMAX];
    float g[KMAX], dot[KMAX];
    // slots past k repeat slot k - 1 (loaded, never used), so every load is
    // unconditional and a chunk's k + 1 loads are in flight together
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        dot[j] = 0.f;
        const size_t i = (size_t)t * k + min(j, k - 1);
        p[j] = pos[i];
        ex[j] = idx[i];
        g[j] = gate[i];
    }
    // CG chunk groups per round: their (k + 1) CG loads are in flight together;
    // each lane still takes its chunks in ascending order, so the dot products
    // accumulate in the same order as one chunk per round
    constexpr int CG = KMAX <= 4 ? 2 : 1;
    for (int c0 = lane; c0 < row_chunks; c0 += 64 * CG) {
        float v[CG][8], w[CG][KMAX][8];
#pragma unroll
        for (int q = 0; q < CG; ++q) {
            const int c = min(c0 + 64 * q, row_chunks - 1);   // a clamped chunk is loaded but not used
            load_chunk<BF>(dy, (size_t)t * row_chunks + c, v[q]);
#pragma unroll
            for (int j = 0; j < KMAX; ++j) load_chunk<BF>(ye, (size_t)p[j] * row_chunks + c, w[q][j]);
        }
#pragma unroll
        for (int q = 0; q < CG; ++q) {
            const int c = c0 + 64 * q;
            if (c >= row_chunks) continue;
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j >= k) continue;
                float o[8];
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    dot[j] = fmaf(v[q][i], w[q][j][i], dot[j]);
                    o[i] = g[j] * v[q][i];
                }
                store_chunk<BF>(dye, (size_t)p[j] * row_chunks + c, o);
            }
        }
    }
    float inner = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j >= k) continue;
        dot[j] = wave_sum(dot[j]);
        inner = fmaf(g[j], dot[j], inner);
    }
    float ds[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (j < k) ds[j] = g[j] * (dot[j] - inner);
    if (lane < k) {
        float mine = 0.f;
        int row = 0;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j == lane) {
                mine = ds[j];
                row = p[j];
            }
        dsel[(size_t)t * k + lane] = mine;
        if (srow != nullptr) srow[row] = mine;   // the same value at the routed row
    }
    for (int e = lane; e < E; e += 64) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k && ex[j] == e) v = ds[j];
        dL[(size_t)t * E + e] = v;
    }
}

// da | db over a | b in place.  Columns of ab interleave 32 gate and 32 up
// columns per 64; thread item = 8 consecutive h of one row.
template <bool BF>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const void* __restrict__ dh, void* __restrict__ ab,
                                                         int R, int H) {
    constexpr int NV = BF ? 8 : 4;
    const int per_row = H / NV;
    const size_t items = (size_t)R * per_row;
    for (size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(it / per_row);
        const int h0 = (int)(it - (size_t)r * per_row) * NV;
        const int ga = 64 * (h0 / 32) + h0 % 32;     // column of gate h0 in a | b
        float d[8], a[8], b[8];
        load_chunk<BF>(dh, ((size_t)r * H + h0) / NV, d);
        load_chunk<BF>(ab, ((size_t)r * 2 * H + ga) / NV, a);
        load_chunk<BF>(ab, ((size_t)r * 2 * H + ga + 32) / NV, b);
        float da[8], db[8];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float s = 1.0f / (1.0f + __expf(-a[i]));
            da[i] = d[i] * b[i] * (s * (1.0f + a[i] * (1.0f - s)));
            db[i] = d[i] * (a[i] * s);
        }
        store_chunk<BF>(ab, ((size_t)r * 2 * H + ga) / NV, da);
        store_chunk<BF>(ab, ((size_t)r * 2 * H + ga + 32) / NV, db);
    }
}

// Weight gradient of one group: C[m][n] = sum over rows r of the group of
// A[r][m] B[r][n] (both row-major over r), float32 FMA through LDS, workgroup
// tile 64 x 64, 16 rows per step, each thread 4 x 4 outputs; rows past the
// group contribute zero.  Group e = blockIdx.z is [offsets[e], offsets[e+1])
// (offsets NULL: one group [0, R)).  OMAP 0: C[e][m][n] (ldc N).  OMAP 1: the
// N axis is a | b interleaved (32 gate, 32 up columns per 64) and column n
// goes to C (gate) or C2 (up) [e][m][h].
template <typename TA, typename TB, int OMAP>
__global__ __launch_bounds__(256) void wgrad_kernel(const TA* __restrict__ A, const TB* __restrict__ B,
                                                    const int32_t* __restrict__ offsets, int R, int M, int N,
                                                    float* __restrict__ C, float* __restrict__ C2) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int e = blockIdx.z;
    const int r0 = offsets ? offsets[e] : 0, r1 = offsets ? offsets[e + 1] : R;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int lr = tid >> 4, lc = (tid & 15) * 4;   // loader: row lr of the step, 4 columns from lc
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int rb = r0; rb < r1; rb += 16) {
        const int r = rb + lr;
        float va[4], vb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = m0 + lc + q, n = n0 + lc + q;
            va[q] = (r < r1 && m < M) ? (float)ldv(A, (size_t)r * M + m) : 0.f;
            vb[q] = (r < r1 && n < N) ? (float)ldv(B, (size_t)r * N + n) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            As[lr][lc + q] = va[q];
            Bs[lr][lc + q] = vb[q];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
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
        const int m = m0 + ty + 16 * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= N) continue;
            if (OMAP == 0) {
                C[((size_t)e * M + m) * N + n] = acc[i][j];
            } else {
                const int Hh = N / 2, h = 32 * (n / 64) + n % 32;
                float* dst = ((n / 32) & 1) ? C2 : C;
                dst[((size_t)e * M + m) * Hh + h] = acc[i][j];
            }
        }
    }
}

// dx[t] = sum_j dxe[pos[t, j]] (slot order) + sum_j dsel[t, j] W_r^T[idx[t, j]]
// (learned router; W_r^T [E][d]), one wave per token.
template <bool BF, int KMAX>
__global__ __launch_bounds__(64 * kTokPerBlock) void dx_kernel(const void* __restrict__ dxe,
                                                               const int32_t* __restrict__ pos,
                                                               const int32_t* __restrict__ idx,
                                                               const float* __restrict__ dsel,
                                                               const void* __restrict__ wrt, void* __restrict__ dx,
                                                               int T, int row_chunks, int E, int k) {
    constexpr int NV = BF ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int p[KMAX], ex[KMAX];
    float ds[KMAX];
    // slots past k repeat slot k - 1 (loaded, never used): unconditional loads
    // keep a chunk's loads in flight together
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const size_t i = (size_t)t * k + min(j, k - 1);
        p[j] = pos[i];
        ex[j] = idx[i];
        ds[j] = dsel[i];
    }
    // all k dxe chunks and k W_r^T chunks of CG chunk groups are loaded
    // together, then summed: the dxe rows in slot order, then the router terms
    // in slot order
    constexpr int CG = KMAX <= 4 ? 2 : 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(dxe);
    const u32x4* wsrc = reinterpret_cast<const u32x4*>(wrt);
    auto val = [](const u32x4& v, int i) {
        return BF ? __uint_as_float((i & 1) ? (v[i / 2] & 0xFFFF0000u) : (v[i / 2] << 16)) : __uint_as_float(v[i]);
    };
    for (int c0 = lane; c0 < row_chunks; c0 += 64 * CG) {
        u32x4 v[KMAX][CG], wv[KMAX][CG];
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
#pragma unroll
            for (int g = 0; g < CG; ++g)
                v[j][g] = __builtin_nontemporal_load(&src[(size_t)p[j] * row_chunks + min(c0 + 64 * g, row_chunks - 1)]);
        if (wrt) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
#pragma unroll
                for (int g = 0; g < CG; ++g)
                    wv[j][g] = wsrc[(size_t)ex[j] * row_chunks + min(c0 + 64 * g, row_chunks - 1)];   // W_r^T rows
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            if (c0 + 64 * g >= row_chunks) continue;
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j >= k) continue;
#pragma unroll
                for (int i = 0; i < NV; ++i) acc[i] += val(v[j][g], i);
            }
            if (wrt) {
#pragma unroll
                for (int j = 0; j < KMAX; ++j) {
                    if (j >= k) continue;
#pragma unroll
                    for (int i = 0; i < NV; ++i) acc[i] = fmaf(ds[j], val(wv[j][g], i), acc[i]);
                }
            }
            store_chunk<BF>(dx, (size_t)t * row_chunks + c0 + 64 * g, acc);
        }
    }
}

// dW_r[c][e] = sum over expert e's rows r of x[row_token[r]][c] srow[r] (the
// token rows themselves: for MXFP8 blocks xe holds their quantised values), in
// two passes.
// Pass 1: the rows are cut into tiles of 64 within each expert (the grouped
// GEMMs' tile schedule with 64-row tiles); a workgroup sums its tile's rows in
// order, 8 columns per thread with 16-byte loads, into part[tile][d], and
// workgroup 0 stores the schedule tstart[E + 1].  Pass 2: dW_r[c][e] = sum of
// part[tile][c] over expert e's tiles in order.
constexpr int kWgBatch = 8;

template <bool BF>
__global__ __launch_bounds__(256) void router_wgrad_rows_kernel(const void* __restrict__ x,
                                                                const int32_t* __restrict__ row_token,
                                                                const float* __restrict__ srow,
                                                                const int32_t* __restrict__ offsets, int E, int d,
                                                                float* __restrict__ part, int32_t* __restrict__ tstart) {
    constexpr int NV = BF ? 8 : 4;
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[256];
    const int MT = build_tile_schedule<64, 256>(offsets, E, s_tstart, s_scan);
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e <= E; e += 256) tstart[e] = s_tstart[e];
    const int tile = blockIdx.x;
    if (tile >= MT) return;
    const int e = tile_expert(s_tstart, E, tile);
    const int row0 = offsets[e] + (tile - s_tstart[e]) * 64;
    const int rows = min(64, offsets[e + 1] - row0);
    const int chunks = d / NV;
    for (int c = threadIdx.x; c < chunks; c += 256) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        // rows in batches of kWgBatch whose loads are issued together (one
        // memory latency per batch); the sum still runs in row order
        for (int r0 = 0; r0 < rows; r0 += kWgBatch) {
            float v[kWgBatch][8], sv[kWgBatch];
#pragma unroll
            for (int u = 0; u < kWgBatch; ++u) {
                const int r = min(r0 + u, rows - 1);
                load_chunk<BF>(x, (size_t)row_token[row0 + r] * chunks + c, v[u]);
                sv[u] = r0 + u < rows ? srow[row0 + r] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kWgBatch; ++u) {
                if (r0 + u < rows) {
#pragma unroll
                    for (int i = 0; i < NV; ++i) acc[i] = fmaf(v[u][i], sv[u], acc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) part[(size_t)tile * d + c * NV + i] = acc[i];
    }
}

__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ part,
                                                                  const int32_t* __restrict__ tstart, int d, int E,
                                                                  float* __restrict__ dw) {
    const int n = d * E;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
        const int c = i / E, e = i - c * E;
        float s = 0.f;
        const int t1 = tstart[e + 1];
        for (int t0 = tstart[e]; t0 < t1; t0 += kWgBatch) {
            float v[kWgBatch];
#pragma unroll
            for (int u = 0; u < kWgBatch; ++u) v[u] = t0 + u < t1 ? part[(size_t)(t0 + u) * d + c] : 0.f;
#pragma unroll
            for (int u = 0; u < kWgBatch; ++u)
                if (t0 + u < t1) s += v[u];
        }
        dw[i] = s;
    }
}

// W_r^T [E][d] from W_r [d][E], for 16-byte reads of one expert's column in dx.
template <typename T>
__global__ __launch_bounds__(256) void transpose_small_kernel(const T* __restrict__ w, int d, int E,
                                                              T* __restrict__ wt) {
    const size_t n = (size_t)d * E;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const int e = (int)(i / d), c = (int)(i % d);
        wt[i] = w[(size_t)c * E + e];
    }
}

// MXFP8 activations to bfloat16: codes [R][K] (or, with `rows`, the code row
// rows[r] of a token matrix: the forward quantised each token once) with E8M0
// scales [K/128][R][4] (the dispatch / GEMM1 layout); 16 codes per thread,
// exact (an E4M3 value times a power of two has at most 4 significant bits).
__global__ __launch_bounds__(256) void dq_mxfp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sc,
                                                       int R, int K, uint16_t* __restrict__ out,
                                                       const int32_t* __restrict__ rows) {
    const int per_row = K / 16;
    const size_t n = (size_t)R * per_row;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const int r = (int)(i / per_row), c16 = (int)(i - (size_t)r * per_row);
        const int blk = c16 / 2;   // 32-value block
        const int se = (int)sc[((size_t)(blk / 4) * R + r) * 4 + (blk % 4)] - 127;
        const size_t src = rows ? (size_t)rows[r] : (size_t)r;
        const u32x4 w = reinterpret_cast<const u32x4*>(q + src * K)[c16];
        uint32_t o[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t word = w[b >> 1];
            const uint32_t c0 = (word >> (16 * (b & 1))) & 0xFFu, c1 = (word >> (16 * (b & 1) + 8)) & 0xFFu;
            o[b] = pack_bf16x2(ldexpf(e4m3_val(c0), se), ldexpf(e4m3_val(c1), se));
        }
        u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)r * K) + 2 * c16;
        dst[0] = (u32x4){o[0], o[1], o[2], o[3]};
        dst[1] = (u32x4){o[4], o[5], o[6], o[7]};
    }
}

// ----------------------------------------------------------------------------- launchers

template <int KMAX>
static void launch_combine_bwd_k(int act, const void* dy, const void* ye, const float* gate, const int32_t* pos,
                                 const int32_t* idx, void* dye, float* dL, float* dsel, float* srow, int T, int d,
                                 int E, int k, hipStream_t s) {
    dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock), block(64 * kTokPerBlock);
    if (act == kF32)
        hipLaunchKernelGGL((combine_bwd_kernel<false, KMAX>), grid, block, 0, s, dy, ye, gate, pos, idx, dye, dL,
                           dsel, srow, T, d / 4, E, k);
    else
        hipLaunchKernelGGL((combine_bwd_kernel<true, KMAX>), grid, block, 0, s, dy, ye, gate, pos, idx, dye, dL,
                           dsel, srow, T, d / 8, E, k);
}

hipError_t launch_combine_bwd(int act, const void* dy, const void* ye, const float* gate, const int32_t* pos,
                              const int32_t* idx, void* dye, float* dL, float* dsel, float* srow, int T, int d, int E,
                              int k, hipStream_t s) {
    if (k <= 2) launch_combine_bwd_k<2>(act, dy, ye, gate, pos, idx, dye, dL, dsel, srow, T, d, E, k, s);
    else if (k <= 4) launch_combine_bwd_k<4>(act, dy, ye, gate, pos, idx, dye, dL, dsel, srow, T, d, E, k, s);
    else if (k <= 8) launch_combine_bwd_k<8>(act, dy, ye, gate, pos, idx, dye, dL, dsel, srow, T, d, E, k, s);
    else launch_combine_bwd_k<kMaxTopK>(act, dy, ye, gate, pos, idx, dye, dL, dsel, srow, T, d, E, k, s);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int act, const void* dh, void* ab, int R, int H, hipStream_t s) {
    const int nv = act == kF32 ? 4 : 8;
    const size_t items = (size_t)R * (H / nv);
    const int grid = (int)std::min<size_t>((items + 255) / 256, 256 * 16);
    if (act == kF32) hipLaunchKernelGGL((swiglu_bwd_kernel<false>), dim3(grid), dim3(256), 0, s, dh, ab, R, H);
    else hipLaunchKernelGGL((swiglu_bwd_kernel<true>), dim3(grid), dim3(256), 0, s, dh, ab, R, H);
    return hipGetLastError();
}

template <typename TA, typename TB, int OMAP>
static void launch_wgrad_t(const void* A, const void* B, const int32_t* offsets, int G, int R, int M, int N,
                           float* C, float* C2, hipStream_t s) {
    dim3 grid((N + 63) / 64, (M + 63) / 64, G), block(256);
    hipLaunchKernelGGL((wgrad_kernel<TA, TB, OMAP>), grid, block, 0, s, static_cast<const TA*>(A),
                       static_cast<const TB*>(B), offsets, R, M, N, C, C2);
}

hipError_t launch_wgrad_down(int act, const void* h, const void* dye, const int32_t* offsets, int E, int R, int H,
                             int d, float* dw_down, hipStream_t s) {
    if (act == kF32) launch_wgrad_t<float, float, 0>(h, dye, offsets, E, R, H, d, dw_down, nullptr, s);
    else launch_wgrad_t<bf16raw, bf16raw, 0>(h, dye, offsets, E, R, H, d, dw_down, nullptr, s);
    return hipGetLastError();
}

hipError_t launch_wgrad_w1(int act, const void* xe, const void* dab, const int32_t* offsets, int E, int R, int d,
                           int H, float* dw_gate, float* dw_up, hipStream_t s) {
    if (act == kF32) launch_wgrad_t<float, float, 1>(xe, dab, offsets, E, R, d, 2 * H, dw_gate, dw_up, s);
    else launch_wgrad_t<bf16raw, bf16raw, 1>(xe, dab, offsets, E, R, d, 2 * H, dw_gate, dw_up, s);
    return hipGetLastError();
}

size_t router_wgrad_part_bytes(int R, int E, int d) {
    return (size_t)(R / 64 + std::min(E, R)) * d * 4 + ((size_t)E + 1) * 4 + 256;
}

hipError_t launch_wgrad_router(int act, const void* x, const int32_t* row_token, const float* srow,
                               const int32_t* offsets, int T, int k, int d, int E, float* part, float* dw_router,
                               hipStream_t s) {
    const int R = T * k;
    const int tiles = R / 64 + std::min(E, R);
    int32_t* tstart = reinterpret_cast<int32_t*>(part + (size_t)tiles * d);
    if (act == kF32)
        hipLaunchKernelGGL(router_wgrad_rows_kernel<false>, dim3(tiles), dim3(256), 0, s, x, row_token, srow, offsets,
                           E, d, part, tstart);
    else
        hipLaunchKernelGGL(router_wgrad_rows_kernel<true>, dim3(tiles), dim3(256), 0, s, x, row_token, srow, offsets,
                           E, d, part, tstart);
    const int n = d * E;
    hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3(std::min((n + 255) / 256, 1024)), dim3(256), 0, s, part,
                       tstart, d, E, dw_router);
    return hipGetLastError();
}

hipError_t launch_router_transpose(int act, const void* w_router, int d, int E, void* wrt, hipStream_t s) {
    const size_t n = (size_t)d * E;
    const int grid = (int)std::min<size_t>((n + 255) / 256, 1024);
    if (act == kF32)
        hipLaunchKernelGGL(transpose_small_kernel<float>, dim3(grid), dim3(256), 0, s,
                           static_cast<const float*>(w_router), d, E, static_cast<float*>(wrt));
    else
        hipLaunchKernelGGL(transpose_small_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                           static_cast<const uint16_t*>(w_router), d, E, static_cast<uint16_t*>(wrt));
    return hipGetLastError();
}

template <int KMAX>
static void launch_dx_k(int act, const void* dxe, const int32_t* pos, const int32_t* idx, const float* dsel,
                        const void* wrt, void* dx, int T, int d, int E, int k, hipStream_t s) {
    dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock), block(64 * kTokPerBlock);
    if (act == kF32)
        hipLaunchKernelGGL((dx_kernel<false, KMAX>), grid, block, 0, s, dxe, pos, idx, dsel, wrt, dx, T, d / 4, E,
                           k);
    else
        hipLaunchKernelGGL((dx_kernel<true, KMAX>), grid, block, 0, s, dxe, pos, idx, dsel, wrt, dx, T, d / 8, E, k);
}

hipError_t launch_dx(int act, const void* dxe, const int32_t* pos, const int32_t* idx, const float* dsel,
                     const void* w_router, void* dx, int T, int d, int E, int k, hipStream_t s) {
    if (k <= 2) launch_dx_k<2>(act, dxe, pos, idx, dsel, w_router, dx, T, d, E, k, s);
    else if (k <= 4) launch_dx_k<4>(act, dxe, pos, idx, dsel, w_router, dx, T, d, E, k, s);
    else if (k <= 8) launch_dx_k<8>(act, dxe, pos, idx, dsel, w_router, dx, T, d, E, k, s);
    else launch_dx_k<kMaxTopK>(act, dxe, pos, idx, dsel, w_router, dx, T, d, E, k, s);
    return hipGetLastError();
}

hipError_t launch_dq_mxfp8(const uint8_t* q, const uint8_t* sc, int R, int K, uint16_t* out, hipStream_t s,
                           const int32_t* rows) {
    const size_t n = (size_t)R * (K / 16);
    const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(dq_mxfp8_kernel, dim3(grid), dim3(256), 0, s, q, sc, R, K, out, rows);
    return hipGetLastError();
}

}  // namespace moe
