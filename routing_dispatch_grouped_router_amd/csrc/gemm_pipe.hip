// Pipelined bf16 grouped GEMM for gfx950: direct global -> LDS loads feeding a
// four-stage LDS ring, 8 waves per workgroup.
//
// Same contract as the register-staged kernel in gemm.hip (expert groups read
// from device offsets, packed [E][N][K] weights, SwiGLU epilogue for GEMM1),
// built for the large-tile case where the register-staged kernel runs out of
// registers: with 2 waves per SIMD a wave has 256 registers, 128 of which hold
// its 128 x 64 accumulator block, so the K-slice prefetch cannot also sit in
// registers.  Here every 16-byte chunk goes from global memory straight into
// LDS (global_load_lds_dwordx4: lane l of a wave writes LDS bytes
// [16 l, 16 l + 16) of a wave-uniform 1 KB block), so no registers are spent
// on staging and three K-slices can be in flight while a fourth is consumed.
//
// Layout of one stage: BM (resp. BN) rows of one 32-wide K slice, 64 bytes =
// 4 chunks per row; chunk c of row r is stored at c ^ ((r >> 2) & 3), which
// keeps the 16 rows read by each 16-lane group of a fragment load on distinct
// banks.  Each stage is its own __shared__ array and the K loop is unrolled
// by the stage count, so every LDS access names its array statically and the
// compiler's wait insertion need not serialise fragment reads behind the
// loads in flight for other stages; the waits for the DMA are explicit.
#include "grouped_sched.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// s_waitcnt vmcnt(N), other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from base + voff (bytes) into LDS bytes [lds + 16 lane, +16).
// Issued as inline asm so the compiler neither spends a 64-bit address per
// load nor makes later LDS reads wait for it: every wait on these loads is the
// explicit wait_vm of the pipeline.  The compiler's own vmcnt waits stay
// correct (only more conservative) because vector loads retire in order.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier for the LDS ring.  __syncthreads() would add a release
// fence, which on this target waits for every DMA still in flight (including
// the prefetches of later stages).  The stage a wave is about to read was
// waited for explicitly (wait_vm), and the fragments it read last step were
// consumed by MFMAs before it arrives here, so a bare s_barrier suffices; the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float silu_mul_p(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

}  // namespace

template <int BM_, int BN_, int WM_, int WN_>
struct PipeTile {
    static constexpr int BM = BM_, BN = BN_, BK = 32, STAGES = 4, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN, NTHR = 64 * NW;
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static constexpr int A_DMA = BM / 16 / NW, B_DMA = BN / 16 / NW;   // 1 KB blocks per wave per stage
    static constexpr int P = A_DMA + B_DMA;                            // DMA instructions per wave per stage
    static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "stage / wave mismatch");
    static_assert(TN % 2 == 0, "a wave's N range must hold whole gate/up pairs");
};

template <class TL>
struct PipeState {
    const void* Ag;              // wave-uniform bases (SGPRs)
    const void* Bg;
    uint32_t offA[TL::A_DMA], offB[TL::B_DMA];   // byte offsets of this lane's chunk, K-tile 0
    int nk;
    int wave, lane;
    int fragA[TL::TM], fragB[TL::TN];
    int fsw;
};

// Issue the DMA of K-tile kt into stage (sa, sb).
template <class TL>
__device__ __forceinline__ void pipe_issue(const PipeState<TL>& st, u32x4* sa, u32x4* sb, int kt) {
    const uint32_t ko = (uint32_t)kt * (TL::BK * 2);
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(sa) + st.wave * TL::A_DMA * 1024);
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(sb) + st.wave * TL::B_DMA * 1024);
#pragma unroll
    for (int i = 0; i < TL::A_DMA; ++i) dma16(st.Ag, st.offA[i] + ko, la + i * 1024);
#pragma unroll
    for (int i = 0; i < TL::B_DMA; ++i) dma16(st.Bg, st.offB[i] + ko, lb + i * 1024);
}

template <class TL>
__device__ __forceinline__ void load_frags(const PipeState<TL>& st, const u32x4* ca, const u32x4* cb, int ks,
                                           bf16x8 (&fa)[TL::TM], bf16x8 (&fb)[TL::TN]) {
    const int c = (2 * ks + (st.lane >> 5)) ^ st.fsw;
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) fa[mi] = __builtin_bit_cast(bf16x8, ca[st.fragA[mi] + c]);
#pragma unroll
    for (int ni = 0; ni < TL::TN; ++ni) fb[ni] = __builtin_bit_cast(bf16x8, cb[st.fragB[ni] + c]);
}

template <class TL>
__device__ __forceinline__ void mfma_block(const bf16x8 (&fa)[TL::TM], const bf16x8 (&fb)[TL::TN],
                                           f32x16 (&acc)[TL::TM][TL::TN]) {
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
}

// Interleave the TM + TN fragment reads issued in a region with its TM * TN MFMAs.
template <class TL>
__device__ __forceinline__ void interleave_hint() {
    constexpr int R = TL::TM + TL::TN, M = TL::TM * TL::TN;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, M / R, 0);    // then MFMAs
    }
}

// One K-tile (two 16-wide k-steps) of the stage (ca, cb).  On entry slot fa0/fb0
// holds k-step 0 of this stage.  k-step 1's fragments are read while k-step 0
// multiplies; then, with those MFMAs queued, the wave waits for K-tile kt + 1
// to land, joins the barrier, starts the DMA of K-tile kt + 3 into the stage
// everyone finished with, and reads k-step 0 of K-tile kt + 1 while k-step 1
// multiplies.
template <class TL>
__device__ __forceinline__ void pipe_step(const PipeState<TL>& st, const u32x4* ca, const u32x4* cb,
                                          const u32x4* nxa, const u32x4* nxb, u32x4* da, u32x4* db, int kt,
                                          bf16x8 (&fa0)[TL::TM], bf16x8 (&fb0)[TL::TN],
                                          f32x16 (&acc)[TL::TM][TL::TN]) {
    bf16x8 fa1[TL::TM], fb1[TL::TN];
    load_frags<TL>(st, ca, cb, 1, fa1, fb1);
    mfma_block<TL>(fa0, fb0, acc);
    interleave_hint<TL>();
    if (kt + 1 < st.nk) {
        if (kt + 2 < st.nk) wait_vm<TL::P>();    // K-tile kt + 2 may stay in flight
        else wait_vm<0>();
        ring_barrier();
        if (kt + 3 < st.nk) pipe_issue<TL>(st, da, db, kt + 3);
        load_frags<TL>(st, nxa, nxb, 0, fa0, fb0);
    }
    mfma_block<TL>(fa1, fb1, acc);
    interleave_hint<TL>();
}

template <class TL, int EPI>   // EPI 0: C = A B (bf16);  1: C = silu(A Bgate) * (A Bup) (bf16, N/2 columns)
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_bf16_pipe_kernel(const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ B,
                                                                  uint16_t* __restrict__ C,
                                                                  const int32_t* __restrict__ offsets,
                                                                  int E, int N, int K, int ldc) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    constexpr int WROWS = BM / TL::WM, WCOLS = BN / TL::WN;
    __shared__ u32x4 sA0[BM * 4], sA1[BM * 4], sA2[BM * 4], sA3[BM * 4];
    __shared__ u32x4 sB0[BN * 4], sB1[BN * 4], sB2[BN * 4], sB3[BN * 4];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];

    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const int kchunks = K / 8;

    PipeState<TL> st;
    st.lane = threadIdx.x & 63;
    st.wave = threadIdx.x >> 6;
    st.nk = K / TL::BK;
    st.Ag = A;
    const int wm = st.wave / TL::WN, wn = st.wave % TL::WN;
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) st.fragA[mi] = (wm * WROWS + mi * 32 + (st.lane & 31)) * 4;
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) st.fragB[ni] = (wn * WCOLS + ni * 32 + (st.lane & 31)) * 4;
    st.fsw = ((st.lane & 31) >> 2) & 3;
    // DMA lane -> (row within its 16-row block, logical chunk)
    const int drow = st.lane >> 2;
    const int dchunk = (st.lane & 3) ^ ((st.lane >> 4) & 3);

    for (int tile = xcd_slot(blockIdx.x, G); tile < total; tile += G) {
        const int mt = tile / NT, nt = tile - mt * NT;
        const int e = tile_expert(s_tstart, E, mt);
        const int row0 = offsets[e] + (mt - s_tstart[e]) * BM;
        const int rows = min(BM, offsets[e + 1] - row0);
        const int n0 = nt * BN;
        {
            const size_t boff = (size_t)__builtin_amdgcn_readfirstlane(e) * N * K;
            st.Bg = B + boff;
        }
#pragma unroll
        for (int i = 0; i < TL::A_DMA; ++i) {
            const int r = 16 * (st.wave * TL::A_DMA + i) + drow;
            st.offA[i] = ((uint32_t)(row0 + min(r, rows - 1)) * kchunks + dchunk) * 16u;
        }
#pragma unroll
        for (int i = 0; i < TL::B_DMA; ++i) {
            const int r = 16 * (st.wave * TL::B_DMA + i) + drow;
            st.offB[i] = ((uint32_t)min(n0 + r, N - 1) * kchunks + dchunk) * 16u;
        }
        // every wave is done reading the previous tile's stages; its epilogue
        // stores may still be in flight, which no later LDS access depends on
        ring_barrier();
        pipe_issue<TL>(st, sA0, sB0, 0);
        if (st.nk > 1) pipe_issue<TL>(st, sA1, sB1, 1);
        if (st.nk > 2) pipe_issue<TL>(st, sA2, sB2, 2);

        f32x16 acc[TM][TN];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        if (st.nk > 2) wait_vm<2 * TL::P>();
        else if (st.nk > 1) wait_vm<TL::P>();
        else wait_vm<0>();
        ring_barrier();
        bf16x8 fa0[TM], fb0[TN];
        load_frags<TL>(st, sA0, sB0, 0, fa0, fb0);
        // stage of K-tile kt is kt % 4; the DMA issued during K-tile kt fills stage (kt + 3) % 4
        for (int kt = 0; kt < st.nk; kt += 4) {
            pipe_step<TL>(st, sA0, sB0, sA1, sB1, sA3, sB3, kt, fa0, fb0, acc);
            if (kt + 1 < st.nk) pipe_step<TL>(st, sA1, sB1, sA2, sB2, sA0, sB0, kt + 1, fa0, fb0, acc);
            if (kt + 2 < st.nk) pipe_step<TL>(st, sA2, sB2, sA3, sB3, sA1, sB1, kt + 2, fa0, fb0, acc);
            if (kt + 3 < st.nk) pipe_step<TL>(st, sA3, sB3, sA0, sB0, sA2, sB2, kt + 3, fa0, fb0, acc);
        }

        // accumulator (mi, ni)[v] holds tile row wm*WROWS + mi*32 + 8*(v/4) + 4*(lane/32) + v%4
        // and tile column wn*WCOLS + ni*32 + lane%32
        const int rbase = wm * WROWS + 4 * (st.lane >> 5);
        if (EPI == 0) {
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni) {
                    const int col = n0 + wn * WCOLS + ni * 32 + (st.lane & 31);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = rbase + mi * 32 + 8 * (v >> 2) + (v & 3);
                        if (r < rows && col < N)
                            C[(size_t)(row0 + r) * ldc + col] = f32_to_bf16(acc[mi][ni][v]);
                    }
                }
        } else {
#pragma unroll
            for (int np = 0; np < TN / 2; ++np) {
                const int pc = n0 + wn * WCOLS + np * 64;
                if (pc >= N) continue;
                const int hcol = pc / 2 + (st.lane & 31);
#pragma unroll
                for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = rbase + mi * 32 + 8 * (v >> 2) + (v & 3);
                        if (r < rows)
                            C[(size_t)(row0 + r) * ldc + hcol] =
                                f32_to_bf16(silu_mul_p(acc[mi][2 * np][v], acc[mi][2 * np + 1][v]));
                    }
            }
        }
    }
}

template <class TL, int EPI>
hipError_t launch_bf16_pipe_tile(const uint16_t* A, const uint16_t* Bw, uint16_t* C, const int32_t* offsets,
                                 int R, int E, int N, int K, int ldc, hipStream_t s) {
    const long mt_bound = (long)R / TL::BM + (long)min(E, R);
    const long tiles = mt_bound * ((N + TL::BN - 1) / TL::BN);
    long g = min(tiles, 256L);
    g = max((g + kXcds - 1) / kXcds * kXcds, (long)kXcds);
    hipLaunchKernelGGL((gemm_bf16_pipe_kernel<TL, EPI>), dim3((unsigned)g), dim3(TL::NTHR), 0, s, A, Bw, C,
                       offsets, E, N, K, ldc);
    return hipGetLastError();
}

using PipeBig = PipeTile<256, 256, 2, 4>;
using PipeBig4 = PipeTile<256, 256, 2, 2>;

hipError_t launch_bf16_pipe(int epi, const uint16_t* A, const uint16_t* Bw, uint16_t* C, const int32_t* offsets,
                            int R, int E, int N, int K, int ldc, hipStream_t s) {
    if (epi == 1) return launch_bf16_pipe_tile<PipeBig, 1>(A, Bw, C, offsets, R, E, N, K, ldc, s);
    return launch_bf16_pipe_tile<PipeBig, 0>(A, Bw, C, offsets, R, E, N, K, ldc, s);
}

}  // namespace moe
