// Pipelined grouped GEMMs for gfx950: direct global -> LDS loads feeding a
// four-stage LDS ring; bf16 (v_mfma_f32_32x32x16_bf16) and MXFP8
// (v_mfma_scale_f32_32x32x64_f8f6f4) variants.
//
// Contract shared with the rest of the library: the rows of expert e are the
// segment [offsets[e], offsets[e+1]) of the expert-major activation buffer,
// read from device memory (grouped_sched.h derives the tile schedule on the
// device; no padding to a common capacity), weights are packed [E][N][K] with
// the contraction axis contiguous, and GEMM1's N axis interleaves 32 gate
// columns with the matching 32 up columns so SwiGLU runs in the epilogue.
//
// Data movement.  Every 16-byte chunk of a K slice goes from global memory
// straight into LDS with global_load_lds_dwordx4 (lane l of a wave writes LDS
// bytes [16 l, 16 l + 16) of a wave-uniform 1 KB block), so no registers are
// spent on staging and three K slices are in flight while a fourth is
// consumed.  The loads are issued from inline asm with an SGPR base and a
// 32-bit lane offset: the compiler spends one VGPR per load and never makes
// LDS reads wait for them; all waits on them are the explicit wait_vm below.
// (The compiler's own vmcnt waits stay correct, only more conservative,
// because vector loads retire in order.)
//
// Stage layout: BM rows of A then BN rows of B, each row one 64-byte K slice
// (32 bf16 or 64 fp8 values) = 4 chunks; chunk c of row r is stored at
// c ^ ((r >> 2) & 3), which keeps the 16 rows read by each 16-lane group of a
// fragment load on distinct banks (16 lanes of a ds_read_b128 are served per
// cycle from 64 banks).  One ring array with a runtime stage offset keeps the
// fragment addresses to a few lane bases plus immediates.
//
// Schedule of one K-tile kt (two bf16 k-steps, or one fp8 k-step):
// multiply the fragments already in registers; with those MFMAs queued, wait
// for K-tile kt + 1, join the barrier (everyone is done with K-tile kt - 1),
// start the DMA of K-tile kt + 3 into that stage, and read K-tile kt + 1's
// fragments.  The barrier is a bare s_barrier: __syncthreads() would add a
// release fence that waits for every DMA in flight.
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

// 16 bytes per lane from base + voff into LDS bytes [lds + 16 lane, +16).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// 4 bytes per lane from base + voff into LDS dword [lds + 4 lane].
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier for the ring: the stage a wave reads next was waited for
// with wait_vm, and the fragments it read last were consumed by MFMAs before
// it arrives, so no fence is needed; the empty asm statements keep the
// compiler from moving LDS accesses across it.
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

// Interleave R fragment reads with M MFMAs in the scheduling region.
template <int R, int M>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
    for (int i = 0; i < R; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, (M + R - 1) / R, 0);        // then MFMAs
    }
}

}  // namespace

// Tile geometry shared by both element types: BM x BN workgroup tile, WM x WN
// waves, 64-byte K slices in a 4-stage ring.
template <int BM_, int BN_, int WM_, int WN_>
struct RingTile {
    static constexpr int BM = BM_, BN = BN_, STAGES = 4, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN, NTHR = 64 * NW;
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static constexpr int WROWS = BM / WM, WCOLS = BN / WN;
    static constexpr int A_DMA = BM / 16 / NW, B_DMA = BN / 16 / NW;   // 1 KB blocks per wave per stage
    static constexpr int P = A_DMA + B_DMA;                            // data DMAs per wave per K-tile
    static constexpr int STAGE_CHUNKS = (BM + BN) * 4;                 // 16-byte chunks per stage
    static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "stage / wave mismatch");
    static_assert(TN % 2 == 0, "a wave's N range must hold whole gate/up pairs");
};

// Per-thread state of the ring: global bases (wave-uniform) and this lane's
// DMA offsets for K-tile 0.
template <class TL>
struct Ring {
    const void* Ag;
    const void* Bg;
    uint32_t offA[TL::A_DMA], offB[TL::B_DMA];
    uint32_t ring_lds;      // LDS byte address of the ring
    int nk, wave, lane;

    // DMA of K-tile kt (64 bytes of every row) into stage kt % 4.
    __device__ __forceinline__ void issue(int kt) const {
        const uint32_t ko = (uint32_t)kt * 64u;
        const uint32_t st = ring_lds + (uint32_t)(kt & 3) * TL::STAGE_CHUNKS * 16u;
        const uint32_t la = __builtin_amdgcn_readfirstlane(st + wave * TL::A_DMA * 1024u);
        const uint32_t lb = __builtin_amdgcn_readfirstlane(st + TL::BM * 64u + wave * TL::B_DMA * 1024u);
#pragma unroll
        for (int i = 0; i < TL::A_DMA; ++i) dma16(Ag, offA[i] + ko, la + i * 1024u);
#pragma unroll
        for (int i = 0; i < TL::B_DMA; ++i) dma16(Bg, offB[i] + ko, lb + i * 1024u);
    }
};

// ============================================================================ bf16

// One ring stage holds 32 K values per row: two 16-wide k-steps; lane l's
// fragment for k-step s is chunk 2 s + l / 32 of its row.
template <class TL>
__device__ __forceinline__ void bf_load(const u32x4* stage, int aoff, int boff, bf16x8 (&fa)[TL::TM],
                                        bf16x8 (&fb)[TL::TN]) {
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) fa[mi] = __builtin_bit_cast(bf16x8, stage[aoff + mi * 128]);
#pragma unroll
    for (int ni = 0; ni < TL::TN; ++ni) fb[ni] = __builtin_bit_cast(bf16x8, stage[boff + ni * 128]);
}

template <class TL>
__device__ __forceinline__ void bf_mfma(const bf16x8 (&fa)[TL::TM], const bf16x8 (&fb)[TL::TN],
                                        f32x16 (&acc)[TL::TM][TL::TN]) {
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
}

template <class TL, int EPI>   // EPI 0: C = A B (bf16);  1: C = silu(A Bgate) * (A Bup) (bf16, N/2 columns)
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_bf16_pipe_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                           uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, int E, int N, int K,
                           int ldc) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    __shared__ u32x4 ring[TL::STAGES * TL::STAGE_CHUNKS];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];

    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const uint32_t rowbytes = (uint32_t)K * 2u;

    Ring<TL> rg;
    rg.lane = threadIdx.x & 63;
    rg.wave = threadIdx.x >> 6;
    rg.nk = K / 32;
    rg.Ag = A;
    rg.ring_lds = lds_addr(ring);
    const int wm = rg.wave / TL::WN, wn = rg.wave % TL::WN;
    const int fsw = ((rg.lane & 31) >> 2) & 3, half = rg.lane >> 5;
    const int arow = (wm * TL::WROWS + (rg.lane & 31)) * 4, brow = (BM + wn * TL::WCOLS + (rg.lane & 31)) * 4;
    const int a0 = arow + ((0 + half) ^ fsw), a1 = arow + ((2 + half) ^ fsw);
    const int b0 = brow + ((0 + half) ^ fsw), b1 = brow + ((2 + half) ^ fsw);
    const int drow = rg.lane >> 2;
    const uint32_t dchunk = (uint32_t)((rg.lane & 3) ^ ((rg.lane >> 4) & 3)) * 16u;

    for (int tile = xcd_slot(blockIdx.x, G); tile < total; tile += G) {
        const int mt = tile / NT, nt = tile - mt * NT;
        const int e = tile_expert(s_tstart, E, mt);
        const int row0 = offsets[e] + (mt - s_tstart[e]) * BM;
        const int rows = min(BM, offsets[e + 1] - row0);
        const int n0 = nt * BN;
        rg.Bg = B + (size_t)__builtin_amdgcn_readfirstlane(e) * N * K;
#pragma unroll
        for (int i = 0; i < TL::A_DMA; ++i) {
            const int r = 16 * (rg.wave * TL::A_DMA + i) + drow;
            rg.offA[i] = (uint32_t)(row0 + min(r, rows - 1)) * rowbytes + dchunk;
        }
#pragma unroll
        for (int i = 0; i < TL::B_DMA; ++i) {
            const int r = 16 * (rg.wave * TL::B_DMA + i) + drow;
            rg.offB[i] = (uint32_t)min(n0 + r, N - 1) * rowbytes + dchunk;
        }
        ring_barrier();   // every wave is done reading the previous tile's stages
        rg.issue(0);
        if (rg.nk > 1) rg.issue(1);
        if (rg.nk > 2) rg.issue(2);

        f32x16 acc[TM][TN];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        if (rg.nk > 2) wait_vm<2 * TL::P>();
        else if (rg.nk > 1) wait_vm<TL::P>();
        else wait_vm<0>();
        ring_barrier();
        bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
        bf_load<TL>(ring, a0, b0, fa0, fb0);
        for (int kt = 0; kt < rg.nk; ++kt) {
            const u32x4* cur = ring + (kt & 3) * TL::STAGE_CHUNKS;
            bf_load<TL>(cur, a1, b1, fa1, fb1);
            bf_mfma<TL>(fa0, fb0, acc);
            interleave_hint<TM + TN, TM * TN>();
            if (kt + 1 < rg.nk) {
                if (kt + 2 < rg.nk) wait_vm<TL::P>();    // K-tile kt + 2 may stay in flight
                else wait_vm<0>();
                ring_barrier();
                if (kt + 3 < rg.nk) rg.issue(kt + 3);
                bf_load<TL>(ring + ((kt + 1) & 3) * TL::STAGE_CHUNKS, a0, b0, fa0, fb0);
            }
            bf_mfma<TL>(fa1, fb1, acc);
            interleave_hint<TM + TN, TM * TN>();
        }

        // accumulator (mi, ni)[v] holds tile row wm*WROWS + mi*32 + 8*(v/4) + 4*(lane/32) + v%4
        // and tile column wn*WCOLS + ni*32 + lane%32
        const int rbase = wm * TL::WROWS + 4 * half;
        if (EPI == 0) {
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni) {
                    const int col = n0 + wn * TL::WCOLS + ni * 32 + (rg.lane & 31);
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
                const int pc = n0 + wn * TL::WCOLS + np * 64;
                if (pc >= N) continue;
                const int hcol = pc / 2 + (rg.lane & 31);
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

// ============================================================================ MXFP8
//
// Operands are E4M3 codes with one E8M0 scale per 32 K values (OCP MX v1.0).
// A ring stage holds 64 K values per row, consumed by one MFMA per fragment
// pair.  In that instruction lane l of half h = l / 32 holds, for row l % 32,
// K values [16 h, 16 h + 16) in its bytes 0..15 and [32 + 16 h, 48 + 16 h) in
// bytes 16..31, and supplies the scale of K block h: scale block b covers
// bytes 0..15 of both halves for b = 0 and bytes 16..31 for b = 1 (measured on
// gfx950).  So a lane's fragment is chunks h and 2 + h of the 64-byte slice,
// and its scale is that of block 2 kt + h.  Scales come in pairs of
// K-tiles: with every even K-tile t each wave DMAs, for its SR rows of A and
// of B, the dword of scale bytes of K blocks 2t .. 2t+3 into a two-slot scale
// ring.  Lanes of the upper half shift that dword right by one byte, so one
// op_sel (byte 0 for even K-tiles, byte 2 for odd ones) gives every lane the
// scale of its own block.  Four waves each own a 128 x 128 block whose 256
// accumulators sit in AGPRs, leaving the VGPRs to the 32-byte fragments (fp8
// halves the LDS bytes per FLOP, so the larger per-wave block suits it).
template <class TL>
struct Fp8Extra {
    static constexpr int PS = 2;                // scale DMAs per wave per even K-tile
    static constexpr int SR = TL::BM / TL::NW;  // scale rows per wave and operand
    static_assert(TL::BM == TL::BN && (SR == 32 || SR == 64), "one scale DMA per wave and operand");
};

template <class TL>
__device__ __forceinline__ void fp8_load(const u32x4* stage, const uint32_t* sslot, int aoff0, int aoff1,
                                         int boff0, int boff1, int arow, int brow, int sh, i32x8 (&fa)[TL::TM],
                                         i32x8 (&fb)[TL::TN], int (&sa)[TL::TM], int (&sb)[TL::TN]) {
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) {
        const u32x4 lo = stage[aoff0 + mi * 128], hi = stage[aoff1 + mi * 128];
        fa[mi] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sa[mi] = (int)(sslot[arow + mi * 32] >> sh);
    }
#pragma unroll
    for (int ni = 0; ni < TL::TN; ++ni) {
        const u32x4 lo = stage[boff0 + ni * 128], hi = stage[boff1 + ni * 128];
        fb[ni] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sb[ni] = (int)(sslot[TL::BM + brow + ni * 32] >> sh);
    }
}

template <class TL, int OPSEL>
__device__ __forceinline__ void fp8_mfma(const i32x8 (&fa)[TL::TM], const i32x8 (&fb)[TL::TN],
                                         const int (&sa)[TL::TM], const int (&sb)[TL::TN],
                                         f32x16 (&acc)[TL::TM][TL::TN]) {
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[mi], fb[ni], acc[mi][ni], 0, 0, OPSEL,
                                                                         sa[mi], OPSEL, sb[ni]);
}

template <class TL, int EPI>   // EPI 0: C = A B (bf16 out);  1: C = MXFP8(silu(A Bgate) * (A Bup)) along N/2
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_fp8_pipe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                          const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, void* __restrict__ C,
                          uint8_t* __restrict__ Cs, const int32_t* __restrict__ offsets, int E, int N, int K,
                          int ldc) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    constexpr int SR = Fp8Extra<TL>::SR, PS = Fp8Extra<TL>::PS;
    __shared__ u32x4 ring[TL::STAGES * TL::STAGE_CHUNKS];
    __shared__ uint32_t sring[2 * (BM + BN)];     // two scale slots: A rows then B rows
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];

    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const int kb = K / 32;            // scale bytes per row

    Ring<TL> rg;
    rg.lane = threadIdx.x & 63;
    rg.wave = threadIdx.x >> 6;
    rg.nk = K / 64;
    rg.Ag = A;
    rg.ring_lds = lds_addr(ring);
    const uint32_t sring_lds = lds_addr(sring);
    const int wm = rg.wave / TL::WN, wn = rg.wave % TL::WN;
    const int fsw = ((rg.lane & 31) >> 2) & 3, half = rg.lane >> 5;
    const int arow_i = wm * TL::WROWS + (rg.lane & 31), brow_i = wn * TL::WCOLS + (rg.lane & 31);
    const int a0 = arow_i * 4 + (half ^ fsw), a1 = arow_i * 4 + ((2 + half) ^ fsw);
    const int b0 = (BM + brow_i) * 4 + (half ^ fsw), b1 = (BM + brow_i) * 4 + ((2 + half) ^ fsw);
    const int sh = half * 8;
    const int drow = rg.lane >> 2;
    const uint32_t dchunk = (uint32_t)((rg.lane & 3) ^ ((rg.lane >> 4) & 3)) * 16u;
    const int srow = SR * rg.wave + (rg.lane & (SR - 1));    // scale DMA row of this lane
    const bool slane = rg.lane < SR;

    for (int tile = xcd_slot(blockIdx.x, G); tile < total; tile += G) {
        const int mt = tile / NT, nt = tile - mt * NT;
        const int e = tile_expert(s_tstart, E, mt);
        const int row0 = offsets[e] + (mt - s_tstart[e]) * BM;
        const int rows = min(BM, offsets[e + 1] - row0);
        const int n0 = nt * BN;
        const size_t eu = (size_t)__builtin_amdgcn_readfirstlane(e);
        rg.Bg = B + eu * N * K;
        const void* Bsg = Bs + eu * N * kb;
#pragma unroll
        for (int i = 0; i < TL::A_DMA; ++i) {
            const int r = 16 * (rg.wave * TL::A_DMA + i) + drow;
            rg.offA[i] = (uint32_t)(row0 + min(r, rows - 1)) * (uint32_t)K + dchunk;
        }
#pragma unroll
        for (int i = 0; i < TL::B_DMA; ++i) {
            const int r = 16 * (rg.wave * TL::B_DMA + i) + drow;
            rg.offB[i] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + dchunk;
        }
        const uint32_t soA = (uint32_t)(row0 + min(srow, rows - 1)) * kb;
        const uint32_t soB = (uint32_t)min(n0 + srow, N - 1) * kb;

        // data of K-tile kt, plus (kt even) the scale dwords of K-tiles kt, kt + 1 into slot (kt / 2) & 1
        auto issue = [&](int kt) {
            rg.issue(kt);
            if ((kt & 1) == 0) {
                const uint32_t slot = sring_lds + (uint32_t)((kt >> 1) & 1) * (BM + BN) * 4u;
                const uint32_t lsa = __builtin_amdgcn_readfirstlane(slot + rg.wave * SR * 4u);
                const uint32_t lsb = __builtin_amdgcn_readfirstlane(slot + BM * 4u + rg.wave * SR * 4u);
                if (slane) {
                    dma4(As, soA + (uint32_t)kt * 2u, lsa);
                    dma4(Bsg, soB + (uint32_t)kt * 2u, lsb);
                }
            }
        };

        ring_barrier();   // every wave is done reading the previous tile's stages and scales
        issue(0);
        if (rg.nk > 1) issue(1);
        if (rg.nk > 2) issue(2);

        f32x16 acc[TM][TN];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        // K-tile 0 (with scales) landed: tiles 1 (P) and 2 (P + PS) may stay in flight
        if (rg.nk > 2) wait_vm<2 * TL::P + PS>();
        else if (rg.nk > 1) wait_vm<TL::P>();
        else wait_vm<0>();
        ring_barrier();
        i32x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
        int sa0[TM], sb0[TN], sa1[TM], sb1[TN];
        fp8_load<TL>(ring, sring, a0, a1, b0, b1, arow_i, brow_i, sh, fa0, fb0, sa0, sb0);
        // nk is even (K % 128 == 0): K-tiles go in pairs (even: register set 0, op_sel 0;
        // odd: register set 1, op_sel 2), the pair's scales in slot (kt / 2) & 1
        for (int kt = 0; kt < rg.nk; kt += 2) {
            fp8_mfma<TL, 0>(fa0, fb0, sa0, sb0, acc);
            if (kt + 2 < rg.nk) wait_vm<TL::P + PS>();      // K-tile kt + 2 (with scales) may stay in flight
            else wait_vm<0>();
            ring_barrier();
            if (kt + 3 < rg.nk) issue(kt + 3);
            fp8_load<TL>(ring + ((kt + 1) & 3) * TL::STAGE_CHUNKS, sring + ((kt >> 1) & 1) * (BM + BN), a0, a1, b0,
                         b1, arow_i, brow_i, sh, fa1, fb1, sa1, sb1);
            interleave_hint<2 * (TM + TN), TM * TN>();
            fp8_mfma<TL, 2>(fa1, fb1, sa1, sb1, acc);
            if (kt + 2 < rg.nk) {
                if (kt + 3 < rg.nk) wait_vm<TL::P>();        // K-tile kt + 3 may stay in flight
                else wait_vm<0>();
                ring_barrier();
                if (kt + 4 < rg.nk) issue(kt + 4);
                fp8_load<TL>(ring + ((kt + 2) & 3) * TL::STAGE_CHUNKS, sring + (((kt + 2) >> 1) & 1) * (BM + BN), a0,
                             a1, b0, b1, arow_i, brow_i, sh, fa0, fb0, sa0, sb0);
                interleave_hint<2 * (TM + TN), TM * TN>();
            }
        }

        const int rbase = wm * TL::WROWS + 4 * half;
        if (EPI == 0) {
            uint16_t* Cb = static_cast<uint16_t*>(C);
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni) {
                    const int col = n0 + wn * TL::WCOLS + ni * 32 + (rg.lane & 31);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = rbase + mi * 32 + 8 * (v >> 2) + (v & 3);
                        if (r < rows && col < N)
                            Cb[(size_t)(row0 + r) * ldc + col] = f32_to_bf16(acc[mi][ni][v]);
                    }
                }
        } else {
            // SwiGLU values of one gate/up column pair (32 h columns) of this
            // wave's rows go through a per-wave LDS region of the ring; each lane
            // then quantises whole 32-value blocks of a row and stores 32 codes
            // with two 16-byte stores plus the block's scale byte.
            ring_barrier();     // every wave is past its last fragment read
            static_assert(TL::WROWS * 32 * 4 * TL::NW <= TL::STAGES * TL::STAGE_CHUNKS * 16, "staging region");
            float* reg = reinterpret_cast<float*>(ring) + rg.wave * TL::WROWS * 32;
            uint8_t* Cq = static_cast<uint8_t*>(C);
#pragma unroll
            for (int np = 0; np < TN / 2; ++np) {
                const int pc = n0 + wn * TL::WCOLS + np * 64;
                // [WROWS rows][32 columns], column c of row r at c ^ (r & 31)
#pragma unroll
                for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                        reg[r * 32 + ((rg.lane & 31) ^ (r & 31))] =
                            silu_mul_p(acc[mi][2 * np][v], acc[mi][2 * np + 1][v]);
                    }
                if (pc < N) {
                    const int hb = pc / 64;              // 32-wide h block of this pair
                    for (int r = rg.lane; r < TL::WROWS; r += 64) {
                        const int grow = wm * TL::WROWS + r;
                        float x[32];
                        float amax = 0.f;
#pragma unroll
                        for (int c = 0; c < 32; ++c) {
                            x[c] = reg[r * 32 + (c ^ (r & 31))];
                            amax = fmaxf(amax, fabsf(x[c]));
                        }
                        const int se = mx_shared_exp(amax);
                        const float inv = mx_inv_scale(se);
                        uint32_t w[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q)
                            w[q] = e4m3_encode(x[4 * q] * inv) | (e4m3_encode(x[4 * q + 1] * inv) << 8) |
                                   (e4m3_encode(x[4 * q + 2] * inv) << 16) | (e4m3_encode(x[4 * q + 3] * inv) << 24);
                        if (grow < rows) {
                            u32x4* dst = reinterpret_cast<u32x4*>(Cq + (size_t)(row0 + grow) * ldc + hb * 32);
                            dst[0] = (u32x4){w[0], w[1], w[2], w[3]};
                            dst[1] = (u32x4){w[4], w[5], w[6], w[7]};
                            Cs[(size_t)(row0 + grow) * (ldc / 32) + hb] = (uint8_t)(se + 127);
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();   // the region is rewritten for the next pair
            }
        }
    }
}

// ============================================================================ launchers

template <class TL>
static unsigned ring_grid(int R, int E, int N) {
    const long mt_bound = (long)R / TL::BM + (long)min(E, R);
    const long tiles = mt_bound * ((N + TL::BN - 1) / TL::BN);
    long g = min(tiles, 256L);
    return (unsigned)max((g + kXcds - 1) / kXcds * kXcds, (long)kXcds);
}

template <class TL, int EPI>
hipError_t launch_bf16_pipe_tile(const uint16_t* A, const uint16_t* Bw, uint16_t* C, const int32_t* offsets,
                                 int R, int E, int N, int K, int ldc, hipStream_t s) {
    hipLaunchKernelGGL((gemm_bf16_pipe_kernel<TL, EPI>), dim3(ring_grid<TL>(R, E, N)), dim3(TL::NTHR), 0, s, A, Bw,
                       C, offsets, E, N, K, ldc);
    return hipGetLastError();
}

template <class TL, int EPI>
hipError_t launch_fp8_pipe_tile(const uint8_t* A, const uint8_t* As, const uint8_t* Bw, const uint8_t* Bs,
                                void* C, uint8_t* Cs, const int32_t* offsets, int R, int E, int N, int K, int ldc,
                                hipStream_t s) {
    hipLaunchKernelGGL((gemm_fp8_pipe_kernel<TL, EPI>), dim3(ring_grid<TL>(R, E, N)), dim3(TL::NTHR), 0, s, A, As,
                       Bw, Bs, C, Cs, offsets, E, N, K, ldc);
    return hipGetLastError();
}

using BfRing = RingTile<256, 256, 2, 4>;    // 8 waves of 128 x 64
using Fp8Ring = RingTile<256, 256, 2, 2>;   // 4 waves of 128 x 128

hipError_t launch_bf16_pipe(int epi, const uint16_t* A, const uint16_t* Bw, uint16_t* C, const int32_t* offsets,
                            int R, int E, int N, int K, int ldc, hipStream_t s) {
    if (epi == 1) return launch_bf16_pipe_tile<BfRing, 1>(A, Bw, C, offsets, R, E, N, K, ldc, s);
    return launch_bf16_pipe_tile<BfRing, 0>(A, Bw, C, offsets, R, E, N, K, ldc, s);
}

hipError_t launch_fp8_pipe(int epi, const uint8_t* A, const uint8_t* As, const uint8_t* Bw, const uint8_t* Bs,
                           void* C, uint8_t* Cs, const int32_t* offsets, int R, int E, int N, int K, int ldc,
                           hipStream_t s) {
    if (epi == 1) return launch_fp8_pipe_tile<Fp8Ring, 1>(A, As, Bw, Bs, C, Cs, offsets, R, E, N, K, ldc, s);
    return launch_fp8_pipe_tile<Fp8Ring, 0>(A, As, Bw, Bs, C, Cs, offsets, R, E, N, K, ldc, s);
}

}  // namespace moe
