// Pipelined grouped GEMMs for gfx950: direct global -> LDS loads feeding an
// LDS ring; bf16 (v_mfma_f32_32x32x16_bf16) and MXFP8
// (v_mfma_scale_f32_32x32x64_f8f6f4) variants.
//
// Contract shared with the rest of the library: the rows of expert e are the
// segment [offsets[e], offsets[e+1]) of the expert-major activation buffer,
// read from device memory (grouped_sched.h derives the tile schedule on the
// device; no padding to a common capacity), weights are packed [E][N][K] with
// the contraction axis contiguous, and GEMM1's N axis interleaves 32 gate
// columns with the matching 32 up columns so SwiGLU runs in the epilogue.
// Called from the whole-block forward, GEMM1 takes expert-major row r from
// the token matrix (bf16 x, or the MXFP8 codes of each token) at row
// row_token[r] instead of from a dispatched copy: each tile's row_token
// entries are DMA'd into an LDS row table a tile or two ahead, and each lane
// turns its A rows into byte offsets once per loop phase.
//
// Data movement.  Every 16-byte chunk of a K slice goes from global memory
// straight into LDS with global_load_lds_dwordx4 (lane l of a wave writes LDS
// bytes [16 l, 16 l + 16) of a wave-uniform 1 KB block), so no registers are
// spent on staging.  The loads are issued from inline asm with an SGPR base
// and a 32-bit lane offset: the compiler spends one VGPR per load and never
// makes LDS reads wait for them; all waits on them are the explicit wait_vm
// below.  (The compiler's own vmcnt waits stay correct, only more
// conservative, because vector loads retire in order.)
//
// Two ring geometries.  The kernels that carry the large blocks (the fused
// bf16 FFN, the fused backward chain, the MXFP8 GEMMs) stream K-tiles of 128
// bytes per row (64 bf16 or 128 fp8 values) in two stages: each DMA
// instruction then moves 8 whole 128-byte lines, so the requests to L2 carry
// twice the bytes they carry with half lines (measured 2-5% faster).  Chunk c
// (of 8) of row r sits at c ^ ((r >> 1) & 7).  The plain bf16 kernel (small d
// or H) keeps K-tiles of 64 bytes (32 values) in
// four stages, chunk c (of 4) of row r at c ^ ((r >> 2) & 3).  Both swizzles
// keep the 16 rows read by each 16-lane group of a fragment load on distinct
// banks (16 lanes of a ds_read_b128 are served per cycle from 64 banks).  One
// ring array with a runtime stage offset keeps the fragment addresses to a
// few lane bases plus immediates.
//
// Schedule of one K-tile: multiply the k-steps whose fragments are in
// registers while reading the next k-step's, then issue a few MFMAs of the
// last k-step, wait for the next K-tile, join the barrier (every wave has all
// of this K-tile in registers by then, so its stage is free), start the DMAs
// of the K-tile one ring length ahead into that stage, and read the next
// K-tile's first fragments between the remaining MFMAs.  The two-stage
// kernels issue only the A blocks (and scales) there and the B blocks between
// the next K-tile's first MFMAs, from the same source: the DMAs slow the
// MFMAs beside them less when spread out (measured 1-3% faster); a tile's
// last K-tile issues its B blocks before the epilogue, and the next tile's
// first K-tile issues them again (identical weight bytes into the same place,
// landed before that K-tile's wait), which keeps the loop free of branches.
// The weight-gradient kernel likewise issues a K-tile's B rows after its first
// k-step's MFMAs.  The barrier is a
// bare s_barrier: __syncthreads() would add a release fence that waits for
// every DMA in flight.  Every issue starts the same number of loads (past the
// last K-tile the loads are clamped and land in a stage nobody reads again),
// so the vmcnt waits are constants and the loop body has no branches.
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

// A wave-uniform pointer forced into SGPRs (the asm operands below need SGPRs
// whatever the compiler's uniformity analysis concludes).
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from base + voff into LDS bytes [lds + 16 lane, +16).
// M0 is set inside each statement; it is listed as clobbered for the reader
// (the compiler treats M0 as reserved and warns that it ignores the entry: no
// code of these kernels keeps a value in M0, LDS instructions on gfx950 do not
// read it, and the only DMAs are these statements).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sgpr_ptr(base))
                 : "memory", "m0");
}

// 4 bytes per lane from base + voff into LDS dword [lds + 4 lane].
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sgpr_ptr(base))
                 : "memory", "m0");
}

// s_waitcnt lgkmcnt(0): every LDS access this wave issued has completed.
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
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

// silu(g) * u with the hardware reciprocal (1 ulp) in place of a division.
__device__ __forceinline__ float silu_mul_p(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
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
    static constexpr int NM = TM * TN;                                 // MFMAs per wave per k-step
    static constexpr int EARLY = TN;                                   // MFMAs issued before a barrier
    static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "stage / wave mismatch");
    static_assert(TN % 2 == 0, "a wave's N range must hold whole gate/up pairs");
};

// Rows and columns of one output tile.  The expert index is wave-uniform, so
// the offsets reads are scalar loads.
struct TileCoord {
    int row0, rows, n0, e;
};

template <int BM, int BN>
__device__ __forceinline__ TileCoord tile_coord(int tile, int MT, int NT, const int* s_tstart, int E,
                                                const int32_t* __restrict__ offsets) {
    int mt, nt;
    block_tile(tile, MT, NT, mt, nt);
    TileCoord c;
    c.e = __builtin_amdgcn_readfirstlane(tile_expert(s_tstart, E, mt));
    const int o0 = offsets[c.e], o1 = offsets[c.e + 1];
    c.row0 = o0 + (mt - __builtin_amdgcn_readfirstlane(s_tstart[c.e])) * BM;
    c.rows = min(BM, o1 - c.row0);
    c.n0 = nt * BN;
    return c;
}

// Source of the K-tiles a loop phase prefetches.  A tile's K loop runs in two
// phases: while kt + 4 < nk the stream prefetches the current tile (kt = rel),
// and in the last four K-tiles it prefetches the tile q ahead (q = 1, or 2
// when a tile has only two K-tiles), kt = rel - q nk; past the last tile the
// current tile's last K-tile stands in (its copy lands in a stage nobody reads
// again).  The K-tile is kt = rel * mul + add, so the loop bodies need no
// selects or branches (a branch there would let the compiler move MFMAs away
// from the loads they are meant to hide).
struct StreamSrc {
    TileCoord t;
    int mul, add;
};


// Output layout.  The MFMAs take the weight fragment as their first operand
// and the activation fragment as their second, so accumulator (mi, ni) is the
// transposed 32 x 32 block: lane l holds tile row mi*32 + l%32 and, in element
// v, tile column ni*32 + 8*(v/4) + 4*(l/32) + v%4.  Each lane thus owns runs of
// four consecutive columns of one row; one v_permlane32_swap per pair of runs
// gives lane halves 0 and 1 the low and high 16 columns of a 32-column block.
//
// w0..w3: the four runs (q = 0..3) of one 32-column block as 32-bit words of
// this lane; on return lane half 0 holds columns 0..15 and half 1 columns
// 16..31 of the block, in order.
__device__ __forceinline__ void gather_halves(uint32_t (&w)[4]) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    w[0] = s02[0];
    w[1] = s02[1];
    w[2] = s13[0];
    w[3] = s13[1];
}

// Cache policy of a device-scope store (sc1): the encoding of an agent-scope
// store on gfx950, complete only once it is coherent across the XCDs' L2s.
constexpr int kCpolSc1 = 16;
// Buffer resource word 3 of a raw (unformatted) gfx9 buffer.
constexpr int kRawBufferWord3 = 0x00020000;
// Two bfloat16 quiet NaNs: the stored output of a tile whose input rows were
// not seen complete (the bounded wait of the fused grouped GEMMs gave up).
constexpr uint32_t kBf16NanPair = 0x7FC07FC0u;

__device__ __forceinline__ void poison_words(uint32_t (&w)[4], bool poison) {
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = poison ? kBf16NanPair : w[q];
}

// bf16 block store: the 16 values of acc (one 32 x 32 block, this lane's row)
// as bf16 columns [col0, col0 + 32) of row `grow` of C (if the row is valid).
// DEV: the two 16-byte stores go through the raw buffer resource `rc` over C
// with device scope (byte offsets past its size are dropped by the hardware).
template <bool DEV = false>
__device__ __forceinline__ void store_bf16_block(uint16_t* __restrict__ C, size_t ldc, int grow, bool valid,
                                                 int col0, const float (&v)[16],
                                                 __amdgpu_buffer_rsrc_t rc = __amdgpu_buffer_rsrc_t(),
                                                 bool poison = false) {
    uint32_t lo[4], hi[4];   // run q: columns 8q + 4 half + (0, 1) and (2, 3)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        lo[q] = pack_bf16x2(v[4 * q], v[4 * q + 1]);
        hi[q] = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
    }
    poison_words(lo, poison);
    poison_words(hi, poison);
    gather_halves(lo);
    gather_halves(hi);
    // half 0: columns 0..15 = runs (w0 = q0 lo/hi of half 0, w1 = q0 of half 1, ...)
    const int half = (threadIdx.x >> 5) & 1;
    if (valid) {
        if constexpr (DEV) {
            const uint32_t off = (uint32_t)((size_t)grow * ldc + col0 + 16 * half) * 2u;
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){lo[0], hi[0], lo[1], hi[1]}, rc, off, 0, kCpolSc1);
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){lo[2], hi[2], lo[3], hi[3]}, rc, off + 16u, 0, kCpolSc1);
        } else {
            u32x4* dst = reinterpret_cast<u32x4*>(C + (size_t)grow * ldc + col0 + 16 * half);
            dst[0] = (u32x4){lo[0], hi[0], lo[1], hi[1]};
            dst[1] = (u32x4){lo[2], hi[2], lo[3], hi[3]};
        }
    }
}

// Row-contiguous device-scope store of one 32 x 32 bf16 block (the 16 values
// of acc of this lane's row, columns [col0, col0 + 32) of rows row0 .. row0 +
// 31; rows at or past nrows and the whole block when !col_ok are skipped):
// the block goes through this wave's LDS buffer `buf` (32 rows x 4 chunks of
// 16 bytes, chunk c of row q at q * 4 + (c ^ (q & 3))) and is read back so that
// 4 lanes cover one row's 64 bytes, which reach memory as whole 64-byte
// segments instead of 16-byte pieces.  The buffer is private to the wave (see
// store_bf16_pair_rows).
__device__ __forceinline__ void store_bf16_block_rows_dev(int row0, int nrows, size_t ldc, int col0, bool col_ok,
                                                          const float (&v)[16], u32x4* __restrict__ buf,
                                                          __amdgpu_buffer_rsrc_t rc, bool poison) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, half = lane >> 5;
    uint32_t lo[4], hi[4];   // run q: columns 8q + 4 half + (0, 1) and (2, 3)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        lo[q] = pack_bf16x2(v[4 * q], v[4 * q + 1]);
        hi[q] = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
    }
    poison_words(lo, poison);
    poison_words(hi, poison);
    gather_halves(lo);
    gather_halves(hi);
    // this lane: row r, columns 16 half .. 16 half + 15 = chunks 2 half, 2 half + 1
    const int sw = r & 3;
    buf[r * 4 + ((2 * half) ^ sw)] = (u32x4){lo[0], hi[0], lo[1], hi[1]};
    buf[r * 4 + ((2 * half + 1) ^ sw)] = (u32x4){lo[2], hi[2], lo[3], hi[3]};
    asm volatile("" ::: "memory");
    wait_lds();
    asm volatile("" ::: "memory");
    u32x4 o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = 16 * j + (lane >> 2), c = lane & 3;
        o[j] = buf[q * 4 + (c ^ (q & 3))];
    }
    asm volatile("" ::: "memory");   // the next block's writes stay after these reads
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = 16 * j + (lane >> 2), c = lane & 3;
        if (q < nrows && col_ok)
            __builtin_amdgcn_raw_buffer_store_b128(o[j], rc, (uint32_t)((size_t)(row0 + q) * ldc + col0 + 8 * c) * 2u,
                                                   0, kCpolSc1);
    }
}

// Row-contiguous store of a 32 x 64 bf16 block pair (blocks g and u, columns
// [pc, pc + 64) of 32 rows starting at global row `row0`; rows at or past
// `nrows` and blocks at or past column N are skipped).  In the MFMA layout
// each lane holds one row, so a direct store puts 32 rows into every
// instruction; instead the pair goes through this wave's LDS buffer `buf`
// (RR x 8 chunks of 16 bytes, RR = rows per round, 16 or 32) and is read back
// so that 8 lanes cover one 128-byte row segment: every store instruction
// then writes whole 128-byte lines of 64 / 8 rows.  Chunk c of buffer row q
// sits at q * 8 + (c ^ (q & 7)) to spread the writes over the LDS banks.
// The buffer is private to the wave, so a wait for the wave's own LDS writes
// (and compiler barriers: lanes read what other lanes wrote) stand in for a
// workgroup barrier.  DEV: the 16-byte stores go through the raw buffer
// resource `rc` over C with device scope (see store_bf16_block).  COUNTED:
// every lane issues each of its 32 / 8 stores, through `rc` whose base is the
// row `rofs` rows above row0 (a tile's first row) and whose size, `oob`
// bytes, ends at that tile's last row; a lane with nothing to store gives the
// offset `oob`, past the resource, where the hardware drops the store.  So a
// call always issues the same number of store instructions, which callers
// count in vmcnt.
template <int RR, bool DEV = false, bool COUNTED = false>
__device__ __forceinline__ void store_bf16_pair_rows(uint16_t* __restrict__ C, size_t ldc, int row0, int nrows,
                                                     int pc, int N, const float (&g)[16], const float (&u)[16],
                                                     u32x4* __restrict__ buf,
                                                     __amdgpu_buffer_rsrc_t rc = __amdgpu_buffer_rsrc_t(),
                                                     bool poison = false, int rofs = 0, uint32_t oob = 0) {
    static_assert(RR == 16 || RR == 32, "rows per round");
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, half = lane >> 5;
    u32x4 ch[4];   // chunks 2 half, 2 half + 1 (block g) and 4 + 2 half, 4 + 2 half + 1 (block u)
    {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lo[q] = pack_bf16x2(g[4 * q], g[4 * q + 1]);
            hi[q] = pack_bf16x2(g[4 * q + 2], g[4 * q + 3]);
        }
        poison_words(lo, poison);
        poison_words(hi, poison);
        gather_halves(lo);
        gather_halves(hi);
        ch[0] = (u32x4){lo[0], hi[0], lo[1], hi[1]};
        ch[1] = (u32x4){lo[2], hi[2], lo[3], hi[3]};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lo[q] = pack_bf16x2(u[4 * q], u[4 * q + 1]);
            hi[q] = pack_bf16x2(u[4 * q + 2], u[4 * q + 3]);
        }
        poison_words(lo, poison);
        poison_words(hi, poison);
        gather_halves(lo);
        gather_halves(hi);
        ch[2] = (u32x4){lo[0], hi[0], lo[1], hi[1]};
        ch[3] = (u32x4){lo[2], hi[2], lo[3], hi[3]};
    }
    const int wq = r % RR, wsw = wq & 7;
    const int c = lane & 7;                  // chunk this lane stores
    const bool col_ok = pc + 32 * (c >> 2) < N;
#pragma unroll
    for (int rho = 0; rho < 32 / RR; ++rho) {
        if (r / RR == rho) {
            buf[wq * 8 + ((2 * half) ^ wsw)] = ch[0];
            buf[wq * 8 + ((2 * half + 1) ^ wsw)] = ch[1];
            buf[wq * 8 + ((4 + 2 * half) ^ wsw)] = ch[2];
            buf[wq * 8 + ((5 + 2 * half) ^ wsw)] = ch[3];
        }
        asm volatile("" ::: "memory");
        wait_lds();
        asm volatile("" ::: "memory");
        u32x4 o[RR / 8];
#pragma unroll
        for (int j = 0; j < RR / 8; ++j) {
            const int q = 8 * j + (lane >> 3);
            o[j] = buf[q * 8 + (c ^ (q & 7))];
        }
        asm volatile("" ::: "memory");   // the next round's writes stay after these reads
#pragma unroll
        for (int j = 0; j < RR / 8; ++j) {
            const int rr = rho * RR + 8 * j + (lane >> 3);
            if constexpr (COUNTED) {
                const uint32_t off = rr < nrows && col_ok ? (uint32_t)((rofs + rr) * ldc + pc + 8 * c) * 2u : oob;
                __builtin_amdgcn_raw_buffer_store_b128(o[j], rc, off, 0, 0);
            } else if (rr < nrows && col_ok) {
                if constexpr (DEV)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        o[j], rc, (uint32_t)((size_t)(row0 + rr) * ldc + pc + 8 * c) * 2u, 0, kCpolSc1);
                else
                    *reinterpret_cast<u32x4*>(C + (size_t)(row0 + rr) * ldc + pc + 8 * c) = o[j];
            }
        }
    }
}

// One accumulator block into VGPRs, at this point of the program: the reads
// are volatile, so the compiler neither hoists all of them to the start of the
// epilogue (which would need 256 VGPRs at once) nor reorders them across the
// stores between blocks.
__device__ __forceinline__ void acc_read(const f32x16& a, float (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[i]) : "a"(a[i]));
}

// Accumulator block of a tile geometry: waves of 128 x 128 (one wave per SIMD)
// keep their 256 accumulators in AGPRs and read them block by block; smaller
// wave tiles keep them in VGPRs.
template <class TL>
__device__ __forceinline__ void acc_block(const f32x16& a, float (&v)[16]) {
    if constexpr (TL::TM * TL::TN >= 16) {
        acc_read(a, v);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = a[i];
    }
}

// ============================================================================ bf16

// One ring stage holds 32 K values per row: two 16-wide k-steps; lane l's
// fragment for k-step s is chunk 2 s + l / 32 of its row.

// Epilogue of the bf16 kernel.  EPI 0: C = acc as bf16.  EPI 1: columns come
// in gate/up pairs of 32; C column (pair column)/2 + j = silu(gate_j) * up_j.
// EPI 2 (SwiGLU backward): the gate/up pairs a, b are rounded to bf16 (the
// values a stored recompute would hold) and, with dh [rows][N/2] (aux), C
// receives da = dh b s (1 + a (1 - s)), db = dh a s, s = sigmoid(a), in the
// layout of a | b.  The dh values of all of a wave's rows are requested
// before any is used.  EPI 3 (SwiGLU backward from stored pre-activations):
// acc holds dh over N hidden units; it is rounded to bf16 (the value the
// recomputing path stores), a | b are read back from aux [rows][2N] (the
// packed layout above), and C receives da | db as EPI 2 computes them, so the
// two paths agree bit for bit when the stored a | b are the recompute's
// values.  DEV: every store goes through the raw buffer resource
// rc over C with device scope (the fused grouped GEMMs, whose next phase reads
// C on other XCDs while the kernel runs).
template <class TL, int EPI, bool DEV = false>
__device__ __forceinline__ void bf_epilogue(const f32x16 (&acc)[TL::TM][TL::TN], uint16_t* __restrict__ C,
                                            int ldc, int N, const TileCoord& c, int wm, int wn,
                                            u32x4* __restrict__ obuf, const uint16_t* __restrict__ aux,
                                            __amdgpu_buffer_rsrc_t rc = __amdgpu_buffer_rsrc_t(),
                                            bool poison = false) {
    const int lane = threadIdx.x & 63;
    static_assert(EPI != 2 || TL::TN == 2, "one gate/up pair per wave row block");
    static_assert(EPI != 3 || TL::WCOLS % 32 == 0, "whole 32-unit hidden blocks per wave");
    uint32_t dhw[EPI == 2 ? TL::TM : 1][4][2];   // dh runs: [mi][q] = 4 bf16 of h 8 q + 4 half + 0..3
    if (EPI == 2) {
        // the wave's 32 hidden units (clamped for a pair past N, whose stores are skipped)
        const int hb = min((c.n0 + wn * TL::WCOLS) / 2, N / 2 - 32) + 4 * (lane >> 5);
#pragma unroll
        for (int mi = 0; mi < TL::TM; ++mi) {
            const int r = min(wm * TL::WROWS + mi * 32 + (lane & 31), c.rows - 1);   // clamped rows not stored
            const uint16_t* src = aux + (size_t)(c.row0 + r) * (N / 2) + hb;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint2 w = *reinterpret_cast<const uint2*>(src + 8 * q);
                dhw[mi][q][0] = w.x;
                dhw[mi][q][1] = w.y;
            }
        }
    }
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) {
        const int r = wm * TL::WROWS + mi * 32 + (lane & 31);
        const bool valid = r < c.rows;
        if (EPI == 3) {
            const int rc_row = min(r, c.rows - 1);   // clamped rows are read, not stored
            const uint16_t* src = aux + (size_t)(c.row0 + rc_row) * (2 * N);
            uint32_t abw[TL::TN][2][4][2];   // [block][a, b][q] = 4 bf16 of units 8 q + 4 half + 0..3
#pragma unroll
            for (int ni = 0; ni < TL::TN; ++ni) {
                const int u0 = min(c.n0 + wn * TL::WCOLS + ni * 32, N - 32);   // a block past N is not stored
#pragma unroll
                for (int ab = 0; ab < 2; ++ab)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint2 w = *reinterpret_cast<const uint2*>(src + 2 * u0 + 32 * ab + 8 * q + 4 * (lane >> 5));
                        abw[ni][ab][q][0] = w.x;
                        abw[ni][ab][q][1] = w.y;
                    }
            }
#pragma unroll
            for (int ni = 0; ni < TL::TN; ++ni) {
                float g[16], u[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t wa = abw[ni][0][i / 4][(i % 4) / 2], wb = abw[ni][1][i / 4][(i % 4) / 2];
                    const float a = __uint_as_float((i & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
                    const float b = __uint_as_float((i & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
                    const float d = bf16_round(acc[mi][ni][i]);
                    const float sg = 1.0f / (1.0f + __expf(-a));
                    g[i] = d * b * (sg * (1.0f + a * (1.0f - sg)));
                    u[i] = d * (a * sg);
                }
                const int rb = wm * TL::WROWS + mi * 32;
                store_bf16_pair_rows<16, DEV>(C, (size_t)ldc, c.row0 + rb, c.rows - rb,
                                              2 * (c.n0 + wn * TL::WCOLS + ni * 32), 2 * N, g, u, obuf, rc, poison);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (EPI == 2) {
            float g[16], u[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = bf16_round(acc[mi][0][i]), b = bf16_round(acc[mi][1][i]);
                const uint32_t w = dhw[mi][i / 4][(i % 4) / 2];
                const float d = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
                const float sg = 1.0f / (1.0f + __expf(-a));
                g[i] = d * b * (sg * (1.0f + a * (1.0f - sg)));
                u[i] = d * (a * sg);
            }
            const int rb = wm * TL::WROWS + mi * 32;
            store_bf16_pair_rows<16, DEV>(C, (size_t)ldc, c.row0 + rb, c.rows - rb, c.n0 + wn * TL::WCOLS, N, g, u,
                                          obuf, rc, poison);
        } else if (EPI == 0) {
#pragma unroll
            for (int np = 0; np < TL::TN / 2; ++np) {
                float g[16], u[16];
                acc_block<TL>(acc[mi][2 * np], g);
                acc_block<TL>(acc[mi][2 * np + 1], u);
                const int rb = wm * TL::WROWS + mi * 32;   // tile row of the block's row 0
                store_bf16_pair_rows<16, DEV>(C, (size_t)ldc, c.row0 + rb, c.rows - rb,
                                              c.n0 + wn * TL::WCOLS + np * 64, N, g, u, obuf, rc, poison);
                __builtin_amdgcn_sched_barrier(0);   // one block pair's values in VGPRs at a time
            }
        } else {
#pragma unroll
            for (int np = 0; np < TL::TN / 2; ++np) {
                const int pc = c.n0 + wn * TL::WCOLS + np * 64;
                float v[16], u[16];
                acc_block<TL>(acc[mi][2 * np], v);
                acc_block<TL>(acc[mi][2 * np + 1], u);
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = silu_mul_p(v[i], u[i]);
                if constexpr (DEV) {
                    const int rb = wm * TL::WROWS + mi * 32;   // tile row of the block's row 0
                    store_bf16_block_rows_dev(c.row0 + rb, c.rows - rb, (size_t)ldc, pc / 2, pc < N, v, obuf, rc, poison);
                } else {
                    store_bf16_block<false>(C, (size_t)ldc, c.row0 + r, valid && pc < N, pc / 2, v, rc, poison);
                }
                __builtin_amdgcn_sched_barrier(0);   // one block pair's values in VGPRs at a time
            }
        }
    }
}

// MFMA number i (row-major over (mi, ni)); i is a constant after unrolling.
template <class TL>
__device__ __forceinline__ void bf_mfma1(int i, const bf16x8 (&fa)[TL::TM], const bf16x8 (&fb)[TL::TN],
                                         f32x16 (&acc)[TL::TM][TL::TN]) {
    const int mi = i / TL::TN, ni = i % TL::TN;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ni], fa[mi], acc[mi][ni], 0, 0, 0);
}

// The persistent bf16 kernel streams K-tiles without a break at tile
// boundaries, like the MXFP8 one below: global K-tile g of this workgroup goes
// through ring stage g % 4, and the DMAs of a tile's last four K-tiles fetch
// the next tile's first four.  A K-tile holds two k-steps.  k-step 0 (set 0,
// read during the previous K-tile) multiplies while k-step 1 is read into
// set 1; then a few MFMAs of set 1, the wait for K-tile g + 1 and the barrier
// (every wave holds all of K-tile g in registers by then, so its stage is
// free), and, one per MFMA, the DMAs of K-tile g + 4 and the reads of K-tile
// g + 1's k-step 0 into set 0.  The epilogue runs between tiles while the
// next tile's first K-tiles are in flight; its stores count in vmcnt after
// those DMAs, which only makes later waits wait longer.
// EPI 0: C = A B (bf16);  1: C = silu(A Bgate) * (A Bup) (bf16, N/2 columns);
// 2: C = the SwiGLU backward of (A Bgate, A Bup) given dh = aux (bf16, N columns)
template <class TL, int EPI>
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_bf16_pipe_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                           uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, int E, int N, int K,
                           int ldc, const uint16_t* __restrict__ aux) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    constexpr int NM = TL::NM, EARLY = TL::EARLY, P = TL::P, SC = TL::STAGE_CHUNKS;
    constexpr int A_DMA = TL::A_DMA, B_DMA = TL::B_DMA;
    static_assert(NM - EARLY >= P && NM >= TM + TN && NM - EARLY >= TM + TN, "one DMA / fragment per MFMA step");
    constexpr int kObufChunks = EPI != 1 ? 128 : 0;   // per wave: 16 rows x 128 bytes of output
    __shared__ u32x4 ring[TL::STAGES * SC];
    __shared__ u32x4 obuf[kObufChunks ? TL::NW * kObufChunks : 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];

    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const uint32_t rowbytes = (uint32_t)K * 2u;
    const int nk = K / 32;
    int tile = xcd_slot(blockIdx.x, G);
    if (tile >= total) return;

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ring_lds = lds_addr(ring);
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    const int fsw = ((lane & 31) >> 2) & 3, half = lane >> 5;
    const int arow = (wm * TL::WROWS + (lane & 31)) * 4, brow = (BM + wn * TL::WCOLS + (lane & 31)) * 4;
    const int a0 = arow + ((0 + half) ^ fsw), a1 = arow + ((2 + half) ^ fsw);
    const int b0 = brow + ((0 + half) ^ fsw), b1 = brow + ((2 + half) ^ fsw);
    const int drow = lane >> 2;
    const uint32_t dchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) * 16u;

    TileCoord c0 = tile_coord<BM, BN>(tile, MT, NT, s_tstart, E, offsets), c1 = c0, c2 = c0;
    if (tile + G < total) c1 = tile_coord<BM, BN>(tile + G, MT, NT, s_tstart, E, offsets);
    if (tile + 2 * G < total) c2 = tile_coord<BM, BN>(tile + 2 * G, MT, NT, s_tstart, E, offsets);
    int kbase = 0;
    const int qa = nk >= 4 ? 1 : 2;   // tiles ahead reached by the last four K-tiles' prefetches
    const int head = max(nk - 4, 0);  // K-tiles whose prefetch stays in the current tile

    // DMA i of global K-tile g (A rows, then B rows) from src.
    auto dma = [&](const StreamSrc& src, int g, int i) {
        const TileCoord& t = src.t;
        const int kt = (g - kbase) * src.mul + src.add;
        const uint32_t st = ring_lds + (uint32_t)(g & 3) * SC * 16u;
        if (i < A_DMA) {
            const int r = 16 * (wave * A_DMA + i) + drow;
            const uint32_t off = (uint32_t)(t.row0 + min(r, t.rows - 1)) * rowbytes + dchunk + (uint32_t)kt * 64u;
            dma16(A, off, st + (uint32_t)(wave * A_DMA + i) * 1024u);
        } else {
            const int j = i - A_DMA;
            const int r = 16 * (wave * B_DMA + j) + drow;
            const uint32_t off = (uint32_t)min(t.n0 + r, N - 1) * rowbytes + dchunk + (uint32_t)kt * 64u;
            dma16(B + (size_t)t.e * N * K, off, st + BM * 64u + (uint32_t)(wave * B_DMA + j) * 1024u);
        }
    };
    auto frag = [&](const u32x4* stage, int aoff, int boff, int i, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
        if (i < TM) fa[i] = __builtin_bit_cast(bf16x8, stage[aoff + i * 128]);
        else if (i < TM + TN) fb[i - TM] = __builtin_bit_cast(bf16x8, stage[boff + (i - TM) * 128]);
    };

    // prologue: K-tiles 0..3 of the stream (for two-K-tile tiles, 2 and 3 are the next tile's)
    {
        const StreamSrc here{c0, 1, 0};
        const bool has1 = tile + G < total;
        const StreamSrc ahead{has1 ? c1 : c0, has1 ? 1 : 0, has1 ? -nk : nk - 1};
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < P; ++i) dma(g < nk ? here : ahead, g, i);
    }
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    wait_vm<3 * P>();   // K-tile 0 landed; 1, 2 and 3 may stay in flight
    ring_barrier();
#pragma unroll
    for (int i = 0; i < TM + TN; ++i) frag(ring, a0, b0, i, fa0, fb0);

    // One K-tile g: k-step 0 (set 0, read during the previous K-tile) multiplies
    // while k-step 1 is read into set 1; then a few MFMAs of set 1, the wait for
    // K-tile g + 1 and the barrier, and, one per MFMA, the DMAs of K-tile g + 4
    // (from src) and the reads of K-tile g + 1's k-step 0 into set 0.
    auto ktile = [&](int g, const StreamSrc& src, f32x16 (&acc)[TM][TN]) {
        const u32x4* stage = ring + (g & 3) * SC;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa0, fb0, acc);
            frag(stage, a1, b1, i, fa1, fb1);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < EARLY; ++i) bf_mfma1<TL>(i, fa1, fb1, acc);
        wait_vm<2 * P>();   // K-tile g + 1 landed; g + 2 and g + 3 may stay in flight
        wait_lds();         // this wave's reads of K-tile g are complete
        ring_barrier();
        const u32x4* nstage = ring + ((g + 1) & 3) * SC;
#pragma unroll
        for (int i = 0; i < NM - EARLY; ++i) {
            bf_mfma1<TL>(EARLY + i, fa1, fb1, acc);
            if (i < P) dma(src, g + 4, i);
            frag(nstage, a0, b0, i, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    for (;;) {
        f32x16 acc[TM][TN];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        const StreamSrc here{c0, 1, 0};
        for (int kt = 0; kt < head; ++kt) ktile(kbase + kt, here, acc);
        const bool has = tile + qa * G < total;
        const StreamSrc ahead{has ? (qa == 1 ? c1 : c2) : c0, has ? 1 : 0, has ? -qa * nk : nk - 1};
        for (int kt = head; kt < nk; ++kt) ktile(kbase + kt, ahead, acc);

        // set 0 now holds k-step 0 of the next tile's first K-tile
        bf_epilogue<TL, EPI>(acc, C, ldc, N, c0, wm, wn, obuf + wave * kObufChunks, aux);
        if (tile + G >= total) break;
        tile += G;
        c0 = c1;
        c1 = c2;
        if (tile + 2 * G < total) c2 = tile_coord<BM, BN>(tile + 2 * G, MT, NT, s_tstart, E, offsets);
        kbase += nk;
    }
    wait_vm<0>();   // no DMA may land in LDS after the workgroup has left
}

// ============================================================================ fused bf16 grouped GEMMs
//
// Up to three grouped GEMMs over the same expert segments in one persistent
// launch, each phase's M tile depending on the previous phase's tiles of the
// same rows.  The phase-table kernel below runs the backward chain: dh = dye
// W_down^T, then the gate/up recompute with the SwiGLU backward in its
// epilogue (da | db, reading dh), then dxe = (da | db) W1^T.  The forward's
// GEMM1 (h = silu(xe W_gate) * (xe W_up)) then GEMM2 (ye = h W_down) follows
// the same design with the two phases written out (gemm_bf16_ffn_kernel,
// after this one).  So no phase ends in a round of tiles on a partly idle chip: with 256
// workgroups and, say, 1040 tiles per GEMM, separate launches each end in a
// round of 16 tiles, while here the workgroups that finish their share of one
// phase go straight on to the next.  The schedule stays device-resident (the
// group sizes never reach the host) and the launch boundaries between the
// projections disappear.
//
// Tile ids: phase 0 takes [0, T0), phase 1 [T0, T0 + T1), ... (M tile major,
// NTp = Np / BN tiles per M tile).  Every tile is computed whole, in the same K
// order and with the same epilogue as by gemm_bf16_pipe_kernel, so the results
// are bitwise those of separate launches, whatever the grid.
//
// Scheduling.  Workgroup b works for "XCD" x = b % 8 (the hardware deals
// workgroups round-robin over the 8 XCDs).  The ids up to the last multiple
// of 256 form blocks of 32 consecutive ids (4 M tiles x 8 N tiles, or 2 x 16),
// and XCD x takes every 8th block from block x, so the tiles running together
// on one XCD share rows and weight slices in its L2; the remaining ids (less
// than one round) are dealt in blocks of 4 the same way, so that every XCD
// gets the same number of tiles.  Within an XCD's sequence the tiles are handed
// out dynamically from a counter (sync[x]): each workgroup holds two tiles
// ahead (the next one is prefetched across the tile boundary; the one after is
// claimed at the end of every tile and read back at the end of the next, by
// when it has long returned, so the atomic's latency never stalls the K loop).
// Placement only affects speed: every ticket maps to one tile, whichever
// workgroup draws it.
//
// Dependencies.  A tile of phase p > 0 and M tile mt reads rows that the NT
// tiles of phase p - 1 and M tile mt write.  Those tiles store with device
// scope (sc1, the encoding of an agent-scope store on gfx950), so a store is
// coherent across the XCDs' L2s once it is complete and no L2 write-back is
// needed; at the end of such a tile every wave waits for its stores, and after
// a barrier one lane adds 1 to the phase's counter of mt.  Before the
// cross-tile prefetch of a dependent tile, wave 0 copies the counter into LDS
// with a device-scope direct-to-LDS load issued among the K-tile DMAs (so its
// completion is covered by the ring's own vmcnt waits and every wave reads the
// same value after a barrier).  If the count is complete the prefetch goes
// ahead; if not, the prefetch slots take a dummy copy and, after the current
// tile's epilogue, the workgroup spins (bounded, with s_sleep) until the count
// is complete, acquires, and restarts the stream.  No workgroup can wait on
// itself (the dependency is only checked for the next tile after the current
// one is finished), and a waiting workgroup holds no unfinished tile of an
// earlier phase (it draws ids in increasing order and earlier phases' ids come
// first), so every wait ends once the earlier tiles, all held by running
// workgroups, are done; the spin bound ends it regardless.  The rows an M tile
// of one phase writes are read by nobody before its count is complete (rows
// are clamped inside each tile), so no cache can hold a stale copy of them.
// The wait is bounded: one lane spins (with s_sleep) on the counter and
// shares the outcome with the workgroup through LDS; if the bound is reached
// the lane raises the error word and the whole tile, computed on rows it could
// not see complete, stores NaN instead of its values, so a caller can detect
// the failure (the error word) and no wrong value passes for a right one.
// sync layout (int32, zeroed before the launch): [0, 8) per-XCD tile
// counters, word kSyncErrWord the error word, then from kSyncHead one array
// of MTmax counters per phase that others wait on.
constexpr int kFusedMaxPhases = 3;

// Epilogue kinds of a fused phase.
enum FusedEpi : int {
    kEpiPlain = 0,     // C = A B (bf16)
    kEpiSwiglu = 1,    // C = silu(A Bgate) * (A Bup)
    kEpiDswiglu = 2,   // C = SwiGLU backward of (A Bgate, A Bup) given dh = aux
    kEpiDswigluKept = 3,   // C = SwiGLU backward of the stored a | b (aux) given dh = A B
};

// An instantiation compiles the epilogues of the (kind, device scope) pairs in
// its KINDS mask only, bit 2 epi + dev, so the forward's kernel does not carry
// the SwiGLU backward's registers.
constexpr int fused_kind_bit(int epi, int dev) { return 1 << (2 * epi + dev); }
constexpr int kFusedBackwardKinds =
    fused_kind_bit(kEpiPlain, 1) | fused_kind_bit(kEpiDswiglu, 1) | fused_kind_bit(kEpiPlain, 0);
constexpr int kFusedBackwardKeptKinds = fused_kind_bit(kEpiDswigluKept, 1) | fused_kind_bit(kEpiPlain, 0);

struct FusedPhase {
    const uint16_t* a;      // A rows [R][K]
    const uint16_t* b;      // B [E][N][K]
    uint16_t* c;            // C [R][ldc]
    const uint16_t* aux;    // kEpiDswiglu: dh [R][N/2]; kEpiDswigluKept: a | b [R][2N]
    int32_t* done;          // counters raised per finished tile (NULL: none)
    const int32_t* need;    // counters of the previous phase waited on (NULL: none)
    int N, K, ldc, epi;
    int need_count;         // tiles of the previous phase per M tile
    int dev;                // stores with device scope (a later phase reads C)
};

struct FusedParams {
    FusedPhase ph[kFusedMaxPhases];
    int nph;
    const int32_t* offsets;
    int32_t* sync;
    int R, E;
    uint32_t spin_limit;
    int force_wait;   // test hook: treat every dependent tile's rows as not yet done at the early check
};

struct FfnTile {
    int row0, rows, n0, e, mt, phase;   // phase -1: no tile
};

// Id of ticket q of XCD x: blocks of 32 ids over the first 256 k32 ids, then
// blocks of 4; XCD x takes every 8th block.
__device__ __forceinline__ int ffn_ticket_id(int x, int q, int k32) {
    if (q < 32 * k32) return 256 * (q >> 5) + 32 * x + (q & 31);
    const int r = q - 32 * k32;
    return 256 * k32 + 32 * (r >> 2) + 4 * x + (r & 3);
}

template <int BM, int BN>
__device__ __forceinline__ FfnTile ffn_tile(const FusedParams& p, int id, int MT, const int* s_tstart) {
    FfnTile c{0, 1, 0, 0, 0, -1};
    int j = id;
    for (int q = 0; q < p.nph; ++q) {
        const int nt_per = (p.ph[q].N + BN - 1) / BN;
        if (j < MT * nt_per) {
            int nt;
            c.phase = q;
            block_tile(j, MT, nt_per, c.mt, nt);
            c.n0 = nt * BN;
            break;
        }
        j -= MT * nt_per;
    }
    if (c.phase < 0) return c;
    // everything below is wave-uniform; saying so keeps it in SGPRs (and the
    // buffer resources built from it out of waterfall loops)
    c.phase = __builtin_amdgcn_readfirstlane(c.phase);
    c.mt = __builtin_amdgcn_readfirstlane(c.mt);
    c.n0 = __builtin_amdgcn_readfirstlane(c.n0);
    c.e = __builtin_amdgcn_readfirstlane(tile_expert(s_tstart, p.E, c.mt));
    const int o0 = p.offsets[c.e], o1 = p.offsets[c.e + 1];
    c.row0 = o0 + (c.mt - __builtin_amdgcn_readfirstlane(s_tstart[c.e])) * BM;
    c.rows = min(BM, o1 - c.row0);
    return c;
}

// K-tile source of one loop phase (see StreamSrc): K-tile kt = rel * mul + add
// of the tile's rows of A and its weight slice B (the expert's packed matrix).
struct FfnSrc {
    const uint16_t* a;
    const uint16_t* b;
    uint32_t rowbytes;
    int row0, rows, n0, nmax, mul, add;
    int gather;   // the tile's A rows are rows s_tab[tab + r] of a (token rows), else rows row0 + r
    int tab;      // first entry of the tile's row table in LDS
};

// Built once per loop phase and wave-uniform throughout (pinned to SGPRs, so
// the K loop does not re-derive the DMA bases from the phase table).
__device__ __forceinline__ FfnSrc ffn_src(const FusedParams& p, const FfnTile& t, int mul, int add) {
    const FusedPhase& q = p.ph[t.phase];
    const int N = __builtin_amdgcn_readfirstlane(q.N), K = __builtin_amdgcn_readfirstlane(q.K);
    FfnSrc s;
    s.a = static_cast<const uint16_t*>(sgpr_ptr(q.a));
    s.b = static_cast<const uint16_t*>(sgpr_ptr(q.b + (size_t)t.e * N * K));
    s.rowbytes = (uint32_t)K * 2u;
    s.nmax = N;
    s.row0 = __builtin_amdgcn_readfirstlane(t.row0);
    s.rows = __builtin_amdgcn_readfirstlane(t.rows);
    s.n0 = t.n0;
    s.mul = mul;
    s.add = __builtin_amdgcn_readfirstlane(add);
    s.gather = 0;
    s.tab = 0;
    return s;
}

// 4 bytes per lane from base + voff into LDS dword [lds + 4 lane], device
// scope (sc1): the load observes atomics performed by other XCDs.
__device__ __forceinline__ void dma4_dev(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 sc1"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sgpr_ptr(base))
                 : "memory", "m0");
}

// One lane's bounded wait for *count >= need: at most `limit` sleeps of 512
// cycles (limit 0: gives up at once without looking, the test hook).  On
// giving up it sets the error word and returns 0; otherwise 1.
__device__ __forceinline__ int bounded_wait(const int32_t* count, int need, uint32_t limit, int32_t* err) {
    for (uint32_t it = 0;; ++it) {
        if (it >= limit) {
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return 0;
        }
        if (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) return 1;
        __builtin_amdgcn_s_sleep(8);
    }
}

template <class TL>
struct Ring128 {
    static constexpr int A_DMA = TL::BM / 8 / TL::NW, B_DMA = TL::BN / 8 / TL::NW;   // 1 KB DMAs per wave
    static constexpr int P = A_DMA + B_DMA;                                            // per wave per K-tile
    static constexpr int SC = (TL::BM + TL::BN) * 8;                                   // 16-byte chunks per stage
    static_assert(TL::BM % (8 * TL::NW) == 0 && TL::BN % (8 * TL::NW) == 0 && A_DMA % 2 == 0 && B_DMA % 2 == 0,
                  "DMA blocks of 8 rows, an even number per wave");
};

template <class TL, int KINDS>
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_bf16_fused_kernel(FusedParams p) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    constexpr int NM = TL::NM, EARLY = TL::EARLY;
    constexpr int A_DMA = Ring128<TL>::A_DMA, B_DMA = Ring128<TL>::B_DMA, P = Ring128<TL>::P, SC = Ring128<TL>::SC;
    constexpr int SL = NM - EARLY;   // MFMA slots after the barrier of a K-tile
    static_assert(NM >= TM + TN && SL >= TM + TN && SL > 0, "one fragment read per MFMA slot");
    constexpr int kObufChunks = 128;   // per wave: 16 rows x 128 bytes of row-contiguous output
    __shared__ u32x4 ring[2 * SC];
    __shared__ u32x4 obuf[TL::NW * kObufChunks];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];
    __shared__ int s_flag[64];
    __shared__ int s_next;
    __shared__ int s_ok;

    const int MT = __builtin_amdgcn_readfirstlane(build_tile_schedule<BM, NTHR>(p.offsets, p.E, s_tstart, s_scan));
    int total = 0;
    for (int q = 0; q < p.nph; ++q) total += MT * ((p.ph[q].N + BN - 1) / BN);
    const int G = gridDim.x, GX = G / kXcds;   // G is a multiple of 8
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int k32 = total / 256;
    const int id0 = ffn_ticket_id(xcd, slot, k32);
    if (id0 >= total) return;
    const int id1 = ffn_ticket_id(xcd, slot + GX, k32);

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ring_lds = lds_addr(ring);
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    const int key = ((lane & 31) >> 1) & 7, half = lane >> 5;
    const int arow = (wm * TL::WROWS + (lane & 31)) * 8, brow = (BM + wn * TL::WCOLS + (lane & 31)) * 8;
    int aoff[4], boff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        aoff[s] = arow + ((2 * s + half) ^ key);
        boff[s] = brow + ((2 * s + half) ^ key);
    }
    const int drow = lane >> 3;
    const uint32_t dch0 = (uint32_t)((lane & 7) ^ (drow >> 1)) * 16u;
    const uint32_t dch1 = (uint32_t)((lane & 7) ^ (4 + (drow >> 1))) * 16u;

    // the ticket after the two static ones, claimed now and read back at the end of the first tile
    int pending = total;
    if (threadIdx.x == 0 && id1 < total)
        pending = ffn_ticket_id(xcd, 2 * GX + __hip_atomic_fetch_add(p.sync + xcd, 1, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT), k32);

    FfnTile c0 = ffn_tile<BM, BN>(p, id0, MT, s_tstart);
    FfnTile c1 = ffn_tile<BM, BN>(p, id1, MT, s_tstart);
    int kbase = 0;

    auto dma = [&](const FfnSrc& src, int g, int i) {
        const int kt = (g - kbase) * src.mul + src.add;
        const uint32_t st = ring_lds + (uint32_t)(g & 1) * SC * 16u;
        const uint32_t dch = (i & 1) ? dch1 : dch0;
        if (i < A_DMA) {
            const int r = 8 * (wave * A_DMA + i) + drow;
            const uint32_t off = (uint32_t)(src.row0 + min(r, src.rows - 1)) * src.rowbytes + dch + (uint32_t)kt * 128u;
            dma16(src.a, off, st + (uint32_t)(wave * A_DMA + i) * 1024u);
        } else {
            const int j = i - A_DMA;
            const int r = 8 * (wave * B_DMA + j) + drow;
            const uint32_t off = (uint32_t)min(src.n0 + r, src.nmax - 1) * src.rowbytes + dch + (uint32_t)kt * 128u;
            dma16(src.b, off, st + BM * 128u + (uint32_t)(wave * B_DMA + j) * 1024u);
        }
    };
    auto frag = [&](const u32x4* stage, int s, int i, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
        if (i < TM) fa[i] = __builtin_bit_cast(bf16x8, stage[aoff[s] + i * 32 * 8]);
        else if (i < TM + TN) fb[i - TM] = __builtin_bit_cast(bf16x8, stage[boff[s] + (i - TM) * 32 * 8]);
    };
    // tile t may start once the previous phase's tiles of its rows are done;
    // false if the bounded wait gave up (error word raised)
    auto wait_rows = [&](const FfnTile& t) -> bool {
        const int32_t* need = p.ph[t.phase].need;
        if (!need) return true;
        if (threadIdx.x == 0)
            s_ok = bounded_wait(need + t.mt, p.ph[t.phase].need_count, p.spin_limit, p.sync + kSyncErrWord);
        wait_lds();
        ring_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return __builtin_amdgcn_readfirstlane(s_ok) != 0;
    };
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    // (re)start the K-tile stream at the first K-tile of tile t (global K-tile kbase)
    auto start_stream = [&](const FfnTile& t) {
        const FfnSrc here = ffn_src(p, t, 1, 0);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < P; ++i) dma(here, kbase + g, i);
        wait_vm<P>();   // the first K-tile landed; the second may stay in flight
        ring_barrier();
#pragma unroll
        for (int i = 0; i < TM + TN; ++i) frag(ring + (kbase & 1) * SC, 0, i, fa0, fb0);
    };

    bool poison = !wait_rows(c0);   // the current tile's rows were not seen complete
    start_stream(c0);

    // one K-tile g of four k-steps, as in gemm_bf16_ffn_kernel below
    auto ktile = [&](int g, const FfnSrc& src, const FfnSrc& prev, f32x16 (&acc)[TM][TN]) {
        const u32x4* stage = ring + (g & 1) * SC;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa0, fb0, acc);
            frag(stage, 1, i, fa1, fb1);
            // the B blocks of K-tile g + 1 (from prev), as in gemm_bf16_ffn_kernel
            if (i % (NM / B_DMA) == NM / B_DMA - 1) dma(prev, g + 1, A_DMA + i / (NM / B_DMA));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa1, fb1, acc);
            frag(stage, 2, i, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa0, fb0, acc);
            frag(stage, 3, i, fa1, fb1);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < EARLY; ++i) bf_mfma1<TL>(i, fa1, fb1, acc);
        wait_vm<0>();   // K-tile g + 1 landed (the only DMAs in flight)
        wait_lds();     // this wave's reads of K-tile g are complete
        ring_barrier();
        const u32x4* nstage = ring + ((g + 1) & 1) * SC;
#pragma unroll
        for (int i = 0; i < SL; ++i) {
            bf_mfma1<TL>(EARLY + i, fa1, fb1, acc);
#pragma unroll
            for (int j = i * A_DMA / SL; j < (i + 1) * A_DMA / SL; ++j) dma(src, g + 2, j);
            frag(nstage, 0, i, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    for (;;) {
        f32x16 acc[TM][TN];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        const int nk = __builtin_amdgcn_readfirstlane(p.ph[c0.phase].K / 64);
        const int head = nk - 2;
        // The count of the next tile's M tile is copied into LDS before K-tile
        // head - 1's wait, which then covers it.
        const int32_t* need1 = c1.phase >= 0 ? p.ph[c1.phase].need : nullptr;
        const bool probe = need1 != nullptr && head >= 1;
        const int split = probe ? head - 1 : head;
        const FfnSrc here = ffn_src(p, c0, 1, 0);
        for (int kt = 0; kt < split; ++kt) ktile(kbase + kt, here, here, acc);
        if (probe && wave == 0) dma4_dev(need1, (uint32_t)c1.mt * 4u, lds_addr(s_flag));
        for (int kt = split; kt < head; ++kt) ktile(kbase + kt, here, here, acc);
        const int flag = __builtin_amdgcn_readfirstlane(s_flag[0]);
        const bool go = c1.phase >= 0 &&
                        (need1 == nullptr || (probe && flag >= p.ph[c1.phase].need_count && !p.force_wait));
        const FfnSrc ahead = go ? ffn_src(p, c1, 1, -nk) : ffn_src(p, c0, 0, nk - 1);
        for (int kt = head; kt < nk; ++kt) ktile(kbase + kt, ahead, kt == head ? here : ahead, acc);
        // the B blocks of the last K-tile's DMAs, before the epilogue (see gemm_bf16_ffn_kernel)
#pragma unroll
        for (int j = A_DMA; j < P; ++j) dma(ahead, kbase + nk + 1, j);
        {
            FusedPhase q = p.ph[c0.phase];
            q.c = static_cast<uint16_t*>(const_cast<void*>(sgpr_ptr(q.c)));
            q.aux = static_cast<const uint16_t*>(sgpr_ptr(q.aux));
            q.N = __builtin_amdgcn_readfirstlane(q.N);
            q.ldc = __builtin_amdgcn_readfirstlane(q.ldc);
            q.epi = __builtin_amdgcn_readfirstlane(q.epi);
            q.dev = __builtin_amdgcn_readfirstlane(q.dev);
            const TileCoord tc{c0.row0, c0.rows, c0.n0, c0.e};
            u32x4* const ob = obuf + wave * kObufChunks;
            // C is [R][ldc] bf16 (below 4 GiB, checked on the host)
            const __amdgpu_buffer_rsrc_t rc =
                __builtin_amdgcn_make_buffer_rsrc(q.c, 0, (int)((uint32_t)p.R * (uint32_t)q.ldc * 2u), kRawBufferWord3);
            const int kind = fused_kind_bit(q.epi, q.dev);
            if ((KINDS & fused_kind_bit(kEpiSwiglu, 1)) && kind == fused_kind_bit(kEpiSwiglu, 1))
                bf_epilogue<TL, 1, true>(acc, q.c, q.ldc, q.N, tc, wm, wn, ob, nullptr, rc, poison);
            else if ((KINDS & fused_kind_bit(kEpiDswiglu, 1)) && kind == fused_kind_bit(kEpiDswiglu, 1))
                bf_epilogue<TL, 2, true>(acc, q.c, q.ldc, q.N, tc, wm, wn, ob, q.aux, rc, poison);
            else if ((KINDS & fused_kind_bit(kEpiDswigluKept, 1)) && kind == fused_kind_bit(kEpiDswigluKept, 1))
                bf_epilogue<TL, 3, true>(acc, q.c, q.ldc, q.N, tc, wm, wn, ob, q.aux, rc, poison);
            else if ((KINDS & fused_kind_bit(kEpiPlain, 1)) && kind == fused_kind_bit(kEpiPlain, 1))
                bf_epilogue<TL, 0, true>(acc, q.c, q.ldc, q.N, tc, wm, wn, ob, nullptr, rc, poison);
            else
                bf_epilogue<TL, 0, false>(acc, q.c, q.ldc, q.N, tc, wm, wn, ob, nullptr, rc, poison);
        }

        // tile end: a counted tile's stores complete (coherent at device
        // scope), the ticket claimed one tile ago published, the tile counted
        int32_t* const done0 = p.ph[c0.phase].done;
        if (done0) wait_vm<0>();
        if (threadIdx.x == 0) s_next = pending;
        wait_lds();
        ring_barrier();
        if (threadIdx.x == 0 && done0)
            __hip_atomic_fetch_add(done0 + c0.mt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int id2 = __builtin_amdgcn_readfirstlane(s_next);
        if (threadIdx.x == 0 && id2 < total)
            pending = ffn_ticket_id(xcd, 2 * GX + __hip_atomic_fetch_add(p.sync + xcd, 1, __ATOMIC_RELAXED,
                                                                           __HIP_MEMORY_SCOPE_AGENT), k32);
        if (c1.phase < 0) break;
        kbase += nk;
        c0 = c1;
        c1 = ffn_tile<BM, BN>(p, id2, MT, s_tstart);
        poison = false;
        if (!go) {
            // the next tile's first K-tiles were not prefetched: wait for its
            // rows, let the dummy copies land, and restart the stream there
            poison = !wait_rows(c0);
            wait_vm<0>();
            ring_barrier();
            start_stream(c0);
        }
    }
    wait_vm<0>();   // no DMA may land in LDS after the workgroup has left
}

// ---------------------------------------------------------------------------- forward, two phases
//
// The forward's expert FFN (GEMM1 with the SwiGLU epilogue into h, then GEMM2
// into ye) has its own kernel with the two phases written out rather than read
// from a phase table: the same schedule, dependency counters and per-tile
// computation as gemm_bf16_fused_kernel, but every per-phase value is a kernel
// argument or a select on them, which keeps the DMA bases in SGPRs.  Measured
// on one box against the phase-table kernel running the same two phases: 395
// against 413 us for the bf16_e8 block's FFN.
struct FfnParams {
    const uint16_t* xe;          // dispatched rows [R][d], or
    const uint16_t* x;           // with row_token: token rows [T][d] read in place of xe
    const int32_t* row_token;    // [R]: token of each expert-major row, or NULL
    const uint16_t* w1;
    uint16_t* h;
    const uint16_t* w2;
    uint16_t* ye;
    uint16_t* ab;                // KEEP: the gate/up pre-activations [R][2H] (bf16 of GEMM1's accumulators)
    const int32_t* offsets;
    int32_t* sync;
    int R, E, d, H;
    uint32_t spin_limit;
    int force_wait;   // test hook: treat every GEMM2 tile's rows as not yet done at the early check
};

template <int BM, int BN>
__device__ __forceinline__ FfnTile ffn_tile(int id, int total, int T1, int NT1, int NT2, const int* s_tstart, int E,
                                            const int32_t* __restrict__ offsets) {
    FfnTile c{0, 1, 0, 0, 0, -1};
    if (id >= total) return c;
    const bool two = id >= T1;
    const int j = two ? id - T1 : id, nt_per = two ? NT2 : NT1;
    int nt;
    block_tile(j, T1 / NT1, nt_per, c.mt, nt);
    c.phase = two ? 1 : 0;
    c.e = __builtin_amdgcn_readfirstlane(tile_expert(s_tstart, E, c.mt));
    const int o0 = offsets[c.e], o1 = offsets[c.e + 1];
    c.row0 = o0 + (c.mt - __builtin_amdgcn_readfirstlane(s_tstart[c.e])) * BM;
    c.rows = min(BM, o1 - c.row0);
    c.n0 = nt * BN;
    return c;
}

__device__ __forceinline__ FfnSrc ffn_src(const FfnParams& p, const FfnTile& t, int mul, int add, int tab) {
    FfnSrc s;
    const bool one = t.phase != 1;
    const bool gather = one && p.row_token != nullptr;
    s.a = one ? (gather ? p.x : p.xe) : p.h;
    s.gather = gather;
    s.tab = tab;
    s.b = one ? p.w1 + (size_t)t.e * (2 * p.H) * p.d : p.w2 + (size_t)t.e * p.d * p.H;
    s.rowbytes = (uint32_t)(one ? p.d : p.H) * 2u;
    s.nmax = one ? 2 * p.H : p.d;
    s.row0 = t.row0;
    s.rows = t.rows;
    s.n0 = t.n0;
    s.mul = mul;
    s.add = add;
    return s;
}

// K-tiles of 64 bf16 values.  A ring stage holds 128 bytes of K per row, so
// every global -> LDS DMA instruction moves 8 whole 128-byte lines (8 lanes per
// row) instead of 16 half lines: the L1 -> L2 path then carries twice the bytes
// per request, which is what bounds this kernel (its data movement alone takes
// most of its time).  Two stages of (BM + BN) x 128 bytes, four 16-wide
// k-steps per K-tile.  Chunk c of row r sits at chunk c ^ ((r >> 1) & 7) of
// the row, so the 16 rows read by each 16-lane group of a fragment load fall
// on 64 distinct banks, and the 8 lanes of one row of a DMA write 8 distinct
// chunks.

template <class TL, bool KEEP>
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_bf16_ffn_kernel(FfnParams p) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    constexpr int NM = TL::NM, EARLY = TL::EARLY;
    constexpr int A_DMA = Ring128<TL>::A_DMA, B_DMA = Ring128<TL>::B_DMA, P = Ring128<TL>::P, SC = Ring128<TL>::SC;
    constexpr int SL = NM - EARLY;   // MFMA slots after the barrier of a K-tile
    static_assert(NM >= TM + TN && SL >= TM + TN && SL > 0, "one fragment read per MFMA slot");
    constexpr int kObufChunks = 128;   // per wave: 16 rows x 128 bytes of GEMM2 output
    __shared__ u32x4 ring[2 * SC];
    __shared__ u32x4 obuf[TL::NW * kObufChunks];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];
    __shared__ int s_flag[64];
    __shared__ int s_next;
    __shared__ int s_ok;
    __shared__ int s_tab[2 * BM];   // token of each A row of the current and the next GEMM1 tile

    const int MT = build_tile_schedule<BM, NTHR>(p.offsets, p.E, s_tstart, s_scan);
    const int NT1 = (2 * p.H + BN - 1) / BN, NT2 = (p.d + BN - 1) / BN;
    const int T1 = MT * NT1, total = T1 + MT * NT2;
    const int nk1 = p.d / 64, nk2 = p.H / 64;
    const int G = gridDim.x, GX = G / kXcds;   // G is a multiple of 8
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int k32 = total / 256;
    const int id0 = ffn_ticket_id(xcd, slot, k32);
    if (id0 >= total) return;
    const int id1 = ffn_ticket_id(xcd, slot + GX, k32);

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ring_lds = lds_addr(ring);
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    // fragments: lane row (lane & 31) of its 32-row block, chunk 2 s + half of k-step s, swizzled
    const int key = ((lane & 31) >> 1) & 7, half = lane >> 5;
    const int arow = (wm * TL::WROWS + (lane & 31)) * 8, brow = (BM + wn * TL::WCOLS + (lane & 31)) * 8;
    int aoff[4], boff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        aoff[s] = arow + ((2 * s + half) ^ key);
        boff[s] = brow + ((2 * s + half) ^ key);
    }
    // DMA lanes: row lane / 8 of an 8-row block, physical chunk lane % 8; block i of a
    // wave starts at row 8 (wave * A_DMA + i), so the row's swizzle key is 4 (i & 1) + (lane / 8) / 2
    const int drow = lane >> 3;
    const uint32_t dch0 = (uint32_t)((lane & 7) ^ (drow >> 1)) * 16u;
    const uint32_t dch1 = (uint32_t)((lane & 7) ^ (4 + (drow >> 1))) * 16u;
    int32_t* const done = p.sync + kSyncHead;
    const __amdgpu_buffer_rsrc_t hrsrc =
        __builtin_amdgcn_make_buffer_rsrc(p.h, 0, (int)((uint32_t)p.R * (uint32_t)p.H * 2u), kRawBufferWord3);

    // the ticket after the two static ones, claimed now and read back at the end of the first tile
    int pending = total;
    if (threadIdx.x == 0 && id1 < total)
        pending = ffn_ticket_id(xcd, 2 * GX + __hip_atomic_fetch_add(p.sync + xcd, 1, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT), k32);

    FfnTile c0 = ffn_tile<BM, BN>(id0, total, T1, NT1, NT2, s_tstart, p.E, p.offsets);
    FfnTile c1 = ffn_tile<BM, BN>(id1, total, T1, NT1, NT2, s_tstart, p.E, p.offsets);
    int kbase = 0;

    // byte offsets of this lane's A rows (one per A DMA, chunk included) in a
    // source: rows of the tile's row table when gathering, else rows row0 + r;
    // taken once per loop phase, so the K loop reads no table
    struct ARows { uint32_t off[A_DMA]; };
    auto arows = [&](const FfnSrc& src) {
        ARows a;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int r = 8 * (wave * A_DMA + i) + drow;
            const int row = src.gather ? s_tab[src.tab + r] : src.row0 + min(r, src.rows - 1);
            a.off[i] = (uint32_t)row * src.rowbytes + ((i & 1) ? dch1 : dch0);
        }
        return a;
    };
    // DMA i of global K-tile g (A blocks, then B blocks) from src
    auto dma = [&](const FfnSrc& src, const ARows& ar, int g, int i) {
        const int kt = (g - kbase) * src.mul + src.add;
        const uint32_t st = ring_lds + (uint32_t)(g & 1) * SC * 16u;
        const uint32_t dch = (i & 1) ? dch1 : dch0;
        if (i < A_DMA) {
            dma16(src.a, ar.off[i] + (uint32_t)kt * 128u, st + (uint32_t)(wave * A_DMA + i) * 1024u);
        } else {
            const int j = i - A_DMA;
            const int r = 8 * (wave * B_DMA + j) + drow;
            const uint32_t off = (uint32_t)min(src.n0 + r, src.nmax - 1) * src.rowbytes + dch + (uint32_t)kt * 128u;
            dma16(src.b, off, st + BM * 128u + (uint32_t)(wave * B_DMA + j) * 1024u);
        }
    };
    // row table of GEMM1 tile t into slot `slot`: row_token of its BM rows
    // (rows past the tile clamped), DMA'd by the first BM / 64 waves; the next
    // K-tile wait and barrier cover it like the K-tile loads
    auto load_tab = [&](const FfnTile& t, int slot) {
        if (p.row_token == nullptr || t.phase != 0 || wave >= BM / 64) return;
        const int r = 64 * wave + lane;
        dma4(p.row_token, (uint32_t)(t.row0 + min(r, t.rows - 1)) * 4u, lds_addr(s_tab + slot * BM + 64 * wave));
    };
    // fragment i (A blocks, then B blocks) of k-step s from a stage
    auto frag = [&](const u32x4* stage, int s, int i, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
        if (i < TM) fa[i] = __builtin_bit_cast(bf16x8, stage[aoff[s] + i * 32 * 8]);
        else if (i < TM + TN) fb[i - TM] = __builtin_bit_cast(bf16x8, stage[boff[s] + (i - TM) * 32 * 8]);
    };
    // GEMM2 tile t may start once all NT1 GEMM1 tiles of its M tile are done;
    // false if the bounded wait gave up (error word raised)
    auto wait_rows = [&](const FfnTile& t) -> bool {
        if (t.phase != 1) return true;
        if (threadIdx.x == 0) s_ok = bounded_wait(done + t.mt, NT1, p.spin_limit, p.sync + kSyncErrWord);
        wait_lds();
        ring_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return __builtin_amdgcn_readfirstlane(s_ok) != 0;
    };
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    // (re)start the K-tile stream at the first K-tile of tile t (global K-tile kbase)
    int cur = 0;   // row-table slot of the current tile (the next tile's is cur ^ 1)
    auto start_stream = [&](const FfnTile& t) {
        const FfnSrc here = ffn_src(p, t, 1, 0, cur * BM);
        const ARows ah = arows(here);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < P; ++i) dma(here, ah, kbase + g, i);
        wait_vm<P>();   // the first K-tile landed; the second may stay in flight
        ring_barrier();
#pragma unroll
        for (int i = 0; i < TM + TN; ++i) frag(ring + (kbase & 1) * SC, 0, i, fa0, fb0);
    };

    load_tab(c0, 0);
    load_tab(c1, 1);
    if (p.row_token) {
        wait_vm<0>();   // both row tables landed before any DMA reads them
        ring_barrier();
    }
    bool poison = !wait_rows(c0);   // the current tile's rows were not seen complete
    start_stream(c0);

    // One K-tile g, four k-steps: k-steps 0..2 multiply while the next one's
    // fragments are read (k-step 0 also issues the B blocks of K-tile g + 1);
    // k-step 3 issues a few MFMAs, waits for K-tile g + 1 and joins the
    // barrier (every wave has all of K-tile g in registers by then, so its
    // stage is free), then, between its remaining MFMAs, starts the A blocks
    // of K-tile g + 2 into that stage and reads K-tile g + 1's k-step 0 into
    // set 0.  prev is the source of K-tile g + 1's DMAs.
    auto ktile = [&](int g, const FfnSrc& src, const ARows& ar, const FfnSrc& prev, f32x16 (&acc)[TM][TN]) {
        const u32x4* stage = ring + (g & 1) * SC;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa0, fb0, acc);
            frag(stage, 1, i, fa1, fb1);
            // the B blocks of K-tile g + 1, whose A blocks went out after the
            // previous K-tile's barrier (from prev, the source those used)
            if (i % (NM / B_DMA) == NM / B_DMA - 1) dma(prev, ar, g + 1, A_DMA + i / (NM / B_DMA));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa1, fb1, acc);
            frag(stage, 2, i, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf_mfma1<TL>(i, fa0, fb0, acc);
            frag(stage, 3, i, fa1, fb1);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < EARLY; ++i) bf_mfma1<TL>(i, fa1, fb1, acc);
        wait_vm<0>();   // K-tile g + 1 landed (the only DMAs in flight)
        wait_lds();     // this wave's reads of K-tile g are complete
        ring_barrier();
        const u32x4* nstage = ring + ((g + 1) & 1) * SC;
#pragma unroll
        for (int i = 0; i < SL; ++i) {
            bf_mfma1<TL>(EARLY + i, fa1, fb1, acc);
#pragma unroll
            for (int j = i * A_DMA / SL; j < (i + 1) * A_DMA / SL; ++j) dma(src, ar, g + 2, j);
            frag(nstage, 0, i, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    for (;;) {
        f32x16 acc[TM][TN];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        const int nk = c0.phase == 0 ? nk1 : nk2;
        const int head = nk - 2;   // K-tiles whose DMAs (two ahead) stay in the current tile
        // The count of the next tile's M tile is copied into LDS before K-tile
        // head - 1's wait, which then covers it.
        const bool probe = c1.phase == 1 && head >= 1;
        const int split = probe ? head - 1 : head;
        const FfnSrc here = ffn_src(p, c0, 1, 0, cur * BM);
        const ARows ah = arows(here);
        for (int kt = 0; kt < split; ++kt) ktile(kbase + kt, here, ah, here, acc);
        if (probe && wave == 0) dma4_dev(done, (uint32_t)c1.mt * 4u, lds_addr(s_flag));
        for (int kt = split; kt < head; ++kt) ktile(kbase + kt, here, ah, here, acc);
        const int flag = __builtin_amdgcn_readfirstlane(s_flag[0]);
        const bool go = c1.phase == 0 || (probe && flag >= NT1 && !p.force_wait);
        const FfnSrc ahead = go ? ffn_src(p, c1, 1, -nk, (cur ^ 1) * BM) : ffn_src(p, c0, 0, nk - 1, cur * BM);
        const ARows aa = arows(ahead);
        for (int kt = head; kt < nk; ++kt) ktile(kbase + kt, ahead, aa, kt == head ? here : ahead, acc);
        // the B blocks of the last K-tile's DMAs go out now rather than after
        // the epilogue (the next tile's first K-tile issues them again: the
        // same bytes into the same place, landed before that K-tile's wait)
#pragma unroll
        for (int j = A_DMA; j < P; ++j) dma(ahead, aa, kbase + nk + 1, j);

        const TileCoord tc{c0.row0, c0.rows, c0.n0, c0.e};
        if (KEEP && c0.phase == 0)   // the pre-activations as GEMM1 computed them, for the backward
            bf_epilogue<TL, 0>(acc, p.ab, 2 * p.H, 2 * p.H, tc, wm, wn, obuf + wave * kObufChunks, nullptr);
        if (c0.phase == 0)
            bf_epilogue<TL, 1, true>(acc, p.h, p.H, 2 * p.H, tc, wm, wn, obuf + wave * kObufChunks, nullptr, hrsrc);
        else
            bf_epilogue<TL, 0>(acc, p.ye, p.d, p.d, tc, wm, wn, obuf + wave * kObufChunks, nullptr,
                               __amdgpu_buffer_rsrc_t(), poison);

        // tile end: a GEMM1 tile's stores complete (h coherent at device
        // scope), the ticket claimed one tile ago published, the finished GEMM1
        // tile counted
        if (c0.phase == 0) wait_vm<0>();
        if (threadIdx.x == 0) s_next = pending;
        wait_lds();
        ring_barrier();
        if (threadIdx.x == 0 && c0.phase == 0)
            __hip_atomic_fetch_add(done + c0.mt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int id2 = __builtin_amdgcn_readfirstlane(s_next);
        if (threadIdx.x == 0 && id2 < total)
            pending = ffn_ticket_id(xcd, 2 * GX + __hip_atomic_fetch_add(p.sync + xcd, 1, __ATOMIC_RELAXED,
                                                                           __HIP_MEMORY_SCOPE_AGENT), k32);
        if (c1.phase < 0) break;
        kbase += nk;
        c0 = c1;
        c1 = ffn_tile<BM, BN>(id2, total, T1, NT1, NT2, s_tstart, p.E, p.offsets);
        // the finished tile's table slot takes the new next tile's rows (every
        // DMA that read it has been issued); the next K-tile wait covers it
        cur ^= 1;
        load_tab(c1, cur ^ 1);
        poison = false;
        if (!go) {
            // the next tile's first K-tiles were not prefetched: wait for its
            // rows, let the dummy copies land, and restart the stream there
            poison = !wait_rows(c0);
            wait_vm<0>();
            ring_barrier();
            start_stream(c0);
        }
    }
    wait_vm<0>();   // no DMA may land in LDS after the workgroup has left
}

// ============================================================================ MXFP8
//
// Operands are E4M3 codes with one E8M0 scale per 32 K values (OCP MX v1.0).
// A ring stage holds 128 K values per row (128 bytes, so every DMA instruction
// moves 8 whole lines, as in the bf16 FFN), consumed as two k-steps of one
// MFMA per fragment pair.  In that instruction lane l of half h = l / 32 holds,
// for row l % 32, K values [16 h, 16 h + 16) of the k-step's 64 in its bytes
// 0..15 and [32 + 16 h, 48 + 16 h) in bytes 16..31, and supplies the scale of
// the k-step's K block h: scale block b covers bytes 0..15 of both halves for
// b = 0 and bytes 16..31 for b = 1 (measured on gfx950).  So a lane's fragment
// of k-step s is chunks 4 s + h and 4 s + 2 + h of the 128-byte row, and its
// scale is that of block 2 s + h of the K-tile.  Scale buffers are stored
// [K/128][rows][4]: the four scales of one K-tile of a row form one dword and
// the dwords of consecutive rows are adjacent, so with every K-tile each wave
// DMAs, for its SR rows of A and of B, one contiguous run of dwords into the
// stage's scale slot.  Each lane reads its own scale byte (byte 2 s + h of its
// row's dword) zero-extended, and the MFMA takes scale byte 0.  Chunk c of row
// r sits at chunk c ^ ((r >> 1) & 7) of the row (bank-conflict-free fragment
// reads).  Four waves each own a 128 x 128 block whose 256 accumulators sit in
// AGPRs, leaving the VGPRs to the 32-byte fragments (fp8 halves the LDS bytes
// per FLOP, so the larger per-wave block suits it).
template <class TL>
struct Fp8Extra {
    static constexpr int PS = 2;                // scale DMAs per wave per K-tile (A rows, B rows)
    static constexpr int SR = TL::BM / TL::NW;  // scale rows per wave and operand
    static constexpr int OBUF_RR = TL::NW == 4 ? 32 : 16;   // output rows staged per round (LDS budget)
    static constexpr int A_DMA = TL::BM / 8 / TL::NW, B_DMA = TL::BN / 8 / TL::NW;   // 1 KB DMAs per wave
    static constexpr int P = A_DMA + B_DMA;     // data DMAs per wave per K-tile
    static constexpr int SC = (TL::BM + TL::BN) * 8;   // 16-byte chunks per stage
    static_assert(TL::BM == TL::BN && (SR == 32 || SR == 64), "one scale DMA per wave and operand");
    static_assert(A_DMA % 2 == 0 && B_DMA % 2 == 0, "DMA blocks of 8 rows, an even number per wave");
};

// Fragment mi of A (or ni of B) of one k-step: two 16-byte chunks of the
// lane's row, and the lane's scale byte read on its own (zero-extended, so the
// MFMA always takes scale byte 0).
template <class TL>
__device__ __forceinline__ void fp8_frag(const u32x4* stage, const uint8_t* sbytes, int off0, int off1, int sbyte,
                                         i32x8& f, int& sc) {
    const u32x4 lo = stage[off0], hi = stage[off1];
    f = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    sc = sbytes[sbyte];
}

// MFMAs [FIRST, FIRST + COUNT) of the TM x TN block, row-major over (mi, ni).
template <class TL, int FIRST, int COUNT>
__device__ __forceinline__ void fp8_mfma(const i32x8 (&fa)[TL::TM], const i32x8 (&fb)[TL::TN],
                                         const int (&sa)[TL::TM], const int (&sb)[TL::TN],
                                         f32x16 (&acc)[TL::TM][TL::TN]) {
#pragma unroll
    for (int i = FIRST; i < FIRST + COUNT; ++i) {
        const int mi = i / TL::TN, ni = i % TL::TN;
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[ni], fa[mi], acc[mi][ni], 0, 0, 0, sb[ni],
                                                                     0, sa[mi]);
    }
}

// MFMA number i (row-major over (mi, ni)); i is a constant after unrolling.
template <class TL>
__device__ __forceinline__ void fp8_mfma1(int i, const i32x8 (&fa)[TL::TM], const i32x8 (&fb)[TL::TN],
                                          const int (&sa)[TL::TM], const int (&sb)[TL::TN],
                                          f32x16 (&acc)[TL::TM][TL::TN]) {
    const int mi = i / TL::TN, ni = i % TL::TN;
    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[ni], fa[mi], acc[mi][ni], 0, 0, 0, sb[ni], 0,
                                                                 sa[mi]);
}

// Epilogue of the MXFP8 kernel.  EPI 0: C = acc as bf16.  EPI 1: h = silu(gate)
// * up per gate/up column pair, quantised to MXFP8 along h: each 32-column
// block of one row is split over lanes l and l ^ 32, which agree on the block
// maximum, take the shared exponent floor(log2 amax) - 8, and encode with
// e4m3x4 (saturating round-to-nearest-even E4M3).  KEEP (EPI 1): the gate/up
// accumulators are also stored as bf16 a | b [rows][N] (the pre-activations,
// for the backward) through the staged row stores.  post(mi) runs once the
// accumulators of row block mi have been read (the caller may reuse them).
template <class TL, int EPI, bool KEEP, class Post>
__device__ __forceinline__ void fp8_epilogue(const f32x16 (&acc)[TL::TM][TL::TN], void* __restrict__ C,
                                             uint8_t* __restrict__ Cs, int ldc, int N, int R, const TileCoord& c,
                                             int wm, int wn, u32x4* __restrict__ obuf, uint16_t* __restrict__ ab,
                                             Post&& post) {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    // EPI 0: the tile's rows of C as a raw buffer resource, for the counted stores
    const uint32_t tile_bytes = (uint32_t)c.rows * (uint32_t)ldc * 2u;
    const __amdgpu_buffer_rsrc_t tile_rc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint16_t*>(C) + (size_t)c.row0 * ldc, 0, (int)tile_bytes, kRawBufferWord3);
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) {
        const int r = wm * TL::WROWS + mi * 32 + (lane & 31);
        const bool valid = r < c.rows;
        const size_t grow = (size_t)(c.row0 + r);
        if (EPI == 0) {
#pragma unroll
            for (int np = 0; np < TL::TN / 2; ++np) {
                float g[16], u[16];
                acc_block<TL>(acc[mi][2 * np], g);
                acc_block<TL>(acc[mi][2 * np + 1], u);
                const int rb = wm * TL::WROWS + mi * 32;   // tile row of the block's row 0
                store_bf16_pair_rows<Fp8Extra<TL>::OBUF_RR, false, true>(
                    static_cast<uint16_t*>(C), (size_t)ldc, c.row0 + rb, c.rows - rb, c.n0 + wn * TL::WCOLS + np * 64,
                    N, g, u, obuf, tile_rc, false, rb, tile_bytes);
                __builtin_amdgcn_sched_barrier(0);   // one block pair's values in VGPRs at a time
            }
        } else {
#pragma unroll
            for (int np = 0; np < TL::TN / 2; ++np) {
                const int pc = c.n0 + wn * TL::WCOLS + np * 64;
                float v[16], u[16];
                acc_block<TL>(acc[mi][2 * np], v);
                acc_block<TL>(acc[mi][2 * np + 1], u);
                if constexpr (KEEP) {
                    const int rb = wm * TL::WROWS + mi * 32;
                    store_bf16_pair_rows<Fp8Extra<TL>::OBUF_RR>(ab, (size_t)N, c.row0 + rb, c.rows - rb, pc, N, v, u,
                                                                obuf);
                }
                float amax = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    v[i] = silu_mul_p(v[i], u[i]);
                    amax = fmaxf(amax, fabsf(v[i]));
                }
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                const int se = mx_shared_exp(amax);
                const float inv = mx_inv_scale(se);
                uint32_t w[4];   // run q: 4 codes of columns 8q + 4 half + 0..3
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = e4m3x4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
                gather_halves(w);
                if (valid && pc < N) {
                    const int hb = pc / 64;   // 32-wide h block of this pair
                    uint8_t* Cq = static_cast<uint8_t*>(C);
                    *reinterpret_cast<u32x4*>(Cq + grow * ldc + hb * 32 + 16 * half) = (u32x4){w[0], w[1], w[2], w[3]};
                    // scale planes [ldc/128][R][4]
                    if (half == 0) Cs[((size_t)(hb >> 2) * R + grow) * 4 + (hb & 3)] = (uint8_t)(se + 127);
                }
                __builtin_amdgcn_sched_barrier(0);   // one block pair's values in VGPRs at a time
            }
        }
        post(mi);
    }
}

// The persistent MXFP8 kernel streams K-tiles without a break at tile
// boundaries: global K-tile g of this workgroup (g = tiles done * nk + kt) goes
// through ring stage and scale slot g % 2, and the DMAs of the last two
// K-tiles of a tile already fetch the first two of the next one (or, when a
// tile has one K-tile, of the tile after).  K-tile g: k-step 0 multiplies
// while k-step 1's fragments are read; then a few MFMAs of k-step 1, the wait
// for K-tile g + 1, the barrier (every wave then holds all of K-tile g in
// registers, so its stage and scale slot are free), and, between the remaining
// MFMAs, the DMAs of K-tile g + 2 and the reads of K-tile g + 1's k-step 0.
// SPLIT (two or more K-tiles per tile): only the A blocks and scales of
// K-tile g + 2 go out there, its B blocks between the first MFMAs of K-tile
// g + 1's k-step 0.
// The epilogue runs between the last MFMA of a tile and the first of the next
// while the next tile's first K-tiles are in flight; its stores count in
// vmcnt after those DMAs, which only makes the next wait wait longer.  EPI 0
// issues a fixed number of stores per wave, so after an overlapped epilogue
// the next tile's first K-tile waits for its own DMAs only and the stores
// drain during that K-tile.
// EPI 0: C = A B (bf16 out);  1: C = MXFP8(silu(A Bgate) * (A Bup)) along N/2, with KEEP also a | b into ab
template <class TL, int EPI, bool SPLIT, bool KEEP>
__global__ __launch_bounds__(TL::NTHR) __attribute__((amdgpu_waves_per_eu(TL::NW / 4, TL::NW / 4)))
void gemm_fp8_pipe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                          const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, void* __restrict__ C,
                          uint8_t* __restrict__ Cs, const int32_t* __restrict__ offsets, int E, int N, int K,
                          int ldc, int R, const int32_t* __restrict__ row_token, uint16_t* __restrict__ ab) {
    constexpr int BM = TL::BM, BN = TL::BN, NTHR = TL::NTHR, TM = TL::TM, TN = TL::TN;
    constexpr int SR = Fp8Extra<TL>::SR, PS = Fp8Extra<TL>::PS;
    constexpr int A_DMA = Fp8Extra<TL>::A_DMA, B_DMA = Fp8Extra<TL>::B_DMA, P = Fp8Extra<TL>::P;
    constexpr int SC = Fp8Extra<TL>::SC, ND = P + PS, ES = ND - B_DMA;   // ES: DMAs issued after a barrier when SPLIT
    constexpr int NM = TL::NM, EARLY = TL::EARLY, SL = NM - EARLY;
    static_assert(SL >= TM + TN && SL > 0, "one fragment read per MFMA slot");
    constexpr int kObufChunks = EPI == 0 || KEEP ? 8 * Fp8Extra<TL>::OBUF_RR : 0;   // per wave: rows x 128 bytes
    // store instructions per wave of an EPI 0 epilogue: TM x TN / 2 counted
    // pair-row stores of 4 each, whatever the tile's rows and columns
    constexpr int kEpiStores = EPI == 0 ? 2 * TM * TN : 0;
    static_assert(kEpiStores < 64, "vmcnt range");
    __shared__ u32x4 ring[2 * SC];
    __shared__ uint32_t sring[2 * (BM + BN)];     // two scale slots: A rows then B rows
    __shared__ u32x4 obuf[kObufChunks ? TL::NW * kObufChunks : 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scan[NTHR];
    __shared__ int s_tab[EPI == 1 ? 3 * BM : 1];   // row tables of gathered A rows (GEMM1 only)

    const int MT = build_tile_schedule<BM, NTHR>(offsets, E, s_tstart, s_scan);
    const int NT = (N + BN - 1) / BN;
    const int total = MT * NT;
    const int G = gridDim.x;
    const int kb = K / 32;            // scale bytes per row
    const int nk = K / 128;           // K-tiles per tile
    int tile = xcd_slot(blockIdx.x, G);
    if (tile >= total) return;

    // wave-uniform values are pinned to SGPRs (derived from threadIdx they would
    // otherwise live in VGPRs)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ring_lds = lds_addr(ring), sring_lds = lds_addr(sring);
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    const int key = ((lane & 31) >> 1) & 7, half = lane >> 5;
    const int arow_i = wm * TL::WROWS + (lane & 31), brow_i = wn * TL::WCOLS + (lane & 31);
    // fragment chunks of k-step s: 4 s + h and 4 s + 2 + h, swizzled
    int a_lo[2], a_hi[2], b_lo[2], b_hi[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        a_lo[s] = arow_i * 8 + ((4 * s + half) ^ key);
        a_hi[s] = arow_i * 8 + ((4 * s + 2 + half) ^ key);
        b_lo[s] = (BM + brow_i) * 8 + ((4 * s + half) ^ key);
        b_hi[s] = (BM + brow_i) * 8 + ((4 * s + 2 + half) ^ key);
    }
    // DMA lanes: row lane / 8 of an 8-row block, physical chunk lane % 8 (key 4 (i & 1) + (lane / 8) / 2)
    const int drow = lane >> 3;
    const uint32_t dch0 = (uint32_t)((lane & 7) ^ (drow >> 1)) * 16u;
    const uint32_t dch1 = (uint32_t)((lane & 7) ^ (4 + (drow >> 1))) * 16u;
    const int srow = SR * wave + (lane & (SR - 1));    // scale DMA row of this lane
    // GEMM1 with row_token: A row r of a tile is code row row_token[row0 + r]
    // of the token matrix A [T][K] (each token quantised once).  Tile i of this
    // workgroup keeps its row_token entries in LDS slot i % 3, DMA'd two tiles
    // ahead (like the K-tiles, covered by the next K-tile wait and barrier);
    // each lane turns its A rows into byte offsets once per loop phase.
    static_assert(EPI == 0 || TL::NW * 64 == BM, "one row-table DMA per wave");
    const bool gather = EPI == 1 && row_token != nullptr;
    auto load_tab = [&](const TileCoord& t, int slot) {
        if constexpr (EPI == 1) {
            if (!gather) return;
            const int r = 64 * wave + lane;
            dma4(row_token, (uint32_t)(t.row0 + min(r, t.rows - 1)) * 4u, lds_addr(s_tab + slot * BM + 64 * wave));
        }
    };
    struct ARows { uint32_t off[A_DMA]; };
    auto arows = [&](const StreamSrc& src, int slot) {
        ARows a;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int r = 8 * (wave * A_DMA + i) + drow;
            int row = src.t.row0 + min(r, src.t.rows - 1);
            if constexpr (EPI == 1) {
                if (gather) row = s_tab[slot * BM + r];
            }
            a.off[i] = (uint32_t)row * (uint32_t)K + ((i & 1) ? dch1 : dch0);
        }
        return a;
    };
    const bool slane = lane < SR;
    // scale byte of this lane in a slot for k-step 0 (+2 for k-step 1): row dword, byte = K block h
    const int sa_byte = arow_i * 4 + half, sb_byte = (BM + brow_i) * 4 + half;

    TileCoord c0 = tile_coord<BM, BN>(tile, MT, NT, s_tstart, E, offsets), c1 = c0, c2 = c0;
    if (tile + G < total) c1 = tile_coord<BM, BN>(tile + G, MT, NT, s_tstart, E, offsets);
    if (tile + 2 * G < total) c2 = tile_coord<BM, BN>(tile + 2 * G, MT, NT, s_tstart, E, offsets);
    int kbase = 0;   // global K-tile index of the current tile's K-tile 0

    const int qa = nk >= 2 ? 1 : 2;   // tiles ahead reached by the last two K-tiles' prefetches
    const int head = max(nk - 2, 0);  // K-tiles whose prefetch stays in the current tile

    // DMA step i of global K-tile g from src: A blocks, then B blocks, then
    // the two scale dword runs (a stand-in K-tile nk - 1 maps to the last plane too)
    auto dma = [&](const StreamSrc& src, const ARows& ar, int g, int i) {
        const TileCoord& t = src.t;
        const int kt = (g - kbase) * src.mul + src.add;
        const uint32_t st = ring_lds + (uint32_t)(g & 1) * SC * 16u;
        const uint32_t dch = (i & 1) ? dch1 : dch0;
        if (i < A_DMA) {
            dma16(A, ar.off[i] + (uint32_t)kt * 128u, st + (uint32_t)(wave * A_DMA + i) * 1024u);
        } else if (i < P) {
            const int j = i - A_DMA;
            const int r = 8 * (wave * B_DMA + j) + drow;
            const uint32_t off = (uint32_t)min(t.n0 + r, N - 1) * (uint32_t)K + dch + (uint32_t)kt * 128u;
            dma16(B + (size_t)t.e * N * K, off, st + BM * 128u + (uint32_t)(wave * B_DMA + j) * 1024u);
        } else {
            const uint32_t slot = sring_lds + (uint32_t)(g & 1) * (BM + BN) * 4u;
            if (SR == 64 || slane) {
                if (i == P)
                    dma4(As, ((uint32_t)kt * (uint32_t)R + (uint32_t)(t.row0 + min(srow, t.rows - 1))) * 4u,
                         slot + (uint32_t)(wave * SR) * 4u);
                else
                    dma4(Bs + (size_t)t.e * N * kb, ((uint32_t)kt * (uint32_t)N + (uint32_t)min(t.n0 + srow, N - 1)) * 4u,
                         slot + BM * 4u + (uint32_t)(wave * SR) * 4u);
            }
        }
    };
    auto frags = [&](const u32x4* stage, const uint8_t* slot, int s, int i, i32x8 (&fa)[TM], i32x8 (&fb)[TN],
                     int (&sa)[TM], int (&sb)[TN]) {
        if (i < TM)
            fp8_frag<TL>(stage, slot, a_lo[s] + i * 256, a_hi[s] + i * 256, sa_byte + 2 * s + i * 128, fa[i], sa[i]);
        else if (i < TM + TN)
            fp8_frag<TL>(stage, slot, b_lo[s] + (i - TM) * 256, b_hi[s] + (i - TM) * 256,
                         sb_byte + 2 * s + (i - TM) * 128, fb[i - TM], sb[i - TM]);
    };
    i32x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    int sa0[TM], sb0[TN], sa1[TM], sb1[TN];

    // one K-tile g: k-step 0 in set 0 (read during the previous K-tile), k-step 1 in set 1
    // MFMA0 false: k-step 0 was multiplied already (during the previous tile's epilogue)
    auto ktile_impl = [&](auto mfma0, int g, const StreamSrc& src, const ARows& ar, const StreamSrc& prev,
                          f32x16 (&acc)[TM][TN]) {
        // after an EPI 0 epilogue (mfma0 false: the tile's first K-tile), K-tile
        // g + 1's B blocks went out before the epilogue's kEpiStores stores, so
        // they are not issued again and the wait leaves those stores in flight
        constexpr bool drain = !decltype(mfma0)::value && EPI == 0 && SPLIT;
        const u32x4* stage = ring + (g & 1) * SC;
        const uint8_t* slot = reinterpret_cast<const uint8_t*>(sring + (g & 1) * (BM + BN));
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if constexpr (decltype(mfma0)::value) fp8_mfma1<TL>(i, fa0, fb0, sa0, sb0, acc);
            frags(stage, slot, 1, i, fa1, fb1, sa1, sb1);
            // SPLIT: the B blocks of K-tile g + 1, whose A blocks and scales
            // went out after the previous K-tile's barrier (from prev, the
            // source those used)
            if (SPLIT && !drain && i < B_DMA) dma(prev, ar, g + 1, A_DMA + i);
            __builtin_amdgcn_sched_barrier(0);
        }
        fp8_mfma<TL, 0, EARLY>(fa1, fb1, sa1, sb1, acc);
        if constexpr (drain)
            wait_vm<kEpiStores>();   // K-tile g + 1 landed; the stores issued after it may not have
        else
            wait_vm<0>();   // K-tile g + 1 landed (the only DMAs in flight)
        wait_lds();     // this wave's reads of K-tile g are complete
        ring_barrier();
        const u32x4* nstage = ring + ((g + 1) & 1) * SC;
        const uint8_t* nslot = reinterpret_cast<const uint8_t*>(sring + ((g + 1) & 1) * (BM + BN));
#pragma unroll
        for (int i = 0; i < SL; ++i) {
            fp8_mfma1<TL>(EARLY + i, fa1, fb1, sa1, sb1, acc);
            if (SPLIT) {   // A blocks and scales
#pragma unroll
                for (int j = i * ES / SL; j < (i + 1) * ES / SL; ++j) dma(src, ar, g + 2, j < A_DMA ? j : j + B_DMA);
            } else {
#pragma unroll
                for (int j = i * ND / SL; j < (i + 1) * ND / SL; ++j) dma(src, ar, g + 2, j);
            }
            frags(nstage, nslot, 0, i, fa0, fb0, sa0, sb0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto ktile = [&](int g, const StreamSrc& src, const ARows& ar, const StreamSrc& prev, f32x16 (&acc)[TM][TN]) {
        ktile_impl(std::integral_constant<bool, true>{}, g, src, ar, prev, acc);
    };
    auto ktile_rest = [&](int g, const StreamSrc& src, const ARows& ar, const StreamSrc& prev, f32x16 (&acc)[TM][TN]) {
        ktile_impl(std::integral_constant<bool, false>{}, g, src, ar, prev, acc);
    };

    int ti = 0;   // tiles this workgroup has finished (row-table slot of the current tile: ti % 3)
    load_tab(c0, 0);
    if (tile + G < total) load_tab(c1, 1);
    if (tile + 2 * G < total) load_tab(c2, 2);
    if (gather) {
        wait_vm<0>();   // the row tables landed before any DMA reads them
        ring_barrier();
    }
    // prologue: K-tiles 0 and 1 of the stream (for one-K-tile tiles, 1 is the next tile's)
    {
        const StreamSrc here{c0, 1, 0};
        const bool has1 = tile + G < total;
        const StreamSrc ahead{has1 ? c1 : c0, has1 ? 1 : 0, has1 ? -nk : nk - 1};
        const ARows ah = arows(here, 0), aa = arows(ahead, has1 ? 1 : 0);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                if (g < nk) dma(here, ah, g, i);
                else dma(ahead, aa, g, i);
            }
    }
    wait_vm<ND>();   // K-tile 0 and its scales landed; K-tile 1 may stay in flight
    ring_barrier();
#pragma unroll
    for (int i = 0; i < TM + TN; ++i)
        frags(ring, reinterpret_cast<const uint8_t*>(sring), 0, i, fa0, fb0, sa0, sb0);

    // With three or more K-tiles per tile the epilogue of a tile multiplies the
    // next tile's k-step 0 (its fragments are in set 0 by then) row block by
    // row block as it frees the accumulators, so the matrix units work while
    // the results are stored; that tile's first K-tile then skips k-step 0.
    const bool overlap_ok = nk >= 3;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
    bool pre = false;   // k-step 0 of this tile's first K-tile is already in acc

    for (;;) {
        const StreamSrc here{c0, 1, 0};
        const bool has = tile + qa * G < total;
        const StreamSrc ahead{has ? (qa == 1 ? c1 : c2) : c0, has ? 1 : 0, has ? -qa * nk : nk - 1};
        const ARows ah = arows(here, ti % 3);
        int kt0 = 0;
        if (pre) {   // head >= 1 here, so K-tile 0 belongs to the first phase
            ktile_rest(kbase, here, ah, here, acc);
            kt0 = 1;
        }
        for (int kt = kt0; kt < head; ++kt) ktile(kbase + kt, here, ah, here, acc);
        const ARows aa = arows(ahead, has ? (ti + qa) % 3 : ti % 3);
        for (int kt = head; kt < nk; ++kt) ktile(kbase + kt, ahead, aa, kt == head ? here : ahead, acc);
        if (SPLIT) {
            // the B blocks of the last K-tile's DMAs go out now rather than
            // after the epilogue (the next tile's first K-tile issues them
            // again: the same bytes into the same place, landed before that
            // K-tile's wait)
#pragma unroll
            for (int j = A_DMA; j < P; ++j) dma(ahead, aa, kbase + nk + 1, j);
        }
        // set 0 now holds k-step 0 of the next tile's first K-tile (or unused data after the last)
        const bool overlap = overlap_ok && tile + G < total;
        fp8_epilogue<TL, EPI, KEEP>(acc, C, Cs, ldc, N, R, c0, wm, wn, obuf + wave * kObufChunks, ab, [&](int mi) {
            if (overlap) {   // row block mi of the next tile's k-step 0, from zero
                const f32x16 z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb0[ni], fa0[mi], z, 0, 0, 0,
                                                                                 sb0[ni], 0, sa0[mi]);
            } else {
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
            }
        });
        pre = overlap;
        if (tile + G >= total) break;
        tile += G;
        c0 = c1;
        c1 = c2;
        ++ti;
        if (tile + 2 * G < total) {
            c2 = tile_coord<BM, BN>(tile + 2 * G, MT, NT, s_tstart, E, offsets);
            load_tab(c2, (ti + 2) % 3);   // the slot of the tile just finished
        }
        kbase += nk;
    }
    wait_vm<0>();   // no DMA may land in LDS after the workgroup has left
}

// ============================================================================ weight gradients

// K-grouped bf16 GEMM on MFMA for the weight gradients: for expert e
//   C[e][m][n] = sum over rows r in [offsets[e], offsets[e+1]) of XA[r][m] XB[r][n]
// with the activations as stored, XA [R][M] and XB [R][N], so no transposed
// copy is made.  Workgroup tile 256 x 256, 8 waves of 128 x 64, a 4-stage
// ring of K-tiles loaded with global_load_lds, one barrier per K-tile, in the
// schedule of the forward kernels: k-step 0 multiplies while k-step 1's
// fragments are read; k-step 1 issues a few MFMAs, waits for K-tile kt + 1,
// joins the barrier (every wave then holds all of kt in registers), and,
// between its remaining MFMAs, sends the DMAs of K-tile kt + 4 into kt's stage
// and reads kt + 1's k-step 0.  An expert without rows writes zeros.  OMAP 0:
// C[e][m][n].  OMAP 1: the N axis interleaves gate and up columns (32 + 32 per
// 64); column n goes to C (gate) or C2 (up) [e][m][h], h = 32 (n / 64) + n %
// 32.  Rows or columns past M, N are clamped in the loads and not stored.  A K-tile is 32 rows:
// each 1 KB DMA brings two 512-byte tile rows (256 columns), lane l's 16 bytes
// landing at chunk l % 32 of row l / 32, which holds global chunk (l % 32) ^
// 4 (row % 4).  The MFMA fragments (8 consecutive rows of one column per
// lane) come from ds_read_b64_tr_b16: in each group of 16 lanes, lane L
// addresses 4 columns of one row and receives element L % 4 of the 64-bit
// reads of lanes 4 j + L / 4, j = 0..3 (measured on gfx950), so lane L
// addressing row k0 + L / 4, columns c + 4 (L % 4) .. + 3 gets rows k0 .. k0
// + 3 of column c + L.  Two such reads give the 8 rows of a fragment; the
// XOR swizzle puts the 4 rows of a read in 4 different 64-byte bank windows.
// Rows past the expert's segment (the last K-tile) are loaded clamped and
// zeroed in the XB fragments.
__device__ __forceinline__ bf16x8 tr_frag(const __attribute__((address_space(3))) char* base, uint32_t b0,
                                          uint32_t b1) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lp;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(base + b0));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(base + b1));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <class WT, int OMAP>
__global__ __launch_bounds__(WT::NTHR, WT::OCC) void gemm_wgrad_rm_kernel(const uint16_t* __restrict__ XA,
                                                                         const uint16_t* __restrict__ XB,
                                                                         const int32_t* __restrict__ offsets, int M,
                                                                         int N, float* __restrict__ C,
                                                                         float* __restrict__ C2) {
    constexpr int BM = WT::BM, BN = WT::BN, STAGES = 4, NW = WT::NW, KT = 32;
    static_assert(BM == 256 && BN == 256, "a 1 KB DMA covers two 512-byte tile rows");
    constexpr uint32_t SA = KT * BM * 2, SBYTES = KT * (BM + BN) * 2;
    constexpr int A_DMA = KT / 2 / NW, B_DMA = KT / 2 / NW, P = A_DMA + B_DMA;
    constexpr int TM = BM / WT::WM / 32, TN = BN / WT::WN / 32;
    constexpr int WROWS = BM / WT::WM, WCOLS = BN / WT::WN;
    __shared__ u32x4 ring[STAGES * SBYTES / 16];
    const int e = blockIdx.z, m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int o0 = offsets[e], len = offsets[e + 1] - o0, nk = (len + KT - 1) / KT;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WT::WN, wn = wave % WT::WN;
    const uint32_t ring_lds = lds_addr(ring);
    const __attribute__((address_space(3))) char* lbase = (const __attribute__((address_space(3))) char*)ring;
    // DMA slot i: tile rows 2 q and 2 q + 1, q = wave * A_DMA + i (A; likewise B)
    const int hr = lane >> 5, ch = lane & 31;
    int trA[A_DMA], trB[B_DMA];
    uint32_t colA[A_DMA], colB[B_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        trA[i] = 2 * (wave * A_DMA + i) + hr;
        colA[i] = (uint32_t)min(m0 + 8 * (ch ^ (4 * (trA[i] & 3))), M - 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        trB[i] = 2 * (wave * B_DMA + i) + hr;
        colB[i] = (uint32_t)min(n0 + 8 * (ch ^ (4 * (trB[i] & 3))), N - 8) * 2u;
    }
    const uint32_t rbA = (uint32_t)M * 2u, rbB = (uint32_t)N * 2u;
    // DMA i of K-tile kt's A rows (or B rows) into stage kt % 4; past the last
    // K-tile a clamped copy lands in a stage whose reads go unused
    auto dma_a = [&](int kt, int i) {
        const int kb = min(kt, nk - 1) * KT;
        const uint32_t st = ring_lds + (uint32_t)(kt & (STAGES - 1)) * SBYTES;
        dma16(XA, (uint32_t)(o0 + min(kb + trA[i], len - 1)) * rbA + colA[i], st + (uint32_t)(wave * A_DMA + i) * 1024u);
    };
    auto dma_b = [&](int kt, int i) {
        const int kb = min(kt, nk - 1) * KT;
        const uint32_t st = ring_lds + (uint32_t)(kt & (STAGES - 1)) * SBYTES;
        dma16(XB, (uint32_t)(o0 + min(kb + trB[i], len - 1)) * rbB + colB[i],
              st + SA + (uint32_t)(wave * B_DMA + i) * 1024u);
    };
    auto issue = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) dma_a(kt, i);
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) dma_b(kt, i);
    };
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // transposed-read addresses (bytes within a stage) of k-step s, read r:
    // row 16 s + 8 h + 4 r + L / 4, column c + 16 (G % 2) + 4 (L % 4)
    const int L = lane & 15, G = lane >> 4, h = lane >> 5;
    auto tr_addr = [&](int s2, int r, int col) -> uint32_t {
        const int row = 16 * s2 + 8 * h + 4 * r + (L >> 2);
        const int c = col + 16 * (G & 1) + 4 * (L & 3);
        return (uint32_t)row * (BM * 2u) + (((uint32_t)c * 2u) ^ (64u * (uint32_t)(L >> 2)));
    };
    // fragment sets: set 0 holds k-step 0 of the current K-tile, set 1 its k-step 1
    constexpr int NM = TM * TN, EARLY = TN, SL = NM - EARLY;
    static_assert(SL >= TM + TN, "one fragment read per MFMA slot");
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    auto frag = [&](int kt, int s2, int i, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
        const __attribute__((address_space(3))) char* sa = lbase + (uint32_t)(kt & (STAGES - 1)) * SBYTES;
        if (i < TM) {
            const int col = wm * WROWS + i * 32;
            fa[i] = tr_frag(sa, tr_addr(s2, 0, col), tr_addr(s2, 1, col));
        } else if (i < TM + TN) {
            const int col = wn * WCOLS + (i - TM) * 32;
            fb[i - TM] = tr_frag(sa + SA, tr_addr(s2, 0, col), tr_addr(s2, 1, col));
        }
    };
    // rows at or past the expert's end (the last K-tile) belong to the next
    // expert or are clamped copies: zero them in the XB fragments
    auto mask = [&](int kt, int s2, bf16x8 (&fb)[TN]) {
        const int rem = len - kt * KT;
        if (rem < KT) {
            wait_lds();
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (16 * s2 + 8 * h + u >= rem) fb[j][u] = (__bf16)0.0f;
        }
    };
    auto mfma1 = [&](int i, const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN]) {
        acc[i / TN][i % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i % TN], fa[i / TN], acc[i / TN][i % TN],
                                                                       0, 0, 0);
    };
    if (nk > 0) {
        issue(0);
        issue(1);
        issue(2);
        issue(3);
        wait_vm<3 * P>();   // K-tile 0 landed; 1, 2 and 3 may still be in flight
        ring_barrier();
#pragma unroll
        for (int i = 0; i < TM + TN; ++i) frag(0, 0, i, fa0, fb0);
        for (int kt = 0; kt < nk; ++kt) {
            mask(kt, 0, fb0);
            // k-step 0 multiplies while k-step 1 is read
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                mfma1(i, fa0, fb0);
                frag(kt, 1, i, fa1, fb1);
                __builtin_amdgcn_sched_barrier(0);
            }
            mask(kt, 1, fb1);
            // k-step 1: a few MFMAs, the wait for K-tile kt + 1 and the barrier
            // (every wave then holds all of kt in registers, so its stage is
            // free), then, between the remaining MFMAs, the DMAs of kt + 4 into
            // that stage and the reads of kt + 1's k-step 0
#pragma unroll
            for (int i = 0; i < EARLY; ++i) mfma1(i, fa1, fb1);
            wait_vm<2 * P>();   // K-tile kt + 1 landed; kt + 2 and kt + 3 may still be in flight
            wait_lds();         // this wave's reads of kt are complete
            ring_barrier();
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                mfma1(EARLY + i, fa1, fb1);
#pragma unroll
                for (int q = i * P / SL; q < (i + 1) * P / SL; ++q) {
                    if (q < A_DMA) dma_a(kt + 4, q);
                    else dma_b(kt + 4, q - A_DMA);
                }
                frag(kt + 1, 0, i, fa0, fb0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    wait_vm<0>();   // every DMA has landed: the ring is free once all waves are past their last reads
    ring_barrier();
    // Epilogue through LDS: each wave owns 1/8 of the ring (16 KB, 64 rows x 64
    // float32) and takes its 128 x 64 block in two rounds of 64 rows.  A lane
    // holds runs of 4 columns of one row (chunk 8 j + 2 q + half of 16 per row,
    // swizzled by the row so 16 lanes of a write hit 64 banks); it reads back
    // chunk l % 16 of row l / 16 + 4 t, so 16 lanes cover a row's 256 bytes and
    // every store instruction writes whole 128-byte lines of 4 rows (direct
    // stores from the MFMA layout wrote 32-byte pieces of 32 rows).  The stores
    // are non-temporal: nothing in the backward reads the weight gradients.
    static_assert(WROWS == 128 && WCOLS == 64 && TN == 2 && NW * 16384 <= STAGES * SBYTES, "epilogue staging");
    const int half = lane >> 5;
    u32x4* stg = reinterpret_cast<u32x4*>(ring) + wave * 1024;
    const int mrow0 = m0 + wm * WROWS;
    const int ncol0 = n0 + wn * WCOLS;
#pragma unroll
    for (int rho = 0; rho < 2; ++rho) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * rho + ii, r = ii * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 8 * j + 2 * q + half;
                    stg[r * 16 + (c ^ (r & 15))] = (u32x4){
                        __float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                        __float_as_uint(acc[i][j][4 * q + 2]), __float_as_uint(acc[i][j][4 * q + 3])};
                }
        }
        asm volatile("" ::: "memory");
        wait_lds();   // this wave's writes are visible to its own lanes (the region is private to the wave)
        asm volatile("" ::: "memory");
        const int c = lane & 15;
        const int n = ncol0 + 4 * c;
        // all 16 reads first, then the stores: a read feeding each store in turn
        // would wait out the LDS latency 16 times
        u32x4 v[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int r = (lane >> 4) + 4 * t;
            v[t] = stg[r * 16 + (c ^ (r & 15))];
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int m = mrow0 + 64 * rho + (lane >> 4) + 4 * t;
            if (m < M && n < N) {
                if (OMAP == 0) {
                    __builtin_nontemporal_store(v[t], reinterpret_cast<u32x4*>(C + ((size_t)e * M + m) * N + n));
                } else {
                    const int Hh = N / 2, hh = 32 * (n / 64) + n % 32;
                    float* dst = ((n / 32) & 1) ? C2 : C;
                    __builtin_nontemporal_store(v[t], reinterpret_cast<u32x4*>(dst + ((size_t)e * M + m) * Hh + hh));
                }
            }
        }
        asm volatile("" ::: "memory");   // the next round's writes stay after these reads
        wait_lds();
        asm volatile("" ::: "memory");
    }
}

// Weight-gradient tile shapes: BM x BN workgroup tile, WM x WN waves, OCC
// workgroups per CU (4 ring stages of (BM + BN) x 64 bytes each).
template <int BM_, int BN_, int WM_, int WN_, int OCC_>
struct WgradTile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NW = WM * WN, NTHR = 64 * NW, OCC = OCC_;
};
using WgradBig = WgradTile<256, 256, 2, 4, 1>;   // 8 waves of 128 x 64, as the forward bf16 tiles

hipError_t launch_wgrad_rows(int omap, const uint16_t* XA, const uint16_t* XB, const int32_t* offsets, int E, int M,
                             int N, float* C, float* C2, hipStream_t s) {
    using WT = WgradBig;
    dim3 grid((N + WT::BN - 1) / WT::BN, (M + WT::BM - 1) / WT::BM, E), block(WT::NTHR);
    if (omap == 1)
        hipLaunchKernelGGL((gemm_wgrad_rm_kernel<WT, 1>), grid, block, 0, s, XA, XB, offsets, M, N, C, C2);
    else
        hipLaunchKernelGGL((gemm_wgrad_rm_kernel<WT, 0>), grid, block, 0, s, XA, XB, offsets, M, N, C, C2);
    return hipGetLastError();
}

// ============================================================================ launchers

template <class TL, int EPI>
hipError_t launch_bf16_pipe_tile(const uint16_t* A, const uint16_t* Bw, uint16_t* C, const int32_t* offsets,
                                 int R, int E, int N, int K, int ldc, const int32_t* host_counts,
                                 const uint16_t* aux, hipStream_t s) {
    const int grid = persistent_grid(R, E, N, TL::BM, TL::BN, 1, host_counts);
    hipLaunchKernelGGL((gemm_bf16_pipe_kernel<TL, EPI>), dim3(grid), dim3(TL::NTHR), 0, s, A, Bw, C, offsets, E, N,
                       K, ldc, aux);
    return hipGetLastError();
}

template <class TL, int EPI, bool KEEP>
hipError_t launch_fp8_pipe_tile(const uint8_t* A, const uint8_t* As, const uint8_t* Bw, const uint8_t* Bs,
                                void* C, uint8_t* Cs, const int32_t* offsets, int R, int E, int N, int K, int ldc,
                                const int32_t* host_counts, hipStream_t s, const int32_t* row_token, uint16_t* ab) {
    const int grid = persistent_grid(R, E, N, TL::BM, TL::BN, 1, host_counts);
    // with two or more K-tiles per tile a K-tile's B blocks are issued in the
    // next K-tile (the source of K-tile g + 1 is then the current tile's or,
    // for the last K-tile, the next one's, as the split code assumes)
    if (K >= 256)
        hipLaunchKernelGGL((gemm_fp8_pipe_kernel<TL, EPI, true, KEEP>), dim3(grid), dim3(TL::NTHR), 0, s, A, As, Bw,
                           Bs, C, Cs, offsets, E, N, K, ldc, R, row_token, ab);
    else
        hipLaunchKernelGGL((gemm_fp8_pipe_kernel<TL, EPI, false, KEEP>), dim3(grid), dim3(TL::NTHR), 0, s, A, As,
                           Bw, Bs, C, Cs, offsets, E, N, K, ldc, R, row_token, ab);
    return hipGetLastError();
}

using BfRing = RingTile<256, 256, 2, 4>;    // 8 waves of 128 x 64
using Fp8Ring = RingTile<256, 256, 2, 2>;   // 4 waves of 128 x 128

hipError_t launch_bf16_pipe(int epi, const uint16_t* A, const uint16_t* Bw, uint16_t* C, const int32_t* offsets,
                            int R, int E, int N, int K, int ldc, const int32_t* host_counts, hipStream_t s,
                            const uint16_t* aux) {
    if (epi == 1) return launch_bf16_pipe_tile<BfRing, 1>(A, Bw, C, offsets, R, E, N, K, ldc, host_counts, aux, s);
    if (epi == 2) return launch_bf16_pipe_tile<BfRing, 2>(A, Bw, C, offsets, R, E, N, K, ldc, host_counts, aux, s);
    return launch_bf16_pipe_tile<BfRing, 0>(A, Bw, C, offsets, R, E, N, K, ldc, host_counts, aux, s);
}

static int g_ffn_force_wait = 0;
static int g_ffn_give_up = 0;

void set_ffn_force_wait(int on) { g_ffn_force_wait = on ? 1 : 0; }
void set_ffn_give_up(int on) { g_ffn_give_up = on ? 1 : 0; }

static uint32_t ffn_spin_limit() { return g_ffn_give_up ? 0u : kFfnSpinLimit; }

namespace {

template <int KINDS>
hipError_t launch_fused(FusedParams& p, int R, int E, int ntiles_n, const int32_t* host_counts, hipStream_t s) {
    using TL = BfRing;
    // the fused launches need their whole grid (a multiple of 8) resident at once
    if (device_compute_units() < kXcds) return hipErrorInvalidConfiguration;
    p.R = R;
    p.E = E;
    p.spin_limit = ffn_spin_limit();
    p.force_wait = g_ffn_force_wait;
    const int grid = persistent_grid(R, E, ntiles_n * TL::BN, TL::BM, TL::BN, 1, host_counts);
    hipLaunchKernelGGL((gemm_bf16_fused_kernel<TL, KINDS>), dim3(grid), dim3(TL::NTHR), 0, s, p);
    return hipGetLastError();
}

int ntiles(int n) { return (n + BfRing::BN - 1) / BfRing::BN; }

}  // namespace

hipError_t launch_bf16_ffn(const uint16_t* xe, const uint16_t* x, const int32_t* row_token, const uint16_t* w1,
                           uint16_t* h, const uint16_t* w2, uint16_t* ye, const int32_t* offsets, int32_t* sync,
                           int R, int E, int d, int H, const int32_t* host_counts, hipStream_t s, uint16_t* ab) {
    using TL = BfRing;
    if (device_compute_units() < kXcds) return hipErrorInvalidConfiguration;
    const int grid = persistent_grid(R, E, 2 * H + d, TL::BM, TL::BN, 1, host_counts);
    const FfnParams p{xe, x, row_token, w1, h, w2, ye, ab, offsets, sync, R, E, d, H, ffn_spin_limit(),
                      g_ffn_force_wait};
    if (ab)
        hipLaunchKernelGGL((gemm_bf16_ffn_kernel<TL, true>), dim3(grid), dim3(TL::NTHR), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_bf16_ffn_kernel<TL, false>), dim3(grid), dim3(TL::NTHR), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bf16_bwd_chain(const uint16_t* dye, const uint16_t* wd, uint16_t* dh, const uint16_t* xe,
                                 const uint16_t* w1, uint16_t* dab, const uint16_t* w1t, uint16_t* dxe,
                                 const int32_t* offsets, int32_t* sync, int R, int E, int d, int H, hipStream_t s) {
    const int mtmax = R / BfRing::BM + E;
    int32_t* done0 = sync + kSyncHead;
    int32_t* done1 = done0 + mtmax;
    FusedParams p{};
    p.ph[0] = FusedPhase{dye, wd, dh, nullptr, done0, nullptr, H, d, H, kEpiPlain, 0, 1};
    p.ph[1] = FusedPhase{xe, w1, dab, dh, done1, done0, 2 * H, d, 2 * H, kEpiDswiglu, ntiles(H), 1};
    p.ph[2] = FusedPhase{dab, w1t, dxe, nullptr, nullptr, done1, d, 2 * H, d, kEpiPlain, ntiles(2 * H), 0};
    p.nph = 3;
    p.offsets = offsets;
    p.sync = sync;
    return launch_fused<kFusedBackwardKinds>(p, R, E, ntiles(H) + ntiles(2 * H) + ntiles(d), nullptr, s);
}

hipError_t launch_bf16_bwd_chain_kept(const uint16_t* dye, const uint16_t* wd, const uint16_t* ab, uint16_t* dab,
                                      const uint16_t* w1t, uint16_t* dxe, const int32_t* offsets, int32_t* sync,
                                      int R, int E, int d, int H, hipStream_t s) {
    int32_t* done0 = sync + kSyncHead;
    FusedParams p{};
    // dh = dye W_down^T with da | db from the stored a | b in its epilogue, then dxe = (da | db) W1^T
    p.ph[0] = FusedPhase{dye, wd, dab, ab, done0, nullptr, H, d, 2 * H, kEpiDswigluKept, 0, 1};
    p.ph[1] = FusedPhase{dab, w1t, dxe, nullptr, nullptr, done0, d, 2 * H, d, kEpiPlain, ntiles(H), 0};
    p.nph = 2;
    p.offsets = offsets;
    p.sync = sync;
    return launch_fused<kFusedBackwardKeptKinds>(p, R, E, ntiles(H) + ntiles(d), nullptr, s);
}

hipError_t launch_fp8_pipe(int epi, const uint8_t* A, const uint8_t* As, const uint8_t* Bw, const uint8_t* Bs,
                           void* C, uint8_t* Cs, const int32_t* offsets, int R, int E, int N, int K, int ldc,
                           const int32_t* host_counts, hipStream_t s, const int32_t* row_token, uint16_t* ab) {
    if (epi == 1 && ab)
        return launch_fp8_pipe_tile<Fp8Ring, 1, true>(A, As, Bw, Bs, C, Cs, offsets, R, E, N, K, ldc, host_counts, s,
                                                      row_token, ab);
    if (epi == 1)
        return launch_fp8_pipe_tile<Fp8Ring, 1, false>(A, As, Bw, Bs, C, Cs, offsets, R, E, N, K, ldc, host_counts,
                                                       s, row_token, nullptr);
    return launch_fp8_pipe_tile<Fp8Ring, 0, false>(A, As, Bw, Bs, C, Cs, offsets, R, E, N, K, ldc, host_counts, s,
                                                   nullptr, nullptr);
}

}  // namespace moe
