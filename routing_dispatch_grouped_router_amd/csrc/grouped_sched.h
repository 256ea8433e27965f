// Device-side tile schedule of the grouped GEMMs.
//
// The group sizes come from the expert offsets in device memory and never
// reach the host ("Supercharging Olmo-core ...", Abstract: device-scheduled
// grouped GEMMs; explainer "Olmo-core 3 ...", section "Olmo-core 3's answer":
// uneven per-expert shapes run without padding every expert to a common
// capacity).  Every workgroup derives the same schedule in LDS:
//   tstart[e] = sum over e' < e of ceil(n_e' / BM)   (M tiles before expert e)
// and walks tile ids in block order (block_tile: 4 M tiles x 8 N tiles per
// block), so the tiles of one expert are consecutive and each run of 32 ids
// shares 4 row blocks and 8 weight slices.  The grid is persistent (bounded by the CU count times the occupancy,
// and by the worst-case tile count the host can bound without reading the
// offsets); workgroup b takes tiles b', b' + G, b' + 2G, ... where b' spreads
// consecutive ids over one XCD (the hardware deals workgroups round-robin over
// the 8 XCDs, each with its own L2), so the workgroups sharing an expert's
// weights and rows mostly share an L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kXcds = 8;

// Logical slot of workgroup `bid` among G (G a multiple of 8): consecutive
// slots land on the same XCD.
__device__ __forceinline__ int xcd_slot(int bid, int G) {
    if (G % kXcds) return bid;
    return (bid % kXcds) * (G / kXcds) + bid / kXcds;
}

// Fills s_tstart[0..E] (E <= 1024) with the M-tile prefix; returns total M tiles.
// Must be called by all threads of the workgroup (contains barriers).
template <int BM, int NTHREADS>
__device__ __forceinline__ int build_tile_schedule(const int32_t* __restrict__ offsets, int E,
                                                   int* s_tstart, int* s_scan) {
    const int tid = threadIdx.x;
    const int per = (E + NTHREADS - 1) / NTHREADS;
    const int e0 = tid * per;
    int local = 0;
    for (int e = e0; e < min(E, e0 + per); ++e) {
        const int n = offsets[e + 1] - offsets[e];
        local += (n + BM - 1) / BM;
    }
    s_scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < NTHREADS; off <<= 1) {
        int v = tid >= off ? s_scan[tid - off] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    int run = s_scan[tid] - local;     // exclusive prefix of this thread's experts
    for (int e = e0; e < min(E, e0 + per); ++e) {
        s_tstart[e] = run;
        const int n = offsets[e + 1] - offsets[e];
        run += (n + BM - 1) / BM;
    }
    if (tid == NTHREADS - 1) s_tstart[E] = s_scan[NTHREADS - 1];
    __syncthreads();
    return s_tstart[E];
}

// Tile j of a GEMM with MT x NT output tiles, in block order: blocks of 4 M
// tiles x 8 N tiles (smaller at the edges), the blocks of one row of 4 M tiles
// in N order, rows in M order, the tiles of a block M-major.  A persistent
// grid deals consecutive runs of 32 tile ids to one XCD, so with this order a
// run is one 4 x 8 block: it reads 4 row blocks of activations and 8 weight
// slices, the fewest distinct bytes (and L2 misses) for 32 tiles, whatever NT
// is (M-major ids give 32 / NT row blocks x NT slices when NT is not 8).
__device__ __forceinline__ void block_tile(int j, int MT, int NT, int& mt, int& nt) {
    const int mg = j / (4 * NT);
    const int r = j - mg * 4 * NT;
    const int mc = min(4, MT - 4 * mg);   // M tiles in this row of blocks
    const int ng = r / (mc * 8);
    const int s = r - ng * mc * 8;
    const int nc = min(8, NT - 8 * ng);   // N tiles in this block
    const int mi = s / nc;
    mt = 4 * mg + mi;
    nt = 8 * ng + (s - mi * nc);
}

// Expert owning global M tile `mt`: the largest e < E with tstart[e] <= mt
// (empty experts share their successor's start and are skipped).
__device__ __forceinline__ int tile_expert(const int* s_tstart, int E, int mt) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (s_tstart[mid] <= mt) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace moe
