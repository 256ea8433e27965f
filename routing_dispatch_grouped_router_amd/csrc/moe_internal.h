// Host-side launch functions of the gfx950 kernels (internal to the library).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Tokens per routing block: per-block expert histograms and within-block ranks
// are computed over this many consecutive tokens.
constexpr int kRouteBlock = 256;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

enum Act { kF32 = 0, kBF16 = 1, kMXFP8 = 2 };

inline int route_blocks(int T) { return (T + kRouteBlock - 1) / kRouteBlock; }

// Lanes per token in top-k selection: the smallest power of two G <= 64 with
// E / G <= 8 (E / 64 <= 16 at E > 512).
inline int route_lanes(int E) {
    int G = 1;
    while (G < 64 && (E + G - 1) / G > 8) G <<= 1;
    return G;
}

// logits[T][E] = x[T][d] . w[d][E]   (x, w float32 or bfloat16; fp32 accumulate).
// bfloat16: wt is scratch for w^T [E][d] (E d bfloat16), then MFMA.
hipError_t launch_router_logits(int act, const void* x, const void* w, float* logits, int T, int d,
                                int E, uint16_t* wt, hipStream_t s);

// Top-k + gates + per-block histogram and within-block ranks.
//   rank[T][k]   : rank of token t among the tokens of its routing block routed to the same expert
//   hist[nblk][E]: per-block expert counts
// psum (optional, [nblk][E]): per-block sums of the full-softmax router probability;
// ppart is then scratch for nblk * route_lanes(E) * E floats.
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                             float* topk_gate, int32_t* rank, int32_t* hist, float* psum, float* ppart,
                             hipStream_t s);

// counts, offsets and base[nblk][E] = offsets[e] + tokens of earlier blocks routed to e;
// with psum non-NULL also the router statistics stats[E + 2] (see route.hip); zero[0, nzero)
// := 0 on the side (the fused FFN's synchronisation words, so that no separate launch clears them).
hipError_t launch_route_scan(const int32_t* hist, int nblk, int E, int32_t* base, int32_t* counts,
                             int32_t* offsets, const float* psum, float* stats, int T, int k, hipStream_t s,
                             int32_t* zero = nullptr, int nzero = 0);

// pos[t][j] (holding the rank on entry) += base[t / kRouteBlock][idx]; row_token[pos] = t.
hipError_t launch_route_finalize(const int32_t* topk_idx, const int32_t* base, int T, int E, int k,
                                 int32_t* pos, int32_t* row_token, hipStream_t s);

// xe[pos[t][j]] = x[t] (copy), or MXFP8 codes + scales for act == kMXFP8.
// With `base` non-NULL, pos holds within-block ranks on entry and is finalised
// here (pos += base[blk][idx], row_token written) before the copy.
hipError_t launch_dispatch(int act, const void* x, int32_t* pos, const int32_t* topk_idx,
                           const int32_t* base, int32_t* row_token, void* xe, uint8_t* xe_scale,
                           int T, int d, int E, int k, hipStream_t s);

// y[t] = sum_j gate[t][j] * ye[pos[t][j]]   (ye/y float32 for kF32, else bfloat16)
// MXFP8 rows in place: codes xq [T][d] and per-token scale dwords xst [T][d/128]
// of each token row, with pos / row_token finalised as by launch_dispatch;
// then the slice-major scales [d/128][R][4] of the expert-major rows gathered
// through row_token.
hipError_t launch_quantize_mxfp8(const void* x, int32_t* pos, const int32_t* topk_idx, const int32_t* base,
                                 int32_t* row_token, void* xq, uint32_t* xst, int T, int d, int E, int k,
                                 hipStream_t s);
hipError_t launch_scale_gather(const uint32_t* xst, const int32_t* row_token, uint8_t* xs, int R, int d,
                               hipStream_t s);
hipError_t launch_combine(int act, const void* ye, const float* gate, const int32_t* pos, void* y,
                          int T, int d, int k, hipStream_t s);

// Grouped GEMMs over expert segments [offsets[e], offsets[e+1]) of R rows.
//   gemm1: h = silu(xe W_gate) * (xe W_up)   (packed W1 [E][2H][d])
//   gemm2: ye = h W_down                      (packed W2 [E][d][H])
// The kernels read the group sizes from `offsets` in device memory.  The grid
// is sized from the worst case R / BM + E M tiles, or, when the host already
// holds the per-expert counts (host_counts, E entries; NULL otherwise), from
// the exact tile count.
// MXFP8 with row_token non-NULL: xe is the token code matrix [T][d] (d >= 256)
// read through row_token, xe_scale the expert-major row scales.
hipError_t launch_gemm1(int act, const void* xe, const uint8_t* xe_scale, const void* w1,
                        const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                        int R, int E, int d, int H, const int32_t* host_counts, hipStream_t s,
                        const int32_t* row_token = nullptr, uint16_t* ab = nullptr);
hipError_t launch_gemm2(int act, const void* h, const uint8_t* h_scale, const void* w2,
                        const uint8_t* w2_scale, const int32_t* offsets, void* ye, int R, int E,
                        int d, int H, const int32_t* host_counts, hipStream_t s);

// Persistent grid: one workgroup per tile up to per_cu * 256, a multiple of the
// 8 XCDs; for the pipelined kernels (per_cu 1) at most the cap set by
// set_pipe_grid_cap (a multiple of 8 up to 256; 0 removes it; -1 if invalid).
int persistent_grid(int R, int E, int N, int BM, int BN, int per_cu, const int32_t* host_counts);
// Compute units of the current device (cached per device; 0 if the query fails).
int device_compute_units();
int set_pipe_grid_cap(int cap);

// Pipelined bf16 grouped GEMM (gemm_pipe.hip); epi 1 = SwiGLU epilogue (C has N/2 columns);
// epi 2 = SwiGLU backward epilogue (C = da | db from the gate/up pairs and dh = aux [R][N/2]).
hipError_t launch_bf16_pipe(int epi, const uint16_t* A, const uint16_t* Bw, uint16_t* C,
                            const int32_t* offsets, int R, int E, int N, int K, int ldc,
                            const int32_t* host_counts, hipStream_t s, const uint16_t* aux = nullptr);

// Fused bf16 grouped GEMMs (gemm_pipe.hip), d and H at least 128, one persistent
// launch each: the forward expert FFN (GEMM1 with the SwiGLU epilogue into h, then
// GEMM2 into ye) and the backward chain (dh = dye W_down^T, then da | db from the
// gate/up recompute and dh, then dxe = (da | db) W1^T, W1T [E][d][2H]).  sync holds
// fused_sync_ints(R, E, phases) int32 (phases = 2 forward, 3 backward) that must be
// zero when the kernel starts: [0, 8) per-XCD tile counters, word kSyncErrWord the
// error word, then from kSyncHead one counter per M tile for every phase that a later
// phase waits on.  A dependent tile waits at most about kFfnSpinLimit sleeps of 512
// cycles (about 2 s) for the previous phase's tiles of its rows, which take tens of
// microseconds unless other work holds the compute units that long.  A tile that
// reaches the bound sets the error word to 1 and writes its output rows as NaN, so the
// failure is visible (moe_fused_status) instead of a hang of the whole GPU.
constexpr uint32_t kFfnSpinLimit = 1u << 22;
constexpr int kSyncErrWord = 8;
constexpr int kSyncHead = 16;
inline int fused_sync_ints(int R, int E, int phases) { return kSyncHead + (phases - 1) * (R / 256 + E); }
inline int ffn_sync_ints(int R, int E) { return fused_sync_ints(R, E, 2); }
// The fused bf16 expert FFN.  GEMM1's A rows are xe [R][d], or, with row_token
// non-NULL, row row_token[r] of the token rows x [T][d] for expert-major row r
// (the rows the dispatch would have copied into xe, read in place).  With ab
// non-NULL GEMM1 also stores its pre-activations a | b [R][2H] (bf16, the
// packed column order of W1) for the backward.
hipError_t launch_bf16_ffn(const uint16_t* xe, const uint16_t* x, const int32_t* row_token, const uint16_t* w1,
                           uint16_t* h, const uint16_t* w2, uint16_t* ye, const int32_t* offsets, int32_t* sync,
                           int R, int E, int d, int H, const int32_t* host_counts, hipStream_t s,
                           uint16_t* ab = nullptr);
// The backward's data-gradient GEMMs in one launch: dh = dye W_down^T, a | b
// = xe W1 recomputed with da | db in its epilogue, dxe = (da | db) W1^T.
hipError_t launch_bf16_bwd_chain(const uint16_t* dye, const uint16_t* wd, uint16_t* dh, const uint16_t* xe,
                                 const uint16_t* w1, uint16_t* dab, const uint16_t* w1t, uint16_t* dxe,
                                 const int32_t* offsets, int32_t* sync, int R, int E, int d, int H, hipStream_t s);
// The same from the forward's stored a | b: dh = dye W_down^T with da | db in
// its epilogue (no recompute), then dxe = (da | db) W1^T.
hipError_t launch_bf16_bwd_chain_kept(const uint16_t* dye, const uint16_t* wd, const uint16_t* ab, uint16_t* dab,
                                      const uint16_t* w1t, uint16_t* dxe, const int32_t* offsets, int32_t* sync,
                                      int R, int E, int d, int H, hipStream_t s);
// Test hooks of the fused GEMMs: force_wait nonzero makes every dependent tile take the
// wait-and-restart path; give_up nonzero makes every such wait end at once as if its bound
// had been reached (error word raised, the tile's output written as NaN).
void set_ffn_force_wait(int on);
void set_ffn_give_up(int on);
// p[0, n) := 0 (a fill kernel, so that callers may capture it in a graph).
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);

// Pipelined MXFP8 grouped GEMM (gemm_pipe.hip): A/B E4M3 codes with E8M0 scales per 32 K,
// scales stored [K/128][rows][4] (A: R rows; B: per expert, N rows).
// epi 0: bf16 C [.., ldc];  epi 1: SwiGLU then MXFP8 C codes [.., ldc] + scales Cs [ldc/128][R][4].
// epi 1 with row_token non-NULL: A row r is row row_token[r] of a token matrix
// A [T][K] (K >= 256), while As stays per expert-major row.  epi 1 with ab
// non-NULL: the gate/up accumulators also go to ab [R][N] as bf16.
hipError_t launch_fp8_pipe(int epi, const uint8_t* A, const uint8_t* As, const uint8_t* Bw, const uint8_t* Bs,
                           void* C, uint8_t* Cs, const int32_t* offsets, int R, int E, int N, int K, int ldc,
                           const int32_t* host_counts, hipStream_t s, const int32_t* row_token = nullptr,
                           uint16_t* ab = nullptr);

// Weight packing (setup).
hipError_t launch_pack(int act, const void* w_gate, const void* w_up, const void* w_down, void* w1,
                       void* w2, uint8_t* s1, uint8_t* s2, int E, int d, int H, hipStream_t s);

// ---------------------------------------------------------------- backward (backward.hip, pack.hip)

// MXFP8 blocks' backward caches (bfloat16, the forward's quantised values): W1T [E][d][2H],
// packed W1 [E][2H][d] and W_down [E][H][d] from bf16 w_gate, w_up, w_down.
hipError_t launch_pack_bwd_mx(const void* w_gate, const void* w_up, const void* w_down, void* w1t, void* w1,
                              void* wdq, int E, int d, int H, hipStream_t s);
hipError_t launch_copy_bytes(const void* src, void* dst, size_t bytes, hipStream_t s);
// MXFP8 codes [R][K] + scales [K/128][R][4] to bfloat16 [R][K].
// out [R][K] bf16 from codes q (row r, or row rows[r] when rows is non-NULL)
// and the slice-major scales sc [K/128][R][4] of row r.
hipError_t launch_dq_mxfp8(const uint8_t* q, const uint8_t* sc, int R, int K, uint16_t* out, hipStream_t s,
                           const int32_t* rows = nullptr);

// W1T [E][d][2H] from w_gate, w_up [E][d][H] (float32 or bfloat16).
hipError_t launch_pack_w1t(int act, const void* w_gate, const void* w_up, void* out, int E, int d, int H,
                           hipStream_t s);

// dye[pos[t][j]] = gate[t][j] dy[t]; dL[T][E] (router gradient through the softmax of
// the selected logits); dsel[t][j] = dL[t][idx[t][j]], and with srow non-NULL also
// srow[pos[t][j]] = dsel[t][j] (T k floats, the router gradient of every routed row).
hipError_t launch_combine_bwd(int act, const void* dy, const void* ye, const float* gate, const int32_t* pos,
                              const int32_t* idx, void* dye, float* dL, float* dsel, float* srow, int T, int d, int E,
                              int k, hipStream_t s);

// ab [R][2H] (a | b interleaved as packed W1) := da | db from dh [R][H].
hipError_t launch_swiglu_bwd(int act, const void* dh, void* ab, int R, int H, hipStream_t s);

// Weight gradients (float32 outputs), contraction over each expert's rows.
hipError_t launch_wgrad_down(int act, const void* h, const void* dye, const int32_t* offsets, int E, int R, int H,
                             int d, float* dw_down, hipStream_t s);
hipError_t launch_wgrad_w1(int act, const void* xe, const void* dab, const int32_t* offsets, int E, int R, int d,
                           int H, float* dw_gate, float* dw_up, hipStream_t s);
// dw_router[c][e] = sum over expert e's rows r of x[row_token[r]][c] srow[r] (= x^T dL, dL
// being zero outside the selected experts; srow from launch_combine_bwd): part
// router_wgrad_part_bytes(T k, E, d) bytes.
size_t router_wgrad_part_bytes(int R, int E, int d);
hipError_t launch_wgrad_router(int act, const void* x, const int32_t* row_token, const float* srow,
                               const int32_t* offsets, int T, int k, int d, int E, float* part, float* dw_router,
                               hipStream_t s);
// W_r^T [E][d] from W_r [d][E] (activation type).
hipError_t launch_router_transpose(int act, const void* w_router, int d, int E, void* wrt, hipStream_t s);

// dx[t] = sum_j dxe[pos[t][j]] (+ sum_j dsel[t][j] W_r^T[idx[t][j]] when wrt [E][d] is given).
hipError_t launch_dx(int act, const void* dxe, const int32_t* pos, const int32_t* idx, const float* dsel,
                     const void* wrt, void* dx, int T, int d, int E, int k, hipStream_t s);

// bf16: da | db [R][2H] (a | b interleaved as packed W1) from the recomputed gate/up
// projections xe W1 (rounded to bf16) and dh [R][H], in one grouped GEMM.
hipError_t launch_gemm_dswiglu(const void* xe, const void* w1, const void* dh, void* dab, const int32_t* offsets,
                               int R, int E, int d, int H, hipStream_t s);

// C = A B^T per expert segment, stored as computed (float32 or bfloat16): the
// grouped GEMM without an epilogue (recompute and data gradients).
hipError_t launch_gemm_plain(int act, const void* A, const void* B, void* C, const int32_t* offsets, int R, int E,
                             int N, int K, int ldc, hipStream_t s);

// bf16 weight gradients on MFMA (gemm_pipe.hip), per expert e over its rows
// [offsets[e], offsets[e+1]) of the row-major activations XA [R][M], XB [R][N]:
// omap 0: C[e][m][n] = sum_r XA[r][m] XB[r][n]; omap 1: XB's columns interleave gate
// and up (32 + 32 per 64) and go to C (gate) or C2 (up) [e][m][N/2].
hipError_t launch_wgrad_rows(int omap, const uint16_t* XA, const uint16_t* XB, const int32_t* offsets, int E, int M,
                             int N, float* C, float* C2, hipStream_t s);

}  // namespace moe
