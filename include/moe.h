/*
 * moe.h - C ABI of the MI355X (gfx950) routed MoE block forward.
 *
 * The block, as the Olmo-core MoE report describes it ("Supercharging Olmo-core
 * for Efficient and Scalable MoE Training", Abstract; "Section 24: Conclusion",
 * 24.1 and Evidence 3 / Figure 74; explainer "Olmo-core 3: an open training
 * stack for trillion-parameter MoE", section "Olmo-core 3's answer: experts
 * resident, data routed"):
 *
 *   router logits -> softmax + top-k -> per-expert counts / offsets / positions
 *   computed and kept on the device -> rowwise dispatch that writes each token
 *   row straight into its expert's segment (no separate permutation) ->
 *   SwiGLU experts as a grouped GEMM whose group sizes never leave the device
 *   (no padding of experts to a common capacity) -> gate-weighted combine
 *   back to token order.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; the caller owns every buffer.  The library never
 *    allocates device memory, never frees, never copies to the host and never
 *    synchronises inside these calls (except moe_kernel_times, the status
 *    query moe_fused_status and the comparison path moe_forward_host_sync,
 *    see there).
 *    All work is enqueued on `stream` (a hipStream_t; NULL = default stream),
 *    so calls on one stream are ordered and the whole sequence is capturable
 *    in a HIP graph.
 *  - Row-major layouts.  T tokens, d = d_model, E experts, k = top_k,
 *    H = d_hidden, R = T*k routed rows.
 *  - Storage types by `act_dtype`:
 *        MOE_F32   : x, xe, h, ye, y float32; weights float32.
 *        MOE_BF16  : x, xe, h, ye, y bfloat16; weights bfloat16; fp32 accumulate.
 *        MOE_MXFP8 : x bfloat16; xe and h are MXFP8 (E4M3 codes, one E8M0
 *                    scale byte per 32 consecutive elements along the GEMM
 *                    contraction axis); weights given bfloat16 and stored
 *                    MXFP8 by moe_pack_weights; ye and y bfloat16.
 *    Logits and gates are always float32; indices int32.
 *  - MXFP8 follows OCP Microscaling (MX) v1.0: E4M3 "FN" (bias 7, max 448, no
 *    infinities), shared exponent floor(log2(amax)) - 8 clamped to [-127,127]
 *    (all-zero block -> 2^-127), elements rounded to nearest-even, saturated
 *    to +-448, sign kept on zero.  Payload 33/32 bytes per value (report
 *    Section 24, Evidence 10).
 *  - Routing: experts ranked by float32 logit, ties to the lower expert index
 *    (-0.0 == +0.0); slot j of a token holds its j-th largest logit.  Gates
 *    are the softmax over all E renormalised over the k selected experts.
 *    Rows of one expert are ordered by ascending token index (stable), experts
 *    back to back without padding: offsets[e] = sum of counts[e' < e].
 *  - Shapes supported: 1 <= k <= min(E, 16), E <= 1024, T >= 1, and
 *    d, H multiples of 64 (MOE_F32, MOE_BF16) or of 128 (MOE_MXFP8); the
 *    bytes of an [R, max(d, H)] activation buffer and of one expert's
 *    [2H, d] weights must each stay below 2^32.
 *  - Errors: every entry point returns MOE_OK or a negative MOE_ERR_* code.
 *    Arguments are validated on the host before anything is enqueued; a
 *    failed check enqueues nothing.  MOE_ERR_LAUNCH reports hipGetLastError()
 *    after a launch.  Faults inside kernels surface at the caller's next
 *    synchronisation.  Preconditions not checked: logits are finite; pos /
 *    offsets buffers come from moe_route for the same problem.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK             0
#define MOE_ERR_NULL      -1   /* a required pointer is NULL                      */
#define MOE_ERR_SHAPE     -2   /* unsupported T, d, E, k or H                      */
#define MOE_ERR_DTYPE     -3   /* unknown act_dtype, or flag not valid for it      */
#define MOE_ERR_WORKSPACE -4   /* ws_bytes smaller than moe_workspace_bytes()      */
#define MOE_ERR_LAUNCH    -5   /* a kernel launch or HIP runtime call failed       */
#define MOE_ERR_STATE     -6   /* no profiled forward yet; inconsistent host counts */
#define MOE_ERR_ARG       -7   /* a setting outside its documented range           */

#define MOE_F32   0
#define MOE_BF16  1
#define MOE_MXFP8 2

/* flags */
#define MOE_LOGITS_GIVEN     1  /* logits are an input; skip the router GEMM x . W_r     */
#define MOE_IDENTITY_EXPERTS 2  /* test mode of moe_forward: ye := xe (f32 / bf16 only)  */
/* MOE_KEEP_GATE_UP: moe_forward also stores the experts' pre-activations
 * a | b = xe W1 (bf16 of GEMM1's float32 accumulators, [T*k][2H] in the
 * packed column order) in its workspace, and moe_backward reads them instead
 * of recomputing xe W1.  The report treats recompute as an option that trades
 * throughput for activation memory ("Section 24: Conclusion", Evidence 11;
 * its per-block recompute cost about a fifth of the throughput); without this
 * flag the library recomputes, with it the forward keeps 4 T k H more bytes.
 * MOE_BF16 (d_model, d_hidden >= 128: the fused FFN's blocks): the gradients
 * are bit for bit those of the recomputing path.  MOE_MXFP8: the stored a | b
 * come from the forward's MXFP8 GEMM, the recompute is a bf16 GEMM of the
 * dequantised values, so the gradients differ by their accumulation order
 * only.  Any other problem with the flag is MOE_ERR_DTYPE.  moe_forward and
 * moe_forward_host_sync honour it; the staged calls ignore it.  moe_backward
 * must be given the problem (flags included) its moe_forward ran with: with
 * the flag it reads a | b from fwd_ws, whose size then includes them (a
 * forward workspace sized without the flag is MOE_ERR_WORKSPACE). */
#define MOE_KEEP_GATE_UP     4

typedef struct moe_problem {
    int32_t T;          /* tokens                                 */
    int32_t d_model;    /* d                                      */
    int32_t n_experts;  /* E                                      */
    int32_t top_k;      /* k                                      */
    int32_t d_hidden;   /* H, expert SwiGLU hidden size           */
    int32_t act_dtype;  /* MOE_F32 | MOE_BF16 | MOE_MXFP8         */
    int32_t flags;      /* MOE_LOGITS_GIVEN | MOE_IDENTITY_EXPERTS | MOE_KEEP_GATE_UP */
} moe_problem;

/* Library version string and a readable name of a status code (host only). */
const char* moe_version(void);
const char* moe_status_string(int32_t status);

/* Device workspace, in bytes, that is enough for every entry point below on
 * problem p (host only, no GPU call).  Contents need no initialisation and are
 * overwritten by every call.  The caller allocates it once and passes it to
 * every call, so the block's buffers keep fixed addresses from step to step
 * (report "Section 24: Conclusion", 24.3: graph replay needs buffers at stable
 * addresses, reused only after their last consumer).  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE / MOE_ERR_DTYPE for an invalid problem. */
int32_t moe_workspace_bytes(const moe_problem* p, size_t* bytes);

/* Size in bytes of the packed expert weights for p (host only, no GPU call):
 * the regions moe_pack_weights writes, described there (report "Section 24:
 * Conclusion", 24.3: weight caches built once, in the layout the GEMM reads).
 * Errors: as moe_workspace_bytes. */
int32_t moe_packed_weight_bytes(const moe_problem* p, size_t* bytes);

/* Packs the expert weights once, outside the timed path: re-lays them out with
 * the contraction axis contiguous and, for MOE_MXFP8, quantises them (report
 * "Section 24: Conclusion", 24.3: MXFP8 weight caches kept beside the
 * high-precision weights, produced by a quantiser in the layout the GEMM
 * consumes, so no per-step conversion kernel runs).  The caller owns both
 * buffers; the inputs are not modified.  Errors: MOE_ERR_NULL for a NULL
 * pointer, shape/dtype errors as moe_workspace_bytes; nothing is enqueued on
 * an error.
 *   w_gate, w_up : device [E, d, H]   (x . W convention), storage type above
 *   w_down       : device [E, H, d]
 *   packed       : device, moe_packed_weight_bytes() bytes, layout:
 *     W1 [E][2H][d] : row n of expert e is gate column h = 32*(n/64) + n%32 when
 *                     (n/32) is even, else up column h (same formula); i.e. 32
 *                     gate columns then the matching 32 up columns, repeated.
 *     W2 [E][d][H]  : W2[e][n][j] = w_down[e][j][n].
 *     Elements are float32 / bfloat16 / E4M3 by act_dtype.  For MOE_MXFP8 the
 *     E8M0 scales follow, each covering 32 consecutive elements of a row and
 *     stored slice-major: S1 [E][d/128][2H][4], then S2 [E][H/128][d][4], where
 *     S[e][s][n][j] is the scale of elements [128 s + 32 j, 128 s + 32 j + 32)
 *     of packed row n (the layout the GEMM loads without conversion).
 *   Regions are W1, W2, S1, S2 in that order, each starting at a multiple of
 *   256 bytes. */
int32_t moe_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up,
                         const void* w_down, void* packed, void* stream);

/* Routing (report: count routes on the GPU, metadata kept on the device,
 * Section 24.1 and Evidence 3).
 *   x        : device [T, d] (storage type of act_dtype; MXFP8: bfloat16);
 *              unused (may be NULL) with MOE_LOGITS_GIVEN
 *   w_router : device [d, E], same type as x; unused with MOE_LOGITS_GIVEN
 *   logits   : device float32 [T, E]; input with MOE_LOGITS_GIVEN, else output
 *   topk_idx : device int32 [T, k] out;  topk_gate : device float32 [T, k] out
 *   counts   : device int32 [E] out;     offsets   : device int32 [E+1] out
 *   pos      : device int32 [T, k] out, row of (token, slot) in the expert-major
 *              buffer: offsets[e] + number of earlier tokens routed to e
 *   row_token: device int32 [R] out, row_token[pos[t][j]] = t
 *   router_stats : device float32 [E + 2] out, or NULL to skip.  The report
 *              asks that the requested route counts be inspected next to the
 *              Switch-style balance scalar, which mixes soft router scores with
 *              hard counts ("Section 24: Conclusion", 24.3 and Evidence 9 /
 *              Figure 45); its formula is not printed, the Switch form is used:
 *                [e]     P_e = mean over tokens of softmax(logits[t])[e]
 *                [E]     E * sum_e (counts[e] / (T k)) * P_e
 *                [E + 1] max_e counts[e] / (T k / E)   (worst-case load / mean)
 *              Computed in the top-k pass; sums run in a fixed order, so the
 *              values are reproducible bit for bit.
 *   ws       : device workspace of ws_bytes bytes */
int32_t moe_route(const moe_problem* p, const void* x, const void* w_router, float* logits,
                  int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                  int32_t* pos, int32_t* row_token, float* router_stats, void* ws, size_t ws_bytes,
                  void* stream);

/* moe_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Arguments, outputs and results are those of moe_route (bit for bit: the
 * same kernels run); there is no workspace argument.  The routing scratch
 * (per-block expert histograms and bases, per-block router-probability
 * partials and, for a bfloat16 / MXFP8 learned router, the transposed router
 * weights) lives in a library-owned device array of MOE_ROUTE_SCRATCH_BYTES
 * bytes, one per GPU, set up on the first call on that GPU and held until
 * the process ends.  The call allocates and frees nothing.
 * The kernels write every scratch byte they read, so no state carries from
 * one call to the next; but every call on one GPU uses that GPU's single
 * array, so calls that overlap on one GPU (other streams, other threads)
 * race and give wrong results: serialise them.
 * Errors: as moe_route; MOE_ERR_WORKSPACE (nothing enqueued) when the
 * problem's routing scratch, the routing part of moe_workspace_bytes' layout
 * (about ceil(T/256) * E * (12 + 4 G) bytes, G <= 64 the lanes per token in
 * top-k selection, plus E * d * 2 for a bfloat16 / MXFP8 learned router,
 * each region rounded up to 256 bytes), exceeds MOE_ROUTE_SCRATCH_BYTES;
 * MOE_ERR_LAUNCH if the array's device address cannot be obtained. */
#define MOE_ROUTE_SCRATCH_BYTES (4 << 20)
int32_t moe_route_noalloc(const moe_problem* p, const void* x, const void* w_router, float* logits,
                          int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                          int32_t* pos, int32_t* row_token, float* router_stats, void* stream);

/* Rowwise dispatch (report Abstract: each token row written directly into its
 * expert's buffer): xe[pos[t][j]] = x[t] for every slot.
 *   x        : device [T, d]
 *   pos      : device int32 [T, k] from moe_route
 *   xe       : device [R, d] out (MOE_MXFP8: uint8 E4M3 codes), 16-byte aligned
 *   xe_scale : device uint8 [d/128][R][4], 4-byte aligned, out for MOE_MXFP8, else ignored (may
 *              be NULL): xe_scale[s][r][j] is the E8M0 scale of elements
 *              [128 s + 32 j, 128 s + 32 j + 32) of row r, so the four scales
 *              of a 128-wide slice of a row form one dword and the dwords of
 *              consecutive rows are adjacent, the layout the grouped GEMM reads
 *              directly (report "Section 24: Conclusion", 24.3: a quantiser
 *              should emit what the consumer reads without conversion) */
int32_t moe_dispatch(const moe_problem* p, const void* x, const int32_t* pos, void* xe,
                     uint8_t* xe_scale, void* stream);

/* Expert SwiGLU FFN as a grouped GEMM whose groups are read from device
 * memory (report: device-scheduled grouped GEMM, no padding to a capacity):
 *   for every expert e and row r in [offsets[e], offsets[e+1]):
 *     h  = silu(xe[r] . W_gate[e]) * (xe[r] . W_up[e])   (stored in workspace)
 *     ye[r] = h . W_down[e]
 *   xe, xe_scale : as written by moe_dispatch
 *   packed_w     : from moe_pack_weights
 *   offsets      : device int32 [E+1] from moe_route
 *   ye           : device [R, d] out (float32 for MOE_F32, else bfloat16)
 *   ws           : workspace (holds h and, for bfloat16, the counters of the
 *                  fused launch, cleared by each call; calls sharing a
 *                  workspace must not overlap)
 * bfloat16 (d_model and d_hidden >= 128) runs both projections in one
 * persistent launch: a GEMM2 tile starts once the GEMM1 tiles of its rows have
 * finished, so neither GEMM ends in a partly filled round.  That wait is
 * bounded (about 2 s) so that the launch cannot hang the GPU: if other work
 * kept this launch's GEMM1 workgroups off the compute units for longer, the
 * GEMM2 tile stops waiting, writes its rows of ye as NaN (never a wrong
 * finite value) and sets an error word in the workspace, which
 * moe_fused_status reports.  The grid never exceeds the device's compute-unit
 * count, so on an otherwise idle GPU every wait ends normally.
 * Every output tile is computed whole by one workgroup in a fixed K order, so
 * the result does not depend on the grid (moe_set_gemm_grid_cap). */
int32_t moe_grouped_swiglu(const moe_problem* p, const void* xe, const uint8_t* xe_scale,
                           const void* packed_w, const int32_t* offsets, void* ye, void* ws,
                           size_t ws_bytes, void* stream);

/* Combine back to token order (report Abstract: combine without a permutation):
 *   y[t] = sum over j = 0..k-1, in slot order, of topk_gate[t][j] * ye[pos[t][j]],
 *   accumulated in float32 and rounded to nearest-even into y.
 *   ye : device [R, d]; y : device [T, d] out (float32 for MOE_F32, else bfloat16) */
int32_t moe_combine(const moe_problem* p, const void* ye, const float* topk_gate,
                    const int32_t* pos, void* y, void* stream);

/* The whole block on one stream: route, dispatch, grouped SwiGLU, combine, with
 * no host synchronisation between them.  For MOE_BF16 with d_model and
 * d_hidden >= 128 the dispatch is not materialised: the fused grouped GEMM
 * reads each expert-major row r straight from x[row_token[r]] (the row the
 * dispatch would have copied), so no xe is written and the routing pass only
 * finalises pos and row_token.  For MOE_MXFP8 with d_model >= 256 each token
 * row is quantised once (codes and scales per token, not per routed row),
 * GEMM1 reads the code rows through row_token, and only the E8M0 scales are
 * laid out per expert-major row.  y is the same either way ("Supercharging Olmo-core ...",
 * Section 2, the design paragraph after Figure 5: no extra permutation, no
 * device-to-host synchronisation and no gap between launches; Abstract:
 * device-scheduled grouped GEMMs).  The caller owns every buffer; ws is at
 * least moe_workspace_bytes(p) bytes, and calls sharing a workspace must not
 * overlap.  All arguments are validated on the host before anything is
 * enqueued: a non-zero status means nothing ran.  Arguments as above; topk_idx,
 * topk_gate, counts, offsets, pos and router_stats are optional outputs (NULL:
 * kept in the workspace only, or for router_stats not computed).  With
 * MOE_IDENTITY_EXPERTS the grouped GEMM is skipped and ye := xe (MOE_F32 /
 * MOE_BF16 only), so y[t] = x[t] * sum_j gate[t][j]. */
int32_t moe_forward(const moe_problem* p, const void* x, const void* w_router, float* logits,
                    const void* packed_w, void* y, int32_t* topk_idx, float* topk_gate,
                    int32_t* counts, int32_t* offsets, int32_t* pos, float* router_stats, void* ws,
                    size_t ws_bytes, void* stream);

/* The same block with one host wait, for comparison with moe_forward: the
 * original MoE path the report measures against needed the per-expert routing
 * counts on the CPU before the grouped-GEMM group sizes were known ("Section
 * 24: Conclusion", 24.1 and Evidence 3 / Figure 74: one device-to-host copy
 * and host wait per routed block).  After routing, the counts are copied to
 * host_counts (host memory of E int32, owned by the caller; pinned memory
 * avoids a staging copy) and the calling thread waits for the stream before it
 * sizes the grouped-GEMM grids from them and enqueues the rest.  Every output
 * is bit-identical to moe_forward's (same kernels; only the grid size and the
 * wait differ).  Not capturable in a HIP graph.  With profiling on (below) the
 * stage "host_count_wait" is the GPU time from the end of routing until work
 * resumes after the wait.  Errors: as moe_forward, MOE_ERR_NULL for a NULL
 * host_counts, MOE_ERR_STATE if the copied counts do not sum to T*k. */
int32_t moe_forward_host_sync(const moe_problem* p, const void* x, const void* w_router, float* logits,
                              const void* packed_w, void* y, int32_t* topk_idx, float* topk_gate,
                              int32_t* counts, int32_t* offsets, int32_t* pos, float* router_stats, void* ws,
                              size_t ws_bytes, void* stream, int32_t* host_counts);

/* Per-kernel timing of moe_forward with HIP events recorded on its stream.
 * moe_set_profiling(1) makes later moe_forward calls record an event before
 * the first kernel and after each kernel (events are created on first use and
 * kept; the last 128 calls keep separate events).  moe_set_profiling resets
 * the count of profiled calls.  moe_kernel_times waits for the last profiled
 * call to finish (this call synchronises on its final event) and writes up to
 * max_n stage names and their durations in milliseconds averaged over the
 * profiled calls (at most the last 128); *n receives the number of stages.
 * Returns MOE_ERR_STATE when no profiled call completed its launches.  Not for
 * use while a graph capture of moe_forward is in progress. */
int32_t moe_set_profiling(int32_t enable);

int32_t moe_kernel_times(const char** names, float* ms, int32_t max_n, int32_t* n);

/* Caps the persistent grid of the bf16 and MXFP8 grouped GEMMs at `cap`
 * workgroups (one per compute unit; a multiple of 8 in [8, 256]), for callers
 * that keep compute units free for concurrent work on another stream; 0
 * removes the cap.  Process-wide, applies to calls launched afterwards; not
 * for use while another thread launches.  Returns MOE_ERR_ARG for any other
 * value. */
int32_t moe_set_gemm_grid_cap(int32_t cap);

/* Test hooks for the fused bfloat16 grouped GEMMs (the forward expert FFN of
 * moe_grouped_swiglu / moe_forward and the backward's data-gradient chain):
 * MOE_TEST_FFN_WAIT makes every dependent tile skip the early check of its
 * rows and start only after waiting for them (the path a tile takes when its
 * rows are not yet done), so tests can show that this path gives the same
 * result; outputs are unchanged, only speed drops.  MOE_TEST_FFN_GIVE_UP makes
 * every such wait end at once as if its bound had been reached, without
 * looking at the counter: the tile writes NaN and raises the error word that
 * moe_fused_status reports (every kernel still runs to completion), so tests
 * can check the failure path.  Process-wide, applies to calls launched
 * afterwards; 0 clears them.  Returns MOE_ERR_ARG for unknown bits. */
#define MOE_TEST_FFN_WAIT 1
#define MOE_TEST_FFN_GIVE_UP 2
int32_t moe_set_test_flags(int32_t flags);

/* Outcome of the bounded dependency waits of the last fused grouped-GEMM
 * launch that used workspace ws (the report's Section 24.3 asks that buffers be
 * reused only after their last consumer has finished and that such
 * dependencies be explicit at component interfaces; in the fused launches one
 * GEMM's tiles consume rows another GEMM's tiles produce, and a tile that
 * stops waiting for its producers makes the broken dependency explicit here).
 *   which  : MOE_STATUS_FORWARD for the workspace of moe_forward /
 *            moe_forward_host_sync / moe_grouped_swiglu (ws_bytes >= the
 *            grouped-GEMM part of moe_workspace_bytes), MOE_STATUS_BACKWARD
 *            for the workspace of moe_backward (ws_bytes >=
 *            moe_backward_workspace_bytes)
 *   status : host int32 out: MOE_OK, or MOE_ERR_STATE if some dependent tile
 *            gave up waiting, in which case its output rows (ye in the
 *            forward; dh, da | db or dxe and what derives from them in the
 *            backward) hold NaN.
 * The word is cleared by every call that launches a fused kernel on ws, so it
 * describes the last such call; for problems that run no fused launch (other
 * dtypes or small d, H) the status is MOE_OK without a device access.
 * Synchronises: the word is copied to the host after the work already queued
 * on `stream` and the calling thread waits for it. */
#define MOE_STATUS_FORWARD 0
#define MOE_STATUS_BACKWARD 1
int32_t moe_fused_status(const moe_problem* p, const void* ws, size_t ws_bytes, int32_t which, int32_t* status,
                         void* stream);

/* ---------------------------------------------------------------- backward
 *
 * Gradients of the block for a loss L with dL/dy = dy (MOE_IDENTITY_EXPERTS
 * returns MOE_ERR_DTYPE).  The report runs the block's backward with the
 * dispatch and combine as each other's transposes, grouped GEMMs for data and
 * weight gradients and the block forward re-executed ("Section 24:
 * Conclusion", Evidence 7 and Evidence 11).  With g the gates (the softmax of
 * the k selected logits):
 *
 *   dgate[t,j] = dy[t] . ye[pos[t,j]]          dye[pos[t,j]] = g[t,j] dy[t]
 *   dlogits[t,e_j] = g_j (dgate_j - sum_i g_i dgate_i), 0 for unselected e
 *   a | b = xe W1 (recomputed, or stored with MOE_KEEP_GATE_UP);  dh = dye W_down^T
 *   da = dh b silu'(a);  db = dh silu(a);  dxe = da W_gate^T + db W_up^T
 *   dw_down[e] = h^T dye,  dw_gate[e] = xe^T da,  dw_up[e] = xe^T db
 *                                              (sums over expert e's rows)
 *   dx[t] = sum_j dxe[pos[t,j]]  (+ dlogits[t] W_r^T for the learned router)
 *   dw_router = x^T dlogits                     (learned router only; summed
 *               per expert over that expert's token rows)
 *
 * Storage: dye, a, b, dh, da, db, dxe and dx in the activation type (bf16
 * rounded to nearest even where stored), dlogits and all weight gradients
 * float32.  MOE_MXFP8 blocks follow Evidence 7 (dequantise, then bf16): the
 * saved MXFP8 xe and h are dequantised to bf16 (exactly), the weights are the
 * bf16 values of the forward's MXFP8 weights, and every step above runs in
 * bf16 (dy, dx bf16).  Every reduction runs in a fixed order: results are
 * bitwise reproducible.  All work is enqueued on `stream`; nothing allocates
 * or synchronises, so the call is capturable in a HIP graph.
 *
 * moe_backward_weight_bytes / moe_pack_weights_backward: the backward weight
 * cache (the report's second weight cache, 24.3), built once from w_gate,
 * w_up [E, d, H] and w_down [E, H, d] (device, the activation type; bf16 for
 * MOE_MXFP8): W1T [E][d][2H], row c holding for each column n of the packed
 * W1 (32 gate then 32 up hidden units per 64) the weight of input c; W_down
 * [E][H][d]; for MOE_MXFP8 also the packed W1 in bf16.  MOE_MXFP8 stores the
 * dequantised MXFP8 values (blocks of 32 along each forward GEMM's
 * contraction axis, as moe_pack_weights quantises them).
 *
 * moe_backward arguments (device pointers unless noted):
 *   dy          [T, d] activation type (bf16 for MOE_MXFP8)
 *   x           [T, d] the forward's input.  Required for the learned router
 *               and for MOE_BF16 blocks with d_model and d_hidden >= 128 (their
 *               forward reads the token rows in place and keeps no dispatched
 *               copy, so the backward gathers them from x again); otherwise
 *               unused and may be NULL
 *   w_router    [d, E] activation type (learned router only; may be NULL with
 *               MOE_LOGITS_GIVEN)
 *   packed_w    the forward weight cache (moe_pack_weights); unused, may be
 *               NULL, for MOE_MXFP8
 *   packed_bwd  the backward weight cache (moe_pack_weights_backward)
 *   topk_idx, topk_gate, offsets, pos : the forward's routing arrays, or NULL
 *               for the copies moe_forward kept in its workspace when it was
 *               given NULL for them
 *   fwd_ws      the workspace of the moe_forward call being differentiated,
 *               unchanged since (it holds h, ye, row_token and the dispatched
 *               rows: none for the gathering bf16 blocks above, one MXFP8
 *               code row per token for MXFP8 blocks with d_model >= 256, one
 *               per routed row otherwise; with MOE_KEEP_GATE_UP also a | b);
 *               fwd_ws_bytes >= moe_workspace_bytes
 *   dx          [T, d] out, activation type (bf16 for MOE_MXFP8)
 *   dlogits     [T, E] out, float32
 *   dw_gate, dw_up [E, d, H] out, dw_down [E, H, d] out, float32
 *   dw_router   [d, E] out, float32 (learned router only; may be NULL with
 *               MOE_LOGITS_GIVEN)
 *   ws          backward workspace, ws_bytes >= moe_backward_workspace_bytes
 * Errors: as moe_forward; MOE_ERR_SHAPE also when T*k*2H elements of the
 * backward's activation type exceed 2^32 bytes. */
int32_t moe_backward_workspace_bytes(const moe_problem* p, size_t* bytes);
int32_t moe_backward_weight_bytes(const moe_problem* p, size_t* bytes);
int32_t moe_pack_weights_backward(const moe_problem* p, const void* w_gate, const void* w_up, const void* w_down,
                                  void* packed_bwd, void* stream);
int32_t moe_backward(const moe_problem* p, const void* dy, const void* x, const void* w_router, const void* packed_w,
                     const void* packed_bwd, const int32_t* topk_idx, const float* topk_gate, const int32_t* offsets,
                     const int32_t* pos, const void* fwd_ws, size_t fwd_ws_bytes, void* dx, float* dlogits,
                     float* dw_gate, float* dw_up, float* dw_down, float* dw_router, void* ws, size_t ws_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
