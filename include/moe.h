/*
 * moe.h - C ABI of the MoE expert-parallel layer forward on one MI355X.
 *
 * The layer is the pages' statement of the problem, run on one GPU's share:
 *   moe_route      router scores and top-k gating
 *   moe_dispatch   per-expert counts, offsets, the token <-> slot layout map
 *                  and the permute-gather into expert-contiguous rows
 *   moe_expert_ffn grouped expert FFN (GEMM-1 + activation, GEMM-2)
 *   moe_combine    gate-weighted sum of each token's k expert outputs
 * plus moe_layer_fused, which runs gather -> GEMM-1 -> GEMM-2 -> combine as
 * one persistent, token-tile-pipelined kernel; the fp8 transport pair
 * moe_dispatch_fp8 / moe_expert_ffn_up_fp8; and the placement hooks
 * moe_place_experts (replicated experts) and moe_expert_load_stats.
 *
 * Conventions (all calls):
 *  - Every pointer is a device pointer unless stated otherwise; the caller
 *    owns every buffer.  The library never allocates or frees memory, never
 *    copies device data to the host and never synchronises: all work is
 *    enqueued on `stream` (0 = the null stream) and the calls can be captured
 *    in a hipGraph.  Sizes that depend on the routing (per-expert counts) are
 *    read on the device, never by the host (TensorRT-LLM large-EP page,
 *    "EP communication kernels": sizes read from GPU memory so that the step
 *    stays graph-capturable).
 *  - Arguments are validated on the host before anything is launched; a
 *    negative return code means nothing was enqueued.  MOE_ERR_HIP means a
 *    launch failed (hipGetLastError).  Faults inside kernels are not reported
 *    synchronously.
 *  - Index type is int32; calls with T*k >= 2^31 are rejected.
 *  - Rows are contiguous with leading dimension H (or I); x, x_perm (and
 *    x_perm_q), h_ws, y_perm, out and the weights must be 16-byte aligned
 *    (checked: MOE_ERR_ARG).  Logits must be finite.
 *  - act_dtype selects the activation format: MOE_DTYPE_F32, MOE_DTYPE_F16
 *    or MOE_DTYPE_BF16.  Expert weights use act_dtype, or MOE_DTYPE_FP8_E4M3
 *    (OCP E4M3FN codes with one float32 scale per 128x128 tile) with bf16
 *    activations.
 *  - Calls are stateless and re-entrant.
 */
#ifndef MOE_ROUTE_MI355X_H
#define MOE_ROUTE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,          /* null pointer, bad size or range            */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but not implemented (dtype, shape)   */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or too small             */
  MOE_ERR_HIP = -4,          /* a kernel launch failed                     */
  MOE_ERR_TOO_LARGE = -5     /* sizes exceed a fixed internal scratch      */
};

enum moe_dtype { MOE_DTYPE_F32 = 0, MOE_DTYPE_F16 = 1, MOE_DTYPE_BF16 = 2,
                 MOE_DTYPE_FP8_E4M3 = 3 };
enum moe_gate { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 };
enum moe_act { MOE_ACT_SWIGLU = 0, MOE_ACT_GELU = 1 };
enum moe_ws_kind { MOE_WS_DISPATCH = 0, MOE_WS_FFN = 1, MOE_WS_FUSED = 2 };

/*
 * moe_route - router logits and top-k gating for T tokens.
 *
 * Defines: a router gives every token one score per expert and the top-k
 * experts are chosen (ThunderEP page, section 1.1); softmax over all experts
 * with an optional temperature, then top-k, the weights being the selected
 * probabilities (GPT-4 MoE page, section 4.1, step 2; temperature default
 * 1.0 in the xDeepServe diary, section 5.3).
 *
 *  x         [T][H] act_dtype activations.
 *  w_router  [E][H] act_dtype router weights, or NULL.  When given, the
 *            call first computes logits[t][e] = sum_h x[t][h]*w_router[e][h]
 *            (float32 accumulation) into `logits`; when NULL, `logits` is an
 *            input and x is not read.
 *  bias      [E] float32 added to the logits before selection, or NULL.
 *  gate      MOE_GATE_SOFTMAX: w = softmax over all E of (s * inv_temperature)
 *            evaluated at the picks; MOE_GATE_SIGMOID: w = 1/(1+exp(-s)).
 *            s = logits + bias (one float32 addition).
 *  renorm    nonzero: the kept weights of a token are divided by their sum
 *            (a token with no kept pick keeps zero weights).
 *  min_prob  minimum-probability threshold in [0, 1] (GPT-4 MoE page,
 *            section 2.3 stage 2 and its section 4.1 sketch).  When it is
 *            above 0, a pick whose gate value (before renorm) is not above
 *            min_prob is dropped: topk_idx -1 and topk_w 0.  Gate values fall
 *            with the pick order, so dropped picks are the last ones of a
 *            token.  0 turns the threshold off.
 *  logits    [T][E] float32 (output, or input when w_router is NULL).
 *  topk_idx  [T][k] int32 output: experts by descending s, ties to the lower
 *            index (-0.0 ties with +0.0); -1 for a dropped pick.
 *  topk_w    [T][k] float32 output: gate weights in the same order.
 * Limits: 1 <= k <= E <= 1024, k <= 32, H % 8 == 0.  An inv_temperature
 * that is negative or not finite, or a min_prob outside [0, 1] (or NaN),
 * returns MOE_ERR_ARG.
 */
int moe_route(const void* x, const void* w_router, int act_dtype,
              const float* bias, int T, int H, int E, int k, int gate,
              int renorm, float inv_temperature, float min_prob, float* logits,
              int32_t* topk_idx, float* topk_w, hipStream_t stream);

/*
 * moe_dispatch - counts, offsets, layout map and permute-gather.
 *
 * Defines: dispatch sends each token once to every one of its k experts
 * (DySHARP page, section 1); the destination keeps an algebraic -> layout
 * index table that packs arriving tokens densely, reused in reverse by
 * combine (DySHARP page, section 3.1, item 3); tokens bound for one expert
 * are gathered into one contiguous buffer (ThunderEP page, sections 3.4 and
 * 5.2).
 *
 *  x          [T][H] act_dtype.
 *  topk_idx   [T][k] int32, each in [0, E) and distinct within a token, or
 *             -1 for a pick dropped by moe_route's threshold.
 *  counts     [E]   int32 output: kept (token, pick) pairs per expert.
 *  offsets    [E+1] int32 output: exclusive prefix sum; offsets[E] is the
 *             number of kept picks (T*k without a threshold).
 *  slot_of    [T][k] int32 output: layout row of pick j of token t
 *             = offsets[e] + (number of earlier tokens that picked e);
 *             -1 for a dropped pick.
 *  row_token  [T*k] int32 output: inverse of slot_of (token of each row);
 *             entries at and past offsets[E] are not written.
 *  x_perm     [T*k][H] act_dtype output: x_perm[r] = x[row_token[r]] for the
 *             rows of local experts e_begin <= e < e_end only (global row
 *             numbering; other rows are not written).
 *  ws         workspace of at least moe_workspace_bytes(MOE_WS_DISPATCH, ...)
 *             bytes (per-tile histograms); contents need not be initialised.
 * Counts, offsets and the layout map cover all E experts.
 */
int moe_dispatch(const void* x, int act_dtype, const int32_t* topk_idx,
                 int T, int H, int E, int k, int e_begin, int e_end,
                 int32_t* counts, int32_t* offsets, int32_t* slot_of,
                 int32_t* row_token, void* x_perm, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/*
 * moe_dispatch_noalloc - moe_dispatch without a workspace argument.
 *
 * For callers that cannot allocate device memory: code under stream capture,
 * tight serving loops, harnesses that forbid allocation.  Arguments, layouts,
 * results and validation are those of moe_dispatch; the workspace is instead
 * a fixed array of MOE_NOALLOC_SCRATCH_BYTES bytes inside the library (one
 * per GPU, held from the library's load until the process ends).  Nothing is
 * allocated or freed by the call.  The first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress; MOE_ERR_HIP if that
 * fails).  Sizes whose workspace (moe_workspace_bytes(MOE_WS_DISPATCH, ...)
 * = 8 * E * ceil(T / 256) bytes) exceeds the array return MOE_ERR_TOO_LARGE
 * before anything is launched.  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (different streams without an
 * ordering between them) race and must not be issued; calls ordered on one
 * stream are safe.  Its contents need no clearing between calls.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (1u << 20)
int moe_dispatch_noalloc(const void* x, int act_dtype, const int32_t* topk_idx,
                         int T, int H, int E, int k, int e_begin, int e_end,
                         int32_t* counts, int32_t* offsets, int32_t* slot_of,
                         int32_t* row_token, void* x_perm, hipStream_t stream);

/*
 * moe_dispatch_fp8 - moe_dispatch with the gathered rows sent in 8 bits.
 *
 * Defines: dispatch transport in FP8 (ThunderEP page, section 3.3: the
 * dispatched activations travel as 8-bit floats, halving the bytes).  Each
 * token's row gets one power-of-two scale 2^e, the smallest with
 * max_h |x[t][h]| <= 448 * 2^e (0 for an all-zero row), so x * 2^-e is exact
 * and never saturates; the codes are OCP E4M3FN, round to nearest even.
 *
 * Arguments as moe_dispatch (act_dtype must be MOE_DTYPE_BF16), except:
 *  x_perm_q   [T*k][H] uint8 output: E4M3 codes of x[row_token[r]] * 2^-e,
 *             rows of local experts only.
 *  x_scale    [T*k] float32 output: 2^e of each local row.
 * Counts, offsets, slot_of and row_token are those of moe_dispatch.
 */
int moe_dispatch_fp8(const void* x, int act_dtype, const int32_t* topk_idx,
                     int T, int H, int E, int k, int e_begin, int e_end,
                     int32_t* counts, int32_t* offsets, int32_t* slot_of,
                     int32_t* row_token, void* x_perm_q, float* x_scale, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_up_fp8 - GEMM-1 + activation on fp8-transported rows.
 *
 * Defines: the expert's first Linear and activation (GPT-4 MoE page,
 * section 3.1 table; SwiGLU's two projections) with both operands in fp8,
 * the ThunderEP page's section 3.3 transport feeding the matrix units
 * directly.  h[r] = act(x_scale[r] * sum_k q[r][k] * W13[n][k]), where
 * W13 = decode(w13) * w13_scale block-wise as for MOE_DTYPE_FP8_E4M3
 * weights; products accumulate in float32 per 128-wide k block, the block
 * scale multiplies each block's sum and the row scale the total.
 *
 *  x_perm_q, x_scale  from moe_dispatch_fp8 (global row numbering).
 *  w13, w13_scale     E4M3 weights and their 128x128 block scales, as for
 *                     moe_expert_ffn with w_dtype MOE_DTYPE_FP8_E4M3.
 *  h_ws               [max_rows][I] bf16 output, row r - offsets[e_begin].
 * Limits: H % 128 == 0, H <= 32768, I % 128 == 0 (MOE_ERR_UNSUPPORTED
 * otherwise).  The 32-row tile serves every row count (it is built for
 * decode batches).
 * GEMM-2 and combine are moe_expert_ffn_down and moe_combine, unchanged.
 */
int moe_expert_ffn_up_fp8(const void* x_perm_q, const float* x_scale,
                          const int32_t* offsets, int H, int I, int e_begin,
                          int e_end, int max_rows, int act, const void* w13,
                          const float* w13_scale, void* h_ws, hipStream_t stream);

/*
 * moe_expert_ffn - grouped expert FFN over the local experts' rows.
 *
 * Defines: each expert is an FFN, Linear -> activation -> Linear (GPT-4 MoE
 * page, section 3.1 table); the gated SwiGLU form uses two first-layer
 * projections.  Expert e (local index g = e - e_begin) owns rows
 * [offsets[e], offsets[e+1]) of x_perm; offsets are read on the device.
 *
 *  x_perm     [*][H] act_dtype, global row numbering (as moe_dispatch).
 *  w13        act MOE_ACT_SWIGLU: [E_loc][2I][H]; rows [0,I) are the gate
 *             projection and rows [I,2I) the up projection.
 *             act MOE_ACT_GELU: [E_loc][I][H].
 *  w2         [E_loc][H][I].
 *  w13_scale, w2_scale  float32 scales, one per 128x128 tile
 *             ([E_loc][rows/128][cols/128]) when w_dtype is FP8_E4M3, else
 *             NULL.
 *  h_ws       [max_rows][I] act_dtype workspace for the activation; row
 *             r - offsets[e_begin].
 *  y_perm     [*][H] act_dtype output, global row numbering; only local rows
 *             are written, so rows of other experts keep what the caller put
 *             there (outputs received from other GPUs).
 *  max_rows   host bound on offsets[e_end] - offsets[e_begin], typically
 *             T*min(k, E_loc); it sizes the grid.
 *  ws         optional workspace of at least
 *             moe_workspace_bytes(MOE_WS_FFN, ...) bytes, or NULL.  With it,
 *             when the tiles of a GEMM leave the last round of workgroups at
 *             most half busy, those tiles are split over K: each part stores
 *             fp32 partial sums in the workspace and the last part to finish
 *             adds them in part order (deterministic for a given GPU) before
 *             the epilogue.  Its first 16 KB are arrival counters: they must
 *             be zero before the workspace is first used (zero-fill it once
 *             when it is allocated); every call leaves them zero again, so
 *             no clearing is needed between calls.  The rest need not be
 *             initialised.  Calls that share a workspace must be ordered
 *             (same stream).  A non-NULL workspace that is too small
 *             returns MOE_ERR_WORKSPACE.
 * Computation: fp32 accumulation; SwiGLU h = silu(x Wg^T) * (x Wu^T), GELU
 * h = gelu_erf(x W1^T), h rounded once to act_dtype; y = h W2^T rounded once.
 * Limits: 16-bit types need H % 256 == 0, and I % 128 == 0 with SwiGLU or
 * I % 256 == 0 with GELU (the first GEMM's weight rows, 2I or I, are cut
 * into 256-row tiles); fp32 needs H % 64 == 0 and I % 64 == 0.  Other sizes
 * return MOE_ERR_UNSUPPORTED before anything is launched.
 */
int moe_expert_ffn(const void* x_perm, const int32_t* offsets, int act_dtype,
                   int H, int I, int e_begin, int e_end, int max_rows, int act,
                   const void* w13, const float* w13_scale, const void* w2,
                   const float* w2_scale, int w_dtype, void* h_ws,
                   void* y_perm, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* The two halves of moe_expert_ffn, same arguments and rules:
 * _up computes h from x_perm (GEMM-1 + activation), _down computes y_perm
 * from h (GEMM-2).  moe_expert_ffn = _up then _down on the same stream. */
int moe_expert_ffn_up(const void* x_perm, const int32_t* offsets,
                      int act_dtype, int H, int I, int e_begin, int e_end,
                      int max_rows, int act, const void* w13,
                      const float* w13_scale, int w_dtype, void* h_ws,
                      void* ws, size_t ws_bytes, hipStream_t stream);
int moe_expert_ffn_down(const int32_t* offsets, int act_dtype, int H, int I,
                        int e_begin, int e_end, int max_rows, const void* w2,
                        const float* w2_scale, int w_dtype, const void* h_ws,
                        void* y_perm, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * moe_combine - gate-weighted un-permute reduction.
 *
 * Defines: combine brings the k expert results of a token back to it and
 * reduces them into one (DySHARP page, section 1), as a weighted sum
 * (ThunderEP page, section 2.1).
 *
 *  y_perm  [T*k][H] act_dtype (global row numbering).
 *  slot_of [T][k] int32, topk_w [T][k] float32 (from dispatch / route).
 *  out     [T][H] act_dtype: out[t] = sum_j topk_w[t][j] * y_perm[slot_of[t][j]],
 *          accumulated in float32 in pick order and rounded once.  Picks
 *          with slot_of -1 (dropped by moe_route's threshold) add nothing;
 *          a token with no kept pick gets a zero row.
 */
int moe_combine(const void* y_perm, const int32_t* slot_of,
                const float* topk_w, int act_dtype, int T, int H, int k,
                void* out, hipStream_t stream);

/*
 * moe_layer_fused - gather -> GEMM-1 -> GEMM-2 -> combine in one persistent
 * kernel, pipelined at 128-row token tiles.
 *
 * Defines: the token-centric fusion of dispatch, both expert GEMMs and
 * combine, with readiness gating per tile and a combine that fires once a
 * token's expert outputs are complete (DySHARP page, section 3.2).
 *
 * Inputs are those of moe_dispatch/moe_expert_ffn/moe_combine after
 * moe_route and moe_dispatch have produced offsets, slot_of and row_token
 * (x_perm is not needed: GEMM-1 gathers its rows from x via row_token).
 * Results equal moe_expert_ffn (without workspace) followed by
 * moe_combine, bit for bit: h_ws, y_perm (local rows) and out are written
 * (dropped picks, slot_of -1, as in moe_combine).  ws must hold
 * moe_workspace_bytes(MOE_WS_FUSED, ...) bytes of queue and readiness
 * counters; the call clears them itself (a small kernel before the fused
 * one), so their contents need not be initialised.  Calls sharing a
 * workspace must be ordered (same stream).
 * Status: the int32 at byte offset 32 of ws (MOE_FUSED_STATUS_BYTE) holds
 * the call's status once the call has completed: 0, or 1 when a readiness
 * wait exceeded its bounded spin (about a second; only possible if the
 * device cannot run the kernel's workgroups to completion, for instance
 * when other work keeps one XCD's compute units busy), in which case h_ws,
 * y_perm and out may be incomplete.  The caller reads it after the call has
 * completed (after a stream synchronisation or an event), without any
 * library call.
 * Supported for 16-bit activations with 16-bit weights and SwiGLU.
 */
#define MOE_FUSED_STATUS_BYTE 32
int moe_layer_fused(const void* x, const int32_t* offsets,
                    const int32_t* slot_of, const int32_t* row_token,
                    const float* topk_w, int act_dtype, int T, int H, int E,
                    int k, int I, int e_begin, int e_end, int act,
                    const void* w13, const void* w2, void* h_ws, void* y_perm,
                    void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_place_experts - logical -> physical expert of every pick.
 *
 * Defines: the routing component of large-scale EP reads the placement
 * information so that hot experts can be replicated and their copies placed
 * on physical expert slots (TensorRT-LLM large-EP page, high-level design:
 * GPU-side routing and MoE components adjusted for dynamic placement).
 *
 *  topk_idx     [T][k] int32 logical experts (moe_route), -1 = dropped.
 *  rep_offsets  [E_log+1] int32: the copies of logical expert e are entries
 *               [rep_offsets[e], rep_offsets[e+1]) of rep_phys (at least one).
 *  rep_phys     int32 physical slot of each copy, in [0, E_phys).
 *  topk_phys    [T][k] int32 output: pick j of token t goes to copy
 *               t mod n_e of its expert (n_e copies): an expert's tokens
 *               take its copies in turn.  Dropped picks stay -1, and so
 *               does a pick whose copy names a slot outside [0, E_phys).
 *               rep_offsets must be nondecreasing and index inside
 *               rep_phys (not checked: device data is never read on the
 *               host).
 * moe_dispatch, moe_expert_ffn and moe_combine then run on topk_phys with
 * E = E_phys, the weights of every physical slot in place (a copy holds its
 * logical expert's weights).  topk_w is unchanged.
 */
int moe_place_experts(const int32_t* topk_idx, int T, int k, int E_log, int E_phys,
                      const int32_t* rep_offsets, const int32_t* rep_phys,
                      int32_t* topk_phys, hipStream_t stream);

/*
 * moe_expert_load_stats - online per-expert load statistics.
 *
 * Defines: the statistics component that counts the traffic of every
 * expert on the GPU, the input of the replication and placement computation
 * (TensorRT-LLM large-EP page, high-level design, GPU side).
 *
 *  topk_idx  [T][k] int32 (-1 = dropped, not counted).
 *  stats     [E] uint64, accumulated: stats[e] += number of picks of e in
 *            this call.  The caller zeroes it when a statistics window
 *            starts; calls on one stream accumulate in order.
 */
int moe_expert_load_stats(const int32_t* topk_idx, int T, int k, int E,
                          uint64_t* stats, hipStream_t stream);

/* Workspace bytes needed by moe_dispatch (MOE_WS_DISPATCH), moe_expert_ffn
 * and its halves (MOE_WS_FFN: 16 KB of counters, zero-filled once by the
 * caller, then one 256 KB partial-sum slot per compute unit of the current
 * device) or moe_layer_fused (MOE_WS_FUSED) for these sizes. */
size_t moe_workspace_bytes(int which, int T, int H, int E, int k, int I);

/* Static, human-readable text for a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_MI355X_H */
