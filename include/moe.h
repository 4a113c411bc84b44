/*
 * moe.h -- C ABI of the routed Mixture-of-Experts FFN layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (vLLM-Moet README: a Mixture-of-Experts layer with 384 routed experts, a resident
 * subset of expert slots on the GPU and "compact" calls whose rows for absent experts are
 * computed by another tier -- MoET hybrid table, rows "identity" and "footprint, power"):
 *
 *   logits  l[t,e]  = x[t,:] . W_r[e,:]            fp32 (+ bias[e], fp32)
 *   top-k   e_tj    = k largest logits of token t, ties to the smaller expert id, j = 0..k-1
 *                     in descending order
 *   gates   w_tj    = s(e_tj) / sum_i s(e_ti)      s = softmax over all E, or sigmoid
 *   FFN_e(x)        = W_d,e ( silu(W_g,e x) * (W_u,e x) ),  silu(z) = z / (1 + e^-z)
 *   out[t]          = sum_{j: slot(e_tj) >= 0} w_tj FFN_{e_tj}(x[t])
 *
 * Rows r = t*k + j whose expert has no resident slot are not computed; they are returned as a
 * (token, expert, weight) list in ascending r for another tier to add.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument named as device memory must be device memory of the current HIP
 *     device; the caller owns it.  The library never allocates, frees or synchronises (except
 *     moe_check_device_error, which says so).  Work is enqueued on `stream` (a hipStream_t;
 *     NULL = the null stream) in call order.
 *   - Arguments are validated on the host before any HIP call.  A failing call returns a
 *     non-zero moe_status, enqueues nothing, and leaves a message for moe_last_error().
 *   - Matrices are row-major.  Weights are stored per slot as [N, K] with K (the input
 *     dimension) contiguous: w_gu [S, 2I, H] (rows [0, I) gate, rows [I, 2I) up) and
 *     w_d [S, H, I].
 *   - Device pointers to weights, activations and outputs must be 16-byte aligned, workspaces
 *     256-byte aligned.
 *   - T = 0 is valid: nothing is enqueued.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* a NULL, negative, inconsistent or misaligned argument        */
  MOE_ERR_UNSUPPORTED = 2,  /* a well-formed request outside what the kernels implement     */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes below the matching *_workspace_size()               */
  MOE_ERR_HIP = 4,          /* a HIP launch or runtime call failed                          */
  MOE_ERR_DEVICE = 5        /* a device-side check failed (see moe_check_device_error)      */
} moe_status;

/* Element formats.  Activation buffers use MOE_F32 or MOE_BF16 only. */
typedef enum moe_dtype {
  MOE_F32 = 0,           /* IEEE binary32                                                    */
  MOE_BF16 = 1,          /* bfloat16 (upper half of a binary32)                              */
  MOE_FP8_E4M3_B128 = 2, /* OCP FP8 E4M3 ("fn": bias 7, max 448, no inf) codes, one byte per
                            weight; scales fp32 [S, ceil(N/128), ceil(K/128)], the value of
                            w[n,k] is code * scale[n/128][k/128]                              */
  MOE_MXFP4 = 3          /* OCP MX FP4: E2M1 codes, two per byte (K index 2j in the low nibble
                            of byte j, 2j+1 in the high nibble); scales E8M0 uint8
                            [S, N, K/32], value = e2m1 * 2^(scale - 127)                      */
} moe_dtype;

typedef enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* Expert-FFN implementation.  GEMV streams each touched slot's weights once per group of rows
 * (any weight dtype).  GEMM runs 128-row tiles on the matrix cores and needs bf16 weights with H
 * and I multiples of 64, or FP8 / MXFP4 weights with H and I multiples of 128 (MXFP4: at most
 * 4096); see moe_mode for mode B.  AUTO picks GEMM when it is available and T*k exceeds c*S,
 * else GEMV, with c by weight format from measured crossovers (MI355X, H = 4096, I = 1024):
 * bf16 2.75, FP8 2, MXFP4 0.5 (the multi-row MXFP4 GEMV decodes every weight per row on the
 * vector units and loses to the matrix cores from about 0.5 rows per slot).  INVARIANT picks
 * GEMM whenever it is available for the weights and mode, else GEMV, whatever T is.
 * moe_resolve_path returns the choice.  Asking for GEMM where it is not available fails with
 * MOE_ERR_UNSUPPORTED.
 * Batch invariance (vLLM-Moet README, RTX PRO 6000 table, row "quality": identical requests give
 * identical results at any batch size): with GEMV, GEMM or INVARIANT a token's output is the
 * same bits whatever batch it is computed in -- each path reduces every output element in a
 * fixed order whatever other rows share its slot or tile, and INVARIANT's choice depends on the
 * weights and mode only.  AUTO is not batch-invariant: its choice depends on T, and the two paths
 * round differently (the GEMM path keeps a = silu(g)*u in bf16, the GEMV path in fp32).
 * GEMM tile order: the tiles are dealt to the GPU's eight XCDs in cost-sorted units of a slot's
 * M tiles.  MOE_PATH_TILES_CONTIGUOUS, or'ed into any path value, deals them in the plain
 * (slot, M tile, N tile) order in eight contiguous runs instead (the order the scheduler falls
 * back to when its tables outgrow its LDS).  The order changes only which compute unit runs a
 * tile, never the arithmetic: both give the same bits. */
typedef enum moe_path {
  MOE_PATH_AUTO = 0,
  MOE_PATH_GEMV = 1,
  MOE_PATH_GEMM = 2,
  MOE_PATH_INVARIANT = 3,
  MOE_PATH_TILES_CONTIGUOUS = 0x100 /* flag, or'ed into one of the above */
} moe_path;

/* Expert-FFN arithmetic.  MODE_A: activations kept in bf16/fp32, weights decoded exactly,
 * fp32 accumulation.  MODE_B: the activations entering each projection (x before gate/up, a
 * before down) are quantised per row and per 32 K-elements as moe_quantize_mx_e4m3 does.  The
 * GEMM path then multiplies the E4M3 codes with the FP8 or MXFP4 weights on the block-scaled
 * matrix cores (FP8 or MXFP4 weights only, H and I multiples of 128 and at most 4096); the GEMV
 * path (any weight dtype, H and I multiples of 32) multiplies the dequantised values, which are
 * exact in bf16/fp32.  Mode B is judged against the same quantisation applied in the reference
 * model of the layer. */
typedef enum moe_mode { MOE_MODE_A = 0, MOE_MODE_B = 1 } moe_mode;

/* The expert weights of one layer, in device memory.  S = number of slots, H = hidden size,
 * I = expert intermediate size.  s_gu / s_d are NULL for MOE_F32 and MOE_BF16. */
typedef struct moe_weights {
  int wdtype; /* moe_dtype */
  int S, H, I;
  const void* w_gu; /* [S, 2I, H]; MXFP4: [S, 2I, H/2] bytes                         */
  const void* s_gu; /* FP8: float [S, ceil(2I/128), ceil(H/128)]; MXFP4: [S, 2I, H/32] */
  const void* w_d;  /* [S, H, I];  MXFP4: [S, H, I/2] bytes                           */
  const void* s_d;  /* FP8: float [S, ceil(H/128), ceil(I/128)];  MXFP4: [S, H, I/32]  */
} moe_weights;

/* Routing configuration.  1 <= k <= min(E, 64), E <= 1024. */
typedef struct moe_routing {
  int E;      /* number of routed experts                                  */
  int k;      /* experts per token                                         */
  int score;  /* moe_score                                                 */
  int renorm; /* non-zero: gates divided by the sum of the k chosen scores */
} moe_routing;

/* ------------------------------------------------------------------------------------------
 * moe_route -- router logits, top-k selection, scores and renormalised gates.
 *
 * Exactly one of w_router / logits is non-NULL.
 *   x         device [T, H], x_dtype MOE_F32 or MOE_BF16; unused (may be NULL) with `logits`
 *   w_router  device fp32 [E, H]: logits are computed as x . W_r^T, fp32 accumulation
 *             (H a multiple of 4, at most 8192; MOE_ERR_UNSUPPORTED otherwise)
 *   logits    device fp32 [T, E]: logits handed in directly
 *   bias      device fp32 [E] or NULL, added to the logits in fp32 before selection
 *   topk_idx  device int32 [T, k] out: expert ids, descending logit, ties to the smaller id
 *   topk_w    device fp32 [T, k] out: gates (renormalised if cfg->renorm)
 *   logits_out device fp32 [T, E] out or NULL: with w_router, where the computed logits (+bias)
 *             are stored; NULL keeps them in the workspace.  With w_router and logits_out given,
 *             topk_idx and topk_w may both be NULL: then only the logits are computed (one launch)
 *   ws        device workspace of moe_route_workspace_size() bytes (may be 0 bytes / NULL)
 * ------------------------------------------------------------------------------------------ */
size_t moe_route_workspace_size(int T, const moe_routing* cfg, int with_router_weights);
int moe_route(const void* x, int x_dtype, int T, int H, const float* w_router,
              const float* logits, const float* bias, const moe_routing* cfg, int32_t* topk_idx,
              float* topk_w, float* logits_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_permute -- expert histogram, slot grouping and the compact miss list.
 *
 * Row r = t*k + j is resident if slot(e) >= 0, where slot(e) = slot_map[e] (slot_map device
 * int32 [E], entries in [-1, S)) or slot(e) = e when slot_map is NULL (then S must equal E).
 *   counts       device int32 [E] out: rows per expert, absent experts included
 *   slot_offsets device int32 [S+1] out: slot s owns positions [off[s], off[s+1]); off[S] is
 *                the number of resident rows n_res
 *   perm         device int32 [T*k] out: perm[p] = r for p < n_res, ordered by (slot, r)
 *   inv_perm     device int32 [T*k] out: position of row r, or -1 if r is not resident
 *   miss_count   device int32 [1] out: number of non-resident rows (required with slot_map)
 *   miss_token / miss_expert (int32) / miss_weight (fp32 = topk_w of the row): device [T*k]
 *                out, the first miss_count entries hold the non-resident rows in ascending r.
 *                Required with slot_map; ignored (may be NULL) without it.
 *   topk_w       device fp32 [T, k]; needed only with slot_map.
 * An expert id outside [0, E) or a slot_map entry outside [-1, S) drops that row (it is
 * neither resident nor a miss, inv_perm = -1) and raises the workspace error word.
 * ------------------------------------------------------------------------------------------ */
size_t moe_permute_workspace_size(int T, const moe_routing* cfg, int S);
int moe_permute(const int32_t* topk_idx, const float* topk_w, int T, const moe_routing* cfg,
                const int32_t* slot_map, int S, int32_t* counts, int32_t* slot_offsets,
                int32_t* perm, int32_t* inv_perm, int32_t* miss_count, int32_t* miss_token,
                int32_t* miss_expert, float* miss_weight, void* ws, size_t ws_bytes,
                void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_route_permute -- moe_route followed by moe_permute in as few launches as possible (for
 * batches of up to 64 tokens the top-k of every token and the permutation share one work-group).
 * Arguments as in those two calls; the results are identical to calling them in sequence.
 *   ws  device workspace of moe_route_permute_workspace_size() bytes; its first 256 bytes hold
 *       the device error word read by moe_check_device_error
 * ------------------------------------------------------------------------------------------ */
size_t moe_route_permute_workspace_size(int T, const moe_routing* cfg, int S, int with_router_weights);
int moe_route_permute(const void* x, int x_dtype, int T, int H, const float* w_router,
                      const float* logits, const float* bias, const moe_routing* cfg,
                      const int32_t* slot_map, int S, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* slot_offsets, int32_t* perm, int32_t* inv_perm,
                      int32_t* miss_count, int32_t* miss_token, int32_t* miss_expert,
                      float* miss_weight, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_expert_ffn -- y_perm[p] = FFN_{slot of p}(x[perm[p] / k]) for every resident position p.
 *
 *   w             weights descriptor (host struct, device pointers inside)
 *   x             device [T, H], x_dtype MOE_F32 or MOE_BF16
 *   perm, slot_offsets  as produced by moe_permute (device)
 *   path          moe_path; mode moe_mode
 *   y_perm        device fp32 [T*k, H] out; rows >= n_res untouched
 *   ws            device workspace of moe_expert_ffn_workspace_size() bytes
 * moe_expert_gate_up and moe_expert_down are its two halves: gate_up leaves
 * a = silu(W_g x) * (W_u x) in the workspace, down reads it.  Call them in that order with the
 * same workspace, weights, T, k, path and mode.
 * Positions whose perm entry names a token outside [0, T) are skipped.
 * ------------------------------------------------------------------------------------------ */
size_t moe_expert_ffn_workspace_size(const moe_weights* w, int T, int k, int path, int mode);

/* Where moe_expert_gate_up leaves the intermediate a in the expert-FFN workspace, for callers that
 * inspect it (tests, debugging).  Fills, for the same (w, T, k, path, mode) as the call:
 *   offsets[0]  byte offset of a: fp32 [T*k, I] on the GEMV path (mode B: the quantised values);
 *               mode A on the GEMM path bf16 [T*k, I], or, where H*I >= 2^25, rows of 2I bf16
 *               values (the I hi halves, then the I lo halves: a = hi + lo)
 *   offsets[1]  byte offset of the E4M3 codes of a, uint8 [T*k, I] (mode B on the GEMM path)
 *   offsets[2]  byte offset of their E8M0 scales, uint8 [T*k, I/32] (same)
 *   offsets[3]  the format of a: 0 = fp32, 1 = bf16, 2 = bf16 (hi, lo) pairs, 3 = E4M3 + E8M0
 * Rows are positions p < slot_offsets[S]; offsets that do not apply are (size_t)-1.  Returns
 * MOE_OK, or MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED as moe_expert_ffn would. */
int moe_expert_ffn_workspace_layout(const moe_weights* w, int T, int k, int path, int mode, size_t offsets[4]);

int moe_expert_ffn(const moe_weights* w, const void* x, int x_dtype, int T, int k,
                   const int32_t* perm, const int32_t* slot_offsets, int path, int mode,
                   float* y_perm, void* ws, size_t ws_bytes, void* stream);
int moe_expert_gate_up(const moe_weights* w, const void* x, int x_dtype, int T, int k,
                       const int32_t* perm, const int32_t* slot_offsets, int path, int mode,
                       void* ws, size_t ws_bytes, void* stream);
int moe_expert_down(const moe_weights* w, int T, int k, const int32_t* slot_offsets, int path,
                    int mode, float* y_perm, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_combine -- out[t] = sum over j ascending of topk_w[t,j] * y_perm[inv_perm[t*k+j]],
 * resident rows only, fp32 accumulation, then rounded (nearest-even) to out_dtype.  A token
 * with no resident row gets a zero row.  H % 4 == 0.
 *   y_perm device fp32 [>= n_res, H]; inv_perm device int32 [T*k]; topk_w device fp32 [T*k];
 *   out device [T, H] of out_dtype (MOE_F32 or MOE_BF16).
 * ------------------------------------------------------------------------------------------ */
int moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int T, int k,
                int H, void* out, int out_dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_combine_tiers -- moe_combine over two tiers of computed rows: the consumer of the compact
 * miss list.  The pages compute the rows routed to absent experts on another tier and add them
 * to the compact output, which then equals the all-resident output (vLLM-Moet README, the
 * compact MoE calls and CPU-computed rows; MoET hybrid table, row "identity").  Here the other
 * tier is a second weight pool with its own slot map: run moe_permute with a map that sends
 * exactly the experts absent from tier a to pool slots (and the others to -1), and
 * moe_expert_ffn on that pool, which gives y_b and inv_b.
 *   y_a, inv_a   tier a rows: fp32 [*, H] and int32 [T*k] positions (-1: not in tier a)
 *   y_b, inv_b   tier b rows, likewise; both NULL = moe_combine
 *   out[t] = sum over j ascending of topk_w[t,j] * (y_a[inv_a[r]] if inv_a[r] >= 0, else
 *            y_b[inv_b[r]] if inv_b[r] >= 0, else nothing), r = t*k + j, fp32, one rounding.
 * Positions at or past T*k count as absent.  Summed in the same order as moe_combine over one
 * pool holding both tiers' experts, so with the same FFN path the output equals that of the
 * one-pool layer bit for bit.  Errors as moe_combine; y_b and inv_b must be given together.
 * ------------------------------------------------------------------------------------------ */
int moe_combine_tiers(const float* y_a, const int32_t* inv_a, const float* y_b, const int32_t* inv_b,
                      const float* topk_w, int T, int k, int H, void* out, int out_dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_layer -- route, permute, expert FFN and combine in one call, one workspace, no host
 * synchronisation.
 *   x, x_dtype, T, w_router / logits, bias, cfg   as moe_route (H = w->H)
 *   slot_map      device int32 [E] or NULL (all resident, w->S == cfg->E)
 *   w, path, mode as moe_expert_ffn
 *   out           device [T, H] out, out_dtype MOE_F32 or MOE_BF16
 *   topk_idx, topk_w  device [T, k] out, or NULL to keep them in the workspace
 *   miss_*        as moe_permute (required with slot_map)
 *   ws            device workspace of moe_layer_workspace_size() bytes; its first 256 bytes
 *                 hold the device error word read by moe_check_device_error
 * ------------------------------------------------------------------------------------------ */
size_t moe_layer_workspace_size(int T, const moe_routing* cfg, const moe_weights* w, int path,
                                int mode, int with_router_weights);
int moe_layer(const void* x, int x_dtype, int T, const float* w_router, const float* logits,
              const float* bias, const moe_routing* cfg, const int32_t* slot_map,
              const moe_weights* w, int path, int mode, void* out, int out_dtype,
              int32_t* topk_idx, float* topk_w, int32_t* miss_count, int32_t* miss_token,
              int32_t* miss_expert, float* miss_weight, void* ws, size_t ws_bytes,
              void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_layer_decode_fused -- whether moe_layer runs this batch as the two-launch decode layer.
 * It does for T <= 4 tokens and T*k <= 32 rows (MXFP4 weights; 8 rows for the others, whose
 * bytes per slot stream better on the staged launches once a batch touches many slots) on the
 * GEMV path (`path` resolved as
 * moe_resolve_path does) in mode A, when the two launches' LDS fits: T rows of x plus the E-entry
 * slot map within 96 KB, and T*k fp32 rows of a plus their output columns within 144 KB.  There
 * every work-group of the first launch selects the batch's experts itself from the logits (a
 * wave per token; the router logits of w_router are computed first, by their own launch) and
 * computes gate/up for one resident slot, and the second launch computes the down projection of
 * every row for 16 output columns and combines them in place.  The outputs (out, top-k ids and
 * gates, miss list and count, the device error word) are the same bits as the staged launches
 * give, since each element is formed by the same arithmetic in the same order; only fewer
 * launches and fewer dependent memory round trips separate a decode layer's inputs from its
 * output (the pages' decode step: MoET hybrid table, row "the step").
 * Returns 1 or 0, or -1 for invalid arguments.
 * ------------------------------------------------------------------------------------------ */
int moe_layer_decode_fused(int T, const moe_routing* cfg, const moe_weights* w, int path, int mode,
                           int x_dtype);

/* ------------------------------------------------------------------------------------------
 * moe_decode_gate_up, moe_decode_down_combine -- the two launches of the decode layer, for
 * callers that schedule them themselves (moe_layer makes exactly these calls, after the router
 * logits when router weights are given).  Shapes as moe_layer_decode_fused requires (T <= 4,
 * T*k <= 32 or 8, the LDS rule); MOE_ERR_UNSUPPORTED otherwise.  Call them in order on one stream.
 *
 * moe_decode_gate_up: routing (top-k of the given logits, scores and gates as moe_route), the
 * slot of each row, the compact miss list (as moe_permute) and a = silu(x W_g^T) * (x W_u^T) of
 * every resident row, stored by row index (not permuted).
 *   x            device [T, H] of x_dtype; logits device fp32 [T, E]; bias device fp32 [E] or NULL
 *   slot_map     device int32 [E] or NULL (then w->S == cfg->E)
 *   topk_idx, topk_w  device [T, k] out
 *   row_slot     device int32 [T*k] out: slot of row t*k+j, -1 when it has none here
 *   a            device fp32 [T*k, I] out (16-byte aligned); rows without a slot are not written
 *   miss_count   device int32 [1] out; miss_token / miss_expert / miss_weight device [T*k] out
 *                (required with slot_map, ignored without)
 *   err          device uint32 word out: 1 when a slot_map entry is outside [-1, S), else 0
 *                (moe_check_device_error reads it)
 * moe_decode_down_combine: out[t] = sum over j ascending of topk_w[t,j] * (a_r W_d^T) for the
 * rows r = t*k+j with row_slot[r] >= 0, fp32, one rounding to out_dtype.
 *   row_slot, topk_w, a  as the first call wrote them; out device [T, H] of out_dtype
 * ------------------------------------------------------------------------------------------ */
int moe_decode_gate_up(const void* x, int x_dtype, int T, const float* logits, const float* bias,
                       const moe_routing* cfg, const int32_t* slot_map, const moe_weights* w,
                       int32_t* topk_idx, float* topk_w, int32_t* row_slot, float* a,
                       int32_t* miss_count, int32_t* miss_token, int32_t* miss_expert,
                       float* miss_weight, uint32_t* err, void* stream);
int moe_decode_down_combine(const moe_weights* w, int T, const moe_routing* cfg,
                            const int32_t* row_slot, const float* topk_w, const float* a, void* out,
                            int out_dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_layer_static -- moe_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that forbid allocation): the same arguments and results without
 * ws / ws_bytes; the workspace is a static array of MOE_STATIC_WORKSPACE_BYTES in the library,
 * one per GPU, held until the process ends.  Nothing is allocated or freed.
 *   Limit: moe_layer_workspace_size() of the call must be at most MOE_STATIC_WORKSPACE_BYTES
 *   (32 MiB: at H = 4096, I = 1024, k = 8 up to 192 tokens), else MOE_ERR_UNSUPPORTED and
 *   nothing is enqueued.
 *   Every call on a GPU uses that GPU's one array: calls that overlap on one GPU (other streams,
 *   other threads) race and must be ordered by the caller.  The array keeps the last call's
 *   contents; nothing in it needs to start at zero (each call writes what it reads, the device
 *   error word included), and moe_check_device_error cannot be pointed at it.
 * ------------------------------------------------------------------------------------------ */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
int moe_layer_static(const void* x, int x_dtype, int T, const float* w_router, const float* logits,
                     const float* bias, const moe_routing* cfg, const int32_t* slot_map,
                     const moe_weights* w, int path, int mode, void* out, int out_dtype,
                     int32_t* topk_idx, float* topk_w, int32_t* miss_count, int32_t* miss_token,
                     int32_t* miss_expert, float* miss_weight, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_quantize_mx_e4m3 -- the mode-B activation quantisation, on its own (OCP MX rule with an
 * E4M3 element type).  For each row and each 32 consecutive elements: X = floor(log2 amax) - 8
 * (X = 0 for an all-zero block; X is kept >= -127), scale byte X + 127 (E8M0), codes = E4M3
 * (e4m3fn) of v / 2^X rounded to nearest even and saturated at +-448.  Quantised value =
 * code * 2^X exactly.
 *   in      device [rows, K], in_dtype MOE_F32 or MOE_BF16, 16-byte aligned; K % 32 == 0
 *   codes   device uint8 [rows, K] out, or NULL
 *   scales  device uint8 [rows, K/32] out, or NULL
 *   deq     device [rows, K] out of deq_dtype (MOE_F32 or MOE_BF16): the quantised values, or
 *           NULL; may be `in` itself when in_dtype == deq_dtype == MOE_F32
 * ------------------------------------------------------------------------------------------ */
int moe_quantize_mx_e4m3(const void* in, int in_dtype, int rows, int K, uint8_t* codes, uint8_t* scales,
                         void* deq, int deq_dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_accumulate_counts / moe_plan_slots -- hot-set placement of the resident slots.  The
 * recipes wiki (Home page, the expert balance) keeps resident the experts the traffic routes to
 * most, chosen from routing histograms by a greedy pick of the largest routing share per byte of
 * weights.  Every expert has the same storage size here, so that share orders as the
 * accumulated count.
 *   moe_accumulate_counts: hist[e] += counts[e] for e < E (counts: device int32 [E], e.g. the
 *       counts output of moe_permute; hist: device int64 [E], 8-byte aligned, zeroed by the
 *       caller before the first call)
 *   moe_plan_slots: slot_map[e] (device int32 [E] out) = the rank of e in (hist descending,
 *       expert id ascending) if that rank is below S, else -1; so slot i holds the i-th hottest
 *       expert.  1 <= S <= E <= 1024.  Deterministic.
 * Errors: MOE_ERR_INVALID_ARG for sizes out of range, NULL or misaligned pointers.
 * ------------------------------------------------------------------------------------------ */
int moe_accumulate_counts(const int32_t* counts, int E, int64_t* hist, void* stream);
int moe_plan_slots(const int64_t* hist, int E, int S, int32_t* slot_map, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_refill_slots -- LRU refill of the resident slots after a call (the pages' "full LRU", where
 * every resident slot is a spare held by the most recently used experts: vLLM-Moet README, the
 * MoET hybrid measurement matrix, the 4x RTX 5090 row with SPARE=110 and its hit rate).  Each
 * expert that missed in the call moves into a slot for the next call:
 *   1. every slot whose expert took rows in the call (counts > 0) gets last_use = step;
 *   2. the missed experts (counts > 0, slot_map -1) in order of (rows descending, id ascending)
 *      take the slots not used in the call in order of (last_use ascending, slot ascending),
 *      as many as both lists allow (empty slots: slot_expert -1 and a last_use below any step);
 *   3. slot_map, slot_expert and last_use are updated and each moved expert's weights are copied
 *      from the store into its slot.
 *   counts       device int32 [E]: the call's rows per expert (moe_permute's counts)
 *   step         the call's number; increasing from call to call
 *   slot_map     device int32 [E] in/out (the layer's slot map); slot_expert device int32 [S]
 *                in/out (its inverse, -1 for an empty slot); last_use device int64 [S] in/out
 *   store        weights of every expert (store->S == E, slot e = expert e): the backing tier
 *   slots        the resident weights (slots->S = S <= E), same format and shape
 *   ws           device workspace of moe_refill_workspace_size(S) bytes, 256-byte aligned; after
 *                the call it holds the number of moves (int32 at byte 0) and the moves as
 *                (slot, expert) int32 pairs from byte 256
 * Deterministic; E <= 1024.  Errors: MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE before any launch.
 * ------------------------------------------------------------------------------------------ */
size_t moe_refill_workspace_size(int S);
int moe_refill_slots(const int32_t* counts, int E, long long step, int32_t* slot_map, int32_t* slot_expert,
                     int64_t* last_use, const moe_weights* store, const moe_weights* slots, void* ws,
                     size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * helpers
 * ------------------------------------------------------------------------------------------ */
/* Reads the error word at the start of a moe_permute / moe_route_permute / moe_layer workspace: synchronises
 * `stream`, returns MOE_OK, MOE_ERR_DEVICE (an out-of-range expert id or slot_map entry was
 * seen) or MOE_ERR_HIP. */
int moe_check_device_error(const void* ws, void* stream);
/* Static description of a status code. */
const char* moe_status_string(int status);
/* Message of the last failing call made by this thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);
/* The implementation moe_expert_ffn / moe_expert_gate_up / moe_expert_down run for these
 * arguments: `path` itself when it is MOE_PATH_GEMV or MOE_PATH_GEMM, AUTO's choice otherwise
 * (see moe_path).  Returns MOE_PATH_GEMV or MOE_PATH_GEMM, or -1 for invalid weights or path. */
int moe_resolve_path(const moe_weights* w, int T, int k, int path, int mode);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
