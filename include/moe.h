/*
 * moe.h — C ABI of the fused MoE routed-expert layer for AMD Instinct MI355X
 * (gfx950).  Library: expert_gemms_amd/libmoe_gfx950.so.
 *
 * The layer is the one the "DeepGEMM MegaMoE experts" page
 * (vllm.model_executor.layers.fused_moe.deep_gemm_mega_moe) describes as a
 * single launch: token dispatch into per-expert groups padded to BLOCK_M, the
 * L1 grouped GEMM against w13 = [gate; up] with the gated activation in its
 * epilogue, quantisation of the L2 input, the L2 grouped GEMM against w2, and
 * the routing-weighted top-k combine back into token order.  The step order
 * is the one of the "fused_moe" page's DeepGemmExperts.apply.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; host pointers are noted as such.  The caller owns
 *     every buffer.  The library never allocates or frees device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously on it; no entry point synchronises the host.
 *   - Arguments are validated before anything is enqueued; on an error the
 *     return value is negative, nothing is enqueued and no output is touched.
 *   - Device pointers must be 16-byte aligned; shapes below are row-major.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_E_INVALID (-1)     /* bad shape, pointer, size or parameter        */
#define MOE_E_UNSUPPORTED (-2) /* device is not gfx950, or activation/format    */
#define MOE_E_WORKSPACE (-3)   /* workspace too small                           */
#define MOE_E_HIP (-4)         /* a HIP call failed (see moe_status_string)     */
#define MOE_E_TOO_LARGE (-5)   /* the layer needs more intermediate memory than
                                  moe_forward_noalloc's fixed scratch holds      */

/* Routed-expert precisions: one row each of the page's feature matrix
 * (MegaMoEWeightFormat; module docstring of the DeepGEMM MegaMoE page). */
/* Weight formats.  moe_format_t is a plain int so that any value a caller
 * passes is well defined on both sides of the ABI; values other than these
 * four are rejected with MOE_E_INVALID. */
typedef int moe_format_t;
enum {
  MOE_FMT_BF16 = 0,  /* BF16 weights, BF16 dispatch, BF16 L2 input            */
  MOE_FMT_MXFP8 = 1, /* E4M3 weights + UE8M0 per 1x32; MXFP8 activations      */
  MOE_FMT_MXFP4 = 2, /* E2M1 weights (2 per byte) + UE8M0 per 1x32; MXFP8
                        activations (W4A8)                                   */
  MOE_FMT_NVFP4 = 3  /* E2M1 weights + E4M3 per 1x16 + per-expert FP32 global;
                        NVFP4 activations: per-token FP32 scale at dispatch,
                        one global scale for every L2 input                  */
};

/* Gated activation fused into the L1 epilogue (MegaMoEActivation on the
 * DeepGEMM MegaMoE page): swiglu = gate * sigmoid(alpha * gate) * (up + beta)
 * after gate <- min(gate, clamp) and up <- clamp(up, -clamp, clamp).
 * kind must be MOE_ACT_SWIGLU; has_clamp = 0 means no clamp; clamp >= 0;
 * alpha and beta finite.  A NULL pointer means plain SwiGLU (alpha 1,
 * beta 0, no clamp). */
#define MOE_ACT_SWIGLU 0
typedef struct {
  int kind;
  int has_clamp;
  float clamp;
  float alpha;
  float beta;
} moe_activation_t;

/* Output-side options (NULL: none).
 *   post_expert_norm_gamma  float32 [H] (device) or NULL: the output row is
 *       RMS-normalised and scaled, y / sqrt(mean(y^2) + eps) * gamma, in
 *       float32 before the BF16 rounding (the Muse-Spark MegaMoE page's
 *       post_expert_norm_gamma / post_expert_norm_eps; a zero-centred gain
 *       is folded into gamma by the caller).  hidden <= 16384; eps >= 0.
 *   apply_router_weight_on_input  nonzero: each token's routing weight
 *       multiplies its input row (float32, one BF16 rounding) before the
 *       experts and the combine weighs the slot by 1 (the "fused_moe" page's
 *       FusedMoE option of that name).  Needs top_k = 1 and no shared
 *       expert. */
typedef struct {
  const float* post_expert_norm_gamma;
  float post_expert_norm_eps;
  int apply_router_weight_on_input;
} moe_options_t;

/* Human-readable text of a status code (a static string). */
const char* moe_status_string(int status);

/* BLOCK_M the expert groups are padded to for `num_tokens` tokens
 * (get_block_m on the DeepGEMM MegaMoE page names the inputs but prints no
 * formula).  This library's rule: with routed group sizes near-Poisson
 * with mean num_tokens * top_k / num_local_experts and shared groups of
 * num_tokens rows, the candidate of 32, 64, 128, 256 (block-scaled formats:
 * up to 128)
 * whose expected padded row count, divided by the tile's relative MFMA
 * efficiency (0.35, 0.55, 0.85, 1.0; NVFP4, measured: 0.70, 1.0, 0.90), is
 * smallest.  Returns BLOCK_M > 0, or MOE_E_INVALID for
 * num_tokens < 0, top_k < 1, num_local_experts < 1, num_shared < 0 or an
 * unknown format.  Host-only; enqueues nothing. */
int moe_get_block_m(int num_tokens, int num_local_experts, int num_shared,
                    int top_k, moe_format_t fmt);

/* Bytes of workspace moe_forward needs for up to `max_tokens` tokens with
 * the given shape and block_m (0 = the largest BLOCK_M, 256, which covers
 * every block_m).  Returns 0 on invalid arguments.  Host-only. */
size_t moe_workspace_bytes(moe_format_t fmt, int max_tokens, int hidden,
                           int inter, int num_local_experts, int num_shared,
                           int top_k, int block_m);

/* Canonical weights -> kernel layout, out of place (every output buffer has
 * the byte size of its input).  The canonical layout is the one of the
 * DeepGEMM MegaMoE page's _create_weights / the Muse-Spark page's NVFP4
 * parameters, with E = num_experts (local routed experts followed by the
 * shared experts):
 *   w13  [E, 2I, H/vpe] (gate rows 0..I-1, then up rows I..2I-1)
 *   w2   [E, H, I/vpe]
 *   vpe = 1 (BF16: 2-byte elements; MXFP8: 1-byte E4M3), 2 (E2M1, element
 *   2i in the low nibble of byte i, 2i+1 in the high nibble).
 *   w13_sf [E, 2I, H/32] uint8 UE8M0 (MX) or [E, 2I, H/16] uint8 E4M3 (NVFP4);
 *   w2_sf  [E, H, I/32] or [E, H, I/16]; NULL for BF16.
 * The kernel layout pairs gate and up rows in 32-row blocks and stores each
 * 32-row x (MFMA K-step) fragment contiguously in MFMA register order; it is
 * private to this library and read only by moe_forward.
 * hidden and inter must be multiples of 128.  Device pointers. */
int moe_transform_weights(moe_format_t fmt, int num_experts, int hidden, int inter,
                          const void* w13, const void* w13_sf,
                          const void* w2, const void* w2_sf,
                          void* w13_k, void* w13_sf_k, void* w2_k, void* w2_sf_k,
                          void* stream);

/* Weight quantiser (the casts the Qwen4-Exp MegaMoE page's _requantize
 * applies; scale rules as in moe_quantize_x below, with the NVFP4 global
 * scale taken per expert).  src: float32 [num_experts, rows, cols] (device).
 * Writes canonical codes [num_experts, rows, cols/vpe] and block scales
 * [num_experts, rows, cols/group]; for NVFP4 also gscale[num_experts] =
 * amax(|W_e|) / (6 * 448) (1 if the expert is all zero).  fmt must be MXFP8,
 * MXFP4 or NVFP4; cols a multiple of 32. */
int moe_quantize_weights(moe_format_t fmt, int num_experts, int rows, int cols,
                         const float* src, void* codes, void* scales,
                         float* gscale, void* stream);

/* Dispatch quantisation of BF16 activations (prepare_megamoe_inputs /
 * prepare_megamoe_nvfp4_inputs on the DeepGEMM MegaMoE page).
 *   MXFP8 and MXFP4 formats (activations are MXFP8): codes [T, H] uint8 E4M3,
 *     scales [T, H/32] uint8 UE8M0; token_scale unused (may be NULL).
 *   NVFP4: token_scale[T] = amax_t / (6 * 448) (1 for a zero row), codes
 *     [T, H/2] packed E2M1, scales [T, H/16] uint8 E4M3.
 * Scale rules: the MX scale is the smallest power of two 2^e with
 * amax32 <= fmax * 2^e (code 127 + e clamped to [1, 254]; code 0 and zero
 * elements for an all-zero block); NVFP4 block scale bs = E4M3(amax16 /
 * (6 g)), elements E2M1(v * (1 / (bs g))), float32 arithmetic.  Rounding is
 * to nearest even, saturating; a value's sign bit is kept on zero codes.
 * x: BF16 [T, H] (device).  hidden a multiple of 32.  Not for BF16. */
int moe_quantize_x(moe_format_t fmt, int num_tokens, int hidden, const void* x,
                   void* codes, void* scales, float* token_scale, void* stream);

/* Size, in int32 values, of moe_dispatch's optional block_counts scratch
 * for num_tokens tokens: ceil(S / 2048) * E' with S = num_tokens * (top_k +
 * num_shared) slots and E' = num_local_experts + num_shared.  Returns -1 on
 * invalid arguments (negative counts, top_k < 1, num_local_experts < 1).
 * Host-only. */
int64_t moe_dispatch_scratch_ints(int num_tokens, int top_k, int num_shared, int num_local_experts);

/* Router top-k: float32 router logits [T, E] (device) -> topk_ids int32
 * [T, top_k] and topk_weights float32 [T, top_k] (device), the input
 * moe_forward takes.  The routing the "fused_moe" page's
 * FusedMoE.select_experts dispatches to (fused_topk, fused_topk_bias,
 * grouped_topk) and the padding-token skip of the DeepGEMM MegaMoE experts
 * page's forward:
 *   scores   softmax over the token's experts (MOE_SCORE_SOFTMAX) or the
 *            sigmoid of each logit (MOE_SCORE_SIGMOID), float32
 *   choice   score + bias[e] (bias: float32 [E] device, or NULL); the bias
 *            only moves the choice
 *   groups   num_groups contiguous groups of E / num_groups experts (1 = no
 *            grouping); a group ranks by its best choice score and the
 *            topk_groups best groups are kept
 *   ids      the top_k kept experts by choice score, best first, ties to
 *            the lower id (groups likewise)
 *   weights  the chosen experts' unbiased scores, divided by their sum if
 *            renormalize != 0, then times routed_scaling_factor
 *   padding  is_padding: uint8 [T] (device) or NULL; a nonzero entry gives
 *            the token ids -1 and weights 0, so moe_forward drops its slots
 * 1 <= E <= 1024, 1 <= top_k <= min(E, 64), 1 <= topk_groups <= num_groups
 * <= 64, num_groups divides E and the kept groups hold at least top_k
 * experts; routed_scaling_factor finite.  MOE_E_INVALID otherwise (nothing
 * enqueued); one wave per token. */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
int moe_route(int num_tokens, int num_experts, int top_k, const float* logits, const float* bias, int scoring,
              int num_groups, int topk_groups, int renormalize, float routed_scaling_factor,
              const uint8_t* is_padding, int32_t* topk_ids, float* topk_weights, void* stream);

/* Routing metadata (the contiguous-layout permutation of the "fused_moe"
 * page's DeepGemmExperts.apply; groups padded to BLOCK_M as
 * compute_aligned_M does).  A slot is (token t, choice j), flat index
 * t * k' + j with k' = top_k + num_shared; choices j >= top_k are the shared
 * experts, local ids num_local_experts + (j - top_k), always selected.  A
 * routed id outside [expert_start, expert_start + num_local_experts)
 * (including -1) drops its slot.  With E' = num_local_experts + num_shared:
 *   counts[E']        slots per local expert
 *   offsets[E'+1]     exclusive scan of counts rounded up to block_m
 *   sorted_slot[M]    slot ids grouped by expert, ascending within a group,
 *                     -1 for padding rows; M = offsets[E'] <= S + E'(block_m-1)
 *   slot_row[S]       row of each slot in sorted_slot, -1 if dropped
 *   tile_expert[M/block_m] expert of each block_m-row tile
 * The buffers must hold the maximum sizes (sorted_slot: S + E'(block_m - 1),
 * tile_expert: that / block_m).  This is the dispatch moe_forward runs; it is
 * exported so the metadata can be checked on its own.  topk_ids: int32
 * [T, top_k] (device).  block_m in {32, 64, 128, 256}; E' = num_local_experts + num_shared <= 1000.
 * block_counts: NULL, or device scratch of ceil(S / 2048) * E' int32 values;
 * with it and S >= 16384 the work is spread over many workgroups (three
 * launches; moe_forward does this from its workspace), without it one
 * workgroup does it all.  The metadata are the same either way. */
int moe_dispatch(int num_tokens, int top_k, int num_shared, int expert_start,
                 int num_local_experts, int block_m, const int32_t* topk_ids,
                 int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                 int32_t* slot_row, int32_t* tile_expert, int32_t* block_counts, void* stream);

/* The layer (DeepGemmMegaMoEExperts.forward on the DeepGEMM MegaMoE page):
 *   out[t] = sum over slots j of w[t, j] * W2_e * act(W13_e * x_t)
 * with the format's dispatch and L2-input quantisation, float32 accumulation,
 * the slot sum in float32 and one round-to-nearest-even to BF16 (the
 * block-scaled formats round each slot's L2 output row to BF16 first, the
 * dtype the fused_moe page's workspace keeps it in).  Shared
 * slots have weight 1.  Tokens whose every slot is dropped get zeros.
 *   x             BF16 [T, H]                        (device)
 *   topk_ids      int32 [T, top_k] global expert ids (device)
 *   topk_weights  float32 [T, top_k]                 (device)
 *   w13_k ... w2_sf_k  kernel-layout weights from moe_transform_weights with
 *                 num_experts = num_local_experts + num_shared (scales NULL
 *                 for BF16)
 *   w13_gscale, w2_gscale  NVFP4 per-expert FP32 global scales [E'] (device),
 *                 NULL otherwise; l2_activation_scale: NVFP4 global scale of
 *                 every L2 input (the max over experts of w2 input_scale, or
 *                 1.0 if that max is 0), finite and > 0; ignored otherwise
 *   block_m       0 = moe_get_block_m(num_tokens, ...), else 32/64/128/256
 *   act, opts     activation and output-side options, NULL for the defaults
 *   out           BF16 [T, H], fully overwritten            (device)
 *   workspace     >= moe_workspace_bytes(fmt, T, ..., block_m) bytes (device)
 * hidden, inter multiples of 128; 1 <= top_k; num_local_experts >= 1;
 * num_tokens >= 0 (0 enqueues nothing); one expert's w13 codes (2 * inter *
 * hidden elements) and, for the block-scaled formats, x's codes
 * (num_tokens * hidden elements) each below 4 GiB, which the GEMMs address
 * with 32-bit offsets.  MOE_E_INVALID otherwise.  Asynchronous; calls on one
 * stream may share a workspace, concurrent calls need their own. */
int moe_forward(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k,
                int expert_start, int num_local_experts, int num_shared, int block_m,
                const moe_activation_t* act, const moe_options_t* opts,
                const void* x, const int32_t* topk_ids, const float* topk_weights,
                const void* w13_k, const void* w13_sf_k,
                const void* w2_k, const void* w2_sf_k,
                const float* w13_gscale, const float* w2_gscale,
                float l2_activation_scale,
                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward with per-step timing: the same computation and arguments,
 * plus `step_events`, a host array of 2 * MOE_NUM_STEPS hipEvent_t created
 * by the caller (NULL, or NULL entries, skip the recording).  Entry 2i is
 * recorded on `stream` just before step i's kernels, entry 2i + 1 just
 * after, so hipEventElapsedTime gives each step's device time.  Steps:
 * dispatch quantisation (MOE_STEP_QUANT_X, empty for BF16), routing
 * metadata, L1 GEMM with activation and L2-input quantisation, L2 GEMM, and
 * the combine. */
#define MOE_STEP_QUANT_X 0
#define MOE_STEP_DISPATCH 1
#define MOE_STEP_L1 2
#define MOE_STEP_L2 3
#define MOE_STEP_COMBINE 4
#define MOE_NUM_STEPS 5
int moe_forward_profiled(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k,
                         int expert_start, int num_local_experts, int num_shared, int block_m,
                         const moe_activation_t* act, const moe_options_t* opts,
                         const void* x, const int32_t* topk_ids, const float* topk_weights,
                         const void* w13_k, const void* w13_sf_k,
                         const void* w2_k, const void* w2_sf_k,
                         const float* w13_gscale, const float* w2_gscale,
                         float l2_activation_scale,
                         void* out, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* step_events);

/* Where moe_forward keeps its intermediate results inside the workspace, for
 * a call with these arguments (the same rules moe_forward applies: the
 * BLOCK_M of moe_get_block_m when block_m is 0, and K splits only when the
 * workspace holds their float32 parts).  Offsets are bytes from the
 * workspace's start, -1 for a buffer the format does not use.  After a
 * forward the buffers hold (M = offsets[E'] padded rows, S slots):
 *   counts, offsets, sorted_slot, slot_row, tile_expert   int32, as
 *       moe_dispatch writes them
 *   xq, xq_sf, x_tok   the dispatch-quantised x as moe_quantize_x writes it
 *       (MX: E4M3 [T, H] + UE8M0 [T, H/32]; NVFP4: packed E2M1 [T, H/2] +
 *       E4M3 [T, H/16] + float32 token scales [T]); -1 for BF16
 *   a1_sf   xq_sf of each sorted row, one plane per K block: byte m of plane
 *       b (at a1_sf + b * sf_plane) is block b's scale of sorted row m
 *   a2, a2_sf   the L2 input of each sorted row: MX E4M3 [M, I] (row
 *       stride a2_ld bytes) with UE8M0 planes per 32 columns; NVFP4 packed
 *       E2M1 [M, I/2] with E4M3 planes per 16 columns (global scale
 *       l2_activation_scale); BF16 stage-blocked [M / block_m][I / 32]
 *       [block_m][32] BF16 values (a2_sf -1)
 *   o       the L2 output by slot: BF16 [S, H] when l2_rows_bf16, else
 *       float32, l2_ksplit parts of [S, H] one after another; a BF16
 *       layer whose L2 has more tiles than the GPU has work slots splits
 *       only the tiles of its partial last round, whose rows are then in an
 *       unlisted parts buffer, not in o
 * The workspace also holds buffers this struct does not list (the
 * GEMMs' per-block tile records, the many-workgroup dispatch's chunk counts,
 * a K-split L1's float32 parts, the split tail's parts).  The layout is for inspection (tests,
 * debugging); it is not a stable interface.  Returns MOE_OK, MOE_E_INVALID
 * (the shape checks of
 * moe_forward) or MOE_E_WORKSPACE.  Host-only. */
typedef struct {
  int block_m;
  int l1_ksplit, l2_ksplit;
  int l2_rows_bf16;
  int64_t sf_plane, a2_ld;
  int64_t counts, offsets, sorted_slot, slot_row, tile_expert;
  int64_t xq, xq_sf, x_tok, a1_sf;
  int64_t a2, a2_sf;
  int64_t o;
  int64_t bytes;
} moe_workspace_layout_t;
int moe_workspace_layout(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k,
                         int num_local_experts, int num_shared, int block_m, size_t workspace_bytes,
                         moe_workspace_layout_t* layout);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and arguments without a workspace.  The intermediate
 * results live in one fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES per
 * GPU, a static device variable of the library that each GPU holds from the
 * first call on it until the process ends.  Calls whose workspace
 * (moe_workspace_bytes with the call's block_m, or the BLOCK_M the rule
 * picks) exceeds it return MOE_E_TOO_LARGE before anything is enqueued; 64
 * MiB holds decode-sized batches, e.g. up to 256 tokens of a hidden-4096,
 * intermediate-1536, 128-expert top-8 MXFP4 layer.  Nothing is allocated:
 * no hipMalloc, no library allocator.  Every call on a GPU shares that GPU's
 * scratch: calls that may overlap on one GPU (different streams, different
 * host threads) race and must be serialised by the caller; calls on one
 * stream are ordered and safe.  The scratch keeps the last call's contents;
 * no step reads anything an earlier call left. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k,
                        int expert_start, int num_local_experts, int num_shared, int block_m,
                        const moe_activation_t* act, const moe_options_t* opts,
                        const void* x, const int32_t* topk_ids, const float* topk_weights,
                        const void* w13_k, const void* w13_sf_k,
                        const void* w2_k, const void* w2_sf_k,
                        const float* w13_gscale, const float* w2_gscale,
                        float l2_activation_scale, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
