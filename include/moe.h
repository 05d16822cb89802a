/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts layer of
 * Reflection's Beam model: hidden 5120, 256 routed experts, 8 per token.
 *
 * The layer, as the pages state it:
 *  - the router is a GEMM of shape (5120, 256) with BF16 output (vLLM PR
 *    #61978 "Day-0 support for Reflection's Beam-1.0", Status table, row
 *    #62042), computed by an FP32 router kernel (UpstreamBeat "vLLM adds
 *    day-zero Reflection Beam serving...", section "Agents worked on the
 *    serving path"; the pre-release router-dtype switch is gone, PR #61978
 *    "What landed differs");
 *  - every token is routed to 8 of 256 experts (vLLM recipe
 *    "reflection/Beam-1.0-501B-A23B", Guide > Overview);
 *  - the expert GEMMs are grouped per expert, gate and up projections are
 *    one merged GEMM ("merged projections", UpstreamBeat, same section);
 *  - a "MoE finalize" step combines the routed outputs per token (PR #61978,
 *    Status table row #62366 and Remaining work);
 *  - the quantised variant stores only the routed experts in NVFP4 and runs
 *    them with BF16 activations (recipe, Guide > Variants).
 * Conventions the pages leave open and this library fixes: softmax over all
 * E logits, top-k by (logit desc, expert id asc), weights renormalised over
 * the k chosen experts; SwiGLU h = silu(g) * u with gate = columns [0, I) and
 * up = columns [I, 2I) of the merged matrix; no biases in the experts.
 *
 * Calling conventions (all entry points):
 *  - Array arguments are DEVICE pointers owned by the caller (for example
 *    torch tensors' data_ptr()), row-major and contiguous, 16-byte aligned.
 *    The library allocates no memory and keeps no global state, except the
 *    device scratch area of moe_forward_noalloc (below).
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on
 *    it and the call returns without synchronising the host, so a whole
 *    forward pass can be captured into a hipGraph.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued and a non-zero moe_status is returned. Device
 *    faults surface at the caller's next synchronisation.
 *  - Supported range: 1 <= k <= 8, k <= E <= 256, H and I multiples of 64,
 *    0 <= T < 2^24 (T == 0 is a successful no-op), T*k < 2^31. Outside it the call
 *    returns MOE_ERR_UNSUPPORTED.
 *  - Dtype combinations: x fp32 with fp32 expert weights (logits fp32), or
 *    x bf16 with bf16, FP8-E4M3 or NVFP4 expert weights. The router weights
 *    are always fp32.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null required pointer, negative size, k > E, bad dtype */
  MOE_ERR_UNSUPPORTED = 2,      /* valid but outside the supported range or combination */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_LAUNCH = 4 /* a HIP launch or runtime call failed */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2, /* OCP E4M3 (bias 7, no infinities, max 448) */
  MOE_FP4_E2M1 = 3  /* NVFP4: E2M1 codes, E4M3 scale per 16 K elements, fp32 scale per expert */
} moe_dtype;

/* Expert weights of one layer (device pointers).
 *  MOE_F32 / MOE_BF16: gate_up [E, H, 2I], down [E, I, H] (N contiguous);
 *      scales NULL.
 *  MOE_FP8_E4M3: gate_up [E, 2I, H] and down [E, H, I] E4M3 codes (K
 *      contiguous); gate_up_scale f32 [E, 2I], down_scale f32 [E, H] (one per
 *      output channel); gscales NULL. W = e4m3(q) * scale.
 *  MOE_FP4_E2M1: gate_up [E, 2I, H/2] and down [E, H, I/2] bytes of two E2M1
 *      codes (element 2j in the low nibble, K contiguous); gate_up_scale
 *      [E, 2I, H/16] and down_scale [E, H, I/16] E4M3 block scales;
 *      gate_up_gscale, down_gscale f32 [E]. W = e2m1(q) * e4m3(s_blk) * s_glob.
 * qmode selects how quantised weights are computed with:
 *  MOE_QMODE_W (0): dequantised exactly to bf16, activations stay bf16, bf16
 *      MFMA (the weight-only W4A16 / W8A16 semantics; vLLM recipe
 *      "reflection/Beam-1.0-501B-A23B", Guide > Variants);
 *  MOE_QMODE_F8 (1): fp8 MFMA: x quantised per token to E4M3 with an fp32
 *      scale (amax / 448), NVFP4 weights re-encoded to E4M3 in registers per
 *      32-deep K block (RNE of e2m1 * s_blk * 2^-s, s = the exponent field of
 *      the block's larger E4M3 scale - 12, 2^s applied as the MFMA's block
 *      scale), h quantised per row and 128-column block to E4M3 with a
 *      power-of-two scale; needs I <= 4096.
 * qmode must be 0 for MOE_F32 / MOE_BF16 weights. */
typedef enum moe_qmode { MOE_QMODE_W = 0, MOE_QMODE_F8 = 1 } moe_qmode;

typedef struct moe_expert_weights {
  int32_t dtype; /* moe_dtype */
  int32_t qmode; /* moe_qmode */
  const void* gate_up;
  const void* down;
  const void* gate_up_scale;
  const void* down_scale;
  const float* gate_up_gscale;
  const float* down_gscale;
} moe_expert_weights;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(int32_t status);

/* ------------------------------------------------------------ router
 * Router GEMM and top-k (steps 1 and 2 of the layer).
 * logit[t, e] = bias[e] + sum_h x[t, h] * w_router[h, e], accumulated in fp32
 * and emitted as logits_dtype (bf16: round to nearest even; fp32 allowed only
 * with fp32 x). Selection works on the emitted logits: p = softmax over all E,
 * ids = the k largest (ties to the lowest id), ordered by (logit desc, id asc),
 * topk_w[t, j] = p[ids[t, j]] / sum_j' p[ids[t, j']].
 *   x          [T, H]  x_dtype (MOE_BF16 or MOE_F32)
 *   w_router   [H, E]  f32
 *   bias       [E]     f32, or NULL for none
 *   logits     [T, E]  logits_dtype, or NULL (then workspace holds them)
 *   logits_f32 [T, E]  f32 pre-rounding logits, or NULL
 *   topk_ids   [T, k]  int32;  topk_w [T, k] f32
 *   workspace          device scratch of moe_route_workspace_size() bytes */
size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E);
moe_status moe_route(const void* x, int32_t x_dtype, int64_t T, int32_t H, const float* w_router,
                     const float* bias, int32_t E, int32_t k, int32_t logits_dtype, void* logits,
                     float* logits_f32, int32_t* topk_ids, float* topk_w, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ permute
 * Token permute by expert (step 3): a stable counting sort of the pairs
 * p = t*k + j by expert id topk_ids[p]. counts[e] = number of pairs routed to
 * e; offsets = exclusive prefix sum of counts (E + 1 entries, offsets[E] =
 * T*k); sorted_pair[r] = the r-th pair in (expert, p) order; pair_pos is its
 * inverse (pair_pos[sorted_pair[r]] = r). Results are deterministic.
 * Ids outside [0, E) are not counted (the router never produces them): such
 * a pair gets pair_pos = -1, offsets[E] is then the number of valid pairs,
 * and sorted_pair[r] = -1 for r >= offsets[E]; moe_experts computes no row
 * for it and the finalize calls add nothing for it. Up to 16384 pairs no
 * workspace is needed (NULL allowed); above, moe_permute_workspace_size()
 * bytes of scratch hold per-segment histograms. */
size_t moe_permute_workspace_size(int64_t T, int32_t k, int32_t E);
moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ experts
 * Grouped SwiGLU expert GEMMs (step 4). For each expert e and each sorted row
 * r in [offsets[e], offsets[e+1]), with token t = sorted_pair[r] / k:
 *   a = x[t] . gate_up[e]  (length 2I, fp32 accumulate)
 *   h = silu(a[0:I]) * a[I:2I]   (rounded to bf16 for bf16 x; fp32 for fp32 x)
 *   y_sorted[r] = h . down[e]    (length H, fp32)
 * offsets and sorted_pair are moe_permute's outputs. On return the workspace
 * begins with h in sorted row order ([T*k, I], bf16, or fp32 for fp32
 * weights), valid until the workspace is reused; in the fp8-MFMA mode this is
 * the bf16 h that the E4M3 quantisation of the down GEMM's operand starts from. */
size_t moe_experts_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  const moe_expert_weights* w);
moe_status moe_experts(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I, int32_t E,
                       int32_t k, const int32_t* offsets, const int32_t* sorted_pair,
                       const moe_expert_weights* w, float* y_sorted, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ compact expert rows
 * Steps 4 and 5 with the expert rows kept compact: the same y_sorted rows,
 * stored as fp16 values with one power-of-two scale per row and 64-column
 * block, y_sorted[r, c] = y16[r, c] * 2^(y16_scale[r, c / 64] - 127). The
 * scale puts each block's largest magnitude into [2^14, 2^15) before the fp16
 * rounding (nearest even; it may round up to 2^15), so no finite row overflows;
 * each value keeps 11 significant bits relative to its block maximum, finer
 * than the error bf16 h already puts in the rows. This halves the traffic of the largest intermediate at prefill
 * sizes, where writing fp32 rows bounds the down GEMM; moe_forward uses these
 * two calls whenever moe_experts_rows16 supports the call.
 * moe_experts_rows16: as moe_experts, writing y16 [T*k, H] (uint16 fp16 bits)
 * and y16_scale [T*k, H/64] (uint8) instead of y_sorted; supported wherever
 * the experts run on the tiled kernels: bf16 and FP8 weights when the experts
 * average at least 32 rows (T*k >= 32*E), NVFP4 weights when they average
 * more than 16 (T*k > 16*E), and the fp8-MFMA mode (MOE_QMODE_F8) at any
 * size; else MOE_ERR_UNSUPPORTED. Same workspace as
 * moe_experts.
 * moe_finalize_rows16: as moe_finalize, reading the compact rows; each value
 * is decoded exactly to fp32 and summed as moe_finalize sums. */
moe_status moe_experts_rows16(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, const int32_t* offsets,
                              const int32_t* sorted_pair, const moe_expert_weights* w,
                              uint16_t* y16, uint8_t* y16_scale, void* workspace,
                              size_t workspace_bytes, void* stream);
moe_status moe_finalize_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                               const int32_t* pair_pos, const float* topk_w, int64_t T, int32_t k,
                               int32_t H, int32_t out_dtype, void* out, float* out_f32,
                               void* stream);

/* ------------------------------------------------------------ finalize
 * MoE finalize (step 5), the weighted un-permute:
 *   out[t] = sum_{j=0..k-1} topk_w[t, j] * y_sorted[pair_pos[t*k + j]]
 * accumulated in fp32 in slot order j = 0..k-1, emitted as out_dtype (bf16:
 * round to nearest even). out_f32 [T, H] (nullable) receives the fp32 sums.
 * A slot whose pair_pos is negative (a pair moe_permute left without a row)
 * adds nothing; every other pair_pos must be a row of y_sorted. */
moe_status moe_finalize(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                        int64_t T, int32_t k, int32_t H, int32_t out_dtype, void* out,
                        float* out_f32, void* stream);

/* ------------------------------------------------------------ finalize + sandwich norms
 * MoE finalize fused with the norms around the routed MoE block (vLLM PR
 * #61978, Status table row #62366 fuses Beam's sandwich norms with MoE
 * finalize and the tensor-parallel all-reduce; one GPU has no all-reduce).
 * The pages define neither the norm nor its epsilon: RMSNorm with a bf16
 * weight vector on a bf16 residual stream is this library's convention. Per
 * token t, with m = the fp32 sum moe_finalize forms (slot order):
 *   post            = m * (1 / sqrt(mean_h(m^2) + eps)) * gamma_post
 *   residual_out[t] = RNE_bf16(residual[t] + post)
 *   normed[t]       = RNE_bf16(residual_out[t] * (1 / sqrt(mean_h(residual_out[t]^2) + eps))
 *                              * gamma_next)
 * all in fp32 (row sums in a fixed order: deterministic). residual,
 * residual_out, normed: [T, H] bf16; gamma_post, gamma_next: [H] bf16;
 * eps >= 0 and finite. residual_out may equal residual (in-place update),
 * else the two must not overlap; normed must not overlap either (overlapping
 * [T, H] ranges return MOE_ERR_INVALID_ARGUMENT). H a multiple of 64 and at
 * most 16384, else MOE_ERR_UNSUPPORTED; errors as for moe_finalize.
 * moe_finalize_norm_rows16: the same over compact rows (y16, y16_scale as
 * moe_experts_rows16 writes them; each value decoded exactly). */
moe_status moe_finalize_norm(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                             int64_t T, int32_t k, int32_t H, const void* residual,
                             const void* gamma_post, const void* gamma_next, float eps,
                             void* residual_out, void* normed, void* stream);
moe_status moe_finalize_norm_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                                    const int32_t* pair_pos, const float* topk_w, int64_t T,
                                    int32_t k, int32_t H, const void* residual,
                                    const void* gamma_post, const void* gamma_next, float eps,
                                    void* residual_out, void* normed, void* stream);

/* ------------------------------------------------------------ whole layer
 * The five steps in order on one stream: route, permute, experts, finalize
 * (with compact expert rows where moe_experts_rows16 supports the call).
 * out [T, H] out_dtype; out_f32, logits, topk_ids, topk_w are optional
 * (NULL: kept in the workspace). logits_dtype as for moe_route. */
size_t moe_forward_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  const moe_expert_weights* w);
moe_status moe_forward(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I, int32_t E,
                       int32_t k, const float* w_router, const float* bias,
                       const moe_expert_weights* w, int32_t out_dtype, void* out, float* out_f32,
                       int32_t logits_dtype, void* logits, int32_t* topk_ids, float* topk_w,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ whole layer + sandwich norms
 * The layer ending in the fused finalize + norms of moe_finalize_norm (vLLM PR
 * #61978, Status table row #62366 fuses MoE finalize with Beam's sandwich
 * norms): route, permute, experts, then, per token, residual_out =
 * RNE_bf16(residual + RMSNorm(m) * gamma_post) and normed = the next
 * sublayer's RMSNorm of residual_out, m being the fp32 finalize sum (never
 * rounded). The expert rows are those moe_forward uses (compact rows on the
 * tiled kernels), so the fused step reads the rows as the plain finalize
 * does. x [T, H] bf16 (bf16, FP8 or NVFP4 expert weights); residual,
 * residual_out, normed [T, H] bf16 and gamma_post, gamma_next [H] bf16 as for
 * moe_finalize_norm (H <= 16384); logits (bf16), topk_ids, topk_w optional;
 * workspace of moe_forward_workspace_size() bytes; errors as moe_forward and
 * moe_finalize_norm. */
moe_status moe_forward_norm(const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                            const float* w_router, const float* bias, const moe_expert_weights* w,
                            const void* residual, const void* gamma_post, const void* gamma_next,
                            float eps, void* residual_out, void* normed, void* logits,
                            int32_t* topk_ids, float* topk_w, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ whole layer, no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * layer as moe_forward (same kernels, bit-identical results), with the
 * workspace taken from a scratch area the library holds in device memory:
 * MOE_NOALLOC_SCRATCH_BYTES on every device the library runs on, held until
 * the process ends. The call allocates nothing (no hipMalloc, no library
 * routine that allocates) and needs no workspace argument; the device is the
 * one `stream` belongs to (the current device for the null stream). The
 * scratch area's address on a device is looked up on the first call on that
 * device.
 *  - Limit: calls whose moe_forward_workspace_size exceeds
 *    MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE_TOO_SMALL and enqueue
 *    nothing (64 MiB covers the Beam decode layer, H = 5120, E = 256, k = 8,
 *    up to T = 128 tokens for I <= 2560 in every weight format; use
 *    moe_forward with a workspace beyond that).
 *  - Every call on one device shares that device's scratch area, and each
 *    call overwrites what the last one left there: calls that overlap on one
 *    device (for example on two streams, or from two host threads without
 *    ordering) race and give undefined results. Calls ordered on one stream
 *    are safe.
 *  - Arguments and errors as moe_forward; MOE_ERR_LAUNCH also when the scratch
 *    area cannot be located on the device. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                               int32_t E, int32_t k, const float* w_router, const float* bias,
                               const moe_expert_weights* w, int32_t out_dtype, void* out,
                               float* out_f32, int32_t logits_dtype, void* logits,
                               int32_t* topk_ids, float* topk_w, void* stream);

/* ------------------------------------------------------------ measurement
 * Not a step of the layer: the HBM read ceiling its bandwidth-bound kernels
 * are quoted against. Reads `bytes` (a multiple of 16) of device memory at buf
 * (16-byte aligned) once, in the decode expert kernels' access pattern
 * (16-byte nontemporal loads, eight in flight per lane; up to 2048 workgroups
 * of 256 lanes, each over a contiguous range), and combines them so that the
 * loads cannot be dropped; sink is
 * one device word the kernel may write. Caller owns both buffers. Errors:
 * MOE_ERR_INVALID_ARGUMENT for null or misaligned pointers or a size not a
 * multiple of 16, MOE_ERR_LAUNCH if the launch fails. */
moe_status moe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
