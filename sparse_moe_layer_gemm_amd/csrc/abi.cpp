// C ABI of the routed MoE layer (include/moe.h): argument validation on the
// host, workspace carving and kernel dispatch on the caller's stream. Nothing
// is enqueued unless every check passes; nothing here synchronises the host.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxPairs = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxTokens = int64_t(1) << 24;  // one select workgroup per token
constexpr int32_t kMaxNormH = 16384;               // fused finalize + norms: row in registers

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_or_null(const void* p) { return p == nullptr || aligned16(p); }

struct Carver {
  char* base;
  size_t cap;
  size_t off = 0;
  void* take(size_t bytes) {
    void* p = base + off;
    off += align_up(bytes);
    return p;
  }
};

moe_status launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// Whether the byte ranges [a, a + n) and [b, b + n) intersect.
bool overlaps(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

// Arguments of the norms fused with finalize (T > 0): bf16 residual, outputs
// and norm weights, 16-byte aligned; normed must not overlap the residual or
// residual_out, and residual_out is either residual itself or disjoint from it.
moe_status check_norm_args(int64_t T, int32_t H, const void* residual, const void* gamma_post,
                           const void* gamma_next, float eps, const void* residual_out,
                           const void* normed) {
  if (!(eps >= 0.f) || eps > 3.4e38f) return MOE_ERR_INVALID_ARGUMENT;  // NaN or inf
  if (!residual || !gamma_post || !gamma_next || !residual_out || !normed)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(residual) || !aligned16(gamma_post) || !aligned16(gamma_next) ||
      !aligned16(residual_out) || !aligned16(normed))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t row_bytes = (size_t)T * H * sizeof(uint16_t);
  if (overlaps(normed, residual, row_bytes) || overlaps(normed, residual_out, row_bytes))
    return MOE_ERR_INVALID_ARGUMENT;
  if (residual_out != residual && overlaps(residual_out, residual, row_bytes))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// -------------------------------------------------------------- shared checks
// Sizes common to every call. T == 0 is valid (no-op).
moe_status check_shape(int64_t T, int32_t H, int32_t E, int32_t k) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (k > 8 || E > 256 || H % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * k > kMaxPairs || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Router split plan: enough K slices that the fp32 router GEMM spreads over
// at least 256 workgroups (16 or 64 tokens x 64 experts each); slices are
// multiples of 32 and there are at most 40 of them (at H = 5120: 128-deep
// slices, one 32-deep step per wavefront).
void router_plan(int64_t T, int32_t H, int32_t E, int* n_split, int* split_len) {
  const int rows = T < (1 << 30) ? moe::router_gemm_rows((int)T) : 64;
  const int64_t blocks = ((T + rows - 1) / rows) * ((E + 63) / 64);
  int64_t s = (256 + blocks - 1) / blocks;
  if (s < 1) s = 1;
  if (s > 40) s = 40;
  const int chunks = H / 32;
  if (s > chunks) s = chunks;
  const int per = (int)((chunks + s - 1) / s);
  *split_len = per * 32;
  *n_split = (chunks + per - 1) / per;
}

// Large bf16 batches run the router as three bf16 GEMMs on the tiled MFMA
// kernel (exact split of the fp32 weights); small ones on the fp32-MFMA kernel.
bool router_use_bf16x3(int32_t x_dtype, int64_t T) {
  return x_dtype == MOE_BF16 && T >= 1024;
}

size_t route_ws_bytes(int64_t T, int32_t H, int32_t E) {
  int S, L;
  router_plan(T, H, E, &S, &L);
  size_t fp32_path = align_up((size_t)S * T * E * sizeof(float));
  size_t bf16x3_path = 0;
  if (T >= 1024)
    bf16x3_path = align_up((size_t)moe::router_bf16x3_splits() * T * 256 * sizeof(float)) +
                  align_up(moe::router_bf16x3_ws_bytes((int)T, H));
  return (fp32_path > bf16x3_path ? fp32_path : bf16x3_path) +
         align_up((size_t)T * E * sizeof(float));
}

moe_status check_weights(const moe_expert_weights* w, int32_t x_dtype, int32_t H, int32_t I) {
  if (!w) return MOE_ERR_INVALID_ARGUMENT;
  if (w->qmode != MOE_QMODE_W && w->qmode != MOE_QMODE_F8) return MOE_ERR_INVALID_ARGUMENT;
  if (w->qmode == MOE_QMODE_F8) {
    if (w->dtype != MOE_FP8_E4M3 && w->dtype != MOE_FP4_E2M1) return MOE_ERR_UNSUPPORTED;
    if (I > 4096) return MOE_ERR_UNSUPPORTED;
  }
  if (!w->gate_up || !w->down) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(w->gate_up) || !aligned16(w->down)) return MOE_ERR_INVALID_ARGUMENT;
  if (I <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (I % 64 != 0 || H % 64 != 0) return MOE_ERR_UNSUPPORTED;
  switch (w->dtype) {
    case MOE_F32:
      if (x_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
      return MOE_OK;
    case MOE_BF16:
      if (x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
      return MOE_OK;
    case MOE_FP8_E4M3:
      if (x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
      if (!w->gate_up_scale || !w->down_scale) return MOE_ERR_INVALID_ARGUMENT;
      if (!aligned16(w->gate_up_scale) || !aligned16(w->down_scale)) return MOE_ERR_INVALID_ARGUMENT;
      return MOE_OK;
    case MOE_FP4_E2M1:
      if (x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
      if (!w->gate_up_scale || !w->down_scale || !w->gate_up_gscale || !w->down_gscale)
        return MOE_ERR_INVALID_ARGUMENT;
      if (!aligned16(w->gate_up_scale) || !aligned16(w->down_scale) ||
          !aligned16(w->gate_up_gscale) || !aligned16(w->down_gscale))
        return MOE_ERR_INVALID_ARGUMENT;
      return MOE_OK;
    default:
      return MOE_ERR_INVALID_ARGUMENT;
  }
}

bool f8_mode(const moe_expert_weights* w) { return w->qmode == MOE_QMODE_F8; }
int wfmt_of(int32_t dtype) {
  return dtype == MOE_BF16 ? moe::W_BF16 : dtype == MOE_FP8_E4M3 ? moe::W_FP8 : moe::W_FP4;
}
// E8M0 block scales per row of h: one per 128 columns, rows padded to 4 bytes
int h_bstride(int32_t I) { return ((I + 127) / 128 + 3) / 4 * 4; }

// h (bf16, or fp32 for the all-fp32 layer) + tile tables (+ fp8-MFMA mode:
// E4M3 x, per-token scales, E4M3 h, block scales; + bf16 weights: split-K
// partial sums of the streaming kernels)
size_t experts_ws_bytes(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                        const moe_expert_weights* w) {
  const size_t P = (size_t)T * k;
  const size_t h_elem = w->dtype == MOE_F32 ? sizeof(float) : sizeof(uint16_t);
  size_t b = align_up(P * I * h_elem) + align_up(moe::expert_tile_ws_bytes((int)P, E, H, I));
  if (f8_mode(w))
    b += align_up((size_t)T * H) + align_up((size_t)T * sizeof(float)) + align_up(P * I) +
         align_up(P * (size_t)h_bstride(I));
  else if (w->dtype != MOE_F32)
    b += align_up(moe::stream_ws_bytes((long long)P, E, H, I, wfmt_of(w->dtype)));  // split-K partials
  return b;
}

// The tiled grouped GEMMs pay off once experts average enough rows to fill
// their 128-row tiles; below that, streaming each weight once per pass of 32
// rows (bf16, FP8) or 8 rows (NVFP4) wins.
bool use_tile_kernel(int32_t w_dtype, int64_t P, int32_t E) {
  if (w_dtype == MOE_F32) return false;
  if (w_dtype == MOE_FP4_E2M1) return P > (int64_t)moe::kStreamMaxRowsPerExpertFp4 * E;
  return P >= (int64_t)moe::kTileMinRowsPerExpert * E;
}

// Sizes whose tiled work lists would overflow int indexing are unsupported.
moe_status check_tile_plan(const moe_expert_weights* w, int64_t T, int32_t k, int32_t E, int32_t H,
                           int32_t I) {
  const int64_t P = T * k;
  const bool tiled = use_tile_kernel(w->dtype, P, E) || w->qmode == MOE_QMODE_F8;
  if (tiled && !moe::expert_tile_fits(P, E, H, I)) return MOE_ERR_UNSUPPORTED;
  const bool quant = w->dtype == MOE_FP8_E4M3 || w->dtype == MOE_FP4_E2M1;
  if (!tiled && quant && P > 0 && !moe::stream_buffers_fit(P, H, I)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Compact expert rows (fp16 + power-of-two scale per 64 columns) are written
// by the tiled kernels: bf16, FP8 and NVFP4 weights with many rows per expert,
// and the fp8-MFMA mode (always tiled).
bool rows16_supported(const moe_expert_weights* w, int64_t P, int32_t E) {
  return w->dtype != MOE_F32 && (w->qmode == MOE_QMODE_F8 || use_tile_kernel(w->dtype, P, E));
}

// -------------------------------------------------------------- enqueue helpers
// (arguments already validated, T > 0)
moe_status enqueue_route(const void* x, int32_t x_dtype, int64_t T, int32_t H, const float* wr,
                         const float* bias, int32_t E, int32_t k, int32_t logits_dtype,
                         void* logits, float* logits_f32, int32_t* ids, float* w, void* ws,
                         hipStream_t st, const moe::PermuteOut* perm = nullptr) {
  int S, L;
  router_plan(T, H, E, &S, &L);
  const bool x3 = router_use_bf16x3(x_dtype, T);
  const size_t part_bytes = x3 ? (size_t)moe::router_bf16x3_splits() * T * 256 * sizeof(float)
                               : (size_t)S * T * E * sizeof(float);
  Carver c{static_cast<char*>(ws), 0};
  float* part = static_cast<float*>(c.take(part_bytes));
  void* x3ws = x3 ? c.take(moe::router_bf16x3_ws_bytes((int)T, H)) : nullptr;
  // the fp32 logits scratch sits at the end of the route workspace
  void* lbuf = static_cast<char*>(ws) + route_ws_bytes(T, H, E) -
               align_up((size_t)T * E * sizeof(float));
  if (!logits) logits = lbuf;
  hipError_t e;
  int nsplit, ldp;
  if (x3) {
    e = moe::launch_router_bf16x3(static_cast<const uint16_t*>(x), (int)T, H, wr, E, part, x3ws, st);
    nsplit = moe::router_bf16x3_splits();
    ldp = 256;
  } else {
    e = moe::launch_router_gemm(x, x_dtype == MOE_BF16, (int)T, H, wr, E, S, L, part, st);
    nsplit = S;
    ldp = E;
  }
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  e = moe::launch_router_select(part, nsplit, ldp, (int)T, E, k, bias, logits_dtype == MOE_BF16,
                                logits, logits_f32, ids, w, st, perm);
  return launch_status(e);
}

// Split partial sums of the down GEMM left for the finalize (S = 0: none).
struct KeptPartials {
  const float* part = nullptr;
  int S = 0;
  long long stride = 0;
};

// With `keep` set, a split-K down GEMM of the streaming kernels leaves its
// partial sums in the workspace (described in *keep) instead of reducing them
// into y_sorted; the caller then finalizes from them.
moe_status enqueue_experts(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                           int32_t E, int32_t k, const int32_t* offsets,
                           const int32_t* sorted_pair, const moe_expert_weights* w,
                           float* y_sorted, void* ws, hipStream_t st, uint16_t* y16 = nullptr,
                           uint8_t* y16_scale = nullptr, KeptPartials* keep = nullptr) {
  const int P = (int)(T * k);
  if (w->dtype == MOE_F32) {
    return launch_status(moe::launch_expert_f32(
        static_cast<const float*>(x), (int)T, H, I, E, k, P, offsets, sorted_pair,
        static_cast<const float*>(w->gate_up), static_cast<const float*>(w->down),
        static_cast<float*>(ws), y_sorted, st));
  }
  (void)x_dtype;
  const int wf = wfmt_of(w->dtype);
  uint16_t* h = static_cast<uint16_t*>(ws);
  void* tile_ws = static_cast<char*>(ws) + align_up((size_t)P * I * sizeof(uint16_t));
  moe::StreamGemmArgs a{};
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.k = k;
  a.E = E;
  a.I = I;
  a.rows = P;
  // gate/up: [T, H] x [H, 2I] -> h [P, I]
  a.a = static_cast<const uint16_t*>(x);
  a.K = H;
  a.N = 2 * I;
  a.w = w->gate_up;
  a.w_scale = w->gate_up_scale;
  a.w_gscale = w->gate_up_gscale;
  a.h_out = h;
  a.y_out = nullptr;
  // down: [P, I] x [I, H] -> y_sorted [P, H]
  moe::StreamGemmArgs d = a;
  d.a = h;
  d.K = I;
  d.N = H;
  d.w = w->down;
  d.w_scale = w->down_scale;
  d.w_gscale = w->down_gscale;
  d.h_out = nullptr;
  d.y_out = y_sorted;
  d.y16 = y16;  // compact rows (tiled paths; the caller checked)
  d.y16_scale = y16_scale;
  if (f8_mode(w)) {
    // the fp8-MFMA mode always runs the tiled kernels
    char* f8ws = static_cast<char*>(tile_ws) + align_up(moe::expert_tile_ws_bytes(P, E, H, I));
    moe::F8Buffers b{};
    b.xq = reinterpret_cast<uint8_t*>(f8ws);
    f8ws += align_up((size_t)T * H);
    b.xs = reinterpret_cast<float*>(f8ws);
    f8ws += align_up((size_t)T * sizeof(float));
    b.hq = reinterpret_cast<uint8_t*>(f8ws);
    f8ws += align_up((size_t)P * I);
    b.hs = reinterpret_cast<uint8_t*>(f8ws);
    b.hs_stride = h_bstride(I);
    return launch_status(moe::launch_expert_f8(wf, a, d, (int)T, P, b, tile_ws, st));
  }
  if (use_tile_kernel(w->dtype, P, E))
    return launch_status(moe::launch_expert_tile(wf, a, d, P, tile_ws, st));
  {
    // few touched experts: split K so that enough wavefronts stream weights
    float* part = reinterpret_cast<float*>(static_cast<char*>(tile_ws) +
                                           align_up(moe::expert_tile_ws_bytes(P, E, H, I)));
    const moe::StreamSplit sg = moe::stream_split_plan(P, E, H, 2 * I, true, wf);
    const moe::StreamSplit sd = moe::stream_split_plan(P, E, I, H, false, wf);
    a.ksplit = sg.ksplit;
    a.ksteps = sg.ksteps;
    a.part = part;
    a.part_stride = (long long)P * 2 * I;
    d.ksplit = sd.ksplit;
    d.ksteps = sd.ksteps;
    d.part = part;
    d.part_stride = (long long)P * H;
    int kr;
    if (moe::stream_fold_h(P, E, H, I, wf, &kr)) {
      // the down kernel forms h from the gate/up partial sums; its own partial
      // sums go after them
      a.keep_partials = true;
      d.h_out = h;  // the down kernel stores the h it forms
      d.hpart = part;
      d.hsplit = sg.ksplit;
      d.hpart_stride = a.part_stride;
      d.hlds_stride = 2 * kr + 16;
      d.part = part + moe::stream_gu_part_bytes(P, E, H, I, wf) / sizeof(float);
    }
    if (keep && d.ksplit > 1) {
      d.keep_partials = true;
      *keep = KeptPartials{d.part, d.ksplit, d.part_stride};
    }
  }
  hipError_t e = moe::launch_expert_stream(wf, true, a, st);
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  return launch_status(moe::launch_expert_stream(wf, false, d, st));
}

}  // namespace

namespace moe {

// Every check moe_forward makes except those on its workspace argument.
moe_status check_forward(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, const float* w_router, const float* bias,
                         const moe_expert_weights* w, int32_t out_dtype, const void* out,
                         const float* out_f32, int32_t logits_dtype, const void* logits,
                         const int32_t* topk_ids, const float* topk_w) {
  moe_status s = check_shape(T, H, E, k);
  if (s != MOE_OK) return s;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (logits_dtype != MOE_F32 && logits_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (logits_dtype == MOE_F32 && x_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  s = check_weights(w, x_dtype, H, I);
  if (s != MOE_OK) return s;
  s = check_tile_plan(w, T, k, E, H, I);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !ok_or_null(bias) || !aligned16(out) ||
      !ok_or_null(out_f32) || !ok_or_null(logits) || !ok_or_null(topk_ids) || !ok_or_null(topk_w))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// The layer's kernels on one stream (arguments checked by check_forward, T > 0,
// workspace of at least moe_forward_workspace_size bytes, 16-byte aligned).
moe_status enqueue_forward(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                           int32_t E, int32_t k, const float* w_router, const float* bias,
                           const moe_expert_weights* w, int32_t out_dtype, void* out,
                           float* out_f32, int32_t logits_dtype, void* logits, int32_t* topk_ids,
                           float* topk_w, void* workspace, size_t workspace_bytes, void* stream,
                           const NormArgs* norm) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t P = (size_t)T * k;
  Carver c{static_cast<char*>(workspace), workspace_bytes};
  void* route_ws = c.take(route_ws_bytes(T, H, E));
  void* lbuf = c.take((size_t)T * E * sizeof(float));
  int32_t* ids = static_cast<int32_t*>(c.take(P * sizeof(int32_t)));
  float* tw = static_cast<float*>(c.take(P * sizeof(float)));
  int32_t* counts = static_cast<int32_t*>(c.take(E * sizeof(int32_t)));
  int32_t* offsets = static_cast<int32_t*>(c.take((E + 1) * sizeof(int32_t)));
  int32_t* sorted_pair = static_cast<int32_t*>(c.take(P * sizeof(int32_t)));
  int32_t* pair_pos = static_cast<int32_t*>(c.take(P * sizeof(int32_t)));
  float* y_sorted = static_cast<float*>(c.take(P * H * sizeof(float)));
  void* exp_ws = c.take(experts_ws_bytes(T, H, I, E, k, w));
  void* perm_ws = c.take(moe::permute_ws_bytes((long long)P, E));
  if (topk_ids) ids = topk_ids;
  if (topk_w) tw = topk_w;
  if (!logits) logits = lbuf;

  // one token: the select kernel also writes the permute (a sort of k distinct ids)
  const moe::PermuteOut perm{counts, offsets, sorted_pair, pair_pos};
  moe_status s = enqueue_route(x, x_dtype, T, H, w_router, bias, E, k, logits_dtype, logits,
                               nullptr, ids, tw, route_ws, st, T == 1 ? &perm : nullptr);
  if (s != MOE_OK) return s;
  if (T != 1) {
    s = launch_status(
        moe::launch_permute(ids, (int)P, E, counts, offsets, sorted_pair, pair_pos, perm_ws, st));
    if (s != MOE_OK) return s;
  }
  if (rows16_supported(w, (int64_t)P, E)) {
    // compact rows in the fp32 rows' space: P*H*2 + P*H/64 bytes
    uint16_t* y16 = reinterpret_cast<uint16_t*>(y_sorted);
    uint8_t* y16_scale = reinterpret_cast<uint8_t*>(y16 + align_up(P * H * sizeof(uint16_t)) / 2);
    s = enqueue_experts(x, x_dtype, T, H, I, E, k, offsets, sorted_pair, w, nullptr, exp_ws, st,
                        y16, y16_scale);
    if (s != MOE_OK) return s;
    if (norm)
      return launch_status(moe::launch_finalize_norm_rows16(
          y16, y16_scale, pair_pos, tw, (int)T, k, H, norm->residual, norm->gamma_post,
          norm->gamma_next, norm->eps, norm->residual_out, norm->normed, st));
    return launch_status(moe::launch_finalize_rows16(y16, y16_scale, pair_pos, tw, (int)T, k, H,
                                                     out_dtype == MOE_BF16, out, out_f32, st));
  }
  KeptPartials kept;
  s = enqueue_experts(x, x_dtype, T, H, I, E, k, offsets, sorted_pair, w, y_sorted, exp_ws, st,
                      nullptr, nullptr, norm ? nullptr : &kept);
  if (s != MOE_OK) return s;
  if (norm)  // fp32 rows (a split-K down GEMM reduces them first)
    return launch_status(moe::launch_finalize_norm(y_sorted, pair_pos, tw, (int)T, k, H,
                                                   norm->residual, norm->gamma_post,
                                                   norm->gamma_next, norm->eps,
                                                   norm->residual_out, norm->normed, st));
  if (kept.S > 1)  // small batches: the down GEMM's split reduction folded into the finalize
    return launch_status(moe::launch_finalize_split(kept.part, kept.S, kept.stride, pair_pos, tw,
                                                    (int)T, k, H, out_dtype == MOE_BF16, out,
                                                    out_f32, st));
  return launch_status(moe::launch_finalize(y_sorted, pair_pos, tw, (int)T, k, H,
                                            out_dtype == MOE_BF16, out, out_f32, st));
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
    default: return "MOE_ERR_UNKNOWN";
  }
}

// ---------------------------------------------------------------- route
size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0 || H % 64 != 0) return 0;
  return route_ws_bytes(T, H, E);
}

moe_status moe_route(const void* x, int32_t x_dtype, int64_t T, int32_t H, const float* w_router,
                     const float* bias, int32_t E, int32_t k, int32_t logits_dtype, void* logits,
                     float* logits_f32, int32_t* topk_ids, float* topk_w, void* workspace,
                     size_t workspace_bytes, void* stream) {
  moe_status s = check_shape(T, H, E, k);
  if (s != MOE_OK) return s;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (logits_dtype != MOE_F32 && logits_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (logits_dtype == MOE_F32 && x_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w || !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !ok_or_null(bias) || !ok_or_null(logits) ||
      !ok_or_null(logits_f32) || !aligned16(topk_ids) || !aligned16(topk_w) ||
      !aligned16(workspace))
    return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < route_ws_bytes(T, H, E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return enqueue_route(x, x_dtype, T, H, w_router, bias, E, k, logits_dtype, logits, logits_f32,
                       topk_ids, topk_w, workspace, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- permute
size_t moe_permute_workspace_size(int64_t T, int32_t k, int32_t E) {
  if (T <= 0 || k <= 0 || E <= 0 || E > 256) return 0;
  return moe::permute_ws_bytes(T * k, E);
}

moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (k > 8 || E > 256) return MOE_ERR_UNSUPPORTED;
  if (T * k > kMaxPairs || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !sorted_pair || !pair_pos) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(topk_ids) || !aligned16(counts) || !aligned16(offsets) ||
      !aligned16(sorted_pair) || !aligned16(pair_pos))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe::permute_ws_bytes(T * k, E);
  if (need > 0) {
    if (!workspace || !aligned16(workspace)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  return launch_status(moe::launch_permute(topk_ids, (int)(T * k), E, counts, offsets, sorted_pair,
                                           pair_pos, workspace, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- experts
size_t moe_experts_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  const moe_expert_weights* w) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || !w) return 0;
  return experts_ws_bytes(T, H, I, E, k, w);
}

moe_status moe_experts(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I, int32_t E,
                       int32_t k, const int32_t* offsets, const int32_t* sorted_pair,
                       const moe_expert_weights* w, float* y_sorted, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moe_status s = check_shape(T, H, E, k);
  if (s != MOE_OK) return s;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  s = check_weights(w, x_dtype, H, I);
  if (s != MOE_OK) return s;
  s = check_tile_plan(w, T, k, E, H, I);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !sorted_pair || !y_sorted || !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(offsets) || !aligned16(sorted_pair) || !aligned16(y_sorted) ||
      !aligned16(workspace))
    return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < experts_ws_bytes(T, H, I, E, k, w)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return enqueue_experts(x, x_dtype, T, H, I, E, k, offsets, sorted_pair, w, y_sorted, workspace,
                         static_cast<hipStream_t>(stream));
}

moe_status moe_experts_rows16(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, const int32_t* offsets,
                              const int32_t* sorted_pair, const moe_expert_weights* w,
                              uint16_t* y16, uint8_t* y16_scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  moe_status s = check_shape(T, H, E, k);
  if (s != MOE_OK) return s;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  s = check_weights(w, x_dtype, H, I);
  if (s != MOE_OK) return s;
  s = check_tile_plan(w, T, k, E, H, I);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!rows16_supported(w, T * k, E)) return MOE_ERR_UNSUPPORTED;
  if (!x || !offsets || !sorted_pair || !y16 || !y16_scale || !workspace)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(offsets) || !aligned16(sorted_pair) || !aligned16(y16) ||
      !aligned16(y16_scale) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < experts_ws_bytes(T, H, I, E, k, w)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return enqueue_experts(x, x_dtype, T, H, I, E, k, offsets, sorted_pair, w, nullptr, workspace,
                         static_cast<hipStream_t>(stream), y16, y16_scale);
}

moe_status moe_finalize_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                               const int32_t* pair_pos, const float* topk_w, int64_t T, int32_t k,
                               int32_t H, int32_t out_dtype, void* out, float* out_f32,
                               void* stream) {
  if (T < 0 || k <= 0 || H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (k > 8 || H % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * k > kMaxPairs || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y16 || !y16_scale || !pair_pos || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y16) || !aligned16(y16_scale) || !aligned16(pair_pos) || !aligned16(topk_w) ||
      !aligned16(out) || !ok_or_null(out_f32))
    return MOE_ERR_INVALID_ARGUMENT;
  return launch_status(moe::launch_finalize_rows16(y16, y16_scale, pair_pos, topk_w, (int)T, k, H,
                                                   out_dtype == MOE_BF16, out, out_f32,
                                                   static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- finalize
moe_status moe_finalize(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                        int64_t T, int32_t k, int32_t H, int32_t out_dtype, void* out,
                        float* out_f32, void* stream) {
  if (T < 0 || k <= 0 || H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (k > 8 || H % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * k > kMaxPairs || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_sorted || !pair_pos || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_sorted) || !aligned16(pair_pos) || !aligned16(topk_w) || !aligned16(out) ||
      !ok_or_null(out_f32))
    return MOE_ERR_INVALID_ARGUMENT;
  return launch_status(moe::launch_finalize(y_sorted, pair_pos, topk_w, (int)T, k, H,
                                            out_dtype == MOE_BF16, out, out_f32,
                                            static_cast<hipStream_t>(stream)));
}

moe_status moe_finalize_norm(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                             int64_t T, int32_t k, int32_t H, const void* residual,
                             const void* gamma_post, const void* gamma_next, float eps,
                             void* residual_out, void* normed, void* stream) {
  if (T < 0 || k <= 0 || H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || eps > 3.4e38f) return MOE_ERR_INVALID_ARGUMENT;  // NaN or inf
  if (k > 8 || H % 64 != 0 || H > kMaxNormH) return MOE_ERR_UNSUPPORTED;
  if (T * k > kMaxPairs || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_sorted || !pair_pos || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_sorted) || !aligned16(pair_pos) || !aligned16(topk_w))
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status s = check_norm_args(T, H, residual, gamma_post, gamma_next, eps, residual_out, normed);
  if (s != MOE_OK) return s;
  return launch_status(moe::launch_finalize_norm(
      y_sorted, pair_pos, topk_w, (int)T, k, H, static_cast<const uint16_t*>(residual),
      static_cast<const uint16_t*>(gamma_post), static_cast<const uint16_t*>(gamma_next), eps,
      static_cast<uint16_t*>(residual_out), static_cast<uint16_t*>(normed),
      static_cast<hipStream_t>(stream)));
}

moe_status moe_finalize_norm_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                                    const int32_t* pair_pos, const float* topk_w, int64_t T,
                                    int32_t k, int32_t H, const void* residual,
                                    const void* gamma_post, const void* gamma_next, float eps,
                                    void* residual_out, void* normed, void* stream) {
  if (T < 0 || k <= 0 || H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || eps > 3.4e38f) return MOE_ERR_INVALID_ARGUMENT;  // NaN or inf
  if (k > 8 || H % 64 != 0 || H > kMaxNormH) return MOE_ERR_UNSUPPORTED;
  if (T * k > kMaxPairs || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y16 || !y16_scale || !pair_pos || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y16) || !aligned16(y16_scale) || !aligned16(pair_pos) || !aligned16(topk_w))
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status s = check_norm_args(T, H, residual, gamma_post, gamma_next, eps, residual_out, normed);
  if (s != MOE_OK) return s;
  return launch_status(moe::launch_finalize_norm_rows16(
      y16, y16_scale, pair_pos, topk_w, (int)T, k, H, static_cast<const uint16_t*>(residual),
      static_cast<const uint16_t*>(gamma_post), static_cast<const uint16_t*>(gamma_next), eps,
      static_cast<uint16_t*>(residual_out), static_cast<uint16_t*>(normed),
      static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- forward
size_t moe_forward_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  const moe_expert_weights* w) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || !w || H % 64 != 0) return 0;
  const size_t P = (size_t)T * k;
  return route_ws_bytes(T, H, E) + align_up((size_t)T * E * sizeof(float)) +
         2 * align_up(P * sizeof(int32_t)) /* ids, w */ + align_up(E * sizeof(int32_t)) +
         align_up((E + 1) * sizeof(int32_t)) + 2 * align_up(P * sizeof(int32_t)) +
         align_up(P * H * sizeof(float)) + experts_ws_bytes(T, H, I, E, k, w) +
         align_up(moe::permute_ws_bytes((long long)P, E));
}

moe_status moe_forward(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I, int32_t E,
                       int32_t k, const float* w_router, const float* bias,
                       const moe_expert_weights* w, int32_t out_dtype, void* out, float* out_f32,
                       int32_t logits_dtype, void* logits, int32_t* topk_ids, float* topk_w,
                       void* workspace, size_t workspace_bytes, void* stream) {
  moe_status s = moe::check_forward(x, x_dtype, T, H, I, E, k, w_router, bias, w, out_dtype, out,
                                    out_f32, logits_dtype, logits, topk_ids, topk_w);
  if (s != MOE_OK || T == 0) return s;
  if (!workspace || !aligned16(workspace)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe_forward_workspace_size(T, H, I, E, k, w))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return moe::enqueue_forward(x, x_dtype, T, H, I, E, k, w_router, bias, w, out_dtype, out, out_f32,
                              logits_dtype, logits, topk_ids, topk_w, workspace, workspace_bytes,
                              stream);
}

moe_status moe_forward_norm(const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                            const float* w_router, const float* bias, const moe_expert_weights* w,
                            const void* residual, const void* gamma_post, const void* gamma_next,
                            float eps, void* residual_out, void* normed, void* logits,
                            int32_t* topk_ids, float* topk_w, void* workspace,
                            size_t workspace_bytes, void* stream) {
  // the layer's output is consumed by the norms: residual_out stands in for
  // `out` in the common checks (bf16, required)
  moe_status s = moe::check_forward(x, MOE_BF16, T, H, I, E, k, w_router, bias, w, MOE_BF16,
                                    residual_out, nullptr, MOE_BF16, logits, topk_ids, topk_w);
  if (s != MOE_OK) return s;
  if (H > kMaxNormH) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  s = check_norm_args(T, H, residual, gamma_post, gamma_next, eps, residual_out, normed);
  if (s != MOE_OK) return s;
  if (!workspace || !aligned16(workspace)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe_forward_workspace_size(T, H, I, E, k, w))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe::NormArgs norm{static_cast<const uint16_t*>(residual),
                           static_cast<const uint16_t*>(gamma_post),
                           static_cast<const uint16_t*>(gamma_next), eps,
                           static_cast<uint16_t*>(residual_out), static_cast<uint16_t*>(normed)};
  return moe::enqueue_forward(x, MOE_BF16, T, H, I, E, k, w_router, bias, w, MOE_BF16, nullptr,
                              nullptr, MOE_BF16, logits, topk_ids, topk_w, workspace,
                              workspace_bytes, stream, &norm);
}

// ---------------------------------------------------------------- measurement
moe_status moe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || !aligned16(buf) || bytes % 16 != 0) return MOE_ERR_INVALID_ARGUMENT;
  return launch_status(moe::launch_hbm_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
