// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"
#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- whole layer (abi.cpp)
// Every check moe_forward makes on its arguments except those on the workspace.
moe_status check_forward(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, const float* w_router, const float* bias,
                         const moe_expert_weights* w, int32_t out_dtype, const void* out,
                         const float* out_f32, int32_t logits_dtype, const void* logits,
                         const int32_t* topk_ids, const float* topk_w);
// The layer's last step fused with the sandwich norms (moe_forward_norm):
// bf16 residual stream, bf16 norm weights, epsilon.
struct NormArgs {
  const uint16_t* residual;
  const uint16_t* gamma_post;
  const uint16_t* gamma_next;
  float eps;
  uint16_t* residual_out;
  uint16_t* normed;
};
// Enqueues the layer (arguments already checked, T > 0, a 16-byte aligned
// workspace of at least moe_forward_workspace_size bytes). With `norm` the
// finalize is fused with the norms and writes residual_out and normed instead
// of out / out_f32.
moe_status enqueue_forward(const void* x, int32_t x_dtype, int64_t T, int32_t H, int32_t I,
                           int32_t E, int32_t k, const float* w_router, const float* bias,
                           const moe_expert_weights* w, int32_t out_dtype, void* out,
                           float* out_f32, int32_t logits_dtype, void* logits, int32_t* topk_ids,
                           float* topk_w, void* workspace, size_t workspace_bytes, void* stream,
                           const NormArgs* norm = nullptr);

// ---------------------------------------------------------------- launchers
// Router GEMM partial sums: part[s][t][e] = sum over K-slice s of x[t,h] w[h,e].
// Tokens per router GEMM workgroup at batch T (16 or 64).
int router_gemm_rows(int T);
hipError_t launch_router_gemm(const void* x, bool x_bf16, int T, int H, const float* w_router,
                              int E, int n_split, int split_len, float* part, hipStream_t st);
// Streaming read of `bytes` (a multiple of 16) from buf; sink: one device word.
hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
// Outputs of the permute (layouts as launch_permute's).
struct PermuteOut {
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_pair = nullptr;
  int32_t* pair_pos = nullptr;
};
// Sum of partials + bias -> logits (bf16 or fp32), softmax, top-k, renormalised weights.
// With `perm` and T == 1 the select also writes the permute of the token's k
// pairs (its experts are distinct, so that is a sort of k ids); otherwise
// `perm` must be null.
hipError_t launch_router_select(const float* part, int n_split, int ldp, int T, int E, int k,
                                const float* bias, bool logits_bf16, void* logits,
                                float* logits_f32, int32_t* ids, float* w, hipStream_t st,
                                const PermuteOut* perm = nullptr);
// Stable counting sort of pairs by expert (one workgroup up to
// kPermuteOneBlockMax pairs, else three kernels with permute_ws_bytes of scratch).
constexpr long long kPermuteOneBlockMax = 16384;
size_t permute_ws_bytes(long long P, int E);
hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* ws, hipStream_t st);

enum WFormat { W_BF16 = 1, W_FP8 = 2, W_FP4 = 3 };

struct StreamGemmArgs {
  const uint16_t* a;       // gate/up: x [T, K] bf16; down: h [P, K] bf16
  const int32_t* offsets;  // [E + 1]
  const int32_t* sorted_pair;
  int k;                   // experts per token (gather divisor)
  int E, K, N, I;          // N = output columns of the matrix (2I or H)
  int rows = 0;            // P = T*k pairs (rows of h and y); 0: unknown
  const void* w;           // expert weights of this matrix
  const void* w_scale;     // FP8: f32 [E, N]; FP4: e4m3 [E, N, K/16]
  const float* w_gscale;   // FP4: f32 [E]
  uint16_t* h_out;         // gate/up output [P, I] bf16
  float* y_out;            // down output [P, N] f32
  // Compact down output instead of y_out (tiled kernel, 8 wavefronts): fp16
  // rows [P, N] with one power-of-two scale byte (2^(b - 127)) per row and
  // 64-column block [P, N / 64]; the block maximum is scaled into [2^14, 2^15).
  uint16_t* y16 = nullptr;
  uint8_t* y16_scale = nullptr;
  // Split-K over blockIdx.y (tiled kernel, down mode only): split s reads the
  // K slice (s % nk_split) of length K from A (row stride lda) and from weight
  // plane (s / nk_split), and writes partial sums to y_out + s * y_split_stride.
  int lda = 0;             // 0: lda = K
  int nsplit = 1, nk_split = 1;
  long long w_plane_stride = 0, y_split_stride = 0;
  // Split-K of the streaming kernels (blockIdx.z): split s covers the K steps
  // [s * ksteps, (s + 1) * ksteps) and writes fp32 partial sums of all N
  // columns to part + s * part_stride ([P, N] row-major); a reduction kernel
  // then forms h (SwiGLU) or y from them in split order.
  int ksplit = 1, ksteps = 0;
  float* part = nullptr;
  long long part_stride = 0;
  // Leave the split partial sums in `part` for their consumer instead of
  // launching the reduction: gate/up's for the down kernel (hpart below),
  // down's for the layer's finalize.
  bool keep_partials = false;
  // Down GEMM of bf16 weights with at most 32 rows per expert: form the h rows
  // a workgroup needs in LDS from the gate/up split partial sums
  // (hpart + s * hpart_stride, [P, 2I], s < hsplit) instead of reading h;
  // hlds_stride = bytes per LDS row. Bit-identical to the reduction kernel.
  const float* hpart = nullptr;
  int hsplit = 0;
  long long hpart_stride = 0;
  int hlds_stride = 0;
};
// fp8-MFMA mode operands: E4M3 codes of x (gate/up) with one fp32 scale per
// token, or of h (down) with one E8M0 scale per row and 128-column block.
struct F8Args {
  const uint8_t* a8;       // [T, H] (gate/up, gathered by token) or [P, I] (down)
  const float* x_scale;    // gate/up: [T]
  const uint8_t* h_bscale; // down: [P, h_bstride] E8M0 codes
  int h_bstride;
};
struct F8Buffers {         // device scratch of the fp8-MFMA mode
  uint8_t* xq;             // [T, H]
  float* xs;               // [T]
  uint8_t* hq;             // [P, I]
  uint8_t* hs;             // [P, hs_stride]
  int hs_stride;           // >= ceil(I / 128), a multiple of 4
};

// Grouped expert GEMM for small row counts per expert: each wavefront owns a
// 128-column slice of one expert's matrix and streams it once per 32 rows (16
// for NVFP4); with few touched experts K is split (StreamGemmArgs::ksplit) and
// a reduction kernel follows. The grid has one row per expert that can have
// rows (min(E, rows)).
// Whether the FP8 / NVFP4 streaming kernels can address A (P rows of H or I
// bf16 values) and one expert's weights with 31-bit byte offsets.
bool stream_buffers_fit(long long P, int H, int I);
// The FP8 / NVFP4 streaming kernels (expert_stream_q.hip): columns per
// wavefront, K values per step, and one launch on the given grid.
int stream_q_cols(int wfmt);
int stream_q_k_step(int wfmt);
hipError_t launch_stream_q(int wfmt, bool gate_up, dim3 grid, const StreamGemmArgs& a, hipStream_t st);
hipError_t launch_expert_stream(int wfmt, bool gate_up, const StreamGemmArgs& a, hipStream_t st);
// Split-K of the streaming kernels for few touched experts: number of splits
// of a K-deep product with N output columns over P rows (at most min(E, P)
// touched experts), the K steps (of `step` K values) per split, and the fp32
// scratch the partial sums need (the larger of the two products of an expert
// FFN).
struct StreamSplit {
  int ksplit, ksteps;
};
constexpr int kMaxStreamSplit = 16;
StreamSplit stream_split_plan(long long P, int E, int K, int N, bool gate_up, int wfmt);
int stream_k_step(int wfmt);  // K values per split unit of the streaming kernels
// Whether the down kernel forms h from the gate/up partial sums itself (bf16
// weights, P <= 32, gate/up split); *kr = the K values of h one down split
// reads (the LDS rows it needs are 32 x (2 kr + 16) bytes).
bool stream_fold_h(long long P, int E, int H, int I, int wfmt, int* kr);
// Bytes of the gate/up split partial sums, rounded up to 256 (where the down
// GEMM's own partial sums start when h is folded).
size_t stream_gu_part_bytes(long long P, int E, int H, int I, int wfmt);
size_t stream_ws_bytes(long long P, int E, int H, int I, int wfmt);

// Grouped expert GEMMs for many rows per expert: bf16 weights on 256 x 256
// tiles (plus 128 x 512 tiles for each expert's last <= 128 rows), quantised
// weights on 128 x 512 tiles, MFMAs fed through a four-stage LDS pipeline.
// Runs gate/up then down; ws holds the tile tables and work lists
// (expert_tile_ws_bytes).
size_t expert_tile_ws_bytes(int P, int E, int H, int I);
// whether the tiled path's work lists stay within int indexing
bool expert_tile_fits(long long P, int E, int H, int I);
// fp8-MFMA mode of the quantised experts (x and h quantised in-kernel; the
// gate/up output h in gate_up.h_out is bf16 scratch of the same size as usual).
hipError_t launch_expert_f8(int wfmt, const StreamGemmArgs& gate_up, const StreamGemmArgs& down,
                            int T, int P, const F8Buffers& bufs, void* tile_ws, hipStream_t st);
// The FP8 / NVFP4 tiled kernels (expert_tile_q.hip), arguments as for
// launch_expert_tile.
hipError_t launch_expert_tile_q(int wfmt, const StreamGemmArgs& gu, const StreamGemmArgs& dn, int P,
                                void* ws, hipStream_t st);
hipError_t launch_expert_tile(int wfmt, const StreamGemmArgs& gate_up, const StreamGemmArgs& down,
                              int P, void* ws, hipStream_t st);
// Router logits as three bf16 GEMMs on the tiled kernel: the fp32 router
// weights split into bf16 planes hi + mid + lo (24 significant bits), x being
// exactly bf16, so every product is exact and accumulation is fp32. Writes
// 3 * n_khalf partial sums [split][T][256] for the select kernel to add.
size_t router_bf16x3_ws_bytes(int T, int H);
int router_bf16x3_splits();
hipError_t launch_router_bf16x3(const uint16_t* x, int T, int H, const float* w_router, int E,
                                float* part, void* ws, hipStream_t st);
// Rows per expert from which the tiled kernel replaces the streaming one.
constexpr int kTileMinRowsPerExpert = 32;
// NVFP4 weights: the streaming kernel reads an expert's weights once per 8
// rows, while the tiled kernel's time hardly depends on the rows (its
// dequantisation is per weight column). Measured at H = 5120, I = 1536,
// E = 256, k = 8: streaming 1.03 / 1.36 / 1.69 / 2.23 ms at 8 / 12 / 16 / 24
// rows per expert, tiled 1.77 ms at each. Tiled above 16 rows per expert.
constexpr int kStreamMaxRowsPerExpertFp4 = 16;

// fp32 expert path (reference-precision layer; fp32 MFMA 16x16x4, fp32 accumulation).
hipError_t launch_expert_f32(const float* x, int T, int H, int I, int E, int k, int P,
                             const int32_t* offsets, const int32_t* sorted_pair,
                             const float* gate_up, const float* down, float* h, float* y,
                             hipStream_t st);

// Weighted un-permute.
hipError_t launch_finalize(const float* y_sorted, const int32_t* pair_pos, const float* w, int T,
                           int k, int H, bool out_bf16, void* out, float* out_f32,
                           hipStream_t st);
// The same from the S fp32 partial sums of a split-K down GEMM
// (part + s * sstride, [P, H] each): every expert row is their sum in split
// order, so the result equals reducing first and then finalizing, bit for bit.
hipError_t launch_finalize_split(const float* part, int S, long long sstride,
                                 const int32_t* pair_pos, const float* w, int T, int k, int H,
                                 bool out_bf16, void* out, float* out_f32, hipStream_t st);
// Weighted un-permute of compact rows (fp16 + per-64-column power-of-two
// scales), otherwise as launch_finalize.
hipError_t launch_finalize_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                                  const int32_t* pair_pos, const float* w, int T, int k, int H,
                                  bool out_bf16, void* out, float* out_f32, hipStream_t st);
// Weighted un-permute + RMS post-norm + residual add + next RMS pre-norm
// (bf16 residual and norm weights); H <= 16384.
hipError_t launch_finalize_norm(const float* y_sorted, const int32_t* pair_pos, const float* w,
                                int T, int k, int H, const uint16_t* residual,
                                const uint16_t* gamma_post, const uint16_t* gamma_next, float eps,
                                uint16_t* residual_out, uint16_t* normed, hipStream_t st);
// The same over compact rows (fp16 + per-64-column power-of-two scales).
hipError_t launch_finalize_norm_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                                       const int32_t* pair_pos, const float* w, int T, int k,
                                       int H, const uint16_t* residual, const uint16_t* gamma_post,
                                       const uint16_t* gamma_next, float eps,
                                       uint16_t* residual_out, uint16_t* normed, hipStream_t st);

}  // namespace moe
