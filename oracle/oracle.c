/*
 * oracle.c -- plain CPU oracle of Beam's routed mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers; the GPU library never
 * links, loads or calls this code, and the two share no source.
 *
 * Everything is computed in double precision, without fast-math, in the
 * order the definition states. Inputs arrive in their storage formats
 * (fp32, bf16 bits, FP8 E4M3 codes, packed FP4 E2M1 codes with E4M3 block
 * scales) and are decoded exactly, element by element, from the format
 * definitions below.
 *
 * What the layer computes, and where it is stated:
 *  - router: a GEMM of shape (5120, 256) with BF16 output (vLLM PR #61978
 *    "Day-0 support for Reflection's Beam-1.0", Status table, row #62042),
 *    accumulated in FP32 (UpstreamBeat, "vLLM adds day-zero Reflection Beam
 *    serving...", section "Agents worked on the serving path": a specialized
 *    FP32 router kernel);
 *  - each token goes to 8 of 256 routed experts (vLLM recipe
 *    "reflection/Beam-1.0-501B-A23B", Guide > Overview);
 *  - routed expert outputs are combined by a "MoE finalize" step (PR #61978,
 *    Status table row #62366 and Remaining work);
 *  - the NVFP4 variant quantises the routed experts only and, on Hopper,
 *    runs them with BF16 activations (recipe, Guide > Variants).
 * The routing function (softmax over all E logits, top-k with ties to the
 * lowest expert id, renormalised weights), SwiGLU with gate columns [0, I)
 * and up columns [I, 2I) of the merged gate/up matrix, and the expert width
 * are conventions the pages leave open; they are the readings this oracle
 * fixes.
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * brute force, closed forms or library routines (see tests/test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_FP8 = 2, ODT_FP4 = 3 };
enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ENOMEM = 2 };

/* ------------------------------------------------------------------ formats */

/* bf16: the upper 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* FP8 E4M3 ("fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits; no
   infinities, S.1111.111 is NaN; exponent 0 is subnormal (m/8 * 2^-6). */
static double e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
   subnormal (m * 0.5). Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static double e2m1_value(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp((double)(2 + m), e - 2); /* (1 + m/2) 2^(e-1) */
  return s ? -v : v;
}

/* Round to the nearest bf16 value, ties to even, in one step from double. */
static double round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
  if (e - 1 < -126) /* below the smallest normal: fixed quantum 2^-133 */
    return ldexp(nearbyint(ldexp(v, 133)), -133);
  return ldexp(nearbyint(ldexp(m, 8)), e - 8); /* 8 significant bits */
}

/* Round to the nearest fp32 value, ties to even (C's conversion). */
static double round_f32(double v) { return (double)(float)v; }

/* Round onto the E4M3 grid, ties to even, saturating at +-448: quantum 2^-9
   below 2^-6 (subnormals), else 2^(floor(log2|v|) - 3) (3 mantissa bits). */
static double q_e4m3(double v) {
  double a = fabs(v), q;
  if (a >= 448.0) return v < 0 ? -448.0 : 448.0;
  if (a < 0.015625) {
    q = ldexp(nearbyint(ldexp(a, 9)), -9);
  } else {
    int e;
    frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1: floor(log2 a) = e - 1 */
    q = ldexp(nearbyint(ldexp(a, 4 - e)), e - 4);
  }
  return v < 0 ? -q : q;
}

/* Power-of-two block scale: the smallest e with 448 * 2^e >= amax, clamped to
   the E8M0 range [-127, 127]; 0 for an all-zero block. With amax = M * 2^E,
   1 <= M < 2: e = E - 8 when M <= 1.75 (448 = 1.75 * 2^8), else E - 7. */
static int block_exp(double amax) {
  if (amax == 0.0) return 0;
  int ex;
  double m = frexp(amax, &ex); /* amax = m * 2^ex, 0.5 <= m < 1 */
  int e = (2.0 * m <= 1.75) ? ex - 1 - 8 : ex - 1 - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

static double x_value(int x_dt, const void* x, int64_t i) {
  return x_dt == ODT_F32 ? (double)((const float*)x)[i] : bf16_value(((const uint16_t*)x)[i]);
}

/* Exported for the format pins. kind: 0 bf16 code, 1 e4m3 code, 2 e2m1 code,
   3 round-to-bf16, 4 round-to-fp32, 5 round-to-E4M3 (saturating), 6 block
   exponent of an amax. Codes are passed as doubles. */
int oracle_format(int kind, const double* in, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    switch (kind) {
      case 0: out[i] = bf16_value((uint16_t)in[i]); break;
      case 1: out[i] = e4m3_value((uint8_t)in[i]); break;
      case 2: out[i] = e2m1_value((uint8_t)in[i]); break;
      case 3: out[i] = round_bf16(in[i]); break;
      case 4: out[i] = round_f32(in[i]); break;
      case 5: out[i] = q_e4m3(in[i]); break;
      case 6: out[i] = (double)block_exp(in[i]); break;
      default: return ORACLE_EINVAL;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ router */

/* logits[i, e] = bias[e] + sum_h x[t, h] * W_r[h, e], h ascending, for the
   tokens t = rows[i] (all tokens when rows is NULL). x is bf16 or fp32, W_r is
   fp32 [H, E]; every product is exact in double (at most 8 + 24 significant
   bits), so the sum is the exact logit up to double rounding of the sum. */
int oracle_logits(int x_dt, const void* x, int64_t T, int32_t H, const float* w_router,
                  const float* bias, int32_t E, const int64_t* rows, int64_t n, double* out) {
  if (!x || !w_router || !out || H <= 0 || E <= 0 || T < 0) return ORACLE_EINVAL;
  if (x_dt != ODT_F32 && x_dt != ODT_BF16) return ORACLE_EINVAL;
  for (int64_t i = 0; i < n; ++i)
    if (rows && (rows[i] < 0 || rows[i] >= T)) return ORACLE_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = rows ? rows[i] : i;
    double* o = out + i * E;
    for (int e = 0; e < E; ++e) o[e] = bias ? (double)bias[e] : 0.0;
    for (int h = 0; h < H; ++h) {
      double xv = x_value(x_dt, x, t * H + h);
      const float* w = w_router + (int64_t)h * E;
      for (int e = 0; e < E; ++e) o[e] += xv * (double)w[e];
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ routing */

typedef struct {
  double v;
  int id;
} cand;

/* larger value first; equal values: lower expert id first */
static int cand_cmp(const void* a, const void* b) {
  const cand* x = (const cand*)a;
  const cand* y = (const cand*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->id > y->id) - (x->id < y->id);
}

/* Routing of n tokens from their logits.
   The selection value is the logit as the router emits it: rounded to bf16
   (sel_dt = BF16) or to fp32 (sel_dt = F32). p = softmax over all E selection
   values; the k chosen experts are the first k in the order (value desc,
   id asc), emitted in that order; w_j = p[S_j] / sum_j' p[S_j'].
   sel (optional, [n, E]) receives the selection values. */
int oracle_route(int sel_dt, const double* logits, int64_t n, int32_t E, int32_t k, int32_t* ids,
                 double* w, double* sel) {
  if (!logits || !ids || !w || E <= 0 || k <= 0 || k > E) return ORACLE_EINVAL;
  if (sel_dt != ODT_F32 && sel_dt != ODT_BF16) return ORACLE_EINVAL;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    cand* c = (cand*)malloc(sizeof(cand) * (size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    if (!c || !p) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t i = 0; i < n; ++i) {
        const double* l = logits + i * E;
        double mx = -INFINITY, z = 0.0, zs = 0.0;
        for (int e = 0; e < E; ++e) {
          double v = sel_dt == ODT_BF16 ? round_bf16(l[e]) : round_f32(l[e]);
          c[e].v = v;
          c[e].id = e;
          if (sel) sel[i * E + e] = v;
          if (v > mx) mx = v;
        }
        for (int e = 0; e < E; ++e) {
          p[e] = exp(c[e].v - mx);
          z += p[e];
        }
        for (int e = 0; e < E; ++e) p[e] /= z;
        qsort(c, (size_t)E, sizeof(cand), cand_cmp);
        for (int j = 0; j < k; ++j) zs += p[c[j].id];
        for (int j = 0; j < k; ++j) {
          ids[i * k + j] = c[j].id;
          w[i * k + j] = p[c[j].id] / zs;
        }
      }
    }
    free(c);
    free(p);
  }
  return err;
}

/* ------------------------------------------------------------------ permute */

/* Stable counting sort of the pair indices p = t*k + j by expert:
   counts[e] = #pairs routed to e; offsets = exclusive prefix sum (E+1 long);
   sorted_pair lists the pairs ordered by (expert, p); pair_pos is its inverse. */
int oracle_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                   int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos) {
  int64_t P = T * k;
  if (!counts || !offsets || E <= 0 || k <= 0 || T < 0) return ORACLE_EINVAL;
  for (int64_t p = 0; p < P; ++p)
    if (ids[p] < 0 || ids[p] >= E) return ORACLE_EINVAL;
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!cursor) return ORACLE_ENOMEM;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[ids[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t p = 0; p < P; ++p) {
    int32_t r = cursor[ids[p]]++;
    sorted_pair[r] = (int32_t)p;
    pair_pos[p] = r;
  }
  free(cursor);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ experts */

typedef struct {
  int dt;
  int32_t H, I;
  const void *gate_up, *down;
  const void *gate_up_scale, *down_scale;
  const float *gate_up_gscale, *down_gscale;
} weights;

/* Row h (K index) of expert e's gate/up matrix, all 2I columns, as doubles.
   f32/bf16 layout [E, H, 2I]; fp8 [E, 2I, H] codes with fp32 [E, 2I] channel
   scales; fp4 [E, 2I, H/2] packed codes (even k in the low nibble) with E4M3
   block scales [E, 2I, H/16] and an fp32 scale per expert. */
static void gate_up_row(const weights* W, int e, int h, double* row) {
  int64_t N = 2 * (int64_t)W->I, H = W->H;
  switch (W->dt) {
    case ODT_F32: {
      const float* s = (const float*)W->gate_up + ((int64_t)e * H + h) * N;
      for (int64_t n = 0; n < N; ++n) row[n] = s[n];
    } break;
    case ODT_BF16: {
      const uint16_t* s = (const uint16_t*)W->gate_up + ((int64_t)e * H + h) * N;
      for (int64_t n = 0; n < N; ++n) row[n] = bf16_value(s[n]);
    } break;
    case ODT_FP8: {
      const uint8_t* q = (const uint8_t*)W->gate_up;
      const float* sc = (const float*)W->gate_up_scale;
      for (int64_t n = 0; n < N; ++n)
        row[n] = e4m3_value(q[((int64_t)e * N + n) * H + h]) * (double)sc[(int64_t)e * N + n];
    } break;
    case ODT_FP4: {
      const uint8_t* q = (const uint8_t*)W->gate_up;
      const uint8_t* sb = (const uint8_t*)W->gate_up_scale;
      double g = W->gate_up_gscale[e];
      for (int64_t n = 0; n < N; ++n) {
        uint8_t byte = q[((int64_t)e * N + n) * (H / 2) + h / 2];
        uint8_t nib = (h & 1) ? (byte >> 4) : (byte & 15);
        row[n] = e2m1_value(nib) * e4m3_value(sb[((int64_t)e * N + n) * (H / 16) + h / 16]) * g;
      }
    } break;
  }
}

/* Row i (K index) of expert e's down matrix, all H columns.
   f32/bf16 [E, I, H]; fp8 [E, H, I] + [E, H]; fp4 [E, H, I/2] + [E, H, I/16] + [E]. */
static void down_row(const weights* W, int e, int i, double* row) {
  int64_t N = W->H, I = W->I;
  switch (W->dt) {
    case ODT_F32: {
      const float* s = (const float*)W->down + ((int64_t)e * I + i) * N;
      for (int64_t n = 0; n < N; ++n) row[n] = s[n];
    } break;
    case ODT_BF16: {
      const uint16_t* s = (const uint16_t*)W->down + ((int64_t)e * I + i) * N;
      for (int64_t n = 0; n < N; ++n) row[n] = bf16_value(s[n]);
    } break;
    case ODT_FP8: {
      const uint8_t* q = (const uint8_t*)W->down;
      const float* sc = (const float*)W->down_scale;
      for (int64_t n = 0; n < N; ++n)
        row[n] = e4m3_value(q[((int64_t)e * N + n) * I + i]) * (double)sc[(int64_t)e * N + n];
    } break;
    case ODT_FP4: {
      const uint8_t* q = (const uint8_t*)W->down;
      const uint8_t* sb = (const uint8_t*)W->down_scale;
      double g = W->down_gscale[e];
      for (int64_t n = 0; n < N; ++n) {
        uint8_t byte = q[((int64_t)e * N + n) * (I / 2) + i / 2];
        uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);
        row[n] = e2m1_value(nib) * e4m3_value(sb[((int64_t)e * N + n) * (I / 16) + i / 16]) * g;
      }
    } break;
  }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One routed expert applied to one token, as a SwiGLU FFN:
   a = x_t W_gu[e] (length 2I), h = silu(a[0:I]) * a[I:2I], y = h W_d[e]
   (length H). Sums run over ascending K; no intermediate rounding. The
   expert's weight rows come from gu [H][2I] and dn [I][H] when the caller
   decoded them, else as stored (gate_up_row / down_row into `row`). */
static void expert_ffn(int x_dt, const void* x, int64_t t, const weights* W, int e,
                       const double* gu, const double* dn, double* a, double* row, double* y,
                       double* h_out) {
  int64_t H = W->H, I = W->I;
  for (int64_t n = 0; n < 2 * I; ++n) a[n] = 0.0;
  for (int64_t h = 0; h < H; ++h) {
    double xv = x_value(x_dt, x, t * H + h);
    const double* r = gu ? gu + h * 2 * I : row;
    if (!gu) gate_up_row(W, e, (int)h, row);
    for (int64_t n = 0; n < 2 * I; ++n) a[n] += xv * r[n];
  }
  for (int64_t i = 0; i < I; ++i) a[i] = silu(a[i]) * a[I + i];
  if (h_out)
    for (int64_t i = 0; i < I; ++i) h_out[i] = a[i];
  for (int64_t n = 0; n < H; ++n) y[n] = 0.0;
  for (int64_t i = 0; i < I; ++i) {
    const double* r = dn ? dn + i * H : row;
    if (!dn) down_row(W, e, (int)i, row);
    for (int64_t n = 0; n < H; ++n) y[n] += a[i] * r[n];
  }
}

/* Row indices grouped by expert: order[start[e] .. start[e + 1]) are the rows
   of expert e, ascending. */
static int group_rows(int64_t n, const int32_t* experts, int32_t E, int64_t** order_out,
                      int64_t** start_out) {
  int64_t* start = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int64_t* cur = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  if (!start || !order || !cur) {
    free(start);
    free(order);
    free(cur);
    return ORACLE_ENOMEM;
  }
  for (int64_t r = 0; r < n; ++r) start[experts[r] + 1]++;
  for (int e = 0; e < E; ++e) start[e + 1] += start[e];
  for (int e = 0; e < E; ++e) cur[e] = start[e];
  for (int64_t r = 0; r < n; ++r) order[cur[experts[r]]++] = r;
  free(cur);
  *order_out = order;
  *start_out = start;
  return ORACLE_OK;
}

static int make_weights(weights* W, int w_dt, int32_t H, int32_t I, const void* gate_up,
                        const void* down, const void* gate_up_scale, const void* down_scale,
                        const float* gate_up_gscale, const float* down_gscale) {
  if (H <= 0 || I <= 0 || !gate_up || !down) return ORACLE_EINVAL;
  if (w_dt < ODT_F32 || w_dt > ODT_FP4) return ORACLE_EINVAL;
  if (w_dt == ODT_FP8 && (!gate_up_scale || !down_scale)) return ORACLE_EINVAL;
  if (w_dt == ODT_FP4 && (!gate_up_scale || !down_scale || !gate_up_gscale || !down_gscale ||
                          H % 16 || I % 16))
    return ORACLE_EINVAL;
  W->dt = w_dt;
  W->H = H;
  W->I = I;
  W->gate_up = gate_up;
  W->down = down;
  W->gate_up_scale = gate_up_scale;
  W->down_scale = down_scale;
  W->gate_up_gscale = gate_up_gscale;
  W->down_gscale = down_gscale;
  return ORACLE_OK;
}

static int expert_rows_grouped(int mode, int x_dt, const void* x, const weights* W, int32_t E,
                               const int32_t* tokens, const int32_t* experts, const double* h_in,
                               int64_t n, double* y, double* h_out, double* hq_out);

/* y[r] = FFN_{experts[r]}(x[tokens[r]]) for n (token, expert) rows;
   optionally also the SwiGLU activations h[r] (length I). */
int oracle_expert_rows(int x_dt, const void* x, int64_t T, int32_t H, int32_t I, int32_t E,
                       int w_dt, const void* gate_up, const void* down, const void* gate_up_scale,
                       const void* down_scale, const float* gate_up_gscale,
                       const float* down_gscale, const int32_t* tokens, const int32_t* experts,
                       int64_t n, double* y, double* h_out) {
  weights W;
  int rc = make_weights(&W, w_dt, H, I, gate_up, down, gate_up_scale, down_scale,
                        gate_up_gscale, down_gscale);
  if (rc) return rc;
  if (!x || !tokens || !experts || !y) return ORACLE_EINVAL;
  for (int64_t r = 0; r < n; ++r)
    if (tokens[r] < 0 || tokens[r] >= T || experts[r] < 0 || experts[r] >= E) return ORACLE_EINVAL;
  return expert_rows_grouped(0, x_dt, x, &W, E, tokens, experts, NULL, n, y, h_out, NULL);
}

/* ------------------------------------------------------------------ fp8-MFMA mode */
/* The quantised experts run on fp8 MFMA ("F8" mode): every operand of both
   expert GEMMs is an E4M3 value, encoded step by step as follows.
   - Activations x (bf16): one fp32 scale per token, s_t = amax_t / 448 (1 for
     an all-zero row), computed in fp32 as the kernel does; codes
     RNE_e4m3(x / s_t) with the division in fp32.
   - FP8 weights are used as stored (their per-channel scale multiplies the
     accumulated sum). NVFP4 weights become E4M3 codes per 32-deep K block
     (two 16-value NVFP4 blocks): with e the exponent field (0..15) of the
     larger of the two E4M3 block scales (0 for a zero or subnormal scale) and
     sigma = e - 12, the codes are RNE_e4m3(e2m1 * s_blk * 2^-sigma). Every
     scale of the block is below 2^(e - 6) (2^-6 if subnormal), so the products
     stay below 6 * 2^6 = 384 <= 448 and never saturate, and the larger scale's
     nonzero products are at least 16: they keep E4M3's full precision whatever
     the scales' range. 2^sigma is the block's scale in the product and s_glob
     multiplies the sum.
   - h = silu(g) * u, rounded to bf16 as in the bf16 path, then per row and
     128-column block a power-of-two scale 2^e (block_exp of the block's amax)
     and codes RNE_e4m3(h * 2^-e).
   - The down GEMM sums each block's code products times its 2^e. */

/* Value of weight (K index kk, column n) of a quantised matrix as the F8 mode
   uses it, without its per-channel / per-expert scale: the E4M3 code (fp8), or
   the re-encoded E4M3 code times its 32-block power of two (fp4); q: codes
   [E, N, K] (fp8) or packed [E, N, K/2] (fp4) with block scales [E, N, K/16]. */
static double w8_value(int dt, const void* q, const void* sb, int64_t N, int64_t K, int e,
                       int64_t n, int64_t kk) {
  if (dt == ODT_FP8) return e4m3_value(((const uint8_t*)q)[((int64_t)e * N + n) * K + kk]);
  uint8_t byte = ((const uint8_t*)q)[((int64_t)e * N + n) * (K / 2) + kk / 2];
  uint8_t nib = (kk & 1) ? (byte >> 4) : (byte & 15);
  const uint8_t* srow = (const uint8_t*)sb + ((int64_t)e * N + n) * (K / 16);
  double s = e4m3_value(srow[kk / 16]);
  int c0 = srow[(kk / 32) * 2] & 0x7F, c1 = srow[(kk / 32) * 2 + 1] & 0x7F;
  int sigma = ((c0 > c1 ? c0 : c1) >> 3) - 12; /* magnitude codes order like values */
  return ldexp(q_e4m3(ldexp(e2m1_value(nib) * s, -sigma)), sigma);
}
static double w8_scale(int dt, const void* sc, const float* gs, int64_t N, int e, int64_t n) {
  return dt == ODT_FP8 ? (double)((const float*)sc)[(int64_t)e * N + n] : (double)gs[e];
}

/* Per-token activation quantisation: xq[h] (E4M3 values) and the fp32 scale. */
static float quantize_x_row(const uint16_t* xr, int64_t H, double* xq) {
  float amax = 0.0f;
  for (int64_t h = 0; h < H; ++h) {
    float v = fabsf((float)bf16_value(xr[h]));
    if (v > amax) amax = v;
  }
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int64_t h = 0; h < H; ++h) xq[h] = q_e4m3((double)((float)bf16_value(xr[h]) / s));
  return s;
}

/* The down stage of F8 mode for one row: h (bf16 values, length I) quantised
   per 128-column block (hq = q * 2^e, length I), then y = hq W_d[e] times the
   column scales. dn8 [H][I]: expert e's down weights as w8_value gives them. */
static void down_f8(const weights* W, int e, const double* dn8, const double* h, double* hq,
                    double* y) {
  int64_t H = W->H, I = W->I;
  for (int64_t b0 = 0; b0 < I; b0 += 128) {
    int64_t b1 = b0 + 128 < I ? b0 + 128 : I;
    double amax = 0.0;
    for (int64_t i = b0; i < b1; ++i) amax = fabs(h[i]) > amax ? fabs(h[i]) : amax;
    int eb = block_exp(amax);
    for (int64_t i = b0; i < b1; ++i) hq[i] = ldexp(q_e4m3(ldexp(h[i], -eb)), eb);
  }
  for (int64_t n = 0; n < H; ++n) {
    const double* wr = dn8 + n * I;
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += hq[i] * wr[i];
    y[n] = acc * w8_scale(W->dt, W->down_scale, W->down_gscale, H, e, n);
  }
}

/* One expert on one token in F8 mode; gu8 [2I][H]: expert e's gate/up weights
   as w8_value gives them. h_out (bf16-rounded h) and hq_out (the dequantised
   codes q * 2^e) are optional. */
static void expert_ffn_f8(const void* x, int64_t t, const weights* W, int e, const double* gu8,
                          const double* dn8, double* a, double* xq, double* y, double* h_out,
                          double* hq_out) {
  int64_t H = W->H, I = W->I, N1 = 2 * I;
  float s_t = quantize_x_row((const uint16_t*)x + t * H, H, xq);
  for (int64_t n = 0; n < N1; ++n) {
    const double* wr = gu8 + n * H;
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h) acc += xq[h] * wr[h];
    a[n] = acc * (double)s_t * w8_scale(W->dt, W->gate_up_scale, W->gate_up_gscale, N1, e, n);
  }
  for (int64_t i = 0; i < I; ++i) a[i] = round_bf16(silu(a[i]) * a[I + i]);
  if (h_out)
    for (int64_t i = 0; i < I; ++i) h_out[i] = a[i];
  down_f8(W, e, dn8, a, a + I, y);
  if (hq_out)
    for (int64_t i = 0; i < I; ++i) hq_out[i] = a[I + i];
}

/* Expert e's weights decoded into dense doubles, once per expert and call.
   mode 0 (weights dequantised exactly, FP8 / NVFP4 only: bf16 and fp32 rows
   are read as stored): gu [H][2I] and dn [I][H], the values gate_up_row and
   down_row give. Modes 1 and 2 (F8): gu [2I][H] and dn [H][I],
   the values w8_value gives (mode 2 needs dn only). A work-shared loop of the
   enclosing parallel region (each ends with a barrier). */
static void decode_expert(int mode, const weights* W, int e, double* gu, double* dn) {
  int64_t H = W->H, I = W->I, N1 = 2 * I;
  if (mode == 0 && (W->dt == ODT_F32 || W->dt == ODT_BF16)) return; /* read as stored */
  if (mode == 0) {
#pragma omp for schedule(static)
    for (int64_t h = 0; h < H; ++h) gate_up_row(W, e, (int)h, gu + h * N1);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < I; ++i) down_row(W, e, (int)i, dn + i * H);
    return;
  }
  if (mode == 1) {
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N1; ++n)
      for (int64_t h = 0; h < H; ++h)
        gu[n * H + h] = w8_value(W->dt, W->gate_up, W->gate_up_scale, N1, H, e, n, h);
  }
#pragma omp for schedule(static)
  for (int64_t n = 0; n < H; ++n)
    for (int64_t i = 0; i < I; ++i) dn[n * I + i] = w8_value(W->dt, W->down, W->down_scale, H, I, e, n, i);
}

/* The expert rows of one call, grouped by expert so that each expert's
   weights are decoded once (decode_expert), then its rows computed one by one
   in parallel. mode 0: FFN with exactly dequantised weights (h_out: h);
   1: F8-mode FFN (h_out: bf16-rounded h, hq_out: dequantised h codes);
   2: F8-mode down stage on the given h rows h_in [n, I]. */
static int expert_rows_grouped(int mode, int x_dt, const void* x, const weights* W, int32_t E,
                               const int32_t* tokens, const int32_t* experts, const double* h_in,
                               int64_t n, double* y, double* h_out, double* hq_out) {
  int64_t H = W->H, I = W->I;
  int64_t *order = NULL, *start = NULL;
  int rc = group_rows(n, experts, E, &order, &start);
  if (rc) return rc;
  /* bf16 / fp32 weights are read as stored; quantised ones decoded per expert */
  const int decode = mode != 0 || (W->dt != ODT_F32 && W->dt != ODT_BF16);
  double* gu = (mode == 2 || !decode) ? NULL : (double*)malloc(sizeof(double) * (size_t)(H * 2 * I));
  double* dn = decode ? (double*)malloc(sizeof(double) * (size_t)(H * I)) : NULL;
  if ((mode != 2 && decode && !gu) || (decode && !dn)) {
    free(gu);
    free(dn);
    free(order);
    free(start);
    return ORACLE_ENOMEM;
  }
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * 2 * (size_t)I);
    double* xq = (double*)malloc(sizeof(double) * (size_t)(H > 2 * I ? H : 2 * I));
    const int bad = !a || !xq;
    if (bad) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    }
    if (!decode) {  /* weights read as stored: every row in parallel */
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < n; ++r)
        if (!bad)
          expert_ffn(x_dt, x, tokens[r], W, experts[r], NULL, NULL, a, xq, y + r * H,
                     h_out ? h_out + r * I : NULL);
    }
    for (int e = 0; decode && e < E; ++e) {
      if (start[e] == start[e + 1]) continue;  /* the same decision in every thread */
      decode_expert(mode, W, e, gu, dn);
#pragma omp for schedule(dynamic, 1)
      for (int64_t q = start[e]; q < start[e + 1]; ++q) {
        if (bad) continue;
        int64_t r = order[q];
        if (mode == 0)  /* xq serves as the row buffer */
          expert_ffn(x_dt, x, tokens[r], W, e, gu, dn, a, xq, y + r * H, h_out ? h_out + r * I : NULL);
        else if (mode == 1)
          expert_ffn_f8(x, tokens[r], W, e, gu, dn, a, xq, y + r * H,
                        h_out ? h_out + r * I : NULL, hq_out ? hq_out + r * I : NULL);
        else
          down_f8(W, e, dn, h_in + r * I, a, y + r * H);
      }
    }
    free(a);
    free(xq);
  }
  free(gu);
  free(dn);
  free(order);
  free(start);
  return err;
}

/* y[r] for n (token, expert) rows as oracle_expert_rows, in F8 mode (bf16 x,
   FP8 or NVFP4 weights); optional h (bf16-rounded) and dequantised h codes. */
int oracle_expert_rows_f8(const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int w_dt,
                          const void* gate_up, const void* down, const void* gate_up_scale,
                          const void* down_scale, const float* gate_up_gscale,
                          const float* down_gscale, const int32_t* tokens, const int32_t* experts,
                          int64_t n, double* y, double* h_out, double* hq_out) {
  weights W;
  if (w_dt != ODT_FP8 && w_dt != ODT_FP4) return ORACLE_EINVAL;
  int rc = make_weights(&W, w_dt, H, I, gate_up, down, gate_up_scale, down_scale,
                        gate_up_gscale, down_gscale);
  if (rc) return rc;
  if (!x || !tokens || !experts || !y) return ORACLE_EINVAL;
  for (int64_t r = 0; r < n; ++r)
    if (tokens[r] < 0 || tokens[r] >= T || experts[r] < 0 || experts[r] >= E) return ORACLE_EINVAL;
  return expert_rows_grouped(1, ODT_BF16, x, &W, E, tokens, experts, NULL, n, y, h_out, hq_out);
}

/* The F8 down stage alone on given h rows (bf16 values [n, I]) of the given
   experts: y [n, H]; lets a caller take the h quantisation decisions on its
   own h. */
int oracle_down_rows_f8(int32_t H, int32_t I, int32_t E, int w_dt, const void* gate_up,
                        const void* down, const void* gate_up_scale, const void* down_scale,
                        const float* gate_up_gscale, const float* down_gscale,
                        const int32_t* experts, int64_t n, const double* h, double* y) {
  weights W;
  if (w_dt != ODT_FP8 && w_dt != ODT_FP4) return ORACLE_EINVAL;
  int rc = make_weights(&W, w_dt, H, I, gate_up, down, gate_up_scale, down_scale,
                        gate_up_gscale, down_gscale);
  if (rc) return rc;
  if (!experts || !h || !y) return ORACLE_EINVAL;
  for (int64_t r = 0; r < n; ++r)
    if (experts[r] < 0 || experts[r] >= E) return ORACLE_EINVAL;
  return expert_rows_grouped(2, ODT_BF16, NULL, &W, E, NULL, experts, h, n, y, NULL, NULL);
}

/* Activation quantisation alone, for the GPU's quantised x: values and scales. */
int oracle_quantize_x(const uint16_t* x, int64_t T, int32_t H, double* xq, float* scale) {
  if (!x || !xq || !scale || H <= 0) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) scale[t] = quantize_x_row(x + t * H, H, xq + t * H);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ finalize */

/* out[i] = sum_{j=0..k-1} w[t, j] * y_sorted[pair_pos[t*k + j]] for t = rows[i]
   (all tokens when rows is NULL), summed in slot order. */
int oracle_finalize(const float* y_sorted, const int32_t* pair_pos, const float* w, int64_t T,
                    int32_t k, int32_t H, const int64_t* rows, int64_t n, double* out) {
  if (!y_sorted || !pair_pos || !w || !out || k <= 0 || H <= 0) return ORACLE_EINVAL;
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = rows ? rows[i] : i;
    if (t < 0 || t >= T) return ORACLE_EINVAL;
    for (int j = 0; j < k; ++j)
      if (pair_pos[t * k + j] < 0 || pair_pos[t * k + j] >= T * k) return ORACLE_EINVAL;
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = rows ? rows[i] : i;
    double* o = out + i * H;
    for (int h = 0; h < H; ++h) o[h] = 0.0;
    for (int j = 0; j < k; ++j) {
      const float* yr = y_sorted + (int64_t)pair_pos[t * k + j] * H;
      double wj = w[t * k + j];
      for (int h = 0; h < H; ++h) o[h] += wj * (double)yr[h];
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ layer */

/* The whole layer for the tokens rows[0..n) (all tokens when rows is NULL):
   logits -> routing -> for each chosen expert its SwiGLU FFN ->
   out[t] = sum_j w[t, j] * FFN_{S[t, j]}(x_t), in slot order.
   Optional outputs: ids [n, k], w [n, k], logits [n, E] (exact, pre-rounding). */
int oracle_expert_rows_f8(const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int w_dt,
                          const void* gate_up, const void* down, const void* gate_up_scale,
                          const void* down_scale, const float* gate_up_gscale,
                          const float* down_gscale, const int32_t* tokens, const int32_t* experts,
                          int64_t n, double* y, double* h_out, double* hq_out);

/* qmode 0: weights dequantised exactly, activations bf16; 1: F8 mode (above). */
int oracle_layer_q(int qmode, int x_dt, const void* x, int64_t T, int32_t H, int32_t I, int32_t E,
                   int32_t k, const float* w_router, const float* bias, int sel_dt, int w_dt,
                   const void* gate_up, const void* down, const void* gate_up_scale,
                   const void* down_scale, const float* gate_up_gscale, const float* down_gscale,
                   const int64_t* rows, int64_t n, double* out, int32_t* ids_out, double* w_out,
                   double* logits_out) {
  if (!out || k <= 0 || k > E) return ORACLE_EINVAL;
  int rc = ORACLE_OK;
  double* lg = logits_out ? logits_out : (double*)malloc(sizeof(double) * (size_t)(n * E + 1));
  int32_t* ids = ids_out ? ids_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(n * k + 1));
  double* w = w_out ? w_out : (double*)malloc(sizeof(double) * (size_t)(n * k + 1));
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n * k + 1));
  double* y = (double*)malloc(sizeof(double) * (size_t)(n * k * (int64_t)H + 1));
  if (!lg || !ids || !w || !tok || !y) {
    rc = ORACLE_ENOMEM;
    goto done;
  }
  rc = oracle_logits(x_dt, x, T, H, w_router, bias, E, rows, n, lg);
  if (rc) goto done;
  rc = oracle_route(sel_dt, lg, n, E, k, ids, w, NULL);
  if (rc) goto done;
  for (int64_t i = 0; i < n; ++i)
    for (int j = 0; j < k; ++j) tok[i * k + j] = (int32_t)(rows ? rows[i] : i);
  if (qmode == 1) {
    if (x_dt != ODT_BF16) {
      rc = ORACLE_EINVAL;
      goto done;
    }
    rc = oracle_expert_rows_f8(x, T, H, I, E, w_dt, gate_up, down, gate_up_scale, down_scale,
                               gate_up_gscale, down_gscale, tok, ids, n * k, y, NULL, NULL);
  } else {
    rc = oracle_expert_rows(x_dt, x, T, H, I, E, w_dt, gate_up, down, gate_up_scale, down_scale,
                            gate_up_gscale, down_gscale, tok, ids, n * k, y, NULL);
  }
  if (rc) goto done;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double* o = out + i * H;
    for (int h = 0; h < H; ++h) o[h] = 0.0;
    for (int j = 0; j < k; ++j) {
      const double* yr = y + (i * k + j) * (int64_t)H;
      for (int h = 0; h < H; ++h) o[h] += w[i * k + j] * yr[h];
    }
  }
done:
  if (!logits_out) free(lg);
  if (!ids_out) free(ids);
  if (!w_out) free(w);
  free(tok);
  free(y);
  return rc;
}

int oracle_layer(int x_dt, const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                 const float* w_router, const float* bias, int sel_dt, int w_dt,
                 const void* gate_up, const void* down, const void* gate_up_scale,
                 const void* down_scale, const float* gate_up_gscale, const float* down_gscale,
                 const int64_t* rows, int64_t n, double* out, int32_t* ids_out, double* w_out,
                 double* logits_out) {
  return oracle_layer_q(0, x_dt, x, T, H, I, E, k, w_router, bias, sel_dt, w_dt, gate_up, down,
                        gate_up_scale, down_scale, gate_up_gscale, down_gscale, rows, n, out,
                        ids_out, w_out, logits_out);
}
