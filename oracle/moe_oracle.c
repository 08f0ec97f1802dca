/*
 * moe_oracle.c -- CPU oracle for the routed MoE layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 statement of
 * what the layer computes.  It is used by the tests, by the GPU smoke check and
 * by the CPU-baseline leg of the benchmark, and by nothing else.  It shares no
 * code, header, table or constant with the HIP library: it does not include
 * any header of that library and that library does not include this file.
 *
 * Sources (page title, then section / equation):
 *   [MM]  CANN operator page "mega_moe": §计算公式 (inputs X, E, G, W1, W2 and
 *         output Y), §约定 (SiLU, round-to-nearest), §计算过程 -> EP Dispatch,
 *         Expert Compute (Linear1, SwiGLU, Linear2), Token Combine, and the
 *         A8W8 block (per-token activation scale, per-output-channel weight
 *         scales, requantisation of the SwiGLU output before Linear2).
 *   [V4]  "Megatron-LM 的 MoE 并行：以 DeepSeek-V4 为例": §模型与入口 (the
 *         layer equation y_t = F_s(x_t) + sum_{e in I_t} g_{t,e} F_e(x_t)),
 *         §路由张量 (gating linear [n,h]->[n,E]; a = sqrt(softplus(l));
 *         I_t = TopK(a + beta); g = alpha * a / sum_{I_t} a; the bias is used
 *         for selection only), §Hash 路由 (a token-id table replaces only the
 *         selection), §计数与重排 (per-expert counts; the first permute copies
 *         each token once per selected expert), §ETP 里的矩阵 (SwiGLU expert
 *         F(X) = (SiLU(X Wg) * X Wu) Wd).
 *   [MD]  "Megatron 分布式训练全维度并行技术文档": §4.1 (router W_gate in
 *         [H,E]) and §4.2 (G(x) = TopK(softmax(x W_gate)), the top-k
 *         probabilities used directly as mixing weights).
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes of the repository):
 *   - top-k order: key descending, ties to the lower expert id;
 *   - row order inside an expert block: ascending flat assignment index
 *     t*k + j (a stable counting sort), one fixed order as [MM] allows;
 *   - SwiGLU split: the first `inter` columns of Linear1 are the gate, the
 *     last `inter` are the up projection ([MM] Expert Compute);
 *   - fp8 (e4m3fn, OCP) replaces INT8 in the A8W8 block: the constant 127
 *     becomes 448, round-to-nearest-even with saturation; a zero row gets
 *     scale 1 and code 0;
 *   - the INT8 A8W8 block itself ([MM] A8W8: s = max|row| / 127, codes in
 *     [-127, 127]): its rounding ⌊z⌉ is read as round half away from zero
 *     (the §约定 wording, 四舍五入); a zero row gets scale 1 and code 0; the
 *     INT8 products are summed exactly as integers before the per-channel
 *     and per-row dequantisation;
 *   - the per-token activation quantisation of X is an integer decision
 *     taken from an input, so it is done in fp32 (the kernel's precision),
 *     everything else is fp64;
 *   - MX block quantisation ([MM] MXFP block: groups of 32 elements along the
 *     contraction dimension share one E8M0 scale, elements FP8 e4m3fn or
 *     FP4 e2m1): the pages name the group size, the element and scale types
 *     and that a shared exponent is extracted per group, but not the rule;
 *     the OCP MX v1.0 rule is taken: shared exponent = floor(log2(max|v|))
 *     - emax(element) (emax 8 for e4m3, 2 for e2m1), clamped to the E8M0
 *     range [-127, 127] (code = exponent + 127; an all-zero group gets code
 *     0), and each element is v / 2^exponent rounded to nearest even and
 *     saturated to the element's largest magnitude (448, 6).
 *
 * Element codes for tensors handed in: 0 = fp32, 1 = bf16 (raw 16-bit words),
 * 2 = fp8 e4m3fn (raw bytes), INT8 weights as int8_t.  MX tensors: e4m3 codes one per byte, e2m1
 * codes two per byte (element 2i in the low nibble), E8M0 scale codes one per
 * byte; MXFP4 weights are stored K-contiguous as on the mega_moe page
 * (codes [E,N,K/2], scales [E,N,K/32]).  All arrays are host memory, row
 * major.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2

#define ORC_SIGMOID 0
#define ORC_SOFTMAX 1
#define ORC_SQRT_SOFTPLUS 2

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32 word. */
/* Thread count of the OpenMP loops below (n < 1: the OpenMP default).  Only
 * the CPU timing in the benchmark sets it; it changes no arithmetic: every
 * parallel loop writes disjoint outputs in a fixed per-item order. */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_set_threads(int n) {
#ifdef _OPENMP
  static int dflt = 0;
  if (dflt == 0) dflt = omp_get_max_threads();
  omp_set_num_threads(n > 0 ? n : dflt);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent field 0 is subnormal. */
double oracle_e4m3_decode(uint8_t code) {
  int sign = (code >> 7) & 1;
  int ex = (code >> 3) & 0xF;
  int man = code & 0x7;
  double v;
  if (ex == 0xF && man == 0x7) return NAN;
  if (ex == 0)
    v = ldexp((double)man / 8.0, -6);
  else
    v = ldexp(1.0 + (double)man / 8.0, ex - 7);
  return sign ? -v : v;
}

/* Nearest e4m3fn value to v, ties to the code with an even mantissa, values
 * beyond the largest finite magnitude (448) saturate to it.  Found by a
 * binary search over the 127 non-negative finite codes, whose values increase
 * with the code. */
uint8_t oracle_e4m3_encode(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = (v < 0.0 || (v == 0.0 && signbit(v))) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int lo = 0, hi = 0x7E; /* value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_decode((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - oracle_e4m3_decode((uint8_t)lo);
  double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
  int pick;
  if (dlo < dhi)
    pick = lo;
  else if (dhi < dlo)
    pick = hi;
  else
    pick = (lo & 1) ? hi : lo; /* tie: even mantissa */
  return (uint8_t)(sign | pick);
}

/* OCP e2m1 (FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit; no
 * infinities or NaN.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_decode(uint8_t code) {
  int sign = (code >> 3) & 1;
  int ex = (code >> 1) & 3;
  int man = code & 1;
  double v = (ex == 0) ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -v : v;
}

/* Nearest e2m1 value, ties to the even mantissa, saturating at 6. */
uint8_t oracle_e2m1_encode(double v) {
  uint8_t sign = (v < 0.0 || (v == 0.0 && signbit(v))) ? 0x8 : 0x0;
  double a = fabs(v);
  if (isnan(v) || a >= 6.0) return (uint8_t)(sign | 0x7);
  int lo = 0, hi = 7; /* value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e2m1_decode((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - oracle_e2m1_decode((uint8_t)lo);
  double dhi = oracle_e2m1_decode((uint8_t)hi) - a;
  int pick = dlo < dhi ? lo : (dhi < dlo ? hi : ((lo & 1) ? hi : lo));
  return (uint8_t)(sign | pick);
}

#define ORC_FMT_E4M3 0
#define ORC_FMT_E2M1 1

/* E8M0 code of the shared scale of a group whose largest magnitude is amax
 * (see the MX reading in the header). */
uint8_t oracle_mx_scale_code(double amax, int fmt) {
  if (!(amax > 0.0)) return 0;
  int e2;
  frexp(amax, &e2); /* amax = m * 2^e2, m in [0.5, 1): floor(log2 amax) = e2 - 1 */
  int x = (e2 - 1) - (fmt == ORC_FMT_E4M3 ? 8 : 2);
  if (x < -127) x = -127;
  if (x > 127) x = 127;
  return (uint8_t)(x + 127);
}

static double element_decode(uint8_t code, int fmt) {
  return fmt == ORC_FMT_E4M3 ? oracle_e4m3_decode(code) : oracle_e2m1_decode(code);
}
static uint8_t element_encode(double v, int fmt) {
  return fmt == ORC_FMT_E4M3 ? oracle_e4m3_encode(v) : oracle_e2m1_encode(v);
}

/* MX quantisation of n values (n a multiple of 32): one element code per
 * value in q (unpacked, one per byte) and one E8M0 code per group in scale. */
void oracle_mx_quantize(int n, const double* x, int fmt, uint8_t* q, uint8_t* scale) {
  for (int g = 0; g < n / 32; ++g) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs(x[g * 32 + i]);
      amax = a > amax ? a : amax;
    }
    uint8_t sc = oracle_mx_scale_code(amax, fmt);
    scale[g] = sc;
    for (int i = 0; i < 32; ++i) q[g * 32 + i] = element_encode(ldexp(x[g * 32 + i], 127 - sc), fmt);
  }
}

/* Value of an MX element: decode(code) * 2^(scale - 127). */
double oracle_mx_value(uint8_t code, uint8_t scale, int fmt) {
  return ldexp(element_decode(code, fmt), (int)scale - 127);
}

/* Values of all 256 e4m3 codes, filled from oracle_e4m3_decode on first use
 * so that the inner loops below do a table read instead of the decode. */
static double e4m3_table[256];
static int e4m3_table_ready = 0;
static void e4m3_table_init(void) {
  if (e4m3_table_ready) return;
  for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_e4m3_decode((uint8_t)c);
  e4m3_table_ready = 1;
}

static double elem(const void* base, int dt, size_t i) {
  if (dt == ORC_F32) return (double)((const float*)base)[i];
  if (dt == ORC_BF16) return bf16_value(((const uint16_t*)base)[i]);
  return e4m3_table[((const uint8_t*)base)[i]];
}

/* ------------------------------------------------------------------ */
/* Routing  ([V4] §路由张量, §Hash 路由; [MD] §4.2)                     */
/* ------------------------------------------------------------------ */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double softplus(double z) { return z > 0 ? z + log1p(exp(-z)) : log1p(exp(z)); }

/* Gating linear: logits[t,e] = sum_c X[t,c] * Wg[c,e] (+ gate_bias[e]). */
void oracle_gate_logits(int T, int hidden, int E, int dt, const void* X, const void* Wg,
                        const double* gate_bias, double* logits) {
  e4m3_table_init();
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double* l = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e) l[e] = 0.0;
    for (int c = 0; c < hidden; ++c) {
      double xc = elem(X, dt, (size_t)t * hidden + c);
      for (int e = 0; e < E; ++e) l[e] += xc * elem(Wg, dt, (size_t)c * E + e);
    }
    for (int e = 0; e < E; ++e) l[e] += gate_bias ? gate_bias[e] : 0.0;
  }
}

/* Affinity a[t,e] from the logits: sigmoid, softmax over the experts, or
 * sqrt(softplus). */
void oracle_affinity(int T, int E, int score_fn, const double* logits, double* aff) {
  for (int t = 0; t < T; ++t) {
    const double* l = logits + (size_t)t * E;
    double* a = aff + (size_t)t * E;
    if (score_fn == ORC_SOFTMAX) {
      double m = l[0];
      for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
      double z = 0.0;
      for (int e = 0; e < E; ++e) z += exp(l[e] - m);
      for (int e = 0; e < E; ++e) a[e] = exp(l[e] - m) / z;
    } else if (score_fn == ORC_SQRT_SOFTPLUS) {
      for (int e = 0; e < E; ++e) a[e] = sqrt(softplus(l[e]));
    } else {
      for (int e = 0; e < E; ++e) a[e] = sigmoid(l[e]);
    }
  }
}

/* Top-k selection on keys[T,E]: the k largest keys, listed by key descending,
 * equal keys in ascending expert id.  margin[t] = k-th largest key minus the
 * (k+1)-th (INFINITY when k == E). */
void oracle_topk(int T, int E, int k, const double* keys, int32_t* ids, double* margin) {
  char* taken = (char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const double* key = keys + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j <= k && j < E; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || key[e] > key[best])) best = e;
      if (j < k) {
        ids[(size_t)t * k + j] = best;
        taken[best] = 1;
      } else if (margin) {
        margin[t] = key[ids[(size_t)t * k + k - 1]] - key[best];
      }
    }
    if (margin && k >= E) margin[t] = INFINITY;
  }
  free(taken);
}

/* Full router.  Score routing: keys = a + beta (beta only selects), ids =
 * TopK(keys).  Hash routing (token_ids and tid2eid both given): ids[t,:] =
 * tid2eid[token_ids[t], :], beta unused.  In both cases the mixing weight is
 * taken from the unbiased affinity: G = alpha * a / sum_{selected} a when
 * renorm, else alpha * a.  keys_out / margin_out may be NULL. */
void oracle_route(int T, int hidden, int E, int k, int dt, const void* X, const void* Wg,
                  const double* gate_bias, const double* beta, int score_fn, int renorm,
                  double alpha, const int32_t* token_ids, const int32_t* tid2eid,
                  int32_t* ids, double* G, double* logits_out, double* keys_out,
                  double* margin_out) {
  double* logits = (double*)malloc(sizeof(double) * (size_t)T * E);
  double* aff = (double*)malloc(sizeof(double) * (size_t)T * E);
  double* keys = (double*)malloc(sizeof(double) * (size_t)T * E);
  oracle_gate_logits(T, hidden, E, dt, X, Wg, gate_bias, logits);
  oracle_affinity(T, E, score_fn, logits, aff);
  int hash = (token_ids != NULL && tid2eid != NULL);
  for (size_t i = 0; i < (size_t)T * E; ++i)
    keys[i] = aff[i] + ((beta && !hash) ? beta[i % (size_t)E] : 0.0);
  if (hash) {
    for (int t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) ids[(size_t)t * k + j] = tid2eid[(size_t)token_ids[t] * k + j];
      if (margin_out) margin_out[t] = INFINITY;
    }
  } else {
    oracle_topk(T, E, k, keys, ids, margin_out);
  }
  for (int t = 0; t < T; ++t) {
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += aff[(size_t)t * E + ids[(size_t)t * k + j]];
    for (int j = 0; j < k; ++j) {
      double a = aff[(size_t)t * E + ids[(size_t)t * k + j]];
      G[(size_t)t * k + j] = renorm ? alpha * a / denom : alpha * a;
    }
  }
  if (logits_out) memcpy(logits_out, logits, sizeof(double) * (size_t)T * E);
  if (keys_out) memcpy(keys_out, keys, sizeof(double) * (size_t)T * E);
  free(logits);
  free(aff);
  free(keys);
}

/* ------------------------------------------------------------------ */
/* Dispatch  ([MM] EP Dispatch; [V4] §计数与重排)                        */
/* ------------------------------------------------------------------ */

/* counts[e] = number of assignments (t,j) with ids[t,j] == e; offsets is the
 * exclusive prefix sum (E+1 entries).  Each assignment gets the destination
 * row dst_row[t*k+j] = offsets[e] + (number of earlier assignments, in flat
 * order t*k+j, to the same expert); src_tok[row] = t.  Returns the number of
 * assignments whose expert id is outside [0,E) (those get dst_row = -1). */
int oracle_dispatch(int T, int k, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                    int32_t* dst_row, int32_t* src_tok) {
  int bad = 0;
  if (E <= 0 || T < 0 || k <= 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (size_t i = 0; i < (size_t)T * k; ++i) {
    int e = ids[i];
    if (e < 0 || e >= E)
      ++bad;
    else
      ++counts[e];
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (size_t i = 0; i < (size_t)T * k; ++i) {
    int e = ids[i];
    if (e < 0 || e >= E) {
      dst_row[i] = -1;
      continue;
    }
    int r = offsets[e] + fill[e]++;
    dst_row[i] = r;
    src_tok[r] = (int32_t)(i / (size_t)k);
  }
  free(fill);
  return bad;
}

/* ------------------------------------------------------------------ */
/* Expert FFN  ([MM] Expert Compute; [V4] §ETP 里的矩阵)                 */
/* ------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* out[0:hidden] = (SiLU(x W1[:, :f]) * (x W1[:, f:])) W2 for one row x,
 * W1 [hidden, 2f] and W2 [f, hidden] of element type wdt. */
static void swiglu_row(int hidden, int f, const double* x, int wdt, const void* W1,
                       const void* W2, double* h1, double* out) {
  for (int n = 0; n < 2 * f; ++n) h1[n] = 0.0;
  for (int c = 0; c < hidden; ++c) {
    double xc = x[c];
    if (xc == 0.0) continue;
    for (int n = 0; n < 2 * f; ++n) h1[n] += xc * elem(W1, wdt, (size_t)c * 2 * f + n);
  }
  for (int n = 0; n < f; ++n) h1[n] = silu(h1[n]) * h1[f + n];
  for (int o = 0; o < hidden; ++o) out[o] = 0.0;
  for (int n = 0; n < f; ++n) {
    double u = h1[n];
    for (int o = 0; o < hidden; ++o) out[o] += u * elem(W2, wdt, (size_t)n * hidden + o);
  }
}

/* Per-token activation quantisation of the A8W8 block, e4m3 form:
 * s = max|x| / 448, q = RNE_sat(x / s), computed in fp32 (see header). */
void oracle_quantize_row_f32(int n, const float* x, uint8_t* q, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    amax = a > amax ? a : amax;
  }
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int i = 0; i < n; ++i) q[i] = oracle_e4m3_encode((double)(x[i] / s));
  *scale = s;
}

/* ⌊z⌉ of [MM] §约定, read as round half away from zero. */
static double round_half_away(double v) { return round(v); /* C round: halves away from 0 */ }

/* Per-token activation quantisation of the INT8 A8W8 block ([MM] A8W8, EP
 * Dispatch): s = max|x| / 127, q = ⌊x / s⌉ in [-127, 127].  The scale and the
 * quotient x / s are fp32 (an integer decision taken from an input, like the
 * e4m3 form), the rounding is exact. */
void oracle_quantize_row_i8_f32(int n, const float* x, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    amax = a > amax ? a : amax;
  }
  float s = amax > 0.0f ? amax / 127.0f : 1.0f;
  for (int i = 0; i < n; ++i) {
    double r = round_half_away((double)(x[i] / s));
    q[i] = (int8_t)(r > 127.0 ? 127.0 : (r < -127.0 ? -127.0 : r));
  }
  *scale = s;
}

/* The INT8 A8W8 expert ([MM] A8W8, Expert Compute 1-3): Linear1 is the
 * integer product Q_e W1[e] (exact), dequantised by the per-channel weight
 * scale and the per-token scale; SwiGLU in fp64; the SwiGLU output is
 * requantised per row (s_a = max|A| / 127, ⌊A / s_a⌉), Linear2 is again an
 * integer product, dequantised by s^{W2} and s_a. */
static void swiglu_row_i8(int hidden, int f, const int8_t* qx, double sx, const int8_t* Wq1,
                          const float* s_w1, const int8_t* Wq2, const float* s_w2, double* h1,
                          double* out) {
  int64_t* acc = (int64_t*)malloc(sizeof(int64_t) * (size_t)(2 * f > hidden ? 2 * f : hidden));
  for (int n = 0; n < 2 * f; ++n) acc[n] = 0;
  for (int c = 0; c < hidden; ++c) {
    int64_t xc = qx[c];
    if (xc == 0) continue;
    for (int n = 0; n < 2 * f; ++n) acc[n] += xc * (int64_t)Wq1[(size_t)c * 2 * f + n];
  }
  for (int n = 0; n < 2 * f; ++n) h1[n] = (double)acc[n] * (double)s_w1[n] * sx;
  double amax = 0.0;
  for (int n = 0; n < f; ++n) {
    h1[n] = silu(h1[n]) * h1[f + n];
    amax = fabs(h1[n]) > amax ? fabs(h1[n]) : amax;
  }
  double sa = amax > 0.0 ? amax / 127.0 : 1.0;
  for (int o = 0; o < hidden; ++o) acc[o] = 0;
  for (int n = 0; n < f; ++n) {
    double r = round_half_away(h1[n] / sa);
    int64_t qa = (int64_t)(r > 127.0 ? 127.0 : (r < -127.0 ? -127.0 : r));
    if (qa == 0) continue;
    for (int o = 0; o < hidden; ++o) acc[o] += qa * (int64_t)Wq2[(size_t)n * hidden + o];
  }
  for (int o = 0; o < hidden; ++o) out[o] = (double)acc[o] * (double)s_w2[o] * sa;
  free(acc);
}

/* The A8W8 (e4m3) expert: x arrives quantised (q_x, s_x).  Linear1 runs on
 * codes, dequantised per output channel and per token; SwiGLU in fp64; the
 * SwiGLU output is requantised per row (s_a = max|A|/448) before Linear2,
 * whose result is dequantised the same way. */
static void swiglu_row_fp8(int hidden, int f, const uint8_t* qx, double sx, const uint8_t* Wq1,
                           const float* s_w1, const uint8_t* Wq2, const float* s_w2,
                           double* h1, double* out) {
  for (int n = 0; n < 2 * f; ++n) h1[n] = 0.0;
  for (int c = 0; c < hidden; ++c) {
    double xc = oracle_e4m3_decode(qx[c]);
    if (xc == 0.0) continue;
    for (int n = 0; n < 2 * f; ++n)
      h1[n] += xc * e4m3_table[Wq1[(size_t)c * 2 * f + n]];
  }
  for (int n = 0; n < 2 * f; ++n) h1[n] = h1[n] * (double)s_w1[n] * sx;
  double amax = 0.0;
  for (int n = 0; n < f; ++n) {
    h1[n] = silu(h1[n]) * h1[f + n];
    amax = fabs(h1[n]) > amax ? fabs(h1[n]) : amax;
  }
  double sa = amax > 0.0 ? amax / 448.0 : 1.0;
  for (int o = 0; o < hidden; ++o) out[o] = 0.0;
  for (int n = 0; n < f; ++n) {
    double qa = oracle_e4m3_decode(oracle_e4m3_encode(h1[n] / sa));
    if (qa == 0.0) continue;
    for (int o = 0; o < hidden; ++o)
      out[o] += qa * e4m3_table[Wq2[(size_t)n * hidden + o]];
  }
  for (int o = 0; o < hidden; ++o) out[o] = out[o] * (double)s_w2[o] * sa;
}

/* Element (c, n) of a K x N MX weight matrix.  MXFP8 stores it K-major:
 * codes [K, N], scales [K/32, N].  MXFP4 keeps the mega_moe page's storage,
 * K-contiguous: codes [N, K/2] (element k of row n in byte k/2, even k in the
 * low nibble), scales [N, K/32]. */
/* Element values and scale factors as tables filled once from
 * element_decode and ldexp (the same numbers as oracle_mx_value; a table
 * read keeps the expert loops fast). */
static double mx_elem_table[2][256];
static double mx_pow2_table[256];
static int mx_tables_ready = 0;
static void mx_tables_init(void) {
  if (mx_tables_ready) return;
  for (int c = 0; c < 256; ++c) {
    mx_elem_table[ORC_FMT_E4M3][c] = element_decode((uint8_t)c, ORC_FMT_E4M3);
    mx_elem_table[ORC_FMT_E2M1][c] = element_decode((uint8_t)(c & 0xF), ORC_FMT_E2M1);
    mx_pow2_table[c] = ldexp(1.0, c - 127);
  }
  mx_tables_ready = 1;
}

static double mx_weight(const uint8_t* W, const uint8_t* S, int K, int N, int c, int n, int fmt) {
  if (fmt == ORC_FMT_E4M3)
    return mx_elem_table[fmt][W[(size_t)c * N + n]] * mx_pow2_table[S[(size_t)(c / 32) * N + n]];
  size_t i = (size_t)n * K + c;
  uint8_t code = (uint8_t)((W[i / 2] >> (4 * (i & 1))) & 0xF);
  return mx_elem_table[fmt][code] * mx_pow2_table[S[(size_t)n * (K / 32) + c / 32]];
}

/* The MX expert of [MM]'s MXFP block: x is quantised per group of 32 along
 * hidden (Q_MX), Linear1 multiplies the dequantised operands (DQ_MX(X^) .
 * DQ_MX(W1)), SwiGLU in fp64, the SwiGLU output is quantised per group of 32
 * along inter and dequantised for Linear2 against DQ_MX(W2). */
static void swiglu_row_mx(int hidden, int f, const double* x, int fmt, const uint8_t* W1,
                          const uint8_t* S1, const uint8_t* W2, const uint8_t* S2, double* xd,
                          uint8_t* qbuf, uint8_t* sbuf, double* h1, double* out) {
  oracle_mx_quantize(hidden, x, fmt, qbuf, sbuf);
  for (int c = 0; c < hidden; ++c) xd[c] = oracle_mx_value(qbuf[c], sbuf[c / 32], fmt);
  for (int n = 0; n < 2 * f; ++n) h1[n] = 0.0;
  for (int c = 0; c < hidden; ++c) {
    double xc = xd[c];
    if (xc == 0.0) continue;
    for (int n = 0; n < 2 * f; ++n) h1[n] += xc * mx_weight(W1, S1, hidden, 2 * f, c, n, fmt);
  }
  for (int n = 0; n < f; ++n) h1[n] = silu(h1[n]) * h1[f + n];
  oracle_mx_quantize(f, h1, fmt, qbuf, sbuf);
  for (int o = 0; o < hidden; ++o) out[o] = 0.0;
  for (int n = 0; n < f; ++n) {
    double u = oracle_mx_value(qbuf[n], sbuf[n / 32], fmt);
    if (u == 0.0) continue;
    for (int o = 0; o < hidden; ++o) out[o] += u * mx_weight(W2, S2, f, hidden, n, o, fmt);
  }
}

/* Everything that describes one layer.  Pointers are host memory. */
typedef struct {
  int T, hidden, E, k, inter, has_shared;
  int precision;        /* 0 = fp32, 1 = bf16, 2 = A8W8 e4m3, 3 = MXFP8, 4 = MXFP4, 5 = A8W8 INT8 */
  const void* X;        /* [T,hidden]: fp32 (precision 0) or bf16 */
  const void* W1;       /* [E,hidden,2f]: fp32 / bf16 / e4m3 codes / int8; MXFP4: [E,2f,hidden/2] */
  const void* W2;       /* [E,f,hidden] */
  const void* w1_scale; /* A8W8 (e4m3, INT8): fp32 [E,2f]; MXFP8: E8M0 [E,hidden/32,2f]; MXFP4 [E,2f,hidden/32] */
  const void* w2_scale; /* A8W8: fp32 [E,hidden]; MXFP8: E8M0 [E,f/32,hidden]; MXFP4 [E,hidden,f/32] */
  const void* Ws1;      /* shared [hidden,2f] or NULL */
  const void* Ws2;      /* shared [f,hidden] */
  const void* ws1_scale;
  const void* ws2_scale;
} oracle_layer;

static int w_dt(int precision) {
  return precision == 0 ? ORC_F32 : (precision == 1 ? ORC_BF16 : ORC_FP8);
}

/* F_e(x_t) for one token and one expert (e == E selects the shared expert). */
static void expert_of_token(const oracle_layer* L, int t, int e, double* xbuf, uint8_t* qbuf,
                            float* fbuf, double* h1, double* out) {
  int h = L->hidden, f = L->inter;
  int shared = (e == L->E);
  const char* W1 = shared ? (const char*)L->Ws1 : (const char*)L->W1;
  const char* W2 = shared ? (const char*)L->Ws2 : (const char*)L->W2;
  int xdt = L->precision == 0 ? ORC_F32 : ORC_BF16;
  if (L->precision == 3 || L->precision == 4) {
    int fmt = L->precision == 3 ? ORC_FMT_E4M3 : ORC_FMT_E2M1;
    size_t d1 = (size_t)h * 2 * f, d2 = (size_t)f * h; /* elements per expert */
    const uint8_t* S1 = shared ? (const uint8_t*)L->ws1_scale
                               : (const uint8_t*)L->w1_scale + (size_t)e * (h / 32) * 2 * f;
    const uint8_t* S2 = shared ? (const uint8_t*)L->ws2_scale
                               : (const uint8_t*)L->w2_scale + (size_t)e * (f / 32) * h;
    if (!shared) {
      W1 += fmt == ORC_FMT_E4M3 ? (size_t)e * d1 : (size_t)e * d1 / 2;
      W2 += fmt == ORC_FMT_E4M3 ? (size_t)e * d2 : (size_t)e * d2 / 2;
    }
    for (int c = 0; c < h; ++c) xbuf[c] = elem(L->X, xdt, (size_t)t * h + c);
    swiglu_row_mx(h, f, xbuf, fmt, (const uint8_t*)W1, S1, (const uint8_t*)W2, S2,
                  xbuf + h, qbuf, qbuf + (h > f ? h : f), h1, out);
    return;
  }
  size_t wb = (L->precision == 0) ? 4 : (L->precision == 1 ? 2 : 1);
  if (!shared) {
    W1 += (size_t)e * h * 2 * f * wb;
    W2 += (size_t)e * f * h * wb;
  }
  if (L->precision == 5) {
    for (int c = 0; c < h; ++c) fbuf[c] = (float)elem(L->X, xdt, (size_t)t * h + c);
    float sx;
    oracle_quantize_row_i8_f32(h, fbuf, (int8_t*)qbuf, &sx);
    const float* s1 = shared ? (const float*)L->ws1_scale : (const float*)L->w1_scale + (size_t)e * 2 * f;
    const float* s2 = shared ? (const float*)L->ws2_scale : (const float*)L->w2_scale + (size_t)e * h;
    swiglu_row_i8(h, f, (const int8_t*)qbuf, (double)sx, (const int8_t*)W1, s1, (const int8_t*)W2,
                  s2, h1, out);
  } else if (L->precision == 2) {
    for (int c = 0; c < h; ++c) fbuf[c] = (float)elem(L->X, xdt, (size_t)t * h + c);
    float sx;
    oracle_quantize_row_f32(h, fbuf, qbuf, &sx);
    const float* s1 = shared ? (const float*)L->ws1_scale : (const float*)L->w1_scale + (size_t)e * 2 * f;
    const float* s2 = shared ? (const float*)L->ws2_scale : (const float*)L->w2_scale + (size_t)e * h;
    swiglu_row_fp8(h, f, qbuf, (double)sx, (const uint8_t*)W1, s1, (const uint8_t*)W2, s2, h1,
                   out);
  } else {
    for (int c = 0; c < h; ++c) xbuf[c] = elem(L->X, xdt, (size_t)t * h + c);
    swiglu_row(h, f, xbuf, w_dt(L->precision), W1, W2, h1, out);
  }
}

/* The layer equation of [V4] §模型与入口, token by token:
 *   y_t = F_s(x_t) + sum_j G[t,j] * F_{ids[t,j]}(x_t)
 * for the tokens listed in tok[0..ntok) (all tokens when tok == NULL).
 * Y is [ntok, hidden] fp64. */
void oracle_layer_tokens(const oracle_layer* L, const int32_t* ids, const double* G, int ntok,
                         const int32_t* tok, double* Y) {
  int h = L->hidden, f = L->inter;
  e4m3_table_init();
  mx_tables_init();
#pragma omp parallel
  {
    double* xbuf = (double*)malloc(sizeof(double) * 2 * h);
    uint8_t* qbuf = (uint8_t*)malloc((size_t)2 * (h > f ? h : f));
    float* fbuf = (float*)malloc(sizeof(float) * h);
    double* h1 = (double*)malloc(sizeof(double) * 2 * f);
    double* fe = (double*)malloc(sizeof(double) * h);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < ntok; ++i) {
      int t = tok ? tok[i] : i;
      double* y = Y + (size_t)i * h;
      for (int o = 0; o < h; ++o) y[o] = 0.0;
      for (int j = 0; j < L->k; ++j) {
        int e = ids[(size_t)t * L->k + j];
        if (e < 0 || e >= L->E) continue;
        expert_of_token(L, t, e, xbuf, qbuf, fbuf, h1, fe);
        double g = G[(size_t)t * L->k + j];
        for (int o = 0; o < h; ++o) y[o] += g * fe[o];
      }
      if (L->has_shared) {
        expert_of_token(L, t, L->E, xbuf, qbuf, fbuf, h1, fe);
        for (int o = 0; o < h; ++o) y[o] += fe[o];
      }
    }
    free(xbuf);
    free(qbuf);
    free(fbuf);
    free(h1);
    free(fe);
  }
}

/* The staged form of [MM]: the rows of the dispatched matrix are the tokens
 * src_tok[r]; row r belongs to the expert whose block [offsets[e],
 * offsets[e+1]) holds it.  Yp[r] = F_e(x_{src_tok[r]}) for the listed rows
 * (all T*k rows when rows == NULL).  Yp is [nrows, hidden] fp64.  With
 * has_shared, rows T*k .. T*k+T-1 stand for the shared expert applied to token
 * r - T*k (src_tok is not read for them). */
void oracle_expert_rows(const oracle_layer* L, const int32_t* offsets, const int32_t* src_tok,
                        int nrows, const int32_t* rows, double* Yp) {
  int h = L->hidden, f = L->inter;
  e4m3_table_init();
  mx_tables_init();
#pragma omp parallel
  {
    double* xbuf = (double*)malloc(sizeof(double) * 2 * h);
    uint8_t* qbuf = (uint8_t*)malloc((size_t)2 * (h > f ? h : f));
    float* fbuf = (float*)malloc(sizeof(float) * h);
    double* h1 = (double*)malloc(sizeof(double) * 2 * f);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < nrows; ++i) {
      int r = rows ? rows[i] : i;
      int routed = L->T * L->k;
      if (r >= routed) {
        expert_of_token(L, r - routed, L->E, xbuf, qbuf, fbuf, h1, Yp + (size_t)i * h);
        continue;
      }
      int e = 0;
      while (e < L->E && offsets[e + 1] <= r) ++e;
      expert_of_token(L, src_tok[r], e, xbuf, qbuf, fbuf, h1, Yp + (size_t)i * h);
    }
    free(xbuf);
    free(qbuf);
    free(fbuf);
    free(h1);
  }
}

/* Token Combine of [MM]: y[t] = sum_j G[t,j] * Yp[dst_row[t,j]] (+ Ys[t]),
 * j ascending.  Yp is [T*k, hidden], Ys [T, hidden] or NULL, all fp64. */
void oracle_combine(int T, int k, int hidden, const double* Yp, const int32_t* dst_row,
                    const double* G, const double* Ys, double* Y) {
  for (int t = 0; t < T; ++t) {
    double* y = Y + (size_t)t * hidden;
    for (int o = 0; o < hidden; ++o) y[o] = 0.0;
    for (int j = 0; j < k; ++j) {
      int r = dst_row[(size_t)t * k + j];
      if (r < 0) continue;
      double g = G[(size_t)t * k + j];
      for (int o = 0; o < hidden; ++o) y[o] += g * Yp[(size_t)r * hidden + o];
    }
    if (Ys)
      for (int o = 0; o < hidden; ++o) y[o] += Ys[(size_t)t * hidden + o];
  }
}

/* ------------------------------------------------------------------ */
/* Backward, local part  ([V4] 反向的通信: the reverse chain on one      */
/* device, unpermute -> expert dgrad / wgrad -> permute, which sums the */
/* k copies; [V4] dX = Ȳ Wᵀ, dW = Xᵀ Ȳ for an expert linear; [MD] §1.8  */
/* SwiGLU backward dA = dH ⊙ U, dU = dH ⊙ A, dG = dA ⊙ [σ(G) + A ⊙ (1 − */
/* σ(G))] with A = SiLU(G))                                             */
/* ------------------------------------------------------------------ */

/* For one row x (fp64) through expert weights W1 [h,2f], W2 [f,h] of element
 * type wdt and the upstream gradient dy [h] of its output: the expert output
 * y (for dG), the SwiGLU output a [f], dh1 [2f] (gradient of the Linear1
 * pre-activations, gate then up) and dx [h].  Buffers are the caller's. */
static void swiglu_row_backward(int hidden, int f, const double* x, int wdt, const void* W1,
                                const void* W2, const double* dy, double* h1, double* a,
                                double* y, double* dh1, double* dx) {
  for (int n = 0; n < 2 * f; ++n) h1[n] = 0.0;
  for (int c = 0; c < hidden; ++c) {
    double xc = x[c];
    if (xc == 0.0) continue;
    for (int n = 0; n < 2 * f; ++n) h1[n] += xc * elem(W1, wdt, (size_t)c * 2 * f + n);
  }
  for (int n = 0; n < f; ++n) a[n] = silu(h1[n]) * h1[f + n];
  for (int o = 0; o < hidden; ++o) y[o] = 0.0;
  for (int n = 0; n < f; ++n)
    for (int o = 0; o < hidden; ++o) y[o] += a[n] * elem(W2, wdt, (size_t)n * hidden + o);
  /* dH (gradient of the SwiGLU output) = dy W2ᵀ, then the SwiGLU backward */
  for (int n = 0; n < f; ++n) {
    double dH = 0.0;
    for (int o = 0; o < hidden; ++o) dH += dy[o] * elem(W2, wdt, (size_t)n * hidden + o);
    double g = h1[n], u = h1[f + n];
    double sg = sigmoid(g), act = silu(g);
    double dA = dH * u;       /* gradient of SiLU(g) */
    dh1[f + n] = dH * act;    /* dU */
    dh1[n] = dA * (sg + act * (1.0 - sg));
  }
  /* dx = dh1 W1ᵀ */
  for (int c = 0; c < hidden; ++c) {
    double s = 0.0;
    for (int n = 0; n < 2 * f; ++n) s += dh1[n] * elem(W1, wdt, (size_t)c * 2 * f + n);
    dx[c] = s;
  }
}

static void expert_weight_ptrs(const oracle_layer* L, int e, const char** W1, const char** W2) {
  size_t wb = (L->precision == 0) ? 4 : 2;
  if (e == L->E) {
    *W1 = (const char*)L->Ws1;
    *W2 = (const char*)L->Ws2;
  } else {
    *W1 = (const char*)L->W1 + (size_t)e * L->hidden * 2 * L->inter * wb;
    *W2 = (const char*)L->W2 + (size_t)e * L->inter * L->hidden * wb;
  }
}

/* Layer backward for the listed tokens (all when tok == NULL), fp32 / bf16
 * layers: given dY [T, hidden] (fp64), writes dX [ntok, hidden] (the expert
 * part: sum over j of the routed experts' dx with upstream G[t,j] dY[t], plus
 * the shared expert's with upstream dY[t]) and dG [ntok, k] (dG[t,j] =
 * dY[t] . F_e(x_t), the unpermute backward of the gate weights).  Returns -1
 * for a quantised layer. */
int oracle_backward_tokens(const oracle_layer* L, const int32_t* ids, const double* G,
                           const double* dY, int ntok, const int32_t* tok, double* dX,
                           double* dG) {
  if (L->precision > 1) return -1;
  int h = L->hidden, f = L->inter, k = L->k;
  int xdt = L->precision == 0 ? ORC_F32 : ORC_BF16, wdt = w_dt(L->precision);
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * h);
    double* dy = (double*)malloc(sizeof(double) * h);
    double* h1 = (double*)malloc(sizeof(double) * 2 * f);
    double* a = (double*)malloc(sizeof(double) * f);
    double* y = (double*)malloc(sizeof(double) * h);
    double* dh1 = (double*)malloc(sizeof(double) * 2 * f);
    double* dx = (double*)malloc(sizeof(double) * h);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < ntok; ++i) {
      int t = tok ? tok[i] : i;
      double* dxt = dX + (size_t)i * h;
      for (int c = 0; c < h; ++c) {
        x[c] = elem(L->X, xdt, (size_t)t * h + c);
        dxt[c] = 0.0;
      }
      for (int j = 0; j < k; ++j) {
        int e = ids[(size_t)t * k + j];
        if (e < 0 || e >= L->E) {
          dG[(size_t)i * k + j] = 0.0;
          continue;
        }
        const char *W1, *W2;
        expert_weight_ptrs(L, e, &W1, &W2);
        double g = G[(size_t)t * k + j];
        for (int o = 0; o < h; ++o) dy[o] = g * dY[(size_t)t * h + o];
        swiglu_row_backward(h, f, x, wdt, W1, W2, dy, h1, a, y, dh1, dx);
        double s = 0.0;
        for (int o = 0; o < h; ++o) s += dY[(size_t)t * h + o] * y[o];
        dG[(size_t)i * k + j] = s;
        for (int c = 0; c < h; ++c) dxt[c] += dx[c];
      }
      if (L->has_shared) {
        const char *W1, *W2;
        expert_weight_ptrs(L, L->E, &W1, &W2);
        swiglu_row_backward(h, f, x, wdt, W1, W2, dY + (size_t)t * h, h1, a, y, dh1, dx);
        for (int c = 0; c < h; ++c) dxt[c] += dx[c];
      }
    }
    free(x);
    free(dy);
    free(h1);
    free(a);
    free(y);
    free(dh1);
    free(dx);
  }
  return 0;
}

/* Weight gradients of the listed experts (e == E: the shared expert):
 * dW1[e] = sum over the rows r routed to e of x_r^T dh1_r  ([hidden, 2f]),
 * dW2[e] = sum of a_r^T dy_r  ([f, hidden]), where dy_r = G[t,j] dY[t] (dY[t]
 * for the shared expert).  Rows are visited in ascending t*k+j.  dW1 / dW2
 * are [nexp, ...] fp64.  Returns -1 for a quantised layer. */
int oracle_backward_weights(const oracle_layer* L, const int32_t* ids, const double* G,
                            const double* dY, int nexp, const int32_t* experts, double* dW1,
                            double* dW2) {
  if (L->precision > 1) return -1;
  int h = L->hidden, f = L->inter, k = L->k, T = L->T;
  int xdt = L->precision == 0 ? ORC_F32 : ORC_BF16, wdt = w_dt(L->precision);
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * h);
    double* dy = (double*)malloc(sizeof(double) * h);
    double* h1 = (double*)malloc(sizeof(double) * 2 * f);
    double* a = (double*)malloc(sizeof(double) * f);
    double* y = (double*)malloc(sizeof(double) * h);
    double* dh1 = (double*)malloc(sizeof(double) * 2 * f);
    double* dx = (double*)malloc(sizeof(double) * h);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < nexp; ++q) {
      int e = experts[q];
      double* w1 = dW1 + (size_t)q * h * 2 * f;
      double* w2 = dW2 + (size_t)q * f * h;
      for (size_t i = 0; i < (size_t)h * 2 * f; ++i) w1[i] = 0.0;
      for (size_t i = 0; i < (size_t)f * h; ++i) w2[i] = 0.0;
      const char *W1, *W2;
      expert_weight_ptrs(L, e, &W1, &W2);
      for (int t = 0; t < T; ++t) {
        for (int j = 0; j < (e == L->E ? 1 : k); ++j) {
          if (e != L->E && ids[(size_t)t * k + j] != e) continue;
          if (e == L->E && !L->has_shared) continue;
          double g = e == L->E ? 1.0 : G[(size_t)t * k + j];
          for (int c = 0; c < h; ++c) x[c] = elem(L->X, xdt, (size_t)t * h + c);
          for (int o = 0; o < h; ++o) dy[o] = g * dY[(size_t)t * h + o];
          swiglu_row_backward(h, f, x, wdt, W1, W2, dy, h1, a, y, dh1, dx);
          for (int c = 0; c < h; ++c) {
            if (x[c] == 0.0) continue;
            for (int n = 0; n < 2 * f; ++n) w1[(size_t)c * 2 * f + n] += x[c] * dh1[n];
          }
          for (int n = 0; n < f; ++n)
            for (int o = 0; o < h; ++o) w2[(size_t)n * h + o] += a[n] * dy[o];
        }
      }
    }
    free(x);
    free(dy);
    free(h1);
    free(a);
    free(y);
    free(dh1);
    free(dx);
  }
  return 0;
}

/* Router backward ([V4] §路由张量: the mixing weights are the selected
 * experts' continuous affinities, α a / Σ a with renorm, else α a; the
 * selection itself is discrete and passes no gradient).  Given the chosen ids
 * and dG [T,k], writes dl [T,E] (gradient of the gating logits: zero outside
 * the chosen experts for sigmoid and sqrt(softplus); softmax spreads it over
 * all experts), and, where not NULL, dWg [hidden,E] = Xᵀ dl, dgate_bias [E] =
 * column sums of dl, and dX [T,hidden] += dl Wgᵀ. */
void oracle_route_backward(int T, int hidden, int E, int k, int dt, const void* X, const void* Wg,
                           const double* gate_bias, int score_fn, int renorm, double alpha,
                           const int32_t* ids, const double* dG, double* dl, double* dWg,
                           double* dgate_bias, double* dX) {
  double* logits = (double*)malloc(sizeof(double) * (size_t)T * E);
  double* aff = (double*)malloc(sizeof(double) * (size_t)T * E);
  double* da = (double*)malloc(sizeof(double) * (size_t)E);
  oracle_gate_logits(T, hidden, E, dt, X, Wg, gate_bias, logits);
  oracle_affinity(T, E, score_fn, logits, aff);
  for (int t = 0; t < T; ++t) {
    const double* a = aff + (size_t)t * E;
    const double* l = logits + (size_t)t * E;
    double* dlt = dl + (size_t)t * E;
    for (int e = 0; e < E; ++e) da[e] = 0.0;
    double S = 0.0, dGa = 0.0;
    for (int j = 0; j < k; ++j) S += a[ids[(size_t)t * k + j]];
    for (int j = 0; j < k; ++j) dGa += dG[(size_t)t * k + j] * a[ids[(size_t)t * k + j]];
    /* G_j = α a_j / S: dG_j/da_i = α (δ_ij / S − a_j / S²) */
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      double g = dG[(size_t)t * k + j];
      da[e] += renorm ? alpha * (g / S - dGa / (S * S)) : alpha * g;
    }
    if (score_fn == ORC_SOFTMAX) {
      double s = 0.0;
      for (int e = 0; e < E; ++e) s += da[e] * a[e];
      for (int e = 0; e < E; ++e) dlt[e] = a[e] * (da[e] - s);
    } else if (score_fn == ORC_SQRT_SOFTPLUS) {
      for (int e = 0; e < E; ++e) dlt[e] = da[e] == 0.0 ? 0.0 : da[e] * sigmoid(l[e]) / (2.0 * a[e]);
    } else {
      for (int e = 0; e < E; ++e) dlt[e] = da[e] * a[e] * (1.0 - a[e]);
    }
  }
  if (dgate_bias) {
    for (int e = 0; e < E; ++e) dgate_bias[e] = 0.0;
    for (int t = 0; t < T; ++t)
      for (int e = 0; e < E; ++e) dgate_bias[e] += dl[(size_t)t * E + e];
  }
  if (dWg) {
#pragma omp parallel for schedule(static)
    for (int c = 0; c < hidden; ++c) {
      double* w = dWg + (size_t)c * E;
      for (int e = 0; e < E; ++e) w[e] = 0.0;
      for (int t = 0; t < T; ++t) {
        double xc = elem(X, dt, (size_t)t * hidden + c);
        if (xc == 0.0) continue;
        for (int e = 0; e < E; ++e) w[e] += xc * dl[(size_t)t * E + e];
      }
    }
  }
  if (dX) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
      for (int c = 0; c < hidden; ++c) {
        double s = 0.0;
        for (int e = 0; e < E; ++e) s += dl[(size_t)t * E + e] * elem(Wg, dt, (size_t)c * E + e);
        dX[(size_t)t * hidden + c] += s;
      }
  }
  free(logits);
  free(aff);
  free(da);
}
