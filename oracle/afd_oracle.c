/*
 * afd_oracle.c -- CPU oracle for one MoE layer's expert FFN (FFN side of
 * Attention-FFN disaggregation).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this.  It shares no code, header, table or constant
 * with the HIP library, and the HIP library never calls it.
 *
 * It computes the plain per-token definition of the layer, slowly and in the
 * obvious way, in double precision:
 *
 *   route   : per token, softmax over all E fp32 router logits; the k experts with
 *             the largest logits (ties -> lower expert index); gates = their softmax
 *             probabilities renormalised to sum to 1.
 *   capacity: the adaptive token dropper (one expert per token, least-loaded
 *             fallback at half gate, drop, adaptive per-expert limits).
 *   permute : counting sort of the T*k (token, slot) pairs by expert: per-expert
 *             counts, exclusive prefix sum, then placement of the pairs in
 *             ascending pair order.
 *   expert  : h = SiLU(x W_gate) * (x W_up), o = h W_down, SiLU(z) = z / (1 + e^-z).
 *   combine : y_t = sum_j g_tj o_tj in slot order, plus the shared expert's output
 *             (gate 1) when there is one.
 *   fp8     : weights are OCP e4m3 codes times one fp32 scale per 128x128 block;
 *             activations (x, and h before the down projection) are quantised per
 *             row and per 128-channel group to e4m3 with scale amax/448, the code
 *             decided in fp32 (the precision the GPU path decides it in).
 *
 * Pages:
 *   [AFD-blog]  "大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §3 (the FFN
 *               service: receive activations, gate routing + expert compute, return).
 *   [MoE-eng]   "MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态专家放置",
 *               §4.1 (top-k router with softmax gates), §4.2 (dynamic token dropping),
 *               §2.2 (per-destination counts, prefix-sum offsets, pack).
 *   [AFD-news]  omica.com.cn AFD article, §2.1 (6*B*H*M FLOPs, arithmetic intensity),
 *               §3.3 (pre-sorting routed tokens, FP8/BF16 mixed precision).
 * Readings where the pages are open (softmax before/after top-k, tie order, the
 * gate/up column split, fp8 scale granularity) follow the workload definition of the
 * layer and are listed with the oracle's pins in the tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { AFDO_F32 = 0, AFDO_BF16 = 1, AFDO_FP8 = 2 };
enum { AFDO_OK = 0, AFDO_EINVAL = -1, AFDO_ENOMEM = -3 };

#define QBLOCK 128

/* ------------------------------------------------------------------ number formats */

/* bfloat16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit float E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds subnormals m/8 * 2^-6; no infinities; the codes with
 * all exponent and mantissa bits set are NaN; the largest finite value is 448. */
double afdo_fp8_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest e4m3 code to a finite fp32 value, ties to the code with an even mantissa.
 * Searched over every finite magnitude, so values beyond 448 land on 448
 * (saturation).  The sign bit is kept, also when the magnitude rounds to zero (-0). */
uint8_t afdo_fp8_encode(float v) {
  double a = fabs((double)v);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 127; ++c) { /* 0x00..0x7E: every finite non-negative code */
    double d = fabs(afdo_fp8_decode((uint8_t)c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = c;
    }
  }
  if (signbit(v)) best |= 0x80;
  return (uint8_t)best;
}

/* Quantise n fp32 values in groups of 128 along the row: scale = amax/448 in fp32
 * (1 when the group is all zero), code = nearest e4m3 of v/scale in fp32.  Writes the
 * dequantised values code*scale (exact in double). */
void afdo_quant_row_fp8(int n, const float* v, uint8_t* codes, float* scales, double* deq) {
  for (int g = 0; g < n / QBLOCK; ++g) {
    float amax = 0.0f;
    for (int i = 0; i < QBLOCK; ++i) {
      float a = fabsf(v[g * QBLOCK + i]);
      if (a > amax) amax = a;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    if (scales) scales[g] = s;
    for (int i = 0; i < QBLOCK; ++i) {
      float q = v[g * QBLOCK + i] / s;
      uint8_t c = afdo_fp8_encode(q);
      if (codes) codes[g * QBLOCK + i] = c;
      if (deq) deq[g * QBLOCK + i] = afdo_fp8_decode(c) * (double)s;
    }
  }
}

/* One weight matrix [rows, cols] of one expert, row-major, in its storage dtype. */
typedef struct {
  int dtype;
  const void* data;
  const float* scales; /* fp8 only: [rows/128, cols/128] */
  int rows, cols;
} mat_t;

/* Decoded value of every e4m3 code, filled once from afdo_fp8_decode. */
static const double* fp8_table(void) {
  static double table[256];
  static int ready = 0;
#pragma omp critical(afdo_fp8_table)
  {
    if (!ready) {
      for (int c = 0; c < 256; ++c) table[c] = afdo_fp8_decode((uint8_t)c);
      ready = 1;
    }
  }
  return table;
}

/* Row r of a weight matrix, decoded to double (fp8: code times its block scale). */
static void mat_row(const mat_t* w, int r, double* out) {
  if (w->dtype == AFDO_F32) {
    const float* p = (const float*)w->data + (size_t)r * w->cols;
    for (int c = 0; c < w->cols; ++c) out[c] = (double)p[c];
  } else if (w->dtype == AFDO_BF16) {
    const uint16_t* p = (const uint16_t*)w->data + (size_t)r * w->cols;
    for (int c = 0; c < w->cols; ++c) out[c] = bf16_to_double(p[c]);
  } else {
    const uint8_t* p = (const uint8_t*)w->data + (size_t)r * w->cols;
    const float* s = w->scales + (size_t)(r / QBLOCK) * (w->cols / QBLOCK);
    const double* dec = fp8_table();
    for (int c = 0; c < w->cols; ++c) out[c] = dec[p[c]] * (double)s[c / QBLOCK];
  }
}

/* ------------------------------------------------------------------ routing */

/* Router projection of the MoE engineering page (§4.1): a bias-free linear map from
 * the hidden size to the experts, plus a per-expert dynamic bias, gives the scores
 * the top-k selects on.  scores[t, e] = sum_h x[t, h] * w[e, h] + bias[e] in double
 * (bias may be NULL: none); x [T, H] and w [E, H] hold fp32 (or bf16-valued) inputs. */
void afdo_router_scores(int T, int E, int H, const float* x, const float* w, const float* bias, double* scores) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* xr = x + (size_t)t * H;
    for (int e = 0; e < E; ++e) {
      const float* wr = w + (size_t)e * H;
      double s = 0.0;
      for (int h = 0; h < H; ++h) s += (double)xr[h] * (double)wr[h];
      scores[(size_t)t * E + e] = s + (bias ? (double)bias[e] : 0.0);
    }
  }
}

/* Per token: softmax over all E logits (double), then the k experts ranked by
 * (logit descending, expert index ascending) compared on the raw fp32 logits, then
 * gates = selected probabilities / their sum.  The rank of expert e is the number of
 * experts that beat it; slot j holds the expert of rank j. */
void afdo_route(int T, int E, int k, const float* logits, int32_t* ids, double* gates) {
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    double m = -INFINITY, z = 0.0, sel = 0.0;
    for (int e = 0; e < E; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
    for (int e = 0; e < E; ++e) {
      int rank = 0;
      for (int i = 0; i < E; ++i)
        if (l[i] > l[e] || (l[i] == l[e] && i < e)) ++rank;
      if (rank < k) ids[(size_t)t * k + rank] = e;
    }
    for (int j = 0; j < k; ++j) sel += exp((double)l[ids[(size_t)t * k + j]] - m) / z;
    for (int j = 0; j < k; ++j)
      gates[(size_t)t * k + j] = (exp((double)l[ids[(size_t)t * k + j]] - m) / z) / sel;
  }
}

/* Router with a selection-only bias.  [MoE-eng] §4.1 steers expert load with a
 * per-expert dynamic bias and names DeepSeek-V3's dynamic bias adjustment; in the
 * variant built here the bias only decides which experts are chosen, while the gate
 * weights come from the unbiased scores.  Per token: key[e] = scores[e] + bias[e]
 * rounded to fp32 (the precision the selection is decided in); the k experts ranked
 * by (key descending, expert index ascending); gates = the softmax probabilities of
 * the unbiased scores (double) of the chosen experts, renormalised to sum to 1. */
void afdo_route_select_bias(int T, int E, int k, const float* scores, const float* bias, int32_t* ids,
                            double* gates) {
  float* key = (float*)malloc(sizeof(float) * (size_t)(E > 0 ? E : 1));
  for (int t = 0; t < T; ++t) {
    const float* s = scores + (size_t)t * E;
    double m = -INFINITY, z = 0.0, sel = 0.0;
    for (int e = 0; e < E; ++e) {
      volatile float v = s[e] + bias[e];
      key[e] = v;
    }
    for (int e = 0; e < E; ++e)
      if ((double)s[e] > m) m = (double)s[e];
    for (int e = 0; e < E; ++e) z += exp((double)s[e] - m);
    for (int e = 0; e < E; ++e) {
      int rank = 0;
      for (int i = 0; i < E; ++i)
        if (key[i] > key[e] || (key[i] == key[e] && i < e)) ++rank;
      if (rank < k) ids[(size_t)t * k + rank] = e;
    }
    for (int j = 0; j < k; ++j) sel += exp((double)s[ids[(size_t)t * k + j]] - m) / z;
    for (int j = 0; j < k; ++j)
      gates[(size_t)t * k + j] = (exp((double)s[ids[(size_t)t * k + j]] - m) / z) / sel;
  }
  free(key);
}

/* Counting sort of pair ids p = t*k + j by expert: counts, exclusive prefix sum
 * (offsets[E] = T*k), then each pair placed at its expert's cursor in ascending p.
 * pair_pos is the inverse permutation of sorted_pair. */
void afdo_permute(int T, int E, int k, const int32_t* ids, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_pair, int32_t* pair_pos) {
  int P = T * k;
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int p = 0; p < P; ++p) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int p = 0; p < P; ++p) {
    int r = cursor[ids[p]]++;
    sorted_pair[r] = p;
    pair_pos[p] = r;
  }
  free(cursor);
}

/* ------------------------------------------------------------------ capacity-aware routing */

/* The adaptive token dropper of the MoE engineering page, §4.2, for one batch.
 * Per-expert counts start at zero (the batch's own load); limits[E] is the adaptive
 * capacity state, read and then updated in place.  Tokens are taken in ascending
 * order.  A token goes to the first expert of its preference list ids[t*k .. t*k+k)
 * whose count is below its limit, with that slot's gate, and to no other expert.
 * When every preferred expert is full, the least-loaded expert (smallest count,
 * lowest index on ties) takes it at half the first slot's gate if its count is below
 * 1.5 times its limit; otherwise the token is dropped (assign = -1, weight = 0).
 * After the batch, when `adaptive` is set, each limit grows by 1.2x (truncated) if
 * the expert's count reached it, else shrinks by 0.9x (truncated, not below `base`)
 * if the count stayed under half of it; the products are taken in double precision
 * as the page's code takes them, and a grown limit saturates at INT32_MAX.
 * counts/offsets/sorted_token list each expert's tokens in token order (the page's
 * per-expert routed lists). */
void afdo_route_capacity(int T, int E, int k, const int32_t* ids, const float* gates, int32_t base, int adaptive,
                         int32_t* limits, int32_t* assign, float* weight, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_token) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int t = 0; t < T; ++t) {
    int chosen = -1;
    float w = 0.0f;
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      if (counts[e] < limits[e]) {
        chosen = e;
        w = gates[(size_t)t * k + j];
        break;
      }
    }
    if (chosen < 0) {
      int least = 0;
      for (int e = 1; e < E; ++e)
        if (counts[e] < counts[least]) least = e;
      if ((double)counts[least] < (double)limits[least] * 1.5) {
        chosen = least;
        w = (float)((double)gates[(size_t)t * k] * 0.5);
      }
    }
    assign[t] = chosen;
    weight[t] = chosen < 0 ? 0.0f : w;
    if (chosen >= 0) counts[chosen] += 1;
  }
  if (adaptive) {
    for (int e = 0; e < E; ++e) {
      double L = (double)limits[e];
      if (counts[e] >= limits[e]) {
        double g = trunc(L * 1.2);
        limits[e] = g > 2147483647.0 ? 2147483647 : (int32_t)g;
      } else if ((double)counts[e] < L * 0.5) {
        int32_t s = (int32_t)trunc(L * 0.9);
        limits[e] = s > base ? s : base;
      }
    }
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int t = 0; t < T; ++t)
    if (assign[t] >= 0) sorted_token[cursor[assign[t]]++] = t;
  free(cursor);
}

/* ------------------------------------------------------------------ expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Scratch arrays of one worker thread. */
typedef struct {
  double *xa, *a, *h, *row;
  float* hf;
} work_t;

/* o[H] = SwiGLU FFN of one token: a = x W_gu ([H] x [H, 2M]), h = SiLU(a[:M]) * a[M:],
 * o = h W_d ([M] x [M, H]).  quant_act: x and h are fp8-quantised per 128 first.
 * Returns the number of multiply-adds executed. */
static int64_t swiglu_ffn(int H, int M, const float* x, const mat_t* wgu, const mat_t* wd, int quant_act,
                          double* o, work_t* w) {
  int64_t macs = 0;
  if (quant_act) {
    afdo_quant_row_fp8(H, x, NULL, NULL, w->xa);
  } else {
    for (int i = 0; i < H; ++i) w->xa[i] = (double)x[i];
  }
  for (int n = 0; n < 2 * M; ++n) w->a[n] = 0.0;
  for (int kk = 0; kk < H; ++kk) {
    mat_row(wgu, kk, w->row);
    for (int n = 0; n < 2 * M; ++n) w->a[n] += w->xa[kk] * w->row[n];
    macs += 2 * M;
  }
  for (int n = 0; n < M; ++n) w->h[n] = silu(w->a[n]) * w->a[M + n];
  if (quant_act) {
    for (int n = 0; n < M; ++n) w->hf[n] = (float)w->h[n];
    afdo_quant_row_fp8(M, w->hf, NULL, NULL, w->h);
  }
  for (int c = 0; c < H; ++c) o[c] = 0.0;
  for (int n = 0; n < M; ++n) {
    mat_row(wd, n, w->row);
    for (int c = 0; c < H; ++c) o[c] += w->h[n] * w->row[c];
    macs += H;
  }
  return macs;
}

/* Problem description shared by the layer entry point. */
typedef struct {
  int H, M, E, k, Ms;
  int dtype;                 /* weights: AFDO_F32 / AFDO_BF16 / AFDO_FP8 */
  const void* const* w_gu;   /* [E] pointers to [H, 2M] (NULL for an expert not needed) */
  const void* const* w_d;    /* [E] pointers to [M, H] */
  const float* const* s_gu;  /* fp8: [E] pointers to [H/128, 2M/128] */
  const float* const* s_d;   /* fp8: [E] pointers to [M/128, H/128] */
  const void* ws_gu;         /* shared expert [H, 2Ms] or NULL */
  const void* ws_d;          /* shared expert [Ms, H] */
  const float* ss_gu;
  const float* ss_d;
} afdo_problem;

/* Whole layer for n tokens given by their fp32 activations x [n, H] (bf16 inputs
 * widened exactly) and fp32 logits [n, E].  Writes ids [n, k], gates [n, k] and
 * y [n, H] (double).  With logits NULL, ids and gates are inputs instead (an
 * assignment made elsewhere, such as the capacity-aware dropper's); a slot with id -1
 * contributes nothing.  *macs receives the number of multiply-adds the expert
 * products executed, counted in their loops (the FLOP count is twice that).  nthreads <= 0 uses the OpenMP default. */
int afdo_layer(const afdo_problem* pb, int n, const float* x, const float* logits, int32_t* ids,
               double* gates, double* y, int64_t* macs, int nthreads) {
  const int H = pb->H, M = pb->M, E = pb->E, k = pb->k, Ms = pb->Ms;
  if (n < 0 || H <= 0 || M <= 0 || E <= 0 || k <= 0 || k > E || Ms < 0) return AFDO_EINVAL;
  if (pb->dtype == AFDO_FP8 && (H % QBLOCK || M % QBLOCK || Ms % QBLOCK)) return AFDO_EINVAL;
  if (logits) afdo_route(n, E, k, logits, ids, gates);
  for (int p = 0; p < n * k; ++p) {
    int e = ids[p];
    if (e < 0 && !logits) continue;
    if (e < 0 || e >= E) return AFDO_EINVAL;
    if (!pb->w_gu[e] || !pb->w_d[e]) return AFDO_EINVAL;
    if (pb->dtype == AFDO_FP8 && (!pb->s_gu[e] || !pb->s_d[e])) return AFDO_EINVAL;
  }
  if (Ms > 0 && (!pb->ws_gu || !pb->ws_d)) return AFDO_EINVAL;
  const int per = k + (Ms > 0 ? 1 : 0); /* FFN evaluations per token */
  const int units = n * per;
  const int Mmax = M > Ms ? M : Ms;
  const int rowlen = 2 * Mmax > H ? 2 * Mmax : H;
  double* outs = (double*)malloc(sizeof(double) * ((size_t)units * H + 1));
  if (!outs) return AFDO_ENOMEM;
  int fail = 0;
  int64_t total = 0;
  const int quant = pb->dtype == AFDO_FP8;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(+ : total)
  {
    work_t w;
    w.xa = (double*)malloc(sizeof(double) * (size_t)H);
    w.a = (double*)malloc(sizeof(double) * 2 * (size_t)Mmax);
    w.h = (double*)malloc(sizeof(double) * (size_t)Mmax);
    w.row = (double*)malloc(sizeof(double) * (size_t)rowlen);
    w.hf = (float*)malloc(sizeof(float) * (size_t)Mmax);
    const int ok = w.xa && w.a && w.h && w.row && w.hf;
    if (!ok) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
      if (!ok) continue;
      int t = u / per, j = u % per;
      mat_t gu, dn;
      if (j < k && ids[(size_t)t * k + j] < 0) {
        for (int c = 0; c < H; ++c) outs[(size_t)u * H + c] = 0.0;
      } else if (j < k) {
        int e = ids[(size_t)t * k + j];
        gu = (mat_t){pb->dtype, pb->w_gu[e], quant ? pb->s_gu[e] : NULL, H, 2 * M};
        dn = (mat_t){pb->dtype, pb->w_d[e], quant ? pb->s_d[e] : NULL, M, H};
        total += swiglu_ffn(H, M, x + (size_t)t * H, &gu, &dn, quant, outs + (size_t)u * H, &w);
      } else {
        gu = (mat_t){pb->dtype, pb->ws_gu, pb->ss_gu, H, 2 * Ms};
        dn = (mat_t){pb->dtype, pb->ws_d, pb->ss_d, Ms, H};
        total += swiglu_ffn(H, Ms, x + (size_t)t * H, &gu, &dn, quant, outs + (size_t)u * H, &w);
      }
    }
    free(w.xa);
    free(w.a);
    free(w.h);
    free(w.row);
    free(w.hf);
  }
  if (fail) {
    free(outs);
    return AFDO_ENOMEM;
  }
  /* combine in slot order, shared expert last with gate 1 */
  for (int t = 0; t < n; ++t) {
    double* yt = y + (size_t)t * H;
    for (int c = 0; c < H; ++c) yt[c] = 0.0;
    for (int j = 0; j < k; ++j) {
      const double g = gates[(size_t)t * k + j];
      const double* o = outs + ((size_t)t * per + j) * H;
      for (int c = 0; c < H; ++c) yt[c] += g * o[c];
    }
    if (Ms > 0) {
      const double* o = outs + ((size_t)t * per + k) * H;
      for (int c = 0; c < H; ++c) yt[c] += o[c];
    }
  }
  free(outs);
  if (macs) *macs = total;
  return AFDO_OK;
}

/* Number of threads the OpenMP runtime would use. */
int afdo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
