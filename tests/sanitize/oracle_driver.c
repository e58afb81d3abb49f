/* Runs every function of the CPU oracle (oracle/afd_oracle.c) on small seeded inputs
 * in a build with AddressSanitizer and UndefinedBehaviorSanitizer, and checks the
 * invariants that do not depend on the arithmetic: a routing is a valid top-k with
 * gates summing to 1, the permutation is a bijection with consistent counts, the
 * capacity walk's lists are consistent, and layer outputs are finite and equal for
 * the same token in different positions.  Exit status 0 and "oracle driver ok" on
 * success; any sanitizer report aborts the run.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int H, M, E, k, Ms;
  int dtype;
  const void* const* w_gu;
  const void* const* w_d;
  const float* const* s_gu;
  const float* const* s_d;
  const void* ws_gu;
  const void* ws_d;
  const float* ss_gu;
  const float* ss_d;
} afdo_problem;

void afdo_router_scores(int T, int E, int H, const float* x, const float* w, const float* bias, double* scores);
void afdo_route(int T, int E, int k, const float* logits, int32_t* ids, double* gates);
void afdo_route_select_bias(int T, int E, int k, const float* scores, const float* bias, int32_t* ids,
                            double* gates);
void afdo_permute(int T, int E, int k, const int32_t* ids, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                  int32_t* pair_pos);
void afdo_route_capacity(int T, int E, int k, const int32_t* ids, const float* gates, int32_t base, int adaptive,
                         int32_t* limits, int32_t* assign, float* weight, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_token);
void afdo_quant_row_fp8(int n, const float* v, uint8_t* codes, float* scales, double* deq);
double afdo_fp8_decode(uint8_t c);
uint8_t afdo_fp8_encode(float v);
int afdo_layer(const afdo_problem* pb, int n, const float* x, const float* logits, int32_t* ids, double* gates,
               double* y, int64_t* macs, int nthreads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
static float nrand(void) { return (float)(sqrt(-2.0 * log(1.0 - urand())) * cos(6.283185307179586 * urand())); }

static int failures = 0;
#define CHECK(c, ...)                      \
  do {                                     \
    if (!(c)) {                            \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");               \
      ++failures;                          \
    }                                      \
  } while (0)

static void check_route(int T, int E, int k, const float* l, const int32_t* ids, const double* g) {
  for (int t = 0; t < T; ++t) {
    double s = 0;
    for (int j = 0; j < k; ++j) {
      const int e = ids[t * k + j];
      CHECK(e >= 0 && e < E, "id out of range");
      for (int i = 0; i < j; ++i) CHECK(ids[t * k + i] != e, "repeated expert");
      s += g[t * k + j];
    }
    CHECK(fabs(s - 1.0) < 1e-12, "gates of token %d sum to %g", t, s);
    /* every unselected logit is at most the smallest selected one */
    float lo = l[t * E + ids[t * k + k - 1]];
    for (int e = 0; e < E; ++e) {
      int sel = 0;
      for (int j = 0; j < k; ++j) sel |= ids[t * k + j] == e;
      if (!sel) CHECK(l[t * E + e] <= lo, "unselected logit above the selection");
    }
  }
}

static void routing(int T, int E, int k) {
  float* l = malloc(sizeof(float) * T * E);
  float* b = malloc(sizeof(float) * E);
  int32_t* ids = malloc(sizeof(int32_t) * T * k);
  double* g = malloc(sizeof(double) * T * k);
  for (int i = 0; i < T * E; ++i) l[i] = (float)(int)(nrand() * 2.0f); /* integer logits: many ties */
  for (int e = 0; e < E; ++e) b[e] = nrand();
  afdo_route(T, E, k, l, ids, g);
  check_route(T, E, k, l, ids, g);
  afdo_route_select_bias(T, E, k, l, b, ids, g);
  for (int t = 0; t < T; ++t) {
    double s = 0;
    for (int j = 0; j < k; ++j) s += g[t * k + j];
    CHECK(fabs(s - 1.0) < 1e-12, "select-bias gates sum");
  }
  int32_t *counts = malloc(sizeof(int32_t) * E), *offsets = malloc(sizeof(int32_t) * (E + 1));
  int32_t *sp = malloc(sizeof(int32_t) * T * k), *pp = malloc(sizeof(int32_t) * T * k);
  afdo_route(T, E, k, l, ids, g);
  afdo_permute(T, E, k, ids, counts, offsets, sp, pp);
  CHECK(offsets[0] == 0 && offsets[E] == T * k, "offsets ends");
  for (int e = 0; e < E; ++e) CHECK(offsets[e + 1] - offsets[e] == counts[e], "offsets are a scan of counts");
  for (int p = 0; p < T * k; ++p) {
    CHECK(sp[p] >= 0 && sp[p] < T * k && pp[sp[p]] == p, "pair_pos inverts sorted_pair");
  }
  /* capacity walk with a small limit, adaptive */
  int32_t *lim = malloc(sizeof(int32_t) * E), *assign = malloc(sizeof(int32_t) * T), *st = malloc(sizeof(int32_t) * T);
  float* wt = malloc(sizeof(float) * T);
  float* gf = malloc(sizeof(float) * T * k);
  for (int i = 0; i < T * k; ++i) gf[i] = (float)g[i];
  for (int e = 0; e < E; ++e) lim[e] = T / E + 1;
  for (int rep = 0; rep < 3; ++rep) {
    afdo_route_capacity(T, E, k, ids, gf, 1, 1, lim, assign, wt, counts, offsets, st);
    int kept = 0;
    for (int t = 0; t < T; ++t) {
      CHECK(assign[t] >= -1 && assign[t] < E, "assign range");
      kept += assign[t] >= 0;
    }
    CHECK(offsets[E] == kept, "kept tokens");
    for (int i = 0; i < kept; ++i) CHECK(st[i] >= 0 && st[i] < T && assign[st[i]] >= 0, "grouped tokens");
  }
  free(l); free(b); free(ids); free(g); free(counts); free(offsets); free(sp); free(pp);
  free(lim); free(assign); free(st); free(wt); free(gf);
}

static void router_scores(void) {
  const int T = 5, E = 7, H = 33;
  float *x = malloc(sizeof(float) * T * H), *w = malloc(sizeof(float) * E * H), *b = malloc(sizeof(float) * E);
  double* s = malloc(sizeof(double) * T * E);
  for (int i = 0; i < T * H; ++i) x[i] = nrand();
  for (int i = 0; i < E * H; ++i) w[i] = nrand();
  for (int e = 0; e < E; ++e) b[e] = nrand();
  afdo_router_scores(T, E, H, x, w, b, s);
  afdo_router_scores(T, E, H, x, w, NULL, s);
  for (int i = 0; i < T * E; ++i) CHECK(isfinite(s[i]), "score finite");
  free(x); free(w); free(b); free(s);
}

static void fp8_codec(void) {
  for (int c = 0; c < 256; ++c) {
    const double v = afdo_fp8_decode((uint8_t)c);
    if ((c & 0x7F) != 0x7F) CHECK(afdo_fp8_encode((float)v) == c || v == 0.0, "fp8 round trip of %d", c);
  }
  float v[384];
  for (int i = 0; i < 384; ++i) v[i] = nrand() * (i < 128 ? 1e-3f : i < 256 ? 0.0f : 300.0f);
  uint8_t codes[384];
  float scales[3];
  double deq[384];
  afdo_quant_row_fp8(384, v, codes, scales, deq);
  CHECK(scales[1] == 1.0f, "all-zero group has scale 1");
}

/* A layer of `dtype` (0 f32, 1 bf16, 2 fp8) with E experts, top-k and a shared expert
 * of Ms: run on n tokens, then on the same tokens reversed; outputs must be finite and
 * match row for row. */
static void layer(int dtype, int H, int M, int E, int k, int Ms, int n) {
  const size_t es = dtype == 0 ? 4 : dtype == 1 ? 2 : 1;
  void** wgu = calloc(E, sizeof(void*));
  void** wd = calloc(E, sizeof(void*));
  float** sgu = calloc(E, sizeof(float*));
  float** sd = calloc(E, sizeof(float*));
  for (int e = 0; e < E; ++e) {
    wgu[e] = malloc(es * H * 2 * M);
    wd[e] = malloc(es * M * H);
    for (size_t i = 0; i < (size_t)H * 2 * M * es; ++i) ((uint8_t*)wgu[e])[i] = (uint8_t)(urand() * 256);
    for (size_t i = 0; i < (size_t)M * H * es; ++i) ((uint8_t*)wd[e])[i] = (uint8_t)(urand() * 256);
    if (dtype == 0) { /* fp32: finite values only */
      for (int i = 0; i < H * 2 * M; ++i) ((float*)wgu[e])[i] = nrand() / sqrtf((float)H);
      for (int i = 0; i < M * H; ++i) ((float*)wd[e])[i] = nrand() / sqrtf((float)M);
    } else if (dtype == 1) {
      for (int i = 0; i < H * 2 * M; ++i) ((uint16_t*)wgu[e])[i] &= 0xBC7F; /* finite, |w| < 1 */
      for (int i = 0; i < M * H; ++i) ((uint16_t*)wd[e])[i] &= 0xBC7F;
    } else {
      for (int i = 0; i < H * 2 * M; ++i) ((uint8_t*)wgu[e])[i] &= 0xF7; /* never the NaN code */
      for (int i = 0; i < M * H; ++i) ((uint8_t*)wd[e])[i] &= 0xF7;
      sgu[e] = malloc(sizeof(float) * (H / 128) * (2 * M / 128));
      sd[e] = malloc(sizeof(float) * (M / 128) * (H / 128));
      for (int i = 0; i < (H / 128) * (2 * M / 128); ++i) sgu[e][i] = (float)(1e-3 * (1 + urand()));
      for (int i = 0; i < (M / 128) * (H / 128); ++i) sd[e][i] = (float)(1e-3 * (1 + urand()));
    }
  }
  void *swgu = NULL, *swd = NULL;
  float *ssgu = NULL, *ssd = NULL;
  if (Ms) {
    swgu = calloc(es * H * 2 * Ms, 1);
    swd = calloc(es * Ms * H, 1);
    if (dtype == 2) {
      ssgu = malloc(sizeof(float) * (H / 128) * (2 * Ms / 128));
      ssd = malloc(sizeof(float) * (Ms / 128) * (H / 128));
      for (int i = 0; i < (H / 128) * (2 * Ms / 128); ++i) ssgu[i] = 1.0f;
      for (int i = 0; i < (Ms / 128) * (H / 128); ++i) ssd[i] = 1.0f;
    }
  }
  afdo_problem pb = {H, M, E, k, Ms, dtype, (const void* const*)wgu, (const void* const*)wd,
                     dtype == 2 ? (const float* const*)sgu : NULL, dtype == 2 ? (const float* const*)sd : NULL,
                     swgu, swd, ssgu, ssd};
  float *x = malloc(sizeof(float) * n * H), *xr = malloc(sizeof(float) * n * H);
  float *l = malloc(sizeof(float) * n * E), *lr = malloc(sizeof(float) * n * E);
  for (int i = 0; i < n * H; ++i) x[i] = nrand();
  for (int i = 0; i < n * E; ++i) l[i] = nrand();
  for (int t = 0; t < n; ++t) {
    memcpy(xr + (size_t)(n - 1 - t) * H, x + (size_t)t * H, sizeof(float) * H);
    memcpy(lr + (size_t)(n - 1 - t) * E, l + (size_t)t * E, sizeof(float) * E);
  }
  int32_t* ids = malloc(sizeof(int32_t) * n * k);
  double *g = malloc(sizeof(double) * n * k), *y = malloc(sizeof(double) * n * H), *yr = malloc(sizeof(double) * n * H);
  int64_t macs = 0;
  CHECK(afdo_layer(&pb, n, x, l, ids, g, y, &macs, 2) == 0, "layer dtype %d", dtype);
  CHECK(macs == 3LL * n * k * H * M + 3LL * n * H * Ms, "MAC count");
  CHECK(afdo_layer(&pb, n, xr, lr, ids, g, yr, &macs, 1) == 0, "layer reversed");
  for (int t = 0; t < n; ++t)
    for (int c = 0; c < H; ++c) {
      const double a = y[(size_t)t * H + c], b = yr[(size_t)(n - 1 - t) * H + c];
      CHECK(isfinite(a) && a == b, "token order equivariance dtype %d", dtype);
    }
  /* an assignment given by the caller (logits NULL), with a dropped token */
  for (int t = 0; t < n; ++t) {
    ids[t * k] = t % 3 == 0 ? -1 : t % E;
    g[t * k] = 0.5;
    for (int j = 1; j < k; ++j) {
      ids[t * k + j] = -1;
      g[t * k + j] = 0.0;
    }
  }
  CHECK(afdo_layer(&pb, n, x, NULL, ids, g, y, &macs, 0) == 0, "layer on an assignment");
  /* invalid arguments are refused */
  afdo_problem bad = pb;
  bad.k = E + 1;
  CHECK(afdo_layer(&bad, n, x, l, ids, g, y, &macs, 0) != 0, "k > E refused");
  for (int e = 0; e < E; ++e) {
    free(wgu[e]); free(wd[e]); free(sgu[e]); free(sd[e]);
  }
  free(wgu); free(wd); free(sgu); free(sd); free(swgu); free(swd); free(ssgu); free(ssd);
  free(x); free(xr); free(l); free(lr); free(ids); free(g); free(y); free(yr);
}

int main(void) {
  routing(37, 8, 2);
  routing(50, 16, 16);
  routing(9, 1, 1);
  routing(64, 48, 3);
  router_scores();
  fp8_codec();
  layer(0, 128, 128, 4, 2, 128, 7);
  layer(1, 128, 256, 5, 3, 0, 6);
  layer(2, 256, 256, 3, 2, 128, 5);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
