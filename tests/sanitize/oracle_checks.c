/*
 * Exercises every function of the fp64 oracle (oracle/oracle.c) for the
 * AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU test suite:
 * both dtypes, SAMPLE and GREEDY, K = 0, V = 1, faulty sequences, -inf rows,
 * NULL optional outputs, probe tokens in and out of range, the shortlisted
 * head with valid and invalid cluster ids, and the KV commit's status cases.
 * Every buffer is a heap block of exactly the size the contract states, so a
 * read or write past it is an ASan report.  Prints "oracle checks ok".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_verify(const void* target, const void* draft, int dtype, const int32_t* tokens, const float* uniforms,
                  int32_t B, int32_t K, int32_t V, float temperature, int mode, int32_t* accepted_len,
                  int32_t* out_tokens, double* p_target, double* p_draft, double* accept_margin,
                  double* sample_margin, double* residual_mass, int32_t* fallbacks, const int32_t* probe_token,
                  double* probe_gap);
int oracle_row_stats(const void* x, int dtype, int32_t R, int32_t V, float temperature, double* m, double* Z);
int oracle_head(const uint16_t* h, const uint16_t* W, const int32_t* cluster_ids, int32_t B, int32_t K, int32_t d,
                int32_t V, int32_t cluster_size, int32_t n_sel, double* compact, double* absdot, double* dense);
int oracle_kv_commit(uint8_t* cache, const uint8_t* staging, const int32_t* accepted_len, int32_t* cache_len,
                     int32_t* status, int32_t P, int32_t B, int32_t K, int32_t Lmax, int64_t row_bytes);

static int failures = 0;
#define EXPECT(cond)                                                               \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform01(void) {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void* logits(int dtype, size_t n, double scale) {
  if (dtype == 0) {
    float* x = (float*)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) x[i] = (float)((uniform01() - 0.5) * scale);
    return x;
  }
  uint16_t* x = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; ++i) x[i] = to_bf16((float)((uniform01() - 0.5) * scale));
  return x;
}

static void set_ninf(void* x, int dtype, size_t i) {
  if (dtype == 0) ((float*)x)[i] = -INFINITY;
  else ((uint16_t*)x)[i] = 0xff80u;
}

static void verify_case(int dtype, int32_t B, int32_t K, int32_t V, int mode, int with_optional, int faults) {
  const size_t tn = (size_t)B * (K + 1) * V, dn = (size_t)B * K * V;
  void* t = logits(dtype, tn, 6.0);
  void* d = mode == 0 ? logits(dtype, dn > 0 ? dn : 1, 6.0) : NULL;
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * K > 0 ? B * K : 1));
  for (int32_t i = 0; i < B * K; ++i) tok[i] = (int32_t)(uniform01() * V);
  float* uni = mode == 0 ? (float*)malloc(sizeof(float) * (size_t)B * (K + 1) * 2) : NULL;
  if (uni)
    for (size_t i = 0; i < (size_t)B * (K + 1) * 2; ++i) uni[i] = (float)uniform01();
  if (faults && B >= 3) {
    if (K > 0) tok[K] = V;                                             /* sequence 1: token out of range */
    for (int32_t v = 0; v < V; ++v) set_ninf(t, dtype, (size_t)2 * (K + 1) * V + v); /* sequence 2: row 0 */
    if (uni) uni[0] = 1.0f;                                            /* sequence 0: boundary uniforms */
    if (uni) uni[2 * K + 1] = 1.0f;
  }
  if (d && V > 2)
    for (int32_t i = 0; i < B * K; ++i) set_ninf(d, dtype, (size_t)i * V + (size_t)(i % V)); /* shortlist holes */
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (K + 1));
  double *pt = NULL, *pd = NULL, *am = NULL, *sm = NULL, *rm = NULL, *pg = NULL;
  int32_t *fb = NULL, *probe = NULL;
  if (with_optional) {
    pt = (double*)malloc(sizeof(double) * (size_t)(B * K > 0 ? B * K : 1));
    pd = (double*)malloc(sizeof(double) * (size_t)(B * K > 0 ? B * K : 1));
    am = (double*)malloc(sizeof(double) * (size_t)(B * K > 0 ? B * K : 1));
    sm = (double*)malloc(sizeof(double) * (size_t)B);
    rm = (double*)malloc(sizeof(double) * (size_t)B);
    fb = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    probe = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    pg = (double*)malloc(sizeof(double) * (size_t)B);
    for (int32_t b = 0; b < B; ++b) probe[b] = (b % 4 == 3) ? V + b : (int32_t)(uniform01() * V) - (b % 5 == 4);
  }
  EXPECT(oracle_verify(t, d, dtype, K > 0 ? tok : NULL, uni, B, K, V, 0.9f, mode, acc, out, pt, pd, am, sm, rm, fb,
                       probe, pg) == 0);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = acc[b];
    EXPECT(n >= -1 && n <= K);
    if (n >= 0) {
      EXPECT(out[(size_t)b * (K + 1) + n] >= 0 && out[(size_t)b * (K + 1) + n] < V);
      for (int32_t i = n + 1; i <= K; ++i) EXPECT(out[(size_t)b * (K + 1) + i] == -1);
      if (pg && mode == 0 && probe[b] >= 0 && probe[b] < V) EXPECT(pg[b] >= 0.0 && pg[b] <= 1.0);
      if (sm && mode == 0) EXPECT(sm[b] >= 0.0 && sm[b] <= 0.5);
    } else {
      for (int32_t i = 0; i <= K; ++i) EXPECT(out[(size_t)b * (K + 1) + i] == -1);
    }
  }
  if (faults && B >= 3) {
    if (K > 0) EXPECT(acc[1] == -1);
    EXPECT(acc[2] == -1);
  }
  free(t); free(d); free(tok); free(uni); free(acc); free(out);
  free(pt); free(pd); free(am); free(sm); free(rm); free(fb); free(probe); free(pg);
}

static void row_stats_cases(void) {
  for (int dtype = 0; dtype < 2; ++dtype) {
    const int32_t R = 5, V = 37;
    void* x = logits(dtype, (size_t)R * V, 8.0);
    for (int32_t v = 0; v < V; ++v) set_ninf(x, dtype, (size_t)V + v);   /* row 1: no finite maximum */
    set_ninf(x, dtype, 3);
    double* m = (double*)malloc(sizeof(double) * R);
    double* Z = (double*)malloc(sizeof(double) * R);
    EXPECT(oracle_row_stats(x, dtype, R, V, 0.7f, m, Z) == 0);
    EXPECT(isnan(Z[1]) && isinf(m[1]));
    EXPECT(Z[0] >= 1.0 && Z[0] <= V);
    free(x); free(m); free(Z);
  }
}

static void head_cases(void) {
  const int32_t B = 3, K = 2, d = 19, cs = 7, nc = 6, V = cs * nc, n_sel = 3;
  uint16_t* h = (uint16_t*)logits(1, (size_t)B * K * d, 2.0);
  uint16_t* W = (uint16_t*)logits(1, (size_t)V * d, 0.1);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * B * n_sel);
  for (int32_t b = 0; b < B; ++b)
    for (int32_t s = 0; s < n_sel; ++s) ids[b * n_sel + s] = s * 2 + (b % 2);
  const size_t L = (size_t)n_sel * cs;
  double* comp = (double*)malloc(sizeof(double) * B * K * L);
  double* absd = (double*)malloc(sizeof(double) * B * K * L);
  double* dense = (double*)malloc(sizeof(double) * B * K * V);
  EXPECT(oracle_head(h, W, ids, B, K, d, V, cs, n_sel, comp, absd, dense) == 0);
  EXPECT(oracle_head(h, W, ids, B, K, d, V, cs, n_sel, comp, NULL, NULL) == 0);
  for (size_t i = 0; i < (size_t)B * K * L; ++i) EXPECT(fabs(comp[i]) <= absd[i]);
  ids[1] = ids[0];                                   /* not strictly ascending */
  EXPECT(oracle_head(h, W, ids, B, K, d, V, cs, n_sel, comp, absd, dense) == 1);
  ids[1] = nc;                                       /* out of range */
  EXPECT(oracle_head(h, W, ids, B, K, d, V, cs, n_sel, comp, absd, dense) == 1);
  free(h); free(W); free(ids); free(comp); free(absd); free(dense);
}

static void kv_cases(void) {
  const int32_t P = 2, B = 4, K = 3, Lmax = 6;
  const int64_t row = 10;
  uint8_t* cache = (uint8_t*)calloc((size_t)P * B * Lmax * row, 1);
  uint8_t* stg = (uint8_t*)malloc((size_t)P * B * K * row);
  for (size_t i = 0; i < (size_t)P * B * K * row; ++i) stg[i] = (uint8_t)(i * 7 + 1);
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * B);
  int32_t* len = (int32_t*)malloc(sizeof(int32_t) * B);
  int32_t* st = (int32_t*)malloc(sizeof(int32_t) * B);
  const int32_t a0[4] = {3, -1, 2, 0}, l0[4] = {3, 1, 5, 6};
  memcpy(acc, a0, sizeof a0);
  memcpy(len, l0, sizeof l0);
  EXPECT(oracle_kv_commit(cache, stg, acc, len, st, P, B, K, Lmax, row) == 0);
  EXPECT(st[0] == 0 && len[0] == 6);  /* fills the cache exactly */
  EXPECT(st[1] == 2 && len[1] == 1);  /* faulty verify */
  EXPECT(st[2] == 1 && len[2] == 5);  /* no room */
  EXPECT(st[3] == 0 && len[3] == 6);  /* nothing to commit at a full cache */
  free(cache); free(stg); free(acc); free(len); free(st);
}

int main(void) {
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int mode = 0; mode < 2; ++mode) {
      verify_case(dtype, 6, 3, 53, mode, 1, 1);
      verify_case(dtype, 6, 3, 53, mode, 0, 0);
      verify_case(dtype, 4, 0, 17, mode, 1, 1);   /* K = 0: bonus (or argmax) only */
      verify_case(dtype, 5, 2, 1, mode, 1, 0);    /* V = 1 */
      verify_case(dtype, 3, 8, 4099, mode, 1, 1);
      verify_case(dtype, 0, 3, 53, mode, 1, 0);   /* empty batch */
    }
  row_stats_cases();
  head_cases();
  kv_cases();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("oracle checks ok\n");
  return 0;
}
