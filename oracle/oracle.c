/*
 * oracle.c -- plain, slow fp64 reference of the speculative-sampling verify step
 * and of the shortlisted drafter head.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source, header, table or helper with the GPU code.
 *
 * Every quantity is computed in IEEE double with scalar loops in token-id order,
 * exactly as the pages state the rule, with no blocking, fusion or reordering:
 *
 *   Speculative Decoding lesson (nextadmin.net), section "Core algorithm",
 *   steps 4-6, and sections "Step 1" (accept_or_reject) and "Step 2"
 *   (residual_dist); LLMs-from-Scratch lesson 25 (aiengineeringfromscratch.com),
 *   sections "The exact rule" and "Greedy case"; RuneLab explainer
 *   (runelab.ai, "speculative decoding"), the single-position figure.
 *
 * Readings taken where the pages leave a step open (each also listed with the
 * design notes):
 *   - temperature T divides the logits of both models before the softmax
 *     (LLMs-from-Scratch lesson 25, "Build it": softmax(q_draft(state)/temperature)
 *     and the target forward with the same temperature);
 *   - one (accept, sample) uniform pair per position, passed in as data;
 *   - accept iff u < min(1, P_t(d)/P_d(d)), strict; P_d(d) = 0 counts as an
 *     infinite ratio (Speculative Decoding lesson, "Step 1");
 *   - residual w = max(0, P_t - P_d) taken elementwise against the whole draft
 *     row at the rejected position (Speculative Decoding lesson, "Step 2"; the
 *     LLMs-from-Scratch listing subtracts a scalar there, which is not the rule
 *     its own "exact rule" section states);
 *   - categorical sample by inverse CDF in token-id order: the smallest v with
 *     C_v > u*S; if rounding leaves none, the largest v with w_v > 0;
 *   - a rejection whose residual mass S is <= 0 (possible only through
 *     rounding) falls back to P_t and is counted;
 *   - greedy: argmax of the raw target logits, lowest id on ties.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_SAMPLE 0
#define OR_GREEDY 1

/* Read element v of a logits row as a double.  bf16 is the top half of an
 * IEEE binary32, so widening is exact. */
static double logit_at(const void* base, int dtype, size_t idx) {
  if (dtype == OR_F32) return (double)((const float*)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Row statistics of softmax(x/T): m = max_v x_v, Z = sum_v exp((x_v - m)/T). */
static void row_stats(const void* base, int dtype, size_t row0, int32_t V, double T,
                      double* m_out, double* Z_out) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v) {
    double x = logit_at(base, dtype, row0 + (size_t)v);
    if (x > m) m = x;
  }
  double Z = 0.0;
  if (isfinite(m)) {
    for (int32_t v = 0; v < V; ++v) {
      double x = logit_at(base, dtype, row0 + (size_t)v);
      Z += exp((x - m) / T);
    }
  } else {
    Z = NAN;
  }
  *m_out = m;
  *Z_out = Z;
}

static double prob_at(const void* base, int dtype, size_t row0, int32_t v, double m, double Z, double T) {
  return exp((logit_at(base, dtype, row0 + (size_t)v) - m) / T) / Z;
}

static int row_ok(double m, double Z) { return isfinite(m) && isfinite(Z) && Z > 0.0; }

/*
 * Verify B independent sequences.
 *   target   [B, K+1, V]   draft [B, K, V]   (dtype OR_F32 or OR_BF16, contiguous)
 *   tokens   [B, K] int32  uniforms [B, K+1, 2] float ([.,i,0] accept, [.,i,1] sample)
 * Outputs (any of the double* may be NULL):
 *   accepted_len [B]      n in [0, K], -1 for a faulty sequence
 *   out_tokens   [B, K+1] d_0..d_{n-1}, sampled token at n, then -1
 *   p_target / p_draft [B, K]  P_t,i(d_i), P_d,i(d_i)  (NaN where not defined)
 *   accept_margin [B, K]  |u_i - min(1, ratio_i)|
 *   sample_margin [B]     distance of u*S to the nearest CDF boundary of the
 *                         chosen token, divided by S
 *   residual_mass [B]     S of the sampled distribution (1 - beta for a residual)
 *   fallbacks     [B]     1 where S <= 0 forced the fallback to P_t
 * Optional probe (both NULL, or both given):
 *   probe_token   [B]     a token id per sequence (for instance another
 *                         implementation's pick at the same position n)
 *   probe_gap     [B] out the mass of the sampled distribution that lies
 *                         between u*S and that token's cumulative interval
 *                         [C_{g-1}, C_g], divided by S: 0 when u*S falls inside
 *                         it, NaN for a faulty sequence, in GREEDY mode, or for
 *                         an id outside [0, V)
 * Returns 0.
 */
int oracle_verify(const void* target, const void* draft, int dtype,
                  const int32_t* tokens, const float* uniforms,
                  int32_t B, int32_t K, int32_t V, float temperature, int mode,
                  int32_t* accepted_len, int32_t* out_tokens,
                  double* p_target, double* p_draft,
                  double* accept_margin, double* sample_margin,
                  double* residual_mass, int32_t* fallbacks,
                  const int32_t* probe_token, double* probe_gap) {
  const double T = (double)temperature;
  double* mt = (double*)malloc(sizeof(double) * (size_t)(K + 1));
  double* Zt = (double*)malloc(sizeof(double) * (size_t)(K + 1));
  double* md = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  double* Zd = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)V);

  for (int32_t b = 0; b < B; ++b) {
    const size_t trow0 = (size_t)b * (size_t)(K + 1) * (size_t)V;
    const size_t drow0 = (size_t)b * (size_t)K * (size_t)V;
    int32_t* out = out_tokens + (size_t)b * (size_t)(K + 1);
    const int32_t* d = tokens + (size_t)b * (size_t)K;
    const float* u = uniforms ? uniforms + (size_t)b * (size_t)(K + 1) * 2 : NULL; /* NULL in GREEDY mode */
    int faulty = 0;
    int32_t n = K;

    for (int32_t i = 0; i < K; ++i) {
      if (d[i] < 0 || d[i] >= V) faulty = 1;
      if (p_target) p_target[(size_t)b * K + i] = NAN;
      if (p_draft) p_draft[(size_t)b * K + i] = NAN;
      if (accept_margin) accept_margin[(size_t)b * K + i] = NAN;
    }
    if (sample_margin) sample_margin[b] = NAN;
    if (residual_mass) residual_mass[b] = NAN;
    if (probe_gap) probe_gap[b] = NAN;
    if (fallbacks) fallbacks[b] = 0;

    if (mode == OR_GREEDY) {
      /* a_i = argmax_v of the raw target logits of row i, first index on ties;
       * n = first i < K with d_i != a_i, else K; the emitted token at n is a_n
       * (LLMs-from-Scratch lesson 25, "Greedy case").  Every row 0..K is read
       * and a row without a finite maximum marks the sequence faulty. */
      int32_t a_n = -1;
      int decided = 0;
      for (int32_t i = 0; i <= K; ++i) {
        double best = -INFINITY;
        int32_t arg = -1;
        for (int32_t v = 0; v < V; ++v) {
          double x = logit_at(target, dtype, trow0 + (size_t)i * V + (size_t)v);
          if (x > best) { best = x; arg = v; }
        }
        if (!isfinite(best)) faulty = 1;
        if (!decided && (i == K || d[i] != arg)) { n = i; a_n = arg; decided = 1; }
      }
      if (faulty) {
        accepted_len[b] = -1;
        for (int32_t i = 0; i <= K; ++i) out[i] = -1;
        continue;
      }
      accepted_len[b] = n;
      for (int32_t i = 0; i < n; ++i) out[i] = d[i];
      out[n] = a_n;
      for (int32_t i = n + 1; i <= K; ++i) out[i] = -1;
      continue;
    }

    /* SAMPLE mode.  Row statistics of every target and draft row. */
    for (int32_t i = 0; i <= K; ++i) row_stats(target, dtype, trow0 + (size_t)i * V, V, T, &mt[i], &Zt[i]);
    for (int32_t i = 0; i < K; ++i) row_stats(draft, dtype, drow0 + (size_t)i * V, V, T, &md[i], &Zd[i]);
    for (int32_t i = 0; i < K; ++i)
      if (!row_ok(mt[i], Zt[i]) || !row_ok(md[i], Zd[i])) faulty = 1;

    if (!faulty) {
      /* Accept test for every draft position, left to right; n = first rejection
       * (Speculative Decoding lesson, "Core algorithm" steps 4-5; "Step 1"). */
      n = K;
      for (int32_t i = 0; i < K; ++i) {
        double pt = prob_at(target, dtype, trow0 + (size_t)i * V, d[i], mt[i], Zt[i], T);
        double pd = prob_at(draft, dtype, drow0 + (size_t)i * V, d[i], md[i], Zd[i], T);
        double ratio = pd > 0.0 ? pt / pd : INFINITY;
        double thr = ratio < 1.0 ? ratio : 1.0;
        double ui = (double)u[2 * i + 0];
        int acc = ui < thr;
        if (p_target) p_target[(size_t)b * K + i] = pt;
        if (p_draft) p_draft[(size_t)b * K + i] = pd;
        if (accept_margin) accept_margin[(size_t)b * K + i] = fabs(ui - thr);
        if (!acc && n == K) n = i;
      }
      if (n == K && !row_ok(mt[K], Zt[K])) faulty = 1;
    }
    if (faulty) {
      accepted_len[b] = -1;
      for (int32_t i = 0; i <= K; ++i) out[i] = -1;
      continue;
    }

    /* The distribution to sample: residual (P_t,n - P_d,n)_+ at a rejection
     * ("Core algorithm" step 5, "Step 2"), else P_t,K for the bonus token
     * (step 6). */
    double S = 0.0;
    const size_t tr = trow0 + (size_t)n * V;
    if (n < K) {
      const size_t dr = drow0 + (size_t)n * V;
      for (int32_t v = 0; v < V; ++v) {
        double diff = prob_at(target, dtype, tr, v, mt[n], Zt[n], T) -
                      prob_at(draft, dtype, dr, v, md[n], Zd[n], T);
        w[v] = diff > 0.0 ? diff : 0.0;
        S += w[v];
      }
      if (!(S > 0.0)) {
        if (fallbacks) fallbacks[b] = 1;
        S = 0.0;
        for (int32_t v = 0; v < V; ++v) { w[v] = prob_at(target, dtype, tr, v, mt[n], Zt[n], T); S += w[v]; }
      }
    } else {
      for (int32_t v = 0; v < V; ++v) { w[v] = prob_at(target, dtype, tr, v, mt[K], Zt[K], T); S += w[v]; }
    }

    /* Inverse CDF in token-id order with the position's sample uniform. */
    const double target_mass = (double)u[2 * n + 1] * S;
    double C = 0.0, Cprev = 0.0;
    int32_t pick = -1;
    for (int32_t v = 0; v < V; ++v) {
      Cprev = C;
      C += w[v];
      if (C > target_mass) { pick = v; break; }
    }
    double margin;
    if (pick < 0) {
      for (int32_t v = V - 1; v >= 0; --v) if (w[v] > 0.0) { pick = v; break; }
      margin = 0.0;
    } else {
      double lo = target_mass - Cprev, hi = C - target_mass;
      margin = (lo < hi ? lo : hi) / S;
    }
    if (sample_margin) sample_margin[b] = margin;
    if (residual_mass) residual_mass[b] = S;

    /* Distance of u*S from the probe token's interval [C_{g-1}, C_g], in the
     * same cumulative sums as the pick above. */
    if (probe_token && probe_gap && probe_token[b] >= 0 && probe_token[b] < V) {
      const int32_t g = probe_token[b];
      double Cg0 = 0.0;
      for (int32_t v = 0; v < g; ++v) Cg0 += w[v];
      const double Cg1 = Cg0 + w[g];
      double gap = 0.0;
      if (target_mass < Cg0) gap = Cg0 - target_mass;
      else if (target_mass > Cg1) gap = target_mass - Cg1;
      probe_gap[b] = gap / S;
    }

    accepted_len[b] = n;
    for (int32_t i = 0; i < n; ++i) out[i] = d[i];
    out[n] = pick;
    for (int32_t i = n + 1; i <= K; ++i) out[i] = -1;
  }
  free(mt); free(Zt); free(md); free(Zd); free(w);
  return 0;
}

/*
 * Row statistics only (for probability checks): m[r], Z[r] for R rows of V.
 */
int oracle_row_stats(const void* x, int dtype, int32_t R, int32_t V, float temperature,
                     double* m, double* Z) {
  for (int32_t r = 0; r < R; ++r) row_stats(x, dtype, (size_t)r * V, V, (double)temperature, &m[r], &Z[r]);
  return 0;
}

/*
 * Acceptance probability of one position: beta = sum_v min(P_t(v), P_d(v)),
 * the chance that the draft token drawn from P_d survives the accept test
 * (RuneLab explainer, the single-position figure: 42/26/16/10/6 against
 * 20/45/10/5/20 is accepted 67 % of the time; the pages print the value, and
 * the sum of the overlap is what produces it).  target and draft hold R rows
 * of V each, paired row by row; beta[r] is NaN for a row without a finite
 * maximum.
 */
int oracle_overlap(const void* target, const void* draft, int dtype, int32_t R, int32_t V, float temperature,
                   double* beta) {
  const double T = (double)temperature;
  for (int32_t r = 0; r < R; ++r) {
    const size_t row0 = (size_t)r * V;
    double mt, Zt, md, Zd;
    row_stats(target, dtype, row0, V, T, &mt, &Zt);
    row_stats(draft, dtype, row0, V, T, &md, &Zd);
    if (!row_ok(mt, Zt) || !row_ok(md, Zd)) { beta[r] = NAN; continue; }
    double s = 0.0;
    for (int32_t v = 0; v < V; ++v) {
      const double pt = prob_at(target, dtype, row0, v, mt, Zt, T);
      const double pd = prob_at(draft, dtype, row0, v, md, Zd, T);
      s += pt < pd ? pt : pd;
    }
    beta[r] = s;
  }
  return 0;
}

/*
 * Shortlisted drafter head (DynaSpec summary, lowest.today: "Model architecture",
 * items 1, 3 and 4): each context b picks n_sel clusters; its shortlist is the
 * union of those clusters, cluster c being the contiguous ids
 * [c*cluster_size, (c+1)*cluster_size).  Draft logits exist only on the
 * shortlist: logit[b,k,t] = sum_j h[b,k,j] * W[t,j].
 *   h   bf16 [B, K, d]     W bf16 [V, d] row-major     cluster_ids int32 [B, n_sel] ascending
 *   compact  [B, K, n_sel*cluster_size]  shortlist logits in ascending token id
 *   absdot   [B, K, n_sel*cluster_size]  sum_j |h*W| (scale for tolerances), may be NULL
 *   dense    [B, K, V]  logits on the shortlist, -inf elsewhere, may be NULL
 * Returns 0, or 1 if cluster ids are out of range or not strictly ascending.
 */
int oracle_head(const uint16_t* h, const uint16_t* W, const int32_t* cluster_ids,
                int32_t B, int32_t K, int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel,
                double* compact, double* absdot, double* dense) {
  const int32_t n_clusters = V / cluster_size;
  const int32_t L = n_sel * cluster_size;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t s = 0; s < n_sel; ++s) {
      int32_t c = cluster_ids[(size_t)b * n_sel + s];
      if (c < 0 || c >= n_clusters) return 1;
      if (s > 0 && c <= cluster_ids[(size_t)b * n_sel + s - 1]) return 1;
    }
  if (dense)
    for (size_t i = 0; i < (size_t)B * K * V; ++i) dense[i] = -INFINITY;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t k = 0; k < K; ++k) {
      const size_t hrow = ((size_t)b * K + k) * (size_t)d;
      for (int32_t s = 0; s < n_sel; ++s) {
        int32_t c = cluster_ids[(size_t)b * n_sel + s];
        for (int32_t t = 0; t < cluster_size; ++t) {
          int32_t tok = c * cluster_size + t;
          double acc = 0.0, aacc = 0.0;
          for (int32_t j = 0; j < d; ++j) {
            double hv = logit_at(h, OR_BF16, hrow + (size_t)j);
            double wv = logit_at(W, OR_BF16, (size_t)tok * d + (size_t)j);
            acc += hv * wv;
            aacc += fabs(hv * wv);
          }
          size_t o = ((size_t)b * K + k) * (size_t)L + (size_t)s * cluster_size + (size_t)t;
          compact[o] = acc;
          if (absdot) absdot[o] = aacc;
          if (dense) dense[((size_t)b * K + k) * (size_t)V + (size_t)tok] = acc;
        }
      }
    }
  return 0;
}

/*
 * KV-cache commit after a verify step (Speculative Decoding lesson,
 * nextadmin.net, section on KV-cache management and exercise 4): the
 * verifier's forward over K drafts produced one KV entry per draft position;
 * after verification the cache must hold only the accepted prefix.  The new
 * entries sit in a staging buffer and the accepted ones are committed.
 *   cache      [P][B][Lmax][row_bytes]  P planes (for instance layers x {K, V})
 *   staging    [P][B][K][row_bytes]     entries of draft positions 0..K-1
 *   accepted_len [B]  n: staging entries 0..n-1 go to cache positions
 *                     cache_len[b] .. cache_len[b]+n-1
 *   cache_len  [B] in/out: advanced by n where the commit happens
 *   status     [B] out: 0 committed, 1 no room (cache_len + n > Lmax),
 *                       2 n outside [0, K] (e.g. -1 from a faulty verify);
 *                       nothing is committed unless the status is 0
 * Plain byte copies, one entry at a time.  Returns 0.
 */
int oracle_kv_commit(uint8_t* cache, const uint8_t* staging, const int32_t* accepted_len,
                     int32_t* cache_len, int32_t* status, int32_t P, int32_t B, int32_t K,
                     int32_t Lmax, int64_t row_bytes) {
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = accepted_len[b];
    const int32_t len = cache_len[b];
    if (n < 0 || n > K) { status[b] = 2; continue; }
    if (len < 0 || len > Lmax - n) { status[b] = 1; continue; }
    for (int32_t p = 0; p < P; ++p)
      for (int32_t j = 0; j < n; ++j) {
        const uint8_t* src = staging + (((size_t)p * B + b) * (size_t)K + (size_t)j) * (size_t)row_bytes;
        uint8_t* dst = cache + (((size_t)p * B + b) * (size_t)Lmax + (size_t)(len + j)) * (size_t)row_bytes;
        for (int64_t q = 0; q < row_bytes; ++q) dst[q] = src[q];
      }
    cache_len[b] = len + n;
    status[b] = 0;
  }
  return 0;
}
