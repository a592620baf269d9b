// Speculative-sampling verify kernels for gfx950.
//
// SAMPLE mode runs three or four kernels on the caller's stream.
//
//  1. stats_kernel streams target rows 0..K-1 and draft rows 0..K-1 once.
//     One wave owns one tile (8 KiB) of one row: 16-byte loads, a per-lane
//     maximum, 2^((x - max) * log2(e)/T) with v_exp_f32, and a wave reduction
//     to a (tile max, tile sum) partial.
//  2. The accept decisions: combine the sequence's partials into (max, Z) per
//     row, evaluate P_t,i(d_i) and P_d,i(d_i) in double, take every decision
//     u < min(1, P_t/P_d) and find the first rejection n (Speculative Decoding
//     lesson, nextadmin.net, "Core algorithm" steps 4-5, "Step 1").  They run
//     in the prologue of every sampling block (the sequence's first block
//     writes the outputs), which saves a launch; only when that prologue is
//     heavy (many rows or many partials per row) and large grids would repeat
//     it in many blocks does decide_kernel take them once per sequence.
//  3. sample_kernel re-reads only what the output token at n needs: its tiles
//     of target and draft row n at a rejection (residual (P_t - P_d)_+,
//     "Step 2"), or of target row K when every draft was accepted (bonus
//     token, step 6), recomputing every element as 2^((x - m) * s) from the
//     exact difference x - m and summing in double.  Small batches use one
//     tile per wave, large ones up to eight.
//  4. pick_kernel (one block per sequence) turns the tile masses into an
//     inverse-CDF choice of tile, then scans that one tile in token-id order.
//
// Kernel boundaries order the passes: partial results cross XCDs through
// the end-of-kernel cache write-back instead of per-block fences.
//
// The statistics pass is deliberately cheap (its normalisers only decide
// accept tests, and its fp32 tile sums are ample for that); the sampling pass
// recomputes the normalisers of the row pair it samples from, summing in
// double, so the inverse-CDF boundaries carry only per-element rounding.  At a
// rejection it takes the statistics pass's tile maxima as its exponent
// references, so it needs no reduction before the exponentials and both
// sampling kernels read the same references.
//
// GREEDY mode runs greedy_kernel (argmax per tile, first index on ties) and
// greedy_finalize_kernel (argmax per row and the longest prefix of drafts equal
// to those argmaxes; LLMs-from-Scratch lesson 25, "Greedy case").

#include <math.h>

#include <algorithm>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

namespace {

constexpr float kNegInf = -__builtin_inff();

struct VerifyArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  int B, K, V;
  int NT, NG;            // statistics pass: tiles (kTile ids) and blocks per row
  int NTs, NGs;          // sampling pass: tiles (kTileS ids) and blocks per row
  int TPWs;              // sampling pass: tiles per wave
  int TPWe;              // early-exit phases: statistics tiles per wave
  float s_hi;            // log2(e)/T rounded to float
  double s64;            // log2(e)/T in double
  double T;
  TileStat* part_a;      // [B][2K][NT]
  SampleRowInfo* rows;   // [B] what pick_kernel needs about the sampled row pair
  SampleTile* part_b;    // [B][NTs]
  float* gx;             // [B][2K] logits at the draft tokens (written by the statistics pass)
  int32_t* cont;         // [K][B] early exit only
  uint32_t* arrive;      // [B] finished sampling blocks per sequence (fused pick)
  int fused_pick;        // SAMPLE: the last sampling block of a sequence picks its token
  // Sparse draft rows (null cids: dense [B][K][V] draft rows).  Position i's
  // draft logits exist on the union of its nsel[i] clusters of cs ids and are
  // stored compactly, [B][K][L], in ascending token id.
  const int32_t* cids;   // [B][K][S] cluster ids per position, ascending
  int L, S, cs;
  int compact_vec;       // compact rows 16-byte aligned with L a whole number of vectors
  int nsel[kMaxK];
  int32_t* accepted_len;
  int32_t* out_tokens;
  float* p_t_out;
  float* p_d_out;
};

// accepted_len and out_tokens.  kCoherent (the fused pick): stored
// write-through at agent scope, because the first sampling block of a
// sequence writes them and its last block (possibly on another XCD, whose L2
// would otherwise write its own dirty copy back later) overwrites position n
// with the picked token.  Elsewhere one launch writes each entry once.
template <bool kCoherent = false>
__device__ __forceinline__ void put_out(int32_t* p, int32_t v) {
  if constexpr (kCoherent) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const void* base, size_t rows_before, int V) {
  return static_cast<const T*>(base) + rows_before * (size_t)V;
}

// ---------------------------------------------------------------------------
// Sparse draft rows.
// ---------------------------------------------------------------------------

// Rank of cluster c among position i's clusters of sequence b, or -1.  Binary
// search over the ascending ids; ids that are not ascending give wrong ranks
// but never an index outside the row.
__device__ __forceinline__ int sparse_rank(const VerifyArgs& a, int b, int i, int c) {
  const int32_t* ids = a.cids + ((size_t)b * a.K + i) * a.S;
  int lo = 0, hi = a.nsel[i] - 1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int v = ids[mid];
    if (v == c) return mid;
    if (v < c) lo = mid + 1;
    else hi = mid - 1;
  }
  return -1;
}

// Storage bits of the draft logits at ids v0 .. v0 + kVec - 1 of row (b, i):
// the compact entry where the id is on the shortlist, -inf elsewhere.
// Rank lookups go through `tab` (rank of every cluster of the row, in LDS)
// when the caller built one, else through sparse_rank.
constexpr int kRankTab = 4096;  // clusters an LDS rank table covers (8 KiB)

__device__ __forceinline__ int rank_of(const VerifyArgs& a, int b, int i, int c, const int16_t* tab) {
  return tab ? (int)tab[c] : sparse_rank(a, b, i, c);
}

// Fill tab (kRankTab entries of LDS) with the rank of every cluster in
// position i's shortlist of sequence b, -1 elsewhere.  Whole block; returns
// tab, or nullptr when the vocabulary has more clusters than the table holds.
__device__ __forceinline__ const int16_t* build_rank_tab(const VerifyArgs& a, int b, int i, int16_t* tab) {
  const int nc = a.V / a.cs;
  if (nc > kRankTab) return nullptr;
  for (int c = threadIdx.x; c < nc; c += kBlock) tab[c] = -1;
  __syncthreads();
  const int32_t* ids = a.cids + ((size_t)b * a.K + i) * a.S;
  for (int r = threadIdx.x; r < a.nsel[i]; r += kBlock) {
    const int c = ids[r];
    if (c >= 0 && c < nc) tab[c] = (int16_t)r;
  }
  __syncthreads();
  return tab;
}

template <typename T>
__device__ __forceinline__ void sparse_group_bits(const VerifyArgs& a, int b, int i, int v0,
                                                  uint32_t (&bits)[Elem<T>::kVec], const int16_t* tab = nullptr) {
  constexpr int V8 = Elem<T>::kVec;
  constexpr uint32_t kNinf = sizeof(T) == 2 ? 0xff80u : 0xff800000u;
  const T* crow = static_cast<const T*>(a.draft) + ((size_t)b * a.K + i) * (size_t)a.L;
  int c = v0 < a.V ? v0 / a.cs : 0, r = v0 < a.V ? rank_of(a, b, i, c, tab) : -1;
#pragma unroll
  for (int q = 0; q < V8; ++q) {
    const int v = v0 + q;
    bits[q] = kNinf;
    if (v < a.V) {
      if (v - c * a.cs >= a.cs) {  // the group crossed into the next cluster
        c = v / a.cs;
        r = rank_of(a, b, i, c, tab);
      }
      if (r >= 0) {
        const T x = crow[r * a.cs + (v - c * a.cs)];
        if constexpr (sizeof(T) == 2) bits[q] = (uint32_t)x;
        else bits[q] = __float_as_uint(x);
      }
    }
  }
}

// The lane's slice of sampling tile t of draft row (b, i) in load_raw's packed form.
template <typename T, int NL>
__device__ __forceinline__ void sparse_tile_raw(const VerifyArgs& a, int b, int i, int t, int lane, u32x4 (&raw)[NL],
                                                const int16_t* tab) {
  constexpr int V8 = Elem<T>::kVec;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    uint32_t bits[V8];
    sparse_group_bits<T>(a, b, i, t * kTileS<T> + j * (kWave * V8) + lane * V8, bits, tab);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (sizeof(T) == 2) raw[j][q] = bits[2 * q] | (bits[2 * q + 1] << 16);
      else raw[j][q] = bits[q];
    }
  }
}

// Load `first` of sampling tile t of draft row (b, i) as floats (load_tile's element order).
template <typename T>
__device__ __forceinline__ void sparse_tile_load(const VerifyArgs& a, int b, int i, int t, int lane, int first,
                                                 float (&x)[Elem<T>::kVec], const int16_t* tab) {
  constexpr int V8 = Elem<T>::kVec;
  uint32_t bits[V8];
  sparse_group_bits<T>(a, b, i, t * kTileS<T> + first * (kWave * V8) + lane * V8, bits, tab);
#pragma unroll
  for (int q = 0; q < V8; ++q) x[q] = sizeof(T) == 2 ? __uint_as_float(bits[q] << 16) : __uint_as_float(bits[q]);
}

// ---------------------------------------------------------------------------
// Row statistics.
// ---------------------------------------------------------------------------

// (tile max, tile sum) of one statistics tile.  Each exponent is one FMA,
// x*s - c with c = RN(ml*s): exact before its single rounding, like
// RN((x - ml)*s), but offset by delta = ml*s - c (exact by FMA), since
// x*s - c = (x - ml)*s + delta.  The offset is taken out once per lane, in
// the factor 2^((ml - M)*s - delta) that scales the lane sum to the tile
// maximum M.  When a lane's maximum is a wide reference (|ml*s| >= 2^26,
// where 2^delta can leave the fp32 range), every lane of the wave takes
// RN((x - ml)*s) instead, with no offset.
template <typename T>
__device__ __forceinline__ void stats_tile(const VerifyArgs& a, const float (&x)[kPerLane<T>], TileStat* out) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & (kWave - 1);
  const float ml = lane_max(x);
  const float c = ml * a.s_hi;
  const bool wide = __ballot(exp_ref_wide(ml, a.s_hi)) != 0;  // uniform over the wave
  const float delta = wide ? 0.0f : __builtin_fmaf(ml, a.s_hi, -c);
  float sl = 0.0f;
  if (ml != kNegInf) {
    if (!wide) {
#pragma unroll
      for (int e = 0; e < kPerLane<T>; ++e) sl += exp2_fast(__builtin_fmaf(x[e], a.s_hi, -c));
    } else {
#pragma unroll
      for (int e = 0; e < kPerLane<T>; ++e) sl += exp2_wide(x[e], ml, a.s_hi);
    }
  }
  const float M = wave_max(ml);
  const float scaled = ml == kNegInf ? 0.0f : sl * exp2_fast((ml - M) * a.s_hi - delta);
  const float S = wave_sum(scaled);
  if (lane == 0) *out = TileStat{M, S};
}

// Block g of the statistics pass over row r of sequence b (r < K: target row
// r, else draft row r - K): one tile per wave, all of its loads issued at
// once.  (Several tiles per wave with the next one loaded during the
// reduction measured 2-6 % slower: the extra registers cost occupancy.)
template <typename T, bool kAligned, bool kSparse = false>
__device__ __forceinline__ void stats_row_block(const VerifyArgs& a, int b, int r, int g) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int K = a.K, R = 2 * K;
  const int t = g * kWavesPerBlock + wave;
  // The drafted token of this row: the wave whose tile holds it also records
  // its logit (re-read from cache) for the accept test.
  const int d = a.tokens[(size_t)b * K + (r < K ? r : r - K)];
  if (kSparse && r >= K) {
    // Sparse draft row: the compact row of position r - K.
    const int i = r - K;
    const T* row = static_cast<const T*>(a.draft) + ((size_t)b * K + i) * (size_t)a.L;
    const int len = a.nsel[i] * a.cs;
    if (t >= a.NT) return;
    TileStat* out = a.part_a + ((size_t)b * R + r) * a.NT + t;
    if (t * kTile<T> >= len) {
      if (lane == 0) *out = TileStat{kNegInf, 0.0f};  // past the compact row
    } else {
      float x[kPerLane<T>];
      if (a.compact_vec) {
        // 16-byte loads up to len rounded up to a vector (inside the L-long
        // row), then ids past len masked
        constexpr int V8 = Elem<T>::kVec;
        load_tile<T, true, kLoads>(row, (len + V8 - 1) / V8 * V8, t, lane, x);
        if ((t + 1) * kTile<T> > len) {
#pragma unroll
          for (int e = 0; e < kPerLane<T>; ++e)
            if (t * kTile<T> + tile_offset<T>(e, lane) >= len) x[e] = kNegInf;
        }
      } else {
        load_tile<T, false, kLoads>(row, len, t, lane, x);
      }
      stats_tile<T>(a, x, out);
    }
    if (t == 0) {
      // The logit at the draft token: its cluster's rank by a wave-wide
      // comparison with the position's cluster ids (one memory round trip).
      const int c = d >= 0 && d < a.V ? d / a.cs : -1;
      const int32_t* ids = a.cids + ((size_t)b * K + i) * a.S;
      int rank = -1;
      for (int base = 0; base < a.nsel[i] && rank < 0; base += kWave) {
        const bool hit = base + lane < a.nsel[i] && c >= 0 && ids[base + lane] == c;
        const uint64_t m = __ballot(hit);
        if (m) rank = base + (int)__builtin_ctzll(m);
      }
      if (lane == 0) a.gx[(size_t)b * R + r] = rank >= 0 ? to_f32(row[rank * a.cs + (d - c * a.cs)]) : kNegInf;
    }
    return;
  }
  const T* row = r < K ? row_ptr<T>(a.target, (size_t)b * (K + 1) + r, a.V)
                       : row_ptr<T>(a.draft, (size_t)b * K + (r - K), a.V);
  if (t < a.NT) {
    float x[kPerLane<T>];
    load_tile<T, kAligned, kLoads>(row, a.V, t, lane, x);
    stats_tile<T>(a, x, a.part_a + ((size_t)b * R + r) * a.NT + t);
    if (lane == 0 && d >= t * kTile<T> && d < (t + 1) * kTile<T> && d < a.V) a.gx[(size_t)b * R + r] = to_f32(row[d]);
  }
}

// Block `blk` of the statistics pass over every row 0..K-1 of target and draft.
template <typename T, bool kAligned, bool kSparse = false>
__device__ __forceinline__ void stats_block(const VerifyArgs& a, int blk) {
  const int R = 2 * a.K;
  const int rb = blk / a.NG;
  stats_row_block<T, kAligned, kSparse>(a, rb / R, rb % R, blk % a.NG);
}

// ---------------------------------------------------------------------------
// Accept decisions of one sequence (run by every block of the sampling pass).
// Combines the statistics partials into (max, Z) per row, evaluates P_t(d_i)
// and P_d(d_i) in double and finds the first rejection n.  With `write` the
// block also writes accepted_len, the accepted tokens, the probability
// outputs and the row data pick_kernel needs.  Returns n, or -1 for a faulty
// sequence.
// ---------------------------------------------------------------------------

// Combines one row's statistics partials into (max, Z): Z = sum over tiles of
// s * 2^((m_tile - max) * log2e/T), summed in double.  One wave; q is the
// lane's tile (tile index = lane) for rows of at most 64 tiles.
__device__ __forceinline__ void combine_row(const TileStat q, const VerifyArgs& a, float& m, double& z) {
  m = wave_max(q.m);
  z = 0.0;
  if (m != kNegInf && q.m != kNegInf) z = (double)q.s * (double)exp2_fast((q.m - m) * a.s_hi);
  z = wave_sum(z);
}

// The same for a row of any length p[0 .. NT): lane l takes tiles l, l+64, ...
// For NT <= 64 the result is bit-identical to combine_row.
__device__ __forceinline__ void combine_row_any(const TileStat* p, const VerifyArgs& a, float& m, double& z) {
  const int lane = threadIdx.x & (kWave - 1);
  m = kNegInf;
  for (int t = lane; t < a.NT; t += kWave) m = fmaxf(m, p[t].m);
  m = wave_max(m);
  z = 0.0;
  if (m != kNegInf) {
    for (int t = lane; t < a.NT; t += kWave) {
      const TileStat q = p[t];
      if (q.m != kNegInf) z += (double)q.s * (double)exp2_fast((q.m - m) * a.s_hi);
    }
  }
  z = wave_sum(z);
}

// The accept test of one position (Speculative Decoding lesson, "Step 1"):
// P_t(d), P_d(d) in double from the row statistics; accept iff
// u < min(1, P_t/P_d), P_d = 0 counting as an infinite ratio.  `bad` marks a
// token outside [0, V) or a row without a finite maximum and normaliser.
__device__ __forceinline__ bool accept_test(const VerifyArgs& a, int d, double xt, double xd, float mt, float md,
                                            double zt, double zd, float u, double& pt, double& pd, bool& bad) {
  bad = d < 0 || d >= a.V || !isfinite(mt) || !isfinite(md) || !(zt > 0.0) || !isfinite(zt) || !(zd > 0.0) ||
        !isfinite(zd);
  pt = __builtin_nan("");
  pd = __builtin_nan("");
  if (bad) return false;
  pt = exp((xt - (double)mt) / a.T) / zt;
  pd = exp((xd - (double)md) / a.T) / zd;
  const double ratio = pd > 0.0 ? pt / pd : __builtin_inf();
  const double thr = ratio < 1.0 ? ratio : 1.0;
  return (double)u < thr;
}

// Decision of position j for sequence b, taken by one wave (wave 0 of every
// block that needs it, which shares the result through LDS; every block gets
// the same result).  Returns the record for the sampling pass with n = -2 if
// the sequence accepted position j and has positions left, else n = j at a
// rejection, K when every position was accepted, -1 for a fault.  (Returned
// by value and inlined, so the record stays in registers.)  The writer wave also stores the outputs that
// position j determines: P_t(d_j), P_d(d_j), cont[j][b], and at the
// sequence's end accepted_len, out_tokens (position n is left for
// pick_kernel) and rows[b].  The caller has checked that the sequence reached
// position j.
__device__ __forceinline__ SampleRowInfo ee_decide(const VerifyArgs& a, int b, int j, bool writer) {
  const int lane = threadIdx.x & (kWave - 1);
  const int K = a.K, R = 2 * K;
  const int32_t* tok = a.tokens + (size_t)b * K;
  // Every draft token is range-checked at position 0, as in the full schedule.
  bool bad_tok = false;
  if (j == 0)
    for (int q = lane; q < K; q += kWave) bad_tok |= tok[q] < 0 || tok[q] >= a.V;
  bad_tok = wave_max((int)bad_tok) != 0;
  const int d = tok[j];
  const float u = a.uniforms[((size_t)b * (K + 1) + j) * 2];
  const double xt = (double)a.gx[(size_t)b * R + j];
  const double xd = (double)a.gx[(size_t)b * R + K + j];
  const TileStat* pb = a.part_a + (size_t)b * R * a.NT;
  float mt, md;
  double zt, zd;
  if (a.NT <= kWave) {
    // loaded into values (a select between the partial and a local default by
    // address would put the default in scratch memory)
    TileStat qt{kNegInf, 0.0f}, qd{kNegInf, 0.0f};
    if (lane < a.NT) {
      qt = pb[(size_t)j * a.NT + lane];
      qd = pb[(size_t)(K + j) * a.NT + lane];
    }
    combine_row(qt, a, mt, zt);
    combine_row(qd, a, md, zd);
  } else {
    combine_row_any(pb + (size_t)j * a.NT, a, mt, zt);
    combine_row_any(pb + (size_t)(K + j) * a.NT, a, md, zd);
  }
  double pt, pd;
  bool bad;
  const bool acc = accept_test(a, d, xt, xd, mt, md, zt, zd, u, pt, pd, bad);
  bad = bad || bad_tok;
  const int n = bad ? -1 : (!acc ? j : (j == K - 1 ? K : -2));  // -2: goes on to position j + 1
  SampleRowInfo sr;
  if (n == -1) sr = SampleRowInfo{0.0f, 0.0f, 1.0, 1.0, -1};
  else if (n == K) sr = SampleRowInfo{0.0f, 0.0f, 1.0, 1.0, K};
  else sr = SampleRowInfo{mt, md, zt, zd, n};
  if (writer) {
    if (lane == 0) {
      if (a.p_t_out) a.p_t_out[(size_t)b * K + j] = bad ? __builtin_nanf("") : (float)pt;
      if (a.p_d_out) a.p_d_out[(size_t)b * K + j] = bad ? __builtin_nanf("") : (float)pd;
      a.cont[(size_t)j * a.B + b] = n == -2 ? 1 : 0;
    }
    if (n != -2) {
      for (int q = lane; q < K; q += kWave) {
        if (n < 0 || q > j) {  // not evaluated (or faulty): NaN
          if (a.p_t_out) a.p_t_out[(size_t)b * K + q] = __builtin_nanf("");
          if (a.p_d_out) a.p_d_out[(size_t)b * K + q] = __builtin_nanf("");
        }
      }
      for (int q = lane; q <= K; q += kWave)
        put_out(&a.out_tokens[(size_t)b * (K + 1) + q], (n >= 0 && q < n) ? tok[q] : -1);
      if (lane == 0) {
        put_out(&a.accepted_len[b], n);
        a.rows[b] = sr;
      }
    }
  }
  return sr;
}

// Returns the record for the sampling pass (n = -1 for a faulty sequence; by
// value and inlined, so it stays in registers).
template <bool kCoherent = false>
__device__ __forceinline__ SampleRowInfo accept_sequence(const VerifyArgs& a, int b, bool write) {
  __shared__ float sh_m[2 * kMaxK];
  __shared__ double sh_z[2 * kMaxK];
  __shared__ int sh_n;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int K = a.K, R = 2 * K;
  if (K == 0) return SampleRowInfo{0.0f, 0.0f, 1.0, 1.0, 0};
  // Loads that do not depend on each other go first: the drafted tokens,
  // their logits (recorded by the statistics pass) and the accept uniforms.
  double xt = 0.0, xd = 0.0;
  float u = 0.0f;
  int d = -1;
  if ((int)threadIdx.x < K) {
    const int i = threadIdx.x;
    d = a.tokens[(size_t)b * K + i];
    u = a.uniforms[((size_t)b * (K + 1) + i) * 2];
    // Loaded whatever the token is, so these loads do not wait for it: the
    // slot of a token outside [0, V) was not written, and the test marks such
    // a position faulty without reading it.
    xt = (double)a.gx[(size_t)b * R + i];
    xd = (double)a.gx[(size_t)b * R + K + i];
  }
  // Row (max, Z).  Wave w owns rows w, w+4, ...  When each row has at most 64
  // tiles and a wave at most kRowsPerWave rows, every partial is loaded
  // before the first reduction, so the block waits for one memory round trip.
  constexpr int kRowsPerWave = 8;
  const int rows_w = (R - wave + kWavesPerBlock - 1) / kWavesPerBlock;
  const TileStat* pb = a.part_a + (size_t)b * R * a.NT;
  if (a.NT <= kWave && rows_w <= kRowsPerWave) {
    TileStat q[kRowsPerWave];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      q[j] = TileStat{kNegInf, 0.0f};
      if (j < rows_w && lane < a.NT) q[j] = pb[(size_t)(wave + j * kWavesPerBlock) * a.NT + lane];
    }
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      if (j < rows_w) {
        float m;
        double z;
        combine_row(q[j], a, m, z);
        if (lane == 0) {
          sh_m[wave + j * kWavesPerBlock] = m;
          sh_z[wave + j * kWavesPerBlock] = z;
        }
      }
    }
  } else {
    for (int r = wave; r < R; r += kWavesPerBlock) {
      float m;
      double z;
      combine_row_any(pb + (size_t)r * a.NT, a, m, z);
      if (lane == 0) {
        sh_m[r] = m;
        sh_z[r] = z;
      }
    }
  }
  __syncthreads();

  double pt = __builtin_nan(""), pd = __builtin_nan("");
  bool acc = true, bad = false;
  if ((int)threadIdx.x < K) {
    const int i = threadIdx.x;
    acc = accept_test(a, d, xt, xd, sh_m[i], sh_m[K + i], sh_z[i], sh_z[K + i], u, pt, pd, bad);
  }
  // Positions 0..K-1 (K <= 64) are the lanes of wave 0: the first rejection
  // is the lowest lane of its ballot.
  if (wave == 0) {
    const uint64_t rej = __ballot(!acc);
    const bool any_bad = __ballot(bad) != 0;
    if (lane == 0) sh_n = any_bad ? -1 : (rej ? (int)__builtin_ctzll(rej) : K);
  }
  __syncthreads();
  const int n = sh_n;
  const SampleRowInfo info = n >= 0 && n < K ? SampleRowInfo{sh_m[n], sh_m[K + n], sh_z[n], sh_z[K + n], n}
                                             : SampleRowInfo{0.0f, 0.0f, 1.0, 1.0, n};
  if (write) {
    const int i = threadIdx.x;
    if (i < K) {
      if (a.p_t_out) a.p_t_out[(size_t)b * K + i] = n < 0 ? __builtin_nanf("") : (float)pt;
      if (a.p_d_out) a.p_d_out[(size_t)b * K + i] = n < 0 ? __builtin_nanf("") : (float)pd;
    }
    // Thread i holds draft token i; position n and the padding get -1 here,
    // pick_kernel overwrites position n with the sampled token.
    if (i <= K) put_out<kCoherent>(&a.out_tokens[(size_t)b * (K + 1) + i], (n >= 0 && i < n) ? d : -1);
    if (i == 0) {
      put_out<kCoherent>(&a.accepted_len[b], n);
      a.rows[b] = info;
    }
  }
  return info;
}

// Per-tile ratio that decides the residual's positive set: element v of a tile
// with maxima (mt, md) is in the set iff e_t * rho > e_d, i.e. P_t(v) > P_d(v)
// with the statistics-pass normalisers, where e_t, e_d are the elements'
// exp2_ref values (so the references' remainders lo enter the ratio).  Both
// sampling kernels evaluate this same function, so they agree on the set.
__device__ __forceinline__ float tile_rho(float mt, float md, const SampleRowInfo& sr, double s64, float s_hi) {
#pragma clang fp contract(off)
  if (mt == kNegInf) return 0.0f;
  if (md == kNegInf) return 1e30f;
  const double lr = ((double)mt - (double)sr.m_t - ((double)md - (double)sr.m_d)) * s64 +
                    log2(sr.za_d) - log2(sr.za_t) + ((double)exp_ref_lo(md, s_hi) - (double)exp_ref_lo(mt, s_hi));
  const double r = exp2(fmin(fmax(lr, -99.0), 99.0));
  return (float)r;
}

// 2^((x - m) * s) for a whole tile slice, as the sampling pass computes it; 0
// when m is -inf (the tile is all -inf).
template <int N>
__device__ __forceinline__ void tile_exp(const float (&x)[N], float m, const VerifyArgs& a, float (&e)[N]) {
  if (exp_ref_wide(m, a.s_hi)) {
#pragma unroll
    for (int i = 0; i < N; ++i) e[i] = exp2_wide(x[i], m, a.s_hi);
    return;
  }
  const float hi = exp_ref_hi(m, a.s_hi);
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = exp2_ref(x[i], a.s_hi, hi);
}

// Value of v in lane l (l the same in every lane of the wave).
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), __builtin_amdgcn_readfirstlane(l)));
}
__device__ __forceinline__ double lane_value(double v, int l) {
  const int i = __builtin_amdgcn_readfirstlane(l);
  return __hiloint2double(__builtin_amdgcn_readlane((int)__double2hiint(v), i),
                          __builtin_amdgcn_readlane((int)__double2loint(v), i));
}

// ---------------------------------------------------------------------------
// Sampling pass: accept decisions, then the tile sums of the sampled row(s).
//
// At a rejection the exponent reference of each sampling tile is the
// statistics pass's maximum of the (twice as long) statistics tile holding it,
// for both rows: no reduction is needed before the exponentials, and the
// positive-set ratio is one value per statistics tile.  The bonus row is not
// read by the statistics pass, so its tiles use their own maxima.
// ---------------------------------------------------------------------------

template <typename T>
constexpr int kSubTiles = kTile<T> / kTileS<T>;  // sampling tiles per statistics tile

// With the fused pick, sampling-pass tile records are written and read with
// agent-scope atomic accesses: write-through stores and loads that are
// coherent across the XCDs' separate L2 caches, so the last block of a
// sequence sees every other block's records once it has seen their arrivals.
// (A separate pick launch reads them after a kernel boundary.)
template <bool kCoherent>
__device__ __forceinline__ void put_sample_tile(SampleTile* p, const SampleTile& v) {
  if constexpr (!kCoherent) {
    *p = v;
  } else {
    const double w[6] = {v.mt, v.md, v.zt, v.zd, v.g, v.h};
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
#pragma unroll
    for (int i = 0; i < 6; ++i)
      __hip_atomic_store(q + i, __builtin_bit_cast(uint64_t, w[i]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool kCoherent>
__device__ __forceinline__ SampleTile get_sample_tile(const SampleTile* p) {
  if constexpr (!kCoherent) {
    return *p;
  } else {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    double w[6];
#pragma unroll
    for (int i = 0; i < 6; ++i)
      w[i] = __builtin_bit_cast(double, __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return SampleTile{w[0], w[1], w[2], w[3], w[4], w[5]};
  }
}

// Residual tile sums of tile t from packed slices cx (target) and cy (draft)
// with references (mt, md) and positive-set ratio rho.
// ht and hd are exp_ref_hi of the references mt and md; the sums are in units
// of 2^(x * s - h), which pick_block rescales by 2^-lo.
template <typename T, int NL, bool kCoherent>
__device__ __forceinline__ void residual_tile(const VerifyArgs& a, int b, int t, float mt, float md, float ht,
                                              float hd, float rho, const u32x4 (&cx)[NL], const u32x4 (&cy)[NL]) {
  constexpr int P = NL * Elem<T>::kVec;
  const int lane = threadIdx.x & (kWave - 1);
  double zt = 0.0, zd = 0.0, gs = 0.0, hs = 0.0;
  auto add = [&](float e, float f) {
    const double et = (double)e, ed = (double)f;
    const double in = e * rho > f ? 1.0 : 0.0;
    zt += et;
    zd += ed;
    gs = __builtin_fma(et, in, gs);
    hs = __builtin_fma(ed, in, hs);
  };
  // The references are uniform over the wave, and so is this branch.
  const bool wt = exp_ref_wide(mt, a.s_hi), wd = exp_ref_wide(md, a.s_hi);
  if (!(wt || wd)) {
#pragma unroll
    for (int i = 0; i < P; ++i)
      add(exp2_ref(raw_elem<T>(cx, i), a.s_hi, ht), exp2_ref(raw_elem<T>(cy, i), a.s_hi, hd));
  } else {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const float x = raw_elem<T>(cx, i), y = raw_elem<T>(cy, i);
      add(wt ? exp2_wide(x, mt, a.s_hi) : exp2_ref(x, a.s_hi, ht),
          wd ? exp2_wide(y, md, a.s_hi) : exp2_ref(y, a.s_hi, hd));
    }
  }
  zt = wave_sum(zt);
  zd = wave_sum(zd);
  gs = wave_sum(gs);
  hs = wave_sum(hs);
  if (lane == 0)
    put_sample_tile<kCoherent>(a.part_b + (size_t)b * a.NTs + t, SampleTile{(double)mt, (double)md, zt, zd, gs, hs});
}

// Bonus-row tile sums of tile t (target row K), referenced to the tile's own maximum.
template <typename T, int NL, bool kCoherent>
__device__ __forceinline__ void bonus_tile(const VerifyArgs& a, int b, int t, const u32x4 (&cx)[NL]) {
  constexpr int P = NL * Elem<T>::kVec;
  const int lane = threadIdx.x & (kWave - 1);
  const float mt = wave_max(raw_lane_max<T>(cx));
  double zt = 0.0;
  if (exp_ref_wide(mt, a.s_hi)) {
#pragma unroll
    for (int i = 0; i < P; ++i) zt += (double)exp2_wide(raw_elem<T>(cx, i), mt, a.s_hi);
  } else if (mt != kNegInf) {
    const float ht = exp_ref_hi(mt, a.s_hi);
#pragma unroll
    for (int i = 0; i < P; ++i) zt += (double)exp2_ref(raw_elem<T>(cx, i), a.s_hi, ht);
  }
  zt = wave_sum(zt);
  if (lane == 0)
    put_sample_tile<kCoherent>(a.part_b + (size_t)b * a.NTs + t,
                               SampleTile{(double)mt, (double)kNegInf, zt, 0.0, 0.0, 0.0});
}

// The token pick of sequence b (defined below): kFused when it runs in the
// sampling launch's last block of the sequence, which passes its own copy of
// the row record and reads the tile records with coherent loads.
template <typename T, bool kAligned, bool kSparse = false, bool kFused = false>
__device__ __forceinline__ void pick_block(const VerifyArgs& a, int b, const SampleRowInfo& sr_local);

// Block `blk` of the sampling pass.
// kFromRows: n and the row record come from the early-exit decisions
// (a.rows) instead of this block's own accept prologue.
// kDecided: decide_kernel has taken every accept decision and left the
// record in rows[b].
// kFused (small grids of the SAMPLE schedule, a.fused_pick): each block
// counts itself in arrive[b] once its tile records are written, and the last
// of the sequence's blocks picks the token.
template <typename T, bool kAligned, bool kFromRows = false, bool kSparse = false, bool kDecided = false,
          bool kFused = false>
__device__ __forceinline__ void sample_block(const VerifyArgs& a, int blk) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int K = a.K;
  const int g = blk % a.NGs;
  const int b = blk / a.NGs;
  // The exponent references of the block's statistics tiles in every row
  // that can be sampled (target rows 0..K-1, then, for dense drafts, draft
  // rows 0..K-1), loaded together with the sequence's record or decision
  // inputs, so that they cost no round trip of their own once n is known.
  // Thread j holds row j / nst, statistics tile T0 + j % nst.
  const int nst = a.TPWs * kWavesPerBlock / kSubTiles<T>;  // statistics tiles the block covers
  const int T0 = g * nst;
  const int nref = (kSparse ? 1 : 2) * K * nst;
  const bool pre = nref <= kBlock;
  float pref = kNegInf;
  if (pre && (int)threadIdx.x < nref && T0 + (int)threadIdx.x % nst < a.NT)
    pref = a.part_a[((size_t)b * 2 * K + threadIdx.x / nst) * a.NT + T0 + threadIdx.x % nst].m;
  SampleRowInfo sr;
  int n;
  if constexpr (kDecided) {
    sr = a.rows[b];
    n = K == 0 ? 0 : sr.n;
  } else if constexpr (kFromRows) {
    // Early exit: a sequence that reached position K - 1 is decided here (by
    // wave 0 of each block, which shares the record through LDS; wave 0 of
    // the first block writes the outputs); the others ended earlier and left
    // their record in rows[b].
    if (K == 0) {
      n = 0;
    } else if (K == 1 || a.cont[(size_t)(K - 2) * a.B + b] != 0) {
      __shared__ SampleRowInfo sh_sr;
      if (wave == 0) {
        sr = ee_decide(a, b, K - 1, g == 0);
        if (lane == 0) sh_sr = sr;
      }
      __syncthreads();
      sr = sh_sr;
      n = sr.n;
    } else {
      sr = a.rows[b];
      n = sr.n;
    }
  } else {
    sr = accept_sequence<kFused>(a, b, g == 0);
    n = sr.n;
  }
  if (n < 0) return;  // faulty sequence: outputs already written
  const bool resid = n < K;
  __shared__ float sh_ref[kBlock];
  if (pre) {
    sh_ref[threadIdx.x] = pref;
    __syncthreads();
  }
  const T* trow = row_ptr<T>(a.target, (size_t)b * (K + 1) + n, a.V);
  const T* drow = resid && !kSparse ? row_ptr<T>(a.draft, (size_t)b * K + n, a.V) : trow;
  constexpr int NL = kLoadsS;
  // The block covers TPWs * 4 consecutive tiles, interleaved over its waves
  // so that the four waves read neighbouring tiles at the same time.  A tile
  // stays packed in registers (about 70 VGPRs); the other waves on the SIMD
  // cover a tile's load latency.  More, smaller blocks (up to seven waves per
  // SIMD) and issuing the next tile's loads before computing the current one
  // (through LDS, no extra registers) both measured no faster.
  auto tile_of = [&](int j) { return (g * a.TPWs + j) * kWavesPerBlock + wave; };
  const int16_t* tab = nullptr;
  if constexpr (kSparse) {
    __shared__ int16_t sh_tab[kRankTab];
    if (resid) tab = build_rank_tab(a, b, n, sh_tab);  // resid is uniform over the block
  }
  if (tile_of(0) < a.NTs) {
    // Residual: lane l holds the references and the ratio of statistics tile T0 + l.
    float ref_t = kNegInf, ref_d = kNegInf, rho_l = 0.0f;
    if (resid && lane < nst && T0 + lane < a.NT) {
      const size_t R = 2 * (size_t)K;
      ref_t = pre ? sh_ref[n * nst + lane] : a.part_a[((size_t)b * R + n) * a.NT + T0 + lane].m;
      // a sparse draft row has no dense tiles: its row maximum is the reference
      if constexpr (kSparse) ref_d = sr.m_d;
      else ref_d = pre ? sh_ref[(K + n) * nst + lane] : a.part_a[((size_t)b * R + K + n) * a.NT + T0 + lane].m;
      rho_l = tile_rho(ref_t, ref_d, sr, a.s64, a.s_hi);
    }
    const float hi_t = exp_ref_hi(ref_t, a.s_hi), hi_d = exp_ref_hi(ref_d, a.s_hi);
    for (int j = 0; j < a.TPWs; ++j) {
      const int t = tile_of(j);
      if (t >= a.NTs) break;
      u32x4 cx[NL], cy[NL];
      load_raw<T, kAligned, kLoadsS>(trow, a.V, t, lane, cx);
      if (resid) {
        if constexpr (kSparse) sparse_tile_raw<T>(a, b, n, t, lane, cy, tab);
        else load_raw<T, kAligned, kLoadsS>(drow, a.V, t, lane, cy);
        const int lt = t / kSubTiles<T> - T0;
        residual_tile<T, NL, kFused>(a, b, t, lane_value(ref_t, lt), lane_value(ref_d, lt), lane_value(hi_t, lt),
                                     lane_value(hi_d, lt), lane_value(rho_l, lt), cx, cy);
      } else {
        bonus_tile<T, NL, kFused>(a, b, t, cx);
      }
    }
  }
  if constexpr (kFused) {
    {
      // This block's tile records have completed (write-through); then it
      // counts itself.  Every block of the sequence reaches this point (n is
      // the same in each), so the last arrival sees all the records.
      __shared__ int sh_last;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        sh_last = __hip_atomic_fetch_add(a.arrive + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (unsigned)(a.NGs - 1);
      __syncthreads();
      if (sh_last) pick_block<T, kAligned, kSparse, true>(a, b, sr);
    }
  }
}

// Two block-wide sums in one round of LDS traffic.
__device__ __forceinline__ void block_sum4(double& x, double& y, double& z, double& w, double* sh) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  x = wave_sum(x);
  y = wave_sum(y);
  z = wave_sum(z);
  w = wave_sum(w);
  if (lane == 0) {
    sh[wv] = x;
    sh[kWavesPerBlock + wv] = y;
    sh[2 * kWavesPerBlock + wv] = z;
    sh[3 * kWavesPerBlock + wv] = w;
  }
  __syncthreads();
  x = y = z = w = 0.0;
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) {
    x += sh[i];
    y += sh[kWavesPerBlock + i];
    z += sh[2 * kWavesPerBlock + i];
    w += sh[3 * kWavesPerBlock + i];
  }
  __syncthreads();
}

__device__ __forceinline__ void block_max2(float& x, float& y, float* sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  x = wave_max(x);
  y = wave_max(y);
  if (lane == 0) {
    sh[w] = x;
    sh[kWavesPerBlock + w] = y;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) {
    x = fmaxf(x, sh[i]);
    y = fmaxf(y, sh[kWavesPerBlock + i]);
  }
  __syncthreads();
}

__device__ __forceinline__ void block_min2(int& x, int& y, int* sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  x = wave_min(x);
  y = wave_min(y);
  if (lane == 0) {
    sh[w] = x;
    sh[kWavesPerBlock + w] = y;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) {
    x = min(x, sh[i]);
    y = min(y, sh[kWavesPerBlock + i]);
  }
  __syncthreads();
}

// One block per sequence, after sample_kernel: the inverse-CDF choice of tile
// from the tile masses, then a four-wave scan of that tile in token-id order.
// The tile sums of the sequence (one per thread for up to 256 tiles) and the
// sample uniforms are loaded together with the row record, so the block waits
// for one memory round trip before the tile choice and one for the tile.
template <typename T, bool kAligned, bool kSparse, bool kFused>
__device__ __forceinline__ void pick_block(const VerifyArgs& a, int b, const SampleRowInfo& sr_local) {
  __shared__ double sh_d[4 * kWavesPerBlock];
  __shared__ float sh_f[2 * kWavesPerBlock];
  __shared__ int sh_i[2 * kWavesPerBlock];
  __shared__ double sh_scan[kWavesPerBlock];
  __shared__ double sh_cbefore;
  constexpr double kNegInfD = -__builtin_inf();
  const int K = a.K, NT = a.NTs;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const SampleTile* P = a.part_b + (size_t)b * NT;
  const bool cached = NT <= kBlock;
  SampleTile q0{kNegInfD, kNegInfD, 0.0, 0.0, 0.0, 0.0};
  if (cached && (int)threadIdx.x < NT) q0 = get_sample_tile<kFused>(P + threadIdx.x);
  // The sample uniforms of every position, loaded before n is known (thread i
  // holds position i's).
  float ui = 0.0f;
  if ((int)threadIdx.x <= K) ui = a.uniforms[((size_t)b * (K + 1) + threadIdx.x) * 2 + 1];
  const SampleRowInfo sr = kFused ? sr_local : a.rows[b];
  const int n = K == 0 ? 0 : sr.n;
  if (n < 0) return;  // uniform over the block: every thread read the same record
  const bool resid = n < K;
  auto tile_at = [&](int tt) -> SampleTile { return cached ? q0 : get_sample_tile<kFused>(P + tt); };

  // Reference maxima: statistics-pass maxima for a residual pair, the maximum
  // over tiles for the bonus row (the statistics pass does not read row K).
  float mref_t = sr.m_t;
  // Tile weights 2^((tile reference - row reference) * s) of the target and
  // draft rows, times 2^-lo of the tile reference (the sampling pass's sums
  // are relative to RN(reference * s)).  One pass gives the rows' normalisers
  // and the residual's two positive-set masses; a thread that owns one tile
  // keeps its weights for the scan below.
  auto w_t = [&](double mt) {
    return mt == kNegInfD ? 0.0 : exp2((mt - (double)mref_t) * a.s64) * exp_ref_scale((float)mt, a.s_hi);
  };
  auto w_d = [&](double md) {
    return md == kNegInfD ? 0.0 : exp2((md - (double)sr.m_d) * a.s64) * exp_ref_scale((float)md, a.s_hi);
  };
  // The choice: P_t(v) = e_t(v) * w_t * izt and P_d(v) = e_d(v) * w_d * izd
  // within a tile (izt, izd the reciprocal row normalisers); the residual mass
  // S = sum (P_t - P_d) over the positive set, where a rejection whose
  // residual rounding left no mass samples P_t instead (fallback, total mass
  // 1); the inverse-CDF point u * S; the tile jstar holding it and the mass
  // before that tile, or, when rounding leaves the point beyond every
  // boundary (no_cross), the last tile with mass.
  double izt = 0.0, izd = 0.0, target = 0.0, cbefore = 0.0;
  int jstar = -1;
  bool fallback = false, no_cross = false, faulty = false;
  auto row_faulty = [&](double zt, double zd) {
    // a sampled row without a finite maximum and normaliser
    return !isfinite(mref_t) || !(zt > 0.0) || !isfinite(zt) || (resid && (!(zd > 0.0) || !isfinite(zd)));
  };
  if (NT <= kWave) {
    // Every tile record is in one lane of wave 0, which takes the choice with
    // wave-wide reductions and passes it on through LDS: one barrier where
    // the block-wide path below takes six.  For NT <= 64 the block-wide path
    // adds the same values in the same order (waves 1-3 only add zeros), so
    // both make the same choice.
    struct Choice {
      double izt, izd, target, cbefore;
      float mref_t;
      int jstar, flags;
    };
    __shared__ Choice sh_c;
    if (wave == 0) {
      const float u_n = n < kWave ? lane_value(ui, n) : a.uniforms[((size_t)b * (K + 1) + n) * 2 + 1];
      const bool has = lane < NT;
      if (!resid) mref_t = wave_max((float)q0.mt);  // q0.mt is -inf past NT
      double zbt = 0.0, zbd = 0.0, G = 0.0, H = 0.0, wt = 0.0, wd = 0.0;
      if (isfinite(mref_t) && has) {
        wt = w_t(q0.mt);
        wd = resid ? w_d(q0.md) : 0.0;
        zbt += q0.zt * wt;
        zbd += q0.zd * wd;
        G += q0.g * wt;
        H += q0.h * wd;
      }
      zbt = wave_sum(zbt);
      zbd = wave_sum(zbd);
      G = wave_sum(G);
      H = wave_sum(H);
      Choice c{0.0, 0.0, 0.0, 0.0, mref_t, -1, 0};
      if (row_faulty(zbt, zbd)) {
        c.flags = 1;
      } else {
        c.izt = 1.0 / zbt;
        c.izd = resid ? 1.0 / zbd : 0.0;
        double S = resid ? G * c.izt - H * c.izd : 1.0;
        const bool fb = resid && !(S > 0.0);
        if (fb) S = 1.0;
        c.target = (double)u_n * S;
        const double ms = !has ? 0.0 : (!resid || fb) ? q0.zt * wt * c.izt : q0.g * wt * c.izt - q0.h * wd * c.izd;
        const double incl = wave_inclusive_scan(ms);
        const uint64_t cross = __ballot(has && incl > c.target);
        const uint64_t mass = __ballot(has && ms > 0.0);
        if (cross) {
          c.jstar = (int)__builtin_ctzll(cross);
          c.cbefore = lane_value(incl - ms, c.jstar);
        } else {
          c.jstar = mass ? 63 - (int)__builtin_clzll(mass) : -1;
          c.flags |= 2;
        }
        if (fb) c.flags |= 4;
      }
      if (lane == 0) sh_c = c;
    }
    __syncthreads();
    const Choice c = sh_c;
    izt = c.izt;
    izd = c.izd;
    target = c.target;
    cbefore = c.cbefore;
    mref_t = c.mref_t;
    jstar = c.jstar;
    faulty = c.flags & 1;
    no_cross = c.flags & 2;
    fallback = c.flags & 4;
  } else {
    __shared__ float sh_u[kMaxK + 1];
    if ((int)threadIdx.x <= K) sh_u[threadIdx.x] = ui;  // read after the barriers below
    if (!resid) {
      float mm = kNegInf, unused = kNegInf;
      for (int tt = threadIdx.x; tt < NT; tt += kBlock) mm = fmaxf(mm, (float)tile_at(tt).mt);
      block_max2(mm, unused, sh_f);
      mref_t = mm;
    }
    double zbt = 0.0, zbd = 0.0, G = 0.0, H = 0.0, wt0 = 0.0, wd0 = 0.0;
    if (isfinite(mref_t)) {
      for (int tt = threadIdx.x; tt < NT; tt += kBlock) {
        const SampleTile q = tile_at(tt);
        const double wt = w_t(q.mt), wd = resid ? w_d(q.md) : 0.0;
        wt0 = wt;
        wd0 = wd;
        zbt += q.zt * wt;
        zbd += q.zd * wd;
        G += q.g * wt;
        H += q.h * wd;
      }
    }
    block_sum4(zbt, zbd, G, H, sh_d);
    faulty = row_faulty(zbt, zbd);
    if (!faulty) {
      izt = 1.0 / zbt;
      izd = resid ? 1.0 / zbd : 0.0;
      double S = resid ? G * izt - H * izd : 1.0;
      fallback = resid && !(S > 0.0);
      if (fallback) S = 1.0;
      auto tile_mass = [&](const SampleTile& q, double wt, double wd) -> double {
        if (!resid || fallback) return q.zt * wt * izt;
        return q.g * wt * izt - q.h * wd * izd;
      };
      target = (double)sh_u[n] * S;
      // Block scan over tiles in id order, 256 tiles per round.
      int last_mass = -1;
      double offset = 0.0;
      for (int c0 = 0; c0 < NT; c0 += kBlock) {
        const int tt = c0 + threadIdx.x;
        double ms = 0.0;
        if (tt < NT) {
          const SampleTile q = tile_at(tt);
          ms = cached ? tile_mass(q, wt0, wd0) : tile_mass(q, w_t(q.mt), resid ? w_d(q.md) : 0.0);
        }
        double incl = wave_inclusive_scan(ms);
        if (lane == kWave - 1) sh_scan[wave] = incl;
        __syncthreads();
        double before_wave = 0.0, total = 0.0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
          if (w < wave) before_wave += sh_scan[w];
          total += sh_scan[w];
        }
        incl += before_wave;
        const bool cross = tt < NT && offset + incl > target;
        // First crossing tile of this round, and its last tile with mass.
        int first = cross ? tt : 0x7fffffff;
        int neg_last = (tt < NT && ms > 0.0) ? -tt : 1;
        block_min2(first, neg_last, sh_i);  // its barriers also retire sh_scan
        if (neg_last <= 0) last_mass = -neg_last;
        if (first != 0x7fffffff) {
          if (tt == first) sh_cbefore = offset + incl - ms;
          __syncthreads();
          cbefore = sh_cbefore;
          jstar = first;
          break;
        }
        offset += total;
      }
      no_cross = jstar < 0;
      if (no_cross) jstar = last_mass;
    }
  }
  if (faulty || jstar < 0) {
    // faulty row, or a row with no mass at all
    for (int i = threadIdx.x; i <= K; i += kBlock) put_out<kFused>(&a.out_tokens[(size_t)b * (K + 1) + i], -1);
    if (threadIdx.x == 0) put_out<kFused>(&a.accepted_len[b], -1);
    return;
  }

  // Scan of tile jstar: wave w owns the tile's load w (kWave*kVec consecutive
  // ids).  The tile maxima and every element value are recomputed exactly as
  // the tile pass computed them.
  const T* trow = row_ptr<T>(a.target, (size_t)b * (K + 1) + n, a.V);
  const T* drow = resid && !kSparse ? row_ptr<T>(a.draft, (size_t)b * K + n, a.V) : nullptr;
  constexpr int V8 = Elem<T>::kVec;
  static_assert(kLoadsS == kWavesPerBlock, "one load of the tile per wave");
  const bool use_d = resid && !fallback;
  const int16_t* sh_tab = nullptr;
  if constexpr (kSparse) {
    __shared__ int16_t sh_rank[kRankTab];
    if (use_d) sh_tab = build_rank_tab(a, b, n, sh_rank);  // use_d is uniform over the block
  }
  float x[V8], y[V8], e[V8], f[V8];
  load_tile<T, kAligned, kLoadsS>(trow, a.V, jstar, lane, x, wave);
  if (use_d) {
    if constexpr (kSparse) sparse_tile_load<T>(a, b, n, jstar, lane, wave, y, sh_tab);
    else load_tile<T, kAligned, kLoadsS>(drow, a.V, jstar, lane, y, wave);
  }
  // Exponent references exactly as the sampling pass took them: the
  // statistics tile maxima for a rejected position, the tile's own maximum
  // for the bonus row.
  float mt, md = kNegInf;
  if (resid) {
    const size_t R = 2 * (size_t)K;
    const int ts = jstar / kSubTiles<T>;
    mt = a.part_a[((size_t)b * R + n) * a.NT + ts].m;
    md = kSparse ? sr.m_d : a.part_a[((size_t)b * R + K + n) * a.NT + ts].m;
  } else {
    mt = lane_max(x);
    float unused = kNegInf;
    block_max2(mt, unused, sh_f);
  }
  const double gt = w_t((double)mt) * izt;
  tile_exp(x, mt, a, e);
  double w[V8];
  if (use_d) {
    const double gd = w_d((double)md) * izd;
    tile_exp(y, md, a, f);
    const float rho = tile_rho(mt, md, sr, a.s64, a.s_hi);
#pragma unroll
    for (int k = 0; k < V8; ++k) w[k] = e[k] * rho > f[k] ? (double)e[k] * gt - (double)f[k] * gd : 0.0;
  } else {
#pragma unroll
    for (int k = 0; k < V8; ++k) w[k] = (double)e[k] * gt;
  }
  const int id0 = jstar * kTileS<T> + wave * (kWave * V8) + lane * V8;
  double cum[V8];
  double acc = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int k = 0; k < V8; ++k) {
    acc += w[k];
    cum[k] = acc;
    if (w[k] > 0.0) last_pos = id0 + k;
  }
  const double incl = wave_inclusive_scan(acc);
  if (lane == kWave - 1) sh_scan[wave] = incl;
  __syncthreads();
  double before = cbefore;
#pragma unroll
  for (int v = 0; v < kWavesPerBlock; ++v)
    if (v < wave) before += sh_scan[v];
  const double base = before + (incl - acc);
  int mine = 0x7fffffff;
  if (!no_cross) {
#pragma unroll
    for (int k = V8 - 1; k >= 0; --k)
      if (base + cum[k] > target) mine = id0 + k;
  }
  int neg_last_pos = -last_pos;
  block_min2(mine, neg_last_pos, sh_i);
  const int token = mine != 0x7fffffff ? mine : -neg_last_pos;
  if (threadIdx.x == 0) {
    put_out<kFused>(&a.out_tokens[(size_t)b * (K + 1) + n], token);
    put_out<kFused>(&a.accepted_len[b], token >= 0 ? n : -1);
    if (token < 0)
      for (int i = 0; i <= K; ++i) put_out<kFused>(&a.out_tokens[(size_t)b * (K + 1) + i], -1);
  }
}

// (Forcing six waves per SIMD here, at most 80 VGPRs, spills one register to
// scratch and measured 16 % slower than the compiler's five.)
template <typename T, bool kAligned, bool kSparse = false>
__global__ void __launch_bounds__(kBlock) stats_kernel(VerifyArgs a) {
  // The sampling launch that follows counts its finished blocks per sequence
  // from zero (the workspace holds the previous call's counts).
  if (a.fused_pick)
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < a.B; i += gridDim.x * kBlock)
      __hip_atomic_store(a.arrive + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  stats_block<T, kAligned, kSparse>(a, blockIdx.x);
}

// Every accept decision of sequence blockIdx.x and its first rejection
// (Speculative Decoding lesson, "Core algorithm" steps 4-5, "Step 1"): the
// outputs up to the first rejection, P(d) at each position, and the record
// the sampling and pick kernels read.  Used for large grids whose sampling
// prologue would be heavy (more than 16 rows or 64 partials per row); other
// shapes take the decisions in the prologue of every sampling block, which
// saves this launch.
__global__ void __launch_bounds__(kBlock) decide_kernel(VerifyArgs a) {
  (void)accept_sequence(a, blockIdx.x, true);
}

template <typename T, bool kAligned, bool kSparse = false, bool kDecided = false, bool kFused = false>
__global__ void __launch_bounds__(kBlock) sample_kernel(VerifyArgs a) {
  sample_block<T, kAligned, false, kSparse, kDecided, kFused>(a, blockIdx.x);
}

template <typename T, bool kAligned, bool kSparse = false>
__global__ void __launch_bounds__(kBlock) pick_kernel(VerifyArgs a) {
  pick_block<T, kAligned, kSparse, false>(a, blockIdx.x, SampleRowInfo{});
}

// ---------------------------------------------------------------------------
// Early-exit schedule: position i is processed only for the sequences that
// accepted every position before it, so rows after a sequence's first
// rejection are never read (they cannot change its output: Speculative
// Decoding lesson, "Core algorithm" step 5).  Phase i = statistics of target
// and draft row i, then one decision wave per sequence.  The statistics and
// decision code is the SAMPLE schedule's, so both schedules take the same
// decisions bit for bit.
// ---------------------------------------------------------------------------

// Statistics tiles per wave in the early-exit phases (a.TPWe): two when the
// phase has at least kEEBlocksForTwo blocks at one tile per wave, which halves
// the decisions taken per position (B=256, K=7, V=262144: phases 255 -> 242
// us), else one (two measured 3-16 % slower for B=8 and B=64).  Loading the
// tile before the decision, so that the two latencies overlap, measured 13 %
// slower over the phases: the tiles of sequences that reject at i - 1 are
// read for nothing.

// Phase i of the early-exit schedule: statistics of target and draft row i
// for the sequences that accepted positions 0..i-1.  For i > 0 every block
// first decides position i - 1 of its sequence (its statistics are complete:
// the previous launch produced them); block 0 of the target row writes the
// outputs of that decision.
template <typename T, bool kAligned>
__global__ void __launch_bounds__(kBlock) ee_phase_kernel(VerifyArgs a, int i) {
  const int wave = threadIdx.x / kWave;
  const int NGe = (a.NT + a.TPWe * kWavesPerBlock - 1) / (a.TPWe * kWavesPerBlock);
  const int b = blockIdx.x / (2 * NGe), rem = blockIdx.x % (2 * NGe);
  const int which = rem / NGe, g = rem % NGe;
  if (i > 0) {
    const bool writer = g == 0 && which == 0 && wave == 0;
    if (i > 1 && a.cont[(size_t)(i - 2) * a.B + b] == 0) {
      // ended earlier: carry the flag forward (the workspace holds stale
      // flags from earlier calls, so every entry a later launch reads is written)
      if (writer && threadIdx.x == 0) a.cont[(size_t)(i - 1) * a.B + b] = 0;
      return;
    }
    // Wave 0 decides for the block; the others wait for its answer.  (Every
    // wave deciding for itself measured 4 % slower over the phases.)
    __shared__ int sh_go;
    if (wave == 0) {
      const int go = ee_decide(a, b, i - 1, writer).n == -2 ? 1 : 0;
      if ((threadIdx.x & (kWave - 1)) == 0) sh_go = go;
    }
    __syncthreads();
    if (!sh_go) return;
  }
  for (int j = 0; j < a.TPWe; ++j) {
    const int t = (g * a.TPWe + j) * kWavesPerBlock + wave;
    if (t >= a.NT) break;
    stats_row_block<T, kAligned>(a, b, which == 0 ? i : a.K + i, t / kWavesPerBlock);
  }
}

template <typename T, bool kAligned>
__global__ void __launch_bounds__(kBlock) ee_sample_kernel(VerifyArgs a) {
  sample_block<T, kAligned, true>(a, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Greedy verify.
// ---------------------------------------------------------------------------

struct GreedyArgs {
  const void* target;
  const int32_t* tokens;
  int B, K, V, NT, NG;
  ArgTile* part;
  int32_t* accepted_len;
  int32_t* out_tokens;
  float* p_t_out;
  float* p_d_out;
};

__device__ __forceinline__ void argmax_merge(float& best, int& idx, float ob, int oi) {
  if (ob > best || (ob == best && oi < idx)) {
    best = ob;
    idx = oi;
  }
}

__device__ void finalize_greedy(const GreedyArgs& a, int b) {
  __shared__ int sh_arg[kMaxK + 1];
  __shared__ int sh_bad;
  const int K = a.K, R = K + 1;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (threadIdx.x == 0) sh_bad = 0;
  __syncthreads();
  // Row r's argmax over its tile records: one wave per row, lane l merging
  // records l, l + 64, ..., then a butterfly.  The merge keeps the largest
  // value and, among equal ones, the lowest id, so its order does not matter.
  for (int r = wave; r < R; r += kWavesPerBlock) {
    const ArgTile* p = a.part + ((size_t)b * R + r) * a.NT;
    float best = kNegInf;
    int idx = 0x7fffffff;
    for (int t = lane; t < a.NT; t += kWave) argmax_merge(best, idx, p[t].v, p[t].i);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(idx, o);
      argmax_merge(best, idx, ob, oi);
    }
    if (lane == 0) {
      if (!isfinite(best)) atomicOr(&sh_bad, 1);
      sh_arg[r] = idx;
    }
  }
  if ((int)threadIdx.x < K) {
    const int d = a.tokens[(size_t)b * K + threadIdx.x];
    if (d < 0 || d >= a.V) atomicOr(&sh_bad, 1);
  }
  __syncthreads();
  if (wave == 0) {
    // n = the first position whose draft differs from the argmax (K <= 64: one ballot)
    const bool bad = sh_bad != 0;
    const int d = lane < K ? a.tokens[(size_t)b * K + lane] : -1;
    const uint64_t miss = __ballot(lane < K && d != sh_arg[lane]);
    const int n = miss ? (int)__builtin_ctzll(miss) : K;
    int32_t* out = a.out_tokens + (size_t)b * R;
    for (int i = lane; i <= K; i += kWave) {
      const int di = i < K ? a.tokens[(size_t)b * K + i] : -1;
      out[i] = bad ? -1 : (i < n ? di : (i == n ? sh_arg[n] : -1));
    }
    if (lane == 0) a.accepted_len[b] = bad ? -1 : n;
  }
  for (int i = threadIdx.x; i < K; i += kBlock) {
    if (a.p_t_out) a.p_t_out[(size_t)b * K + i] = __builtin_nanf("");
    if (a.p_d_out) a.p_d_out[(size_t)b * K + i] = __builtin_nanf("");
  }
}

template <typename T, bool kAligned>
__global__ void __launch_bounds__(kBlock) greedy_kernel(GreedyArgs a) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int K = a.K, R = K + 1;
  const int g = blockIdx.x % a.NG;
  const int rb = blockIdx.x / a.NG;
  const int r = rb % R;
  const int b = rb / R;
  const T* row = row_ptr<T>(a.target, (size_t)b * R + r, a.V);
  const int t = g * kWavesPerBlock + wave;
  if (t < a.NT) {
    float x[kPerLane<T>];
    load_tile<T, kAligned, kLoads>(row, a.V, t, lane, x);
    float best = kNegInf;
    int idx = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < kPerLane<T>; ++e)
      if (x[e] > best) {
        best = x[e];
        idx = t * kTile<T> + tile_offset<T>(e, lane);
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(idx, o);
      argmax_merge(best, idx, ob, oi);
    }
    if (lane == 0) a.part[((size_t)b * R + r) * a.NT + t] = ArgTile{best, idx};
  }
}

__global__ void __launch_bounds__(kBlock) greedy_finalize_kernel(GreedyArgs a) { finalize_greedy(a, blockIdx.x); }

template <typename K1, typename K2, typename K3, typename K4, typename... Args>
hipError_t dispatch4(int dtype, bool aligned, dim3 grid, hipStream_t st, K1 k_b_a, K2 k_b_u, K3 k_f_a, K4 k_f_u,
                     Args... args) {
  if (dtype == 1) {
    if (aligned) hipLaunchKernelGGL(k_b_a, grid, dim3(kBlock), 0, st, args...);
    else hipLaunchKernelGGL(k_b_u, grid, dim3(kBlock), 0, st, args...);
  } else {
    if (aligned) hipLaunchKernelGGL(k_f_a, grid, dim3(kBlock), 0, st, args...);
    else hipLaunchKernelGGL(k_f_u, grid, dim3(kBlock), 0, st, args...);
  }
  return hipGetLastError();
}

double log2e_over(float temperature) { return 1.4426950408889634073599 / (double)temperature; }

}  // namespace

static VerifyArgs verify_args(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws) {
  VerifyArgs a{};
  a.target = io.target;
  a.draft = io.draft;
  a.tokens = io.tokens;
  a.uniforms = io.uniforms;
  a.B = s.B;
  a.K = s.K;
  a.V = s.V;
  a.NT = s.NT;
  a.NG = s.NG;
  a.NTs = s.NT_s;
  a.NGs = s.NG_s;
  a.TPWs = s.TPW_s;
  a.TPWe = s.TPW_e;
  a.s64 = log2e_over(io.temperature);
  a.s_hi = (float)a.s64;
  a.T = (double)io.temperature;
  a.part_a = ws.part_a;
  a.rows = ws.rows;
  a.part_b = ws.part_b;
  a.gx = ws.gx;
  a.cont = ws.cont;
  a.arrive = ws.arrive;
  a.fused_pick = 0;
  a.cids = io.cids;
  if (io.cids) {
    a.L = io.L;
    a.S = io.S;
    a.cs = io.cs;
    a.compact_vec = (io.L % (s.dtype == 1 ? 8 : 4) == 0) && ((uintptr_t)io.draft % 16 == 0);
    for (int i = 0; i < s.K; ++i) a.nsel[i] = io.nsel[i];
  }
  a.accepted_len = io.accepted_len;
  a.out_tokens = io.out_tokens;
  a.p_t_out = io.p_target;
  a.p_d_out = io.p_draft;
  return a;
}

template <bool kSparse>
static hipError_t sample_pipeline(const VerifyShape& s, const VerifyArgs& a, hipStream_t st, void* const* events,
                                  int n_events) {
  int k = 0;
  auto record = [&]() {
    if (events && k < n_events && events[k]) (void)hipEventRecord(static_cast<hipEvent_t>(events[k]), st);
    ++k;
  };
  hipError_t e = hipSuccess;
  if (s.K > 0) {
    record();
    e = dispatch4(s.dtype, s.aligned, dim3((unsigned)((size_t)s.B * 2 * s.K * s.NG)), st,
                  stats_kernel<uint16_t, true, kSparse>, stats_kernel<uint16_t, false, kSparse>,
                  stats_kernel<float, true, kSparse>, stats_kernel<float, false, kSparse>, a);
  }
  record();
  const dim3 sgrid((unsigned)((size_t)s.B * s.NG_s));
  if (s.decide) {
    if (e == hipSuccess) {
      hipLaunchKernelGGL(decide_kernel, dim3((unsigned)s.B), dim3(kBlock), 0, st, a);
      e = hipGetLastError();
    }
    record();
    if (e == hipSuccess)
      e = dispatch4(s.dtype, s.aligned, sgrid, st, sample_kernel<uint16_t, true, kSparse, true>,
                    sample_kernel<uint16_t, false, kSparse, true>, sample_kernel<float, true, kSparse, true>,
                    sample_kernel<float, false, kSparse, true>, a);
  } else if (e == hipSuccess && s.fused_pick) {
    e = dispatch4(s.dtype, s.aligned, sgrid, st, sample_kernel<uint16_t, true, kSparse, false, true>,
                  sample_kernel<uint16_t, false, kSparse, false, true>, sample_kernel<float, true, kSparse, false, true>,
                  sample_kernel<float, false, kSparse, false, true>, a);
  } else if (e == hipSuccess) {
    e = dispatch4(s.dtype, s.aligned, sgrid, st, sample_kernel<uint16_t, true, kSparse>,
                  sample_kernel<uint16_t, false, kSparse>, sample_kernel<float, true, kSparse>,
                  sample_kernel<float, false, kSparse>, a);
  }
  if (!s.fused_pick) {
    record();
    if (e == hipSuccess)
      e = dispatch4(s.dtype, s.aligned, dim3((unsigned)s.B), st, pick_kernel<uint16_t, true, kSparse>,
                    pick_kernel<uint16_t, false, kSparse>, pick_kernel<float, true, kSparse>,
                    pick_kernel<float, false, kSparse>, a);
  }
  record();
  return e;
}

// Three dedicated kernels.  (Splitting the batch into groups and running the
// statistics of one group in the same launch as the sampling of the previous
// one measured 0-2 % faster at best: both passes are VALU-heavy, so running
// them side by side gains little over running them back to back.)  A sparse
// draft (io.cids set) uses the same three kernels compiled for compact draft
// rows.
hipError_t launch_sample_pipeline(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                  hipStream_t st, void* const* events, int n_events) {
  if (s.B == 0) return hipSuccess;
  VerifyArgs a = verify_args(s, io, ws);
  a.fused_pick = s.fused_pick ? 1 : 0;
  return io.cids ? sample_pipeline<true>(s, a, st, events, n_events)
                 : sample_pipeline<false>(s, a, st, events, n_events);
}

hipError_t launch_early_exit_pipeline(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                      hipStream_t st, void* const* events, int n_events) {
  if (s.B == 0) return hipSuccess;
  const VerifyArgs a = verify_args(s, io, ws);
  int k = 0;
  auto record = [&]() {
    if (events && k < n_events && events[k]) (void)hipEventRecord(static_cast<hipEvent_t>(events[k]), st);
    ++k;
  };
  hipError_t e = hipSuccess;
  const int NGe = (s.NT + s.TPW_e * kWavesPerBlock - 1) / (s.TPW_e * kWavesPerBlock);
  const dim3 phase_grid((unsigned)((size_t)s.B * 2 * NGe));
  for (int i = 0; i < s.K && e == hipSuccess; ++i) {
    record();
    e = dispatch4(s.dtype, s.aligned, phase_grid, st, ee_phase_kernel<uint16_t, true>,
                  ee_phase_kernel<uint16_t, false>, ee_phase_kernel<float, true>, ee_phase_kernel<float, false>, a,
                  i);
  }
  record();
  if (e == hipSuccess)
    e = dispatch4(s.dtype, s.aligned, dim3((unsigned)((size_t)s.B * s.NG_s)), st, ee_sample_kernel<uint16_t, true>,
                  ee_sample_kernel<uint16_t, false>, ee_sample_kernel<float, true>, ee_sample_kernel<float, false>,
                  a);
  record();
  if (e == hipSuccess)
    e = dispatch4(s.dtype, s.aligned, dim3((unsigned)s.B), st, pick_kernel<uint16_t, true>,
                  pick_kernel<uint16_t, false>, pick_kernel<float, true>, pick_kernel<float, false>, a);
  record();
  return e;
}

hipError_t launch_greedy(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  GreedyArgs a{};
  a.target = io.target;
  a.tokens = io.tokens;
  a.B = s.B;
  a.K = s.K;
  a.V = s.V;
  a.NT = s.NT;
  a.NG = s.NG;
  a.part = ws.part_g;
  a.accepted_len = io.accepted_len;
  a.out_tokens = io.out_tokens;
  a.p_t_out = io.p_target;
  a.p_d_out = io.p_draft;
  const dim3 grid((unsigned)((size_t)s.B * (s.K + 1) * s.NG));
  return dispatch4(s.dtype, s.aligned, grid, st, greedy_kernel<uint16_t, true>, greedy_kernel<uint16_t, false>,
                   greedy_kernel<float, true>, greedy_kernel<float, false>, a);
}

hipError_t launch_greedy_finalize(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                  hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  GreedyArgs a{};
  a.tokens = io.tokens;
  a.B = s.B;
  a.K = s.K;
  a.V = s.V;
  a.NT = s.NT;
  a.NG = s.NG;
  a.part = ws.part_g;
  a.accepted_len = io.accepted_len;
  a.out_tokens = io.out_tokens;
  a.p_t_out = io.p_target;
  a.p_d_out = io.p_draft;
  hipLaunchKernelGGL(greedy_finalize_kernel, dim3(s.B), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
