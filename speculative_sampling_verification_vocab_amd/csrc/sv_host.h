// Host half of libspecverify: launch geometry, workspace layout and the
// argument checks of every entry point.  Plain C++ with no HIP types, so the
// same source also builds with g++ for the AddressSanitizer / UBSan run of the
// host checks.  The kernels and launches (sv_*.hip) include it through
// sv_internal.h / sv_common.h.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"

namespace sv {

// ---- geometry shared by host and device code ----------------------------------

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kLoads = 8;   // 16-byte loads per lane per tile of the streaming passes
constexpr int kLoadsS = 4;  // 16-byte loads per lane per tile of the sampling pass
constexpr int kMaxK = SPEC_MAX_K;

// elements per 16-byte vector, per streaming tile (one wave) and per sampling tile
constexpr int vec_elems(int elem_bytes) { return 16 / elem_bytes; }
constexpr int stat_tile_elems(int elem_bytes) { return kWave * vec_elems(elem_bytes) * kLoads; }
constexpr int sample_tile_elems(int elem_bytes) { return kWave * vec_elems(elem_bytes) * kLoadsS; }

// Sampling tiles per wave: several amortise the per-block accept prologue
// over more work; small batches take fewer so the grid still fills the chip.
constexpr int kMaxTilesPerWaveS = 8;
constexpr int kSampleBlocksWanted = 1024;  // 4 per CU
constexpr int kEEBlocksForTwo = 4096;      // early-exit phase blocks at one tile per wave from which waves take two
constexpr long long kFusedPickMaxBlocks = 512;  // sampling grids up to this size pick in their last block
constexpr int kHeadMaxCtx = 1024;          // contexts the shortlist head lists per cluster
constexpr size_t kMaxGrid = 0x7fffffffu;

// ---- records the verify kernels exchange through the workspace -----------------

// Per-tile partial of the row-statistics pass: tile max and sum of 2^((x-max)*s).
struct TileStat {
  float m;
  float s;
};

// Per-tile partial of the sampling pass (see sample_kernel).
struct SampleTile {
  double mt, md;   // tile maxima of the target / draft row (as double)
  double zt, zd;   // sums of 2^((x - tile max) * s) over the tile (fp64)
  double g, h;     // the same sums restricted to the residual's positive set
};

// What the token pick needs about a sequence's sampled position n (written by
// the sampling pass): statistics-pass maxima and normalisers of target and
// draft row n (residual), and n itself (-1 for a faulty sequence).
struct SampleRowInfo {
  float m_t, m_d;
  double za_t, za_d;
  int n;
};

struct ArgTile {
  float v;
  int i;
};

struct VerifyShape {
  int B, K, V;
  int dtype;     // 0 f32, 1 bf16
  bool aligned;  // 16-byte aligned rows and V % (16 / sizeof(elem)) == 0
  int tile;      // elements per tile (one wave)
  int NT;        // tiles per row
  int NG;        // blocks (4 tiles each) per row
  int NT_s;      // sampling-pass tiles per row
  int NG_s;      // sampling-pass blocks per row
  int TPW_s;     // sampling-pass tiles per wave
  int TPW_e;     // early-exit phases: statistics tiles per wave
  bool decide;   // SAMPLE: a separate decision launch before the sampling pass
  bool fused_pick;  // SAMPLE: the last sampling block of each sequence picks its token (K > 0)
};

struct VerifyWorkspace {
  TileStat* part_a;     // [B][2K][NT]
  SampleRowInfo* rows;  // [B]
  SampleTile* part_b;   // [B][NT_s]
  ArgTile* part_g;      // [B][K+1][NT]
  float* gx;            // [B][2K] logits at the draft tokens: target rows 0..K-1, then draft rows
  int32_t* cont;        // [K][B] early exit: 1 if the sequence accepted positions 0..j and goes on
  uint32_t* arrive;     // [B] SAMPLE: sampling blocks of the sequence that have finished (zeroed by the statistics pass)
};

struct VerifyIO {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  float temperature;
  int32_t* accepted_len;
  int32_t* out_tokens;
  float* p_target;
  float* p_draft;
  // sparse draft (null cids: dense draft rows)
  const int32_t* cids;  // [B][K][S]
  int L, S, cs;
  const int32_t* nsel;  // host [K]
};

inline int tile_elems(int dtype) { return stat_tile_elems(dtype == 1 ? 2 : 4); }

inline VerifyShape make_shape(int B, int K, int V, int dtype, bool aligned) {
  VerifyShape s;
  s.B = B;
  s.K = K;
  s.V = V;
  s.dtype = dtype;
  s.aligned = aligned;
  s.tile = tile_elems(dtype);
  s.NT = (V + s.tile - 1) / s.tile;
  s.NG = (s.NT + kWavesPerBlock - 1) / kWavesPerBlock;
  const int tile_s = sample_tile_elems(dtype == 1 ? 2 : 4);
  s.NT_s = (V + tile_s - 1) / tile_s;
  s.TPW_s = 1;
  for (int tpw = kMaxTilesPerWaveS; tpw > 1; tpw /= 2) {
    const long long blocks = (long long)B * ((s.NT_s + tpw * kWavesPerBlock - 1) / (tpw * kWavesPerBlock));
    if (blocks >= kSampleBlocksWanted) {
      s.TPW_s = tpw;
      break;
    }
  }
  s.NG_s = (s.NT_s + s.TPW_s * kWavesPerBlock - 1) / (s.TPW_s * kWavesPerBlock);
  s.TPW_e = (long long)B * 2 * s.NG >= kEEBlocksForTwo ? 2 : 1;
  // Every sampling block takes its sequence's accept decisions in its
  // prologue, unless that prologue is heavy (more than 16 rows, four per
  // wave, or more than 64 partials per row) in a grid of blocks that cover
  // several sampling tiles: then a separate launch takes them once per
  // sequence.  (B=256, K=7, V=262144: 346.6 -> 345.5 us without that launch;
  // B=8, K=5, V=128256: 21.8 -> 24.5 us with it.)
  s.decide = s.TPW_s > 1 && (2 * K > 4 * kWavesPerBlock || s.NT > kWave);
  // Small sampling grids pick the token in their last block per sequence
  // instead of a launch of their own (B=1, K=4, V=32000: 20 -> 14 us; B=8,
  // K=5, V=128256: 19.5 -> 18 us).  A statistics launch precedes them to
  // clear the arrival counters.  Large grids keep the separate pick: there the
  // arrival round trip and the pick's registers in every sampling block cost
  // more than the launch (B=256, K=7, V=262144: 66 -> 71 us).
  s.fused_pick = K > 0 && !s.decide && (long long)B * s.NG_s <= kFusedPickMaxBlocks;
  return s;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bytes of the verify workspace for shape s in `mode` (spec_mode_t value), and,
// with base and out set, the offsets of its parts inside base.
inline size_t verify_workspace_layout(const VerifyShape& s, int mode, void* base, VerifyWorkspace* out) {
  const size_t B = (size_t)s.B, K = (size_t)s.K;
  const bool greedy = mode == 1, early = mode == 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  size_t o_pa = 0, o_rows = 0, o_pb = 0, o_pg = 0, o_gx = 0, o_cont = 0, o_arr = 0;
  if (greedy) {
    o_pg = take(B * (K + 1) * (size_t)s.NT * sizeof(ArgTile));
  } else {
    o_pa = take(B * 2 * K * (size_t)s.NT * sizeof(TileStat));
    o_rows = take(B * sizeof(SampleRowInfo));
    o_pb = take(B * (size_t)s.NT_s * sizeof(SampleTile));
    o_gx = take(B * 2 * (K > 0 ? K : 1) * sizeof(float));
    if (early) o_cont = take(B * (K > 0 ? K : 1) * sizeof(int32_t));
    else o_arr = take(B * sizeof(uint32_t));
  }
  if (out && base) {
    VerifyWorkspace w{};
    char* p = static_cast<char*>(base);
    if (greedy) {
      w.part_g = reinterpret_cast<ArgTile*>(p + o_pg);
    } else {
      w.part_a = reinterpret_cast<TileStat*>(p + o_pa);
      w.rows = reinterpret_cast<SampleRowInfo*>(p + o_rows);
      w.part_b = reinterpret_cast<SampleTile*>(p + o_pb);
      w.gx = reinterpret_cast<float*>(p + o_gx);
      if (early) w.cont = reinterpret_cast<int32_t*>(p + o_cont);
      else w.arrive = reinterpret_cast<uint32_t*>(p + o_arr);
    }
    *out = w;
  }
  return off;
}

// statistics (K > 0), decisions (large batches), sampling, and the pick when
// it is not fused into the sampling launch
inline int sample_launches(const VerifyShape& s) {
  return s.B == 0 ? 0 : (s.K > 0 ? 1 : 0) + (s.decide ? 1 : 0) + 1 + (s.fused_pick ? 0 : 1);
}
inline int early_exit_launches(const VerifyShape& s) { return s.B == 0 ? 0 : s.K + 2; }

// ---- argument checks ------------------------------------------------------------

inline bool valid_dtype(spec_dtype_t d) { return d == SPEC_F32 || d == SPEC_BF16; }
inline bool valid_mode(spec_mode_t m) {
  return m == SPEC_MODE_SAMPLE || m == SPEC_MODE_GREEDY || m == SPEC_MODE_SAMPLE_EARLY_EXIT;
}
inline bool sampling(spec_mode_t m) { return m == SPEC_MODE_SAMPLE || m == SPEC_MODE_SAMPLE_EARLY_EXIT; }
inline size_t elem_size(spec_dtype_t d) { return d == SPEC_BF16 ? 2 : 4; }

// Shape checks shared by the sizing functions and the verify entry points.
inline spec_status_t check_shape(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, spec_mode_t mode) {
  if (!valid_dtype(dtype) || !valid_mode(mode)) return SPEC_ERR_INVALID_ARG;
  if (B < 0 || K < 0 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (K > SPEC_MAX_K) return SPEC_ERR_UNSUPPORTED;
  if (V > (1 << 30)) return SPEC_ERR_UNSUPPORTED;  // token ids and tile offsets stay in int32
  // element counts must fit size_t with room for byte offsets
  const size_t rows = (size_t)B * (size_t)(K + 1);
  if ((size_t)B != 0 && rows / (size_t)B != (size_t)(K + 1)) return SPEC_ERR_INVALID_ARG;
  if (rows != 0 && (size_t)V > SIZE_MAX / 8 / rows) return SPEC_ERR_INVALID_ARG;
  const VerifyShape s = make_shape(B, K, V, dtype == SPEC_BF16 ? 1 : 0, false);
  const size_t per_seq_rows = mode == SPEC_MODE_GREEDY ? (size_t)(K + 1) : (size_t)(2 * K);
  if ((size_t)B * per_seq_rows * (size_t)s.NG > kMaxGrid) return SPEC_ERR_UNSUPPORTED;
  if ((size_t)B * (2 * (size_t)K * s.NG + s.NG_s + 1) > kMaxGrid) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

// Everything spec_verify and spec_verify_sparse_draft check before a launch.
// On SPEC_OK, *shape and *need hold the launch shape and the workspace bytes;
// *empty is set when there is nothing to launch (B == 0).
inline spec_status_t validate_verify(const void* target_logits, const void* draft_logits,
                                     const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                                     int32_t V, spec_dtype_t dtype, float temperature, spec_mode_t mode,
                                     const int32_t* accepted_len, const int32_t* out_tokens, const void* workspace,
                                     size_t workspace_bytes, bool sparse_draft, VerifyShape* shape, size_t* need,
                                     bool* empty) {
  const spec_status_t sc = check_shape(B, K, V, dtype, mode);
  if (sc != SPEC_OK) return sc;
  const bool sample = sampling(mode);
  if (sample && !(temperature > 0.0f && isfinite(temperature))) return SPEC_ERR_INVALID_ARG;
  *empty = B == 0;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !accepted_len || !out_tokens) return SPEC_ERR_INVALID_ARG;
  if (K > 0 && !draft_tokens) return SPEC_ERR_INVALID_ARG;
  if (sample && K > 0 && !draft_logits) return SPEC_ERR_INVALID_ARG;
  if (sample && !uniforms) return SPEC_ERR_INVALID_ARG;
  const size_t vec = (size_t)vec_elems((int)elem_size(dtype));
  bool aligned = ((size_t)V % vec == 0) && ((uintptr_t)target_logits % 16 == 0);
  if (sample && K > 0 && !sparse_draft) aligned = aligned && ((uintptr_t)draft_logits % 16 == 0);
  *shape = make_shape(B, K, V, dtype == SPEC_BF16 ? 1 : 0, aligned);
  *need = verify_workspace_layout(*shape, (int)mode, nullptr, nullptr);
  if (!workspace || workspace_bytes < *need || ((uintptr_t)workspace % 256) != 0) return SPEC_ERR_WORKSPACE;
  return SPEC_OK;
}

// The sparse-draft arguments of spec_verify_sparse_draft (n_sel is host memory, K entries).
inline spec_status_t validate_sparse_draft(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                           const int32_t* cluster_ids, const int32_t* n_sel, int32_t L, int32_t S,
                                           int32_t cluster_size) {
  const spec_status_t sc = check_shape(B, K, V, dtype, SPEC_MODE_SAMPLE);
  if (sc != SPEC_OK) return sc;
  if (B > 0 && K > 0) {
    if (!cluster_ids || !n_sel || cluster_size < 1 || L < 1 || S < 1) return SPEC_ERR_INVALID_ARG;
    if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
    if (S > V / cluster_size) return SPEC_ERR_INVALID_ARG;
    if ((size_t)B * (size_t)K * (size_t)L > SIZE_MAX / 8 || (size_t)B * (size_t)K * (size_t)S > SIZE_MAX / 8)
      return SPEC_ERR_INVALID_ARG;
    for (int i = 0; i < K; ++i) {
      if (n_sel[i] < 1 || n_sel[i] > S) return SPEC_ERR_INVALID_ARG;
      const long long len = (long long)n_sel[i] * cluster_size;
      if (len > L || len > V) return SPEC_ERR_INVALID_ARG;
    }
  }
  return SPEC_OK;
}

// spec_draft_head_shortlist; *empty when there is nothing to launch.
inline spec_status_t validate_head_shortlist(const void* h, const void* W, const int32_t* cluster_ids, int32_t B,
                                             int32_t K, int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel,
                                             const float* logits_compact, const void* dense_out,
                                             spec_dtype_t dense_dtype, bool* empty) {
  if (B < 0 || K < 0 || d < 1 || V < 1 || cluster_size < 1 || n_sel < 0) return SPEC_ERR_INVALID_ARG;
  if (!valid_dtype(dense_dtype)) return SPEC_ERR_INVALID_ARG;
  if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
  if (n_sel > V / cluster_size) return SPEC_ERR_INVALID_ARG;
  *empty = B == 0 || K == 0;
  if (*empty) return SPEC_OK;
  if (B > kHeadMaxCtx || n_sel > 0xffff) return SPEC_ERR_UNSUPPORTED;
  if ((size_t)B * (size_t)n_sel > 0x7fffffffu || (size_t)B * K * (size_t)V > SIZE_MAX / 8) return SPEC_ERR_INVALID_ARG;
  if (!h || !W || (!cluster_ids && n_sel > 0) || (!logits_compact && !dense_out)) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

// spec_draft_head_positions (n_sel is host memory, K entries).
inline spec_status_t validate_head_positions(const void* h, const void* W, const int32_t* cluster_ids,
                                             const int32_t* n_sel, int32_t B, int32_t K, int32_t d, int32_t V,
                                             int32_t cluster_size, int32_t S, int32_t L, const void* logits_compact,
                                             spec_dtype_t compact_dtype, bool* empty) {
  if (B < 0 || K < 0 || d < 1 || V < 1 || cluster_size < 1 || S < 1 || L < 1) return SPEC_ERR_INVALID_ARG;
  if (!valid_dtype(compact_dtype)) return SPEC_ERR_INVALID_ARG;
  if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
  *empty = B == 0 || K == 0;
  if (*empty) return SPEC_OK;
  if (K > SPEC_MAX_K || (size_t)B * K > (size_t)kHeadMaxCtx || S > 0xffff) return SPEC_ERR_UNSUPPORTED;
  if (S > V / cluster_size || (size_t)B * K * (size_t)S > 0x7fffffffu || (size_t)B * K * (size_t)L > SIZE_MAX / 8)
    return SPEC_ERR_INVALID_ARG;
  if (!h || !W || !cluster_ids || !n_sel || !logits_compact) return SPEC_ERR_INVALID_ARG;
  for (int i = 0; i < K; ++i)
    if (n_sel[i] < 0 || n_sel[i] > S || (long long)n_sel[i] * cluster_size > L) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

// Launch plan of spec_draft_head_static.  Rows of d % 64 == 0 dims with
// 16-byte alignment take the LDS-DMA kernel: 128 x 128 output tiles when the
// shortlist gives at least kStaticWideTiles of them (M = 128: N >= 24577),
// else, with a workspace, 128 x 128 tiles whose K stages are split over
// ksplit blocks (fp32 partial tiles in the workspace, added in a fixed order
// by a second launch), or, without one, 64 x 32 tiles over the whole K.
// Other shapes take the register-staged kernel (no split).
constexpr long long kStaticWideTiles = 192;
constexpr int kStaticMaxSplit = 8;

inline int head_static_split(int32_t M, int32_t d, int32_t N) {
  if (M < 1 || N < 1 || d % 64 != 0) return 1;
  const long long t128 = (long long)((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= kStaticWideTiles) return 1;
  // about one block per CU (256): 63 tiles at M = 128, N = 8016 take 4 slices
  long long s = (256 + t128 / 2) / t128;
  const long long stages = d / 64;
  if (s > kStaticMaxSplit) s = kStaticMaxSplit;
  if (s > stages / 4) s = stages / 4;  // at least four stages per slice
  return s < 1 ? 1 : (int)s;
}

// Workspace bytes that let spec_draft_head_static split K (0: no split).
inline size_t head_static_workspace_bytes(int32_t M, int32_t d, int32_t N) {
  const int s = head_static_split(M, d, N);
  return s > 1 ? align256((size_t)s * (size_t)M * (size_t)N * sizeof(float)) : 0;
}

// spec_draft_head_static.
inline spec_status_t validate_head_static(const void* h, const void* W, const int32_t* cluster_ids, int32_t M,
                                          int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel,
                                          const void* logits, spec_dtype_t out_dtype, const void* workspace,
                                          size_t workspace_bytes, bool* empty) {
  if (M < 0 || d < 1 || V < 1 || cluster_size < 1 || n_sel < 0) return SPEC_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return SPEC_ERR_INVALID_ARG;
  if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
  if (n_sel > V / cluster_size) return SPEC_ERR_INVALID_ARG;
  *empty = M == 0 || n_sel == 0;
  if (*empty) return SPEC_OK;
  if (!h || !W || !cluster_ids || !logits) return SPEC_ERR_INVALID_ARG;
  if ((uintptr_t)h % 2 || (uintptr_t)W % 2 || (uintptr_t)cluster_ids % 4 ||
      (uintptr_t)logits % elem_size(out_dtype))
    return SPEC_ERR_INVALID_ARG;
  const size_t N = (size_t)n_sel * (size_t)cluster_size;
  if ((size_t)M * N > SIZE_MAX / 8 || (size_t)M * (size_t)d > SIZE_MAX / 8) return SPEC_ERR_INVALID_ARG;
  if (((N + 31) / 32) * (((size_t)M + 127) / 128) > 0x7fffffffu) return SPEC_ERR_UNSUPPORTED;  // 1-D grid of tiles
  if (workspace && ((uintptr_t)workspace % 256 != 0 ||
                    workspace_bytes < head_static_workspace_bytes(M, d, (int32_t)N)))
    return SPEC_ERR_WORKSPACE;
  return SPEC_OK;
}

// How spec_kv_commit copies: planes with work, vector or element units.
struct KvPlan {
  bool copies;  // P > 0, K > 0 and E > 0
  bool vec;     // 16-byte units
  size_t row;   // bytes per entry
};

// spec_kv_commit; *empty when there is nothing to launch.
inline spec_status_t validate_kv_commit(const void* cache, const void* staging, const int32_t* accepted_len,
                                        const int32_t* cache_len, int32_t P, int32_t B, int32_t K, int32_t L_max,
                                        int32_t E, spec_dtype_t dtype, KvPlan* plan, bool* empty) {
  if (!valid_dtype(dtype)) return SPEC_ERR_INVALID_ARG;
  if (P < 0 || B < 0 || K < 0 || L_max < 0 || E < 0) return SPEC_ERR_INVALID_ARG;
  *empty = B == 0;
  if (*empty) return SPEC_OK;
  if (!accepted_len || !cache_len) return SPEC_ERR_INVALID_ARG;
  const size_t esz = elem_size(dtype);
  const size_t row = (size_t)E * esz;
  // the larger buffer must fit size_t byte offsets
  const size_t planes = (size_t)P * (size_t)B;
  const size_t rows = planes * (size_t)(L_max > K ? L_max : K);
  if (planes / (size_t)B != (size_t)P || (row != 0 && rows > SIZE_MAX / 2 / row)) return SPEC_ERR_INVALID_ARG;
  const bool copies = P > 0 && K > 0 && E > 0;
  if (copies && (!cache || !staging)) return SPEC_ERR_INVALID_ARG;
  if (copies && ((uintptr_t)cache % esz != 0 || (uintptr_t)staging % esz != 0)) return SPEC_ERR_INVALID_ARG;
  const bool vec = row % 16 == 0 && ((uintptr_t)cache % 16 == 0) && ((uintptr_t)staging % 16 == 0);
  const size_t units = copies ? (vec ? row / 16 : (size_t)E) : 0;
  if (copies && units > 0x7fffffffu / (size_t)K) return SPEC_ERR_UNSUPPORTED;  // K > 0 when copies
  if (copies && planes > kMaxGrid) return SPEC_ERR_UNSUPPORTED;
  plan->copies = copies;
  plan->vec = vec;
  plan->row = row;
  return SPEC_OK;
}

inline int32_t position_budget(int32_t t, int32_t k_max) {
  if (t < 0 || k_max < 1) return -1;
  if (t < 2) return k_max;
  return (int32_t)((int64_t)k_max / (((int64_t)t + 1) * 2));
}

}  // namespace sv
