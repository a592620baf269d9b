// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

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
};

struct VerifyWorkspace {
  TileStat* part_a;     // [B][2K][NT]
  SampleRowInfo* rows;  // [B]
  SampleTile* part_b;   // [B][NT_s]
  ArgTile* part_g;      // [B][K+1][NT]
  float* gx;            // [B][2K] logits at the draft tokens: target rows 0..K-1, then draft rows
  int32_t* cont;        // [K][B] early exit: 1 if the sequence accepted positions 0..j and goes on
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

int tile_elems(int dtype);
VerifyShape make_shape(int B, int K, int V, int dtype, bool aligned);
// mode: 0 SAMPLE, 1 GREEDY, 2 SAMPLE_EARLY_EXIT (spec_mode_t values).
size_t verify_workspace_layout(const VerifyShape& s, int mode, void* base, VerifyWorkspace* out);

// SAMPLE: statistics, then either decisions and sampling (s.decide) or
// sampling with the decisions in its prologue, then pick: four or three
// launches.  events[k] (if present, k < n_events) is recorded before launch k
// and events[launches] after the last one.
int sample_launches(const VerifyShape& s);
hipError_t launch_sample_pipeline(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                  hipStream_t st, void* const* events, int n_events);
// SAMPLE_EARLY_EXIT: K + 2 launches (position i's statistics, each block
// first deciding position i - 1 of its sequence; then sampling, which decides
// position K - 1, and pick); events as above.
int early_exit_launches(const VerifyShape& s);
hipError_t launch_early_exit_pipeline(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                      hipStream_t st, void* const* events, int n_events);
// GREEDY: greedy -> greedy_finalize.
hipError_t launch_greedy(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws, hipStream_t st);
hipError_t launch_greedy_finalize(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                  hipStream_t st);

// nsel_pos (host, nsel_period entries) set: context x uses the first
// nsel_pos[x % nsel_period] of its S cluster ids and writes compact rows of
// stride L; otherwise every context uses n_sel ids and rows of n_sel * cs.
hipError_t launch_head(const void* h, const void* W, const int32_t* cluster_ids, int B, int K, int d, int V,
                       int cluster_size, int n_sel, void* compact, void* dense, int dense_dtype,
                       hipStream_t st, const int32_t* nsel_pos = nullptr, int nsel_period = 0, int S = 0,
                       int L = 0, int compact_dtype = 0);
int head_max_contexts();

// Head over one shortlist shared by every row: C[M, n_sel*cs] = h[M, d] * W_S^T.
hipError_t launch_head_static(const void* h, const void* W, const int32_t* cluster_ids, int M, int d, int V,
                              int cluster_size, int n_sel, void* out, int out_dtype, hipStream_t st);

// KV-cache commit: copy, then lengths and status (two launches).
hipError_t launch_kv_commit(void* cache, const void* staging, const int32_t* accepted_len, int32_t* cache_len,
                            int32_t* status, int P, int B, int K, int Lmax, int64_t row_bytes, int elem_bytes,
                            bool vec_ok, hipStream_t st);

}  // namespace sv
