// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sv_host.h"

namespace sv {

// SAMPLE: statistics, then either decisions and sampling (s.decide) or
// sampling with the decisions in its prologue, then pick: four or three
// launches.  events[k] (if present, k < n_events) is recorded before launch k
// and events[launches] after the last one.
hipError_t launch_sample_pipeline(const VerifyShape& s, const VerifyIO& io, const VerifyWorkspace& ws,
                                  hipStream_t st, void* const* events, int n_events);
// SAMPLE_EARLY_EXIT: K + 2 launches (position i's statistics, each block
// first deciding position i - 1 of its sequence; then sampling, which decides
// position K - 1, and pick); events as above.
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

// Head over one shortlist shared by every row: C[M, n_sel*cs] = h[M, d] * W_S^T.
// partial (null: no K split) holds head_static_workspace_bytes(M, d, N).
hipError_t launch_head_static(const void* h, const void* W, const int32_t* cluster_ids, int M, int d, int V,
                              int cluster_size, int n_sel, void* out, int out_dtype, float* partial,
                              hipStream_t st);

// Read-only stream of bytes (a multiple of 32 KiB) for the roofline reference.
hipError_t launch_read_stream(const void* src, size_t bytes, void* sink, hipStream_t st);

// KV-cache commit: copy, then lengths and status (two launches).
hipError_t launch_kv_commit(void* cache, const void* staging, const int32_t* accepted_len, int32_t* cache_len,
                            int32_t* status, int P, int B, int K, int Lmax, int64_t row_bytes, int elem_bytes,
                            bool vec_ok, hipStream_t st);

}  // namespace sv
