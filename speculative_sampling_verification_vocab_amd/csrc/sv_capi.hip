// C ABI of libspecverify.so: argument validation, workspace sizing, launches.
// Declarations and the contract of every entry point are in include/specverify.h.

#include <math.h>
#include <stdint.h>

#include "../../include/specverify.h"
#include "sv_internal.h"

namespace {

constexpr size_t kMaxGrid = 0x7fffffffu;

bool valid_dtype(spec_dtype_t d) { return d == SPEC_F32 || d == SPEC_BF16; }
bool valid_mode(spec_mode_t m) {
  return m == SPEC_MODE_SAMPLE || m == SPEC_MODE_GREEDY || m == SPEC_MODE_SAMPLE_EARLY_EXIT;
}
bool sampling(spec_mode_t m) { return m == SPEC_MODE_SAMPLE || m == SPEC_MODE_SAMPLE_EARLY_EXIT; }
size_t elem_size(spec_dtype_t d) { return d == SPEC_BF16 ? 2 : 4; }

// Shape checks shared by the sizing function and the entry points.
spec_status_t check_shape(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, spec_mode_t mode) {
  if (!valid_dtype(dtype) || !valid_mode(mode)) return SPEC_ERR_INVALID_ARG;
  if (B < 0 || K < 0 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (K > SPEC_MAX_K) return SPEC_ERR_UNSUPPORTED;
  if (V > (1 << 30)) return SPEC_ERR_UNSUPPORTED;  // token ids and tile offsets stay in int32
  // element counts must fit size_t with room for byte offsets
  const size_t rows = (size_t)B * (size_t)(K + 1);
  if ((size_t)B != 0 && rows / (size_t)B != (size_t)(K + 1)) return SPEC_ERR_INVALID_ARG;
  if (rows != 0 && (size_t)V > SIZE_MAX / 8 / rows) return SPEC_ERR_INVALID_ARG;
  const sv::VerifyShape s = sv::make_shape(B, K, V, dtype == SPEC_BF16 ? 1 : 0, false);
  const size_t per_seq_rows = mode == SPEC_MODE_GREEDY ? (size_t)(K + 1) : (size_t)(2 * K);
  if ((size_t)B * per_seq_rows * (size_t)s.NG > kMaxGrid) return SPEC_ERR_UNSUPPORTED;
  if ((size_t)B * (2 * (size_t)K * s.NG + s.NG_s + 1) > kMaxGrid) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

struct SparseDraft {
  const int32_t* cids;
  const int32_t* nsel;  // host
  int L, S, cs;
};

spec_status_t verify_impl(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                          const float* uniforms, int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                          float temperature, spec_mode_t mode, int32_t* accepted_len, int32_t* out_tokens,
                          float* p_target_at_draft, float* p_draft_at_draft, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events, int n_events,
                          const SparseDraft* sparse = nullptr) {
  const spec_status_t sc = check_shape(B, K, V, dtype, mode);
  if (sc != SPEC_OK) return sc;
  const bool sample = sampling(mode);
  const bool early = mode == SPEC_MODE_SAMPLE_EARLY_EXIT;
  if (sample && !(temperature > 0.0f && isfinite(temperature))) return SPEC_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto record = [&](int i) {
    if (events && i < n_events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
  };
  if (B == 0) {
    record(0);
    return SPEC_OK;
  }
  if (!target_logits || !accepted_len || !out_tokens) return SPEC_ERR_INVALID_ARG;
  if (K > 0 && !draft_tokens) return SPEC_ERR_INVALID_ARG;
  if (sample && K > 0 && !draft_logits) return SPEC_ERR_INVALID_ARG;
  if (sample && !uniforms) return SPEC_ERR_INVALID_ARG;

  const size_t esz = elem_size(dtype);
  const size_t vec = 16 / esz;
  bool aligned = ((size_t)V % vec == 0) && ((uintptr_t)target_logits % 16 == 0);
  if (sample && K > 0 && !sparse) aligned = aligned && ((uintptr_t)draft_logits % 16 == 0);
  const sv::VerifyShape s = sv::make_shape(B, K, V, dtype == SPEC_BF16 ? 1 : 0, aligned);

  const size_t need = sv::verify_workspace_layout(s, (int)mode, nullptr, nullptr);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 256) != 0) return SPEC_ERR_WORKSPACE;
  sv::VerifyWorkspace ws{};
  sv::verify_workspace_layout(s, (int)mode, workspace, &ws);

  sv::VerifyIO io{};
  io.target = target_logits;
  io.draft = draft_logits;
  io.tokens = draft_tokens;
  io.uniforms = uniforms;
  io.temperature = temperature;
  io.accepted_len = accepted_len;
  io.out_tokens = out_tokens;
  io.p_target = p_target_at_draft;
  io.p_draft = p_draft_at_draft;
  if (sparse && K > 0) {
    io.cids = sparse->cids;
    io.nsel = sparse->nsel;
    io.L = sparse->L;
    io.S = sparse->S;
    io.cs = sparse->cs;
  }

  (void)hipGetLastError();  // clear a stale error so the checks below see only ours
  hipError_t e = hipSuccess;
  if (early) {
    e = sv::launch_early_exit_pipeline(s, io, ws, st, events, n_events);
  } else if (sample) {
    e = sv::launch_sample_pipeline(s, io, ws, st, events, n_events);
  } else {
    record(0);
    e = sv::launch_greedy(s, io, ws, st);
    record(1);
    if (e == hipSuccess) e = sv::launch_greedy_finalize(s, io, ws, st);
    record(2);
  }
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

const char* spec_status_string(spec_status_t status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG: return "SPEC_ERR_INVALID_ARG: invalid argument";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED: shape outside what the library supports";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP: a HIP launch failed";
  }
  return "unknown spec_status_t";
}

size_t spec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, spec_mode_t mode) {
  if (check_shape(B, K, V, dtype, mode) != SPEC_OK || B == 0) return 0;
  const sv::VerifyShape s = sv::make_shape(B, K, V, dtype == SPEC_BF16 ? 1 : 0, false);
  return sv::verify_workspace_layout(s, (int)mode, nullptr, nullptr);
}

spec_status_t spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                          const float* uniforms, int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                          float temperature, spec_mode_t mode, int32_t* accepted_len, int32_t* out_tokens,
                          float* p_target_at_draft, float* p_draft_at_draft, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, B, K, V, dtype, temperature, mode,
                     accepted_len, out_tokens, p_target_at_draft, p_draft_at_draft, workspace, workspace_bytes,
                     stream, nullptr, 0);
}

spec_status_t spec_verify_timed(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                                const float* uniforms, int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                float temperature, spec_mode_t mode, int32_t* accepted_len, int32_t* out_tokens,
                                float* p_target_at_draft, float* p_draft_at_draft, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* events, int32_t n_events) {
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, B, K, V, dtype, temperature, mode,
                     accepted_len, out_tokens, p_target_at_draft, p_draft_at_draft, workspace, workspace_bytes,
                     stream, events, n_events);
}

spec_status_t spec_verify_sparse_draft(const void* target_logits, const void* draft_compact,
                                       const int32_t* cluster_ids, const int32_t* n_sel, int32_t L, int32_t S,
                                       int32_t cluster_size, const int32_t* draft_tokens, const float* uniforms,
                                       int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, float temperature,
                                       int32_t* accepted_len, int32_t* out_tokens, float* p_target_at_draft,
                                       float* p_draft_at_draft, void* workspace, size_t workspace_bytes,
                                       void* stream) {
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
  const SparseDraft sp{cluster_ids, n_sel, L, S, cluster_size};
  return verify_impl(target_logits, draft_compact, draft_tokens, uniforms, B, K, V, dtype, temperature,
                     SPEC_MODE_SAMPLE, accepted_len, out_tokens, p_target_at_draft, p_draft_at_draft, workspace,
                     workspace_bytes, stream, nullptr, 0, &sp);
}

int32_t spec_verify_launch_count(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, spec_mode_t mode) {
  if (check_shape(B, K, V, dtype, mode) != SPEC_OK || B == 0) return 0;
  if (mode == SPEC_MODE_GREEDY) return 2;
  const sv::VerifyShape s = sv::make_shape(B, K, V, dtype == SPEC_BF16 ? 1 : 0, false);
  return mode == SPEC_MODE_SAMPLE_EARLY_EXIT ? sv::early_exit_launches(s) : sv::sample_launches(s);
}

spec_status_t spec_draft_head_shortlist(const void* h, const void* W, const int32_t* cluster_ids, int32_t B,
                                        int32_t K, int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel,
                                        float* logits_compact, void* dense_out, spec_dtype_t dense_dtype,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (B < 0 || K < 0 || d < 1 || V < 1 || cluster_size < 1 || n_sel < 0) return SPEC_ERR_INVALID_ARG;
  if (!valid_dtype(dense_dtype)) return SPEC_ERR_INVALID_ARG;
  if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
  if (n_sel > V / cluster_size) return SPEC_ERR_INVALID_ARG;
  if (B == 0 || K == 0) return SPEC_OK;
  if (B > sv::head_max_contexts() || n_sel > 0xffff) return SPEC_ERR_UNSUPPORTED;
  if ((size_t)B * (size_t)n_sel > 0x7fffffffu || (size_t)B * K * (size_t)V > SIZE_MAX / 8) return SPEC_ERR_INVALID_ARG;
  if (!h || !W || (!cluster_ids && n_sel > 0) || (!logits_compact && !dense_out)) return SPEC_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_head(h, W, cluster_ids, B, K, d, V, cluster_size, n_sel, logits_compact,
                                       dense_out, dense_dtype == SPEC_BF16 ? 1 : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_draft_head_positions(const void* h, const void* W, const int32_t* cluster_ids,
                                        const int32_t* n_sel, int32_t B, int32_t K, int32_t d, int32_t V,
                                        int32_t cluster_size, int32_t S, int32_t L, void* logits_compact,
                                        spec_dtype_t compact_dtype, void* stream) {
  if (B < 0 || K < 0 || d < 1 || V < 1 || cluster_size < 1 || S < 1 || L < 1) return SPEC_ERR_INVALID_ARG;
  if (!valid_dtype(compact_dtype)) return SPEC_ERR_INVALID_ARG;
  if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
  if (B == 0 || K == 0) return SPEC_OK;
  if (K > SPEC_MAX_K || (size_t)B * K > (size_t)sv::head_max_contexts() || S > 0xffff) return SPEC_ERR_UNSUPPORTED;
  if (S > V / cluster_size || (size_t)B * K * (size_t)S > 0x7fffffffu || (size_t)B * K * (size_t)L > SIZE_MAX / 8)
    return SPEC_ERR_INVALID_ARG;
  if (!h || !W || !cluster_ids || !n_sel || !logits_compact) return SPEC_ERR_INVALID_ARG;
  for (int i = 0; i < K; ++i)
    if (n_sel[i] < 0 || n_sel[i] > S || (long long)n_sel[i] * cluster_size > L) return SPEC_ERR_INVALID_ARG;
  (void)hipGetLastError();
  // every (context, position) is a context of its own with one row
  const hipError_t e = sv::launch_head(h, W, cluster_ids, B * K, 1, d, V, cluster_size, 0, logits_compact, nullptr,
                                       0, static_cast<hipStream_t>(stream), n_sel, K, S, L,
                                       compact_dtype == SPEC_BF16 ? 1 : 0);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_draft_head_static(const void* h, const void* W, const int32_t* cluster_ids, int32_t M,
                                     int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel, void* logits,
                                     spec_dtype_t out_dtype, void* stream) {
  if (M < 0 || d < 1 || V < 1 || cluster_size < 1 || n_sel < 0) return SPEC_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return SPEC_ERR_INVALID_ARG;
  if (V % cluster_size != 0) return SPEC_ERR_UNSUPPORTED;
  if (n_sel > V / cluster_size) return SPEC_ERR_INVALID_ARG;
  if (M == 0 || n_sel == 0) return SPEC_OK;
  if (!h || !W || !cluster_ids || !logits) return SPEC_ERR_INVALID_ARG;
  if ((uintptr_t)h % 2 || (uintptr_t)W % 2 || (uintptr_t)cluster_ids % 4 ||
      (uintptr_t)logits % elem_size(out_dtype))
    return SPEC_ERR_INVALID_ARG;
  const size_t N = (size_t)n_sel * (size_t)cluster_size;
  if ((size_t)M * N > SIZE_MAX / 8 || (size_t)M * (size_t)d > SIZE_MAX / 8) return SPEC_ERR_INVALID_ARG;
  if (((N + 31) / 32) * (((size_t)M + 127) / 128) > 0x7fffffffu) return SPEC_ERR_UNSUPPORTED;  // 1-D grid of tiles
  (void)hipGetLastError();
  const hipError_t e = sv::launch_head_static(h, W, cluster_ids, M, d, V, cluster_size, n_sel, logits,
                                              out_dtype == SPEC_BF16 ? 1 : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_kv_commit(void* cache, const void* staging, const int32_t* accepted_len, int32_t* cache_len,
                             int32_t* status, int32_t P, int32_t B, int32_t K, int32_t L_max, int32_t E,
                             spec_dtype_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return SPEC_ERR_INVALID_ARG;
  if (P < 0 || B < 0 || K < 0 || L_max < 0 || E < 0) return SPEC_ERR_INVALID_ARG;
  if (B == 0) return SPEC_OK;
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
  (void)hipGetLastError();
  const hipError_t e = sv::launch_kv_commit(copies ? cache : nullptr, copies ? staging : nullptr, accepted_len,
                                            cache_len, status, copies ? P : 0, B, K, L_max, (int64_t)row,
                                            (int)esz, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // extern "C"
