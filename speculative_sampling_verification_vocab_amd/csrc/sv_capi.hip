// C ABI of libspecverify.so: launches behind the host checks of sv_host.h.
// Declarations and the contract of every entry point are in include/specverify.h.

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/specverify.h"
#include "sv_internal.h"

// Scratch of spec_verify_noalloc: one copy per GPU, at a different device
// address on each.  In host code this name is only a stand-in for the symbol:
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

using sv::check_shape;

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until located
std::mutex g_scratch_mu;

// Device address of the current device's scratch, located on first use with
// that device current.  `stream` (if not null) must belong to that device.
spec_status_t noalloc_scratch(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SPEC_ERR_HIP;
  if (dev >= kMaxDevices) return SPEC_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return SPEC_ERR_HIP;
    if (sdev != dev) return SPEC_ERR_INVALID_ARG;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return SPEC_ERR_HIP;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
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
  sv::VerifyShape s{};
  size_t need = 0;
  bool empty = false;
  const spec_status_t sc =
      sv::validate_verify(target_logits, draft_logits, draft_tokens, uniforms, B, K, V, dtype, temperature, mode,
                          accepted_len, out_tokens, workspace, workspace_bytes, sparse != nullptr, &s, &need, &empty);
  if (sc != SPEC_OK) return sc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto record = [&](int i) {
    if (events && i < n_events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
  };
  if (empty) {
    record(0);
    return SPEC_OK;
  }
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
  if (mode == SPEC_MODE_SAMPLE_EARLY_EXIT) {
    e = sv::launch_early_exit_pipeline(s, io, ws, st, events, n_events);
  } else if (mode == SPEC_MODE_SAMPLE) {
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

spec_status_t spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                                  const float* uniforms, int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                  float temperature, spec_mode_t mode, int32_t* accepted_len, int32_t* out_tokens,
                                  float* p_target_at_draft, float* p_draft_at_draft, void* stream) {
  // Every argument check of spec_verify first, with the scratch size as the
  // workspace size and a stand-in address: nothing is located or enqueued
  // for a call that fails them.
  sv::VerifyShape s{};
  size_t need = 0;
  bool empty = false;
  void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
  const spec_status_t sc =
      sv::validate_verify(target_logits, draft_logits, draft_tokens, uniforms, B, K, V, dtype, temperature, mode,
                          accepted_len, out_tokens, stand_in, SPEC_NOALLOC_SCRATCH_BYTES, false, &s, &need, &empty);
  if (sc != SPEC_OK) return sc;
  void* ws = nullptr;
  if (!empty) {
    const spec_status_t ss = noalloc_scratch(stream, &ws);
    if (ss != SPEC_OK) return ss;
  }
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, B, K, V, dtype, temperature, mode,
                     accepted_len, out_tokens, p_target_at_draft, p_draft_at_draft, empty ? stand_in : ws,
                     SPEC_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

spec_status_t spec_verify_sparse_draft(const void* target_logits, const void* draft_compact,
                                       const int32_t* cluster_ids, const int32_t* n_sel, int32_t L, int32_t S,
                                       int32_t cluster_size, const int32_t* draft_tokens, const float* uniforms,
                                       int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, float temperature,
                                       int32_t* accepted_len, int32_t* out_tokens, float* p_target_at_draft,
                                       float* p_draft_at_draft, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const spec_status_t sc = sv::validate_sparse_draft(B, K, V, dtype, cluster_ids, n_sel, L, S, cluster_size);
  if (sc != SPEC_OK) return sc;
  const SparseDraft sp{cluster_ids, n_sel, L, S, cluster_size};
  return verify_impl(target_logits, draft_compact, draft_tokens, uniforms, B, K, V, dtype, temperature,
                     SPEC_MODE_SAMPLE, accepted_len, out_tokens, p_target_at_draft, p_draft_at_draft, workspace,
                     workspace_bytes, stream, nullptr, 0, &sp);
}

int32_t spec_position_budget(int32_t t, int32_t k_max) { return sv::position_budget(t, k_max); }

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
  bool empty = false;
  const spec_status_t sc = sv::validate_head_shortlist(h, W, cluster_ids, B, K, d, V, cluster_size, n_sel,
                                                       logits_compact, dense_out, dense_dtype, &empty);
  if (sc != SPEC_OK || empty) return sc;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_head(h, W, cluster_ids, B, K, d, V, cluster_size, n_sel, logits_compact,
                                       dense_out, dense_dtype == SPEC_BF16 ? 1 : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_draft_head_positions(const void* h, const void* W, const int32_t* cluster_ids,
                                        const int32_t* n_sel, int32_t B, int32_t K, int32_t d, int32_t V,
                                        int32_t cluster_size, int32_t S, int32_t L, void* logits_compact,
                                        spec_dtype_t compact_dtype, void* stream) {
  bool empty = false;
  const spec_status_t sc = sv::validate_head_positions(h, W, cluster_ids, n_sel, B, K, d, V, cluster_size, S, L,
                                                       logits_compact, compact_dtype, &empty);
  if (sc != SPEC_OK || empty) return sc;
  (void)hipGetLastError();
  // every (context, position) is a context of its own with one row
  const hipError_t e = sv::launch_head(h, W, cluster_ids, B * K, 1, d, V, cluster_size, 0, logits_compact, nullptr,
                                       0, static_cast<hipStream_t>(stream), n_sel, K, S, L,
                                       compact_dtype == SPEC_BF16 ? 1 : 0);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_draft_head_static_workspace_bytes(int32_t M, int32_t d, int32_t V, int32_t cluster_size,
                                             int32_t n_sel) {
  if (M < 1 || d < 1 || V < 1 || cluster_size < 1 || n_sel < 1 || V % cluster_size != 0) return 0;
  const long long N = (long long)n_sel * cluster_size;
  if (N > 0x7fffffffLL) return 0;
  return sv::head_static_workspace_bytes(M, d, (int32_t)N);
}

spec_status_t spec_draft_head_static(const void* h, const void* W, const int32_t* cluster_ids, int32_t M,
                                     int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel, void* logits,
                                     spec_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  bool empty = false;
  const spec_status_t sc = sv::validate_head_static(h, W, cluster_ids, M, d, V, cluster_size, n_sel, logits,
                                                    out_dtype, workspace, workspace_bytes, &empty);
  if (sc != SPEC_OK || empty) return sc;
  (void)hipGetLastError();
  const hipError_t e =
      sv::launch_head_static(h, W, cluster_ids, M, d, V, cluster_size, n_sel, logits, out_dtype == SPEC_BF16 ? 1 : 0,
                             static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_kv_commit(void* cache, const void* staging, const int32_t* accepted_len, int32_t* cache_len,
                             int32_t* status, int32_t P, int32_t B, int32_t K, int32_t L_max, int32_t E,
                             spec_dtype_t dtype, void* stream) {
  sv::KvPlan plan{};
  bool empty = false;
  const spec_status_t sc =
      sv::validate_kv_commit(cache, staging, accepted_len, cache_len, P, B, K, L_max, E, dtype, &plan, &empty);
  if (sc != SPEC_OK || empty) return sc;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_kv_commit(plan.copies ? cache : nullptr, plan.copies ? staging : nullptr,
                                            accepted_len, cache_len, status, plan.copies ? P : 0, B, K, L_max,
                                            (int64_t)plan.row, (int)sv::elem_size(dtype), plan.vec,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_read_stream_probe(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 32768 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0)
    return SPEC_ERR_INVALID_ARG;
  if (bytes / 32768 > 0x7fffffffu) return SPEC_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_read_stream(src, bytes, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // extern "C"
