// Exercises the library's host half (sv_host.h: shape arithmetic, workspace
// layout and the argument checks of every entry point) for the
// AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU test suite.
// Plain C++; no GPU, no HIP.  Prints "host checks ok" and exits 0 when every
// expectation holds; a sanitizer finding aborts with a report.
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../speculative_sampling_verification_vocab_amd/csrc/sv_host.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

// Fake device addresses: validation never dereferences them.
static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static void layouts() {
  const int Bs[] = {0, 1, 3, 8, 64, 256, 1000};
  const int Ks[] = {0, 1, 4, 7, 64};
  const int Vs[] = {1, 7, 33, 4096, 5003, 32000, 262144, 1 << 20};
  for (int B : Bs)
    for (int K : Ks)
      for (int V : Vs)
        for (int dt = 0; dt < 2; ++dt)
          for (int mode = 0; mode < 3; ++mode) {
            const spec_status_t sc = sv::check_shape(B, K, V, (spec_dtype_t)dt, (spec_mode_t)mode);
            EXPECT(sc == SPEC_OK);
            if (B == 0) continue;
            const sv::VerifyShape s = sv::make_shape(B, K, V, dt, true);
            EXPECT(s.NT >= 1 && s.NG >= 1 && s.NT_s >= 1 && s.NG_s >= 1);
            EXPECT((long long)s.NT * s.tile >= V && (long long)(s.NT - 1) * s.tile < V);
            EXPECT((long long)s.NG * sv::kWavesPerBlock >= s.NT);
            EXPECT((long long)s.NG_s * s.TPW_s * sv::kWavesPerBlock >= s.NT_s);
            const size_t need = sv::verify_workspace_layout(s, mode, nullptr, nullptr);
            if (need > ((size_t)64 << 20)) continue;
            // lay the workspace out in a heap buffer of exactly `need` bytes and
            // fill every part: an overflow of the buffer is an ASan report, and
            // parts must not overlap
            std::vector<unsigned char> buf(need + 256);
            unsigned char* base = buf.data() + (256 - ((uintptr_t)buf.data() % 256)) % 256;
            unsigned char* exact = static_cast<unsigned char*>(malloc(need));
            sv::VerifyWorkspace w{};
            sv::verify_workspace_layout(s, mode, base, &w);
            struct Part { void* p; size_t bytes; } parts[6];
            int np = 0;
            const size_t Bz = (size_t)B, Kz = (size_t)K;
            if (mode == 1) {
              parts[np++] = {w.part_g, Bz * (Kz + 1) * s.NT * sizeof(sv::ArgTile)};
            } else {
              parts[np++] = {w.part_a, Bz * 2 * Kz * s.NT * sizeof(sv::TileStat)};
              parts[np++] = {w.rows, Bz * sizeof(sv::SampleRowInfo)};
              parts[np++] = {w.part_b, Bz * s.NT_s * sizeof(sv::SampleTile)};
              parts[np++] = {w.gx, Bz * 2 * (Kz > 0 ? Kz : 1) * sizeof(float)};
              if (mode == 2) parts[np++] = {w.cont, Bz * (Kz > 0 ? Kz : 1) * sizeof(int32_t)};
            }
            for (int i = 0; i < np; ++i) {
              const size_t off = (size_t)((unsigned char*)parts[i].p - base);
              EXPECT(off % 256 == 0);
              EXPECT(off + parts[i].bytes <= need);
              if (parts[i].bytes) {
                memset(exact + off, 0x40 + i, parts[i].bytes);
                memset(base + off, 0x40 + i, parts[i].bytes);
              }
            }
            for (int i = 0; i < np; ++i) {
              const size_t off = (size_t)((unsigned char*)parts[i].p - base);
              if (parts[i].bytes) {
                EXPECT(exact[off] == 0x40 + i);
                EXPECT(exact[off + parts[i].bytes - 1] == 0x40 + i);
              }
            }
            free(exact);
          }
}

static void shape_limits() {
  EXPECT(sv::check_shape(4, 3, 1000, (spec_dtype_t)7, SPEC_MODE_SAMPLE) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::check_shape(4, 3, 1000, SPEC_BF16, (spec_mode_t)9) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::check_shape(-1, 3, 1000, SPEC_BF16, SPEC_MODE_SAMPLE) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::check_shape(4, -1, 1000, SPEC_BF16, SPEC_MODE_SAMPLE) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::check_shape(4, 3, 0, SPEC_BF16, SPEC_MODE_SAMPLE) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::check_shape(4, 65, 1000, SPEC_BF16, SPEC_MODE_SAMPLE) == SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::check_shape(4, 3, (1 << 30) + 1, SPEC_BF16, SPEC_MODE_SAMPLE) == SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::check_shape(4, 3, INT_MAX, SPEC_F32, SPEC_MODE_GREEDY) == SPEC_ERR_UNSUPPORTED);
  // grids beyond 2^31 - 1 blocks
  EXPECT(sv::check_shape(INT_MAX, 64, 1 << 30, SPEC_F32, SPEC_MODE_SAMPLE) != SPEC_OK);
  EXPECT(sv::check_shape(INT_MAX, 0, 1, SPEC_BF16, SPEC_MODE_SAMPLE) == SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::check_shape(INT_MAX, 64, 1, SPEC_BF16, SPEC_MODE_GREEDY) == SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::check_shape(1 << 20, 64, 1, SPEC_BF16, SPEC_MODE_GREEDY) == SPEC_OK);
  for (int B : {0, 1, 255, 65536, INT_MAX})
    for (int K : {0, 1, 63, 64})
      for (int V : {1, 4095, 4096, 4097, 1 << 30})
        for (int dt = 0; dt < 2; ++dt)
          for (int mode = 0; mode < 3; ++mode) {
            const spec_status_t sc = sv::check_shape(B, K, V, (spec_dtype_t)dt, (spec_mode_t)mode);
            if (sc == SPEC_OK && B > 0) {
              const sv::VerifyShape s = sv::make_shape(B, K, V, dt, false);
              (void)sv::verify_workspace_layout(s, mode, nullptr, nullptr);
              EXPECT((size_t)B * (size_t)s.NG_s <= sv::kMaxGrid);
            }
          }
}

static void verify_args() {
  sv::VerifyShape s{};
  size_t need = 0;
  bool empty = false;
  void* t = fake(0x10000);
  void* d = fake(0x20000);
  const int32_t* tok = static_cast<const int32_t*>(fake(0x30000));
  const float* uni = static_cast<const float*>(fake(0x40000));
  int32_t* acc = static_cast<int32_t*>(fake(0x50000));
  int32_t* out = static_cast<int32_t*>(fake(0x60000));
  void* ws = fake(0x100000);
  auto call = [&](const void* tt, const void* dd, const int32_t* tk, const float* un, int B, int K, int V, int dt,
                  float T, int mode, int32_t* a, int32_t* o, void* w, size_t wb, bool sparse = false) {
    return sv::validate_verify(tt, dd, tk, un, B, K, V, (spec_dtype_t)dt, T, (spec_mode_t)mode, a, o, w, wb, sparse,
                               &s, &need, &empty);
  };
  const size_t big = (size_t)1 << 40;
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_OK && !empty && need > 0);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 0.0f, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, -1.0f, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, NAN, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, INFINITY, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 0.0f, 1, acc, out, ws, big) == SPEC_OK);  // greedy ignores T
  EXPECT(call(nullptr, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, nullptr, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, nullptr, tok, nullptr, 2, 3, 1000, 1, 1.0f, 1, acc, out, ws, big) == SPEC_OK);
  EXPECT(call(t, d, nullptr, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, nullptr, nullptr, uni, 2, 0, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_OK);
  EXPECT(call(t, d, tok, nullptr, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, nullptr, out, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, nullptr, ws, big) == SPEC_ERR_INVALID_ARG);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, nullptr, big) == SPEC_ERR_WORKSPACE);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, fake(0x100010), big) == SPEC_ERR_WORKSPACE);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, 0) == SPEC_ERR_WORKSPACE);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_OK);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, need) == SPEC_OK);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, need - 1) == SPEC_ERR_WORKSPACE);
  // empty batch: nothing else is looked at
  EXPECT(call(nullptr, nullptr, nullptr, nullptr, 0, 3, 1000, 1, 1.0f, 0, nullptr, nullptr, nullptr, 0) == SPEC_OK &&
         empty);
  // alignment decides the load path, not validity
  EXPECT(call(fake(0x10002), d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_OK && !s.aligned);
  EXPECT(call(t, d, tok, uni, 2, 3, 1001, 1, 1.0f, 0, acc, out, ws, big) == SPEC_OK && !s.aligned);
  EXPECT(call(t, d, tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big) == SPEC_OK && s.aligned);
  EXPECT(call(t, fake(0x20002), tok, uni, 2, 3, 1000, 1, 1.0f, 0, acc, out, ws, big, true) == SPEC_OK && s.aligned);
}

static void sparse_args() {
  const int32_t* cids = static_cast<const int32_t*>(fake(0x70000));
  for (int K = 1; K <= 8; ++K) {
    // n_sel on the heap with exactly K entries: reading past it is an ASan report
    int32_t* ns = static_cast<int32_t*>(malloc(sizeof(int32_t) * K));
    for (int i = 0; i < K; ++i) ns[i] = 1 + i % 3;
    EXPECT(sv::validate_sparse_draft(4, K, 6000, SPEC_BF16, cids, ns, 1500, 3, 500) == SPEC_OK);
    ns[K - 1] = 0;
    EXPECT(sv::validate_sparse_draft(4, K, 6000, SPEC_BF16, cids, ns, 1500, 3, 500) == SPEC_ERR_INVALID_ARG);
    ns[K - 1] = 4;
    EXPECT(sv::validate_sparse_draft(4, K, 6000, SPEC_BF16, cids, ns, 1500, 3, 500) == SPEC_ERR_INVALID_ARG);
    ns[K - 1] = 3;
    EXPECT(sv::validate_sparse_draft(4, K, 6000, SPEC_BF16, cids, ns, 1499, 3, 500) == SPEC_ERR_INVALID_ARG);
    free(ns);
  }
  int32_t one = 1;
  EXPECT(sv::validate_sparse_draft(4, 1, 6001, SPEC_BF16, cids, &one, 1500, 3, 500) == SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::validate_sparse_draft(4, 1, 6000, SPEC_BF16, nullptr, &one, 1500, 3, 500) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_sparse_draft(4, 1, 6000, SPEC_BF16, cids, nullptr, 1500, 3, 500) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_sparse_draft(4, 1, 6000, SPEC_BF16, cids, &one, 1500, 13, 500) == SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_sparse_draft(4, 0, 6000, SPEC_BF16, nullptr, nullptr, 0, 0, 0) == SPEC_OK);
  EXPECT(sv::validate_sparse_draft(INT_MAX, 64, 1 << 30, SPEC_F32, cids, &one, INT_MAX, INT_MAX, 1) != SPEC_OK);
}

static void head_args() {
  bool empty = false;
  void* h = fake(0x10000);
  void* W = fake(0x20000);
  const int32_t* c = static_cast<const int32_t*>(fake(0x30000));
  float* o = static_cast<float*>(fake(0x40000));
  EXPECT(sv::validate_head_shortlist(h, W, c, 32, 4, 4096, 128256, 501, 16, o, nullptr, SPEC_F32, &empty) == SPEC_OK);
  EXPECT(sv::validate_head_shortlist(h, W, c, 32, 4, 4096, 128257, 501, 16, o, nullptr, SPEC_F32, &empty) ==
         SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::validate_head_shortlist(h, W, c, 1025, 4, 64, 1000, 10, 2, o, nullptr, SPEC_F32, &empty) ==
         SPEC_ERR_UNSUPPORTED);
  EXPECT(sv::validate_head_shortlist(h, W, c, 2, 4, 64, 1000, 10, 101, o, nullptr, SPEC_F32, &empty) ==
         SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_head_shortlist(h, W, c, 2, 4, 64, 1000, 10, 2, nullptr, nullptr, SPEC_F32, &empty) ==
         SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_head_shortlist(nullptr, W, c, 0, 4, 64, 1000, 10, 2, nullptr, nullptr, SPEC_F32, &empty) ==
             SPEC_OK && empty);
  EXPECT(sv::validate_head_shortlist(h, W, c, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1, INT_MAX, o, nullptr, SPEC_F32,
                                     &empty) != SPEC_OK);
  for (int K = 1; K <= 8; ++K) {
    int32_t* ns = static_cast<int32_t*>(malloc(sizeof(int32_t) * K));
    for (int i = 0; i < K; ++i) ns[i] = i % 3;
    EXPECT(sv::validate_head_positions(h, W, c, ns, 4, K, 64, 1000, 10, 2, 20, o, SPEC_BF16, &empty) == SPEC_OK);
    ns[K - 1] = 3;
    EXPECT(sv::validate_head_positions(h, W, c, ns, 4, K, 64, 1000, 10, 2, 20, o, SPEC_BF16, &empty) ==
           SPEC_ERR_INVALID_ARG);
    free(ns);
  }
  EXPECT(sv::validate_head_static(h, W, c, 128, 4096, 128256, 1, 32768, o, SPEC_F32, nullptr, 0, &empty) == SPEC_OK);
  EXPECT(sv::validate_head_static(fake(0x10001), W, c, 128, 4096, 128256, 1, 32768, o, SPEC_F32, nullptr, 0, &empty) ==
         SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_head_static(h, W, c, 128, 4096, 128256, 1, 32768, fake(0x40002), SPEC_F32, nullptr, 0, &empty) ==
         SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_head_static(h, W, c, 128, 4096, 128256, 1, 32768, fake(0x40002), SPEC_BF16, nullptr, 0, &empty) ==
         SPEC_OK);
  EXPECT(sv::validate_head_static(h, W, c, INT_MAX, INT_MAX, 1 << 30, 1, 1 << 30, o, SPEC_F32, nullptr, 0, &empty) != SPEC_OK);
  EXPECT(sv::validate_head_static(h, W, c, 0, 64, 100, 10, 3, o, SPEC_F32, nullptr, 0, &empty) == SPEC_OK && empty);
  // the K split: 4 slices of 128 x 8016 fp32 at M = 128, N = 8016; wide shortlists do not split
  EXPECT(sv::head_static_split(128, 4096, 8016) == 4);
  EXPECT(sv::head_static_split(128, 4096, 32768) == 1);
  EXPECT(sv::head_static_split(128, 4000, 8016) == 1);
  EXPECT(sv::head_static_split(1, 256, 64) == 1);
  const size_t need = sv::head_static_workspace_bytes(128, 4096, 8016);
  EXPECT(need == (size_t)4 * 128 * 8016 * 4);
  EXPECT(sv::validate_head_static(h, W, c, 128, 4096, 128256, 501, 16, o, SPEC_F32, fake(0x100000), need, &empty) ==
         SPEC_OK);
  EXPECT(sv::validate_head_static(h, W, c, 128, 4096, 128256, 501, 16, o, SPEC_F32, fake(0x100000), need - 1,
                                  &empty) == SPEC_ERR_WORKSPACE);
  EXPECT(sv::validate_head_static(h, W, c, 128, 4096, 128256, 501, 16, o, SPEC_F32, fake(0x100080), need, &empty) ==
         SPEC_ERR_WORKSPACE);
  for (int M : {1, 7, 128, 1000})
    for (int N : {1, 64, 8016, 20000, 32768})
      for (int d : {64, 128, 4096, 4100}) {
        const int s = sv::head_static_split(M, d, N);
        EXPECT(s >= 1 && s <= sv::kStaticMaxSplit && (s == 1 || s * 4 <= d / 64));
      }
}

static void kv_args() {
  bool empty = false;
  sv::KvPlan plan{};
  void* cache = fake(0x100000);
  void* stg = fake(0x200000);
  const int32_t* a = static_cast<const int32_t*>(fake(0x300000));
  const int32_t* l = static_cast<const int32_t*>(fake(0x400000));
  EXPECT(sv::validate_kv_commit(cache, stg, a, l, 64, 256, 7, 128, 1024, SPEC_BF16, &plan, &empty) == SPEC_OK &&
         plan.copies && plan.vec && plan.row == 2048);
  EXPECT(sv::validate_kv_commit(cache, stg, a, l, 2, 3, 4, 10, 5, SPEC_BF16, &plan, &empty) == SPEC_OK && !plan.vec);
  EXPECT(sv::validate_kv_commit(fake(0x100001), stg, a, l, 2, 3, 4, 10, 5, SPEC_BF16, &plan, &empty) ==
         SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_kv_commit(cache, stg, nullptr, l, 2, 3, 4, 10, 5, SPEC_BF16, &plan, &empty) ==
         SPEC_ERR_INVALID_ARG);
  EXPECT(sv::validate_kv_commit(nullptr, nullptr, a, l, 0, 3, 4, 10, 5, SPEC_BF16, &plan, &empty) == SPEC_OK &&
         !plan.copies);
  EXPECT(sv::validate_kv_commit(cache, stg, a, l, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, SPEC_F32, &plan,
                                &empty) != SPEC_OK);
  EXPECT(sv::validate_kv_commit(cache, stg, a, l, -1, 3, 4, 10, 5, SPEC_BF16, &plan, &empty) == SPEC_ERR_INVALID_ARG);
}

static void budget() {
  const int want16[] = {16, 16, 2, 2, 1, 1, 1, 1, 0, 0};
  for (int t = 0; t < 10; ++t) EXPECT(sv::position_budget(t, 16) == want16[t]);
  EXPECT(sv::position_budget(INT_MAX, INT_MAX) == 0);
  EXPECT(sv::position_budget(1, INT_MAX) == INT_MAX);
  EXPECT(sv::position_budget(-1, 4) == -1 && sv::position_budget(0, 0) == -1);
}

int main() {
  layouts();
  shape_limits();
  verify_args();
  sparse_args();
  head_args();
  kv_args();
  budget();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
