// Shortlisted drafter head (DynaSpec summary, lowest.today, "Model
// architecture", items 1, 3 and 4): each context scores clusters, keeps the
// union of its top clusters as the drafter's shortlist, and computes draft
// logits only there.  P_d is 0 (logit -inf) off the shortlist.
//
// Cluster-major gather-GEMM on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16,
// fp32 accumulation).  One block owns a slab of 64 consecutive tokens of one
// cluster (W rows are contiguous, so the slab is one 512 KiB block of W for
// d = 4096).  It finds the contexts that selected the cluster, stages their
// hidden rows in LDS chunk by chunk, and streams its W slab through MFMA once
// per pass of up to 32 (context, position) rows.  The same block writes -inf
// into the dense output for every context that did not select the cluster, so
// each dense element is written exactly once.

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSlabTok = 64;       // tokens per block: 4 waves x 16 MFMA columns
constexpr int kPassRows = 32;      // A rows per pass over W: two 16-row MFMA chunks
constexpr int kDChunk = 512;       // hidden dims staged in LDS per step
constexpr int kAStride = kDChunk + 8;  // LDS row stride: 16-byte skew per row avoids bank conflicts
constexpr int kMaxCtx = 2048;      // contexts listed per cluster (host-checked: B <= kMaxCtx)

struct HeadArgs {
  const uint16_t* h;    // bf16 [B, K, d]
  const uint16_t* W;    // bf16 [V, d]
  const int32_t* cids;  // [B, n_sel]
  int B, K, d, V, cs, n_sel;
  float* compact;       // [B, K, n_sel*cs] or null
  void* dense;          // [B, K, V] or null
  int dense_bf16;
  int vec_ok;           // d % 8 == 0 and h, W 16-byte aligned: 16-byte row loads
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_dense(const HeadArgs& a, size_t idx, float v) {
  if (a.dense_bf16) static_cast<uint16_t*>(a.dense)[idx] = f32_to_bf16_rne(v);
  else static_cast<float*>(a.dense)[idx] = v;
}

__global__ void __launch_bounds__(kBlock) head_mfma_kernel(HeadArgs a) {
  __shared__ int sh_ctx[kMaxCtx];     // (b << 16) | s of every context that selected this cluster
  __shared__ uint32_t sh_sel[kMaxCtx / 32];
  __shared__ int sh_count;
  __shared__ __attribute__((aligned(16))) uint16_t sh_a[kPassRows * kAStride];  // 32.5 KiB

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c = blockIdx.x;
  const int tok_in0 = blockIdx.y * kSlabTok;
  const int ntok = min(kSlabTok, a.cs - tok_in0);
  const int tok0 = c * a.cs + tok_in0;

  // 1. The contexts that selected cluster c, listed in (b, s) order.
  __shared__ int sh_wcount[kWavesPerBlock];
  if (threadIdx.x == 0) sh_count = 0;
  for (int i = threadIdx.x; i < kMaxCtx / 32; i += kBlock) sh_sel[i] = 0u;
  __syncthreads();
  const int entries = a.B * a.n_sel;
  for (int e0 = 0; e0 < entries; e0 += kBlock) {
    const int e = e0 + threadIdx.x;
    const bool hit = e < entries && a.cids[e] == c;
    const uint64_t mask = __ballot(hit);
    if (lane == 0) sh_wcount[wave] = __popcll(mask);
    __syncthreads();
    int before = sh_count, tot = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      if (w < wave) before += sh_wcount[w];
      tot += sh_wcount[w];
    }
    if (hit) {
      const int pos = before + __popcll(mask & ((1ull << lane) - 1ull));
      const int b = e / a.n_sel, s = e % a.n_sel;
      if (pos < kMaxCtx) sh_ctx[pos] = (b << 16) | s;
      atomicOr(&sh_sel[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    if (threadIdx.x == 0) sh_count += tot;
    __syncthreads();
  }
  const int nctx = min(sh_count, kMaxCtx);
  const int K = a.K, L = a.n_sel * a.cs;

  // 2. -inf for every (context, position) that did not select c.
  if (a.dense) {
    const int total = a.B * K * ntok;
    for (int i = threadIdx.x; i < total; i += kBlock) {
      const int t = i % ntok;
      const int bk = i / ntok;
      const int b = bk / K;
      if (!((sh_sel[b >> 5] >> (b & 31)) & 1u)) store_dense(a, (size_t)bk * a.V + tok0 + t, -__builtin_inff());
    }
  }
  if (nctx == 0) return;

  // 3. Passes of up to kPassRows A rows (row r = context p*, position k).
  const int ctx_per_pass = max(1, kPassRows / K);
  const int my_tok = wave * 16 + (lane & 15);                 // MFMA column of this lane
  const bool tok_ok = my_tok < ntok;
  const uint16_t* wrow = a.W + (size_t)(tok0 + (tok_ok ? my_tok : 0)) * a.d;
  const int kgrp = lane >> 4;                                 // 0..3: which 8 of the 32 k's
  for (int p0 = 0; p0 < nctx; p0 += ctx_per_pass) {
    const int np = min(ctx_per_pass, nctx - p0);
    const int rows = np * K;  // <= kPassRows unless K > kPassRows
    for (int r0 = 0; r0 < rows; r0 += kPassRows) {
      const int nr = min(kPassRows, rows - r0);
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      for (int d0 = 0; d0 < a.d; d0 += kDChunk) {
        const int dn = min(kDChunk, a.d - d0);
        // Stage A rows [r0, r0+nr) x dims [d0, d0+dn) in LDS (zero padding).
        __syncthreads();
        for (int i = threadIdx.x; i < kPassRows * kDChunk / 8; i += kBlock) {
          const int r = i / (kDChunk / 8), j8 = (i % (kDChunk / 8)) * 8;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (r < nr && j8 < dn) {
            const int rr = r0 + r;
            const int ctx = sh_ctx[p0 + rr / K];
            const int b = ctx >> 16, k = rr % K;
            const uint16_t* src = a.h + ((size_t)b * K + k) * a.d + d0 + j8;
            if (a.vec_ok && j8 + 8 <= dn) {
              v = *reinterpret_cast<const u32x4*>(src);
            } else {
              uint32_t t4[4] = {0u, 0u, 0u, 0u};
              for (int e = 0; e < 8; ++e)
                if (j8 + e < dn) t4[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
              v = u32x4{t4[0], t4[1], t4[2], t4[3]};
            }
          }
          *reinterpret_cast<u32x4*>(&sh_a[r * kAStride + j8]) = v;
        }
        __syncthreads();
        // MFMA over this chunk, 32 k per instruction; this lane supplies
        // W[my_tok][k..k+8).  Four k-steps of W are loaded before their MFMAs.
        for (int kk0 = 0; kk0 < dn; kk0 += 4 * 32) {
          u32x4 wv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kofs = kk0 + q * 32 + kgrp * 8;
            wv[q] = u32x4{0u, 0u, 0u, 0u};
            if (tok_ok && kofs < dn) {
              if (a.vec_ok && kofs + 8 <= dn) {
                wv[q] = *reinterpret_cast<const u32x4*>(wrow + d0 + kofs);
              } else {
                uint32_t t4[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8; ++e)
                  if (kofs + e < dn) t4[e >> 1] |= (uint32_t)wrow[d0 + kofs + e] << (16 * (e & 1));
                wv[q] = u32x4{t4[0], t4[1], t4[2], t4[3]};
              }
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kofs = kk0 + q * 32 + kgrp * 8;
            if (kk0 + q * 32 >= dn) break;
            const bf16x8 bfrag = __builtin_bit_cast(bf16x8, wv[q]);
#pragma unroll
            for (int mc = 0; mc < 2; ++mc) {
              const u32x4 av = *reinterpret_cast<const u32x4*>(&sh_a[(mc * 16 + (lane & 15)) * kAStride + kofs]);
              acc[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bfrag, acc[mc], 0, 0,
                                                                0);
            }
          }
        }
      }
      // Epilogue: lane holds D[m = 4*(lane/16) + i][n = lane%16] of each chunk.
      if (tok_ok) {
#pragma unroll
        for (int mc = 0; mc < 2; ++mc) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mc * 16 + 4 * kgrp + i;
            if (r < nr) {
              const int rr = r0 + r;
              const int ctx = sh_ctx[p0 + rr / K];
              const int b = ctx >> 16, s = ctx & 0xffff, k = rr % K;
              const float v = acc[mc][i];
              const size_t bk = (size_t)b * K + k;
              if (a.compact) a.compact[bk * L + (size_t)s * a.cs + tok_in0 + my_tok] = v;
              if (a.dense) store_dense(a, bk * a.V + tok0 + my_tok, v);
            }
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_head(const void* h, const void* W, const int32_t* cluster_ids, int B, int K, int d, int V,
                       int cluster_size, int n_sel, float* compact, void* dense, int dense_dtype, hipStream_t st) {
  HeadArgs a{};
  a.h = static_cast<const uint16_t*>(h);
  a.W = static_cast<const uint16_t*>(W);
  a.cids = cluster_ids;
  a.B = B;
  a.K = K;
  a.d = d;
  a.V = V;
  a.cs = cluster_size;
  a.n_sel = n_sel;
  a.compact = compact;
  a.dense = dense;
  a.dense_bf16 = dense_dtype == 1;
  a.vec_ok = (d % 8 == 0) && ((uintptr_t)h % 16 == 0) && ((uintptr_t)W % 16 == 0);
  const int n_clusters = V / cluster_size;
  const dim3 grid((unsigned)n_clusters, (unsigned)((cluster_size + kSlabTok - 1) / kSlabTok));
  hipLaunchKernelGGL(head_mfma_kernel, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

int head_max_contexts() { return kMaxCtx; }

}  // namespace sv
