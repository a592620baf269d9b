// Shortlisted drafter head (DynaSpec summary, lowest.today, "Model
// architecture", items 1, 3 and 4): each context scores clusters, keeps the
// union of its top clusters as the drafter's shortlist, and computes draft
// logits only there.  P_d is 0 (logit -inf) off the shortlist.
//
// Cluster-major gather-GEMM on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16,
// fp32 accumulation).  One block owns a slab of 64 consecutive tokens of one
// cluster (W rows are contiguous, so the slab is one 512 KiB block of W for
// d = 4096).  It finds the contexts that selected the cluster and streams its
// W slab through MFMA once per pass of up to 32 (context, position) rows,
// staging W and the hidden rows through LDS so that global loads stay fully
// coalesced while MFMA reads its lane-major fragments.  A dense output is
// first filled with -inf by a separate pass of whole-line stores; the head
// then writes the shortlist's logits into it.

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPassRows = 32;      // A rows per pass over W: two 16-row MFMA chunks
constexpr int kStageK = 256;       // hidden dims per LDS stage (128 and 512 measured slower)
// LDS rows of a stage are unpadded; the 16-byte chunks of row r are stored
// XOR-permuted by r % 16, so a fragment read (16 rows, one chunk) and a row
// store both touch distinct banks.  Without the 16-byte row skew the block
// needs 53.4 KB, and three blocks fit a CU instead of two (1-2 % faster).
constexpr int kLdsStride = kStageK;
// Element offset of (row, 8-aligned column) in a staged LDS tile.
__device__ __forceinline__ int lds_at(int row, int col) { return row * kLdsStride + (((col >> 3) ^ (row & 15)) << 3); }
constexpr int kMaxCtx = kHeadMaxCtx;  // contexts listed per cluster (host-checked: B <= kMaxCtx)

struct HeadArgs {
  const uint16_t* h;    // bf16 [B, K, d]
  const uint16_t* W;    // bf16 [V, d]
  const int32_t* cids;  // [B, n_sel]
  int B, K, d, V, cs, n_sel;
  void* compact;        // [B, K, L] fp32 (or bf16 with compact_bf16) or null
  int compact_bf16;
  void* dense;          // [B, K, V] or null
  int dense_bf16;
  int vec_ok;           // d % 8 == 0 and h, W 16-byte aligned: 16-byte row loads
  int S;                // entries per row of cids (n_sel for one shortlist per context)
  int L;                // compact row stride
  int nsel_period;      // 0: every context uses n_sel; else context x uses nsel_pos[x % period]
  int nsel_pos[kMaxK];
  int dense_filled;     // the dense output already holds -inf everywhere (dense_fill_kernel)
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

// 8 consecutive bf16 of a row starting at k (zero beyond d).
__device__ __forceinline__ u32x4 load8(const uint16_t* row, int k, int d, int vec_ok) {
  if (vec_ok && k + 8 <= d) return *reinterpret_cast<const u32x4*>(row + k);
  uint32_t t4[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < 8; ++e)
    if (k + e < d) t4[e >> 1] |= (uint32_t)row[k + e] << (16 * (e & 1));
  return u32x4{t4[0], t4[1], t4[2], t4[3]};
}

// Steps 1 and 2 of both kernels: list the contexts that selected cluster c in
// (b, s) order (sh_ctx, count returned), and write -inf into the dense output
// for every (context, position) that did not select it.  Every thread of the
// block must call this.
template <int NTH>
__device__ __forceinline__ int list_contexts(const HeadArgs& a, int c, int tok0, int ntok, int* sh_ctx,
                                             uint32_t* sh_sel) {
  constexpr int NW = NTH / kWave;
  __shared__ int sh_count;
  __shared__ int sh_wcount[NW];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (threadIdx.x == 0) sh_count = 0;
  for (int i = threadIdx.x; i < kMaxCtx / 32; i += NTH) sh_sel[i] = 0u;
  __syncthreads();
  const int entries = a.B * a.S;
  for (int e0 = 0; e0 < entries; e0 += NTH) {
    const int e = e0 + threadIdx.x;
    const int used = a.nsel_period ? a.nsel_pos[(e / a.S) % a.nsel_period] : a.n_sel;
    const bool hit = e < entries && e % a.S < used && a.cids[e] == c;
    const uint64_t mask = __ballot(hit);
    if (lane == 0) sh_wcount[wave] = __popcll(mask);
    __syncthreads();
    int before = sh_count, tot = 0;
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += sh_wcount[w];
      tot += sh_wcount[w];
    }
    if (hit) {
      const int pos = before + __popcll(mask & ((1ull << lane) - 1ull));
      const int b = e / a.S, s = e % a.S;
      if (pos < kMaxCtx) sh_ctx[pos] = (b << 16) | s;
      atomicOr(&sh_sel[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    if (threadIdx.x == 0) sh_count += tot;
    __syncthreads();
  }
  const int nctx = min(sh_count, kMaxCtx);
  if (a.dense && !a.dense_filled) {
    const int total = a.B * a.K * ntok;
    for (int i = threadIdx.x; i < total; i += NTH) {
      const int t = i % ntok;
      const int bk = i / ntok;
      const int b = bk / a.K;
      if (!((sh_sel[b >> 5] >> (b & 31)) & 1u)) store_dense(a, (size_t)bk * a.V + tok0 + t, -__builtin_inff());
    }
  }
  return nctx;
}

// Epilogue of one pass: lane holds D[m = 4*(lane/16) + i][n = lane%16] of
// each 16-row chunk; row r of the pass is A row r0 + r.
__device__ __forceinline__ void store_pass(const HeadArgs& a, const f32x4 (&acc)[2], const int* sh_ctx, int p0,
                                           int r0, int nr, int tok0, int tok_in0, int my_tok, int ntok, int kgrp) {
  if (my_tok >= ntok) return;
  const int K = a.K;
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
        if (a.compact) {
          const size_t o = bk * a.L + (size_t)s * a.cs + tok_in0 + my_tok;
          if (a.compact_bf16) static_cast<uint16_t*>(a.compact)[o] = f32_to_bf16_rne(v);
          else static_cast<float*>(a.compact)[o] = v;
        }
        if (a.dense) store_dense(a, bk * a.V + tok0 + my_tok, v);
      }
    }
  }
}

// -inf over the whole dense output, in 16-byte stores (whole cache lines),
// ahead of the head kernel, which then writes only the shortlist's logits.
// Filling per cluster slab inside the head kernel wrote 128-byte pieces that
// straddle lines (clusters of 501 tokens do not start on line boundaries) and
// cost about 27 us at B=32, K=4, V=128256; with this pass the dense output
// costs about 10 us.  (An LDS-DMA variant of the head kernel, as in the
// static-shortlist head, measured 3-5 % slower here: with about two contexts
// per cluster the kernel is bound by the W stream, not by LDS traffic.)
__global__ void __launch_bounds__(kBlock) dense_fill_kernel(void* dense, size_t elems, int bf16) {
  const uint32_t pat = bf16 ? 0xff80ff80u : 0xff800000u;
  const size_t bytes = elems * (bf16 ? 2 : 4);
  const size_t stride = (size_t)gridDim.x * kBlock;
  const size_t first = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if ((uintptr_t)dense % 16 == 0) {
    const u32x4 v = {pat, pat, pat, pat};
    for (size_t i = first; i < bytes / 16; i += stride)  // nontemporal: about 3 us less over 33 MB
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dense) + i);
    for (size_t i = bytes / 16 * 16 / (bf16 ? 2 : 4) + first; i < elems; i += stride) {
      if (bf16) static_cast<uint16_t*>(dense)[i] = 0xff80u;
      else static_cast<uint32_t*>(dense)[i] = pat;
    }
  } else {
    for (size_t i = first; i < elems; i += stride) {
      if (bf16) static_cast<uint16_t*>(dense)[i] = 0xff80u;
      else static_cast<uint32_t*>(dense)[i] = pat;
    }
  }
}

// SLAB tokens per block (SLAB / 16 waves of 16 MFMA columns); one stage of
// loads in flight in registers.  kFull: d % kStageK == 0 and 16-byte aligned
// rows, so every load is a whole 16-byte piece inside its row; the loads are
// then issued without per-lane guards (W rows past the slab re-read its last
// row, A rows past the pass read h's first row; none of it reaches an
// output).  Otherwise loads are guarded per lane and zero-filled past d.
template <int SLAB, bool kFull>
__global__ void __launch_bounds__(SLAB / 16 * kWave, 3) head_mfma_kernel(HeadArgs a) {
  constexpr int NTH = SLAB / 16 * kWave;
  constexpr int kCols = kStageK / 8, kRowsPerLoad = NTH / kCols;
  constexpr int kWL = SLAB / kRowsPerLoad;        // 16-byte W loads per thread per stage
  constexpr int kAL = kPassRows / kRowsPerLoad;   // 16-byte A loads per thread per stage
  static_assert(SLAB % kRowsPerLoad == 0 && kPassRows % kRowsPerLoad == 0, "load split");
  __shared__ int sh_ctx[kMaxCtx];     // (b << 16) | s of every context that selected this cluster
  __shared__ uint32_t sh_sel[kMaxCtx / 32];
  __shared__ __attribute__((aligned(16))) uint16_t sh_w[SLAB * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sh_a[kPassRows * kLdsStride];

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  // Block -> (cluster, slab).  Workgroup i runs on XCD i % 8, so the slabs of
  // one cluster are made consecutive blocks of one XCD: they run together and
  // share, through that XCD's L2, the hidden rows of the contexts that
  // selected the cluster (B=32, K=4, d=4096, top 16 of 256 clusters: 167 ->
  // 164 us).  The bytes fetched beyond W and h, about 5 % of W, did not change
  // with this order, with other cache policies for the W loads, or with the
  // hidden-row loads reduced to one row (a probe), so they are not re-reads
  // of h.
  const int nslab = (a.cs + SLAB - 1) / SLAB;
  const int xcd = (int)(blockIdx.x & 7u), j = (int)(blockIdx.x >> 3);
  const int c = (j / nslab) * 8 + xcd;
  if (c >= a.V / a.cs) return;
  const int tok_in0 = (j % nslab) * SLAB;
  const int ntok = min(SLAB, a.cs - tok_in0);
  const int tok0 = c * a.cs + tok_in0;

  // 1, 2. The contexts that selected cluster c; -inf for the others.
  const int nctx = list_contexts<NTH>(a, c, tok0, ntok, sh_ctx, sh_sel);
  if (nctx == 0) return;
  const int K = a.K;

  // 3. Passes of up to kPassRows A rows (row r = context p*, position k).
  //    Per stage of kStageK hidden dims the block loads its W rows with fully
  //    coalesced 16-byte loads (each wave instruction covers two rows x 512
  //    bytes) and the pass's A rows likewise, stores them to LDS, and every
  //    wave reads the lane-major MFMA fragments of its 16 tokens from LDS.
  const int my_tok = wave * 16 + (lane & 15);  // MFMA column of this lane
  const int kgrp = lane >> 4;                  // 0..3: which 8 of the 32 k's
  const int lrow = threadIdx.x / kCols, c8 = (threadIdx.x % kCols) * 8;
  const uint16_t* wrow[kWL];
#pragma unroll
  for (int i = 0; i < kWL; ++i) {
    const int r = kRowsPerLoad * i + lrow;
    wrow[i] = (kFull || r < ntok) ? a.W + (size_t)(tok0 + min(r, ntok - 1)) * a.d : nullptr;
  }
  const int ctx_per_pass = max(1, kPassRows / K);
  const int nstage = (a.d + kStageK - 1) / kStageK;
  for (int p0 = 0; p0 < nctx; p0 += ctx_per_pass) {
    const int np = min(ctx_per_pass, nctx - p0);
    const int rows = np * K;
    for (int r0 = 0; r0 < rows; r0 += kPassRows) {
      const int nr = min(kPassRows, rows - r0);
      const uint16_t* arow[kAL];
#pragma unroll
      for (int i = 0; i < kAL; ++i) {
        const int r = kRowsPerLoad * i + lrow;
        arow[i] = kFull ? a.h : nullptr;
        if (r < nr) {
          const int rr = r0 + r;
          const int ctx = sh_ctx[p0 + rr / K];
          arow[i] = a.h + ((size_t)(ctx >> 16) * K + rr % K) * a.d;
        }
      }
      u32x4 wreg[kWL], areg[kAL];
      auto load_stage = [&](int st) {
        const int k = st * kStageK + c8;
        if (kFull) {
#pragma unroll
          for (int i = 0; i < kWL; ++i)  // W streams once per pass: nontemporal
            wreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[i] + k));
#pragma unroll
          for (int i = 0; i < kAL; ++i) areg[i] = *reinterpret_cast<const u32x4*>(arow[i] + k);
        } else {
#pragma unroll
          for (int i = 0; i < kWL; ++i) wreg[i] = wrow[i] ? load8(wrow[i], k, a.d, a.vec_ok) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int i = 0; i < kAL; ++i) areg[i] = arow[i] ? load8(arow[i], k, a.d, a.vec_ok) : u32x4{0u, 0u, 0u, 0u};
        }
      };
      auto stage_to_lds = [&]() {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kWL; ++i) *reinterpret_cast<u32x4*>(&sh_w[lds_at(kRowsPerLoad * i + lrow, c8)]) = wreg[i];
#pragma unroll
        for (int i = 0; i < kAL; ++i) *reinterpret_cast<u32x4*>(&sh_a[lds_at(kRowsPerLoad * i + lrow, c8)]) = areg[i];
        __syncthreads();
      };
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      const bool two = nr > 16;
      auto mfma_stage = [&]() {
#pragma unroll
        for (int q = 0; q < kStageK / 32; ++q) {
          const int kofs = q * 32 + kgrp * 8;
          const u32x4 bv = *reinterpret_cast<const u32x4*>(&sh_w[lds_at(my_tok, kofs)]);
          const bf16x8 bfrag = __builtin_bit_cast(bf16x8, bv);
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(&sh_a[lds_at(lane & 15, kofs)]);
          acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), bfrag, acc[0], 0, 0, 0);
          if (two) {
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(&sh_a[lds_at(16 + (lane & 15), kofs)]);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), bfrag, acc[1], 0, 0, 0);
          }
        }
      };
      // One stage in flight: the next stage's loads are issued before the
      // MFMA work on the current one; the last stage issues none.
      load_stage(0);
      for (int st = 0; st + 1 < nstage; ++st) {
        stage_to_lds();
        load_stage(st + 1);
        mfma_stage();
      }
      stage_to_lds();
      mfma_stage();
      store_pass(a, acc, sh_ctx, p0, r0, nr, tok0, tok_in0, my_tok, ntok, kgrp);
    }
  }
}

template <int SLAB>
void launch_head_cfg(const HeadArgs& a, int n_clusters, bool full, hipStream_t st) {
  // a multiple of 8 clusters (the excess exits at once), times the slabs of each
  const size_t nslab = (size_t)(a.cs + SLAB - 1) / SLAB;
  const dim3 grid((unsigned)(((size_t)n_clusters + 7) / 8 * 8 * nslab)), block(SLAB / 16 * kWave);
  if (full) hipLaunchKernelGGL((head_mfma_kernel<SLAB, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((head_mfma_kernel<SLAB, false>), grid, block, 0, st, a);
}

}  // namespace

hipError_t launch_head(const void* h, const void* W, const int32_t* cluster_ids, int B, int K, int d, int V,
                       int cluster_size, int n_sel, void* compact, void* dense, int dense_dtype, hipStream_t st,
                       const int32_t* nsel_pos, int nsel_period, int S, int L, int compact_dtype) {
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
  a.compact_bf16 = compact_dtype == 1;
  a.dense = dense;
  a.dense_bf16 = dense_dtype == 1;
  a.vec_ok = (d % 8 == 0) && ((uintptr_t)h % 16 == 0) && ((uintptr_t)W % 16 == 0);
  a.S = nsel_pos ? S : n_sel;
  a.L = nsel_pos ? L : n_sel * cluster_size;
  a.nsel_period = nsel_pos ? nsel_period : 0;
  for (int i = 0; nsel_pos && i < nsel_period; ++i) a.nsel_pos[i] = nsel_pos[i];
  const int n_clusters = V / cluster_size;
  if (dense) {
    const size_t elems = (size_t)B * K * V;
    const size_t chunks = (elems * (dense_dtype == 1 ? 2 : 4) + 16 * kBlock - 1) / (16 * kBlock);
    const unsigned blocks = (unsigned)(chunks < 4096 ? (chunks > 0 ? chunks : 1) : 4096);
    hipLaunchKernelGGL(dense_fill_kernel, dim3(blocks), dim3(kBlock), 0, st, dense, elems, a.dense_bf16);
    a.dense_filled = 1;
  }
  const bool full = a.vec_ok && d % kStageK == 0;
  // 64-token slabs with one stage in flight: 32-token slabs (more, smaller
  // blocks) and two stages in flight both measured slower.
  launch_head_cfg<64>(a, n_clusters, full, st);
  return hipGetLastError();
}


}  // namespace sv
