// Drafter head over a static shortlist shared by every context (the
// fixed-subset methods the DynaSpec summary contrasts with, FR-Spec and
// VocabTrim: one frequency-ranked subset of the vocabulary for all contexts).
// With one shortlist the head is a dense GEMM, C[M, N] = h[M, d] * W_S[N, d]^T,
// M = B*K rows of hidden states and N = n_sel * cluster_size shortlist tokens
// whose W rows are gathered cluster by cluster.
//
// For the drafting shapes (M = B*K up to a few hundred, d = 4096, N of 8k to
// 32k) the GEMM is bound by the stream of W_S from HBM: 2 flops per byte per
// row of M, far below the MFMA/HBM balance of about 300.  Two kernels:
//   * head_static_dma_kernel (d % 64 == 0, 16-byte aligned rows): both
//     operands go straight from memory into LDS with global_load_lds, four
//     to six stages of 64 dims deep, XOR-swizzled so fragment reads are free
//     of bank conflicts; explicit vmcnt waits and one barrier per stage;
//   * head_static_kernel (any d and alignment): global -> registers -> LDS in
//     stages of 64 dims (two LDS buffers, P stages in flight in registers);
//     the loads are issued without branches and masked on the way to LDS,
//     which keeps the compiler's wait counts partial.
// Both: one block per (kMt x kNt) output tile, h (1 MiB at M = 128) re-read
// from L2 by every column tile, so kNt is as wide as the grid allows; each
// wave computes TM x TN chunks of 16 x 16 with v_mfma_f32_16x16x32_bf16 from
// LDS fragments (lane l: row l % 16, k offset 8 * (l / 16)), fp32
// accumulation; WK > 1 splits the MFMA k-steps of a stage between waves and
// adds the partial tiles at the end.
// Loading W straight into B-fragment registers (no LDS for W) measured
// slower: a B fragment spans 16 rows, so each such load touches twice the
// cache lines per byte.
// Cluster ids are not checked on the host; an id outside [0, V / cluster_size)
// contributes zero columns.

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


struct StaticArgs {
  const uint16_t* h;     // bf16 [M, d]
  const uint16_t* W;     // bf16 [V, d]
  const int32_t* cids;   // [n_sel], any order
  int M, d, cs, N;
  int nclusters;         // V / cs: ids outside [0, nclusters) read as zero rows
  int m_tiles;           // row tiles; column tile = v / m_tiles
  int remap;             // XCD-aware tile order (grid a multiple of 8, m_tiles > 1)
  void* out;             // [M, N] fp32 or bf16
  int out_bf16;
  int pair16;            // bf16 out, N even, out 4-byte aligned: dword stores of column pairs
  int ksplit;            // LDS-DMA kernel: blocks per output tile, each over a slice of the K stages
  int split_stages;      // stages per slice
  float* partial;        // ksplit > 1: fp32 partial tiles [ksplit][M][N], added by head_static_reduce_kernel
};

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 8 consecutive bf16 of a row from k, zeros past d (any d, any alignment).
__device__ __forceinline__ u32x4 load8_slow(const uint16_t* row, int k, int d) {
  uint32_t t4[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < 8; ++e)
    if (k + e < d) t4[e >> 1] |= (uint32_t)row[k + e] << (16 * (e & 1));
  return u32x4{t4[0], t4[1], t4[2], t4[3]};
}

// WK > 1: the waves of k-group wk (0 .. WK - 1) hold partial sums of the same
// tiles as group 0.  One row chunk i at a time, groups 1.. park their sums in
// LDS (red, room for (WK - 1) * NWMN * 64 * TN * 4 floats) and group 0 adds
// them in a fixed order.  Every wave of the block must call this.
template <int NWMN, int WK, int TM, int TN>
__device__ __forceinline__ void add_split_k(f32x4 (&acc)[TM][TN], float* red, int wk, int wmn, int lane) {
  constexpr int kE = TN * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (wk > 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(((wk - 1) * NWMN + wmn) * kE + j * 4 + r) * kWave + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int k2 = 1; k2 < WK; ++k2)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] += red[(((k2 - 1) * NWMN + wmn) * kE + j * 4 + r) * kWave + lane];
    }
    __syncthreads();
  }
}

// Column n of the shortlist reads a W row of an in-range cluster.
__device__ __forceinline__ bool live_column(const StaticArgs& a, int n) {
  if (n >= a.N) return false;
  const int c = a.cids[n / a.cs];
  return c >= 0 && c < a.nclusters;
}

// Write a wave's TM x TN chunks of 16 x 16 at rows mw.., columns nw.. (lane
// holds D[4 * (lane / 16) + r][lane % 16] of each chunk).  check_cols: zero
// the columns of out-of-range clusters (their W rows were not masked).
template <int TM, int TN>
__device__ __forceinline__ void store_tile(const StaticArgs& a, f32x4 (&acc)[TM][TN], int mw, int nw, int lane,
                                           bool check_cols) {
  if (check_cols) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
      if (!live_column(a, nw + 16 * j + (lane & 15)))
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (a.pair16) {
    // bf16 pairs: lanes c and c ^ 1 (columns n, n + 1) swap two of their
    // four rows, so each lane stores two rows as one dword per row (the even
    // lane rows 0 and 1, the odd lane rows 2 and 3) instead of four shorts.
    const int odd = lane & 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nc = nw + 16 * j + (lane & 14);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const f32x4 v = acc[i][j];
        const float r0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? v[0] : v[2]), 0xb1, 0xf, 0xf, false));
        const float r1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? v[1] : v[3]), 0xb1, 0xf, 0xf, false));
        if (nc >= a.N) continue;
        const int mb = mw + 16 * i + 4 * (lane >> 4) + 2 * odd;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int m = mb + q;
          if (m >= a.M) continue;
          const float lo = odd ? (q ? r1 : r0) : v[q];
          const float hi = odd ? v[2 + q] : (q ? r1 : r0);
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + (size_t)m * a.N + nc) =
              (uint32_t)to_bf16_rne(lo) | ((uint32_t)to_bf16_rne(hi) << 16);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = nw + 16 * j + (lane & 15);
    if (n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mw + 16 * i + 4 * (lane >> 4) + r;
        if (m < a.M) {
          const size_t o = (size_t)m * a.N + n;
          if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = to_bf16_rne(acc[i][j][r]);
          else static_cast<float*>(a.out)[o] = acc[i][j][r];
        }
      }
    }
  }
}

// WM x WN x WK waves; each wave TM x TN chunks of 16 x 16 over every WK-th
// MFMA k-step of a stage (WK > 1: the WK partial sums are added through LDS
// at the end); P (even) stages in flight; rows of kStage + kPad bf16 in LDS.
// kVec: d % 8 == 0 and 16-byte aligned rows (eight dims are all inside d or
// all past it).
template <int WM, int WN, int WK, int TM, int TN, int P, int kStage, int kPad, bool kVec>
__global__ void __launch_bounds__(kWave * WM * WN * WK) head_static_kernel(StaticArgs a) {
  constexpr int kStride = kStage + kPad;
  constexpr int kCols = kStage / 8;     // sixteen-byte columns per row and stage
  constexpr int kThreads = kWave * WM * WN * WK;
  constexpr int kMt = 16 * WM * TM, kNt = 16 * WN * TN, kRows = kMt + kNt;
  constexpr int kR = kThreads / kCols;          // rows one load slot covers across the block
  constexpr int kL = kRows / kR;                // load slots per thread and stage
  constexpr int kLA = kMt / kR;                 // the first kLA slots are h rows
  static_assert(kThreads % kCols == 0 && kMt % kR == 0 && kNt % kR == 0, "tile / block mismatch");
  static_assert(P % 2 == 0, "stage parity must be static");
  static_assert(kStage % (32 * WK) == 0 && kPad % 8 == 0, "stage / split mismatch");
  static_assert((WK - 1) * WM * WN * kWave * TN * 4 * 4 <= 2 * kRows * kStride * 2, "reduction space");
  __shared__ __attribute__((aligned(16))) uint16_t sh[2][kRows * kStride];

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int wk = wave / (WM * WN), wmn = wave % (WM * WN);
  const int wm = wmn / WN, wn = wmn % WN;
  int v = blockIdx.x;
  if (a.remap) v = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int n0 = (v / a.m_tiles) * kNt, m0 = (v % a.m_tiles) * kMt;

  const int lrow = threadIdx.x / kCols, c8 = (threadIdx.x % kCols) * 8;
  // Every slot loads from a valid row (h row 0 stands in for rows past M,
  // past N or of an out-of-range cluster) and masks the value: loads under a
  // branch would make the compiler wait for all of them before each stage.
  const uint16_t* src[kL];
  uint32_t live[kL];
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    const int r = lrow + kR * j;
    src[j] = a.h;
    live[j] = 0u;
    if (j < kLA) {
      const int m = m0 + r;
      if (m < a.M) src[j] = a.h + (size_t)m * a.d, live[j] = ~0u;
    } else {
      const int n = n0 + r - kMt;
      if (n < a.N) {
        const int s = n / a.cs;
        const int c = a.cids[s];
        if (c >= 0 && c < a.nclusters) src[j] = a.W + ((size_t)c * a.cs + (n - s * a.cs)) * a.d, live[j] = ~0u;
      }
    }
  }
  const int nst = (a.d + kStage - 1) / kStage;
  u32x4 R[P][kL];
  // Loads of stage s.  Dims past d (the ragged last stage, and the stages up
  // to the next multiple of P, which the loop runs as zeros) load from the
  // row start and are zeroed when the slot is written to LDS, with rows that
  // are not live; masking at load time would make the wave wait for the
  // loads at once, and a branch around them makes the compiler wait for all
  // loads in flight.
  auto issue = [&](u32x4 (&slot)[kL], int s) {
    const int k = s * kStage + c8;
    if (kVec) {
      const int kk = k < a.d ? k : 0;
#pragma unroll
      for (int j = 0; j < kL; ++j) {
        const u32x4* p = reinterpret_cast<const u32x4*>(src[j] + kk);
        slot[j] = j < kLA ? *p : __builtin_nontemporal_load(p);  // W streams once: nontemporal
      }
    } else {
#pragma unroll
      for (int j = 0; j < kL; ++j) slot[j] = live[j] ? load8_slow(src[j], k, a.d) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto put = [&](const u32x4 (&slot)[kL], int buf, int s) {
    const uint32_t kin = s * kStage + c8 < a.d ? ~0u : 0u;
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      const uint32_t m = live[j] & kin;
      *reinterpret_cast<u32x4*>(&sh[buf][(lrow + kR * j) * kStride + c8]) =
          u32x4{slot[j][0] & m, slot[j][1] & m, slot[j][2] & m, slot[j][3] & m};
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Slot by slot, in the order the loop issues them (no interleaving by the
  // scheduler), so the loads in flight at the loop head are the same on entry
  // and on the back edge and the compiler's wait counts stay partial.
#pragma unroll
  for (int q = 0; q < P; ++q) {
    issue(R[q], q);
    __builtin_amdgcn_sched_barrier(0);
  }
  put(R[0], 0, 0);
  issue(R[0], P);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  const int frow = lane & 15, fk = 8 * (lane >> 4);
  const int arow0 = wm * 16 * TM + frow, brow0 = kMt + wn * 16 * TN + frow;
  // Stage s lives in LDS buffer s & 1 (P is even, so q & 1) and in register
  // slot s % P before that.  No exit inside the unrolled body: every path
  // through the loop issues the same loads.
  for (int s0 = 0; s0 < nst; s0 += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int s = s0 + q;
      const int buf = q & 1;
#pragma unroll
      for (int kk = 0; kk < kStage / (32 * WK); ++kk) {
        const int ks = 32 * (kk * WK + wk);
        bf16x8 bf[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                 &sh[buf][(brow0 + 16 * j) * kStride + ks + fk]));
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                           &sh[buf][(arow0 + 16 * i) * kStride + ks + fk]));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
      // The other LDS buffer was last read in stage s - 1, before the
      // previous barrier.
      put(R[(q + 1) % P], buf ^ 1, s + 1);
      issue(R[(q + 1) % P], s + 1 + P);
      __syncthreads();
    }
  }

  if (WK > 1) {
    // The loop ended on a barrier: LDS is free.
    add_split_k<WM * WN, WK, TM, TN>(acc, reinterpret_cast<float*>(&sh[0][0]), wk, wmn, lane);
    if (wk > 0) return;
  }
  store_tile<TM, TN>(a, acc, m0 + wm * 16 * TM, n0 + wn * 16 * TN, lane, false);
}

// LDS-DMA form, for d % 64 == 0 and 16-byte aligned rows: global_load_lds
// moves each stage straight from memory into LDS (no register staging, no
// ds_write), NBUF stages deep.  One DMA instruction writes 1 KiB: 8 rows of
// 64 dims.  Within a 128-byte row the 16-byte chunk c sits in slot
// c ^ ((row >> 1) & 7): the 16 rows that one fragment read touches then fall
// on distinct banks, and a DMA lane picks its source chunk to match its slot.
// Rows past M, past N or of out-of-range clusters load h's first row: their
// outputs are not stored, or (out-of-range clusters) stored as zeros.
// The compiler does not track LDS-DMA completion, so the waits are explicit:
// before a stage is read, every wave waits until at most the later stages'
// DMAs are in flight, then the block meets at a barrier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte global_load_lds per lane: lane l's bytes land at lds + 16 * l
// (lds is the wave's uniform base).  The default cache policy: the
// nontemporal one measured 10-35 % slower in this kernel.
__device__ __forceinline__ void dma16(const uint16_t* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#endif
}

// Block epilogue through LDS: the waves that hold final sums (own) write
// their chunks into a row-major kMt x kNt fp32 tile in LDS (stage, room for
// kMt * (kNt + 4) floats), then the whole block stores it row by row, 16
// bytes per thread where the output rows allow it, so every row leaves as
// whole cache lines.  Columns of out-of-range clusters are stored as zeros.
// Every thread of the block must call this.
template <int kMt, int kNt, int TM, int TN>
__device__ __forceinline__ void store_block_tile(const StaticArgs& a, const f32x4 (&acc)[TM][TN], float* stage,
                                                 int m0, int n0, bool own, int mw, int nw, int lane, void* dst,
                                                 bool dst_bf16) {
  constexpr int kLd = kNt + 4;  // row stride in floats: the four row groups of a write land on distinct banks
  if (own) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stage[(mw + 16 * i + 4 * (lane >> 4) + r) * kLd + nw + 16 * j + (lane & 15)] = acc[i][j][r];
  }
  __syncthreads();
  // Thread t stores 4 consecutive columns: kNt / 4 threads per row.
  constexpr int kTpr = kNt / 4;
  const int nthreads = blockDim.x;
  const int c4 = (threadIdx.x % kTpr) * 4;
  const int esz = dst_bf16 ? 2 : 4;
  const bool vec = (size_t)a.N * esz % (dst_bf16 ? 8 : 16) == 0 &&
                   (uintptr_t)dst % (dst_bf16 ? 8 : 16) == 0 && n0 + kNt <= a.N;
  uint32_t keep = 0;  // bit e: column n0 + c4 + e is stored with its value (not zero)
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (live_column(a, n0 + c4 + e)) keep |= 1u << e;
  for (int r = threadIdx.x / kTpr; r < kMt; r += nthreads / kTpr) {
    const int m = m0 + r;
    if (m >= a.M) break;
    const float* src = stage + r * kLd + c4;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (keep >> e & 1u) ? src[e] : 0.0f;
    const size_t o = (size_t)m * a.N + n0 + c4;
    if (vec) {
      if (dst_bf16) {
        const uint32_t lo = (uint32_t)to_bf16_rne(v[0]) | ((uint32_t)to_bf16_rne(v[1]) << 16);
        const uint32_t hi = (uint32_t)to_bf16_rne(v[2]) | ((uint32_t)to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + o) = uint2{lo, hi};
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(dst) + o) = float4{v[0], v[1], v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n0 + c4 + e >= a.N) break;
        if (dst_bf16) static_cast<uint16_t*>(dst)[o + e] = to_bf16_rne(v[e]);
        else static_cast<float*>(dst)[o + e] = v[e];
      }
    }
  }
}

template <int WM, int WN, int WK, int TM, int TN, int NBUF>
__global__ void __launch_bounds__(kWave * WM * WN * WK) head_static_dma_kernel(StaticArgs a) {
  constexpr int NW = WM * WN * WK;
  constexpr int kMt = 16 * WM * TM, kNt = 16 * WN * TN, kRows = kMt + kNt;
  constexpr int kStage = 64;                      // dims per stage: 128 bytes of a row
  constexpr int kInst = kRows / 8;                // DMA instructions per stage
  constexpr int kIW = kInst / NW;                 // per wave
  static_assert(kRows % 8 == 0 && kInst % NW == 0, "DMA split");
  static_assert(NBUF >= 3 && (NBUF - 2) * kIW < 64, "pipeline depth");
  static_assert(kStage % (32 * WK) == 0, "k split");
  static_assert((WK - 1) * WM * WN * kWave * TN * 4 * 4 <= NBUF * kRows * 128, "reduction space");
  static_assert(kMt * (kNt + 4) * 4 <= NBUF * kRows * 128, "epilogue space");
  static_assert(kWave * NW % (kNt / 4) == 0, "epilogue rows per pass");
  __shared__ __attribute__((aligned(1024))) uint8_t sh[NBUF][kRows * 128];

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int wk = wave / (WM * WN), wmn = wave % (WM * WN);
  const int wm = wmn / WN, wn = wmn % WN;
  int v = blockIdx.x;
  if (a.remap) v = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  // Slice-major order: the blocks of one K slice are consecutive, so an XCD's
  // share of the grid reuses the same slice of h from its L2.
  const int tiles = (int)(gridDim.x / (unsigned)a.ksplit);
  const int split = v / tiles;
  v -= split * tiles;
  const int n0 = (v / a.m_tiles) * kNt, m0 = (v % a.m_tiles) * kMt;

  // DMA instruction j of this wave covers tile rows 8 * (j * NW + wave) ..;
  // lane i fills slot i % 8 of row 8 * (j * NW + wave) + i / 8.
  const uint16_t* src[kIW];
#pragma unroll
  for (int j = 0; j < kIW; ++j) {
    const int r = 8 * (j * NW + wave) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const uint16_t* row = a.h;
    if (r < kMt) {
      if (m0 + r < a.M) row = a.h + (size_t)(m0 + r) * a.d;
    } else {
      const int n = n0 + r - kMt;
      if (n < a.N) {
        const int sc = n / a.cs;
        const int cl = a.cids[sc];
        if (cl >= 0 && cl < a.nclusters) row = a.W + ((size_t)cl * a.cs + (n - sc * a.cs)) * a.d;
      }
    }
    src[j] = row + 8 * c;
  }
  // This block's stages: s0 .. s0 + nst - 1 of the a.d / kStage in the row.
  const int s0 = split * a.split_stages;
  const int nst = min(a.d / kStage - s0, a.split_stages);
  auto issue = [&](int s) {
    uint8_t* dst = &sh[s % NBUF][0];
#pragma unroll
    for (int j = 0; j < kIW; ++j)
      dma16(src[j] + (s0 + s) * kStage, dst + 1024 * (j * NW + wave));
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NBUF - 1; ++s)
    if (s < nst) issue(s);

  const int frow = lane & 15, fc = lane >> 4;
  const int arow0 = wm * 16 * TM + frow, brow0 = kMt + wn * 16 * TN + frow;
  for (int s = 0; s < nst; ++s) {
    // Stage s has landed once only the later stages' DMAs can be in flight.
    if (s + NBUF - 2 < nst) wait_vmcnt<(NBUF - 2) * kIW>();
    else wait_vmcnt<0>();
    block_barrier();
    // Every wave has finished stage s - 1, whose buffer the next DMA refills.
    if (s + NBUF - 1 < nst) issue(s + NBUF - 1);
    const uint8_t* buf = &sh[s % NBUF][0];
#pragma unroll
    for (int kk = 0; kk < kStage / (32 * WK); ++kk) {
      const int c = 4 * (kk * WK + wk) + fc;       // 16-byte chunk of the 64-dim stage
      bf16x8 bf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = brow0 + 16 * j;
        bf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + r * 128 + 16 * (c ^ ((r >> 1) & 7))));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = arow0 + 16 * i;
        const bf16x8 af =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + r * 128 + 16 * (c ^ ((r >> 1) & 7))));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  // Every DMA has landed (the last stages waited for vmcnt 0).
  __syncthreads();  // all fragment reads done before LDS is reused
  float* stage = reinterpret_cast<float*>(&sh[0][0]);
  if (WK > 1) add_split_k<WM * WN, WK, TM, TN>(acc, stage, wk, wmn, lane);
  if (a.ksplit == 1)
    store_block_tile<kMt, kNt, TM, TN>(a, acc, stage, m0, n0, wk == 0, wm * 16 * TM, wn * 16 * TN, lane, a.out,
                                       a.out_bf16 != 0);
  else
    store_block_tile<kMt, kNt, TM, TN>(a, acc, stage, m0, n0, wk == 0, wm * 16 * TM, wn * 16 * TN, lane,
                                       a.partial + (size_t)split * a.M * a.N, false);
}

// out[m, n] = sum over slices s = 0 .. ksplit - 1 of partial[s][m][n], added
// in that order (deterministic), then stored as fp32 or bf16.  Four
// consecutive outputs per thread; 16-byte partial loads when N % 4 == 0.
__global__ void __launch_bounds__(kBlock) head_static_reduce_kernel(StaticArgs a) {
  const size_t MN = (size_t)a.M * a.N;
  const size_t q = ((size_t)blockIdx.x * kBlock + threadIdx.x) * 4;
  if (q >= MN) return;
  const bool vec_in = a.N % 4 == 0;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.ksplit; ++s) {
    const float* p = a.partial + (size_t)s * MN + q;
    if (vec_in) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += __uint_as_float(x[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (q + e < MN) v[e] += p[e];
    }
  }
  const bool vec_out = vec_in && (uintptr_t)a.out % (a.out_bf16 ? 8 : 16) == 0;
  if (vec_out) {
    if (a.out_bf16) {
      const uint32_t lo = (uint32_t)to_bf16_rne(v[0]) | ((uint32_t)to_bf16_rne(v[1]) << 16);
      const uint32_t hi = (uint32_t)to_bf16_rne(v[2]) | ((uint32_t)to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + q) = uint2{lo, hi};
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + q) = float4{v[0], v[1], v[2], v[3]};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (q + e >= MN) break;
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[q + e] = to_bf16_rne(v[e]);
      else static_cast<float*>(a.out)[q + e] = v[e];
    }
  }
}

// ksplit > 1 needs a.partial with room for ksplit * M * N floats.
template <int WM, int WN, int WK, int TM, int TN, int NBUF>
hipError_t launch_dma(StaticArgs a, int ksplit, hipStream_t st) {
  constexpr int kMt = 16 * WM * TM, kNt = 16 * WN * TN;
  a.m_tiles = (a.M + kMt - 1) / kMt;
  const long long tiles = (long long)((a.N + kNt - 1) / kNt) * a.m_tiles;
  const int nst = a.d / 64;
  if (ksplit < 1 || ksplit > nst || (ksplit > 1 && !a.partial)) return hipErrorInvalidValue;
  a.split_stages = (nst + ksplit - 1) / ksplit;
  a.ksplit = (nst + a.split_stages - 1) / a.split_stages;  // no empty slice
  const long long total = tiles * a.ksplit;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  a.remap = (a.m_tiles > 1 || a.ksplit > 1) && total % 8 == 0;
  hipLaunchKernelGGL((head_static_dma_kernel<WM, WN, WK, TM, TN, NBUF>), dim3((unsigned)total),
                     dim3(kWave * WM * WN * WK), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1) return e;
  const size_t quads = ((size_t)a.M * a.N + 3) / 4;
  hipLaunchKernelGGL(head_static_reduce_kernel, dim3((unsigned)((quads + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     a);
  return hipGetLastError();
}

template <int WM, int WN, int WK, int TM, int TN, int P, int KS = 64, int KP = 8>
hipError_t launch_cfg(StaticArgs a, bool vec, hipStream_t st) {
  constexpr int kMt = 16 * WM * TM, kNt = 16 * WN * TN;
  a.m_tiles = (a.M + kMt - 1) / kMt;
  const long long total = (long long)((a.N + kNt - 1) / kNt) * a.m_tiles;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  a.remap = a.m_tiles > 1 && total % 8 == 0;
  const dim3 grid((unsigned)total), block(kWave * WM * WN * WK);
  if (vec) hipLaunchKernelGGL((head_static_kernel<WM, WN, WK, TM, TN, P, KS, KP, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((head_static_kernel<WM, WN, WK, TM, TN, P, KS, KP, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_head_static(const void* h, const void* W, const int32_t* cluster_ids, int M, int d, int V,
                              int cluster_size, int n_sel, void* out, int out_dtype, float* partial,
                              hipStream_t st) {
  StaticArgs a{};
  a.h = static_cast<const uint16_t*>(h);
  a.W = static_cast<const uint16_t*>(W);
  a.cids = cluster_ids;
  a.M = M;
  a.d = d;
  a.cs = cluster_size;
  a.N = n_sel * cluster_size;
  a.nclusters = V / cluster_size;
  a.out = out;
  a.out_bf16 = out_dtype == 1;
  a.pair16 = a.out_bf16 && a.N % 2 == 0 && (uintptr_t)out % 4 == 0;
  const bool vec = (d % 8 == 0) && ((uintptr_t)h % 16 == 0) && ((uintptr_t)W % 16 == 0);
  // Widest column tile whose grid still gives most CUs a block: 128 x 128
  // tiles on 8 waves (2 x 4, each 64 x 32) for wide shortlists.  Narrow
  // shortlists: with a workspace, 128 x 128 tiles with the K stages split
  // over about one block per CU (head_static_split), the slices' fp32 tiles
  // added by a second launch (M = 128, N = 8016: 26.9 against 34.9 us with
  // W_S from HBM); without one, 64 x 32 tiles whose waves split each stage's
  // MFMA k-steps in two.  The LDS-DMA kernel takes d % 64 == 0 with 16-byte
  // aligned rows; the register-staged kernel everything else (128 x 32 narrow
  // tiles, 4 waves; LDS rows of 64 + 16 bf16).
  const long long t128 = (long long)((M + 127) / 128) * ((a.N + 127) / 128);
  const bool wide = t128 >= kStaticWideTiles;
  if (vec && d % 64 == 0) {
    if (wide) return launch_dma<2, 4, 1, 4, 2, 4>(a, 1, st);
    const int split = head_static_split(M, d, a.N);
    if (partial && split > 1) {
      a.partial = partial;
      return launch_dma<2, 4, 1, 4, 2, 3>(a, split, st);
    }
    return launch_dma<1, 2, 2, 4, 1, 6>(a, 1, st);
  }
  return wide ? launch_cfg<2, 4, 1, 4, 2, 4, 64, 16>(a, vec, st) : launch_cfg<2, 1, 2, 4, 2, 4, 64, 16>(a, vec, st);
}

}  // namespace sv
