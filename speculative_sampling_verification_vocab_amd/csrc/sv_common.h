// Device-side building blocks shared by the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_host.h"

namespace sv {

// Storage element types: bf16 logits are handled as their uint16 bit patterns.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kVec = vec_elems(2); };
template <> struct Elem<float> { static constexpr int kVec = vec_elems(4); };

template <typename T> constexpr int kPerLane = Elem<T>::kVec * kLoads;    // 64 bf16, 32 f32
template <typename T> constexpr int kTile = kWave * kPerLane<T>;           // 4096 bf16, 2048 f32
template <typename T> constexpr int kPerLaneS = Elem<T>::kVec * kLoadsS;  // 32 bf16, 16 f32
template <typename T> constexpr int kTileS = kWave * kPerLaneS<T>;        // 2048 bf16, 1024 f32

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float to_f32(float f) { return f; }

// Position of lane element e inside a tile: 16-byte load j = e / kVec covers
// kWave*kVec consecutive ids, lane l owns ids [l*kVec, l*kVec + kVec) of it.
// A lane's elements are therefore in increasing token-id order.
template <typename T>
__device__ __forceinline__ int tile_offset(int e, int lane) {
  constexpr int V8 = Elem<T>::kVec;
  return (e / V8) * (kWave * V8) + lane * V8 + (e % V8);
}

// One 16-byte streaming load of logits: nontemporal, so the line is not kept
// in the caches for reuse.  A read-only probe over 1.88 GB in 8 KiB pieces per
// wave streams at 6.8 TB/s this way against 6.06 TB/s with plain loads, and the
// statistics pass went from 314 to 281 us at B=256, K=7, V=262144.  The
// sampling pass keeps plain loads (its raw-tile loader below): nontemporal
// ones measured the same there.
__device__ __forceinline__ u32x4 stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Load the lane's L*kVec elements of tile t (tiles of kWave*L*kVec ids) of a
// row of V logits as float; ids >= V read as -inf.  kAligned requires a
// 16-byte aligned row and V % kVec == 0, so a 16-byte vector is either fully
// inside the row or fully out.  `first` skips the tile's first loads (a wave
// that owns only part of a tile).
template <typename T, bool kAligned, int L, int N>
__device__ __forceinline__ void load_tile(const T* __restrict__ row, int V, int t, int lane, float (&x)[N],
                                          int first = 0) {
  constexpr int V8 = Elem<T>::kVec;
  static_assert(N % V8 == 0 && N / V8 <= L, "tile slice");
  constexpr int kL = N / V8;
  const int base = t * (kWave * L * V8) + first * (kWave * V8) + lane * V8;
  if constexpr (kAligned) {
    u32x4 raw[kL];
    // A slice wholly inside the row (every slice but the last of a row whose
    // length is not a tile multiple) loads without per-vector range checks.
    if (t * (kWave * L * V8) + (first + kL) * (kWave * V8) <= V) {
#pragma unroll
      for (int j = 0; j < kL; ++j) raw[j] = stream16(row + base + j * (kWave * V8));
    } else {
#pragma unroll
      for (int j = 0; j < kL; ++j) {
        const int off = base + j * (kWave * V8);
        if (off < V) {
          raw[j] = stream16(row + off);
        } else {
          const uint32_t ninf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
          raw[j] = u32x4{ninf, ninf, ninf, ninf};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[j * 8 + 2 * q] = bf16_lo(raw[j][q]);
          x[j * 8 + 2 * q + 1] = bf16_hi(raw[j][q]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[j * 4 + q] = __uint_as_float(raw[j][q]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kL; ++j) {
#pragma unroll
      for (int k = 0; k < V8; ++k) {
        const int off = base + j * (kWave * V8) + k;
        x[j * V8 + k] = off < V ? to_f32(row[off]) : -__builtin_inff();
      }
    }
  }
}

// The same tile slice kept in its storage format: NL 16-byte vectors per lane
// (8 bf16 or 4 f32 each), -inf beyond V.  Kernels that hold a tile across a
// long computation keep it packed (half the registers for bf16) and unpack an
// element when they use it with raw_elem; the values are bit-identical to
// load_tile's.
template <typename T, bool kAligned, int L, int NL>
__device__ __forceinline__ void load_raw(const T* __restrict__ row, int V, int t, int lane, u32x4 (&raw)[NL]) {
  constexpr int V8 = Elem<T>::kVec;
  static_assert(NL <= L, "tile slice");
  const int base = t * (kWave * L * V8) + lane * V8;
  constexpr uint32_t kNinf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
  if constexpr (kAligned) {
    if (t * (kWave * L * V8) + NL * (kWave * V8) <= V) {
#pragma unroll
      for (int j = 0; j < NL; ++j) raw[j] = *reinterpret_cast<const u32x4*>(row + base + j * (kWave * V8));
    } else {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int off = base + j * (kWave * V8);
        raw[j] = off < V ? *reinterpret_cast<const u32x4*>(row + off) : u32x4{kNinf, kNinf, kNinf, kNinf};
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (sizeof(T) == 2) {
          const int off = base + j * (kWave * V8) + 2 * q;
          const uint32_t lo = off < V ? (uint32_t)row[off] : 0xff80u;
          const uint32_t hi = off + 1 < V ? (uint32_t)row[off + 1] : 0xff80u;
          raw[j][q] = lo | (hi << 16);
        } else {
          const int off = base + j * (kWave * V8) + q;
          raw[j][q] = off < V ? __float_as_uint(row[off]) : kNinf;
        }
      }
    }
  }
}

// Element e (0 .. NL*kVec-1, in the lane's token-id order) of a packed slice.
template <typename T, int NL>
__device__ __forceinline__ float raw_elem(const u32x4 (&raw)[NL], int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = raw[e / 8][(e % 8) / 2];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return __uint_as_float(raw[e / 4][e % 4]);
  }
}

template <typename T, int NL>
__device__ __forceinline__ float raw_lane_max(const u32x4 (&raw)[NL]) {
  float m = raw_elem<T>(raw, 0);
#pragma unroll
  for (int e = 1; e < NL * Elem<T>::kVec; ++e) m = fmaxf(m, raw_elem<T>(raw, e));
  return m;
}

template <int N>
__device__ __forceinline__ float lane_max(const float (&x)[N]) {
  float m = x[0];
#pragma unroll
  for (int e = 1; e < N; ++e) m = fmaxf(m, x[e]);
  return m;
}

// Wave-wide reductions with DPP lane moves (gfx9 encodings): two quad
// permutes, the half-row and row mirrors, then row_bcast15 / row_bcast31
// carry row results into rows 1 and 3, 2 and 3.  Lane 63 ends with the
// result, which readlane returns to every lane.  No LDS traffic, one VALU
// operation per step.
namespace dpp {
constexpr int kQuadSwap1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kBcast15 = 0x142;
constexpr int kBcast31 = 0x143;
constexpr int kShr1 = 0x111;  // row_shr:1 (within rows of 16 lanes)
constexpr int kShr2 = 0x112;
constexpr int kShr4 = 0x114;
constexpr int kShr8 = 0x118;

template <int kCtrl, int kRowMask>
__device__ __forceinline__ int mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, kCtrl, kRowMask, 0xf, false);
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float mov(float old, float v) {
  return __int_as_float(mov<kCtrl, kRowMask>(__float_as_int(old), __float_as_int(v)));
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double mov(double old, double v) {
  const int lo = mov<kCtrl, kRowMask>((int)__double2loint(old), (int)__double2loint(v));
  const int hi = mov<kCtrl, kRowMask>((int)__double2hiint(old), (int)__double2hiint(v));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ __forceinline__ float lane63(float v) { return __int_as_float(lane63(__float_as_int(v))); }
__device__ __forceinline__ double lane63(double v) {
  return __hiloint2double(lane63((int)__double2hiint(v)), lane63((int)__double2loint(v)));
}

// Reduce with op; `id` is op's identity (what disabled lanes contribute).
template <typename V, typename Op>
__device__ __forceinline__ V reduce(V v, V id, Op op) {
  v = op(v, mov<kQuadSwap1, 0xf>(id, v));
  v = op(v, mov<kQuadSwap2, 0xf>(id, v));
  v = op(v, mov<kHalfMirror, 0xf>(id, v));
  v = op(v, mov<kMirror, 0xf>(id, v));
  v = op(v, mov<kBcast15, 0xa>(id, v));
  v = op(v, mov<kBcast31, 0xc>(id, v));
  return lane63(v);
}
}  // namespace dpp

__device__ __forceinline__ float wave_max(float v) {
  return dpp::reduce(v, -__builtin_inff(), [](float x, float y) { return fmaxf(x, y); });
}

__device__ __forceinline__ float wave_sum(float v) {
  return dpp::reduce(v, 0.0f, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ double wave_sum(double v) {
  return dpp::reduce(v, 0.0, [](double x, double y) { return x + y; });
}

__device__ __forceinline__ int wave_min(int v) {
  return dpp::reduce(v, 0x7fffffff, [](int x, int y) { return min(x, y); });
}

__device__ __forceinline__ int wave_max(int v) {
  return dpp::reduce(v, (int)0x80000000, [](int x, int y) { return max(x, y); });
}

// Inclusive prefix sum over the 64 lanes in lane order, with DPP lane moves:
// row shifts by 1, 2, 4 and 8 scan each row of 16 lanes (a lane shifted in
// from outside its row adds 0), then row_bcast15 adds row 0's total to row 1
// and row 2's to row 3, and row_bcast31 the total of rows 0-1 to rows 2-3.
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  v += dpp::mov<dpp::kShr1, 0xf>(0.0, v);
  v += dpp::mov<dpp::kShr2, 0xf>(0.0, v);
  v += dpp::mov<dpp::kShr4, 0xf>(0.0, v);
  v += dpp::mov<dpp::kShr8, 0xf>(0.0, v);
  v += dpp::mov<dpp::kBcast15, 0xa>(0.0, v);
  v += dpp::mov<dpp::kBcast31, 0xc>(0.0, v);
  return v;
}

// Block-wide reductions for a 256-thread block; `sh` is kWavesPerBlock doubles of LDS.
__device__ __forceinline__ double block_sum(double v, double* sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_sum(v);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) r += sh[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float* sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_max(v);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kWavesPerBlock; ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_min(int v, int* sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_min(v);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int i = 1; i < kWavesPerBlock; ++i) r = min(r, sh[i]);
  __syncthreads();
  return r;
}

// Fast 2^((x - m) * s) for the row statistics pass: hardware v_exp_f32 on a
// float32 argument.  Used where relative errors of ~1e-7 are harmless.
__device__ __forceinline__ float exp2_fast(float a) { return __builtin_amdgcn_exp2f(a); }

// Exponentials of the sampling pass.  A tile with reference (maximum) m
// takes hi = RN(m * s) once; each element is then 2^RN(x * s - hi): one FMA
// (x * s - hi exact before its single rounding) and v_exp_f32, under one ulp.
// The exact remainder lo = m * s - hi is put back where tiles are combined, as
// the factor 2^-lo on the tile's weight and in the positive-set ratio, so
// every value is 2^((x - m) * s) to within that rounding.  An earlier form,
// RN((x - m) * s) with a clamp for -inf tiles, took three instructions per
// element instead of one and has the same per-element error (a float32-exact
// emulation over B=256, K=7, V=262144 rows: RMS 2.95e-7 against fp64 for
// both); a compensated form that also recovered the product's rounding
// error took five more and gave no better agreement with the fp64 oracle.
// A reference of -inf (a tile that is all -inf) gets hi = +inf, so every
// element's argument is -inf and its value 0 without a per-element select.
__device__ __forceinline__ float exp_ref_hi(float m, float s) {
#pragma clang fp contract(off)
  return m == -__builtin_inff() ? __builtin_inff() : m * s;
}

// Wide references: |m * s| at or above 2^26.  The remainder lo of RN(m * s)
// is half an ulp of m * s at most, so it grows with |m * s| (up to 2 at 2^26,
// hundreds past 2^32), and once it nears 128 the one-FMA element value
// 2^((x - m) * s + lo) leaves the fp32 range: every element of a row
// overflows or underflows.  Elements of a tile with a wide reference take
// RN((x - m) * s) instead (x - m is exact for every x near enough to m to
// carry weight, since |m| is then far above the distance), and such a
// reference has no remainder to take out (exp_ref_lo returns 0).  This is
// the case only when the logits' magnitude over T exceeds about 2^25.5
// (logits near 10 at T below about 2e-7).  -inf references are never wide.
constexpr float kExpRefWide = 67108864.0f;  // 2^26
__device__ __forceinline__ bool exp_ref_wide(float m, float s) {
#pragma clang fp contract(off)
  return m != -__builtin_inff() && !(__builtin_fabsf(m * s) < kExpRefWide);
}

// 2^RN((x - m) * s), the element value under a wide reference.
__device__ __forceinline__ float exp2_wide(float x, float m, float s) {
#pragma clang fp contract(off)
  return __builtin_amdgcn_exp2f((x - m) * s);
}

// lo = m * s - RN(m * s), exact; |lo| <= 2^-25 |m * s|; 0 when m is -inf or
// wide.
__device__ __forceinline__ float exp_ref_lo(float m, float s) {
#pragma clang fp contract(off)
  if (m == -__builtin_inff() || exp_ref_wide(m, s)) return 0.0f;
  const float hi = m * s;
  return __builtin_fmaf(m, s, -hi);
}

// 2^-lo in fp64: e^-t with t = lo ln 2, five Taylor terms (relative error
// under t^5 / 120 < 1e-17 while |t| < 1e-3, i.e. |m * s| below about 4.8e4).
__device__ __forceinline__ double exp_ref_scale(float m, float s) {
  const double t = (double)exp_ref_lo(m, s) * 0.69314718055994530942;
  if (__builtin_fabs(t) >= 1e-3) return exp(-t);
  return 1.0 + t * (-1.0 + t * (0.5 + t * (-1.0 / 6.0 + t * (1.0 / 24.0))));
}

__device__ __forceinline__ float exp2_ref(float x, float s, float hi) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, s, -hi));
}

}  // namespace sv
