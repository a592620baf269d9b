// Shortlisted drafter head: logits only on the union of the clusters each
// context selects (DynaSpec summary, lowest.today, "Model architecture",
// items 1, 3 and 4).  First version: one wave per (context, token), the hidden
// rows of the context's K positions against one W row, fp32 accumulation.

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

namespace {

struct HeadArgs {
  const uint16_t* h;   // bf16 [B, K, d]
  const uint16_t* W;   // bf16 [V, d]
  const int32_t* cids; // [B, n_sel]
  int B, K, d, V, cs, n_sel;
  float* compact;      // [B, K, n_sel*cs] or null
  void* dense;         // [B, K, V] or null
  int dense_bf16;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void __launch_bounds__(kBlock) fill_neg_inf(void* dense, size_t n, int bf16) {
  const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t k = i; k < n; k += stride) {
    if (bf16) static_cast<uint16_t*>(dense)[k] = 0xff80u;
    else static_cast<float*>(dense)[k] = -__builtin_inff();
  }
}

constexpr int kHeadMaxK = 8;

__global__ void __launch_bounds__(kBlock) head_rowdot_kernel(HeadArgs a) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int b = blockIdx.y;
  const int s = blockIdx.z;
  const int tok_in = blockIdx.x * kWavesPerBlock + wave;
  if (tok_in >= a.cs) return;
  const int c = a.cids[(size_t)b * a.n_sel + s];
  const int n_clusters = a.V / a.cs;
  if (c < 0 || c >= n_clusters) return;
  if (s > 0 && a.cids[(size_t)b * a.n_sel + s - 1] >= c) return;
  const int tok = c * a.cs + tok_in;
  const uint16_t* wrow = a.W + (size_t)tok * a.d;
  const int L = a.n_sel * a.cs;
  for (int k0 = 0; k0 < a.K; k0 += kHeadMaxK) {
    const int kn = min(kHeadMaxK, a.K - k0);
    float acc[kHeadMaxK];
#pragma unroll
    for (int k = 0; k < kHeadMaxK; ++k) acc[k] = 0.0f;
    for (int j = lane; j < a.d; j += kWave) {
      const float w = to_f32(wrow[j]);
#pragma unroll
      for (int k = 0; k < kHeadMaxK; ++k)
        if (k < kn) acc[k] = __builtin_fmaf(w, to_f32(a.h[((size_t)b * a.K + k0 + k) * a.d + j]), acc[k]);
    }
#pragma unroll
    for (int k = 0; k < kHeadMaxK; ++k) {
      if (k >= kn) break;
      const float v = wave_sum(acc[k]);
      if (lane == 0) {
        const size_t bk = (size_t)b * a.K + k0 + k;
        if (a.compact) a.compact[bk * L + (size_t)s * a.cs + tok_in] = v;
        if (a.dense) {
          if (a.dense_bf16) static_cast<uint16_t*>(a.dense)[bk * a.V + tok] = f32_to_bf16_rne(v);
          else static_cast<float*>(a.dense)[bk * a.V + tok] = v;
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
  if (dense) {
    const size_t n = (size_t)B * K * V;
    const unsigned blocks = (unsigned)std::min<size_t>((n + kBlock - 1) / kBlock, 8192);
    hipLaunchKernelGGL(fill_neg_inf, dim3(blocks), dim3(kBlock), 0, st, dense, n, a.dense_bf16);
  }
  if (n_sel > 0) {
    const dim3 grid((unsigned)((cluster_size + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)B, (unsigned)n_sel);
    hipLaunchKernelGGL(head_rowdot_kernel, grid, dim3(kBlock), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sv
