// Read-only streaming reference for the roofline figures: the statistics
// pass's access pattern (each wave reads 8 KiB contiguous in 16-byte
// nontemporal loads, four waves per block) with no arithmetic beyond an XOR,
// so its rate is the ceiling the streaming passes can be compared with.

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

namespace {

__global__ void __launch_bounds__(kBlock) read_stream_kernel(const u32x4* __restrict__ src, uint32_t* sink,
                                                             uint32_t magic) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const size_t base = ((size_t)blockIdx.x * kWavesPerBlock + wave) * (kWave * kLoads);
  u32x4 v[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) v[j] = __builtin_nontemporal_load(src + base + j * kWave + lane);
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  // data-dependent store, so no load can be dropped; never taken for real data
  if (x == magic) sink[0] = x;
}

}  // namespace

hipError_t launch_read_stream(const void* src, size_t bytes, void* sink, hipStream_t st) {
  const size_t per_block = (size_t)kBlock * kLoads * 16;  // 32 KiB
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)(bytes / per_block)), dim3(kBlock), 0, st,
                     static_cast<const u32x4*>(src), static_cast<uint32_t*>(sink), 0x9e3779b9u);
  return hipGetLastError();
}

}  // namespace sv
