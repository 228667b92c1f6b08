// Streaming-read probe for MI355X (gfx950): the practical HBM read rate of
// this machine, measured with the access pattern of the attention kernels
// (each wave streams its own contiguous region with 16-byte non-temporal
// loads, sixteen in flight per lane: the fastest of the patterns measured,
// 6.9 TB/s over 1 GiB against 6.4-6.6 with eight).  It gives the attention
// roofline a measured ceiling next to the published 8 TB/s.  Every 16-byte unit is read
// exactly once; thread t writes the XOR of the words it read to sink[t], so
// a caller can check that the whole buffer was read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hda.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void hda_read_probe_kernel(const u32x4* __restrict__ p,
                                                                       int64_t n16,
                                                                       uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const int64_t wave = t >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * kProbeThreads) >> 6;
  const int64_t per = (n16 + n_waves - 1) / n_waves;      // 16-byte units per wave
  const int64_t begin = wave * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  uint32_t acc = 0;
  int64_t i = begin + lane;
  for (; i + 64 * (kProbeUnroll - 1) < end; i += 64 * kProbeUnroll) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + 64 * u);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += 64) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[t] = acc;
}

}  // namespace

extern "C" int hda_read_probe(const void* buf, int64_t bytes, int32_t n_workgroups,
                              uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || n_workgroups < 1) return HDA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return HDA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(hda_read_probe_kernel, dim3(n_workgroups), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? HDA_OK : HDA_ERR_HIP;
}
