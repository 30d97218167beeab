// HBM read probe: the rate at which this GPU streams a buffer it reads once, as the
// achievable ceiling that the kernels' rates are compared with (next to the nominal
// 8 TB/s).  Each thread loads 16-byte pieces at a grid stride, every load of a
// round in flight before any is used, and folds them into one word per workgroup
// so that no load can be dropped.
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* buf, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= buf[i];
  const uint32_t w = wave_reduce_u32(acc[0] ^ acc[1] ^ acc[2] ^ acc[3], [](uint32_t a, uint32_t b) { return a ^ b; }, 0u);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = w;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s, int tid) {
  V4A_LAUNCH(tid, read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s,
             reinterpret_cast<const u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace v4a
