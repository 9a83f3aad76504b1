// Streaming-read probe: the device's practical read ceiling for the row kernels'
// access pattern (16-byte non-temporal loads, eight in flight per lane).
#include <algorithm>

#include "vrt_dev.hpp"
#include "vrt_internal.hpp"

namespace vrt {
namespace {

constexpr int kPT = 256;   // threads per block
constexpr int kPL = 8;     // 16-byte loads in flight per lane

__global__ __launch_bounds__(kPT) void k_read_probe(const u32x4_t* buf, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kPT * kPL;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * kPT * kPL + threadIdx.x; base < n16; base += stride) {
    u32x4_t v[kPL];
#pragma unroll
    for (int q = 0; q < kPL; ++q) {
      const int64_t k = base + (int64_t)q * kPT;
      v[q] = k < n16 ? __builtin_nontemporal_load(buf + k) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < kPL; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
  }
  acc = wave_reduce(acc, [](uint32_t x, uint32_t y) { return x ^ y; });
  if (lane_id() == 0 && acc == 0x9E3779B9u) sink[0] = acc;  // practically never taken
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int dev = 0, cus = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t need = (n16 + (int64_t)kPT * kPL - 1) / ((int64_t)kPT * kPL);
  const int blocks = (int)std::min<int64_t>(need, (int64_t)cus * 8);
  hipLaunchKernelGGL(k_read_probe, dim3(blocks > 0 ? blocks : 1), dim3(kPT), 0, stream,
                     (const u32x4_t*)buf, n16, sink);
  return hipGetLastError();
}

}  // namespace vrt
