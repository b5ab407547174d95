// Bandwidth calibration: a plain streaming read or copy of a device buffer,
// the yardstick the HBM-bound kernels of this library are measured against.
// Each workgroup streams one contiguous chunk of the buffer, each thread with
// sixteen 16-byte loads in flight (contiguous chunks measured ahead of a
// grid-stride loop, and sixteen loads ahead of four or eight, on a 1 GiB
// buffer); a read-only pass folds its data into one word per thread that is
// written only when the (never given) sink pointer is set, so the loads stay.
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int CAL_THREADS = 256;
constexpr int CAL_UNROLL = 16;
constexpr int64_t CAL_GRID = 2048;  // eight workgroups per compute unit

__global__ __launch_bounds__(CAL_THREADS) void calib_stream_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n16, int64_t chunk,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
  uint32_t acc = 0u;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += (int64_t)CAL_THREADS * CAL_UNROLL) {
    u32x4 v[CAL_UNROLL];
#pragma unroll
    for (int u = 0; u < CAL_UNROLL; ++u) {
      const int64_t j = i + (int64_t)CAL_THREADS * u;
      v[u] = j < b1 ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
    if (dst != nullptr) {
#pragma unroll
      for (int u = 0; u < CAL_UNROLL; ++u) {
        const int64_t j = i + (int64_t)CAL_THREADS * u;
        if (j < b1) __builtin_nontemporal_store(v[u], dst + j);
      }
    } else {
#pragma unroll
      for (int u = 0; u < CAL_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (sink != nullptr) sink[(int64_t)blockIdx.x * CAL_THREADS + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_calib_stream(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t grid = n16 < CAL_GRID ? (n16 < 1 ? 1 : n16) : CAL_GRID;
  const int64_t chunk = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(calib_stream_kernel, dim3((unsigned)grid), dim3(CAL_THREADS), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16, chunk,
                     static_cast<uint32_t*>(nullptr));
  return hipGetLastError();
}

}  // namespace dsa
