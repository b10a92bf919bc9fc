// msa_stream.hip -- a plain streaming read of a device buffer: the practical
// HBM read ceiling the index scan is measured against (the scan is a read of
// 72 B per context token with a few operations per byte, so its bound is
// this kernel's rate, below the 8 TB/s the part is rated for).
//
// Every workgroup reads one contiguous share of the buffer with 16-byte
// non-temporal loads (the scan's own load form), four per thread in flight,
// and folds them into one XOR that is stored only if it equals a value no
// input produces by chance, so the loads cannot be removed and almost
// nothing is written.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint8_t* __restrict__ src, int64_t n16,
                                                                     int64_t per_wg, uint32_t* __restrict__ sink) {
  const int64_t lo = (int64_t)blockIdx.x * per_wg, hi = min(lo + per_wg, n16);
  uint32_t acc = 0;
  constexpr int64_t kStep = (int64_t)kStreamThreads * kStreamUnroll;
  int64_t i = lo + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * kStreamThreads < hi; i += kStep) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = nt_load4(src + (i + u * kStreamThreads) * 16);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kStreamThreads) {
    const uint4 v = nt_load4(src + i * 16);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace msa

using namespace msa;

extern "C" int msa_launch_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink,
                                      hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kStreamThreads), 0, s, (const uint8_t*)src, n16,
                     per_wg, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
