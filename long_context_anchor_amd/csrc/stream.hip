// Stream-read reference: reads a buffer once with the same 16-byte
// nontemporal loads the decode passes use and folds it into one word, so a
// read bandwidth can be measured beside the decode kernels' rates (a device
// copy both reads and writes, and library reductions read slower than the
// decode passes themselves).  Not part of the method.
#include "common.h"

namespace kc {

namespace {

constexpr int kStreamThreads = 1024;
constexpr int kStreamInFlight = 4;   // 16-byte loads per lane per iteration

// *sink ^= XOR of every 32-bit word of src[0 : n16) (n16 >= 1 words of 16
// bytes).  Workgroup b reads one contiguous range, [b*per, (b+1)*per): long
// per-CU streams measured faster than a grid-stride interleave (6.95 vs
// 6.43 TB/s over 4 GiB with one workgroup per CU).
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4* __restrict__ src, int64_t n16,
                                                                uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (int64_t base = lo + threadIdx.x; base < hi; base += (int64_t)kStreamThreads * kStreamInFlight) {
    uint4 v[kStreamInFlight];
    // reads clamped into the range and issued unconditionally; words past
    // its end count as zero
#pragma unroll
    for (int u = 0; u < kStreamInFlight; ++u) {
      const int64_t i = base + (int64_t)u * kStreamThreads;
      const uint4 w = ld16_nt(src + (i < hi ? i : hi - 1));
      v[u] = i < hi ? w : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kStreamInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, int grid, hipStream_t s) {
  if (n16 < 1 || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kStreamThreads), 0, s, reinterpret_cast<const uint4*>(src),
                     n16, sink);
  return hipGetLastError();
}

}  // namespace kc
