// Calibration of the achievable HBM read rate.  The decode is bound by the
// bandwidth of its cache read (onedev.kr review, "Premises and limits":
// decode is dominated by reading the cache), so its rate is stated beside
// a plain streaming read of the same bytes with the same load form: 16-byte
// non-temporal loads, eight in flight per lane, each block over one
// contiguous range.  The words read are folded into a 32-bit XOR per block,
// so no load can be dropped and the result can be checked exactly.
#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               size_t n16,
                                                               uint32_t* __restrict__ xor_out) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = min(n16, per * blockIdx.x);
  const size_t end = min(n16, begin + per);
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < end; i += kThreads) acc ^= __builtin_nontemporal_load(src + i);
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ unsigned red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) r ^= red[w];
    xor_out[blockIdx.x] = r;
  }
}

}  // namespace

// bytes a multiple of 16 and buf 16-byte aligned (checked by the caller);
// every one of the `blocks` output words is written.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* xor_out, int blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, xor_out);
  return hipGetLastError();
}

}  // namespace gva
