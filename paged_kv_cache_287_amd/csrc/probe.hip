// Streaming-read bandwidth probe: the attainable HBM read rate that the decode kernel is
// compared against. Every lane reads 16-byte chunks in a grid-stride loop with four
// independent loads in flight and folds them into a register; the single conditional store
// keeps the loads live without adding traffic.
#include "pa_internal.hpp"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) +
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n = bytes / 16;
  stream_read_kernel<<<8192, 256, 0, stream>>>(static_cast<const uint4*>(buf), n, sink);
  return hipGetLastError();
}

}  // namespace pa
