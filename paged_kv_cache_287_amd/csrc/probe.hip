// Streaming-read bandwidth probe: the attainable HBM read rate that the decode kernel is
// compared against. Every lane reads 16-byte chunks with non-temporal loads in a grid-stride
// loop with four independent loads in flight and folds them into a register; the single
// conditional store keeps the loads live without adding traffic. The shape (non-temporal,
// four loads in flight, 65536 workgroups of 256) was the fastest of a sweep over grid sizes,
// loads in flight and chunking on MI355X.
#include "pa_internal.hpp"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 nt_load(const uint4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = nt_load(p + i), b = nt_load(p + i + stride), c = nt_load(p + i + 2 * stride),
                d = nt_load(p + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) +
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n; i += stride) {
    const u32x4 a = nt_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n = bytes / 16;
  stream_read_kernel<<<65536, 256, 0, stream>>>(static_cast<const uint4*>(buf), n, sink);
  return hipGetLastError();
}

}  // namespace pa
