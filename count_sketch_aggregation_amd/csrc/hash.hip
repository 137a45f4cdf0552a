// hash.hip -- test hook exposing the device bucket/sign hashes of Algorithm 1
// (S2 Reducer, arXiv 2110.02140, Section 3.1: items are "randomly mapped" to a bucket by
// h_j with a random sign s_j).  Uses the very device functions the encode and decode
// kernels call.
#include "s2r_launch.hpp"

namespace s2r {

template <int D>
__global__ __launch_bounds__(256) void k_hash(HashArgs h, const uint32_t* __restrict__ keys,
                                              uint64_t m, uint32_t* __restrict__ buckets,
                                              int8_t* __restrict__ signs) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < m; t += stride) {
    const uint32_t i = keys[t];
    const uint32_t part = partition_of(h, i);
#pragma unroll
    for (int j = 0; j < D; ++j) {
      buckets[(uint64_t)j * m + t] = bucket_of(h, part, j, i);
      signs[(uint64_t)j * m + t] = sign_mask(h, j, i) ? (int8_t)-1 : (int8_t)1;
    }
  }
}

hipError_t launch_hash(const HashArgs& h, const uint32_t* keys, uint64_t m, uint32_t* buckets,
                       int8_t* signs, hipStream_t s) {
  if (m == 0) return hipSuccess;
  uint64_t blocks = (m + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  trace_mark(s, "k_hash");
  S2R_DISPATCH_D(h.d, hipLaunchKernelGGL((k_hash<D>), dim3((uint32_t)blocks), dim3(256), 0, s, h,
                                         keys, m, buckets, signs));
  return hipGetLastError();
}

}  // namespace s2r
