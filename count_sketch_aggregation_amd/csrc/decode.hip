// decode.hip -- decompression: merged bitmap + merged sketch -> dense g_hat.
//
// S2 Reducer (arXiv 2110.02140) Section 3.1 "Decompressing Sparse Gradient" and the query
// loop of Algorithm 1: recover the indices from the set bits of the merged bitmap and, for
// each, take the median over rows j of s_j(i) * S[j, h_j(i)]; clear bits decode to +0.0.
//
// k_decode_direct: one workgroup per 4096 output elements (64 bitmap words).  Wave 0 loads
// the words, ranks the set bits with a wave prefix sum and lists their local offsets in LDS;
// every thread then takes whole items (d hashed gathers from the sketch + a register
// median) and writes the result into an LDS copy of the output tile, which is finally
// stored with 128-bit coalesced writes (zeros included).
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecTile = 4096;
constexpr int kDecWords = kDecTile / 64;

template <int D>
__global__ __launch_bounds__(kDecThreads) void k_decode_direct(
    HashArgs h, uint64_t n, uint64_t nwords, const uint64_t* __restrict__ bitmap,
    const float* __restrict__ sketch, uint64_t w, float* __restrict__ out) {
  __shared__ float otile[kDecTile];
  __shared__ uint16_t items[kDecTile];
  __shared__ uint32_t count;
  const int tid = threadIdx.x;
  const uint64_t base = (uint64_t)blockIdx.x * kDecTile;

  for (int c = tid; c < kDecTile; c += kDecThreads) otile[c] = 0.f;
  if (tid < kWave) {
    const uint64_t q = (uint64_t)blockIdx.x * kDecWords + tid;
    uint64_t wv = q < nwords ? bitmap[q] : 0ull;
    const uint64_t first = q * 64;  // bits at or beyond n are ignored
    if (first >= n) wv = 0;
    else if (n - first < 64) wv &= (1ull << (n - first)) - 1ull;
    const uint32_t pc = (uint32_t)__popcll(wv);
    const uint32_t inc = wave_inclusive_sum(pc);
    uint32_t slot = inc - pc;
    while (wv) {
      const int b = __builtin_ctzll(wv);
      wv &= wv - 1;
      items[slot++] = (uint16_t)(tid * 64 + b);
    }
    if (tid == kWave - 1) count = inc;
  }
  __syncthreads();
  const uint32_t cnt = count;
  for (uint32_t e = tid; e < cnt; e += kDecThreads) {
    const uint32_t li = items[e];
    const uint32_t i = (uint32_t)(base + li);
    const uint32_t part = partition_of(h, i);
    float v[D];
#pragma unroll
    for (int j = 0; j < D; ++j)
      v[j] = apply_sign(sketch[(uint64_t)j * w + bucket_of(h, part, j, i)], sign_mask(h, j, i));
    otile[li] = median_of<D>(v);
  }
  __syncthreads();
  if (base + kDecTile <= n) {
    f32x4* o = reinterpret_cast<f32x4*>(out + base);
    for (int c = tid; c < kDecTile / 4; c += kDecThreads)
      o[c] = *reinterpret_cast<const f32x4*>(&otile[4 * c]);
  } else {
    for (int c = tid; c < kDecTile; c += kDecThreads)
      if (base + c < n) out[base + c] = otile[c];
  }
}

hipError_t launch_decode_direct(const HashArgs& h, uint64_t n, const uint64_t* bitmap,
                                const float* sketch, uint64_t w, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t blocks = (n + kDecTile - 1) / kDecTile;
  const uint64_t nwords = (n + 63) / 64;
  S2R_DISPATCH_D(h.d, hipLaunchKernelGGL((k_decode_direct<D>), dim3((uint32_t)blocks),
                                         dim3(kDecThreads), 0, s, h, n, nwords, bitmap, sketch, w,
                                         out));
  return hipGetLastError();
}

}  // namespace s2r
