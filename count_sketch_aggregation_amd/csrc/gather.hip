// gather.hip -- the lossless comparator: the exact sum of the workers' sparse gradients from
// their compacted (index, value) lists, the quantity the sketch path estimates.
//
// S2 Reducer (arXiv 2110.02140) Section 1 and Section 2.2 with Fig. 1(b): without a
// mergeable structure, sparse gradients are synchronised by gathering every worker's indices
// and values and adding them afterwards.  On one GPU the W gathered lists are resident
// already (s2r_encode writes them), so what remains is the scatter-add:
//   k_gather_fill   out = +0.0 with 128-bit stores;
//   k_gather_add    one launch per worker k = 0..W-1, in that order: every entry t of worker
//                   k's list adds val[k][t] into out[idx[k][t]].  A worker's indices are
//                   distinct, so the adds of one launch never collide and need no atomics;
//                   the launches run in worker order on one stream, so each element is the
//                   fp32 sum of its contributions in worker order, the same on every run.
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kGatherPer = 4;  // list entries per thread, loads issued together

__global__ __launch_bounds__(kGatherThreads) void k_gather_fill(float* __restrict__ out,
                                                                uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kGatherThreads;
  const uint64_t n4 = n / 4;
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  for (uint64_t q = (uint64_t)blockIdx.x * kGatherThreads + threadIdx.x; q < n4; q += stride)
    o4[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) out[4 * n4 + threadIdx.x] = 0.f;
}

// Entries [0, min(nnz, cap)) of one worker's list; entries whose index is not below n are
// skipped.  The first worker's adds go into the zeros just written, so they store
// 0.0f + v without reading (the same value an add into +0.0 gives).
template <bool FIRST>
__global__ __launch_bounds__(kGatherThreads) void k_gather_add(const uint32_t* __restrict__ idx,
                                                               const float* __restrict__ val,
                                                               const uint64_t* __restrict__ nnz,
                                                               uint64_t cap, uint64_t n,
                                                               float* __restrict__ out) {
  const uint64_t len = *nnz < cap ? *nnz : cap;
  const uint64_t base = ((uint64_t)blockIdx.x * kGatherThreads) * kGatherPer + threadIdx.x;
  if (base >= len) return;
  uint32_t ii[kGatherPer];
  float vv[kGatherPer];
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const uint64_t t = base + (uint64_t)u * kGatherThreads;
    const uint64_t tc = t < len ? t : len - 1;  // len > 0 here: clamped, so all loads issue
    ii[u] = idx[tc];
    vv[u] = val[tc];
  }
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const uint64_t t = base + (uint64_t)u * kGatherThreads;
    if (t < len && ii[u] < n) {
      if (FIRST) out[ii[u]] = 0.f + vv[u];
      else out[ii[u]] += vv[u];
    }
  }
}

hipError_t launch_gather_sum(uint32_t W, const uint32_t* idx, const float* val, uint64_t cap,
                             const uint64_t* nnz, uint64_t n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  uint64_t blocks = (n / 4 + kGatherThreads - 1) / kGatherThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  trace_mark(s, "k_gather_fill");
  hipLaunchKernelGGL(k_gather_fill, dim3((uint32_t)blocks), dim3(kGatherThreads), 0, s, out, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || cap == 0) return e;
  const uint64_t per_block = (uint64_t)kGatherThreads * kGatherPer;
  const uint64_t gb = (cap + per_block - 1) / per_block;
  for (uint32_t k = 0; k < W; ++k) {
    trace_mark(s, "k_gather_add");
    if (k == 0)
      hipLaunchKernelGGL(k_gather_add<true>, dim3((uint32_t)gb), dim3(kGatherThreads), 0, s,
                         idx, val, nnz, cap, n, out);
    else
      hipLaunchKernelGGL(k_gather_add<false>, dim3((uint32_t)gb), dim3(kGatherThreads), 0, s,
                         idx + (uint64_t)k * cap, val + (uint64_t)k * cap, nnz + k, cap, n, out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace s2r
