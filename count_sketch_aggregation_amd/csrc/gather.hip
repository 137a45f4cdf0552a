// gather.hip -- the lossless comparator: the exact sum of the workers' sparse gradients from
// their compacted (index, value) lists, the quantity the sketch path estimates.
//
// S2 Reducer (arXiv 2110.02140) Section 1 and Section 2.2 with Fig. 1(b): without a
// mergeable structure, sparse gradients are synchronised by gathering every worker's indices
// and values and adding them afterwards.  On one GPU the W gathered lists are resident
// already (s2r_encode writes them), so what remains is the scatter-add:
//   k_gather_fill   out = +0.0 with 128-bit stores, one workgroup per 32 KiB in XCD runs
//                   (non-temporal when the output exceeds the Infinity Cache);
//   k_gather_add    one launch per worker k = 0..W-1, in that order: every entry t of worker
//                   k's list adds val[k][t] into out[idx[k][t]].  A worker's indices are
//                   distinct, so the adds of one launch never collide and need no atomics;
//                   the launches run in worker order on one stream, so each element is the
//                   fp32 sum of its contributions in worker order, the same on every run.
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kGatherPer = 4;    // list entries per thread, loads issued together
constexpr int kFillStores = 8;   // float4 stores per thread: 32 KiB per workgroup

// Workgroup b (in XCD runs of 64, 2 MiB) zeroes float4 groups [b, b + 1) * 2048, each store
// instruction of a wave covering 1 KiB; workgroup 0 also zeroes the n % 4 trailing floats.
template <bool NT>
__global__ __launch_bounds__(kGatherThreads) void k_gather_fill(float* __restrict__ out,
                                                                uint64_t n) {
  const uint64_t n4 = n / 4;
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const uint64_t base = xcd_run_item(blockIdx.x, gridDim.x, 64) * kGatherThreads * kFillStores;
#pragma unroll
  for (int r = 0; r < kFillStores; ++r) {
    const uint64_t q = base + threadIdx.x + (uint64_t)kGatherThreads * r;
    if (q < n4) {
      if (NT) __builtin_nontemporal_store(z, &o4[q]);
      else o4[q] = z;
    }
  }
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
  const uint64_t per = (uint64_t)kGatherThreads * kFillStores;
  uint64_t blocks = (n / 4 + per - 1) / per;
  if (blocks == 0) blocks = 1;  // n < 4: workgroup 0 writes the trailing floats
  // an output larger than the Infinity Cache is written past it (measured on MI355X: the
  // 10^9-element workload's 4 GB fill 0.80 ms with cached stores)
  trace_mark(s, "k_gather_fill");
  if (n * sizeof(float) > kCacheResidentBytes)
    hipLaunchKernelGGL(k_gather_fill<true>, dim3((uint32_t)blocks), dim3(kGatherThreads), 0, s,
                       out, n);
  else
    hipLaunchKernelGGL(k_gather_fill<false>, dim3((uint32_t)blocks), dim3(kGatherThreads), 0, s,
                       out, n);
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
