// diag.hip -- measurement helpers (include/s2r_diag.h): a plain streaming read, so the
// benchmark can state the achievable HBM read rate of the GPU it runs on.
#include "s2r_diag.h"
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDiagThreads = 256;
constexpr int kDiagLoads = 1;  // float4 loads per lane and iteration

__global__ __launch_bounds__(kDiagThreads) void k_diag_read(const f32x4* __restrict__ in,
                                                            uint64_t n4, float* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kDiagThreads;
  float acc = 0.f;
  for (uint64_t i0 = (uint64_t)blockIdx.x * kDiagThreads + threadIdx.x; i0 < n4;
       i0 += stride * kDiagLoads) {
    f32x4 v[kDiagLoads];
#pragma unroll
    for (int u = 0; u < kDiagLoads; ++u) {
      const uint64_t i = i0 + (uint64_t)u * stride;
      v[u] = i < n4 ? __builtin_nontemporal_load(in + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kDiagLoads; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  // keeps the loads alive; the sink receives one lane's value only when the sum is exactly 1
  if (acc == 1.0f) *sink = acc;
}

// 128-bit non-temporal stores of `value`, shaped like the decode's output pass: one
// 256-thread workgroup per 32 KiB, each thread storing kDiagStores float4 groups
// tid + 256 r (every store instruction of a wave covers 1 KiB), the workgroups in XCD runs
// of 2 MiB (xcd_run_item; measured on MI355X: 6.2-6.3 TB/s against 5.6 in round-robin order).
constexpr int kDiagStores = 8;

__global__ __launch_bounds__(kDiagThreads) void k_diag_write(f32x4* __restrict__ out, uint64_t n4,
                                                             float value) {
  const f32x4 v = {value, value, value, value};
  const uint64_t base = xcd_run_item(blockIdx.x, gridDim.x, 64) * kDiagThreads * kDiagStores;
#pragma unroll
  for (int r = 0; r < kDiagStores; ++r) {
    const uint64_t i = base + threadIdx.x + (uint64_t)kDiagThreads * r;
    if (i < n4) __builtin_nontemporal_store(v, &out[i]);
  }
}

}  // namespace s2r

extern "C" s2r_status s2r_diag_stream_write(void* buf, size_t bytes, float value, void* stream) {
  if (!buf) return S2R_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || bytes % 16 != 0) return S2R_ERR_ALIGN;
  const uint64_t n4 = bytes / 16;
  if (n4 == 0) return S2R_OK;
  const uint64_t per = (uint64_t)s2r::kDiagThreads * s2r::kDiagStores;
  const uint64_t blocks = (n4 + per - 1) / per;
  if (blocks > 0x7fffffffull) return S2R_ERR_DIM;
  s2r::trace_mark(static_cast<hipStream_t>(stream), "k_diag_write");
  hipLaunchKernelGGL(s2r::k_diag_write, dim3((uint32_t)blocks), dim3(s2r::kDiagThreads), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<s2r::f32x4*>(buf), n4,
                     value);
  return hipGetLastError() == hipSuccess ? S2R_OK : S2R_ERR_HIP;
}

extern "C" s2r_status s2r_diag_stream_read(const void* buf, size_t bytes, float* sink,
                                           void* stream) {
  if (!buf || !sink) return S2R_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || bytes % 16 != 0) return S2R_ERR_ALIGN;
  const uint64_t n4 = bytes / 16;
  if (n4 == 0) return S2R_OK;
  uint64_t blocks = (n4 + s2r::kDiagThreads * s2r::kDiagLoads - 1) /
                    (s2r::kDiagThreads * s2r::kDiagLoads);
  if (blocks > 2048) blocks = 2048;  // 2048 x 256 lanes, grid-stride: the best measured shape
  s2r::trace_mark(static_cast<hipStream_t>(stream), "k_diag_read");
  hipLaunchKernelGGL(s2r::k_diag_read, dim3((uint32_t)blocks), dim3(s2r::kDiagThreads), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const s2r::f32x4*>(buf),
                     n4, sink);
  return hipGetLastError() == hipSuccess ? S2R_OK : S2R_ERR_HIP;
}
