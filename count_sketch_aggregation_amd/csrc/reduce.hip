// reduce.hip -- aggregation of W workers' sketches and bitmaps on one GPU.
//
// S2 Reducer (arXiv 2110.02140) Section 3.1 "Collecting Sparse-Sketch with AllReduce": the
// sketch is the linear map A^T g, so the sketches of W workers add element-wise to the
// sketch of the summed gradient; the merged bitmap marks the union of non-zero positions.
// With the W workers resident as W buffers of one GPU, the AllReduce becomes this
// streaming pass: sum in worker order k = 0..W-1 (fixed, so the fp32 result is
// reproducible) and OR of the bitmap words.  HBM-bound: W reads + 1 write per cell.
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroups [0, sblocks) sum the sketches, the rest OR the bitmaps, so that every
// workgroup streams one kind of data.  Grid-stride over each range.
template <bool VS, bool VB>
__global__ __launch_bounds__(256) void k_reduce(uint32_t W, uint64_t cells, uint64_t words,
                                                uint32_t sblocks,
                                                const uint64_t* __restrict__ bitmaps,
                                                const float* sketches, uint64_t* bitmap_out,
                                                float* sketch_out) {
  // no __restrict__ on sketches / sketch_out: they may alias (in place into slot 0)
  if (blockIdx.x < sblocks) {
    const uint64_t stride = (uint64_t)sblocks * blockDim.x;
    // 4 KiB of each worker per workgroup and pass: XCD runs of 2 MiB (xcd_run_item)
    const uint64_t gid = xcd_run_item(blockIdx.x, sblocks, 512) * blockDim.x + threadIdx.x;
    if constexpr (VS) {
      const uint64_t c4 = cells / 4;
      const f32x4* in = reinterpret_cast<const f32x4*>(sketches);
      f32x4* out = reinterpret_cast<f32x4*>(sketch_out);
      for (uint64_t c = gid; c < c4; c += stride) {
        f32x4 acc = __builtin_nontemporal_load(in + c);
        for (uint32_t k = 1; k < W; ++k) acc += __builtin_nontemporal_load(in + (uint64_t)k * c4 + c);
        // non-temporal: the merged sketch is read once by the decode, well after this pass
        // (measured on MI355X: 9 us faster over the 1e9-element workload's 2.6 GB, same elsewhere)
        __builtin_nontemporal_store(acc, out + c);
      }
    } else {
      for (uint64_t c = gid; c < cells; c += stride) {
        float acc = sketches[c];
        for (uint32_t k = 1; k < W; ++k) acc += sketches[(uint64_t)k * cells + c];
        sketch_out[c] = acc;
      }
    }
    return;
  }
  const uint32_t bblocks = gridDim.x - sblocks;
  const uint64_t stride = (uint64_t)bblocks * blockDim.x;
  const uint64_t gid = xcd_run_item(blockIdx.x - sblocks, bblocks, 512) * blockDim.x + threadIdx.x;
  if constexpr (VB) {  // pairs of words, 128-bit loads (words even, 16-byte aligned rows)
    // non-temporal loads: the bitmaps are read once (measured on MI355X: 455 -> 437 us over
    // the 1e9-element workload's 2.6 GB, no change on the smaller ones)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint64_t w2 = words / 2;
    const u32x4* in = reinterpret_cast<const u32x4*>(bitmaps);
    u32x4* out = reinterpret_cast<u32x4*>(bitmap_out);
    for (uint64_t q = gid; q < w2; q += stride) {
      u32x4 m = __builtin_nontemporal_load(in + q);
      for (uint32_t k = 1; k < W; ++k) m |= __builtin_nontemporal_load(in + (uint64_t)k * w2 + q);
      out[q] = m;
    }
  } else {
    for (uint64_t q = gid; q < words; q += stride) {
      uint64_t m = 0;
      for (uint32_t k = 0; k < W; ++k) m |= bitmaps[(uint64_t)k * words + q];
      bitmap_out[q] = m;
    }
  }
}

hipError_t launch_reduce(uint32_t W, uint64_t cells, uint64_t words, const uint64_t* bitmaps,
                         const float* sketches, uint64_t* bitmap_out, float* sketch_out,
                         hipStream_t s) {
  const bool vs = (cells % 4 == 0) && (reinterpret_cast<uintptr_t>(sketches) % 16 == 0) &&
                  (reinterpret_cast<uintptr_t>(sketch_out) % 16 == 0);
  const bool vb = (words % 2 == 0) && (reinterpret_cast<uintptr_t>(bitmaps) % 16 == 0) &&
                  (reinterpret_cast<uintptr_t>(bitmap_out) % 16 == 0);
  const uint64_t su = vs ? cells / 4 : cells, bu = vb ? words / 2 : words;
  // grid-stride beyond 65536 workgroups in all (measured on MI355X over 2.6 GB: 2% faster
  // than a cap of 16384, 7% faster than 4096), split in proportion to the units of each part
  const uint64_t total = su + bu;
  if (total == 0) return hipSuccess;
  uint64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  uint64_t sblocks = su ? (blocks * su + total - 1) / total : 0;
  if (su && sblocks == 0) sblocks = 1;
  // a multiple of 8, so that the bitmap part's workgroups start on XCD 0 (xcd_run_item)
  if (sblocks > kXcds) sblocks = (sblocks + kXcds - 1) / kXcds * kXcds;
  uint64_t bblocks = blocks > sblocks ? blocks - sblocks : 0;
  if (bu && bblocks == 0) bblocks = 1;
  const dim3 grid((uint32_t)(sblocks + bblocks));
  trace_mark(s, "k_reduce");
  if (vs && vb)
    hipLaunchKernelGGL((k_reduce<true, true>), grid, dim3(256), 0, s, W, cells, words,
                       (uint32_t)sblocks, bitmaps, sketches, bitmap_out, sketch_out);
  else if (vs)
    hipLaunchKernelGGL((k_reduce<true, false>), grid, dim3(256), 0, s, W, cells, words,
                       (uint32_t)sblocks, bitmaps, sketches, bitmap_out, sketch_out);
  else if (vb)
    hipLaunchKernelGGL((k_reduce<false, true>), grid, dim3(256), 0, s, W, cells, words,
                       (uint32_t)sblocks, bitmaps, sketches, bitmap_out, sketch_out);
  else
    hipLaunchKernelGGL((k_reduce<false, false>), grid, dim3(256), 0, s, W, cells, words,
                       (uint32_t)sblocks, bitmaps, sketches, bitmap_out, sketch_out);
  return hipGetLastError();
}

}  // namespace s2r
