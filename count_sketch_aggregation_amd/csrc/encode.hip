// encode.hip -- compression kernels: gradient -> bitmap + ordered non-zero list + sketch.
//
// Follows S2 Reducer (arXiv 2110.02140) Section 3.1 "Compressing Sparse Gradient" and the
// compression loop of Algorithm 1: mark every non-zero position in a bitmap, then add
// s_j(i) * g(i) into bucket h_j(i) of each row j for every non-zero g(i).
//
// Pipeline on gfx950 (all W workers batched in every launch):
//   k_stream      streams the gradient once with 128-bit loads; four 64-lane ballots per
//                 load round give four element-ordered bitmap words; writes the bitmap and
//                 one non-zero count per 8192-element tile.
//   k_scan        per worker: exclusive prefix of the tile counts (list offsets), the exact
//                 nnz, and for every 8192-entry list chunk the tile where it starts.
//   k_list_*      per list chunk: expands the chunk's bitmap bits into ascending
//                 (index, value) pairs in LDS, re-reading only the 16-byte groups of the
//                 gradient that hold a set bit, and writes the list with coalesced stores.
//                 Then either
//                   _atomic: adds every pair into the d rows with global fp32 atomics, or
//                   _bin:    counting-sorts the chunk by partition P(i) in LDS and writes
//                            the partition-ordered copy plus per-partition offsets;
//   k_accumulate  (partitioned path) one workgroup per (worker, partition): accumulates the
//                 partition's d x 2^K buckets in LDS with ds_add_f32 and writes them to the
//                 sketch with dense coalesced stores (no zero fill, no global atomics).
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// k_stream: grid (tiles, W), 256 threads.  Wave w of a tile owns 2048 consecutive elements
// (8 load rounds of 256): lane l of round r holds elements base + 256 r + 4 l .. +3, so the
// ballot of component c has bit l = element 4 l + c; interleaving the four ballots' 16-bit
// slices gives the 64-bit words of elements base + 256 r + 64 q.
__global__ __launch_bounds__(kStreamThreads) void k_stream(
    const float* __restrict__ grad, uint64_t n, uint64_t ld, uint64_t tiles, uint64_t words,
    uint64_t* __restrict__ bitmaps, uint32_t* __restrict__ counts) {
  const uint32_t t = blockIdx.x, k = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* row = grad + (uint64_t)k * ld;
  const uint64_t wave_base = (uint64_t)t * kTile + (uint64_t)wave * (kTile / 4);

  f32x4 v[kStreamVec];
#pragma unroll
  for (int r = 0; r < kStreamVec; ++r) {
    const uint64_t e = wave_base + r * 256 + lane * 4;
    // e is a multiple of 4 and ld % 4 == 0, so e < n <= ld keeps all four lanes in the row
    if (e < n) v[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e));
    else v[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint64_t myword = 0;
#pragma unroll
  for (int r = 0; r < kStreamVec; ++r) {
    const uint64_t e = wave_base + r * 256 + lane * 4;
    const uint64_t b0 = __ballot(e + 0 < n && nonzero_bits(v[r].x));
    const uint64_t b1 = __ballot(e + 1 < n && nonzero_bits(v[r].y));
    const uint64_t b2 = __ballot(e + 2 < n && nonzero_bits(v[r].z));
    const uint64_t b3 = __ballot(e + 3 < n && nonzero_bits(v[r].w));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sh = 16 * q;
      const uint64_t word = spread4(b0 >> sh) | (spread4(b1 >> sh) << 1) |
                            (spread4(b2 >> sh) << 2) | (spread4(b3 >> sh) << 3);
      if (lane == r * 4 + q) myword = word;
    }
  }
  const uint64_t gw = (uint64_t)t * kTileWords + wave * 32 + lane;
  if (lane < 32 && gw < words) bitmaps[(uint64_t)k * words + gw] = myword;

  uint32_t c = wave_sum(lane < 32 ? (uint32_t)__popcll(myword) : 0u);
  __shared__ uint32_t wcount[kStreamThreads / kWave];
  if (lane == 0) wcount[wave] = c;
  __syncthreads();
  if (tid == 0) counts[(uint64_t)k * tiles + t] = wcount[0] + wcount[1] + wcount[2] + wcount[3];
}

// ---------------------------------------------------------------------------------------
// k_scan: grid W, 1024 threads.  Thread t owns a contiguous run of tiles.
__global__ __launch_bounds__(kScanThreads) void k_scan(
    uint64_t tiles, const uint32_t* __restrict__ counts, uint32_t* __restrict__ offsets,
    uint64_t* __restrict__ nnz, uint32_t* __restrict__ chunk_tile, uint64_t chunks,
    uint64_t cap) {
  const uint32_t k = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t* cnt = counts + (uint64_t)k * tiles;
  uint32_t* off = offsets + (uint64_t)k * (tiles + 1);
  uint32_t* ct = chunk_tile + (uint64_t)k * chunks;

  const uint64_t per = (tiles + kScanThreads - 1) / kScanThreads;
  const uint64_t lo = (uint64_t)tid * per;
  const uint64_t hi = lo + per < tiles ? lo + per : tiles;
  uint32_t sum = 0;
#pragma unroll 8
  for (uint64_t t = lo; t < hi; ++t) sum += cnt[t];

  __shared__ uint32_t wsum[kScanThreads / kWave];
  const uint32_t inc = wave_inclusive_sum(sum);
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint32_t x = lane < kScanThreads / kWave ? wsum[lane] : 0u;
    const uint32_t xi = wave_inclusive_sum(x);
    if (lane < kScanThreads / kWave) wsum[lane] = xi - x;
  }
  __syncthreads();
  uint32_t run = wsum[wave] + inc - sum;
  const uint64_t limit = cap;  // list positions that get a chunk: [0, min(nnz, cap))
  for (uint64_t t = lo; t < hi; ++t) {
    const uint32_t c_t = cnt[t];
    off[t] = run;
    // chunks whose first position falls inside this tile start here
    uint64_t c0 = ((uint64_t)run + kChunk - 1) / kChunk;
    for (; c0 < chunks && c0 * kChunk < (uint64_t)run + c_t && c0 * kChunk < limit; ++c0)
      ct[c0] = (uint32_t)t;
    run += c_t;
  }
  if (tid == kScanThreads - 1) {
    off[tiles] = run;
    nnz[k] = run;
  }
}

// ---------------------------------------------------------------------------------------
// Shared front half of k_list_*: fill lidx/lval[0..cnt) with list positions
// [start, start + cnt) of worker k in ascending order.  Returns cnt (uniform).
struct ListChunk {
  uint32_t k, c;
  uint64_t start, end;
};

__device__ __forceinline__ bool next_chunk(uint64_t& g, uint32_t W, uint64_t chunks,
                                           const uint32_t* offsets, uint64_t tiles,
                                           uint64_t cap, ListChunk& out) {
  // walk global chunk ids g, g + gridDim.x, ... skipping chunks beyond a worker's list
  for (; g < (uint64_t)W * chunks; g += gridDim.x) {
    const uint32_t k = (uint32_t)(g / chunks);
    const uint32_t c = (uint32_t)(g % chunks);
    const uint64_t total = offsets[(uint64_t)k * (tiles + 1) + tiles];
    const uint64_t lim = total < cap ? total : cap;
    const uint64_t start = (uint64_t)c * kChunk;
    if (start >= lim) continue;
    out.k = k;
    out.c = c;
    out.start = start;
    out.end = start + kChunk < lim ? start + kChunk : lim;
    return true;
  }
  return false;
}

template <int NT>
__device__ void expand_chunk(const ListChunk& ch, const float* __restrict__ grad, uint64_t ld,
                             uint64_t tiles, const uint64_t* __restrict__ bitmaps,
                             uint64_t words, const uint32_t* __restrict__ offsets,
                             const uint32_t* __restrict__ chunk_tile, uint64_t chunks,
                             uint32_t* lidx, float* lval, uint64_t* lwords, uint32_t* lwoff) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t* off = offsets + (uint64_t)ch.k * (tiles + 1);
  const uint64_t* bm = bitmaps + (uint64_t)ch.k * words;
  const float* row = grad + (uint64_t)ch.k * ld;
  for (uint64_t t = chunk_tile[(uint64_t)ch.k * chunks + ch.c]; t < tiles; ++t) {
    const uint64_t o_t = off[t];
    if (o_t >= ch.end) break;
    if (off[t + 1] == o_t) continue;  // empty tile
    // the tile's 128 words and their exclusive popcount prefix
    if (tid < kTileWords) {
      const uint64_t q = t * kTileWords + tid;
      const uint64_t wv = q < words ? bm[q] : 0ull;
      const uint32_t pc = (uint32_t)__popcll(wv);
      const uint32_t inc = wave_inclusive_sum(pc);
      lwords[tid] = wv;
      lwoff[tid] = inc - pc;
      if (lane == kWave - 1) lwoff[kTileWords + wave] = inc;  // per-wave totals
    }
    __syncthreads();
    // 2048 groups of four elements per tile
    for (int gidx = tid; gidx < kTile / 4; gidx += NT) {
      const int q = gidx >> 4;
      const uint64_t wv = lwords[q];
      const uint32_t nib = (uint32_t)(wv >> (4 * (gidx & 15))) & 0xFu;
      if (!nib) continue;
      const uint32_t below = (uint32_t)__popcll(wv & ((1ull << (4 * (gidx & 15))) - 1ull));
      const uint32_t wbase = lwoff[q] + (q >= kWave ? lwoff[kTileWords] : 0u);
      const uint64_t pos0 = o_t + wbase + below;
      // a set bit lies below n <= ld and the group is 4-aligned: the 16-byte load stays in
      // the row
      const uint64_t e0 = t * kTile + (uint64_t)gidx * 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + e0);
      uint32_t r = 0;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        if (nib & (1u << c4)) {
          const uint64_t pos = pos0 + r;
          ++r;
          if (pos >= ch.start && pos < ch.end) {
            const uint32_t slot = (uint32_t)(pos - ch.start);
            lidx[slot] = (uint32_t)(e0 + c4);
            lval[slot] = v[c4];
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(kListThreads) void k_list_atomic(
    HashArgs h, uint32_t W, const float* __restrict__ grad, uint64_t ld, uint64_t tiles,
    const uint64_t* __restrict__ bitmaps, uint64_t words, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ chunk_tile, uint32_t* __restrict__ idx,
    float* __restrict__ val, uint64_t cap, uint64_t chunks, float* __restrict__ sketches,
    uint64_t dw) {
  __shared__ uint32_t lidx[kChunk];
  __shared__ float lval[kChunk];
  __shared__ uint64_t lwords[kTileWords];
  __shared__ uint32_t lwoff[kTileWords + 2];
  const uint64_t w = dw / D;
  ListChunk ch;
  for (uint64_t g = blockIdx.x; next_chunk(g, W, chunks, offsets, tiles, cap, ch);
       g += gridDim.x) {
    expand_chunk<kListThreads>(ch, grad, ld, tiles, bitmaps, words, offsets, chunk_tile, chunks,
                               lidx, lval, lwords, lwoff);
    const uint32_t cnt = (uint32_t)(ch.end - ch.start);
    uint32_t* oi = idx + (uint64_t)ch.k * cap + ch.start;
    float* ov = val + (uint64_t)ch.k * cap + ch.start;
    for (uint32_t s = threadIdx.x; s < cnt; s += kListThreads) {
      oi[s] = lidx[s];
      ov[s] = lval[s];
    }
    float* sk = sketches + (uint64_t)ch.k * dw;
    for (uint32_t pr = threadIdx.x; pr < cnt * D; pr += kListThreads) {
      const uint32_t s = pr / D;
      const int j = (int)(pr - s * D);
      const uint32_t i = lidx[s];
      const uint32_t b = bucket_of(h, partition_of(h, i), j, i);
      unsafeAtomicAdd(sk + (uint64_t)j * w + b, apply_sign(lval[s], sign_mask(h, j, i)));
    }
    __syncthreads();
  }
}

// Partitioned path, first half: list + partition-ordered copy of each chunk.
//   bidx/bval[k][c * kChunk + X[p] ...]: chunk c's pairs grouped by partition p
//   prefix[k][p][c] = X[p] (p = 0..P), the start of partition p inside chunk c
__global__ __launch_bounds__(kListThreads) void k_list_bin(
    HashArgs h, uint32_t W, const float* __restrict__ grad, uint64_t ld, uint64_t tiles,
    const uint64_t* __restrict__ bitmaps, uint64_t words, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ chunk_tile, uint32_t* __restrict__ idx,
    float* __restrict__ val, uint64_t cap, uint64_t chunks, uint32_t partitions,
    uint32_t* __restrict__ bidx, float* __restrict__ bval, uint32_t* __restrict__ prefix) {
  __shared__ uint32_t lidx[kChunk];
  __shared__ float lval[kChunk];
  __shared__ uint64_t lwords[kTileWords];
  __shared__ uint32_t lwoff[kTileWords + 2];
  __shared__ uint32_t wtot[kListThreads / kWave];
  extern __shared__ uint32_t hist[];  // partitions + 1 counters
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t P = partitions;
  ListChunk ch;
  for (uint64_t g = blockIdx.x; next_chunk(g, W, chunks, offsets, tiles, cap, ch);
       g += gridDim.x) {
    for (uint32_t p = tid; p <= P; p += kListThreads) hist[p] = 0;
    expand_chunk<kListThreads>(ch, grad, ld, tiles, bitmaps, words, offsets, chunk_tile, chunks,
                               lidx, lval, lwords, lwoff);
    const uint32_t cnt = (uint32_t)(ch.end - ch.start);
    uint32_t* oi = idx + (uint64_t)ch.k * cap + ch.start;
    float* ov = val + (uint64_t)ch.k * cap + ch.start;
    for (uint32_t s = tid; s < cnt; s += kListThreads) {
      const uint32_t i = lidx[s];
      oi[s] = i;
      ov[s] = lval[s];
      atomicAdd(&hist[partition_of(h, i)], 1u);
    }
    __syncthreads();
    // exclusive scan of hist[0..P) in place; each thread owns a contiguous run
    const uint32_t per = (P + kListThreads - 1) / kListThreads;
    const uint32_t lo = tid * per < P ? tid * per : P;
    const uint32_t hi = lo + per < P ? lo + per : P;
    uint32_t sum = 0;
    for (uint32_t p = lo; p < hi; ++p) sum += hist[p];
    const uint32_t inc = wave_inclusive_sum(sum);
    if (lane == kWave - 1) wtot[wave] = inc;
    __syncthreads();
    uint32_t run = inc - sum;
    for (int v = 0; v < wave; ++v) run += wtot[v];
    for (uint32_t p = lo; p < hi; ++p) {
      const uint32_t x = hist[p];
      hist[p] = run;
      run += x;
    }
    __syncthreads();
    uint32_t* pf = prefix + (uint64_t)ch.k * (P + 1) * chunks + ch.c;
    for (uint32_t p = tid; p < P; p += kListThreads) pf[(uint64_t)p * chunks] = hist[p];
    if (tid == 0) pf[(uint64_t)P * chunks] = cnt;
    __syncthreads();
    // scatter into partition order; hist[] now serves as the running cursor
    const uint64_t bbase = ((uint64_t)ch.k * chunks + ch.c) * kChunk;
    for (uint32_t s = tid; s < cnt; s += kListThreads) {
      const uint32_t i = lidx[s];
      const uint32_t pos = atomicAdd(&hist[partition_of(h, i)], 1u);
      bidx[bbase + pos] = i;
      bval[bbase + pos] = lval[s];
    }
    __syncthreads();
  }
}

// Partitioned path, second half: grid (P, W).  The partition tile is d x 2^K fp32 in LDS.
template <int D>
__global__ __launch_bounds__(kAccThreads) void k_accumulate(
    HashArgs h, uint64_t tiles, const uint32_t* __restrict__ offsets, uint64_t cap,
    uint64_t chunks, uint32_t partitions, const uint32_t* __restrict__ bidx,
    const float* __restrict__ bval, const uint32_t* __restrict__ prefix,
    float* __restrict__ sketches, uint64_t w, int vec4) {
  extern __shared__ float tile[];  // D * 2^K
  const uint32_t p = blockIdx.x, k = blockIdx.y;
  const int tid = threadIdx.x;
  const uint32_t pw = 1u << h.K;
  const uint32_t cells = D * pw;
  for (uint32_t c = tid; c < cells; c += kAccThreads) tile[c] = 0.f;
  __syncthreads();

  const uint64_t total = offsets[(uint64_t)k * (tiles + 1) + tiles];
  const uint64_t lim = total < cap ? total : cap;
  const uint64_t nch = (lim + kChunk - 1) / kChunk;
  const uint32_t* pf = prefix + ((uint64_t)k * (partitions + 1) + p) * chunks;
  for (uint64_t c = tid; c < nch; c += kAccThreads) {
    const uint32_t lo = pf[c], hi = pf[chunks + c];
    const uint64_t base = ((uint64_t)k * chunks + c) * kChunk;
    for (uint32_t e = lo; e < hi; ++e) {
      const uint32_t i = bidx[base + e];
      const float g = bval[base + e];
#pragma unroll
      for (int j = 0; j < D; ++j)
        atomicAdd(&tile[j * pw + row_bucket(h, j, i)], apply_sign(g, sign_mask(h, j, i)));
    }
  }
  __syncthreads();

  float* sk = sketches + (uint64_t)k * D * w + (uint64_t)p * pw;
  if (vec4) {
    const uint32_t pw4 = pw / 4;
    for (uint32_t c = tid; c < D * pw4; c += kAccThreads) {
      const uint32_t j = c / pw4, q = c - j * pw4;
      const f32x4 x = *reinterpret_cast<const f32x4*>(&tile[j * pw + 4 * q]);
      *reinterpret_cast<f32x4*>(sk + (uint64_t)j * w + 4 * q) = x;
    }
  } else {
    for (uint32_t c = tid; c < cells; c += kAccThreads) {
      const uint32_t j = c / pw, q = c - j * pw;
      sk[(uint64_t)j * w + q] = tile[c];
    }
  }
}

__global__ void k_fill_zero(float* __restrict__ p, uint64_t count) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    p[i] = 0.f;
}

// ---------------------------------------------------------------------------------------
// host launchers

hipError_t launch_stream(uint32_t W, const float* grad, uint64_t n, uint64_t ld, uint64_t tiles,
                         uint64_t* bitmaps, uint32_t* counts, hipStream_t s) {
  if (tiles == 0) return hipSuccess;
  const uint64_t words = (n + 63) / 64;
  hipLaunchKernelGGL(k_stream, dim3((uint32_t)tiles, W), dim3(kStreamThreads), 0, s, grad, n, ld,
                     tiles, words, bitmaps, counts);
  return hipGetLastError();
}

hipError_t launch_scan(uint32_t W, uint64_t tiles, const uint32_t* counts, uint32_t* offsets,
                       uint64_t* nnz, uint32_t* chunk_tile, uint64_t chunks, uint64_t cap,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(W), dim3(kScanThreads), 0, s, tiles, counts, offsets, nnz,
                     chunk_tile, chunks, cap);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, uint64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_fill_zero, dim3((uint32_t)blocks), dim3(256), 0, s, p, count);
  return hipGetLastError();
}

static uint32_t list_grid(uint32_t W, uint64_t chunks) {
  const uint64_t total = (uint64_t)W * chunks;
  return (uint32_t)(total < 2048 ? total : 2048);
}

hipError_t launch_list_atomic(const HashArgs& h, uint32_t W, const float* grad, uint64_t ld,
                              uint64_t tiles, const uint64_t* bitmaps, uint64_t words,
                              const uint32_t* offsets, const uint32_t* chunk_tile, uint32_t* idx,
                              float* val, uint64_t cap, uint64_t chunks, float* sketches,
                              uint64_t dw, hipStream_t s) {
  if (chunks == 0) return hipSuccess;
  const uint32_t grid = list_grid(W, chunks);
  S2R_DISPATCH_D(h.d, hipLaunchKernelGGL((k_list_atomic<D>), dim3(grid), dim3(kListThreads), 0,
                                         s, h, W, grad, ld, tiles, bitmaps, words, offsets,
                                         chunk_tile, idx, val, cap, chunks, sketches, dw));
  return hipGetLastError();
}

hipError_t launch_list_bin(const HashArgs& h, uint32_t W, const float* grad, uint64_t ld,
                           uint64_t tiles, const uint64_t* bitmaps, uint64_t words,
                           const uint32_t* offsets, const uint32_t* chunk_tile, uint32_t* idx,
                           float* val, uint64_t cap, uint64_t chunks, uint64_t partitions,
                           uint32_t* bidx, float* bval, uint32_t* prefix, hipStream_t s) {
  if (chunks == 0) return hipSuccess;
  const uint32_t grid = list_grid(W, chunks);
  const size_t lds = (partitions + 1) * sizeof(uint32_t);
  // static LDS (66 KiB) + the histogram exceeds the default dynamic limit
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_list_bin),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_list_bin, dim3(grid), dim3(kListThreads), lds, s, h, W, grad, ld, tiles,
                     bitmaps, words, offsets, chunk_tile, idx, val, cap, chunks,
                     (uint32_t)partitions, bidx, bval, prefix);
  return hipGetLastError();
}

hipError_t launch_accumulate(const HashArgs& h, uint32_t W, uint64_t tiles,
                             const uint32_t* offsets, uint64_t cap, uint64_t chunks,
                             uint64_t partitions, const uint32_t* bidx, const float* bval,
                             const uint32_t* prefix, float* sketches, uint64_t w,
                             hipStream_t s) {
  const size_t lds = ((size_t)h.d << h.K) * sizeof(float);
  const int vec4 = (h.K >= 2 && (reinterpret_cast<uintptr_t>(sketches) % 16) == 0) ? 1 : 0;
  hipError_t e = hipSuccess;
  S2R_DISPATCH_D(h.d, {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_accumulate<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      hipLaunchKernelGGL((k_accumulate<D>), dim3((uint32_t)partitions, W), dim3(kAccThreads), lds,
                         s, h, tiles, offsets, cap, chunks, (uint32_t)partitions, bidx, bval,
                         prefix, sketches, w, vec4);
  });
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace s2r
