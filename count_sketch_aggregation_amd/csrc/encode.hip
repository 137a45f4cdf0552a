// encode.hip -- compression kernels: gradient -> bitmap + ordered non-zero list + sketch.
//
// Follows S2 Reducer (arXiv 2110.02140) Section 3.1 "Compressing Sparse Gradient" and the
// compression loop of Algorithm 1: mark every non-zero position in a bitmap, then add
// s_j(i) * g(i) into bucket h_j(i) of each row j for every non-zero g(i).
//
// Pipeline on gfx950 (all W workers batched in every launch):
//   k_stream      streams the gradient once with 128-bit loads, packs the non-zero tests
//                 into element-ordered bitmap words through LDS; writes the bitmap and one
//                 non-zero count per 4096-element tile.
//   k_scan_sum, k_scan
//                 per (4096-tile block, worker): exclusive prefix of the tile counts (list
//                 offsets), nnz, and the lists of non-empty tile pairs, sparse and dense.
//   k_blockbits   (block-granular bitmaps only) folds the element bitmap into block bits.
//   k_expand_dense, k_expand_sparse
//                 per non-empty tile pair: expands the bitmap words into ascending
//                 (index, value) pairs at their list offsets, re-reading only the 16-byte
//                 gradient groups that hold a set bit (a workgroup per dense pair, a wave
//                 per sparse one).
//   then either (d x w table larger than LDS, independent rows)
//     k_scatter   reads 8192-entry list chunks and adds each pair into the d rows with
//                 global fp32 atomics (after a zero fill), or (partitioned path)
//     k_bin       counting-sorts each list chunk by partition P(i) and writes the
//                 partition-ordered copy plus per-partition offsets;
//     k_accumulate one workgroup per (worker, partition): accumulates the partition's
//                 d x 2^K buckets in LDS and writes them to the sketch with dense coalesced
//                 stores (no zero fill, no global atomics).
#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// k_stream: grid (tiles, W), 512 threads.  Wave w of a 4096-element tile owns 512
// consecutive elements (2 load rounds of 256): lane l of round r holds elements
// base + 256 r + 4 l .. +3 in one 128-bit load.  Each lane folds its four non-zero tests
// into a nibble with vector ops (min(bits << 1, 1) is 1 exactly when the magnitude bits are
// not all zero), a DPP swap pairs adjacent lanes' nibbles into one byte, and the even lanes
// drop the bytes into LDS in element order, so the tile's 64 bitmap words assemble in LDS
// with no scalar-unit work and leave with one coalesced non-temporal 512-byte store.
// Measured on MI355X: this shape (one short-lived workgroup per tile, 2 loads per lane)
// beats 4 loads x 256 lanes (4%), 1 x 1024 (40%), cached loads (9%) and a persistent grid
// that loads the next tile while packing the current one (10-20%).
__device__ __forceinline__ uint32_t nz_bit(float x) { return min(__float_as_uint(x) << 1, 1u); }

template <bool TAIL>
__device__ __forceinline__ uint32_t stream_tile(const float* __restrict__ row, uint64_t wave_base,
                                                uint64_t n, uint8_t* lbytes, int lane) {
  f32x4 v[kStreamVec];
#pragma unroll
  for (int r = 0; r < kStreamVec; ++r) {
    const uint64_t e = wave_base + r * 256 + lane * 4;
    // e is a multiple of 4 and ld % 4 == 0, so e < n <= ld keeps all four lanes in the row
    if (!TAIL || e < n) v[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e));
    else v[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int r = 0; r < kStreamVec; ++r) {
    uint32_t nib = nz_bit(v[r].x) | (nz_bit(v[r].y) << 1) | (nz_bit(v[r].z) << 2) |
                   (nz_bit(v[r].w) << 3);
    if (TAIL) {  // clear the bits of elements at or beyond n
      const uint64_t e = wave_base + r * 256 + lane * 4;
      const uint64_t left = e < n ? n - e : 0;
      nib &= left >= 4 ? 0xFu : ((1u << left) - 1u);
    }
    cnt += __popc(nib);
    const uint32_t odd = __builtin_amdgcn_mov_dpp(nib, 0xB1, 0xF, 0xF, false);  // lane ^ 1
    if (!(lane & 1)) lbytes[r * 32 + (lane >> 1)] = (uint8_t)(nib | (odd << 4));
  }
  return cnt;
}

__global__ __launch_bounds__(kStreamThreads) void k_stream(
    const float* __restrict__ grad, uint64_t n, uint64_t ld, uint64_t tiles, uint64_t words,
    uint64_t* __restrict__ bitmaps, uint32_t* __restrict__ counts) {
  __shared__ uint64_t lwords[kTileWords];
  __shared__ uint32_t wcount[kStreamThreads / kWave];
  // tiles in XCD runs of 2 MiB (xcd_run_item); the grid is x-fastest over (tile, worker)
  const uint64_t item =
      xcd_run_item(blockIdx.x + (uint64_t)blockIdx.y * gridDim.x, (uint64_t)gridDim.x * gridDim.y,
                   (2u << 20) / (kTile * sizeof(float)));
  const uint32_t t = (uint32_t)(item % gridDim.x), k = (uint32_t)(item / gridDim.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* row = grad + (uint64_t)k * ld;
  const uint64_t tile_base = (uint64_t)t * kTile;
  const uint64_t wave_base = tile_base + (uint64_t)wave * kStreamWaveSpan;
  uint8_t* lbytes = reinterpret_cast<uint8_t*>(lwords) + wave * (kStreamWaveSpan / 8);
  uint32_t c = (tile_base + kTile <= n) ? stream_tile<false>(row, wave_base, n, lbytes, lane)
                                        : stream_tile<true>(row, wave_base, n, lbytes, lane);
  c = wave_sum(c);
  if (lane == 0) wcount[wave] = c;
  __syncthreads();
  if (tid < kTileWords) {
    const uint64_t gw = (uint64_t)t * kTileWords + tid;
    // non-temporal: ordinary stores mixed into this read stream cost the pass ~20% on MI355X
    if (gw < words) __builtin_nontemporal_store(lwords[tid], &bitmaps[(uint64_t)k * words + gw]);
  }
  if (tid == 0) {
    uint32_t sum = 0;
#pragma unroll
    for (int v = 0; v < kStreamThreads / kWave; ++v) sum += wcount[v];
    counts[(uint64_t)k * tiles + t] = sum;
  }
}

// ---------------------------------------------------------------------------------------
// k_scan: grid (blocks, W), 1024 threads; block b of worker k scans tiles
// [b * kScanPass, (b + 1) * kScanPass): coalesced loads into LDS, one contiguous run of
// kScanPass / 1024 per thread for the block scan (read with a 1-in-16 padding), offsets
// written back through LDS with coalesced stores.  The block starts from the
// totals of the blocks before it (btot, from k_scan_sum; none with one block).
// Optionally (spans != nullptr) it also lists the spans (tile pairs) that hold a non-zero,
// for k_expand: the sparse ones (at most kDenseSpan non-zeros) in order from the front of
// the worker's list, the dense ones from its back, with the two counts in nspan[2k],
// nspan[2k + 1].  And, for every chunk of kChunk consecutive list positions below `limit`,
// it records the tile holding its first position.
__device__ __forceinline__ uint32_t scan_pad(uint32_t i) { return i + (i >> 4); }

// p[i] for i < n, else 0: an unconditional load of a clamped index, so that a thread's
// loads issue back to back rather than as one guarded round trip each.  With n == 0 there
// is no element to clamp to, so nothing is loaded (n is uniform across the grid).
__device__ __forceinline__ uint32_t load_or_zero(const uint32_t* p, uint64_t i, uint64_t n) {
  if (n == 0) return 0u;
  const uint32_t v = p[i < n ? i : n - 1];
  return i < n ? v : 0u;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_sum(uint64_t tiles,
                                                           const uint32_t* __restrict__ counts,
                                                           uint4* __restrict__ btot) {
  __shared__ uint32_t wsum[3][kScanThreads / kWave];
  const uint32_t b = blockIdx.x, k = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t* cnt = counts + (uint64_t)k * tiles;
  const uint64_t base = (uint64_t)b * kScanPass;
  constexpr int U = kScanPass / 2 / kScanThreads;
  uint32_t x[2 * U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t i = base + 2 * (uint64_t)(tid + kScanThreads * u);  // a span's first tile
    x[2 * u] = load_or_zero(cnt, i, tiles);
    x[2 * u + 1] = load_or_zero(cnt, i + 1, tiles);
  }
  uint32_t sum = 0, ns = 0, nd = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t c = x[2 * u] + x[2 * u + 1];
    sum += c;
    ns += (c && c <= kDenseSpan) ? 1u : 0u;
    nd += c > kDenseSpan ? 1u : 0u;
  }
  sum = wave_sum(sum);
  ns = wave_sum(ns);
  nd = wave_sum(nd);
  if (lane == 0) {
    wsum[0][wave] = sum;
    wsum[1][wave] = ns;
    wsum[2][wave] = nd;
  }
  __syncthreads();
  if (tid == 0) {
    uint4 t = {0u, 0u, 0u, 0u};
    for (int v = 0; v < kScanThreads / kWave; ++v) {
      t.x += wsum[0][v];
      t.y += wsum[1][v];
      t.z += wsum[2][v];
    }
    btot[(uint64_t)k * gridDim.x + b] = t;
  }
}

__global__ __launch_bounds__(kScanThreads) void k_scan(
    uint64_t tiles, const uint32_t* __restrict__ counts, uint32_t* __restrict__ offsets,
    uint64_t* __restrict__ nnz, uint32_t* __restrict__ chunk_tile, uint64_t chunks,
    uint64_t limit, const uint4* __restrict__ btot, uint2* __restrict__ spans,
    uint32_t* __restrict__ nspan) {
  constexpr int PER = kScanPass / kScanThreads;  // tiles per thread, whole spans
  static_assert(PER % 2 == 0, "a thread's run holds whole spans");
  constexpr int NW = kScanThreads / kWave;
  __shared__ uint32_t lc[kScanPass + kScanPass / 16];
  __shared__ uint32_t wsum[3][NW];
  const uint32_t b = blockIdx.x, k = blockIdx.y, nb = gridDim.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t* cnt = counts + (uint64_t)k * tiles;
  uint32_t* off = offsets + (uint64_t)k * (tiles + 1);
  uint32_t* ct = chunk_tile + (uint64_t)k * chunks;
  const uint64_t nsp = (tiles + 1) / 2;
  uint2* sp = spans ? spans + (uint64_t)k * nsp : nullptr;
  const uint64_t base = (uint64_t)b * kScanPass;
  uint32_t carry = 0, scarry = 0, dcarry = 0;
  if (b > 0) {  // totals of the blocks before this one
    uint32_t c = 0, e = 0, f = 0;
    for (uint32_t i = tid; i < b; i += kScanThreads) {
      const uint4 t = btot[(uint64_t)k * nb + i];
      c += t.x;
      e += t.y;
      f += t.z;
    }
    c = wave_sum(c);
    e = wave_sum(e);
    f = wave_sum(f);
    if (lane == 0) {
      wsum[0][wave] = c;
      wsum[1][wave] = e;
      wsum[2][wave] = f;
    }
    __syncthreads();
    for (int v = 0; v < NW; ++v) {
      carry += wsum[0][v];
      scarry += wsum[1][v];
      dcarry += wsum[2][v];
    }
    __syncthreads();  // wsum is reused below
  }
  {
    uint32_t x[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) x[u] = load_or_zero(cnt, base + tid + kScanThreads * u, tiles);
#pragma unroll
    for (int u = 0; u < PER; ++u) lc[scan_pad(tid + kScanThreads * u)] = x[u];
  }
  __syncthreads();
  uint32_t v[PER], sum = 0, ns = 0, nd = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    v[u] = lc[scan_pad(tid * PER + u)];
    sum += v[u];
    if (u & 1) {
      const uint32_t c = v[u - 1] + v[u];
      ns += (c && c <= kDenseSpan) ? 1u : 0u;
      nd += c > kDenseSpan ? 1u : 0u;
    }
  }
  const uint32_t inc = wave_inclusive_sum(sum);
  const uint32_t sinc = wave_inclusive_sum(ns);
  const uint32_t dinc = wave_inclusive_sum(nd);
  if (lane == kWave - 1) {
    wsum[0][wave] = inc;
    wsum[1][wave] = sinc;
    wsum[2][wave] = dinc;
  }
  __syncthreads();
  uint32_t run = carry + inc - sum, block_total = 0;
  uint32_t srun = scarry + sinc - ns, block_sparse = 0;
  uint32_t drun = dcarry + dinc - nd, block_dense = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      run += wsum[0][w];
      srun += wsum[1][w];
      drun += wsum[2][w];
    }
    block_total += wsum[0][w];
    block_sparse += wsum[1][w];
    block_dense += wsum[2][w];
  }
  const uint64_t t0 = base + (uint64_t)tid * PER;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    lc[scan_pad(tid * PER + u)] = run;
    if (chunks && t0 + u < tiles) {
      // chunks whose first position falls inside this tile start here
      for (uint64_t c0 = ((uint64_t)run + kChunk - 1) / kChunk;
           c0 < chunks && c0 * kChunk < (uint64_t)run + v[u] && c0 * kChunk < limit; ++c0)
        ct[c0] = (uint32_t)(t0 + u);
    }
    if (sp && (u & 1)) {
      const uint32_t c = v[u - 1] + v[u];
      // the span and the list position of its first pair (run still holds v[u - 1])
      const uint2 span = make_uint2((uint32_t)((t0 + u) >> 1), run - v[u - 1]);
      if (c > kDenseSpan) sp[nsp - 1 - drun++] = span;
      else if (c) sp[srun++] = span;
    }
    run += v[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t i = tid + kScanThreads * u;
    if (base + i < tiles) off[base + i] = lc[scan_pad(i)];
  }
  if (b == nb - 1 && tid == 0) {
    off[tiles] = carry + block_total;
    nnz[k] = carry + block_total;
    if (nspan) {
      nspan[2 * k] = scarry + block_sparse;
      nspan[2 * k + 1] = dcarry + block_dense;
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_expand_dense / k_expand_sparse: list the non-empty spans (tile pairs of 8192 elements and
// 128 words, from k_scan, each with the list position of its first pair), so empty regions
// cost nothing.  Each writes a span's pairs at that position + (rank within the span),
// re-reading only the 16-byte gradient groups that hold a set bit; the next span's entry is
// loaded while the current one is expanded.
//   dense spans (more than kDenseSpan non-zeros), grid (G, W), 256 threads: a workgroup per
//     span; the words and their popcount prefix go to LDS and each thread takes 8 groups of
//     four elements, all 8 loads issued before use;
//   sparse spans, grid (G, W), 256 threads: a wave per span, so four spans per workgroup are
//     in flight with no workgroup barrier; lane l loads words 2l and 2l+1, a wave prefix sum
//     of their popcounts gives every word's rank offset, both go to the wave's own LDS rows,
//     and lane l owns the groups g = l + 64 m (m = 0..31): it lists those holding a set bit
//     and loads them kExpandUnroll at a time.
constexpr int kExpandSpan = 2 * kTile;
constexpr int kExpandWords = kExpandSpan / 64;  // 128
constexpr int kExpandWaves = kExpandThreads / kWave;
constexpr int kExpandUnroll = 4;

// store the pairs of one group of four elements (nib = its set bits): a whole group whose
// list slots are 16-byte aligned in both lists leaves with two 128-bit stores (measured on
// MI355X: the expansion of the Transformer and embedding workloads 250 -> 168 us and
// 81 -> 54 us against four scalar stores per list), any other with one store per set bit
__device__ __forceinline__ void expand_store(uint32_t* oi, float* ov, uint64_t cap, uint64_t pos,
                                             uint32_t e0, uint32_t nib, const f32x4& v) {
  if (nib == 0xFu && pos + 4 <= cap &&
      ((reinterpret_cast<uintptr_t>(oi + pos) | reinterpret_cast<uintptr_t>(ov + pos)) & 15u) == 0) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4*>(oi + pos) = u32x4{e0, e0 + 1, e0 + 2, e0 + 3};
    *reinterpret_cast<f32x4*>(ov + pos) = v;
    return;
  }
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    if (nib & (1u << c4)) {
      if (pos < cap) {
        oi[pos] = e0 + c4;
        ov[pos] = v[c4];
      }
      ++pos;
    }
  }
}

__global__ __launch_bounds__(kExpandThreads) void k_expand_dense(
    const float* __restrict__ grad, uint64_t ld, uint64_t tiles,
    const uint64_t* __restrict__ bitmaps, uint64_t words, const uint2* __restrict__ spans,
    const uint32_t* __restrict__ nspan, uint32_t* __restrict__ idx, float* __restrict__ val,
    uint64_t cap) {
  const uint32_t k = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t nsp = (tiles + 1) / 2;
  const uint2* sl = spans + (uint64_t)k * nsp;
  const uint32_t nd = nspan[2 * k + 1];
  __shared__ uint64_t lwords[kExpandWords];
  __shared__ uint32_t lwoff[kExpandWords + 2];
  uint32_t* oi = idx + (uint64_t)k * cap;
  float* ov = val + (uint64_t)k * cap;
  uint2 next = blockIdx.x < nd ? sl[nsp - 1 - blockIdx.x] : make_uint2(0u, 0u);
  for (uint32_t si = blockIdx.x; si < nd; si += gridDim.x) {
    const uint32_t t = next.x;
    const uint64_t o_t = next.y;
    // the following span's entry, one round trip ahead
    if (si + gridDim.x < nd) next = sl[nsp - 1 - (si + gridDim.x)];
    if (o_t >= cap) continue;  // beyond the list capacity (uniform)
    if (tid < kExpandWords) {
      const uint64_t q = (uint64_t)t * kExpandWords + tid;
      const uint64_t wv = q < words ? bitmaps[(uint64_t)k * words + q] : 0ull;
      const uint32_t pc = (uint32_t)__popcll(wv);
      const uint32_t inc = wave_inclusive_sum(pc);
      lwords[tid] = wv;
      lwoff[tid] = inc - pc;
      if (lane == kWave - 1) lwoff[kExpandWords + wave] = inc;
    }
    __syncthreads();
    const float* row = grad + (uint64_t)k * ld + (uint64_t)t * kExpandSpan;
    constexpr int G = kExpandSpan / 4 / kExpandThreads;  // groups per thread
    f32x4 v[G];
    uint32_t nib[G], pos0[G];
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const int gidx = tid + kExpandThreads * m;
      const int q = gidx >> 4, sh = 4 * (gidx & 15);
      const uint64_t wv = lwords[q];
      nib[m] = (uint32_t)(wv >> sh) & 0xFu;
      pos0[m] = lwoff[q] + (q >= kWave ? lwoff[kExpandWords] : 0u) +
                (uint32_t)__popcll(wv & ((1ull << sh) - 1ull));
      // a set bit lies below n <= ld and the group is 4-aligned: the load stays in the row
      if (nib[m]) v[m] = *reinterpret_cast<const f32x4*>(row + 4 * gidx);
    }
    wait_vector_memory();  // one wait for the loads, then the stores issue back to back
#pragma unroll
    for (int m = 0; m < G; ++m)
      if (nib[m])
        expand_store(oi, ov, cap, o_t + pos0[m],
                     t * (uint32_t)kExpandSpan + 4u * (uint32_t)(tid + kExpandThreads * m), nib[m],
                     v[m]);
    __syncthreads();  // lwords and lwoff are rewritten for the next span
  }
}

// LDS written by some lanes of a wave and read by others: order the two within the wave
// (no workgroup barrier: the waves of a workgroup run different spans).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// six waves per SIMD: the kernel is latency-bound, and the vector-store path of expand_store
// would otherwise take it to 82 registers and five
__global__ __launch_bounds__(kExpandThreads) __attribute__((amdgpu_waves_per_eu(6)))
void k_expand_sparse(
    const float* __restrict__ grad, uint64_t ld, uint64_t tiles,
    const uint64_t* __restrict__ bitmaps, uint64_t words, const uint2* __restrict__ spans,
    const uint32_t* __restrict__ nspan, uint32_t* __restrict__ idx, float* __restrict__ val,
    uint64_t cap) {
  const uint32_t k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t nsp = (tiles + 1) / 2;
  const uint2* sl = spans + (uint64_t)k * nsp;
  const uint32_t ns = nspan[2 * k];
  __shared__ uint64_t lwords[kExpandWaves][kExpandWords];
  __shared__ uint32_t lwoff[kExpandWaves][kExpandWords];
  uint64_t* lw = lwords[wave];
  uint32_t* lo = lwoff[wave];
  uint32_t* oi = idx + (uint64_t)k * cap;
  float* ov = val + (uint64_t)k * cap;
  const uint32_t stride = gridDim.x * kExpandWaves;
  const uint32_t s0 = blockIdx.x * kExpandWaves + wave;
  uint2 next = s0 < ns ? sl[s0] : make_uint2(0u, 0u);
  for (uint32_t si = s0; si < ns; si += stride) {
    const uint32_t t = next.x;
    const uint64_t o_t = next.y;
    if (si + stride < ns) next = sl[si + stride];  // one round trip ahead
    if (o_t >= cap) continue;  // beyond the list capacity (wave-uniform)
    uint64_t wv[2];
    uint32_t pc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint64_t q = (uint64_t)t * kExpandWords + 2 * lane + j;
      wv[j] = q < words ? bitmaps[(uint64_t)k * words + q] : 0ull;
      pc[j] = (uint32_t)__popcll(wv[j]);
    }
    const uint32_t inc = wave_inclusive_sum(pc[0] + pc[1]);
    wave_lds_sync();  // the previous span's reads of lw / lo are done
    lw[2 * lane] = wv[0];
    lw[2 * lane + 1] = wv[1];
    lo[2 * lane] = inc - pc[0] - pc[1];
    lo[2 * lane + 1] = inc - pc[1];
    wave_lds_sync();
    const float* row = grad + (uint64_t)k * ld + (uint64_t)t * kExpandSpan;
    // lane l owns groups g = l + 64 m (m = 0..31): word (l >> 4) + 4 m, nibble 4 (l & 15).
    // Its set groups are listed first, then taken kExpandUnroll at a time, so the wave makes
    // one round trip per kExpandUnroll set groups of its busiest lane.
    const int sh = 4 * (lane & 15), qb = lane >> 4;
    uint32_t mask = 0;
#pragma unroll
    for (int m = 0; m < kExpandSpan / 4 / kWave; ++m)
      mask |= (uint32_t)(((lw[qb + 4 * m] >> sh) & 0xFull) != 0ull) << m;
    constexpr int UN = kExpandUnroll;
    while (__ballot(mask != 0u) != 0ull) {
      f32x4 v[UN];
      uint32_t nib[UN], pos0[UN], g[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const bool has = mask != 0u;
        const int m = has ? __builtin_ctz(mask) : 0;
        mask &= mask - 1u;  // 0 stays 0
        g[u] = (uint32_t)(lane + kWave * m);
        const int q = qb + 4 * m;
        const uint64_t w = lw[q];
        nib[u] = has ? (uint32_t)(w >> sh) & 0xFu : 0u;
        pos0[u] = lo[q] + (uint32_t)__popcll(w & ((1ull << sh) - 1ull));
        // unconditional, so the loads issue together: a lane with nothing left reads the
        // span's first group, which lies inside the row (the span holds a set bit, and
        // ld % 4 == 0); a set group lies below n <= ld, 4-aligned
        v[u] = *reinterpret_cast<const f32x4*>(row + (has ? 4u * g[u] : 0u));
      }
      wait_vector_memory();  // one wait for the loads, then the stores issue back to back
#pragma unroll
      for (int u = 0; u < UN; ++u) asm volatile("" : "+v"(v[u]));  // keeps the loads above it
#pragma unroll
      for (int u = 0; u < UN; ++u)
        if (nib[u])
          expand_store(oi, ov, cap, o_t + pos0[u], t * (uint32_t)kExpandSpan + 4u * g[u], nib[u],
                       v[u]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_scatter (independent-row path when the table exceeds LDS): grid (chunks, W).  Reads the
// chunk's list entries and adds s_j(i) g(i) into every row with global fp32 atomics.
template <int D>
__global__ __launch_bounds__(kScatterThreads) void k_scatter(
    HashArgs h, uint64_t tiles, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ idx, const float* __restrict__ val, uint64_t cap,
    float* __restrict__ sketches, uint64_t w) {
  const uint32_t c = blockIdx.x, k = blockIdx.y;
  const uint64_t total = offsets[(uint64_t)k * (tiles + 1) + tiles];
  const uint64_t lim = total < cap ? total : cap;
  const uint64_t start = (uint64_t)c * kChunk;
  if (start >= lim) return;
  const uint32_t cnt = (uint32_t)(lim - start < kChunk ? lim - start : kChunk);
  const uint32_t* li = idx + (uint64_t)k * cap + start;
  const float* lv = val + (uint64_t)k * cap + start;
  float* sk = sketches + (uint64_t)k * D * w;
  for (uint32_t s = threadIdx.x; s < cnt; s += kScatterThreads) {
    const uint32_t i = li[s];
    const float g = lv[s];
    const uint32_t part = partition_of(h, i);
#pragma unroll
    for (int j = 0; j < D; ++j)
      unsafeAtomicAdd(sk + (uint64_t)j * w + bucket_of(h, part, j, i),
                      apply_sign(g, sign_mask(h, j, i)));
  }
}

// ---------------------------------------------------------------------------------------
// Block-wide exclusive scan of hist[0..P) in place (each thread owns a contiguous run).
template <int NT>
__device__ __forceinline__ void block_exclusive_scan(uint32_t* hist, uint32_t P, uint32_t* wtot) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t per = (P + NT - 1) / NT;
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
}

// k_bin (partitioned path): grid (chunks, W), 512 threads.  Counting-sorts the chunk's list
// entries by partition P(i) (u32 LDS atomics give each entry its slot), assembles the sorted
// chunk in LDS and writes it out with coalesced 128-bit stores:
//   bins[k][c * kChunk + X[p] ...]        the chunk's (index, value bits) pairs grouped by
//                                         partition, interleaved so a segment is one run
//   prefix[k][c][p] = X[p], p = 0..P       the start of partition p inside chunk c (one
//                                          contiguous row per chunk, so the stores coalesce)
__global__ __launch_bounds__(kBinThreads) void k_bin(
    HashArgs h, uint64_t tiles, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ idx, const float* __restrict__ val, uint64_t cap,
    uint64_t chunks, uint32_t P, uint2* __restrict__ bins, uint32_t* __restrict__ prefix) {
  extern __shared__ uint32_t hist[];  // P + 1 counters
  __shared__ __align__(16) uint2 spair[kChunk];
  __shared__ uint32_t wtot[kBinThreads / kWave];
  const uint32_t c = blockIdx.x, k = blockIdx.y;
  const int tid = threadIdx.x;
  // start < min(cap, n): the grid has ceil(min(cap, n) / kChunk) chunks
  const uint64_t start = (uint64_t)c * kChunk;
  constexpr int R = kChunk / kBinThreads;
  uint32_t ii[R], pp[R], rk[R];
  float gg[R];
  const uint32_t* li = idx + (uint64_t)k * cap + start;
  const float* lv = val + (uint64_t)k * cap + start;
  // The chunk's entries are read in the same round trip as the list length: indices are
  // clamped inside the worker's list capacity, so every load issues unconditionally, and
  // entries at or past the length are ignored below.
  const uint64_t room = cap - start;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t s = tid + kBinThreads * r;
    const uint64_t sc = s < room ? s : room - 1;
    ii[r] = li[sc];
    gg[r] = lv[sc];
  }
  const uint64_t total = offsets[(uint64_t)k * (tiles + 1) + tiles];
  const uint64_t lim = total < cap ? total : cap;
  if (start >= lim) return;
  const uint32_t cnt = (uint32_t)(lim - start < kChunk ? lim - start : kChunk);
  for (uint32_t p = tid; p <= P; p += kBinThreads) hist[p] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t s = tid + kBinThreads * r;
    if (s < cnt) {
      pp[r] = partition_of(h, ii[r]);
      rk[r] = atomicAdd(&hist[pp[r]], 1u);
    }
  }
  __syncthreads();
  block_exclusive_scan<kBinThreads>(hist, P, wtot);
  uint32_t* pf = prefix + ((uint64_t)k * chunks + c) * (P + 1);
  for (uint32_t p = tid; p < P; p += kBinThreads) pf[p] = hist[p];
  if (tid == 0) pf[P] = cnt;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t s = tid + kBinThreads * r;
    if (s < cnt) {
      const uint32_t pos = hist[pp[r]] + rk[r];
      spair[pos] = make_uint2(ii[r], __float_as_uint(gg[r]));
    }
  }
  __syncthreads();
  uint2* out = bins + ((uint64_t)k * chunks + c) * kChunk;  // 16-byte aligned
  const uint32_t cnt2 = cnt / 2;
  for (uint32_t q = tid; q < cnt2; q += kBinThreads)
    *reinterpret_cast<uint4*>(out + 2 * q) = *reinterpret_cast<const uint4*>(&spair[2 * q]);
  if ((cnt & 1u) && tid == 0) out[cnt - 1] = spair[cnt - 1];
}

// One group of k_accumulate's entries, e0 + u * kAccThreads (u < UN) of a batch of E > 0
// flattened entries: each entry's segment (branch-free search) and its (index, value bits)
// pair.  Entries at or past E are read as entry E - 1, so every load issues unconditionally;
// acc_add drops them.
template <int UN>
__device__ __forceinline__ void acc_fetch(const uint32_t* seg_off, const uint32_t* seg_src,
                                          uint32_t nb, uint32_t E, const uint2* kb, uint32_t e0,
                                          uint2* pr) {
  uint32_t x[UN], c[UN];
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const uint32_t e = e0 + u * kAccThreads;
    x[u] = e < E ? e : E - 1;
  }
  segments_of<UN>(seg_off, nb, x, c);
#pragma unroll
  for (int u = 0; u < UN; ++u) pr[u] = kb[seg_src[c[u]] + (x[u] - seg_off[c[u]])];
}

// Adds the group's pairs (entries below E) into the LDS tile: s_j(i) g(i) into row j's
// bucket Q_j(i), all D x UN compare-and-swaps in flight together.
template <int D, int UN>
__device__ __forceinline__ void acc_add(const HashArgs& h, float* tile, uint32_t pw, uint32_t E,
                                        uint32_t e0, const uint2* pr) {
  uint32_t cell[UN * D];
  float add[UN * D];
  bool live[UN * D];
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const bool on = e0 + u * kAccThreads < E;
    const uint32_t i = pr[u].x;
    const float g = __uint_as_float(pr[u].y);
#pragma unroll
    for (int j = 0; j < D; ++j) {
      live[u * D + j] = on;
      cell[u * D + j] = j * pw + row_bucket(h, j, i);
      add[u * D + j] = apply_sign(g, sign_mask(h, j, i));
    }
  }
  lds_add_f32_many<UN * D>(tile, cell, add, live);
}

// Item v of k_accumulate's sequence (v < items) -> (worker, partition) item: XCD x runs the
// x-th eighth of the items in order, so that neighbouring partitions, whose chunk offsets
// share cache lines, run on one XCD at about the same time.  Workgroup b runs on XCD b % 8
// and walks v = b, b + G, b + 2G, ... with G (the grid) a multiple of 8, so v % 8 stays b's
// XCD.  Identity when either count is not a multiple of 8.
__device__ __forceinline__ uint32_t acc_item(uint32_t v, uint32_t items) {
  if (items % kXcds != 0 || gridDim.x % kXcds != 0) return v;
  return (v % kXcds) * (items / kXcds) + v / kXcds;
}

// Issues the loads of a chunk batch's segment bounds: chunk row (cb + c) of the partition's
// column pf, for c = tid * PER + u below nb (clamped, unconditional loads: all in flight at
// once; rows past nb re-read row cb + nb - 1 and are dropped by acc_flatten).
template <int PER>
__device__ __forceinline__ void acc_bounds(const uint32_t* pf, uint32_t partitions, uint64_t cb,
                                           uint64_t nb, uint32_t* lo, uint32_t* hi) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint64_t c = (uint64_t)tid * PER + u < nb ? (uint64_t)tid * PER + u : nb - 1;
    const uint64_t row = (cb + c) * (partitions + 1);
    lo[u] = pf[row];
    hi[u] = pf[row + 1];
  }
}

// Flattens the segments of chunks [cb, cb + nb) (bounds lo/hi from acc_bounds) into
// seg_src / seg_off and returns their total entry count E.  Whole workgroup, two barriers;
// seg_src, seg_off and wtot must be free on entry.
template <int PER>
__device__ __forceinline__ uint32_t acc_flatten(uint32_t cb, uint32_t nb, const uint32_t* lo,
                                                const uint32_t* hi, uint32_t* seg_src,
                                                uint32_t* seg_off, uint32_t* wtot) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t len[PER], sum = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t c = tid * PER + u;
    len[u] = 0;
    if (c < nb) {
      seg_src[c] = (cb + c) * (uint32_t)kChunk + lo[u];
      len[u] = hi[u] - lo[u];
    }
    sum += len[u];
  }
  const uint32_t inc = wave_inclusive_sum(sum);
  if (lane == kWave - 1) wtot[wave] = inc;
  __syncthreads();
  uint32_t run = inc - sum;
  for (int v = 0; v < wave; ++v) run += wtot[v];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t c = tid * PER + u;
    if (c <= nb) seg_off[c] = run;  // seg_off[nb] = total entries of the batch
    run += len[u];
  }
  if (tid == kAccThreads - 1 && nb == (uint32_t)kSegBatch) seg_off[kSegBatch] = run;
  __syncthreads();
  return seg_off[nb];
}

// Adds the E > 0 flattened entries of a batch into the tile; the thread's first group
// (entries tid + u * kAccThreads) is already in pa.  Software pipeline: the segment search
// and list loads of the next group issue before the current group's adds, so one group's
// global round trip overlaps the previous group's LDS work.  The register sets a and b
// alternate, so no loaded register is ever copied (a copy would wait for its load).
template <int D, int UN>
__device__ __forceinline__ void acc_batch(const HashArgs& h, float* tile, uint32_t pw,
                                          const uint32_t* seg_off, const uint32_t* seg_src,
                                          uint32_t nb, uint32_t E, const uint2* kb, uint2* pa) {
  constexpr uint32_t kStep = kAccThreads * UN;
  uint2 pb[UN];
  for (uint32_t e0 = threadIdx.x; e0 < E; e0 += 2 * kStep) {
    acc_fetch<UN>(seg_off, seg_src, nb, E, kb, e0 + kStep, pb);
    acc_add<D, UN>(h, tile, pw, E, e0, pa);
    if (e0 + kStep >= E) break;
    acc_fetch<UN>(seg_off, seg_src, nb, E, kb, e0 + 2 * kStep, pa);
    acc_add<D, UN>(h, tile, pw, E, e0 + kStep, pb);
  }
}

// k_accumulate (partitioned path): a grid of G workgroups (a multiple of 8 where the item
// count allows), 512 threads; workgroup b accumulates items v = b, b + G, ... of the P x W
// (partition, worker) items in turn (acc_item): one item each when G = P W, else a resident
// grid walking the items.  The partition's d x 2^K buckets live in LDS.  Its entries are
// spread over one short segment per list chunk; the segments of up to kSegBatch chunks are
// flattened with a prefix sum so that consecutive threads read consecutive entries, several
// per thread in flight.  The next item's list length and first segment bounds load while
// this item accumulates, and its first segments are flattened and its first entries loaded
// before this item's tile is written, so its two dependent round trips overlap this item's
// adds and tile write.  The tile leaves with dense coalesced stores (non-temporal when nt
// is set) and, on a walking grid, is cleared in LDS as it is read.  WALK = false compiles
// the one-item-per-workgroup form, without the next item's registers.
template <int D, bool WALK>
__global__ __launch_bounds__(kAccThreads) void k_accumulate(
    HashArgs h, uint64_t tiles, const uint32_t* __restrict__ offsets, uint64_t cap,
    uint64_t chunks, uint32_t partitions, uint32_t items, const uint2* __restrict__ bins,
    const uint32_t* __restrict__ prefix, float* __restrict__ sketches, uint64_t w, int vec4,
    int nt) {
  extern __shared__ __align__(16) float tile[];  // D * 2^K
  __shared__ uint32_t seg_src[kSegBatch];
  __shared__ uint32_t seg_off[kSegBatch + 1];
  __shared__ uint32_t wtot[kAccThreads / kWave];
  constexpr int UN = acc_unroll(D);
  constexpr int PER = kSegBatch / kAccThreads;
  const int tid = threadIdx.x;
  const uint32_t pw = 1u << h.K;
  const uint32_t cells = D * pw;
  uint32_t v = blockIdx.x;
  if (v >= items) return;  // uniform
  uint32_t item = acc_item(v, items);
  uint32_t p = item % partitions, k = item / partitions;

  // The first item's list length and first batch of segment bounds: rows up to the
  // workspace's last chunk are in bounds, and those past the filled ones are dropped.  With
  // no list capacity (chunks == 0) nothing is listed and every tile is written as zeros.
  uint32_t lo[PER], hi[PER];
  if (chunks > 0)
    acc_bounds<PER>(prefix + (uint64_t)k * chunks * (partitions + 1) + p, partitions, 0, chunks,
                    lo, hi);
  const uint64_t total = offsets[(uint64_t)k * (tiles + 1) + tiles];
  for (uint32_t c = tid; c < cells; c += kAccThreads) tile[c] = 0.f;
  uint32_t nch = (uint32_t)(((total < cap ? total : cap) + kChunk - 1) / kChunk);
  uint32_t nb = nch < (uint32_t)kSegBatch ? nch : (uint32_t)kSegBatch;
  uint32_t E = nb ? acc_flatten<PER>(0, nb, lo, hi, seg_src, seg_off, wtot) : 0u;
  uint2 pa[UN];
  if (E) acc_fetch<UN>(seg_off, seg_src, nb, E, bins + (uint64_t)k * chunks * kChunk, tid, pa);

  while (true) {
    const uint32_t* pf = prefix + (uint64_t)k * chunks * (partitions + 1) + p;
    const uint2* kb = bins + (uint64_t)k * chunks * kChunk;
    // the next item's list length and first segment bounds, in flight during this item
    const uint32_t nv = v + gridDim.x;
    const bool more = WALK && nv < items;  // uniform
    const uint32_t nitem = more ? acc_item(nv, items) : item;
    const uint32_t np = nitem % partitions, nk = nitem / partitions;
    uint32_t nlo[PER], nhi[PER];
    uint64_t ntotal = 0;
    if (more) {
      if (chunks > 0)
        acc_bounds<PER>(prefix + (uint64_t)nk * chunks * (partitions + 1) + np, partitions, 0,
                        chunks, nlo, nhi);
      ntotal = offsets[(uint64_t)nk * (tiles + 1) + tiles];
    }
    // this item's batches; the first is flattened and its first group loaded already
    for (uint32_t cb = 0; cb < nch; cb += kSegBatch) {
      if (cb > 0) {
        nb = nch - cb < (uint32_t)kSegBatch ? nch - cb : (uint32_t)kSegBatch;
        acc_bounds<PER>(pf, partitions, cb, nb, lo, hi);
        __syncthreads();  // the previous batch is consumed
        E = acc_flatten<PER>(cb, nb, lo, hi, seg_src, seg_off, wtot);
        if (E) acc_fetch<UN>(seg_off, seg_src, nb, E, kb, tid, pa);
      }
      if (E) acc_batch<D, UN>(h, tile, pw, seg_off, seg_src, nb, E, kb, pa);
    }
    __syncthreads();  // the tile is complete; the segment arrays are free
    if (more) {  // the next item's first batch, before this tile is written
      nch = (uint32_t)(((ntotal < cap ? ntotal : cap) + kChunk - 1) / kChunk);
      nb = nch < (uint32_t)kSegBatch ? nch : (uint32_t)kSegBatch;
      E = nb ? acc_flatten<PER>(0, nb, nlo, nhi, seg_src, seg_off, wtot) : 0u;
      if (E) acc_fetch<UN>(seg_off, seg_src, nb, E, bins + (uint64_t)nk * chunks * kChunk, tid, pa);
    }
    float* sk = sketches + (uint64_t)k * D * w + (uint64_t)p * pw;
    if (vec4) {
      const uint32_t pw4 = pw / 4;
      f32x4* t4 = reinterpret_cast<f32x4*>(tile);
      for (uint32_t c = tid; c < D * pw4; c += kAccThreads) {
        const uint32_t j = c / pw4, q = c - j * pw4;
        const f32x4 x = t4[c];  // = tile[j pw + 4 q]
        if constexpr (WALK) t4[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4* dst = reinterpret_cast<f32x4*>(sk + (uint64_t)j * w + 4 * q);
        if (nt) __builtin_nontemporal_store(x, dst);
        else *dst = x;
      }
    } else {
      for (uint32_t c = tid; c < cells; c += kAccThreads) {
        const uint32_t j = c / pw, q = c - j * pw;
        sk[(uint64_t)j * w + q] = tile[c];
        if constexpr (WALK) tile[c] = 0.f;
      }
    }
    if (!more) break;
    __syncthreads();  // the tile is clear before the next item's adds
    v = nv;
    item = nitem;
    p = np;
    k = nk;
  }
}

// ---------------------------------------------------------------------------------------
// k_blockbits (block-granular bitmaps): grid (ceil(bwords / 4), W), 256 threads.  Wave v
// builds output word q = 4 blockIdx.x + v: lane l tests block b = 64 q + l, the OR of the
// element bits of elements [b B, b B + B) (whole words for B >= 64, a B-bit field of one
// word otherwise; element bits at or beyond n are already 0), and a ballot forms the word.
__global__ __launch_bounds__(256) void k_blockbits(const uint64_t* __restrict__ ebm,
                                                   uint64_t ewords, uint64_t n, uint32_t lb,
                                                   uint64_t bwords, uint64_t* __restrict__ bbm) {
  const uint32_t k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t q = (uint64_t)blockIdx.x * 4 + wave;
  if (q >= bwords) return;  // whole wave
  const uint64_t first = (q * 64 + lane) << lb;
  const uint64_t* e = ebm + (uint64_t)k * ewords;
  bool any = false;
  if (first < n) {
    if (lb >= 6) {
      const uint64_t w0 = first >> 6;
      uint64_t w1 = w0 + (1ull << (lb - 6));
      if (w1 > ewords) w1 = ewords;
      uint64_t acc = 0;
      for (uint64_t x = w0; x < w1; ++x) acc |= e[x];
      any = acc != 0ull;
    } else {
      const uint64_t field = (1ull << (1u << lb)) - 1ull;  // B <= 32 bits
      any = ((e[first >> 6] >> (first & 63)) & field) != 0ull;
    }
  }
  const uint64_t word = __ballot(any);
  if (lane == 0) bbm[(uint64_t)k * bwords + q] = word;
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
  trace_mark(s, "k_stream");
  hipLaunchKernelGGL(k_stream, dim3((uint32_t)tiles, W), dim3(kStreamThreads), 0, s, grad, n, ld,
                     tiles, words, bitmaps, counts);
  return hipGetLastError();
}

uint32_t scan_blocks(uint64_t tiles) {
  return (uint32_t)((tiles + kScanPass - 1) / kScanPass);
}

hipError_t launch_scan(uint32_t W, uint64_t tiles, const uint32_t* counts, uint32_t* offsets,
                       uint64_t* nnz, uint32_t* chunk_tile, uint64_t chunks, uint64_t cap,
                       uint4* btot, uint2* spans, uint32_t* nspan, hipStream_t s) {
  const uint32_t nb = tiles > 0 ? scan_blocks(tiles) : 1;
  if (nb > 1) {
    trace_mark(s, "k_scan_sum");
    hipLaunchKernelGGL(k_scan_sum, dim3(nb, W), dim3(kScanThreads), 0, s, tiles, counts, btot);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  trace_mark(s, "k_scan");
  hipLaunchKernelGGL(k_scan, dim3(nb, W), dim3(kScanThreads), 0, s, tiles, counts, offsets, nnz,
                     chunk_tile, chunks, cap, btot, spans, nspan);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, uint64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  trace_mark(s, "k_fill_zero");
  hipLaunchKernelGGL(k_fill_zero, dim3((uint32_t)blocks), dim3(256), 0, s, p, count);
  return hipGetLastError();
}

hipError_t launch_blockbits(uint32_t W, const uint64_t* ebm, uint64_t ewords, uint64_t n,
                            uint32_t log2_block, uint64_t bwords, uint64_t* bbm, hipStream_t s) {
  if (bwords == 0) return hipSuccess;
  trace_mark(s, "k_blockbits");
  hipLaunchKernelGGL(k_blockbits, dim3((uint32_t)((bwords + 3) / 4), W), dim3(256), 0, s, ebm, ewords,
                     n, log2_block, bwords, bbm);
  return hipGetLastError();
}

hipError_t launch_expand(uint32_t W, const float* grad, uint64_t ld, uint64_t tiles,
                         const uint64_t* bitmaps, uint64_t words, const uint2* spans,
                         const uint32_t* nspan, uint32_t* idx, float* val, uint64_t cap,
                         hipStream_t s) {
  if (tiles == 0 || cap == 0) return hipSuccess;
  const uint64_t nsp = (tiles + 1) / 2;
  uint64_t g = (kExpandGroups + W - 1) / W;
  if (g > nsp) g = nsp;
  trace_mark(s, "k_expand_dense");
  hipLaunchKernelGGL(k_expand_dense, dim3((uint32_t)g, W), dim3(kExpandThreads), 0, s, grad, ld,
                     tiles, bitmaps, words, spans, nspan, idx, val, cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint64_t gs = (nsp + kExpandWaves - 1) / kExpandWaves;
  if (gs > g) gs = g;
  trace_mark(s, "k_expand_sparse");
  hipLaunchKernelGGL(k_expand_sparse, dim3((uint32_t)gs, W), dim3(kExpandThreads), 0, s, grad, ld,
                     tiles, bitmaps, words, spans, nspan, idx, val, cap);
  return hipGetLastError();
}

hipError_t launch_scatter(const HashArgs& h, uint32_t W, uint64_t tiles, const uint32_t* offsets,
                          const uint32_t* idx, const float* val, uint64_t cap, uint64_t chunks,
                          float* sketches, uint64_t w, hipStream_t s) {
  if (chunks == 0) return hipSuccess;
  trace_mark(s, "k_scatter");
  S2R_DISPATCH_D(h.d, hipLaunchKernelGGL((k_scatter<D>), dim3((uint32_t)chunks, W),
                                         dim3(kScatterThreads), 0, s, h, tiles, offsets, idx, val,
                                         cap, sketches, w));
  return hipGetLastError();
}

hipError_t launch_bin(const HashArgs& h, uint32_t W, uint64_t tiles, const uint32_t* offsets,
                      const uint32_t* idx, const float* val, uint64_t cap, uint64_t chunks,
                      uint64_t partitions, uint2* bins, uint32_t* prefix, hipStream_t s) {
  if (chunks == 0) return hipSuccess;
  const size_t lds = (partitions + 1) * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bin),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  trace_mark(s, "k_bin");
  hipLaunchKernelGGL(k_bin, dim3((uint32_t)chunks, W), dim3(kBinThreads), lds, s, h, tiles,
                     offsets, idx, val, cap, chunks, (uint32_t)partitions, bins, prefix);
  return hipGetLastError();
}

hipError_t launch_accumulate(const HashArgs& h, uint32_t W, uint64_t tiles,
                             const uint32_t* offsets, uint64_t cap, uint64_t chunks,
                             uint64_t partitions, const uint2* bins, const uint32_t* prefix,
                             float* sketches, uint64_t w, hipStream_t s) {
  const size_t lds = ((size_t)h.d << h.K) * sizeof(float);
  const int vec4 = (h.K >= 2 && (reinterpret_cast<uintptr_t>(sketches) % 16) == 0) ? 1 : 0;
  // sketches larger than the Infinity Cache go out with non-temporal stores; smaller ones
  // stay cached for the reduce that reads them next (both measured faster on MI355X)
  const int nt = (uint64_t)W * ((uint64_t)h.d * w) * sizeof(float) > kCacheResidentBytes ? 1 : 0;
  const uint64_t items = partitions * W;
  if (items == 0) return hipSuccess;
  if (items > 0xffffffffull) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  // Partitions with few entries (the list capacity over P, at most kAccWalkEntries) are
  // bound by each item's two dependent round trips: a resident grid that walks the items
  // overlaps them with the previous item's adds and tile write.  Partitions with many
  // entries are bound by the LDS adds, and one workgroup per item, each slot refilled as
  // its workgroup ends, is faster.  Measured on MI355X, one workgroup per item against the
  // walking grid: 244 entries per partition 392 -> 355 us, about 2000 40 -> 37 us; about
  // 4000 the walk loses, 116 -> 125 us and 486 -> 503 us.
  const bool walk = cap / partitions <= kAccWalkEntries;
  int cus = 0;
  if (walk) {
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  S2R_DISPATCH_D(h.d, {
    const void* kfn = walk ? reinterpret_cast<const void*>(&k_accumulate<D, true>)
                           : reinterpret_cast<const void*>(&k_accumulate<D, false>);
    e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    uint64_t grid = items;
    if (e == hipSuccess && walk) {
      int per_cu = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, kAccThreads, lds);
      // as many workgroups as are resident at once, a multiple of 8 (acc_item), spread so
      // that every workgroup gets the same number of items to within one
      uint64_t most = (uint64_t)(per_cu > 0 ? per_cu : 1) * (uint64_t)(cus > 0 ? cus : 1);
      if (most > kXcds) most -= most % kXcds;
      const uint64_t rounds = (items + most - 1) / most;
      grid = (items + rounds - 1) / rounds;
      if (grid > kXcds) grid = (grid + kXcds - 1) / kXcds * kXcds;
      if (grid > most) grid = most;
      if (grid > items) grid = items;
    }
    if (e == hipSuccess) {
      trace_mark(s, "k_accumulate");
      if (walk)
        hipLaunchKernelGGL((k_accumulate<D, true>), dim3((uint32_t)grid), dim3(kAccThreads), lds,
                           s, h, tiles, offsets, cap, chunks, (uint32_t)partitions,
                           (uint32_t)items, bins, prefix, sketches, w, vec4, nt);
      else
        hipLaunchKernelGGL((k_accumulate<D, false>), dim3((uint32_t)grid), dim3(kAccThreads), lds,
                           s, h, tiles, offsets, cap, chunks, (uint32_t)partitions,
                           (uint32_t)items, bins, prefix, sketches, w, vec4, nt);
    }
  });
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace s2r
