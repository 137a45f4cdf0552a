// decode.hip -- decompression: merged bitmap + merged sketch -> dense g_hat.
//
// S2 Reducer (arXiv 2110.02140) Section 3.1 "Decompressing Sparse Gradient" and the query
// loop of Algorithm 1: recover the indices from the set bits of the merged bitmap and, for
// each, take the median over rows j of s_j(i) * S[j, h_j(i)]; clear bits decode to +0.0.
//
// Two paths.
//
// Direct (no workspace, or a table small enough to stay cache-resident): k_dwrite_direct
// gathers, for every set bit of its 8192-element tile, the d sketch cells from memory (the
// gathers of several set bits in flight per thread) and takes a register median; the tile
// is written with 128-bit coalesced stores, zeros included.
// Random gathers into a table larger than L2 run at ~55-80 G/s on MI355X, so this path is
// bound by the d*U gathers.
//
// Partitioned (h_j(i) = P(i) 2^K + Q_j(i), all rows of an item in one partition):
//   k_dcount   popcount per 8192-element tile of the merged bitmap;
//   k_scan     tile rank offsets, the number U of set bits, and the tile where every chunk
//              of 8192 consecutive ranks starts;
//   k_dbin     per rank chunk: expands its indices from the bitmap (a round's words
//              spread over every wave where a chunk fills less than a round), counting-sorts
//              them by partition in LDS, writes them partition-ordered with 16-bit
//              per-partition offsets, and records for every rank its slot in that order;
//   k_dmedian  per partition (split over rank-chunk ranges): loads the partition's d x 2^K
//              cells into LDS and takes every item's median from LDS, writing it at the
//              item's slot;
//   k_dunsort  per rank chunk: moves the medians from slot order to rank order, when set
//              bits are dense (U >= n / kDecSparseRatio);
//   k_dwrite   per tile: reads the medians of its set bits (in rank order, or through
//              each rank's slot when set bits are sparse) and writes the tile.
// If U exceeds the workspace capacity, k_dbin, k_dmedian and k_dunsort do nothing and
// k_dwrite falls back to the direct gathers, decided on the device.
// With a block-granular bitmap (one bit per 2^lb elements) every kernel reads element words
// built from the block bits (masked_word), so the set bits above are the elements of set
// blocks.
#include <string.h>

#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecTile = 8192;
constexpr int kDecWords = kDecTile / 64;     // 128
constexpr uint64_t kDirectTableBytes = 4ull << 20;  // one XCD's L2
constexpr int kDBinThreads = 512;         // dense bitmaps: a chunk's set bits span few words
constexpr int kDBinThreadsWide = 1024;    // sparse bitmaps: a chunk spans many rounds of words
constexpr int kDUnsortThreads = 512;
// Below one set bit in kDecSparseRatio elements the medians stay in slot order and k_dwrite
// reads each through its slot: a tile then holds few set bits, and the gathers cost less
// than the unsort pass (measured on MI355X: at 0.8% density the decode is 63 us faster
// over 10^9 elements; at 7.7% and 27% the gathers are 11 and 175 us slower).
constexpr uint64_t kDecSparseRatio = 32;
constexpr int kDMedianUnroll = 4;  // items in flight per thread (stride kAccThreads)
constexpr int kTileLoads = 8;      // 16-byte cell loads per thread in flight when a tile fills
// Workgroups k_dmedian aims for when partitions are few: each split reloads its partition's
// cells, so fewer splits trade parallelism for cell traffic (measured on MI355X with 128
// partitions of 48 KiB, the ResNet-50 workload: 8 splits 25.5 us, 4 splits 21 us, 3 or
// 2 splits 23-24 us)
constexpr uint64_t kDMedianTargetGroups = 512;
constexpr uint32_t kDMedianMaxSplits = 8;
// Set bits per k_dmedian workgroup above which a partition's chunks are split further
// (measured on MI355X: about 21K per workgroup -> 11K took the Transformer workload's
// k_dmedian 349 -> 317 us; below about 7K the extra cell loads cost more than they save)
constexpr uint64_t kDMedianGroupItems = 16384;
constexpr int kDBinWordsPerThread = 4;

// Element word q (elements 64q .. 64q+63) of the query set, bits at or beyond n cleared.
// nwords = ceil(n / 64).  With a block-granular bitmap (lb = log2 B > 0) the word is built
// from the block bits: all ones or zeros for B >= 64, else each of its 64/B block bits
// spread over B element bits.
// The bitmap word that element word q (< nwords) is built from: q itself, or the word
// holding q's block bits.
__device__ __forceinline__ uint64_t masked_src(uint64_t q, uint32_t lb) {
  return lb == 0 ? q : ((q * 64) >> lb) >> 6;
}

// Element word q built from raw = bitmap[masked_src(q, lb)]; 0 for q >= nwords.
__device__ __forceinline__ uint64_t masked_from(uint64_t raw, uint64_t nwords, uint64_t n,
                                                uint64_t q, uint32_t lb) {
  if (q >= nwords) return 0ull;
  const uint64_t first = q * 64;
  uint64_t wv;
  if (lb == 0) {
    wv = raw;
  } else if (lb >= 6) {
    const uint64_t b = first >> lb;
    wv = ((raw >> (b & 63)) & 1ull) ? ~0ull : 0ull;
  } else {
    const uint32_t B = 1u << lb, per = 64u >> lb;  // B <= 32, per <= 32
    const uint64_t b0 = first >> lb;               // a multiple of per: one bitmap word
    const uint64_t bits = (raw >> (b0 & 63)) & ((1ull << per) - 1ull);
    const uint64_t ones = (1ull << B) - 1ull;
    wv = 0ull;
    for (uint32_t t = 0; t < per; ++t)
      if ((bits >> t) & 1ull) wv |= ones << (t * B);
  }
  if (n - first < 64) wv &= (1ull << (n - first)) - 1ull;
  return wv;
}

// Element word q (0 for q >= nwords; nwords > 0): the load is unconditional, at a clamped
// index, so that several of them issue back to back.
__device__ __forceinline__ uint64_t masked_word(const uint64_t* __restrict__ bitmap,
                                                uint64_t nwords, uint64_t n, uint64_t q,
                                                uint32_t lb) {
  const uint64_t raw = bitmap[masked_src(q < nwords ? q : nwords - 1, lb)];
  return masked_from(raw, nwords, n, q, lb);
}

// ---------------------------------------------------------------------------------------
// k_dcount: 256 threads, a wave per two 8192-element tiles (no barrier): lane l takes words
// 4l .. 4l + 3 of the wave's 256 (lanes 0-31 the first tile, 32-63 the second), all four
// loads issued before any is masked, and a half-wave sum gives each tile's count.
constexpr int kDcountThreads = 256;
constexpr int kDcountTiles = 2 * kDcountThreads / kWave;  // tiles per workgroup

// Sum over the 32 lanes of each half of the wave.
__device__ __forceinline__ uint32_t half_wave_sum(uint32_t x) {
#pragma unroll
  for (int off = kWave / 4; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__global__ __launch_bounds__(kDcountThreads) void k_dcount(const uint64_t* __restrict__ bitmap,
                                                           uint64_t n, uint64_t nwords,
                                                           uint64_t tiles, uint32_t lb,
                                                           uint32_t* __restrict__ tcount) {
  const int lane = threadIdx.x & 63;
  const uint64_t vb = xcd_run_item(blockIdx.x, gridDim.x, 256);  // 2 MiB of bitmap per XCD run
  const uint64_t t0 = (vb * (kDcountThreads / kWave) + (threadIdx.x >> 6)) * 2;
  if (t0 >= tiles) return;  // wave-uniform
  const uint64_t q0 = t0 * kDecWords + 4 * lane;
  uint64_t r[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = bitmap[masked_src(q0 + u < nwords ? q0 + u : nwords - 1, lb)];
  uint32_t c = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) c += (uint32_t)__popcll(masked_from(r[u], nwords, n, q0 + u, lb));
  c = half_wave_sum(c);
  const uint64_t t = t0 + (lane >> 5);
  if ((lane & 31) == 0 && t < tiles) tcount[t] = c;
}

// ---------------------------------------------------------------------------------------
// The partitioned path's workspace, shared by k_dbin, k_dmedian, k_dunsort and k_dwrite.
struct DecodeWs {
  const uint32_t* toff;       // [tiles + 1] rank offset of every tile
  const uint32_t* chunk_tile; // [chunks] tile holding rank c * kChunk
  uint32_t* bidx;             // [chunks][kChunk] indices, partition-ordered per chunk
  uint16_t* slot;             // [chunks][kChunk] rank -> slot in that order
  float* gval;                // [chunks][kChunk] median of the item at each slot (k_dmedian),
                              // then of each rank (k_dunsort, dense set bits only)
  uint16_t* prefix;           // [chunks][P + 1] partition starts per chunk (<= kChunk)
  uint64_t chunks;            // capacity in chunks (max_set rounded up)
  uint64_t max_set;
  uint64_t sparse_below;      // U below this: no unsort pass; k_dwrite reads through slots
};

// List expansion of bitmap words held in registers: thread t owns words
// qbase + t * tstride + u * ustride (u < WPT), whose first set bit has list rank rank[u].
// Writes item[r - start] = 64 * word + bit for every set bit with rank r in [start, end).
// The wave visits only lanes whose word is non-empty and meets the range (a ballot),
// broadcasts that word, and expands its 64 bits with one lane per bit (v_mbcnt gives each
// bit's rank), so the cost follows the set bits in range, not the span of words.  Word
// indices and ranks fit 32 bits: n < 2^32 elements have fewer than 2^26 words and set bits.
template <int WPT>
__device__ __forceinline__ void expand_owned_words(const uint64_t* wv, const uint32_t* rank,
                                                   uint32_t qbase, uint32_t tstride,
                                                   uint32_t ustride, uint32_t start,
                                                   uint32_t end, uint32_t* item, int tid) {
  const int lane = tid & (kWave - 1);
  const uint32_t qwave = qbase + (uint32_t)(tid - lane) * tstride;
#pragma unroll
  for (int u = 0; u < WPT; ++u) {
    const uint32_t pc = (uint32_t)__popcll(wv[u]);
    uint64_t m = __ballot(pc != 0 && rank[u] < end && rank[u] + pc > start);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const uint64_t w = readlane64(wv[u], l);
      const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)rank[u], l) + bits_below_lane(w);
      const uint32_t q = qwave + (uint32_t)l * tstride + (uint32_t)u * ustride;
      if (((w >> lane) & 1ull) && r >= start && r < end) item[r - start] = q * 64u + (uint32_t)lane;
    }
  }
}

// Word u (< kDBinWordsPerThread) of thread tid in a k_dbin round starting at word q0.
// Interleaved (IL): q0 + u * NT + tid, so a run of set bits shorter than the round spreads
// over every wave (dense bitmaps, where a chunk's set bits fill a fraction of one round);
// else blocked: q0 + kDBinWordsPerThread * tid + u (sparse bitmaps, where a chunk spans
// several rounds and every wave already meets it).
template <int NT, bool IL>
__device__ __forceinline__ uint32_t dbin_word_index(uint32_t q0, int u, int tid) {
  return IL ? q0 + (uint32_t)(u * NT + tid) : q0 + (uint32_t)(kDBinWordsPerThread * tid + u);
}

// Raw bitmap words of a k_dbin round (clamped below q_end, so every load issues
// unconditionally; masked in dbin_round).
template <int NT, bool IL>
__device__ __forceinline__ void dbin_words(const uint64_t* __restrict__ bitmap, uint32_t q0,
                                           uint32_t q_end, uint32_t lb, int tid, uint64_t* wv) {
#pragma unroll
  for (int u = 0; u < kDBinWordsPerThread; ++u) {
    const uint32_t q = dbin_word_index<NT, IL>(q0, u, tid);
    wv[u] = bitmap[masked_src(q < q_end ? q : q_end - 1, lb)];
  }
}

// One round of k_dbin's rank expansion over words [q0, q0 + NT * kDBinWordsPerThread):
// masks the thread's raw words (in place), ranks them in word order and expands the set bits
// whose rank lies in [start, end) into litem; advances q0 and rank0.  Blocked: one workgroup
// scan of the threads' popcount sums.  Interleaved: slice u (every thread's word u) precedes
// slice u + 1; the four popcounts go through the wave scan as 16-bit fields of two words (a
// wave's field sums stay below 2^13) and the per-wave sums are combined in full words.
// Called by the whole workgroup (two barriers).
template <int NT, bool IL>
__device__ __forceinline__ void dbin_round(uint64_t* wv, uint64_t n, uint64_t nwords,
                                           uint32_t q_end, uint32_t lb, uint32_t start,
                                           uint32_t end, uint32_t& q0, uint32_t& rank0,
                                           uint32_t* litem, uint4* wtot, int tid) {
  static_assert(kDBinWordsPerThread == 4, "four slices packed in two scan words");
  constexpr int NW = NT / kWave;
  const int wave = tid >> 6, lane = tid & 63;
  uint32_t pc[kDBinWordsPerThread];
#pragma unroll
  for (int u = 0; u < kDBinWordsPerThread; ++u) {
    const uint32_t q = dbin_word_index<NT, IL>(q0, u, tid);
    wv[u] = q < q_end ? masked_from(wv[u], nwords, n, q, lb) : 0ull;  // masked in place
    pc[u] = (uint32_t)__popcll(wv[u]);
  }
  uint32_t rk0[kDBinWordsPerThread];
  if constexpr (IL) {
    const uint32_t a = pc[0] | (pc[1] << 16), b = pc[2] | (pc[3] << 16);
    const uint32_t ia = wave_inclusive_sum(a), ib = wave_inclusive_sum(b);
    if (lane == kWave - 1) wtot[wave] = make_uint4(ia & 0xFFFFu, ia >> 16, ib & 0xFFFFu, ib >> 16);
    __syncthreads();
    const uint32_t ea = ia - a, eb = ib - b;  // exclusive, within the wave
    uint32_t before[kDBinWordsPerThread] = {ea & 0xFFFFu, ea >> 16, eb & 0xFFFFu, eb >> 16};
    uint32_t total[kDBinWordsPerThread] = {0u, 0u, 0u, 0u};
#pragma unroll 4
    for (int v = 0; v < NW; ++v) {
      const uint4 t = wtot[v];
      if (v < wave) {
        before[0] += t.x; before[1] += t.y; before[2] += t.z; before[3] += t.w;
      }
      total[0] += t.x; total[1] += t.y; total[2] += t.z; total[3] += t.w;
    }
    uint32_t base = rank0;
#pragma unroll
    for (int u = 0; u < kDBinWordsPerThread; ++u) {
      rk0[u] = base + before[u];
      base += total[u];
    }
    rank0 = base;
  } else {
    const uint32_t sum = pc[0] + pc[1] + pc[2] + pc[3];
    const uint32_t inc = wave_inclusive_sum(sum);
    if (lane == kWave - 1) wtot[wave].x = inc;
    __syncthreads();
    uint32_t before = inc - sum, total = 0;
    for (int v = 0; v < NW; ++v) {
      if (v < wave) before += wtot[v].x;
      total += wtot[v].x;
    }
#pragma unroll
    for (int u = 0; u < kDBinWordsPerThread; ++u) {
      rk0[u] = rank0 + before;
      before += pc[u];
    }
    rank0 += total;
  }
  expand_owned_words<kDBinWordsPerThread>(wv, rk0, q0, IL ? 1u : (uint32_t)kDBinWordsPerThread,
                                          IL ? (uint32_t)NT : 1u, start, end, litem, tid);
  q0 += (uint32_t)(NT * kDBinWordsPerThread);
  __syncthreads();  // wtot is reused next round
}

// k_dbin: grid = rank chunks, NT threads; IL selects the word layout of the rank expansion
// (dbin_word_index).  The 512-thread kernel is held to six waves per SIMD, so three
// workgroups (40 KiB of LDS each with P = 2048) share a CU.
template <int NT, bool IL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT <= 512 ? 6 : 4)))
void k_dbin(HashArgs h, uint64_t n, const uint64_t* __restrict__ bitmap, uint64_t nwords,
            uint64_t tiles, DecodeWs ws, uint32_t P) {
  extern __shared__ uint32_t hist[];  // P + 1
  // the chunk's indices in rank order, then (once every thread holds its own in registers)
  // in partition order
  __shared__ __align__(16) uint32_t litem[kChunk];
  __shared__ uint4 wtot[NT / kWave];
  const uint32_t c = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t U = ws.toff[tiles];
  const uint32_t t0 = ws.chunk_tile[c];  // loaded with U (c < chunks); meaningful if start < U
  if (U > ws.max_set) return;  // over capacity: k_dwrite decodes directly
  // ranks and bitmap word indices below fit 32 bits (U <= n < 2^32, nwords < 2^26)
  const uint32_t start = c * (uint32_t)kChunk;
  if (start >= U) return;
  const uint32_t cnt = (uint32_t)(U - start < kChunk ? U - start : kChunk);
  const uint32_t end = start + cnt;

  // 1. expand ranks [start, end) into litem, NT * kDBinWordsPerThread bitmap words per round
  //    (expand_owned_words visits only the non-empty words that meet the chunk).  The
  //    chunk's last rank lies at or before the tile where the next chunk starts, so words
  //    past that tile are not read (a thread past it re-reads the last word in range and
  //    drops it).
  uint32_t q0 = t0 * (uint32_t)kDecWords;
  uint32_t rank0 = ws.toff[t0];
  const uint64_t t_last = end < U ? (uint64_t)ws.chunk_tile[c + 1] : tiles - 1;
  const uint32_t q_end =
      (uint32_t)((t_last + 1) * kDecWords < nwords ? (t_last + 1) * kDecWords : nwords);
  // The next round's words are loaded before the current round is expanded (register sets
  // a and b alternate, so no loaded register is copied); past q_end they re-read the last
  // word in range and are never used.
  constexpr uint32_t kRound = (uint32_t)(NT * kDBinWordsPerThread);  // words per round
  uint64_t wa[kDBinWordsPerThread], wb[kDBinWordsPerThread];
  dbin_words<NT, IL>(bitmap, q0, q_end, h.lb, tid, wa);
  while (rank0 < end && q0 < q_end) {
    dbin_words<NT, IL>(bitmap, q0 + kRound, q_end, h.lb, tid, wb);
    dbin_round<NT, IL>(wa, n, nwords, q_end, h.lb, start, end, q0, rank0, litem, wtot, tid);
    if (!(rank0 < end && q0 < q_end)) break;
    dbin_words<NT, IL>(bitmap, q0 + kRound, q_end, h.lb, tid, wa);
    dbin_round<NT, IL>(wb, n, nwords, q_end, h.lb, start, end, q0, rank0, litem, wtot, tid);
  }
  for (uint32_t p = tid; p <= P; p += NT) hist[p] = 0;
  __syncthreads();

  // 2. counting sort by partition; each thread keeps its items in registers, so litem can
  //    take the sorted order
  constexpr int R = kChunk / NT;
  uint32_t it[R], rk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t s = tid + NT * r;
    if (s < cnt) {
      it[r] = litem[s];
      rk[r] = atomicAdd(&hist[partition_of(h, it[r])], 1u);
    }
  }
  __syncthreads();
  {  // exclusive scan of hist[0..P) in place
    const uint32_t per = (P + NT - 1) / NT;
    const uint32_t lo = tid * per < P ? tid * per : P;
    const uint32_t hi = lo + per < P ? lo + per : P;
    uint32_t sum = 0;
    for (uint32_t p = lo; p < hi; ++p) sum += hist[p];
    const uint32_t inc = wave_inclusive_sum(sum);
    if (lane == kWave - 1) wtot[wave].x = inc;
    __syncthreads();
    uint32_t run = inc - sum;
    for (int v = 0; v < wave; ++v) run += wtot[v].x;
    for (uint32_t p = lo; p < hi; ++p) {
      const uint32_t x = hist[p];
      hist[p] = run;
      run += x;
    }
    __syncthreads();
  }
  uint16_t* pf = ws.prefix + (uint64_t)c * (P + 1);  // one contiguous row per chunk
  for (uint32_t p = tid; p < P; p += NT) pf[p] = (uint16_t)hist[p];
  if (tid == 0) pf[P] = (uint16_t)cnt;
  uint16_t* sl = ws.slot + start;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t s = tid + NT * r;
    if (s < cnt) {
      const uint32_t pos = hist[partition_of(h, it[r])] + rk[r];
      litem[pos] = it[r];
      sl[s] = (uint16_t)pos;
    }
  }
  __syncthreads();
  uint32_t* bo = ws.bidx + start;
  const uint32_t cnt4 = cnt / 4;
  for (uint32_t q = tid; q < cnt4; q += NT)
    *reinterpret_cast<uint4*>(bo + 4 * q) = *reinterpret_cast<const uint4*>(&litem[4 * q]);
  for (uint32_t s = 4 * cnt4 + tid; s < cnt; s += NT) bo[s] = litem[s];
}

// ---------------------------------------------------------------------------------------
// The d x 2^K cells of one partition (rows w apart, 16-byte aligned) into the LDS tile,
// kTileLoads 128-bit loads per thread in flight.  NT: non-temporal loads, for cells that
// no other workgroup reads.
template <int D, bool NT>
__device__ __forceinline__ void dmedian_cells(const float* __restrict__ sk, uint64_t w,
                                              uint32_t pw, float* tile, int tid) {
  const uint32_t pw4 = pw / 4, n4 = D * pw4;
  for (uint32_t c0 = tid; c0 < n4; c0 += kAccThreads * kTileLoads) {
    f32x4 v[kTileLoads];
#pragma unroll
    for (int u = 0; u < kTileLoads; ++u) {
      const uint32_t c = c0 + u * kAccThreads < n4 ? c0 + u * kAccThreads : n4 - 1;
      const uint32_t j = c / pw4, q = c - j * pw4;
      const f32x4* src = reinterpret_cast<const f32x4*>(sk + (uint64_t)j * w + 4 * q);
      v[u] = NT ? __builtin_nontemporal_load(src) : *src;
    }
#pragma unroll
    for (int u = 0; u < kTileLoads; ++u) {
      const uint32_t c = c0 + u * kAccThreads;
      if (c < n4) *reinterpret_cast<f32x4*>(&tile[4 * c]) = v[u];  // j pw + 4 q = 4 c
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_dmedian: grid (partitions, splits), kAccThreads threads, items XCD-grouped.  LDS holds
// the partition's d x 2^K cells (non-temporal loads when nt: with one split no other
// workgroup reads them); workgroup (p, s) takes the partition-p items of the s-th of
// `splits` equal ranges of rank chunks (their segments flattened as in the encode
// accumulation, kDMedianUnroll items per thread in flight) and writes each median at its
// item's slot.
template <int D>
__global__ __launch_bounds__(kAccThreads) void k_dmedian(HashArgs h, uint64_t tiles,
                                                         const float* __restrict__ sketch,
                                                         uint64_t w, DecodeWs ws, uint32_t P,
                                                         int vec4, int nt) {
  extern __shared__ __align__(16) float tile[];  // D * 2^K
  __shared__ uint32_t seg_src[kSegBatch];
  __shared__ uint32_t seg_off[kSegBatch + 1];
  __shared__ uint32_t wtot[kAccThreads / kWave];
  const uint32_t item = xcd_grouped_item();
  const uint32_t p = item % P, split = item / P;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t U = ws.toff[tiles];
  const uint32_t pw = 1u << h.K;
  const float* sk = sketch + (uint64_t)p * pw;
  // The partition's cells are loaded in the same round trip as U (they do not depend on
  // it), kTileLoads per thread with every load issued before any is stored to LDS.
  if (vec4) {
    if (nt) dmedian_cells<D, true>(sk, w, pw, tile, tid);
    else dmedian_cells<D, false>(sk, w, pw, tile, tid);
  } else {
    for (uint32_t c = tid; c < D * pw; c += kAccThreads) {
      const uint32_t j = c / pw, q = c - j * pw;
      tile[c] = sk[(uint64_t)j * w + q];
    }
  }
  if (U > ws.max_set || U == 0) return;
  const uint64_t nch = (U + kChunk - 1) / kChunk;
  const uint32_t c_lo = (uint32_t)(nch * split / gridDim.y);
  const uint32_t c_hi = (uint32_t)(nch * (split + 1) / gridDim.y);
  if (c_lo >= c_hi) return;
  const uint16_t* pf = ws.prefix + p;  // column p of the chunk-major offsets
  constexpr int PER = kSegBatch / kAccThreads;
  for (uint32_t cb = c_lo; cb < c_hi; cb += kSegBatch) {
    const uint32_t nb = c_hi - cb < (uint32_t)kSegBatch ? c_hi - cb : (uint32_t)kSegBatch;
    __syncthreads();  // the previous batch is consumed (and the tile is loaded)
    uint32_t lo[PER], hi[PER], len[PER], sum = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {  // clamped, unconditional loads: all in flight at once
      const uint32_t c = tid * PER + u < nb ? tid * PER + u : nb - 1;
      const uint64_t row = (uint64_t)(cb + c) * (P + 1);
      lo[u] = pf[row];
      hi[u] = pf[row + 1];
    }
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
      if (c <= nb) seg_off[c] = run;
      run += len[u];
    }
    if (tid == kAccThreads - 1 && nb == (uint32_t)kSegBatch) seg_off[kSegBatch] = run;
    __syncthreads();
    const uint32_t E = seg_off[nb];
    for (uint32_t e0 = tid; e0 < E; e0 += kAccThreads * kDMedianUnroll) {
      uint32_t e[kDMedianUnroll], c[kDMedianUnroll];
#pragma unroll
      for (int u = 0; u < kDMedianUnroll; ++u) e[u] = e0 + u * kAccThreads;
      segments_of<kDMedianUnroll>(seg_off, nb, e, c);
      uint32_t at[kDMedianUnroll], ii[kDMedianUnroll];
      // Unconditional loads (an item at or past E is read as item E - 1 of the last segment,
      // which its search returned, and dropped below); the empty asm uses the values so the
      // compiler cannot sink a load into the branch that consumes it, after other stores.
#pragma unroll
      for (int u = 0; u < kDMedianUnroll; ++u) {
        const uint32_t x = e[u] < E ? e[u] : E - 1;
        at[u] = seg_src[c[u]] + (x - seg_off[c[u]]);
        ii[u] = ws.bidx[at[u]];
      }
#pragma unroll
      for (int u = 0; u < kDMedianUnroll; ++u) asm volatile("" : "+v"(ii[u]));
#pragma unroll
      for (int u = 0; u < kDMedianUnroll; ++u) {
        if (e[u] < E) {
          float v[D];
#pragma unroll
          for (int j = 0; j < D; ++j)
            v[j] = apply_sign(tile[j * pw + row_bucket(h, j, ii[u])], sign_mask(h, j, ii[u]));
          ws.gval[at[u]] = median_of<D>(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_dunsort: grid = rank chunks, kDUnsortThreads threads.  Puts a chunk's medians from slot
// order into rank order in place: the chunk's 8192 values are staged in LDS with coalesced
// loads, then rank r takes the value at its slot, with coalesced slot reads and stores.  The
// slot reads issue together with the value loads, before the barrier (clamped indices, so
// every load issues unconditionally; the workspace holds whole chunks, so index 0 and the
// first 16 bytes of the chunk are always in bounds).
__global__ __launch_bounds__(kDUnsortThreads) void k_dunsort(uint64_t tiles, DecodeWs ws) {
  __shared__ __align__(16) float lv[kChunk];
  constexpr int VPT = kChunk / kDUnsortThreads;  // 16 ranks per thread
  const uint32_t c = blockIdx.x;
  const int tid = threadIdx.x;
  const uint64_t U = ws.toff[tiles];
  if (U > ws.max_set || U < ws.sparse_below) return;
  const uint64_t start = (uint64_t)c * kChunk;
  if (start >= U) return;
  const uint32_t cnt = (uint32_t)(U - start < kChunk ? U - start : kChunk);
  float* g = ws.gval + start;
  const uint16_t* sl = ws.slot + start;
  const uint32_t cnt4 = cnt / 4;
  f32x4 gv[VPT / 4];
  uint32_t sv[VPT];
#pragma unroll
  for (int m = 0; m < VPT / 4; ++m) {
    const uint32_t q = tid + kDUnsortThreads * m;
    gv[m] = *reinterpret_cast<const f32x4*>(g + 4 * (q < cnt4 ? q : 0u));
  }
#pragma unroll
  for (int m = 0; m < VPT; ++m) {
    const uint32_t r = tid + kDUnsortThreads * m;
    sv[m] = sl[r < cnt ? r : 0u];
  }
#pragma unroll
  for (int m = 0; m < VPT / 4; ++m) {
    const uint32_t q = tid + kDUnsortThreads * m;
    if (q < cnt4) *reinterpret_cast<f32x4*>(&lv[4 * q]) = gv[m];
  }
  for (uint32_t s = 4 * cnt4 + tid; s < cnt; s += kDUnsortThreads) lv[s] = g[s];
  __syncthreads();
#pragma unroll
  for (int m = 0; m < VPT; ++m) {
    const uint32_t r = tid + kDUnsortThreads * m;
    if (r < cnt) g[r] = lv[sv[m]];
  }
}

// ---------------------------------------------------------------------------------------
// k_dwrite (partitioned path): grid = tiles, 256 threads.  Thread t writes the float4 groups
// g = t + 256 r (elements base + 4g .. 4g + 3, r = 0..7) straight from registers, zeros
// included.  The tile's 128 bitmap words and their rank offsets sit in LDS; the set bits of
// a group take consecutive ranks starting at the word's offset plus the popcount of the
// bits below the group, and their medians are read in rank order (after k_dunsort), or, with
// sparse set bits, each through its rank's slot.  If U exceeds the workspace capacity (the
// other partitioned kernels then did nothing), each set bit instead gathers its d cells and
// takes the median in registers.
template <int D>
__global__ __launch_bounds__(kDecThreads) void k_dwrite(HashArgs h, uint64_t n, uint64_t nwords,
                                                        const uint64_t* __restrict__ bitmap,
                                                        const float* __restrict__ sketch,
                                                        uint64_t w, float* __restrict__ out,
                                                        DecodeWs ws, uint64_t tiles) {
  __shared__ uint64_t lw[kDecWords];
  __shared__ uint32_t lwo[kDecWords];
  __shared__ uint32_t wtot[2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t tile = xcd_run_item(blockIdx.x, gridDim.x, 64);  // 2 MiB of output per XCD run
  const uint64_t base = tile * kDecTile;
  uint64_t wv = 0;
  if (tid < kDecWords)
    wv = masked_word(bitmap, nwords, n, tile * kDecWords + tid, h.lb);
  const uint32_t pc = (uint32_t)__popcll(wv);
  const uint32_t inc = wave_inclusive_sum(pc);
  if (tid < kDecWords) {
    lw[tid] = wv;
    if (lane == kWave - 1) wtot[wave] = inc;
  }
  __syncthreads();
  if (tid < kDecWords) lwo[tid] = inc - pc + (wave ? wtot[0] : 0u);
  __syncthreads();
  const uint64_t U = ws.toff[tiles];
  const bool direct = U > ws.max_set;
  const bool via_slot = U < ws.sparse_below;  // k_dunsort did nothing
  const uint32_t rank0 = ws.toff[tile];  // ranks fit 32 bits (U <= n < 2^32)
  constexpr int RPT = kDecTile / 4 / kDecThreads;  // 8 groups per thread
  uint32_t nib[RPT], rk[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const uint32_t g = tid + kDecThreads * r;
    const uint32_t q = g >> 4, sh = 4 * (g & 15);
    const uint64_t word = lw[q];
    nib[r] = (uint32_t)(word >> sh) & 0xFu;
    rk[r] = lwo[q] + (uint32_t)__popcll(word & ((1ull << sh) - 1ull));
  }
  f32x4 o[RPT];
  if (!direct && !via_slot) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      // a group's set bits have consecutive ranks
      float v[4];
      uint32_t k = rk[r];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[b] = 0.f;
        if ((nib[r] >> b) & 1u) v[b] = ws.gval[rank0 + k++];
      }
      o[r] = f32x4{v[0], v[1], v[2], v[3]};
    }
  } else if (!direct) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      float v[4];
      uint32_t k = rk[r];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[b] = 0.f;
        if ((nib[r] >> b) & 1u) {
          const uint32_t R = rank0 + k++;  // median at its chunk's slot
          v[b] = ws.gval[(R & ~(uint32_t)(kChunk - 1)) + ws.slot[R]];
        }
      }
      o[r] = f32x4{v[0], v[1], v[2], v[3]};
    }
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      float m[4] = {0.f, 0.f, 0.f, 0.f};
      if (nib[r]) {
        const uint32_t i0 = (uint32_t)(base + 4 * (tid + kDecThreads * r));
        float v[4][D];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if ((nib[r] >> b) & 1u) {
            const uint32_t i = i0 + b;
            const uint32_t part = partition_of(h, i);
#pragma unroll
            for (int j = 0; j < D; ++j)
              v[b][j] = apply_sign(sketch[(uint64_t)j * w + bucket_of(h, part, j, i)],
                                   sign_mask(h, j, i));
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if ((nib[r] >> b) & 1u) m[b] = median_of<D>(v[b]);
      }
      o[r] = f32x4{m[0], m[1], m[2], m[3]};
    }
  }
  if (base + kDecTile <= n) {
    // non-temporal: the output is not read again by this path, and cached stores leave it
    // dirty in L2 and the Infinity Cache, where the next encode's gradient stream has to
    // evict it (measured on MI355X: whole steps 0.4-1.1% faster, though this kernel alone
    // is up to 15% slower on the embedding workload)
    f32x4* o4 = reinterpret_cast<f32x4*>(out + base);
#pragma unroll
    for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(o[r], &o4[tid + kDecThreads * r]);
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const uint64_t e = base + 4 * (uint64_t)(tid + kDecThreads * r);
      if (e + 0 < n) out[e + 0] = o[r].x;
      if (e + 1 < n) out[e + 1] = o[r].y;
      if (e + 2 < n) out[e + 2] = o[r].z;
      if (e + 3 < n) out[e + 3] = o[r].w;
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_dwrite_direct: the direct path (no partitioned workspace), grid = tiles, 256 threads.
// Thread t owns the float4 groups g = t + 256 r (r = 0..7) of its 8192-element tile, as in
// k_dwrite, and collects the set bits of those 32 elements into one mask.  It then walks
// the mask direct_batch<D>() set bits at a time (8 for d <= 3, else 4): the d gathers of
// every bit in the batch issue before any median is taken, so a thread waits once per
// batch rather than once per group.
// Each median goes to the element's place in an LDS copy of the tile; the thread reads its
// own groups back (no barrier: no other thread touches them) and stores them, zeros at
// clear bits, with 128-bit stores.
template <int D>
constexpr int direct_batch() { return D <= 3 ? 8 : 4; }

template <int D>
__global__ __launch_bounds__(kDecThreads) void k_dwrite_direct(
    HashArgs h, uint64_t n, uint64_t nwords, const uint64_t* __restrict__ bitmap,
    const float* __restrict__ sketch, uint64_t w, float* __restrict__ out) {
  __shared__ __align__(16) float lout[kDecTile];
  const int tid = threadIdx.x;
  const uint64_t tile = xcd_run_item(blockIdx.x, gridDim.x, 64);  // 2 MiB of output per XCD run
  const uint64_t base = tile * kDecTile;
  constexpr int RPT = kDecTile / 4 / kDecThreads;  // 8 groups per thread
  // group g = tid + 256 r lies in word g >> 4 = (tid >> 4) + 16 r at bit 4 (tid & 15)
  uint64_t raw[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {  // all eight loads first, then the (branchy) masking
    const uint64_t q = tile * kDecWords + (tid >> 4) + 16 * r;
    raw[r] = bitmap[masked_src(q < nwords ? q : nwords - 1, h.lb)];
  }
  uint32_t mask = 0;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const uint64_t q = tile * kDecWords + (tid >> 4) + 16 * r;
    const uint64_t wv = masked_from(raw[r], nwords, n, q, h.lb);
    mask |= (uint32_t)((wv >> (4 * (tid & 15))) & 0xFu) << (4 * r);
  }
  constexpr int B = direct_batch<D>();
  for (uint32_t left = mask; left != 0;) {
    uint32_t slot[B];
    bool on[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      on[u] = left != 0;
      const uint32_t q = on[u] ? (uint32_t)__builtin_ctz(left) : 0u;  // bit 4r + b
      left &= left - 1u;                                                // 0 stays 0
      slot[u] = 4u * (tid + kDecThreads * (q >> 2)) + (q & 3u);         // element in the tile
    }
    float v[B][D];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t i = (uint32_t)(base + slot[u]);
      const uint32_t part = partition_of(h, i);
      // unconditional: a lane past its last set bit gathers element `base`'s cells (the
      // same cells for all such lanes) and drops them, so no load waits on a branch
#pragma unroll
      for (int j = 0; j < D; ++j)
        v[u][j] = apply_sign(sketch[(uint64_t)j * w + bucket_of(h, part, j, i)],
                             sign_mask(h, j, i));
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (on[u]) lout[slot[u]] = median_of<D>(v[u]);
  }
  f32x4 o[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const uint32_t nib = (mask >> (4 * r)) & 0xFu;
    const f32x4 x = *reinterpret_cast<const f32x4*>(&lout[4 * (tid + kDecThreads * r)]);
    o[r] = f32x4{(nib & 1u) ? x.x : 0.f, (nib & 2u) ? x.y : 0.f, (nib & 4u) ? x.z : 0.f,
                 (nib & 8u) ? x.w : 0.f};
  }
  if (base + kDecTile <= n) {
    f32x4* o4 = reinterpret_cast<f32x4*>(out + base);
#pragma unroll
    for (int r = 0; r < RPT; ++r) o4[tid + kDecThreads * r] = o[r];
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const uint64_t e = base + 4 * (uint64_t)(tid + kDecThreads * r);
      if (e + 0 < n) out[e + 0] = o[r].x;
      if (e + 1 < n) out[e + 1] = o[r].y;
      if (e + 2 < n) out[e + 2] = o[r].z;
      if (e + 3 < n) out[e + 3] = o[r].w;
    }
  }
}

// ---------------------------------------------------------------------------------------
// host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(const s2r_params& p, uint64_t n, uint64_t max_set) {
  DecodeLayout L;
  L.tiles = (n + kDecTile - 1) / kDecTile;
  const uint64_t cap = max_set < n ? max_set : n;
  L.chunks = (cap + kChunk - 1) / kChunk;
  L.partitioned = use_partitioned(p) && n > 0;
  L.partitions = 1ull << (p.log2_w - p.log2_part);
  size_t off = 0;
  L.off_tcount = off;
  off = align256(off + L.tiles * 4);
  L.off_toff = off;
  off = align256(off + (L.tiles + 1) * 4);
  L.off_btot = off;
  off = align256(off + (size_t)scan_blocks(L.tiles) * 16);
  L.off_total = off;
  off = align256(off + 8);
  L.off_chunk_tile = off;
  off = align256(off + L.chunks * 4);
  L.off_bidx = off;
  off = align256(off + L.chunks * kChunk * 4);
  L.off_slot = off;
  off = align256(off + L.chunks * kChunk * 2);
  L.off_gval = off;
  off = align256(off + L.chunks * kChunk * 4);
  L.off_prefix = off;
  off = align256(off + (L.partitions + 1) * L.chunks * 2);
  L.total = L.partitioned ? off : 0;
  return L;
}

hipError_t launch_decode(const HashArgs& h, const s2r_params& p, uint64_t n,
                         const uint64_t* bitmap, const float* sketch, float* out,
                         uint64_t max_set, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t w = 1ull << p.log2_w;
  const uint64_t nwords = (n + 63) / 64;
  const DecodeLayout L = decode_layout(p, n, max_set);
  // direct gathers win while the table fits one XCD's L2; past it every gather pulls a
  // line from the Infinity Cache or HBM (measured on MI355X: a 6 MiB table decodes 1.3x
  // faster partitioned, a 21 MiB one 2.5x)
  const uint64_t table_bytes = ((uint64_t)p.d << p.log2_w) * sizeof(float);
  const bool part = L.partitioned && workspace != nullptr && ws_bytes >= L.total &&
                    table_bytes > kDirectTableBytes;
  DecodeWs ws;
  memset(&ws, 0, sizeof(ws));
  if (part) {
    char* b = static_cast<char*>(workspace);
    uint32_t* tcount = reinterpret_cast<uint32_t*>(b + L.off_tcount);
    uint32_t* toff = reinterpret_cast<uint32_t*>(b + L.off_toff);
    uint32_t* chunk_tile = reinterpret_cast<uint32_t*>(b + L.off_chunk_tile);
    ws.toff = toff;
    ws.chunk_tile = chunk_tile;
    ws.bidx = reinterpret_cast<uint32_t*>(b + L.off_bidx);
    ws.slot = reinterpret_cast<uint16_t*>(b + L.off_slot);
    ws.gval = reinterpret_cast<float*>(b + L.off_gval);
    ws.prefix = reinterpret_cast<uint16_t*>(b + L.off_prefix);
    ws.chunks = L.chunks;
    ws.max_set = L.chunks * kChunk < max_set ? L.chunks * kChunk : max_set;
    if (ws.max_set > n) ws.max_set = n;
    ws.sparse_below = n / kDecSparseRatio;
    trace_mark(s, "k_dcount");
    hipLaunchKernelGGL(k_dcount, dim3((uint32_t)((L.tiles + kDcountTiles - 1) / kDcountTiles)),
                       dim3(kDcountThreads), 0, s, bitmap, n, nwords, L.tiles, h.lb,
                       tcount);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_scan(1, L.tiles, tcount, toff, reinterpret_cast<uint64_t*>(b + L.off_total),
                    chunk_tile, L.chunks, ws.max_set, reinterpret_cast<uint4*>(b + L.off_btot),
                    nullptr, nullptr, s);
    if (e != hipSuccess) return e;
    if (L.chunks > 0) {
      const size_t lds = (L.partitions + 1) * sizeof(uint32_t);
      // A chunk of kChunk set bits spans about nwords * kChunk / U bitmap words (max_set
      // stands in for U on the host).  Where that is more than four rounds of the 512-thread
      // kernel, twice the threads halve the rounds (measured on MI355X: 99 -> 80 us on a
      // 1e9-element bitmap at 0.8% density; on denser ones the wide kernel is 40-65% slower)
      const bool wide = nwords * (uint64_t)kChunk >
                        4 * (uint64_t)kDBinThreads * kDBinWordsPerThread * ws.max_set;
      const void* kfn = wide ? reinterpret_cast<const void*>(&k_dbin<kDBinThreadsWide, false>)
                             : reinterpret_cast<const void*>(&k_dbin<kDBinThreads, true>);
      e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      trace_mark(s, "k_dbin");
      if (wide)
        hipLaunchKernelGGL((k_dbin<kDBinThreadsWide, false>), dim3((uint32_t)L.chunks),
                           dim3(kDBinThreadsWide), lds, s, h, n, bitmap, nwords, L.tiles, ws,
                           (uint32_t)L.partitions);
      else
        hipLaunchKernelGGL((k_dbin<kDBinThreads, true>), dim3((uint32_t)L.chunks), dim3(kDBinThreads),
                           lds, s, h, n, bitmap, nwords, L.tiles, ws, (uint32_t)L.partitions);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const size_t tlds = ((size_t)p.d << p.log2_part) * sizeof(float);
      const int vec4 = (p.log2_part >= 2 && (reinterpret_cast<uintptr_t>(sketch) % 16) == 0);
      // about kDMedianTargetGroups workgroups, and at most about kDMedianGroupItems set bits
      // per workgroup (max_set stands in for U); each split reloads the partition's cells,
      // so never more splits than rank chunks
      uint32_t splits = (uint32_t)((kDMedianTargetGroups + L.partitions - 1) / L.partitions);
      const uint64_t by_items =
          (ws.max_set + L.partitions * kDMedianGroupItems - 1) / (L.partitions * kDMedianGroupItems);
      if (by_items > splits) splits = (uint32_t)(by_items < kDMedianMaxSplits ? by_items : kDMedianMaxSplits);
      if (splits > kDMedianMaxSplits) splits = kDMedianMaxSplits;
      if (splits > L.chunks) splits = (uint32_t)L.chunks;
      if (splits < 1) splits = 1;
      // with one split every partition's cells are read by one workgroup only: they stream
      // past the caches (measured on MI355X: the 1e9-element workload's k_dmedian 99 -> 87 us
      // and its k_dwrite 718 -> 706 us; with two or more splits the cached loads are faster)
      const int nt = splits == 1 ? 1 : 0;
      S2R_DISPATCH_D(p.d, {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dmedian<D>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)tlds);
        if (e == hipSuccess) {
          trace_mark(s, "k_dmedian");
          hipLaunchKernelGGL((k_dmedian<D>), dim3((uint32_t)L.partitions, splits), dim3(kAccThreads), tlds,
                             s, h, L.tiles, sketch, w, ws, (uint32_t)L.partitions, vec4, nt);
        }
      });
      if (e != hipSuccess) return e;
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      // U <= max_set < sparse_below, or U > max_set (direct): no unsort either way
      if (ws.max_set >= ws.sparse_below) {
        trace_mark(s, "k_dunsort");
        hipLaunchKernelGGL(k_dunsort, dim3((uint32_t)L.chunks), dim3(kDUnsortThreads), 0, s,
                           L.tiles, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  const uint64_t tiles = (n + kDecTile - 1) / kDecTile;
  if (part) {
    trace_mark(s, "k_dwrite");
    S2R_DISPATCH_D(p.d, hipLaunchKernelGGL((k_dwrite<D>), dim3((uint32_t)tiles),
                                           dim3(kDecThreads), 0, s, h, n, nwords, bitmap, sketch,
                                           w, out, ws, tiles));
  } else {
    trace_mark(s, "k_dwrite_direct");
    S2R_DISPATCH_D(p.d, hipLaunchKernelGGL((k_dwrite_direct<D>), dim3((uint32_t)tiles),
                                           dim3(kDecThreads), 0, s, h, n, nwords, bitmap, sketch,
                                           w, out));
  }
  return hipGetLastError();
}

}  // namespace s2r
