// s2r_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libs2r).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "s2r_device.hpp"

namespace s2r {

// ---- encode geometry -------------------------------------------------------------------
constexpr int kStreamThreads = 512;                 // 8 waves
constexpr int kStreamVec = 2;                       // float4 loads per thread
constexpr int kTile = kStreamThreads * kStreamVec * 4;  // 4096 elements per tile
constexpr int kTileWords = kTile / 64;              // 64 bitmap words per tile
constexpr int kStreamWaveSpan = kTile / (kStreamThreads / 64);  // elements per wave

constexpr int kExpandThreads = 256;
constexpr uint64_t kExpandGroups = 8192;             // expand workgroups per launch, all workers
constexpr uint32_t kDenseSpan = 1024;                // non-zeros above which a span is expanded
                                                     // by a whole workgroup, not one wave
constexpr int kScatterThreads = 256;
constexpr int kChunk = 8192;                        // list entries per chunk
constexpr int kBinThreads = 512;                    // 16 entries per thread
constexpr int kMaxPartitions = 8192;                // LDS histogram limit of the binning pass
constexpr int kAccThreads = 512;
// entries in flight per thread of the encode accumulation (measured on MI355X at d = 5:
// one is 1-5% faster than two, whose ten compare-and-swaps in flight cost registers; at
// d = 3 two win); one for many rows keeps it out of scratch
constexpr int acc_unroll(int d) { return d <= 3 ? 2 : 1; }
constexpr int kSegBatch = 1024;                     // chunk segments flattened per batch
constexpr uint64_t kAccWalkEntries = 2048;          // entries per partition up to which the
                                                    // accumulation walks items on a resident grid
constexpr size_t kAccLdsBytes = 64 * 1024;          // LDS of one partition tile
constexpr uint64_t kCacheResidentBytes = 256ull << 20;  // MI355X Infinity Cache

constexpr int kScanThreads = 1024;
// tiles per scan block: small enough that the blocks spread over many CUs (one CU writes
// its offsets and span lists slowly), four per thread so the loads all fly together
constexpr uint32_t kScanPass = kScanThreads * 4;

// Workspace layout of s2r_encode (every section 256-byte aligned).
struct EncodeLayout {
  uint64_t tiles;        // tiles per worker
  uint64_t chunks;       // list chunks per worker (bounded by min(cap, n))
  uint64_t partitions;   // 2^(L-K) on the partitioned path, 0 otherwise
  bool partitioned;
  size_t off_counts, off_offsets, off_btot, off_spans, off_nspan, off_ebm, off_bins, off_prefix,
      total;
};
EncodeLayout encode_layout(const s2r_params& p, uint32_t W, uint64_t n, uint64_t cap);
bool use_partitioned(const s2r_params& p);

HashArgs make_hash_args(const s2r_params& p);

// Kernel trace (s2r_diag_trace_attach): with a trace attached to the calling host thread,
// records its next event on `s` and names it `name`, the kernel about to be launched (or
// "end" after a call's last launch); does nothing otherwise.
void trace_mark(hipStream_t s, const char* name);

hipError_t launch_stream(uint32_t W, const float* grad, uint64_t n, uint64_t ld,
                         uint64_t tiles, uint64_t* bitmaps, uint32_t* counts, hipStream_t s);
// tiles are scanned in blocks of kScanPass; more than one block needs W * scan_blocks(tiles)
// uint4 block totals.  spans (W * ceil(tiles / 2) uint2: span, list position of its first
// pair) and nspan (2 W uint32) may be null.
uint32_t scan_blocks(uint64_t tiles);
hipError_t launch_scan(uint32_t W, uint64_t tiles, const uint32_t* counts, uint32_t* offsets,
                       uint64_t* nnz, uint32_t* chunk_tile, uint64_t chunks, uint64_t cap,
                       uint4* btot, uint2* spans, uint32_t* nspan, hipStream_t s);
hipError_t launch_fill_zero(float* p, uint64_t count, hipStream_t s);
// block-granular bitmaps [W][bwords] from element bitmaps [W][ewords]
hipError_t launch_blockbits(uint32_t W, const uint64_t* ebm, uint64_t ewords, uint64_t n,
                            uint32_t log2_block, uint64_t bwords, uint64_t* bbm, hipStream_t s);
hipError_t launch_expand(uint32_t W, const float* grad, uint64_t ld, uint64_t tiles,
                         const uint64_t* bitmaps, uint64_t words, const uint2* spans,
                         const uint32_t* nspan, uint32_t* idx, float* val, uint64_t cap,
                         hipStream_t s);
hipError_t launch_scatter(const HashArgs& h, uint32_t W, uint64_t tiles, const uint32_t* offsets,
                          const uint32_t* idx, const float* val, uint64_t cap, uint64_t chunks,
                          float* sketches, uint64_t w, hipStream_t s);
hipError_t launch_bin(const HashArgs& h, uint32_t W, uint64_t tiles, const uint32_t* offsets,
                      const uint32_t* idx, const float* val, uint64_t cap, uint64_t chunks,
                      uint64_t partitions, uint2* bins, uint32_t* prefix, hipStream_t s);
hipError_t launch_accumulate(const HashArgs& h, uint32_t W, uint64_t tiles,
                             const uint32_t* offsets, uint64_t cap, uint64_t chunks,
                             uint64_t partitions, const uint2* bins, const uint32_t* prefix,
                             float* sketches, uint64_t w, hipStream_t s);

hipError_t launch_reduce(uint32_t W, uint64_t cells, uint64_t words, const uint64_t* bitmaps,
                         const float* sketches, uint64_t* bitmap_out, float* sketch_out,
                         hipStream_t s);

// Workspace layout of the partitioned decode (total == 0 when the direct path applies).
struct DecodeLayout {
  uint64_t tiles, chunks, partitions;
  bool partitioned;
  size_t off_tcount, off_toff, off_btot, off_total, off_chunk_tile, off_bidx, off_slot, off_gval,
      off_prefix, total;
};
DecodeLayout decode_layout(const s2r_params& p, uint64_t n, uint64_t max_set);
hipError_t launch_decode(const HashArgs& h, const s2r_params& p, uint64_t n,
                         const uint64_t* bitmap, const float* sketch, float* out,
                         uint64_t max_set, void* workspace, size_t ws_bytes, hipStream_t s);

// Workspace of s2r_topk_ef: fp64 keys [W][key_stride] (nb rounded up to even), a kept-block
// bitmap [W][sel_words] (used when the caller passes none), the select's per-worker scratch
// (global digit histograms and candidate count), gathered candidates [W][16384] and the
// per-worker select outcome.
struct TopkLayout {
  uint64_t nb, key_stride, sel_words;
  uint32_t scratch_words;
  size_t off_keys, off_sel, off_scratch, off_gcand, off_outcome, total;
};
TopkLayout topk_layout(uint32_t W, uint64_t n, uint64_t block);
hipError_t launch_topk(uint32_t W, const float* grad, float* residual, uint64_t n, uint64_t ld,
                       uint64_t block, uint64_t K, float* out, uint64_t* selected,
                       void* workspace, hipStream_t s);

hipError_t launch_gather_sum(uint32_t W, const uint32_t* idx, const float* val, uint64_t cap,
                             const uint64_t* nnz, uint64_t n, float* out, hipStream_t s);

hipError_t launch_hash(const HashArgs& h, const uint32_t* keys, uint64_t m, uint32_t* buckets,
                       int8_t* signs, hipStream_t s);

}  // namespace s2r
