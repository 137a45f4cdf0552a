// api.hip -- the C ABI of libs2r (declared in include/s2r.h): host-side validation,
// SplitMix64 derivation of the hash constants, workspace layout and kernel launches.
// Every check runs before the first enqueue, so a call that returns an error has enqueued
// nothing.
#include <string.h>

#include <mutex>

#include "s2r_diag.h"
#include "s2r_launch.hpp"

namespace s2r {

static inline uint64_t splitmix64_step(uint64_t& state) {
  // SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): gamma increment, then mix
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static bool params_ok(const s2r_params* p) {
  return p && p->d >= 1 && p->d <= S2R_MAX_ROWS && p->log2_w <= 31 && p->log2_part <= p->log2_w &&
         p->log2_block <= S2R_MAX_LOG2_BLOCK;
}

HashArgs make_hash_args(const s2r_params& p) {
  HashArgs h;
  memset(&h, 0, sizeof(h));
  h.d = p.d;
  h.K = p.log2_part;
  h.lb = p.log2_block;
  h.shift_part = 32u - (p.log2_w - p.log2_part);
  h.shift_row = 32u - p.log2_part;
  h.pA = p.pA;
  h.pB = p.pB;
  for (uint32_t j = 0; j < p.d; ++j) {
    h.hA[j] = p.hA[j];
    h.hB[j] = p.hB[j];
    h.sA[j] = p.sA[j];
    h.sB[j] = p.sB[j];
  }
  return h;
}

// The trace of the calling host thread, set only by s2r_diag_trace_attach.
static thread_local s2r_trace* t_trace = nullptr;

void trace_mark(hipStream_t s, const char* name) {
  s2r_trace* t = t_trace;
  if (t == nullptr || t->count >= t->capacity) return;
  if (hipEventRecord(static_cast<hipEvent_t>(t->events[t->count]), s) != hipSuccess) {
    (void)hipGetLastError();  // an unusable event is skipped; the launch is not affected
    return;
  }
  t->names[t->count++] = name;
}

bool use_partitioned(const s2r_params& p) {
  const uint64_t tile_bytes = ((uint64_t)p.d << p.log2_part) * sizeof(float);
  const uint64_t parts = 1ull << (p.log2_w - p.log2_part);
  return tile_bytes <= kAccLdsBytes && parts <= (uint64_t)kMaxPartitions;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

EncodeLayout encode_layout(const s2r_params& p, uint32_t W, uint64_t n, uint64_t cap) {
  EncodeLayout L;
  L.tiles = (n + kTile - 1) / kTile;
  const uint64_t listable = cap < n ? cap : n;
  L.chunks = (listable + kChunk - 1) / kChunk;
  L.partitioned = use_partitioned(p);
  L.partitions = L.partitioned ? (1ull << (p.log2_w - p.log2_part)) : 0;
  size_t off = 0;
  L.off_counts = off;
  off = align256(off + (size_t)W * L.tiles * 4);
  L.off_offsets = off;
  off = align256(off + (size_t)W * (L.tiles + 1) * 4);
  L.off_btot = off;
  off = align256(off + (size_t)W * scan_blocks(L.tiles) * 16);
  L.off_spans = off;
  off = align256(off + (size_t)W * ((L.tiles + 1) / 2) * 8);
  L.off_nspan = off;
  off = align256(off + (size_t)W * 8);
  L.off_ebm = off;  // element bitmaps when the output bitmap is block-granular
  if (p.log2_block > 0) off = align256(off + (size_t)W * ((n + 63) / 64) * 8);
  L.off_bins = L.off_prefix = off;
  if (L.partitioned) {
    const size_t slots = (size_t)W * L.chunks * kChunk;
    L.off_bins = off;
    off = align256(off + slots * 8);
    L.off_prefix = off;
    off = align256(off + (size_t)W * (L.partitions + 1) * L.chunks * 4);
  }
  L.total = off > 0 ? off : 256;
  return L;
}

}  // namespace s2r

using namespace s2r;

extern "C" {

s2r_status s2r_params_from_seed(uint64_t seed, uint32_t d, uint32_t log2_w, uint32_t log2_part,
                                s2r_params* out) {
  if (!out) return S2R_ERR_NULL;
  if (d < 1 || d > S2R_MAX_ROWS || log2_w > 31 || log2_part > log2_w) return S2R_ERR_DIM;
  memset(out, 0, sizeof(*out));
  out->d = d;
  out->log2_w = log2_w;
  out->log2_part = log2_part;
  uint64_t st = seed;
  out->pA = splitmix64_step(st);
  out->pB = splitmix64_step(st);
  for (uint32_t j = 0; j < d; ++j) {
    out->hA[j] = splitmix64_step(st);
    out->hB[j] = splitmix64_step(st);
    out->sA[j] = splitmix64_step(st);
    out->sB[j] = splitmix64_step(st);
  }
  return S2R_OK;
}

uint32_t s2r_default_log2_part(uint32_t d, uint32_t log2_w) {
  if (d < 1 || d > S2R_MAX_ROWS || log2_w > 31) return 0;
  uint32_t K = log2_w;
  while (K > 0 && ((uint64_t)d << K) * sizeof(float) > kAccLdsBytes) --K;
  return K;
}

double s2r_sketch_lambda(uint32_t rows, uint32_t log2_w, uint64_t nnz, int per_row) {
  if (nnz == 0 || rows < 1 || rows > S2R_MAX_ROWS || log2_w > 31) return 0.0;
  const double cells = (double)(per_row ? 1u : rows) * (double)(1ull << log2_w);
  return cells / (double)nnz;
}

uint32_t s2r_log2_w_for_lambda(uint32_t rows, uint64_t nnz, double lambda, int per_row) {
  if (rows < 1 || rows > S2R_MAX_ROWS || !(lambda > 0.0) || !(lambda <= 1.7e308))
    return UINT32_MAX;
  if (nnz == 0) return 0;
  for (uint32_t L = 0; L <= 31; ++L)
    if (s2r_sketch_lambda(rows, L, nnz, per_row) >= lambda) return L;
  return UINT32_MAX;
}

uint64_t s2r_bitmap_words(uint64_t n) { return (n + 63) / 64; }

uint64_t s2r_block_bitmap_words(uint64_t n, uint32_t log2_block) {
  if (log2_block > 63) return 0;
  const uint64_t blocks = (n >> log2_block) + ((n & ((1ull << log2_block) - 1)) ? 1 : 0);
  return (blocks + 63) / 64;
}

size_t s2r_encode_workspace_bytes(const s2r_params* p, uint32_t W, uint64_t n, uint64_t cap) {
  if (!params_ok(p) || W == 0 || n >= (1ull << 32)) return 0;
  return encode_layout(*p, W, n, cap).total;
}

static inline bool aligned(const void* ptr, size_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) % a) == 0;
}

#define S2R_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return S2R_ERR_HIP; \
  } while (0)

// Workspace of s2r_encode_noalloc: a file-scope device array, one copy per GPU, which the
// GPU holds until the process ends.  In host code `scratch` names a host-side stand-in, so
// it is never passed to a kernel or copy: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept here.
static __device__ __align__(256) unsigned char scratch[S2R_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the device `s` runs on, which must be the current
// device; nullptr when the device cannot be determined or the lookup fails.
static void* scratch_address(hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (s != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev) {
      (void)hipGetLastError();
      return nullptr;
    }
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Argument checks of s2r_encode and s2r_encode_noalloc, workspace aside (a caller-given
// workspace is checked for NULL and alignment with the other pointers).
static s2r_status encode_check(const s2r_params* p, uint32_t W, const float* grad, uint64_t n,
                               uint64_t ld, const uint64_t* bitmaps, const float* sketches,
                               const uint32_t* idx, const float* val, uint64_t cap,
                               const uint64_t* nnz, bool ws_arg, const void* workspace) {
  if (!p || (!bitmaps && n > 0) || !sketches || !nnz || (ws_arg && !workspace)) return S2R_ERR_NULL;
  if (n > 0 && !grad) return S2R_ERR_NULL;
  if (cap > 0 && (!idx || !val)) return S2R_ERR_NULL;
  if (!params_ok(p) || W == 0 || W > 65535 || n >= (1ull << 32) || ld < n) return S2R_ERR_DIM;
  if (ld % 4 != 0 || !aligned(grad, 16) || !aligned(bitmaps, 8) || !aligned(sketches, 4) ||
      !aligned(nnz, 8) || (ws_arg && !aligned(workspace, 16)) ||
      (cap > 0 && (!aligned(idx, 4) || !aligned(val, 4))))
    return S2R_ERR_ALIGN;
  return S2R_OK;
}

// The encode kernels, in launch order, with workspace `ws` laid out as L.
static s2r_status encode_launch(const s2r_params* p, uint32_t W, const float* grad, uint64_t n,
                                uint64_t ld, uint64_t* bitmaps, float* sketches, uint32_t* idx,
                                float* val, uint64_t cap, uint64_t* nnz, const EncodeLayout& L,
                                char* ws, hipStream_t s) {
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.off_counts);
  uint32_t* offsets = reinterpret_cast<uint32_t*>(ws + L.off_offsets);
  const uint64_t w = 1ull << p->log2_w;
  const uint64_t dw = (uint64_t)p->d * w;
  const uint64_t words = s2r_bitmap_words(n);
  const HashArgs h = make_hash_args(*p);

  // block-granular output: the element bitmaps the list step needs stay in the workspace
  uint64_t* ebm = p->log2_block ? reinterpret_cast<uint64_t*>(ws + L.off_ebm) : bitmaps;
  if (!L.partitioned) S2R_TRY(launch_fill_zero(sketches, (uint64_t)W * dw, s));
  S2R_TRY(launch_stream(W, grad, n, ld, L.tiles, ebm, counts, s));
  if (p->log2_block)
    S2R_TRY(launch_blockbits(W, ebm, words, n, p->log2_block,
                             s2r_block_bitmap_words(n, p->log2_block), bitmaps, s));
  uint2* spans = reinterpret_cast<uint2*>(ws + L.off_spans);
  uint32_t* nspan = reinterpret_cast<uint32_t*>(ws + L.off_nspan);
  S2R_TRY(launch_scan(W, L.tiles, counts, offsets, nnz, nullptr, 0, cap,
                      reinterpret_cast<uint4*>(ws + L.off_btot), spans, nspan, s));
  S2R_TRY(launch_expand(W, grad, ld, L.tiles, ebm, words, spans, nspan, idx, val, cap, s));
  if (L.partitioned) {
    uint2* bins = reinterpret_cast<uint2*>(ws + L.off_bins);
    uint32_t* prefix = reinterpret_cast<uint32_t*>(ws + L.off_prefix);
    S2R_TRY(launch_bin(h, W, L.tiles, offsets, idx, val, cap, L.chunks, L.partitions, bins, prefix,
                       s));
    S2R_TRY(launch_accumulate(h, W, L.tiles, offsets, cap, L.chunks, L.partitions, bins, prefix,
                              sketches, w, s));
  } else {
    S2R_TRY(launch_scatter(h, W, L.tiles, offsets, idx, val, cap, L.chunks, sketches, w, s));
  }
  trace_mark(s, "end");
  return S2R_OK;
}

s2r_status s2r_encode(const s2r_params* p, uint32_t W, const float* grad, uint64_t n,
                      uint64_t ld, uint64_t* bitmaps, float* sketches, uint32_t* idx,
                      float* val, uint64_t cap, uint64_t* nnz, void* workspace,
                      size_t ws_bytes, void* stream) {
  const s2r_status st =
      encode_check(p, W, grad, n, ld, bitmaps, sketches, idx, val, cap, nnz, true, workspace);
  if (st != S2R_OK) return st;
  const EncodeLayout L = encode_layout(*p, W, n, cap);
  if (ws_bytes < L.total) return S2R_ERR_WORKSPACE;
  return encode_launch(p, W, grad, n, ld, bitmaps, sketches, idx, val, cap, nnz, L,
                       static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

s2r_status s2r_encode_noalloc(const s2r_params* p, uint32_t W, const float* grad, uint64_t n,
                              uint64_t ld, uint64_t* bitmaps, float* sketches, uint32_t* idx,
                              float* val, uint64_t cap, uint64_t* nnz, void* stream) {
  const s2r_status st =
      encode_check(p, W, grad, n, ld, bitmaps, sketches, idx, val, cap, nnz, false, nullptr);
  if (st != S2R_OK) return st;
  const EncodeLayout L = encode_layout(*p, W, n, cap);
  if (L.total > (size_t)S2R_NOALLOC_SCRATCH_BYTES) return S2R_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(scratch_address(s));
  if (ws == nullptr) return S2R_ERR_HIP;
  return encode_launch(p, W, grad, n, ld, bitmaps, sketches, idx, val, cap, nnz, L, ws, s);
}

s2r_status s2r_reduce(const s2r_params* p, uint32_t W, uint64_t n, const uint64_t* bitmaps,
                      const float* sketches, uint64_t* bitmap_out, float* sketch_out,
                      void* stream) {
  if (!p || !sketches || !sketch_out) return S2R_ERR_NULL;
  if (n > 0 && (!bitmaps || !bitmap_out)) return S2R_ERR_NULL;
  if (!params_ok(p) || W == 0 || n >= (1ull << 32)) return S2R_ERR_DIM;
  if (!aligned(sketches, 4) || !aligned(sketch_out, 4) || !aligned(bitmaps, 8) ||
      !aligned(bitmap_out, 8))
    return S2R_ERR_ALIGN;
  const uint64_t cells = (uint64_t)p->d << p->log2_w;
  S2R_TRY(launch_reduce(W, cells, s2r_block_bitmap_words(n, p->log2_block), bitmaps, sketches,
                        bitmap_out, sketch_out, static_cast<hipStream_t>(stream)));
  trace_mark(static_cast<hipStream_t>(stream), "end");
  return S2R_OK;
}

size_t s2r_decode_workspace_bytes(const s2r_params* p, uint64_t n, uint64_t max_set) {
  if (!params_ok(p) || n >= (1ull << 32)) return 0;
  return decode_layout(*p, n, max_set).total;
}

s2r_status s2r_decode(const s2r_params* p, uint64_t n, const uint64_t* bitmap,
                      const float* sketch, float* out, uint64_t max_set, void* workspace,
                      size_t ws_bytes, void* stream) {
  if (!p || !sketch) return S2R_ERR_NULL;
  if (n > 0 && (!bitmap || !out)) return S2R_ERR_NULL;
  if (!params_ok(p) || n >= (1ull << 32)) return S2R_ERR_DIM;
  if (!aligned(bitmap, 8) || !aligned(sketch, 4) || !aligned(out, 16) || !aligned(workspace, 16))
    return S2R_ERR_ALIGN;
  if (workspace && ws_bytes > 0 && ws_bytes < decode_layout(*p, n, max_set).total)
    return S2R_ERR_WORKSPACE;
  S2R_TRY(launch_decode(make_hash_args(*p), *p, n, bitmap, sketch, out, max_set, workspace,
                        ws_bytes, static_cast<hipStream_t>(stream)));
  trace_mark(static_cast<hipStream_t>(stream), "end");
  return S2R_OK;
}

s2r_status s2r_hash(const s2r_params* p, const uint32_t* keys, uint64_t m, uint32_t* buckets,
                    int8_t* signs, void* stream) {
  if (!p) return S2R_ERR_NULL;
  if (m > 0 && (!keys || !buckets || !signs)) return S2R_ERR_NULL;
  if (!params_ok(p)) return S2R_ERR_DIM;
  if (!aligned(keys, 4) || !aligned(buckets, 4)) return S2R_ERR_ALIGN;
  S2R_TRY(launch_hash(make_hash_args(*p), keys, m, buckets, signs,
                      static_cast<hipStream_t>(stream)));
  trace_mark(static_cast<hipStream_t>(stream), "end");
  return S2R_OK;
}

s2r_status s2r_gather_sum(uint32_t W, const uint32_t* idx, const float* val, uint64_t cap,
                          const uint64_t* nnz, uint64_t n, float* out, void* stream) {
  if (n > 0 && !out) return S2R_ERR_NULL;
  if (n > 0 && cap > 0 && (!idx || !val || !nnz)) return S2R_ERR_NULL;
  if (W == 0 || W > 65535 || n >= (1ull << 32)) return S2R_ERR_DIM;
  if (!aligned(out, 16) || !aligned(idx, 4) || !aligned(val, 4) || !aligned(nnz, 8))
    return S2R_ERR_ALIGN;
  S2R_TRY(launch_gather_sum(W, idx, val, cap, nnz, n, out, static_cast<hipStream_t>(stream)));
  trace_mark(static_cast<hipStream_t>(stream), "end");
  return S2R_OK;
}

size_t s2r_topk_workspace_bytes(uint32_t W, uint64_t n, uint64_t block) {
  if (W == 0 || block == 0 || n >= (1ull << 32)) return 0;
  return topk_layout(W, n, block).total;
}

s2r_status s2r_topk_ef(uint32_t W, const float* grad, float* residual, uint64_t n, uint64_t ld,
                       uint64_t block, uint64_t K, float* out, uint64_t* selected,
                       void* workspace, size_t ws_bytes, void* stream) {
  if (n > 0 && (!grad || !out || !workspace)) return S2R_ERR_NULL;
  if (W == 0 || W > 65535 || block == 0 || n >= (1ull << 32) || ld < n) return S2R_ERR_DIM;
  if (ld % 4 != 0 || !aligned(grad, 16) || !aligned(residual, 16) || !aligned(out, 16) ||
      !aligned(selected, 8) || !aligned(workspace, 16))
    return S2R_ERR_ALIGN;
  if (n > 0 && ws_bytes < topk_layout(W, n, block).total) return S2R_ERR_WORKSPACE;
  if (n > 0 && residual == grad) return S2R_ERR_DIM;
  S2R_TRY(launch_topk(W, grad, residual, n, ld, block, K, out, selected, workspace,
                      static_cast<hipStream_t>(stream)));
  trace_mark(static_cast<hipStream_t>(stream), "end");
  return S2R_OK;
}

s2r_status s2r_diag_trace_attach(s2r_trace* t) {
  if (t && (t->capacity > S2R_TRACE_MAX || t->count > t->capacity)) return S2R_ERR_DIM;
  t_trace = t;
  return S2R_OK;
}

const char* s2r_status_string(s2r_status s) {
  switch (s) {
    case S2R_OK: return "ok";
    case S2R_ERR_NULL: return "null pointer argument";
    case S2R_ERR_DIM: return "size or parameter out of range";
    case S2R_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case S2R_ERR_WORKSPACE: return "workspace too small";
    case S2R_ERR_HIP: return "HIP launch failed";
    case S2R_ERR_SCRATCH: return "workspace need exceeds the static scratch of the allocation-free call";
  }
  return "unknown status";
}

}  // extern "C"
