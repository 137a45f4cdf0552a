/* s2r.h -- C ABI of the sparse-sketch gradient aggregation library (libs2r.so, gfx950).
 *
 * The operation is the data-parallel hot path of S2 Reducer ("S2 Reducer: High-Performance
 * Sparse Communication to Accelerate Distributed Deep Learning", Ge et al., arXiv
 * 2110.02140):
 *
 *   s2r_encode  -- Section 3.1 "Compressing Sparse Gradient" and the compression loop of
 *                  Algorithm 1: every worker's gradient becomes a bitmap of its non-zero
 *                  positions plus a d x w count-sketch in which each non-zero g(i) adds
 *                  s_j(i) * g(i) to bucket h_j(i) of every row j.
 *   s2r_reduce  -- Section 3.1 "Collecting Sparse-Sketch with AllReduce" (the AllReduce of
 *                  Algorithm 1): sketches add element-wise, bitmaps merge by OR.  On one
 *                  GPU the W workers are W buffers and the AllReduce is this local step.
 *   s2r_decode  -- Section 3.1 "Decompressing Sparse Gradient" and the query loop of
 *                  Algorithm 1: for every set bit i, g_hat(i) = median over rows j of
 *                  s_j(i) * S[j, h_j(i)]; every clear bit decodes to +0.0.
 *   s2r_hash    -- the bucket and sign hashes of Algorithm 1 on arbitrary keys (test hook).
 *   s2r_gather_sum -- the lossless comparator of Section 1 and Section 2.2 (Fig. 1(b)):
 *                  the exact sum of the workers' (index, value) lists.
 *   s2r_topk_ef -- Section 2.2 and Appendix A.2: block-wise Top-K sparsification with error
 *                  feedback, which produces the sparse gradients that s2r_encode compresses.
 *
 * Conventions shared by every call:
 *   - Device arrays are caller-owned device memory (hipMalloc / torch tensors).  The
 *     library never allocates, frees or synchronises.  Its only state is the static scratch
 *     of s2r_encode_noalloc (one array per GPU, with its device address looked up once per
 *     GPU under a lock) and the per-thread trace pointer of s2r_diag.h; calls from several
 *     host threads are safe as long as their buffers differ (for s2r_encode_noalloc see
 *     there).
 *   - Work is only enqueued on `stream` (a hipStream_t; NULL = the default stream).  Every
 *     argument check happens on the host before anything is enqueued, so a call that
 *     returns an error has enqueued nothing.  S2R_ERR_HIP means a launch failed.
 *   - Indices are the element positions 0..n-1 of a worker's gradient, so n < 2^32.
 *   - Bitmap layout: one bit per block of B = 2^log2_block consecutive elements (B = 1:
 *     one bit per element).  s2r_block_bitmap_words(n, log2_block) uint64 words per
 *     bitmap; bit b (block b, elements b*B .. b*B+B-1) = bit (b % 64) of word b / 64, least
 *     significant bit first; bits of blocks at or beyond ceil(n/B) are 0 on output.
 *   - Sketch layout: fp32 [d][w] row-major per worker, w = 2^log2_w.
 *   - "Non-zero" means (bits(x) & 0x7fffffff) != 0: +0 and -0 are zero, subnormals are
 *     not.  By the same test +-Inf and NaN are non-zero: they are listed with their bits,
 *     and the sketch cells and sums they reach are non-finite as IEEE arithmetic gives them
 *     (NaN where both infinite signs or a NaN meet).  Decoding a non-finite cell is outside
 *     the contract.
 */
#ifndef S2R_H
#define S2R_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S2R_MAX_ROWS 16
#define S2R_MAX_LOG2_BLOCK 16

typedef enum {
  S2R_OK = 0,
  S2R_ERR_NULL = 1,      /* a required pointer is NULL                                 */
  S2R_ERR_DIM = 2,       /* a size or parameter is out of range                        */
  S2R_ERR_ALIGN = 3,     /* a pointer or leading dimension breaks an alignment rule     */
  S2R_ERR_WORKSPACE = 4, /* the workspace is smaller than the *_workspace_bytes query    */
  S2R_ERR_HIP = 5,       /* a HIP launch failed                                        */
  S2R_ERR_SCRATCH = 6    /* s2r_encode_noalloc: the call needs more workspace than the
                            static scratch holds (S2R_NOALLOC_SCRATCH_BYTES)             */
} s2r_status;

/* Hash constants shared by every worker and by encode and decode (Algorithm 1 draws its
 * sign hashes {s_j} and bucket hashes {h_j} once, before the worker loop).  Host memory;
 * copied at call time.
 *
 *   MAS_b(a, c; x) = ((a * x + c) mod 2^64) >> (64 - b)   (the top b bits; 0 when b = 0)
 *   P(i)   = MAS_{L-K}(pA, pB; i)          partition hash, shared by all rows
 *   Q_j(i) = MAS_K(hA[j], hB[j]; i)        row hash
 *   h_j(i) = P(i) * 2^K + Q_j(i)           bucket in row j, 0 <= h_j(i) < 2^L
 *   s_j(i) = +1 if MAS_1(sA[j], sB[j]; i) == 0 else -1
 *
 * with L = log2_w and K = log2_part.  K == L makes every row an independent
 * multiply-add-shift hash (Dietzfelbinger 1996).  K < L keeps each row a uniform
 * 2-independent map onto 2^L buckets but groups all rows of an item into the same
 * partition of 2^K buckets per row; the library then accumulates and queries one
 * partition at a time in LDS instead of through global atomics and gathers.
 */
typedef struct {
  uint32_t d;         /* rows (the pages' r), 1..S2R_MAX_ROWS                         */
  uint32_t log2_w;    /* L: w = 2^L buckets per row (the pages' c, also m), 0..31        */
  uint32_t log2_part; /* K: 0..L, see above                                            */
  uint32_t log2_block; /* bitmap granularity B = 2^log2_block elements per bit, 0..16;
                          0 (the s2r_params_from_seed default) = one bit per element.
                          Section 3.1 sizes the bitmap by embedding rows or gradient
                          blocks: a block's bit is set if any of its elements is non-zero,
                          and decoding queries every element of every set block.       */
  uint64_t pA, pB;
  uint64_t hA[S2R_MAX_ROWS], hB[S2R_MAX_ROWS];
  uint64_t sA[S2R_MAX_ROWS], sB[S2R_MAX_ROWS];
} s2r_params;

/* Fill *out from a 64-bit seed: SplitMix64 (Steele, Lea & Flood 2014) seeded with `seed`
 * yields pA, pB, then hA[j], hB[j], sA[j], sB[j] for j = 0..d-1; log2_block = 0 (set it
 * afterwards for a block-granular bitmap).  Pure host code.
 * Errors: S2R_ERR_NULL (out), S2R_ERR_DIM (d, log2_w or log2_part out of range). */
s2r_status s2r_params_from_seed(uint64_t seed, uint32_t d, uint32_t log2_w, uint32_t log2_part,
                                s2r_params* out);

/* The largest K <= log2_w whose partition tile (d rows x 2^K fp32 buckets) fits the LDS
 * budget of the partitioned path; pure host code. */
uint32_t s2r_default_log2_part(uint32_t d, uint32_t log2_w);

/* Sketch-size ratio lambda (Section 3.1 "Decompressing Sparse Gradient": the sketch
 * compresses when lambda = m / (alpha d) < 1, alpha d being the number of non-zeros of a
 * d-element gradient; Appendix B.3 calls lambda the ratio of the sketch's size to the
 * number of non-zeros and finds 0.5 best for its models).  The pages size a single-row
 * sketch of m buckets in Section 3.1 but a rows x columns table in Algorithm 1, so both
 * readings are offered:
 *   per_row == 0:  lambda = rows * 2^log2_w / nnz   (every cell of the table)
 *   per_row != 0:  lambda = 2^log2_w / nnz          (one row, the pages' m)
 * nnz is whichever non-zero count the caller sizes for (one worker's, or the merged
 * union).  Returns 0.0 when nnz == 0 or rows is outside 1..S2R_MAX_ROWS or log2_w > 31.
 * Pure host code. */
double s2r_sketch_lambda(uint32_t rows, uint32_t log2_w, uint64_t nnz, int per_row);

/* The smallest log2_w in 0..31 whose sketch reaches the target ratio under the same
 * reading, s2r_sketch_lambda(rows, log2_w, nnz, per_row) >= lambda (widths are powers of
 * two, so the ratio reached lies in [lambda, 2 lambda) unless log2_w = 0 already exceeds
 * it).  Returns 0 for nnz == 0, and UINT32_MAX when rows is outside 1..S2R_MAX_ROWS, lambda
 * is not a positive finite number, or no log2_w <= 31 reaches it.  Pure host code. */
uint32_t s2r_log2_w_for_lambda(uint32_t rows, uint64_t nnz, double lambda, int per_row);

/* ceil(n / 64): uint64 words of an element-granular bitmap. */
uint64_t s2r_bitmap_words(uint64_t n);

/* ceil(ceil(n / 2^log2_block) / 64): uint64 words of a bitmap of n elements at granularity
 * 2^log2_block (the size of every bitmap argument below, with log2_block from the params). */
uint64_t s2r_block_bitmap_words(uint64_t n, uint32_t log2_block);

/* Bytes of device workspace s2r_encode needs for W workers of n elements with list
 * capacity `cap` per worker (0 if the arguments are invalid). */
size_t s2r_encode_workspace_bytes(const s2r_params* p, uint32_t W, uint64_t n, uint64_t cap);

/* Compression of W workers' gradients in one call (Section 3.1; Algorithm 1, steps before
 * the AllReduce).
 *   grad      [W][ld] fp32, row k = worker k; 16-byte aligned, ld % 4 == 0, ld >= n.
 *   bitmaps   [W][s2r_block_bitmap_words(n, p->log2_block)] uint64 out.
 *   sketches  [W][d][w] fp32 out (fully overwritten; need not be initialised).
 *   idx, val  [W][cap] out: worker k's non-zero indices in ascending order and their
 *             exact fp32 values (the compacted Sparse(g_k)); may be NULL only if cap == 0.
 *   nnz       [W] uint64 out: exact non-zero count of each worker.
 *   workspace device memory of at least s2r_encode_workspace_bytes(p, W, n, cap) bytes,
 *             256-byte aligned; its contents on entry do not matter.
 * Capacity: if nnz[k] > cap, the bitmap and nnz of worker k are still exact, but its
 * list holds only the first cap entries and its sketch is unspecified; cap >= n is always
 * safe.  Sketch cells are fp32 sums whose order is unspecified (each differs from the
 * exact sum by at most (count-1) * 2^-24 * sum|contributions|).
 * Aliasing: no output may overlap grad or another output.
 * Errors (nothing enqueued): S2R_ERR_NULL, S2R_ERR_DIM (W == 0, n >= 2^32, ld < n, bad
 * params), S2R_ERR_ALIGN, S2R_ERR_WORKSPACE; S2R_ERR_HIP on a failed launch.
 * n == 0 writes nnz = 0 and zero sketches. */
s2r_status s2r_encode(const s2r_params* p, uint32_t W, const float* grad, uint64_t n,
                      uint64_t ld, uint64_t* bitmaps, float* sketches, uint32_t* idx,
                      float* val, uint64_t cap, uint64_t* nnz, void* workspace,
                      size_t ws_bytes, void* stream);

/* Bytes of the static scratch that s2r_encode_noalloc uses as its workspace. */
#define S2R_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* s2r_encode without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops that forbid allocation, harnesses that
 * disallow hipMalloc.  Same arguments, kernels, results and errors as s2r_encode, except:
 *   - the workspace is a static device array of S2R_NOALLOC_SCRATCH_BYTES inside the
 *     library, one per GPU, held from the library's first use on that GPU until the process
 *     ends; nothing is allocated or freed by the call (no hipMalloc, no hipFree);
 *   - a call whose s2r_encode_workspace_bytes(p, W, n, cap) exceeds that size returns
 *     S2R_ERR_SCRATCH and enqueues nothing (at the five built-in workloads' sizes, the
 *     1e9-element, ResNet-50, embedding and tiny ones fit; the 160M-element one does not);
 *   - `stream` must belong to the current device (else S2R_ERR_HIP, nothing enqueued); the
 *     first call on a device looks up that device's scratch address;
 *   - every call on one GPU shares that GPU's scratch, which keeps the last call's
 *     contents (the kernels need nothing cleared): calls whose work overlaps on one GPU
 *     (other streams, other host threads) race on it and give unspecified results, so they
 *     must be ordered, e.g. on one stream. */
s2r_status s2r_encode_noalloc(const s2r_params* p, uint32_t W, const float* grad, uint64_t n,
                              uint64_t ld, uint64_t* bitmaps, float* sketches, uint32_t* idx,
                              float* val, uint64_t cap, uint64_t* nnz, void* stream);

/* Aggregation (Section 3.1; the AllReduce of Algorithm 1) of W workers on one GPU:
 *   sketch_out[c] = sum_{k=0..W-1} sketches[k][c]   (fp32, added in order k = 0, 1, ...)
 *   bitmap_out[q] = OR_k bitmaps[k][q]
 * sketches [W][d][w] and bitmaps [W][words] in, sketch_out [d][w] and bitmap_out [words]
 * out, words = s2r_block_bitmap_words(n, p->log2_block).  sketch_out may equal `sketches` and bitmap_out may equal
 * `bitmaps` (in place into worker 0's slot); other overlaps are not allowed.
 * Errors: S2R_ERR_NULL, S2R_ERR_DIM, S2R_ERR_ALIGN (sketch pointers not 4-byte aligned or
 * bitmap pointers not 8-byte aligned), S2R_ERR_HIP. */
s2r_status s2r_reduce(const s2r_params* p, uint32_t W, uint64_t n, const uint64_t* bitmaps,
                      const float* sketches, uint64_t* bitmap_out, float* sketch_out,
                      void* stream);

/* Bytes of device workspace that let s2r_decode take the partitioned path for up to
 * `max_set` set bits (0 when the params do not partition, i.e. the d x 2^K partition tile
 * does not fit the LDS budget; then s2r_decode always gathers directly). */
size_t s2r_decode_workspace_bytes(const s2r_params* p, uint64_t n, uint64_t max_set);

/* Decompression (Section 3.1; the query loop of Algorithm 1):
 *   out[i] = median_j s_j(i) * sketch[j][h_j(i)]  if the bit of i's block is set,
 *   out[i] = +0.0                                 otherwise,           for i < n.
 * For even d the median is the mean of the two middle values, rounded once to fp32.
 * "Set bits" below count the elements i < n of set blocks.
 * bitmap [s2r_block_bitmap_words(n, p->log2_block)] uint64 (bits of blocks at or beyond
 * ceil(n/B) are ignored), sketch [d][w] fp32,
 * out [n] fp32, 16-byte aligned.  Must use the same params as the encode that produced
 * the sketch.  out may not overlap the inputs.
 * Paths: with workspace == NULL (or ws_bytes == 0) every set bit gathers its d cells from
 * the sketch directly.  With a workspace of s2r_decode_workspace_bytes(p, n, max_set)
 * bytes (contents on entry irrelevant) and a sketch larger than 4 MiB, the set bits are
 * grouped by partition and each partition's cells are read once into LDS (smaller sketches
 * stay cache-resident and are gathered directly); if the bitmap turns out to hold more than
 * max_set set bits below n, the call still completes correctly through direct gathers
 * (decided on the device).  Both paths give identical results.
 * Errors: S2R_ERR_NULL, S2R_ERR_DIM, S2R_ERR_ALIGN, S2R_ERR_WORKSPACE (a non-NULL workspace
 * smaller than the query), S2R_ERR_HIP. */
s2r_status s2r_decode(const s2r_params* p, uint64_t n, const uint64_t* bitmap,
                      const float* sketch, float* out, uint64_t max_set, void* workspace,
                      size_t ws_bytes, void* stream);

/* Lossless comparator: the exact sum of the workers' sparse gradients, formed from their
 * compacted lists -- the aggregate the sketch path estimates.  Section 1 and Section 2.2
 * (Fig. 1(b)) describe it: without a mergeable structure, workers gather one another's
 * indices and values and add them afterwards.  On one GPU the W lists are already resident
 * (s2r_encode writes them), so this is the add.  For i < n:
 *   out[i] = the fp32 sum, in worker order k = 0, 1, ..., W-1 starting from +0.0, of
 *            val[k][t] over the entries t < min(nnz[k], cap) with idx[k][t] == i;
 *   out[i] = +0.0 where no worker lists i.
 * idx [W][cap] uint32, val [W][cap] fp32 and nnz [W] uint64 are device memory, read-only,
 * in the layout s2r_encode writes; the indices of one worker must be distinct (s2r_encode's
 * are strictly ascending; repeated indices give an unspecified sum at those elements).
 * Entries with idx >= n are skipped.  out [n] fp32, 16-byte aligned, may not overlap the
 * inputs.  Deterministic: the same inputs give the same bits on every run.
 * Errors: S2R_ERR_NULL, S2R_ERR_DIM (W == 0 or W > 65535, n >= 2^32), S2R_ERR_ALIGN
 * (out not 16-byte aligned, idx / val not 4-byte or nnz not 8-byte aligned), S2R_ERR_HIP. */
s2r_status s2r_gather_sum(uint32_t W, const uint32_t* idx, const float* val, uint64_t cap,
                          const uint64_t* nnz, uint64_t n, float* out, void* stream);

/* Test hook: the same device hash the other calls use, on arbitrary keys.
 *   buckets[j * m + t] = h_j(keys[t]),  signs[j * m + t] = s_j(keys[t])  (int8, +1/-1)
 * Errors: S2R_ERR_NULL, S2R_ERR_DIM, S2R_ERR_HIP. */
s2r_status s2r_hash(const s2r_params* p, const uint32_t* keys, uint64_t m, uint32_t* buckets,
                    int8_t* signs, void* stream);

/* Bytes of device workspace s2r_topk_ef needs for W workers of n elements in blocks of
 * `block` elements (0 if the arguments are invalid). */
size_t s2r_topk_workspace_bytes(uint32_t W, uint64_t n, uint64_t block);

/* Block-wise Top-K sparsification with error feedback, the step that produces the sparse
 * gradients compressed above (Section 2.2: the l2 norm of every block, the K largest blocks
 * are kept; Appendix A.2: the error sequence e_{t+1} = g_t - C(g_t), g_t = gradient_t + e_t,
 * taken here against the Top-K output itself).  Per worker k, with nb = ceil(n / block)
 * blocks (the last may be short):
 *   g[i]        = grad[i] + residual[i]    (one fp32 addition; g = grad if residual == NULL)
 *   norm2(q)    = sum over block q of g[i]^2, accumulated in fp64
 *   kept blocks = the K largest norm2, ties to the lower block id (all blocks if K >= nb)
 *   out[i]      = g[i] in kept blocks, +0.0 elsewhere        (= sparse(g))
 *   residual[i] = 0 in kept blocks, g[i] elsewhere          (= g - sparse(g))
 *   grad      [W][ld] fp32 in; residual [W][ld] fp32 in/out or NULL; out [W][ld] fp32 out
 *             (elements n..ld-1 of a row are not touched); all 16-byte aligned, ld % 4 == 0.
 *   selected  [W][ceil(nb / 64)] uint64 out, bit q = block q kept (bits >= nb are 0); may
 *             be NULL.
 *   workspace at least s2r_topk_workspace_bytes(W, n, block) bytes; contents irrelevant.
 * The squared norms are fp64 sums in the kernel's own order (per-lane partial sums, then a
 * butterfly across the wave), so a block whose norm ties another's only to within fp64
 * rounding may be ordered either way.
 * Aliasing: out may not overlap grad or residual; residual may not equal grad.
 * Errors: S2R_ERR_NULL, S2R_ERR_DIM (W == 0, block == 0, n >= 2^32, ld < n), S2R_ERR_ALIGN,
 * S2R_ERR_WORKSPACE, S2R_ERR_HIP. */
s2r_status s2r_topk_ef(uint32_t W, const float* grad, float* residual, uint64_t n, uint64_t ld,
                       uint64_t block, uint64_t K, float* out, uint64_t* selected,
                       void* workspace, size_t ws_bytes, void* stream);

/* Static string naming a status code. */
const char* s2r_status_string(s2r_status s);

#ifdef __cplusplus
}
#endif

#endif /* S2R_H */
