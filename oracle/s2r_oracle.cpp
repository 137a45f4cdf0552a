// s2r_oracle.cpp -- plain, slow, fp64 CPU oracle for sparse-sketch gradient aggregation.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load or call this library.  The GPU library never links it and
// shares no code, header, table or helper with it.
//
// What it computes follows "S2 Reducer: High-Performance Sparse Communication to
// Accelerate Distributed Deep Learning" (Ge et al., arXiv 2110.02140):
//   * Section 3.1, "Compressing Sparse Gradient": a bitmap marks the non-zero positions
//     and every non-zero g(i) adds s(i)*g(i) to bucket h(i); zeros change nothing.
//   * Section 3.1, "Collecting Sparse-Sketch with AllReduce": sketches of W workers are
//     summed element-wise (the sketch is the linear map A^T g), bitmaps are merged.
//   * Section 3.1, "Decompressing Sparse Gradient" and Algorithm 1: for every set bit
//     i of the merged bitmap, g_hat(i) is the median over the r rows of
//     s_j(i) * S[j, h_j(i)].
//   * Section 1 and Section 2.2 (Fig. 1(b)): the lossless alternative the sketch is
//     measured against, the gathered (index, value) lists of all workers added up.
//
// Readings taken where the pages leave a step open (each also listed in the design notes):
//   * one bitmap bit per block of 2^log2_block consecutive elements (the pages give the
//     bitmap one entry per embedding row or gradient block); log2_block = 0 is one bit per
//     element.
//     A block's bit is set when any of its elements is non-zero, and decoding queries every
//     element of every set block;
//   * "non-zero" is the bit test (bits(x) & 0x7fffffff) != 0: +0 and -0 are zero;
//   * hashes are multiply-add-shift (Dietzfelbinger 1996) on the element index with
//     64-bit constants drawn from SplitMix64 (Steele, Lea & Flood 2014);
//   * bucket of row j: the high L-K bits are a partition hash P(i) shared by all rows and
//     the low K bits are a per-row hash Q_j(i); K == L gives fully independent rows;
//   * merge of bitmaps = bitwise OR; aggregation = sum (no division by W);
//   * even row count: median = mean of the two middle values.
//
// Arithmetic: sketch cells are accumulated in fp64 from the fp32 inputs, and an
// "absolute mass" table A (sum of |contribution| per cell) is carried alongside; it
// is the scale of the fp32 rounding error a faithful GPU implementation may show.
// Built with -ffp-contract=off.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

extern "C" {

// Oracle-local parameter block.  Same field order as the GPU library's by convention
// (the Python side fills each from its own derivation), but declared here separately.
#define ORC_MAX_ROWS 16
struct orc_params {
  uint32_t d;          // rows (the pages' r)
  uint32_t log2_w;     // L: w = 2^L buckets per row (the pages' c, also m)
  uint32_t log2_part;  // K: low bucket bits hashed per row; the high L-K bits are shared
  uint32_t log2_block;  // bitmap granularity: one bit per 2^log2_block elements
  uint64_t pA, pB;                 // shared partition hash constants
  uint64_t hA[ORC_MAX_ROWS], hB[ORC_MAX_ROWS];  // per-row bucket hash constants
  uint64_t sA[ORC_MAX_ROWS], sB[ORC_MAX_ROWS];  // per-row sign hash constants
};

// ---------------------------------------------------------------------------------
// SplitMix64, from its published definition (Steele, Lea & Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014): advance the state by the golden
// gamma, then apply the variant-13 finaliser of MurmurHash3.
uint64_t orc_splitmix64_next(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Draw the hash constants: pA, pB, then for each row j: hA_j, hB_j, sA_j, sB_j.
int orc_params_from_seed(uint64_t seed, uint32_t d, uint32_t log2_w, uint32_t log2_part,
                         orc_params* out) {
  if (!out || d < 1 || d > ORC_MAX_ROWS || log2_w > 31 || log2_part > log2_w) return 1;
  std::memset(out, 0, sizeof(*out));
  out->d = d;
  out->log2_w = log2_w;
  out->log2_part = log2_part;
  uint64_t st = seed;
  out->pA = orc_splitmix64_next(&st);
  out->pB = orc_splitmix64_next(&st);
  for (uint32_t j = 0; j < d; ++j) {
    out->hA[j] = orc_splitmix64_next(&st);
    out->hB[j] = orc_splitmix64_next(&st);
    out->sA[j] = orc_splitmix64_next(&st);
    out->sB[j] = orc_splitmix64_next(&st);
  }
  return 0;
}

// ---------------------------------------------------------------------------------
// Multiply-add-shift: the top `bits` bits of (a*x + c) mod 2^64.  The product is formed
// exactly in 128 bits and reduced, as the textbook definition reads.
static uint64_t mas_top(uint64_t a, uint64_t c, uint64_t x, unsigned bits) {
  if (bits == 0) return 0;
  unsigned __int128 full = (unsigned __int128)a * (unsigned __int128)x + c;
  uint64_t low64 = (uint64_t)full;  // mod 2^64
  return low64 >> (64 - bits);
}

// Bucket of element index i in row j: the pages' h_j(i) (Algorithm 1, bucket hashes).
uint32_t orc_bucket(const orc_params* p, uint32_t j, uint32_t i) {
  unsigned L = p->log2_w, K = p->log2_part;
  uint64_t part = mas_top(p->pA, p->pB, i, L - K);
  uint64_t low = mas_top(p->hA[j], p->hB[j], i, K);
  return (uint32_t)((part << K) | low);
}

// Sign of element index i in row j: the pages' s_j(i) in {-1,+1} (Algorithm 1, sign hashes).
int orc_sign(const orc_params* p, uint32_t j, uint32_t i) {
  return 1 - 2 * (int)mas_top(p->sA[j], p->sB[j], i, 1);
}

// Hash probe: buckets[j*m + t] and signs[j*m + t] for keys[t].
void orc_hash(const orc_params* p, const uint32_t* keys, uint64_t m, uint32_t* buckets,
              int8_t* signs) {
  for (uint32_t j = 0; j < p->d; ++j)
    for (uint64_t t = 0; t < m; ++t) {
      buckets[(uint64_t)j * m + t] = orc_bucket(p, j, keys[t]);
      signs[(uint64_t)j * m + t] = (int8_t)orc_sign(p, j, keys[t]);
    }
}

// ---------------------------------------------------------------------------------
// "Non-zero" reading: the magnitude bits of the fp32 pattern are not all zero.
static bool is_nonzero(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (u & 0x7FFFFFFFu) != 0;
}

static void insert(const orc_params* p, uint32_t i, float g, double* S, double* A) {
  uint64_t w = 1ull << p->log2_w;
  for (uint32_t j = 0; j < p->d; ++j) {
    uint64_t cell = (uint64_t)j * w + orc_bucket(p, j, i);
    S[cell] += (double)orc_sign(p, j, i) * (double)g;
    A[cell] += std::fabs((double)g);
  }
}

// Bitmap granularity (Section 3.1, "Compressing Sparse Gradient": one bitmap entry per
// embedding row or gradient block): element i belongs to block i >> log2_block.
static uint64_t block_of(const orc_params* p, uint64_t i) { return i >> p->log2_block; }

// ceil(ceil(n / 2^log2_block) / 64) words: bit b = bit (b%64) of word b/64.
uint64_t orc_bitmap_words(const orc_params* p, uint64_t n) {
  const uint64_t blocks = (n + (1ull << p->log2_block) - 1) >> p->log2_block;
  return (blocks + 63) / 64;
}

// Compression of one worker's dense gradient g[0..n) (Section 3.1, Algorithm 1):
// initialise bitmap and table, set the bit of the block of every non-zero, list the
// non-zeros in ascending index order, and insert each into every row of the sketch.
// bitmap: orc_bitmap_words(p, n) words.  S, A: d*w doubles.
// idx/val receive at most `cap` entries; *nnz receives the exact count.
int orc_encode_dense(const orc_params* p, const float* g, uint64_t n, uint64_t* bitmap,
                     double* S, double* A, uint32_t* idx, float* val, uint64_t cap,
                     uint64_t* nnz) {
  if (n >= (1ull << 32)) return 2;
  uint64_t words = orc_bitmap_words(p, n), cells = (uint64_t)p->d << p->log2_w;
  std::memset(bitmap, 0, words * 8);
  std::memset(S, 0, cells * 8);
  std::memset(A, 0, cells * 8);
  uint64_t count = 0;
  for (uint64_t i = 0; i < n; ++i) {
    if (!is_nonzero(g[i])) continue;
    const uint64_t b = block_of(p, i);
    bitmap[b / 64] |= 1ull << (b % 64);
    if (count < cap) {
      idx[count] = (uint32_t)i;
      val[count] = g[i];
    }
    ++count;
    insert(p, (uint32_t)i, g[i], S, A);
  }
  *nnz = count;
  return 0;
}

// Compression from Sparse(g) given as (index, value) pairs -- Algorithm 1's own input
// form.  Indices must be < n; each pair is inserted as a non-zero.
int orc_encode_sparse(const orc_params* p, const uint32_t* idx, const float* val,
                      uint64_t k, uint64_t n, uint64_t* bitmap, double* S, double* A) {
  if (n >= (1ull << 32)) return 2;
  uint64_t words = orc_bitmap_words(p, n), cells = (uint64_t)p->d << p->log2_w;
  std::memset(bitmap, 0, words * 8);
  std::memset(S, 0, cells * 8);
  std::memset(A, 0, cells * 8);
  for (uint64_t t = 0; t < k; ++t) {
    if (idx[t] >= n) return 3;
    if (!is_nonzero(val[t])) continue;
    const uint64_t b = block_of(p, idx[t]);
    bitmap[b / 64] |= 1ull << (b % 64);
    insert(p, idx[t], val[t], S, A);
  }
  return 0;
}

// Aggregation (Section 3.1, AllReduce step): S = sum_k S_k and A = sum_k A_k in worker
// order k = 0..W-1; bitmap = OR_k bitmap_k.  Inputs are [W][cells] and [W][words].
void orc_reduce(uint32_t W, uint64_t cells, uint64_t words, const uint64_t* bitmaps,
                const double* S, const double* A, uint64_t* bm_out, double* S_out,
                double* A_out) {
  for (uint64_t c = 0; c < cells; ++c) {
    double s = 0.0, a = 0.0;
    for (uint32_t k = 0; k < W; ++k) {
      s += S[(uint64_t)k * cells + c];
      a += A[(uint64_t)k * cells + c];
    }
    S_out[c] = s;
    A_out[c] = a;
  }
  for (uint64_t q = 0; q < words; ++q) {
    uint64_t m = 0;
    for (uint32_t k = 0; k < W; ++k) m |= bitmaps[(uint64_t)k * words + q];
    bm_out[q] = m;
  }
}

// Decompression (Section 3.1, "Decompressing Sparse Gradient"; Algorithm 1 query loop):
// recover the indices from the bitmap -- every element i < n whose block bit is set -- and,
// for each, take the median over rows of s_j(i) * S[j, h_j(i)].  Output is sparse: ascending indices with value and
// tolerance tol(i) = 1e-5 * max_j A[j, h_j(i)] + 1e-12.  Returns the number of set bits;
// at most `cap` entries are written.
uint64_t orc_decode(const orc_params* p, uint64_t n, const uint64_t* bitmap, const double* S,
                    const double* A, uint32_t* out_idx, double* out_val, double* out_tol,
                    uint64_t cap) {
  uint64_t w = 1ull << p->log2_w;
  uint32_t d = p->d;
  std::vector<double> est(d);
  uint64_t count = 0;
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t b = block_of(p, i);
    if (!((bitmap[b / 64] >> (b % 64)) & 1ull)) continue;
    double amax = 0.0;
    for (uint32_t j = 0; j < d; ++j) {
      uint64_t cell = (uint64_t)j * w + orc_bucket(p, j, (uint32_t)i);
      est[j] = (double)orc_sign(p, j, (uint32_t)i) * S[cell];
      amax = std::max(amax, A[cell]);
    }
    std::sort(est.begin(), est.end());
    double med = (d % 2) ? est[(d - 1) / 2] : 0.5 * (est[d / 2 - 1] + est[d / 2]);
    if (count < cap) {
      out_idx[count] = (uint32_t)i;
      out_val[count] = med;
      out_tol[count] = 1e-5 * amax + 1e-12;
    }
    ++count;
  }
  return count;
}

// ---------------------------------------------------------------------------------
// Lossless aggregation, the comparator the sketch is measured against (Section 1 and
// Section 2.2 with Fig. 1(b): without a mergeable structure, workers gather one another's
// indices and values and add them).  For each worker k = 0..W-1 in turn, every entry t below
// len[k] of its list adds val[k][t] to element idx[k][t]; entries at or beyond n are skipped.
//   idx, val [W][stride]; out [n] = the exact sum in fp64; mass [n] = the sum of |value|.
void orc_gather_sum(uint32_t W, const uint32_t* idx, const float* val, const uint64_t* len,
                    uint64_t stride, uint64_t n, double* out, double* mass) {
  for (uint64_t i = 0; i < n; ++i) {
    out[i] = 0.0;
    mass[i] = 0.0;
  }
  for (uint32_t k = 0; k < W; ++k)
    for (uint64_t t = 0; t < len[k]; ++t) {
      const uint64_t i = idx[(uint64_t)k * stride + t];
      if (i >= n) continue;
      const double v = (double)val[(uint64_t)k * stride + t];
      out[i] += v;
      mass[i] += std::fabs(v);
    }
}

// ---------------------------------------------------------------------------------
// Block-wise Top-K sparsification with error feedback, the step that produces the sparse
// gradients the method compresses (Section 2.2: l2 norm of every block, the K largest
// blocks are kept; Appendix A.2: the error sequence e_{t+1} = g_t - C(g_t) with
// g_t = gradient_t + e_t).  Readings: the residual is taken against the Top-K output
// itself, e_{t+1} = g_t - sparse(g_t); blocks are ordered by squared norm, larger first,
// then by lower block id; the squared norm is the plain fp64 sum of the squares of the
// block's fp32 elements in index order, and g_t = gradient_t + e_t is one fp32 addition.
//   grad [n], residual [n] (in/out; NULL = no error feedback), out [n] = sparse(g),
//   sel [ceil(nb/64)] bitmap of the kept blocks, norm2 [nb]; nb = ceil(n / block).
int orc_topk_ef(const float* grad, float* residual, uint64_t n, uint64_t block, uint64_t K,
                float* out, uint64_t* sel, double* norm2) {
  if (block == 0) return 1;
  const uint64_t nb = (n + block - 1) / block;
  std::vector<float> g(n);
  for (uint64_t i = 0; i < n; ++i) g[i] = residual ? grad[i] + residual[i] : grad[i];
  for (uint64_t q = 0; q < nb; ++q) {
    double s = 0.0;
    for (uint64_t i = q * block; i < n && i < (q + 1) * block; ++i) s += (double)g[i] * (double)g[i];
    norm2[q] = s;
  }
  std::vector<uint64_t> order(nb);
  for (uint64_t q = 0; q < nb; ++q) order[q] = q;
  std::sort(order.begin(), order.end(), [&](uint64_t a, uint64_t b) {
    return norm2[a] > norm2[b] || (norm2[a] == norm2[b] && a < b);
  });
  std::memset(sel, 0, ((nb + 63) / 64) * 8);
  for (uint64_t r = 0; r < K && r < nb; ++r) sel[order[r] / 64] |= 1ull << (order[r] % 64);
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t q = i / block;
    const bool kept = (sel[q / 64] >> (q % 64)) & 1ull;
    out[i] = kept ? g[i] : 0.0f;
    if (residual) residual[i] = kept ? 0.0f : g[i];
  }
  return 0;
}

}  // extern "C"
