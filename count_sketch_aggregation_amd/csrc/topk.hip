// topk.hip -- block-wise Top-K sparsification with error feedback, the step that produces
// the sparse gradients the method compresses.
//
// S2 Reducer (arXiv 2110.02140) Section 2.2: the gradient is cut into blocks, the l2 norm of
// every block is taken and the K largest blocks are kept; Appendix A.2 carries the error
// sequence e_{t+1} = g_t - C(g_t) with g_t = gradient_t + e_t.  Here the residual is taken
// against the Top-K output itself, e_{t+1} = g_t - sparse(g_t).
//
// Three passes per call, all W workers batched (grid y = worker):
//   k_tk_norm    one wave per block: g = grad + residual (one fp32 add), the fp64 sum of g^2
//                (per-lane partial sums in index order, then a butterfly across the wave),
//                stored as the block's 64-bit key; with error feedback g is written back
//                into the residual, so the last pass reads one array instead of two;
//   k_tk_select  one workgroup per worker: radix select over the keys (up to eight digits,
//                sign and exponent first; non-negative fp64 bit patterns order as their
//                values; the surviving candidates move to LDS once they fit; it stops
//                early once every key matching the digits chosen so far is taken) finds the
//                K-th largest key T and how many keys equal to T are taken; kept = key > T,
//                plus the lowest-id keys equal to T when fewer than all of them fit; writes
//                the kept-block bitmap;
//   k_tk_apply   every element: out = g in kept blocks and 0 elsewhere; the residual of
//                kept blocks becomes 0 (the rest already holds g).
// HBM traffic with error feedback: 12 B per element in the first pass (read gradient and
// residual, write g) and 8 B in the last (read g, write out), plus 4 B per kept element.
// These streams go past the caches (non-temporal loads and stores): each array is read or
// written once per pass, and on the ResNet-50-sized workload (W = 16) each is 1.6 GB, far
// beyond the Infinity Cache (measured on MI355X: step 1.49 -> 1.41 ms against cached ones).

#include "s2r_launch.hpp"

namespace s2r {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTkNormThreads = 256;   // 4 waves, one block each
constexpr int kTkSelThreads = 1024;
constexpr int kTkApplyThreads = 256;

// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kTkNormThreads) void k_tk_norm(const float* __restrict__ grad,
                                                            float* __restrict__ residual,
                                                            uint64_t n, uint64_t ld,
                                                            uint64_t block, uint64_t nb,
                                                            uint64_t key_stride,
                                                            uint64_t* __restrict__ keys,
                                                            int vec4,
                                                            uint32_t* __restrict__ zero,
                                                            uint32_t zero_words) {
  // (group, worker) items in XCD runs of 512 groups (xcd_run_item), the grid x-fastest
  const uint64_t item =
      xcd_run_item(blockIdx.x + (uint64_t)blockIdx.y * gridDim.x, (uint64_t)gridDim.x * gridDim.y, 512);
  const uint32_t x = (uint32_t)(item % gridDim.x), k = (uint32_t)(item / gridDim.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (x == 0)  // the worker's select histograms and candidate count start at zero
    for (uint32_t i = threadIdx.x; i < zero_words; i += kTkNormThreads)
      zero[(uint64_t)k * zero_words + i] = 0u;
  const uint64_t q = (uint64_t)x * (kTkNormThreads / kWave) + wave;
  if (q >= nb) return;  // whole wave
  const uint64_t first = q * block;
  const uint64_t len = first + block <= n ? block : n - first;
  const float* gr = grad + (uint64_t)k * ld + first;
  float* rs = residual ? residual + (uint64_t)k * ld + first : nullptr;
  double acc = 0.0;
  if (vec4) {  // block % 4 == 0 and ld % 4 == 0: every float4 lies inside the block
    for (uint64_t e = 4 * (uint64_t)lane; e < len; e += 4 * kWave) {
      if (e + 4 <= len) {
        f32x4 g = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gr + e));
        if (rs) {
          g += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rs + e));
          __builtin_nontemporal_store(g, reinterpret_cast<f32x4*>(rs + e));
        }
        acc += (double)g.x * (double)g.x;
        acc += (double)g.y * (double)g.y;
        acc += (double)g.z * (double)g.z;
        acc += (double)g.w * (double)g.w;
      } else {
        for (uint64_t c = e; c < len; ++c) {
          float g = gr[c];
          if (rs) {
            g += rs[c];
            rs[c] = g;
          }
          acc += (double)g * (double)g;
        }
      }
    }
  } else {
    for (uint64_t e = lane; e < len; e += kWave) {
      float g = gr[e];
      if (rs) {
        g += rs[e];
        rs[e] = g;
      }
      acc += (double)g * (double)g;
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane == 0) keys[(uint64_t)k * key_stride + q] = (uint64_t)__double_as_longlong(acc);
}

// ---------------------------------------------------------------------------------------
// Radix select of the K largest keys of each worker.  Digits, most significant first: the 12
// bits of sign and exponent, six 8-bit digits of the mantissa, its last 4 bits.  The first
// digit splits the keys by binade (a top 8-bit digit would not: it holds the sign and the
// exponent's high bits, alike for every norm).  After each digit's histogram, the digit
// taken is the largest b whose count from the top (bins >= b) reaches the number still to
// take; the keys matching the digits taken so far are the candidates of the next digit.
//
// The first three digits are histogrammed by wide grids (k_tk_hist, one launch per digit,
// global histograms), every workgroup first replaying the earlier choices from the global
// histograms.  The first of those passes whose candidates fit in cand_cap keys also gathers
// them into a global list.  k_tk_select (one workgroup per worker) replays the three choices,
// finishes from the gathered list in LDS (or, if nothing fitted, from the keys, gathering into
// LDS as soon as the candidates fit), and in the rare case that only some keys equal to the
// K-th largest are taken writes the kept-block bitmap itself; otherwise k_tk_bitmap writes it
// from the threshold, over a wide grid.
constexpr int kTkLoads = 8;
constexpr int kTkHistWords = 4096;       // 2^12 bins of the first digit
constexpr int kTkGlobalPasses = 3;       // digits histogrammed by the wide grids
constexpr int kTkHistThreads = 256;
constexpr uint32_t kTkSliceKeys = 2048;  // keys per k_tk_hist workgroup
constexpr uint32_t kTkCandBig = 16384;   // 128 KiB of candidates where the device allows it
constexpr uint32_t kTkCandSmall = 6000;  // else 47 KiB (with the histograms under 64 KiB)
// Per-worker select scratch (uint32 words): the global histograms of the first three digits,
// then the gathered-candidate count.
constexpr uint32_t kTkScratchCount = kTkHistWords + 2 * 256;
constexpr uint32_t kTkScratchWords = kTkScratchCount + 4;
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// Digit p of a key: its lowest bit and its width.
__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 52 : (p < 7 ? 52 - 8 * p : 0); }
__device__ __forceinline__ int digit_bits(int p) { return p == 0 ? 12 : (p < 7 ? 8 : 4); }
// Offset of digit p's histogram in a worker's global histograms (p < kTkGlobalPasses).
__device__ __forceinline__ int ghist_offset(int p) { return p == 0 ? 0 : kTkHistWords + 256 * (p - 1); }

// Select state: the digits taken so far (prefix), how many keys matching them are still to
// be taken (rem) and how many match (eq); 1 <= rem <= eq.
struct TkState {
  uint64_t prefix, rem, eq;
};

// Counts each lane with `on` set into h[digit]; the lanes holding the first live lane's digit
// add together (same-address LDS atomics of one instruction serialise, and the keys' leading
// digits are mostly alike).
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t digit, bool on, int lane) {
  const uint64_t live = __ballot(on);
  if (live == 0) return;
  const int leader = __ffsll((unsigned long long)live) - 1;
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)digit, leader);
  const uint64_t same = __ballot(on && digit == d0);
  if (lane == leader) atomicAdd(&h[d0], (uint32_t)__popcll(same));
  else if (on && digit != d0) atomicAdd(&h[digit], 1u);
}

// Appends v to list (count in *n, LDS or global; room for cap) for each lane with `on` set:
// one atomic per wave.  The callers append exactly as many keys as fit; the bound is a guard.
__device__ __forceinline__ void wave_append(uint64_t* list, uint32_t* n, uint32_t cap,
                                            uint64_t v, bool on, int lane) {
  const uint64_t m = __ballot(on);
  if (m == 0) return;
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, (uint32_t)__popcll(m));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  const uint32_t at = base + bits_below_lane(m);
  if (on && at < cap) list[at] = v;
}

// Chooses digit p from its histogram h[0 .. 2^bits) (LDS) and returns the new state to every
// thread of the block.  Thread t holds a run of bins; with suf(t) the count of the bins of
// threads >= t, the one thread with suf(t) >= rem > suf(t + 1) holds the digit.  wsum: one
// slot per wave; out: LDS.  Ends with a barrier.
template <int THREADS>
__device__ TkState choose_digit(const uint32_t* h, int p, TkState st, uint64_t* wsum,
                                TkState* out) {
  constexpr int PER = kTkHistWords / THREADS;
  constexpr int NW = THREADS / kWave;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbins = 1 << digit_bits(p);
  uint64_t c[PER], tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = PER * tid + j < nbins ? h[PER * tid + j] : 0u;
    tot += c[j];
  }
  uint64_t suf = tot;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint64_t t = __shfl_down(suf, off, kWave);
    if (lane + off < kWave) suf += t;
  }
  if (lane == 0) wsum[wave] = suf;
  __syncthreads();
  for (int v = wave + 1; v < NW; ++v) suf += wsum[v];
  uint64_t above = suf - tot;  // suf(t + 1)
  if (suf >= st.rem && above < st.rem) {
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      if (above + c[j] >= st.rem) {
        TkState r;
        r.rem = st.rem - above;
        r.prefix = st.prefix | ((uint64_t)(PER * tid + j) << digit_shift(p));
        r.eq = c[j];
        *out = r;
        break;
      }
      above += c[j];
    }
  }
  __syncthreads();
  const TkState r = *out;
  __syncthreads();  // out and wsum may be rewritten next
  return r;
}

// Replays the choices of digits 0 .. upto-1 from the worker's global histograms; eqs[q]
// receives the candidate count after digit q.  True when a choice took every candidate
// (rem == eq): the select is then complete, with the keys >= prefix kept.
template <int THREADS>
__device__ bool replay_digits(const uint32_t* gh, int upto, TkState& st, uint64_t* eqs,
                              uint32_t* hist, uint64_t* wsum, TkState* out) {
  for (int q = 0; q < upto; ++q) {
    const int nbins = 1 << digit_bits(q);
    for (int i = threadIdx.x; i < nbins; i += THREADS) hist[i] = gh[ghist_offset(q) + i];
    __syncthreads();
    st = choose_digit<THREADS>(hist, q, st, wsum, out);
    eqs[q] = st.eq;
    if (st.rem == st.eq) return true;
  }
  return false;
}

// The pass whose gathered candidates the select reads: the first of passes 1 .. 2 whose
// candidate count (after the previous digit) fits, else 0.
__device__ __forceinline__ int gather_pass(const uint64_t* eqs, uint32_t cap) {
  if (eqs[0] <= cap) return 1;
  if (eqs[1] <= cap) return 2;
  return 0;
}

// k_tk_hist: grid (ceil(nb / kTkSliceKeys), W), 256 threads; histograms digit p over the
// workgroup's slice of the keys matching the digits already taken, adds it into the global
// histogram, and gathers those keys into the global list when this pass is the gather pass.
__global__ __launch_bounds__(kTkHistThreads) void k_tk_hist(
    const uint64_t* __restrict__ keys, uint64_t nb, uint64_t stride, uint64_t K, int p,
    uint32_t* __restrict__ ghist, uint32_t ghist_words, uint64_t* __restrict__ gcand,
    uint32_t cand_cap) {
  constexpr int NW = kTkHistThreads / kWave;
  __shared__ uint32_t hist[kTkHistWords];
  __shared__ uint64_t wsum[NW];
  __shared__ TkState s_out;
  const uint32_t k = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  if (K == 0 || K >= nb) return;  // nothing to select
  // the slice's keys are loaded first: their latency overlaps the replay
  const uint64_t* key = keys + (uint64_t)k * stride;  // stride even: 16-byte aligned rows
  const u64x2* key2 = reinterpret_cast<const u64x2*>(key);
  const uint64_t lo = (uint64_t)blockIdx.x * kTkSliceKeys;  // even
  const uint64_t hi = lo + kTkSliceKeys < nb ? lo + kTkSliceKeys : nb;
  constexpr int U = kTkSliceKeys / 2 / kTkHistThreads;  // 16-byte loads per thread
  u64x2 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t pi = lo / 2 + (uint64_t)u * kTkHistThreads + tid;
    x[u] = key2[2 * pi < hi ? pi : (hi - 1) / 2];  // clamped: the loads issue together
  }
  uint32_t* gh = ghist + (uint64_t)k * ghist_words;
  TkState st = {0ull, K, nb};
  uint64_t eqs[kTkGlobalPasses] = {nb, nb, nb};
  if (replay_digits<kTkHistThreads>(gh, p, st, eqs, hist, wsum, &s_out)) return;
  const bool gather = p >= 1 && gather_pass(eqs, cand_cap) == p;
  for (int i = tid; i < kTkHistWords; i += kTkHistThreads) hist[i] = 0u;
  __syncthreads();
  const int shift = digit_shift(p), bits = digit_bits(p);
  const uint32_t dmask = (1u << bits) - 1u;
  const uint64_t hi_mask = shift + bits >= 64 ? 0ull : ~0ull << (shift + bits);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t pi = lo / 2 + (uint64_t)u * kTkHistThreads + tid;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint64_t xv = e ? x[u].y : x[u].x;
      const bool on = 2 * pi + e < hi && ((xv ^ st.prefix) & hi_mask) == 0;
      hist_add(hist, (uint32_t)(xv >> shift) & dmask, on, lane);
      if (gather)
        wave_append(gcand + (uint64_t)k * cand_cap, gh + kTkScratchCount, cand_cap, xv, on, lane);
    }
  }
  __syncthreads();
  for (int i = tid; i < (1 << bits); i += kTkHistThreads)
    if (hist[i]) atomicAdd(&gh[ghist_offset(p) + i], hist[i]);
}

// Per-worker outcome of the select for k_tk_bitmap: keys >= thr are kept (mode 0), all keys
// (1), none (2), or the bitmap is already written (3).
struct TkOutcome {
  uint64_t thr;
  uint64_t mode;
};

// k_tk_select: grid W, 1024 threads.  Per-wave 256-bin histograms in LDS for the digits it
// histograms itself, summed before each choice.  Passes over global keys read two keys per
// 16-byte load, kTkLoads loads in flight per thread.
__global__ __launch_bounds__(kTkSelThreads) void k_tk_select(const uint64_t* __restrict__ keys,
                                                             uint64_t nb, uint64_t stride,
                                                             uint64_t K,
                                                             uint64_t* __restrict__ sel,
                                                             uint64_t sel_words,
                                                             uint32_t cand_cap,
                                                             const uint32_t* __restrict__ ghist,
                                                             uint32_t ghist_words,
                                                             const uint64_t* __restrict__ gcand,
                                                             TkOutcome* __restrict__ outcome) {
  constexpr int NW = kTkSelThreads / kWave;
  static_assert(kTkHistWords == NW * 256, "the per-wave histograms share the first digit's");
  __shared__ uint32_t hist[kTkHistWords];
  extern __shared__ uint64_t cand[];  // cand_cap keys
  __shared__ uint32_t s_ncand;
  __shared__ uint64_t wsum[NW];
  __shared__ TkState s_out;
  const uint32_t k = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t* key = keys + (uint64_t)k * stride;  // stride even: 16-byte aligned rows
  const u64x2* key2 = reinterpret_cast<const u64x2*>(key);
  const uint64_t npairs = (nb + 1) / 2;
  uint64_t* out = sel + (uint64_t)k * sel_words;

  TkState st = {0ull, K, nb};
  const bool all = K >= nb, none = K == 0;
  if (!all && !none) {
    uint64_t eqs[kTkGlobalPasses] = {nb, nb, nb};
    if (!replay_digits<kTkSelThreads>(ghist + (uint64_t)k * ghist_words, kTkGlobalPasses, st,
                                      eqs, hist, wsum, &s_out)) {
      bool in_lds = false;
      uint32_t ncand = 0;
      if (tid == 0) s_ncand = 0;
      const int gp = gather_pass(eqs, cand_cap);
      if (gp > 0) {  // the gathered candidates: every key matching the digits before pass gp
        ncand = ghist[(uint64_t)k * ghist_words + kTkScratchCount];  // == eqs[gp - 1] <= cap
        if (ncand > cand_cap) ncand = cand_cap;
        const uint64_t* gc = gcand + (uint64_t)k * cand_cap;
        for (uint32_t i = tid; i < ncand; i += kTkSelThreads) cand[i] = gc[i];
        in_lds = true;
      }
      for (int p = kTkGlobalPasses; p < 8; ++p) {
        const int shift = digit_shift(p), bits = digit_bits(p);
        const uint32_t dmask = (1u << bits) - 1u;
        for (int i = tid; i < kTkHistWords; i += kTkSelThreads) hist[i] = 0u;
        __syncthreads();
        // keys whose digits above this one equal the prefix chosen so far
        const uint64_t hi_mask = shift + bits >= 64 ? 0ull : ~0ull << (shift + bits);
        uint32_t* h = hist + wave * 256;
        if (in_lds) {
          for (uint32_t i0 = 0; i0 < ncand; i0 += kTkSelThreads) {
            const uint32_t i = i0 + tid;
            const uint64_t x = i < ncand ? cand[i] : 0ull;
            hist_add(h, (uint32_t)(x >> shift) & dmask,
                     i < ncand && ((x ^ st.prefix) & hi_mask) == 0, lane);
          }
        } else {
          const bool gather = st.eq <= (uint64_t)cand_cap;
          for (uint64_t p0 = 0; p0 < npairs; p0 += (uint64_t)kTkSelThreads * kTkLoads) {
            u64x2 x[kTkLoads];
#pragma unroll
            for (int u = 0; u < kTkLoads; ++u) {
              const uint64_t pi = p0 + (uint64_t)u * kTkSelThreads + tid;
              if (pi < npairs) x[u] = key2[pi];
            }
#pragma unroll
            for (int u = 0; u < kTkLoads; ++u) {
              const uint64_t pi = p0 + (uint64_t)u * kTkSelThreads + tid;
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const uint64_t xv = e ? x[u].y : x[u].x;
                const bool on = 2 * pi + e < nb && ((xv ^ st.prefix) & hi_mask) == 0;
                hist_add(h, (uint32_t)(xv >> shift) & dmask, on, lane);
                if (gather) wave_append(cand, &s_ncand, cand_cap, xv, on, lane);
              }
            }
          }
          if (gather) in_lds = true;  // uniform: st is the same in every thread
        }
        __syncthreads();
        if (gp == 0) ncand = s_ncand < cand_cap ? s_ncand : cand_cap;  // gathered here, if any
        if (tid < 256) {
          uint32_t c = 0;
          for (int v = 0; v < NW; ++v) c += hist[v * 256 + tid];
          hist[tid] = c;
        }
        __syncthreads();
        st = choose_digit<kTkSelThreads>(hist, p, st, wsum, &s_out);
        // every key matching the prefix is taken: the keys kept are those >= the prefix
        if (st.rem == st.eq) break;
      }
    }
  }
  const uint64_t T = st.prefix, take_eq = st.rem, n_eq = st.eq;  // 1 <= take_eq <= n_eq

  if (all || none || take_eq == n_eq) {
    if (tid == 0) {
      TkOutcome o;
      o.thr = T;
      o.mode = all ? 1u : (none ? 2u : 0u);
      outcome[k] = o;
    }
    return;
  }
  if (tid == 0) {
    TkOutcome o;
    o.thr = T;
    o.mode = 3u;
    outcome[k] = o;
  }
  // only some keys equal to T fit: they go to the lowest block ids, so the tie rank is a
  // prefix count in id order, chunk by chunk
  uint64_t carry = 0;
  for (uint64_t base = 0; base < nb; base += kTkSelThreads) {
    const uint64_t i = base + tid;
    const uint64_t x = i < nb ? key[i] : 0ull;
    const bool tie = i < nb && x == T;
    const uint64_t tb = __ballot(tie);
    if (lane == 0) wsum[wave] = (uint64_t)__popcll(tb);
    __syncthreads();
    uint64_t before = carry, total = 0;
    for (int v = 0; v < NW; ++v) {
      if (v < wave) before += wsum[v];
      total += wsum[v];
    }
    const uint64_t rank = before + bits_below_lane(tb);
    const bool kept = i < nb && (x > T || (tie && rank < take_eq));
    const uint64_t word = __ballot(kept);
    if (lane == 0 && i < nb) out[i / 64] = word;
    carry += total;
    __syncthreads();  // wsum is rewritten next chunk
  }
}

// k_tk_bitmap: grid (ceil(sel_words / 4), W), 256 threads: one wave per kept-block word from
// the select's outcome (nothing to do where the select wrote the bitmap itself).
__global__ __launch_bounds__(256) void k_tk_bitmap(const uint64_t* __restrict__ keys,
                                                   uint64_t nb, uint64_t stride,
                                                   const TkOutcome* __restrict__ outcome,
                                                   uint64_t* __restrict__ sel,
                                                   uint64_t sel_words) {
  const uint32_t k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t q = (uint64_t)blockIdx.x * 4 + wave;
  const TkOutcome o = outcome[k];
  if (q >= sel_words || o.mode == 3u) return;  // whole wave
  const uint64_t i = q * 64 + lane;
  const uint64_t x = i < nb && o.mode == 0u ? keys[(uint64_t)k * stride + i] : 0ull;
  const bool kept = i < nb && (o.mode == 1u || (o.mode == 0u && x >= o.thr));
  const uint64_t word = __ballot(kept);
  if (lane == 0) sel[(uint64_t)k * sel_words + q] = word;
}

// ---------------------------------------------------------------------------------------
// k_tk_apply: grid (ceil(n / (4 * 256 * kTkApplyIters)), W).  Each thread takes
// kTkApplyIters float4 groups, 1024 elements apart.  A group's first element gives its block
// by a multiply-high division (below); the others follow by counting.  Away from the row's
// end every load of the thread (data and kept-block words) is issued before any is used.
constexpr int kTkApplyIters = 4;

// Unsigned division by a divisor fixed for the launch, exact for every 32-bit dividend:
// the round-up multiplier method of Granlund & Montgomery, "Division by invariant integers
// using multiplication" (1994), Section 4.  With l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1 and t = mulhi(m, x): x / d = (t + ((x - t) >> s1)) >> s2,
// s1 = min(l, 1), s2 = max(l - 1, 0).
struct DivU32 {
  uint32_t d, m, s1, s2;
};
__device__ __forceinline__ uint32_t div_u32(const DivU32& v, uint32_t x) {
  const uint32_t t = __umulhi(v.m, x);
  return (t + ((x - t) >> v.s1)) >> v.s2;
}
static DivU32 make_div_u32(uint32_t d) {  // d >= 1
  DivU32 v;
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;
  v.d = d;
  v.m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
  v.s1 = l < 1 ? l : 1;
  v.s2 = l > 0 ? l - 1 : 0;
  return v;
}

__global__ __launch_bounds__(kTkApplyThreads) void k_tk_apply(const float* __restrict__ grad,
                                                              float* __restrict__ residual,
                                                              uint64_t n, uint64_t ld, DivU32 dv,
                                                              const uint64_t* __restrict__ sel,
                                                              uint64_t sel_words,
                                                              float* __restrict__ out) {
  // (group, worker) items in XCD runs of 128 groups of 16 KiB (xcd_run_item)
  const uint64_t item =
      xcd_run_item(blockIdx.x + (uint64_t)blockIdx.y * gridDim.x, (uint64_t)gridDim.x * gridDim.y, 128);
  const uint32_t x = (uint32_t)(item % gridDim.x), k = (uint32_t)(item / gridDim.x);
  const uint64_t* sk = sel + (uint64_t)k * sel_words;
  // with error feedback the residual holds g (k_tk_norm), else g is the gradient itself
  const float* src = residual ? residual + (uint64_t)k * ld : grad + (uint64_t)k * ld;
  float* rs = residual ? residual + (uint64_t)k * ld : nullptr;
  float* o = out + (uint64_t)k * ld;
  const uint32_t d = dv.d;  // the block size, or n when the block holds the whole row
  constexpr uint64_t kStep = 4ull * kTkApplyThreads;
  const uint64_t e0 = 4 * ((uint64_t)x * kTkApplyThreads * kTkApplyIters + threadIdx.x);
  if (e0 + kStep * (kTkApplyIters - 1) + 4 <= n) {
    // every group whole and inside the row (ld % 4 == 0: aligned float4 groups)
    f32x4 g[kTkApplyIters];
    uint64_t w0[kTkApplyIters], w1[kTkApplyIters];
    uint32_t q[kTkApplyIters], r[kTkApplyIters];
#pragma unroll
    for (int it = 0; it < kTkApplyIters; ++it) {
      const uint32_t e = (uint32_t)(e0 + kStep * it);
      q[it] = div_u32(dv, e);
      r[it] = e - q[it] * d;
      const uint32_t q3 = div_u32(dv, e + 3);  // block of the group's last element
      w0[it] = sk[q[it] >> 6];
      w1[it] = sk[q3 >> 6];  // the group's blocks span at most these two words
      g[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + e));
    }
#pragma unroll
    for (int it = 0; it < kTkApplyIters; ++it) {
      const uint64_t e = e0 + kStep * it;
      bool kept[4];
      uint32_t qc = q[it], rc = r[it];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t w = (qc >> 6) == (q[it] >> 6) ? w0[it] : w1[it];
        kept[c] = (w >> (qc & 63)) & 1ull;
        if (++rc == d) {
          rc = 0;
          ++qc;
        }
      }
      f32x4 v;
      v.x = kept[0] ? g[it].x : 0.f;
      v.y = kept[1] ? g[it].y : 0.f;
      v.z = kept[2] ? g[it].z : 0.f;
      v.w = kept[3] ? g[it].w : 0.f;
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o + e));
      if (rs && (kept[0] | kept[1] | kept[2] | kept[3])) {
        f32x4 z;
        z.x = kept[0] ? 0.f : g[it].x;
        z.y = kept[1] ? 0.f : g[it].y;
        z.z = kept[2] ? 0.f : g[it].z;
        z.w = kept[3] ? 0.f : g[it].w;
        *reinterpret_cast<f32x4*>(rs + e) = z;
      }
    }
    return;
  }
  // the row's end: group by group, element by element past n
  for (int it = 0; it < kTkApplyIters; ++it) {
    const uint64_t e = e0 + kStep * it;
    if (e >= n) break;
    uint32_t qc = div_u32(dv, (uint32_t)e);
    uint32_t rc = (uint32_t)e - qc * d;
    for (int c = 0; c < 4 && e + c < n; ++c) {
      const bool kept = (sk[qc >> 6] >> (qc & 63)) & 1ull;
      const float gv = src[e + c];
      o[e + c] = kept ? gv : 0.f;
      if (rs && kept) rs[e + c] = 0.f;
      if (++rc == d) {
        rc = 0;
        ++qc;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// host side

// The select kernel stages up to kTkCandBig candidates in dynamic LDS; where the device
// refuses that much, it stages fewer.  Asked on every call (the library caches nothing).
static uint32_t select_cand_cap() {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_tk_select),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)(kTkCandBig * sizeof(uint64_t))) != hipSuccess) {
    (void)hipGetLastError();
    return kTkCandSmall;
  }
  return kTkCandBig;
}

TopkLayout topk_layout(uint32_t W, uint64_t n, uint64_t block) {
  TopkLayout L;
  L.nb = block ? (n + block - 1) / block : 0;
  L.key_stride = (L.nb + 1) & ~(uint64_t)1;
  L.sel_words = (L.nb + 63) / 64;
  size_t off = 0;
  L.off_keys = off;
  off += ((size_t)W * L.key_stride * 8 + 255) & ~(size_t)255;
  L.off_sel = off;
  off += ((size_t)W * L.sel_words * 8 + 255) & ~(size_t)255;
  L.scratch_words = kTkScratchWords;
  L.off_scratch = off;
  off += ((size_t)W * L.scratch_words * 4 + 255) & ~(size_t)255;
  L.off_gcand = off;
  off += (size_t)W * kTkCandBig * 8;
  L.off_outcome = off;
  off += ((size_t)W * sizeof(TkOutcome) + 255) & ~(size_t)255;
  L.total = off;
  return L;
}

hipError_t launch_topk(uint32_t W, const float* grad, float* residual, uint64_t n, uint64_t ld,
                       uint64_t block, uint64_t K, float* out, uint64_t* selected,
                       void* workspace, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const TopkLayout L = topk_layout(W, n, block);
  char* ws = static_cast<char*>(workspace);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.off_keys);
  uint64_t* sel = selected ? selected : reinterpret_cast<uint64_t*>(ws + L.off_sel);
  uint32_t* scratch = reinterpret_cast<uint32_t*>(ws + L.off_scratch);  // [W][scratch_words]
  uint64_t* gcand = reinterpret_cast<uint64_t*>(ws + L.off_gcand);
  TkOutcome* outcome = reinterpret_cast<TkOutcome*>(ws + L.off_outcome);
  const int vec4 = (block % 4 == 0) && (ld % 4 == 0);
  const uint64_t ngroups = (L.nb + kTkNormThreads / kWave - 1) / (kTkNormThreads / kWave);
  trace_mark(s, "k_tk_norm");
  hipLaunchKernelGGL(k_tk_norm, dim3((uint32_t)ngroups, W), dim3(kTkNormThreads), 0, s, grad,
                     residual, n, ld, block, L.nb, L.key_stride, keys, vec4, scratch,
                     L.scratch_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t cap = select_cand_cap();
  if (K > 0 && K < L.nb) {  // else the select has nothing to histogram
    const uint32_t slices = (uint32_t)((L.nb + kTkSliceKeys - 1) / kTkSliceKeys);
    for (int p = 0; p < kTkGlobalPasses; ++p) {
      trace_mark(s, "k_tk_hist");
      hipLaunchKernelGGL(k_tk_hist, dim3(slices, W), dim3(kTkHistThreads), 0, s, keys, L.nb,
                         L.key_stride, K, p, scratch, L.scratch_words, gcand, cap);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  trace_mark(s, "k_tk_select");
  hipLaunchKernelGGL(k_tk_select, dim3(W), dim3(kTkSelThreads), cap * sizeof(uint64_t), s, keys,
                     L.nb, L.key_stride, K, sel, L.sel_words, cap, scratch, L.scratch_words,
                     gcand, outcome);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_mark(s, "k_tk_bitmap");
  hipLaunchKernelGGL(k_tk_bitmap, dim3((uint32_t)((L.sel_words + 3) / 4), W), dim3(256), 0, s,
                     keys, L.nb, L.key_stride, outcome, sel, L.sel_words);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t per = 4ull * kTkApplyThreads * kTkApplyIters;
  // blocks beyond n hold the whole row: dividing by n gives the same block ids (all 0)
  const DivU32 dv = make_div_u32((uint32_t)(block < n ? block : n));
  trace_mark(s, "k_tk_apply");
  hipLaunchKernelGGL(k_tk_apply, dim3((uint32_t)((n + per - 1) / per), W), dim3(kTkApplyThreads), 0,
                     s, grad, residual, n, ld, dv, sel, L.sel_words, out);
  return hipGetLastError();
}

}  // namespace s2r
