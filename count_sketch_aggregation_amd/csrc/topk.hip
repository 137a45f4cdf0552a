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
//   k_tk_select  one workgroup per worker: radix select over the keys (eight 8-bit digits,
//                most significant first; non-negative fp64 bit patterns order as their
//                values; the surviving candidates move to LDS once they fit) finds the K-th
//                largest key T and how many keys equal to T are taken; kept = key > T, plus
//                the lowest-id keys equal to T when fewer than all of them fit; writes the
//                kept-block bitmap;
//   k_tk_apply   every element: out = g in kept blocks and 0 elsewhere; the residual of
//                kept blocks becomes 0 (the rest already holds g).
// HBM traffic with error feedback: 12 B per element in the first pass (read gradient and
// residual, write g) and 8 B in the last (read g, write out), plus 4 B per kept element.
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
                                                            uint64_t* __restrict__ keys,
                                                            int vec4) {
  const uint32_t k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t q = (uint64_t)blockIdx.x * (kTkNormThreads / kWave) + wave;
  if (q >= nb) return;  // whole wave
  const uint64_t first = q * block;
  const uint64_t len = first + block <= n ? block : n - first;
  const float* gr = grad + (uint64_t)k * ld + first;
  float* rs = residual ? residual + (uint64_t)k * ld + first : nullptr;
  double acc = 0.0;
  if (vec4) {  // block % 4 == 0 and ld % 4 == 0: every float4 lies inside the block
    for (uint64_t e = 4 * (uint64_t)lane; e < len; e += 4 * kWave) {
      if (e + 4 <= len) {
        f32x4 g = *reinterpret_cast<const f32x4*>(gr + e);
        if (rs) {
          g += *reinterpret_cast<const f32x4*>(rs + e);
          *reinterpret_cast<f32x4*>(rs + e) = g;
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
  if (lane == 0) keys[(uint64_t)k * nb + q] = (uint64_t)__double_as_longlong(acc);
}

// ---------------------------------------------------------------------------------------
// k_tk_select: grid W, 1024 threads.  Per-wave 256-bin histograms in LDS (64 lanes hitting
// one bin serialise within a wave only), summed before each digit is chosen.  Passes over
// global keys keep kTkLoads loads in flight per thread.  As soon as the keys that match the
// digits chosen so far fit in LDS (kTkCand), the next pass also gathers them there, and the
// remaining passes read only those.
constexpr int kTkCand = 6000;  // candidate keys staged in LDS (47 KiB; with the histograms under 64 KiB)
constexpr int kTkLoads = 8;
__global__ __launch_bounds__(kTkSelThreads) void k_tk_select(const uint64_t* __restrict__ keys,
                                                             uint64_t nb, uint64_t K,
                                                             uint64_t* __restrict__ sel,
                                                             uint64_t sel_words) {
  constexpr int NW = kTkSelThreads / kWave;
  __shared__ uint32_t hist[NW][256];
  __shared__ uint64_t cand[kTkCand];
  __shared__ uint64_t s_prefix;
  __shared__ uint64_t s_rem, s_eq;
  __shared__ uint32_t s_ncand;
  __shared__ uint32_t wsum[NW];
  const uint32_t k = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t* key = keys + (uint64_t)k * nb;
  uint64_t* out = sel + (uint64_t)k * sel_words;

  uint64_t T = 0, take_eq = 0, n_eq = 0;
  const bool all = K >= nb, none = K == 0;
  if (!all && !none) {
    if (tid == 0) {
      s_prefix = 0;
      s_rem = K;
      s_eq = nb;  // keys matching the (empty) prefix
      s_ncand = 0;
    }
    bool in_lds = false;
    uint32_t ncand = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int b = tid; b < NW * 256; b += kTkSelThreads) (&hist[0][0])[b] = 0u;
      __syncthreads();
      const uint64_t prefix = s_prefix;
      // keys whose digits above `shift` equal the prefix chosen so far
      const uint64_t hi_mask = shift == 56 ? 0ull : ~0ull << (shift + 8);
      if (in_lds) {
        for (uint32_t i = tid; i < ncand; i += kTkSelThreads) {
          const uint64_t x = cand[i];
          if (((x ^ prefix) & hi_mask) == 0) atomicAdd(&hist[wave][(x >> shift) & 255u], 1u);
        }
      } else {
        const bool gather = s_eq <= (uint64_t)kTkCand;
        for (uint64_t i0 = tid; i0 < nb; i0 += (uint64_t)kTkSelThreads * kTkLoads) {
          uint64_t x[kTkLoads];
#pragma unroll
          for (int u = 0; u < kTkLoads; ++u) {
            const uint64_t i = i0 + (uint64_t)u * kTkSelThreads;
            x[u] = i < nb ? key[i] : 0ull;
          }
#pragma unroll
          for (int u = 0; u < kTkLoads; ++u) {
            const uint64_t i = i0 + (uint64_t)u * kTkSelThreads;
            if (i < nb && ((x[u] ^ prefix) & hi_mask) == 0) {
              atomicAdd(&hist[wave][(x[u] >> shift) & 255u], 1u);
              if (gather) cand[atomicAdd(&s_ncand, 1u)] = x[u];
            }
          }
        }
        if (gather) in_lds = true;  // uniform: s_eq was read by every thread
      }
      __syncthreads();
      ncand = s_ncand;
      if (tid < 256) {
        uint32_t c = 0;
        for (int v = 0; v < NW; ++v) c += hist[v][tid];
        hist[0][tid] = c;
      }
      __syncthreads();
      if (tid == 0) {
        // from the largest digit down: the digit where the running count reaches s_rem
        uint64_t rem = s_rem, above = 0;
        int b = 255;
        for (; b > 0; --b) {
          if (above + hist[0][b] >= rem) break;
          above += hist[0][b];
        }
        s_rem = rem - above;
        s_prefix = prefix | ((uint64_t)b << shift);
        s_eq = hist[0][b];
      }
      __syncthreads();
    }
    T = s_prefix;
    take_eq = s_rem;  // 1 <= take_eq <= n_eq
    n_eq = s_eq;
  }

  // kept-block bitmap, 64 keys per wave step
  if (all || none || take_eq == n_eq) {
    constexpr int U = 4;
    for (uint64_t b0 = (uint64_t)wave * kWave; b0 < nb; b0 += (uint64_t)kTkSelThreads * U) {
      uint64_t x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t i = b0 + (uint64_t)u * kTkSelThreads + lane;
        x[u] = (i < nb && !all && !none) ? key[i] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t base = b0 + (uint64_t)u * kTkSelThreads;
        const bool kept = base + lane < nb && (all || (!none && x[u] >= T));
        const uint64_t word = __ballot(kept);
        if (lane == 0 && base < nb) out[base / 64] = word;
      }
    }
  } else {
    // only some keys equal to T fit: they go to the lowest block ids, so the tie rank is a
    // prefix count in id order, chunk by chunk
    uint64_t carry = 0;
    for (uint64_t base = 0; base < nb; base += kTkSelThreads) {
      const uint64_t i = base + tid;
      const uint64_t x = i < nb ? key[i] : 0ull;
      const bool tie = i < nb && x == T;
      const uint64_t tb = __ballot(tie);
      if (lane == 0) wsum[wave] = (uint32_t)__popcll(tb);
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
}

// ---------------------------------------------------------------------------------------
// k_tk_apply: grid (ceil(n / (4 * 256 * kTkApplyIters)), W).  Each thread takes float4
// groups; the group's first element fixes its block by one division, the others follow.
constexpr int kTkApplyIters = 4;
__global__ __launch_bounds__(kTkApplyThreads) void k_tk_apply(const float* __restrict__ grad,
                                                              float* __restrict__ residual,
                                                              uint64_t n, uint64_t ld,
                                                              uint64_t block,
                                                              const uint64_t* __restrict__ sel,
                                                              uint64_t sel_words,
                                                              float* __restrict__ out) {
  const uint32_t k = blockIdx.y;
  const uint64_t* sk = sel + (uint64_t)k * sel_words;
  // with error feedback the residual holds g (k_tk_norm), else g is the gradient itself
  const float* src = residual ? residual + (uint64_t)k * ld : grad + (uint64_t)k * ld;
  float* rs = residual ? residual + (uint64_t)k * ld : nullptr;
  float* o = out + (uint64_t)k * ld;
#pragma unroll
  for (int it = 0; it < kTkApplyIters; ++it) {
    const uint64_t e = 4 * ((uint64_t)blockIdx.x * kTkApplyThreads * kTkApplyIters +
                            (uint64_t)it * kTkApplyThreads + threadIdx.x);
    if (e >= n) break;
    uint64_t q = e / block;
    uint64_t r = e - q * block;
    bool kept[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kept[c] = e + c < n && ((sk[q >> 6] >> (q & 63)) & 1ull);
      if (++r == block) {
        r = 0;
        ++q;
      }
    }
    if (e + 4 <= n) {  // ld % 4 == 0 and e % 4 == 0: the group is aligned and inside the row
      const f32x4 g = *reinterpret_cast<const f32x4*>(src + e);
      f32x4 v;
      v.x = kept[0] ? g.x : 0.f;
      v.y = kept[1] ? g.y : 0.f;
      v.z = kept[2] ? g.z : 0.f;
      v.w = kept[3] ? g.w : 0.f;
      *reinterpret_cast<f32x4*>(o + e) = v;
      if (rs && (kept[0] | kept[1] | kept[2] | kept[3])) {
        f32x4 z;
        z.x = kept[0] ? 0.f : g.x;
        z.y = kept[1] ? 0.f : g.y;
        z.z = kept[2] ? 0.f : g.z;
        z.w = kept[3] ? 0.f : g.w;
        *reinterpret_cast<f32x4*>(rs + e) = z;
      }
    } else {
      for (int c = 0; c < 4 && e + c < n; ++c) {
        const float g = src[e + c];
        o[e + c] = kept[c] ? g : 0.f;
        if (rs && kept[c]) rs[e + c] = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// host side

TopkLayout topk_layout(uint32_t W, uint64_t n, uint64_t block) {
  TopkLayout L;
  L.nb = block ? (n + block - 1) / block : 0;
  L.sel_words = (L.nb + 63) / 64;
  size_t off = 0;
  L.off_keys = off;
  off += ((size_t)W * L.nb * 8 + 255) & ~(size_t)255;
  L.off_sel = off;
  off += ((size_t)W * L.sel_words * 8 + 255) & ~(size_t)255;
  L.total = off > 0 ? off : 256;
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
  const int vec4 = (block % 4 == 0) && (ld % 4 == 0);
  const uint64_t ngroups = (L.nb + kTkNormThreads / kWave - 1) / (kTkNormThreads / kWave);
  hipLaunchKernelGGL(k_tk_norm, dim3((uint32_t)ngroups, W), dim3(kTkNormThreads), 0, s, grad,
                     residual, n, ld, block, L.nb, keys, vec4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tk_select, dim3(W), dim3(kTkSelThreads), 0, s, keys, L.nb, K, sel,
                     L.sel_words);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t per = 4ull * kTkApplyThreads * kTkApplyIters;
  hipLaunchKernelGGL(k_tk_apply, dim3((uint32_t)((n + per - 1) / per), W), dim3(kTkApplyThreads), 0,
                     s, grad, residual, n, ld, block, sel, L.sel_words, out);
  return hipGetLastError();
}

}  // namespace s2r
