// s2r_device.hpp -- device helpers shared by the gfx950 kernels of libs2r.
//
// Hash: multiply-add-shift (Dietzfelbinger 1996) on the 32-bit element index with 64-bit
// constants, as the public header defines: the top b bits of (a*x + c) mod 2^64.  For
// b <= 32 those bits lie in the high word, which costs one v_mad_u64_u32 (low word of a
// times x plus c, a 64-bit result that wraps mod 2^64) and one 32-bit multiply-add for
// the high word of a -- no 64x64 product is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "s2r.h"

namespace s2r {

constexpr int kWave = 64;
constexpr uint32_t kXcds = 8;  // accelerator complex dies of an MI355X

// Kernel-argument copy of the hash constants.  Shifts are precomputed on the host so
// kernels need no branches on K or L: top b bits of a 32-bit word = (uint64)hi >> (32-b),
// which is 0 for b = 0.
struct HashArgs {
  uint32_t d;
  uint32_t shift_part;  // 32 - (L - K)
  uint32_t shift_row;   // 32 - K
  uint32_t K;
  uint32_t lb;          // log2 of the bitmap block size
  uint64_t pA, pB;
  uint64_t hA[S2R_MAX_ROWS], hB[S2R_MAX_ROWS];
  uint64_t sA[S2R_MAX_ROWS], sB[S2R_MAX_ROWS];
};

// High 32 bits of (a*x + c) mod 2^64.
__device__ __forceinline__ uint32_t mas_hi32(uint64_t a, uint64_t c, uint32_t x) {
  uint64_t t = (uint64_t)(uint32_t)a * (uint64_t)x + c;
  return (uint32_t)(t >> 32) + (uint32_t)(a >> 32) * x;
}

__device__ __forceinline__ uint32_t top_bits(uint32_t hi, uint32_t shift) {
  return (uint32_t)((uint64_t)hi >> shift);
}

// P(i): the partition of index i (shared by all rows).
__device__ __forceinline__ uint32_t partition_of(const HashArgs& h, uint32_t i) {
  return top_bits(mas_hi32(h.pA, h.pB, i), h.shift_part);
}

// Q_j(i): bucket of index i within its partition, row j.
__device__ __forceinline__ uint32_t row_bucket(const HashArgs& h, int j, uint32_t i) {
  return top_bits(mas_hi32(h.hA[j], h.hB[j], i), h.shift_row);
}

// h_j(i) = P(i) * 2^K + Q_j(i)
__device__ __forceinline__ uint32_t bucket_of(const HashArgs& h, uint32_t part, int j,
                                              uint32_t i) {
  return (part << h.K) | row_bucket(h, j, i);
}

// 0x80000000 when s_j(i) = -1, else 0: xor-ing it into an fp32 pattern multiplies by s_j(i)
// exactly.
__device__ __forceinline__ uint32_t sign_mask(const HashArgs& h, int j, uint32_t i) {
  return mas_hi32(h.sA[j], h.sB[j], i) & 0x80000000u;
}

__device__ __forceinline__ float apply_sign(float v, uint32_t mask) {
  return __uint_as_float(__float_as_uint(v) ^ mask);
}

// Median of D values (D <= 16), exact selection for odd D; even D gives the mean of the
// two middle values rounded once (halving is exact away from the subnormal range).
template <int D>
__device__ __forceinline__ float median_of(float* v) {
  if constexpr (D == 1) {
    return v[0];
  } else if constexpr (D == 2) {
    return 0.5f * v[0] + 0.5f * v[1];
  } else if constexpr (D == 3) {
    return __builtin_amdgcn_fmed3f(v[0], v[1], v[2]);
  } else if constexpr (D == 5) {
    // the median of five is the median of e and the two inner values of the sorted pairs
    float lo = fmaxf(fminf(v[0], v[1]), fminf(v[2], v[3]));
    float hi = fminf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    return __builtin_amdgcn_fmed3f(v[4], lo, hi);
  } else {
    // odd-even transposition sort: D rounds of compare-exchange sort D values
#pragma unroll
    for (int r = 0; r < D; ++r) {
#pragma unroll
      for (int a = (r & 1); a + 1 < D; a += 2) {
        float x = v[a], y = v[a + 1];
        v[a] = fminf(x, y);
        v[a + 1] = fmaxf(x, y);
      }
    }
    if constexpr (D % 2) return v[(D - 1) / 2];
    else return 0.5f * v[D / 2 - 1] + 0.5f * v[D / 2];
  }
}

// Wave-wide inclusive prefix sum (64 lanes).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Number of set bits of w below this lane's position (v_mbcnt_lo/hi): with one lane per bit
// of a 64-bit word, it is the rank of the lane's bit among the word's set bits.
__device__ __forceinline__ uint32_t bits_below_lane(uint64_t w) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(w >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)w, 0u));
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Adds v[r] into tile[cell[r]] (an LDS array) for R independent cells: all reads and the
// first compare-and-swap of every cell are issued back to back (R LDS round trips in
// flight instead of R in sequence), then only cells that lost a race retry.  Same fp32
// additions as ds_add_f32, which gfx950 executes about 9x slower at scattered addresses.
template <int R>
__device__ __forceinline__ void lds_add_f32_many(float* tile, const uint32_t* cell,
                                                 const float* v, const bool* on) {
  uint32_t* t = reinterpret_cast<uint32_t*>(tile);
  uint32_t old[R], got[R];
#pragma unroll
  for (int r = 0; r < R; ++r) old[r] = on[r] ? t[cell[r]] : 0u;
#pragma unroll
  for (int r = 0; r < R; ++r)
    got[r] = on[r] ? atomicCAS(&t[cell[r]], old[r], __float_as_uint(__uint_as_float(old[r]) + v[r]))
                   : old[r];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    while (got[r] != old[r]) {
      old[r] = got[r];
      got[r] = atomicCAS(&t[cell[r]], old[r], __float_as_uint(__uint_as_float(old[r]) + v[r]));
    }
  }
}

// Waits for every outstanding vector memory operation of the wave (s_waitcnt vmcnt(0), the
// other counters left alone).  Placed once after a batch of loads whose values are stored
// under data-dependent branches: past the branch joins the compiler can no longer count
// which operations are still in flight and would otherwise wait before each store for the
// previous store's completion.
__device__ __forceinline__ void wait_vector_memory() {
  __builtin_amdgcn_sched_barrier(0);   // no instruction is scheduled across the wait
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each XCD has its own
// L2.  This maps the linear id so that XCD x runs the x-th eighth of the (x-fastest) work
// items in order: neighbouring items, which share cache lines at their edges, then run on one
// XCD at about the same time.  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_grouped_item() {
  const uint32_t lin = blockIdx.x + blockIdx.y * gridDim.x;
  const uint32_t total = gridDim.x * gridDim.y;
  if (total % kXcds != 0) return lin;
  return (lin % kXcds) * (total / kXcds) + lin / kXcds;
}

// Streaming kernels: workgroups are dispatched to the 8 XCDs round-robin by linear id, and
// each XCD translates addresses through its own L2 TLB.  With consecutive work items on
// consecutive XCDs every XCD touches every page of the stream; this maps the linear id so
// that each XCD takes runs of `run` consecutive work items (one 2 MiB page of the stream),
// the 8 XCDs taking 8 adjacent runs at a time, so the stream still advances as one front.
// Measured on MI355X for the gradient stream (16 KiB per item): runs of 2 MiB beat 0.5, 1
// and 4 MiB, and the 32 GB stream of the 10^9-element workload ran 8% faster than
// round-robin order (5.29 -> 4.81 ms), the 1.6-5 GB ones 4-7% faster.  Items past the last
// whole group of 8 runs keep their own id.
__device__ __forceinline__ uint64_t xcd_run_item(uint64_t lin, uint64_t total, uint32_t run) {
  const uint64_t span = (uint64_t)kXcds * run;
  if (lin >= total / span * span) return lin;
  const uint64_t j = lin / kXcds;
  return (j / run) * span + (lin % kXcds) * run + j % run;
}

// For each of U positions e[u]: the largest c in [0, nb) with off[c] <= e[u] (off
// non-decreasing, off[0] = 0).  Branch-free search whose step count depends only on nb, so
// the U searches advance together with U independent LDS reads per step.
template <int U>
__device__ __forceinline__ void segments_of(const uint32_t* off, uint32_t nb, const uint32_t* e,
                                            uint32_t* c) {
#pragma unroll
  for (int u = 0; u < U; ++u) c[u] = 0;
  uint32_t len = nb;
  while (len > 1) {
    const uint32_t half = len >> 1;
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] += (off[c[u] + half] <= e[u]) ? half : 0u;
    len -= half;
  }
}

}  // namespace s2r

// Expand a template call over D = 1..16 (every row count the header allows).
#define S2R_DISPATCH_D(d, CALL)                        \
  switch (d) {                                         \
    case 1: { constexpr int D = 1; CALL; } break;      \
    case 2: { constexpr int D = 2; CALL; } break;      \
    case 3: { constexpr int D = 3; CALL; } break;      \
    case 4: { constexpr int D = 4; CALL; } break;      \
    case 5: { constexpr int D = 5; CALL; } break;      \
    case 6: { constexpr int D = 6; CALL; } break;      \
    case 7: { constexpr int D = 7; CALL; } break;      \
    case 8: { constexpr int D = 8; CALL; } break;      \
    case 9: { constexpr int D = 9; CALL; } break;      \
    case 10: { constexpr int D = 10; CALL; } break;    \
    case 11: { constexpr int D = 11; CALL; } break;    \
    case 12: { constexpr int D = 12; CALL; } break;    \
    case 13: { constexpr int D = 13; CALL; } break;    \
    case 14: { constexpr int D = 14; CALL; } break;    \
    case 15: { constexpr int D = 15; CALL; } break;    \
    case 16: { constexpr int D = 16; CALL; } break;    \
    default: break;                                    \
  }
