// select.hpp -- block-wide helpers of the per-row top-k: prefix scans and
// the first radix digit taken from a 4096-bin histogram of the top 12
// order-key bits.
#pragma once

#include "common.hpp"

namespace misa {

// Per-row counters of the selection workspace (zeroed with the histogram):
//   [0] columns above the threshold digit reserved so far
//   [1] threshold-digit candidates reserved so far
//   [4] b1  [5] above  [6] eq  [7] kk  -- the row's threshold, for the finish
constexpr int kRowCounters = 8;

struct Thresh {
  int b1;          // the digit holding the kk-th largest key
  uint32_t above;  // valid columns with digit > b1
  uint32_t eq;     // valid columns with digit == b1
  uint32_t kk;     // min(k, valid columns)
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide inclusive scan of one value per thread, NT threads (a multiple
// of 64).  sh needs NT/64 words.  Returns the inclusive prefix; `total` is
// the block sum.  Contains two barriers: call with uniform control flow.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *sh, uint32_t &total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) sh[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t x = sh[i];
    if (i < wave) base += x;
    total += x;
  }
  __syncthreads();
  return base + incl;
}

// Threshold digit from a 4096-bin histogram in LDS.  The first 256 threads
// own 16 consecutive bins each, counted from the top; the others add zero.
// sh needs NT/64 + 4 words.
template <int NT>
__device__ __forceinline__ Thresh threshold_from_lds(const uint32_t *lh, uint32_t k, uint32_t *sh) {
  static_assert(NT >= 256, "one thread per 16 bins");
  const int tid = threadIdx.x;
  const int top = kHistBins - 1 - 16 * tid;
  uint32_t v[16];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = tid < 256 ? lh[top - i] : 0u;
    s += v[i];
  }
  uint32_t total;
  const uint32_t incl = block_scan<NT>(s, sh, total);
  const uint32_t excl = incl - s;
  const uint32_t kk = min(k, total);
  uint32_t *res = sh + NT / kWave;
  if (kk > 0 && excl < kk && kk <= incl) {
    uint32_t cum = excl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (cum + v[i] >= kk) {
        res[0] = (uint32_t)(top - i);
        res[1] = cum;
        res[2] = v[i];
        break;
      }
      cum += v[i];
    }
  }
  __syncthreads();
  Thresh th;
  th.kk = kk;
  th.b1 = kk ? (int)res[0] : kHistBins;
  th.above = kk ? res[1] : 0;
  th.eq = kk ? res[2] : 0;
  __syncthreads();
  return th;
}

}  // namespace misa
