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

// A selection key that orders (score, token) pairs: the score's order key in
// the high word and the complemented token in the low word, so that of equal
// scores the lower token ranks higher (the row's ties are broken by token).
__device__ __forceinline__ uint64_t composite(uint32_t key, int tok) {
  return ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)tok);
}


// ------------------------------------------------------- chunk candidate lists
// The two-stage top-k of few long rows.  A row is cut into chunks (one per
// workgroup of the kernel that produces its scores); each chunk keeps a
// short list of its best entries -- every valid entry whose 12-bit digit is
// at least a cutoff `cut` -- and records the cutoff, so that every entry it
// dropped has a digit below `cut`.  The row's top-k is then exact if it is
// taken from the union of the lists and its k-th key has a digit no lower
// than every chunk's cutoff (topk_merge_kernel checks this, and otherwise
// selects from the whole score row).
//
// A chunk of n columns out of a row of n_row valid columns holds, on
// average, E = k n / n_row of the row's top k; it keeps its best
// quota = E + 6 sqrt(E) + 16 entries (rounded up to whole digits), so a
// chunk holding more of the row's top-k than that -- which makes the check
// fail -- is a six-sigma event on unstructured scores.
__device__ __forceinline__ uint32_t chunk_quota(int k, int n, int n_row) {
  if (n_row <= 0) return 0u;
  const float e = (float)k * (float)n / (float)n_row;
  const float q = ceilf(e + 6.f * sqrtf(e) + 16.f);
  return q >= (float)n ? (uint32_t)n : (uint32_t)q;
}

// List entry: (order key, token id); header: (entries, cutoff digit,
// largest key in the list, 0).
// sc: the chunk's n scores in LDS; lh: the 4096-bin histogram of the top 12
// key bits of its nvalid valid entries (LDS); valid(i) / tok(i): entry i's
// validity and token id.  Every thread of the NT-thread workgroup calls this
// with uniform arguments (it contains barriers); sh needs 2 NT/64 + 8 words.
// At most cap entries are written to out.
template <int NT, int MAXPER, typename Valid, typename Tok>
__device__ __forceinline__ void chunk_list(const float *sc, int n, const uint32_t *lh, uint32_t nvalid,
                                           uint32_t quota, uint32_t cap, Valid valid, Tok tok, uint2 *out,
                                           uint4 *head, uint32_t *sh) {
  const int tid = threadIdx.x;
  uint32_t cut = 0;  // keep every valid entry
  if (quota < nvalid) {
    const Thresh th = threshold_from_lds<NT>(lh, quota, sh);
    // the digit holding the quota-th best entry, or the one above it when
    // that digit's entries would overflow the list
    cut = th.above + th.eq <= cap ? (uint32_t)th.b1 : (uint32_t)th.b1 + 1u;
  }
  uint32_t hits = 0, kmax = 0;
#pragma unroll
  for (int u = 0; u < MAXPER; ++u) {
    const int i = tid + NT * u;
    const uint32_t key = order_key(sc[min(i, max(n - 1, 0))]);
    if (i < n && valid(i) && (key >> kHistShift) >= cut) {
      hits |= 1u << u;
      kmax = max(kmax, key);
    }
  }
  kmax = wave_max_u32(kmax);
  if (lane_id() == 0) sh[NT / kWave + 7 + threadIdx.x / kWave] = kmax;
  uint32_t total;
  uint32_t pos = block_scan<NT>((uint32_t)__popc(hits), sh, total) - (uint32_t)__popc(hits);
#pragma unroll
  for (int u = 0; u < MAXPER; ++u) {
    if ((hits >> u) & 1u) {
      const int i = tid + NT * u;
      if (pos < cap) out[pos] = make_uint2(order_key(sc[i]), (uint32_t)tok(i));
      ++pos;
    }
  }
  if (tid == 0) {
    uint32_t m = 0;
    for (int w = 0; w < NT / kWave; ++w) m = max(m, sh[NT / kWave + 7 + w]);
    *head = make_uint4(min(total, cap), total <= cap ? cut : 0xFFFFFFFFu, m, 0u);
  }
}

}  // namespace misa
