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

// Threshold digit from a 4096-bin histogram in LDS, counted from the top:
// the bin holding the k-th largest key.  The first wave alone resolves it
// (lane l sums the 64 bins [4096 - 64 (l + 1), 4096 - 64 l); a scan over
// the lanes finds the lane whose bins cross k, and a scan over that lane's
// 64 bins, one per lane, finds the bin); the workgroup reads the result
// from sh[NT/64 .. NT/64 + 2] between two barriers, so the caller may reuse
// those words at once.  sh needs NT/64 + 3 words; call with uniform control
// flow.
template <int NT>
__device__ __forceinline__ Thresh threshold_from_lds(const uint32_t *lh, uint32_t k, uint32_t *sh) {
  static_assert(NT % kWave == 0 && kHistBins == 64 * kWave, "one wave, 64 bins a lane");
  uint32_t *res = sh + NT / kWave;
  if (threadIdx.x < kWave) {
    const int lane = (int)threadIdx.x;
    const int lo = kHistBins - 64 * (lane + 1);
    uint32_t s = 0;
    // (neighbouring lanes start at different 4-bin chunks: lanes 256 bytes
    // apart would all hit one bank group)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 v = *(const uint4 *)(lh + lo + 4 * ((j + lane) & 15));
      s += (v.x + v.y) + (v.z + v.w);
    }
    const uint32_t incl = wave_incl_scan(s);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    const uint32_t kk = min(k, total);
    uint32_t b1 = kHistBins, above = 0, eq = 0;
    if (kk > 0) {
      const int L = __ffsll((unsigned long long)__ballot(incl >= kk)) - 1;
      const uint32_t aboveL = (uint32_t)__builtin_amdgcn_readlane((int)(incl - s), L);
      const int loL = kHistBins - 64 * (L + 1);
      const uint32_t x = lh[loL + 63 - lane];  // lane i: bin loL + 63 - i
      const uint32_t inc2 = wave_incl_scan(x) + aboveL;
      const int i = __ffsll((unsigned long long)__ballot(inc2 >= kk)) - 1;
      b1 = (uint32_t)(loL + 63 - i);
      above = (uint32_t)__builtin_amdgcn_readlane((int)(inc2 - x), i);
      eq = (uint32_t)__builtin_amdgcn_readlane((int)x, i);
    }
    if (lane == 0) {
      res[0] = b1;
      res[1] = above;
      res[2] = eq;
    }
  }
  __syncthreads();
  Thresh th;
  th.b1 = (int)res[0];
  th.above = res[1];
  th.eq = res[2];
  // the bins below the crossing one are empty when the histogram holds
  // fewer than k keys, so min(k, above + eq) is min(k, total)
  th.kk = th.b1 < kHistBins ? min(k, th.above + th.eq) : 0u;
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
