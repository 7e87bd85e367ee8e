// tiles.hpp -- the tile table of a batch of several sequences with a few
// query rows each: runs of equal q_seq (rows of one sequence kept
// contiguous) cut into tiles of qwg rows, so that the MFMA tiling of
// prefill.hip streams each sequence's keys once per tile rather than once
// per row.  Built by one workgroup: a running maximum over the run starts
// (a Hillis-Steele scan in LDS) gives each row its run's first row, and a
// block scan of the tile starts places the tiles.
#pragma once

#include "common.hpp"
#include "select.hpp"

namespace misa {

// One workgroup of NT threads; smax: NT ints of LDS, sh: NT/64 + 4 words.
// tiles[i] = (first row, sequence) for i < *ntiles.  When the tiles would
// pass `bound` (the rows of a sequence are not contiguous), *ntiles = 0 and
// *fallback = T (the per-row scoring then takes every row), else
// *fallback = 0.
template <int NT>
__device__ __forceinline__ void build_tile_table(const int32_t *q_seq, int T, int qwg, int bound, int2 *tiles,
                                                 uint32_t *ntiles, uint32_t *fallback, int *smax, uint32_t *sh) {
  const int tid = threadIdx.x;
  int carry_rs = 0;
  uint32_t carry_n = 0;
  for (int base = 0; base < T; base += NT) {
    const int t = base + tid;
    const int q = t < T ? q_seq[t] : 0;
    smax[tid] = (t < T && (t == 0 || q != q_seq[t - 1])) ? t : -1;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int v = tid >= off ? smax[tid - off] : -1;
      __syncthreads();
      smax[tid] = max(smax[tid], v);
      __syncthreads();
    }
    const int rs = max(smax[tid], carry_rs);  // the row's run start
    const uint32_t ts = (t < T && (t - rs) % qwg == 0) ? 1u : 0u;
    uint32_t total;
    const uint32_t pos = carry_n + block_scan<NT>(ts, sh, total) - ts;
    if (ts && pos < (uint32_t)bound) tiles[pos] = make_int2(t, q);
    carry_rs = max(carry_rs, smax[NT - 1]);
    carry_n += total;
    __syncthreads();
  }
  if (tid == 0) {
    const bool fits = carry_n <= (uint32_t)bound;
    *ntiles = fits ? carry_n : 0u;
    *fallback = fits ? 0u : (uint32_t)T;
  }
}

}  // namespace misa
