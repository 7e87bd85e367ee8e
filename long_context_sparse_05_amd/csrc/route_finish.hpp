// route_finish.hpp -- the last step of the block-pooled head router, shared
// by route_final_kernel and the fused scoring kernel's prologue so that both
// give the same heads bit for bit.
//
// ("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
// Inference", Technical Summary, Methodology: MISA -- Lightweight
// Block-Pooled Router.)  A query's importance of head j is its weight times
// the sum over the query's blocks of max(0, q_j . Kbar_b); the router
// kernel leaves that sum as partial sums over chunks of blocks, [nparts][H].
// Four waves sum contiguous quarters of the partials (eight loads in flight
// per lane, clamped and masked, added in order), the quarters are combined
// in a fixed order, weighted (w, or |w| in mode 1), and every head computes
// its rank under (g desc, head id asc); the heads of rank < h are routed.
#pragma once

#include "common.hpp"

namespace misa {

// Every thread of the workgroup calls this (it contains barriers); threads
// 0..255 do the sums, threads 0..H-1 the ranking.  red / gs: LDS scratch.
// g_out [H] and heads_out [h] (global) and heads_lds [h] may be null.
__device__ __forceinline__ void route_finish(const float *pp, int nparts, int H, const float *wrow,
                                             int mode, int h, float (*red)[MISA_MAX_HEADS_DEV],
                                             float *gs, float *g_out, int32_t *heads_out,
                                             int32_t *heads_lds) {
  const int tid = threadIdx.x, lane = lane_id(), quarter = tid >> 6;
  const int per = (nparts + 3) / 4;
  const int c0 = quarter * per, c1 = min(nparts, c0 + per);
  const float wpre = wrow[min(tid, H - 1)];
  if (quarter < 4) {
    for (int u = 0; u < 2 && 64 * u < H; ++u) {
      const int j = lane + 64 * u;
      const float *pj = pp + min(j, H - 1);
      float s = 0.f;
      for (int c = c0; c < c1; c += 8) {
        float v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const uint32_t m = c + x < c1 ? 0xFFFFFFFFu : 0u;
          v[x] = __uint_as_float(__float_as_uint(pj[(size_t)min(c + x, c1 - 1) * H]) & m);
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) s += v[x];
      }
      if (j < H) red[quarter][j] = s;
    }
  }
  __syncthreads();
  if (tid < H) {
    const float s = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    const float wj = mode == 1 ? fabsf(wpre) : wpre;
    gs[tid] = wj * s;
    if (g_out) g_out[tid] = gs[tid];
  }
  __syncthreads();
  if (tid < H) {
    const float gj = gs[tid];
    int rank = 0;
    for (int i = 0; i < H; ++i) {
      const float gi = gs[i];
      rank += (gi > gj || (gi == gj && i < tid)) ? 1 : 0;
    }
    if (rank < h) {
      if (heads_out) heads_out[rank] = tid;
      if (heads_lds) heads_lds[rank] = tid;
    }
  }
}

}  // namespace misa
