// hisa.hip -- the hierarchical indexer's coarse stage: block scores.
//
// "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse Attention"
// (abstract) searches in two passes: a cheap pass ranks whole blocks of the
// prefix by a score computed on each block's pooled summary and drops the
// low-ranked blocks, and the unchanged token-level indexer then looks only
// at the tokens of the blocks that survive.  Here
// a block's representation is its mean key (the pooled-key cache MISA's
// router reads, "MISA: Mixture of Indexer Sparse Attention for Long-Context
// LLM Inference", Technical Summary, Methodology: Lightweight Block-Pooled
// Router) and its score is the indexer's own form on that mean,
//   s_b = sum_{j in heads} w_j * max(0, q_j . Kbar_b),
// over all H heads, or over the routed heads when MISA's router runs first.
//
// hisa_block_kernel: one workgroup per (query, 64 complete blocks), as the
// decode router: the (gathered) head rows are the A operand of
// v_mfma_f32_16x16x32_bf16, 16 pooled blocks per B tile, each fp32 pooled
// key split exactly into three bf16 terms (exact products, fp32
// accumulation).  The epilogue weights and ReLUs the four head rows a lane
// holds and sums the four lane groups, giving one score per block column.
// The extra workgroup per query scores the query's own last block, pooled
// from the raw keys of [bt*B, p], and writes the query's block count.
// The refinement's scoring kernel expands the kept block ids into token
// lists itself (score.hip, the kept-block gather).
#include "common.hpp"
#include "kernels.hpp"

namespace misa {

// A 16-byte value with every word ANDed with m (0 or all ones): masks a value
// loaded from a clamped address, with no branch around the load.
static __device__ __forceinline__ uint4 mask_u4(uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

template <int HT>
__global__ __launch_bounds__(256) void hisa_block_kernel(HisaArgs a) {
  __shared__ float red[4][kD];
  __shared__ float mean[kD];
  __shared__ float wsum[4];
  const int t = blockIdx.y, ch = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int p = a.q_pos[t];
  const int bt = p / a.B;  // complete blocks are [0, bt); block bt is the query's own
  const int sq = a.q_seq[t];
  float *srow = a.bscore + (size_t)t * a.Mmax;
  auto head_of = [&](int m) { return a.heads ? a.heads[(size_t)t * a.nh + m] : m; };

  if (ch == a.nchunks) {  // the query's own last block: [bt*B, p]
    const int lo = bt * a.B;
    const int dc = tid & 15, kl = tid >> 4;
    const uint16_t *kb = a.keys + (size_t)sq * a.Lmax * kD + dc * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = lo + kl; i0 <= p; i0 += 16 * 8) {  // 8 loads in flight per thread
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const uint4 *)(kb + (size_t)min(i0 + 16 * u, p) * kD);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + 16 * u > p) break;
        const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(x[e] << 16);
          acc[2 * e + 1] += __uint_as_float(x[e] & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += __shfl_xor(acc[e], 16, kWave);
      acc[e] += __shfl_xor(acc[e], 32, kWave);
    }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][dc * 8 + e] = acc[e];
    }
    __syncthreads();
    if (tid < kD)
      mean[tid] = (((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid]) / (float)(p - lo + 1);
    __syncthreads();
    // head dots against the tail mean: thread = (head row m, 32-dim quarter)
    const int qq = tid & 3;
    float contrib = 0.f;
    for (int m0 = 0; m0 < a.nh; m0 += 64) {
      const int m = m0 + (tid >> 2);
      float x = 0.f;
      // loads from a clamped head, rows past nh masked (no branch around them)
      const uint32_t mm = m < a.nh ? 0xFFFFFFFFu : 0u;
      const uint16_t *qv = a.q + ((size_t)t * a.H + head_of(min(m, a.nh - 1))) * kD + qq * 32;
      uint4 qx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) qx[u] = mask_u4(*(const uint4 *)(qv + u * 8), mm);
      {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 v = qx[u];
          const uint32_t y[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = qq * 32 + u * 8 + 2 * e;
            x = fmaf(__uint_as_float(y[e] << 16), mean[c], x);
            x = fmaf(__uint_as_float(y[e] & 0xFFFF0000u), mean[c + 1], x);
          }
        }
      }
      x += __shfl_xor(x, 1, kWave);
      x += __shfl_xor(x, 2, kWave);
      if (m < a.nh && qq == 0) contrib += a.w[(size_t)t * a.H + head_of(m)] * fmaxf(x, 0.f);
    }
    contrib = wave_sum(contrib);
    if (lane == 0) wsum[wave] = contrib;
    __syncthreads();
    if (tid == 0) {
      srow[bt] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
      a.mt[t] = bt + 1;
    }
    return;
  }

  const int b0 = ch * kHisaChunk;
  const int b = b0 + wave * 16 + col;
  if (b0 >= bt) {  // no complete block here: -inf past the query's own block
    for (int bb = b0 + tid; bb < min(b0 + kHisaChunk, a.Mmax); bb += 256)
      if (bb > bt) srow[bb] = -INFINITY;
    return;
  }
  // Head rows (A operand) and the weights of this lane's rows: two batched
  // rounds of loads (head ids, then rows and weights) from clamped indices,
  // rows past nh masked, so that no load waits behind a branch
  bf16x8 qa[HT][4];
  float wv[HT][4];
  {
    int jq[HT], jw[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      jq[ht] = head_of(min(ht * 16 + col, a.nh - 1));
#pragma unroll
      for (int r = 0; r < 4; ++r) jw[ht][r] = head_of(min(ht * 16 + grp * 4 + r, a.nh - 1));
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint32_t mq = ht * 16 + col < a.nh ? 0xFFFFFFFFu : 0u;
      const uint16_t *qr = a.q + ((size_t)t * a.H + jq[ht]) * kD + grp * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) qa[ht][s] = as_bf16x8(mask_u4(*(const uint4 *)(qr + s * 32), mq));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t wb = __float_as_uint(a.w[(size_t)t * a.H + jw[ht][r]]);
        wv[ht][r] = __uint_as_float(wb & (ht * 16 + grp * 4 + r < a.nh ? 0xFFFFFFFFu : 0u));
      }
    }
  }
  const bool ok = b < bt;
  const float *pb = a.pooled + ((size_t)sq * a.Mmax + (ok ? b : 0)) * kD + grp * 8;
  f32x4 acc[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) acc[ht] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float4 x0 = *(const float4 *)(pb + s * 32);
    const float4 x1 = *(const float4 *)(pb + s * 32 + 4);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    u16x8 hi, mi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t h16, m16, l16;
      split3(xs[e], h16, m16, l16);
      hi[e] = h16;
      mi[e] = m16;
      lo[e] = l16;
    }
    const bf16x8 bh = __builtin_bit_cast(bf16x8, hi);
    const bf16x8 bm = __builtin_bit_cast(bf16x8, mi);
    const bf16x8 bl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      acc[ht] = mfma16(qa[ht][s], bh, acc[ht]);
      acc[ht] = mfma16(qa[ht][s], bm, acc[ht]);
      acc[ht] = mfma16(qa[ht][s], bl, acc[ht]);
    }
  }
  // weighted ReLU over the lane's four head rows, then over the lane groups
  float part = 0.f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) part += wv[ht][r] * fmaxf(acc[ht][r], 0.f);
  part += __shfl_xor(part, 16, kWave);
  part += __shfl_xor(part, 32, kWave);
  if (grp == 0 && b < a.Mmax) {
    if (ok) srow[b] = part;
    else if (b > bt) srow[b] = -INFINITY;
  }
}

hipError_t launch_hisa_blocks(const HisaArgs &a, hipStream_t st) {
  dim3 grid(a.nchunks + 1, a.T);
  if (a.nh <= 16) hipLaunchKernelGGL(hisa_block_kernel<1>, grid, dim3(256), 0, st, a);
  else if (a.nh <= 32) hipLaunchKernelGGL(hisa_block_kernel<2>, grid, dim3(256), 0, st, a);
  else if (a.nh <= 64) hipLaunchKernelGGL(hisa_block_kernel<4>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(hisa_block_kernel<8>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
