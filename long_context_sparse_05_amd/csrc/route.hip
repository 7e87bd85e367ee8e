// route.hip -- the block-pooled head router.
//
// Per query row t ("MISA: Mixture of Indexer Sparse Attention for
// Long-Context LLM Inference", Technical Summary, Methodology: MISA --
// Lightweight Block-Pooled Router): affinities of every head j against the
// mean-pooled keys of the query's M_t = floor(p_t/B) + 1 prefix blocks,
// summed over blocks and scaled by the head weight, then the top-h heads:
//   g_j = w'_j * sum_b max(0, q_j . Kbar_b),   w' = w (mode 0) or |w| (mode 1).
// Blocks b < floor(p_t/B) are complete and come from the pooled cache; the
// query's own last block is pooled here from the raw keys of [bB, p_t].
//
// route_partial_kernel: one workgroup per (query, 64 complete blocks); the
// H x 64 affinities are an MFMA contraction over d = 128 with the query's
// head rows as A and 16 pooled blocks per B tile.  The pooled keys are fp32;
// each is split exactly into three bf16 terms (hi + mid + lo), so three
// bf16 MFMAs give the fp32 dot product with exact products and fp32
// accumulation.  The extra workgroup per query (index nchunks) pools the
// tail block and does its dot products on the vector ALUs.
// route_final_kernel: one wave per query sums the partials in a fixed order,
// applies the weight and selects the top-h heads by (g desc, head id asc).
#include "common.hpp"
#include "kernels.hpp"

namespace misa {

template <int HT>
__global__ __launch_bounds__(256) void route_partial_kernel(RouteArgs a) {
  __shared__ float part[4][HT * 16];
  __shared__ float red[4][kD];
  __shared__ float mean[kD];
  const int t = blockIdx.y, ch = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int p = a.q_pos[t];
  const int bt = p / a.B;  // complete blocks are [0, bt)
  const int sq = a.q_seq[t];
  float *out = a.partial + ((size_t)t * (a.nchunks + 1) + ch) * a.H;

  if (ch == a.nchunks) {  // the query's own last block: [bt*B, p]
    // Mean of the tail keys.  Thread = (8-dim slice dc, key lane kl): 16 key
    // lanes stream the block with 16-byte loads; the 4 key lanes of a wave
    // are folded with xor shuffles, the 4 waves through LDS.
    const int lo = bt * a.B;
    const int dc = tid & 15, kl = tid >> 4;
    // this thread's query slices for the head dots below, requested first:
    // thread = (head j = tid/4 + 64*round, 32-dim quarter qq)
    const int qq = tid & 3;
    uint4 qv[2][4];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int j = rd * 64 + (tid >> 2);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        qv[rd][u] = j < a.H ? ((const uint4 *)(a.q + ((size_t)t * a.H + j) * kD + qq * 32))[u]
                            : make_uint4(0, 0, 0, 0);
    }
    const uint16_t *kb = a.keys + (size_t)sq * a.Lmax * kD + dc * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = lo + kl; i0 <= p; i0 += 16 * 8) {  // 8 loads in flight per thread
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + 16 * u;
        v[u] = i <= p ? *(const uint4 *)(kb + (size_t)i * kD) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
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
    // Head dots against the tail mean: thread = (head j, 32-dim quarter).
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int j = rd * 64 + (tid >> 2);
      float x = 0.f;
      if (j < a.H) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 v = qv[rd][u];
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
      if (j < a.H && qq == 0) out[j] = fmaxf(x, 0.f);
    }
    return;
  }

  const int b0 = ch * kRouteChunk;
  if (b0 >= bt) {  // no complete block of this chunk in the prefix
    for (int j = tid; j < a.H; j += 256) out[j] = 0.f;
    return;
  }

  bf16x8 qa[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int m = ht * 16 + col;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < a.H) v = *(const uint4 *)(a.q + ((size_t)t * a.H + m) * kD + s * 32 + grp * 8);
      qa[ht][s] = as_bf16x8(v);
    }
  }
  const int b = b0 + wave * 16 + col;
  const bool ok = b < bt;
  const float *pb = a.pooled + ((size_t)sq * a.Mmax + (ok ? b : 0)) * kD + grp * 8;
  f32x4 acc[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) acc[ht] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (ok) {
      x0 = *(const float4 *)(pb + s * 32);
      x1 = *(const float4 *)(pb + s * 32 + 4);
    }
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
  // ReLU, then sum over this wave's 16 blocks (the 16 lanes of a group).
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = row_sum16(ok ? fmaxf(acc[ht][r], 0.f) : 0.f);
      if (col == 0) part[wave][ht * 16 + grp * 4 + r] = v;
    }
  }
  __syncthreads();
  for (int j = tid; j < a.H; j += 256) out[j] = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
}

// One workgroup per query: four thread quarters sum contiguous quarters of
// the partials (loads in flight together), combined in a fixed order; then
// every head computes its own rank, and ranks below h are written.  In the
// fused indexer call it also clears the query's selection histogram, which
// saves the scoring step a separate fill launch.
__global__ __launch_bounds__(256) void route_final_kernel(RouteArgs a) {
  __shared__ float red[4][MISA_MAX_HEADS_DEV];
  __shared__ float gs[MISA_MAX_HEADS_DEV];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), quarter = tid >> 6;
  const int nparts = a.nchunks + 1;
  const float *pp = a.partial + (size_t)t * nparts * a.H;
  const int per = (nparts + 3) / 4;
  const int c0 = quarter * per, c1 = min(nparts, c0 + per);
  if (a.zero_hist) {  // fused indexer call: clear this query's selection histogram
    uint4 *zh = (uint4 *)(a.zero_hist + (size_t)t * kHistBins);
    for (int i = tid; i < kHistBins / 4; i += 256) zh[i] = make_uint4(0, 0, 0, 0);
    if (tid < 8) a.zero_ctr[(size_t)t * 8 + tid] = 0u;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = lane + 64 * u;
    if (j < a.H) {
      float s = 0.f;
      int c = c0;
      for (; c + 8 <= c1; c += 8) {
        float v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = pp[(size_t)(c + x) * a.H + j];
#pragma unroll
        for (int x = 0; x < 8; ++x) s += v[x];
      }
      for (; c < c1; ++c) s += pp[(size_t)c * a.H + j];
      red[quarter][j] = s;
    }
  }
  __syncthreads();
  if (tid < a.H) {
    const float s = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    float wj = a.w[(size_t)t * a.H + tid];
    if (a.mode == 1) wj = fabsf(wj);
    gs[tid] = wj * s;
    if (a.g) a.g[(size_t)t * a.H + tid] = gs[tid];
  }
  __syncthreads();
  // rank of head j under (g desc, id asc); the heads of rank < h are routed
  if (tid < a.H) {
    const float gj = gs[tid];
    int rank = 0;
    for (int i = 0; i < a.H; ++i) {
      const float gi = gs[i];
      rank += (gi > gj || (gi == gj && i < tid)) ? 1 : 0;
    }
    if (rank < a.h) a.heads[(size_t)t * a.h + rank] = tid;
  }
}

template <int HT>
static void launch_partial(const RouteArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((route_partial_kernel<HT>), dim3(a.nchunks + 1, a.T), dim3(256), 0, st, a);
}

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.H <= 16) launch_partial<1>(a, st);
  else if (a.H <= 32) launch_partial<2>(a, st);
  else if (a.H <= 64) launch_partial<4>(a, st);
  else launch_partial<8>(a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_final_kernel, dim3(a.T), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
