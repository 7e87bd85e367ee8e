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
  __shared__ float red[2][kD];
  __shared__ float mean[kD];
  const int t = blockIdx.y, ch = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int p = a.q_pos[t];
  const int bt = p / a.B;  // complete blocks are [0, bt)
  const int sq = a.q_seq[t];
  float *out = a.partial + ((size_t)t * (a.nchunks + 1) + ch) * a.H;

  if (ch == a.nchunks) {  // the query's own last block: [bt*B, p]
    const int lo = bt * a.B;
    const int c = tid & (kD - 1), half = tid >> 7;
    const uint16_t *kb = a.keys + (size_t)sq * a.Lmax * kD + c;
    float s = 0.f;
    for (int i = lo + half; i <= p; i += 2) s += bf16_to_f32(kb[(size_t)i * kD]);
    red[half][c] = s;
    __syncthreads();
    if (tid < kD) mean[tid] = (red[0][tid] + red[1][tid]) / (float)(p - lo + 1);
    __syncthreads();
    for (int j = tid; j < a.H; j += 256) {
      const uint16_t *qj = a.q + ((size_t)t * a.H + j) * kD;
      float x = 0.f;
      for (int cc = 0; cc < kD; ++cc) x = fmaf(bf16_to_f32(qj[cc]), mean[cc], x);
      out[j] = fmaxf(x, 0.f);
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
      float v = ok ? fmaxf(acc[ht][r], 0.f) : 0.f;
      v += __shfl_xor(v, 1, kWave);
      v += __shfl_xor(v, 2, kWave);
      v += __shfl_xor(v, 4, kWave);
      v += __shfl_xor(v, 8, kWave);
      if (col == 0) part[wave][ht * 16 + grp * 4 + r] = v;
    }
  }
  __syncthreads();
  for (int j = tid; j < a.H; j += 256) out[j] = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
}

__global__ __launch_bounds__(64) void route_final_kernel(RouteArgs a) {
  const int t = blockIdx.x;
  const int lane = lane_id();
  const float *pp = a.partial + (size_t)t * (a.nchunks + 1) * a.H;
  float gv[2];
  bool avail[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = lane + 64 * u;
    avail[u] = j < a.H;
    gv[u] = 0.f;
    if (avail[u]) {
      float s = 0.f;
      for (int c = 0; c <= a.nchunks; ++c) s += pp[(size_t)c * a.H + j];
      float wj = a.w[(size_t)t * a.H + j];
      if (a.mode == 1) wj = fabsf(wj);
      gv[u] = wj * s;
      if (a.g) a.g[(size_t)t * a.H + j] = gv[u];
    }
  }
  for (int r = 0; r < a.h; ++r) {
    // this lane's best remaining head under (g desc, id asc)
    float bg = 0.f;
    int bj = 0x7FFFFFFF;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = lane + 64 * u;
      if (avail[u] && (bj == 0x7FFFFFFF || gv[u] > bg)) {
        bg = gv[u];
        bj = j;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float og = __shfl_xor(bg, o, kWave);
      const int oj = __shfl_xor(bj, o, kWave);
      const bool better = oj != 0x7FFFFFFF &&
                          (bj == 0x7FFFFFFF || og > bg || (!(og < bg) && oj < bj));
      if (better) {
        bg = og;
        bj = oj;
      }
    }
    if (lane == 0) a.heads[(size_t)t * a.h + r] = bj;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (lane + 64 * u == bj) avail[u] = false;
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
  hipLaunchKernelGGL(route_final_kernel, dim3(a.T), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
