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
// route_partial_kernel: one workgroup per (query, kRouteChunk complete
// blocks); the H x kRouteChunk affinities are an MFMA contraction over
// d = 128 with the query's head rows as A and 16 pooled blocks per B tile.
// The pooled keys are fp32; each is split exactly into three bf16 terms
// (hi + mid + lo), so three bf16 MFMAs give the fp32 dot product with exact
// products and fp32 accumulation.  The extra workgroup per query (index nchunks) pools the
// tail block and does its dot products on the vector ALUs.
// route_final_kernel: one wave per query sums the partials in a fixed order,
// applies the weight and selects the top-h heads by (g desc, head id asc).
#include "common.hpp"
#include "kernels.hpp"
#include "route_finish.hpp"
#include "tiles.hpp"

namespace misa {

// A 16-byte value with every word ANDed with m (0 or all ones): masks a value
// loaded from a clamped address, with no branch around the load.
static __device__ __forceinline__ uint4 mask_u4(uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

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
    // (loads from clamped indices, masked afterwards: a load under a branch
    // would make each wait for every load before it)
    uint4 qv[2][4];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int j = rd * 64 + (tid >> 2);
      const uint32_t mj = j < a.H ? 0xFFFFFFFFu : 0u;
      const uint4 *qr = (const uint4 *)(a.q + ((size_t)t * a.H + min(j, a.H - 1)) * kD + qq * 32);
#pragma unroll
      for (int u = 0; u < 4; ++u) qv[rd][u] = mask_u4(qr[u], mj);
    }
    const uint16_t *kb = a.keys + (size_t)sq * a.Lmax * kD + dc * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = lo + kl; i0 <= p; i0 += 16 * 8) {  // 8 loads in flight per thread
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + 16 * u;
        v[u] = mask_u4(*(const uint4 *)(kb + (size_t)min(i, p) * kD), i <= p ? 0xFFFFFFFFu : 0u);
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

  // every load issued at once, from clamped indices, and masked afterwards
  // (a load under a branch would make each step wait for all before it)
  bf16x8 qa[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int m = ht * 16 + col;
    const uint32_t mq = m < a.H ? 0xFFFFFFFFu : 0u;
    const uint16_t *qr = a.q + ((size_t)t * a.H + min(m, a.H - 1)) * kD + grp * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[ht][s] = as_bf16x8(mask_u4(*(const uint4 *)(qr + s * 32), mq));
  }
  // The wave's G groups of 16 blocks (group g: blocks b0 + (4g + wave)*16 ..
  // + 15, one per lane column): all loads first, then per group the three
  // MFMA planes, the ReLU and the sum over the group's blocks.
  constexpr int G = kRouteChunk / 64;
  static_assert(G * 64 == kRouteChunk, "whole groups of 16 blocks for each of the four waves");
  uint4 xr[G][4][2];
  bool okg[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int b = b0 + (g * 4 + wave) * 16 + col;
    const bool ok = b < bt;
    okg[g] = ok;
    const uint32_t mb = ok ? 0xFFFFFFFFu : 0u;
    const float *pb = a.pooled + ((size_t)sq * a.Mmax + (ok ? b : 0)) * kD + grp * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      xr[g][s][0] = mask_u4(*(const uint4 *)(pb + s * 32), mb);
      xr[g][s][1] = mask_u4(*(const uint4 *)(pb + s * 32 + 4), mb);
    }
  }
  float rs[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) rs[ht][r] = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 x0 = xr[g][s][0], x1 = xr[g][s][1];
      const float xs[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z),
                           __uint_as_float(x0.w), __uint_as_float(x1.x), __uint_as_float(x1.y),
                           __uint_as_float(x1.z), __uint_as_float(x1.w)};
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
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) rs[ht][r] += row_sum16(okg[g] ? fmaxf(acc[ht][r], 0.f) : 0.f);
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (col == 0) part[wave][ht * 16 + grp * 4 + r] = rs[ht][r];
  __syncthreads();
  for (int j = tid; j < a.H; j += 256) out[j] = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
}

// One workgroup per query: the partial sums reduced in a fixed order,
// weighted and ranked (route_finish.hpp).  With a tile table requested, one
// more workgroup (the last) builds it for the grouped scoring that follows.
__global__ __launch_bounds__(256) void route_final_kernel(RouteArgs a) {
  __shared__ float red[4][MISA_MAX_HEADS_DEV];
  __shared__ float gs[MISA_MAX_HEADS_DEV];
  const int t = blockIdx.x;
  if (t == a.T) {  // uniform: the tile table
    __shared__ int smax[256];
    __shared__ uint32_t tsh[256 / kWave + 4];
    build_tile_table<256>(a.q_seq, a.T, a.tqwg, a.tbound, a.tiles, a.tcount, a.tcount + 1, smax, tsh);
    return;
  }
  const int nparts = a.nchunks + 1;
  route_finish(a.partial + (size_t)t * nparts * a.H, nparts, a.H, a.w + (size_t)t * a.H, a.mode, a.h,
               red, gs, a.g ? a.g + (size_t)t * a.H : nullptr, a.heads + (size_t)t * a.h, nullptr);
}

// ------------------------------------------------------------ tile router
// Many queries of one sequence (a prefill chunk): the (query, head) x block
// affinities form one GEMM.  A workgroup takes QWG consecutive queries (16
// with H <= 32, 8 with H <= 64); each of its 8 waves holds two 32-row tiles
// of query head rows (the A operand of v_mfma_f32_32x32x16_bf16, in
// registers).  The pooled blocks stream through LDS 32 at a time, split once
// per workgroup into three exact bf16 planes (B), so each dot product is,
// as in the decode router, exact products with fp32 accumulation.  Each
// lane keeps a ReLU running sum per accumulator row over the blocks that are
// complete for its query; one more B tile holds the queries' own tail-block
// means (column i = query i of the workgroup).  The sums are reduced across
// lanes once, weighted, ranked and written: no partials, no second kernel.
constexpr int kRtRowLds = 272;  // bytes per block row of a plane in LDS (256 + 16)

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int HT, int NW>  // 32-head row tiles per query (H <= 32 * HT), waves
__global__ __launch_bounds__(NW * 64) void route_tile_kernel(RouteArgs a) {
  constexpr int RT = 2, NT = NW * 64;
  constexpr int QWG = NW * RT / HT;
  constexpr int CH = 32 * 16 / NT;  // 8-float chunks of a 32-block tile per thread
  constexpr int PLANE = 32 * kRtRowLds;  // bytes of one plane of a 32-block tile
  __shared__ uint4 tiles[2][3 * PLANE / 16];
  __shared__ float gsum[QWG][32 * HT];
  __shared__ int sh_bt[QWG];
  __shared__ int sh_nb;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int qt0 = blockIdx.x * QWG;
  const int sq = a.q_seq[qt0];  // the host sends only batches of one sequence here
  const float *pbase = a.pooled + (size_t)sq * a.Mmax * kD;

  if (tid == 0) sh_nb = 0;
  __syncthreads();
  if (tid < QWG) {
    const int t = qt0 + tid;
    const int bt = t < a.T ? a.q_pos[t] / a.B : 0;  // complete blocks [0, bt)
    sh_bt[tid] = bt;
    atomicMax(&sh_nb, bt);
  }
  __syncthreads();
  const int nb = __builtin_amdgcn_readfirstlane(sh_nb);

  // A fragments: row tile rt of this wave = (query qi, 32-head tile ht)
  bf16x8 qa[RT][8];
  int qi_[RT], bt_[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ti = wave * RT + rt, qi = ti / HT, ht = ti % HT;
    const int t = qt0 + qi, j = ht * 32 + l32;
    qi_[rt] = qi;
    bt_[rt] = sh_bt[qi];
    const bool ok = t < a.T && j < a.H;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *(const uint4 *)(a.q + ((size_t)t * a.H + j) * kD + s * 16 + g * 8);
      qa[rt][s] = as_bf16x8(v);
    }
  }

  // staging: chunk c = tid + NT * i of a tile = (block row c / 16, 8-float
  // slice c % 16 of d)
  auto fetch = [&](int tile, float (&x)[CH][8]) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + NT * i, br = c >> 4, dc = c & 15;
      const int b = min(tile * 32 + br, a.Mmax - 1);  // rows past nb are masked below
      const float4 x0 = *(const float4 *)(pbase + (size_t)b * kD + dc * 8);
      const float4 x1 = *(const float4 *)(pbase + (size_t)b * kD + dc * 8 + 4);
      x[i][0] = x0.x; x[i][1] = x0.y; x[i][2] = x0.z; x[i][3] = x0.w;
      x[i][4] = x1.x; x[i][5] = x1.y; x[i][6] = x1.z; x[i][7] = x1.w;
    }
  };
  auto stage = [&](int buf, int row, int dc, const float (&x)[8]) {
    u16x8 hi, mi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t h16, m16, l16;
      split3(x[e], h16, m16, l16);
      hi[e] = h16;
      mi[e] = m16;
      lo[e] = l16;
    }
    char *base = (char *)tiles[buf] + row * kRtRowLds + dc * 16;
    *(u16x8 *)(base) = hi;
    *(u16x8 *)(base + PLANE) = mi;
    *(u16x8 *)(base + 2 * PLANE) = lo;
  };

  float rs[RT][16];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) rs[rt][r] = 0.f;
  const f32x16 zero = {};
  // one 32-block tile: 24 MFMAs per row tile (8 d-steps x 3 planes), then
  // ReLU into the running sums of the columns on for each query
  auto consume = [&](int buf, int bbase, bool tail) {
    const char *base = (const char *)tiles[buf] + l32 * kRtRowLds + g * 16;
    f32x16 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = zero;
    // B fragments one d-step ahead of the MFMAs that use them (each feeds
    // both row tiles)
    uint4 bv[2][3];
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) bv[0][pl] = *(const uint4 *)(base + pl * PLANE);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) {
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
          bv[(s + 1) & 1][pl] = *(const uint4 *)(base + pl * PLANE + (s + 1) * 32);
      }
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rt][s], as_bf16x8(bv[s & 1][pl]), acc[rt],
                                                            0, 0, 0);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bool on = tail ? l32 == qi_[rt] : bbase + l32 < bt_[rt];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        rs[rt][r] += on ? __int_as_float(max(__float_as_int(acc[rt][r]), 0)) : 0.f;
    }
  };

  // The tail means accumulate inside the tile loop: per iteration each
  // thread loads four of its query's tail keys with the pooled fetch and adds
  // them after the MFMAs.  thread = (query tq, key lane tkl of 2, 8-dim
  // slice tdc); loads are clamped into the prefix and added only when in it.
  static_assert(NT / 32 >= QWG, "one 32-thread group per query");
  const int tq = tid >> 5, tkl = (tid >> 4) & 1, tdc = tid & 15;
  const bool tval = tq < QWG && qt0 + tq < a.T;
  const int tp = tval ? a.q_pos[qt0 + tq] : -1;
  const int tlo = tval ? (tp / a.B) * a.B : 0;
  const uint16_t *tkb = a.keys + (size_t)sq * a.Lmax * kD + tdc * 8;
  float tacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int tnext = tlo + tkl;  // this thread's next tail key
  uint4 tv[4];
  auto tail_load = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) tv[u] = *(const uint4 *)(tkb + (size_t)min(tnext + 2 * u, max(tp, 0)) * kD);
  };
  auto tail_add = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (tnext + 2 * u <= tp) {
        const uint32_t w4[4] = {tv[u].x, tv[u].y, tv[u].z, tv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tacc[2 * e] += __uint_as_float(w4[e] << 16);
          tacc[2 * e + 1] += __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      }
    }
    tnext += 8;
  };

  const int ntile = (nb + 31) / 32;
  float x[CH][8];
  auto stage_all = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + NT * i;
      stage(buf, c >> 4, c & 15, x[i]);
    }
  };
  if (ntile > 0) {
    fetch(0, x);
    stage_all(0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntile; ++tile) {
    // the next tile is fetched and staged unconditionally (the last
    // iteration re-reads a clamped tile into the buffer the tail tile then
    // overwrites): a conditional fetch would leave the compiler unable to
    // count the loads in flight, and it would wait for them before the MFMAs
    const int buf = tile & 1;
    fetch(min(tile + 1, ntile - 1), x);
    tail_load();
    // keep the order: loads out first, the staging (which waits for them)
    // after every MFMA of this tile
    __builtin_amdgcn_sched_barrier(0);
    consume(buf, tile * 32, false);
    __builtin_amdgcn_sched_barrier(0);
    tail_add();
    stage_all(buf ^ 1);
    __syncthreads();
  }

  // the rest of the tail keys (short prefixes, large blocks), then the
  // tail tile: query tq's mean of its own last block [bt*B, p] in row tq
  while (tnext <= tp) {
    tail_load();
    tail_add();
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    tacc[e] += __shfl_xor(tacc[e], 16, kWave);
    tacc[e] = tval ? tacc[e] / (float)(tp - tlo + 1) : 0.f;
  }
  if (tkl == 0 && tq < QWG) stage(ntile & 1, tq, tdc, tacc);
  __syncthreads();
  consume(ntile & 1, 0, true);

  // reduce each row's sum over the 32 column lanes, then per query: weight,
  // rank by (g desc, head id asc), write the first h
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ht = (wave * RT + rt) % HT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = row_sum16(rs[rt][r]);
      v += __shfl_xor(v, 16, kWave);
      if (l32 == 0) gsum[qi_[rt]][ht * 32 + 8 * (r >> 2) + 4 * g + (r & 3)] = v;
    }
  }
  __syncthreads();
  for (int qi = wave; qi < QWG; qi += NW) {
    const int t = qt0 + qi;
    if (t >= a.T) break;
    float gj = 0.f;
    const int j = lane;
    if (j < a.H) {
      float wj = a.w[(size_t)t * a.H + j];
      if (a.mode == 1) wj = fabsf(wj);
      gj = wj * gsum[qi][j];
      if (a.g) a.g[(size_t)t * a.H + j] = gj;
    }
    // the wave's 64 lanes hold every head (H <= 64): ranks from LDS
    __builtin_amdgcn_wave_barrier();
    if (j < a.H) gsum[qi][j] = gj;
    __builtin_amdgcn_wave_barrier();
    if (j < a.H) {
      int rank = 0;
      for (int i = 0; i < a.H; ++i) {
        const float gi = gsum[qi][i];
        rank += (gi > gj || (gi == gj && i < j)) ? 1 : 0;
      }
      if (rank < a.h) a.heads[(size_t)t * a.h + rank] = j;
    }
  }
}

constexpr int kRtWaves = 4;  // two workgroups per CU: one stages while the other multiplies

hipError_t launch_route_tile(const RouteArgs &a, hipStream_t st) {
  constexpr int q1 = kRtWaves * 2, q2 = kRtWaves;  // queries per workgroup
  if (a.H <= 32) {
    hipLaunchKernelGGL((route_tile_kernel<1, kRtWaves>), dim3((a.T + q1 - 1) / q1), dim3(kRtWaves * 64),
                       0, st, a);
  } else if (a.H <= 64) {
    hipLaunchKernelGGL((route_tile_kernel<2, kRtWaves>), dim3((a.T + q2 - 1) / q2), dim3(kRtWaves * 64),
                       0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HT>
static void launch_partial(const RouteArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((route_partial_kernel<HT>), dim3(a.nchunks + 1, a.T), dim3(256), 0, st, a);
}

hipError_t launch_route_partial(const RouteArgs &a, hipStream_t st) {
  if (a.H <= 16) launch_partial<1>(a, st);
  else if (a.H <= 32) launch_partial<2>(a, st);
  else if (a.H <= 64) launch_partial<4>(a, st);
  else launch_partial<8>(a, st);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  hipError_t e = launch_route_partial(a, st);
  if (e != hipSuccess) return e;
  if (a.tiles && (!a.tcount || a.tqwg < 1 || a.tbound < 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_final_kernel, dim3(a.T + (a.tiles ? 1 : 0)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
