// score.hip -- indexer token scoring on MFMA (decode and rerank paths).
//
// Computes, for query row t and column c of its score row,
//   s(c) = sum_{j in heads_t} w[t][j] * max(0, q[t][j] . K[token(c)])
// ("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
// Inference", Technical Summary, Methodology: MISA -- Sparse Token Scoring;
// with all H heads it is the DSA indexer of the Problem Statement, and over a
// candidate list it is the Fine Stage of the Hierarchical Variant).
//
// The head-token products are a dense contraction over d = 128, so they run
// on v_mfma_f32_16x16x32_bf16: A = the query's (gathered) head rows, padded to
// 16-row tiles and held in registers for the whole workgroup; B = 16 keys per
// MFMA column tile.  Keys are streamed from HBM exactly once with coalesced
// non-temporal 16-byte loads (a wave instruction covers four whole 256-byte
// keys, 1 KiB contiguous), then passed through a per-wave LDS tile whose rows
// are padded to 272 bytes, so the MFMA-layout reads (lane = key column,
// lane group = 8-element slice of d) hit 16 distinct bank groups.  The
// weighted ReLU and the head reduction run on the accumulators in registers
// (four rows per lane), then a reduce-scatter across the four lane groups
// leaves each group the whole sums of one tile, so a wave stores the scores
// of 32 consecutive columns at once.  The scores of the workgroup's chunk
// collect in LDS and leave in one burst of 16-byte stores at the end: score
// stores spread through the key stream cost more HBM time than their bytes.
// For the top-k of few long rows the epilogue also keeps the chunk's
// candidate list: a 4096-bin LDS histogram of the top 12 bits of each
// score's order key gives the cutoff digit of the chunk's share of the row's
// top k, and the entries at or above it are written out (select.hpp).
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"
#include "route_finish.hpp"
#include "select.hpp"

namespace misa {

constexpr int kKeyRowLds = 272;  // bytes per key row in the LDS tile (256 + 16)
// Waves per workgroup: eight where one 16-row head tile keeps a wave within
// 128 registers (two workgroups, sixteen waves, per CU: more key loads in
// flight), and for direct rows of four tiles (64 heads: 200 registers, two
// waves per SIMD, about 256 workgroups of 4096 keys -- 46.6 -> 46.0 us at
// 32 x 32768 keys); four otherwise.  (RLIST launches of four tiles keep
// four: eight would spill there.)
template <int HT, bool GATHER, bool RLIST = false>
constexpr int score_waves() {
  return !GATHER && (HT == 1 || (HT == 4 && !RLIST)) ? 8 : 4;
}

// One (chunk, row) of the scoring: the body of score_rows_kernel.
template <int HT, bool GATHER, bool ROUTE, int U, int NW>
__device__ __forceinline__ void score_row_chunk(const ScoreArgs &a, const int t) {
  constexpr int NT = NW * 64;
  static_assert(!(ROUTE && GATHER), "the router prologue serves direct rows");
  __shared__ alignas(16) uint32_t lds_hist[kHistBins];
  __shared__ float rred[ROUTE ? 4 : 1][MISA_MAX_HEADS_DEV];  // router prologue scratch
  __shared__ float rgs[ROUTE ? MISA_MAX_HEADS_DEV : 1];
  __shared__ int32_t rheads[ROUTE ? MISA_MAX_HEADS_DEV : 1];  // the routed heads
  __shared__ uint4 tile[NW][16 * kKeyRowLds / 16];
  __shared__ int32_t ctok[GATHER ? kMaxScoreChunk : 1];  // the chunk's candidate tokens
  __shared__ float csc[kMaxScoreChunk];                   // the chunk's scores
  __shared__ uint32_t lsh[2 * NW + 9];                    // scan scratch; [2 NW + 8] valid-entry count
  const int lane = lane_id();
  // wave-uniform, and known to be: the step loop below branches on scalars
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // MFMA column (key) / 16-byte slice of a key row
  const int grp = lane >> 4;   // lane group: k sub-slice / accumulator rows / key of a load
  const bool lists = a.lists != nullptr;

  const int c0 = blockIdx.x * a.chunk;
  const int c1 = min(c0 + a.chunk, a.ncols);
  // Valid columns: the causal prefix 0..p_t for direct rows; every slot
  // holding a token id for gathered (candidate) rows.
  const int nvalid = GATHER ? a.ncols : min(a.ncols, a.q_pos[t] + 1);
  float *srow = a.scores + (size_t)t * a.ld;

  if (lists) {
    for (int b = threadIdx.x; b < kHistBins; b += NT) lds_hist[b] = 0;
    if (threadIdx.x == 0) lsh[2 * NW + 8] = 0;
    if (GATHER) __syncthreads();  // the count is zero before the candidate loop adds to it
  }
  if (!GATHER && c0 >= nvalid) {  // uniform across the workgroup: no barrier follows
    for (int c = c0 + threadIdx.x; c < c1; c += NT) srow[c] = -INFINITY;
    if (lists && threadIdx.x == 0) a.lhead[(size_t)t * gridDim.x + blockIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }

  const size_t seq_base = (size_t)a.q_seq[t] * a.Lmax;
  // Direct rows request their first step's keys (those of load_step below)
  // before the router prologue and the query loads, so that the stream is
  // under way while the heads are ranked and loaded.
  uint4 ka[U][4];
  if constexpr (!GATHER) {
    const int cw = c0 + wave * 16 * U + grp;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ka[u][i] = load_nt16(a.keys + (seq_base + (size_t)min(cw + u * 16 + 4 * i, c1 - 1)) * kD + col * 8);
  }
  if constexpr (ROUTE) {  // the router's last step: reduce the partials, rank the heads
    route_finish(a.partial + (size_t)t * a.nparts * a.H, a.nparts, a.H, a.w + (size_t)t * a.H, a.mode,
                 a.nh, rred, rgs, (blockIdx.x == 0 && a.g_out) ? a.g_out + (size_t)t * a.H : nullptr,
                 blockIdx.x == 0 ? a.heads_out + (size_t)t * a.nh : nullptr, rheads);
    __syncthreads();
  }

  // Query head fragments (A operand) and the weights of this lane's rows:
  // two batched rounds of loads (head ids, then rows and weights), indices
  // clamped and rows past nh masked, so that no load waits behind a branch
  bf16x8 qa[HT][4];
  float wv[HT][4];
  {
    int jq[HT], jw[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int m = min(ht * 16 + col, a.nh - 1);
      jq[ht] = ROUTE ? rheads[m] : a.heads ? a.heads[(size_t)t * a.nh + m] : m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mr = min(ht * 16 + grp * 4 + r, a.nh - 1);
        jw[ht][r] = ROUTE ? rheads[mr] : a.heads ? a.heads[(size_t)t * a.nh + mr] : mr;
      }
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint32_t mq = ht * 16 + col < a.nh ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 v = *(const uint4 *)(a.q + ((size_t)t * a.H + jq[ht]) * kD + s * 32 + grp * 8);
        qa[ht][s] = as_bf16x8(make_uint4(v.x & mq, v.y & mq, v.z & mq, v.w & mq));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t wb = __float_as_uint(a.w[(size_t)t * a.H + jw[ht][r]]);
        wv[ht][r] = __uint_as_float(wb & (ht * 16 + grp * 4 + r < a.nh ? 0xFFFFFFFFu : 0u));
      }
    }
  }
  if (GATHER) {
    if (a.kept) {  // the tokens of the kept blocks, also written out for the select
      const int32_t *krow = a.kept + (size_t)t * a.nkept;
      int32_t *orow = a.cand_out + (size_t)t * a.ncols;
      const int p = a.q_pos[t];
      uint32_t nv = 0;
      for (int c = c0 + threadIdx.x; c < c1; c += NT) {
        const int i = c / a.blk, b = krow[i], tok = b * a.blk + (c - i * a.blk);
        const int v = (b >= 0 && tok <= p) ? tok : -1;
        ctok[c - c0] = v;
        orow[c] = v;
        nv += v >= 0 ? 1u : 0u;
      }
      if (lists && nv) atomicAdd(&lsh[2 * NW + 8], nv);
    } else {
      const int32_t *crow = a.cand + (size_t)t * a.ncols;
      uint32_t nv = 0;
      for (int c = c0 + threadIdx.x; c < c1; c += NT) {
        const int v = crow[c];
        ctok[c - c0] = v;
        nv += v >= 0 ? 1u : 0u;
      }
      if (lists && nv) atomicAdd(&lsh[2 * NW + 8], nv);
    }
  }
  if (lists || GATHER) __syncthreads();
  char *wt = (char *)tile[wave];
  // U tiles of 16 keys per step; load i of tile u covers keys 4i..4i+3
  // Every load is issued unconditionally, from a column clamped into
  // [c0, c1) (and token 0 for an empty candidate slot): a load under a
  // branch leaves the compiler unable to count the loads in flight, and it
  // then waits for all of them -- the next step's included -- before each
  // step.  The epilogue masks the columns that are not valid.
  auto load_step = [&](int base, uint4 (&kv)[U][4]) {
    int tok[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = min(base + u * 16 + 4 * i + grp, c1 - 1);
        tok[u][i] = GATHER ? max(ctok[c - c0], 0) : c;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kv[u][i] = load_nt16(a.keys + (seq_base + (size_t)tok[u][i]) * kD + col * 8);
  };
  const int stride = NW * 16 * U;
  const int wstart = c0 + wave * 16 * U;
  const int nsteps = wstart < c1 ? (c1 - wstart + stride - 1) / stride : 0;
  uint4 kb2[U][4];

  auto process_step = [&](int base, const uint4 (&kv)[U][4]) {
    float part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // transpose through LDS: row = key within the tile, 16-byte slices
#pragma unroll
      for (int i = 0; i < 4; ++i) *(uint4 *)(wt + (4 * i + grp) * kKeyRowLds + col * 16) = kv[u][i];
      uint4 kb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kb[s] = *(const uint4 *)(wt + col * kKeyRowLds + (4 * s + grp) * 16);
      part[u] = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(qa[ht][s], as_bf16x8(kb[s]), acc);
        // ReLU as a signed-integer max of the bits (-0 and negatives -> +0)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          part[u] += wv[ht][r] * __int_as_float(max(__float_as_int(acc[r]), 0));
      }
    }
    // reduce-scatter over the four lane groups (each holds four head rows):
    // afterwards groups 0 and 1 hold the whole sum of tile 0, groups 2 and 3
    // that of tile 1, so one LDS store covers 32 consecutive columns
    static_assert(U == 2, "two tiles per step");
    const bool lo = grp < 2;
    float own = (lo ? part[0] : part[1]) + __shfl_xor(lo ? part[1] : part[0], 32, kWave);
    own += __shfl_xor(own, 16, kWave);
    const int c = base + (grp >> 1) * 16 + col;
    if ((grp & 1) == 0 && c < c1) {
      const bool ok = c < nvalid && (!GATHER || ctok[c - c0] >= 0);
      const float sc = ok ? own : -INFINITY;
      csc[c - c0] = sc;
      if (lists && ok) atomicAdd(&lds_hist[order_key(sc) >> kHistShift], 1u);
    }
  };
  // software pipeline over two register buffers: the next step's loads are
  // in flight while the current step is transposed, contracted and stored.
  // Every path that goes on has issued the next step's loads (the last
  // steps leave the loop), so the compiler waits only for the step it
  // processes.
  if (nsteps > 0) {
    if constexpr (GATHER) load_step(wstart, ka);
    for (int st = 0;; st += 2) {
      const int b0 = wstart + st * stride;
      if (st + 1 >= nsteps) {
        process_step(b0, ka);
        break;
      }
      load_step(b0 + stride, kb2);
      process_step(b0, ka);
      if (st + 2 >= nsteps) {
        process_step(b0 + stride, kb2);
        break;
      }
      load_step(b0 + 2 * stride, ka);
      process_step(b0 + stride, kb2);
    }
  }
  __syncthreads();
  if (lists) {  // the chunk's share of the row's top k, for the merge (before the
    // score stores: work after them would wait for the stores to land)
    const uint32_t nvc = GATHER ? lsh[2 * NW + 8] : (uint32_t)max(0, min(c1, nvalid) - c0);
    const uint32_t quota = chunk_quota(a.k, (int)nvc, nvalid);
    const uint32_t cap = min((uint32_t)a.lcap, 2u * quota + 64u);
    const size_t slot = (size_t)t * gridDim.x + blockIdx.x;
    chunk_list<NT, kMaxScoreChunk / NT>(
        csc, c1 - c0, lds_hist, nvc, quota, cap,
        [&](int i) { return GATHER ? ctok[i] >= 0 : c0 + i < nvalid; },
        [&](int i) { return GATHER ? ctok[i] : c0 + i; }, a.lists + slot * a.lcap, a.lhead + slot, lsh);
  }
  // the chunk's scores, in 16-byte non-temporal stores where aligned
  {
    const int n = c1 - c0;
    if ((n & 3) == 0 && (((size_t)t * a.ld + c0) & 3) == 0) {
      for (int i = threadIdx.x * 4; i < n; i += 4 * NT) {
        const float4 v = *(const float4 *)&csc[i];
        __builtin_nontemporal_store((f32x4){v.x, v.y, v.z, v.w}, (f32x4 *)(srow + c0 + i));
      }
    } else {
      for (int i = threadIdx.x; i < n; i += NT) srow[c0 + i] = csc[i];
    }
  }
}

// Grid (chunks, rows): workgroup (x, y) scores chunk x of row y -- or, with
// a row count (RLIST), of rows rowlist[y], rowlist[y + gridDim.y], ...
// (rows y, y + gridDim.y, ... without a list) below *rowcount, one after
// another.
template <int HT, bool GATHER, bool ROUTE, int U, int NW, bool RLIST>
__global__ __launch_bounds__(NW * 64) void score_rows_kernel(ScoreArgs a) {
  if constexpr (RLIST) {
    const uint32_t nrows = *a.rowcount;
    for (uint32_t y = blockIdx.y; y < nrows; y += gridDim.y) {
      score_row_chunk<HT, GATHER, ROUTE, U, NW>(a, a.rowlist ? a.rowlist[y] : (int)y);
      __syncthreads();  // the next row reuses the shared memory
    }
  } else {
    score_row_chunk<HT, GATHER, ROUTE, U, NW>(a, (int)blockIdx.y);
  }
}

// workgroup rows of a row-list launch (each walks its share of the list)
constexpr int kRowListGrid = 64;

template <int HT, bool GATHER, bool ROUTE>
static hipError_t launch_ht(const ScoreArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.rowcount) {  // (at most 64 heads: rows a prefill or grouped call hands back)
    if constexpr (HT <= 4 && !GATHER && !ROUTE) {
      if (!a.rowcount || ev0 || ev1 || a.chunk > kMaxScoreChunk) return hipErrorInvalidValue;
      constexpr int U = 2, NW = score_waves<HT, false, true>();
      const dim3 grid((a.ncols + a.chunk - 1) / a.chunk, a.T < kRowListGrid ? a.T : kRowListGrid);
      hipLaunchKernelGGL((score_rows_kernel<HT, false, false, U, NW, true>), grid, dim3(NW * 64), 0, st, a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  dim3 grid((a.ncols + a.chunk - 1) / a.chunk, a.T);
  // two 16-key tiles per wave step: fewer registers, more waves per CU
  constexpr int U = 2;
  constexpr int NW = score_waves<HT, GATHER>();
  if (a.chunk > kMaxScoreChunk) return hipErrorInvalidValue;
  if (ev0 || ev1)  // the measurement hook: events stamped with the kernel's begin and end
    hipExtLaunchKernelGGL((score_rows_kernel<HT, GATHER, ROUTE, U, NW, false>), grid, dim3(NW * 64), 0, st, ev0,
                          ev1, 0, a);
  else
    hipLaunchKernelGGL((score_rows_kernel<HT, GATHER, ROUTE, U, NW, false>), grid, dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <bool GATHER, bool ROUTE>
static hipError_t launch_g(const ScoreArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.nh <= 16) return launch_ht<1, GATHER, ROUTE>(a, st, ev0, ev1);
  if (a.nh <= 32) return launch_ht<2, GATHER, ROUTE>(a, st, ev0, ev1);
  if (a.nh <= 64) return launch_ht<4, GATHER, ROUTE>(a, st, ev0, ev1);
  return launch_ht<8, GATHER, ROUTE>(a, st, ev0, ev1);
}

hipError_t launch_score_rows(const ScoreArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.T <= 0 || a.ncols <= 0) {  // nothing to launch: the events mark the empty interval
    if (ev0 && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
    if (ev1 && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
    return hipSuccess;
  }
  if (a.partial) {  // the fused indexer call: the router's last step in the prologue
    if (a.cand || a.kept || !a.heads_out || a.nh > a.H) return hipErrorInvalidValue;
    return launch_g<false, true>(a, st, ev0, ev1);
  }
  return (a.cand || a.kept) ? launch_g<true, false>(a, st, ev0, ev1) : launch_g<false, false>(a, st, ev0, ev1);
}

}  // namespace misa
