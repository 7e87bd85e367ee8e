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
// MFMA column tile, loaded straight from HBM into registers (each lane loads
// 16 contiguous bytes of one key, so a wave reads 16 whole 256-byte keys in
// four instructions).  Keys are read exactly once.  The weighted ReLU and the
// head reduction run on the accumulators in registers (four rows per lane,
// then two cross-lane adds).  The epilogue also builds a 4096-bin histogram
// of the top 12 bits of each score's order key, the first radix digit of the
// per-row top-k, so the selection needs no extra pass over the scores.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {

template <int HT, bool GATHER, int U>
__global__ __launch_bounds__(256) void score_rows_kernel(ScoreArgs a) {
  __shared__ uint32_t lds_hist[kHistBins];
  const int t = blockIdx.y;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;   // MFMA column (key) within a 16-key tile
  const int grp = lane >> 4;   // lane group: k sub-slice / accumulator rows
  const bool hist = a.hist != nullptr;

  const int c0 = blockIdx.x * a.chunk;
  const int c1 = min(c0 + a.chunk, a.ncols);
  // Valid columns: the causal prefix 0..p_t for direct rows; every slot
  // holding a token id for gathered (candidate) rows.
  const int nvalid = GATHER ? a.ncols : min(a.ncols, a.q_pos[t] + 1);
  float *srow = a.scores + (size_t)t * a.ld;

  if (hist) {
    for (int b = threadIdx.x; b < kHistBins; b += 256) lds_hist[b] = 0;
  }
  if (!GATHER && c0 >= nvalid) {
    for (int c = c0 + threadIdx.x; c < c1; c += 256) srow[c] = -INFINITY;
    return;  // uniform across the workgroup: no barrier follows for it
  }

  // Query head fragments (A operand) and the weights of this lane's rows.
  const size_t seq_base = (size_t)a.q_seq[t] * a.Lmax;
  bf16x8 qa[HT][4];
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int m = ht * 16 + col;
    int j = -1;
    if (m < a.nh) j = a.heads ? a.heads[(size_t)t * a.nh + m] : m;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j >= 0)
        v = *(const uint4 *)(a.q + ((size_t)t * a.H + j) * kD + s * 32 + grp * 8);
      qa[ht][s] = as_bf16x8(v);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mr = ht * 16 + grp * 4 + r;
      float wr = 0.f;
      if (mr < a.nh) {
        const int jr = a.heads ? a.heads[(size_t)t * a.nh + mr] : mr;
        wr = a.w[(size_t)t * a.H + jr];
      }
      wv[ht][r] = wr;
    }
  }
  if (hist) __syncthreads();

  const int32_t *crow = GATHER ? a.cand + (size_t)t * a.ncols : nullptr;
  for (int base = c0 + wave * 16 * U; base < c1; base += 4 * 16 * U) {
    uint4 kv[U][4];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * 16 + col;
      int tok = -1;
      if (c < c1 && c < nvalid) tok = GATHER ? crow[c] : c;
      ok[u] = tok >= 0;
      const uint16_t *kp = a.keys + (seq_base + (size_t)(tok >= 0 ? tok : 0)) * kD + grp * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kv[u][s] = ok[u] ? *(const uint4 *)(kp + s * 32) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(qa[ht][s], as_bf16x8(kv[u][s]), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) part += wv[ht][r] * fmaxf(acc[r], 0.f);
      }
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      const int c = base + u * 16 + col;
      if (grp == 0 && c < c1) {
        const float sc = ok[u] ? part : -INFINITY;
        srow[c] = sc;
        if (hist && ok[u]) atomicAdd(&lds_hist[order_key(sc) >> kHistShift], 1u);
      }
    }
  }
  if (hist) {
    __syncthreads();
    uint32_t *grow = a.hist + (size_t)t * kHistBins;
    for (int b = threadIdx.x; b < kHistBins; b += 256) {
      const uint32_t v = lds_hist[b];
      if (v) atomicAdd(&grow[b], v);
    }
  }
}

template <int HT, bool GATHER>
static hipError_t launch_ht(const ScoreArgs &a, hipStream_t st) {
  dim3 grid((a.ncols + a.chunk - 1) / a.chunk, a.T);
  hipLaunchKernelGGL((score_rows_kernel<HT, GATHER, 4>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool GATHER>
static hipError_t launch_g(const ScoreArgs &a, hipStream_t st) {
  if (a.nh <= 16) return launch_ht<1, GATHER>(a, st);
  if (a.nh <= 32) return launch_ht<2, GATHER>(a, st);
  if (a.nh <= 64) return launch_ht<4, GATHER>(a, st);
  return launch_ht<8, GATHER>(a, st);
}

hipError_t launch_score_rows(const ScoreArgs &a, hipStream_t st) {
  if (a.T <= 0 || a.ncols <= 0) return hipSuccess;
  return a.cand ? launch_g<true>(a, st) : launch_g<false>(a, st);
}

}  // namespace misa
