// topk.hip -- per-row top-k by (score desc, token id asc), as a radix select.
//
// The indexer keeps the k best-scoring prefix tokens of each query ("MISA:
// Mixture of Indexer Sparse Attention for Long-Context LLM Inference",
// Technical Summary, Problem Statement; the selected set is shared by all
// heads, MISA abstract).  Every valid column is given the 64-bit composite
// key (order_key(score) << 32) | ~token: keys are unique and their order is
// exactly the ranking, so the top-k is "every key >= the k-th largest key".
//
//  1. histogram of the top 12 bits (fused into the scoring epilogue, or
//     topk_hist_kernel for caller-provided scores);
//  2. topk_filter_kernel (many workgroups per row): every workgroup finds the
//     digit b1 holding the k-th key from the 4096-bin histogram; columns
//     above b1 are written straight to the output (wave-aggregated atomics),
//     columns equal to b1 are appended to a per-row candidate list;
//  3. topk_finish_kernel (one workgroup per row): the candidates are loaded
//     into LDS (up to 16384 of them; beyond that they are re-read from the
//     score row) and the remaining 52 key bits are resolved with 8-bit digit
//     passes over LDS histograms, emitting every key above each pass's
//     crossing digit, until the crossing bin holds exactly what is needed.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {

constexpr int kFinishCap = 16384;  // candidates resolved in LDS (128 KiB)

struct Thresh {
  int b1;          // first digit holding the kk-th key
  uint32_t above;  // keys with first digit > b1
  uint32_t eq;     // keys with first digit == b1
  uint32_t kk;     // min(k, number of valid columns)
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide inclusive scan of one value per thread (256 threads, 4 waves).
__device__ __forceinline__ uint32_t block_scan256(uint32_t v, uint32_t *sh4, uint32_t &total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) sh4[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = sh4[i];
    if (i < wave) base += x;
    total += x;
  }
  __syncthreads();
  return base + incl;
}

// Threshold digit of one row from its 4096-bin histogram (256 threads).
// Thread tid owns 16 consecutive bins, counted from the top.
__device__ Thresh row_threshold(const uint32_t *hrow, uint32_t k, uint32_t *sh) {
  const int tid = threadIdx.x;
  const int top = kHistBins - 1 - 16 * tid;
  uint32_t v[16];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = hrow[top - i];
    s += v[i];
  }
  uint32_t total;
  const uint32_t incl = block_scan256(s, sh, total);
  const uint32_t excl = incl - s;
  const uint32_t kk = min(k, total);
  if (kk > 0 && excl < kk && kk <= incl) {
    uint32_t cum = excl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (cum + v[i] >= kk) {
        sh[4] = (uint32_t)(top - i);
        sh[5] = cum;
        sh[6] = v[i];
        break;
      }
      cum += v[i];
    }
  }
  __syncthreads();
  Thresh th;
  th.kk = kk;
  th.b1 = kk ? (int)sh[4] : kHistBins;
  th.above = kk ? sh[5] : 0;
  th.eq = kk ? sh[6] : 0;
  __syncthreads();
  return th;
}

__device__ __forceinline__ int row_valid_len(const TopkArgs &a, int r) {
  return a.row_len ? max(0, min(a.ld, a.row_len[r] + a.row_len_add)) : a.ld;
}

// ---------------------------------------------------------------- histogram
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a, uint32_t *hist) {
  __shared__ uint32_t h[kHistBins];
  const int r = blockIdx.y;
  for (int b = threadIdx.x; b < kHistBins; b += 256) h[b] = 0;
  __syncthreads();
  const int n = row_valid_len(a, r);
  const int c0 = blockIdx.x * a.chunk, c1 = min(c0 + a.chunk, n);
  const float *srow = a.scores + (size_t)r * a.ld;
  for (int c = c0 + threadIdx.x; c < c1; c += 256) {
    if (a.map && a.map[(size_t)r * a.ld + c] < 0) continue;
    atomicAdd(&h[order_key(srow[c]) >> kHistShift], 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kHistBins; b += 256)
    if (h[b]) atomicAdd(&hist[(size_t)r * kHistBins + b], h[b]);
}

// ------------------------------------------------------------------- filter
template <bool MAP>
__global__ __launch_bounds__(256) void topk_filter_kernel(TopkArgs a) {
  __shared__ uint32_t sh[8];
  const int r = blockIdx.y;
  const Thresh th = row_threshold(a.hist + (size_t)r * kHistBins, (uint32_t)a.k, sh);
  if (th.kk == 0) return;
  const int n = row_valid_len(a, r);
  const int c0 = blockIdx.x * a.chunk, c1 = min(c0 + a.chunk, n);
  const bool keep = th.eq <= (uint32_t)a.cap;
  const int lane = lane_id();
  uint32_t *cnt = a.counters + (size_t)r * 4;
  const float *srow = a.scores + (size_t)r * a.ld;
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;
  uint2 *crow = a.cand + (size_t)r * a.cap;
  for (int cb = c0; cb < c1; cb += 256) {  // same trip count for every lane
    const int c = cb + threadIdx.x;
    bool valid = c < c1;
    int tok = c;
    if (MAP && valid) {
      tok = a.map[(size_t)r * a.ld + c];
      valid = tok >= 0;
    }
    const float s = valid ? srow[c] : 0.f;
    const uint32_t key = order_key(s);
    const int dg = (int)(key >> kHistShift);
    const bool sel = valid && dg > th.b1;
    const bool cnd = valid && keep && dg == th.b1;
    const uint64_t ms = __ballot(sel);
    if (ms) {
      const int leader = __ffsll((unsigned long long)ms) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&cnt[0], (uint32_t)__popcll(ms));
      base = __shfl(base, leader, kWave);
      if (sel) {
        const uint32_t pos = base + lanes_below(ms);
        if (pos < th.above) {
          irow[pos] = tok;
          if (vrow) vrow[pos] = s;
        }
      }
    }
    const uint64_t mc = __ballot(cnd);
    if (mc) {
      const int leader = __ffsll((unsigned long long)mc) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&cnt[1], (uint32_t)__popcll(mc));
      base = __shfl(base, leader, kWave);
      if (cnd) {
        const uint32_t pos = base + lanes_below(mc);
        if (pos < (uint32_t)a.cap) crow[pos] = make_uint2(key, (uint32_t)c);
      }
    }
  }
}

// ------------------------------------------------------------------- finish
template <bool MAP>
__global__ __launch_bounds__(256) void topk_finish_kernel(TopkArgs a) {
  __shared__ uint64_t cs[kFinishCap];
  __shared__ uint32_t hs[256];
  __shared__ uint32_t sh[16];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const Thresh th = row_threshold(a.hist + (size_t)r * kHistBins, (uint32_t)a.k, sh);
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;
  for (int i = (int)th.kk + tid; i < a.k; i += 256) {
    irow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
  if (th.kk == 0) return;

  const bool in_lds = th.eq <= (uint32_t)a.cap;
  const int ncand = in_lds ? (int)th.eq : 0;
  const int n = row_valid_len(a, r);
  const float *srow = a.scores + (size_t)r * a.ld;
  const int32_t *mrow = MAP ? a.map + (size_t)r * a.ld : nullptr;
  if (in_lds) {
    const uint2 *crow = a.cand + (size_t)r * a.cap;
    for (int i = tid; i < ncand; i += 256) {
      const uint2 e = crow[i];
      const int tok = MAP ? mrow[e.y] : (int)e.y;
      cs[i] = ((uint64_t)e.x << 32) | (uint32_t)(~(uint32_t)tok);
    }
  }
  if (tid == 0) sh[8] = th.above;  // next output slot
  __syncthreads();

  // Visit every candidate composite key: from LDS, or (too many candidates)
  // straight from the score row.
  auto for_each = [&](auto &&fn) {
    if (in_lds) {
      for (int i = tid; i < ncand; i += 256) fn(cs[i]);
    } else {
      for (int c = tid; c < n; c += 256) {
        int tok = c;
        if (MAP) {
          tok = mrow[c];
          if (tok < 0) continue;
        }
        fn(((uint64_t)order_key(srow[c]) << 32) | (uint32_t)(~(uint32_t)tok));
      }
    }
  };
  auto emit = [&](uint64_t ck) {
    const uint32_t pos = atomicAdd(&sh[8], 1u);
    if (pos < th.kk) {
      irow[pos] = (int32_t)(~(uint32_t)ck);
      if (vrow) vrow[pos] = key_to_float((uint32_t)(ck >> 32));
    }
  };

  uint32_t need = th.kk - th.above;
  uint64_t prefix = (uint64_t)(uint32_t)th.b1 << 52;
  uint64_t mask = 0xFFFull << 52;
  for (int pass = 0; pass < 7; ++pass) {
    const int shift = pass < 6 ? 44 - 8 * pass : 0;
    hs[tid] = 0;
    __syncthreads();
    for_each([&](uint64_t ck) {
      if ((ck & mask) == prefix) atomicAdd(&hs[(uint32_t)(ck >> shift) & 0xFFu], 1u);
    });
    __syncthreads();
    const uint32_t v = hs[255 - tid];  // thread 0 holds the largest digit
    uint32_t total;
    const uint32_t incl = block_scan256(v, sh, total);
    const uint32_t excl = incl - v;
    if (excl < need && need <= incl) {
      sh[4] = 255 - tid;
      sh[5] = excl;
      sh[6] = v;
    }
    __syncthreads();
    const uint32_t d = sh[4], above_d = sh[5], cnt_d = sh[6];
    for_each([&](uint64_t ck) {
      if ((ck & mask) == prefix && ((uint32_t)(ck >> shift) & 0xFFu) > d) emit(ck);
    });
    need -= above_d;
    prefix |= (uint64_t)d << shift;
    mask |= 0xFFull << shift;
    if (cnt_d == need || pass == 6) {
      for_each([&](uint64_t ck) {
        if ((ck & mask) == prefix) emit(ck);
      });
      break;
    }
    __syncthreads();
  }
}

// -------------------------------------------------------------------- fill
__global__ void fill_u32_kernel(uint32_t *p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const TopkArgs &a, uint32_t *hist, hipStream_t st) {
  dim3 grid((a.ld + a.chunk - 1) / a.chunk, a.rows);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(256), 0, st, a, hist);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const TopkArgs &a, hipStream_t st) {
  dim3 grid((a.ld + a.chunk - 1) / a.chunk, a.rows);
  if (a.map)
    hipLaunchKernelGGL(topk_filter_kernel<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(topk_filter_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_finish(const TopkArgs &a, hipStream_t st) {
  if (a.cap > kFinishCap) return hipErrorInvalidValue;
  if (a.map)
    hipLaunchKernelGGL(topk_finish_kernel<true>, dim3(a.rows), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(topk_finish_kernel<false>, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
