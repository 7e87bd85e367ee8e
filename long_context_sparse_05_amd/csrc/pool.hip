// pool.hip -- block mean-pool of the indexing keys.
//
// The router summarises the prefix with M = ceil(L/B) mean-pooled indexing
// keys ("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
// Inference", Technical Summary, Methodology: MISA -- Lightweight
// Block-Pooled Router).  pooled[s][b] = mean of keys[s][i] over the keys
// present in [bB, bB+B); a block with none is zeros.
//
// misa_pool_append reuses the kernel for a streaming key cache: after keys
// are appended only the blocks that now hold them change, so the cost per
// decode step is O(B d) instead of a pass over the cache (the router's
// per-query cost is then O(H_I M) with no pooling pass).
//
// One wave per block: each lane loads 16 bytes (8 bf16) of one of 4
// consecutive keys per step, so a wave streams 1 KiB contiguous per load
// (non-temporal: the keys are read once here, and plain loads stream at
// about half the rate on this part);
// fp32 partial sums are combined across the 4 lane groups with two xor
// shuffles and the 16 lanes of the first group store the 512-byte row.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace misa {

// With old_lens (an append), block b of sequence s counts from
// floor(old_lens[s] / B), and blocks with no key present are left alone:
// only the blocks that hold an appended key are recomputed.
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t *keys, const int32_t *seq_lens,
                                                   const int32_t *old_lens, int Lmax, int B,
                                                   int Mmax, float *pooled) {
  const int s = blockIdx.y;
  const int b = (old_lens ? old_lens[s] / B : 0) + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= Mmax) return;  // wave-uniform; no barrier in this kernel
  const int lane = lane_id();
  const int g = lane >> 4, cc = lane & 15;
  const int lo = b * B;
  const int hi = min(lo + B, min(seq_lens[s], Lmax));
  if (old_lens && lo >= hi) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t *base = keys + (size_t)s * Lmax * kD + cc * 8;
  int i = lo + g;
  for (; i + 12 < hi; i += 16) {  // four keys per lane in flight
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load_nt16(base + (size_t)(i + 4 * u) * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(x[e] << 16);
        acc[2 * e + 1] += __uint_as_float(x[e] & 0xFFFF0000u);
      }
    }
  }
  for (; i < hi; i += 4) {
    const uint4 v = load_nt16(base + (size_t)i * kD);
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(x[e] << 16);
      acc[2 * e + 1] += __uint_as_float(x[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 16, kWave);
    acc[e] += __shfl_xor(acc[e], 32, kWave);
  }
  if (g == 0) {
    const int cnt = hi - lo;
    float4 o0, o1;
    if (cnt > 0) {
      const float fc = (float)cnt;
      o0 = make_float4(acc[0] / fc, acc[1] / fc, acc[2] / fc, acc[3] / fc);
      o1 = make_float4(acc[4] / fc, acc[5] / fc, acc[6] / fc, acc[7] / fc);
    } else {
      o0 = o1 = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float *dst = pooled + ((size_t)s * Mmax + b) * kD + cc * 8;
    *(float4 *)dst = o0;
    *(float4 *)(dst + 4) = o1;
  }
}

hipError_t launch_pool(const uint16_t *keys, const int32_t *seq_lens, int S, int Lmax, int B,
                       float *pooled, hipStream_t st) {
  const int Mmax = (Lmax + B - 1) / B;
  dim3 grid((Mmax + 3) / 4, S);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(256), 0, st, keys, seq_lens, nullptr, Lmax, B, Mmax,
                     pooled);
  return hipGetLastError();
}

hipError_t launch_pool_append(const uint16_t *keys, const int32_t *seq_lens,
                              const int32_t *old_lens, int max_new, int S, int Lmax, int B,
                              float *pooled, hipStream_t st) {
  const int Mmax = (Lmax + B - 1) / B;
  // appending n keys touches at most ceil(n / B) + 1 blocks of a sequence
  const int nb = std::min(Mmax, (max_new + B - 1) / B + 1);
  dim3 grid((nb + 3) / 4, S);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(256), 0, st, keys, seq_lens, old_lens, Lmax, B, Mmax,
                     pooled);
  return hipGetLastError();
}

}  // namespace misa
