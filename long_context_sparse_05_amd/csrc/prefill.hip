// prefill.hip -- routed token scoring for a chunk of many queries of one
// sequence (a prefill chunk), as a dense MFMA contraction.
//
// s(t, i) = sum_{j in heads_t} w[t][j] * max(0, q[t][j] . K[i]),  i <= p_t
// ("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
// Inference", Technical Summary, Methodology: MISA -- Sparse Token Scoring).
//
// When many queries share the key sequence, the gathered (query, routed
// head) rows form the A operand of v_mfma_f32_32x32x16_bf16 and the keys the
// B operand.  The 32 rows of a tile are laid out so that each lane's 16
// accumulator rows are whole head sets of its queries: with HP = h rounded
// up to a power of two (HP <= 16), lane group g of the 32x32 tile holds, in
// accumulator r, query g*(16/HP) + r/HP and head slot r%HP.  The weighted
// ReLU head reduction is therefore a register-local sum, with no cross-lane
// traffic.  A workgroup owns QWG consecutive queries x one split of the key
// range; keys stream through a double-buffered LDS tile of 64 keys (rows
// padded to 272 bytes), loaded with coalesced 16-byte loads one tile ahead.
// Key tiles beyond the workgroup's last query position are skipped
// (causality); columns past a query's position are written as -inf.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kPfKeys = 64;       // keys per LDS tile
constexpr int kPfRowLds = 272;    // bytes per key row in LDS (256 + 16)
constexpr int kPfWaves = 4;

template <int HP, int RT>
__global__ __launch_bounds__(kPfWaves * 64) void score_prefill_kernel(PrefillArgs a) {
  constexpr int QPT = 32 / HP;                  // queries per 32-row tile
  constexpr int QPL = 16 / HP;                  // queries per lane (per tile)
  constexpr int QWG = kPfWaves * RT * QPT;      // queries per workgroup
  __shared__ uint4 ktile[2][kPfKeys * kPfRowLds / 16];
  __shared__ int sh_pmax;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int qt0 = blockIdx.y * QWG;
  const int k0 = blockIdx.x * a.split;
  const int k1 = min(k0 + a.split, a.Lmax);

  // last position of the workgroup's queries: keys past it are never needed
  if (tid == 0) sh_pmax = -1;
  __syncthreads();
  if (tid < QWG && qt0 + tid < a.T) atomicMax(&sh_pmax, a.q_pos[qt0 + tid]);
  __syncthreads();
  const int kend = min(k1, sh_pmax + 1);

  // A fragments: row l32 of tile rt holds (query, head slot) of the layout above
  bf16x8 qa[RT][8];
  float wv[RT][16];
  int tq[RT][QPL];   // this lane's queries (row ids), -1 when past T
  int pq[RT][QPL];   // their positions
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tile_q0 = qt0 + (wave * RT + rt) * QPT;
    {
      const int gg = (l32 >> 2) & 1, rr = ((l32 >> 3) << 2) | (l32 & 3);
      const int t = tile_q0 + gg * QPL + rr / HP, slot = rr % HP;
      int j = -1;
      if (t < a.T && slot < a.h) j = a.heads[(size_t)t * a.h + slot];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j >= 0) v = *(const uint4 *)(a.q + ((size_t)t * a.H + j) * kD + s * 16 + g * 8);
        qa[rt][s] = as_bf16x8(v);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tile_q0 + g * QPL + r / HP, slot = r % HP;
      float wr = 0.f;
      if (t < a.T && slot < a.h) wr = a.w[(size_t)t * a.H + a.heads[(size_t)t * a.h + slot]];
      wv[rt][r] = wr;
    }
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      const int t = tile_q0 + g * QPL + qq;
      tq[rt][qq] = t < a.T ? t : -1;
      pq[rt][qq] = t < a.T ? a.q_pos[t] : -1;
    }
  }

  // coalesced tile load: thread = (key lane tid/16, 16-byte slice tid%16), 4 rounds
  const uint16_t *kseq = a.keys + (size_t)a.seq * a.Lmax * kD;
  auto load_tile = [&](int kt, uint4 (&kr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt + 16 * i + (tid >> 4);
      kr[i] = key < kend ? load_nt16(kseq + (size_t)key * kD + (tid & 15) * 8)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 kr[4];
  if (k0 < kend) load_tile(k0, kr);
  int buf = 0;
  for (int kt = k0; kt < kend; kt += kPfKeys, buf ^= 1) {
    char *lt = (char *)ktile[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint4 *)(lt + (16 * i + (tid >> 4)) * kPfRowLds + (tid & 15) * 16) = kr[i];
    __syncthreads();
    if (kt + kPfKeys < kend) load_tile(kt + kPfKeys, kr);  // in flight during the MFMAs
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 bv = *(const uint4 *)(lt + (half * 32 + l32) * kPfRowLds + s * 32 + g * 16);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32(qa[rt][s], as_bf16x8(bv), acc[rt]);
      }
      const int key = kt + half * 32 + l32;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int qq = 0; qq < QPL; ++qq) {
          float sc = 0.f;
#pragma unroll
          for (int hs = 0; hs < HP; ++hs) sc += wv[rt][qq * HP + hs] * fmaxf(acc[rt][qq * HP + hs], 0.f);
          const int t = tq[rt][qq];
          if (t >= 0 && key < k1) a.scores[(size_t)t * a.ld + key] = key <= pq[rt][qq] ? sc : -INFINITY;
        }
      }
    }
  }
  // columns of this split past every query of the workgroup
  for (int qi = 0; qi < QWG; ++qi) {
    const int t = qt0 + qi;
    if (t >= a.T) break;
    for (int c = max(kend, k0) + tid; c < k1; c += kPfWaves * 64) a.scores[(size_t)t * a.ld + c] = -INFINITY;
  }
}

template <int HP>
static hipError_t launch_hp(const PrefillArgs &a, hipStream_t st) {
  constexpr int RT = 2;
  constexpr int QWG = kPfWaves * RT * (32 / HP);
  dim3 grid((a.Lmax + a.split - 1) / a.split, (a.T + QWG - 1) / QWG);
  hipLaunchKernelGGL((score_prefill_kernel<HP, RT>), grid, dim3(kPfWaves * 64), 0, st, a);
  return hipGetLastError();
}

int prefill_queries_per_wg(int h) {
  const int hp = h <= 1 ? 1 : h <= 2 ? 2 : h <= 4 ? 4 : h <= 8 ? 8 : 16;
  return kPfWaves * 2 * (32 / hp);
}

hipError_t launch_score_prefill(const PrefillArgs &a, hipStream_t st) {
  if (a.h <= 1) return launch_hp<1>(a, st);
  if (a.h <= 2) return launch_hp<2>(a, st);
  if (a.h <= 4) return launch_hp<4>(a, st);
  if (a.h <= 8) return launch_hp<8>(a, st);
  if (a.h <= 16) return launch_hp<16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace misa
