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
// range; keys stream through a double-buffered LDS tile of 128 keys (rows
// padded to 272 bytes), loaded with coalesced 16-byte loads one tile ahead.
// Within a tile each wave pipelines its 32-key column blocks: the MFMA chain
// of the next block is issued before the epilogue of the previous one.
// Key tiles beyond the workgroup's last query position are skipped
// (causality); columns past a query's position are written as -inf.  The
// epilogue is kept lean because on CDNA every wave64 VALU op costs four
// cycles against 32 for one 32x32x16 MFMA: the first MFMA of each chain
// takes a zero accumulator, store addresses are per-row pointers set up
// once, and tiles below every query's position store without a mask.
#include <climits>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace misa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kPfRowLds = 272;    // bytes per key row in LDS (256 + 16)

template <int HP, int RT, int NW, int KT>
__global__ __launch_bounds__(NW * 64) void score_prefill_kernel(PrefillArgs a) {
  constexpr int QPT = 32 / HP;                  // queries per 32-row tile
  constexpr int QPL = 16 / HP;                  // queries per lane (per tile)
  constexpr int QWG = NW * RT * QPT;            // queries per workgroup
  constexpr int NT = NW * 64;
  constexpr int LPT = KT * 16 / NT;             // 16-byte key loads per thread per tile
  static_assert(LPT * NT == KT * 16, "tile load split");
  __shared__ uint4 ktile[2][KT * kPfRowLds / 16];
  __shared__ int sh_pmax, sh_pmin;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int qt0 = blockIdx.y * QWG;
  const int k0 = blockIdx.x * a.split;
  const int k1 = min(k0 + a.split, a.Lmax);

  // positions of the workgroup's queries: keys past the last one are never
  // needed; tiles below the first one need no causal mask
  if (tid == 0) {
    sh_pmax = -1;
    sh_pmin = 0x7FFFFFFF;
  }
  __syncthreads();
  if (tid < QWG && qt0 + tid < a.T) {
    const int p = a.q_pos[qt0 + tid];
    atomicMax(&sh_pmax, p);
    atomicMin(&sh_pmin, p);
  }
  __syncthreads();
  // (read back through readfirstlane: the tile loops below branch on scalars)
  const int kend = __builtin_amdgcn_readfirstlane(min(k1, sh_pmax + 1));
  const bool all_rows = qt0 + QWG <= a.T;
  const int kfull = __builtin_amdgcn_readfirstlane(all_rows ? min(k1, sh_pmin + 1) : 0);

  // A fragments: row l32 of tile rt holds (query, head slot) of the layout above
  bf16x8 qa[RT][8];
  float wv[RT][16];
  // this lane's query rows of the score matrix, as byte offsets from the
  // workgroup's first row (at most QWG rows of ld floats: 32 bits suffice),
  // and their positions (INT_MIN past T: nothing is stored for such rows)
  char *const wg_rows = (char *)(a.scores + (size_t)qt0 * a.ld);
  uint32_t rowo[RT][QPL];
  int pq[RT][QPL];
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
      rowo[rt][qq] = (uint32_t)(((t - qt0) * a.ld + l32) * 4);
      pq[rt][qq] = t < a.T ? a.q_pos[t] : INT_MIN;
    }
  }

  // coalesced tile load: thread = (key lane tid/16, 16-byte slice tid%16).
  // Every load is issued, from a key clamped below kend (the epilogue masks
  // those keys), and the next tile is always prefetched (the last one again
  // at the end): loads under branches leave the compiler unable to count the
  // memory operations in flight, and it then waits for all of them -- the
  // previous tile's score stores included -- before each tile.
  const uint16_t *kseq = a.keys + (size_t)a.seq * a.Lmax * kD;
  auto load_tile = [&](int kt, uint4 (&kr)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = min(kt + (NT / 16) * i + (tid >> 4), kend - 1);
      kr[i] = load_nt16(kseq + (size_t)key * kD + (tid & 15) * 8);
    }
  };
  const f32x16 zero = {};
  uint4 kr[LPT];
  const int ntile = kend > k0 ? (kend - k0 + KT - 1) / KT : 0;
  // tiles [0, nfull) lie below every query's position: no mask
  const int nfull = kfull > k0 ? min(ntile, (kfull - k0) / KT) : 0;
  if (ntile > 0) load_tile(k0, kr);
  int buf = 0;
  auto run_tile = [&](int it, auto full_tag) {
    const int kt = k0 + it * KT;
    char *lt = (char *)ktile[buf];
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      *(uint4 *)(lt + ((NT / 16) * i + (tid >> 4)) * kPfRowLds + (tid & 15) * 16) = kr[i];
    __syncthreads();
    load_tile(k0 + min(it + 1, ntile - 1) * KT, kr);  // in flight during the MFMAs
    // software pipeline over the tile's 32-key column blocks: the MFMA chain
    // of block c+1 is issued before the epilogue of block c, so the vector
    // ALU work overlaps the matrix core.  Tiles below every query's position
    // (FULL) take a straight-line body with unmasked stores.
    {
      constexpr bool FULL = decltype(full_tag)::value;
      auto chain = [&](int cb, f32x16 (&acc)[RT]) {
        const char *kr0 = lt + (cb * 32 + l32) * kPfRowLds + g * 16;
        // the block's eight B fragments are read before its MFMAs issue
        uint4 bvs[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) bvs[s] = *(const uint4 *)(kr0 + s * 32);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32(qa[rt][0], as_bf16x8(bvs[0]), zero);
#pragma unroll
        for (int s = 1; s < 8; ++s)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32(qa[rt][s], as_bf16x8(bvs[s]), acc[rt]);
      };
      auto epilogue = [&](int cb, const f32x16 (&acc)[RT]) {
        const int kb = kt + cb * 32;  // this lane's key is kb + l32
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int qq = 0; qq < QPL; ++qq) {
            // ReLU as a signed-integer max of the bits: negative floats
            // (and -0) have the sign bit set, so they become +0
            float sc = wv[rt][qq * HP] * __int_as_float(max(__float_as_int(acc[rt][qq * HP]), 0));
#pragma unroll
            for (int hs = 1; hs < HP; ++hs)
              sc += wv[rt][qq * HP + hs] * __int_as_float(max(__float_as_int(acc[rt][qq * HP + hs]), 0));
            float *dst = (float *)(wg_rows + (size_t)kb * 4 + rowo[rt][qq]);
            if (FULL) {
              *dst = sc;
            } else if (pq[rt][qq] != INT_MIN && kb + l32 < k1) {
              *dst = kb + l32 <= pq[rt][qq] ? sc : -INFINITY;
            }
          }
        }
      };
      f32x16 acc0[RT], acc1[RT];
      chain(0, acc0);
#pragma unroll
      for (int cb = 1; cb < KT / 32; ++cb) {
        if (cb & 1) {
          chain(cb, acc1);
          epilogue(cb - 1, acc0);
        } else {
          chain(cb, acc0);
          epilogue(cb - 1, acc1);
        }
      }
      if ((KT / 32) & 1) epilogue(KT / 32 - 1, acc0); else epilogue(KT / 32 - 1, acc1);
    }
    buf ^= 1;
  };
  // The first full tile is peeled: the loop is then entered, like its back
  // edge, with one tile's loads and then its 16 score stores in flight, so
  // the wait at its top is for the loads alone.
  if (nfull > 0) run_tile(0, std::true_type{});
  for (int it = 1; it < nfull; ++it) run_tile(it, std::true_type{});
  for (int it = nfull; it < ntile; ++it) run_tile(it, std::false_type{});
  // columns of this split past every query of the workgroup
  for (int qi = 0; qi < QWG; ++qi) {
    const int t = qt0 + qi;
    if (t >= a.T) break;
    for (int c = max(kend, k0) + tid; c < k1; c += NT) a.scores[(size_t)t * a.ld + c] = -INFINITY;
  }
}

constexpr int kPfWaves = 8, kPfKeys = kPrefillKeyTile;
// row tiles per wave: two where a lane's rows are few whole head sets; one
// where a lane holds many queries (HP <= 2), whose row pointers would not
// fit in registers beside two pipelined accumulator sets
constexpr int pf_rt(int hp) { return hp >= 4 ? 2 : 1; }

template <int HP>
static hipError_t launch_hp(const PrefillArgs &a, hipStream_t st) {
  constexpr int RT = pf_rt(HP);
  constexpr int QWG = kPfWaves * RT * (32 / HP);
  if (a.split % kPfKeys) return hipErrorInvalidValue;
  if ((uint64_t)QWG * a.ld * 4 > 0xFFFFFFFFull) return hipErrorInvalidValue;  // 32-bit row offsets
  dim3 grid((a.Lmax + a.split - 1) / a.split, (a.T + QWG - 1) / QWG);
  hipLaunchKernelGGL((score_prefill_kernel<HP, RT, kPfWaves, kPfKeys>), grid,
                     dim3(kPfWaves * 64), 0, st, a);
  return hipGetLastError();
}

bool prefill_supported(int h, int ld) {
  return h >= 1 && h <= 16 && (uint64_t)prefill_queries_per_wg(h) * ld * 4 <= 0xFFFFFFFFull;
}

int prefill_queries_per_wg(int h) {
  const int hp = h <= 1 ? 1 : h <= 2 ? 2 : h <= 4 ? 4 : h <= 8 ? 8 : 16;
  return kPfWaves * pf_rt(hp) * (32 / hp);
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
