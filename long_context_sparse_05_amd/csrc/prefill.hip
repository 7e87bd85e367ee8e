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
// accumulator r, query g*(16/HP) + r/HP and head slot r%HP, so the weighted
// ReLU head reduction is a register-local sum.  A workgroup (8 waves, two
// per SIMD) owns QWG consecutive queries, whose A fragments stay in
// registers, and one split of the key range, which streams through LDS in
// tiles of 128 keys:
//
//  * key tiles are copied from global memory straight into LDS by buffer
//    loads with the LDS bit (no registers, no ds_write), two tiles ahead of
//    use, into two buffers; chunk c (16 bytes) of key row r lands in slot
//    r*16 + (c ^ (r & 15)), so a B-fragment read (one chunk of 32 rows)
//    touches every bank once;
//  * within a wave, each B fragment is re-read for the next 32-key column
//    block right after its two MFMAs, a whole block ahead of use, and the
//    previous block's epilogue (ReLU, weights, head sums, stores) is split
//    into eight slices issued beside the eight MFMA pairs;
//  * one barrier per tile, before its last block: every wave then holds the
//    tile's fragments and its own copy of the next tile has landed (an
//    explicit vmcnt wait that leaves the score stores issued since in
//    flight), so the buffer may be refilled.
//
// Measured on MI355X with random bf16 data the matrix pipe is power-bound
// well below its nominal rate, so the epilogue's vector work and the score
// stores, not the LDS feed, set the remaining gap.
#include <climits>
#include <type_traits>

#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace misa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt bits
// [3:0] and [15:14]; expcnt and lgkmcnt at their maxima, i.e. not waited on)
#define PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

enum { kEpiNone = 0, kEpiFull = 1, kEpiCausal = 2, kEpiGeneric = 3 };
template <int E> using epi_t = std::integral_constant<int, E>;

// GEN = false: every row of the workgroup is a query and its key split is a
// whole number of tiles (the host launches only such workgroups here);
// GEN = true: ragged workgroups, every store checked.  qtile0 / split0 offset
// the grid into the workgroup space.
template <int HP, int RT, int NW, int KT, bool GEN>
__global__ __launch_bounds__(NW * 64) void score_prefill_kernel(PrefillArgs a, int qtile0, int split0) {
  constexpr int QPT = 32 / HP;                  // queries per 32-row tile
  constexpr int QPL = 16 / HP;                  // queries per lane (per tile)
  constexpr int QWG = NW * RT * QPT;            // queries per workgroup
  constexpr int NT = NW * 64;
  constexpr int NB = KT / 32;                   // 32-key column blocks per tile
  constexpr int NDMA = KT / (4 * NW);           // 16-byte DMA loads per thread per tile
  constexpr int TB = KT * 256;                  // bytes per key tile
  constexpr int OUT = RT * QPL;                 // score stores per lane per column block
  static_assert(NDMA * 4 * NW == KT && NW % 4 == 0 && NB == 4, "tile shape");
  // the two key-tile buffers are separate arrays so that the compiler can
  // tell reads of one from DMA writes into the other
  __shared__ uint4 ktile0[TB / 16], ktile1[TB / 16];
  __shared__ int sh_pmax, sh_pmin;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int qt0 = (blockIdx.y + qtile0) * QWG;
  const int k0 = (blockIdx.x + split0) * a.split;
  const int k1 = min(k0 + a.split, a.Lmax);

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
  const int kend = __builtin_amdgcn_readfirstlane(min(k1, sh_pmax + 1));
  const bool all_rows = qt0 + QWG <= a.T;
  const int kfull = __builtin_amdgcn_readfirstlane(all_rows ? min(k1, sh_pmin + 1) : 0);

  bf16x8 qa[RT][8];
  float wv[RT][16];
  char *const wg_rows = (char *)(a.scores + (size_t)qt0 * a.ld);
  uint32_t rowo[RT][QPL];
  int lim[RT][QPL];   // position - l32: key kb + l32 is in the prefix iff kb <= lim
  bool rowok[RT][QPL];
  // The lane's rows: A row l32 of tile rt is (query tA, head slot sA); its
  // accumulator rows r are (query tile_q0 + g*QPL + r/HP, slot r%HP).  Every
  // index is clamped so that all loads of a round are issued together (two
  // dependent rounds: head ids and positions, then query rows and weights).
  const int Tm = a.T - 1, hm = a.h - 1;
  int jq[RT], jw[RT][16], pos[RT][QPL];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tile_q0 = qt0 + (wave * RT + rt) * QPT;
    const int gg = (l32 >> 2) & 1, rr = ((l32 >> 3) << 2) | (l32 & 3);
    const int tA = tile_q0 + gg * QPL + rr / HP, sA = rr % HP;
    jq[rt] = a.heads[(size_t)min(tA, Tm) * a.h + min(sA, hm)];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      jw[rt][r] = a.heads[(size_t)min(tile_q0 + g * QPL + r / HP, Tm) * a.h + min(r % HP, hm)];
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) pos[rt][qq] = a.q_pos[min(tile_q0 + g * QPL + qq, Tm)];
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tile_q0 = qt0 + (wave * RT + rt) * QPT;
    const int gg = (l32 >> 2) & 1, rr = ((l32 >> 3) << 2) | (l32 & 3);
    const int tA = tile_q0 + gg * QPL + rr / HP, sA = rr % HP;
    // (rows past T or past h are zeroed with a mask, not a select: a select
    // of a loaded value may be turned into a branch around the load)
    const uint32_t mA = (tA < a.T && sA < a.h) ? 0xFFFFFFFFu : 0u;
    const uint16_t *qrow = a.q + ((size_t)min(tA, Tm) * a.H + jq[rt]) * kD + g * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 v = *(const uint4 *)(qrow + s * 16);
      qa[rt][s] = as_bf16x8(make_uint4(v.x & mA, v.y & mA, v.z & mA, v.w & mA));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tile_q0 + g * QPL + r / HP, slot = r % HP;
      const uint32_t wb = __float_as_uint(a.w[(size_t)min(t, Tm) * a.H + jw[rt][r]]);
      wv[rt][r] = __uint_as_float(wb & ((t < a.T && slot < a.h) ? 0xFFFFFFFFu : 0u));
    }
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      const int t = tile_q0 + g * QPL + qq;
      rowo[rt][qq] = (uint32_t)(((t - qt0) * a.ld + l32) * 4);
      rowok[rt][qq] = t < a.T;
      lim[rt][qq] = t < a.T ? pos[rt][qq] - l32 : INT_MIN;
    }
  }

  // Key tiles go straight from global memory into LDS (buffer loads with the
  // LDS-DMA bit): each wave instruction writes 64 consecutive 16-byte slots,
  // four key rows.  Chunk c of key row r sits in slot r*16 + (c ^ (r & 15)),
  // so the 32 rows one B-fragment read touches spread over all banks.  The
  // buffer's record limit is the tile's key range below kend: slots of keys
  // past it read as zero (their scores are masked).
  const int rr = 4 * wave + (lane >> 4);
  const uint32_t dvoff = (uint32_t)(rr * 256 + (((lane & 15) ^ (rr & 15)) * 16));
  const char *kseq = (const char *)(a.keys + (size_t)a.seq * a.Lmax * kD);
  auto buf_of = [&](auto b) -> char * {
    if constexpr (decltype(b)::value == 0) return (char *)ktile0; else return (char *)ktile1;
  };
  const int ntile = kend > k0 ? (kend - k0 + KT - 1) / KT : 0;
  const int nfull = kfull > k0 ? min(ntile, (kfull - k0) / KT) : 0;
  auto dma_tile = [&](int it, auto buf) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      // rows [kr, kr + 4 NW) of the tile, through a buffer of the keys from kr on
      const int kr = k0 + it * KT + 4 * NW * i;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(kseq + (size_t)kr * 256), (short)0, max(kend - kr, 0) * 256, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void *)(buf_of(buf) + (NW * i + wave) * 1024), 16, dvoff, 0, 0, 0);
    }
  };
  // B-fragment read addresses: lane (l32, g) of step s reads chunk 2s + g of
  // key row cb*32 + l32; the column block and buffer come in as offsets
  uint32_t raddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) raddr[s] = (uint32_t)(l32 * 256 + (((2 * s + g) ^ (l32 & 15)) * 16));

  // the workgroup's score rows (at most QWG rows of ld floats: 32-bit offsets)
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void *)wg_rows, (short)0, (int)((uint32_t)QWG * a.ld * 4u), 0x00020000);
  const f32x16 zero = {};
  f32x16 acc[2][RT];
  uint4 bfr[8];
  float sc[OUT];

  // one 32-key column block: the MFMA chain of `cur` from bfr, each fragment
  // replaced right after its MFMAs by the same fragment of the next block
  // (NEXT_CB: that block's index in the buffer raddr points at), and the
  // previous block's epilogue (head sums of `prev`, then stores at key base
  // kbp) spread over the eight steps so the vector ALU runs beside the MFMAs
  auto block = [&](f32x16 (&cur)[RT], const f32x16 (&prev)[RT], auto next_buf, auto next_cb, int kbp, auto epi) {
    constexpr int NEXT = decltype(next_cb)::value;
    const char *const nb = buf_of(next_buf);
    constexpr int EPI = decltype(epi)::value;

#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) cur[rt] = mfma32(qa[rt][s], as_bf16x8(bfr[s]), s ? cur[rt] : zero);
      bfr[s] = *(const uint4 *)(nb + raddr[s] + NEXT * 32 * 256);
      if (EPI != kEpiNone) {
#pragma unroll
        for (int v = s * 2 * RT; v < (s + 1) * 2 * RT; ++v) {
          const int rt = v / 16, r = v % 16, o = v / HP, hs = v % HP;
          const float x = __int_as_float(max(__float_as_int(prev[rt][r]), 0));
          sc[o] = hs == 0 ? wv[rt][r] * x : fmaf(wv[rt][r], x, sc[o]);
          if (hs == HP - 1) {
            const int ort = o / QPL, oq = o % QPL;
            if (EPI == kEpiFull) {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc[o]), srs, rowo[ort][oq], kbp * 4, 0);
            } else if (EPI == kEpiCausal) {
              const float y = kbp <= lim[ort][oq] ? sc[o] : -INFINITY;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), srs, rowo[ort][oq], kbp * 4, 0);
            } else if (rowok[ort][oq] && kbp + l32 < k1) {
              *(float *)(wg_rows + (size_t)kbp * 4 + rowo[ort][oq]) = kbp <= lim[ort][oq] ? sc[o] : -INFINITY;
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Tile `it` lives in buffer it % 2.  Its blocks 0..NB-2 run on fragments
  // read during the previous block.  Before the last block: this wave's DMA
  // of tile it+1 has landed (the stores issued after it are not waited for)
  // and every wave holds its fragments of tile it, so after the barrier the
  // DMA of tile it+2 may overwrite buffer it % 2 and the last block reads
  // tile it+1's first fragments.
  auto tile = [&](int it, auto prev_epi, auto cur_epi, auto buf) {
    constexpr int PE = decltype(prev_epi)::value, CE = decltype(cur_epi)::value, B = decltype(buf)::value;
    using cur_b = std::integral_constant<int, B>;
    using nxt_b = std::integral_constant<int, B ^ 1>;
    const int kt = k0 + it * KT;
    block(acc[0], acc[1], cur_b{}, std::integral_constant<int, 1>{}, kt - 32, prev_epi);
    block(acc[1], acc[0], cur_b{}, std::integral_constant<int, 2>{}, kt, cur_epi);
    block(acc[0], acc[1], cur_b{}, std::integral_constant<int, 3>{}, kt + 32, cur_epi);
    if (PE == kEpiGeneric || CE == kEpiGeneric) {
      PF_WAIT_VM(0);
    } else if (PE == kEpiNone) {
      PF_WAIT_VM((NB - 2) * OUT < 63 ? (NB - 2) * OUT : 63);
    } else {
      PF_WAIT_VM(NB * OUT < 63 ? NB * OUT : 63);
    }
    __syncthreads();
    if (it + 2 < ntile) dma_tile(it + 2, cur_b{});
    block(acc[1], acc[0], nxt_b{}, std::integral_constant<int, 0>{}, kt + 64, cur_epi);
  };
  if (ntile > 0) {
    dma_tile(0, std::integral_constant<int, 0>{});
    if (ntile > 1) {
      dma_tile(1, std::integral_constant<int, 1>{});
      PF_WAIT_VM(NDMA);
    } else {
      PF_WAIT_VM(0);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) bfr[s] = *(const uint4 *)((const char *)ktile0 + raddr[s]);
    // tile it sits in buffer it % 2: after tile 0, tiles go in (odd, even)
    // pairs so that every call names its buffer at compile time
    constexpr int E = GEN ? kEpiGeneric : kEpiCausal;
    using b0 = std::integral_constant<int, 0>;
    using b1 = std::integral_constant<int, 1>;
    tile(0, epi_t<kEpiNone>{}, epi_t<E>{}, b0{});
    int it = 1;
    // tiles [0, nfull) lie below every query's position; a pair takes the
    // unmasked epilogue when both of its tiles do (block 0 of a tile holds the
    // previous tile's last epilogue: below nfull too, or masked, which is
    // always right)
    if (!GEN) {
      for (; it + 1 < nfull; it += 2) {
        tile(it, epi_t<kEpiFull>{}, epi_t<kEpiFull>{}, b1{});
        tile(it + 1, epi_t<kEpiFull>{}, epi_t<kEpiFull>{}, b0{});
      }
    }
    for (; it + 1 < ntile; it += 2) {
      tile(it, epi_t<E>{}, epi_t<E>{}, b1{});
      tile(it + 1, epi_t<E>{}, epi_t<E>{}, b0{});
    }
    if (it < ntile) tile(it, epi_t<E>{}, epi_t<E>{}, b1{});
    // the last block's epilogue (its MFMAs ran in the final tile's last block)
    const int kbp = k0 + ntile * KT - 32;
    f32x16 dummy[RT];
    block(dummy, acc[1], b0{}, std::integral_constant<int, 0>{}, kbp, epi_t<E>{});
  }
  // columns of this split past every query of the workgroup
  const int cstart = min(k1, k0 + ntile * KT);
  for (int qi = 0; qi < QWG; ++qi) {
    const int t = qt0 + qi;
    if (t >= a.T) break;
    for (int c = cstart + tid; c < k1; c += NT) a.scores[(size_t)t * a.ld + c] = -INFINITY;
  }
}

constexpr int kPfWaves = 8, kPfKeys = kPrefillKeyTile;
constexpr int pf_rt(int hp) { return hp >= 4 ? 2 : 1; }

template <int HP>
static hipError_t launch_hp(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int RT = pf_rt(HP);
  constexpr int QWG = kPfWaves * RT * (32 / HP);
  if (a.split % kPfKeys) return hipErrorInvalidValue;
  if ((uint64_t)QWG * a.ld * 4 > 0x7FFFFFFFull) return hipErrorInvalidValue;
  if ((uint64_t)a.Lmax * 256 > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const int nsplit = (a.Lmax + a.split - 1) / a.split, nqt = (a.T + QWG - 1) / QWG;
  // whole workgroups: every row a query, every split a whole number of tiles
  const int nq_full = a.T / QWG;
  const int ns_full = (a.Lmax % kPfKeys == 0) ? nsplit : nsplit - 1;
  const bool l0 = nq_full > 0 && ns_full > 0, l1 = nq_full < nqt, l2 = ns_full < nsplit && nq_full > 0;
  // the start event goes with the first launch issued, the stop event with the last
  const int first = l0 ? 0 : l1 ? 1 : l2 ? 2 : -1, last = l2 ? 2 : l1 ? 1 : l0 ? 0 : -1;
  auto e0 = [&](int i) { return i == first ? ev0 : nullptr; };
  auto e1 = [&](int i) { return i == last ? ev1 : nullptr; };
  // plain launches unless the measurement hook asks for events
  auto launch = [&](int i, auto kernel, dim3 grid, int qtile0, int split0) {
    if (e0(i) || e1(i))
      hipExtLaunchKernelGGL(kernel, grid, dim3(kPfWaves * 64), 0, st, e0(i), e1(i), 0, a, qtile0, split0);
    else
      hipLaunchKernelGGL(kernel, grid, dim3(kPfWaves * 64), 0, st, a, qtile0, split0);
  };
  if (l0) launch(0, score_prefill_kernel<HP, RT, kPfWaves, kPfKeys, false>, dim3(ns_full, nq_full), 0, 0);
  if (l1)  // the ragged last row of query tiles, all splits
    launch(1, score_prefill_kernel<HP, RT, kPfWaves, kPfKeys, true>, dim3(nsplit, 1), nq_full, 0);
  if (l2)  // the ragged last split, whole query tiles
    launch(2, score_prefill_kernel<HP, RT, kPfWaves, kPfKeys, true>, dim3(1, nq_full), 0, ns_full);
  if (first < 0) {  // nothing to launch: the events mark the empty interval
    if (ev0 && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
    if (ev1 && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int prefill_queries_per_wg(int h) {
  const int hp = h <= 1 ? 1 : h <= 2 ? 2 : h <= 4 ? 4 : h <= 8 ? 8 : 16;
  return kPfWaves * pf_rt(hp) * (32 / hp);
}

bool prefill_supported(int h, int ld, int Lmax) {
  return h >= 1 && h <= 16 && ld >= Lmax && (uint64_t)prefill_queries_per_wg(h) * ld * 4 <= 0x7FFFFFFFull &&
         (uint64_t)Lmax * 256 <= 0x7FFFFFFFull;
}

hipError_t launch_score_prefill(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.h <= 1) return launch_hp<1>(a, st, ev0, ev1);
  if (a.h <= 2) return launch_hp<2>(a, st, ev0, ev1);
  if (a.h <= 4) return launch_hp<4>(a, st, ev0, ev1);
  if (a.h <= 8) return launch_hp<8>(a, st, ev0, ev1);
  if (a.h <= 16) return launch_hp<16>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

}  // namespace misa
