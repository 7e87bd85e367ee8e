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
// ReLU head reduction is a register-local sum.  Wider head sets (HP = 32:
// a tile per query; HP = 64: the wave's two tiles per query, e.g. every head
// of a dense DSA indexer with H_I = 64) give each lane group 16 or 32 of a
// query's slots, and the two groups' partial sums meet in one lane swap
// (v_permlane32_swap).  A workgroup (8 waves, two
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
#include "select.hpp"
#include "tiles.hpp"

namespace misa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
// LISTS: instead of the score rows, every score >= tau[row] goes to the
// row's threshold list for this key split (kernels.hpp, PrefillArgs::tau) as
// (score bits, column).  Column blocks are taken in pairs: one lane swap
// (v_permlane32_swap) trades the upper lane group of the first block's
// scores for the lower group of the second's, after which a register holds
// one row over 64 consecutive columns, so the hits' places come from one
// ballot and the row's hit count is a scalar.  A row's hits lie side by
// side after those of the earlier blocks, so its list is one contiguous run
// and a store touches one or two cache lines.  The list stores are issued
// by every lane (a lane without a hit, or past the capacity, stores out of
// the buffer's range and is dropped), so the vmcnt waits count them.  The
// row's hit count (which may pass the capacity: the list overflowed) is
// written at the end.
template <int HP, int RT, int NW, int KT, bool GEN, bool LISTS>
__global__ __launch_bounds__(NW * 64) void score_prefill_kernel(PrefillArgs a, int qtile0, int split0) {
  constexpr bool WIDE = HP > 16;                // a query's slots span both lane groups
  constexpr int QPT = WIDE ? 1 : 32 / HP;       // queries per 32-row tile (HP <= 32)
  constexpr int QPL = WIDE ? 1 : 16 / HP;       // queries per lane (per tile, HP <= 16)
  constexpr int QPW = RT * 32 / HP;             // queries per wave
  constexpr int QWG = NW * QPW;                 // queries per workgroup
  constexpr int LS = WIDE ? (HP == 32 ? 16 : 32) : HP;  // accumulator rows per lane and output
  constexpr int NT = NW * 64;
  constexpr int NB = KT / 32;                   // 32-key column blocks per tile
  constexpr int NDMA = KT / (4 * NW);           // 16-byte DMA loads per thread per tile
  constexpr int TB = KT * 256;                  // bytes per key tile
  constexpr int OUT = RT * 16 / LS;             // scores per lane per column block (one store each)
  static_assert(!WIDE || (RT == 2 && (HP == 32 || HP == 64) && !LISTS), "wide head sets");
  // stores per lane per column block that the waits count: a score row
  // store per output, or with lists 2 OUT list stores for every second block
  // (the waits come after an even number of blocks since the last DMA)
  constexpr int VMO = OUT;
  static_assert(NDMA * 4 * NW == KT && NW % 4 == 0 && NB % 2 == 0 && NB >= 4, "tile shape");
  // the two key-tile buffers are separate arrays so that the compiler can
  // tell reads of one from DMA writes into the other
  __shared__ uint4 ktile0[TB / 16], ktile1[TB / 16];
  __shared__ int sh_pmax, sh_pmin;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // the workgroup's query rows: QWG consecutive rows from qt0 of sequence
  // a.seq, or with a tile table the rows of tile blockIdx.y's sequence
  int qt0 = (blockIdx.y + qtile0) * QWG, seq = a.seq;
  if (a.tiles) {  // uniform
    if (blockIdx.y >= *a.ntiles) return;
    const int2 tl = a.tiles[blockIdx.y];
    qt0 = tl.x;
    seq = tl.y;
  }
  const int k0 = (blockIdx.x + split0) * a.split;
  const int k1 = min(k0 + a.split, a.Lmax);

  __shared__ uint8_t sh_in[QWG];  // row qt0 + i belongs to the workgroup
  __shared__ int sh_nin;
  if (tid == 0) {
    sh_pmax = -1;
    sh_pmin = 0x7FFFFFFF;
    sh_nin = 0;
  }
  __syncthreads();
  if (tid < QWG) {
    const int t = qt0 + tid;
    const bool in = t < a.T && (!a.tiles || a.q_seq[t] == seq);
    sh_in[tid] = in;
    if (in) {
      const int p = a.q_pos[t];
      atomicMax(&sh_pmax, p);
      atomicMin(&sh_pmin, p);
      atomicAdd(&sh_nin, 1);
    }
  }
  __syncthreads();
  auto row_in = [&](int t) { return sh_in[t - qt0] != 0; };  // t in [qt0, qt0 + QWG)
  const int kend = __builtin_amdgcn_readfirstlane(min(k1, sh_pmax + 1));
  const bool all_rows = sh_nin == QWG;
  const int kfull = __builtin_amdgcn_readfirstlane(all_rows ? min(k1, sh_pmin + 1) : 0);

  bf16x8 qa[RT][8];
  float wv[RT][16];
  char *const wg_rows = (char *)(a.scores + (size_t)qt0 * a.ld);
  // per output o of the lane (its query out_q(o)): score-row offset, prefix
  // limit, validity and, with lists, the cut and the hit count
  uint32_t rowo[OUT];
  int lim[OUT];       // position - l32: key kb + l32 is in the prefix iff kb <= lim
  bool rowok[OUT];
  // LISTS: per row of the wave (2 OUT of them, index 2 o + lane group),
  // its cut and its hits so far -- both uniform over the wave
  float rtau[LISTS ? 2 * OUT : 1];
  uint32_t rcnt[LISTS ? 2 * OUT : 1];
  // (query, head slot) of A row (gg, rr) of tile rt -- also of accumulator r
  // of lane group gg -- and the query of output o.  HP <= 16: tile rt holds
  // queries tile_q0 + gg*QPL + rr/HP, slot rr%HP; HP = 32: tile rt is query
  // rt of the wave, slot gg*16 + rr; HP = 64: both tiles are the wave's
  // query, slot rt*32 + gg*16 + rr.
  auto row_q = [&](int rt, int gg, int rr) {
    if constexpr (!WIDE) return qt0 + (wave * RT + rt) * QPT + gg * QPL + rr / HP;
    else return qt0 + wave * QPW + (HP == 32 ? rt : 0);
  };
  auto row_s = [&](int rt, int gg, int rr) {
    if constexpr (!WIDE) return rr % HP;
    else return (HP == 64 ? rt * 32 : 0) + gg * 16 + rr;
  };
  auto out_q = [&](int o) {
    if constexpr (!WIDE) return qt0 + (wave * RT + o / QPL) * QPT + g * QPL + o % QPL;
    else return qt0 + wave * QPW + o;
  };
  // the query of output o in lane group gg (LISTS: the row of list register 2 o + gg)
  auto out_qg = [&](int o, int gg) { return qt0 + (wave * RT + o / QPL) * QPT + gg * QPL + o % QPL; };
  // head id of slot sl of query t: the routed list, or head sl itself (dense)
  auto head_of = [&](int t, int sl) { return a.heads ? a.heads[(size_t)t * a.h + sl] : sl; };
  // Every index is clamped so that all loads of a round are issued together
  // (two dependent rounds: head ids and positions, then query rows and
  // weights).
  const int Tm = a.T - 1, hm = a.h - 1;
  int jq[RT], jw[RT][16], pos[OUT];
  const int ag = (l32 >> 2) & 1, ar = ((l32 >> 3) << 2) | (l32 & 3);  // A row l32 = (group, row)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    jq[rt] = head_of(min(row_q(rt, ag, ar), Tm), min(row_s(rt, ag, ar), hm));
#pragma unroll
    for (int r = 0; r < 16; ++r) jw[rt][r] = head_of(min(row_q(rt, g, r), Tm), min(row_s(rt, g, r), hm));
  }
#pragma unroll
  for (int o = 0; o < OUT; ++o) pos[o] = a.q_pos[min(out_q(o), Tm)];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tA = row_q(rt, ag, ar), sA = row_s(rt, ag, ar);
    // (rows past T or past h are zeroed with a mask, not a select: a select
    // of a loaded value may be turned into a branch around the load)
    const uint32_t mA = (row_in(tA) && sA < a.h) ? 0xFFFFFFFFu : 0u;
    const uint16_t *qrow = a.q + ((size_t)min(tA, Tm) * a.H + jq[rt]) * kD + g * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 v = *(const uint4 *)(qrow + s * 16);
      qa[rt][s] = as_bf16x8(make_uint4(v.x & mA, v.y & mA, v.z & mA, v.w & mA));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = row_q(rt, g, r), slot = row_s(rt, g, r);
      const uint32_t wb = __float_as_uint(a.w[(size_t)min(t, Tm) * a.H + jw[rt][r]]);
      wv[rt][r] = __uint_as_float(wb & ((row_in(t) && slot < a.h) ? 0xFFFFFFFFu : 0u));
    }
  }
#pragma unroll
  for (int o = 0; o < OUT; ++o) {
    const int t = out_q(o);
    rowo[o] = (uint32_t)(((t - qt0) * a.ld + l32) * 4);
    rowok[o] = row_in(t);
    lim[o] = rowok[o] ? pos[o] - l32 : INT_MIN;
  }
  if constexpr (LISTS) {
#pragma unroll
    for (int i = 0; i < 2 * OUT; ++i) {
      rtau[i] = a.tau[min(out_qg(i / 2, i % 2), Tm)];
      rcnt[i] = 0;
    }
  }
  // wide head sets: the lane group that stores output o (the other holds
  // the same sum after the swap)
  auto stores = [&](int o) { return !WIDE || g == (HP == 32 ? o : 0); };

  // Key tiles go straight from global memory into LDS (buffer loads with the
  // LDS-DMA bit): each wave instruction writes 64 consecutive 16-byte slots,
  // four key rows.  Chunk c of key row r sits in slot r*16 + (c ^ (r & 15)),
  // so the 32 rows one B-fragment read touches spread over all banks.  The
  // buffer's record limit is the tile's key range below kend: slots of keys
  // past it read as zero (their scores are masked).
  const int rr = 4 * wave + (lane >> 4);
  const uint32_t dvoff = (uint32_t)(rr * 256 + (((lane & 15) ^ (rr & 15)) * 16));
  const char *kseq = (const char *)(a.keys + (size_t)seq * a.Lmax * kD);
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
  // the workgroup's threshold lists for this split: rows qt0.. of
  // [split][T][tcap] entries, one buffer over the workgroup's valid rows; a
  // row's list starts at its scalar offset (which the range check counts).
  // A lane without a hit stores at an offset past the range (dropped), and
  // once a row's hits pass the capacity no lane stores: the merge leaves an
  // overflowed list unread (the row is rescored), so its contents are free.
  const int split_id = blockIdx.x + split0;
  uint2 *const wg_lists = LISTS ? a.tlists + ((size_t)split_id * a.T + qt0) * a.tcap : nullptr;
  const uint32_t lrow = LISTS ? (uint32_t)a.tcap * 8u : 0u;
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)wg_lists, (short)0, LISTS ? (int)((uint32_t)min(QWG, a.T - qt0) * lrow) : 0, 0x00020000);
  // list register i of a block pair (row out_qg(i / 2, i % 2), columns
  // x0 .. x0 + 63): its hits after the row's earlier ones
  auto list_put = [&](int i, float v, int x0) __attribute__((always_inline)) {
    const bool hit = v >= rtau[i];  // (false for the NaN of a masked column)
    const uint64_t m = __ballot(hit);
    const uint32_t nh = (uint32_t)__popcll(m);
    const bool room = rcnt[i] + nh <= (uint32_t)a.tcap;  // uniform
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint32_t voff = hit && room ? (rcnt[i] + below) * 8u : 0x80000000u;
    rcnt[i] += nh;
    const u32x2 ent = {__float_as_uint(v), (uint32_t)(x0 + lane)};
    __builtin_amdgcn_raw_buffer_store_b64(ent, lrs, voff, (int)((uint32_t)(out_qg(i / 2, i % 2) - qt0) * lrow), 0);
  };
  const f32x16 zero = {};
  f32x16 acc[2][RT];
  uint4 bfr[8];
  // the head sums of a block; with lists, [0] and [1] hold the two blocks of a pair
  float scs[LISTS ? 2 : 1][OUT];

  // one 32-key column block: the MFMA chain of `cur` from bfr, each fragment
  // replaced right after its MFMAs by the same fragment of the next block
  // (NEXT_CB: that block's index in the buffer raddr points at), and the
  // previous block's epilogue (head sums of `prev`, then stores at key base
  // kbp) spread over the eight steps so the vector ALU runs beside the MFMAs.
  // PAIR (lists): 0 for the first block of a pair, 1 for the second, whose
  // epilogue also places the pair's hits.
  // (forced inline: an outlined call would pass the accumulators through scratch)
  auto block = [&](f32x16 (&cur)[RT], const f32x16 (&prev)[RT], auto next_buf, auto next_cb, int kbp, auto epi,
                   auto pair) __attribute__((always_inline)) {
    constexpr int NEXT = decltype(next_cb)::value;
    const char *const nb = buf_of(next_buf);
    constexpr int EPI = decltype(epi)::value;
    constexpr int PAIR = LISTS ? decltype(pair)::value : 0;
    float(&sc)[OUT] = scs[PAIR];

#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) cur[rt] = mfma32(qa[rt][s], as_bf16x8(bfr[s]), s ? cur[rt] : zero);
      bfr[s] = *(const uint4 *)(nb + raddr[s] + NEXT * 32 * 256);
      if (EPI != kEpiNone) {
#pragma unroll
        for (int v = s * 2 * RT; v < (s + 1) * 2 * RT; ++v) {
          const int rt = v / 16, r = v % 16, o = v / LS, hs = v % LS;
          const float x = __int_as_float(max(__float_as_int(prev[rt][r]), 0));
          sc[o] = hs == 0 ? wv[rt][r] * x : fmaf(wv[rt][r], x, sc[o]);
          if (hs == LS - 1) {
            if constexpr (WIDE) {  // plus the other lane group's slots of the query
              const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[o]), __float_as_uint(sc[o]),
                                                               false, false);
              sc[o] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            const bool st = stores(o);
            bool in = true;  // the column is in the row's prefix (and in range)
            if (EPI == kEpiFull) {
              if (!LISTS && st)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc[o]), srs, rowo[o], kbp * 4, 0);
            } else if (EPI == kEpiCausal) {
              in = kbp <= lim[o];
              const float y = in ? sc[o] : -INFINITY;
              if (!LISTS && st) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), srs, rowo[o], kbp * 4, 0);
            } else {
              in = rowok[o] && kbp + l32 < k1 && kbp <= lim[o];
              if (!LISTS && st && rowok[o] && kbp + l32 < k1)
                *(float *)(wg_rows + (size_t)kbp * 4 + rowo[o]) = in ? sc[o] : -INFINITY;
            }
            if constexpr (LISTS) {
              if (EPI != kEpiFull && !in) sc[o] = __uint_as_float(0x7FC00000u);  // NaN: never a hit
              if constexpr (PAIR == 1) {
                // lanes 32..63 of the first block's sums trade places with
                // lanes 0..31 of the second's: [0] is then row out_qg(o, 0),
                // [1] row out_qg(o, 1), each over the pair's 64 columns
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(scs[0][o]),
                                                                 __float_as_uint(scs[1][o]), false, false);
                list_put(2 * o, __uint_as_float(sw[0]), kbp - 32);
                list_put(2 * o + 1, __uint_as_float(sw[1]), kbp - 32);
              }
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
  auto tile = [&](int it, auto prev_epi, auto cur_epi, auto buf) __attribute__((always_inline)) {
    constexpr int PE = decltype(prev_epi)::value, CE = decltype(cur_epi)::value, B = decltype(buf)::value;
    using cur_b = std::integral_constant<int, B>;
    using nxt_b = std::integral_constant<int, B ^ 1>;
    const int kt = k0 + it * KT;
    using first = std::integral_constant<int, 0>;
    using second = std::integral_constant<int, 1>;
    // block j (0 .. NB-2) of the tile runs its MFMAs on acc[j % 2] and the
    // epilogue of block j - 1 (block 0: the previous tile's last); even
    // blocks close a pair of epilogues
    block(acc[0], acc[1], cur_b{}, std::integral_constant<int, 1>{}, kt - 32, prev_epi, second{});
    auto mid = [&](auto self, auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j <= NB - 2) {
        block(acc[j & 1], acc[(j + 1) & 1], cur_b{}, std::integral_constant<int, j + 1>{}, kt + 32 * (j - 1), cur_epi,
              std::integral_constant<int, (j & 1) ? 0 : 1>{});
        self(self, std::integral_constant<int, j + 1>{});
      }
    };
    mid(mid, std::integral_constant<int, 1>{});
    if (PE == kEpiGeneric || CE == kEpiGeneric) {
      PF_WAIT_VM(0);
    } else if (PE == kEpiNone) {
      PF_WAIT_VM((NB - 2) * VMO < 63 ? (NB - 2) * VMO : 63);  // (fewer is only more conservative)
    } else {
      PF_WAIT_VM(NB * VMO < 63 ? NB * VMO : 63);
    }
    __syncthreads();
    if (it + 2 < ntile) dma_tile(it + 2, cur_b{});
    block(acc[(NB - 1) & 1], acc[NB & 1], nxt_b{}, std::integral_constant<int, 0>{}, kt + 32 * (NB - 2), cur_epi,
          first{});
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
    block(dummy, acc[1], b0{}, std::integral_constant<int, 0>{}, kbp, epi_t<E>{}, std::integral_constant<int, 1>{});
  }
  if constexpr (LISTS) {  // the rows' hit counts: [split][T]
#pragma unroll
    for (int i = 0; i < 2 * OUT; ++i) {
      const int t = out_qg(i / 2, i % 2);
      if (lane == 0 && t < a.T) a.tcount[(size_t)split_id * a.T + t] = rcnt[i];
    }
  }
  if (LISTS) return;  // no score rows
  // columns of this split past every query of the workgroup
  const int cstart = min(k1, k0 + ntile * KT);
  for (int qi = 0; qi < QWG; ++qi) {
    if (!sh_in[qi]) continue;  // uniform
    const int t = qt0 + qi;
    for (int c = cstart + tid; c < k1; c += NT) a.scores[(size_t)t * a.ld + c] = -INFINITY;
  }
}

constexpr int kPfWaves = 8, kPfKeys = kPrefillKeyTile;
constexpr int pf_rt(int hp) { return hp >= 4 ? 2 : 1; }
// A tile table (several sequences, a handful of queries each): four waves
// and one A tile per wave (two for wide head sets), so a tile of a short run
// of queries carries less padding through the MFMAs.
constexpr int kPfGroupWaves = 4;
constexpr int pf_group_rt(int hp) { return hp > 16 ? 2 : 1; }

template <int HP, bool LISTS>
static hipError_t launch_hp(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int RT = pf_rt(HP);
  constexpr int QWG = kPfWaves * RT * 32 / HP;
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
  if (a.tiles) {  // a tile table: every workgroup checked (ragged tiles and splits)
    if (LISTS || !a.ntiles || !a.q_seq || a.ntile_bound < 1 || a.ntile_bound > 65535) return hipErrorInvalidValue;
    constexpr int GRT = pf_group_rt(HP);
    const dim3 grid(nsplit, a.ntile_bound), block(kPfGroupWaves * 64);
    if (ev0 || ev1)
      hipExtLaunchKernelGGL((score_prefill_kernel<HP, GRT, kPfGroupWaves, kPfKeys, true, false>), grid, block, 0, st,
                            ev0, ev1, 0, a, 0, 0);
    else
      hipLaunchKernelGGL((score_prefill_kernel<HP, GRT, kPfGroupWaves, kPfKeys, true, false>), grid, block, 0, st, a,
                         0, 0);
    return hipGetLastError();
  }
  if (l0) launch(0, score_prefill_kernel<HP, RT, kPfWaves, kPfKeys, false, LISTS>, dim3(ns_full, nq_full), 0, 0);
  if (l1)  // the ragged last row of query tiles, all splits
    launch(1, score_prefill_kernel<HP, RT, kPfWaves, kPfKeys, true, LISTS>, dim3(nsplit, 1), nq_full, 0);
  if (l2)  // the ragged last split, whole query tiles
    launch(2, score_prefill_kernel<HP, RT, kPfWaves, kPfKeys, true, LISTS>, dim3(1, nq_full), 0, ns_full);
  if (first < 0) {  // nothing to launch: the events mark the empty interval
    if (ev0 && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
    if (ev1 && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int head_slots(int h) { return h <= 1 ? 1 : h <= 2 ? 2 : h <= 4 ? 4 : h <= 8 ? 8 : h <= 16 ? 16 : h <= 32 ? 32 : 64; }

int prefill_queries_per_wg(int h) {
  const int hp = head_slots(h);
  return kPfWaves * pf_rt(hp) * 32 / hp;
}

int prefill_group_queries_per_wg(int h) {
  const int hp = head_slots(h);
  return kPfGroupWaves * pf_group_rt(hp) * 32 / hp;
}

bool prefill_supported(int h, int ld, int Lmax) {
  return h >= 1 && h <= kPrefillMaxHeads && ld >= Lmax &&
         (uint64_t)prefill_queries_per_wg(h) * ld * 4 <= 0x7FFFFFFFull && (uint64_t)Lmax * 256 <= 0x7FFFFFFFull;
}

// The threshold lists cost two registers per (lane, row): the tilings with
// one, two or four head slots per query (8 to 16 rows per lane) have none to
// spare and run without lists.
bool prefill_lists_supported(int h) { return h >= 5 && h <= 16; }

template <bool LISTS>
static hipError_t launch_lists(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if constexpr (!LISTS) {
    if (a.h <= 1) return launch_hp<1, false>(a, st, ev0, ev1);
    if (a.h <= 2) return launch_hp<2, false>(a, st, ev0, ev1);
    if (a.h <= 4) return launch_hp<4, false>(a, st, ev0, ev1);
  }
  if (a.h >= 5 && a.h <= 8) return launch_hp<8, LISTS>(a, st, ev0, ev1);
  if (a.h >= 9 && a.h <= 16) return launch_hp<16, LISTS>(a, st, ev0, ev1);
  if constexpr (!LISTS) {
    if (a.h <= 32) return launch_hp<32, false>(a, st, ev0, ev1);
    if (a.h <= 64) return launch_hp<64, false>(a, st, ev0, ev1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score_prefill(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (!a.tau) return launch_lists<false>(a, st, ev0, ev1);
  if (!prefill_lists_supported(a.h) || !a.tlists || !a.tcount || a.tcap < 1 ||
      (uint64_t)prefill_queries_per_wg(a.h) * a.tcap * 8 > 0x7FFFFFF0ull)
    return hipErrorInvalidValue;
  return launch_lists<true>(a, st, ev0, ev1);
}

// One workgroup walks the rows 1024 at a time: a run starts where q_seq
// changes; the run start of every row is a running maximum (a scan in LDS);
// a tile starts at every run start and every qwg rows after it; tile slots
// come from a block scan of those starts.
__global__ __launch_bounds__(1024) void prefill_tiles_kernel(const int32_t *q_seq, int T, int qwg, int bound,
                                                             int2 *tiles, uint32_t *ntiles, uint32_t *fallback) {
  constexpr int NT = 1024;
  __shared__ int smax[NT];
  __shared__ uint32_t sh[NT / kWave + 4];
  build_tile_table<NT>(q_seq, T, qwg, bound, tiles, ntiles, fallback, smax, sh);
}

hipError_t launch_prefill_tiles(const int32_t *q_seq, int T, int h, int bound, int2 *tiles, uint32_t *ntiles,
                                uint32_t *fallback, hipStream_t st) {
  if (T < 1 || bound < 1 || !prefill_supported(h, 1, 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_tiles_kernel, dim3(1), dim3(1024), 0, st, q_seq, T, prefill_group_queries_per_wg(h), bound,
                     tiles, ntiles, fallback);
  return hipGetLastError();
}

}  // namespace misa
