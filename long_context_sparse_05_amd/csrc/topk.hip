// topk.hip -- per-row top-k by (score desc, token id asc), as a radix select.
//
// The indexer keeps the k best-scoring prefix tokens of each query ("MISA:
// Mixture of Indexer Sparse Attention for Long-Context LLM Inference",
// Technical Summary, Problem Statement; the selected set is shared by all
// heads, MISA abstract).  Every valid column is given the 64-bit composite
// key (order_key(score) << 32) | ~token: keys are unique and their order is
// exactly the ranking, so the top-k is "every key >= the k-th largest key".
//
// Few long rows (decode: a handful of queries, 32K..128K columns each) take
// two stages:
//  1. each chunk of a row -- the columns one workgroup of the scoring kernel
//     produced, or of topk_lists_kernel for caller-provided scores -- keeps
//     a list of its best entries, every valid entry whose top 12 key bits
//     are at least a cutoff digit chosen from an LDS histogram of the chunk
//     so that the list holds a little more than the chunk's expected share
//     of the row's top-k (select.hpp, chunk_list);
//  2. topk_merge_kernel, one 1024-thread workgroup per row, loads the
//     union of the lists into LDS, takes its exact top-k (a 4096-bin
//     histogram over the union's key range, then the keys of the crossing
//     bin ranked among themselves)
//     and checks that the k-th key's digit is no lower than every chunk's
//     cutoff, which proves no dropped entry belongs in the top-k; if the
//     check fails (a chunk holds far more than its share, heavy ties) the
//     same workgroup runs the exact row select over the row's scores.
// Many rows, or short rows: one workgroup per row (topk_rowselect_kernel),
// or for rows of 16K..128K columns first the streamed select of
// topk_stream_kernel.
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace misa {

constexpr int kSelThreads = 1024;
constexpr int kSelCap = 16384;      // candidates resolved in LDS (128 KiB)
constexpr int kSelCompact = 2048;   // survivors compacted after each pass

// The LDS of a 1024-thread row select, declared once by each kernel that
// runs one (the merge kernel reuses it, so its fallback to the exact row
// select needs no second copy).
struct alignas(16) SelLds {
  uint64_t cs[kSelCap];
  uint64_t cs2[kSelCompact];
  uint32_t hs[256];
  uint32_t sh[kSelThreads / kWave + 16];
  unsigned long long cnt64;
};

__device__ __forceinline__ int row_valid_len(const TopkArgs &a, int r) {
  return a.row_len ? max(0, min(a.ld, a.row_len[r] + a.row_len_add)) : a.ld;
}

// Wave-aggregated append to an LDS counter: one atomic per wave.
__device__ __forceinline__ bool lds_append(bool pred, uint32_t *counter, uint32_t &pos) {
  const uint64_t m = __ballot(pred);
  if (!m) return false;
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  pos = base + lanes_below(m);
  return pred;
}

// Resolve the candidates of the threshold digit: 8-bit digit passes over
// LDS histograms of the remaining 52 composite-key bits, emitting every key
// above each pass's crossing digit (wave-aggregated LDS atomics for the
// output slots, starting at ctr[0]) and compacting the survivors, until the
// crossing bin holds exactly the keys still needed.  Candidates come from
// `cur` (keep) or are re-read from the score row (more than fit in LDS).
//
// The candidates are those whose composite key matches (prefix0, mask0); the
// first pass takes the 8-bit digit at shift0 and later passes the digits
// below it.  Candidates held in LDS may carry keys relative to key_base
// (the emitted score is key_to_float(key + key_base)).
template <bool MAP, int NT>
__device__ __forceinline__ void resolve_candidates(
    uint64_t *cur, int ncur, bool keep, int n, const float *srow, const int32_t *mrow,
    const Thresh th, int32_t *irow, float *vrow, uint64_t *cs, uint64_t *cs2, uint32_t *hs,
    uint32_t *sh, uint32_t *ctr, uint32_t *res, uint64_t prefix0, uint64_t mask0, int shift0,
    uint32_t key_base) {
  const int tid = threadIdx.x;
  // Visit every candidate that matches (prefix, mask) in uniform rounds of NT
  // (wave ballots stay legal): from LDS, or (too many ties) from the row.
  auto for_each = [&](uint64_t prefix, uint64_t mask, auto &&fn) {
    const int total = keep ? ncur : n;
    for (int b = 0; b < total; b += NT) {
      const int i = b + tid;
      bool ok = i < total;
      uint64_t ck = 0;
      if (ok) {
        if (keep) {
          ck = cur[i];
        } else {
          int tok = i;
          if (MAP) {
            tok = mrow[i];
            ok = tok >= 0;
          }
          if (ok) ck = composite(order_key(srow[i]), tok);
        }
      }
      fn(ok && (ck & mask) == prefix, ck);
    }
  };
  auto emit = [&](bool pred, uint64_t ck) {
    uint32_t pos;
    if (lds_append(pred, &ctr[0], pos) && pos < th.kk) {
      irow[pos] = (int32_t)(~(uint32_t)ck);
      if (vrow) vrow[pos] = key_to_float((uint32_t)(ck >> 32) + key_base);
    }
  };

  uint32_t need = th.kk - th.above;
  uint64_t prefix = prefix0;
  uint64_t mask = mask0;
  for (int pass = 0;; ++pass) {
    const int shift = max(shift0 - 8 * pass, 0);
    if (tid < 256) hs[tid] = 0;
    __syncthreads();
    for_each(prefix, mask, [&](bool ok, uint64_t ck) {
      if (ok) atomicAdd(&hs[(uint32_t)(ck >> shift) & 0xFFu], 1u);
    });
    __syncthreads();
    const uint32_t v = tid < 256 ? hs[255 - tid] : 0u;  // thread 0: the largest digit
    uint32_t total;
    const uint32_t incl = block_scan<NT>(v, sh, total);
    const uint32_t excl = incl - v;
    if (tid < 256 && excl < need && need <= incl) {
      res[0] = 255 - tid;
      res[1] = excl;
      res[2] = v;
    }
    __syncthreads();
    const uint32_t d = res[0], above_d = res[1], cnt_d = res[2];
    for_each(prefix, mask, [&](bool ok, uint64_t ck) {
      emit(ok && ((uint32_t)(ck >> shift) & 0xFFu) > d, ck);
    });
    need -= above_d;
    prefix |= (uint64_t)d << shift;
    mask |= 0xFFull << shift;
    if (cnt_d == need || shift == 0) {
      for_each(prefix, mask, [&](bool ok, uint64_t ck) { emit(ok, ck); });
      break;
    }
    if (keep && cnt_d <= (uint32_t)kSelCompact) {  // keep only the survivors
      uint64_t *dst = (cur == cs) ? cs2 : cs;
      if (tid == 0) ctr[1] = 0;
      __syncthreads();
      for_each(prefix, mask, [&](bool ok, uint64_t ck) {
        uint32_t pos;
        if (lds_append(ok, &ctr[1], pos) && pos < (uint32_t)(dst == cs2 ? kSelCompact : kSelCap))
          dst[pos] = ck;
      });
      __syncthreads();
      cur = dst;
      ncur = (int)cnt_d;
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- row select
// With enough rows to fill the GPU, one 1024-thread workgroup per row does
// the whole selection: pass 1 builds the row's first-digit histogram in LDS,
// pass 2 writes the columns above the threshold digit and collects the
// digit's candidates in LDS, and the candidates are resolved.  No global
// atomics and no zeroed workspace.  Rows of at most kRegCols columns with
// ld % 4 == 0 (REG) are read from HBM once: each thread keeps its 64 scores
// in registers from pass 1 to pass 2 (and the sample threshold first tries
// to skip the histogram).  Other rows are streamed twice.
constexpr int kSelU = 4;                                    // float4 loads per thread per round
constexpr int kSelRound = kSelThreads * 4 * kSelU;          // columns per round
constexpr int kRegRounds = 4;
constexpr int kRegCols = kSelRound * kRegRounds;            // 65536

// Sample threshold for a register-resident row of n columns (every column
// valid) when k is a small fraction of n.  One score per thread -- 16
// windows of 256 columns spread over the row -- gives an estimate tau of a
// key a little below the k-th largest (a two-level 12-bit radix select of the
// sample at rank ~ 1.25 k ns / n plus a margin).  One pass over the
// registers collects the columns whose scores are >= tau (one compare
// each); when there are at least k of them and no thread holds more than
// 15, their keys relative to tau are ranked: a 12-bit digit histogram emits
// every key above the k-th key's digit and the 8-bit passes resolve that
// digit.  Otherwise nothing has been written and the caller runs the exact
// histogram path.  Returns true when done.
constexpr int kSampleMinCols = 8192;

__device__ __forceinline__ bool sample_collect(const TopkArgs &a, int n,
                                               const float (&sv)[kRegRounds][kSelU][4],
                                               uint64_t *cs, uint32_t *sh, uint32_t &cnt_out,
                                               uint32_t &tau_out, uint32_t &kk_out) {
  constexpr int NT = kSelThreads;
  constexpr int NW = NT / kWave;
  static_assert(NW == kRegRounds * kSelU, "one sample window per wave");
  const int tid = threadIdx.x, wave = tid >> 6;
  const uint32_t kk = (uint32_t)min(a.k, n);
  if (n < kSampleMinCols || kk * 8u > (uint32_t)n) return false;
  uint32_t *lh = (uint32_t *)cs;
  uint32_t *res = sh + NW + 4;

  // the sample: wave w takes element 0 of its (round, group) w
  float smp = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (wave == i) smp = sv[i / kSelU][i % kSelU][0];
  const int scol = (wave / kSelU) * kSelRound + (wave % kSelU) * NT * 4 + 4 * tid;
  const bool sok = scol < n;
  const uint32_t skey = order_key(smp);

  for (int i = tid; i < kHistBins; i += NT) lh[i] = 0;
  __syncthreads();
  if (sok) atomicAdd(&lh[skey >> kHistShift], 1u);
  // block-wide values read back from LDS are uniform: readfirstlane lets the
  // compiler see that, so the early exits are scalar branches and the row's
  // registers are not kept live through the resolve below
  const int ns = __builtin_amdgcn_readfirstlane(__syncthreads_count(sok));
  const float m = (float)kk * (float)ns / (float)n;
  const int rs = (int)ceilf(1.25f * m + 3.f * sqrtf(m) + 4.f);
  if (rs >= ns) return false;  // uniform; the histogram is rebuilt by the caller
  Thresh t1 = threshold_from_lds<NT>(lh, (uint32_t)rs, sh);
  t1.b1 = __builtin_amdgcn_readfirstlane(t1.b1);
  t1.above = __builtin_amdgcn_readfirstlane(t1.above);
  for (int i = tid; i < kHistBins; i += NT) lh[i] = 0;
  if (tid == 0) {
    res[3] = 0;  // candidates
    res[4] = 0;  // a thread ran out of slots
    res[5] = 0;  // largest relative key
  }
  __syncthreads();
  if (sok && (int)(skey >> kHistShift) == t1.b1) atomicAdd(&lh[(skey >> 8) & 0xFFFu], 1u);
  __syncthreads();
  const Thresh t2 = threshold_from_lds<NT>(lh, (uint32_t)rs - t1.above, sh);
  const uint32_t b2 = __builtin_amdgcn_readfirstlane(t2.b1);
  const uint32_t tau = ((uint32_t)t1.b1 << kHistShift) | (b2 << 8);
  // tau must name a normal float or an infinity: then "score >= tf" agrees
  // with "order_key(score) >= tau" whatever the denormal mode
  if (tau < 0x00800000u || tau > 0xFF800000u || (tau >= 0x7F800000u && tau <= 0x807FFFFFu))
    return false;
  const float tf = key_to_float(tau);

  // one branch-free pass: each thread appends the columns with score >= tf
  // to its own slots (slot j of thread t at j*NT + t, so a wave's stores hit
  // consecutive words whatever its lanes' counts); a column below tf is
  // written to the next free slot and overwritten by the next hit.  A thread
  // keeps at most SLOTS - 1 hits (the last slot is the scratch).
  constexpr int SLOTS = kSelCap / NT;
  uint32_t *cv = (uint32_t *)cs;  // scores
  uint32_t *cc = cv + kSelCap;    // columns
  uint32_t cnt = 0;
#pragma unroll
  for (int rr = 0; rr < kRegRounds; ++rr) {
    const int base = rr * kSelRound;
    if (base < n) {
      const bool all = base + kSelRound <= n;
#pragma unroll
      for (int u = 0; u < kSelU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = base + u * NT * 4 + 4 * tid + e;
          const uint32_t at = min(cnt, (uint32_t)SLOTS - 1) * NT + tid;
          cv[at] = __float_as_uint(sv[rr][u][e]);
          cc[at] = (uint32_t)c;
          cnt += ((all || c < n) && sv[rr][u][e] >= tf) ? 1u : 0u;
        }
    }
  }
  const uint32_t wsum = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt), kWave - 1);
  const bool wover = __ballot(cnt >= (uint32_t)SLOTS) != 0;
  if (lane_id() == 0) {
    atomicAdd(&res[3], wsum);
    if (wover) atomicOr(&res[4], 1u);
  }
  __syncthreads();
  const uint32_t total = __builtin_amdgcn_readfirstlane(res[3]);
  if (__builtin_amdgcn_readfirstlane(res[4]) || total < kk) return false;
  cnt_out = cnt;
  tau_out = tau;
  kk_out = kk;
  return true;
}

// The ranking of the candidates sample_collect left in LDS (thread t's
// slots j < cnt at j*NT + t).  The row's registers are dead here: this is
// entered only when the collection succeeded, and the kernel ends after it.
__device__ __forceinline__ void sample_finish(const TopkArgs &a, int r, int n, uint32_t kk, uint32_t tau,
                                              uint32_t cnt, uint64_t *cs, uint64_t *cs2,
                                              uint32_t *hs, uint32_t *sh) {
  constexpr int NT = kSelThreads;
  constexpr int NW = NT / kWave;
  constexpr int SLOTS = kSelCap / NT;
  const int tid = threadIdx.x;
  uint32_t *lh = (uint32_t *)cs;
  uint32_t *ctr = sh + NW;
  uint32_t *res = sh + NW + 4;
  const uint32_t *cv = (const uint32_t *)cs;
  const uint32_t *cc = cv + kSelCap;

  // the candidates' keys relative to tau and their columns stay in
  // registers (two 32-bit arrays, every element written: a conditionally
  // written 64-bit array is kept as one vector and copied whole)
  uint32_t rk[SLOTS - 1], col[SLOTS - 1];
  uint32_t kmax = 0;
#pragma unroll
  for (int jj = 0; jj < SLOTS - 1; ++jj) {
    const bool ok = jj < (int)cnt;
    const uint32_t at = ok ? jj * NT + tid : tid;
    const uint32_t rel = order_key(__uint_as_float(cv[at])) - tau;
    rk[jj] = rel;
    col[jj] = cc[at];
    kmax = ok ? max(kmax, rel) : kmax;
  }
  kmax = wave_max_u32(kmax);
  if (lane_id() == 0 && kmax) atomicMax(&res[5], kmax);
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;
  for (int i = (int)kk + tid; i < a.k; i += NT) {
    irow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
  __syncthreads();  // every slot read: the LDS is free for the histogram
  const uint32_t top = __builtin_amdgcn_readfirstlane(res[5]);
  const int bits = top ? 32 - __clz(top) : 0;  // relative keys fit in `bits` bits
  const int dshift = max(bits - kHistBits, 0);

  // 12-bit digit of the relative key: emit the keys above the digit of the
  // kk-th key, then resolve that digit's keys
  for (int i = tid; i < kHistBins; i += NT) lh[i] = 0;
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < SLOTS - 1; ++jj)
    if (jj < (int)cnt) atomicAdd(&lh[rk[jj] >> dshift], 1u);
  __syncthreads();
  Thresh th = threshold_from_lds<NT>(lh, kk, sh);
  th.b1 = __builtin_amdgcn_readfirstlane(th.b1);
  th.above = __builtin_amdgcn_readfirstlane(th.above);
  th.eq = __builtin_amdgcn_readfirstlane(th.eq);
  const bool take_eq = th.eq == kk - th.above;  // the digit holds exactly the keys still needed
  // positions from one block scan of packed per-thread counts (at most 15
  // each, 15360 in all): emitted keys (digit above b1, or b1 itself when it
  // holds exactly the keys still needed) high, the digit's keys to resolve low
  uint32_t ne = 0, nq = 0;
#pragma unroll
  for (int jj = 0; jj < SLOTS - 1; ++jj) {
    const bool ok = jj < (int)cnt;
    const int dg = (int)(rk[jj] >> dshift);
    ne += (ok && (dg > th.b1 || (take_eq && dg == th.b1))) ? 1u : 0u;
    nq += (ok && !take_eq && dg == th.b1) ? 1u : 0u;
  }
  const uint32_t mine = (ne << 16) | nq;
  uint32_t tot;
  const uint32_t excl = block_scan<NT>(mine, sh, tot) - mine;
  uint32_t pe = excl >> 16, pq = excl & 0xFFFFu;
  uint64_t *eqk = cs;  // every slot has been read: the words are free
#pragma unroll
  for (int jj = 0; jj < SLOTS - 1; ++jj) {
    const bool ok = jj < (int)cnt;
    const int dg = (int)(rk[jj] >> dshift);
    if (ok && (dg > th.b1 || (take_eq && dg == th.b1))) {
      if (pe < kk) {
        irow[pe] = (int32_t)col[jj];
        if (vrow) vrow[pe] = key_to_float(rk[jj] + tau);
      }
      ++pe;
    }
    if (ok && !take_eq && dg == th.b1) eqk[pq++] = composite(rk[jj], (int)col[jj]);
  }
  if (take_eq) return;  // uniform
  if (tid == 0) ctr[0] = th.above;  // next output slot
  __syncthreads();
  resolve_candidates<false, NT>(eqk, (int)th.eq, true, n, nullptr, nullptr, th, irow, vrow, cs, cs2,
                                hs, sh, ctr, res, 0ull, 0ull, max(32 + dshift - 8, 0), tau);
}

template <bool MAP, bool REG>
__device__ __forceinline__ void rowselect_row(const TopkArgs &a, const int r, SelLds &L) {
  constexpr int NT = kSelThreads;
  constexpr int NW = NT / kWave;
  constexpr int U = kSelU;
  constexpr int RR = REG ? kRegRounds : 1;  // rounds held in registers
  uint64_t *cs = L.cs;
  uint64_t *cs2 = L.cs2;
  uint32_t *hs = L.hs;
  uint32_t *sh = L.sh;
  uint32_t *ctr = sh + NW;       // [0] next output slot [1] compacted
  uint32_t *res = sh + NW + 4;   // [0] digit [1] count above it [2] count in it
  unsigned long long &cnt64 = L.cnt64;  // (above emitted << 32) | candidates collected
  uint32_t *lh = (uint32_t *)cs;  // pass-1 histogram lives in the candidate array
  const int tid = threadIdx.x;
  const int n = row_valid_len(a, r);
  const float *srow = a.scores + (size_t)r * a.ld;
  const int32_t *mrow = MAP ? a.map + (size_t)r * a.ld : nullptr;
  const bool vec = (a.ld % 4) == 0 && ((uintptr_t)a.scores & 15) == 0;  // 16-byte aligned rows

  auto load_round = [&](int base, float (&sv)[U][4]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cf = base + u * NT * 4 + 4 * tid;
      if (vec && cf + 3 < n) {
        const float4 x = *(const float4 *)(srow + cf);
        sv[u][0] = x.x; sv[u][1] = x.y; sv[u][2] = x.z; sv[u][3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[u][e] = cf + e < n ? srow[cf + e] : 0.f;
      }
    }
  };
  // a round's map entries (token ids, -1 = empty slot), all loads issued at
  // once from columns clamped into the row: a load under a branch would wait
  // for every load before it
  auto load_map = [&](int base, int32_t (&mv)[U][4]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) mv[u][e] = mrow[min(base + u * NT * 4 + 4 * tid + e, n - 1)];
  };
  auto hist_round = [&](int base, const float (&sv)[U][4]) {
    const bool all = !MAP && base + kSelRound <= n;  // uniform: no per-column test
    int32_t mv[U][4];
    if constexpr (MAP) load_map(base, mv);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = base + u * NT * 4 + 4 * tid + e;
        if (all || (c < n && (!MAP || mv[u][e] >= 0)))
          atomicAdd(&lh[order_key(sv[u][e]) >> kHistShift], 1u);
      }
  };

  float sv[RR][U][4];
  if constexpr (REG) {
    // every load of the row in flight at once: float4 loads with the column
    // clamped into the row (ld % 4 == 0, so a float4 at c < ld stays inside
    // it); columns at or past n hold stale values that every use masks out
#pragma unroll
    for (int rr = 0; rr < RR; ++rr)
      if (rr * kSelRound < n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t cf = (uint32_t)min(rr * kSelRound + u * NT * 4 + 4 * tid, a.ld - 4);
          const float4 x = *(const float4 *)((const char *)srow + cf * 4u);
          sv[rr][u][0] = x.x; sv[rr][u][1] = x.y; sv[rr][u][2] = x.z; sv[rr][u][3] = x.w;
        }
      }
    if constexpr (!MAP) {
      uint32_t cnt, tau, kk;
      if (sample_collect(a, n, sv, cs, sh, cnt, tau, kk)) {  // uniform
        sample_finish(a, r, n, kk, tau, cnt, cs, cs2, hs, sh);
        return;
      }
    }
  }
  for (int i = tid; i < kHistBins; i += NT) lh[i] = 0;
  __syncthreads();
  if (REG) {  // pass 1: the histogram of the registers
#pragma unroll
    for (int rr = 0; rr < RR; ++rr)
      if (rr * kSelRound < n) hist_round(rr * kSelRound, sv[rr]);
  } else {
    for (int base = 0; base < n; base += kSelRound) {
      load_round(base, sv[0]);
      hist_round(base, sv[0]);
    }
  }
  __syncthreads();
  const Thresh th = threshold_from_lds<NT>(lh, (uint32_t)a.k, sh);
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;
  for (int i = (int)th.kk + tid; i < a.k; i += NT) {
    irow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
  if (th.kk == 0) return;  // uniform
  const bool keep = th.eq <= (uint32_t)kSelCap;
  if (tid == 0) {
    cnt64 = 0;
    ctr[0] = th.above;
  }
  __syncthreads();
  // pass 2: emit the columns above b1, collect the columns equal to b1
  auto emit_round = [&](int base, const float (&sv)[U][4]) {
    int32_t mv[U][4];
    if constexpr (MAP) load_map(base, mv);
    uint32_t fs = 0, fc = 0;  // this thread's 16 columns: above b1 / equal to b1
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = base + u * NT * 4 + 4 * tid + e;
        const bool valid = c < n && (!MAP || mv[u][e] >= 0);
        const int dg = (int)(order_key(sv[u][e]) >> kHistShift);
        fs |= (valid && dg > th.b1 ? 1u : 0u) << (u * 4 + e);
        fc |= (valid && keep && dg == th.b1 ? 1u : 0u) << (u * 4 + e);
      }
    }
    // positions: a wave-wide scan of the packed counts and one 64-bit LDS
    // atomic per wave (at most 1024 of each kind per wave and round)
    const uint32_t mine = ((uint32_t)__popc(fs) << 16) | (uint32_t)__popc(fc);
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    uint64_t wbase = 0;
    if (lane_id() == 0 && wtot)
      wbase = atomicAdd(&cnt64, ((uint64_t)(wtot >> 16) << 32) | (uint64_t)(wtot & 0xFFFFu));
    wbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(wbase >> 32), 0) << 32) |
            (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)wbase, 0);
    const uint32_t excl = incl - mine;
    uint32_t so = (uint32_t)(wbase >> 32) + (excl >> 16);
    uint32_t co = (uint32_t)wbase + (excl & 0xFFFFu);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bit = u * 4 + e;
        const int c = base + u * NT * 4 + 4 * tid + e;
        if ((fs >> bit) & 1u) {
          if (so < th.above) {
            irow[so] = MAP ? mv[u][e] : c;
            if (vrow) vrow[so] = sv[u][e];
          }
          ++so;
        }
        if ((fc >> bit) & 1u) {
          if (co < (uint32_t)kSelCap) cs[co] = composite(order_key(sv[u][e]), MAP ? mv[u][e] : c);
          ++co;
        }
      }
    }
  };
  if (REG) {
#pragma unroll
    for (int rr = 0; rr < RR; ++rr)
      if (rr * kSelRound < n) emit_round(rr * kSelRound, sv[rr]);
  } else {
    for (int base = 0; base < n; base += kSelRound) {
      load_round(base, sv[0]);
      emit_round(base, sv[0]);
    }
  }
  __syncthreads();
  resolve_candidates<MAP, NT>(cs, keep ? (int)th.eq : 0, keep, n, srow, mrow, th, irow, vrow, cs,
                              cs2, hs, sh, ctr, res, (uint64_t)(uint32_t)th.b1 << 52, 0xFFFull << 52,
                              44, 0u);
}

// One workgroup per row.
template <bool MAP, bool REG>
__global__ __launch_bounds__(kSelThreads) void topk_rowselect_kernel(TopkArgs a) {
  __shared__ SelLds L;
  rowselect_row<MAP, REG>(a, blockIdx.x, L);
}

// The rows the streamed select left (counter 7 set): a grid of at most 256
// workgroups walks the rows, so a row it settled costs one flag read. It
// takes the streamed (register-free) form of the row select: wrapped in this
// loop the register-resident form spills, and the rows that come here are
// few.
__global__ __launch_bounds__(kSelThreads) void topk_flagged_kernel(TopkArgs a) {
  // this workgroup's rows r = blockIdx.x + i * gridDim.x, their flags read
  // 1024 at a time in one round of loads
  __shared__ uint32_t fl[kSelThreads];
  __shared__ SelLds L;
  for (int i0 = 0; blockIdx.x + i0 * gridDim.x < a.rows; i0 += kSelThreads) {
    {
      const int r = blockIdx.x + (i0 + threadIdx.x) * gridDim.x;
      fl[threadIdx.x] = r < a.rows ? a.counters[(size_t)r * kRowCounters + 7] : 0u;
    }
    __syncthreads();
    for (int i = 0; i < kSelThreads; ++i) {
      const int r = blockIdx.x + (i0 + i) * gridDim.x;
      if (r >= a.rows) break;
      if (fl[i] == 0u) continue;  // uniform
      rowselect_row<false, false>(a, r, L);
      __syncthreads();  // the next row reuses the LDS
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ merge
// One workgroup per row: the exact top-k of the union of the row's chunk
// lists, or the row select over its scores when the union cannot prove it.
//  1. headers and the first entries of every list in one round of loads
//     (a list's slot holds at least 256 entries: the first min(512, slot)
//     are loaded before its length is known);
//  2. the entries as composite keys into LDS, with a histogram of 4096
//     bins over the union's own key range [lo, hi] -- lo the lowest cutoff,
//     hi the largest key, both from the headers -- so bins are fine where
//     the k-th key lies;
//  3. the bin holding the kk-th key; when it holds more keys than are still
//     needed they are ranked among themselves (each against all, few keys),
//     giving the kk-th composite key K (a bin of more than 1024 keys -- heavy
//     ties -- takes the row select);
//  4. the exactness check (K's digit against every cutoff), then one pass
//     writes every key >= K, positions from a block scan.
// above this many outputs a row's merge writes them in runs per wave (fewer
// cache lines a store); below, the block scan's layout costs less
constexpr uint32_t kRunOutMin = 4096;

// SPEC: entries per lane loaded ahead, per list (in the first round of
// loads; the rest of a longer list follows in further rounds)
template <bool MAP, int SPEC>
__global__ __launch_bounds__(kSelThreads) void topk_merge_kernel(TopkArgs a) {
  constexpr int NT = kSelThreads, NW = NT / kWave;
  constexpr int PER = kSelCap / NT;
  constexpr int NB = kHistBins;  // bins over the union's key range
  __shared__ SelLds L;
  __shared__ uint32_t off[kMaxLists], cnt[kMaxLists];
  // [0] largest cutoff [1] lowest key bound [2] largest key [3] keys of the
  // crossing bin; later [0..1] hold the kk-th composite key
  __shared__ alignas(8) uint32_t red[4];
  uint32_t *sh = L.sh;
  uint32_t *lh = (uint32_t *)L.cs2;  // the union's histogram (16 KiB)
  const int r = blockIdx.x, tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = a.nwg;
  const uint4 *hd = a.lhead + (size_t)r * nl;
  const uint2 *lrow = a.lists + (size_t)r * nl * a.lcap;
  const uint32_t spec = (uint32_t)min(SPEC * kWave, a.lcap);
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;

  // 1. headers (thread = list) and, per wave, lists wave and wave + NW
  const uint4 h = tid < nl ? hd[tid] : make_uint4(0u, 0u, 0u, 0u);
  const uint2 *la = lrow + (size_t)min(wave, nl - 1) * a.lcap;
  const uint2 *lb = lrow + (size_t)min(wave + NW, nl - 1) * a.lcap;
  uint2 ea[SPEC], eb[SPEC];
#pragma unroll
  for (int u = 0; u < SPEC; ++u) {
    const uint32_t j = min((uint32_t)(lane + kWave * u), spec - 1u);
    ea[u] = la[j];
    eb[u] = lb[j];
  }
  for (int i = tid; i < NB; i += NT) lh[i] = 0;
  if (tid < 4) red[tid] = tid == 1 ? 0xFFFFFFFFu : 0u;
  uint32_t total;
  const uint32_t incl = block_scan<NT>(h.x, sh, total);
  if (tid < nl) {
    off[tid] = incl - h.x;
    cnt[tid] = h.x;
  }
  {  // largest cutoff; lowest bound of a list's keys (its cutoff digit, 0 when
     // it kept everything); largest key
    const bool on = tid < nl && h.x > 0;
    const uint32_t mc = wave_max_u32(tid < nl ? h.y : 0u);
    const uint32_t lo = ~wave_max_u32(on ? ~(h.y >= (uint32_t)kHistBins ? 0u : h.y << kHistShift) : 0u);
    const uint32_t hi = wave_max_u32(on ? h.z : 0u);
    if (lane == 0) {
      if (mc) atomicMax(&red[0], mc);
      atomicMin(&red[1], lo);
      if (hi) atomicMax(&red[2], hi);
    }
  }
  __syncthreads();
  total = __builtin_amdgcn_readfirstlane(total);
  const uint32_t cut = __builtin_amdgcn_readfirstlane(red[0]);
  // (readfirstlane returns int: compare as unsigned)
  const uint32_t khi = (uint32_t)__builtin_amdgcn_readfirstlane(red[2]);
  const uint32_t klo = min((uint32_t)__builtin_amdgcn_readfirstlane(red[1]), khi);
  const uint32_t kk = min((uint32_t)a.k, total);
  // bin of a key: (key - klo) >> bs, in [0, NB) for every key of the union
  // (clamped all the same, so no LDS access can leave the histogram)
  const int bs = max(0, 32 - (int)__clz(khi - klo) - kHistBits);
  auto bin_of = [&](uint32_t key) { return min((key - klo) >> bs, (uint32_t)NB - 1u); };

  bool fits = total <= (uint32_t)kSelCap;
  uint64_t kth = 0;  // the kk-th largest composite key
  if (fits && kk > 0) {  // uniform
    // 2. the entries into LDS (list w at off[w]) and their histogram
    auto place = [&](int w, const uint2 &e, uint32_t j) {
      if (j < cnt[w]) {
        L.cs[off[w] + j] = composite(e.x, (int)e.y);
        atomicAdd(&lh[bin_of(e.x)], 1u);
      }
    };
#pragma unroll
    for (int u = 0; u < SPEC; ++u) {
      const uint32_t j = (uint32_t)(lane + kWave * u);
      if (wave < nl) place(wave, ea[u], j);
      if (wave + NW < nl) place(wave + NW, eb[u], j);
    }
    // the rest: entries past the first `spec` of these lists, and whole
    // lists past the first 2 NW
    for (int w = wave; w < nl; w += NW) {
      const uint32_t c = cnt[w];
      const uint2 *lw = lrow + (size_t)w * a.lcap;
      for (uint32_t j0 = w < 2 * NW ? spec : 0u; j0 < c; j0 += SPEC * kWave) {
        uint2 e[SPEC];
#pragma unroll
        for (int u = 0; u < SPEC; ++u) e[u] = lw[min(j0 + lane + kWave * u, c - 1u)];
#pragma unroll
        for (int u = 0; u < SPEC; ++u) place(w, e[u], j0 + lane + kWave * u);
      }
    }
    __syncthreads();
    // 3. the bin holding the kk-th key, counted from the top
    const Thresh th = threshold_from_lds<NT>(lh, kk, sh);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane(th.b1);
    const uint32_t need = kk - __builtin_amdgcn_readfirstlane(th.above);
    const uint32_t inb = __builtin_amdgcn_readfirstlane(th.eq);
    if (inb > (uint32_t)NT) {  // uniform: heavy ties in one bin
      fits = false;
    } else {
      // the bin's keys into the (now free) histogram words, one per thread,
      // each ranked against all of them: the key of rank need - 1 is K
      uint64_t *bkeys = (uint64_t *)lh;
      if (tid == 0) red[3] = 0;
      __syncthreads();
      for (uint32_t i0 = 0; i0 < total; i0 += NT) {
        const uint32_t i = i0 + tid;
        const uint64_t ck = i < total ? L.cs[i] : 0ull;
        uint32_t pos;
        if (lds_append(i < total && bin_of((uint32_t)(ck >> 32)) == b, &red[3], pos) && pos < (uint32_t)NT)
          bkeys[pos] = ck;
      }
      __syncthreads();
      if ((uint32_t)tid < inb) {
        const uint64_t mine = bkeys[tid];
        uint32_t rank = 0;
        for (uint32_t j = 0; j < inb; ++j) rank += bkeys[j] > mine ? 1u : 0u;
        if (rank == need - 1u) ((uint64_t *)&red[0])[0] = mine;  // red[0..1]: K (cutoff already read)
      }
      __syncthreads();
      kth = ((const uint64_t *)&red[0])[0];
    }
  }
  // 4. exact when no chunk dropped anything, or the union holds k keys and
  // K's digit is at least every cutoff
  const bool exact = fits && (cut == 0u || (kk == (uint32_t)a.k && (uint32_t)(kth >> 52) >= cut));
  if (!exact) {  // uniform: the exact select over the whole score row
    __syncthreads();
    rowselect_row<MAP, false>(a, r, L);
    return;
  }
  // every key >= K: exactly kk of them, in any order
  uint32_t selbits = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t i = (uint32_t)(tid + NT * u);
    if (kk > 0 && i < total && L.cs[i] >= kth) selbits |= 1u << u;
  }
  if (kk > kRunOutMin) {  // uniform
    // many: wave w's entries of slot u follow those of its slots < u and the
    // waves' runs follow one another, so each store writes one short run
    uint32_t wtot = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) wtot += (uint32_t)__popcll(__ballot((selbits >> u) & 1u));
    __syncthreads();  // sh is free again
    if (lane == 0) sh[wave] = wtot;
    __syncthreads();
    uint32_t pos = 0;
    for (int w = 0; w < NW; ++w) pos += w < wave ? sh[w] : 0u;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const bool s_u = (selbits >> u) & 1u;
      const uint64_t m = __ballot(s_u);
      if (s_u) {
        const uint64_t ck = L.cs[tid + NT * u];
        const uint32_t p = pos + lanes_below(m);
        irow[p] = (int32_t)(~(uint32_t)ck);
        if (vrow) vrow[p] = key_to_float((uint32_t)(ck >> 32));
      }
      pos += (uint32_t)__popcll(m);
    }
  } else {  // few: each thread's entries side by side, positions from a block scan
    const uint32_t mine = (uint32_t)__popc(selbits);
    uint32_t tot;
    uint32_t pos = block_scan<NT>(mine, sh, tot) - mine;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if ((selbits >> u) & 1u) {
        const uint64_t ck = L.cs[tid + NT * u];
        if (pos < kk) {
          irow[pos] = (int32_t)(~(uint32_t)ck);
          if (vrow) vrow[pos] = key_to_float((uint32_t)(ck >> 32));
        }
        ++pos;
      }
    }
  }
  for (int i = (int)kk + tid; i < a.k; i += NT) {
    irow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
}

// Chunk lists of caller-provided score rows (misa_topk with few long rows):
// one 256-thread workgroup per (chunk of kListChunk columns, row).
template <bool MAP>
__global__ __launch_bounds__(256) void topk_lists_kernel(TopkArgs a) {
  constexpr int NT = 256, PER = kListChunk / NT;
  __shared__ float sc[kListChunk];
  __shared__ alignas(16) uint32_t lh[kHistBins];
  __shared__ int32_t tk[MAP ? kListChunk : 1];
  __shared__ uint32_t sh[2 * NT / kWave + 9];
  const int r = blockIdx.y, tid = threadIdx.x;
  const int n_row = row_valid_len(a, r);
  const int c0 = blockIdx.x * kListChunk, c1 = min(c0 + kListChunk, n_row);
  const float *srow = a.scores + (size_t)r * a.ld;
  const int32_t *mrow = MAP ? a.map + (size_t)r * a.ld : nullptr;
  for (int b = tid; b < kHistBins; b += NT) lh[b] = 0;
  __syncthreads();
  uint32_t nv = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + NT * u, c = c0 + i;
    const float x = c < c1 ? srow[c] : -INFINITY;
    const int32_t t = MAP ? (c < c1 ? mrow[c] : -1) : c;
    const bool ok = c < c1 && (!MAP || t >= 0);
    sc[i] = x;
    if (MAP) tk[i] = t;
    if (ok) {
      atomicAdd(&lh[order_key(x) >> kHistShift], 1u);
      ++nv;
    }
  }
  uint32_t nvalid;
  block_scan<NT>(nv, sh, nvalid);  // (its barriers also publish sc, tk and lh)
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const int n = max(0, c1 - c0);
  const uint32_t quota = chunk_quota(a.k, (int)nvalid, n_row);
  const uint32_t cap = min((uint32_t)a.lcap, 2u * quota + 64u);
  chunk_list<NT, PER>(sc, n, lh, nvalid, quota, cap,
                      [&](int i) { return !MAP || tk[i] >= 0; },
                      [&](int i) { return MAP ? tk[i] : c0 + i; },
                      a.lists + ((size_t)r * a.nwg + blockIdx.x) * a.lcap,
                      a.lhead + (size_t)r * a.nwg + blockIdx.x, sh);
}

hipError_t launch_topk_merge(const TopkArgs &a, hipStream_t st) {
  if (a.nwg < 1 || a.nwg > kMaxLists) return hipErrorInvalidValue;
  // a list's expected length (its chunk's quota when the rows are whole):
  // four entries a lane ahead cover it when it is at most 240 (k = 2048 over
  // 32 lists: about 128), eight otherwise (k' = 8192: about 370)
  const double e = (double)a.k / a.nwg;
  const bool short_lists = e + 6.0 * std::sqrt(e) + 16.0 <= 240.0;
  const dim3 grid(a.rows), block(kSelThreads);
  if (a.map) {
    if (short_lists) hipLaunchKernelGGL((topk_merge_kernel<true, 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((topk_merge_kernel<true, 8>), grid, block, 0, st, a);
  } else {
    if (short_lists) hipLaunchKernelGGL((topk_merge_kernel<false, 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((topk_merge_kernel<false, 8>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_topk_lists(const TopkArgs &a, hipStream_t st) {
  if (a.nwg != (a.ld + kListChunk - 1) / kListChunk || a.lcap < kListChunk) return hipErrorInvalidValue;
  const dim3 grid(a.nwg, a.rows);
  if (a.map)
    hipLaunchKernelGGL(topk_lists_kernel<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(topk_lists_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ streamed select
// Many long rows (the score rows of a prefill chunk): one 256-thread
// workgroup per row, several rows per CU at once, each row read from HBM
// once (the register-resident row select holds one row per CU and cannot
// overlap a row's ranking with the next row's loads).
//  1. A 4096-score sample -- 16 windows of 256 columns spread over the row --
//     brackets the k-th largest key: with m = kk 4096 / n, tau_lo is the
//     lower edge of the histogram bin holding the sample's
//     (m + 4 sqrt(m) + 4)-th largest key and tau_hi the upper edge of the
//     bin holding its (m - 4 sqrt(m) - 4)-th (a 1024-bin histogram over the
//     sample's own key range, its crossing bins split again into 1024).
//  2. One streamed pass (non-temporal 16-byte loads, the next round's in
//     flight) appends the columns with key >= tau_lo to an LDS list of
//     composite keys (key relative to tau_lo << 32 | ~column; positions from
//     a wave scan and one LDS atomic per wave and round) and counts those
//     >= tau_hi.
//  3. If no more than kk columns lie at or above tau_hi and the list holds
//     at least kk and fits, the entries >= tau_hi are output and the
//     kk - above still needed are resolved among the band [tau_lo, tau_hi)
//     by 10-bit digit passes from the highest bit in use, every key above a
//     pass's crossing digit emitted, until the crossing digit holds exactly
//     the keys still needed.  Otherwise nothing is written and the row's
//     flag (counter 7) is set: the register-resident row select takes it.
constexpr int kStThreads = 256;
constexpr int kStCap = kStreamSelectCap;           // candidates held per row
constexpr int kStU = 4;                            // float4 per thread per round
constexpr int kStRound = kStThreads * 4 * kStU;    // 4096 columns
constexpr int kStMinCols = kStreamSelectMinCols;
constexpr int kStSample = kStreamSelectSample;
constexpr int kStBins = 1024;                      // histogram bins (sample, band digits)

__global__ __launch_bounds__(kStThreads) void topk_stream_kernel(TopkArgs a) {
  constexpr int NT = kStThreads, NW = NT / kWave;
  __shared__ uint64_t cand[kStCap];
  __shared__ uint32_t hh[kStBins];
  __shared__ uint32_t sh[NW + 16];
  __shared__ uint32_t ctr[2];  // [0] candidates appended [1] output slots used
  const int r = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = row_valid_len(a, r);
  const float *srow = a.scores + (size_t)r * a.ld;
  uint32_t *flag = a.counters + (size_t)r * kRowCounters + 7;
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;
  const uint32_t kk = (uint32_t)min(a.k, n);
  if (n < kStMinCols || kk == 0) {  // uniform: the exact select takes the row
    if (tid == 0) *flag = 1u;
    return;
  }
  // The bin of an NB-bin histogram in hh where the count from the top
  // crosses `need` (need <= the histogram's total), the count above it and
  // the bin's own count, to sh[NW..NW+2].  Uniform control flow.
  auto crossing = [&](uint32_t need, auto nb) {
    constexpr int NB = decltype(nb)::value;
    constexpr int PER = NB / NT;
    const int top = NB - 1 - PER * tid;
    uint32_t v[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      v[i] = hh[top - i];
      sum += v[i];
    }
    uint32_t total;
    const uint32_t incl = block_scan<NT>(sum, sh, total), excl = incl - sum;
    if (excl < need && need <= incl) {
      uint32_t cum = excl;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (cum + v[i] >= need) {
          sh[NW] = (uint32_t)(top - i);
          sh[NW + 1] = cum;
          sh[NW + 2] = v[i];
          break;
        }
        cum += v[i];
      }
    }
    __syncthreads();
  };
  using BBIG = std::integral_constant<int, kStBins>;

  // 1. the sample: thread t reads 16 consecutive columns of window t / 16
  uint32_t skey[16];
  {
    const int wbase = (int)(((long long)(tid >> 4) * (n - 256)) / 15) & ~3;
    const int cs = wbase + (tid & 15) * 16;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 x = *(const float4 *)(srow + cs + 4 * u);
      skey[4 * u + 0] = order_key(x.x);
      skey[4 * u + 1] = order_key(x.y);
      skey[4 * u + 2] = order_key(x.z);
      skey[4 * u + 3] = order_key(x.w);
    }
  }
  const float m = (float)kk * (float)kStSample / (float)n;
  const float marg = 4.f * sqrtf(m) + 4.f;
  const uint32_t rs_lo = (uint32_t)ceilf(m + marg);   // rank of tau_lo in the sample
  const int rs_hi = (int)floorf(m - marg);            // rank of tau_hi (none if < 1)
  if (rs_lo >= (uint32_t)kStSample) {
    if (tid == 0) *flag = 1u;
    return;
  }
  // one histogram of the sample over its own key range, kStBins bins of
  // 2^s keys: tau_lo = the lower edge of the bin holding the rs_lo-th
  // largest sample key, tau_hi = the upper edge of the bin of the rs_hi-th
  uint32_t kmin = ~0u, kmax = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    kmin = min(kmin, skey[e]);
    kmax = max(kmax, skey[e]);
  }
  kmax = wave_max_u32(kmax);
  kmin = ~wave_max_u32(~kmin);
  if (lane == 0) {
    sh[wave] = kmax;
    sh[NW + 8 + wave] = kmin;
  }
  for (int i = tid; i < kStBins; i += NT) hh[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    kmax = max(kmax, sh[i]);
    kmin = min(kmin, sh[NW + 8 + i]);
  }
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  const int rbits = kmax > kmin ? 32 - (int)__clz(kmax - kmin) : 0;
  const int s1 = max(0, rbits - 10), s2 = max(0, s1 - 10);
#pragma unroll
  for (int e = 0; e < 16; ++e) atomicAdd(&hh[(skey[e] - kmin) >> s1], 1u);
  __syncthreads();
  crossing(rs_lo, BBIG{});
  const uint32_t blo = __builtin_amdgcn_readfirstlane(sh[NW]);
  const uint32_t alo = __builtin_amdgcn_readfirstlane(sh[NW + 1]);
  __syncthreads();
  uint32_t bhi = 0, ahi = 0;
  if (rs_hi >= 1) {
    crossing((uint32_t)rs_hi, BBIG{});
    bhi = __builtin_amdgcn_readfirstlane(sh[NW]);
    ahi = __builtin_amdgcn_readfirstlane(sh[NW + 1]);
  }
  // the first level's bins are coarse where the range spans many octaves:
  // the crossing bins are split again into kStBins sub-bins of 2^s2 keys
  auto refine = [&](uint32_t b1, uint32_t rank) -> uint32_t {
    __syncthreads();
    for (int i = tid; i < kStBins; i += NT) hh[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t d = skey[e] - kmin;
      if ((d >> s1) == b1) atomicAdd(&hh[(d - (b1 << s1)) >> s2], 1u);
    }
    __syncthreads();
    crossing(rank, BBIG{});
    const uint32_t b2 = __builtin_amdgcn_readfirstlane(sh[NW]);
    __syncthreads();
    return b2;
  };
  const uint32_t tau_lo = kmin + (blo << s1) + (refine(blo, rs_lo - alo) << s2);
  uint64_t tau_hi = 1ull << 32;  // keys >= tau_hi rank in the top kk when no more than kk lie there
  if (rs_hi >= 1)
    tau_hi = (uint64_t)kmin + ((uint64_t)bhi << s1) + ((uint64_t)(refine(bhi, (uint32_t)rs_hi - ahi) + 1) << s2);
  if (tid == 0) {
    ctr[0] = 0;
    ctr[1] = 0;
  }
  __syncthreads();

  // 2. the streamed pass
  auto load_round = [&](int base, float4 (&v)[kStU]) {
#pragma unroll
    for (int u = 0; u < kStU; ++u) {
      const uint32_t cf = (uint32_t)min(base + u * NT * 4 + 4 * tid, a.ld - 4);
      const uint4 t = load_nt16((const char *)srow + cf * 4u);  // read once
      v[u] = make_float4(__uint_as_float(t.x), __uint_as_float(t.y), __uint_as_float(t.z),
                         __uint_as_float(t.w));
    }
  };
  uint32_t nhi = 0;  // this thread's columns above tau_hi
  auto scan_round = [&](int base, const float4 (&v)[kStU]) {
    uint32_t bits = 0;
#pragma unroll
    for (int u = 0; u < kStU; ++u) {
      const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = base + u * NT * 4 + 4 * tid + e;
        const uint32_t key = order_key(x[e]);
        const bool ok = c < n && key >= tau_lo;
        nhi += (ok && (uint64_t)key >= tau_hi) ? 1u : 0u;
        bits |= (ok ? 1u : 0u) << (u * 4 + e);
      }
    }
    const uint32_t mine = (uint32_t)__popc(bits);
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    uint32_t wb = 0;
    if (lane == kWave - 1 && wtot) wb = atomicAdd(&ctr[0], wtot);
    uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)wb, kWave - 1) + incl - mine;
#pragma unroll
    for (int u = 0; u < kStU; ++u) {
      const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((bits >> (u * 4 + e)) & 1u) {
          if (pos < (uint32_t)kStCap) cand[pos] = composite(order_key(x[e]) - tau_lo, base + u * NT * 4 + 4 * tid + e);
          ++pos;
        }
      }
    }
  };
  {
    float4 va[kStU], vb[kStU];
    load_round(0, va);
    for (int base = 0;; base += 2 * kStRound) {
      load_round(base + kStRound, vb);
      scan_round(base, va);
      if (base + kStRound >= n) break;
      load_round(base + 2 * kStRound, va);
      scan_round(base + kStRound, vb);
      if (base + 2 * kStRound >= n) break;
    }
  }
  uint32_t nh_total;
  block_scan<NT>(nhi, sh, nh_total);
  const uint32_t nabove = __builtin_amdgcn_readfirstlane(nh_total);
  const uint32_t total = __builtin_amdgcn_readfirstlane(ctr[0]);
  if (nabove > kk || total > (uint32_t)kStCap || total < kk) {  // uniform
    // (the flag names the reason: 2 too many above tau_hi, 3 the list
    // overflowed, 4 too few at or above tau_lo; 1 is a row this select does
    // not take)
    if (tid == 0) *flag = nabove > kk ? 2u : total > (uint32_t)kStCap ? 3u : 4u;
    return;
  }
  if (tid == 0) *flag = 0u;
  // list entries at or above tau_hi (relative key >= hib) are in (they leave
  // with the first band pass's emissions); the band below supplies the
  // kk - nabove still needed
  const uint64_t hib = tau_hi >= (1ull << 32) ? ~0ull : (tau_hi - tau_lo) << 32;

  // 3. the kk - nabove best of the band: 10-bit digit passes
  uint32_t need = kk - nabove;
  if (need == 0) {
    for (uint32_t i0 = 0; i0 < total; i0 += NT) {
      const uint32_t i = i0 + tid;
      const uint64_t x = i < total ? cand[i] : 0ull;
      uint32_t pos;
      if (lds_append(i < total && x >= hib, &ctr[1], pos) && pos < kk) {
        irow[pos] = (int32_t)~(uint32_t)x;
        if (vrow) vrow[pos] = key_to_float((uint32_t)(x >> 32) + tau_lo);
      }
    }
  } else {
    uint32_t hmax = 0;
    for (uint32_t i = tid; i < total; i += NT)
      if (cand[i] < hib) hmax = max(hmax, (uint32_t)(cand[i] >> 32));
    hmax = wave_max_u32(hmax);
    if (lane == 0) sh[wave] = hmax;
    __syncthreads();
    uint32_t top = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) top = max(top, sh[i]);
    top = __builtin_amdgcn_readfirstlane(top);
    // the highest bit in use: in the relative key, or else in the column word
    int shift = top ? 32 + max(0, 31 - (int)__clz(top) - 9) : 22;
    uint64_t prefix = 0, pmask = 0;
    for (bool first = true;; first = false) {
      __syncthreads();
      for (int i = tid; i < kStBins; i += NT) hh[i] = 0;
      __syncthreads();
      for (uint32_t i = tid; i < total; i += NT) {
        const uint64_t x = cand[i];
        if (x < hib && (x & pmask) == prefix) atomicAdd(&hh[(uint32_t)(x >> shift) & (kStBins - 1)], 1u);
      }
      __syncthreads();
      crossing(need, BBIG{});
      const uint32_t b = __builtin_amdgcn_readfirstlane(sh[NW]);
      const uint32_t above = __builtin_amdgcn_readfirstlane(sh[NW + 1]);
      const uint32_t inb = __builtin_amdgcn_readfirstlane(sh[NW + 2]);
      const bool last = inb == need - above;  // the crossing digit holds exactly the keys still needed
      // every thread visits the same number of list slots, so the wave-level
      // appends inside run with all lanes present
      for (uint32_t i0 = 0; i0 < total; i0 += NT) {
        const uint32_t i = i0 + tid;
        const uint64_t x = i < total ? cand[i] : 0ull;
        const uint32_t d = (uint32_t)(x >> shift) & (kStBins - 1);
        const bool out = i < total && (x < hib ? (x & pmask) == prefix && (d > b || (last && d == b)) : first);
        uint32_t pos;
        if (lds_append(out, &ctr[1], pos) && pos < kk) {
          irow[pos] = (int32_t)~(uint32_t)x;
          if (vrow) vrow[pos] = key_to_float((uint32_t)(x >> 32) + tau_lo);
        }
      }
      if (last) break;
      need -= above;
      prefix |= (uint64_t)b << shift;
      pmask |= (uint64_t)(kStBins - 1) << shift;
      shift = max(shift - 10, 0);
    }
  }
  for (int i = (int)kk + tid; i < a.k; i += NT) {
    irow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
}

hipError_t launch_topk_stream(const TopkArgs &a, hipStream_t st) {
  if (a.map || a.ld % 4 || ((uintptr_t)a.scores & 15) || a.ld < kStMinCols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_stream_kernel, dim3(a.rows), dim3(kStThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_rowselect(const TopkArgs &a, hipStream_t st) {
  if (a.only_flagged) {
    if (a.map) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_flagged_kernel, dim3(a.rows < 256 ? a.rows : 256), dim3(kSelThreads), 0,
                       st, a);
    return hipGetLastError();
  }
  // the register-resident form reads 16-byte vectors
  const bool reg = a.ld <= kRegCols && a.ld % 4 == 0 && ((uintptr_t)a.scores & 15) == 0;
  const dim3 grid(a.rows);
  if (a.map) {
    if (reg)
      hipLaunchKernelGGL((topk_rowselect_kernel<true, true>), grid, dim3(kSelThreads), 0, st, a);
    else
      hipLaunchKernelGGL((topk_rowselect_kernel<true, false>), grid, dim3(kSelThreads), 0, st, a);
  } else {
    if (reg)
      hipLaunchKernelGGL((topk_rowselect_kernel<false, true>), grid, dim3(kSelThreads), 0, st, a);
    else
      hipLaunchKernelGGL((topk_rowselect_kernel<false, false>), grid, dim3(kSelThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace misa
