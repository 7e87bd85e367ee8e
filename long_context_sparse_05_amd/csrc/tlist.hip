// tlist.hip -- the per-row top-k of a prefill chunk (many long score rows)
// without re-reading its score matrix: a sampled lower bound of each row's
// k-th score, lists of the scores at or above it written by the scoring
// kernel, and an exact selection from those lists.
//
// The indexer keeps the k best-scoring prefix tokens of every query ("MISA:
// Mixture of Indexer Sparse Attention for Long-Context LLM Inference",
// Technical Summary, Methodology: MISA -- Sparse Token Scoring).  For a
// prefill chunk of thousands of queries the score matrix is a gigabyte;
// reading it back costs more than a quarter of the step.  Instead:
//
//  1. tlist_gather_kernel copies NS keys spread evenly over the shortest
//     prefix of the chunk into a small contiguous cache (and a position
//     array that makes every sampled key visible to every row);
//  2. the prefill scoring kernel scores every row against that sample
//     (the same MFMA tiling, NS columns);
//  3. tlist_tau_kernel takes, per row, the r-th largest sample score with
//     r = m + 4 sqrt(m) + 8 for m = k NS / n_row: about r n / NS of the
//     row's scores reach it, and fewer than k only four standard deviations
//     out on unstructured scores;
//  4. the full scoring pass writes no score rows: every score >= tau goes
//     to the row's list for its key split (prefill.hip);
//  5. tlist_merge_kernel, one workgroup per row: the union of the row's
//     lists is exactly the set of its scores >= tau; when none overflowed
//     and it holds at least k entries, its top-k is the row's top-k, found
//     by radix digits of the composite (score, column) keys.  Otherwise the
//     row goes on the merge's list of flagged rows, which are rescored one
//     by one (score_rows_kernel) and take the row select
//     (topk_flagged_kernel).
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace misa {

// ------------------------------------------------------------------ sample
// Grid: enough 256-thread workgroups to copy NS keys; each also reduces the
// rows' shortest prefix itself (T positions, cheap) so no pass precedes it.
__global__ __launch_bounds__(256) void tlist_gather_kernel(const uint16_t *keys, const int32_t *q_pos,
                                                           int T, int Lmax, int ns, uint16_t *sample,
                                                           int32_t *spos, uint32_t *fcount) {
  __shared__ int smin;
  const int tid = threadIdx.x;
  if (tid == 0) smin = 0x7FFFFFFF;
  __syncthreads();
  int m = 0x7FFFFFFF;
#pragma unroll 8
  for (int t = tid; t < T; t += 256) m = min(m, q_pos[t]);
  atomicMin(&smin, m);
  __syncthreads();
  // every row sees keys 0 .. n-1 (at least key 0, at most the cache)
  const int64_t n = min(max((int64_t)smin + 1, (int64_t)1), (int64_t)Lmax);
  // thread = (sample key j, 16-byte chunk c)
  for (int i = blockIdx.x * 256 + tid; i < ns * 16; i += gridDim.x * 256) {
    const int j = i >> 4, c = i & 15;
    const int64_t p = (int64_t)j * n / ns;
    ((uint4 *)sample)[(size_t)j * 16 + c] = ((const uint4 *)keys)[(size_t)p * 16 + c];
  }
  if (blockIdx.x == 0) {
    for (int t = tid; t < T; t += 256) spos[t] = ns - 1;
    if (tid == 0) *fcount = 0;  // the merge's list of flagged rows starts empty
  }
}

// One wave per row, four rows per workgroup: tau[t] = the r-th largest of
// the row's NS sample scores, its order key rounded down to a multiple of
// 65536 (a lower bound, at most about 1% below that score: the float keeps
// its sign, exponent and 7 mantissa bits): the largest such key K with at
// least r sample keys >= K, found bit by bit from the top, each step one
// count over the row.
// r >= NS (a short row) gives -inf: every score is kept.
template <int NS>
__global__ __launch_bounds__(256) void tlist_tau_kernel(const float *ss, const int32_t *q_pos, int T, int k,
                                                        float *tau) {
  constexpr int PER = NS / kWave;
  static_assert(NS % kWave == 0, "sample shape");
  const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = lane_id();
  if (t >= T) return;  // wave-uniform
  const float n = (float)max(q_pos[t], 0) + 1.f;
  const float m = (float)k * (float)NS / n;
  const float rf = ceilf(m + kTlistSigma * sqrtf(m) + 8.f);
  if (rf >= (float)NS) {
    if (lane == 0) tau[t] = -INFINITY;
    return;
  }
  const uint32_t r = (uint32_t)rf;
  const float *row = ss + (size_t)t * NS;
  uint32_t key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) key[u] = order_key(row[lane + kWave * u]);
  uint32_t K = 0;
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t cand = K | (1u << bit);
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) c += key[u] >= cand ? 1u : 0u;
    c = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(c), kWave - 1);
    if (c >= r) K = cand;
  }
  if (lane == 0) tau[t] = key_to_float(K);
}

// ------------------------------------------------------------------- merge
// One 256-thread workgroup per row.  The row's lists (one per key split,
// contiguous) are loaded into registers in one round: list s takes slots
// [first_s, first_s + ceil(len_s / 256)) of every thread, slot u of thread
// i holding entry (u - first_s) 256 + i.  Their keys go into a histogram of
// 4096 bins over the union's own key range [tau, largest key]; the bin
// holding the kk-th key is ranked among itself (at most 256 keys, else the
// row is flagged), giving the kk-th composite key K, and every entry >= K is
// written, positions from a block scan.
constexpr int kTmThreads = kTlistMergeThreads;
constexpr int kTmPer = kTlistUnionCap / kTmThreads;

__global__ __launch_bounds__(kTmThreads) void tlist_merge_kernel(TlistArgs a) {
  constexpr int NT = kTmThreads, NW = NT / kWave, PER = kTmPer, NB = kHistBins;
  static_assert(kMaxTlists <= kWave && PER <= NT, "one wave scans the lists");
  __shared__ alignas(16) uint32_t lh[NB];  // histogram, then the crossing bin's keys (64-bit)
  __shared__ uint32_t sh[NW + 8];
  __shared__ uint32_t slen[kMaxTlists], sfirst[kMaxTlists];
  __shared__ alignas(8) uint32_t red[4];  // [0] overflow [1] largest key [2] crossing-bin keys; then K
  const int r = blockIdx.x, tid = threadIdx.x, lane = lane_id();
  const int ns = a.nsplit;
  uint32_t *flag = a.counters + (size_t)r * kRowCounters + 7;
  int32_t *irow = a.idx + (size_t)r * a.k;
  float *vrow = a.val ? a.val + (size_t)r * a.k : nullptr;
  const int n = max(0, min(a.ld, a.q_pos[r] + 1));
  const uint32_t kk = (uint32_t)min(a.k, n);
  const float tau = a.tau[r];
  // the row goes to the row select: flag it and append it to the row list
  auto flag_row = [&]() {
    if (tid == 0) {
      *flag = 1u;
      a.flist[atomicAdd(a.fcount, 1u)] = r;
    }
  };

  for (int i = tid; i < NB; i += NT) lh[i] = 0;
  if (tid < 4) red[tid] = 0;
  __syncthreads();
  if (tid < kWave) {  // wave 0: the lists' lengths and first slots
    const uint32_t c = tid < ns ? a.tcount[(size_t)tid * a.T + r] : 0u;
    const uint32_t len = min(c, (uint32_t)a.tcap), nslot = (len + NT - 1) / NT;
    const uint32_t ie = wave_incl_scan(len), is = wave_incl_scan(nslot);
    if (tid < ns) {
      slen[tid] = len;
      sfirst[tid] = is - nslot;
    }
    if (c > (uint32_t)a.tcap) red[0] = 1;  // a list overflowed
    if (tid == kWave - 1) {
      sh[NW] = ie;
      sh[NW + 1] = is;
    }
  }
  __syncthreads();
  const uint32_t total = __builtin_amdgcn_readfirstlane(sh[NW]);
  const uint32_t slots = __builtin_amdgcn_readfirstlane(sh[NW + 1]);
  // the union holds every score >= tau: its top-k is the row's when it holds
  // at least kk of them and none was dropped
  const bool ok = red[0] == 0 && total >= kk && slots <= (uint32_t)PER && tau > -INFINITY;
  if (!ok) {  // uniform: the row select on the rescored row
    flag_row();
    return;
  }
  // the entries as composite keys (order key << 32 | ~column).  Lane l of
  // every wave holds list l's first slot and length; slot u's list is the
  // last one starting at or before u (a ballot), its figures read from that
  // lane -- all wave-uniform
  const uint32_t klo = order_key(tau);
  const uint32_t my_first = lane < ns ? sfirst[lane] : 0xFFFFFFFFu, my_len = lane < ns ? slen[lane] : 0u;
  uint64_t ck[PER];
  uint32_t valid = 0, kmax = 0;
  {
    uint2 e[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const uint64_t starts = __ballot(my_first <= (uint32_t)u);
      const int l = starts ? 63 - __clzll((long long)starts) : 0;
      const uint32_t first = (uint32_t)__builtin_amdgcn_readlane((int)my_first, l);
      const uint32_t len = (uint32_t)__builtin_amdgcn_readlane((int)my_len, l);
      const uint32_t j = (starts ? (uint32_t)u - first : 0u) * NT + tid;
      const bool v = u < (int)slots && j < len;
      if (v) valid |= 1u << u;
      // (a slot of a list past its entries reads the list's first; slots past
      // the row's last list load nothing: `slots` is uniform)
      e[u] = make_uint2(0u, 0u);
      if (u < (int)slots) e[u] = a.tlists[((size_t)l * a.T + r) * a.tcap + (v ? j : 0u)];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const uint32_t key = order_key(__uint_as_float(e[u].x));
      const bool v = (valid >> u) & 1u;
      ck[u] = v ? composite(key, (int)e[u].y) : 0ull;
      kmax = max(kmax, v ? key : 0u);
    }
  }
  kmax = wave_max_u32(kmax);
  if (lane == 0) atomicMax(&red[1], kmax);
  if (kk == 0) {  // uniform: nothing to select
    for (int i = tid; i < a.k; i += NT) {
      irow[i] = -1;
      if (vrow) vrow[i] = -INFINITY;
    }
    if (tid == 0) *flag = 0u;
    return;
  }
  __syncthreads();
  const uint32_t khi = max((uint32_t)__builtin_amdgcn_readfirstlane(red[1]), klo);
  // The kk-th composite key: 12-bit digits of (key - lo) over a range
  // [lo, lo + 2^wb) that holds it -- first the union's own range (its keys
  // from klo to khi, any column), then the crossing digit's -- until the
  // crossing digit holds at most NT keys, which are ranked among themselves.
  // Composite keys are distinct (one per column), so this ends by the digit
  // of single keys at the latest.
  uint64_t lo = (uint64_t)klo << 32;
  int wb = 32 + (khi > klo ? 32 - (int)__clz(khi - klo) : 0);
  uint32_t need = kk, inb = 0;
  auto in_range = [&](uint64_t c) { return c >= lo && (wb >= 64 || ((c - lo) >> wb) == 0); };
  for (int pass = 0;; ++pass) {
    const int ds = max(wb - kHistBits, 0);
    if (pass > 0) {
      for (int i = tid; i < NB; i += NT) lh[i] = 0;
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (((valid >> u) & 1u) && in_range(ck[u])) atomicAdd(&lh[(uint32_t)((ck[u] - lo) >> ds)], 1u);
    __syncthreads();
    const Thresh th = threshold_from_lds<NT>(lh, need, sh);
    lo += (uint64_t)__builtin_amdgcn_readfirstlane(th.b1) << ds;
    need -= (uint32_t)__builtin_amdgcn_readfirstlane(th.above);
    inb = (uint32_t)__builtin_amdgcn_readfirstlane(th.eq);
    wb = ds;
    if (inb <= (uint32_t)NT || ds == 0) break;
  }
  if (inb > (uint32_t)NT) {  // uniform: equal composite keys, which valid lists never hold
    flag_row();
    return;
  }
  if (tid == 0) {
    *flag = 0u;
    red[0] = red[1] = 0xFFFFFFFFu;  // no composite key is all ones (NaN never reaches tau)
  }
  // the crossing digit's keys into the histogram's words, ranked among themselves
  uint64_t *bkeys = (uint64_t *)lh;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bool inbin = ((valid >> u) & 1u) && in_range(ck[u]);
    const uint64_t msk = __ballot(inbin);
    if (msk) {
      const int leader = __ffsll((unsigned long long)msk) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&red[2], (uint32_t)__popcll(msk));
      const uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)base, leader) + lanes_below(msk);
      if (inbin) bkeys[pos] = ck[u];
    }
  }
  __syncthreads();
  if ((uint32_t)tid < inb) {
    const uint64_t mine = bkeys[tid];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < inb; ++j) rank += bkeys[j] > mine ? 1u : 0u;
    if (rank == need - 1u) ((uint64_t *)red)[0] = mine;
  }
  __syncthreads();
  const uint64_t kth = ((const uint64_t *)red)[0];
  if (kth == ~0ull) {  // uniform: no key of rank kk, which valid lists always have
    flag_row();
    return;
  }
  // every key >= K: exactly kk of them.  Output order is free: wave w's
  // selected entries of slot u follow those of its slots < u, the waves'
  // runs one after another -- staged in the (now free) histogram words when
  // they fit, then written with coalesced stores, else written directly.
  const bool stage = kk <= (uint32_t)(NB / 2);  // uniform
  uint32_t wtot = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    wtot += (uint32_t)__popcll(__ballot(((valid >> u) & 1u) && ck[u] >= kth));
  const int wave = tid >> 6;
  if (lane == 0) sh[wave] = wtot;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) base += w < wave ? sh[w] : 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bool s_u = ((valid >> u) & 1u) && ck[u] >= kth;
    const uint64_t m = __ballot(s_u);
    const uint32_t pos = base + lanes_below(m);
    if (s_u && pos < kk) {  // (exactly kk are selected; the bound keeps a bad list in the row)
      if (stage) {
        bkeys[pos] = ck[u];
      } else {
        irow[pos] = (int32_t)(~(uint32_t)ck[u]);
        if (vrow) vrow[pos] = key_to_float((uint32_t)(ck[u] >> 32));
      }
    }
    base += (uint32_t)__popcll(m);
  }
  if (stage) {
    __syncthreads();
    for (uint32_t i = (uint32_t)tid; i < kk; i += NT) {
      const uint64_t c = bkeys[i];
      irow[i] = (int32_t)(~(uint32_t)c);
      if (vrow) vrow[i] = key_to_float((uint32_t)(c >> 32));
    }
  }
  for (int i = (int)kk + tid; i < a.k; i += NT) {
    irow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
}

hipError_t launch_tlist_gather(const uint16_t *keys, const int32_t *q_pos, int T, int Lmax, int ns,
                               uint16_t *sample, int32_t *spos, uint32_t *fcount, hipStream_t st) {
  if (T < 1 || Lmax < 1 || ns < 1) return hipErrorInvalidValue;
  const int grid = (ns * 16 + 255) / 256;
  hipLaunchKernelGGL(tlist_gather_kernel, dim3(grid < 64 ? grid : 64), dim3(256), 0, st, keys, q_pos, T, Lmax,
                     ns, sample, spos, fcount);
  return hipGetLastError();
}

hipError_t launch_tlist_tau(const float *ss, const int32_t *q_pos, int T, int ns, int k, float *tau,
                            hipStream_t st) {
  if (ns != kTlistSample || T < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tlist_tau_kernel<kTlistSample>, dim3((T + 3) / 4), dim3(256), 0, st, ss, q_pos, T, k, tau);
  return hipGetLastError();
}

hipError_t launch_tlist_merge(const TlistArgs &a, hipStream_t st) {
  if (a.nsplit < 1 || a.nsplit > kMaxTlists || a.tcap < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tlist_merge_kernel, dim3(a.T), dim3(kTmThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
