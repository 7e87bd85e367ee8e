// api.hip -- the C ABI (include/misa_indexer.h): argument validation,
// workspace layout and kernel launch sequences.  Every check runs before
// any HIP call; every call only enqueues work on the caller's stream.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/misa_indexer.h"
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

using namespace misa;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxRows = 65535;  // rows go on grid dimension y

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Keys, queries, pooled keys, workspaces and misa_score's output are moved in
// 16-byte vectors: their base addresses must be 16-byte aligned.
bool a16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int check_batch(const misa_batch *b, bool need_q) {
  if (!b) return MISA_ERR_NULL;
  if (!b->keys) return MISA_ERR_NULL;
  if (need_q && (!b->q || !b->w || !b->q_seq || !b->q_pos)) return MISA_ERR_NULL;
  if (b->d != MISA_D) return MISA_ERR_UNSUPPORTED;
  if (!a16(b->keys) || (need_q && !a16(b->q))) return MISA_ERR_UNSUPPORTED;
  if (b->S < 1 || b->Lmax < 1) return MISA_ERR_SHAPE;
  if (need_q) {
    if (b->T < 1 || b->H < 1) return MISA_ERR_SHAPE;
    if (b->H > MISA_MAX_HEADS) return MISA_ERR_UNSUPPORTED;
    if (b->T > kMaxRows) return MISA_ERR_UNSUPPORTED;
  }
  return MISA_OK;
}

int score_chunk(int rows, int ncols, bool wide = false) {
  // about 512 workgroups over the whole launch (two per CU), 256..4096 columns
  // each; 256 for direct rows of more than 16 head slots (the four-wave
  // kernel, whose per-workgroup prologue and epilogue weigh more than a
  // second wave per SIMD: 58.4 -> 57.0 us at 32 x 32768 keys, 64 heads)
  const size_t work = (size_t)rows * ncols;
  const size_t target = wide ? 256 : 512;
  size_t c = (work + target - 1) / target;
  c = (c + 255) / 256 * 256;
  c = std::max<size_t>(256, std::min<size_t>(4096, c));
  return (int)c;
}

// Selection over rows of ld columns.  Few long rows: the two-stage select --
// [score rows + chunk lists | chunk lists of the given scores] -> merge.
// Enough rows to fill the GPU, or short rows: [score rows] -> one workgroup
// per row (topk_rowselect_kernel, after the streamed select for long rows).
constexpr int kRowSelectMinRows = 256;
// Rows this short are one workgroup's work whatever their number.
constexpr int kRowSelectMaxShortRow = 16384;

// The two-stage select takes few long rows whose lists are expected to fit
// the merge's LDS: about k + nwg (6 sqrt(k / nwg) + 16) entries per row,
// with room to spare.
bool list_mode(int rows, int ld, int k) {
  if (rows >= kRowSelectMinRows || ld <= kRowSelectMaxShortRow) return false;
  const int cs = score_chunk(rows, ld);
  const int nwg = std::max((ld + cs - 1) / cs, (ld + kListChunk - 1) / kListChunk);
  if (nwg > kMaxLists) return false;
  const double e = (double)k / nwg;
  return (double)k + nwg * (6.0 * std::sqrt(e) + 17.0) <= 0.85 * 16384.0;
}

// Layout of the selection workspace for `rows` score rows of `ld` columns:
// fp32 score rows (when the call computes them), per-row counters (the
// streamed select's flags), and in the two-stage mode the chunk lists
// (at most ld + 4096 entries per row, whatever the chunk) and their headers.
struct SelectLayout {
  size_t scores, counters, lhead, lists, total;
  bool lists_on;
};
SelectLayout select_layout(size_t rows, size_t ld, int k, bool with_scores) {
  SelectLayout L;
  L.lists_on = list_mode((int)std::min<size_t>(rows, 1u << 30), (int)std::min<size_t>(ld, 1u << 30), k);
  size_t off = 0;
  L.scores = off;
  if (with_scores) off = align_up(off + rows * ld * sizeof(float));
  L.counters = off;
  off = align_up(off + rows * kRowCounters * sizeof(uint32_t));
  L.lhead = off;
  if (L.lists_on) off = align_up(off + rows * (size_t)kMaxLists * sizeof(uint4));
  L.lists = off;
  if (L.lists_on) off = align_up(off + rows * (ld + (size_t)kListChunk) * sizeof(uint2));
  L.total = off;
  return L;
}

size_t route_bytes(const misa_batch *b, int B) {
  const int Mmax = (b->Lmax + B - 1) / B;
  const int nchunks = (Mmax + kRouteChunk - 1) / kRouteChunk;
  return align_up((size_t)b->T * (nchunks + 1) * b->H * sizeof(float));
}

// The hierarchical indexer's workspace: block scores, block counts, kept
// blocks, candidate tokens, then the block select and the token select.
struct HisaLayout {
  size_t bscore, mt, kept, cand, bsel, tsel, total;
  SelectLayout LB, LT;
};
HisaLayout hisa_layout(const misa_batch *b, int B, int m, int k) {
  HisaLayout H;
  const size_t T = (size_t)b->T, Mmax = (size_t)(b->Lmax + B - 1) / B, kc = (size_t)m * B;
  size_t off = 0;
  H.bscore = off;
  off = align_up(off + T * Mmax * sizeof(float));
  H.mt = off;
  off = align_up(off + T * sizeof(int32_t));
  H.kept = off;
  off = align_up(off + T * (size_t)m * sizeof(int32_t));
  H.cand = off;
  off = align_up(off + T * kc * sizeof(int32_t));
  H.LB = select_layout(T, Mmax, m, false);
  H.bsel = off;
  off = align_up(off + H.LB.total);
  H.LT = select_layout(T, kc, k, true);
  H.tsel = off;
  off = align_up(off + H.LT.total);
  H.total = off;
  return H;
}

// Many queries of one sequence, routed (h heads) or dense (every head,
// heads == nullptr): the MFMA tiling of prefill.hip, for up to 64 head slots
// per query.  Otherwise each query row streams the keys itself.
constexpr int kPrefillMinRows = 64;
bool use_prefill(const misa_batch *b, const int32_t *heads, int h) {
  const int nh = heads ? h : b->H;
  return b->S == 1 && b->T >= kPrefillMinRows && prefill_supported(nh, b->Lmax, b->Lmax);
}

// Key columns per prefill workgroup: about one workgroup per compute unit
// (one fits at a time: its A rows fill the registers), query tiles x key
// splits of whole key tiles.
int prefill_split(int T, int h, int Lmax) {
  const int nqt = (T + prefill_queries_per_wg(h) - 1) / prefill_queries_per_wg(h);
  const int nsplit = std::max(1, std::min((Lmax + 1023) / 1024, (256 + nqt / 2) / nqt));
  const int split = (Lmax + nsplit - 1) / nsplit;
  return (split + kPrefillKeyTile - 1) / kPrefillKeyTile * kPrefillKeyTile;
}

PrefillArgs make_prefill_args(const misa_batch *b, const int32_t *heads, int h, float *scores) {
  if (!heads) h = b->H;  // dense: every head
  PrefillArgs p{};
  p.keys = b->keys;
  p.q = b->q;
  p.w = b->w;
  p.q_pos = b->q_pos;
  p.heads = heads;
  p.scores = scores;
  p.seq = 0;
  p.h = h;
  p.H = b->H;
  p.Lmax = b->Lmax;
  p.T = b->T;
  p.ld = b->Lmax;
  p.split = prefill_split(b->T, h, b->Lmax);
  return p;
}

// The prefill chunk's select from threshold lists (tlist.hip): the scores of
// kTlistSample keys spread over the shortest prefix give every row a lower
// bound tau of its k-th score; the scoring kernel keeps the scores >= tau in
// one list per (key split, row) of tcap entries besides the score rows, and
// one workgroup per row selects from their union.  The score rows are not
// written: the rows whose lists cannot prove their top-k (a list overflowed,
// fewer than k scores reached tau) are rescored one by one (score_rows_kernel
// over the merge's list of them) and take the row select.  Taken
// for many long rows (where the streamed select would read the whole matrix)
// when the expected union of a row fits the merge's registers.
struct TlistLayout {
  size_t sample, spos, sscore, tau, tcount, tlists, flist, total;
  int nsplit, tcap;
  bool on;
};
TlistLayout tlist_layout(const misa_batch *b, int h, int k) {
  TlistLayout L{};
  const int T = b->T, n = b->Lmax;
  if (!(b->S == 1 && T >= kRowSelectMinRows && n > kRowSelectMaxShortRow && h >= 1 &&
        prefill_supported(h, n, n) && prefill_lists_supported(h) && k >= 1 && k <= n))
    return L;
  const int split = prefill_split(T, h, n);
  L.nsplit = (n + split - 1) / split;
  if (L.nsplit > kMaxTlists) return L;
  // a row of n columns: tau is the r-th of the row's sample scores with
  // m = k NS / n and r = m + sigma sqrt(m) + 8 (tlist_tau_kernel), so about
  // u = r n / NS of its scores reach it, give or take sqrt(r) n / NS
  const double ns = kTlistSample, m = (double)k * ns / n, r = m + kTlistSigma * std::sqrt(m) + 8.0;
  if (r >= ns) return L;
  const double u = r * n / ns, sd = std::sqrt(r) * n / ns;
  if (u + 4.0 * sd > 0.9 * kTlistUnionCap) return L;
  // the merge's register slots: ceil(len / threads) per list
  if ((u + 4.0 * sd) / kTlistMergeThreads + L.nsplit > kTlistUnionCap / kTlistMergeThreads) return L;
  // a list takes one split of one row: u split / n hits on average, with
  // room for rows up to 1.5x as dense (shorter prefixes)
  const double mu = 1.5 * u * split / n;
  L.tcap = ((int)std::ceil(mu + 6.0 * std::sqrt(mu) + 32.0) + 7) / 8 * 8;
  if ((uint64_t)prefill_queries_per_wg(h) * L.tcap * 8 > 0x7FFFFFF0ull) return L;
  size_t off = 0;
  L.sample = off;
  off = align_up(off + (size_t)kTlistSample * MISA_D * sizeof(uint16_t));
  L.spos = off;
  off = align_up(off + (size_t)T * sizeof(int32_t));
  L.sscore = off;
  off = align_up(off + (size_t)T * kTlistSample * sizeof(float));
  L.tau = off;
  off = align_up(off + (size_t)T * sizeof(float));
  L.tcount = off;
  off = align_up(off + (size_t)L.nsplit * T * sizeof(uint32_t));
  L.tlists = off;
  off = align_up(off + (size_t)L.nsplit * T * L.tcap * sizeof(uint2));
  L.flist = off;  // the count, then the flagged rows
  off = align_up(off + (size_t)(T + 1) * sizeof(int32_t));
  L.total = off;
  L.on = true;
  return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MISA_OK : MISA_ERR_HIP; }

// The streamed select keeps the columns at or above a sampled bracket of
// the k-th score in a list of kStreamSelectCap entries per row; a row whose
// list overflows goes on to the row select.  With m = k * sample / ld, the
// list holds about r = m + 4 sqrt(m) + 4 sample ranks' worth of columns,
// r * ld / sample entries with a standard deviation of about
// sqrt(r) * ld / sample; rows take the streamed select when two standard
// deviations above the mean still fit (ld is the longest row: shorter rows
// make smaller lists).
bool stream_select_fits(int k, int ld) {
  const double m = (double)k * kStreamSelectSample / ld;
  const double r = m + 4.0 * std::sqrt(m) + 4.0;
  return (r + 2.0 * std::sqrt(r)) * ld / kStreamSelectSample <= (double)kStreamSelectCap;
}

int run_select(const ScoreArgs *score, const float *scores_in, int rows, int ld,
               const int32_t *row_len, int row_len_add, const int32_t *map, int k,
               int32_t *idx, float *val, void *ws, const SelectLayout &L, hipStream_t st,
               void *ev_start = nullptr, void *ev_stop = nullptr) {
  hipError_t e = hipSuccess;
  TopkArgs t{};
  t.counters = (uint32_t *)((char *)ws + L.counters);
  t.scores = score ? score->scores : scores_in;
  t.row_len = row_len;
  t.row_len_add = row_len_add;
  t.map = map;
  t.idx = idx;
  t.val = val;
  t.rows = rows;
  t.ld = ld;
  t.k = k;
  if (L.lists_on) {
    t.lists = (uint2 *)((char *)ws + L.lists);
    t.lhead = (uint4 *)((char *)ws + L.lhead);
    t.lcap = score ? score->chunk : kListChunk;
    t.nwg = (ld + t.lcap - 1) / t.lcap;
  }
  if (score) {
    ScoreArgs s = *score;
    s.lists = t.lists;
    s.lhead = t.lhead;
    s.lcap = t.lcap;
    s.k = k;
    e = launch_score_rows(s, st, (hipEvent_t)ev_start, (hipEvent_t)ev_stop);
    if (e != hipSuccess) return MISA_ERR_HIP;
  }
  if (L.lists_on) {
    if (!score && (e = launch_topk_lists(t, st)) != hipSuccess) return MISA_ERR_HIP;
    return hip_status(launch_topk_merge(t, st));
  }
  // many long rows without a column map: the streamed select, then the
  // register-resident select on the rows it could not settle
  if (rows >= kRowSelectMinRows && !map && ld % 4 == 0 && ((uintptr_t)t.scores & 15) == 0 &&
      ld >= kStreamSelectMinCols && ld <= kStreamSelectMaxCols && stream_select_fits(k, ld)) {
    if ((e = launch_topk_stream(t, st)) != hipSuccess) return MISA_ERR_HIP;
    t.only_flagged = 1;
  }
  return hip_status(launch_topk_rowselect(t, st));
}

ScoreArgs make_score_args(const misa_batch *b, const int32_t *heads, int nh) {
  ScoreArgs s{};
  s.keys = b->keys;
  s.q = b->q;
  s.w = b->w;
  s.q_seq = b->q_seq;
  s.q_pos = b->q_pos;
  s.heads = heads;
  s.nh = nh;
  s.H = b->H;
  s.Lmax = b->Lmax;
  s.T = b->T;
  return s;
}

// A prefill chunk: the MFMA scoring of prefill.hip, then the select -- from
// threshold lists when TL.on (the tlist workspace follows the select's),
// else over the score matrix.  The events bracket the main scoring kernel.
int prefill_select(const misa_batch *b, const int32_t *heads, int h, int k, int32_t *idx, float *val,
                   void *ws, const SelectLayout &L, const TlistLayout &TL, hipStream_t st, void *ev_start,
                   void *ev_stop) {
  float *sc = (float *)((char *)ws + L.scores);
  PrefillArgs p = make_prefill_args(b, heads, h, sc);
  if (!TL.on) {
    if (launch_score_prefill(p, st, (hipEvent_t)ev_start, (hipEvent_t)ev_stop) != hipSuccess)
      return MISA_ERR_HIP;
    return run_select(nullptr, sc, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, ws, L, st);
  }
  char *tw = (char *)ws + L.total;
  uint16_t *sample = (uint16_t *)(tw + TL.sample);
  int32_t *spos = (int32_t *)(tw + TL.spos);
  float *ss = (float *)(tw + TL.sscore);
  float *tau = (float *)(tw + TL.tau);
  uint32_t *tcount = (uint32_t *)(tw + TL.tcount);
  uint2 *tlists = (uint2 *)(tw + TL.tlists);
  uint32_t *fcount = (uint32_t *)(tw + TL.flist);
  int32_t *flist = (int32_t *)(tw + TL.flist) + 1;
  // the sample's scores: the same tiling over kTlistSample keys every row sees
  if (launch_tlist_gather(b->keys, b->q_pos, b->T, b->Lmax, kTlistSample, sample, spos, fcount, st) !=
      hipSuccess)
    return MISA_ERR_HIP;
  PrefillArgs ps = p;
  ps.keys = sample;
  ps.q_pos = spos;
  ps.scores = ss;
  ps.seq = 0;
  ps.Lmax = ps.ld = kTlistSample;
  ps.split = kTlistSample / 4;  // four key splits: about one workgroup per compute unit at 4096 rows
  if (launch_score_prefill(ps, st) != hipSuccess) return MISA_ERR_HIP;
  if (launch_tlist_tau(ss, b->q_pos, b->T, kTlistSample, k, tau, st) != hipSuccess) return MISA_ERR_HIP;
  // the lists (no score rows)
  p.tau = tau;
  p.tlists = tlists;
  p.tcount = tcount;
  p.tcap = TL.tcap;
  if ((p.Lmax + p.split - 1) / p.split != TL.nsplit) return MISA_ERR_HIP;  // layouts out of step
  if (launch_score_prefill(p, st, (hipEvent_t)ev_start, (hipEvent_t)ev_stop) != hipSuccess)
    return MISA_ERR_HIP;
  TlistArgs ta{};
  ta.tlists = tlists;
  ta.tcount = tcount;
  ta.tau = tau;
  ta.q_pos = b->q_pos;
  ta.counters = (uint32_t *)((char *)ws + L.counters);
  ta.idx = idx;
  ta.val = val;
  ta.T = b->T;
  ta.nsplit = TL.nsplit;
  ta.tcap = TL.tcap;
  ta.ld = b->Lmax;
  ta.k = k;
  ta.flist = flist;
  ta.fcount = fcount;
  if (launch_tlist_merge(ta, st) != hipSuccess) return MISA_ERR_HIP;
  // the rows the lists could not settle (flagged by the merge): their score
  // rows, then the row select over them
  ScoreArgs s = make_score_args(b, heads, h);
  s.scores = sc;
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = kMaxScoreChunk;
  s.rowlist = flist;
  s.rowcount = fcount;
  if (launch_score_rows(s, st) != hipSuccess) return MISA_ERR_HIP;
  TopkArgs t{};
  t.counters = ta.counters;
  t.scores = sc;
  t.row_len = b->q_pos;
  t.row_len_add = 1;
  t.idx = idx;
  t.val = val;
  t.rows = b->T;
  t.ld = b->Lmax;
  t.k = k;
  t.only_flagged = 1;
  return hip_status(launch_topk_rowselect(t, st));
}

// Several query rows per sequence (S > 1, at least two rows per sequence on
// average, up to 64 head slots): the MFMA tiling over a tile table built on
// the device, so that the rows of a sequence share one pass over its keys.
// Rows of one sequence must be contiguous for this to pay; when they are not
// (more tiles than the bound), every row is scored on its own instead.
bool use_grouped(const misa_batch *b, const int32_t *heads, int h) {
  const int nh = heads ? h : b->H;
  return b->S > 1 && b->T >= 2 * b->S && prefill_supported(nh, b->Lmax, b->Lmax);
}
size_t grouped_bytes(const misa_batch *b) {
  return b->S > 1 ? align_up((size_t)b->T * sizeof(int2)) + kAlign : 0;
}

// The grouped scoring's tile table: rows per tile, the grid's bound on the
// tiles, and where the table and its counts sit in its workspace.
struct GroupedTiles {
  int qwg, bound;
  int2 *tiles;
  uint32_t *cnt;
};
GroupedTiles grouped_tiles(const misa_batch *b, int nh, void *gws) {
  GroupedTiles g;
  g.qwg = prefill_group_queries_per_wg(nh);
  g.bound = std::min(b->T, (b->T + g.qwg - 1) / g.qwg + b->S);
  g.tiles = (int2 *)gws;
  g.cnt = (uint32_t *)((char *)gws + align_up((size_t)b->T * sizeof(int2)));
  return g;
}

// The grouped scoring into sc [T][Lmax] (gws: grouped_bytes of workspace);
// tiles_built: the router's final kernel already built the tile table.
int grouped_score(const misa_batch *b, const int32_t *heads, int h, float *sc, void *gws, hipStream_t st,
                  void *ev_start = nullptr, void *ev_stop = nullptr, bool tiles_built = false) {
  const int nh = heads ? h : b->H;
  const GroupedTiles gt = grouped_tiles(b, nh, gws);
  const int bound = gt.bound;
  int2 *tiles = gt.tiles;
  uint32_t *cnt = gt.cnt;
  if (!tiles_built && launch_prefill_tiles(b->q_seq, b->T, nh, bound, tiles, cnt, cnt + 1, st) != hipSuccess)
    return MISA_ERR_HIP;
  PrefillArgs p = make_prefill_args(b, heads, h, sc);
  p.q_seq = b->q_seq;
  p.tiles = tiles;
  p.ntiles = cnt;
  p.ntile_bound = bound;
  // about two four-wave workgroups per compute unit over the tiles, at
  // least 512 keys a split
  const int nsplit = std::max(1, std::min((b->Lmax + 511) / 512, (512 + bound / 2) / bound));
  const int split = (b->Lmax + nsplit - 1) / nsplit;
  p.split = (split + kPrefillKeyTile - 1) / kPrefillKeyTile * kPrefillKeyTile;
  if (launch_score_prefill(p, st, (hipEvent_t)ev_start, (hipEvent_t)ev_stop) != hipSuccess) return MISA_ERR_HIP;
  // rows not contiguous by sequence: each row on its own (cnt[1] = T), else nothing
  ScoreArgs s = make_score_args(b, heads, nh);
  s.scores = sc;
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax, s.nh > 16);
  s.rowcount = cnt + 1;
  return hip_status(launch_score_rows(s, st));
}


}  // namespace

extern "C" {

const char *misa_status_str(int status) {
  switch (status) {
    case MISA_OK: return "ok";
    case MISA_ERR_NULL: return "a required pointer is NULL";
    case MISA_ERR_SHAPE: return "a size or count is out of range";
    case MISA_ERR_UNSUPPORTED: return "unsupported argument (the library does not handle it)";
    case MISA_ERR_WORKSPACE: return "workspace is smaller than required";
    case MISA_ERR_HIP: return "a HIP launch or runtime call failed";
    case MISA_ERR_TOO_LARGE:
      return "the request needs more scratch than the allocation-free call's static buffer holds";
    default: return "unknown status";
  }
}

int misa_workspace_bytes(const misa_batch *b, int32_t op, int32_t B, int32_t h, int32_t k,
                         int32_t kc, size_t *bytes) {
  if (!b || !bytes) return MISA_ERR_NULL;
  if (b->d != MISA_D) return MISA_ERR_UNSUPPORTED;
  if (b->S < 1 || b->Lmax < 1 || b->T < 1 || b->H < 1) return MISA_ERR_SHAPE;
  switch (op) {
    case MISA_OP_ROUTE:
      if (B < 1 || B > b->Lmax || h < 1 || h > b->H) return MISA_ERR_SHAPE;
      *bytes = route_bytes(b, B);
      return MISA_OK;
    case MISA_OP_DENSE:
    case MISA_OP_SCORE_TOPK:
      if (k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
      *bytes = select_layout(b->T, b->Lmax, k, true).total +
               (op == MISA_OP_SCORE_TOPK ? tlist_layout(b, h, k).total : 0) + grouped_bytes(b);
      return MISA_OK;
    case MISA_OP_RERANK:
      if (k < 1 || kc < k || kc > b->Lmax) return MISA_ERR_SHAPE;
      *bytes = select_layout(b->T, kc, k, true).total;
      return MISA_OK;
    case MISA_OP_INDEXER:
      if (B < 1 || B > b->Lmax || h < 1 || h > b->H || k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
      *bytes = route_bytes(b, B) + select_layout(b->T, b->Lmax, k, true).total + tlist_layout(b, h, k).total +
               grouped_bytes(b);
      return MISA_OK;
    case MISA_OP_TOPK:
      if (k < 1) return MISA_ERR_SHAPE;
      *bytes = select_layout(b->T, b->Lmax, k, false).total;
      return MISA_OK;
    case MISA_OP_HISA: {  // kc carries m, the number of kept blocks
      const int Mmax = B >= 1 ? (b->Lmax + B - 1) / B : 0;
      if (B < 1 || B > b->Lmax || kc < 1 || kc > Mmax || k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
      *bytes = hisa_layout(b, B, kc, k).total;
      return MISA_OK;
    }
    default:
      return MISA_ERR_SHAPE;
  }
}

int misa_pool(const misa_batch *b, int32_t B, float *pooled, void *stream) {
  int rc = check_batch(b, false);
  if (rc) return rc;
  if (!b->seq_lens || !pooled) return MISA_ERR_NULL;
  if (!a16(pooled)) return MISA_ERR_UNSUPPORTED;
  if (B < 1 || B > b->Lmax) return MISA_ERR_SHAPE;
  if (b->S > kMaxRows) return MISA_ERR_UNSUPPORTED;
  return hip_status(launch_pool(b->keys, b->seq_lens, b->S, b->Lmax, B, pooled,
                                (hipStream_t)stream));
}

int misa_pool_append(const misa_batch *b, int32_t B, const int32_t *old_lens, int32_t max_new,
                     float *pooled, void *stream) {
  int rc = check_batch(b, false);
  if (rc) return rc;
  if (!b->seq_lens || !old_lens || !pooled) return MISA_ERR_NULL;
  if (!a16(pooled)) return MISA_ERR_UNSUPPORTED;
  if (B < 1 || B > b->Lmax || max_new < 0 || max_new > b->Lmax) return MISA_ERR_SHAPE;
  if (b->S > kMaxRows) return MISA_ERR_UNSUPPORTED;
  return hip_status(launch_pool_append(b->keys, b->seq_lens, old_lens, max_new, b->S, b->Lmax, B,
                                       pooled, (hipStream_t)stream));
}

static RouteArgs make_route_args(const misa_batch *b, const float *pooled, int32_t B, int32_t h,
                                 int32_t mode, int32_t *heads, float *head_score, void *ws) {
  RouteArgs a{};
  a.keys = b->keys;
  a.q = b->q;
  a.w = b->w;
  a.q_seq = b->q_seq;
  a.q_pos = b->q_pos;
  a.pooled = pooled;
  a.partial = (float *)ws;
  a.heads = heads;
  a.g = head_score;
  a.S = b->S;
  a.Lmax = b->Lmax;
  a.T = b->T;
  a.H = b->H;
  a.B = B;
  a.h = h;
  a.mode = mode;
  a.Mmax = (b->Lmax + B - 1) / B;
  a.nchunks = (a.Mmax + kRouteChunk - 1) / kRouteChunk;
  return a;
}

// Many queries of one sequence (a prefill chunk) with at most 64 heads: the
// tiled one-kernel router.  Otherwise the per-query partial + final pair,
// whose final kernel also clears the selection histogram of the fused call.
constexpr int kRouteTileMinRows = 64;
bool route_tiled(const misa_batch *b) { return b->S == 1 && b->T >= kRouteTileMinRows && b->H <= 64; }
hipError_t dispatch_route(const misa_batch *b, const RouteArgs &a, hipStream_t st) {
  return route_tiled(b) ? launch_route_tile(a, st) : launch_route(a, st);
}

int misa_route(const misa_batch *b, const float *pooled, int32_t B, int32_t h, int32_t mode,
               int32_t *heads, float *head_score, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!pooled || !heads || !ws) return MISA_ERR_NULL;
  if (!a16(pooled) || !a16(ws)) return MISA_ERR_UNSUPPORTED;
  if (B < 1 || B > b->Lmax || h < 1 || h > b->H) return MISA_ERR_SHAPE;
  if (mode != 0 && mode != 1) return MISA_ERR_SHAPE;
  if (ws_bytes < route_bytes(b, B)) return MISA_ERR_WORKSPACE;
  const RouteArgs a = make_route_args(b, pooled, B, h, mode, heads, head_score, ws);
  return hip_status(dispatch_route(b, a, (hipStream_t)stream));
}

int misa_score(const misa_batch *b, const int32_t *heads, int32_t h, float *scores,
               void *stream) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!scores) return MISA_ERR_NULL;
  if (!a16(scores)) return MISA_ERR_UNSUPPORTED;
  if (heads && (h < 1 || h > b->H)) return MISA_ERR_SHAPE;
  if (use_prefill(b, heads, h))
    return hip_status(launch_score_prefill(make_prefill_args(b, heads, h, scores),
                                           (hipStream_t)stream));
  ScoreArgs s = make_score_args(b, heads, heads ? h : b->H);
  s.scores = scores;
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax, s.nh > 16);
  return hip_status(launch_score_rows(s, (hipStream_t)stream));
}

int misa_topk(const float *scores, int32_t rows, int32_t ld, const int32_t *row_len, int32_t k,
              int32_t *idx, float *val, void *ws, size_t ws_bytes, void *stream) {
  if (!scores || !row_len || !idx || !ws) return MISA_ERR_NULL;
  if (!a16(ws)) return MISA_ERR_UNSUPPORTED;
  if (rows < 1 || ld < 1 || k < 1) return MISA_ERR_SHAPE;
  if (rows > kMaxRows) return MISA_ERR_UNSUPPORTED;
  const SelectLayout L = select_layout(rows, ld, k, false);
  if (ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  return run_select(nullptr, scores, rows, ld, row_len, 0, nullptr, k, idx, val, ws, L,
                    (hipStream_t)stream);
}

int misa_score_topk_ev(const misa_batch *b, const int32_t *heads, int32_t h, int32_t k,
                       int32_t *idx, float *val, void *ws, size_t ws_bytes, void *stream,
                       void *ev_start, void *ev_stop) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!idx || !ws) return MISA_ERR_NULL;
  if (!a16(ws)) return MISA_ERR_UNSUPPORTED;
  if (heads && (h < 1 || h > b->H)) return MISA_ERR_SHAPE;
  if (k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
  const SelectLayout L = select_layout(b->T, b->Lmax, k, true);
  const TlistLayout TL = heads ? tlist_layout(b, h, k) : TlistLayout{};
  if (ws_bytes < L.total + TL.total + grouped_bytes(b)) return MISA_ERR_WORKSPACE;
  if (use_prefill(b, heads, h))
    return prefill_select(b, heads, h, k, idx, val, ws, L, TL, (hipStream_t)stream, ev_start, ev_stop);
  if (use_grouped(b, heads, h)) {
    float *sc = (float *)((char *)ws + L.scores);
    rc = grouped_score(b, heads, h, sc, (char *)ws + L.total + TL.total, (hipStream_t)stream, ev_start, ev_stop);
    if (rc) return rc;
    return run_select(nullptr, sc, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, ws, L, (hipStream_t)stream);
  }
  ScoreArgs s = make_score_args(b, heads, heads ? h : b->H);
  s.scores = (float *)((char *)ws + L.scores);
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax, s.nh > 16);
  return run_select(&s, nullptr, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, ws, L,
                    (hipStream_t)stream, ev_start, ev_stop);
}

int misa_score_topk(const misa_batch *b, const int32_t *heads, int32_t h, int32_t k,
                    int32_t *idx, float *val, void *ws, size_t ws_bytes, void *stream) {
  return misa_score_topk_ev(b, heads, h, k, idx, val, ws, ws_bytes, stream, nullptr, nullptr);
}

int indexer_dense(const misa_batch *b, int32_t k, int32_t *idx, float *val, void *ws,
                  size_t ws_bytes, void *stream) {
  return misa_score_topk(b, nullptr, 0, k, idx, val, ws, ws_bytes, stream);
}

}  // extern "C"

// misa_indexer's checks of everything but the workspace
static int indexer_check(const misa_batch *b, const float *pooled, int32_t B, int32_t h,
                         int32_t mode, int32_t k, const int32_t *heads, const int32_t *idx) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!pooled || !heads || !idx) return MISA_ERR_NULL;
  if (!a16(pooled)) return MISA_ERR_UNSUPPORTED;
  if (B < 1 || B > b->Lmax || h < 1 || h > b->H) return MISA_ERR_SHAPE;
  if (mode != 0 && mode != 1) return MISA_ERR_SHAPE;
  if (k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
  return MISA_OK;
}

extern "C" {

int misa_indexer_ev(const misa_batch *b, const float *pooled, int32_t B, int32_t h, int32_t mode,
                    int32_t k, int32_t *heads, float *head_score, int32_t *idx, float *val,
                    void *ws, size_t ws_bytes, void *stream, void *ev_start, void *ev_stop) {
  int rc = indexer_check(b, pooled, B, h, mode, k, heads, idx);
  if (rc) return rc;
  if (!ws) return MISA_ERR_NULL;
  if (!a16(ws)) return MISA_ERR_UNSUPPORTED;
  const size_t rbytes = route_bytes(b, B);
  const SelectLayout L = select_layout(b->T, b->Lmax, k, true);
  const TlistLayout TL = tlist_layout(b, h, k);
  if (ws_bytes < rbytes + L.total + TL.total + grouped_bytes(b)) return MISA_ERR_WORKSPACE;
  void *sws = (char *)ws + rbytes;
  RouteArgs ra = make_route_args(b, pooled, B, h, mode, heads, head_score, ws);
  // many queries of one sequence: the tiled router writes the heads; the
  // prefill and grouped tilings read them from memory (the grouped one's
  // tile table built by one more workgroup of the router's final kernel);
  // otherwise the router kernel leaves partial sums that the scoring
  // kernel's prologue reduces and ranks
  const bool tiled_router = route_tiled(b), prefill = use_prefill(b, heads, h);
  const bool grouped = !prefill && use_grouped(b, heads, h);
  if (grouped && !tiled_router) {
    const GroupedTiles gt = grouped_tiles(b, h, (char *)sws + L.total + TL.total);
    ra.tiles = gt.tiles;
    ra.tcount = gt.cnt;
    ra.tqwg = gt.qwg;
    ra.tbound = gt.bound;
  }
  const bool in_prologue = !tiled_router && !prefill && !grouped;
  hipError_t re = tiled_router          ? launch_route_tile(ra, (hipStream_t)stream)
                  : (prefill || grouped) ? launch_route(ra, (hipStream_t)stream)
                                         : launch_route_partial(ra, (hipStream_t)stream);
  if (re != hipSuccess) return MISA_ERR_HIP;
  if (prefill)
    return prefill_select(b, heads, h, k, idx, val, sws, L, TL, (hipStream_t)stream, ev_start, ev_stop);
  if (grouped) {
    float *sc = (float *)((char *)sws + L.scores);
    rc = grouped_score(b, heads, h, sc, (char *)sws + L.total + TL.total, (hipStream_t)stream, ev_start, ev_stop,
                       ra.tiles != nullptr);
    if (rc) return rc;
    return run_select(nullptr, sc, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, sws, L, (hipStream_t)stream);
  }
  ScoreArgs s = make_score_args(b, heads, h);
  if (in_prologue) {  // heads come from the router's partial sums
    s.heads = nullptr;
    s.partial = ra.partial;
    s.nparts = ra.nchunks + 1;
    s.mode = mode;
    s.heads_out = heads;
    s.g_out = head_score;
  }
  s.scores = (float *)((char *)sws + L.scores);
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax, s.nh > 16);
  return run_select(&s, nullptr, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, sws, L,
                    (hipStream_t)stream, ev_start, ev_stop);
}

int misa_indexer(const misa_batch *b, const float *pooled, int32_t B, int32_t h, int32_t mode,
                 int32_t k, int32_t *heads, float *head_score, int32_t *idx, float *val, void *ws,
                 size_t ws_bytes, void *stream) {
  return misa_indexer_ev(b, pooled, B, h, mode, k, heads, head_score, idx, val, ws, ws_bytes,
                         stream, nullptr, nullptr);
}

}  // extern "C"

// ------------------------------------------------- the allocation-free call
// misa_indexer_noalloc's workspace: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes `scratch` itself
// (in host code the name is a host-side stand-in, not a device address): the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// taken once per device on the first call there and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[MISA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, or nullptr on failure.
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace

extern "C" {

int misa_indexer_noalloc(const misa_batch *b, const float *pooled, int32_t B, int32_t h,
                         int32_t mode, int32_t k, int32_t *heads, float *head_score, int32_t *idx,
                         float *val, void *stream) {
  int rc = indexer_check(b, pooled, B, h, mode, k, heads, idx);
  if (rc) return rc;
  size_t need = 0;
  rc = misa_workspace_bytes(b, MISA_OP_INDEXER, B, h, k, 0, &need);
  if (rc) return rc;
  if (need > (size_t)MISA_NOALLOC_SCRATCH_BYTES) return MISA_ERR_TOO_LARGE;
  void *ws = scratch_address();  // the first HIP call
  if (!ws) return MISA_ERR_HIP;
  return misa_indexer_ev(b, pooled, B, h, mode, k, heads, head_score, idx, val, ws,
                         (size_t)MISA_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

int misa_rerank(const misa_batch *b, const int32_t *cand, int32_t kc, int32_t k, int32_t *idx,
                float *val, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!cand || !idx || !ws) return MISA_ERR_NULL;
  if (!a16(ws)) return MISA_ERR_UNSUPPORTED;
  if (k < 1 || kc < k || kc > b->Lmax) return MISA_ERR_SHAPE;
  const SelectLayout L = select_layout(b->T, kc, k, true);
  if (ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  ScoreArgs s = make_score_args(b, nullptr, b->H);
  s.scores = (float *)((char *)ws + L.scores);
  s.cand = cand;
  s.ncols = kc;
  s.ld = kc;
  s.chunk = score_chunk(b->T, kc);
  return run_select(&s, nullptr, b->T, kc, nullptr, 0, cand, k, idx, val, ws, L,
                    (hipStream_t)stream);
}

static HisaArgs make_hisa_args(const misa_batch *b, const float *pooled, int B, const int32_t *heads,
                               int h, void *ws, const HisaLayout &HL, float *bscore) {
  HisaArgs a{};
  a.keys = b->keys;
  a.q = b->q;
  a.w = b->w;
  a.q_seq = b->q_seq;
  a.q_pos = b->q_pos;
  a.pooled = pooled;
  a.heads = heads;
  a.bscore = bscore ? bscore : (float *)((char *)ws + HL.bscore);
  a.mt = (int32_t *)((char *)ws + HL.mt);
  a.S = b->S;
  a.Lmax = b->Lmax;
  a.T = b->T;
  a.H = b->H;
  a.nh = heads ? h : b->H;
  a.B = B;
  a.Mmax = (b->Lmax + B - 1) / B;
  a.nchunks = (a.Mmax + kHisaChunk - 1) / kHisaChunk;
  return a;
}

static int hisa_check(const misa_batch *b, const float *pooled, int B, int m, const int32_t *heads,
                      int h, int k) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!pooled) return MISA_ERR_NULL;
  if (!a16(pooled)) return MISA_ERR_UNSUPPORTED;
  if (B < 1 || B > b->Lmax) return MISA_ERR_SHAPE;
  const int Mmax = (b->Lmax + B - 1) / B;
  if (m < 1 || m > Mmax || k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
  if (heads ? (h < 1 || h > b->H) : h != 0) return MISA_ERR_SHAPE;
  return MISA_OK;
}

// block scores and the m kept blocks (the coarse stage alone)
static int hisa_coarse(const misa_batch *b, const float *pooled, int B, int m, const int32_t *heads,
                       int h, void *ws, const HisaLayout &HL, int32_t *kept, float *bscore,
                       hipStream_t st) {
  const HisaArgs a = make_hisa_args(b, pooled, B, heads, h, ws, HL, bscore);
  if (launch_hisa_blocks(a, st) != hipSuccess) return MISA_ERR_HIP;
  return run_select(nullptr, a.bscore, b->T, a.Mmax, a.mt, 0, nullptr, m, kept, nullptr,
                    (char *)ws + HL.bsel, HL.LB, st);
}

int hisa_blocks(const misa_batch *b, const float *pooled, int32_t B, int32_t m,
                const int32_t *heads, int32_t h, float *block_scores, int32_t *blocks, void *ws,
                size_t ws_bytes, void *stream) {
  int rc = hisa_check(b, pooled, B, m, heads, h, 1);
  if (rc) return rc;
  if (!ws) return MISA_ERR_NULL;
  if (!a16(ws)) return MISA_ERR_UNSUPPORTED;
  const HisaLayout HL = hisa_layout(b, B, m, 1);
  if (ws_bytes < HL.total) return MISA_ERR_WORKSPACE;
  const hipStream_t st = (hipStream_t)stream;
  int32_t *kept = blocks ? blocks : (int32_t *)((char *)ws + HL.kept);
  return hisa_coarse(b, pooled, B, m, heads, h, ws, HL, kept, block_scores, st);
}

int hisa_indexer_ev(const misa_batch *b, const float *pooled, int32_t B, int32_t m,
                    const int32_t *heads, int32_t h, int32_t k, int32_t *idx, float *val, void *ws,
                    size_t ws_bytes, void *stream, void *ev_start, void *ev_stop) {
  int rc = hisa_check(b, pooled, B, m, heads, h, k);
  if (rc) return rc;
  if (!idx || !ws) return MISA_ERR_NULL;
  if (!a16(ws)) return MISA_ERR_UNSUPPORTED;
  const HisaLayout HL = hisa_layout(b, B, m, k);
  if (ws_bytes < HL.total) return MISA_ERR_WORKSPACE;
  const hipStream_t st = (hipStream_t)stream;
  int32_t *kept = (int32_t *)((char *)ws + HL.kept);
  int32_t *cand = (int32_t *)((char *)ws + HL.cand);
  rc = hisa_coarse(b, pooled, B, m, heads, h, ws, HL, kept, nullptr, st);
  if (rc) return rc;
  // token-level refinement: the indexer over the kept blocks' tokens (the
  // scoring kernel expands the block ids and writes the token lists the
  // select maps its columns through)
  const int kc = m * B;
  void *tws = (char *)ws + HL.tsel;
  ScoreArgs s = make_score_args(b, heads, heads ? h : b->H);
  s.scores = (float *)((char *)tws + HL.LT.scores);
  s.cand = nullptr;
  s.kept = kept;
  s.cand_out = cand;
  s.nkept = m;
  s.blk = B;
  s.ncols = kc;
  s.ld = kc;
  s.chunk = score_chunk(b->T, kc);
  return run_select(&s, nullptr, b->T, kc, nullptr, 0, cand, k, idx, val, tws, HL.LT, st, ev_start,
                    ev_stop);
}

int hisa_indexer(const misa_batch *b, const float *pooled, int32_t B, int32_t m,
                 const int32_t *heads, int32_t h, int32_t k, int32_t *idx, float *val, void *ws,
                 size_t ws_bytes, void *stream) {
  return hisa_indexer_ev(b, pooled, B, m, heads, h, k, idx, val, ws, ws_bytes, stream, nullptr,
                         nullptr);
}

}  // extern "C"
