// api.hip -- the C ABI (include/misa_indexer.h): argument validation,
// workspace layout and kernel launch sequences.  Every check runs before
// any HIP call; every call only enqueues work on the caller's stream.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

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

int hist_chunk(int rows, int ncols) {
  // about 1024 workgroups; many rows -> whole rows per workgroup, so each
  // non-empty bin is merged into the row histogram once
  const size_t work = (size_t)rows * ncols;
  size_t c = (work + 1023) / 1024;
  c = (c + 255) / 256 * 256;
  c = std::max<size_t>(4096, std::min<size_t>((size_t)ncols, c));
  return (int)c;
}

int filter_chunk(int rows, int ncols) {
  // about 512 filter workgroups, each a multiple of 4096 columns (one round)
  const int per_row = std::max(1, 512 / std::max(1, rows));
  int c = (ncols + per_row - 1) / per_row;
  c = (c + 4095) / 4096 * 4096;
  return std::max(4096, c);
}

// Layout of the selection workspace for `rows` score rows of `ld` columns:
// fp32 score rows (when the call computes them), the first-digit histograms
// and per-row counters (zeroed together by the call), and the per-row
// threshold-digit candidate lists.
struct SelectLayout {
  size_t scores, hist, counters, cand, total;
  int cap;
};
SelectLayout select_layout(size_t rows, size_t ld, int k, bool with_scores) {
  (void)k;
  SelectLayout L;
  L.cap = (int)std::min<size_t>(ld, 16384);
  size_t off = 0;
  L.scores = off;
  if (with_scores) off = align_up(off + rows * ld * sizeof(float));
  L.hist = off;
  off = align_up(off + rows * kHistBins * sizeof(uint32_t));
  L.counters = off;  // directly after the histograms: one fill clears both
  off = align_up(off + rows * kRowCounters * sizeof(uint32_t));
  L.cand = off;
  off = align_up(off + rows * (size_t)L.cap * sizeof(uint2));
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

int score_chunk(int rows, int ncols) {
  // about 512 workgroups over the whole launch (two per CU), 256..4096 columns each
  const size_t work = (size_t)rows * ncols;
  size_t c = (work + 511) / 512;
  c = (c + 255) / 256 * 256;
  c = std::max<size_t>(256, std::min<size_t>(4096, c));
  return (int)c;
}

// Many queries of one sequence with a few routed heads: the dense MFMA
// tiling of prefill.hip.  Otherwise each query row streams the keys itself.
constexpr int kPrefillMinRows = 64;
bool use_prefill(const misa_batch *b, const int32_t *heads, int h) {
  return heads && b->S == 1 && b->T >= kPrefillMinRows && prefill_supported(h, b->Lmax, b->Lmax);
}

PrefillArgs make_prefill_args(const misa_batch *b, const int32_t *heads, int h, float *scores) {
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
  // about one workgroup per compute unit (one fits at a time: its A rows fill
  // the registers): query tiles x key splits of whole key tiles
  const int nqt = (b->T + prefill_queries_per_wg(h) - 1) / prefill_queries_per_wg(h);
  const int nsplit = std::max(1, std::min((b->Lmax + 1023) / 1024, (256 + nqt / 2) / nqt));
  int split = (b->Lmax + nsplit - 1) / nsplit;
  p.split = (split + kPrefillKeyTile - 1) / kPrefillKeyTile * kPrefillKeyTile;
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MISA_OK : MISA_ERR_HIP; }

// Selection over rows of ld columns.  Few long rows: zero the histograms ->
// [score rows + histogram | histogram] -> multi-workgroup filter -> finish.
// Enough rows to fill the GPU, or short rows: [score rows] -> one workgroup
// per row.
constexpr int kRowSelectMinRows = 256;
// Rows this short are one workgroup's work whatever their number: a single
// select kernel beats the fill + histogram + filter + finish chain.
constexpr int kRowSelectMaxShortRow = 16384;

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
               void *ev_start = nullptr, void *ev_stop = nullptr, bool zeroed = false) {
  const bool row_mode = rows >= kRowSelectMinRows || ld <= kRowSelectMaxShortRow;
  uint32_t *hist = (uint32_t *)((char *)ws + L.hist);
  hipError_t e = hipSuccess;
  if (!zeroed && !row_mode) {  // the fused indexer call clears these in its router kernel
    e = launch_fill_u32(hist, (L.cand - L.hist) / sizeof(uint32_t), 0u, st);
    if (e != hipSuccess) return MISA_ERR_HIP;
  }
  TopkArgs t{};
  t.counters = (uint32_t *)((char *)ws + L.counters);
  t.cand = (uint2 *)((char *)ws + L.cand);
  t.cap = L.cap;
  t.scores = score ? score->scores : scores_in;
  t.row_len = row_len;
  t.row_len_add = row_len_add;
  t.map = map;
  t.hist = hist;
  t.idx = idx;
  t.val = val;
  t.rows = rows;
  t.ld = ld;
  t.k = k;
  if (score) {
    ScoreArgs s = *score;
    s.hist = row_mode ? nullptr : hist;
    e = launch_score_rows(s, st, (hipEvent_t)ev_start, (hipEvent_t)ev_stop);
    if (e != hipSuccess) return MISA_ERR_HIP;
  }
  if (row_mode) {
    // many long rows without a column map: the streamed select, then the
    // register-resident select on the rows it could not settle
    if (rows >= kRowSelectMinRows && !map && ld % 4 == 0 && ((uintptr_t)t.scores & 15) == 0 &&
        ld >= kStreamSelectMinCols && ld <= kStreamSelectMaxCols && stream_select_fits(k, ld)) {
      if ((e = launch_topk_stream(t, st)) != hipSuccess) return MISA_ERR_HIP;
      t.only_flagged = 1;
    }
    return hip_status(launch_topk_rowselect(t, st));
  }
  if (!score) {
    t.chunk = hist_chunk(rows, ld);
    if ((e = launch_topk_hist(t, hist, st)) != hipSuccess) return MISA_ERR_HIP;
  }
  t.chunk = filter_chunk(rows, ld);
  if ((e = launch_topk_select(t, st)) != hipSuccess) return MISA_ERR_HIP;
  return MISA_OK;
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
      *bytes = select_layout(b->T, b->Lmax, k, true).total;
      return MISA_OK;
    case MISA_OP_RERANK:
      if (k < 1 || kc < k || kc > b->Lmax) return MISA_ERR_SHAPE;
      *bytes = select_layout(b->T, kc, k, true).total;
      return MISA_OK;
    case MISA_OP_INDEXER:
      if (B < 1 || B > b->Lmax || h < 1 || h > b->H || k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
      *bytes = route_bytes(b, B) + select_layout(b->T, b->Lmax, k, true).total;
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
hipError_t dispatch_route(const misa_batch *b, const RouteArgs &a, hipStream_t st, bool &zeroed) {
  if (b->S == 1 && b->T >= kRouteTileMinRows && b->H <= 64) {
    zeroed = false;
    return launch_route_tile(a, st);
  }
  zeroed = a.zero_hist != nullptr;
  return launch_route(a, st);
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
  bool zeroed;
  return hip_status(dispatch_route(b, a, (hipStream_t)stream, zeroed));
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
  s.hist = nullptr;
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax);
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
  if (ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  if (use_prefill(b, heads, h)) {
    float *sc = (float *)((char *)ws + L.scores);
    if (launch_score_prefill(make_prefill_args(b, heads, h, sc), (hipStream_t)stream,
                             (hipEvent_t)ev_start, (hipEvent_t)ev_stop) != hipSuccess)
      return MISA_ERR_HIP;
    return run_select(nullptr, sc, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, ws, L,
                      (hipStream_t)stream);
  }
  ScoreArgs s = make_score_args(b, heads, heads ? h : b->H);
  s.scores = (float *)((char *)ws + L.scores);
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax);
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

int misa_indexer_ev(const misa_batch *b, const float *pooled, int32_t B, int32_t h, int32_t mode,
                    int32_t k, int32_t *heads, float *head_score, int32_t *idx, float *val,
                    void *ws, size_t ws_bytes, void *stream, void *ev_start, void *ev_stop) {
  int rc = check_batch(b, true);
  if (rc) return rc;
  if (!pooled || !heads || !idx || !ws) return MISA_ERR_NULL;
  if (!a16(pooled) || !a16(ws)) return MISA_ERR_UNSUPPORTED;
  if (B < 1 || B > b->Lmax || h < 1 || h > b->H) return MISA_ERR_SHAPE;
  if (mode != 0 && mode != 1) return MISA_ERR_SHAPE;
  if (k < 1 || k > b->Lmax) return MISA_ERR_SHAPE;
  const size_t rbytes = route_bytes(b, B);
  const SelectLayout L = select_layout(b->T, b->Lmax, k, true);
  if (ws_bytes < rbytes + L.total) return MISA_ERR_WORKSPACE;
  void *sws = (char *)ws + rbytes;
  RouteArgs ra = make_route_args(b, pooled, B, h, mode, heads, head_score, ws);
  ra.zero_hist = (uint32_t *)((char *)sws + L.hist);
  ra.zero_ctr = (uint32_t *)((char *)sws + L.counters);
  bool zeroed;
  if (dispatch_route(b, ra, (hipStream_t)stream, zeroed) != hipSuccess) return MISA_ERR_HIP;
  if (use_prefill(b, heads, h)) {
    float *sc = (float *)((char *)sws + L.scores);
    if (launch_score_prefill(make_prefill_args(b, heads, h, sc), (hipStream_t)stream,
                             (hipEvent_t)ev_start, (hipEvent_t)ev_stop) != hipSuccess)
      return MISA_ERR_HIP;
    return run_select(nullptr, sc, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, sws, L,
                      (hipStream_t)stream, nullptr, nullptr, zeroed);
  }
  ScoreArgs s = make_score_args(b, heads, h);
  s.scores = (float *)((char *)sws + L.scores);
  s.cand = nullptr;
  s.ncols = b->Lmax;
  s.ld = b->Lmax;
  s.chunk = score_chunk(b->T, b->Lmax);
  return run_select(&s, nullptr, b->T, b->Lmax, b->q_pos, 1, nullptr, k, idx, val, sws, L,
                    (hipStream_t)stream, ev_start, ev_stop, zeroed);
}

int misa_indexer(const misa_batch *b, const float *pooled, int32_t B, int32_t h, int32_t mode,
                 int32_t k, int32_t *heads, float *head_score, int32_t *idx, float *val, void *ws,
                 size_t ws_bytes, void *stream) {
  return misa_indexer_ev(b, pooled, B, h, mode, k, heads, head_score, idx, val, ws, ws_bytes,
                         stream, nullptr, nullptr);
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
  a.nchunks = (a.Mmax + kRouteChunk - 1) / kRouteChunk;
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
