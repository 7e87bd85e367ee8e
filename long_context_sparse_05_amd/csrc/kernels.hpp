// kernels.hpp -- argument blocks and host launchers of the gfx950 kernels.
// Internal to the library: the public boundary is include/misa_indexer.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

// Token scoring over score rows (score.hip).
struct ScoreArgs {
  const uint16_t *keys;    // bf16 [S][Lmax][128]
  const uint16_t *q;       // bf16 [T][H][128]
  const float *w;          // [T][H]
  const int32_t *q_seq;    // [T]
  const int32_t *q_pos;    // [T]
  const int32_t *heads;    // [T][nh] or nullptr (rows 0..nh-1 = heads 0..nh-1)
  const int32_t *cand;     // [T][ncols] token ids (-1 empty) or nullptr (column = token)
  // With kept != nullptr the candidates are the tokens of kept blocks:
  // column c is token kept[t][c / blk] * blk + c % blk (-1 for an empty block
  // slot or past q_pos[t]); the kernel computes them and writes them to
  // cand_out [T][ncols] for the select that follows.
  const int32_t *kept;     // [T][nkept] block ids (-1 empty) or nullptr
  int32_t *cand_out;
  int nkept, blk;
  float *scores;           // [T][ld]
  // Chunk candidate lists for the two-stage top-k (select.hpp), or nullptr:
  // workgroup x of row t writes list [t][x][lcap] and its header [t][x]
  // (entries, cutoff digit), keeping its share of the row's top k.
  uint2 *lists;
  uint4 *lhead;
  int lcap, k;
  // The router's partial sums [T][nparts][H] (route_partial_kernel), or
  // nullptr: the prologue then reduces and ranks them (route_finish.hpp)
  // into the nh routed heads instead of reading `heads`; workgroup 0 of
  // each row writes them to heads_out [T][nh] and g to g_out [T][H].
  const float *partial;
  int nparts, mode;
  int32_t *heads_out;
  float *g_out;
  // A row count (optional; direct rows, nh <= 64): the rows rowlist[0 ..
  // *rowcount) -- rows 0 .. *rowcount-1 when rowlist is nullptr -- are
  // scored instead of rows 0 .. T-1 (T bounds the count).
  const int32_t *rowlist;
  const uint32_t *rowcount;
  int nh, H, Lmax, T;
  int ncols, ld, chunk;
};
constexpr int kMaxScoreChunk = 4096;  // columns per workgroup of score_rows_kernel
// ev0 / ev1 (optional): hipExtLaunchKernelGGL stamps them with the begin of
// the first and the end of the last kernel a launcher issues, so
// hipEventElapsedTime(ev0, ev1) is the kernels' own duration.
hipError_t launch_score_rows(const ScoreArgs &a, hipStream_t st, hipEvent_t ev0 = nullptr,
                             hipEvent_t ev1 = nullptr);

// Routed scoring of many queries of one sequence (prefill.hip).
struct PrefillArgs {
  const uint16_t *keys;    // bf16 [S][Lmax][128]
  const uint16_t *q;       // bf16 [T][H][128]
  const float *w;          // [T][H]
  const int32_t *q_pos;    // [T]
  const int32_t *heads;    // [T][h] routed heads, or nullptr: slot j is head j (dense, h = H)
  float *scores;           // [T][ld]
  int seq;                 // the one sequence all rows read
  int h, H, Lmax, T, ld;
  int split;               // key columns per workgroup, a multiple of 64
  // Threshold lists (optional, tau != nullptr): instead of the score rows
  // (scores is not written), every score >= tau[t] goes to tlists
  // [nsplit][T][tcap] as (score bits, column) -- list [split][t] holds row
  // t's hits in the columns of that split, in no set order -- and the count
  // of hits (which may exceed tcap: the list overflowed) to tcount
  // [nsplit][T].
  const float *tau;
  uint2 *tlists;
  uint32_t *tcount;
  int tcap;
  // Several sequences (optional, tiles != nullptr): workgroup row y takes
  // tile y of the table -- (first row, sequence), the rows from there on
  // with that q_seq, at most the tiling's queries per workgroup -- if y <
  // *ntiles; the grid has ntile_bound rows.  seq is then unused.
  const int32_t *q_seq;
  const int2 *tiles;
  const uint32_t *ntiles;
  int ntile_bound;
};
// The tile table of a batch of several sequences (prefill.hip): runs of
// equal q_seq cut into tiles of prefill_group_queries_per_wg(h) rows.  When the
// rows of a sequence are not contiguous and the tiles would pass `bound`,
// *ntiles = 0 and *fallback = T (the per-row scoring then takes every row);
// else *fallback = 0.
hipError_t launch_prefill_tiles(const int32_t *q_seq, int T, int h, int bound, int2 *tiles, uint32_t *ntiles,
                                uint32_t *fallback, hipStream_t st);
// key tile of the prefill kernel: PrefillArgs::split must be a multiple
constexpr int kPrefillKeyTile = 128;
constexpr int kPrefillMaxHeads = 64;  // head slots per query the tiling takes
hipError_t launch_score_prefill(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0 = nullptr,
                                hipEvent_t ev1 = nullptr);
int prefill_queries_per_wg(int h);
int prefill_group_queries_per_wg(int h);  // with a tile table
bool prefill_supported(int h, int ld, int Lmax);  // the launch shape fits h, the row length and the keys
bool prefill_lists_supported(int h);              // the tiling for h heads can write threshold lists

// Per-row top-k selection (topk.hip).
struct TopkArgs {
  const float *scores;     // [rows][ld]
  const int32_t *row_len;  // [rows] or nullptr (all ld columns)
  int row_len_add;         // valid columns = row_len[r] + row_len_add
  const int32_t *map;      // [rows][ld] column -> token id (-1 = empty) or nullptr
  uint32_t *counters;      // [rows][kRowCounters] (select.hpp)
  // the rows' chunk candidate lists [rows][nwg][lcap] and headers [rows][nwg]
  // (two-stage top-k of few long rows: topk_merge_kernel)
  uint2 *lists;
  uint4 *lhead;
  int nwg, lcap;
  int32_t *idx;            // [rows][k]
  float *val;              // [rows][k] or nullptr
  int rows, ld, k;
  int only_flagged;        // row select: skip rows whose counter 7 is 0 (streamed select done)
};
constexpr int kMaxLists = 1024;   // chunk lists per row the merge takes
constexpr int kListChunk = 4096;  // columns per workgroup of topk_lists_kernel
hipError_t launch_topk_merge(const TopkArgs &a, hipStream_t st);
hipError_t launch_topk_lists(const TopkArgs &a, hipStream_t st);
hipError_t launch_topk_rowselect(const TopkArgs &a, hipStream_t st);
hipError_t launch_topk_stream(const TopkArgs &a, hipStream_t st);  // then the row select on flagged rows
constexpr int kStreamSelectMinCols = 16384;   // rows of kStreamSelectMinCols..kStreamSelectMaxCols
constexpr int kStreamSelectMaxCols = 131072;  // columns take the streamed select
constexpr int kStreamSelectCap = 4096;        // its list of bracketed columns, per row
constexpr int kStreamSelectSample = 4096;     // its sample, per row

// The prefill chunk's top-k from threshold lists (tlist.hip).
struct TlistArgs {
  const uint2 *tlists;     // [nsplit][T][tcap] (score bits, column)
  const uint32_t *tcount;  // [nsplit][T] hits (> tcap: the list overflowed)
  const float *tau;        // [T] the lists' lower bound
  const int32_t *q_pos;    // [T]
  uint32_t *counters;      // [T][kRowCounters]: counter 7 = 1 flags the row for the row select
  int32_t *flist;          // [T] the flagged rows, *fcount of them (zeroed by tlist_gather_kernel)
  uint32_t *fcount;
  int32_t *idx;            // [T][k]
  float *val;              // [T][k] or nullptr
  int T, nsplit, tcap, ld, k;
};
constexpr int kMaxTlists = 64;         // lists (key splits) per row
constexpr int kTlistSample = 2048;     // sampled keys that set tau
// tau is the sample's r-th largest score, r = m + kTlistSigma sqrt(m) + 8 for
// m = k NS / n: fewer than k of the row's scores reach it only kTlistSigma
// standard deviations out (unstructured scores)
constexpr float kTlistSigma = 4.f;
constexpr int kTlistUnionCap = 8192;   // union entries the merge holds (in registers)
constexpr int kTlistMergeThreads = 256;
hipError_t launch_tlist_gather(const uint16_t *keys, const int32_t *q_pos, int T, int Lmax, int ns,
                               uint16_t *sample, int32_t *spos, uint32_t *fcount, hipStream_t st);
hipError_t launch_tlist_tau(const float *ss, const int32_t *q_pos, int T, int ns, int k, float *tau,
                            hipStream_t st);
hipError_t launch_tlist_merge(const TlistArgs &a, hipStream_t st);

// Block mean-pool (pool.hip).
hipError_t launch_pool(const uint16_t *keys, const int32_t *seq_lens, int S, int Lmax,
                       int B, float *pooled, hipStream_t st);
hipError_t launch_pool_append(const uint16_t *keys, const int32_t *seq_lens,
                              const int32_t *old_lens, int max_new, int S, int Lmax, int B,
                              float *pooled, hipStream_t st);

// Head router (route.hip).
struct RouteArgs {
  const uint16_t *keys;
  const uint16_t *q;
  const float *w;
  const int32_t *q_seq;
  const int32_t *q_pos;
  const float *pooled;     // [S][Mmax][128]
  float *partial;          // [T][nchunks + 1][H]
  int32_t *heads;          // [T][h]
  float *g;                // [T][H] or nullptr
  // optional, launch_route: the tile table of the grouped scoring built by
  // one more workgroup of the final kernel (tiles.hpp); tcount[0] = tiles,
  // tcount[1] = the fallback row count
  int2 *tiles;
  uint32_t *tcount;
  int tqwg, tbound;
  int S, Lmax, T, H, B, h, mode, Mmax, nchunks;
};
// complete blocks per router workgroup: each of its four waves takes
// kRouteChunk / 64 groups of 16 blocks (128: 7.1 us at 16 x 1024 blocks,
// against 8.9 us for 64 and 10.3 us for 256)
constexpr int kRouteChunk = 128;
constexpr int kHisaChunk = 64;  // blocks per workgroup of hisa_block_kernel (one group a wave)

// The hierarchical indexer's block scores (hisa.hip).
struct HisaArgs {
  const uint16_t *keys;
  const uint16_t *q;
  const float *w;
  const int32_t *q_seq;
  const int32_t *q_pos;
  const float *pooled;     // [S][Mmax][128]
  const int32_t *heads;    // [T][nh] routed heads, or nullptr = all H heads
  float *bscore;           // [T][Mmax]: block scores, -inf past the query's blocks
  int32_t *mt;             // [T]: the query's block count floor(p/B) + 1
  int S, Lmax, T, H, nh, B, Mmax, nchunks;
};
hipError_t launch_hisa_blocks(const HisaArgs &a, hipStream_t st);
hipError_t launch_route(const RouteArgs &a, hipStream_t st);
// the partial sums alone: the fused indexer call ranks the heads in the
// scoring kernel's prologue (ScoreArgs::partial)
hipError_t launch_route_partial(const RouteArgs &a, hipStream_t st);
// many queries of one sequence, H <= 64: one kernel, heads written directly
hipError_t launch_route_tile(const RouteArgs &a, hipStream_t st);

}  // namespace misa
