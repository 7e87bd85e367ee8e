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
  uint32_t *hist;          // [T][4096] first-digit histogram (accumulated), or nullptr
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
  const int32_t *heads;    // [T][h], h <= 16
  float *scores;           // [T][ld]
  int seq;                 // the one sequence all rows read
  int h, H, Lmax, T, ld;
  int split;               // key columns per workgroup, a multiple of 64
};
// key tile of the prefill kernel: PrefillArgs::split must be a multiple
constexpr int kPrefillKeyTile = 128;
hipError_t launch_score_prefill(const PrefillArgs &a, hipStream_t st, hipEvent_t ev0 = nullptr,
                                hipEvent_t ev1 = nullptr);
int prefill_queries_per_wg(int h);
bool prefill_supported(int h, int ld, int Lmax);  // the launch shape fits h, the row length and the keys

// Per-row top-k selection (topk.hip).
struct TopkArgs {
  const float *scores;     // [rows][ld]
  const int32_t *row_len;  // [rows] or nullptr (all ld columns)
  int row_len_add;         // valid columns = row_len[r] + row_len_add
  const int32_t *map;      // [rows][ld] column -> token id (-1 = empty) or nullptr
  const uint32_t *hist;    // [rows][4096] first-digit histogram of the valid columns
  uint32_t *counters;      // [rows][kRowCounters] (select.hpp)
  uint2 *cand;             // [rows][cap] threshold-digit candidates (order key, column)
  int cap;                 // <= 16384
  int32_t *idx;            // [rows][k]
  float *val;              // [rows][k] or nullptr
  int rows, ld, k, chunk;  // chunk: columns per workgroup (histogram / filter)
  int only_flagged;        // row select: skip rows whose counter 7 is 0 (streamed select done)
};
hipError_t launch_topk_hist(const TopkArgs &a, uint32_t *hist, hipStream_t st);
hipError_t launch_topk_select(const TopkArgs &a, hipStream_t st);
hipError_t launch_topk_rowselect(const TopkArgs &a, hipStream_t st);
hipError_t launch_topk_stream(const TopkArgs &a, hipStream_t st);  // then the row select on flagged rows
constexpr int kStreamSelectMinCols = 16384;   // rows of kStreamSelectMinCols..kStreamSelectMaxCols
constexpr int kStreamSelectMaxCols = 131072;  // columns take the streamed select
constexpr int kStreamSelectCap = 4096;        // its list of bracketed columns, per row
constexpr int kStreamSelectSample = 4096;     // its sample, per row
hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t st);

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
  uint32_t *zero_hist;     // [T][4096] zeroed by route_final (fused indexer call), or nullptr
  uint32_t *zero_ctr;      // [T][8] zeroed with it
  int S, Lmax, T, H, B, h, mode, Mmax, nchunks;
};
constexpr int kRouteChunk = 64;  // complete blocks per router workgroup

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
// many queries of one sequence, H <= 64: one kernel, heads written directly
hipError_t launch_route_tile(const RouteArgs &a, hipStream_t st);

}  // namespace misa
