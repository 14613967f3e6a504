// Host-side internals shared by the C-ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

constexpr int kPage = CSA_PAGE_ENTRIES;
constexpr int kD = CSA_HEAD_DIM;
constexpr int kDI = CSA_IDX_DIM;

// ------------------------------------------------------------------ compress

constexpr int kCompressMaxItems = 64;

struct CompressItem {
  int32_t seq, old_len, n_new, row_off, page0, n_pages;
};

struct CompressArgs {
  const void *raw_k, *raw_v, *gate;               // packed new rows [sum n_new][D]
  const void *block_stage;                        // open-block gate/K/V rows [max_seqs][3][r][D]
  const float *proj;                              // [D][D_I] or null
  void *kbar, *vbar, *kidx;                       // pools
  uint8_t *kbar_gs, *vbar_gs;                     // fp4 group scales [pool_pages][64][D/16]
  float *kbar_scale, *vbar_scale, *kidx_scale;    // fp8 page scales
  float *kbar_stage, *vbar_stage, *kidx_stage;    // fp8 open-page staging
  const int32_t *block_table;
  uint32_t *err;
  int32_t r, R, bt_stride, pool_pages, write_idx, n_items;
  CompressItem it[kCompressMaxItems];
  int32_t wg0[kCompressMaxItems + 1];             // first page workgroup of each item (set by the launcher)
};

struct RingArgs {
  const void *raw_k, *raw_v, *gate;
  void *ring_k, *ring_v;                          // [max_seqs][R][D] act dtype, or E4M3 codes
  float *ring_k_scale, *ring_v_scale;             // [max_seqs][R] row scales (fp8 ring)
  void *block_stage;                              // [max_seqs][3][r][D]
  int32_t r, R, n_items, rows_per_wg;
  int32_t write_stage;                            // 0: window rows only (a replay)
  int32_t chunks[kCompressMaxItems];              // WGs per item
  CompressItem it[kCompressMaxItems];
  int32_t wg0[kCompressMaxItems + 1];             // first workgroup of each item (set by the launcher)
};

// The fields of RingArgs that one item's ring rows need.
struct RingPtrs {
  const void *raw_k, *raw_v, *gate;
  void *ring_k, *ring_v;
  float *ring_k_scale, *ring_v_scale;
  void *block_stage;
  int32_t r, R, rows_per_wg, write_stage;
};

void launch_compress_pages(const CompressArgs &a, int n_wg, int kv, int act, hipStream_t s);
void launch_compress_ring(const RingArgs &a, int n_wg, int act, bool ring_fp8, hipStream_t s);
// One workgroup per item (a.n_items of them, fp8 or fp4 pages), for calls in
// which every item writes at most one page and at most rp.rows_per_wg ring
// rows: the item's page (it.n_pages = 0 or 1, at it.page0), then its ring and
// block-staging rows, in one launch.
void launch_compress_step(const CompressArgs &a, const RingPtrs &rp, int kv, int act, bool ring_fp8, hipStream_t s);

// ------------------------------------------------------------------ index (decode)

constexpr int kIdxMaxQ = 128;        // queries per decode launch group
constexpr int kScanPagesPerWave = 2;                     // indexer-key pages per scan wave
constexpr int kScanWaves = 4;                            // waves per scan workgroup
constexpr int kIdxChunk = kScanWaves * kScanPagesPerWave * 64;   // entries per scan workgroup
constexpr int kRescanChunk = kScanWaves * 64;                   // pool positions per Reindex scoring workgroup
constexpr int kFilterSlice = 4096;   // scores per filter workgroup
constexpr int kMaxGroups = 8192;     // group maxima per query (threshold select in LDS)
constexpr int kMaxSlices = 512;      // filter slices per query (<= 2M visible entries)

struct IdxQuery {
  int32_t seq, n_vis, chunk0, glog2;  // visible entries, first scan-WG index, log2 group size
};

struct IdxScanArgs {
  const void *kidx;
  const float *kidx_scale;
  const int32_t *block_table;
  const void *q_idx;   // [n_q][H_I][D_I] (this group's rows)
  const float *w_idx;  // [n_q][H_I]
  float *S;            // [n_q][s_stride]
  float *M;            // [n_q][s_stride]
  float *B;            // [n_q][s_stride] maxima of aligned 8-entry blocks (first N/8 used), or null
  uint32_t *err;
  int32_t bt_stride, pool_pages, h_i, s_stride, n_q, total_wg;
  IdxQuery q[kIdxMaxQ];
};

// candidate pool of a Full-mode layer: blocks of 8 entries
constexpr int kPoolBlock = 8;

// Reindex scores: positions p of a query's pool row map to entries
// pool[p / 8] * 8 + p % 8; q[i].n_vis counts positions, n_ent visible entries
struct IdxRescanArgs {
  const void *kidx;
  const float *kidx_scale;
  const int32_t *block_table;
  const void *q_idx;
  const float *w_idx;
  const int32_t *pool;   // [n_q][pool_stride]
  float *S, *M;          // [n_q][s_stride] position scores and group maxima
  uint32_t *err;
  int32_t bt_stride, pool_pages, h_i, s_stride, n_q, total_wg, pool_stride;
  IdxQuery q[kIdxMaxQ];
  int32_t n_ent[kIdxMaxQ];
};

struct IdxFilterArgs {
  const float *S, *M;
  float *cand_s;       // [n_q][s_stride]: slice i's candidates at [i * kFilterSlice, ...), index order
  int32_t *cand_j;     // [n_q][s_stride]
  int32_t *cnt;        // [n_q][max_slices] candidates per slice
  int32_t s_stride, k, n_q, max_slices;
  int32_t slice0[kIdxMaxQ + 1];   // prefix of filter WGs
  int32_t n_vis[kIdxMaxQ];
  int32_t glog2[kIdxMaxQ];
  int32_t uniform;                // filter WGs per query when every query has as many, else 0
};

struct IdxFinalArgs {
  const float *S;
  const float *cand_s;
  const int32_t *cand_j;
  const int32_t *cnt;
  int32_t *topk;       // [n_q][k]
  uint32_t *err;
  const int32_t *pool; // null, or [n_q][pool_stride]: selected positions map through the pool row
  int32_t s_stride, k, n_q, max_slices, pool_stride;
  int32_t n_vis[kIdxMaxQ];
  int32_t n_ent[kIdxMaxQ];   // with a pool: visible entries (mapped entries past it become -1)
};

// chunk (prefill) index: all queries of one sequence at consecutive positions
constexpr int kChunkSample = 16;     // the sample GEMM scores entries 16m + 15
constexpr int kChunkCandCap = 4096;  // candidates one select keeps in LDS
constexpr int kChunkTileCand = 64;   // candidate slots per (query, 256-entry tile)
constexpr int kChunkMaxTiles = 1024; // 256-entry tiles per query the chunk select takes
constexpr int kChunkMaxEntries = kChunkMaxTiles * 256;   // larger chunks are indexed query by query

struct IdxChunkArgs {
  const void *kidx;
  const float *kidx_scale;
  const int32_t *bt_row;   // block-table row of the sequence
  const void *q_idx;       // [n_tok][H_I][D_I]
  const float *w_idx;      // [n_tok][H_I]
  float *ss;               // [n_tok][ss_stride] sampled scores
  float *tau;              // [n_tok] thresholds
  int32_t *cnt;            // [n_tok][n_etiles] candidates per (query, entry tile)
  uint64_t *cand;          // [n_tok][n_etiles][kChunkTileCand] candidates (entry << 32 | score bits), entry order
  float *fb_rows;          // [n_tok][fb_stride] full rows for the exact fallback
  int32_t *topk;           // [n_tok][k]
  uint32_t *err;
  // candidate pool (null when not built): 8-entry block maxima [n_tok][bm_stride],
  // stored in fb_rows (the pool select runs before the Top-K select may need them)
  float *bmax;
  int32_t *pool;           // [n_tok][n_pool] ascending block ids, -1 padding
  int32_t pool_pages, h_i, ss_stride, fb_stride, n_tok, pos0, r, k, m_s, n_etiles, n_stiles, kv_dtype, act_dtype;
  int32_t bm_stride, n_pool;
};

// ev0/ev1 (may be null): events stamped with the start and end of the launch
// that does the score work (the scan; in chunk mode the full-score GEMM pass).
void launch_idx_scan(const IdxScanArgs &a, int kv, int act, hipStream_t s, hipEvent_t ev0 = nullptr,
                     hipEvent_t ev1 = nullptr);
// Short rows: a query with at most kSmallEntries visible entries and at most
// kSmallBytes of indexer keys is scored and selected by one workgroup (one
// launch for the group; topk rows as for the final kernel).
constexpr int kSmallEntries = 4096;
constexpr int kSmallBytes = 256 << 10;
void launch_idx_small(const IdxScanArgs &a, int kv, int act, int32_t *topk, int k, hipStream_t s,
                      hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
void launch_idx_filter(const IdxFilterArgs &a, int n_wg, hipStream_t s);
void launch_idx_final(const IdxFinalArgs &a, hipStream_t s);
void launch_idx_chunk(const IdxChunkArgs &a, int kv, int act, hipStream_t s, hipEvent_t ev0 = nullptr,
                      hipEvent_t ev1 = nullptr);
void launch_idx_chunk_select(const IdxChunkArgs &a, hipStream_t s);
void launch_idx_chunk_pool(const IdxChunkArgs &a, hipStream_t s);
void launch_idx_rescan(const IdxRescanArgs &a, int kv, int act, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);

// ------------------------------------------------------------------ attend

constexpr int kAttMaxQ = 128;
constexpr int kKeyBlock = 64;        // keys per attention block

struct AttQuery {
  int32_t seq, pos, swa;   // swa: replay start s of the window branch
};

constexpr uint32_t kAttMaxBufferBytes = 0xfffff000u;   // largest K/V pool or ring an attention gather addresses
constexpr int kAttMaxSplitKeys = 2304;   // keys one workgroup resolves up front (36 blocks)
constexpr int kAttKeyStreams = 1;        // 64-key blocks a decode workgroup processes per round
constexpr int kAttChunkKeyStreams = 1;   // the same for a prefill chunk (one workgroup per query)
constexpr int kAttMaxSplits = 80;        // splits per query combined by the merge kernel
constexpr int kAttSplitBudget = kAttMaxQ * 40;   // queries x splits of one launch (partials workspace)

// Most splits a launch of nq queries may use: the partials of nq x splits fit the budget.
inline int att_max_splits(int nq) {
  const int b = kAttSplitBudget / (nq > 0 ? nq : 1);
  return b < 1 ? 1 : (b < kAttMaxSplits ? b : kAttMaxSplits);
}

struct AttendArgs {
  const void *q;            // [n_q][H][D]
  void *out;                // [n_q][H][D]
  const int32_t *topk;      // [n_q][k]
  const void *kbar, *vbar;
  const float *kbar_scale, *vbar_scale;
  const uint8_t *kbar_gs, *vbar_gs;         // fp4 group scales [pool_pages][64][D/16]
  const void *ring_k, *ring_v;
  const float *ring_k_scale, *ring_v_scale;   // per-row scales of an fp8 ring
  uint32_t pool_bytes, ring_bytes, gs_bytes;  // bytes of each K (= V) pool, ring and fp4 group-scale pool
  const int32_t *block_table;
  float *part_o;            // [n_q][n_splits][H][D] unnormalised partial outputs
  float *part_ml;           // [n_q][n_splits][2][H] running max and sum
  uint32_t *err;
  float scale;
  int32_t k, W, R, r, bt_stride, pool_pages, H;
  int32_t n_sparse_blocks, n_blocks, blocks_per_split, n_splits, n_q;
  int32_t act_f32;          // outputs are fp32 (else bf16)
  int32_t chunk;            // 1: queries are a chunk (seq0, pos0 + i)
  int32_t dense;            // 1: the sparse keys are every visible entry (topk unused)
  int32_t seq0, pos0, swa0;
  AttQuery qd[kAttMaxQ];
};

constexpr int kAttSplitMaxKeys = 2048;   // keys one decode-kernel workgroup resolves up front (32 blocks)
constexpr int kAttDenseSplits = 64;      // splits per dense query at most: a workgroup takes ceil(blocks / 64) rounds
constexpr int kAttWideBatch = 512;       // decode (query, block) pairs above which a workgroup takes two blocks

// Decode and dense attention with bf16 compute (kv: bf16, fp8 or fp4): one
// workgroup per (query, split), one 64-key block per round, a.blocks_per_split
// blocks per split; with several splits the merge kernel follows.
// n_wg = n_q x n_splits.
void launch_attend_decode(const AttendArgs &a, int n_wg, int kv, bool ring_fp8, hipStream_t s,
                          hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// ev0/ev1 (may be null): events stamped with the start and end of the attention kernel launch.
void launch_attend(const AttendArgs &a, int n_wg, int kv, int act, bool ring_fp8, hipStream_t s,
                   hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);


}  // namespace csa
