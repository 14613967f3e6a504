/*
 * csa.h - C ABI of the MI355X (gfx950) Compressed Sparse Attention hot path.
 *
 * One CSA layer group over one shared, paged, compressed global KV cache:
 *   csa_compress    gated pooling of every r raw KV rows into one entry,
 *                   indexer-key projection, quantisation into cache pages;
 *   csa_index_topk  lightning-indexer scores and the per-query Top-K;
 *   csa_attend      one softmax over the gathered Top-K entries plus the
 *                   last W raw rows (sliding window).
 *
 * Sources (cited by page title and section):
 *   [Walkthrough] "DeepSeek-V4.1-Flash technical report" chaptered walkthrough:
 *       "Compressed Sparse Attention 2" (modes table; "The indexer selects, SWA
 *       covers the rest"; "A simpler compressor"), "Causal Encoder-Decoder"
 *       ("One hidden state feeds the decoder"), "SWA Bounded Replay"
 *       ("Replay only the window").
 *   [Atlas] "Model architectures" atlas: compressed-KV (CSA/HCA) entry,
 *       sliding-window entry, MQA/GQA entry, IndexCache entry.
 *
 * Conventions
 * -----------
 * - Every pointer named "dev" is device memory; every other pointer is host
 *   memory. The library never allocates device memory: the caller allocates
 *   every buffer (e.g. torch tensors) and keeps it alive while the handle
 *   lives. (The one exception is csa_attend_noalloc's fixed device array,
 *   part of the library's code object.) Nothing here synchronises a stream except csa_read_errors().
 * - All work is enqueued on the caller's stream, in call order. A handle is
 *   not thread-safe and must be used from one stream at a time.
 * - Every entry point validates its arguments on the host before enqueuing
 *   anything. On error it enqueues nothing, leaves the handle unchanged and
 *   returns a status; csa_last_error() then holds a message. No C++
 *   exception crosses this boundary.
 * - Device-side bounds checks (page ids outside the pool, a Top-K index past
 *   the visible entries) never fault: the offending read or write is skipped
 *   and a bit is set in the device error word (csa_read_errors).
 * - Element layouts are row-major and dense unless stated.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_MAX_LAYERS 8      /* layers sharing one handle (one Top-K selection) */
#define CSA_PAGE_ENTRIES 64   /* compressed entries per cache page */
#define CSA_HEAD_DIM 128      /* D: the one supported KV head dimension */
#define CSA_IDX_DIM 64        /* D_I: the one supported indexer key dimension */
#define CSA_MAX_IDX_HEADS 4   /* H_I <= 4 */
#define CSA_MAX_TOPK 2048     /* k <= 2048 */
#define CSA_POOL_BLOCK 8          /* entries per candidate-pool block */
#define CSA_MAX_POOL_BLOCKS 2048  /* blocks per candidate pool (16,384 entries) */

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null/destroyed handle, bad pointer, bad index */
  CSA_ERR_SHAPE = 2,       /* sizes inconsistent with the config */
  CSA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination */
  CSA_ERR_CAPACITY = 4,    /* sequence, page, ring or workspace capacity exceeded */
  CSA_ERR_UNSUPPORTED = 5, /* valid request outside the library's limits */
  CSA_ERR_HIP = 6          /* a HIP runtime call failed */
} csa_status;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_FP4_E2M1 = 3 } csa_dtype;

/* Static shape of a layer group's cache.
 * Supported (kv_dtype, act_dtype): (F32, F32), (BF16, BF16), (FP8_E4M3, BF16),
 * (FP4_E2M1, BF16).
 * FP4_E2M1 ([Walkthrough] "FP4 main KV cache": E2M1 elements, one E4M3 scale
 * per 16 channels, no second-level scale) applies to the compressed K/V only:
 * element pairs pack into bytes (channel 2i in the low nibble), each entry's 8
 * group scales are E4M3 codes of amax/6 (round to nearest; a zero scale stores
 * zero elements), and the indexer keys stay FP8_E4M3 with page scales. */
typedef struct csa_config {
  int32_t ratio;             /* r in [1, 256]: raw rows per compressed entry (1 keeps main KV uncompressed) */
  int32_t head_dim;          /* D, must be CSA_HEAD_DIM */
  int32_t q_heads;           /* H_q: query heads sharing the single KV head, multiple of 16, <= 128 */
  int32_t idx_heads;         /* H_I: indexer query heads, 0..CSA_MAX_IDX_HEADS. 0: no indexer - a
                                heavily compressed (HCA) layer group, attended with csa_attend_dense */
  int32_t idx_dim;           /* D_I, must be CSA_IDX_DIM */
  int32_t window;            /* W >= 0: sliding-window length in raw rows (0 disables the branch) */
  int32_t ring_rows;         /* R: raw rows kept per sequence and layer; >= max(W, r, 1).
                                A prefill chunk of n tokens needs R >= n + W - 1. */
  int32_t n_layers;          /* 1..CSA_MAX_LAYERS; layer 0 is the indexing (Full) layer */
  int32_t max_seqs;          /* sequences addressable through the block table */
  int32_t max_pages_per_seq; /* block-table row length */
  int32_t pool_pages;        /* physical pages in every pool. Each layer's K (or V) pool,
                                pool_pages * 64 rows, and its window ring, max_seqs * R rows,
                                must each fit in 0xfffff000 bytes (attention addresses
                                them with 32-bit offsets): CSA_ERR_UNSUPPORTED otherwise */
  int32_t kv_dtype;          /* csa_dtype of compressed entries and indexer keys (FP4_E2M1: see above) */
  int32_t act_dtype;         /* csa_dtype of raw rows, queries and outputs (F32 or BF16) */
  int32_t swa_dtype;         /* csa_dtype of the window ring: act_dtype, or CSA_FP8_E4M3 with
                                BF16 activations (E4M3 codes, one fp32 scale amax/448 per row) */
} csa_config;

/* Device buffers of one handle (all caller-allocated, all "dev").
 * Pools are indexed by physical page: entry j of sequence b lives at slot
 * j % 64 of physical page block_table[b * max_pages_per_seq + j / 64].
 * Per-layer arrays use entries [0, n_layers); unused entries may be NULL.
 * Page scale and page staging arrays of K/V are used only when kv_dtype ==
 * CSA_FP8_E4M3, those of the indexer keys with FP8_E4M3 or FP4_E2M1, group
 * scales only with FP4_E2M1, ring scales only when swa_dtype == CSA_FP8_E4M3
 * (else NULL). */
typedef struct csa_buffers {
  void *kbar[CSA_MAX_LAYERS];        /* [pool_pages][64][D] kv_dtype: compressed keys ([..][D/2] bytes for fp4) */
  void *vbar[CSA_MAX_LAYERS];        /* [pool_pages][64][D] kv_dtype: compressed values */
  float *kbar_scale[CSA_MAX_LAYERS]; /* [pool_pages] fp32 page scale (fp8) */
  float *vbar_scale[CSA_MAX_LAYERS];
  float *kbar_stage[CSA_MAX_LAYERS]; /* [max_seqs][64][D] fp32 values of each sequence's open page (fp8) */
  float *vbar_stage[CSA_MAX_LAYERS];
  uint8_t *kbar_gscale[CSA_MAX_LAYERS]; /* [pool_pages][64][D/16] E4M3 group scales (fp4) */
  uint8_t *vbar_gscale[CSA_MAX_LAYERS];
  void *ring_k[CSA_MAX_LAYERS];      /* [max_seqs][R][D] swa_dtype: last R raw keys (row i at slot i % R) */
  void *ring_v[CSA_MAX_LAYERS];      /* [max_seqs][R][D] swa_dtype: last R raw values */
  float *ring_k_scale[CSA_MAX_LAYERS]; /* [max_seqs][R] fp32 row scales (fp8 ring) */
  float *ring_v_scale[CSA_MAX_LAYERS];
  void *block_stage[CSA_MAX_LAYERS]; /* [max_seqs][3][r][D] act_dtype: gate logits, raw keys and raw
                                        values of each sequence's open (incomplete) r-block */
  void *kidx;                        /* [pool_pages][64][D_I] indexer keys (layer 0), kv_dtype (fp8 when
                                        kv_dtype is fp4); NULL if idx_heads == 0 */
  float *kidx_scale;                 /* [pool_pages] fp32 (fp8/fp4; NULL if idx_heads == 0) */
  float *kidx_stage;                 /* [max_seqs][64][D_I] fp32 (fp8/fp4; NULL if idx_heads == 0) */
  const int32_t *block_table;        /* [max_seqs][max_pages_per_seq] physical page ids */
  void *workspace;                   /* scratch, >= csa_workspace_size() bytes, 256-byte aligned,
                                        zero-filled before csa_cache_create */
  size_t workspace_bytes;
} csa_buffers;

/* Byte sizes of the buffers above for a config (for the caller's allocator). */
typedef struct csa_buffer_sizes {
  size_t kv_pool;      /* each kbar[l] / vbar[l] */
  size_t idx_pool;     /* kidx */
  size_t page_scale;   /* each *_scale (0 unless fp8 or fp4) */
  size_t kv_stage;     /* each kbar_stage[l] / vbar_stage[l] (0 unless fp8) */
  size_t idx_stage;    /* kidx_stage (0 unless fp8 or fp4) */
  size_t group_scale;  /* each kbar_gscale[l] / vbar_gscale[l] (0 unless fp4) */
  size_t ring;         /* each ring_k[l] / ring_v[l] */
  size_t ring_scale;   /* each ring_k_scale[l] / ring_v_scale[l] (0 unless the ring is fp8) */
  size_t block_stage;  /* each block_stage[l] */
  size_t block_table;  /* block_table */
} csa_buffer_sizes;

typedef struct csa_cache *csa_cache_t;

/* Human-readable name of a status. Never NULL. */
const char *csa_status_string(csa_status s);

/* Message describing the last failed call on this host thread ("" if none). */
const char *csa_last_error(void);

/* Fills *out for cfg. Returns CSA_ERR_* if cfg is invalid. */
csa_status csa_buffer_sizes_for(const csa_config *cfg, csa_buffer_sizes *out);

/* Workspace bytes needed for calls with up to max_queries queries per call
 * (a prefill chunk counts its tokens) and k <= max_k. 0 if cfg is invalid. */
size_t csa_workspace_size(const csa_config *cfg, int32_t max_queries, int32_t max_k);

/* Creates a handle over caller-owned buffers. Every sequence starts empty. */
csa_status csa_cache_create(const csa_config *cfg, const csa_buffers *bufs, csa_cache_t *out);

/* Destroys a handle (host memory only; the caller's buffers are untouched). */
csa_status csa_cache_destroy(csa_cache_t h);

/* Marks sequence `seq` empty in every layer (host bookkeeping only). */
csa_status csa_seq_reset(csa_cache_t h, int32_t seq);

/* Raw rows appended so far to (layer, seq); -1 on bad arguments. */
int64_t csa_seq_len(csa_cache_t h, int32_t layer, int32_t seq);

/* Restores the length of (layer, seq) after the caller restored its buffer
 * contents (checkpoint / resume). len must fit the sequence's block table. */
csa_status csa_seq_set_len(csa_cache_t h, int32_t layer, int32_t seq, int64_t len);

/* Sets the replay start s of sequence `seq` (every layer): its window branch
 * then covers raw rows [max(s, t - W + 1), t] for a query at t.
 * [Walkthrough] "SWA Bounded Replay" > "Replay only the window" (the window is
 * truncated to the replay segment that starts at s). s = 0 (the default, and
 * after csa_seq_reset) leaves the window untruncated. Host state only. */
csa_status csa_seq_set_swa_start(csa_cache_t h, int32_t seq, int32_t start);

/*
 * csa_compress - append raw rows to sequences of one layer and build the
 * compressed entries of every r-block they complete.
 * [Atlas] compressed-KV entry (every r KV rows squeezed into one entry with
 * learned compression weights); [Walkthrough] "A simpler compressor" (no
 * overlap between groups, no positional embedding, indexer K projected from
 * the main-KV entry) and "One hidden state feeds the decoder" (entries and
 * compression weights are projections of one hidden state).
 *
 * For block j (rows [j*r, (j+1)*r)) and channel d: w_i = softmax_i(Z[i][d]),
 * Kbar[j][d] = sum_i w_i K[i][d], Vbar likewise with the same w,
 * KI[j] = Kbar[j] @ proj_idx (before rounding). Entries are rounded to
 * kv_dtype; with FP8 each page of each stream carries one fp32 scale
 * amax/448 over its filled entries, and a page that gains entries is
 * re-quantised whole from fp32 staging, so incremental appends produce the
 * same bytes as one bulk call.
 *
 *   layer       0..n_layers-1. With an indexer (idx_heads > 0) layer 0 must
 *               pass proj_idx (it writes the indexer keys); every other call
 *               passes NULL.
 *   n_seqs      number of sequences appended to (>= 1); seq_ids (host) are distinct.
 *   n_new       (host) rows appended per sequence, >= 0.
 *   raw_k, raw_v, gate (dev) [sum(n_new)][D] act_dtype, sequences packed in
 *               seq_ids order.
 *   proj_idx    (dev) [D][D_I] fp32, or NULL.
 * The block table must map every page the new entries land on.
 * Errors: CSA_ERR_CAPACITY if a sequence would outgrow its block-table row.
 */
csa_status csa_compress(csa_cache_t h, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                        const int32_t *n_new, const void *raw_k, const void *raw_v, const void *gate,
                        const float *proj_idx, hipStream_t stream);

/*
 * csa_ring_write - rewrite window-ring rows of already appended positions
 * without touching the compressed cache: the bounded replay regenerates only
 * the local (SWA) keys and values and reuses the cached global KV
 * ([Walkthrough] "SWA Bounded Replay" > "Encoder SWA Bounded Replay").
 *
 *   n_seqs, seq_ids (host): sequences; pos0, n_rows (host) [n_seqs]: rows
 *   [pos0, pos0 + n_rows) are replaced; raw_k, raw_v (dev) [sum(n_rows)][D]
 *   act_dtype, packed in seq_ids order. Rows are stored in the ring format
 *   (fp8 rows take a fresh per-row scale).
 * Errors: CSA_ERR_INVALID_ARG for rows not appended yet; CSA_ERR_CAPACITY for
 * rows older than the ring holds (pos0 < len - R).
 */
csa_status csa_ring_write(csa_cache_t h, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *pos0,
                          const int32_t *n_rows, const void *raw_k, const void *raw_v, hipStream_t stream);

/*
 * csa_index_topk - lightning-indexer scores and per-query Top-K over the
 * entries each query may see. [Walkthrough] CSA2 "The indexer selects, SWA
 * covers the rest" (indexer query against indexer key, top entries per
 * query); [Atlas] trained-sparse-attention entry (lightning indexer run as
 * MQA, several indexer heads over one shared key).
 *
 *   s[t][j] = sum_h w[t][h] * max(0, q_idx[t][h] . KI[j]), for the entries
 *   visible to a query at raw position t: (j+1)*r <= t+1.
 *   topk[t] = the k visible j with the largest s (ties -> lower j), ascending;
 *   -1 pads the row when fewer than k entries are visible.
 *
 *   n_q         queries (>= 1). q_seq, q_pos (host) [n_q]: sequence and raw
 *               position of each query; q_pos < csa_seq_len(h, 0, q_seq).
 *               When all queries share one sequence at consecutive positions
 *               (a prefill chunk), the chunk kernels run.
 *   q_idx       (dev) [n_q][H_I][D_I] act_dtype.   w_idx (dev) [n_q][H_I] fp32, >= 0.
 *   k           1..CSA_MAX_TOPK.   topk (dev) [n_q][k] int32 output.
 * Errors: CSA_ERR_UNSUPPORTED on a group without an indexer (idx_heads == 0).
 */
csa_status csa_index_topk(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                          const void *q_idx, const float *w_idx, int32_t k, int32_t *topk,
                          hipStream_t stream);

/*
 * csa_index_topk_pool - csa_index_topk for the group's Full-mode layer that
 * also builds each query's candidate pool for deeper Reindex-mode layers.
 * [Walkthrough] CSA2 "The Hierarchical Sparse Indexer" (the first Full layer
 * scores every causally visible entry; blocks of 8 entries score the maximum
 * of their entries; the best 2,048 blocks form a 16,384-entry pool).
 *
 *   Arguments as csa_index_topk, plus
 *   n_pool_blocks  1..CSA_MAX_POOL_BLOCKS.
 *   pool           (dev) [n_q][n_pool_blocks] int32 output: block ids b
 *                  (entries [8b, 8b+8)) of the n_pool_blocks blocks with the
 *                  largest block maximum max_{8b <= j < min(8b+8, N)} s[t][j]
 *                  (ties -> lower b), ascending; -1 pads the row when fewer
 *                  blocks are visible.
 * Chunk queries take the chunk kernels (the score GEMM also writes the block
 * maxima); other queries the per-query kernels.
 * Errors: as csa_index_topk; CSA_ERR_UNSUPPORTED for n_pool_blocks out of range.
 */
csa_status csa_index_topk_pool(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                               const void *q_idx, const float *w_idx, int32_t k, int32_t *topk,
                               int32_t n_pool_blocks, int32_t *pool, hipStream_t stream);

/*
 * csa_index_reindex - Top-K of a Reindex-mode layer: its own indexer query
 * and weights score only the entries of each query's candidate pool (the
 * shared indexer keys are reused). [Walkthrough] CSA2 "Full, Reindex, and
 * Reuse" (Reindex rescores the reused keys with its own query) and "The
 * Hierarchical Sparse Indexer" (deeper indexers search only the pool).
 *
 *   s[t][j] as csa_index_topk, for the visible entries j of the blocks in
 *   pool[t]; topk[t] = the k of them with the largest s (ties -> lower j),
 *   ascending; -1 pads the row when the pool holds fewer than k entries.
 *
 *   q_seq, q_pos, q_idx, w_idx, k, topk as csa_index_topk.
 *   n_pool_blocks, pool (dev) [n_q][n_pool_blocks]: rows as
 *   csa_index_topk_pool writes them (ascending block ids, -1 only as trailing
 *   padding). A block past the visible entries is skipped and sets bit 1
 *   (a Top-K index outside the visible range) of the csa_read_errors word.
 * Errors: as csa_index_topk; CSA_ERR_UNSUPPORTED for n_pool_blocks out of range.
 */
csa_status csa_index_reindex(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                             const void *q_idx, const float *w_idx, int32_t n_pool_blocks, const int32_t *pool,
                             int32_t k, int32_t *topk, hipStream_t stream);

/*
 * csa_attend - one layer's attention for n_q queries: one softmax over the
 * gathered Top-K entries of that layer's compressed cache plus the raw rows
 * [max(s, t-W+1), t] of its window ring (s: the sequence's replay start). [Walkthrough] CSA2 "The indexer
 * selects, SWA covers the rest"; "SWA Bounded Replay" > "Replay only the
 * window" (window rule); [Atlas] MQA/GQA entry (all query heads share the one
 * KV head). Reuse-mode layers call this with the Top-K rows produced for the
 * indexing layer ([Walkthrough] CSA2 "Full, Reindex, and Reuse").
 *
 *   out[t][h] = sum_key p * v,  p = softmax over keys of scale * q[t][h] . key
 *   keys = {Kbar[j] : j in topk[t], j >= 0} u {K[i] : max(0,t-W+1) <= i <= t}
 *   (no de-duplication between the two branches; entries with fp8 storage
 *   are dequantised with their page scales).
 *
 *   layer       0..n_layers-1.  q_seq, q_pos (host) [n_q] as for csa_index_topk,
 *               q_pos < csa_seq_len(h, layer, q_seq).
 *   q           (dev) [n_q][H_q][D] act_dtype.   topk (dev) [n_q][k] int32, k >= 0.
 *   scale       logit scale (1/sqrt(D) in the method).
 *   out         (dev) [n_q][H_q][D] act_dtype.
 * Errors: CSA_ERR_INVALID_ARG for a bad layer, pointer or position;
 * CSA_ERR_CAPACITY when a query's window rows already left the ring or the
 * workspace cannot hold the split partials; CSA_ERR_UNSUPPORTED for k outside
 * [0, CSA_MAX_TOPK] or when a decode query's keys (k + W) need more splits
 * than the merge takes: min(80, 5120 / min(n_q, 128)) splits of 2,048 keys
 * (2,304 for fp32 caches), i.e. 163,840 keys for batches of up to 64.
 * Prefill chunks (consecutive positions of one sequence) have no such bound.
 */
csa_status csa_attend(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq,
                      const int32_t *q_pos, const void *q, const int32_t *topk, int32_t k, float scale,
                      void *out, hipStream_t stream);

/*
 * csa_attend_noalloc - csa_attend for callers that cannot allocate or pass
 * scratch memory per call (code under HIP graph capture that must not touch
 * the handle's workspace, tight serving loops, harnesses that forbid
 * allocation). Same arguments, results and errors as csa_attend; the split
 * partials go to a fixed 16 MiB device array of the library (one per GPU,
 * held until the process ends; its address is looked up on the first call on
 * each device) instead of the handle's workspace. Nothing is allocated and
 * nothing needs clearing: every partial is written before it is read.
 * A call needs n_q x splits x (H x D + 2 H) x 4 bytes of it (at most 80
 * splits per query; a decode query has one split per 64 keys of Top-K and
 * window): CSA_ERR_CAPACITY when that exceeds 16 MiB, before any launch.
 * All calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads, other handles) race and must be serialised by the
 * caller. Records no profiling events.
 */
csa_status csa_attend_noalloc(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq,
                              const int32_t *q_pos, const void *q, const int32_t *topk, int32_t k, float scale,
                              void *out, hipStream_t stream);

/*
 * csa_attend_dense - heavily compressed attention (HCA): one softmax over every
 * compressed entry visible to the query ((j+1)*r <= t+1) plus the window rows,
 * with no indexer selection. [Atlas] compressed-KV entry (HCA applies the same
 * compression primitive far more aggressively and runs ordinary dense
 * attention over the short compressed stream).
 *
 *   Arguments as for csa_attend, without topk and k.
 *   out[t][h] = sum_key p * v over keys {Kbar[j] : j < (t+1)/r} u window rows.
 * Errors: as csa_attend, with k replaced by the visible entries: a decode
 * query may see up to 163,840 keys (entries + W) in batches of up to 64.
 */
csa_status csa_attend_dense(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq,
                            const int32_t *q_pos, const void *q, float scale, void *out,
                            hipStream_t stream);

/* Synchronises `stream`, returns the device error word in *flags (bit 0: a
 * page id outside the pool was met; bit 1: a Top-K index outside the visible
 * range was met; bit 2: an internal capacity fallback ran) and clears it. */
csa_status csa_read_errors(csa_cache_t h, hipStream_t stream, uint32_t *flags);

/* Kernel timing. csa_profile_begin(h, kernels) starts recording, for every
 * later call on h issued outside stream capture, a HIP event pair stamped by
 * the kernel launch itself (hipExtLaunchKernelGGL) around:
 *   CSA_PROFILE_INDEX   the indexer score kernel of csa_index_topk (the decode
 *                       scan; in chunk mode the GEMM pass that scores every
 *                       visible entry);
 *   CSA_PROFILE_ATTEND  the attention kernel of csa_attend (not its split merge).
 * csa_profile_end(h, kernel, ...) synchronises and returns the summed elapsed
 * milliseconds and the number of timed launches of one kind (one bit), and
 * stops recording that kind. Errors: CSA_ERR_INVALID_ARG for a bad mask. */
#define CSA_PROFILE_INDEX 1
#define CSA_PROFILE_ATTEND 2
csa_status csa_profile_begin(csa_cache_t h, int32_t kernels);
csa_status csa_profile_end(csa_cache_t h, int32_t kernel, double *total_ms, int32_t *launches);

/* ---- Test and measurement hooks (not part of the method) ---------------- */

/* Test hook: runs the device number-format routines on n values (the codec
 * tests compare them with the oracle's encoders bit for bit):
 * kind 0: fp8 e4m3 codes (uint8) -> fp32 as the attention/indexer kernels decode them;
 * kind 1: fp8 e4m3 codes (uint8) -> bf16 bits (uint16) as the MFMA operands are built;
 * kind 2: fp32 -> fp8 e4m3 codes (uint8) as the compressor encodes (RNE, saturating);
 * kind 3: fp32 -> bf16 bits (RNE);
 * kind 4: fp4 byte pairs (uint8, n a multiple of 4) -> 2n fp32 (low nibble first) as the
 *         attention kernel decodes packed E2M1 rows;
 * kind 5: fp32 -> E2M1 codes (uint8, low 4 bits) as the compressor encodes.
 * in/out are device pointers. */
csa_status csa_debug_convert(int32_t kind, const void *in, void *out, int64_t n, hipStream_t stream);

/* Measurement hook: a streaming-read reference for the indexer scan's
 * bandwidth, reported by the benchmark beside the scan. Reads `bytes` of
 * device memory per launch with
 * 16-byte non-temporal loads (the scan's load form), `reps` launches rotating
 * over the n_bufs device buffers bufs[i] (each >= bytes, 16-byte aligned; use
 * enough of them to exceed the last-level cache), each launch timed by events
 * it stamps itself. Writes nothing to device memory. Synchronises `stream`;
 * *avg_us receives the mean launch duration in microseconds. Errors:
 * CSA_ERR_INVALID_ARG for null or misaligned buffers, bytes not a positive
 * multiple of 16, reps < 1; CSA_ERR_HIP on a launch or event failure. */
csa_status csa_debug_stream_read(const void *const *bufs, int32_t n_bufs, int64_t bytes, int32_t reps,
                                 hipStream_t stream, float *avg_us);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
