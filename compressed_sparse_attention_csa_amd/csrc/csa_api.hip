// C ABI of the CSA hot path: handle, host-side validation and launch planning.
// The kernels live in compress.hip, index.hip and attend.hip.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include <hip/hip_ext.h>

#include "csa_device.h"
#include "csa_internal.h"

using namespace csa;

// Scratch of csa_attend_noalloc: a device array of this library, one copy per
// GPU the library runs on, held until the process ends. Host code never uses
// the array's name as an address: each device's copy is looked up once, with
// that device current, and kept per device (static_scratch below).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

struct csa_cache {
  uint64_t magic;
  csa_config cfg;
  csa_buffers buf;
  std::vector<int64_t> len;  // [n_layers][max_seqs] raw rows appended
  std::vector<int32_t> swa_start;  // [max_seqs] replay start s of the window branch
  uint32_t *err;             // device error word (workspace head)
  char *scratch;             // workspace after the head
  size_t scratch_bytes;
  int32_t profiling;                 // CSA_PROFILE_* bits being recorded
  std::vector<hipEvent_t> events;    // start/stop pairs
  std::vector<int32_t> event_kind;   // CSA_PROFILE_* bit of each pair
  size_t events_used;                // pairs in use
};

namespace {

constexpr uint64_t kMagic = 0x4353414d49333535ull;  // "CSAMI355"
constexpr size_t kHead = 256;       // device error word
thread_local std::string g_last_error;

csa_status fail(csa_status s, const char *fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof(msg), fmt, ap);
  va_end(ap);
  g_last_error = msg;
  return s;
}

bool handle_ok(csa_cache_t h) { return h != nullptr && h->magic == kMagic; }

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (nullptr on failure, with the message set).
char *static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(CSA_ERR_HIP, "no current device for the static scratch");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      fail(CSA_ERR_HIP, "hipGetSymbolAddress of the static scratch failed on device %d", dev);
      return nullptr;
    }
    scratch_ptr[dev] = p;
  }
  return static_cast<char *>(scratch_ptr[dev]);
}

int dt_bytes(int dt) { return dt == CSA_F32 ? 4 : (dt == CSA_BF16 ? 2 : 1); }

// Kernel dtypes of the compressed K/V and of the indexer keys (fp8 when K/V are fp4).
int main_dt(const csa_config &c) {
  return c.kv_dtype == CSA_F32 ? DT_F32 : c.kv_dtype == CSA_BF16 ? DT_BF16 : c.kv_dtype == CSA_FP8_E4M3 ? DT_FP8 : DT_FP4;
}
int idx_dt(const csa_config &c) {
  return c.kv_dtype == CSA_F32 ? DT_F32 : c.kv_dtype == CSA_BF16 ? DT_BF16 : DT_FP8;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bytes of one compressed K (or V) row, one window-ring row, and each layer's
// K (or V) pool and ring
uint64_t pool_row_bytes(const csa_config &c) {
  return c.kv_dtype == CSA_FP4_E2M1 ? kD / 2 : static_cast<uint64_t>(kD) * dt_bytes(c.kv_dtype);
}
uint64_t ring_row_bytes(const csa_config &c) {
  return c.swa_dtype == CSA_FP8_E4M3 ? kD : static_cast<uint64_t>(kD) * dt_bytes(c.act_dtype);
}
uint64_t pool_bytes_of(const csa_config &c) { return static_cast<uint64_t>(c.pool_pages) * kPage * pool_row_bytes(c); }
uint64_t ring_bytes_of(const csa_config &c) {
  return static_cast<uint64_t>(c.max_seqs) * static_cast<uint64_t>(c.ring_rows) * ring_row_bytes(c);
}

csa_status check_config(const csa_config *c) {
  if (!c) return fail(CSA_ERR_INVALID_ARG, "config is NULL");
  if (c->ratio < 1 || c->ratio > 256) return fail(CSA_ERR_UNSUPPORTED, "ratio %d outside [1, 256]", c->ratio);
  if (c->head_dim != CSA_HEAD_DIM) return fail(CSA_ERR_UNSUPPORTED, "head_dim %d != %d", c->head_dim, CSA_HEAD_DIM);
  if (c->idx_dim != CSA_IDX_DIM) return fail(CSA_ERR_UNSUPPORTED, "idx_dim %d != %d", c->idx_dim, CSA_IDX_DIM);
  if (!(c->q_heads == 16 || c->q_heads == 32 || c->q_heads == 64 || c->q_heads == 128))
    return fail(CSA_ERR_UNSUPPORTED, "q_heads %d not in {16, 32, 64, 128}", c->q_heads);
  if (c->idx_heads < 0 || c->idx_heads > CSA_MAX_IDX_HEADS)
    return fail(CSA_ERR_UNSUPPORTED, "idx_heads %d outside [0, %d]", c->idx_heads, CSA_MAX_IDX_HEADS);
  if (c->window < 0) return fail(CSA_ERR_SHAPE, "window %d < 0", c->window);
  if (c->ring_rows < std::max(std::max(c->window, c->ratio), 1))
    return fail(CSA_ERR_SHAPE, "ring_rows %d < max(window, ratio, 1)", c->ring_rows);
  if (c->n_layers < 1 || c->n_layers > CSA_MAX_LAYERS)
    return fail(CSA_ERR_SHAPE, "n_layers %d outside [1, %d]", c->n_layers, CSA_MAX_LAYERS);
  if (c->max_seqs < 1 || c->max_pages_per_seq < 1 || c->pool_pages < 1)
    return fail(CSA_ERR_SHAPE, "max_seqs, max_pages_per_seq and pool_pages must be >= 1");
  if (static_cast<int64_t>(c->pool_pages) * CSA_PAGE_ENTRIES >= (1ll << 31) ||
      static_cast<int64_t>(c->max_seqs) * c->ring_rows >= (1ll << 31))
    return fail(CSA_ERR_UNSUPPORTED, "pool_pages * 64 and max_seqs * ring_rows must stay below 2^31 rows");
  if (static_cast<int64_t>(c->max_pages_per_seq) * CSA_PAGE_ENTRIES * c->ratio > (1ll << 30))
    return fail(CSA_ERR_UNSUPPORTED, "max_pages_per_seq * 64 * ratio exceeds 2^30 raw rows");
  const bool ok = (c->kv_dtype == CSA_F32 && c->act_dtype == CSA_F32) ||
                  (c->kv_dtype == CSA_BF16 && c->act_dtype == CSA_BF16) ||
                  (c->kv_dtype == CSA_FP8_E4M3 && c->act_dtype == CSA_BF16) ||
                  (c->kv_dtype == CSA_FP4_E2M1 && c->act_dtype == CSA_BF16);
  if (!ok) return fail(CSA_ERR_DTYPE, "unsupported (kv_dtype, act_dtype) = (%d, %d)", c->kv_dtype, c->act_dtype);
  if (c->swa_dtype != c->act_dtype && !(c->swa_dtype == CSA_FP8_E4M3 && c->act_dtype == CSA_BF16))
    return fail(CSA_ERR_DTYPE, "swa_dtype %d must be act_dtype, or FP8_E4M3 with BF16 activations", c->swa_dtype);
  // attention gathers address each K/V pool and ring with 32-bit byte offsets
  if (pool_bytes_of(*c) > kAttMaxBufferBytes || ring_bytes_of(*c) > kAttMaxBufferBytes)
    return fail(CSA_ERR_UNSUPPORTED, "each K/V pool and ring must hold at most %u bytes (pool %llu, ring %llu)",
                kAttMaxBufferBytes, static_cast<unsigned long long>(pool_bytes_of(*c)),
                static_cast<unsigned long long>(ring_bytes_of(*c)));
  return CSA_OK;
}

struct Plan {  // workspace needs
  size_t idx_decode, idx_chunk, attend;
};

int64_t ecap(const csa_config &c) { return static_cast<int64_t>(c.max_pages_per_seq) * CSA_PAGE_ENTRIES; }

int64_t max_slices_for(int64_t s_stride) { return (s_stride + kFilterSlice - 1) / kFilterSlice; }

// S, M, candidate scores, candidate indices (each [nq][s_stride]), per-slice
// counts and the 8-entry block maxima of the candidate pool
size_t idx_decode_bytes(int nq, int64_t s_stride) {
  return align_up(static_cast<size_t>(nq) * s_stride * 4, 256) * 4 +
         align_up(static_cast<size_t>(nq) * max_slices_for(s_stride) * 4, 256) +
         align_up(static_cast<size_t>(nq) * s_stride * 4, 256);
}
// sampled scores, tau, per-tile counts, per-tile candidate regions, fallback rows
// Workgroups per query when every one of the nq queries has the same
// non-zero count (first_of(i): query i's first workgroup, total: all of
// them), else 0: the filter kernel then finds a workgroup's query by division.
template <typename First>
int uniform_count(First first_of, int nq, int total) {
  if (nq <= 0 || total <= 0 || total % nq != 0) return 0;
  const int per = total / nq;
  for (int i = 0; i < nq; ++i)
    if (first_of(i) != i * per) return 0;
  return per;
}

size_t idx_chunk_bytes(int nq, int64_t ss_stride, int64_t fb_stride) {
  const int64_t tiles = (fb_stride + 255) / 256;
  return align_up(static_cast<size_t>(nq) * ss_stride * 4, 256) + align_up(static_cast<size_t>(nq) * 4, 256) +
         align_up(static_cast<size_t>(nq) * tiles * 4, 256) +
         align_up(static_cast<size_t>(nq) * tiles * kChunkTileCand * 8, 256) +
         align_up(static_cast<size_t>(nq) * fb_stride * 4, 256);
}

size_t attend_bytes(int nq, int n_splits, int H) {
  return align_up(static_cast<size_t>(nq) * n_splits * H * kD * 4, 256) + align_up(static_cast<size_t>(nq) * n_splits * H * 2 * 4, 256);
}

int n_blocks_for(int k, int W) { return (k + kKeyBlock - 1) / kKeyBlock + (W > 0 ? (W + kKeyBlock - 1) / kKeyBlock : 0); }


// Blocks of 64 keys per attention workgroup for a decode batch of nq queries
// with nb blocks each: enough workgroups to spread the gathers over the chip,
// few enough splits that the fused merge stays cheap.
int attend_blocks_per_split(int nq, int nb) {
  // Latency-bound: a workgroup that walks several blocks in sequence waits a
  // memory round trip per block, so decode batches take one round per split.
  int bps = kAttKeyStreams;
  const int ms = att_max_splits(nq);
  bps = std::max(bps, (nb + ms - 1) / ms);
  bps = std::min(bps, kAttMaxSplitKeys / kKeyBlock);
  return std::max(1, bps);
}

bool is_chunk(int n, const int32_t *seq, const int32_t *pos) {
  if (n < 2) return false;
  for (int i = 1; i < n; ++i)
    if (seq[i] != seq[0] || pos[i] != pos[0] + i) return false;
  return true;
}

// A chunk is indexed as one (shared score GEMM, per-query candidate select)
// while its last query sees at most kChunkMaxEntries entries; past that, query
// by query (the decode path scans up to 2M entries per query).
bool index_as_chunk(const csa_config &c, int n, const int32_t *seq, const int32_t *pos) {
  return is_chunk(n, seq, pos) && (static_cast<int64_t>(pos[n - 1]) + 1) / c.ratio <= kChunkMaxEntries;
}

// Event pair for the next profiled launch, or {nullptr, nullptr} when profiling
// is off or the stream is being captured. The launcher hands the pair to
// hipExtLaunchKernelGGL, which stamps them with the kernel's own start and end.
struct ProfPair { hipEvent_t start = nullptr, stop = nullptr; };

ProfPair prof_events(csa_cache_t h, hipStream_t s, int32_t kind) {
  if (!(h->profiling & kind)) return {};
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return {};
  if (2 * (h->events_used + 1) > h->events.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return {};
    if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return {}; }
    h->events.push_back(a);
    h->events.push_back(b);
    h->event_kind.push_back(0);
  }
  ProfPair p{h->events[2 * h->events_used], h->events[2 * h->events_used + 1]};
  h->event_kind[h->events_used] = kind;
  ++h->events_used;
  return p;
}

// ------------------------------------------------------------------ debug conversions
__global__ void debug_convert_kernel(int kind, const void *in, void *out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (kind == 0) {
    const uint32_t c = reinterpret_cast<const uint8_t *>(in)[i];
    reinterpret_cast<float *>(out)[i] = fp8x2_to_f32<false>(c)[0];
  } else if (kind == 1) {
    const uint32_t c = reinterpret_cast<const uint8_t *>(in)[i];
    reinterpret_cast<uint16_t *>(out)[i] = __builtin_bit_cast(uint16_t, fp8x2_to_bf16<false>(c)[0]);
  } else if (kind == 2) {
    reinterpret_cast<uint8_t *>(out)[i] = static_cast<uint8_t>(f32_to_e4m3(reinterpret_cast<const float *>(in)[i]));
  } else if (kind == 3) {
    reinterpret_cast<uint16_t *>(out)[i] = f32_to_bf16(reinterpret_cast<const float *>(in)[i]);
  } else if (kind == 4) {
    // byte i of the input sits at byte i % 4 of its 32-bit word, as in a packed row
    const uint32_t w = reinterpret_cast<const uint32_t *>(in)[i >> 2];
    f32x2_t v;
    switch (i & 3) {
      case 0: v = fp4x2_to_f32<0>(w); break;
      case 1: v = fp4x2_to_f32<1>(w); break;
      case 2: v = fp4x2_to_f32<2>(w); break;
      default: v = fp4x2_to_f32<3>(w); break;
    }
    reinterpret_cast<float *>(out)[2 * i] = v[0];
    reinterpret_cast<float *>(out)[2 * i + 1] = v[1];
  } else {
    reinterpret_cast<uint8_t *>(out)[i] = static_cast<uint8_t>(f32_to_e2m1(reinterpret_cast<const float *>(in)[i]));
  }
}

// Streaming read of n16 16-byte words with non-temporal loads. The xor of the
// words feeds an empty volatile asm statement, so the loads stay and nothing
// is written.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *p, int64_t n16) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + u * 256;
    if (i < n16) acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i);
  }
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  asm volatile("" : : "v"(x));
}

}  // namespace

extern "C" {

const char *csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE";
    case CSA_ERR_DTYPE: return "CSA_ERR_DTYPE";
    case CSA_ERR_CAPACITY: return "CSA_ERR_CAPACITY";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
  }
  return "CSA_ERR_UNKNOWN";
}

const char *csa_last_error(void) { return g_last_error.c_str(); }

csa_status csa_buffer_sizes_for(const csa_config *cfg, csa_buffer_sizes *out) {
  csa_status st = check_config(cfg);
  if (st != CSA_OK) return st;
  if (!out) return fail(CSA_ERR_INVALID_ARG, "out is NULL");
  const size_t P = cfg->pool_pages, S = cfg->max_seqs;
  const bool fp8 = cfg->kv_dtype == CSA_FP8_E4M3, fp4 = cfg->kv_dtype == CSA_FP4_E2M1;
  const int kb = dt_bytes(cfg->kv_dtype), ab = dt_bytes(cfg->act_dtype);
  out->kv_pool = fp4 ? P * kPage * kD / 2 : P * kPage * kD * kb;
  const bool idx = cfg->idx_heads > 0;
  out->idx_pool = idx ? P * kPage * kDI * kb : 0;
  out->page_scale = fp8 || fp4 ? P * 4 : 0;
  out->kv_stage = fp8 ? S * kPage * kD * 4 : 0;
  out->idx_stage = (fp8 || fp4) && idx ? S * kPage * kDI * 4 : 0;
  out->group_scale = fp4 ? P * kPage * (kD / kFp4Group) : 0;
  const bool ring8 = cfg->swa_dtype == CSA_FP8_E4M3;
  out->ring = S * static_cast<size_t>(cfg->ring_rows) * kD * (ring8 ? 1 : ab);
  out->ring_scale = ring8 ? S * static_cast<size_t>(cfg->ring_rows) * 4 : 0;
  out->block_stage = S * 3 * static_cast<size_t>(cfg->ratio) * kD * ab;
  out->block_table = S * static_cast<size_t>(cfg->max_pages_per_seq) * 4;
  return CSA_OK;
}

size_t csa_workspace_size(const csa_config *cfg, int32_t max_queries, int32_t max_k) {
  if (check_config(cfg) != CSA_OK || max_queries < 1 || max_k < 0 || max_k > CSA_MAX_TOPK) return 0;
  const int64_t E = ecap(*cfg);
  const int64_t s_dec = (E + kIdxChunk - 1) / kIdxChunk * kIdxChunk;
  const int nq_dec = std::min<int>(max_queries, kIdxMaxQ);
  const size_t a = idx_decode_bytes(nq_dec, s_dec);
  const int64_t s_chunk = (E + 63) / 64 * 64;
  const int64_t ss_chunk = (E / kChunkSample + 255) / 256 * 256 + 256;
  const size_t b = max_queries > 1 ? idx_chunk_bytes(max_queries, ss_chunk, s_chunk) : 0;
  // attention partials: a launch of nq <= nq_att queries uses nq x att_max_splits(nq)
  // query-splits, at most min(nq_att x kAttMaxSplits, kAttSplitBudget)
  const int nq_att = std::min<int>(max_queries, kAttMaxQ);
  const size_t c = attend_bytes(1, std::min(nq_att * kAttMaxSplits, kAttSplitBudget), cfg->q_heads);
  return kHead + std::max(a, std::max(b, c)) + 1024;
}

csa_status csa_cache_create(const csa_config *cfg, const csa_buffers *bufs, csa_cache_t *out) {
  csa_status st = check_config(cfg);
  if (st != CSA_OK) return st;
  if (!bufs || !out) return fail(CSA_ERR_INVALID_ARG, "buffers or out is NULL");
  const bool fp8 = cfg->kv_dtype == CSA_FP8_E4M3, fp4 = cfg->kv_dtype == CSA_FP4_E2M1;
  for (int l = 0; l < cfg->n_layers; ++l) {
    if (!bufs->kbar[l] || !bufs->vbar[l] || !bufs->ring_k[l] || !bufs->ring_v[l] || !bufs->block_stage[l])
      return fail(CSA_ERR_INVALID_ARG, "layer %d: kbar, vbar, ring_k, ring_v and block_stage are required", l);
    if (cfg->swa_dtype == CSA_FP8_E4M3 && (!bufs->ring_k_scale[l] || !bufs->ring_v_scale[l]))
      return fail(CSA_ERR_INVALID_ARG, "layer %d: an fp8 window ring needs ring_k_scale and ring_v_scale", l);
    if (fp8 && (!bufs->kbar_scale[l] || !bufs->vbar_scale[l] || !bufs->kbar_stage[l] || !bufs->vbar_stage[l]))
      return fail(CSA_ERR_INVALID_ARG, "layer %d: fp8 caches need scale and staging buffers", l);
    if (fp4 && (!bufs->kbar_gscale[l] || !bufs->vbar_gscale[l]))
      return fail(CSA_ERR_INVALID_ARG, "layer %d: fp4 caches need kbar_gscale and vbar_gscale", l);
  }
  if (!bufs->block_table || !bufs->workspace)
    return fail(CSA_ERR_INVALID_ARG, "block_table and workspace are required");
  if (cfg->idx_heads > 0 && !bufs->kidx) return fail(CSA_ERR_INVALID_ARG, "kidx is required when idx_heads > 0");
  if (cfg->idx_heads > 0 && (fp8 || fp4) && (!bufs->kidx_scale || !bufs->kidx_stage))
    return fail(CSA_ERR_INVALID_ARG, "fp8 and fp4 caches need kidx_scale and kidx_stage");
  if (reinterpret_cast<uintptr_t>(bufs->workspace) % 256 != 0) return fail(CSA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (bufs->workspace_bytes < kHead + 1024) return fail(CSA_ERR_CAPACITY, "workspace too small");
  csa_cache *h = new (std::nothrow) csa_cache();
  if (!h) return fail(CSA_ERR_INVALID_ARG, "out of host memory");
  h->magic = kMagic;
  h->cfg = *cfg;
  h->buf = *bufs;
  h->len.assign(static_cast<size_t>(cfg->n_layers) * cfg->max_seqs, 0);
  h->swa_start.assign(static_cast<size_t>(cfg->max_seqs), 0);
  h->err = reinterpret_cast<uint32_t *>(bufs->workspace);
  h->scratch = reinterpret_cast<char *>(bufs->workspace) + kHead;
  h->scratch_bytes = bufs->workspace_bytes - kHead;
  h->profiling = 0;
  h->events_used = 0;
  *out = h;
  return CSA_OK;
}

csa_status csa_cache_destroy(csa_cache_t h) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->magic = 0;
  delete h;
  return CSA_OK;
}

csa_status csa_seq_reset(csa_cache_t h, int32_t seq) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  if (seq < 0 || seq >= h->cfg.max_seqs) return fail(CSA_ERR_INVALID_ARG, "seq %d out of range", seq);
  for (int l = 0; l < h->cfg.n_layers; ++l) h->len[static_cast<size_t>(l) * h->cfg.max_seqs + seq] = 0;
  h->swa_start[seq] = 0;
  return CSA_OK;
}

csa_status csa_seq_set_swa_start(csa_cache_t h, int32_t seq, int32_t start) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  if (seq < 0 || seq >= h->cfg.max_seqs) return fail(CSA_ERR_INVALID_ARG, "seq %d out of range", seq);
  if (start < 0) return fail(CSA_ERR_INVALID_ARG, "swa start %d < 0", start);
  h->swa_start[seq] = start;
  return CSA_OK;
}

int64_t csa_seq_len(csa_cache_t h, int32_t layer, int32_t seq) {
  if (!handle_ok(h) || layer < 0 || layer >= h->cfg.n_layers || seq < 0 || seq >= h->cfg.max_seqs) return -1;
  return h->len[static_cast<size_t>(layer) * h->cfg.max_seqs + seq];
}

csa_status csa_seq_set_len(csa_cache_t h, int32_t layer, int32_t seq, int64_t len) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  if (layer < 0 || layer >= h->cfg.n_layers || seq < 0 || seq >= h->cfg.max_seqs)
    return fail(CSA_ERR_INVALID_ARG, "layer/seq out of range");
  if (len < 0 || len / h->cfg.ratio > ecap(h->cfg) || len > (1ll << 30))
    return fail(CSA_ERR_CAPACITY, "length %lld exceeds the block-table row", static_cast<long long>(len));
  h->len[static_cast<size_t>(layer) * h->cfg.max_seqs + seq] = len;
  return CSA_OK;
}

csa_status csa_compress(csa_cache_t h, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *n_new,
                        const void *raw_k, const void *raw_v, const void *gate, const float *proj_idx,
                        hipStream_t stream) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  const csa_config &c = h->cfg;
  if (layer < 0 || layer >= c.n_layers) return fail(CSA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (n_seqs < 1 || !seq_ids || !n_new) return fail(CSA_ERR_INVALID_ARG, "n_seqs >= 1 with seq_ids and n_new required");
  if ((layer == 0 && h->cfg.idx_heads > 0) != (proj_idx != nullptr))
    return fail(CSA_ERR_INVALID_ARG, "layer 0 (and only layer 0) of a group with an indexer must pass proj_idx");
  int64_t total = 0;
  std::vector<char> seen(c.max_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    if (s < 0 || s >= c.max_seqs) return fail(CSA_ERR_INVALID_ARG, "seq_ids[%d] = %d out of range", i, s);
    if (seen[s]) return fail(CSA_ERR_INVALID_ARG, "seq %d listed twice", s);
    seen[s] = 1;
    if (n_new[i] < 0) return fail(CSA_ERR_SHAPE, "n_new[%d] < 0", i);
    const int64_t nl = h->len[static_cast<size_t>(layer) * c.max_seqs + s] + n_new[i];
    if (nl > (1ll << 30) || nl / c.ratio > ecap(c))
      return fail(CSA_ERR_CAPACITY, "seq %d would hold %lld rows, more than its block-table row maps", s, static_cast<long long>(nl));
    total += n_new[i];
  }
  if (total > 0 && (!raw_k || !raw_v || !gate)) return fail(CSA_ERR_INVALID_ARG, "raw_k, raw_v and gate are required");
  if (total == 0) return CSA_OK;
  if (total > (1ll << 31) / kD) return fail(CSA_ERR_UNSUPPORTED, "too many rows in one call");

  // pages whose earlier entries are re-quantised from staging: fp8 K/V, or the fp8 indexer keys of fp4
  const bool fp8 = c.kv_dtype == CSA_FP8_E4M3 || (c.kv_dtype == CSA_FP4_E2M1 && proj_idx != nullptr);
  const int kv = main_dt(c);
  const int act = c.act_dtype == CSA_F32 ? DT_F32 : DT_BF16;
  CompressArgs base{};
  base.raw_k = raw_k; base.raw_v = raw_v; base.gate = gate;
  base.block_stage = h->buf.block_stage[layer];
  base.proj = proj_idx;
  base.kbar = h->buf.kbar[layer]; base.vbar = h->buf.vbar[layer]; base.kidx = h->buf.kidx;
  base.kbar_gs = h->buf.kbar_gscale[layer]; base.vbar_gs = h->buf.vbar_gscale[layer];
  base.kbar_scale = h->buf.kbar_scale[layer]; base.vbar_scale = h->buf.vbar_scale[layer]; base.kidx_scale = h->buf.kidx_scale;
  base.kbar_stage = h->buf.kbar_stage[layer]; base.vbar_stage = h->buf.vbar_stage[layer]; base.kidx_stage = h->buf.kidx_stage;
  base.block_table = h->buf.block_table;
  base.err = h->err;
  base.r = c.ratio; base.R = c.ring_rows; base.bt_stride = c.max_pages_per_seq; base.pool_pages = c.pool_pages;
  base.write_idx = proj_idx != nullptr;

  // items in call order; row offsets into the packed input
  std::vector<CompressItem> items;
  int64_t off = 0;
  for (int i = 0; i < n_seqs; ++i) {
    CompressItem it{};
    it.seq = seq_ids[i];
    it.old_len = static_cast<int32_t>(h->len[static_cast<size_t>(layer) * c.max_seqs + it.seq]);
    it.n_new = n_new[i];
    it.row_off = static_cast<int32_t>(off);
    off += n_new[i];
    if (it.n_new > 0) items.push_back(it);
  }

  RingArgs ring{};
  ring.raw_k = raw_k; ring.raw_v = raw_v; ring.gate = gate;
  ring.ring_k = h->buf.ring_k[layer]; ring.ring_v = h->buf.ring_v[layer];
  ring.ring_k_scale = h->buf.ring_k_scale[layer]; ring.ring_v_scale = h->buf.ring_v_scale[layer];
  ring.block_stage = h->buf.block_stage[layer];
  ring.r = c.ratio; ring.R = c.ring_rows; ring.rows_per_wg = 64; ring.write_stage = 1;
  const bool ring8 = c.swa_dtype == CSA_FP8_E4M3;

  const RingPtrs rp{raw_k, raw_v, gate, ring.ring_k, ring.ring_v, ring.ring_k_scale, ring.ring_v_scale,
                    ring.block_stage, ring.r, ring.R, ring.rows_per_wg, ring.write_stage};
  for (size_t g0 = 0; g0 < items.size(); g0 += kCompressMaxItems) {
    const size_t g1 = std::min(items.size(), g0 + kCompressMaxItems);
    // fp8 / fp4 pages, every item writing at most one page and one chunk of
    // ring rows (a single-token append): one workgroup per item does both
    bool one_step = (fp8 || kv == DT_FP4) && act == DT_BF16;
    for (size_t i = g0; i < g1 && one_step; ++i) {
      const CompressItem &it = items[i];
      const int nb_old = it.old_len / c.ratio, nb_new = (it.old_len + it.n_new) / c.ratio;
      if (nb_new > nb_old && nb_old / kPage != (nb_new - 1) / kPage) one_step = false;
      const int new_len = it.old_len + it.n_new;
      const int first = std::min(std::max(it.old_len, new_len - c.ring_rows), std::max(it.old_len, (new_len / c.ratio) * c.ratio));
      if (new_len - first > ring.rows_per_wg) one_step = false;
    }
    if (one_step) {
      CompressArgs F = base;
      F.n_items = 0;
      for (size_t i = g0; i < g1; ++i) {
        CompressItem it = items[i];
        const int nb_old = it.old_len / c.ratio, nb_new = (it.old_len + it.n_new) / c.ratio;
        it.page0 = nb_old / kPage;
        it.n_pages = nb_new > nb_old ? 1 : 0;
        F.it[F.n_items++] = it;
      }
      launch_compress_step(F, rp, kv, act, ring8, stream);
      continue;
    }
    // page launches: A = first pages holding earlier entries (fp8 only), B = the rest
    CompressArgs A = base, B = base;
    A.n_items = B.n_items = 0;
    int wgA = 0, wgB = 0;
    for (size_t i = g0; i < g1; ++i) {
      CompressItem it = items[i];
      const int nb_old = it.old_len / c.ratio, nb_new = (it.old_len + it.n_new) / c.ratio;
      if (nb_new <= nb_old) continue;
      const int p0 = nb_old / kPage, p1 = (nb_new - 1) / kPage;
      int first = p0;
      if (fp8 && nb_old % kPage != 0) {
        CompressItem a = it;
        a.page0 = p0; a.n_pages = 1;
        A.it[A.n_items++] = a;
        wgA += 1;
        first = p0 + 1;
      }
      if (first <= p1) {
        CompressItem b = it;
        b.page0 = first; b.n_pages = p1 - first + 1;
        B.it[B.n_items++] = b;
        wgB += b.n_pages;
      }
    }
    launch_compress_pages(A, wgA, kv, act, stream);
    launch_compress_pages(B, wgB, kv, act, stream);
    // ring / gate staging
    RingArgs R = ring;
    R.n_items = 0;
    int wgR = 0;
    for (size_t i = g0; i < g1; ++i) {
      const CompressItem &it = items[i];
      const int new_len = it.old_len + it.n_new;
      const int lo = std::max(it.old_len, new_len - c.ring_rows);
      const int glo = std::max(it.old_len, (new_len / c.ratio) * c.ratio);
      const int first = std::min(lo, glo);
      const int rows = new_len - first;
      if (rows <= 0) continue;
      R.it[R.n_items] = it;
      R.chunks[R.n_items] = (rows + R.rows_per_wg - 1) / R.rows_per_wg;
      wgR += R.chunks[R.n_items];
      R.n_items++;
    }
    launch_compress_ring(R, wgR, act, ring8, stream);
  }
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed in csa_compress");
  for (int i = 0; i < n_seqs; ++i) h->len[static_cast<size_t>(layer) * c.max_seqs + seq_ids[i]] += n_new[i];
  return CSA_OK;
}

csa_status csa_ring_write(csa_cache_t h, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *pos0,
                          const int32_t *n_rows, const void *raw_k, const void *raw_v, hipStream_t stream) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  const csa_config &c = h->cfg;
  if (layer < 0 || layer >= c.n_layers) return fail(CSA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (n_seqs < 1 || !seq_ids || !pos0 || !n_rows) return fail(CSA_ERR_INVALID_ARG, "n_seqs >= 1 with seq_ids, pos0, n_rows");
  int64_t total = 0;
  std::vector<CompressItem> items;
  std::vector<char> seen(c.max_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    if (s < 0 || s >= c.max_seqs) return fail(CSA_ERR_INVALID_ARG, "seq_ids[%d] out of range", i);
    if (seen[s]) return fail(CSA_ERR_INVALID_ARG, "seq %d listed twice", s);
    seen[s] = 1;
    if (n_rows[i] < 0 || pos0[i] < 0) return fail(CSA_ERR_INVALID_ARG, "negative pos0 or n_rows at %d", i);
    const int64_t L = h->len[static_cast<size_t>(layer) * c.max_seqs + s];
    if (pos0[i] + static_cast<int64_t>(n_rows[i]) > L)
      return fail(CSA_ERR_INVALID_ARG, "rows [%d, %lld) of seq %d are not appended yet", pos0[i],
                  static_cast<long long>(pos0[i]) + n_rows[i], s);
    if (pos0[i] < L - c.ring_rows)
      return fail(CSA_ERR_CAPACITY, "row %d of seq %d already left the %d-row ring", pos0[i], s, c.ring_rows);
    CompressItem it{};
    it.seq = s; it.old_len = pos0[i]; it.n_new = n_rows[i]; it.row_off = static_cast<int32_t>(total);
    total += n_rows[i];
    if (it.n_new > 0) items.push_back(it);
  }
  if (total > 0 && (!raw_k || !raw_v)) return fail(CSA_ERR_INVALID_ARG, "raw_k and raw_v are required");
  if (total == 0) return CSA_OK;
  const int act = c.act_dtype == CSA_F32 ? DT_F32 : DT_BF16;
  RingArgs ring{};
  ring.raw_k = raw_k; ring.raw_v = raw_v; ring.gate = nullptr;
  ring.ring_k = h->buf.ring_k[layer]; ring.ring_v = h->buf.ring_v[layer];
  ring.ring_k_scale = h->buf.ring_k_scale[layer]; ring.ring_v_scale = h->buf.ring_v_scale[layer];
  ring.block_stage = h->buf.block_stage[layer];
  ring.r = c.ratio; ring.R = c.ring_rows; ring.rows_per_wg = 64; ring.write_stage = 0;
  for (size_t g0 = 0; g0 < items.size(); g0 += kCompressMaxItems) {
    const size_t g1 = std::min(items.size(), g0 + kCompressMaxItems);
    RingArgs R = ring;
    R.n_items = 0;
    int wg = 0;
    for (size_t i = g0; i < g1; ++i) {
      R.it[R.n_items] = items[i];
      R.chunks[R.n_items] = (items[i].n_new + R.rows_per_wg - 1) / R.rows_per_wg;
      wg += R.chunks[R.n_items];
      R.n_items++;
    }
    launch_compress_ring(R, wg, act, c.swa_dtype == CSA_FP8_E4M3, stream);
  }
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed in csa_ring_write");
  return CSA_OK;
}

namespace {

// Argument checks shared by the index entry points.
csa_status check_index_args(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos, const void *q_idx,
                            const float *w_idx, int32_t k, const int32_t *topk) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  const csa_config &c = h->cfg;
  if (c.idx_heads == 0) return fail(CSA_ERR_UNSUPPORTED, "this layer group has no indexer (idx_heads = 0)");
  if (n_q < 1 || !q_seq || !q_pos || !q_idx || !w_idx || !topk)
    return fail(CSA_ERR_INVALID_ARG, "n_q >= 1 and all pointers are required");
  if (k < 1 || k > CSA_MAX_TOPK) return fail(CSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, CSA_MAX_TOPK);
  for (int i = 0; i < n_q; ++i) {
    if (q_seq[i] < 0 || q_seq[i] >= c.max_seqs) return fail(CSA_ERR_INVALID_ARG, "q_seq[%d] out of range", i);
    const int64_t L = h->len[q_seq[i]];
    if (q_pos[i] < 0 || q_pos[i] >= L)
      return fail(CSA_ERR_INVALID_ARG, "q_pos[%d] = %d not below the sequence length %lld", i, q_pos[i], static_cast<long long>(L));
  }
  return CSA_OK;
}

// Group size G = 2^glog2 of the threshold maxima for n scores and Top-k: at
// least 4k groups where possible, at most kMaxGroups, G <= 2^gmax.
int group_log2(int n, int k, int gmax) {
  int glog2 = 0;
  while (glog2 < gmax && (((n + (2 << glog2) - 1) >> (glog2 + 1)) >= 4 * k)) ++glog2;
  while (glog2 < gmax && ((n + (1 << glog2) - 1) >> glog2) > kMaxGroups) ++glog2;
  return glog2;
}

struct DecodeScratch {
  float *S, *M, *cs, *B;
  int32_t *cj, *cnt;
  int32_t max_slices;
};

DecodeScratch carve_decode(csa_cache_t h, int nq, int64_t s_stride) {
  DecodeScratch d{};
  char *p = h->scratch;
  const size_t row = align_up(static_cast<size_t>(nq) * s_stride * 4, 256);
  d.S = reinterpret_cast<float *>(p); p += row;
  d.M = reinterpret_cast<float *>(p); p += row;
  d.cs = reinterpret_cast<float *>(p); p += row;
  d.cj = reinterpret_cast<int32_t *>(p); p += row;
  d.cnt = reinterpret_cast<int32_t *>(p); p += align_up(static_cast<size_t>(nq) * max_slices_for(s_stride) * 4, 256);
  d.B = reinterpret_cast<float *>(p);
  d.max_slices = static_cast<int32_t>(max_slices_for(s_stride));
  return d;
}

// Prefill chunk: queries of one sequence at consecutive positions.
csa_status index_chunk(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos, const void *q_idx,
                       const float *w_idx, int32_t k, int32_t *topk, int32_t n_pool, int32_t *pool, hipStream_t stream) {
  const csa_config &c = h->cfg;
  const int kv = idx_dt(c);
  const int act = c.act_dtype == CSA_F32 ? DT_F32 : DT_BF16;
  const int pos0 = q_pos[0];
  const int n_max = (pos0 + n_q) / c.ratio;
  const int64_t ss_stride = (static_cast<int64_t>(n_max) / kChunkSample + 255) / 256 * 256 + 256;
  const int64_t fb_stride = (static_cast<int64_t>(n_max) + 63) / 64 * 64;
  const size_t need = idx_chunk_bytes(n_q, ss_stride, fb_stride);
  if (need > h->scratch_bytes) return fail(CSA_ERR_CAPACITY, "workspace too small for a %d-token chunk (%zu > %zu bytes)", n_q, need, h->scratch_bytes);
  char *p = h->scratch;
  IdxChunkArgs s{};
  s.ss = reinterpret_cast<float *>(p); p += align_up(static_cast<size_t>(n_q) * ss_stride * 4, 256);
  const int64_t tiles = (fb_stride + 255) / 256;
  s.tau = reinterpret_cast<float *>(p); p += align_up(static_cast<size_t>(n_q) * 4, 256);
  s.cnt = reinterpret_cast<int32_t *>(p); p += align_up(static_cast<size_t>(n_q) * tiles * 4, 256);
  s.cand = reinterpret_cast<uint64_t *>(p); p += align_up(static_cast<size_t>(n_q) * tiles * kChunkTileCand * 8, 256);
  s.fb_rows = reinterpret_cast<float *>(p);
  s.kidx = h->buf.kidx; s.kidx_scale = h->buf.kidx_scale;
  s.bt_row = h->buf.block_table + static_cast<int64_t>(q_seq[0]) * c.max_pages_per_seq;
  s.q_idx = q_idx; s.w_idx = w_idx; s.topk = topk; s.err = h->err;
  s.pool_pages = c.pool_pages; s.h_i = c.idx_heads; s.ss_stride = static_cast<int32_t>(ss_stride);
  s.fb_stride = static_cast<int32_t>(fb_stride); s.n_tok = n_q; s.pos0 = pos0; s.r = c.ratio; s.k = k;
  s.m_s = std::max(1, (2 * k + kChunkSample - 1) / kChunkSample);
  s.n_etiles = (n_max + 255) / 256;
  s.n_stiles = (n_max / kChunkSample + 255) / 256;
  s.kv_dtype = kv; s.act_dtype = act;
  // pool: block maxima in the fallback rows, selected before the Top-K select can reuse them
  s.pool = pool; s.n_pool = n_pool;
  s.bmax = pool ? s.fb_rows : nullptr; s.bm_stride = s.fb_stride;
  const ProfPair ev = prof_events(h, stream, CSA_PROFILE_INDEX);
  launch_idx_chunk(s, kv, act, stream, ev.start, ev.stop);
  launch_idx_chunk_pool(s, stream);
  launch_idx_chunk_select(s, stream);
  return CSA_OK;
}

// Per-query path: scan -> filter -> final, plus the candidate pool when pool
// is not null.
csa_status index_per_query(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos, const void *q_idx,
                           const float *w_idx, int32_t k, int32_t *topk, int32_t n_pool, int32_t *pool,
                           hipStream_t stream) {
  const csa_config &c = h->cfg;
  const int kv = idx_dt(c);
  const int act = c.act_dtype == CSA_F32 ? DT_F32 : DT_BF16;
  const int ab = dt_bytes(c.act_dtype);
  for (int g0 = 0; g0 < n_q; g0 += kIdxMaxQ) {
    const int nq = std::min(kIdxMaxQ, n_q - g0);
    int nmax = 0;
    for (int i = 0; i < nq; ++i) nmax = std::max(nmax, (q_pos[g0 + i] + 1) / c.ratio);
    // short rows (no pool): one workgroup per query scores and selects
    const int key_bytes = kv == DT_F32 ? 4 : (kv == DT_BF16 ? 2 : 1);
    if (!pool && nmax <= kSmallEntries && static_cast<int64_t>(nmax) * kDI * key_bytes <= kSmallBytes) {
      IdxScanArgs s{};
      s.kidx = h->buf.kidx; s.kidx_scale = h->buf.kidx_scale; s.block_table = h->buf.block_table;
      s.q_idx = reinterpret_cast<const char *>(q_idx) + static_cast<int64_t>(g0) * c.idx_heads * kDI * ab;
      s.w_idx = w_idx + static_cast<int64_t>(g0) * c.idx_heads;
      s.err = h->err;
      s.bt_stride = c.max_pages_per_seq; s.pool_pages = c.pool_pages; s.h_i = c.idx_heads; s.n_q = nq;
      for (int i = 0; i < nq; ++i) {
        s.q[i].seq = q_seq[g0 + i];
        s.q[i].n_vis = (q_pos[g0 + i] + 1) / c.ratio;
      }
      const ProfPair ev = prof_events(h, stream, CSA_PROFILE_INDEX);
      launch_idx_small(s, kv, act, topk + static_cast<int64_t>(g0) * k, k, stream, ev.start, ev.stop);
      continue;
    }
    const int64_t s_stride = std::max<int64_t>(kIdxChunk, (static_cast<int64_t>(nmax) + kIdxChunk - 1) / kIdxChunk * kIdxChunk);
    const size_t need = idx_decode_bytes(nq, s_stride);
    if (need > h->scratch_bytes)
      return fail(CSA_ERR_CAPACITY, "workspace too small for %d queries indexed one by one (%zu > %zu bytes)", nq, need,
                  h->scratch_bytes);
    const DecodeScratch d = carve_decode(h, nq, s_stride);

    IdxScanArgs s{};
    s.kidx = h->buf.kidx; s.kidx_scale = h->buf.kidx_scale; s.block_table = h->buf.block_table;
    s.q_idx = reinterpret_cast<const char *>(q_idx) + static_cast<int64_t>(g0) * c.idx_heads * kDI * ab;
    s.w_idx = w_idx + static_cast<int64_t>(g0) * c.idx_heads;
    s.S = d.S; s.M = d.M; s.B = pool ? d.B : nullptr; s.err = h->err;
    s.bt_stride = c.max_pages_per_seq; s.pool_pages = c.pool_pages; s.h_i = c.idx_heads;
    s.s_stride = static_cast<int32_t>(s_stride); s.n_q = nq;
    IdxFilterArgs f{};
    f.S = d.S; f.M = d.M; f.cand_s = d.cs; f.cand_j = d.cj; f.cnt = d.cnt; f.s_stride = s.s_stride; f.k = k; f.n_q = nq;
    f.max_slices = d.max_slices;
    IdxFinalArgs fin{};
    fin.S = d.S; fin.cand_s = d.cs; fin.cand_j = d.cj; fin.cnt = d.cnt; fin.err = h->err;
    fin.topk = topk + static_cast<int64_t>(g0) * k; fin.s_stride = s.s_stride; fin.k = k; fin.n_q = nq;
    fin.max_slices = d.max_slices;
    // the pool reuses filter and final on the block maxima B: a group of G >= 8
    // entries is a group of G / 8 whole blocks, so the topk's group maxima M
    // are maxima of distinct blocks and bound the n_pool-th block maximum
    IdxFilterArgs pf = f;
    pf.S = d.B; pf.k = n_pool;
    IdxFinalArgs pfin = fin;
    pfin.S = d.B; pfin.k = n_pool; pfin.topk = pool ? pool + static_cast<int64_t>(g0) * n_pool : nullptr;
    int wg = 0, slices = 0, pslices = 0;
    for (int i = 0; i < nq; ++i) {
      const int N = (q_pos[g0 + i] + 1) / c.ratio;
      // groups of G <= 256 entries that stay within one scan workgroup
      constexpr int kGMax = kIdxChunk < 256 ? (kIdxChunk < 128 ? 6 : 7) : 8;
      static_assert(kIdxChunk >= 64, "a scan workgroup covers whole pages");
      const int glog2 = group_log2(N, k, kGMax);
      if (((N + (1 << glog2) - 1) >> glog2) > kMaxGroups)
        return fail(CSA_ERR_UNSUPPORTED, "query %d sees %d entries; at most %d are supported for k = %d", g0 + i, N, kMaxGroups << kGMax, k);
      s.q[i].seq = q_seq[g0 + i];
      s.q[i].n_vis = N;
      s.q[i].chunk0 = wg;
      s.q[i].glog2 = glog2;
      wg += (N + kIdxChunk - 1) / kIdxChunk;
      f.slice0[i] = slices;
      f.n_vis[i] = N;
      f.glog2[i] = glog2;
      slices += N > k ? (N + kFilterSlice - 1) / kFilterSlice : 0;
      fin.n_vis[i] = N;
      const int nb = (N + kPoolBlock - 1) / kPoolBlock;
      pf.slice0[i] = pslices;
      pf.n_vis[i] = nb;
      // groups smaller than a block give no bound: a huge group count of 1 turns the threshold off
      pf.glog2[i] = glog2 >= 3 ? glog2 - 3 : 30;
      pslices += nb > n_pool ? (nb + kFilterSlice - 1) / kFilterSlice : 0;
      pfin.n_vis[i] = nb;
    }
    f.slice0[nq] = slices;
    pf.slice0[nq] = pslices;
    s.total_wg = wg;
    f.uniform = uniform_count([&](int i) { return f.slice0[i]; }, nq, slices);
    pf.uniform = uniform_count([&](int i) { return pf.slice0[i]; }, nq, pslices);
    const ProfPair ev = prof_events(h, stream, CSA_PROFILE_INDEX);
    launch_idx_scan(s, kv, act, stream, ev.start, ev.stop);
    launch_idx_filter(f, slices, stream);
    launch_idx_final(fin, stream);
    if (pool) {
      launch_idx_filter(pf, pslices, stream);
      launch_idx_final(pfin, stream);
    }
  }
  return CSA_OK;
}

}  // namespace

csa_status csa_index_topk(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos, const void *q_idx,
                          const float *w_idx, int32_t k, int32_t *topk, hipStream_t stream) {
  csa_status st = check_index_args(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk);
  if (st != CSA_OK) return st;
  st = index_as_chunk(h->cfg, n_q, q_seq, q_pos)
           ? index_chunk(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk, 0, nullptr, stream)
           : index_per_query(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk, 0, nullptr, stream);
  if (st != CSA_OK) return st;
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed in csa_index_topk");
  return CSA_OK;
}

csa_status csa_index_topk_pool(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                               const void *q_idx, const float *w_idx, int32_t k, int32_t *topk,
                               int32_t n_pool_blocks, int32_t *pool, hipStream_t stream) {
  csa_status st = check_index_args(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk);
  if (st != CSA_OK) return st;
  if (n_pool_blocks < 1 || n_pool_blocks > CSA_MAX_POOL_BLOCKS)
    return fail(CSA_ERR_UNSUPPORTED, "n_pool_blocks = %d outside [1, %d]", n_pool_blocks, CSA_MAX_POOL_BLOCKS);
  if (!pool) return fail(CSA_ERR_INVALID_ARG, "pool is required");
  st = index_as_chunk(h->cfg, n_q, q_seq, q_pos)
           ? index_chunk(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk, n_pool_blocks, pool, stream)
           : index_per_query(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk, n_pool_blocks, pool, stream);
  if (st != CSA_OK) return st;
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed in csa_index_topk_pool");
  return CSA_OK;
}

csa_status csa_index_reindex(csa_cache_t h, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                             const void *q_idx, const float *w_idx, int32_t n_pool_blocks, const int32_t *pool,
                             int32_t k, int32_t *topk, hipStream_t stream) {
  csa_status st = check_index_args(h, n_q, q_seq, q_pos, q_idx, w_idx, k, topk);
  if (st != CSA_OK) return st;
  if (n_pool_blocks < 1 || n_pool_blocks > CSA_MAX_POOL_BLOCKS)
    return fail(CSA_ERR_UNSUPPORTED, "n_pool_blocks = %d outside [1, %d]", n_pool_blocks, CSA_MAX_POOL_BLOCKS);
  if (!pool) return fail(CSA_ERR_INVALID_ARG, "pool is required");
  const csa_config &c = h->cfg;
  const int kv = idx_dt(c);
  const int act = c.act_dtype == CSA_F32 ? DT_F32 : DT_BF16;
  const int ab = dt_bytes(c.act_dtype);
  for (int g0 = 0; g0 < n_q; g0 += kIdxMaxQ) {
    const int nq = std::min(kIdxMaxQ, n_q - g0);
    // positions of query i: min(pool blocks, visible blocks) * 8, cut at the visible entries
    std::vector<int> npos(nq), nent(nq);
    int vmax = 0;
    for (int i = 0; i < nq; ++i) {
      nent[i] = (q_pos[g0 + i] + 1) / c.ratio;
      const int nb = std::min(n_pool_blocks, (nent[i] + kPoolBlock - 1) / kPoolBlock);
      npos[i] = std::min(nb * kPoolBlock, nent[i]);
      vmax = std::max(vmax, npos[i]);
    }
    const int64_t s_stride = std::max<int64_t>(kIdxChunk, (static_cast<int64_t>(vmax) + kIdxChunk - 1) / kIdxChunk * kIdxChunk);
    const size_t need = idx_decode_bytes(nq, s_stride);
    if (need > h->scratch_bytes)
      return fail(CSA_ERR_CAPACITY, "workspace too small for %d queries indexed one by one (%zu > %zu bytes)", nq, need,
                  h->scratch_bytes);
    const DecodeScratch d = carve_decode(h, nq, s_stride);
    IdxRescanArgs s{};
    s.kidx = h->buf.kidx; s.kidx_scale = h->buf.kidx_scale; s.block_table = h->buf.block_table;
    s.q_idx = reinterpret_cast<const char *>(q_idx) + static_cast<int64_t>(g0) * c.idx_heads * kDI * ab;
    s.w_idx = w_idx + static_cast<int64_t>(g0) * c.idx_heads;
    s.pool = pool + static_cast<int64_t>(g0) * n_pool_blocks; s.pool_stride = n_pool_blocks;
    s.S = d.S; s.M = d.M; s.err = h->err;
    s.bt_stride = c.max_pages_per_seq; s.pool_pages = c.pool_pages; s.h_i = c.idx_heads;
    s.s_stride = static_cast<int32_t>(s_stride); s.n_q = nq;
    IdxFilterArgs f{};
    f.S = d.S; f.M = d.M; f.cand_s = d.cs; f.cand_j = d.cj; f.cnt = d.cnt; f.s_stride = s.s_stride; f.k = k; f.n_q = nq;
    f.max_slices = d.max_slices;
    IdxFinalArgs fin{};
    fin.S = d.S; fin.cand_s = d.cs; fin.cand_j = d.cj; fin.cnt = d.cnt; fin.err = h->err;
    fin.topk = topk + static_cast<int64_t>(g0) * k; fin.s_stride = s.s_stride; fin.k = k; fin.n_q = nq;
    fin.max_slices = d.max_slices;
    fin.pool = s.pool; fin.pool_stride = n_pool_blocks;
    int wg = 0, slices = 0;
    for (int i = 0; i < nq; ++i) {
      const int V = npos[i];
      const int glog2 = group_log2(V, k, 4);   // groups stay inside one 16-position MFMA tile
      s.q[i].seq = q_seq[g0 + i];
      s.q[i].n_vis = V;
      s.q[i].chunk0 = wg;
      s.q[i].glog2 = glog2;
      s.n_ent[i] = nent[i];
      wg += (V + kRescanChunk - 1) / kRescanChunk;
      f.slice0[i] = slices;
      f.n_vis[i] = V;
      f.glog2[i] = glog2;
      slices += V > k ? (V + kFilterSlice - 1) / kFilterSlice : 0;
      fin.n_vis[i] = V;
      fin.n_ent[i] = nent[i];
    }
    f.slice0[nq] = slices;
    s.total_wg = wg;
    f.uniform = uniform_count([&](int i) { return f.slice0[i]; }, nq, slices);
    const ProfPair ev = prof_events(h, stream, CSA_PROFILE_INDEX);
    launch_idx_rescan(s, kv, act, stream, ev.start, ev.stop);
    launch_idx_filter(f, slices, stream);
    launch_idx_final(fin, stream);
  }
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed in csa_index_reindex");
  return CSA_OK;
}

namespace {

// Shared by csa_attend (keys = the Top-K rows) and csa_attend_dense (keys =
// every visible entry: topk is NULL and k is replaced by the largest visible count).
// scratch: where the split partials go (the handle's workspace, or the static
// scratch of csa_attend_noalloc, which also records no profiling events)
csa_status attend_impl(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                       const void *q, const int32_t *topk, int32_t k, bool dense, float scale, void *out,
                       hipStream_t stream, char *scratch_base, size_t scratch_bytes, bool profile) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  const csa_config &c = h->cfg;
  if (layer < 0 || layer >= c.n_layers) return fail(CSA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (n_q < 1 || !q_seq || !q_pos || !q || !out) return fail(CSA_ERR_INVALID_ARG, "n_q >= 1 and q_seq, q_pos, q, out required");
  if (!dense) {
    if (k < 0 || k > CSA_MAX_TOPK) return fail(CSA_ERR_UNSUPPORTED, "k = %d outside [0, %d]", k, CSA_MAX_TOPK);
    if (k > 0 && !topk) return fail(CSA_ERR_INVALID_ARG, "topk required when k > 0");
  }
  for (int i = 0; i < n_q; ++i) {
    if (q_seq[i] < 0 || q_seq[i] >= c.max_seqs) return fail(CSA_ERR_INVALID_ARG, "q_seq[%d] out of range", i);
    const int64_t L = h->len[static_cast<size_t>(layer) * c.max_seqs + q_seq[i]];
    if (q_pos[i] < 0 || q_pos[i] >= L)
      return fail(CSA_ERR_INVALID_ARG, "q_pos[%d] = %d not below the layer's sequence length %lld", i, q_pos[i], static_cast<long long>(L));
    if (c.window > 0 && (L - 1 - q_pos[i]) > c.ring_rows - c.window)
      return fail(CSA_ERR_CAPACITY, "query %d: window rows already left the %d-row ring", i, c.ring_rows);
  }
  if (dense) {
    k = 0;
    for (int i = 0; i < n_q; ++i) k = std::max(k, (q_pos[i] + 1) / c.ratio);
  }
  const int kv = main_dt(c);
  // the splits of one query (the keys a workgroup resolves up front times the
  // splits the merge combines) bound the keys a decode query can attend to
  {
    const int ms = att_max_splits(std::min(n_q, kAttMaxQ));
    const int per_split = kv == DT_F32 ? kAttMaxSplitKeys : kAttSplitMaxKeys;
    const int64_t nb = n_blocks_for(k, c.window);
    if (!is_chunk(n_q, q_seq, q_pos) && nb > static_cast<int64_t>(ms) * (per_split / kKeyBlock))
      return fail(CSA_ERR_UNSUPPORTED, "a query attends to %lld keys (%d entries + window %d); at most %d are supported",
                  static_cast<long long>(nb * kKeyBlock), k, c.window, ms * per_split);
  }
  const int act = c.act_dtype == CSA_F32 ? DT_F32 : DT_BF16;
  const int ab = dt_bytes(c.act_dtype);
  AttendArgs a{};
  a.kbar = h->buf.kbar[layer]; a.vbar = h->buf.vbar[layer];
  a.kbar_scale = h->buf.kbar_scale[layer]; a.vbar_scale = h->buf.vbar_scale[layer];
  a.kbar_gs = h->buf.kbar_gscale[layer]; a.vbar_gs = h->buf.vbar_gscale[layer];
  a.ring_k = h->buf.ring_k[layer]; a.ring_v = h->buf.ring_v[layer];
  a.ring_k_scale = h->buf.ring_k_scale[layer]; a.ring_v_scale = h->buf.ring_v_scale[layer];
  a.pool_bytes = static_cast<uint32_t>(pool_bytes_of(c));   // check_config bounds both by kAttMaxBufferBytes
  a.ring_bytes = static_cast<uint32_t>(ring_bytes_of(c));
  a.gs_bytes = kv == DT_FP4 ? static_cast<uint32_t>(static_cast<uint64_t>(c.pool_pages) * kPage * (kD / kFp4Group)) : 0u;
  const bool ring8 = c.swa_dtype == CSA_FP8_E4M3;
  a.block_table = h->buf.block_table;
  a.err = h->err;
  a.scale = scale; a.k = k; a.W = c.window; a.R = c.ring_rows; a.r = c.ratio; a.dense = dense ? 1 : 0;
  a.bt_stride = c.max_pages_per_seq; a.pool_pages = c.pool_pages; a.H = c.q_heads;
  a.act_f32 = act == DT_F32 ? 1 : 0;
  a.n_sparse_blocks = (k + kKeyBlock - 1) / kKeyBlock;
  a.n_blocks = n_blocks_for(k, c.window);
  const size_t qrow = static_cast<size_t>(c.q_heads) * kD * ab;

  if (is_chunk(n_q, q_seq, q_pos) && a.n_blocks * kKeyBlock <= kAttMaxSplitKeys) {
    a.q = q; a.out = out; a.topk = topk;
    a.chunk = 1; a.seq0 = q_seq[0]; a.pos0 = q_pos[0]; a.swa0 = h->swa_start[q_seq[0]];
    a.blocks_per_split = std::max(1, a.n_blocks); a.n_splits = 1; a.n_q = n_q;
    const ProfPair ev = profile ? prof_events(h, stream, CSA_PROFILE_ATTEND) : ProfPair{};
    launch_attend(a, n_q, kv, act, ring8, stream, ev.start, ev.stop);
  } else if (kv != DT_F32) {
    // decode and dense queries: one 64-key block per workgroup for a decode
    // query (its blocks' gathers run side by side on as many CUs); several
    // rounds of one block per workgroup for a dense query, whose many blocks
    // would otherwise leave the merge with too many partials
    for (int g0 = 0; g0 < n_q; g0 += kAttMaxQ) {
      const int nq = std::min(kAttMaxQ, n_q - g0);
      AttendArgs b = a;
      b.q = reinterpret_cast<const char *>(q) + g0 * qrow;
      b.out = reinterpret_cast<char *>(out) + g0 * qrow;
      b.topk = topk && !dense ? topk + static_cast<int64_t>(g0) * k : nullptr;
      b.chunk = 0; b.n_q = nq;
      for (int i = 0; i < nq; ++i) {
        b.qd[i].seq = q_seq[g0 + i];
        b.qd[i].pos = q_pos[g0 + i];
        b.qd[i].swa = h->swa_start[q_seq[g0 + i]];
      }
      const int nb = std::max(1, b.n_blocks);
      const int ms = att_max_splits(nq);
      // a large decode batch already fills the chip: two blocks per workgroup
      // halve the partials the merge reads
      int rounds = dense ? (nb + kAttDenseSplits - 1) / kAttDenseSplits : (nq * nb > kAttWideBatch ? 2 : 1);
      rounds = std::max(rounds, (nb + ms - 1) / ms);
      rounds = std::min(rounds, kAttSplitMaxKeys / kKeyBlock);
      const int splits = (nb + rounds - 1) / rounds;
      if (splits > ms) return fail(CSA_ERR_UNSUPPORTED, "too many attention splits per query");
      b.blocks_per_split = rounds;
      b.n_splits = splits;
      if (splits > 1) {
        const size_t need = attend_bytes(nq, splits, c.q_heads);
        if (need > scratch_bytes)
          return fail(CSA_ERR_CAPACITY, "attention partials need %zu bytes of scratch, %zu available", need, scratch_bytes);
        b.part_o = reinterpret_cast<float *>(scratch_base);
        b.part_ml = reinterpret_cast<float *>(scratch_base + align_up(static_cast<size_t>(nq) * splits * c.q_heads * kD * 4, 256));
      }
      const ProfPair ev = profile ? prof_events(h, stream, CSA_PROFILE_ATTEND) : ProfPair{};
      launch_attend_decode(b, nq * splits, kv, ring8, stream, ev.start, ev.stop);
    }
  } else {
    for (int g0 = 0; g0 < n_q; g0 += kAttMaxQ) {
      const int nq = std::min(kAttMaxQ, n_q - g0);
      AttendArgs b = a;
      b.q = reinterpret_cast<const char *>(q) + g0 * qrow;
      b.out = reinterpret_cast<char *>(out) + g0 * qrow;
      b.topk = topk && !dense ? topk + static_cast<int64_t>(g0) * k : nullptr;
      b.chunk = 0; b.n_q = nq;
      for (int i = 0; i < nq; ++i) {
        b.qd[i].seq = q_seq[g0 + i];
        b.qd[i].pos = q_pos[g0 + i];
        b.qd[i].swa = h->swa_start[q_seq[g0 + i]];
      }
      const int nb = std::max(1, b.n_blocks);
      b.blocks_per_split = attend_blocks_per_split(nq, nb);
      b.n_splits = (nb + b.blocks_per_split - 1) / b.blocks_per_split;
      if (b.n_splits > kAttMaxSplits) return fail(CSA_ERR_UNSUPPORTED, "too many attention splits per query");
      if (b.n_splits > 1) {
        const size_t need = attend_bytes(nq, b.n_splits, c.q_heads);
        if (need > scratch_bytes)
          return fail(CSA_ERR_CAPACITY, "attention partials need %zu bytes of scratch, %zu available", need, scratch_bytes);
        b.part_o = reinterpret_cast<float *>(scratch_base);
        b.part_ml = reinterpret_cast<float *>(scratch_base + align_up(static_cast<size_t>(nq) * b.n_splits * c.q_heads * kD * 4, 256));
      }
      const ProfPair ev = profile ? prof_events(h, stream, CSA_PROFILE_ATTEND) : ProfPair{};
      launch_attend(b, nq * b.n_splits, kv, act, ring8, stream, ev.start, ev.stop);
    }
  }
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed in csa_attend");
  return CSA_OK;
}

}  // namespace

csa_status csa_attend(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos, const void *q,
                      const int32_t *topk, int32_t k, float scale, void *out, hipStream_t stream) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  return attend_impl(h, layer, n_q, q_seq, q_pos, q, topk, k, false, scale, out, stream, h->scratch, h->scratch_bytes,
                     true);
}

csa_status csa_attend_noalloc(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                              const void *q, const int32_t *topk, int32_t k, float scale, void *out,
                              hipStream_t stream) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  char *p = static_scratch();
  if (!p) return CSA_ERR_HIP;
  return attend_impl(h, layer, n_q, q_seq, q_pos, q, topk, k, false, scale, out, stream, p, kStaticScratchBytes,
                     false);
}

csa_status csa_attend_dense(csa_cache_t h, int32_t layer, int32_t n_q, const int32_t *q_seq, const int32_t *q_pos,
                            const void *q, float scale, void *out, hipStream_t stream) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  return attend_impl(h, layer, n_q, q_seq, q_pos, q, nullptr, 0, true, scale, out, stream, h->scratch,
                     h->scratch_bytes, true);
}

csa_status csa_read_errors(csa_cache_t h, hipStream_t stream, uint32_t *flags) {
  if (!handle_ok(h) || !flags) return fail(CSA_ERR_INVALID_ARG, "invalid handle or flags");
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(CSA_ERR_HIP, "stream synchronize failed");
  uint32_t v = 0;
  if (hipMemcpy(&v, h->err, 4, hipMemcpyDeviceToHost) != hipSuccess) return fail(CSA_ERR_HIP, "error-word read failed");
  if (hipMemset(h->err, 0, 4) != hipSuccess) return fail(CSA_ERR_HIP, "error-word clear failed");
  *flags = v;
  return CSA_OK;
}

csa_status csa_profile_begin(csa_cache_t h, int32_t kernels) {
  if (!handle_ok(h)) return fail(CSA_ERR_INVALID_ARG, "invalid handle");
  if (kernels <= 0 || (kernels & ~(CSA_PROFILE_INDEX | CSA_PROFILE_ATTEND)))
    return fail(CSA_ERR_INVALID_ARG, "kernels must be a nonzero mask of CSA_PROFILE_INDEX / CSA_PROFILE_ATTEND");
  h->profiling = kernels;
  h->events_used = 0;
  return CSA_OK;
}

csa_status csa_profile_end(csa_cache_t h, int32_t kernel, double *total_ms, int32_t *launches) {
  if (!handle_ok(h) || !total_ms || !launches) return fail(CSA_ERR_INVALID_ARG, "invalid arguments");
  if (kernel != CSA_PROFILE_INDEX && kernel != CSA_PROFILE_ATTEND)
    return fail(CSA_ERR_INVALID_ARG, "kernel must be CSA_PROFILE_INDEX or CSA_PROFILE_ATTEND");
  double tot = 0.0;
  int32_t n = 0;
  for (size_t i = 0; i < h->events_used; ++i) {
    if (h->event_kind[i] != kernel) continue;
    if (hipEventSynchronize(h->events[2 * i + 1]) != hipSuccess) return fail(CSA_ERR_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, h->events[2 * i], h->events[2 * i + 1]) != hipSuccess)
      return fail(CSA_ERR_HIP, "elapsed time failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  h->profiling &= ~kernel;
  if (h->profiling == 0) h->events_used = 0;
  return CSA_OK;
}

csa_status csa_debug_stream_read(const void *const *bufs, int32_t n_bufs, int64_t bytes, int32_t reps,
                                 hipStream_t stream, float *avg_us) {
  if (!bufs || n_bufs < 1 || !avg_us || reps < 1 || bytes <= 0 || bytes % 16 != 0)
    return fail(CSA_ERR_INVALID_ARG, "bad stream-read arguments");
  for (int i = 0; i < n_bufs; ++i)
    if (!bufs[i] || reinterpret_cast<uintptr_t>(bufs[i]) % 16 != 0)
      return fail(CSA_ERR_INVALID_ARG, "buffer %d is null or not 16-byte aligned", i);
  const int64_t n16 = bytes / 16, blocks = (n16 + 1023) / 1024;
  std::vector<hipEvent_t> ev(2 * static_cast<size_t>(reps), nullptr);
  csa_status st = CSA_OK;
  for (auto &e : ev)
    if (hipEventCreate(&e) != hipSuccess) { st = fail(CSA_ERR_HIP, "event creation failed"); break; }
  if (st == CSA_OK) {
    for (int r = 0; r < reps; ++r)
      hipExtLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ev[2 * r],
                            ev[2 * r + 1], 0, reinterpret_cast<const uint4 *>(bufs[r % n_bufs]), n16);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) {
      st = fail(CSA_ERR_HIP, "stream-read launch failed");
    } else {
      double tot = 0.0;
      for (int r = 0; r < reps; ++r) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]) != hipSuccess) { st = fail(CSA_ERR_HIP, "event timing failed"); break; }
        tot += ms;
      }
      if (st == CSA_OK) *avg_us = static_cast<float>(tot * 1e3 / reps);
    }
  }
  for (auto &e : ev)
    if (e) (void)hipEventDestroy(e);
  return st;
}

csa_status csa_debug_convert(int32_t kind, const void *in, void *out, int64_t n, hipStream_t stream) {
  if (kind < 0 || kind > 5 || !in || !out || n < 0) return fail(CSA_ERR_INVALID_ARG, "bad debug conversion arguments");
  if (kind == 4 && n % 4 != 0) return fail(CSA_ERR_INVALID_ARG, "kind 4 takes whole 32-bit words (n % 4 == 0)");
  if (n == 0) return CSA_OK;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(debug_convert_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, kind, in, out, n);
  if (hipGetLastError() != hipSuccess) return fail(CSA_ERR_HIP, "kernel launch failed");
  return CSA_OK;
}

}  // extern "C"
