// csa_index_topk kernels: lightning-indexer scores over the paged indexer-key
// cache and an exact per-query Top-K.
//
// Method: DeepSeek-V4.1-Flash technical-report walkthrough, "Compressed Sparse
// Attention 2" > "The indexer selects, SWA covers the rest" (indexer query
// scores the main-KV entries through their indexer keys; the top entries per
// query are kept); Model-architectures atlas, trained-sparse-attention entry
// (a lightning indexer run as MQA, several query heads over one key).
// Score: s[t][j] = sum_h w[t][h] * max(0, q[t][h] . KI[j]).
//
// Decode (one query per sequence):
//   scan   - one workgroup per 1,024 visible entries of a query. MFMA with the
//            indexer heads as rows (16x16 tiles, rows >= H_I zero) and 16
//            entries as columns; writes fp32 scores and the max of every group
//            of G consecutive scores.
//   filter - tau = the k-th largest group maximum is a lower bound of the
//            k-th largest score (the maxima are k distinct scores). Each
//            workgroup re-derives tau by an LDS radix select and appends the
//            scores >= tau of its slice to a candidate list.
//   final  - exact selection among the candidates on 64-bit keys
//            (score bits, ~index), so ties go to the lower index; bitonic sort
//            of the chosen indices; -1 padding.
// Prefill chunk (queries of one sequence at consecutive positions):
//   chunk scan   - MFMA GEMM tile of 32 queries x 256 entries, with (query,
//                  head) pairs as the 16 rows of each tile, so every lane's 4
//                  accumulators are the 4 heads of one (query, entry) score.
//   chunk select - per query: tau from its group maxima, filter, exact select.
#include <type_traits>

#include "csa_device.h"
#include <hip/hip_ext.h>

#include "csa_internal.h"

namespace csa {

namespace {

template <int KV> struct ComputeT { using type = __bf16; };
template <> struct ComputeT<DT_F32> { using type = float; };

template <int SD> constexpr int elem_bytes() { return SD == DT_F32 ? 4 : (SD == DT_BF16 ? 2 : 1); }

// ------------------------------------------------------------------ block radix select

// Value of the k-th largest (1 <= k <= n) of n 64-bit keys produced by get(i),
// by MSB-first radix passes over 8-bit digits with an LDS histogram.
template <typename Get>
__device__ uint64_t kth_largest_u64(Get get, int n, int k, int *hist, int *sh) {
  const int t = threadIdx.x, bd = blockDim.x, lane = t & 63;
  uint64_t prefix = 0;
  int rem = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int i = t; i < 256; i += bd) hist[i] = 0;
    __syncthreads();
    for (int i = t; i < n; i += bd) {
      const uint64_t v = get(i);
      if ((v & hmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1);
    }
    __syncthreads();
    if (t < 64) {
      int c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; s += c[j]; }
      int incl = s;
      incl = wave_incl_sum(incl);
      const int excl = incl - s;
      if (excl < rem && rem <= incl) {
        int cum = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= rem) { sh[0] = 255 - 4 * lane - j; sh[1] = rem - cum; break; }
          cum += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= static_cast<uint64_t>(sh[0]) << shift;
    rem = sh[1];
    __syncthreads();
  }
  return prefix;
}

// max(x, 0) as one integer max on the bit pattern (negative floats, -0.0
// included, are negative integers); no NaN quieting step.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sort keys: a score's 32 bits in an order-preserving form (non-negative
// scores get the sign bit set, negative ones - a missing page's -1 - have
// every bit flipped, so they sort below every real score; -0 counts as +0),
// then ~index so that equal scores go to the lower index.
__device__ __forceinline__ uint32_t score_bits(float s) {
  const uint32_t u = s == 0.f ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float bits_score(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}
__device__ __forceinline__ uint64_t score_key(float s, int j) {
  return (static_cast<uint64_t>(score_bits(s)) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(j));
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key & 0xffffffffull));
}

// Ascending bitonic sort of n (power of two) ints in LDS.
__device__ void bitonic_sort(int *arr, int n) {
  const int t = threadIdx.x, bd = blockDim.x;
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < (n >> 1); i += bd) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int x = arr[lo], y = arr[hi];
        if ((x > y) == asc) { arr[lo] = y; arr[hi] = x; }
      }
      __syncthreads();
    }
  }
}

constexpr int kSelCap = 6144;   // candidates held in LDS by the select kernels
constexpr int kTauBins = 1024;

__device__ __forceinline__ float block_reduce_max(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_reduce_min(float v, float *red) {
  v = wave_min(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fminf(r, red[i]);
  return r;
}

// Block-wide min and max in one exchange (red holds >= 2 x waves floats).
__device__ __forceinline__ void block_reduce_minmax(float &lo, float &hi, float *red) {
  lo = wave_min(lo);
  hi = wave_max(hi);
  const int nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6] = lo; red[nw + (threadIdx.x >> 6)] = hi; }
  __syncthreads();
  lo = red[0];
  hi = red[nw];
  for (int i = 1; i < nw; ++i) { lo = fminf(lo, red[i]); hi = fmaxf(hi, red[nw + i]); }
}

// A threshold tau <= the k-th largest of n (> k) non-negative values given by
// get(i): values are binned linearly between their min and max, the highest
// bins holding at least k values are kept, and tau is the smallest value in
// them (an actual element, so at least k elements are >= tau). Any tau below
// the k-th largest keeps the filter exact; binning only decides how tight it is.
__device__ __forceinline__ float f4_elem(const float4 &f, int i) {
  return i == 0 ? f.x : (i == 1 ? f.y : (i == 2 ? f.z : f.w));
}

// The bin holding the k-th largest of the values counted in hist (bins in
// ascending value order): suffix counts from the top bin down, thread t owning
// bins [kTauBins-1-4t-3, kTauBins-1-4t].
__device__ int kth_bin_from_top(const int *hist, int k, int *sh) {
  const int t = threadIdx.x;
  if (t == 0) sh[0] = 0;
  __syncthreads();
  int c4[4], tot = 0;
  const bool owner = t < kTauBins / 4;
  if (owner) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { c4[j] = hist[kTauBins - 1 - 4 * t - j]; tot += c4[j]; }
  }
  // block-wide inclusive scan of tot in thread order
  int incl = owner ? tot : 0;
  const int lane = t & 63, w = t >> 6;
  incl = wave_incl_sum(incl);
  __shared__ int wsum[16];
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  incl += base;
  const int excl = incl - (owner ? tot : 0);
  if (owner && excl < k && incl >= k) {
    int cum = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cum += c4[j];
      if (cum >= k) { sh[0] = kTauBins - 1 - 4 * t - j; break; }
    }
  }
  __syncthreads();
  return sh[0];
}

// A threshold tau <= the k-th largest of n (> k) non-negative values given by
// get(i): values are binned linearly between their min and max, the highest
// bins holding at least k values are kept, and tau is the smallest value in
// them (an actual element, so at least k elements are >= tau). Any tau below
// the k-th largest keeps the filter exact; binning only decides how tight it is.
template <typename Get>
__device__ float tau_lower_bound(Get get, int n, int k, int *hist, float *red, int *sh) {
  const int t = threadIdx.x, bd = blockDim.x;
  float lo = INFINITY, hi = -INFINITY;
  for (int i = t; i < n; i += bd) {
    const float v = get(i);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  block_reduce_minmax(lo, hi, red);
  if (!(hi > lo)) return lo;
  const float sc = static_cast<float>(kTauBins - 1) / (hi - lo);
  for (int i = t; i < kTauBins; i += bd) hist[i] = 0;
  __syncthreads();
  for (int i = t; i < n; i += bd) {
    const int b = min(kTauBins - 1, static_cast<int>((get(i) - lo) * sc));
    atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  const int bstar = kth_bin_from_top(hist, k, sh);
  float m = INFINITY;
  for (int i = t; i < n; i += bd) {
    const float v = get(i);
    if (min(kTauBins - 1, static_cast<int>((v - lo) * sc)) >= bstar) m = fminf(m, v);
  }
  return block_reduce_min(m, red);
}

// The same threshold over values held in registers by a 256-thread block:
// thread t holds values 4 (256 u + t) + q (q < 4) in v[u], those below n valid.
template <int U>
__device__ float tau_lower_bound_regs(const float4 (&v)[U], int n, int k, int *hist, float *red, int *sh) {
  const int t = threadIdx.x;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * (256 * u + t) + q < n) {
        lo = fminf(lo, f4_elem(v[u], q));
        hi = fmaxf(hi, f4_elem(v[u], q));
      }
  block_reduce_minmax(lo, hi, red);
  if (!(hi > lo)) return lo;
  const float sc = static_cast<float>(kTauBins - 1) / (hi - lo);
  for (int i = t; i < kTauBins; i += 256) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * (256 * u + t) + q < n) atomicAdd(&hist[min(kTauBins - 1, static_cast<int>((f4_elem(v[u], q) - lo) * sc))], 1);
  __syncthreads();
  const int bstar = kth_bin_from_top(hist, k, sh);
  float m = INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x = f4_elem(v[u], q);
      if (4 * (256 * u + t) + q < n && min(kTauBins - 1, static_cast<int>((x - lo) * sc)) >= bstar) m = fminf(m, x);
    }
  return block_reduce_min(m, red);
}

// Ascending bitonic sort of n (power of two) 64-bit keys in LDS.
__device__ void bitonic_sort_u64(uint64_t *arr, int n) {
  const int t = threadIdx.x, bd = blockDim.x;
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < (n >> 1); i += bd) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const uint64_t x = arr[lo], y = arr[hi];
        if ((x > y) == asc) { arr[lo] = y; arr[hi] = x; }
      }
      __syncthreads();
    }
  }
}

// Output maps of the selects: the selected index itself, or (Reindex) the
// entry that a pool position stands for.
struct IdMap {
  __device__ int32_t operator()(int i) const { return i; }
};
struct PoolMap {
  const int32_t *row;   // the query's pool row (ascending block ids)
  int n_ent;            // visible entries
  __device__ int32_t operator()(int p) const {
    const int b = row[p >> 3];
    const int e = b * 8 + (p & 7);
    return (b >= 0 && e < n_ent) ? e : -1;
  }
};

// Exact Top-K from c candidate keys already in LDS (k <= c <= kSelCap): sort
// the keys, keep the k largest (keys are unique: score bits, then ~index, so
// ties go to the lower index), sort their indices ascending, write out[0..k).
__device__ void select_sorted_and_write(uint64_t *keys, int c, int k, int *sel, int32_t *out) {
  int np = 1;
  while (np < c) np <<= 1;
  for (int i = c + threadIdx.x; i < np; i += blockDim.x) keys[i] = 0ull;
  __syncthreads();
  bitonic_sort_u64(keys, np);
  int np2 = 1;
  while (np2 < k) np2 <<= 1;
  for (int i = threadIdx.x; i < np2; i += blockDim.x) sel[i] = i < k ? key_index(keys[np - 1 - i]) : 0x7fffffff;
  __syncthreads();
  bitonic_sort(sel, np2);
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = sel[i];
}

// Exact Top-K of one query from `n` candidates given by a getter (any n >= k;
// slow multi-pass radix path, used only when candidates overflow LDS),
// written ascending into out[0..k). sel is LDS of >= next_pow2(k) ints.
template <typename GetKey, typename Map = IdMap>
__device__ void select_and_write(GetKey key_of, int n, int k, int *sel, int *hist, int *sh, int32_t *out,
                                 Map map = Map()) {
  const uint64_t kth = kth_largest_u64(key_of, n, k, hist, sh);
  if (threadIdx.x == 0) sh[2] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t key = key_of(i);
    if (key >= kth) {
      const int p = atomicAdd(&sh[2], 1);
      sel[p] = key_index(key);
    }
  }
  __syncthreads();
  int np2 = 1;
  while (np2 < k) np2 <<= 1;
  for (int i = k + threadIdx.x; i < np2; i += blockDim.x) sel[i] = 0x7fffffff;
  __syncthreads();
  bitonic_sort(sel, np2);
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = map(sel[i]);
}


// Exact Top-K of c candidates held in LDS in ascending index order (keys
// cand_key[i] = score_key(score, index)), written ascending
// into out[0..k), c >= k. The k-th largest key is found without sorting:
// a linear histogram of the scores locates the bin b* holding it; every
// candidate in a higher bin is selected; inside b* the (k - above) largest
// keys are found by exact ranking. The selected candidates are then compacted
// in their (index) order. Returns false (and writes nothing) when bin b*
// holds more than kRankCap candidates; the caller then takes a slower path.
constexpr int kRankCap = 1024;
constexpr int kSelBins = 2048;

// The bin b* of hist (kSelBins counts, bins ascending in value) that holds the
// k-th largest counted value, and how many values lie in higher bins:
// sh[0] = b*, sh[1] = that count. Suffix counts, kSelBins / blockDim bins per
// thread from the top; ends with a barrier.
__device__ void boundary_bin(const int *hist, int k, int *sh) {
  const int t = threadIdx.x, bd = blockDim.x, lane = t & 63, w = t >> 6;
  constexpr int kMaxPer = kSelBins / 256;
  const int per = kSelBins / bd;
  int cnt[kMaxPer], tot = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    cnt[j] = j < per ? hist[kSelBins - 1 - per * t - j] : 0;
    tot += cnt[j];
  }
  int incl = tot;
  incl = wave_incl_sum(incl);
  __shared__ int wsum_b[16];
  if (lane == 63) wsum_b[w] = incl;
  __syncthreads();
  for (int i = 0; i < w; ++i) incl += wsum_b[i];
  const int excl = incl - tot;
  if (excl < k && incl >= k) {
    int cum = excl;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      if (j < per && cum + cnt[j] >= k) { sh[0] = kSelBins - 1 - per * t - j; sh[1] = cum; break; }
      cum += cnt[j];
    }
  }
  __syncthreads();
}

template <typename Map = IdMap>
__device__ bool select_ordered(const uint64_t *cand_key, int c, int k, int *hist, float *red, int *sh,
                               uint64_t *bin_keys, int32_t *out, Map map = Map()) {
  const int t = threadIdx.x, bd = blockDim.x, lane = t & 63, w = t >> 6, nw = bd >> 6;
  float lo = INFINITY, hi = -INFINITY;
  for (int i = t; i < c; i += bd) {
    const float v = bits_score(static_cast<uint32_t>(cand_key[i] >> 32));
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  block_reduce_minmax(lo, hi, red);
  const float sc = hi > lo ? static_cast<float>(kSelBins - 1) / (hi - lo) : 0.f;
  auto bin_of = [&](uint64_t key) {
    return min(kSelBins - 1, static_cast<int>((bits_score(static_cast<uint32_t>(key >> 32)) - lo) * sc));
  };
  for (int i = t; i < kSelBins; i += bd) hist[i] = 0;
  __syncthreads();
  for (int i = t; i < c; i += bd) atomicAdd(&hist[bin_of(cand_key[i])], 1);
  __syncthreads();
  boundary_bin(hist, k, sh);
  const int bstar = sh[0], above = sh[1];
  const int need = k - above;            // keys to take from bin b*
  const int m = hist[bstar];
  if (m > kRankCap) return false;
  if (t == 0) sh[2] = 0;
  __syncthreads();
  for (int i = t; i < c; i += bd)
    if (bin_of(cand_key[i]) == bstar) bin_keys[atomicAdd(&sh[2], 1)] = cand_key[i];
  __syncthreads();
  // threshold key: the need-th largest key of the bin, by exact rank
  for (int i = t; i < m; i += bd) {
    const uint64_t x = bin_keys[i];
    int r = 0;
    for (int j = 0; j < m; ++j) r += bin_keys[j] > x;
    if (r == need - 1) sh[3] = static_cast<int>(i);
  }
  __syncthreads();
  const uint64_t kth = bin_keys[sh[3]];
  // ordered compaction of the selected candidates (keys >= kth): thread-contiguous ranges
  const int span = (c + bd - 1) / bd;
  const int i0 = min(c, t * span), i1 = min(c, i0 + span);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += cand_key[i] >= kth;
  int inc2 = mine;
  inc2 = wave_incl_sum(inc2);
  __shared__ int wsum2[16];
  if (lane == 63) wsum2[w] = inc2;
  __syncthreads();
  for (int i = 0; i < w; ++i) inc2 += wsum2[i];
  int pos = inc2 - mine;
  for (int i = i0; i < i1; ++i)
    if (cand_key[i] >= kth) out[pos++] = map(key_index(cand_key[i]));
  (void)nw;
  return true;
}

// The same selection over candidates held in registers by the block: thread t
// holds candidates [t s, t s + s) (s = ceil(c / blockDim) <= P) in kr[0..s),
// so every thread's candidates are consecutive and the compaction keeps their
// order. No pass re-reads the candidates from LDS; each key's bin is computed
// once.
// ok[u] marks the slots that hold a candidate: the candidates of all threads,
// taken in thread order and then slot order, are in ascending index order.
template <int P, typename Map = IdMap>
__device__ __forceinline__ bool select_ordered_regs_ok(const uint64_t (&kr)[P], const bool (&ok)[P], int k, int *hist, float *red,
                                       int *sh, uint64_t *bin_keys, int32_t *out, Map map = Map()) {
  const int t = threadIdx.x, bd = blockDim.x, lane = t & 63, w = t >> 6;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int u = 0; u < P; ++u) {
    if (ok[u]) {
      const float v = bits_score(static_cast<uint32_t>(kr[u] >> 32));
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
  }
  for (int i = t; i < kSelBins; i += bd) hist[i] = 0;
  block_reduce_minmax(lo, hi, red);   // its barriers also order the clear before the counts
  const float sc = hi > lo ? static_cast<float>(kSelBins - 1) / (hi - lo) : 0.f;
  int bn[P];
#pragma unroll
  for (int u = 0; u < P; ++u) {
    bn[u] = -1;
    if (ok[u]) {
      bn[u] = min(kSelBins - 1, static_cast<int>((bits_score(static_cast<uint32_t>(kr[u] >> 32)) - lo) * sc));
      atomicAdd(&hist[bn[u]], 1);
    }
  }
  __syncthreads();
  boundary_bin(hist, k, sh);
  const int bstar = sh[0], above = sh[1];
  const int need = k - above;            // keys to take from bin b*
  const int m = hist[bstar];
  if (m > kRankCap) return false;
  if (t == 0) sh[2] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (bn[u] == bstar) bin_keys[atomicAdd(&sh[2], 1)] = kr[u];
  __syncthreads();
  // threshold key: the need-th largest key of the bin, by exact rank
  for (int i = t; i < m; i += bd) {
    const uint64_t x = bin_keys[i];
    int r = 0;
    for (int j = 0; j < m; ++j) r += bin_keys[j] > x;
    if (r == need - 1) sh[3] = static_cast<int>(i);
  }
  __syncthreads();
  const uint64_t kth = bin_keys[sh[3]];
  int mine = 0;
#pragma unroll
  for (int u = 0; u < P; ++u) mine += (ok[u] && kr[u] >= kth) ? 1 : 0;
  int inc = wave_incl_sum(mine);
  __shared__ int wsum_r[16];
  if (lane == 63) wsum_r[w] = inc;
  __syncthreads();
  for (int i = 0; i < w; ++i) inc += wsum_r[i];
  int pos = inc - mine;
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (ok[u] && kr[u] >= kth) out[pos++] = map(key_index(kr[u]));
  return true;
}

// Thread t holds candidates [t s, t s + s) of c (s = ceil(c / blockDim) <= P).
template <int P, typename Map = IdMap>
__device__ __forceinline__ bool select_ordered_regs(const uint64_t (&kr)[P], int c, int k, int *hist, float *red, int *sh,
                                    uint64_t *bin_keys, int32_t *out, Map map = Map()) {
  const int span = (c + blockDim.x - 1) / blockDim.x, i0 = threadIdx.x * span;
  bool ok[P];
#pragma unroll
  for (int u = 0; u < P; ++u) ok[u] = u < span && i0 + u < c;
  return select_ordered_regs_ok(kr, ok, k, hist, red, sh, bin_keys, out, map);
}


// In-place inclusive prefix sum of arr[1..n] in LDS (arr[0] = 0 is left as is):
// thread-contiguous chunks, wave scan of chunk totals, block combine.
__device__ void block_prefix_sum(int *arr, int n, int *wsum) {
  const int t = threadIdx.x, bd = blockDim.x, lane = t & 63, w = t >> 6;
  const int span = (n + bd - 1) / bd;
  const int i0 = 1 + min(n, t * span), i1 = 1 + min(n, t * span + span);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += arr[i];
  int incl = mine;
  incl = wave_incl_sum(incl);
  __syncthreads();
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  for (int i = 0; i < w; ++i) incl += wsum[i];
  int run = incl - mine;
  for (int i = i0; i < i1; ++i) {
    run += arr[i];
    arr[i] = run;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ decode scan

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

// A wave-uniform load of data no kernel of this launch writes, through the
// scalar cache into a scalar register (no vector register, and its wait is
// separate from the vector loads' counter).
template <typename T>
__device__ __forceinline__ T scalar_load(const T *p) {
  return *(const __attribute__((address_space(4))) T *)(p);
}

// One workgroup = kScanWaves waves, each owning kScanPagesPerWave consecutive pages of
// one query's visible entries. A wave reads its page ids, issues every key
// load of its pages at once, and scores 16 entries per MFMA (indexer heads as
// rows, entries as columns). Small workgroups keep many of them resident per
// CU, so one workgroup's block-table round trip overlaps others' key streams.
template <int ACT, int KV>
__global__ __launch_bounds__(kScanWaves * 64) void idx_scan_kernel(const IdxScanArgs a) {
  using CT = typename ComputeT<KV>::type;
  constexpr int PPW = kScanPagesPerWave;
  const int wg = blockIdx.x;
  // owning query: the last one whose first workgroup is <= wg
  int qlo = 0, qhi = a.n_q;
  while (qhi - qlo > 1) {
    const int mid = (qlo + qhi) >> 1;
    if (a.q[mid].chunk0 <= wg) qlo = mid; else qhi = mid;
  }
  const int qi = qlo;
  const IdxQuery Q = a.q[qi];
  const int chunk = wg - Q.chunk0;
  const int N = Q.n_vis;

  const int lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int AE = elem_bytes<ACT>(), KE = elem_bytes<KV>();

  const int glog2 = Q.glog2, G = 1 << glog2;
  // a group of more than one page: its maximum is gathered across the wave's
  // pages (run) and, when it spans several waves, through LDS
  static_assert(kScanPagesPerWave <= 2, "a group of G > 64 entries is whole waves");
  const bool cross = G > kPage;
  float *Srow = a.S + static_cast<int64_t>(qi) * a.s_stride;
  float *Mrow = a.M + static_cast<int64_t>(qi) * a.s_stride;
  const int wave_e0 = chunk * kIdxChunk + w * (PPW * kPage);
  float run = -INFINITY;

  if (wave_e0 < N) {
    // this lane's head row (placed in the tile col / 4 whose rows it
    // supplies), issued first: in flight during the block-table round trip
    // instead of behind the key stream
    Frag<CT> qv[2];
    qv[0] = qv[1] = zero_frag<CT>();
    if ((col & 3) < a.h_i) {
      const char *qrow = reinterpret_cast<const char *>(a.q_idx) + (static_cast<int64_t>(qi) * a.h_i + (col & 3)) * kDI * AE;
#pragma unroll
      for (int c = 0; c < 2; ++c) qv[c] = LoadFrag<ACT, CT>::load(qrow + (16 * g + 8 * c) * AE);
    }
    const int32_t *bt = a.block_table + static_cast<int64_t>(Q.seq) * a.bt_stride;
    const char *kbase = reinterpret_cast<const char *>(a.kidx);
    int pps[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) pps[p] = wave_e0 + p * kPage < N ? bt[(wave_e0 >> 6) + p] : -1;

    // A operands, one per 16-entry tile of a page: the indexer heads in rows
    // [4 tl, 4 tl + 4), zero elsewhere. The page's four tiles accumulate into
    // one MFMA result whose lane (g, col) holds the heads' dot products for
    // entry 16 g + col of the page, so the epilogue runs once per page with
    // every lane scoring one entry (rows >= H_I of a tile are zero).
    // every key load of the wave in flight together: lane (g, col) reads dims
    // [16g, 16g + 16) of entry col of each 16-entry tile; the key stream is
    // read once, so the loads are non-temporal
    constexpr int RW = KE;   // uint4 per lane per tile
    uint4 raw[PPW][4][RW];
    bool okp[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int pp = pps[p];
      okp[p] = pp >= 0 && pp < a.pool_pages;
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        const int e = wave_e0 + p * kPage + tl * 16 + col;
        if (okp[p] && e < N) {
          const uint4 *src = reinterpret_cast<const uint4 *>(kbase + ((static_cast<int64_t>(pp) * kPage + (e & 63)) * kDI + 16 * g) * KE);
#pragma unroll
          for (int u = 0; u < RW; ++u) {
            const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(src + u));
            raw[p][tl][u] = make_uint4(t.x, t.y, t.z, t.w);
          }
        } else {
#pragma unroll
          for (int u = 0; u < RW; ++u) raw[p][tl][u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    float scs[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      if (!okp[p] && lane == 0 && wave_e0 + p * kPage < N) flag_error(a.err, ERR_PAGE);
      scs[p] = (KV == DT_FP8 && okp[p]) ? scalar_load(a.kidx_scale + pps[p]) : 1.f;
    }
    // head weights and page scales are scalar loads issued after the keys:
    // scalar loads complete out of order, so any earlier one would hold the
    // block-table wait
    float wv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) wv[v] = v < a.h_i ? scalar_load(a.w_idx + qi * a.h_i + v) : 0.f;
    // tiles outer, pages inner: only one tile's A operands are live at a time
    f32x4_t accp[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) accp[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) {
      const Frag<CT> qa0 = (col >> 2) == tl ? qv[0] : zero_frag<CT>();
      const Frag<CT> qa1 = (col >> 2) == tl ? qv[1] : zero_frag<CT>();
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        if (wave_e0 + p * kPage + tl * 16 >= N) continue;
        Frag<CT> kb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char *rp = reinterpret_cast<const char *>(&raw[p][tl][0]) + 8 * c * KE;
          if constexpr (KV == DT_FP8) kb[c] = LoadFrag<DT_FP8, __bf16>::load(rp);
          else if constexpr (KV == DT_BF16) kb[c] = LoadFrag<DT_BF16, __bf16>::load(rp);
          else kb[c] = LoadFrag<DT_F32, float>::load(rp);
        }
        accp[p] = mma(qa0, kb[0], accp[p]);
        accp[p] = mma(qa1, kb[1], accp[p]);
      }
    }

#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int e_page = wave_e0 + p * kPage;
      if (e_page >= N) break;
      const f32x4_t acc = accp[p];
      const int e = e_page + lane;   // lane = 16 g + col
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) s += wv[v] * fmaxf(acc[v], 0.f);
      s = okp[p] ? s * scs[p] : -1.f;   // a missing page scores -1 (and is flagged)
      if (e < N) Srow[e] = s;
      if (a.B) {   // maxima of aligned 8-entry blocks (candidate pool)
        float m8 = e < N ? s : -INFINITY;
        m8 = group_max(m8, kPoolBlock);
        if ((col & (kPoolBlock - 1)) == 0 && e < N) a.B[static_cast<int64_t>(qi) * a.s_stride + (e >> 3)] = m8;
      }
      // group maxima: entries past N do not take part; a group of G <= 64
      // entries is G consecutive lanes
      float m = e < N ? s : -INFINITY;
      m = group_max(m, G < 16 ? G : 16);
      if (G >= 32) m = max_xor16(m);
      if (G >= 64) m = max_xor32(m);
      if (!cross) {
        if ((lane & (G - 1)) == 0 && e < N) Mrow[e >> glog2] = m;
      } else {
        run = fmaxf(run, m);
      }
    }
  }
  if (cross) {
    // groups of G entries = G / (PPW * 64) consecutive waves (at least one), all inside this workgroup
    __shared__ float wmax[kScanWaves];
    if (lane == 0) wmax[w] = run;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int wpg = G / (PPW * kPage);
      for (int w0 = 0; w0 < kScanWaves; w0 += wpg) {
        const int e0 = chunk * kIdxChunk + w0 * (PPW * kPage);
        if (e0 >= N) break;
        float m = -INFINITY;
        for (int u = 0; u < wpg; ++u) m = fmaxf(m, wmax[w0 + u]);
        Mrow[e0 >> glog2] = m;
      }
    }
  }
}

// ------------------------------------------------------------------ short rows
//
// A query whose visible indexer keys are few (at most kSmallEntries, and at
// most kSmallBytes of keys) is scored and selected by one workgroup: its 16
// waves score pages w, w + 16, ... with the scan's MFMA tile (small_batch
// pages' loads in flight at once), the keys go to LDS, and the same exact
// select as the final kernel writes the ascending row. One launch instead of
// scan, filter and final.
constexpr int kSmallWaves = 16;
template <int KV> constexpr int small_batch() { return 4 / elem_bytes<KV>(); }

template <int ACT, int KV>
__global__ __launch_bounds__(kSmallWaves * 64) void idx_small_kernel(const IdxScanArgs a, int32_t *topk, int k) {
  using CT = typename ComputeT<KV>::type;
  constexpr int AE = elem_bytes<ACT>(), KE = elem_bytes<KV>();
  constexpr int RW = KE;                 // uint4 per lane per 16-entry tile
  constexpr int PB = small_batch<KV>();  // pages per wave in flight
  __shared__ uint64_t keys[kSmallEntries];
  __shared__ uint64_t bin_keys[kRankCap];
  __shared__ int hist[kSelBins];
  __shared__ float red[32];
  __shared__ int sh[4];
  const int qi = blockIdx.x, tid = threadIdx.x;
  const IdxQuery Q = a.q[qi];
  const int N = Q.n_vis;
  int32_t *out = topk + static_cast<int64_t>(qi) * k;
  if (N <= k) {
    for (int i = tid; i < k; i += kSmallWaves * 64) out[i] = i < N ? i : -1;
    return;
  }
  const int lane = tid & 63, g = lane >> 4, col = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_pages = (N + kPage - 1) / kPage;   // <= 64: 4 per wave
  const int32_t *bt = a.block_table + static_cast<int64_t>(Q.seq) * a.bt_stride;
  // lane j holds the physical id of this wave's j-th page (page w + 16 j)
  const int my_pp = (lane < 4 && w + kSmallWaves * lane < n_pages) ? bt[w + kSmallWaves * lane] : -1;
  Frag<CT> qv[2];
  qv[0] = qv[1] = zero_frag<CT>();
  if ((col & 3) < a.h_i) {
    const char *qrow = reinterpret_cast<const char *>(a.q_idx) + (static_cast<int64_t>(qi) * a.h_i + (col & 3)) * kDI * AE;
#pragma unroll
    for (int c = 0; c < 2; ++c) qv[c] = LoadFrag<ACT, CT>::load(qrow + (16 * g + 8 * c) * AE);
  }
  float wv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) wv[v] = v < a.h_i ? a.w_idx[qi * a.h_i + v] : 0.f;
  const char *kbase = reinterpret_cast<const char *>(a.kidx);

  for (int j0 = 0; w + kSmallWaves * j0 < n_pages; j0 += PB) {
    uint4 raw[PB][4][RW];
    bool okp[PB];
    int pps[PB];
#pragma unroll
    for (int jj = 0; jj < PB; ++jj) {
      const int page = w + kSmallWaves * (j0 + jj);
      pps[jj] = __builtin_amdgcn_readlane(my_pp, (j0 + jj) & 63);
      okp[jj] = page < n_pages && pps[jj] >= 0 && pps[jj] < a.pool_pages;
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        const int e = page * kPage + tl * 16 + col;
        if (okp[jj] && e < N) {
          const uint4 *src = reinterpret_cast<const uint4 *>(kbase + ((static_cast<int64_t>(pps[jj]) * kPage + (e & 63)) * kDI + 16 * g) * KE);
#pragma unroll
          for (int u = 0; u < RW; ++u) raw[jj][tl][u] = src[u];
        } else {
#pragma unroll
          for (int u = 0; u < RW; ++u) raw[jj][tl][u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    float scs[PB];
#pragma unroll
    for (int jj = 0; jj < PB; ++jj) {
      const int page = w + kSmallWaves * (j0 + jj);
      if (page < n_pages && !okp[jj] && lane == 0) flag_error(a.err, ERR_PAGE);
      scs[jj] = (KV == DT_FP8 && okp[jj]) ? a.kidx_scale[pps[jj]] : 1.f;
    }
#pragma unroll
    for (int jj = 0; jj < PB; ++jj) {
      const int page = w + kSmallWaves * (j0 + jj);
      if (page >= n_pages) break;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        Frag<CT> kb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char *rp = reinterpret_cast<const char *>(&raw[jj][tl][0]) + 8 * c * KE;
          if constexpr (KV == DT_FP8) kb[c] = LoadFrag<DT_FP8, __bf16>::load(rp);
          else if constexpr (KV == DT_BF16) kb[c] = LoadFrag<DT_BF16, __bf16>::load(rp);
          else kb[c] = LoadFrag<DT_F32, float>::load(rp);
        }
        // this lane's head row only in the tile whose rows it supplies
        const bool mine = (col >> 2) == tl;
        acc = mma(mine ? qv[0] : zero_frag<CT>(), kb[0], acc);
        acc = mma(mine ? qv[1] : zero_frag<CT>(), kb[1], acc);
      }
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) s += wv[v] * fmaxf(acc[v], 0.f);
      s = okp[jj] ? s * scs[jj] : -1.f;   // a missing page scores -1 (and is flagged)
      const int e = page * kPage + lane;
      if (e < N) keys[e] = score_key(s, e);
    }
  }
  __syncthreads();
  if (!select_ordered(keys, N, k, hist, red, sh, bin_keys, out)) {
    // heavy ties: the exact radix select over the same keys
    if (tid == 0) flag_error(a.err, ERR_FALLBACK);
    __syncthreads();
    select_and_write([&](int i) { return keys[i]; }, N, k, reinterpret_cast<int *>(bin_keys), hist, sh, out);
  }
}

// ------------------------------------------------------------------ decode filter

__global__ __launch_bounds__(256) void idx_filter_kernel(const IdxFilterArgs a) {
  __shared__ int hist[kTauBins];
  __shared__ float red[32];
  __shared__ int sh[4];
  __shared__ int wcnt[4];
  const int wg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int qi = 0;   // owning query: the last one whose first workgroup is <= wg
  if (a.uniform > 0) {
    qi = __builtin_amdgcn_readfirstlane(wg / a.uniform);
  } else {
    int hi = a.n_q;
    while (hi - qi > 1) {
      const int mid = (qi + hi) >> 1;
      if (a.slice0[mid] <= wg) qi = mid; else hi = mid;
    }
  }
  const int slice = wg - a.slice0[qi];
  const int N = a.n_vis[qi];
  const int glog2 = a.glog2[qi];
  const int nG = (N + (1 << glog2) - 1) >> glog2;
  const float *Srow = a.S + static_cast<int64_t>(qi) * a.s_stride;
  const float *Mrow = a.M + static_cast<int64_t>(qi) * a.s_stride;
  const int e_begin = slice * kFilterSlice, e_end = min(N, e_begin + kFilterSlice);

  // this slice's scores, 16 consecutive per thread (so a thread-order prefix
  // keeps ascending index order), and the query's group maxima in registers:
  // U float4 per thread, the smallest of 2, 4, 8 that holds its nG maxima (M
  // rows are padded to 256 floats). Both sets of loads sit in one branch-free
  // stretch per U, maxima first, so they share one round trip.
  constexpr int kPer = kFilterSlice / 256;
  const int t0 = e_begin + tid * kPer;
  float sv[kPer];
  static_assert(kMaxGroups == 8 * 1024, "at most 8 float4 of group maxima per thread");
  auto load_threshold = [&](auto u_tag) {
    constexpr int U = decltype(u_tag)::value;
    // addresses are clamped into the row instead of guarded, so no load waits
    // on a branch; values past nG (maxima) or e_end (scores) are never used
    float4 mv[U];
    const int last4 = max(0, (nG - 1) >> 2);
#pragma unroll
    for (int u = 0; u < U; ++u) mv[u] = *reinterpret_cast<const float4 *>(Mrow + 4 * min(256 * u + tid, last4));
    const int smax = a.s_stride - 4;
#pragma unroll
    for (int u = 0; u < kPer; u += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(Srow + min(t0 + u, smax));
      sv[u] = v.x; sv[u + 1] = v.y; sv[u + 2] = v.z; sv[u + 3] = v.w;
    }
    return nG > a.k ? tau_lower_bound_regs(mv, nG, a.k, hist, red, sh) : 0.f;
  };
  const float tau = nG <= 2048 ? load_threshold(std::integral_constant<int, 2>{})
                  : nG <= 4096 ? load_threshold(std::integral_constant<int, 4>{})
                               : load_threshold(std::integral_constant<int, 8>{});

  // ordered compaction into this slice's own region
  int mine = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) mine += (t0 + u < e_end && sv[u] >= tau) ? 1 : 0;
  int incl = mine;
  incl = wave_incl_sum(incl);
  if (lane == 63) wcnt[w] = incl;
  __syncthreads();
  int pos = incl - mine;
  for (int i = 0; i < w; ++i) pos += wcnt[i];
  const int64_t region = static_cast<int64_t>(qi) * a.s_stride + static_cast<int64_t>(slice) * kFilterSlice;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (t0 + u < e_end && sv[u] >= tau) {
      a.cand_s[region + pos] = sv[u];
      a.cand_j[region + pos] = t0 + u;
      ++pos;
    }
  }
  if (tid == 0) a.cnt[static_cast<int64_t>(qi) * a.max_slices + slice] = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
}

// ------------------------------------------------------------------ decode final

// Speculative candidate load of the final select: queries with at most
// kFinalSpecSlices filter slices read every slice's first 512 / ns2 * 8 slots
// together with the counts (8 per thread of 512).
constexpr int kFinalSpecSlices = 64;
constexpr int kFinalSpecPer = 8;

struct FinalLds {
  uint64_t bin_keys[kRankCap];
  int sel[CSA_MAX_TOPK];
  int hist[kSelBins];
  int soff[kMaxSlices + 1];
  float red[32];
  int sh[4];
  int wsum_f[16];
};

template <typename Map>
__device__ __forceinline__ void final_select(const IdxFinalArgs &a, FinalLds &L, int qi, int N, int k, int32_t *out, Map map) {
  uint64_t *bin_keys = L.bin_keys;
  int *sel = L.sel, *hist = L.hist, *soff = L.soff, *sh = L.sh, *wsum_f = L.wsum_f;
  float *red = L.red;
  const int tid = threadIdx.x;
  if (N <= k) {
    for (int i = tid; i < k; i += blockDim.x) out[i] = i < N ? map(i) : -1;
    return;
  }
  const int ns = (N + kFilterSlice - 1) / kFilterSlice;
  const int32_t *cnts = a.cnt + static_cast<int64_t>(qi) * a.max_slices;
  if (ns <= kFinalSpecSlices) {
    // the slice counts and the first slots of every slice in one round trip:
    // 512 / ns2 threads per slice (ns2 = ns rounded up to a power of two),
    // 8 consecutive slots each, so thread order then slot order is index order
    int ns2 = 1;
    while (ns2 < ns) ns2 <<= 1;
    const int tps = 512 / ns2, sl = tid / tps, j0 = (tid % tps) * kFinalSpecPer;
    const int e0 = sl * kFilterSlice;
    const int n_sl = sl < ns ? min(kFilterSlice, N - e0) : 0;   // entries (and slots) of the slice
    const int64_t o0 = static_cast<int64_t>(qi) * a.s_stride + e0 + j0;
    const int cs = sl < ns ? cnts[sl] : 0;
    float ts[kFinalSpecPer];
    int tj[kFinalSpecPer];
    if (j0 + kFinalSpecPer <= n_sl) {
#pragma unroll
      for (int u = 0; u < kFinalSpecPer; u += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(a.cand_s + o0 + u);
        const int4 j = *reinterpret_cast<const int4 *>(a.cand_j + o0 + u);
        ts[u] = v.x; ts[u + 1] = v.y; ts[u + 2] = v.z; ts[u + 3] = v.w;
        tj[u] = j.x; tj[u + 1] = j.y; tj[u + 2] = j.z; tj[u + 3] = j.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kFinalSpecPer; ++u) {
        ts[u] = j0 + u < n_sl ? a.cand_s[o0 + u] : 0.f;
        tj[u] = j0 + u < n_sl ? a.cand_j[o0 + u] : 0;
      }
    }
    bool ok[kFinalSpecPer];
    uint64_t tk[kFinalSpecPer];
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kFinalSpecPer; ++u) {
      ok[u] = j0 + u < cs;
      tk[u] = score_key(ts[u], tj[u]);
      mine += ok[u] ? 1 : 0;
    }
    // every slice's candidates inside its slots, and at least k of them
    const bool over = (tid % tps) == tps - 1 && cs > j0 + kFinalSpecPer;
    int incl = wave_incl_sum(mine);
    if ((tid & 63) == 63) wsum_f[tid >> 6] = incl;
    const bool any_over = __syncthreads_or(over);
    int c = 0;
    for (int i = 0; i < 8; ++i) c += wsum_f[i];
    if (!any_over && c >= k && select_ordered_regs_ok(tk, ok, k, hist, red, sh, bin_keys, out, map)) return;
    __syncthreads();   // the general path below reuses the same LDS
  }
  // slice counts -> offsets (slices in index order, each region already ordered)
  for (int i = tid; i < ns; i += blockDim.x) soff[i + 1] = cnts[i];
  if (tid == 0) soff[0] = 0;
  __syncthreads();
  block_prefix_sum(soff, ns, wsum_f);
  const int c = soff[ns];
  bool done = false;
  if (c >= k && c <= kSelCap) {
    const int64_t qbase = static_cast<int64_t>(qi) * a.s_stride;
    // the slice of every candidate position, written slice by slice into
    // bin_keys (free until the select) when the candidates fit it
    constexpr int kMapCap = kRankCap * 4;   // 16-bit entries in bin_keys
    static_assert(kMaxSlices <= 65536, "slice ids fit 16 bits");
    uint16_t *slice_of = reinterpret_cast<uint16_t *>(bin_keys);
    const bool mapped = c <= kMapCap;
    if (mapped) {
      for (int t = tid; t < ns; t += blockDim.x)
        for (int i = soff[t]; i < soff[t + 1]; ++i) slice_of[i] = static_cast<uint16_t>(t);
      __syncthreads();
    }
    // thread tid holds candidates [tid s, tid s + s), s = ceil(c / 512), in
    // registers; the code is unrolled for the smallest P >= s of 4, 8, 12
    static_assert((kSelCap + 511) / 512 <= 12, "at most 12 candidates per thread");
    const int span = (c + 511) / 512, i0 = tid * span;
    auto gather_select = [&](auto per_tag) {
      constexpr int P = decltype(per_tag)::value;
      float ts[P];
      int tj[P];
#pragma unroll
      for (int u = 0; u < P; ++u) {   // every load first, then the keys
        const int i = i0 + u;
        ts[u] = 0.f;
        tj[u] = 0;
        if (u < span && i < c) {
          int lo = 0;                     // slice s with soff[s] <= i < soff[s+1]
          if (mapped) {
            lo = slice_of[i];
          } else {
            int hi = ns;
            while (hi - lo > 1) {
              const int mid = (lo + hi) >> 1;
              if (soff[mid] <= i) lo = mid; else hi = mid;
            }
          }
          const int64_t o = qbase + static_cast<int64_t>(lo) * kFilterSlice + (i - soff[lo]);
          ts[u] = a.cand_s[o];
          tj[u] = a.cand_j[o];
        }
      }
      uint64_t tk[P];
#pragma unroll
      for (int u = 0; u < P; ++u) tk[u] = score_key(ts[u], tj[u]);
      // (the select's first barrier comes after every read of slice_of, which it then reuses)
      return select_ordered_regs(tk, c, k, hist, red, sh, bin_keys, out, map);
    };
    if (span <= 4) done = gather_select(std::integral_constant<int, 4>{});
    else if (span <= 8) done = gather_select(std::integral_constant<int, 8>{});
    else done = gather_select(std::integral_constant<int, 12>{});
  }
  if (!done) {
    // heavy ties or too many candidates: exact select straight from the scores
    if (tid == 0) flag_error(a.err, ERR_FALLBACK);
    const float *Srow = a.S + static_cast<int64_t>(qi) * a.s_stride;
    select_and_write([&](int i) { return score_key(Srow[i], i); }, N, k, sel, hist, sh, out, map);
  }
}

__global__ __launch_bounds__(512) void idx_final_kernel(const IdxFinalArgs a) {
  __shared__ FinalLds lds;
  const int qi = blockIdx.x;
  int32_t *out = a.topk + static_cast<int64_t>(qi) * a.k;
  if (a.pool)
    final_select(a, lds, qi, a.n_vis[qi], a.k, out, PoolMap{a.pool + static_cast<int64_t>(qi) * a.pool_stride, a.n_ent[qi]});
  else
    final_select(a, lds, qi, a.n_vis[qi], a.k, out, IdMap{});
}

// ------------------------------------------------------------------ Reindex scores
//
// The scan's MFMA scoring over pool positions instead of consecutive pages:
// lane (g, col) of tile tl holds position p = wave_p0 + 16 tl + col, entry
// pool[p / 8] * 8 + p % 8, so every lane resolves its own page. Positions whose
// entry is not visible (the tail of the last block) score 0: equal scores go
// to the lower position, so they are only picked when the pool holds fewer
// than k entries, and then map to -1.

template <int ACT, int KV>
__global__ __launch_bounds__(kScanWaves * 64) void idx_rescan_kernel(const IdxRescanArgs a) {
  using CT = typename ComputeT<KV>::type;
  const int wg = blockIdx.x;
  int qlo = 0, qhi = a.n_q;
  while (qhi - qlo > 1) {
    const int mid = (qlo + qhi) >> 1;
    if (a.q[mid].chunk0 <= wg) qlo = mid; else qhi = mid;
  }
  const int qi = qlo;
  const IdxQuery Q = a.q[qi];
  const int V = Q.n_vis, n_ent = a.n_ent[qi];
  const int lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_p0 = (wg - Q.chunk0) * kRescanChunk + w * 64;
  if (wave_p0 >= V) return;   // no barriers below
  constexpr int AE = elem_bytes<ACT>(), KE = elem_bytes<KV>();
  const int32_t *prow = a.pool + static_cast<int64_t>(qi) * a.pool_stride;
  const int32_t *bt = a.block_table + static_cast<int64_t>(Q.seq) * a.bt_stride;
  float *Srow = a.S + static_cast<int64_t>(qi) * a.s_stride;
  float *Mrow = a.M + static_cast<int64_t>(qi) * a.s_stride;
  const int glog2 = Q.glog2, G = 1 << glog2;

  // the four block ids, then the four pages, each set in one round trip:
  // addresses are clamped into the rows instead of guarded, so no load waits
  // behind the error checks (V >= 1 here; the block-table row has >= 1 entry)
  int bid[4], ent[4], pg[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) bid[tl] = prow[min(wave_p0 + tl * 16 + col, V - 1) >> 3];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const int p = wave_p0 + tl * 16 + col;
    const int b = p < V ? bid[tl] : -1;
    const int e = b * 8 + (p & 7);
    ent[tl] = (p < V && b >= 0 && e < n_ent) ? e : -1;
  }
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) pg[tl] = bt[max(ent[tl], 0) >> 6];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const int p = wave_p0 + tl * 16 + col;
    const int b = p < V ? bid[tl] : -1;
    if (p < V && (b < 0 || b * 8 >= n_ent) && g == 0 && (p & 7) == 0) flag_error(a.err, ERR_TOPK);
    if (ent[tl] < 0) pg[tl] = -1;
  }

  constexpr int RW = KE;
  const char *kbase = reinterpret_cast<const char *>(a.kidx);
  uint4 raw[4][RW];
  bool ok[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    ok[tl] = ent[tl] >= 0 && pg[tl] >= 0 && pg[tl] < a.pool_pages;
    if (ent[tl] >= 0 && !ok[tl] && g == 0) flag_error(a.err, ERR_PAGE);
    if (ok[tl]) {
      const uint4 *src = reinterpret_cast<const uint4 *>(
          kbase + ((static_cast<int64_t>(pg[tl]) * kPage + (ent[tl] & 63)) * kDI + 16 * g) * KE);
#pragma unroll
      for (int u = 0; u < RW; ++u) raw[tl][u] = src[u];
    } else {
#pragma unroll
      for (int u = 0; u < RW; ++u) raw[tl][u] = make_uint4(0, 0, 0, 0);
    }
  }
  float sc[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) sc[tl] = (KV == DT_FP8 && ok[tl]) ? a.kidx_scale[pg[tl]] : 1.f;
  // (after the key loads) this lane's head row, in the tile (col / 4) whose
  // rows it supplies: the four tiles accumulate into one MFMA result whose
  // lane (g, col) holds the heads of position 16 g + col, as in the scan
  Frag<CT> qv[2];
  qv[0] = qv[1] = zero_frag<CT>();
  if ((col & 3) < a.h_i) {
    const char *qrow = reinterpret_cast<const char *>(a.q_idx) + (static_cast<int64_t>(qi) * a.h_i + (col & 3)) * kDI * AE;
#pragma unroll
    for (int c = 0; c < 2; ++c) qv[c] = LoadFrag<ACT, CT>::load(qrow + (16 * g + 8 * c) * AE);
  }
  float wv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) wv[v] = v < a.h_i ? a.w_idx[qi * a.h_i + v] : 0.f;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    if (wave_p0 + tl * 16 >= V) break;
    Frag<CT> kb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const char *rp = reinterpret_cast<const char *>(&raw[tl][0]) + 8 * c * KE;
      if constexpr (KV == DT_FP8) kb[c] = LoadFrag<DT_FP8, __bf16>::load(rp);
      else if constexpr (KV == DT_BF16) kb[c] = LoadFrag<DT_BF16, __bf16>::load(rp);
      else kb[c] = LoadFrag<DT_F32, float>::load(rp);
    }
    const Frag<CT> q0 = (col >> 2) == tl ? qv[0] : zero_frag<CT>(), q1 = (col >> 2) == tl ? qv[1] : zero_frag<CT>();
    acc = mma(q0, kb[0], acc);
    acc = mma(q1, kb[1], acc);
  }
  // lane (g, col): position 16 g + col of the wave, its tile g's scale and validity
  const float scl = g == 0 ? sc[0] : (g == 1 ? sc[1] : (g == 2 ? sc[2] : sc[3]));
  const bool okl = g == 0 ? ok[0] : (g == 1 ? ok[1] : (g == 2 ? ok[2] : ok[3]));
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) s += wv[v] * fmaxf(acc[v], 0.f);
  s = okl ? s * scl : 0.f;
  const int p = wave_p0 + lane;
  if (p < V) Srow[p] = s;
  float m = p < V ? s : -INFINITY;
  m = group_max(m, G);
  if ((col & (G - 1)) == 0 && p < V) Mrow[p >> glog2] = m;
}

// ------------------------------------------------------------------ chunk (prefill) index
//
// Queries of one sequence at consecutive positions share the indexer keys, so
// scores are an MFMA GEMM: tiles of 32 queries x 256 entries, the 16 rows of
// each MFMA tile being 4 queries x 4 indexer heads, so each lane's 4
// accumulators are the 4 heads of one (query, entry) pair.
// The full score matrix is never written. A sample GEMM over every 16th entry
// gives each query a threshold tau (about its (2k/16)-th best sample, so about
// 2k entries of the row score >= tau); the main GEMM keeps only scores >= tau.
// The select kernel checks it got at least k of them (otherwise it recomputes
// the row and selects exactly), finds the exact k-th key by binning plus an
// exact rank inside one bin, and orders the output with an LDS bitmap.

// 4 queries per MFMA row tile, kMT row tiles per wave, 4 waves: 32 queries per
// workgroup keeps the wave at 3 per SIMD (64 would need 2 more row tiles of
// accumulators and query fragments, leaving room for 2)
constexpr int kMT = 2;
constexpr int kCQ = 16 * kMT;   // queries per tile
constexpr int kCE = 256;    // entries per tile
constexpr int kLdsRow = kDI + 8;
constexpr int kWgCand = kChunkTileCand;
constexpr int kChunkTilesPerWg = 4;   // entry tiles a full-score workgroup walks (next tile prefetched)
// the sample pass touches 64 pages per tile and has few tiles: one tile per workgroup
template <int MODE> constexpr int chunk_tiles_per_wg() { return MODE == 0 ? 1 : kChunkTilesPerWg; }
constexpr int kMaxChunkTiles = kChunkMaxTiles;  // entry tiles per query the select accepts (262,144 entries)
static_assert(kMaxChunkTiles * kCE == kChunkMaxEntries, "host routing and the select agree on the limit");

template <int ACT, int KV, int MODE>
__global__ __launch_bounds__(256) void idx_chunk_gemm_kernel(const IdxChunkArgs a) {
  using CT = typename ComputeT<KV>::type;
  constexpr int AE = elem_bytes<ACT>(), KE = elem_bytes<KV>();
  constexpr bool SAMPLE = MODE == 0;
  constexpr bool POOL = MODE == 2;   // the full pass also writes 8-entry block maxima
  constexpr int kChunkElems = 16 / KE;                 // elements per 16-byte load
  constexpr int kChunksPerRow = kDI / kChunkElems;
  constexpr int kLoads = kCE * kChunksPerRow / 256;    // 16-byte loads per thread per tile
  constexpr int kPagesPerTile = SAMPLE ? kCE * kChunkSample / kPage : kCE / kPage;
  constexpr int TPW = chunk_tiles_per_wg<MODE>();
  __shared__ CT kt[kCE][kLdsRow];
  __shared__ float rsc[kCE];
  __shared__ int32_t pid[TPW * kPagesPerTile];

  const int n_et = SAMPLE ? a.n_stiles : a.n_etiles;
  const int n_eg = (n_et + TPW - 1) / TPW;   // entry-tile groups
  const int qt = blockIdx.x / n_eg, eg = blockIdx.x % n_eg;
  const int q0 = qt * kCQ;
  const int qlast = min(a.n_tok, q0 + kCQ) - 1;
  const int nvis_max = (a.pos0 + qlast + 1) / a.r;
  auto entry_of = [&](int m) { return SAMPLE ? m * kChunkSample + (kChunkSample - 1) : m; };
  const int et_begin = eg * TPW;
  int et_end = min(n_et, et_begin + TPW);
  while (et_end > et_begin && entry_of((et_end - 1) * kCE) >= nvis_max) --et_end;
  if (et_end <= et_begin) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
  const int qw = q0 + 4 * kMT * w;   // the wave's first query
  const char *kbase = reinterpret_cast<const char *>(a.kidx);

  // physical page of every page the walked tiles touch (pages are contiguous
  // per tile in both modes), read once, in the same round trip as the queries
  const int page0 = et_begin * kPagesPerTile;
  for (int i = tid; i < (et_end - et_begin) * kPagesPerTile; i += 256) {
    const int lp = page0 + i;
    pid[i] = lp * kPage < nvis_max ? a.bt_row[lp] : -1;
  }

  // A operands: (query, head) pairs as rows: row = 4*q + h
  Frag<CT> qa[kMT][2];
  float wq[kMT][4], tq[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int qq = qw + 4 * mt + (col >> 2), hh = col & 3;
    qa[mt][0] = qa[mt][1] = zero_frag<CT>();
    if (qq < a.n_tok && hh < a.h_i) {
      const char *qrow = reinterpret_cast<const char *>(a.q_idx) + (static_cast<int64_t>(qq) * a.h_i + hh) * kDI * AE;
#pragma unroll
      for (int c = 0; c < 2; ++c) qa[mt][c] = LoadFrag<ACT, CT>::load(qrow + (16 * g + 8 * c) * AE);
    }
    const int qo = qw + 4 * mt + g;   // the query this lane scores
#pragma unroll
    for (int v = 0; v < 4; ++v) wq[mt][v] = (qo < a.n_tok && v < a.h_i) ? a.w_idx[qo * a.h_i + v] : 0.f;
    tq[mt] = INFINITY;
    if constexpr (!SAMPLE) tq[mt] = qo < a.n_tok ? a.tau[qo] : INFINITY;
  }
  // visibility of each of the lane's queries, and of the wave's first (smallest) one
  int nvis[kMT];
  bool qok[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int qo = qw + 4 * mt + g;
    qok[mt] = qo < a.n_tok;
    nvis[mt] = (a.pos0 + qo + 1) / a.r;
  }
  const int nvis_lo = (a.pos0 + qw + 1) / a.r;
  __syncthreads();   // pid ready

  // register prefetch of one tile's indexer keys: all loads of a thread in flight together
  uint4 raw[kLoads];
  float rscale = 1.f;
  auto page_of = [&](int et, int e) { return pid[(et - et_begin) * kPagesPerTile + ((e >> 6) - et * kPagesPerTile)]; };
  auto load_tile = [&](int et) {
    const int m0 = et * kCE;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int i = u * 256 + tid;
      const int le = i / kChunksPerRow, ch = i % kChunksPerRow;
      const int e = entry_of(m0 + le);
      const int pp = e < nvis_max ? page_of(et, e) : -1;
      raw[u] = (pp >= 0 && pp < a.pool_pages)
                   ? *reinterpret_cast<const uint4 *>(kbase + ((static_cast<int64_t>(pp) * kPage + (e & 63)) * kDI + ch * kChunkElems) * KE)
                   : make_uint4(0, 0, 0, 0);
    }
    const int e = entry_of(m0 + tid);
    const int pp = e < nvis_max ? page_of(et, e) : -1;
    const bool ok = pp >= 0 && pp < a.pool_pages;
    if (e < nvis_max && !ok) flag_error(a.err, ERR_PAGE);
    rscale = (KV == DT_FP8 && ok) ? a.kidx_scale[pp] : 1.f;
  };
  auto commit_tile = [&]() {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int i = u * 256 + tid;
      const int le = i / kChunksPerRow, ch = i % kChunksPerRow;
      CT *dst = &kt[le][ch * kChunkElems];
      if constexpr (KV == DT_FP8) {
        const uint32_t wds[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x2_t lo = fp8x2_to_bf16<false>(wds[q]), hi = fp8x2_to_bf16<true>(wds[q]);
          dst[4 * q + 0] = lo[0]; dst[4 * q + 1] = lo[1]; dst[4 * q + 2] = hi[0]; dst[4 * q + 3] = hi[1];
        }
      } else {
        *reinterpret_cast<uint4 *>(dst) = raw[u];
      }
    }
    rsc[tid] = rscale;
  };

  load_tile(et_begin);
  for (int et = et_begin; et < et_end; ++et) {
    const int m0 = et * kCE;
    __syncthreads();                 // previous tile's LDS reads are done
    commit_tile();
    __syncthreads();
    if (et + 1 < et_end) load_tile(et + 1);   // in flight during this tile's MFMAs

    // candidates of (query, this tile) so far; every lane of a 16-lane group
    // scores the same query, so the group's ballot orders its slots by entry
    int run[kMT] = {};
    uint64_t *cand_t[kMT];   // this tile's candidate slots of each of the lane's queries
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      cand_t[mt] = a.cand + (static_cast<int64_t>(min(qw + 4 * mt + g, a.n_tok - 1)) * a.n_etiles + et) * kWgCand;
    // every (query, entry) pair of the wave visible in this tile: skip the per-score test
    // (the tile's code comes in two copies: without any visibility test for
    // the common fully visible tile, and with it)
    auto tile_body = [&](auto full_tag) {
    constexpr bool full = decltype(full_tag)::value;
#pragma unroll 1
    for (int pg = 0; pg < kCE / 64; ++pg) {
      float psc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) psc[nt] = KV == DT_FP8 ? rsc[pg * 64 + nt * 16 + col] : 1.f;
      f32x4_t acc[kMT][4];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int le = pg * 64 + nt * 16 + col;
        Frag<CT> kb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const CT *src = &kt[le][16 * g + 8 * c];
          if constexpr (KV == DT_F32) kb[c] = LoadFrag<DT_F32, float>::load(src);
          else kb[c] = LoadFrag<DT_BF16, __bf16>::load(src);
        }
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          acc[mt][nt] = mma(qa[mt][0], kb[0], acc[mt][nt]);
          acc[mt][nt] = mma(qa[mt][1], kb[1], acc[mt][nt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int qo = qw + 4 * mt + g;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int le = pg * 64 + nt * 16 + col;
          const int e = entry_of(m0 + le);
          float s = 0.f;
#pragma unroll
          for (int v = 0; v < 4; ++v) s += wq[mt][v] * relu_bits(acc[mt][nt][v]);
          if constexpr (KV == DT_FP8) s *= psc[nt];
          const bool vis = full || (qok[mt] && e < nvis[mt]);
          if constexpr (POOL) {
            // the 8 lanes of an aligned block hold consecutive entries of one query
            float m8 = vis ? s : -INFINITY;
            m8 = group_max(m8, kPoolBlock);
            if ((col & (kPoolBlock - 1)) == 0 && qok[mt] && e < nvis[mt])
              a.bmax[static_cast<int64_t>(qo) * a.bm_stride + (e >> 3)] = m8;
          }
          if constexpr (SAMPLE) {
            if (vis) a.ss[static_cast<int64_t>(qo) * a.ss_stride + m0 + le] = s;
          } else {
            const bool take = vis && s >= tq[mt];
            const uint32_t seg = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(take) >> (16 * g)) & 0xffffu;
            if (take) {
              // a tile with more than kWgCand candidates sends its query to the
              // select's exact fallback, which ignores the slots: the index is
              // clamped instead of tested
              const uint32_t slot = min(static_cast<uint32_t>(run[mt]) + __popc(seg & ((1u << col) - 1u)),
                                        static_cast<uint32_t>(kWgCand - 1));
              cand_t[mt][slot] = (static_cast<uint64_t>(static_cast<uint32_t>(e)) << 32) | __float_as_uint(s);
            }
            run[mt] += __popc(seg);
          }
        }
      }
    }
    };
    if (qw + 4 * kMT - 1 < a.n_tok && entry_of(m0 + kCE - 1) < nvis_lo) tile_body(std::true_type{});
    else tile_body(std::false_type{});
    if constexpr (!SAMPLE) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int qo = qw + 4 * mt + g;
        if (col == 0 && qo < a.n_tok) a.cnt[static_cast<int64_t>(qo) * a.n_etiles + et] = run[mt];
      }
    }
  }
}

// Per query: tau from its sampled scores.
// U float4 per thread hold a query's samples when ns <= 1024 U (the host picks
// the smallest U of 1, 2, 4, 8, 16 that covers the chunk's last query; each U is
// its own kernel so the common small case keeps few registers and many
// workgroups per CU). The loads take one round trip (rows are padded to 256
// floats; addresses past the last sample are clamped and those values ignored).
template <int U>
__global__ __launch_bounds__(256) void idx_chunk_tau_kernel(const IdxChunkArgs a) {
  __shared__ int hist[kTauBins];
  __shared__ float red[32];
  __shared__ int sh[4];
  const int qi = blockIdx.x;
  const int N = (a.pos0 + qi + 1) / a.r;
  const int ns = N / kChunkSample;          // visible samples: entries 16m + 15 < N
  float tau = 0.f;
  if (ns > a.m_s) {
    const float *row = a.ss + static_cast<int64_t>(qi) * a.ss_stride;
    float4 v[U];
    const int last4 = (ns - 1) >> 2;
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float4 *>(row + 4 * min(256 * u + static_cast<int>(threadIdx.x), last4));
    tau = tau_lower_bound_regs(v, ns, a.m_s, hist, red, sh);
  }
  if (threadIdx.x == 0) a.tau[qi] = tau;
}

// Element loads for the fallback's plain re-scoring of one row.
__device__ __forceinline__ float chunk_q(const IdxChunkArgs &a, int q, int h, int d) {
  const int64_t i = (static_cast<int64_t>(q) * a.h_i + h) * kDI + d;
  return a.act_dtype == DT_F32 ? reinterpret_cast<const float *>(a.q_idx)[i]
                               : bf16_to_f32(reinterpret_cast<const uint16_t *>(a.q_idx)[i]);
}
__device__ __forceinline__ float chunk_k(const IdxChunkArgs &a, int pp, int slot, int d) {
  const int64_t i = (static_cast<int64_t>(pp) * kPage + slot) * kDI + d;
  if (a.kv_dtype == DT_F32) return reinterpret_cast<const float *>(a.kidx)[i];
  if (a.kv_dtype == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(a.kidx)[i]);
  return fp8x2_to_f32<false>(reinterpret_cast<const uint8_t *>(a.kidx)[i])[0];
}

// Per query: its candidates (per-tile slot runs, already in entry order) are
// gathered into LDS and the exact Top-K is selected and written ascending.
__global__ __launch_bounds__(512) void idx_chunk_select_kernel(const IdxChunkArgs a) {
  __shared__ uint64_t bin_keys[kRankCap];
  __shared__ int hist[kSelBins];
  __shared__ float red[32];
  __shared__ int sh[4];
  __shared__ int wsum[16];
  __shared__ int toff[kMaxChunkTiles + 1];
  __shared__ int sel[CSA_MAX_TOPK];           // the fallback's index list
  const int qi = blockIdx.x, tid = threadIdx.x, bd = blockDim.x;
  const int N = (a.pos0 + qi + 1) / a.r, k = a.k;
  int32_t *out = a.topk + static_cast<int64_t>(qi) * k;
  if (N <= k) {
    for (int i = tid; i < k; i += bd) out[i] = i < N ? i : -1;
    return;
  }
  // per-tile candidate counts of this query -> offsets (tiles past its visible range hold none)
  // (the host sends longer rows query by query; a longer one here goes to the fallback)
  const int n_tiles = (N + kCE - 1) / kCE;
  const bool fits = n_tiles <= kMaxChunkTiles;
  const int32_t *tc = a.cnt + static_cast<int64_t>(qi) * a.n_etiles;
  if (tid == 0) { toff[0] = 0; sh[3] = fits ? 0 : 1; }
  __syncthreads();
  int c = 0;
  if (fits) {
    for (int i = tid; i < n_tiles; i += bd) {
      const int v = tc[i];
      if (v > kWgCand) sh[3] = 1;          // a tile overflowed its slots
      toff[i + 1] = min(v, kWgCand);
    }
    __syncthreads();
    block_prefix_sum(toff, n_tiles, wsum);
    c = toff[n_tiles];
  }
  bool done = false;
  if (sh[3] == 0 && c >= k && c <= kChunkCandCap) {
    const uint64_t *cq = a.cand + static_cast<int64_t>(qi) * a.n_etiles * kWgCand;
    // the tile of every candidate position, written tile by tile (bin_keys is
    // free until the select; c <= kChunkCandCap 16-bit entries fit it)
    static_assert(kChunkCandCap * 2 <= kRankCap * 8 && kMaxChunkTiles <= 65536, "tile map fits bin_keys");
    uint16_t *tile_of = reinterpret_cast<uint16_t *>(bin_keys);
    for (int t = tid; t < n_tiles; t += bd)
      for (int i = toff[t]; i < toff[t + 1]; ++i) tile_of[i] = static_cast<uint16_t>(t);
    __syncthreads();
    // thread tid holds candidates [tid s, tid s + s), s = ceil(c / 512), in
    // registers; the code is unrolled for the smallest P >= s of 4 and 8
    static_assert(kChunkCandCap / 512 == 8, "at most 8 candidates per thread");
    const int span = (c + 511) / 512, i0 = tid * span;
    auto gather_select = [&](auto per_tag) {
      constexpr int P = decltype(per_tag)::value;
      uint64_t tk[P];
#pragma unroll
      for (int u = 0; u < P; ++u) {   // every load first, then the keys
        const int i = i0 + u;
        tk[u] = 0;
        if (u < span && i < c) {
          const int lo = tile_of[i];
          tk[u] = cq[static_cast<int64_t>(lo) * kWgCand + (i - toff[lo])];   // entry << 32 | score bits
        }
      }
#pragma unroll
      for (int u = 0; u < P; ++u)
        tk[u] = score_key(__uint_as_float(static_cast<uint32_t>(tk[u])), static_cast<int>(tk[u] >> 32));
      // (the select's first barrier comes after every read of tile_of, which it then reuses)
      return select_ordered_regs(tk, c, k, hist, red, sh, bin_keys, out);
    };
    done = span <= 4 ? gather_select(std::integral_constant<int, 4>{}) : gather_select(std::integral_constant<int, 8>{});
    __syncthreads();
  }
  if (!done) {
    // too few or too many candidates, or heavy ties: score the whole row and select exactly
    if (tid == 0) flag_error(a.err, ERR_FALLBACK);
    __syncthreads();
    float *row = a.fb_rows + static_cast<int64_t>(qi) * a.fb_stride;
    const int t = a.pos0 + qi;
    (void)t;
    for (int e = tid; e < N; e += bd) {
      const int pp = a.bt_row[e >> 6];
      float sres = -1.f;
      if (pp >= 0 && pp < a.pool_pages) {
        const float sc = a.kv_dtype == DT_FP8 ? a.kidx_scale[pp] : 1.f;
        float acc = 0.f;
        for (int h = 0; h < a.h_i; ++h) {
          float dot = 0.f;
          for (int d = 0; d < kDI; ++d) dot += chunk_q(a, qi, h, d) * chunk_k(a, pp, e & 63, d);
          acc += a.w_idx[qi * a.h_i + h] * fmaxf(dot, 0.f);
        }
        sres = acc * sc;
      }
      row[e] = sres;
    }
    __syncthreads();
    select_and_write([&](int i) { return score_key(row[i], i); }, N, k, sel, hist, sh, out);
  }
}

// Candidate pool of each chunk query: the n_pool best 8-entry blocks by the
// block maxima the full pass wrote (ties -> lower block), ascending.
__global__ __launch_bounds__(512) void idx_chunk_pool_kernel(const IdxChunkArgs a) {
  __shared__ uint64_t keys[kSelCap];
  __shared__ uint64_t bin_keys[kRankCap];
  __shared__ int sel[CSA_MAX_POOL_BLOCKS];
  __shared__ int hist[kSelBins];
  __shared__ float red[32];
  __shared__ int sh[4];
  const int qi = blockIdx.x, tid = threadIdx.x, bd = blockDim.x;
  const int N = (a.pos0 + qi + 1) / a.r, P = a.n_pool;
  const int nB = (N + kPoolBlock - 1) / kPoolBlock;
  int32_t *out = a.pool + static_cast<int64_t>(qi) * P;
  const float *row = a.bmax + static_cast<int64_t>(qi) * a.bm_stride;
  if (nB <= P) {
    for (int i = tid; i < P; i += bd) out[i] = i < nB ? i : -1;
    return;
  }
  bool done = false;
  if (nB <= kSelCap) {
    // every load issued before the first use (clamped addresses, one round trip)
    constexpr int kPer = (kSelCap + 511) / 512;
    float v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u] = row[min(tid + u * bd, nB - 1)];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (tid + u * bd < nB) keys[tid + u * bd] = score_key(v[u], tid + u * bd);
    __syncthreads();
    done = select_ordered(keys, nB, P, hist, red, sh, bin_keys, out);
  }
  if (!done) select_and_write([&](int i) { return score_key(row[i], i); }, nB, P, sel, hist, sh, out);
}

}  // namespace

void launch_idx_chunk_pool(const IdxChunkArgs &a, hipStream_t s) {
  if (a.n_tok <= 0 || !a.pool) return;
  hipLaunchKernelGGL(idx_chunk_pool_kernel, dim3(a.n_tok), dim3(512), 0, s, a);
}

void launch_idx_scan(const IdxScanArgs &a, int kv, int act, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.total_wg <= 0) return;
  if (kv == DT_F32 && act == DT_F32)
    hipExtLaunchKernelGGL((idx_scan_kernel<DT_F32, DT_F32>), dim3(a.total_wg), dim3(kScanWaves * 64), 0, s, ev0, ev1, 0, a);
  else if (kv == DT_BF16 && act == DT_BF16)
    hipExtLaunchKernelGGL((idx_scan_kernel<DT_BF16, DT_BF16>), dim3(a.total_wg), dim3(kScanWaves * 64), 0, s, ev0, ev1, 0, a);
  else if (kv == DT_FP8 && act == DT_BF16)
    hipExtLaunchKernelGGL((idx_scan_kernel<DT_BF16, DT_FP8>), dim3(a.total_wg), dim3(kScanWaves * 64), 0, s, ev0, ev1, 0, a);
}

void launch_idx_small(const IdxScanArgs &a, int kv, int act, int32_t *topk, int k, hipStream_t s, hipEvent_t ev0,
                      hipEvent_t ev1) {
  if (a.n_q <= 0) return;
  if (kv == DT_F32 && act == DT_F32)
    hipExtLaunchKernelGGL((idx_small_kernel<DT_F32, DT_F32>), dim3(a.n_q), dim3(kSmallWaves * 64), 0, s, ev0, ev1, 0, a, topk, k);
  else if (kv == DT_BF16 && act == DT_BF16)
    hipExtLaunchKernelGGL((idx_small_kernel<DT_BF16, DT_BF16>), dim3(a.n_q), dim3(kSmallWaves * 64), 0, s, ev0, ev1, 0, a, topk, k);
  else if (kv == DT_FP8 && act == DT_BF16)
    hipExtLaunchKernelGGL((idx_small_kernel<DT_BF16, DT_FP8>), dim3(a.n_q), dim3(kSmallWaves * 64), 0, s, ev0, ev1, 0, a, topk, k);
}

void launch_idx_filter(const IdxFilterArgs &a, int n_wg, hipStream_t s) {
  if (n_wg <= 0) return;
  hipLaunchKernelGGL(idx_filter_kernel, dim3(n_wg), dim3(256), 0, s, a);
}

void launch_idx_final(const IdxFinalArgs &a, hipStream_t s) {
  if (a.n_q <= 0) return;
  hipLaunchKernelGGL(idx_final_kernel, dim3(a.n_q), dim3(512), 0, s, a);
}

void launch_idx_rescan(const IdxRescanArgs &a, int kv, int act, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.total_wg <= 0) return;
  if (kv == DT_F32 && act == DT_F32)
    hipExtLaunchKernelGGL((idx_rescan_kernel<DT_F32, DT_F32>), dim3(a.total_wg), dim3(kScanWaves * 64), 0, s, ev0, ev1, 0, a);
  else if (kv == DT_BF16 && act == DT_BF16)
    hipExtLaunchKernelGGL((idx_rescan_kernel<DT_BF16, DT_BF16>), dim3(a.total_wg), dim3(kScanWaves * 64), 0, s, ev0, ev1, 0, a);
  else if (kv == DT_FP8 && act == DT_BF16)
    hipExtLaunchKernelGGL((idx_rescan_kernel<DT_BF16, DT_FP8>), dim3(a.total_wg), dim3(kScanWaves * 64), 0, s, ev0, ev1, 0, a);
}

void launch_idx_chunk(const IdxChunkArgs &a, int kv, int act, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int n_qt = (a.n_tok + kCQ - 1) / kCQ;
  auto gemm = [&](auto mode_tag, int n_et, hipEvent_t e0, hipEvent_t e1) {
    constexpr int M = decltype(mode_tag)::value;
    const int n_wg = n_qt * ((n_et + chunk_tiles_per_wg<M>() - 1) / chunk_tiles_per_wg<M>());
    if (n_wg <= 0) return;
    if (kv == DT_F32 && act == DT_F32)
      hipExtLaunchKernelGGL((idx_chunk_gemm_kernel<DT_F32, DT_F32, M>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a);
    else if (kv == DT_BF16 && act == DT_BF16)
      hipExtLaunchKernelGGL((idx_chunk_gemm_kernel<DT_BF16, DT_BF16, M>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a);
    else if (kv == DT_FP8 && act == DT_BF16)
      hipExtLaunchKernelGGL((idx_chunk_gemm_kernel<DT_BF16, DT_FP8, M>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a);
  };
  gemm(std::integral_constant<int, 0>{}, a.n_stiles, nullptr, nullptr);
  static_assert(kChunkMaxEntries / kChunkSample <= 16 * 1024, "at most 16 float4 of samples per thread");
  const int ns_max = (a.pos0 + a.n_tok) / a.r / kChunkSample;   // the last query sees the most
  const dim3 tg(a.n_tok), tb(256);
  if (ns_max <= 1024) hipLaunchKernelGGL(idx_chunk_tau_kernel<1>, tg, tb, 0, s, a);
  else if (ns_max <= 2048) hipLaunchKernelGGL(idx_chunk_tau_kernel<2>, tg, tb, 0, s, a);
  else if (ns_max <= 4096) hipLaunchKernelGGL(idx_chunk_tau_kernel<4>, tg, tb, 0, s, a);
  else if (ns_max <= 8192) hipLaunchKernelGGL(idx_chunk_tau_kernel<8>, tg, tb, 0, s, a);
  else hipLaunchKernelGGL(idx_chunk_tau_kernel<16>, tg, tb, 0, s, a);
  if (a.pool) gemm(std::integral_constant<int, 2>{}, a.n_etiles, ev0, ev1);
  else gemm(std::integral_constant<int, 1>{}, a.n_etiles, ev0, ev1);
}

void launch_idx_chunk_select(const IdxChunkArgs &a, hipStream_t s) {
  if (a.n_tok <= 0) return;
  hipLaunchKernelGGL(idx_chunk_select_kernel, dim3(a.n_tok), dim3(512), 0, s, a);
}

}  // namespace csa
