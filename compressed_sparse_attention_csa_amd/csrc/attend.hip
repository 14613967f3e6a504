// csa_attend kernel: one softmax over the gathered Top-K compressed entries
// and the sliding-window raw rows, for all query heads sharing the one KV head.
//
// Method: DeepSeek-V4.1-Flash technical-report walkthrough, "Compressed Sparse
// Attention 2" > "The indexer selects, SWA covers the rest" (the query attends
// to the selected entries together with the layer-local window KV) and "SWA
// Bounded Replay" > "Replay only the window" (window keys [max(s, i-W+1), i]);
// Model-architectures atlas, MQA/GQA entry (many query heads, one KV head).
//
// Work decomposition: the keys of a query are cut into blocks of 64 (Top-K
// blocks first, then window blocks). A 256-thread workgroup owns (query,
// split), a split being a run of blocks:
//   1. it resolves the source of every key of the split once (Top-K index ->
//      page -> pool row and page scales, or window row -> ring row) into LDS;
//   2. per block, the 64 K and V rows (fp8 codes converted exactly to bf16)
//      go to LDS, K row-major and V transposed, while the next block's rows
//      are already being loaded into registers;
//   3. each active wave takes 16 heads: S^T[key][head] = K . Q^T with keys as
//      MFMA rows and heads as columns, so a lane holds one head and 4 keys per
//      16-key tile; after the online-softmax update those probabilities are
//      already the A operand of O = P . V (heads as rows, keys contracted),
//      paired with V^T from LDS.
// With one split per query the workgroup writes the normalised output. With
// several, each writes (m, l, O) partials; the last split of a query to finish
// (release fence + arrival counter) merges them with the log-sum-exp
// rescaling, which equals one softmax over the union of keys.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

template <int KV> struct ComputeT { using type = __bf16; };
template <> struct ComputeT<DT_F32> { using type = float; };

template <typename CT> constexpr int kpad() { return sizeof(CT) == 2 ? 8 : 4; }

template <typename CT>
__device__ __forceinline__ CT to_ct(float x) {
  if constexpr (sizeof(CT) == 4) {
    return x;
  } else {
    return __builtin_bit_cast(__bf16, f32_to_bf16(x));
  }
}

constexpr int kThreads = 256;
constexpr int kMaxSplits = kAttMaxSplits;

// Raw bytes of one 32-element segment of a row, by storage dtype.
template <int SD> struct Seg { uint4 u[SD == DT_F32 ? 8 : (SD == DT_BF16 ? 4 : 2)]; };

template <int SD>
__device__ __forceinline__ void load_seg(Seg<SD> &s, const char *src) {
  const uint4 *p = reinterpret_cast<const uint4 *>(src);
#pragma unroll
  for (int q = 0; q < static_cast<int>(sizeof(s.u) / 16); ++q) s.u[q] = p[q];
}
template <int SD>
__device__ __forceinline__ void zero_seg(Seg<SD> &s) {
#pragma unroll
  for (int q = 0; q < static_cast<int>(sizeof(s.u) / 16); ++q) s.u[q] = make_uint4(0, 0, 0, 0);
}

// Segment -> 32 compute-type values.
template <int SD, typename CT>
__device__ __forceinline__ void seg_values(const Seg<SD> &s, CT *dst) {
  if constexpr (SD == DT_F32) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dst[4 * q + 0] = to_ct<CT>(__uint_as_float(s.u[q].x)); dst[4 * q + 1] = to_ct<CT>(__uint_as_float(s.u[q].y));
      dst[4 * q + 2] = to_ct<CT>(__uint_as_float(s.u[q].z)); dst[4 * q + 3] = to_ct<CT>(__uint_as_float(s.u[q].w));
    }
  } else if constexpr (SD == DT_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {s.u[q].x, s.u[q].y, s.u[q].z, s.u[q].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dst[8 * q + 2 * u + 0] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(w[u] & 0xffffu));
        dst[8 * q + 2 * u + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(w[u] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w[4] = {s.u[q].x, s.u[q].y, s.u[q].z, s.u[q].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x2_t lo = fp8x2_to_bf16<false>(w[u]), hi = fp8x2_to_bf16<true>(w[u]);
        dst[16 * q + 4 * u + 0] = lo[0]; dst[16 * q + 4 * u + 1] = lo[1];
        dst[16 * q + 4 * u + 2] = hi[0]; dst[16 * q + 4 * u + 3] = hi[1];
      }
    }
  }
}

// AW: waves that compute (min(4, H/16)); NHT: 16-head tiles per computing wave.
template <int ACT, int KV, int AW, int NHT>
__global__ __launch_bounds__(kThreads) void attend_kernel(const AttendArgs a) {
  using CT = typename ComputeT<KV>::type;
  constexpr int KE = KV == DT_F32 ? 4 : (KV == DT_BF16 ? 2 : 1);
  constexpr int AE = ACT == DT_F32 ? 4 : 2;
  constexpr int KS = kD + kpad<CT>();          // K row stride (elements)
  constexpr int VS = kKeyBlock + kpad<CT>();   // V^T row stride (elements)
  constexpr int H = AW * NHT * 16;
  __shared__ CT Ks[kKeyBlock * KS];
  __shared__ CT Vt[kD * VS];
  __shared__ int32_t src_row[kAttMaxSplitKeys];   // >= 0 pool row; < 0: -(ring row) - 1
  __shared__ uint8_t kvalid[kAttMaxSplitKeys];
  __shared__ float ksc[kKeyBlock], vsc[kKeyBlock];  // page scales of the block in LDS

  const int qi = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
  const int seq = a.chunk ? a.seq0 : a.qd[qi].seq;
  const int t = a.chunk ? a.pos0 + qi : a.qd[qi].pos;
  const int n_vis = (t + 1) / a.r;
  const int swa_lo = max(0, t - a.W + 1);
  const int b_begin = split * a.blocks_per_split;
  const int b_end = min(a.n_blocks, b_begin + a.blocks_per_split);
  const int n_keys = (b_end - b_begin) * kKeyBlock;
  const int32_t *bt = a.block_table + static_cast<int64_t>(seq) * a.bt_stride;
  const int32_t *trow = a.topk + static_cast<int64_t>(qi) * a.k;
  const int tid = threadIdx.x;

  // ---------------- 1. resolve every key of the split
  for (int i = tid; i < n_keys; i += kThreads) {
    const int b = b_begin + i / kKeyBlock, kk = i % kKeyBlock;
    int valid = 0;
    int32_t row = 0;
    if (b < a.n_sparse_blocks) {
      const int slot = b * kKeyBlock + kk;
      const int j = slot < a.k ? trow[slot] : -1;
      if (j >= 0) {
        if (j >= n_vis) {
          flag_error(a.err, ERR_TOPK);
        } else {
          const int pp = bt[j >> 6];
          if (pp >= 0 && pp < a.pool_pages) {
            valid = 1;
            row = pp * kPage + (j & 63);
          } else {
            flag_error(a.err, ERR_PAGE);
          }
        }
      }
    } else {
      const int r = swa_lo + (b - a.n_sparse_blocks) * kKeyBlock + kk;
      if (r <= t) {
        valid = 1;
        row = -(seq * a.R + r % a.R) - 1;
      }
    }
    src_row[i] = row;
    kvalid[i] = valid;
  }
  __syncthreads();

  // ---------------- register prefetch of one block: thread owns (key, 32-dim segment)
  const int pk = tid & 63, psg = tid >> 6;
  Seg<KV> kseg, vseg;
  Seg<ACT> kraw, vraw;
  float pks = 1.f, pvs = 1.f;
  auto prefetch = [&](int b) {
    const int i = (b - b_begin) * kKeyBlock + pk;
    const int64_t row = src_row[i];
    pks = 1.f;
    pvs = 1.f;
    if (kvalid[i] == 0) {
      zero_seg(kseg); zero_seg(vseg); zero_seg(kraw); zero_seg(vraw);
    } else if (row >= 0) {
      const int64_t off = (row * kD + 32 * psg) * KE;
      load_seg(kseg, reinterpret_cast<const char *>(a.kbar) + off);
      load_seg(vseg, reinterpret_cast<const char *>(a.vbar) + off);
      if constexpr (KV == DT_FP8) {
        if (psg == 0) { pks = a.kbar_scale[row >> 6]; pvs = a.vbar_scale[row >> 6]; }
      }
    } else {
      const int64_t off = ((-row - 1) * kD + 32 * psg) * AE;
      load_seg(kraw, reinterpret_cast<const char *>(a.ring_k) + off);
      load_seg(vraw, reinterpret_cast<const char *>(a.ring_v) + off);
    }
  };
  auto commit = [&](int b) {
    const int i = (b - b_begin) * kKeyBlock + pk;
    CT kv[32], vv[32];
    if (src_row[i] >= 0 || !kvalid[i]) {
      seg_values<KV, CT>(kseg, kv);
      seg_values<KV, CT>(vseg, vv);
    } else {
      seg_values<ACT, CT>(kraw, kv);
      seg_values<ACT, CT>(vraw, vv);
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) Ks[pk * KS + 32 * psg + u] = kv[u];
#pragma unroll
    for (int u = 0; u < 32; ++u) Vt[(32 * psg + u) * VS + pk] = vv[u];
    if (psg == 0) { ksc[pk] = pks; vsc[pk] = pvs; }
  };

  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
  const bool computes = w < AW;

  // Q fragments (B operand of S^T) for this wave's head tiles
  Frag<CT> qf[NHT][4];
  f32x4_t O[NHT][8];
  float m_run[NHT], l_run[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int head = 16 * (w + AW * ht) + col;
    if (computes) {
      const char *qrow = reinterpret_cast<const char *>(a.q) + (static_cast<int64_t>(qi) * H + head) * kD * AE;
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[ht][c] = LoadFrag<ACT, CT>::load(qrow + (32 * g + 8 * c) * AE);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) O[ht][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }

  if (b_begin < b_end) prefetch(b_begin);
  for (int b = b_begin; b < b_end; ++b) {
    __syncthreads();                 // previous block's LDS reads are done
    commit(b);
    __syncthreads();
    if (b + 1 < b_end) prefetch(b + 1);   // in flight during this block's math
    if (!computes) continue;
    const int kb0 = (b - b_begin) * kKeyBlock;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      // S^T = K . Q^T
      f32x4_t S[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        S[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const CT *src = &Ks[(16 * kt + col) * KS + 32 * g + 8 * c];
          Frag<CT> kf;
          if constexpr (sizeof(CT) == 4) kf = LoadFrag<DT_F32, float>::load(src);
          else kf = LoadFrag<DT_BF16, __bf16>::load(src);
          S[kt] = mma(kf, qf[ht][c], S[kt]);
        }
      }
      // logits and online softmax (lane's head = col; keys 16*kt + 4*g + v)
      float x[4][4];
      float bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = kb0 + 16 * kt + 4 * g + v;
          x[kt][v] = kvalid[key] ? S[kt][v] * (a.scale * ksc[key - kb0]) : -INFINITY;
          bm = fmaxf(bm, x[kt][v]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run[ht], bm);
      const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run[ht] - m_new);
      float psum = 0.f;
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[kt][v] = (x[kt][v] == -INFINITY) ? 0.f : __expf(x[kt][v] - m_new);
          psum += p[kt][v];
        }
      l_run[ht] = l_run[ht] * alpha + psum;
      m_run[ht] = m_new;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
        for (int n = 0; n < 8; ++n) O[ht][n][v] *= av;
      }
      // O += P . V
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float pv[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[v] = p[2 * kc][v] * vsc[32 * kc + 4 * g + v];
          pv[4 + v] = p[2 * kc + 1][v] * vsc[32 * kc + 16 + 4 * g + v];
        }
        const Frag<CT> pf = frag_from_f32(pv, static_cast<Frag<CT> *>(nullptr));
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const CT *vr = &Vt[(16 * n + col) * VS + 32 * kc + 4 * g];
          Frag<CT> vf;
          if constexpr (sizeof(CT) == 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) { vf.v[u] = vr[u]; vf.v[4 + u] = vr[16 + u]; }
          } else {
            const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
            const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
            vf.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          }
          O[ht][n] = mma(pf, vf, O[ht][n]);
        }
      }
    }
  }

  // ---------------- finish
  if (a.n_splits == 1) {
    if (!computes) return;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float l_tot = l_run[ht] + __shfl_xor(l_run[ht], 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * (w + AW * ht) + 4 * g + v;
        const float lh = __shfl(l_tot, 4 * g + v, 64);
        const float inv = lh > 0.f ? 1.f / lh : 0.f;
        const int64_t ob = (static_cast<int64_t>(qi) * H + h) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float o = O[ht][n][v] * inv;
          if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[ob + 16 * n + col] = o;
          else reinterpret_cast<uint16_t *>(a.out)[ob + 16 * n + col] = f32_to_bf16(o);
        }
      }
    }
    return;
  }

  const int64_t pbase = static_cast<int64_t>(qi) * a.n_splits + split;
  if (computes) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float l_tot = l_run[ht] + __shfl_xor(l_run[ht], 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const int h0 = 16 * (w + AW * ht);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float *po = a.part_o + (pbase * H + h0 + 4 * g + v) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) po[16 * n + col] = O[ht][n][v];
      }
      if (g == 0) {
        a.part_ml[(pbase * 2 + 0) * H + h0 + col] = m_run[ht];
        a.part_ml[(pbase * 2 + 1) * H + h0 + col] = l_tot;
      }
    }
  }
}

// Combines the split partials of (query, head): one softmax over the union of
// every split's keys. Thread d owns output dimension d; all of its loads are
// independent, so the whole merge is about one memory round trip.
template <int ACT>
__global__ __launch_bounds__(kD) void attend_merge_kernel(const AttendArgs a) {
  const int qi = blockIdx.x / a.H, h = blockIdx.x % a.H, d = threadIdx.x;
  const int64_t q0 = static_cast<int64_t>(qi) * a.n_splits;
  float m[kMaxSplits], l[kMaxSplits], o[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const bool ok = s < a.n_splits;
    m[s] = ok ? a.part_ml[((q0 + s) * 2 + 0) * a.H + h] : -INFINITY;
    l[s] = ok ? a.part_ml[((q0 + s) * 2 + 1) * a.H + h] : 0.f;
    o[s] = ok ? a.part_o[((q0 + s) * a.H + h) * kD + d] : 0.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) mx = fmaxf(mx, m[s]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const float e = (m[s] == -INFINITY) ? 0.f : __expf(m[s] - mx);
    L += e * l[s];
    acc += e * o[s];
  }
  const float out = L > 0.f ? acc / L : 0.f;
  const int64_t oi = (static_cast<int64_t>(qi) * a.H + h) * kD + d;
  if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[oi] = out;
  else reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16(out);
}

template <int ACT, int KV>
void launch_attend_t(const AttendArgs &a, int n_wg, hipStream_t s) {
  switch (a.H) {
    case 16: hipLaunchKernelGGL((attend_kernel<ACT, KV, 1, 1>), dim3(n_wg), dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((attend_kernel<ACT, KV, 2, 1>), dim3(n_wg), dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL((attend_kernel<ACT, KV, 4, 1>), dim3(n_wg), dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((attend_kernel<ACT, KV, 4, 2>), dim3(n_wg), dim3(kThreads), 0, s, a); break;
    default: break;
  }
}

}  // namespace

void launch_attend(const AttendArgs &a, int n_wg, int kv, int act, hipStream_t s) {
  if (n_wg <= 0) return;
  if (kv == DT_F32 && act == DT_F32) launch_attend_t<DT_F32, DT_F32>(a, n_wg, s);
  else if (kv == DT_BF16 && act == DT_BF16) launch_attend_t<DT_BF16, DT_BF16>(a, n_wg, s);
  else if (kv == DT_FP8 && act == DT_BF16) launch_attend_t<DT_BF16, DT_FP8>(a, n_wg, s);
  if (a.n_splits > 1) {
    if (act == DT_F32) hipLaunchKernelGGL(attend_merge_kernel<DT_F32>, dim3(a.n_q * a.H), dim3(kD), 0, s, a);
    else hipLaunchKernelGGL(attend_merge_kernel<DT_BF16>, dim3(a.n_q * a.H), dim3(kD), 0, s, a);
  }
}

}  // namespace csa
