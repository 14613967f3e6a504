// csa_attend kernel: one softmax over the gathered Top-K compressed entries
// and the sliding-window raw rows, for all query heads sharing the one KV head.
//
// Method: DeepSeek-V4.1-Flash technical-report walkthrough, "Compressed Sparse
// Attention 2" > "The indexer selects, SWA covers the rest" (the query attends
// to the selected entries together with the layer-local window KV) and "SWA
// Bounded Replay" > "Replay only the window" (window keys [max(s, i-W+1), i]);
// Model-architectures atlas, MQA/GQA entry (many query heads, one KV head).
//
// Work decomposition. The keys of a query are cut into blocks of 64 (Top-K
// blocks first, then window blocks). A workgroup owns (query, split), a split
// being a run of blocks, and has HG x KSTR waves: HG head groups times KSTR
// key streams. Each round it gathers KSTR blocks (one per stream) into LDS, K
// row-major and V transposed in the MFMA compute type (fp8 codes convert
// exactly to bf16; page scales are applied to the logits and probabilities),
// while the next round's rows are already being loaded into registers. Wave
// (head group, stream) then runs, for its 16-head tiles and its stream's block:
//   S^T[key][head] = K . Q^T  (keys as MFMA rows, heads as columns), so a lane
//   holds one head and 4 keys per 16-key tile; after the online-softmax update
//   those probabilities are already the A operand of O = P . V (heads as rows,
//   keys contracted) against V^T from LDS.
// The streams' (m, l, O) are merged in LDS at the end. With one split per
// query the workgroup writes the output; with several, each writes its (m, l,
// O) partial and a merge kernel combines them with the log-sum-exp rescaling,
// which equals one softmax over the union of all keys. (A merge by the last
// split to finish would need a device-scope release fence per workgroup, which
// on this multi-XCD part writes back the L2 and costs more than the launch.)
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

__device__ __forceinline__ float f4_at(const float4 &f, int i) {
  return i == 0 ? f.x : (i == 1 ? f.y : (i == 2 ? f.z : f.w));
}

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


// One gather item: 32 dims of one key's K and V row, as raw bytes of either
// the pool format (KV) or the window-ring format (ACT); kind says which.
template <int ACT, int KV>
struct Item {
  static constexpr int RW = (sizeof(Seg<KV>) > sizeof(Seg<ACT>) ? sizeof(Seg<KV>) : sizeof(Seg<ACT>)) / 16;
  uint4 k[RW], v[RW];
  float ks, vs;
  int kind;   // 0 masked, 1 pool row, 2 ring row
};

template <int SD, int RW>
__device__ __forceinline__ const Seg<SD> &as_seg(const uint4 (&u)[RW]) {
  return *reinterpret_cast<const Seg<SD> *>(&u[0]);
}

// HG: head groups (waves per stream); NTW: 16-head tiles per wave; KSTR: key streams.
template <int ACT, int KV, int HG, int NTW, int KSTR>
__global__ __launch_bounds__(HG * KSTR * 64) void attend_kernel(const AttendArgs a) {
  using CT = typename ComputeT<KV>::type;
  constexpr int NT = HG * KSTR * 64;
  constexpr int H = HG * NTW * 16;
  constexpr int KE = KV == DT_F32 ? 4 : (KV == DT_BF16 ? 2 : 1);
  constexpr int AE = ACT == DT_F32 ? 4 : 2;
  constexpr int KS = kD + kpad<CT>();          // K row stride (elements)
  constexpr int VS = kKeyBlock + kpad<CT>();   // V^T row stride (elements)
  constexpr int ITEMS = KSTR * 256 / NT;       // gather items per thread per round
  constexpr bool PREFETCH = KV != DT_F32;      // fp32 rows are too large to hold a round in registers
  constexpr int KV_LDS = KSTR * (kKeyBlock * KS + kD * VS) * static_cast<int>(sizeof(CT));
  static_assert((KSTR - 1) * H * kD * 4 <= KV_LDS, "stream partials must fit in the K/V buffers");

  __shared__ __align__(16) char kv_lds[KV_LDS];
  __shared__ int32_t src_row[kAttMaxSplitKeys];   // >= 0 pool row; < 0: -(ring row) - 1
  __shared__ uint8_t kvalid[kAttMaxSplitKeys];
  // per key of the block: logit = S * kmul + kbias (kmul = scale x page scale,
  // kbias = -inf for a masked key), probability weight vsc = value page scale
  __shared__ __align__(16) float kmul[KSTR][kKeyBlock];
  __shared__ __align__(16) float kbias[KSTR][kKeyBlock];
  __shared__ __align__(16) float vsc[KSTR][kKeyBlock];
  __shared__ float sm_m[KSTR][H], sm_l[KSTR][H];
  CT *Ks = reinterpret_cast<CT *>(kv_lds);                       // [KSTR][64][KS]
  CT *Vt = Ks + KSTR * kKeyBlock * KS;                           // [KSTR][D][VS]

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

  // ---------------- 1. resolve every key of the split once: all Top-K reads
  // of a thread first, then all of its block-table reads (two round trips)
  constexpr int kMaxPer = (kAttMaxSplitKeys + NT - 1) / NT;
  int jv[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    const int i = tid + u * NT;
    jv[u] = -1;
    if (i < n_keys) {
      const int b = b_begin + i / kKeyBlock, kk = i % kKeyBlock;
      if (b < a.n_sparse_blocks) {
        const int slot = b * kKeyBlock + kk;
        jv[u] = slot < a.k ? trow[slot] : -1;
      }
    }
  }
  int pv[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    const int j = jv[u];
    pv[u] = (j >= 0 && j < n_vis) ? bt[j >> 6] : -1;
  }
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    const int i = tid + u * NT;
    if (i >= n_keys) continue;
    const int b = b_begin + i / kKeyBlock, kk = i % kKeyBlock;
    int valid = 0;
    int32_t row = 0;
    if (b < a.n_sparse_blocks) {
      const int j = jv[u], pp = pv[u];
      if (j >= 0) {
        if (j >= n_vis) {
          flag_error(a.err, ERR_TOPK);
        } else if (pp >= 0 && pp < a.pool_pages) {
          valid = 1;
          row = pp * kPage + (j & 63);
        } else {
          flag_error(a.err, ERR_PAGE);
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

  // ---------------- gather: item = (stream, key, 32-dim segment)
  using It = Item<ACT, KV>;
  auto load_item = [&](It &x, int gi, int r) {
    const int st = gi >> 8, pk = gi & 63, psg = (gi >> 6) & 3;
    const int b = b_begin + r * KSTR + st;
    const int i = (b - b_begin) * kKeyBlock + pk;
    x.ks = 1.f;
    x.vs = 1.f;
    x.kind = 0;
    if (b >= b_end || kvalid[i] == 0) return;
    const int64_t row = src_row[i];
    if (row >= 0) {
      x.kind = 1;
      const int64_t off = (row * kD + 32 * psg) * KE;
      load_seg(*reinterpret_cast<Seg<KV> *>(&x.k[0]), reinterpret_cast<const char *>(a.kbar) + off);
      load_seg(*reinterpret_cast<Seg<KV> *>(&x.v[0]), reinterpret_cast<const char *>(a.vbar) + off);
      if constexpr (KV == DT_FP8) {
        if (psg == 0) { x.ks = a.kbar_scale[row >> 6]; x.vs = a.vbar_scale[row >> 6]; }
      }
    } else {
      x.kind = 2;
      const int64_t off = ((-row - 1) * kD + 32 * psg) * AE;
      load_seg(*reinterpret_cast<Seg<ACT> *>(&x.k[0]), reinterpret_cast<const char *>(a.ring_k) + off);
      load_seg(*reinterpret_cast<Seg<ACT> *>(&x.v[0]), reinterpret_cast<const char *>(a.ring_v) + off);
    }
  };
  auto commit_item = [&](const It &x, int gi) {
    const int st = gi >> 8, pk = gi & 63, psg = (gi >> 6) & 3;
    CT kv[32], vv[32];
    if (x.kind == 1) {
      seg_values<KV, CT>(as_seg<KV>(x.k), kv);
      seg_values<KV, CT>(as_seg<KV>(x.v), vv);
    } else if (x.kind == 2) {
      seg_values<ACT, CT>(as_seg<ACT>(x.k), kv);
      seg_values<ACT, CT>(as_seg<ACT>(x.v), vv);
    } else {
#pragma unroll
      for (int u = 0; u < 32; ++u) { kv[u] = to_ct<CT>(0.f); vv[u] = to_ct<CT>(0.f); }
    }
    CT *kd = Ks + (st * kKeyBlock + pk) * KS + 32 * psg;
    CT *vd = Vt + st * kD * VS + (32 * psg) * VS + pk;
#pragma unroll
    for (int u = 0; u < 32; ++u) kd[u] = kv[u];
#pragma unroll
    for (int u = 0; u < 32; ++u) vd[u * VS] = vv[u];
    if (psg == 0) {
      kmul[st][pk] = x.kind != 0 ? a.scale * x.ks : 0.f;
      kbias[st][pk] = x.kind != 0 ? 0.f : -INFINITY;
      vsc[st][pk] = x.vs;
    }
  };
  It items[PREFETCH ? ITEMS : 1];
  auto load_round = [&](int r) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) load_item(items[it], tid + it * NT, r);
  };
  auto commit_round = [&](int r) {
    if constexpr (PREFETCH) {
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) commit_item(items[it], tid + it * NT);
    } else {
      for (int it = 0; it < ITEMS; ++it) {
        load_item(items[0], tid + it * NT, r);
        commit_item(items[0], tid + it * NT);
      }
    }
  };

  const int lane = tid & 63, w = tid >> 6, hg = w % HG, ks = w / HG, g = lane >> 4, col = lane & 15;

  // Q fragments (B operand of S^T) for this wave's head tiles
  Frag<CT> qf[NTW][4];
  f32x4_t O[NTW][8];
  float m_run[NTW], l_run[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int head = 16 * (hg + HG * j) + col;
    const char *qrow = reinterpret_cast<const char *>(a.q) + (static_cast<int64_t>(qi) * H + head) * kD * AE;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[j][c] = LoadFrag<ACT, CT>::load(qrow + (32 * g + 8 * c) * AE);
#pragma unroll
    for (int n = 0; n < 8; ++n) O[j][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }

  const int n_rounds = (b_end - b_begin + KSTR - 1) / KSTR;
  if constexpr (PREFETCH) {
    if (n_rounds > 0) load_round(0);
  }
  for (int r = 0; r < n_rounds; ++r) {
    __syncthreads();                   // previous round's LDS reads are done
    commit_round(r);
    __syncthreads();
    if constexpr (PREFETCH) {
      if (r + 1 < n_rounds) load_round(r + 1);   // in flight during this round's math
    }
    const int b = b_begin + r * KSTR + ks;
    if (b >= b_end) continue;
    const int kb0 = (b - b_begin) * kKeyBlock;
    const CT *Kb = Ks + ks * kKeyBlock * KS;
    const CT *Vb = Vt + ks * kD * VS;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      // S^T tiles; the next tile's K fragments are read while this one multiplies
      f32x4_t S[4];
      Frag<CT> kf[2][4];
      auto load_kf = [&](Frag<CT> (&dst)[4], int kt) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const CT *src = Kb + (16 * kt + col) * KS + 32 * g + 8 * c;
          if constexpr (sizeof(CT) == 4) dst[c] = LoadFrag<DT_F32, float>::load(src);
          else dst[c] = LoadFrag<DT_BF16, __bf16>::load(src);
        }
      };
      load_kf(kf[0], 0);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if (kt + 1 < 4) load_kf(kf[(kt + 1) & 1], kt + 1);
        S[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) S[kt] = mma(kf[kt & 1][c], qf[j][c], S[kt]);
      }
      // per-key factors of the lane's keys 16*kt + 4*g + v, four at a time
      float4 km[4], kbi[4], vs4[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        km[kt] = *reinterpret_cast<const float4 *>(&kmul[ks][16 * kt + 4 * g]);
        kbi[kt] = *reinterpret_cast<const float4 *>(&kbias[ks][16 * kt + 4 * g]);
        vs4[kt] = *reinterpret_cast<const float4 *>(&vsc[ks][16 * kt + 4 * g]);
      }
      // logits and online softmax (lane's head = col; keys 16*kt + 4*g + v)
      float x[4][4];
      float bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[kt][v] = fmaf(S[kt][v], f4_at(km[kt], v), f4_at(kbi[kt], v));
          bm = fmaxf(bm, x[kt][v]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run[j], bm);
      const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run[j] - m_new);
      float psum = 0.f;
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[kt][v] = (x[kt][v] == -INFINITY) ? 0.f : __expf(x[kt][v] - m_new);
          psum += p[kt][v];
        }
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
        for (int n = 0; n < 8; ++n) O[j][n][v] *= av;
      }
      // O += P . V over the two 32-key halves; V^T fragments read one step ahead
      auto load_vf = [&](int kc, int n) {
        const CT *vr = Vb + (16 * n + col) * VS + 32 * kc + 4 * g;
        Frag<CT> vf;
        if constexpr (sizeof(CT) == 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) { vf.v[u] = vr[u]; vf.v[4 + u] = vr[16 + u]; }
        } else {
          const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
          const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
          vf.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
        return vf;
      };
      Frag<CT> vfb[2];
      vfb[0] = load_vf(0, 0);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float pv[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[v] = p[2 * kc][v] * f4_at(vs4[2 * kc], v);
          pv[4 + v] = p[2 * kc + 1][v] * f4_at(vs4[2 * kc + 1], v);
        }
        const Frag<CT> pf = frag_from_f32(pv, static_cast<Frag<CT> *>(nullptr));
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int step = kc * 8 + n;
          if (step + 1 < 16) vfb[(step + 1) & 1] = load_vf((step + 1) >> 3, (step + 1) & 7);
          O[j][n] = mma(pf, vfb[step & 1], O[j][n]);
        }
      }
    }
  }

  // ---------------- 2. merge the key streams in LDS (stream 0 keeps the result)
  float *po = reinterpret_cast<float *>(kv_lds);   // [KSTR-1][H][D] partial outputs of streams >= 1
  __syncthreads();                                 // all rounds done: K/V buffers are free
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int h0 = 16 * (hg + HG * j);
    float l_tot = l_run[j] + __shfl_xor(l_run[j], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (g == 0) {
      sm_m[ks][h0 + col] = m_run[j];
      sm_l[ks][h0 + col] = l_tot;
    }
    if (ks > 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int n = 0; n < 8; ++n) po[((ks - 1) * H + h0 + 4 * g + v) * kD + 16 * n + col] = O[j][n][v];
    }
  }
  __syncthreads();
  float Lh[NTW][4];   // per O row (head 4g + v of each tile): merged denominator and max
  float Mh[NTW][4];
  if (ks == 0) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int h0 = 16 * (hg + HG * j);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = h0 + 4 * g + v;
        float mx = -INFINITY;
#pragma unroll
        for (int s = 0; s < KSTR; ++s) mx = fmaxf(mx, sm_m[s][h]);
        float L = 0.f;
        float al[KSTR];
#pragma unroll
        for (int s = 0; s < KSTR; ++s) {
          al[s] = (sm_m[s][h] == -INFINITY) ? 0.f : __expf(sm_m[s][h] - mx);
          L += al[s] * sm_l[s][h];
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          float o = al[0] * O[j][n][v];
#pragma unroll
          for (int s = 1; s < KSTR; ++s) o += al[s] * po[((s - 1) * H + h) * kD + 16 * n + col];
          O[j][n][v] = o;
        }
        Lh[j][v] = L;
        Mh[j][v] = mx;
      }
    }
  }

  if (a.n_splits == 1) {
    if (ks != 0) return;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * (hg + HG * j) + 4 * g + v;
        const float inv = Lh[j][v] > 0.f ? 1.f / Lh[j][v] : 0.f;
        const int64_t ob = (static_cast<int64_t>(qi) * H + h) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float o = O[j][n][v] * inv;
          if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[ob + 16 * n + col] = o;
          else reinterpret_cast<uint16_t *>(a.out)[ob + 16 * n + col] = f32_to_bf16(o);
        }
      }
    return;
  }

  // ---------------- 3. several splits: write this split's partial; the merge kernel combines them
  const int64_t pbase = static_cast<int64_t>(qi) * a.n_splits + split;
  if (ks == 0) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * (hg + HG * j) + 4 * g + v;
        float *pr = a.part_o + (pbase * H + h) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) pr[16 * n + col] = O[j][n][v];
        if (col == 0) {
          a.part_ml[(pbase * 2 + 0) * H + h] = Mh[j][v];
          a.part_ml[(pbase * 2 + 1) * H + h] = Lh[j][v];
        }
      }
  }
}

// Combines the split partials of (query, head): one softmax over the union of
// every split's keys. Thread d owns output dimension d; all of its loads are
// independent, so the merge costs about one memory round trip.
template <int ACT>
__global__ __launch_bounds__(kD) void attend_merge_kernel(const AttendArgs a) {
  const int qi = blockIdx.x / a.H, h = blockIdx.x % a.H, d = threadIdx.x;
  const int64_t q0 = static_cast<int64_t>(qi) * a.n_splits;
  float m[kAttMaxSplits], l[kAttMaxSplits], o[kAttMaxSplits];
#pragma unroll
  for (int s = 0; s < kAttMaxSplits; ++s) {
    const bool ok = s < a.n_splits;
    m[s] = ok ? a.part_ml[((q0 + s) * 2 + 0) * a.H + h] : -INFINITY;
    l[s] = ok ? a.part_ml[((q0 + s) * 2 + 1) * a.H + h] : 0.f;
    o[s] = ok ? a.part_o[((q0 + s) * a.H + h) * kD + d] : 0.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kAttMaxSplits; ++s) mx = fmaxf(mx, m[s]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int s = 0; s < kAttMaxSplits; ++s) {
    const float e = (m[s] == -INFINITY) ? 0.f : __expf(m[s] - mx);
    L += e * l[s];
    acc += e * o[s];
  }
  const float out = L > 0.f ? acc / L : 0.f;
  const int64_t oi = (static_cast<int64_t>(qi) * a.H + h) * kD + d;
  if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[oi] = out;
  else reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16(out);
}

template <int ACT, int KV, int KSTR>
void launch_attend_k(const AttendArgs &a, int n_wg, hipStream_t s) {
  switch (a.H) {
    case 16: hipLaunchKernelGGL((attend_kernel<ACT, KV, 1, 1, KSTR>), dim3(n_wg), dim3(1 * KSTR * 64), 0, s, a); break;
    case 32: hipLaunchKernelGGL((attend_kernel<ACT, KV, 2, 1, KSTR>), dim3(n_wg), dim3(2 * KSTR * 64), 0, s, a); break;
    case 64: hipLaunchKernelGGL((attend_kernel<ACT, KV, 4, 1, KSTR>), dim3(n_wg), dim3(4 * KSTR * 64), 0, s, a); break;
    case 128: hipLaunchKernelGGL((attend_kernel<ACT, KV, 4, 2, KSTR>), dim3(n_wg), dim3(4 * KSTR * 64), 0, s, a); break;
    default: break;
  }
}

template <int ACT, int KV>
void launch_attend_t(const AttendArgs &a, int n_wg, hipStream_t s) {
  // decode: one block per split (latency-bound); a prefill chunk walks all of a
  // query's blocks in one workgroup, two blocks per round
  if (a.chunk && KV != DT_F32) launch_attend_k<ACT, KV, kAttChunkKeyStreams>(a, n_wg, s);
  else launch_attend_k<ACT, KV, kAttKeyStreams>(a, n_wg, s);
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
