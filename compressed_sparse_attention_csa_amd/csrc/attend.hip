// csa_attend kernels: one softmax over the gathered Top-K compressed entries
// and the sliding-window raw rows, for all query heads sharing the one KV head.
//
// Method: DeepSeek-V4.1-Flash technical-report walkthrough, "Compressed Sparse
// Attention 2" > "The indexer selects, SWA covers the rest" (the query attends
// to the selected entries together with the layer-local window KV) and "SWA
// Bounded Replay" > "Replay only the window" (window keys [max(s, i-W+1), i]);
// Model-architectures atlas, MQA/GQA entry (many query heads, one KV head).
//
// Work decomposition: the keys of a query are cut into blocks of 64 (Top-K
// blocks first, then window blocks). A workgroup owns (query, split), a split
// being a run of blocks, and loops over its blocks with an online softmax.
// Per block the workgroup gathers the 64 keys into LDS (K row-major, V
// transposed, both in the MFMA compute type, fp8 codes converted exactly to
// bf16 with the page scales kept aside), then each wave takes 16 heads:
//   S^T[key][head] = K . Q^T  (keys as MFMA rows, heads as columns), so each
//   lane holds one head and 4 keys per 16-key tile;
//   those probabilities are already laid out as the A operand of O = P . V
//   (heads as rows, keys as the contraction), paired with V^T from LDS.
// With one split per query the workgroup writes the normalised output; with
// several it writes (m, l, O) partials that the merge kernel combines with the
// usual log-sum-exp rescaling, which is one softmax over the union of keys.
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

// Convert 32 contiguous elements of storage dtype SD at src into dst[0..32) (compute type).
template <int SD, typename CT>
__device__ __forceinline__ void load32(const char *src, CT *dst) {
  if constexpr (SD == DT_F32) {
    const float4 *s = reinterpret_cast<const float4 *>(src);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = s[q];
      dst[4 * q + 0] = to_ct<CT>(v.x); dst[4 * q + 1] = to_ct<CT>(v.y);
      dst[4 * q + 2] = to_ct<CT>(v.z); dst[4 * q + 3] = to_ct<CT>(v.w);
    }
  } else if constexpr (SD == DT_BF16) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = s[q];
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dst[8 * q + 2 * u + 0] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(wds[u] & 0xffffu));
        dst[8 * q + 2 * u + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(wds[u] >> 16));
      }
    }
  } else {  // fp8 -> bf16, exact
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 v = s[q];
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x2_t lo = fp8x2_to_bf16<false>(wds[u]), hi = fp8x2_to_bf16<true>(wds[u]);
        dst[16 * q + 4 * u + 0] = lo[0]; dst[16 * q + 4 * u + 1] = lo[1];
        dst[16 * q + 4 * u + 2] = hi[0]; dst[16 * q + 4 * u + 3] = hi[1];
      }
    }
  }
}

template <int ACT, int KV, int NW>
__global__ __launch_bounds__(NW * 64) void attend_kernel(const AttendArgs a) {
  using CT = typename ComputeT<KV>::type;
  constexpr int KE = KV == DT_F32 ? 4 : (KV == DT_BF16 ? 2 : 1);
  constexpr int AE = ACT == DT_F32 ? 4 : 2;
  constexpr int KS = kD + kpad<CT>();          // K row stride (elements)
  constexpr int VS = kKeyBlock + kpad<CT>();   // V^T row stride (elements)
  __shared__ CT Ks[kKeyBlock * KS];
  __shared__ CT Vt[kD * VS];
  __shared__ float sK[kKeyBlock], sV[kKeyBlock];
  __shared__ int kval[kKeyBlock];

  const int qi = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
  const int seq = a.chunk ? a.seq0 : a.qd[qi].seq;
  const int t = a.chunk ? a.pos0 + qi : a.qd[qi].pos;
  const int n_vis = (t + 1) / a.r;
  const int swa_lo = max(0, t - a.W + 1);
  const int b_begin = split * a.blocks_per_split;
  const int b_end = min(a.n_blocks, b_begin + a.blocks_per_split);
  const int32_t *bt = a.block_table + static_cast<int64_t>(seq) * a.bt_stride;
  const int32_t *trow = a.topk + static_cast<int64_t>(qi) * a.k;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, col = lane & 15;
  const int head = 16 * w + col;   // head owned in S^T (column)

  // Q fragments (B operand of S^T): dims [32g + 8c, +8)
  Frag<CT> qf[4];
  {
    const char *qrow = reinterpret_cast<const char *>(a.q) + (static_cast<int64_t>(qi) * a.H + head) * kD * AE;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = LoadFrag<ACT, CT>::load(qrow + (32 * g + 8 * c) * AE);
  }

  f32x4_t O[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) O[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int b = b_begin; b < b_end; ++b) {
    // ---------------- gather 64 keys of block b into LDS
    __syncthreads();
    for (int item = threadIdx.x; item < kKeyBlock * 4; item += NW * 64) {
      const int kk = item & 63, sg = item >> 6;
      CT kbuf[32], vbuf[32];
      bool valid = false;
      float sk = 1.f, sv = 1.f;
      if (b < a.n_sparse_blocks) {
        const int slot = b * kKeyBlock + kk;
        const int j = slot < a.k ? trow[slot] : -1;
        if (j >= 0) {
          if (j >= n_vis) {
            if (sg == 0) flag_error(a.err, ERR_TOPK);
          } else {
            const int pp = bt[j >> 6];
            if (pp >= 0 && pp < a.pool_pages) {
              valid = true;
              const int64_t off = ((static_cast<int64_t>(pp) * kPage + (j & 63)) * kD + 32 * sg) * KE;
              load32<KV, CT>(reinterpret_cast<const char *>(a.kbar) + off, kbuf);
              load32<KV, CT>(reinterpret_cast<const char *>(a.vbar) + off, vbuf);
              if constexpr (KV == DT_FP8) { sk = a.kbar_scale[pp]; sv = a.vbar_scale[pp]; }
            } else if (sg == 0) {
              flag_error(a.err, ERR_PAGE);
            }
          }
        }
      } else {
        const int row = swa_lo + (b - a.n_sparse_blocks) * kKeyBlock + kk;
        if (row <= t) {
          valid = true;
          const int64_t off = ((static_cast<int64_t>(seq) * a.R + row % a.R) * kD + 32 * sg) * AE;
          load32<ACT, CT>(reinterpret_cast<const char *>(a.ring_k) + off, kbuf);
          load32<ACT, CT>(reinterpret_cast<const char *>(a.ring_v) + off, vbuf);
        }
      }
      if (!valid) {
#pragma unroll
        for (int u = 0; u < 32; ++u) { kbuf[u] = to_ct<CT>(0.f); vbuf[u] = to_ct<CT>(0.f); }
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) Ks[kk * KS + 32 * sg + u] = kbuf[u];
#pragma unroll
      for (int u = 0; u < 32; ++u) Vt[(32 * sg + u) * VS + kk] = vbuf[u];
      if (sg == 0) {
        sK[kk] = sk;
        sV[kk] = sv;
        kval[kk] = valid ? 1 : 0;
      }
    }
    __syncthreads();

    // ---------------- S^T = K . Q^T for this wave's 16 heads
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
        S[kt] = mma(kf, qf[c], S[kt]);
      }
    }
    // logits, online softmax (lane's head = col; keys 16*kt + 4*g + v)
    float x[4][4];
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = 16 * kt + 4 * g + v;
        x[kt][v] = kval[key] ? S[kt][v] * (a.scale * sK[key]) : -INFINITY;
        bm = fmaxf(bm, x[kt][v]);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    float psum = 0.f;
    float p[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[kt][v] = (x[kt][v] == -INFINITY) ? 0.f : __expf(x[kt][v] - m_new);
        psum += p[kt][v];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // rescale O rows (heads 4g + v of this wave)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
      for (int n = 0; n < 8; ++n) O[n][v] *= av;
    }

    // ---------------- O += P . V  (P: heads x keys, V^T from LDS)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      float pv[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[v] = p[2 * kc][v] * sV[32 * kc + 4 * g + v];
        pv[4 + v] = p[2 * kc + 1][v] * sV[32 * kc + 16 + 4 * g + v];
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
        O[n] = mma(pf, vf, O[n]);
      }
    }
  }

  // ---------------- finish: per-head totals
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  if (a.n_splits == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * w + 4 * g + v;
      const float lh = __shfl(l_tot, 4 * g + v, 64);
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      const int64_t ob = (static_cast<int64_t>(qi) * a.H + h) * kD;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float o = O[n][v] * inv;
        if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[ob + 16 * n + col] = o;
        else reinterpret_cast<uint16_t *>(a.out)[ob + 16 * n + col] = f32_to_bf16(o);
      }
    }
  } else {
    float *pb = a.part + (static_cast<int64_t>(qi) * a.n_splits + split) * a.H * (kD + 2);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * w + 4 * g + v;
#pragma unroll
      for (int n = 0; n < 8; ++n) pb[h * (kD + 2) + 16 * n + col] = O[n][v];
    }
    if (g == 0) {
      pb[head * (kD + 2) + kD] = m_run;
      pb[head * (kD + 2) + kD + 1] = l_tot;
    }
  }
}

// Combines split partials: one softmax over the union of every split's keys.
template <int ACT>
__global__ __launch_bounds__(256) void attend_merge_kernel(const MergeArgs a) {
  const int qi = blockIdx.x / (a.H / 2);
  const int h = (blockIdx.x % (a.H / 2)) * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  const float *pb = a.part + static_cast<int64_t>(qi) * a.n_splits * a.H * (kD + 2);
  float m = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) m = fmaxf(m, pb[(s * a.H + h) * (kD + 2) + kD]);
  float L = 0.f, o = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < a.n_splits; ++s) {
      const float *ps = pb + (s * a.H + h) * (kD + 2);
      const float ms = ps[kD];
      if (ms == -INFINITY) continue;
      const float f = __expf(ms - m);
      L += f * ps[kD + 1];
      o += f * ps[d];
    }
  }
  o = L > 0.f ? o / L : 0.f;
  const int64_t oi = (static_cast<int64_t>(qi) * a.H + h) * kD + d;
  if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[oi] = o;
  else reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16(o);
}

template <int ACT, int KV>
void launch_attend_t(const AttendArgs &a, int n_wg, hipStream_t s) {
  switch (a.H / 16) {
    case 1: hipLaunchKernelGGL((attend_kernel<ACT, KV, 1>), dim3(n_wg), dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attend_kernel<ACT, KV, 2>), dim3(n_wg), dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attend_kernel<ACT, KV, 4>), dim3(n_wg), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attend_kernel<ACT, KV, 8>), dim3(n_wg), dim3(512), 0, s, a); break;
    default: break;
  }
}

}  // namespace

void launch_attend(const AttendArgs &a, int n_wg, int kv, int act, hipStream_t s) {
  if (n_wg <= 0) return;
  if (kv == DT_F32 && act == DT_F32) launch_attend_t<DT_F32, DT_F32>(a, n_wg, s);
  else if (kv == DT_BF16 && act == DT_BF16) launch_attend_t<DT_BF16, DT_BF16>(a, n_wg, s);
  else if (kv == DT_FP8 && act == DT_BF16) launch_attend_t<DT_BF16, DT_FP8>(a, n_wg, s);
}

void launch_attend_merge(const MergeArgs &a, int act, hipStream_t s) {
  const int n_wg = a.n_q * (a.H / 2);
  if (n_wg <= 0) return;
  if (act == DT_F32) hipLaunchKernelGGL(attend_merge_kernel<DT_F32>, dim3(n_wg), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attend_merge_kernel<DT_BF16>, dim3(n_wg), dim3(256), 0, s, a);
}

}  // namespace csa
