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
// being a run of blocks, and has HG waves (head groups). Each round it gathers
// one block into LDS, K row-major and V transposed in the MFMA compute type
// (fp8 codes convert exactly to bf16; page scales are applied to the logits
// and probabilities): a block's rows move as 16-byte chunks, CPR consecutive
// lanes per row, as raw buffer loads whose 32-bit offsets come from a per-key
// table built once per split (a key that takes no part points past the end
// of the buffer and reads zeros, so no lane branches), and the next block is
// already in flight in registers during this block's math. Each wave then
// runs, for its 16-head tiles:
//   S^T[key][head] = K . Q^T  (keys as MFMA rows, heads as columns), so a lane
//   holds one head and 4 keys per 16-key tile; after the online-softmax update
//   those probabilities are already the A operand of O = P . V (heads as rows,
//   keys contracted) against V^T from LDS.
// With one split per query the workgroup writes the output; with several,
// each writes its (m, l, O) partial and a merge kernel combines them with the
// log-sum-exp rescaling, which equals one softmax over the union of all keys.
// (A merge by the last split to finish would need a device-scope release
// fence per workgroup, which on this multi-XCD part writes back the L2 and
// costs more than the launch.)
#include <type_traits>

#include <hip/hip_ext.h>

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

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i supplies the address of
// 4 consecutive 16-bit values D[i][0..3]; lane j receives D[4q + j/4][j%4],
// q = 0..3 (a transposed 16 x 4 tile).
__device__ __forceinline__ uint2 lds_read_tr16(const void *p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t *)(const_cast<void *>(p)));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ float f4_at(const float4 &f, int i) {
  return i == 0 ? f.x : (i == 1 ? f.y : (i == 2 ? f.z : f.w));
}

// 16 bytes of a row (E = 16 / element size elements) -> compute type. An fp4
// chunk holds 32 elements, two 16-channel groups whose E4M3 scale codes are
// bytes 0 and 1 of gsc; E2M1 x E4M3 products are exact in bf16.
template <int SD, typename CT>
__device__ __forceinline__ void chunk_values(const uint4 &u, CT *dst, uint32_t gsc = 0) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (SD == DT_FP4) {
    const float s0 = e4m3_to_f32(gsc & 0xffu), s1 = e4m3_to_f32((gsc >> 8) & 0xffu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sc = q < 2 ? s0 : s1;
      const f32x2_t v0 = fp4x2_to_f32<0>(w[q]), v1 = fp4x2_to_f32<1>(w[q]);
      const f32x2_t v2 = fp4x2_to_f32<2>(w[q]), v3 = fp4x2_to_f32<3>(w[q]);
      dst[8 * q + 0] = to_ct<CT>(v0[0] * sc); dst[8 * q + 1] = to_ct<CT>(v0[1] * sc);
      dst[8 * q + 2] = to_ct<CT>(v1[0] * sc); dst[8 * q + 3] = to_ct<CT>(v1[1] * sc);
      dst[8 * q + 4] = to_ct<CT>(v2[0] * sc); dst[8 * q + 5] = to_ct<CT>(v2[1] * sc);
      dst[8 * q + 6] = to_ct<CT>(v3[0] * sc); dst[8 * q + 7] = to_ct<CT>(v3[1] * sc);
    }
  } else if constexpr (SD == DT_F32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = to_ct<CT>(__uint_as_float(w[q]));
  } else if constexpr (SD == DT_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dst[2 * q + 0] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(w[q] & 0xffffu));
      dst[2 * q + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(w[q] >> 16));
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2_t lo = fp8x2_to_bf16<false>(w[q]), hi = fp8x2_to_bf16<true>(w[q]);
      dst[4 * q + 0] = lo[0]; dst[4 * q + 1] = lo[1];
      dst[4 * q + 2] = hi[0]; dst[4 * q + 3] = hi[1];
    }
  }
}

// Gathers are buffer loads: a row's address is a 32-bit byte offset into its
// pool (or ring) buffer, and a key that takes no part gets an offset past the
// buffer's end, where the load returns zeros without touching memory. Buffers
// hold at most kOobOffset bytes, so no in-row chunk offset wraps back in range.
constexpr uint32_t kOobOffset = kAttMaxBufferBytes;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *p, uint32_t bytes) {
  // stride 0 (raw buffer: range check on the byte offset), 32-bit dword format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.f;             // log2 headroom of the lazily rescaled softmax

// 2^x with the hardware instruction alone (results below 2^-126 flush to 0,
// which a softmax weight can lose).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int SD> constexpr int elem_bytes_of() { return SD == DT_F32 ? 4 : (SD == DT_BF16 ? 2 : 1); }
template <int SD> constexpr int row_bytes_of() { return SD == DT_FP4 ? kD / 2 : kD * elem_bytes_of<SD>(); }

// RS: storage type of the window ring (ACT, or E4M3 with one scale per row);
// HG: head groups; NTW: 16-head tiles per wave; KH: key halves. The HG x KH
// waves split each staged 64-key block: wave (hg, kh) takes head tiles
// hg + HG j and, with KH = 2, only the block's keys [32 kh, 32 kh + 32), so a
// key's K and V are read from LDS by HG waves instead of all of them. With
// KH = 2 the two halves keep their own softmax states (m, l, O) and combine
// them through LDS at the end.
template <int ACT, int KV, int RS, int HG, int NTW, int KH>
__global__ __launch_bounds__(HG * KH * 64) void attend_kernel(const AttendArgs a) {
  using CT = typename ComputeT<KV>::type;
  static_assert(KH == 1 || KH == 2, "one or two key halves");
  constexpr int NT = HG * KH * 64;
  constexpr int NKT = 4 / KH;                  // 16-key tiles of a block per wave
  constexpr int H = HG * NTW * 16;
  constexpr int AE = elem_bytes_of<ACT>();
  constexpr bool VSCALE = KV == DT_FP8 || RS == DT_FP8;   // value rows carry a page or row scale
  constexpr int64_t PRB = row_bytes_of<KV>(), RRB = row_bytes_of<RS>();   // pool / ring row bytes
  constexpr int KS = kD + kpad<CT>();          // K row stride (elements)
  // bf16: V row-major like K, read as transposed MFMA fragments; fp32: V^T.
  // A transposed read covers 4 rows x 32 bytes per 16 lanes, so bf16 V rows are
  // padded by 32 bytes (8 banks) to keep those rows on disjoint banks.
  constexpr bool VROW = sizeof(CT) == 2;
  constexpr int VS = VROW ? kD + 16 : kKeyBlock + kpad<CT>();   // V (or V^T) row stride (elements)
  // a block's K and V rows move as 16-byte chunks, 16 consecutive lanes per
  // 256-byte row, so every wave load covers whole rows
  constexpr int CPR_P = row_bytes_of<KV>() / 16, CPR_R = row_bytes_of<RS>() / 16;   // chunks per pool / ring row
  constexpr int CPR_MAX = CPR_P > CPR_R ? CPR_P : CPR_R;
  static_assert((CPR_P & (CPR_P - 1)) == 0 && (CPR_R & (CPR_R - 1)) == 0, "chunks per row are powers of two");
  constexpr int U = 2 * kKeyBlock * CPR_MAX / NT;              // chunk slots per thread per block
  constexpr bool PREFETCH = U <= 8;                            // whole block held in registers
  constexpr int KV_STAGE = (kKeyBlock * KS + (VROW ? kKeyBlock : kD) * VS) * static_cast<int>(sizeof(CT));
  // the second key half's (m, l, O) per head group, after the last block
  constexpr int OSTR = kD + 4;
  constexpr int HALF_LDS = KH == 2 ? HG * NTW * 16 * (OSTR + 2) * 4 : 0;
  constexpr int KV_LDS = KV_STAGE > HALF_LDS ? KV_STAGE : HALF_LDS;

  __shared__ __align__(16) char kv_lds[KV_LDS];
  // byte offset of each key's row in the pool (Top-K blocks) or ring (window
  // blocks) buffer; kOobOffset for a key that takes no part
  __shared__ uint32_t src_off[kAttMaxSplitKeys];
  __shared__ uint8_t kvalid[kAttMaxSplitKeys];
  // per key of the block: logit = S * kmul + kbias (kmul = scale x page scale,
  // kbias = -inf for a masked key), probability weight vsc = value page scale.
  // Without page or row scales kmul is one constant and the block's masked
  // keys are the zero bits of kmask.
  __shared__ __align__(16) float kmul[VSCALE ? kKeyBlock : 1];
  __shared__ __align__(16) float kbias[VSCALE ? kKeyBlock : 1];
  __shared__ __align__(16) float vsc[VSCALE ? kKeyBlock : 1];
  __shared__ uint64_t kmask;
  CT *Ks = reinterpret_cast<CT *>(kv_lds);                       // [64][KS]
  CT *Vt = Ks + kKeyBlock * KS;                                  // [64][VS] (bf16) or [D][VS]

  const int qi = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
  const int seq = a.chunk ? a.seq0 : a.qd[qi].seq;
  const int t = a.chunk ? a.pos0 + qi : a.qd[qi].pos;
  const int n_vis = (t + 1) / a.r;
  const int swa_lo = max(a.chunk ? a.swa0 : a.qd[qi].swa, t - a.W + 1);   // replay start s bounds the window
  const int b_begin = split * a.blocks_per_split;
  const int b_end = min(a.n_blocks, b_begin + a.blocks_per_split);
  const int n_keys = (b_end - b_begin) * kKeyBlock;
  const int32_t *bt = a.block_table + static_cast<int64_t>(seq) * a.bt_stride;
  const int32_t *trow = a.dense ? nullptr : a.topk + static_cast<int64_t>(qi) * a.k;
  const int tid = threadIdx.x;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hg = wave % HG, kh = wave / HG, g = lane >> 4, col = lane & 15;

  // Q fragments (B operand of S^T) for this wave's head tiles, loaded first:
  // in flight during the key resolution
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
        jv[u] = a.dense ? (slot < n_vis ? slot : -1) : (slot < a.k ? trow[slot] : -1);
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
    uint32_t off = kOobOffset;
    if (b < a.n_sparse_blocks) {
      const int j = jv[u], pp = pv[u];
      if (j >= 0) {
        if (j >= n_vis) {
          flag_error(a.err, ERR_TOPK);
        } else if (pp >= 0 && pp < a.pool_pages) {
          valid = 1;
          off = static_cast<uint32_t>(pp * kPage + (j & 63)) * static_cast<uint32_t>(PRB);
        } else {
          flag_error(a.err, ERR_PAGE);
        }
      }
    } else {
      const int r = swa_lo + (b - a.n_sparse_blocks) * kKeyBlock + kk;
      if (r <= t) {
        valid = 1;
        off = static_cast<uint32_t>(seq * a.R + r % a.R) * static_cast<uint32_t>(RRB);
      }
    }
    src_off[i] = off;
    kvalid[i] = valid;
  }
  __syncthreads();

  // ---------------- gather: slot u of a thread in a block whose rows have CPR
  // 16-byte chunks is chunk (tid mod CPR) of key ((u NT + tid) mod 64 CPR) / CPR,
  // of K for the first 64 CPR slots of the block and of V for the next; slots
  // past 2 x 64 CPR are unused. Which slots are K, V or unused is known at
  // compile time per u, and a K slot and its V slot share one row offset.
  const __amdgpu_buffer_rsrc_t pool_k = buffer_of(a.kbar, a.pool_bytes), pool_v = buffer_of(a.vbar, a.pool_bytes);
  const __amdgpu_buffer_rsrc_t ring_k = buffer_of(a.ring_k, a.ring_bytes), ring_v = buffer_of(a.ring_v, a.ring_bytes);
  constexpr int UW = U < 8 ? U : 8;      // slots in registers at once
  uint4 raw[UW];
  uint32_t graw[KV == DT_FP4 ? UW : 1];  // fp4: the chunk's two group-scale codes
  float ks_pref = 1.f, vs_pref = 1.f;   // page (or ring row) scales of key tid (tid < 64)
  // the loads of slots [u0, u0 + UW) of block b (rows stored as SD) into v[], gs[]
  auto gather = [&](auto sd_tag, int b, int u0, uint4 *v, uint32_t *gs) {
    constexpr int SD = decltype(sd_tag)::value;
    constexpr int CPR = row_bytes_of<SD>() / 16;
    constexpr bool POOL_SD = SD == KV;
    const bool pool = b < a.n_sparse_blocks;
    const __amdgpu_buffer_rsrc_t rk = pool ? pool_k : ring_k, rv = pool ? pool_v : ring_v;
    const uint32_t *offs = src_off + (b - b_begin) * kKeyBlock;
    const uint32_t chunk_off = static_cast<uint32_t>(tid & (CPR - 1)) * 16u;
#pragma unroll
    for (int w = 0; w < UW; ++w) {
      const int u = u0 + w;
      if (u * NT >= 2 * kKeyBlock * CPR) break;
      const bool is_v = u * NT >= kKeyBlock * CPR;
      const int key = ((u * NT) % (kKeyBlock * CPR) + tid) / CPR;
      const uint32_t row_off = offs[key];
      v[w] = buffer_load16(is_v ? rv : rk, row_off + chunk_off);
      if constexpr (KV == DT_FP4 && POOL_SD) {
        // 8 scale bytes per fp4 row (64 B): two per 16-byte chunk
        const uint8_t *gbase = is_v ? a.vbar_gs : a.kbar_gs;
        const uint32_t goff = row_off >= kOobOffset ? kOobOffset : (row_off >> 3) + chunk_off / 8u;
        gs[w] = __builtin_amdgcn_raw_buffer_load_b16(buffer_of(gbase, a.gs_bytes), goff, 0, 0);
      }
    }
  };
  auto load_scales = [&](int b) {
    ks_pref = vs_pref = 1.f;
    if (tid < kKeyBlock) {
      const uint32_t off = src_off[(b - b_begin) * kKeyBlock + tid];
      if constexpr (KV == DT_FP8) {
        if (b < a.n_sparse_blocks && off != kOobOffset) {   // page scales
          const uint32_t page = off / static_cast<uint32_t>(PRB * kPage);
          ks_pref = a.kbar_scale[page];
          vs_pref = a.vbar_scale[page];
        }
      }
      if constexpr (RS == DT_FP8) {
        if (b >= a.n_sparse_blocks && off != kOobOffset) {  // ring row scales
          const uint32_t row = off / static_cast<uint32_t>(RRB);
          ks_pref = a.ring_k_scale[row];
          vs_pref = a.ring_v_scale[row];
        }
      }
    }
  };
  // slots [u0, u0 + UW) of a block (rows stored as SD) -> compute type -> K
  // row-major and V row-major (bf16) or V^T (fp32) in LDS
  auto commit = [&](auto sd_tag, int u0, const uint4 *v, const uint32_t *gs) {
    constexpr int SD = decltype(sd_tag)::value;
    constexpr int E = SD == DT_FP4 ? 32 : 16 / elem_bytes_of<SD>();
    constexpr int CPR = kD / E;
#pragma unroll
    for (int w = 0; w < UW; ++w) {
      const int u = u0 + w;
      if (u * NT >= 2 * kKeyBlock * CPR) break;
      const bool is_v = u * NT >= kKeyBlock * CPR;
      const int key = ((u * NT) % (kKeyBlock * CPR) + tid) / CPR, d0 = (tid & (CPR - 1)) * E;
      CT vals[E];
      uint32_t gsc = 0;
      if constexpr (SD == DT_FP4) gsc = gs[w];
      chunk_values<SD, CT>(v[w], vals, gsc);
      if (!is_v) {
        CT *kd = Ks + key * KS + d0;
#pragma unroll
        for (int q = 0; q < E; ++q) kd[q] = vals[q];
      } else if constexpr (VROW) {
        CT *vd = Vt + key * VS + d0;
#pragma unroll
        for (int q = 0; q < E; ++q) vd[q] = vals[q];
      } else {
        CT *vd = Vt + d0 * VS + key;
#pragma unroll
        for (int q = 0; q < E; ++q) vd[q * VS] = vals[q];
      }
    }
  };
  auto load_round = [&](int r) {
    const int b = b_begin + r;
    if (b >= b_end) return;
    if constexpr (PREFETCH) {
      if (b < a.n_sparse_blocks) gather(std::integral_constant<int, KV>{}, b, 0, raw, graw);
      else gather(std::integral_constant<int, RS>{}, b, 0, raw, graw);
    }
    load_scales(b);
  };
  auto commit_round = [&](int r) {
    const int b = b_begin + r;
    if constexpr (PREFETCH) {
      if (b < a.n_sparse_blocks) commit(std::integral_constant<int, KV>{}, 0, raw, graw);
      else commit(std::integral_constant<int, RS>{}, 0, raw, graw);
    } else {
      // rows too wide to hold a block in registers (fp32): gather and commit
      // UW slots at a time
      auto slices = [&](auto sd_tag) {
#pragma unroll
        for (int u0 = 0; u0 < U; u0 += UW) {
          gather(sd_tag, b, u0, raw, graw);
          commit(sd_tag, u0, raw, graw);
        }
      };
      if (b < a.n_sparse_blocks) slices(std::integral_constant<int, KV>{});
      else slices(std::integral_constant<int, RS>{});
    }
    if (tid < kKeyBlock) {   // wave 0
      const bool valid = kvalid[(b - b_begin) * kKeyBlock + tid] != 0;
      if constexpr (VSCALE) {
        kmul[tid] = valid ? a.scale * kLog2e * ks_pref : 0.f;   // logits in log2 units
        kbias[tid] = valid ? 0.f : -INFINITY;
        vsc[tid] = vs_pref;
      } else {
        const uint64_t m = __builtin_amdgcn_ballot_w64(valid);
        if (tid == 0) kmask = m;
      }
    }
  };


  const int n_rounds = b_end - b_begin;
  if (n_rounds > 0) load_round(0);
  for (int r = 0; r < n_rounds; ++r) {
    __syncthreads();                   // previous round's LDS reads are done
    commit_round(r);
    __syncthreads();
    if (r + 1 < n_rounds) load_round(r + 1);   // in flight during this round's math
    const CT *Kb = Ks;
    const CT *Vb = Vt;
    // S^T tiles of this wave's keys (tile i is block key tile kt0 + i) for all
    // of its head tiles: each K fragment is read from LDS once, and the next
    // tile's are read while this one multiplies
    const int kt0 = kh * NKT;
    f32x4_t S[NTW][NKT];
    {
      Frag<CT> kf[2][4];
      auto load_kf = [&](Frag<CT> (&dst)[4], int kt) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const CT *src = Kb + (16 * kt + col) * KS + 32 * g + 8 * c;
          if constexpr (sizeof(CT) == 4) dst[c] = LoadFrag<DT_F32, float>::load(src);
          else dst[c] = LoadFrag<DT_BF16, __bf16>::load(src);
        }
      };
      load_kf(kf[0], kt0);
#pragma unroll
      for (int i = 0; i < NKT; ++i) {
        if (i + 1 < NKT) load_kf(kf[(i + 1) & 1], kt0 + i + 1);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          S[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) S[j][i] = mma(kf[i & 1][c], qf[j][c], S[j][i]);
        }
      }
    }
    // per-key factors of the lane's keys 16*(kt0 + i) + 4*g + v, four at a time
    float4 km[NKT], kbi[NKT];
    if constexpr (VSCALE) {
#pragma unroll
      for (int i = 0; i < NKT; ++i) {
        km[i] = *reinterpret_cast<const float4 *>(&kmul[16 * (kt0 + i) + 4 * g]);
        kbi[i] = *reinterpret_cast<const float4 *>(&kbias[16 * (kt0 + i) + 4 * g]);
      }
    } else {
      const float c = a.scale * kLog2e;   // logits in log2 units
      const uint64_t mk = kmask;
#pragma unroll
      for (int i = 0; i < NKT; ++i) {
        km[i] = make_float4(c, c, c, c);
        kbi[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (mk != ~0ull) {
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
          const uint32_t nib = static_cast<uint32_t>(mk >> (16 * (kt0 + i) + 4 * g)) & 0xfu;
          kbi[i] = make_float4((nib & 1u) ? 0.f : -INFINITY, (nib & 2u) ? 0.f : -INFINITY,
                               (nib & 4u) ? 0.f : -INFINITY, (nib & 8u) ? 0.f : -INFINITY);
        }
      }
    }
    float4 vs4[NKT];
#pragma unroll
    for (int i = 0; i < NKT; ++i)
      if constexpr (VSCALE) vs4[i] = *reinterpret_cast<const float4 *>(&vsc[16 * (kt0 + i) + 4 * g]);
      else vs4[i] = make_float4(1.f, 1.f, 1.f, 1.f);
    // logits and online softmax per head tile (lane's head = col)
    constexpr int NKC = NKT / 2;   // 32-key halves of this wave
    Frag<CT> pf[NTW][NKC];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      float x[NKT][4];
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < NKT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[i][v] = fmaf(S[j][i][v], f4_at(km[i], v), f4_at(kbi[i], v));
          bm = fmaxf(bm, x[i][v]);
        }
      bm = max_xor32(max_xor16(bm));
      // Lazy rescaling: O and l stay relative to the reference max m_run, which
      // moves only when a head's block max exceeds it by more than kRescale
      // (probabilities stay <= 2^kRescale); the wave rescales all its heads then.
      if (__builtin_amdgcn_ballot_w64(bm > m_run[j] + kRescale) != 0) {
        const float m_new = fmaxf(m_run[j], bm);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[j] - m_new);
        l_run[j] *= alpha;
        m_run[j] = m_new;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
          for (int n = 0; n < 8; ++n) O[j][n][v] *= av;
        }
      }
      const float m_ref = m_run[j] == -INFINITY ? 0.f : m_run[j];   // masked keys: exp2(-inf) = 0
      float psum = 0.f;
      float p[NKT][4];
#pragma unroll
      for (int i = 0; i < NKT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[i][v] = fast_exp2(x[i][v] - m_ref);
          psum += p[i][v];
        }
      l_run[j] += psum;
#pragma unroll
      for (int c2 = 0; c2 < NKC; ++c2) {
        float pv[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[v] = p[2 * c2][v] * f4_at(vs4[2 * c2], v);
          pv[4 + v] = p[2 * c2 + 1][v] * f4_at(vs4[2 * c2 + 1], v);
        }
        pf[j][c2] = frag_from_f32(pv, static_cast<Frag<CT> *>(nullptr));
      }
    }
    // O += P . V over this wave's 32-key halves: each V^T fragment is read
    // once (one step ahead) and serves every head tile
    auto load_vf = [&](int kc, int n) {
      Frag<CT> vf;
      if constexpr (VROW) {
        // keys 32kc + 4g + (0..3) and + 16 for dim 16n + col: in each 16-lane
        // group lane i reads 4 dims of key 4g + i/4, and the transposing read
        // hands lane col those 4 keys at its dim
        const CT *vr = Vb + (32 * kc + 4 * g + (col >> 2)) * VS + 16 * n + 4 * (col & 3);
        const uint2 lo = lds_read_tr16(vr);
        const uint2 hi = lds_read_tr16(vr + 16 * VS);
        vf.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
      } else {
        const CT *vr = Vb + (16 * n + col) * VS + 32 * kc + 4 * g;
#pragma unroll
        for (int u = 0; u < 4; ++u) { vf.v[u] = vr[u]; vf.v[4 + u] = vr[16 + u]; }
      }
      return vf;
    };
    const int kc0 = kh * NKC;
    Frag<CT> vfb[2];
    vfb[0] = load_vf(kc0, 0);
#pragma unroll
    for (int c2 = 0; c2 < NKC; ++c2)
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int step = c2 * 8 + n;
        if (step + 1 < NKC * 8) vfb[(step + 1) & 1] = load_vf(kc0 + ((step + 1) >> 3), (step + 1) & 7);
#pragma unroll
        for (int j = 0; j < NTW; ++j) O[j][n] = mma(pf[j][c2], vfb[step & 1], O[j][n]);
      }
  }

  // ---------------- 2. per O row (head 16*tile + 4g + v): its running max and sum
  float Lh[NTW][4], Mh[NTW][4];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const float l_tot = sum_xor32(sum_xor16(l_run[j]));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      Mh[j][v] = __shfl(m_run[j], 4 * g + v, 64);
      Lh[j][v] = __shfl(l_tot, 4 * g + v, 64);
    }
  }

  if constexpr (KH == 2) {
    // the second key half hands its (m, l, O) to the first through LDS; the
    // first rescales both to their common maximum and carries on alone
    float *ho = reinterpret_cast<float *>(kv_lds) + hg * NTW * 16 * (OSTR + 2);   // [NTW*16][OSTR] O, then m, l
    float *hm = ho + NTW * 16 * OSTR;
    __syncthreads();                   // every wave is done with the last block's K and V
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int hr = 16 * j + 4 * g + v;
#pragma unroll
          for (int n = 0; n < 8; ++n) ho[hr * OSTR + 16 * n + col] = O[j][n][v];
          if (col == 0) { hm[2 * hr] = Mh[j][v]; hm[2 * hr + 1] = Lh[j][v]; }
        }
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int hr = 16 * j + 4 * g + v;
        const float m1 = hm[2 * hr], l1 = hm[2 * hr + 1], m0 = Mh[j][v];
        const float mx = fmaxf(m0, m1);
        const float s0 = mx == -INFINITY ? 0.f : fast_exp2(m0 - mx), s1 = mx == -INFINITY ? 0.f : fast_exp2(m1 - mx);
        Mh[j][v] = mx;
        Lh[j][v] = Lh[j][v] * s0 + l1 * s1;
#pragma unroll
        for (int n = 0; n < 8; ++n) O[j][n][v] = O[j][n][v] * s0 + ho[hr * OSTR + 16 * n + col] * s1;
      }
  }

  if (a.n_splits == 1) {
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

// ------------------------------------------------------------------ decode and dense queries
//
// One workgroup per (query, split); a split is a run of 64-key blocks taken
// one per round, the next block's gather in flight in registers during this
// block's math. The HG waves are head groups, as in the chunk kernel above, so
// one gathered block serves all 16 HG NTW heads. A decode query's workgroups
// take one block each (the gathers of a query's blocks run side by side on as
// many CUs, which is what bounds this latency-bound step; a wide batch takes
// two); a dense query's take a few rounds each, so that the merge combines at
// most kAttDenseSplits partials. The split's softmax state (m, l, O) goes out
// straight from the MFMA accumulators: the output when the query has one
// split, else the partial state that attend_merge_kernel combines.

template <int SD> __device__ __forceinline__ constexpr int cpr_of() { return row_bytes_of<SD>() / 16; }

// 16 bytes of a stored row -> its values as bf16, packed two per 32-bit word
// (E / 8 16-byte words: bf16 1, fp8 2, fp4 4). fp4: the chunk's two
// 16-channel groups take the E4M3 scale codes in bytes 0 and 1 of gsc
// (E2M1 x E4M3 products are exact in bf16).
template <int SD>
__device__ __forceinline__ void pack_bf16(const uint4 &u, uint32_t gsc, uint4 *dst) {
  if constexpr (SD == DT_BF16) {
    dst[0] = u;
  } else if constexpr (SD == DT_FP8) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16<false>(w[q]));
      o[2 * q + 1] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16<true>(w[q]));
    }
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
    static_assert(SD == DT_FP4, "bf16, fp8 or fp4 storage");
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const float s0 = e4m3_to_f32(gsc & 0xffu), s1 = e4m3_to_f32((gsc >> 8) & 0xffu);
    uint32_t o[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sc = q < 2 ? s0 : s1;
      const f32x2_t v0 = fp4x2_to_f32<0>(w[q]), v1 = fp4x2_to_f32<1>(w[q]);
      const f32x2_t v2 = fp4x2_to_f32<2>(w[q]), v3 = fp4x2_to_f32<3>(w[q]);
      o[4 * q + 0] = f32x2_to_bf16x2(v0[0] * sc, v0[1] * sc);
      o[4 * q + 1] = f32x2_to_bf16x2(v1[0] * sc, v1[1] * sc);
      o[4 * q + 2] = f32x2_to_bf16x2(v2[0] * sc, v2[1] * sc);
      o[4 * q + 3] = f32x2_to_bf16x2(v3[0] * sc, v3[1] * sc);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
  }
}

// Two waves per SIMD at most (amdgpu_waves_per_eu), so the compiler may give
// each wave up to 256 registers instead of spilling.
template <int KV, int RS, int HG, int NTW>
__global__ __launch_bounds__(HG * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void attend_decode_kernel(const AttendArgs a) {
  using CT = __bf16;
  static_assert(KV != DT_F32, "bf16 compute path");
  constexpr int NT = HG * 64;
  constexpr int H = HG * NTW * 16;
  constexpr bool VSCALE = KV == DT_FP8 || RS == DT_FP8;
  constexpr int64_t PRB = row_bytes_of<KV>(), RRB = row_bytes_of<RS>();
  constexpr int KSTR = kD + 8;                 // K row stride (bf16 elements)
  constexpr int VSTR = kD + 16;                // V row stride: conflict-free transposed reads
  constexpr int KV_LDS = kKeyBlock * (KSTR + VSTR) * 2;
  // 16-byte slots per thread per block of pool (P) and ring (R) rows; a block
  // is held in registers between rounds (prefetched) when its slots fit UW
  constexpr int U_P = 2 * kKeyBlock * cpr_of<KV>() / NT, U_R = 2 * kKeyBlock * cpr_of<RS>() / NT;
  constexpr int UCAP = 8;
  constexpr int UW = (U_P > U_R ? U_P : U_R) < UCAP ? (U_P > U_R ? U_P : U_R) : UCAP;
  constexpr bool PRE_P = U_P <= UW, PRE_R = U_R <= UW;

  __shared__ __align__(16) char kv_lds[KV_LDS];
  __shared__ __align__(16) uint32_t off_t[kAttSplitMaxKeys];   // byte offset of every key (kOobOffset: none)
  __shared__ __align__(16) float kmul[VSCALE ? kKeyBlock : 1];
  __shared__ __align__(16) float kbias[VSCALE ? kKeyBlock : 1];
  __shared__ __align__(16) float vscl[VSCALE ? kKeyBlock : 1];
  __shared__ uint64_t kmask;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave;                         // head group (wave-uniform)
  const int g = lane >> 4, col = lane & 15;
  const int qi = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
  const int seq = a.qd[qi].seq, t = a.qd[qi].pos;
  const int n_vis = (t + 1) / a.r;
  const int swa_lo = max(a.qd[qi].swa, t - a.W + 1);
  const int b_begin = split * a.blocks_per_split;
  const int b_end = min(a.n_blocks, b_begin + a.blocks_per_split);
  const int n_keys = (b_end - b_begin) * kKeyBlock;
  const int32_t *bt = a.block_table + static_cast<int64_t>(seq) * a.bt_stride;
  const int32_t *trow = a.dense ? nullptr : a.topk + static_cast<int64_t>(qi) * a.k;

  // queries first: their loads overlap the key resolution
  Frag<CT> qf[NTW][4];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int head = 16 * (hg + HG * j) + col;
    const char *qrow = reinterpret_cast<const char *>(a.q) + (static_cast<int64_t>(qi) * H + head) * kD * 2;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[j][c] = LoadFrag<DT_BF16, CT>::load(qrow + (32 * g + 8 * c) * 2);
  }

  // ---------------- resolve every key of the split to a row offset (Top-K
  // entry -> page through the block table, window row -> ring slot)
  for (int i = tid; i < n_keys; i += NT) {
    const int b = b_begin + (i >> 6), kk = i & 63;
    uint32_t off = kOobOffset;
    if (b < a.n_sparse_blocks) {
      const int slot = b * kKeyBlock + kk;
      const int j = a.dense ? (slot < n_vis ? slot : -1) : (slot < a.k ? trow[slot] : -1);
      if (j >= n_vis) {
        flag_error(a.err, ERR_TOPK);
      } else if (j >= 0) {
        const int pp = bt[j >> 6];
        if (pp >= 0 && pp < a.pool_pages) off = static_cast<uint32_t>(pp * kPage + (j & 63)) * static_cast<uint32_t>(PRB);
        else flag_error(a.err, ERR_PAGE);
      }
    } else {
      const int row = swa_lo + (b - a.n_sparse_blocks) * kKeyBlock + kk;
      if (row <= t) off = static_cast<uint32_t>(seq * a.R + row % a.R) * static_cast<uint32_t>(RRB);
    }
    off_t[i] = off;
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t pool_k = buffer_of(a.kbar, a.pool_bytes), pool_v = buffer_of(a.vbar, a.pool_bytes);
  const __amdgpu_buffer_rsrc_t ring_k = buffer_of(a.ring_k, a.ring_bytes), ring_v = buffer_of(a.ring_v, a.ring_bytes);
  CT *Ks = reinterpret_cast<CT *>(kv_lds);
  CT *Vs = Ks + kKeyBlock * KSTR;

  // a block's 16-byte slots in registers, one array per row kind (pool rows
  // of the Top-K blocks, ring rows of the window blocks): one array written
  // along two paths of different widths would be demoted to scratch
  constexpr int WP = U_P < UW ? U_P : UW, WR = U_R < UW ? U_R : UW;
  uint4 rawp[WP], rawr[WR];
  uint32_t graw[KV == DT_FP4 ? WP : 1];
  float ks_pref = 1.f, vs_pref = 1.f;
  // slots [u0, u0 + W) of block b (pool rows when POOL): slot u of
  // thread tid is chunk tid % CPR of key ((u NT + tid) mod 64 CPR) / CPR, of K for
  // the first 64 CPR slots and of V for the next
  auto gather = [&](auto pool_tag, int b, int u0) {
    constexpr bool POOL = decltype(pool_tag)::value;
    constexpr int SD = POOL ? KV : RS;
    constexpr int CPR = cpr_of<SD>();
    constexpr int W = POOL ? WP : WR;
    uint4 *raw = POOL ? rawp : rawr;
    const __amdgpu_buffer_rsrc_t rk = POOL ? pool_k : ring_k, rv = POOL ? pool_v : ring_v;
    const uint32_t *offs = off_t + (b - b_begin) * kKeyBlock;
    const uint32_t chunk_off = static_cast<uint32_t>(tid & (CPR - 1)) * 16u;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int u = u0 + w;
      if (u * NT >= 2 * kKeyBlock * CPR) break;
      const bool is_v = u * NT >= kKeyBlock * CPR;
      const uint32_t row_off = offs[((u * NT) % (kKeyBlock * CPR) + tid) / CPR];
      raw[w] = buffer_load16(is_v ? rv : rk, row_off + chunk_off);
      if constexpr (KV == DT_FP4 && POOL) {
        const uint8_t *gbase = is_v ? a.vbar_gs : a.kbar_gs;
        const uint32_t goff = row_off >= kOobOffset ? kOobOffset : (row_off >> 3) + chunk_off / 8u;
        graw[w] = __builtin_amdgcn_raw_buffer_load_b16(buffer_of(gbase, a.gs_bytes), goff, 0, 0);
      }
    }
  };
  auto load_scales = [&](int b) {
    ks_pref = vs_pref = 1.f;
    if (tid < kKeyBlock) {
      const uint32_t off = off_t[(b - b_begin) * kKeyBlock + tid];
      if constexpr (KV == DT_FP8) {
        if (b < a.n_sparse_blocks && off != kOobOffset) {
          const uint32_t page = off / static_cast<uint32_t>(PRB * kPage);
          ks_pref = a.kbar_scale[page];
          vs_pref = a.vbar_scale[page];
        }
      }
      if constexpr (RS == DT_FP8) {
        if (b >= a.n_sparse_blocks && off != kOobOffset) {
          const uint32_t row = off / static_cast<uint32_t>(RRB);
          ks_pref = a.ring_k_scale[row];
          vs_pref = a.ring_v_scale[row];
        }
      }
    }
  };
  auto commit = [&](auto pool_tag, int u0) {
    constexpr bool POOL = decltype(pool_tag)::value;
    constexpr int SD = POOL ? KV : RS;
    constexpr int E = SD == DT_FP4 ? 32 : 16 / elem_bytes_of<SD>();
    constexpr int CPR = kD / E;
    constexpr int W = POOL ? WP : WR;
    const uint4 *raw = POOL ? rawp : rawr;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int u = u0 + w;
      if (u * NT >= 2 * kKeyBlock * CPR) break;
      const bool is_v = u * NT >= kKeyBlock * CPR;
      const int key = ((u * NT) % (kKeyBlock * CPR) + tid) / CPR, d0 = (tid & (CPR - 1)) * E;
      uint4 packed[E / 8];
      pack_bf16<SD>(raw[w], KV == DT_FP4 && POOL ? graw[KV == DT_FP4 ? w : 0] : 0u, packed);
      uint4 *dst = reinterpret_cast<uint4 *>(is_v ? Vs + key * VSTR + d0 : Ks + key * KSTR + d0);
#pragma unroll
      for (int q = 0; q < E / 8; ++q) dst[q] = packed[q];
    }
  };
  using PoolTag = std::integral_constant<bool, true>;
  using RingTag = std::integral_constant<bool, false>;
  auto load_round = [&](int r) {
    const int b = b_begin + r;
    if (b >= b_end) return;
    if (b < a.n_sparse_blocks) {
      if constexpr (PRE_P) gather(PoolTag{}, b, 0);
    } else {
      if constexpr (PRE_R) gather(RingTag{}, b, 0);
    }
    load_scales(b);
  };
  // rows too wide to be held for a whole block: gather and commit W slots at a time
  auto slices = [&](auto pool_tag, int b) {
    constexpr bool POOL = decltype(pool_tag)::value;
    constexpr int US = POOL ? U_P : U_R;
    constexpr int W = POOL ? WP : WR;
#pragma unroll
    for (int u0 = 0; u0 < US; u0 += W) {
      gather(pool_tag, b, u0);
      commit(pool_tag, u0);
    }
  };
  auto commit_round = [&](int r) {
    const int b = b_begin + r;
    if (b >= b_end) return;
    if (b < a.n_sparse_blocks) {
      if constexpr (PRE_P) commit(PoolTag{}, 0);
      else slices(PoolTag{}, b);
    } else {
      if constexpr (PRE_R) commit(RingTag{}, 0);
      else slices(RingTag{}, b);
    }
    if (tid < kKeyBlock) {   // the first wave
      const bool valid = off_t[(b - b_begin) * kKeyBlock + tid] != kOobOffset;
      if constexpr (VSCALE) {
        kmul[tid] = valid ? a.scale * kLog2e * ks_pref : 0.f;
        kbias[tid] = valid ? 0.f : -INFINITY;
        vscl[tid] = vs_pref;
      } else {
        const uint64_t m = __builtin_amdgcn_ballot_w64(valid);
        if (tid == 0) kmask = m;
      }
    }
  };

  f32x4_t O[NTW][8];
  float m_run[NTW], l_run[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
#pragma unroll
    for (int n = 0; n < 8; ++n) O[j][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }

  const int n_rounds = b_end - b_begin;
  load_round(0);
  for (int r = 0; r < n_rounds; ++r) {
    if (r > 0) __syncthreads();          // previous round's LDS reads are done
    commit_round(r);
    __syncthreads();
    if (r + 1 < n_rounds) load_round(r + 1);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      // S^T tiles: keys as MFMA rows, the wave's 16 heads as columns
      f32x4_t S[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        Frag<CT> kf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[c] = LoadFrag<DT_BF16, CT>::load(Ks + (16 * kt + col) * KSTR + 32 * g + 8 * c);
        S[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) S[kt] = mma(kf[c], qf[j][c], S[kt]);
      }
      // logits in log2 units of the lane's keys 16 kt + 4 g + v, masked keys -inf
      float bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if constexpr (VSCALE) {
          const float4 km = *reinterpret_cast<const float4 *>(&kmul[16 * kt + 4 * g]);
          const float4 kb = *reinterpret_cast<const float4 *>(&kbias[16 * kt + 4 * g]);
          S[kt][0] = fmaf(S[kt][0], km.x, kb.x); S[kt][1] = fmaf(S[kt][1], km.y, kb.y);
          S[kt][2] = fmaf(S[kt][2], km.z, kb.z); S[kt][3] = fmaf(S[kt][3], km.w, kb.w);
        } else {
          const float c = a.scale * kLog2e;
          const uint32_t nib = static_cast<uint32_t>(kmask >> (16 * kt + 4 * g)) & 0xfu;
#pragma unroll
          for (int v = 0; v < 4; ++v) S[kt][v] = (nib >> v) & 1u ? S[kt][v] * c : -INFINITY;
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) bm = fmaxf(bm, S[kt][v]);
      }
      bm = max_xor32(max_xor16(bm));
      // lazily rescaled online softmax: O and l move to a new reference max
      // only when a head's block max exceeds it by more than kRescale
      if (__builtin_amdgcn_ballot_w64(bm > m_run[j] + kRescale) != 0) {
        const float m_new = fmaxf(m_run[j], bm);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[j] - m_new);
        l_run[j] *= alpha;
        m_run[j] = m_new;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
          for (int n = 0; n < 8; ++n) O[j][n][v] *= av;
        }
      }
      const float m_ref = m_run[j] == -INFINITY ? 0.f : m_run[j];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          S[kt][v] = fast_exp2(S[kt][v] - m_ref);
          psum += S[kt][v];
        }
      l_run[j] += psum;
      // O += P . V: heads as rows, keys contracted, V fragments by transposed reads
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float pv[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[v] = S[2 * kc][v];
          pv[4 + v] = S[2 * kc + 1][v];
        }
        if constexpr (VSCALE) {
          const float4 s0 = *reinterpret_cast<const float4 *>(&vscl[32 * kc + 4 * g]);
          const float4 s1 = *reinterpret_cast<const float4 *>(&vscl[32 * kc + 16 + 4 * g]);
          pv[0] *= s0.x; pv[1] *= s0.y; pv[2] *= s0.z; pv[3] *= s0.w;
          pv[4] *= s1.x; pv[5] *= s1.y; pv[6] *= s1.z; pv[7] *= s1.w;
        }
        const Frag<CT> pf = frag_from_f32(pv, static_cast<Frag<CT> *>(nullptr));
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const CT *vr = Vs + (32 * kc + 4 * g + (col >> 2)) * VSTR + 16 * n + 4 * (col & 3);
          const uint2 lo = lds_read_tr16(vr);
          const uint2 hi = lds_read_tr16(vr + 16 * VSTR);
          Frag<CT> vf;
          vf.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          O[j][n] = mma(pf, vf, O[j][n]);
        }
      }
    }
  }

  // the state goes out straight from the MFMA accumulators
  // (lane (g, col) holds dims 16 n + col of heads 4 g + v)
  const int64_t pb = static_cast<int64_t>(qi) * a.n_splits + split;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const float l_tot = sum_xor32(sum_xor16(l_run[j]));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * (hg + HG * j) + 4 * g + v;
      if (a.n_splits == 1) {
        const float lv = __shfl(l_tot, 4 * g + v, 64);
        const float inv = lv > 0.f ? 1.f / lv : 0.f;
        uint16_t *dst = reinterpret_cast<uint16_t *>(a.out) + (static_cast<int64_t>(qi) * H + h) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) dst[16 * n + col] = f32_to_bf16(O[j][n][v] * inv);
      } else {
        float *dst = a.part_o + (pb * H + h) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) dst[16 * n + col] = O[j][n][v];
      }
    }
    if (a.n_splits > 1 && g == 0) {
      const int h = 16 * (hg + HG * j) + col;
      a.part_ml[(pb * 2 + 0) * H + h] = m_run[j];
      a.part_ml[(pb * 2 + 1) * H + h] = l_tot;
    }
  }
}

// Combines the split partials of (query, head): one softmax over the union of
// every split's keys. Thread d owns output dimension d. Threads s < MS load
// split s's (m, l) with one vector load each and stage them through LDS; the
// partial loads take a clamped split index instead of a guard, so every load
// is issued unconditionally and the merge costs about one memory round trip
// (a split past the query's count repeats the last one with weight 0).
template <int ACT, int MS>
__global__ __launch_bounds__(kD) void attend_merge_kernel(const AttendArgs a) {
  const int qi = blockIdx.x / a.H, h = blockIdx.x % a.H, d = threadIdx.x;
  const int n = a.n_splits;
  const int64_t q0 = static_cast<int64_t>(qi) * n;
  static_assert(MS <= kD, "one thread per split stages (m, l)");
  __shared__ float ms_st[MS], ls_st[MS];
  const float *ml = a.part_ml + q0 * 2 * a.H + h;               // split s: m at [2 s H], l at [(2 s + 1) H]
  const float *po = a.part_o + (q0 * a.H + h) * kD + d;         // split s at [s H kD]
  const int sd = min(d, n - 1), HD = a.H * kD;
  const float mv = ml[2 * sd * a.H], lv = ml[(2 * sd + 1) * a.H];
  float o[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) o[s] = po[min(s, n - 1) * HD];
  if (d < MS) {
    ms_st[d] = d < n ? mv : -INFINITY;
    ls_st[d] = d < n ? lv : 0.f;
  }
  __syncthreads();
  float m[MS], l[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    m[s] = ms_st[s];
    l[s] = ls_st[s];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s) mx = fmaxf(mx, m[s]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const float e = (m[s] == -INFINITY) ? 0.f : fast_exp2(m[s] - mx);   // running maxima are in log2 units
    L += e * l[s];
    acc += e * o[s];
  }
  const float out = L > 0.f ? acc / L : 0.f;
  const int64_t oi = (static_cast<int64_t>(qi) * a.H + h) * kD + d;
  if constexpr (ACT == DT_F32) reinterpret_cast<float *>(a.out)[oi] = out;
  else reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16(out);
}

template <int ACT, int KV, int RS>
void launch_attend_t(const AttendArgs &a, int n_wg, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (a.H) {
    // 16 heads: two waves, each on half of every block's keys; more heads:
    // one wave per 16-head tile (two tiles for 128), every wave on all keys
    case 16: hipExtLaunchKernelGGL((attend_kernel<ACT, KV, RS, 1, 1, 2>), dim3(n_wg), dim3(128), 0, s, e0, e1, 0, a); break;
    case 32: hipExtLaunchKernelGGL((attend_kernel<ACT, KV, RS, 2, 1, 1>), dim3(n_wg), dim3(128), 0, s, e0, e1, 0, a); break;
    case 64: hipExtLaunchKernelGGL((attend_kernel<ACT, KV, RS, 4, 1, 1>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a); break;
    case 128: hipExtLaunchKernelGGL((attend_kernel<ACT, KV, RS, 4, 2, 1>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a); break;
    default: break;
  }
}

template <int KV, int RS>
void launch_attend_decode_t(const AttendArgs &a, int n_wg, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (a.H) {
    case 16: hipExtLaunchKernelGGL((attend_decode_kernel<KV, RS, 1, 1>), dim3(n_wg), dim3(64), 0, s, e0, e1, 0, a); break;
    case 32: hipExtLaunchKernelGGL((attend_decode_kernel<KV, RS, 2, 1>), dim3(n_wg), dim3(128), 0, s, e0, e1, 0, a); break;
    case 64: hipExtLaunchKernelGGL((attend_decode_kernel<KV, RS, 4, 1>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a); break;
    case 128: hipExtLaunchKernelGGL((attend_decode_kernel<KV, RS, 4, 2>), dim3(n_wg), dim3(256), 0, s, e0, e1, 0, a); break;
    default: break;
  }
}

// The same combination for queries with at most MS splits, 8 (query, head)
// pairs per workgroup: 32 threads per pair, each owning 4 contiguous output
// dims (16-byte partial loads, all issued before the first use). Eight times
// fewer workgroups than one per pair: at these sizes the launch of the many
// small workgroups, not the loads, set the merge's time.
template <int ACT, int MS>
__global__ __launch_bounds__(256) void attend_merge_wide_kernel(const AttendArgs a) {
  const int tid = threadIdx.x;
  const int pair = blockIdx.x * 8 + (tid >> 5);
  if (pair >= a.n_q * a.H) return;   // no barriers below
  const int qi = pair / a.H, h = pair - qi * a.H, d0 = 4 * (tid & 31);
  const int n = a.n_splits;
  const int64_t q0 = static_cast<int64_t>(qi) * n;
  float m[MS], l[MS];
  float4 o[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const bool ok = s < n;
    m[s] = ok ? a.part_ml[((q0 + s) * 2 + 0) * a.H + h] : -INFINITY;
    l[s] = ok ? a.part_ml[((q0 + s) * 2 + 1) * a.H + h] : 0.f;
    o[s] = ok ? *reinterpret_cast<const float4 *>(a.part_o + ((q0 + s) * a.H + h) * kD + d0)
              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s) mx = fmaxf(mx, m[s]);
  float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const float e = (m[s] == -INFINITY) ? 0.f : fast_exp2(m[s] - mx);   // running maxima are in log2 units
    L += e * l[s];
    acc[0] += e * o[s].x; acc[1] += e * o[s].y; acc[2] += e * o[s].z; acc[3] += e * o[s].w;
  }
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = L > 0.f ? acc[i] / L : 0.f;
  const int64_t oi = (static_cast<int64_t>(qi) * a.H + h) * kD + d0;
  if constexpr (ACT == DT_F32)
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + oi) = make_float4(r[0], r[1], r[2], r[3]);
  else
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + oi) =
        make_uint2(f32x2_to_bf16x2(r[0], r[1]), f32x2_to_bf16x2(r[2], r[3]));
}


// Merge kernels: with at least 1,024 (query, head) pairs and up to 24 splits,
// 8 pairs per workgroup; otherwise one workgroup per pair (measured faster
// when the pairs are few: 256 pairs of 18 splits), with (m, l) in registers
// up to 40 splits and staged through LDS beyond. Each kernel is unrolled for
// the smallest split count MS >= the query's: the guarded loads of unused
// splits still cost issue slots (44 splits: 5.1 us at MS = 80, 4.3 at 48).
template <int ACT>
void launch_merge_t(const AttendArgs &a, hipStream_t s) {
  const int n = a.n_splits;
  const dim3 grid(a.n_q * a.H), block(kD);
  const dim3 grid_w((a.n_q * a.H + 7) / 8), block_w(256);
  if (a.n_q * a.H >= 1024 && n <= 24) {
    if (n <= 8) hipLaunchKernelGGL((attend_merge_wide_kernel<ACT, 8>), grid_w, block_w, 0, s, a);
    else hipLaunchKernelGGL((attend_merge_wide_kernel<ACT, 24>), grid_w, block_w, 0, s, a);
  } else if (n <= 8) {
    hipLaunchKernelGGL((attend_merge_kernel<ACT, 8>), grid, block, 0, s, a);
  } else if (n <= 24) {
    hipLaunchKernelGGL((attend_merge_kernel<ACT, 24>), grid, block, 0, s, a);
  } else if (n <= 40) {
    hipLaunchKernelGGL((attend_merge_kernel<ACT, 40>), grid, block, 0, s, a);
  } else if (n <= 48) {
    hipLaunchKernelGGL((attend_merge_kernel<ACT, 48>), grid, block, 0, s, a);
  } else if (n <= 64) {
    hipLaunchKernelGGL((attend_merge_kernel<ACT, 64>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((attend_merge_kernel<ACT, kAttMaxSplits>), grid, block, 0, s, a);
  }
}

void launch_merge(const AttendArgs &a, hipStream_t s) {
  if (a.n_splits <= 1) return;
  if (a.act_f32) launch_merge_t<DT_F32>(a, s);
  else launch_merge_t<DT_BF16>(a, s);
}

}  // namespace

void launch_attend_decode(const AttendArgs &a, int n_wg, int kv, bool ring_fp8, hipStream_t s, hipEvent_t ev0,
                          hipEvent_t ev1) {
  if (n_wg <= 0) return;
  if (kv == DT_BF16 && !ring_fp8) launch_attend_decode_t<DT_BF16, DT_BF16>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_BF16) launch_attend_decode_t<DT_BF16, DT_FP8>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP8 && !ring_fp8) launch_attend_decode_t<DT_FP8, DT_BF16>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP8) launch_attend_decode_t<DT_FP8, DT_FP8>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP4 && !ring_fp8) launch_attend_decode_t<DT_FP4, DT_BF16>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP4) launch_attend_decode_t<DT_FP4, DT_FP8>(a, n_wg, s, ev0, ev1);
  launch_merge(a, s);
}

void launch_attend(const AttendArgs &a, int n_wg, int kv, int act, bool ring_fp8, hipStream_t s, hipEvent_t ev0,
                   hipEvent_t ev1) {
  if (n_wg <= 0) return;
  if (kv == DT_F32 && act == DT_F32) launch_attend_t<DT_F32, DT_F32, DT_F32>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_BF16 && act == DT_BF16 && !ring_fp8) launch_attend_t<DT_BF16, DT_BF16, DT_BF16>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_BF16 && act == DT_BF16) launch_attend_t<DT_BF16, DT_BF16, DT_FP8>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP8 && act == DT_BF16 && !ring_fp8) launch_attend_t<DT_BF16, DT_FP8, DT_BF16>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP8 && act == DT_BF16) launch_attend_t<DT_BF16, DT_FP8, DT_FP8>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP4 && act == DT_BF16 && !ring_fp8) launch_attend_t<DT_BF16, DT_FP4, DT_BF16>(a, n_wg, s, ev0, ev1);
  else if (kv == DT_FP4 && act == DT_BF16) launch_attend_t<DT_BF16, DT_FP4, DT_FP8>(a, n_wg, s, ev0, ev1);
  launch_merge(a, s);
}

}  // namespace csa
