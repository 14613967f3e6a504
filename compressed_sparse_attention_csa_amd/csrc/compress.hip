// csa_compress kernels: gated pooling of r raw rows into one compressed entry,
// indexer-key projection, and the page write (with per-page FP8 scaling).
//
// Method: Model-architectures atlas, compressed-KV entry (every r KV rows
// folded into one entry with learned compression weights); DeepSeek-V4.1-Flash
// technical-report walkthrough, "Compressed Sparse Attention 2" > "A simpler
// compressor" (non-overlapping groups, no absolute positional embedding,
// indexer K projected from the main-KV entry) and "Causal Encoder-Decoder" >
// "One hidden state feeds the decoder" (entries C and compression weights Z).
//
// One workgroup owns one (sequence, page) - for fp32 and bf16 pages, one of
// its 8-slot parts: it computes the new entries in fp32, then writes them. For FP8 pages it also re-quantises the page's
// earlier entries (kept in fp32 staging) under the page's new amax, so the
// bytes of a page never depend on how its entries were appended.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

template <int ACT>
__device__ __forceinline__ float2 load2(const void *base, int64_t elem) {
  if constexpr (ACT == DT_F32) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(base) + elem);
  } else {
    uint32_t w = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(base) + elem);
    return make_float2(bf16_to_f32(static_cast<uint16_t>(w & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(w >> 16)));
  }
}

template <int KV>
__device__ __forceinline__ void store2(void *base, int64_t elem, float a, float b) {
  if constexpr (KV == DT_F32) {
    *reinterpret_cast<float2 *>(reinterpret_cast<float *>(base) + elem) = make_float2(a, b);
  } else if constexpr (KV == DT_BF16) {
    uint32_t w = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(base) + elem) = w;
  }
}

template <int KV>
__device__ __forceinline__ void store1(void *base, int64_t elem, float a) {
  if constexpr (KV == DT_F32) {
    reinterpret_cast<float *>(base)[elem] = a;
  } else if constexpr (KV == DT_BF16) {
    reinterpret_cast<uint16_t *>(base)[elem] = f32_to_bf16(a);
  }
}

// The item a workgroup belongs to: the last one whose first workgroup is <= wg
// (a binary search over the launcher's prefix, log2(items) dependent loads).
__device__ __forceinline__ int item_of(const int32_t *wg0, int n_items, int wg) {
  int lo = 0, hi = n_items;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (wg0[mid] <= wg) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kThreads = 256;
constexpr int kPageParts = 8;   // workgroups per fp32 / bf16 page

// fp32 / bf16 pages: each page is split over kPageParts workgroups of SPW
// slots; fp8 and fp4 pages need a page-wide amax and stay whole
template <int KV> constexpr int page_parts() { return (KV == DT_F32 || KV == DT_BF16) ? kPageParts : 1; }

// The workgroup's share of one (sequence, page): slots [slot0, slot0 + SPW) of
// page `page` of item `it`.
template <int ACT, int KV>
__device__ void compress_page(const CompressArgs &a, const CompressItem &it, int page, int slot0) {
  constexpr int PARTS = page_parts<KV>();
  constexpr int SPW = kPage / PARTS, SPT = SPW / (kThreads / 64);   // slots per workgroup / thread
  __shared__ float kb_s[SPW][kD];
  __shared__ float p_s[kD][kDI];   // indexer projection, staged once
  __shared__ float red[48];

  const int seq = it.seq;
  const int r = a.r;
  const int new_len = it.old_len + it.n_new;
  const int nb_old = it.old_len / r, nb_new = new_len / r;
  const int pstart = page * kPage;
  const int e0 = max(pstart, nb_old), e1 = min(pstart + kPage, nb_new);
  const int filled = e1 - pstart;                     // slots [0, filled) hold entries after this call
  const int pp = a.block_table[static_cast<int64_t>(seq) * a.bt_stride + page];
  const bool page_ok = pp >= 0 && pp < a.pool_pages;
  if (!page_ok && threadIdx.x == 0) flag_error(a.err, ERR_PAGE);

  const int t = threadIdx.x, dp = t & 63, eb = t >> 6;
  const int d0 = 2 * dp;
  if (a.write_idx) {
    // 8 independent 16-byte loads per thread
    const float4 *src = reinterpret_cast<const float4 *>(a.proj);
    float4 tmp[kD * kDI / 4 / kThreads];
#pragma unroll
    for (int u = 0; u < kD * kDI / 4 / kThreads; ++u) tmp[u] = src[u * kThreads + t];
#pragma unroll
    for (int u = 0; u < kD * kDI / 4 / kThreads; ++u) reinterpret_cast<float4 *>(&p_s[0][0])[u * kThreads + t] = tmp[u];
  }

  // A row of entry e's block: from the packed input when this call appends it,
  // else from open-block staging (appended by an earlier call).
  auto row_src = [&](int row, int plane, const void *fresh) -> float2 {
    const bool is_new = row >= it.old_len;
    const void *base = is_new ? fresh : a.block_stage;
    const int64_t off = is_new ? static_cast<int64_t>(it.row_off + row - it.old_len) * kD + d0
                               : ((static_cast<int64_t>(seq) * 3 + plane) * r + row % r) * kD + d0;
    return load2<ACT>(base, off);
  };

  float kk[SPT][2], vv[SPT][2];
#pragma unroll
  for (int m = 0; m < SPT; ++m) {
    const int slot = slot0 + eb + 4 * m, e = pstart + slot;   // the same for every lane of a wave
    float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
    if (e >= e0 && e < e1) {
      // gated pooling over rows [e*r, e*r + r): softmax of the gate per channel
      float zm0 = -INFINITY, zm1 = -INFINITY;
#pragma unroll 4
      for (int u = 0; u < r; ++u) {
        const float2 z = row_src(e * r + u, 0, a.gate);
        zm0 = fmaxf(zm0, z.x);
        zm1 = fmaxf(zm1, z.y);
      }
      float ws0 = 0.f, ws1 = 0.f;
#pragma unroll 4
      for (int u = 0; u < r; ++u) {
        const int row = e * r + u;
        const float2 z = row_src(row, 0, a.gate), kx = row_src(row, 1, a.raw_k), vx = row_src(row, 2, a.raw_v);
        const float w0 = expf(z.x - zm0), w1 = expf(z.y - zm1);
        ws0 += w0; ws1 += w1;
        k0 += w0 * kx.x; k1 += w1 * kx.y;
        v0 += w0 * vx.x; v1 += w1 * vx.y;
      }
      k0 /= ws0; k1 /= ws1; v0 /= ws0; v1 /= ws1;
    }
    kk[m][0] = k0; kk[m][1] = k1;
    vv[m][0] = v0; vv[m][1] = v1;
    if (a.write_idx) {
      kb_s[slot - slot0][d0] = k0;
      kb_s[slot - slot0][d0 + 1] = k1;
    }
  }

  // fp8 pages: the fp32 values of the page's earlier entries, from staging,
  // loaded after the new entries' rows (which the pooling above waited for).
  // Every slot of a sequence's staging page is valid memory, so the loads are
  // issued for every slot (all in flight together) and selected afterwards.
  if constexpr (KV == DT_FP8) {
    float2 stk[SPT], stv[SPT];
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      const int64_t so = (static_cast<int64_t>(seq) * kPage + slot0 + eb + 4 * m) * kD + d0;
      stk[m] = *reinterpret_cast<const float2 *>(a.kbar_stage + so);
      stv[m] = *reinterpret_cast<const float2 *>(a.vbar_stage + so);
    }
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      const int slot = slot0 + eb + 4 * m, e = pstart + slot;
      if (slot < filled && e < e0) {   // an entry appended by an earlier call
        kk[m][0] = stk[m].x; kk[m][1] = stk[m].y;
        vv[m][0] = stv[m].x; vv[m][1] = stv[m].y;
      }
    }
  }

  // ---- indexer key: KI = Kbar @ P (fp32, before any rounding); thread owns column c
  const int c = dp;
  float ki[SPT];
#pragma unroll
  for (int m = 0; m < SPT; ++m) ki[m] = 0.f;
  // fp8 indexer keys of earlier entries from staging, issued before the projection
  float sti[SPT];
  if constexpr (KV == DT_FP8 || KV == DT_FP4) {
    if (a.write_idx) {
#pragma unroll
      for (int m = 0; m < SPT; ++m)
        sti[m] = a.kidx_stage[(static_cast<int64_t>(seq) * kPage + slot0 + eb + 4 * m) * kDI + c];
    }
  }
  if (a.write_idx) {
    __syncthreads();
    // new entries only (a slot is new for every lane of its wave or for none):
    // an earlier entry's key comes from staging (fp8 keys) or is not rewritten
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      const int e = pstart + slot0 + eb + 4 * m;
      if (e >= e0 && e < e1) {
        const float *kr = &kb_s[eb + 4 * m][0];
        // four partial sums (d mod 4) shorten the dependent chain
        float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll 8
        for (int d = 0; d < kD; d += 4) {
          const float4 k4 = *reinterpret_cast<const float4 *>(kr + d);
          acc0 += k4.x * p_s[d][c];
          acc1 += k4.y * p_s[d + 1][c];
          acc2 += k4.z * p_s[d + 2][c];
          acc3 += k4.w * p_s[d + 3][c];
        }
        ki[m] = (acc0 + acc1) + (acc2 + acc3);
      }
    }
    if constexpr (KV == DT_FP8 || KV == DT_FP4) {   // fp8 indexer keys
#pragma unroll
      for (int m = 0; m < SPT; ++m) {
        const int slot = slot0 + eb + 4 * m, e = pstart + slot;
        if (slot < filled && e < e0) ki[m] = sti[m];
      }
    }
  }

  const int64_t kv_page = static_cast<int64_t>(pp) * kPage * kD;
  const int64_t ki_page = static_cast<int64_t>(pp) * kPage * kDI;

  if constexpr (KV == DT_FP4) {
    // ---- FP4 K/V: every entry on its own, one E4M3 scale amax/6 per 16
    // channels (8 lanes of a wave); only the new entries are written
    uint8_t *kp = reinterpret_cast<uint8_t *>(a.kbar) + static_cast<int64_t>(pp) * kPage * (kD / 2);
    uint8_t *vp = reinterpret_cast<uint8_t *>(a.vbar) + static_cast<int64_t>(pp) * kPage * (kD / 2);
    uint8_t *kg = a.kbar_gs + static_cast<int64_t>(pp) * kPage * (kD / kFp4Group);
    uint8_t *vg = a.vbar_gs + static_cast<int64_t>(pp) * kPage * (kD / kFp4Group);
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      const int slot = slot0 + eb + 4 * m, e = pstart + slot;
      float mk = fmaxf(fabsf(kk[m][0]), fabsf(kk[m][1]));
      float mv = fmaxf(fabsf(vv[m][0]), fabsf(vv[m][1]));
#pragma unroll
      for (int o = 1; o < kFp4Group / 2; o <<= 1) {
        mk = fmaxf(mk, __shfl_xor(mk, o, 64));
        mv = fmaxf(mv, __shfl_xor(mv, o, 64));
      }
      const uint32_t gk = f32_to_e4m3(mk / 6.0f), gv = f32_to_e4m3(mv / 6.0f);
      const float sk = e4m3_to_f32(gk), sv = e4m3_to_f32(gv);
      const uint32_t ck = sk > 0.f ? f32_to_e2m1(kk[m][0] / sk) | (f32_to_e2m1(kk[m][1] / sk) << 4) : 0u;
      const uint32_t cv = sv > 0.f ? f32_to_e2m1(vv[m][0] / sv) | (f32_to_e2m1(vv[m][1] / sv) << 4) : 0u;
      if (page_ok && e >= e0 && e < e1) {
        kp[slot * (kD / 2) + dp] = static_cast<uint8_t>(ck);
        vp[slot * (kD / 2) + dp] = static_cast<uint8_t>(cv);
        if ((dp & (kFp4Group / 2 - 1)) == 0) {
          kg[slot * (kD / kFp4Group) + dp / (kFp4Group / 2)] = static_cast<uint8_t>(gk);
          vg[slot * (kD / kFp4Group) + dp / (kFp4Group / 2)] = static_cast<uint8_t>(gv);
        }
      }
    }
    if (!a.write_idx) return;
    // ---- FP8 indexer keys: one scale per page, amax over the filled slots
    float ai = 0.f;
#pragma unroll
    for (int m = 0; m < SPT; ++m)
      if (slot0 + eb + 4 * m < filled) ai = fmaxf(ai, fabsf(ki[m]));
    ai = block_max(ai, red + 8);
    const float si = ai > 0.f ? ai / 448.0f : 1.0f;
    if (page_ok) {
      uint8_t *ip = reinterpret_cast<uint8_t *>(a.kidx) + ki_page;
#pragma unroll
      for (int m = 0; m < SPT; ++m) {
        const int slot = slot0 + eb + 4 * m;
        if (slot < filled) ip[slot * kDI + c] = static_cast<uint8_t>(f32_to_e4m3(ki[m] / si));
      }
      if (threadIdx.x == 0) a.kidx_scale[pp] = si;
    }
    if (filled < kPage) {
#pragma unroll
      for (int m = 0; m < SPT; ++m) {
        const int slot = slot0 + eb + 4 * m, e = pstart + slot;
        if (e >= e0 && e < e1) a.kidx_stage[(static_cast<int64_t>(seq) * kPage + slot) * kDI + c] = ki[m];
      }
    }
  } else if constexpr (KV != DT_FP8) {
    if (!page_ok) return;
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      const int slot = slot0 + eb + 4 * m, e = pstart + slot;
      if (e >= e0 && e < e1) {
        store2<KV>(a.kbar, kv_page + slot * kD + d0, kk[m][0], kk[m][1]);
        store2<KV>(a.vbar, kv_page + slot * kD + d0, vv[m][0], vv[m][1]);
        if (a.write_idx) store1<KV>(a.kidx, ki_page + slot * kDI + c, ki[m]);
      }
    }
  } else {
    // ---- FP8: one scale per page and stream, amax over the filled slots
    float ak = 0.f, av = 0.f, ai = 0.f;
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      if (slot0 + eb + 4 * m < filled) {
        ak = fmaxf(ak, fmaxf(fabsf(kk[m][0]), fabsf(kk[m][1])));
        av = fmaxf(av, fmaxf(fabsf(vv[m][0]), fabsf(vv[m][1])));
        ai = fmaxf(ai, fabsf(ki[m]));
      }
    }
    block_max3(ak, av, ai, red);
    const float sk = ak > 0.f ? ak / 448.0f : 1.0f;
    const float sv = av > 0.f ? av / 448.0f : 1.0f;
    const float si = ai > 0.f ? ai / 448.0f : 1.0f;
    const bool open_after = filled < kPage;
    if (page_ok) {
      uint8_t *kp = reinterpret_cast<uint8_t *>(a.kbar) + kv_page;
      uint8_t *vp = reinterpret_cast<uint8_t *>(a.vbar) + kv_page;
      uint8_t *ip = reinterpret_cast<uint8_t *>(a.kidx) + ki_page;
#pragma unroll
      for (int m = 0; m < SPT; ++m) {
        const int slot = slot0 + eb + 4 * m;
        if (slot < filled) {
          const uint32_t ck = f32x2_to_e4m3x2(kk[m][0] / sk, kk[m][1] / sk);
          const uint32_t cv = f32x2_to_e4m3x2(vv[m][0] / sv, vv[m][1] / sv);
          *reinterpret_cast<uint16_t *>(kp + slot * kD + d0) = static_cast<uint16_t>(ck);
          *reinterpret_cast<uint16_t *>(vp + slot * kD + d0) = static_cast<uint16_t>(cv);
          if (a.write_idx) ip[slot * kDI + c] = static_cast<uint8_t>(f32_to_e4m3(ki[m] / si));
        }
      }
      if (threadIdx.x == 0) {
        a.kbar_scale[pp] = sk;
        a.vbar_scale[pp] = sv;
        if (a.write_idx) a.kidx_scale[pp] = si;
      }
    }
    if (open_after) {
#pragma unroll
      for (int m = 0; m < SPT; ++m) {
        const int slot = slot0 + eb + 4 * m, e = pstart + slot;
        if (e >= e0 && e < e1) {
          const int64_t so = (static_cast<int64_t>(seq) * kPage + slot) * kD + d0;
          *reinterpret_cast<float2 *>(a.kbar_stage + so) = make_float2(kk[m][0], kk[m][1]);
          *reinterpret_cast<float2 *>(a.vbar_stage + so) = make_float2(vv[m][0], vv[m][1]);
          if (a.write_idx) a.kidx_stage[(static_cast<int64_t>(seq) * kPage + slot) * kDI + c] = ki[m];
        }
      }
    }
  }
}

template <int ACT, int KV>
__global__ __launch_bounds__(kThreads) void compress_pages_kernel(const CompressArgs a) {
  // which (sequence, page) this workgroup owns: with as many page workgroups
  // as items every item has one page, and the item is the workgroup
  constexpr int PARTS = page_parts<KV>();
  const int wg = blockIdx.x / PARTS;
  const int item = static_cast<int>(gridDim.x) / PARTS == a.n_items ? wg : item_of(a.wg0, a.n_items, wg);
  const CompressItem it = a.it[item];
  compress_page<ACT, KV>(a, it, it.page0 + (wg - a.wg0[item]), (blockIdx.x % PARTS) * (kPage / PARTS));
}

// Copies the newest raw rows into the window ring (as E4M3 codes with one
// fp32 scale amax/448 per row when RING8) and the open r-block's gate, key
// and value rows into block staging. Runs after the page kernel, which still
// reads the previous staging contents for a block straddling two calls.
// Ring and block-staging rows of one item, chunk `chunk` of rows_per_wg rows
// (RA: RingArgs or RingPtrs).
template <int ACT, bool RING8, typename RA>
__device__ void compress_ring_rows(const RA &a, const CompressItem &it, int chunk) {
  const int new_len = it.old_len + it.n_new;
  const int lo = max(it.old_len, new_len - a.R);
  const int glo = a.write_stage ? max(it.old_len, (new_len / a.r) * a.r) : new_len;
  constexpr int kEsz = ACT == DT_F32 ? 4 : 2;
  constexpr int kVec = kD * kEsz / 16;                 // 16-byte vectors per row
  static_assert(64 % kVec == 0, "a row's vectors stay inside one wave");
  const int row_begin = min(lo, glo) + chunk * a.rows_per_wg;
  const int row_end = min(new_len, row_begin + a.rows_per_wg);
  const int n_vec = (row_end - row_begin) * kVec;
  for (int base = 0; base < n_vec; base += blockDim.x) {
    const int v = base + threadIdx.x;
    const bool live = v < n_vec;           // whole rows are live or not (n_vec is a multiple of kVec)
    const int row = row_begin + v / kVec, col = v % kVec;
    const int64_t src = static_cast<int64_t>(it.row_off + row - it.old_len) * kVec + col;
    uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
    if (live) {
      kx = reinterpret_cast<const uint4 *>(a.raw_k)[src];
      vx = reinterpret_cast<const uint4 *>(a.raw_v)[src];
    }
    const int64_t slot = static_cast<int64_t>(it.seq) * a.R + row % a.R;
    if constexpr (RING8) {
      // row scale: amax over the row's kVec lanes (bf16 values are exact in fp32)
      float fk[8], fv[8], mk = 0.f, mv = 0.f;
      const uint32_t wk[4] = {kx.x, kx.y, kx.z, kx.w}, wv[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        fk[2 * q] = bf16_to_f32(static_cast<uint16_t>(wk[q] & 0xffffu));
        fk[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(wk[q] >> 16));
        fv[2 * q] = bf16_to_f32(static_cast<uint16_t>(wv[q] & 0xffffu));
        fv[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(wv[q] >> 16));
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) { mk = fmaxf(mk, fabsf(fk[q])); mv = fmaxf(mv, fabsf(fv[q])); }
#pragma unroll
      for (int o = 1; o < kVec; o <<= 1) {
        mk = fmaxf(mk, __shfl_xor(mk, o, 64));
        mv = fmaxf(mv, __shfl_xor(mv, o, 64));
      }
      const float sk = mk > 0.f ? mk / 448.0f : 1.0f;
      const float sv = mv > 0.f ? mv / 448.0f : 1.0f;
      if (live && row >= lo) {
        uint32_t ck[2] = {0u, 0u}, cv[2] = {0u, 0u};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          ck[q >> 2] |= f32_to_e4m3(fk[q] / sk) << (8 * (q & 3));
          cv[q >> 2] |= f32_to_e4m3(fv[q] / sv) << (8 * (q & 3));
        }
        reinterpret_cast<uint2 *>(a.ring_k)[slot * kVec + col] = make_uint2(ck[0], ck[1]);
        reinterpret_cast<uint2 *>(a.ring_v)[slot * kVec + col] = make_uint2(cv[0], cv[1]);
        if (col == 0) {
          a.ring_k_scale[slot] = sk;
          a.ring_v_scale[slot] = sv;
        }
      }
    } else {
      if (live && row >= lo) {
        reinterpret_cast<uint4 *>(a.ring_k)[slot * kVec + col] = kx;
        reinterpret_cast<uint4 *>(a.ring_v)[slot * kVec + col] = vx;
      }
    }
    if (live && row >= glo) {
      const int64_t dst = ((static_cast<int64_t>(it.seq) * 3) * a.r + row % a.r) * kVec + col;
      const int64_t plane = static_cast<int64_t>(a.r) * kVec;
      uint4 *st = reinterpret_cast<uint4 *>(a.block_stage);
      st[dst] = reinterpret_cast<const uint4 *>(a.gate)[src];
      st[dst + plane] = kx;
      st[dst + 2 * plane] = vx;
    }
  }
}

// One workgroup per item, each writing at most one page and one chunk of ring
// rows (a single-token decode append): the page first, then the ring and
// block-staging rows. The page reads the open block's staged rows before the
// ring part overwrites block staging (the barrier between them), and the
// items are distinct sequences, so workgroups touch disjoint staging. One
// launch instead of the page and ring kernels.
template <int ACT, int KV, bool RING8>
__global__ __launch_bounds__(kThreads) void compress_step_kernel(const CompressArgs a, const RingPtrs rp) {
  static_assert(page_parts<KV>() == 1, "whole pages only");
  const CompressItem it = a.it[blockIdx.x];
  if (it.n_pages > 0) compress_page<ACT, KV>(a, it, it.page0, 0);
  __syncthreads();
  compress_ring_rows<ACT, RING8>(rp, it, 0);
}

template <int ACT, bool RING8>
__global__ __launch_bounds__(256) void compress_ring_kernel(const RingArgs a) {
  const int wg = blockIdx.x;
  const int item = item_of(a.wg0, a.n_items, wg);
  compress_ring_rows<ACT, RING8>(a, a.it[item], wg - a.wg0[item]);
}

}  // namespace

void launch_compress_pages(const CompressArgs &args, int n_wg, int kv, int act, hipStream_t s) {
  if (n_wg <= 0) return;
  CompressArgs a = args;
  a.wg0[0] = 0;
  for (int i = 0; i < a.n_items; ++i) a.wg0[i + 1] = a.wg0[i] + a.it[i].n_pages;
  if (kv == DT_F32 && act == DT_F32)
    hipLaunchKernelGGL((compress_pages_kernel<DT_F32, DT_F32>), dim3(n_wg * kPageParts), dim3(kThreads), 0, s, a);
  else if (kv == DT_BF16 && act == DT_BF16)
    hipLaunchKernelGGL((compress_pages_kernel<DT_BF16, DT_BF16>), dim3(n_wg * kPageParts), dim3(kThreads), 0, s, a);
  else if (kv == DT_FP8 && act == DT_BF16)
    hipLaunchKernelGGL((compress_pages_kernel<DT_BF16, DT_FP8>), dim3(n_wg), dim3(kThreads), 0, s, a);
  else if (kv == DT_FP4 && act == DT_BF16)
    hipLaunchKernelGGL((compress_pages_kernel<DT_BF16, DT_FP4>), dim3(n_wg), dim3(kThreads), 0, s, a);
}

void launch_compress_step(const CompressArgs &a, const RingPtrs &rp, int kv, int act, bool ring_fp8, hipStream_t s) {
  if (a.n_items <= 0 || act != DT_BF16) return;
  const dim3 grid(a.n_items), block(kThreads);
  if (kv == DT_FP8 && ring_fp8) hipLaunchKernelGGL((compress_step_kernel<DT_BF16, DT_FP8, true>), grid, block, 0, s, a, rp);
  else if (kv == DT_FP8) hipLaunchKernelGGL((compress_step_kernel<DT_BF16, DT_FP8, false>), grid, block, 0, s, a, rp);
  else if (kv == DT_FP4 && ring_fp8) hipLaunchKernelGGL((compress_step_kernel<DT_BF16, DT_FP4, true>), grid, block, 0, s, a, rp);
  else if (kv == DT_FP4) hipLaunchKernelGGL((compress_step_kernel<DT_BF16, DT_FP4, false>), grid, block, 0, s, a, rp);
}

void launch_compress_ring(const RingArgs &args, int n_wg, int act, bool ring_fp8, hipStream_t s) {
  if (n_wg <= 0) return;
  RingArgs a = args;
  a.wg0[0] = 0;
  for (int i = 0; i < a.n_items; ++i) a.wg0[i + 1] = a.wg0[i] + a.chunks[i];
  if (act == DT_F32)
    hipLaunchKernelGGL((compress_ring_kernel<DT_F32, false>), dim3(n_wg), dim3(256), 0, s, a);
  else if (ring_fp8)
    hipLaunchKernelGGL((compress_ring_kernel<DT_BF16, true>), dim3(n_wg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((compress_ring_kernel<DT_BF16, false>), dim3(n_wg), dim3(256), 0, s, a);
}

}  // namespace csa
