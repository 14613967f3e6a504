// Device-side building blocks shared by the CSA kernels (gfx950, wave64).
//
// Number formats: bf16 is stored as uint16 bits; fp8 is OCP E4M3 (e4m3fn:
// bias 7, no infinities, max 448) stored as uint8 codes with one fp32 scale
// per 64-entry page.
//
// MFMA fragments: every dot-product tile here uses the 16x16 MFMA shapes
// (bf16 16x16x32, fp32 16x16x4). In both, lane l supplies operand row/column
// l % 16 and the lanes of quarter g = l / 16 supply one quarter of the
// contraction slice; the output element (row 4*g + v, column l % 16) lands in
// accumulator register v of lane l. A contraction is split into "chunks" of 32
// elements and quarter g of chunk c takes 8 contiguous elements starting at
// g * (len / 4) + 8 * c of the full vector; since the A and B operands use the
// same rule, which hardware k-slot a pair lands in does not matter.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_FP4 = 3 };

constexpr int kFp4Group = 16;   // channels sharing one E4M3 scale in an fp4 entry

// error-word bits (see csa_read_errors)
enum : uint32_t { ERR_PAGE = 1u, ERR_TOPK = 2u, ERR_FALLBACK = 4u };

__device__ __forceinline__ void flag_error(uint32_t *err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16: the compiler emits gfx950's
// v_cvt_pk_bf16_f32 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two at once (one v_cvt_pk_bf16_f32): lo in bits 0-15, hi in bits 16-31.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ------------------------------------------------------------------ fp8 e4m3

// Two fp8 codes (byte pair `hi` of a 32-bit word) -> two fp32 values.
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
}

// Two fp8 codes -> two bf16 values (exact: every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI);
}

// fp32 -> E4M3 codes, round-to-nearest-even, saturating to +-448 (NaN
// saturates too): the input is clamped, then gfx950's v_cvt_pk_fp8_f32
// rounds it. The sign bit is the sign of the input (a negative value that
// rounds to zero gives 0x80). Two at once: lo in bits 0-7, hi in bits 8-15.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float lo, float hi) {
  const float a = fminf(fmaxf(lo, -448.0f), 448.0f), b = fminf(fmaxf(hi, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  return f32x2_to_e4m3x2(x, x) & 0xffu;
}

// One E4M3 code (low byte) -> fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return fp8x2_to_f32<false>(code)[0];
}

// ------------------------------------------------------------------ fp4 e2m1

// fp32 -> E2M1 code (bits 0-2 magnitude index of 0, .5, 1, 1.5, 2, 3, 4, 6;
// bit 3 the input's sign): nearest magnitude, a tie going to the even code,
// saturating at 6 (NaN saturates too).
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fabsf(x);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return sign | c;
}

// Two E2M1 codes (byte `SEL` of w: low nibble first) -> two fp32 values, exact
// (gfx950's fp4 conversion with a unit scale).
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(static_cast<int>(w), 1.0f, SEL);
}

// ------------------------------------------------------------------ fragments

// 8 contiguous operand elements of one lane, in the compute type.
template <typename CT> struct Frag;
template <> struct Frag<float> { float v[8]; };
template <> struct Frag<__bf16> { bf16x8_t v; };

__device__ __forceinline__ f32x4_t mma(const Frag<__bf16> &a, const Frag<__bf16> &b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma(const Frag<float> &a, const Frag<float> &b, f32x4_t acc) {
#pragma unroll
  for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[u], b.v[u], acc, 0, 0, 0);
  return acc;
}

// Load 8 contiguous elements of storage dtype SD from p (element pointer) as compute type CT.
template <int SD, typename CT> struct LoadFrag;

template <> struct LoadFrag<DT_F32, float> {
  static __device__ __forceinline__ Frag<float> load(const void *p) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
    float4 a = q[0], b = q[1];
    Frag<float> f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
};
template <> struct LoadFrag<DT_BF16, __bf16> {
  static __device__ __forceinline__ Frag<__bf16> load(const void *p) {
    Frag<__bf16> f;
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    f.v = __builtin_bit_cast(bf16x8_t, u);
    return f;
  }
};
template <> struct LoadFrag<DT_FP8, __bf16> {
  static __device__ __forceinline__ Frag<__bf16> load(const void *p) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    bf16x2_t a = fp8x2_to_bf16<false>(u.x), b = fp8x2_to_bf16<true>(u.x);
    bf16x2_t c = fp8x2_to_bf16<false>(u.y), d = fp8x2_to_bf16<true>(u.y);
    Frag<__bf16> f;
    f.v = bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return f;
  }
};

// Frag from 8 fp32 values (rounded to the compute type).
__device__ __forceinline__ Frag<float> frag_from_f32(const float *x, Frag<float> *) {
  Frag<float> f;
#pragma unroll
  for (int u = 0; u < 8; ++u) f.v[u] = x[u];
  return f;
}
__device__ __forceinline__ Frag<__bf16> frag_from_f32(const float *x, Frag<__bf16> *) {
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) w[u] = f32x2_to_bf16x2(x[2 * u], x[2 * u + 1]);
  Frag<__bf16> f;
  f.v = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
  return f;
}

template <typename CT>
__device__ __forceinline__ Frag<CT> zero_frag() {
  const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  return frag_from_f32(z, static_cast<Frag<CT> *>(nullptr));
}

// ------------------------------------------------------------------ element access

template <int SD> struct Elem;
template <> struct Elem<DT_F32> {
  static constexpr int bytes = 4;
  static __device__ __forceinline__ float get(const void *p, int64_t i) { return reinterpret_cast<const float *>(p)[i]; }
};
template <> struct Elem<DT_BF16> {
  static constexpr int bytes = 2;
  static __device__ __forceinline__ float get(const void *p, int64_t i) {
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
  }
};

// ------------------------------------------------------------------ reductions

// Lane exchange inside each row of 16 lanes by DPP: a register-to-register
// move, where __shfl_xor would go through the LDS crossbar (ds_bpermute).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppSwap1 = 0xb1;        // quad_perm [1,0,3,2]: lane i <- i ^ 1
constexpr int kDppSwap2 = 0x4e;        // quad_perm [2,3,0,1]: lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i of each 8 <- 7 - i (the other quad)
constexpr int kDppRowMirror = 0x140;   // lane i of each 16 <- 15 - i (the other 8)

// Inclusive prefix sum over the 64 lanes in lane order (every lane active):
// shifts by 1, 2, 4 and 8 inside each row of 16 (a lane past its row's start
// adds 0), then row 0's total into row 1 and row 2's into row 3, then rows 0-1's
// total into rows 2 and 3.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// Max over the aligned group of n lanes holding this lane, n in {1, 2, 4, 8,
// 16}; n is the same on every lane, and every lane of the wave is active.
__device__ __forceinline__ float group_max(float v, int n) {
  if (n > 1) v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  if (n > 2) v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  if (n > 4) v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  if (n > 8) v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return v;
}

// Lane i combined with lane i ^ 16 (i ^ 32), on every lane: the permlane swaps
// exchange rows 0 <-> 1 and 2 <-> 3 (halves 0 <-> 1) between two copies of v,
// and the combine is symmetric, so either copy may come first.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max (min) over the 64 lanes, on every lane (every lane active): each row
// of 16 by DPP, then the four row results read as scalars.
__device__ __forceinline__ float wave_max(float v) {
  v = group_max(v, 16);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_min(float v) {
  v = -group_max(-v, 16);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fminf(fminf(r0, r1), fminf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide max of non-negative values over blockDim.x threads (multiple of 64).
__device__ __forceinline__ float block_max(float v, float *scratch /* >= 16 floats of LDS */) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, scratch[i]);
  return r;
}

// Block-wide maxima of three values at once (two barriers instead of six).
__device__ __forceinline__ void block_max3(float &a, float &b, float &c, float *scratch /* >= 48 floats of LDS */) {
  a = wave_max(a);
  b = wave_max(b);
  c = wave_max(c);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { scratch[w] = a; scratch[16 + w] = b; scratch[32 + w] = c; }
  __syncthreads();
  a = scratch[0];
  b = scratch[16];
  c = scratch[32];
  for (int i = 1; i < nw; ++i) {
    a = fmaxf(a, scratch[i]);
    b = fmaxf(b, scratch[16 + i]);
    c = fmaxf(c, scratch[32 + i]);
  }
}

}  // namespace csa
