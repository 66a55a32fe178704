// device_utils.h -- gfx950 device helpers of the MoE finalize kernels: 128-bit activation
// packing, wavefront reductions over DPP, and exact FP8/FP4 encoders (software ones and ones
// built on the gfx950 conversion instructions).
//
// Sources (cited by key): [FI6631] flashinfer PR #6631 "perf(comm): gather MoE-finalize routes
// together and accumulate in FP32"; [FI3385] flashinfer PR #3385 "feat: MNNVL Allreduce quant
// fusion and performance optimization".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfin {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum : int { ACT_BF16 = 0, ACT_FP16 = 1 };

// --- activation packing: 8 elements of bf16/fp16 in one 128-bit word ---------------------------
template <int ACT>
struct Act;

template <>
struct Act<ACT_BF16> {
  static __device__ __forceinline__ void unpack(const u32x4 v, float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, v[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
    }
  }
  // Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ u32x4 pack(const float f[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 x = {f[2 * i], f[2 * i + 1]};
      r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    }
    return r;
  }
  static __device__ __forceinline__ float scalar(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
};

template <>
struct Act<ACT_FP16> {
  static __device__ __forceinline__ void unpack(const u32x4 v, float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Copy the element out first: bit-casting a vector-element lvalue directly has been seen
      // to read element 0 for every i.
      const uint32_t word = v[i];
      f32x2 x = __builtin_convertvector(__builtin_bit_cast(f16x2, word), f32x2);
      f[2 * i] = x[0];
      f[2 * i + 1] = x[1];
    }
  }
  // Round-to-nearest-even float -> fp16 (default rounding mode; never the RTZ pack).
  static __device__ __forceinline__ u32x4 pack(const float f[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x2 h;
      h[0] = (_Float16)f[2 * i];
      h[1] = (_Float16)f[2 * i + 1];
      r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
  }
};

// --- workgroup barrier for LDS traffic only ----------------------------------------------------
// __syncthreads() also orders global memory, which makes every wavefront wait until its pending
// global stores are acknowledged before the barrier. The kernels only exchange data through LDS,
// so this barrier fences LDS alone and lets outstanding stores drain in the background.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// --- wavefront sum over DPP ---------------------------------------------------------------------
// Sums v over the 64 lanes of a wavefront in a fixed order (so the result is bitwise
// reproducible): quad swaps, half-row and row mirrors give every lane its 16-lane row sum, then
// the four row sums (lanes 15, 31, 47, 63) are added in row order. Returns the sum in all lanes.
#define MFIN_DPP_ADD(v, ctrl)                                                                   \
  (v) += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                                 \
             0, __builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))

__device__ __forceinline__ float wave_sum(float v) {
  MFIN_DPP_ADD(v, 0xB1);   // quad_perm [1,0,3,2]
  MFIN_DPP_ADD(v, 0x4E);   // quad_perm [2,3,0,1]
  MFIN_DPP_ADD(v, 0x141);  // row_half_mirror
  MFIN_DPP_ADD(v, 0x140);  // row_mirror: every lane now holds its row (16 lanes) sum
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  return (r0 + r1) + (r2 + r3);
}

// Maximum of v and the value of lane ^ 1 (the other half of a 16-element NVFP4 block).
__device__ __forceinline__ uint32_t pair_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  return max(v, o);
}

// The value of lane + N within the lane's row of 16 (DPP row_shl:N, one VALU operation instead
// of an LDS permute); lanes whose lane + N leaves the row get 0.
template <int N>
__device__ __forceinline__ uint32_t row_shl_dpp(uint32_t v) {
  static_assert(N >= 1 && N <= 15, "row shift");
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xF, 0xF, false);
}

// --- exact-decision narrow encoders ------------------------------------------------------------
// Branch-free: every lane runs the same instruction stream, so the codes of a lane's 8 elements
// are independent chains the compiler can interleave. e4m3_code, e4m3_value and e2m1_code are
// the software encoders (float64 and per-midpoint FMA tests); the kernels use them only for
// NVFP4 global scales outside [2^-100, 2^100]. The hardware-conversion encoders further down
// (e4m3_block_scale_exact, e4m3_pack8_exact, e2m1_pack_exact) serve every other call.
//
// OCP E4M3 ("fn") of an exact float64 magnitude y: bias 7, 3 mantissa bits, subnormals m * 2^-9,
// max 448. Round to nearest even, saturate at 448. y >= 0, finite, infinite or NaN. Returns the
// 7-bit magnitude code.
__device__ __forceinline__ uint32_t e4m3_code(double y) {
  const double yc = __builtin_fmin(y, 448.0);   // saturation (a NaN y is handled at the end)
  // yc = m * 2^e with m in [1, 2); below 2^-6 (zero included) the spacing stays 2^-9
  const int e = yc < 0x1p-6 ? -6 : __builtin_amdgcn_frexp_exp(yc) - 1;
  const double r = __builtin_rint(__builtin_amdgcn_ldexp(yc, 3 - e));  // exact scale, RNE
  // normal: r in [8, 16]; subnormal: r in [0, 8]. A carry to 16 moves to the next binade, and
  // 448 itself gives 0x7E.
  const uint32_t c = (uint32_t)((e + 7) * 8 + (int)r - 8);
  return y == y ? c : 0x7Fu;
}

__device__ __forceinline__ double e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 0xFu, m = c & 7u;
  const uint32_t mant = ex ? 8u + m : m;          // subnormal: m * 2^-9
  const int sh = ex ? (int)ex - 10 : -9;          // normal: (8 + m) * 2^(ex - 10)
  return __builtin_amdgcn_ldexp((double)mant, sh);
}

__device__ __forceinline__ uint32_t sign_bit(float x) {
  return __builtin_bit_cast(uint32_t, x) >> 31;
}

// E2M1 magnitude code of a*gs/sf for a = |x| (a bf16/fp16 value), the float32 global scale gs
// and the E4M3 block scale sf > 0: round to nearest even among {0, .5, 1, 1.5, 2, 3, 4, 6}
// (codes 0..7), saturate at 6; 0 for NaN. No division: each decision compares a*gs with
// m*sf for a rounding midpoint m. m*sf is exact in float32 (a 3-bit by 4-bit product), and
// fma(a, gs, -m*sf) rounds the exact difference a*gs - m*sf once, so its sign is the exact
// sign unless that difference underflows to zero. It cannot: near a decision a*gs is close to
// m*sf >= 2^-11, and a*gs carries at most 35 significant bits (an fp16 significand of 11 bits
// times a float32 one of 24; bf16 gives 32), so both are multiples of about 2^-46 there and a
// nonzero difference is at least that large, far above the float32 subnormals; far from a
// decision the difference is large anyway. Each test is the sign bit of one FMA: no compare
// result goes through VCC, and the seven tests of a lane's eight elements overlap.
__device__ __forceinline__ uint32_t e2m1_code(float a, float gs, float sf) {
  // ties to the even code: midpoints 0.25, 1.25, 2.5, 5 go down (count a*gs > m*sf);
  // 0.75, 1.75, 3.5 go up (count a*gs >= m*sf, i.e. 1 - [a*gs < m*sf])
  const uint32_t above = sign_bit(__builtin_fmaf(-a, gs, 0.25f * sf)) +
                         sign_bit(__builtin_fmaf(-a, gs, 1.25f * sf)) +
                         sign_bit(__builtin_fmaf(-a, gs, 2.5f * sf)) +
                         sign_bit(__builtin_fmaf(-a, gs, 5.0f * sf));
  const uint32_t below = sign_bit(__builtin_fmaf(a, gs, -0.75f * sf)) +
                         sign_bit(__builtin_fmaf(a, gs, -1.75f * sf)) +
                         sign_bit(__builtin_fmaf(a, gs, -3.5f * sf));
  return a == a ? above + 3u - below : 0u;
}

// The value of E4M3 code c (gfx950 v_cvt_f32_fp8, OCP E4M3; code 0x7F gives NaN).
__device__ __forceinline__ float e4m3_value_hw(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// E4M3 code of amax * gs / 6 rounded to nearest even exactly, saturating at 448 (0x7E), for a
// block maximum amax >= 0 (a bf16 / fp16 magnitude or infinity, not NaN) and gs in
// [2^-100, 2^100]. The same three steps as e2m1_pack_exact on the E4M3 grid (gfx950
// v_cvt_pk_fp8_f32: round to nearest even on the float32 input; it gives NaN from 464 up, so
// inputs are clamped to 448 first): the codes of v (1 -+ 2^-19), v = amax * (gs * (1/6))
// within three float32 roundings of amax * gs / 6, bracket the exact one; S = 2m from their
// values (a midpoint m, or twice a value); the exact sign of amax * gs - 3S from one FMA
// (3S is exact, and amax * gs has at most 35 significant bits); S moved by
// clamp(d * 2^16, +-S * 2^-6), halved, then converted. A cell of the E4M3 grid is at least
// 1/15 of its value wide, so the +-2^-6 move stays inside it.
__device__ __forceinline__ uint32_t e4m3_block_scale_exact(float amax, float gs) {
  const float v = amax * (gs * (1.f / 6.f));
  const float v_lo = fminf(v * (1.f - 0x1p-19f), 448.f), v_hi = fminf(v * (1.f + 0x1p-19f), 448.f);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v_lo, v_hi, 0, false);
  const auto s = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
  const float s2 = s[0] + s[1];
  const float d = __builtin_fmaf(amax, gs, -3.f * s2);
  const float bd = 0x1p-22f * s2;
  const float y = 0.5f * __builtin_fmaf(__builtin_amdgcn_fmed3f(d, -bd, bd), 0x1p16f, s2);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFFu;
}

// OCP E4M3 codes of x[i] * s8 (i < 8, byte i of the pair of words) rounded to nearest even
// exactly, saturating at 448 (0x7E); a NaN gives 0x7F whatever its sign. The float32 product p
// is made round-to-odd (p one step toward zero when the exact FMA residual is negative, then
// the last bit set when it is nonzero), which keeps every rounding decision to the 4-bit E4M3
// significand (round-to-odd at 24 bits followed by a rounding to at most 22 is a single correct
// rounding: Boldo and Melquiond's result); gfx950
// v_cvt_pk_fp8_f32 then rounds it to nearest even. Products above 448 (infinities included)
// are clamped first, since the conversion gives NaN from 464 up; a NaN code's sign bit is
// cleared in the packed words.
__device__ __forceinline__ u32x2 e4m3_pack8_exact(const float x[8], float s8) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = __builtin_fabsf(x[i]);
    const float p = a * s8;
    const uint32_t rb = __builtin_bit_cast(uint32_t, __builtin_fmaf(a, s8, -p));
    const uint32_t t = (__builtin_bit_cast(uint32_t, p) - (rb >> 31)) | min(rb, 1u);
    const float m = p > 448.f ? 448.f : __builtin_bit_cast(float, t);   // a NaN stays NaN
    y[i] = __builtin_copysignf(m, x[i]);
  }
  u32x2 w;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * j], y[4 * j + 1], 0, false);
    v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * j + 2], y[4 * j + 3], (int)v, true);
    // bytes whose magnitude is 0x7F (NaN; finite codes stop at 0x7E) lose their sign bit
    const uint32_t nan_bytes = ((v & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    w[j] = v & ~nan_bytes;
  }
  return w;
}

// gfx950 E2M1 conversion (v_cvt_scalef32_pk_fp4_f32) of N = 4 or 8 float32 values y[i] / hw,
// packed 4 bits each, element i in bits 4i..4i+3. hw must be a power of two (the instruction
// divides by 2^exponent(hw), exactly). Round to nearest even on the float32 input, saturating at
// 6, sign kept; a NaN gives magnitude 7.
template <int N>
__device__ __forceinline__ uint32_t e2m1_cvt(const float* y, float hw) {
  static_assert(N == 4 || N == 8, "four or eight elements");
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], hw, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], hw, 1);
  if constexpr (N == 8) {
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], hw, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], hw, 3);
  }
  return w;
}

// The inverse (v_cvt_scalef32_pk_f32_fp4, scale 1): the values of the N codes packed in w.
template <int N>
__device__ __forceinline__ void e2m1_values(uint32_t w, float v[N]) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 1);
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  if constexpr (N == 8) {
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 3);
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
  }
}

// E2M1 codes (sign and magnitude, packed as by e2m1_cvt) of x[i] * gs / sf rounded to nearest
// even exactly, for an E4M3 block scale sf (0 gives the signed zeros of the x[i]) and a global
// scale gs in [2^-100, 2^100]; x[i] are bf16 or fp16 values, not NaN.
// 1. q = gs * rcp(sf) is within three float32 roundings of gs / sf, so the hardware codes of
//    x * q (1 - 2^-19) and x * q (1 + 2^-19) bracket the exact code: equal, or c and c + 1
//    when x * gs / sf lies within ~2^-18 of the midpoint m between them (or on it).
// 2. From the two codes' values, S = 2m in the bracketed case and S = 2 * value otherwise, and
//    d = fma(|x|, gs, -(S / 2) * sf), whose sign is the exact sign of x * gs - m * sf (the same
//    argument as for e2m1_code: (S / 2) * sf is exact and the difference cannot underflow).
// 3. S + clamp(d * 2^17 / sf, +-2^-5), divided by 2 in the conversion, is m moved off the
//    midpoint by at least two float32 steps in the exact direction (a nonzero |x * gs - m * sf|
//    is at least 2^-36 of m * sf: x * gs has at most 35 significant bits), or m itself on a
//    tie, which the conversion then rounds to even; away from midpoints it stays within 2^-6
//    of the value, inside that code's interval. About 12 instructions per element, no branch.
template <int N>
__device__ __forceinline__ uint32_t e2m1_pack_exact(const float* x, float gs, float sf) {
  const float r = sf != 0.f ? __builtin_amdgcn_rcpf(sf) : 0.f;
  const float q = gs * r, q_lo = q * (1.f - 0x1p-19f), q_hi = q * (1.f + 0x1p-19f);
  float y[N];
#pragma unroll
  for (int i = 0; i < N; ++i) y[i] = x[i] * q_lo;
  const uint32_t w_lo = e2m1_cvt<N>(y, 1.f);
#pragma unroll
  for (int i = 0; i < N; ++i) y[i] = x[i] * q_hi;
  const uint32_t w_hi = e2m1_cvt<N>(y, 1.f);
  float v_lo[N], v_hi[N];
  e2m1_values<N>(w_lo & 0x77777777u, v_lo);
  e2m1_values<N>(w_hi & 0x77777777u, v_hi);
  const float hsf = 0.5f * sf, k2 = 0x1p17f * r, bd = 0x1p-22f * sf;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float s2 = v_lo[i] + v_hi[i];
    const float d = __builtin_fmaf(__builtin_fabsf(x[i]), gs, -(s2 * hsf));
    y[i] = __builtin_fmaf(__builtin_amdgcn_fmed3f(d, -bd, bd), k2, s2);
  }
  return (e2m1_cvt<N>(y, 2.f) & 0x77777777u) | (w_lo & 0x88888888u);
}

}  // namespace mfin
