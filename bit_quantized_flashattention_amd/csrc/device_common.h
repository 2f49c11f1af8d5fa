// Device helpers shared by the gfx950 kernels of libhifa4.
//
// Format (the HiFA4 abstract names the 4-bit format HIF4 without a bit layout; this library
// substitutes): E2M1 codes with one power-of-two E8M0 scale per block of 32 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 32;      // elements per scale block
constexpr int kTileKeys = 128;  // keys held per LDS tile (one 16x16x128 MFMA contraction)

// Block exponent from the block's largest magnitude: the smallest e with 6 * 2^e >= amax
// (no element is clipped), clamped to [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex;
  const float m = frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
  const int e = (m <= 0.75f) ? ex - 3 : ex - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as the FP32 scale operand of the FP4 converter, which reads the operand's biased exponent
// field as an E8M0 value (e = -127 is the subnormal 2^-127, exponent field 0).
__device__ __forceinline__ float e8m0_as_float(int e) {
  return __uint_as_float(e <= -127 ? 0x00400000u : (uint32_t)(e + 127) << 23);
}

// RNE of (a / scale) and (b / scale) onto E2M1, saturating at 6, written to byte SEL of old
// (a in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// Packs 8 values (already relative to nothing: the scale argument divides them) into one dword.
__device__ __forceinline__ uint32_t pack8_fp4(const float* v, float scale) {
  uint32_t w = 0;
  w = cvt_fp4x2<0>(w, v[0], v[1], scale);
  w = cvt_fp4x2<1>(w, v[2], v[3], scale);
  w = cvt_fp4x2<2>(w, v[4], v[5], scale);
  w = cvt_fp4x2<3>(w, v[6], v[7], scale);
  return w;
}

// P-tilde's exp2: X(w) = 2^floor(w) * g(fract(w)), g(t) = ((c3 t + c2) t + c1) t + 1 with one
// rounding per fma.  g is the cubic through (0, 1) and the E2M1 rounding midpoints
// (log2 1.25, 1.25), (log2 1.5, 1.5), (log2 1.75, 1.75), so a 4-bit decision on X(w) is the
// round-to-nearest decision on the true 2^w except within ~1e-7 of a midpoint.
__device__ __forceinline__ float exp2_x(float w, float c1, float c2, float c3) {
  const float f = __builtin_amdgcn_fractf(w);
  const float fl = __builtin_floorf(w);
  const float g = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c3, f, c2), f, c1), f, 1.0f);
  return __builtin_ldexpf(g, (int)fl);
}

__device__ __forceinline__ v4f mfma_fp4(const uint4& a, uint32_t sa, const uint4& b, uint32_t sb,
                                         v4f c) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands E2M1; byte 0 of sa / sb is the E8M0 scale of this lane's
  // 32-element block.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the gfx950 row-swap
// permutes, which are VALU operations (no LDS round trip).  Swapping a value with itself leaves
// the lower partner's copy in the first result and the upper partner's in the second, in every
// lane: v_permlane16_swap pairs rows (0,1) and (2,3), v_permlane32_swap pairs halves.
__device__ __forceinline__ float group_max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// (x0 + x1) + (x2 + x3) with x_g the value of lane group g, the same bits in every lane
__device__ __forceinline__ float group_sum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace hifa4
