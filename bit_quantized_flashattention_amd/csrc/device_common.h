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

// The shared-exponent rule of the OCP microscaling format, an accuracy variant: e = floor(log2
// amax) - 2 (2 = the largest E2M1 exponent), clamped; -127 for an all-zero block.  Magnitudes in
// (6, 8) * 2^e then saturate to 6 in the conversion.
__device__ __forceinline__ int mx_exponent_floor(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex;
  (void)frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
  const int e = ex - 3;
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

// Inputs of one 32-element block quantization: 32 FP16 values and their 32 FP32 channel scales.
struct Block32In {
  uint4 x[4];
  float4 s[8];
};

// Issues the loads of one block: x points at 32 FP16 values (16-byte aligned), s at their FP32
// channel scales; either may be nullptr to leave that part of in untouched.
__device__ __forceinline__ void load_block32(const uint16_t* x, const float* s, Block32In& in) {
  if (x != nullptr) {
    const uint4* src = reinterpret_cast<const uint4*>(x);
#pragma unroll
    for (int i = 0; i < 4; i++) in.x[i] = src[i];
  }
  if (s != nullptr) {
    const float4* sc = reinterpret_cast<const float4*>(s);
#pragma unroll
    for (int i = 0; i < 8; i++) in.s[i] = sc[i];
  }
}

// 4-bit quantization of 32 FP32 values: the block exponent comes from the largest magnitude and
// the codes are RNE onto E2M1 relative to 2^e.  Returns the E8M0 scale byte (e + 127); the 16
// code bytes go to *codes (element 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t quantize_values32(const float* v, uint4* codes, bool floor_rule = false) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  const int e = floor_rule ? mx_exponent_floor(amax) : mx_exponent(amax);
  const float scale = e8m0_as_float(e);
  codes->x = pack8_fp4(v + 0, scale);
  codes->y = pack8_fp4(v + 8, scale);
  codes->z = pack8_fp4(v + 16, scale);
  codes->w = pack8_fp4(v + 24, scale);
  return (uint32_t)(e + 127);
}

// The 32 FP16 values of a loaded block as FP32 (exact).
__device__ __forceinline__ void unpack_block32(const Block32In& in, float* v) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t w[4] = {in.x[i].x, in.x[i].y, in.x[i].z, in.x[i].w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[i * 8 + 2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFF));
      v[i * 8 + 2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
    }
  }
}

// Smooth-QK rescale and 4-bit quantization of one loaded block (scaled: apply in.s).  Each value
// becomes fp32(x * s) (one rounding; contraction is off), then quantize_values32.
__device__ __forceinline__ uint32_t quantize_loaded32(const Block32In& in, bool scaled, uint4* codes,
                                                      bool floor_rule = false) {
  float v[32];
  unpack_block32(in, v);
  if (scaled) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      v[4 * i + 0] = v[4 * i + 0] * in.s[i].x;
      v[4 * i + 1] = v[4 * i + 1] * in.s[i].y;
      v[4 * i + 2] = v[4 * i + 2] * in.s[i].z;
      v[4 * i + 3] = v[4 * i + 3] * in.s[i].w;
    }
  }
  return quantize_values32(v, codes, floor_rule);
}

// RoPE (rotate-half, FP32), Smooth-QK and 4-bit quantization of block blk of one FP16 row of
// width D before RoPE: cos_row and sin_row are the D/2 table entries of the row's position, s
// the 32 channel scales of the block or nullptr.  A block in the first half takes
// y = x c - x' s with x' its partner D/2 channels later; a block in the second half takes
// y = x c + x' s with x' its partner D/2 channels earlier; each product and sum is rounded once.
// All loads are issued before any arithmetic (one memory round trip): without Smooth-QK scales
// the factors read are the cos entries and are replaced by 1 (y * 1 = y exactly), so no load
// depends on a branch.
__device__ __forceinline__ uint32_t quantize_block32_rope(const uint16_t* row, int blk, int D, const float* cos_row,
                                                          const float* sin_row, const float* s, uint4* codes) {
  const int half = D / 2;
  const int c0 = kBlock * blk;
  const bool first = c0 < half;
  const int i0 = first ? c0 : c0 - half;  // table column of the block's first channel
  const uint4* own = reinterpret_cast<const uint4*>(row + c0);
  const uint4* partner = reinterpret_cast<const uint4*>(row + (first ? c0 + half : c0 - half));
  const float4* cp = reinterpret_cast<const float4*>(cos_row + i0);
  const float4* sp = reinterpret_cast<const float4*>(sin_row + i0);
  const float4* mp = reinterpret_cast<const float4*>(s != nullptr ? s : cos_row + i0);
  uint4 xo[4], xq[4];
  float4 cv[8], sv[8], mv[8];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    xo[k] = own[k];
    xq[k] = partner[k];
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    cv[k] = cp[k];
    sv[k] = sp[k];
    mv[k] = mp[k];
  }
  float y[32];
#pragma unroll
  for (int t = 0; t < 32; t++) {
    const uint32_t wo = (&xo[t / 8].x)[(t % 8) / 2], wq = (&xq[t / 8].x)[(t % 8) / 2];
    const float x = (float)__builtin_bit_cast(_Float16, (uint16_t)((t & 1) ? (wo >> 16) : (wo & 0xFFFF)));
    const float xp = (float)__builtin_bit_cast(_Float16, (uint16_t)((t & 1) ? (wq >> 16) : (wq & 0xFFFF)));
    const float c = (&cv[t / 4].x)[t % 4], sn = (&sv[t / 4].x)[t % 4];
    const float m = s != nullptr ? (&mv[t / 4].x)[t % 4] : 1.0f;
    y[t] = (first ? x * c - xp * sn : x * c + xp * sn) * m;
  }
  return quantize_values32(y, codes);
}

// Both steps for one block (see load_block32 and quantize_loaded32).
__device__ __forceinline__ uint32_t quantize_block32(const uint16_t* x, const float* s, uint4* codes) {
  Block32In in;
  load_block32(x, s, in);
  return quantize_loaded32(in, s != nullptr, codes);
}

// The softmax scale in the log2 domain, C = fp32(log2(e) / sqrt(d)), as a compile-time constant
// per head dimension: the per-score fma(S, C, offset) then takes the literal-operand form, which
// the vector ALU issues at twice the rate of the three-register form.
template <int D>
struct SoftmaxC;
template <>
struct SoftmaxC<64> {
  static constexpr float value = 0x1.715476p-3f;
};
template <>
struct SoftmaxC<128> {
  static constexpr float value = 0x1.0527dcp-3f;
};
template <>
struct SoftmaxC<256> {
  static constexpr float value = 0x1.715476p-4f;
};

// log2(6) rounded to the nearest FP32 (0x40257007): 6 is the largest E2M1 magnitude.
constexpr float kLog2Six = 0x1.4ae00ep+1f;

// Exponent e of a P-hat scale 2^e (one per query row and 32-key block; per row and tile in the
// per-tile variant), as an integer-valued float: the smallest power of two that keeps the
// largest probability 2^v it covers inside the E2M1 range, ceil(fp32(v - log2 6)), clamped below
// at -127 (v = -inf: no visible key).
__device__ __forceinline__ float tile_exponent(float v) {
  return fmaxf(__builtin_ceilf(v - kLog2Six), -127.0f);
}

// Direct-P constants (nearest FP32 values).  delta = 1/4 - log2(1.5)/2: a log2-domain value x is
// turned into 2^floor(x) (1 + frac(x)), whose E2M1 rounding points (mantissa 1.25 and 1.75) then
// sit at the log2-domain midpoints of neighbouring E2M1 values once delta is added to the score.
// kDirectTop = delta - 2.5: that value reaches 6, the largest E2M1 magnitude, at x = 2.5.
constexpr float kDirectDelta = -0x1.5c01a4p-5f;
constexpr float kDirectTop = -0x1.457006p+1f;

// Direct-P block exponent: the smallest e keeping the block maximum's value at most 6,
// ceil(fp32(v + (delta - 2.5))), clamped below at -127.
__device__ __forceinline__ float direct_exponent(float v) {
  return fmaxf(__builtin_ceilf(v + kDirectTop), -127.0f);
}

// float -> uint32 with the hardware conversion's saturation: negative values and -inf give 0
// (the C cast leaves them undefined, and a clamp would cost a second instruction)
__device__ __forceinline__ uint32_t cvt_u32_sat(float y) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(y));
  return r;
}

// float -> int32 with the hardware conversion's rules: NaN gives 0, out-of-range values (and
// +-inf) saturate (the C cast leaves all of these undefined)
__device__ __forceinline__ int cvt_i32_sat(float y) {
  int r;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(y));
  return r;
}

// rn16(2^x) of both FP16 halves of h.  v_exp_f16 is correctly rounded on every FP16 input;
// the SDWA form writes the high half and keeps the low one, so no pack is needed.  A
// transcendental result is not forwarded to the next instruction: the SDWA form reads the low
// half back (to keep it) only after one wait state, and so does the VALU consumer of r.
__device__ __forceinline__ uint32_t exp2_h2(uint32_t h) {
  uint32_t r;
  asm("v_exp_f16 %0, %1\n\t"
      "s_nop 0\n\t"
      "v_exp_f16_sdwa %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
      "s_nop 0"
      : "=&v"(r)
      : "v"(h));
  return r;
}

// Packs the two FP16 values of p (scale 1) as E2M1 codes, RNE and saturating, into byte SEL
// of old (the low half in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_h(uint32_t old, uint32_t p) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(old, __builtin_bit_cast(h2, p), 1.0f, SEL);
}

// (FP16 a, FP16 b) in one dword, each rounded to nearest even
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}

// The FP32 value x as it is, kept from being folded into a mixed-precision instruction: the
// log2-domain scores are rounded to FP32 by their fma first and only then to FP16.
__device__ __forceinline__ float keep_f32(float x) {
  asm("" : "+v"(x));
  return x;
}

// One (query row, key tile) step of the online softmax, from the row's largest visible score
// rmax (-inf if none) and the running max m (-inf before the first visible key).
struct RowStep {
  float m_new;      // integer running max ceil(fp32(max S * C)), exact in FP16
  _Float16 alpha;   // rn16(2^(m - m_new)), the FP16 rescale of O and l (see row_step)
  float mm;         // m_new, or a finite stand-in below every real m while m_new = -inf
};

// The P-hat scale of one lane's 32 keys and the offset of their log2-domain scores, from the
// largest visible score emax the scale covers (the lane's own block, or the row's tile maximum
// in the per-tile variant; -inf if none), under code rule DIRECT (Direct-P) or the FP16 exp2.
struct PhatScale {
  float e;          // scale exponent (integer-valued); -127 for a block without a visible key
  float neg_big_m;  // -(mm + e): offset of the scores relative to 2^e
};

template <bool DIRECT>
__device__ __forceinline__ PhatScale phat_scale(float emax, float C, float mm) {
  PhatScale p;
  const float v = __builtin_fmaf(emax, C, -mm);
  p.e = DIRECT ? direct_exponent(v) : tile_exponent(v);
  // held negated in a register: a negation folded into the per-score fma as an operand modifier
  // would force its slower three-register form
  p.neg_big_m = keep_f32(-(mm + p.e));
  return p;
}

// max of two FP32 values that are never NaN, as one v_max_f32 (fmaxf would first quiet operands
// the compiler cannot prove canonical, such as cross-lane results and loop-carried values)
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// min of two FP32 values that are never NaN, as one v_min_f32 (see max_nn)
__device__ __forceinline__ float min_nn(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ RowStep row_step(float rmax, float m, float C) {
  RowStep r;
  r.m_new = max_nn(m, __builtin_ceilf(rmax * C));
  // 2^(m - m_new) straight in FP16: exact down to 2^-24; below that the result underflows to 0
  // (2^-25 is a tie to even), and so it does for m = -inf (d = -inf saturates).  While no key of
  // the row has been visible (m = m_new = -inf, d = NaN, converted to 0) alpha is 1, which
  // multiplies the row's zero state: the same state as alpha = 0.  No compare and select: a
  // select on the condition register issues far slower than this arithmetic
  const float d = m - r.m_new;
  r.alpha = __builtin_ldexpf16((_Float16)1.0f, cvt_i32_sat(d));
  // m_new = -inf only for a row with no visible key yet: any finite stand-in below every real
  // m keeps e = -127 and every code 0
  r.mm = max_nn(r.m_new, -0x1p100f);
  return r;
}

// The same step under the round-to-nearest running max (an accuracy variant, not the method's
// reading): m_new = max(m, rn16(fp32(max S * C))), an FP16 value; alpha = rn16(2^rn16(fp32(m -
// m_new))) from v_exp_f16 (correctly rounded; 0 while m = -inf, and below 2^-30 where rn16
// gives 0 anyway); m_new + e is rounded once to FP32 (phat_scale).
__device__ __forceinline__ RowStep row_step_nearest16(float rmax, float m, float C) {
  RowStep r;
  // the product is rounded to FP32 first (keep_f32: not fused into one rounding to FP16)
  r.m_new = max_nn(m, (float)(_Float16)keep_f32(rmax * C));
  const float d = m - r.m_new;
  const uint32_t a2 = exp2_h2(pack_h2(d, d));
  r.alpha = d >= -30.0f ? __builtin_bit_cast(h2, a2)[0] : (_Float16)0.0f;
  r.mm = max_nn(r.m_new, -0x1p100f);
  return r;
}

// Key and channel maps of the 16x16x128 MFMAs (all offsets inside one 128-key tile).
//
// Scores are computed transposed, S^T = K-hat Q-hat^T, with the 16 MFMA columns = 16 queries.
// Score MFMA t (t = 0..7) takes key kappa(t, r) = 32 (r/4) + 8 (r%4) + t as its row r; its output
// register i of lane group g then holds key 32 g + 8 i + t, so after the 8 MFMAs lane (g, col)
// holds all 32 keys of block g of its query (s[4 t + i]), the slice the PV MFMA consumes as its
// B operand, and the 8 keys whose scales row r = col needs (t = 0..7) are adjacent.
__device__ __forceinline__ int score_row_key(int t, int r) { return 32 * (r >> 2) + 8 * (r & 3) + t; }
// key offset (inside the lane group's 32-key block) of accumulator value s[k]
__device__ __host__ constexpr int s_key(int k) { return 8 * (k & 3) + (k >> 2); }
// accumulator index holding key offset j of the block
__device__ __host__ constexpr int s_index(int j) { return 4 * (j & 7) + (j >> 3); }
// PV MFMA cb takes channel chi(cb, r) = 16 cb + r as its row r: the 16 lanes of a lane group
// read 16 adjacent V-hat cells.  Lane (g, col) needs the scales of channels col, 16 + col, ...,
// which the V-hat scale layout keeps adjacent, and its output register i of block cb holds
// channel 16 cb + 4 g + i of its query.

// P-hat codes of a lane's 32 keys: E2M1 of rn16(2^rn16(fma32(s_k, C, -(m + e)))), packed two
// per byte in key order (key 2j of the block in the low nibble of byte j); a score of -inf
// (masked key) gives the code 0.  The FP16 probabilities are left in p16 (pairs of keys
// (2j, 2j + 1)) for callers that sum them.
__device__ __forceinline__ uint4 phat_codes(const float* s, float C, float nbm, uint32_t* p16) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    // every byte of x is written by one of the four conversions below, so its initial value does
    // not matter: the first conversion writes into the probabilities' own register (no move of 0)
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int k = 8 * q + 2 * j;  // key offsets k, k + 1
      const float u0 = keep_f32(__builtin_fmaf(s[s_index(k)], C, nbm));
      const float u1 = keep_f32(__builtin_fmaf(s[s_index(k + 1)], C, nbm));
      const uint32_t pr = exp2_h2(pack_h2(u0, u1));
      p16[k / 2] = pr;
      if (j == 0) x = cvt_fp4x2_h<0>(pr, pr);
      if (j == 1) x = cvt_fp4x2_h<1>(x, pr);
      if (j == 2) x = cvt_fp4x2_h<2>(x, pr);
      if (j == 3) x = cvt_fp4x2_h<3>(x, pr);
    }
    w[q] = x;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Direct-P codes of a lane's 32 keys (FA4 prior art: scores mapped straight to FP4
// probabilities, no exponential): with K = fp32(fp32(127 - (m + e)) + delta), the single FP32
// rounding y = fma(s_k, C 2^23, K 2^23) holds (x + 127) 2^23 for the log2-domain value
// x = fma32(s_k, C, K) - 127; its integer part (0 for y <= 0, so a masked key gives 0), read as
// the bits of an FP32 number, is 2^floor(x) (1 + frac(x)), and the converter rounds that to E2M1
// (RNE, saturating at 6).  Packed two per byte in key order like phat_codes.
__device__ __forceinline__ uint4 phat_codes_direct(float* s, float C, float neg_big_m) {
  const float k = (127.0f + neg_big_m) + kDirectDelta;
  const float b = k * 0x1p23f;
  const float c23 = C * 0x1p23f;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    // the values replace the scores in place, eight keys at a time (no second set of live registers)
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int i = s_index(8 * q + j);
      s[i] = __uint_as_float(cvt_u32_sat(__builtin_fmaf(s[i], c23, b)));
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int kk = 8 * q + 2 * j;
      const float z0 = s[s_index(kk)], z1 = s[s_index(kk + 1)];
      if (j == 0) x = cvt_fp4x2<0>(x, z0, z1, 1.0f);
      if (j == 1) x = cvt_fp4x2<1>(x, z0, z1, 1.0f);
      if (j == 2) x = cvt_fp4x2<2>(x, z0, z1, 1.0f);
      if (j == 3) x = cvt_fp4x2<3>(x, z0, z1, 1.0f);
    }
    w[q] = x;
    __builtin_amdgcn_sched_barrier(0);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// FP32 sum of the 32 FP16 probabilities of a lane in the fixed tree order: pairs (k, k + 16),
// then (k, k + 8), (k, k + 4), (k, k + 2), (0, 1).
__device__ __forceinline__ float tree_sum32_h(const uint32_t* p16) {
  float t[32];
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const h2 v = __builtin_bit_cast(h2, p16[j]);
    t[2 * j] = (float)v[0];
    t[2 * j + 1] = (float)v[1];
  }
#pragma unroll
  for (int w = 16; w >= 1; w /= 2) {
#pragma unroll
    for (int k = 0; k < w; k++) t[k] = t[k] + t[k + w];
  }
  return t[0];
}

// O <- fma16(alpha, O, rn16(pv)) for the four FP16 outputs of one accumulator tile.
__device__ __forceinline__ void state_update(h2* o, _Float16 alpha, const v4f& pv) {
  const h2 a2 = h2{alpha, alpha};
  o[0] = __builtin_elementwise_fma(a2, o[0], __builtin_bit_cast(h2, pack_h2(pv[0], pv[1])));
  o[1] = __builtin_elementwise_fma(a2, o[1], __builtin_bit_cast(h2, pack_h2(pv[2], pv[3])));
}

// Writes one query's output row fp16(O / l) from the FP16 state of CB channel blocks: register i
// (i = 0..3) of block cb holds channel 16 cb + 4 g + i, so each block gives 4 adjacent channels
// (8 bytes); dst points at channel 4 g of the row (a row of LDS: the prefill stages its output
// tile there and stores it row-contiguous).
//
// The quotient: fp16(x / l) for FP16 values x and l > 0.  q = x r with r ~ 1/l (hardware
// reciprocal, ~1 ulp) is corrected once with the exact residual, which leaves the corrected value
// within about 2^-45 (relative) of x / l; it is then rounded to FP32 and only then to FP16.  A
// quotient of two FP16 values that is an FP16 rounding tie (possible only in the subnormal range,
// e.g. 9 * 2^-24 / 6) has at most 12 significant bits, so the FP32 rounding returns it exactly and
// the conversion breaks the tie to even; any other quotient lies farther from every tie than the
// FP32 rounding moves it.  tests/test_gpu_quotient.py checks every pair of finite FP16 x and
// positive finite FP16 l.  The residual is taken negated, d = fma(l, q, -x) (the same rounding of
// the same exact value with the opposite sign), and the correction is q - d r: then x = -0 keeps
// its sign through every step (q = -0, d = +0, -0 * r + -0 = -0) without a separate sign copy.
__device__ __forceinline__ float quot_h(float x, float l, float r) {
  const float q = x * r;
  const float d = __builtin_fmaf(l, q, -x);
  return __builtin_fmaf(-d, r, q);
}

// fp16(x / l) with r = rcp(l): the FP32 quotient is kept as it is (keep_f32), so the compiler
// cannot fuse the last fma with the conversion into a mixed-precision fma that rounds once to
// FP16 (that form rounds exact ties in the wrong direction)
__device__ __forceinline__ _Float16 quot_h16(float x, float l, float r) {
  return (_Float16)keep_f32(quot_h(x, l, r));
}

template <int CB>
__device__ __forceinline__ void write_out_row(uint8_t* dst, const h2 (*o)[2], float l) {
  const float r = __builtin_amdgcn_rcpf(l);
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      w[j] = __builtin_bit_cast(uint32_t, h2{quot_h16((float)o[cb][j][0], l, r), quot_h16((float)o[cb][j][1], l, r)});
    }
    *reinterpret_cast<uint2*>(dst + 32 * cb) = make_uint2(w[0], w[1]);
  }
}

__device__ __forceinline__ v4f mfma_fp4(const uint4& a, uint32_t sa, const uint4& b, uint32_t sb,
                                         v4f c) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands E2M1; byte 0 of sa / sb is the E8M0 scale of this lane's
  // 32-element block.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// The same with the scale bytes taken from byte SA of sa and byte SB of sb (the instruction's
// scale-select fields), so four scales packed in one register need no unpacking.
template <int SA, int SB>
__device__ __forceinline__ v4f mfma_fp4_sel(const uint4& a, uint32_t sa, const uint4& b, uint32_t sb, v4f c) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, SA, (int)sa, SB, (int)sb);
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the gfx950 row-swap
// permutes, which are VALU operations (no LDS round trip).  Swapping a value with itself leaves
// the lower partner's copy in the first result and the upper partner's in the second, in every
// lane: v_permlane16_swap pairs rows (0,1) and (2,3), v_permlane32_swap pairs halves.
__device__ __forceinline__ float group_max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// (x0 + x1) + (x2 + x3) with x_g the value of lane group g, the same bits in every lane
__device__ __forceinline__ float group_sum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace hifa4
