// Test helpers (not part of the library).
//
// mfma_probe_run: one scaled FP4 matrix instruction per wave on operands read from buffers, raw
// FP32 results written back, so a GPU test can compare the instruction's accumulation with the
// oracle's model on randomized operands.  Wave w, lane l reads a[w*64 + l] (16 bytes: 32 E2M1
// codes, two per byte, low nibble first), the scale byte sa[w*64 + l] (E8M0), b and sb likewise,
// and the accumulator input c[w*64 + l] (4 floats); it writes d[w*64 + l] (4 floats).  The
// instruction is the 16x16x128 scaled FP4 MFMA: lane l supplies row l % 16 of A (and column
// l % 16 of B) for the 32-element block l / 16, and register i of lane l holds output row
// 4 (l / 16) + i, column l % 16.
//
// quot_probe_run: the library's output quotient (hifa4::quot_h16 of device_common.h, used by the
// prefill epilogue) against the correctly rounded FP16 quotient, for every finite FP16 x and
// every positive finite FP16 l.
//
// prim_probe_run: the library's elementwise P-hat helpers (device_common.h) on given FP16 inputs:
// hifa4::exp2_h2 (both halves) and the E2M1 conversions of FP16 (hifa4::cvt_fp4x2_h) and FP32
// (hifa4::cvt_fp4x2) values at scale 1, for a GPU test to compare with the oracle.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

typedef int probe_v8i __attribute__((ext_vector_type(8)));
typedef float probe_v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint4* a, const uint32_t* sa, const uint4* b,
                                                        const uint32_t* sb, const float4* c, float4* d, int n) {
  if ((int)blockIdx.x >= n) return;
  const int i = blockIdx.x * 64 + threadIdx.x;
  const uint4 av = a[i], bv = b[i];
  const float4 cv = c[i];
  const probe_v8i A = {(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
  const probe_v8i B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
  const probe_v4f C = {cv.x, cv.y, cv.z, cv.w};
  // cbsz = blgp = 4: both operands E2M1; byte 0 of each scale register
  const probe_v4f D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, 4, 4, 0, (int)sa[i], 0, (int)sb[i]);
  d[i] = make_float4(D[0], D[1], D[2], D[3]);
}

// Device pointers (16-byte aligned), n waves; launches on the given stream (may be null).
// Returns the HIP status of the launch.
extern "C" int mfma_probe_run(const void* a, const void* sa, const void* b, const void* sb, const void* c, void* d,
                              int n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((uint32_t)n), dim3(64), 0, (hipStream_t)stream,
                     (const uint4*)a, (const uint32_t*)sa, (const uint4*)b, (const uint32_t*)sb, (const float4*)c,
                     (float4*)d, n);
  return (int)hipGetLastError();
}

// RNE of a finite FP64 value to FP16 (one rounding, subnormals and overflow to infinity included)
__device__ uint16_t f64_to_f16_rne(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int e = (int)((b >> 52) & 0x7FF);
  if (e == 0) return sign;  // zero (the quotients here are never FP64 subnormals)
  const int E = e - 1023;
  const uint64_t sig = (b & ((1ull << 52) - 1)) | (1ull << 52);
  // keep the bits down to 2^-10 of the leading one (normal), or down to 2^-24 (subnormal range)
  const int shift = E >= -14 ? 42 : 42 + (-14 - E);
  if (shift >= 64) return sign;  // below 2^-25: rounds to zero
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  if (E >= -14) {
    int e16 = E + 15;
    if (q == 2048) {
      q = 1024;
      e16++;
    }
    if (e16 >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (e16 << 10) | (uint32_t)(q - 1024));
  }
  return (uint16_t)(sign | q);  // q = 1024 is the smallest normal, exponent field 1
}

// one thread per l (bits 0x0001 .. 0x7BFF), all finite x; counts[0] = mismatches, first[0] = the
// first mismatch seen as (l bits << 16) | x bits
__global__ __launch_bounds__(256) void quot_probe_kernel(unsigned long long* counts, uint32_t* first) {
  const uint32_t lb = blockIdx.x * blockDim.x + threadIdx.x + 1;
  if (lb > 0x7BFFu) return;
  const float l = (float)__builtin_bit_cast(_Float16, (uint16_t)lb);
  const float r = __builtin_amdgcn_rcpf(l);
  unsigned long long n = 0;
  for (uint32_t xb = 0; xb < 0x10000u; xb++) {
    if ((xb & 0x7C00u) == 0x7C00u) continue;  // infinities and NaNs
    const float x = (float)__builtin_bit_cast(_Float16, (uint16_t)xb);
    const uint16_t got = __builtin_bit_cast(uint16_t, hifa4::quot_h16(x, l, r));
    // the FP64 quotient is correctly rounded (relative error below 2^-53), and an exact quotient of
    // two FP16 values that is not itself an FP16 tie lies more than 2^-40 (relative) from one, so
    // the FP64 value sits on the same side of every FP16 rounding boundary: one more rounding gives
    // fp16(x / l)
    const uint16_t want = f64_to_f16_rne((double)x / (double)l);
    if (got != want) {
      n++;
      atomicCAS(first, 0u, (lb << 16) | xb);
    }
  }
  if (n) atomicAdd(counts, n);
}

// counts: 1 zeroed unsigned 64-bit counter, first: 1 zeroed 32-bit word (device pointers).
extern "C" int quot_probe_run(void* counts, void* first, void* stream) {
  hipLaunchKernelGGL(quot_probe_kernel, dim3((0x7BFFu + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                     (unsigned long long*)counts, (uint32_t*)first);
  return (int)hipGetLastError();
}

// thread i: h[i] in both halves of a dword; exp_out[2 i], exp_out[2 i + 1] = the two halves of
// exp2_h2; code16[i] = the byte of cvt_fp4x2_h (low nibble from the low half); code32[i] = the
// byte of cvt_fp4x2 on the FP32 value, scale 1
__global__ __launch_bounds__(256) void prim_probe_kernel(const uint16_t* h, uint16_t* exp_out, uint8_t* code16,
                                                         uint8_t* code32, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t v = h[i];
  const uint32_t packed = v | (v << 16);
  const uint32_t e = hifa4::exp2_h2(packed);
  exp_out[2 * i] = (uint16_t)(e & 0xFFFF);
  exp_out[2 * i + 1] = (uint16_t)(e >> 16);
  code16[i] = (uint8_t)(hifa4::cvt_fp4x2_h<0>(0u, packed) & 0xFF);
  const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)v);
  code32[i] = (uint8_t)(hifa4::cvt_fp4x2<0>(0u, f, f, 1.0f) & 0xFF);
}

// device pointers: h [n] FP16 bits, exp_out [2 n], code16 [n], code32 [n]
extern "C" int prim_probe_run(const void* h, void* exp_out, void* code16, void* code32, int n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(prim_probe_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)h, (uint16_t*)exp_out, (uint8_t*)code16, (uint8_t*)code32, n);
  return (int)hipGetLastError();
}
