// Test helper (not part of the library): one scaled FP4 matrix instruction per wave on operands
// read from buffers, raw FP32 results written back, so a GPU test can compare the instruction's
// accumulation with the oracle's model on randomized operands.
//
// Wave w, lane l reads a[w*64 + l] (16 bytes: 32 E2M1 codes, two per byte, low nibble first),
// the scale byte sa[w*64 + l] (E8M0), b and sb likewise, and the accumulator input c[w*64 + l]
// (4 floats); it writes d[w*64 + l] (4 floats).  The instruction is the 16x16x128 scaled FP4
// MFMA: lane l supplies row l % 16 of A (and column l % 16 of B) for the 32-element block l / 16,
// and register i of lane l holds output row 4 (l / 16) + i, column l % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
