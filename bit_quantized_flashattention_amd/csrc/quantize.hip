// K1: Smooth-QK element-wise rescale + 4-bit block quantization (HBM-bound).
//
// HiFA4 abstract: Smooth-QK leaves only "a fusible element-wise scaling" at inference; here it is
// fused into the quantizer, so Q and K are read once in FP16 and written once as 4-bit codes.
#include "device_common.h"
#include "launch.h"

namespace hifa4 {

// One thread per 32-element block along d: 64 B of FP16 in, 16 B of codes + 1 scale byte out.
// Consecutive threads own consecutive blocks, so loads and stores are contiguous per wave.
// K-hat scales are written as block planes [B*H, d/32, len32] (one row of key scales per
// 32-channel block, what the attention kernels stage per tile); threads past the last key of
// a row write the zero scale bytes of the padding.  When all rows of a work-group belong to one
// (batch, head), its Smooth-QK scale row is staged in LDS once instead of every thread reading
// its 128 bytes of scales through the vector memory path.
template <int D, bool PLANES>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantRowsArgs a) {
  constexpr int NB = D / kBlock;
  __shared__ __attribute__((aligned(16))) float s_row[D];
  const int64_t n_rows = PLANES ? a.rows / a.len * a.len32 : a.rows;
  const int64_t n_items = n_rows * NB;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x;
  const int64_t t = t0 + threadIdx.x;
  // (batch, head) index of the work-group's first and last row; uniform across the group
  const int64_t t_last = (t0 + blockDim.x < n_items ? t0 + blockDim.x : n_items) - 1;
  const int64_t rows_per_bh = PLANES ? a.len32 : a.len;
  const int64_t bh_first = t0 / NB / rows_per_bh, bh_last = t_last / NB / rows_per_bh;
  const bool staged = a.scale != nullptr && bh_first == bh_last;
  if (staged) {
    const int h = (int)(bh_first % a.heads);
    const float* src = a.scale + (int64_t)(h / a.heads_per_scale_row) * D;
    for (int i = threadIdx.x; i < D; i += blockDim.x) s_row[i] = src[i];
    __syncthreads();
  }
  if (t >= n_items) return;
  const int blk = (int)(t % NB);
  int64_t row = t / NB;
  uint8_t* scale_dst;
  if (PLANES) {
    const int64_t bh = row / a.len32, tok = row % a.len32;
    scale_dst = a.scales + (bh * NB + blk) * a.len32 + tok;
    if (tok >= a.len) {
      *scale_dst = 0;
      return;
    }
    row = bh * a.len + tok;
  } else {
    scale_dst = a.scales + row * NB + blk;
  }
  Block32In in;
  load_block32(a.x + row * D + blk * kBlock, nullptr, in);
  if (staged) {
    const float4* ls = reinterpret_cast<const float4*>(s_row + blk * kBlock);
#pragma unroll
    for (int i = 0; i < 8; i++) in.s[i] = ls[i];
  } else if (a.scale != nullptr) {
    const int h = (int)((row / a.len) % a.heads);
    load_block32(nullptr, a.scale + (int64_t)(h / a.heads_per_scale_row) * D + blk * kBlock, in);
  }
  uint4 out;
  const uint32_t e8 = quantize_loaded32(in, a.scale != nullptr, &out);
  *reinterpret_cast<uint4*>(a.codes + row * (D / 2) + blk * 16) = out;
  *scale_dst = (uint8_t)e8;
}

// V: blocks run along tokens, so a work-group stages 128 tokens x d channels in LDS and each
// thread quantizes (channel, 32-token block) items.  The output is block-major (for each
// 32-token block, all channels), so consecutive threads write consecutive 16-byte cells.
template <int D>
constexpr int vt_tokens() { return D >= 256 ? 64 : 128; }  // LDS tile stays below 64 KB

template <int D>
__global__ __launch_bounds__(256) void quantize_vt_kernel(QuantVtArgs a) {
  constexpr int TOK = vt_tokens<D>();
  constexpr int NBT = TOK / kBlock;  // 32-token blocks per tile
  constexpr int ROW = D + 8;  // FP16 elements per LDS row (padding breaks bank aliasing)
  __shared__ _Float16 tile[TOK * ROW];
  const int64_t bh = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * TOK;
  const uint16_t* src = a.v + bh * a.len * D;
  constexpr int CPR = D / 8;  // 16-byte chunks per token row
  for (int c = threadIdx.x; c < TOK * CPR; c += blockDim.x) {
    const int r = c / CPR, cc = c % CPR;
    uint4 val = {0u, 0u, 0u, 0u};
    if (t0 + r < a.len) val = *reinterpret_cast<const uint4*>(src + (t0 + r) * D + cc * 8);
    *reinterpret_cast<uint4*>(&tile[r * ROW + cc * 8]) = val;
  }
  __syncthreads();
  const int64_t nblk = (a.len32 - t0) / kBlock < NBT ? (a.len32 - t0) / kBlock : NBT;
  for (int w = threadIdx.x; w < D * NBT; w += blockDim.x) {
    const int jb = w / D, ch = w % D;
    if (jb >= nblk) continue;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) {
      v[i] = (float)tile[(jb * kBlock + i) * ROW + ch];
      amax = fmaxf(amax, fabsf(v[i]));
    }
    const int e = mx_exponent(amax);
    const float sc = e8m0_as_float(e);
    uint4 out;
    out.x = pack8_fp4(v + 0, sc);
    out.y = pack8_fp4(v + 8, sc);
    out.z = pack8_fp4(v + 16, sc);
    out.w = pack8_fp4(v + 24, sc);
    // block-major V-hat: [bh][token block][channel] -> 16 code bytes; the block's scale bytes
    // are stored channel ch at (D/16) (ch % 16) + ch / 16, so the D/16 channels ch, ch + 16, ...
    // that one MFMA lane serves have adjacent scale bytes
    const int64_t blk_row = (bh * (a.len32 / kBlock) + t0 / kBlock + jb) * D;
    *reinterpret_cast<uint4*>(a.codes + (blk_row + ch) * 16) = out;
    a.scales[blk_row + (D / 16) * (ch % 16) + ch / 16] = (uint8_t)(e + 127);
  }
}

template <int D>
static hipError_t quant_rows_d(const QuantRowsArgs& a, hipStream_t s) {
  const int64_t rows = a.block_planes ? a.rows / a.len * a.len32 : a.rows;
  const int64_t items = rows * (D / kBlock);
  const int64_t grid = (items + 255) / 256;
  if (a.block_planes) hipLaunchKernelGGL((quantize_rows_kernel<D, true>), dim3((uint32_t)grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((quantize_rows_kernel<D, false>), dim3((uint32_t)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return quant_rows_d<64>(a, s);
    case 128: return quant_rows_d<128>(a, s);
    case 256: return quant_rows_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t quant_vt_d(const QuantVtArgs& a, hipStream_t s) {
  const int64_t tiles = (a.len + vt_tokens<D>() - 1) / vt_tokens<D>();
  hipLaunchKernelGGL(quantize_vt_kernel<D>, dim3((uint32_t)tiles, (uint32_t)a.bh), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_vt(const QuantVtArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return quant_vt_d<64>(a, s);
    case 128: return quant_vt_d<128>(a, s);
    case 256: return quant_vt_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hifa4
