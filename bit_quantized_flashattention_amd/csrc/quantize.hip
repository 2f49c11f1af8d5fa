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
  const uint32_t e8 = quantize_loaded32(in, a.scale != nullptr, &out, a.scale_rule == 1);
  *reinterpret_cast<uint4*>(a.codes + row * (D / 2) + blk * 16) = out;
  *scale_dst = (uint8_t)e8;
}

// V: blocks run along tokens, so a work-group stages one 32-token block x d channels in LDS and
// each thread quantizes (channel, block) items.  The output is block-major (for each 32-token
// block, all channels), so consecutive threads write consecutive 16-byte cells.  Small LDS tiles
// keep many work-groups in flight per CU (measured at B8 L4096 d128: 32-token tiles about 4 us
// faster than 128-token ones).
template <int D>
constexpr int vt_tokens() { return 32; }

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
    const int e = a.scale_rule == 1 ? mx_exponent_floor(amax) : mx_exponent(amax);
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

// RoPE (FP32, rotate-half), Smooth-QK and 4-bit quantization of pre-RoPE rows, fused.  A
// work-group serves kRopeMaxPos consecutive positions of one batch entry for all H heads, so the
// cos/sin rows of those positions (and the Smooth-QK scale table when it is small) are staged in
// LDS once and shared by every head.  An item is one (position, head, block pair j): channels
// 32 j .. 32 j + 31 and their rotation partners 32 j + d/2 .. , so each item writes two
// quantization blocks.  Rounding, as the rotation is defined for this prologue: each product
// and each sum once in FP32, no fused multiply-add (contraction is off), then fp32(y * s).
constexpr int kRopeMaxPos = 32;          // positions per work-group at most
constexpr int kRopeMaxScaleFloats = 4096;  // Smooth-QK tables up to 16 KB are staged in LDS

template <int D, bool PLANES>
__global__ __launch_bounds__(256) void quantize_rope_kernel(QuantRopeArgs a) {
  constexpr int NB = D / kBlock;
  constexpr int NP = NB / 2;  // block pairs per row
  constexpr int H2 = D / 2;
  __shared__ __attribute__((aligned(16))) float s_cos[kRopeMaxPos * H2];
  __shared__ __attribute__((aligned(16))) float s_sin[kRopeMaxPos * H2];
  __shared__ __attribute__((aligned(16))) float s_scale[kRopeMaxScaleFloats];
  const int P = a.pos_per_wg;
  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * P;  // first token of the work-group
  const int64_t n_tok = PLANES ? a.len32 : a.len;
  const int np = (int)(n_tok - t0 < P ? n_tok - t0 : P);
  const int nrot = (int)(a.len - t0 < np ? (a.len - t0 > 0 ? a.len - t0 : 0) : np);  // tokens with data
  for (int i = threadIdx.x; i < nrot * H2; i += blockDim.x) {
    const int64_t src = (a.pos0 + t0 + i / H2) * H2 + i % H2;
    s_cos[i] = a.rope_cos[src];
    s_sin[i] = a.rope_sin[src];
  }
  const bool staged = a.scale != nullptr && a.scale_rows * D <= kRopeMaxScaleFloats;
  if (staged)
    for (int i = threadIdx.x; i < a.scale_rows * D; i += blockDim.x) s_scale[i] = a.scale[i];
  __syncthreads();
  // items ordered (head, position, block pair): the threads of a wave read consecutive rows of
  // one head, i.e. one contiguous run of HBM
  const int items = P * a.heads * NP;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int j = it % NP;
    const int pl = (it / NP) % P;
    const int h = it / (NP * P);
    if (pl >= np) continue;
    const int64_t tok = t0 + pl;
    const int64_t bh = b * a.heads + h;
    if (tok >= a.len) {  // padding key of a scale plane: zero scale bytes for both blocks
      if (PLANES) {
        a.scales[(bh * NB + j) * a.len32 + tok] = 0;
        a.scales[(bh * NB + j + NP) * a.len32 + tok] = 0;
      }
      continue;
    }
    const int64_t row = bh * a.len + tok;
    Block32In lo_in, hi_in;
    load_block32(a.x + row * D + kBlock * j, nullptr, lo_in);
    load_block32(a.x + row * D + H2 + kBlock * j, nullptr, hi_in);
    float lo[32], hi[32];
    unpack_block32(lo_in, lo);
    unpack_block32(hi_in, hi);
    const float* cs = s_cos + pl * H2 + kBlock * j;
    const float* sn = s_sin + pl * H2 + kBlock * j;
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const float x0 = lo[i], x1 = hi[i];
      const float c = cs[i], s = sn[i];
      lo[i] = x0 * c - x1 * s;  // RN32 of each product, then of the difference
      hi[i] = x1 * c + x0 * s;
    }
    if (a.scale != nullptr) {
      const int srow = h / a.heads_per_scale_row;
      const float* sc = staged ? s_scale + srow * D : a.scale + (int64_t)srow * D;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        lo[i] = lo[i] * sc[kBlock * j + i];
        hi[i] = hi[i] * sc[H2 + kBlock * j + i];
      }
    }
    uint4 c_lo, c_hi;
    const uint32_t e_lo = quantize_values32(lo, &c_lo);
    const uint32_t e_hi = quantize_values32(hi, &c_hi);
    *reinterpret_cast<uint4*>(a.codes + row * (D / 2) + 16 * j) = c_lo;
    *reinterpret_cast<uint4*>(a.codes + row * (D / 2) + 16 * (j + NP)) = c_hi;
    if (PLANES) {
      a.scales[(bh * NB + j) * a.len32 + tok] = (uint8_t)e_lo;
      a.scales[(bh * NB + j + NP) * a.len32 + tok] = (uint8_t)e_hi;
    } else {
      a.scales[row * NB + j] = (uint8_t)e_lo;
      a.scales[row * NB + j + NP] = (uint8_t)e_hi;
    }
  }
}

template <int D>
static hipError_t quant_rope_d(QuantRopeArgs a, hipStream_t s) {
  const int p = kRopeMaxPos;
  a.pos_per_wg = p;
  const int64_t n_tok = a.block_planes ? a.len32 : a.len;
  dim3 grid((uint32_t)((n_tok + p - 1) / p), (uint32_t)a.batch);
  if (a.block_planes) hipLaunchKernelGGL((quantize_rope_kernel<D, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((quantize_rope_kernel<D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_rope(QuantRopeArgs a, hipStream_t s) {
  switch (a.d) {
    case 64: return quant_rope_d<64>(a, s);
    case 128: return quant_rope_d<128>(a, s);
    case 256: return quant_rope_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Append n keys to a 4-bit cache, one work-group per (batch, KV head).  K-hat rows are
// independent: each new key is rotated (optional), rescaled and quantized into its row and its
// scale-plane column.  V-hat blocks run along keys, so every block the new keys touch is
// quantized again from FP16: keys before len0 come from the stage (the FP16 keys of the block
// that was still open), new keys from v_new, and positions past len0 + n are zero, exactly as
// the whole-sequence quantizer pads the last block.  The stage then receives the keys of the
// block left open, after every read of the old stage has happened (one barrier).
template <int D>
__global__ __launch_bounds__(256) void cache_append_kernel(CacheAppendArgs a) {
  constexpr int NB = D / kBlock;
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % a.heads_kv);
  const int64_t end = a.len0 + a.n;
  // K-hat: one thread per (new key, 32-channel block)
  for (int64_t it = threadIdx.x; it < a.n * NB; it += blockDim.x) {
    const int blk = (int)(it % NB);
    const int64_t t = it / NB, pos = a.len0 + t;
    const uint16_t* x = a.k_new + (bh * a.n + t) * D;
    const float* sc = a.inv_s ? a.inv_s + (int64_t)h * D + kBlock * blk : nullptr;
    uint4 out;
    const uint32_t e8 = a.rope_cos ? quantize_block32_rope(x, blk, D, a.rope_cos + pos * (D / 2),
                                                           a.rope_sin + pos * (D / 2), sc, &out)
                                   : quantize_block32(x + kBlock * blk, sc, &out);
    *reinterpret_cast<uint4*>(a.k_codes + (bh * a.rows + pos) * (D / 2) + 16 * blk) = out;
    a.k_scales[(bh * NB + blk) * a.rows32 + pos] = (uint8_t)e8;
  }
  // V-hat: every touched 32-key block, one thread per channel
  const int64_t open0 = a.len0 - a.len0 % kBlock;  // first key of the block that was open
  for (int64_t jb = a.len0 / kBlock; jb * kBlock < end; jb++) {
    for (int ch = threadIdx.x; ch < D; ch += blockDim.x) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; i++) {
        const int64_t p = jb * kBlock + i;
        uint16_t bits = 0;
        if (p < a.len0) bits = a.v_stage[(bh * kBlock + (p - open0)) * D + ch];
        else if (p < end) bits = a.v_new[(bh * a.n + (p - a.len0)) * D + ch];
        v[i] = (float)__builtin_bit_cast(_Float16, bits);
      }
      uint4 out;
      const uint32_t e8 = quantize_values32(v, &out);
      const int64_t blk_row = (bh * (a.rows32 / kBlock) + jb) * D;
      *reinterpret_cast<uint4*>(a.v_codes + (blk_row + ch) * 16) = out;
      a.v_scales[blk_row + (D / 16) * (ch % 16) + ch / 16] = (uint8_t)e8;
    }
  }
  __syncthreads();
  // the block left open: its keys (FP16) go to the stage for the next append
  const int64_t open1 = end - end % kBlock;
  for (int64_t it = threadIdx.x; it < (end - open1) * D; it += blockDim.x) {
    const int64_t p = open1 + it / D;
    const int ch = (int)(it % D);
    if (p >= a.len0)  // keys before len0 are in the stage already, in the same slot
      a.v_stage[(bh * kBlock + (p - open1)) * D + ch] = a.v_new[(bh * a.n + (p - a.len0)) * D + ch];
  }
}

hipError_t launch_cache_append(const CacheAppendArgs& a, hipStream_t s) {
  const dim3 grid((uint32_t)a.bh);
  switch (a.d) {
    case 64: hipLaunchKernelGGL(cache_append_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(cache_append_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(cache_append_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
