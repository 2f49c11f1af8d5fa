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
__device__ __forceinline__ void quantize_rows_block(const QuantRowsArgs& a, int64_t block) {
  constexpr int NB = D / kBlock;
  __shared__ __attribute__((aligned(16))) float s_row[D];
  const int64_t n_rows = PLANES ? a.rows / a.len * a.len32 : a.rows;
  const int64_t n_items = n_rows * NB;
  const int64_t t0 = block * blockDim.x;
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

template <int D, bool PLANES>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantRowsArgs a) {
  quantize_rows_block<D, PLANES>(a, blockIdx.x);
}

// V: blocks run along tokens, so a work-group stages one 32-token block x d channels in LDS and
// each thread quantizes (channel, block) items.  The output is block-major (for each 32-token
// block, all channels), so consecutive threads write consecutive 16-byte cells.  Small LDS tiles
// keep many work-groups in flight per CU (measured at B8 L4096 d128: 32-token tiles about 4 us
// faster than 128-token ones).
template <int D>
constexpr int vt_tokens() { return 32; }

template <int D>
__device__ __forceinline__ void quantize_vt_block(const QuantVtArgs& a, int64_t tile_idx, int64_t bh) {
  constexpr int TOK = vt_tokens<D>();
  constexpr int NBT = TOK / kBlock;  // 32-token blocks per tile
  constexpr int ROW = D + 8;  // FP16 elements per LDS row (padding breaks bank aliasing)
  __shared__ _Float16 tile[TOK * ROW];
  const int64_t t0 = tile_idx * TOK;
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

template <int D>
__global__ __launch_bounds__(256) void quantize_vt_kernel(QuantVtArgs a) {
  quantize_vt_block<D>(a, blockIdx.x, blockIdx.y);
}

// K-hat (block planes) and V-hat in one launch: work-groups [0, k_blocks) quantize K rows, the
// rest V tiles (tile fastest), so the K tail and the V start overlap instead of being separated
// by a kernel boundary.
template <int D>
__global__ __launch_bounds__(256) void quantize_kv_kernel(QuantRowsArgs ka, QuantVtArgs va, int64_t k_blocks,
                                                          int64_t v_tiles) {
  const int64_t blk = blockIdx.x;
  if (blk < k_blocks) {
    quantize_rows_block<D, true>(ka, blk);
  } else {
    const int64_t vb = blk - k_blocks;
    quantize_vt_block<D>(va, vb % v_tiles, vb / v_tiles);
  }
}

// RoPE (FP32, rotate-half), Smooth-QK and 4-bit quantization of pre-RoPE rows, fused.  An item
// is one (position, block pair j): channels 32 j .. 32 j + 31 of a row and their rotation
// partners 32 j + d/2 .., so each item writes two quantization blocks.  Four adjacent lanes
// share an item: lane q rotates channels 8 q .. 8 q + 7 of both blocks, the two block maxima are
// reduced over the four lanes, and each lane packs its 8 + 8 codes (4 bytes of each block's 16).
// A work-group takes 64 items (64 / (d/64) consecutive positions) of kRopeHeads heads of one
// batch entry: a lane reads its cos/sin entries once from the (L2-resident) tables and applies
// them to the same item of each head, and consecutive work-groups read consecutive rows of each
// head.  The heads' Smooth-QK rows are staged in LDS.  Rounding, as the rotation is defined for
// this prologue: each product and each sum once in FP32, no fused multiply-add (contraction is
// off), then fp32(y * s).
constexpr int kRopeHeads = 4;  // heads per work-group sharing each lane's cos/sin registers

template <int D>
constexpr int rope_positions() { return 64 / (D / 64); }

// Largest of v over the four lanes of an aligned quad (all four lanes active).
__device__ __forceinline__ float quad_max(float v) {
  const int b = __builtin_bit_cast(int, v);
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));  // lanes 1 0 3 2
  const int c = __builtin_bit_cast(int, v);
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(c, c, 0x4E, 0xF, 0xF, false)));  // 2 3 0 1
}

// The 8 FP16 values of one 16-byte load as FP32 (exact).
__device__ __forceinline__ void unpack8(const uint4& w, float* v) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[i] & 0xFFFF));
    v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[i] >> 16));
  }
}

// Work-group (bx, by, bz) of the RoPE quantizer's grid: position group bx, heads G by .. G by +
// G - 1, batch entry bz.
template <int D, bool PLANES>
__device__ __forceinline__ void quantize_rope_block(const QuantRopeArgs& a, int64_t bx, int by, int64_t bz) {
  constexpr int NB = D / kBlock;
  constexpr int NP = NB / 2;  // block pairs per row
  constexpr int H2 = D / 2;
  constexpr int G = kRopeHeads;
  constexpr int P = rope_positions<D>();  // P * NP = 64 items, one per quad
  constexpr int SV = (G * D + 255) / 256;  // staged Smooth-QK values per thread
  __shared__ __attribute__((aligned(16))) float s_scale[G * D];
  const int h0 = by * G;
  const int64_t b = bz;
  const int64_t tok = bx * P + (threadIdx.x >> 2) / NP;
  const int j = (threadIdx.x >> 2) % NP;
  const int q = threadIdx.x & 3;
  const int c = kBlock * j + 8 * q;  // the lane's first channel in the low block
  const bool scaled = a.scale != nullptr;
  // the loads go out in this order: the heads' Smooth-QK rows, then the table entries and the
  // rows, as straight-line code (the compiler counts loads in flight only outside branches); the
  // LDS writes wait for the first loads only, so the barrier and the rows' loads overlap in one
  // memory round trip.  Unscaled calls read unused table entries instead, heads past H and
  // tokens past the data read head H - 1 and row len - 1 without using them.
  float sv[SV];
#pragma unroll
  for (int i = 0; i < SV; i++) {
    const int e = i * 256 + threadIdx.x;  // (head g, channel) = (e / D, e % D)
    const int hs = min(h0 + (e / D) % G, a.heads - 1);
    sv[i] = scaled ? a.scale[(int64_t)(hs / a.heads_per_scale_row) * D + e % D] : a.rope_cos[e % H2];
  }
  __builtin_amdgcn_sched_barrier(0);  // keeps those loads ahead of the rows' loads
  const bool live = tok < a.len;
  const int64_t tc = live ? tok : a.len - 1;
  const float4* cp = reinterpret_cast<const float4*>(a.rope_cos + (a.pos0 + tc) * H2 + c);
  const float4* sp = reinterpret_cast<const float4*>(a.rope_sin + (a.pos0 + tc) * H2 + c);
  const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
  uint4 xl[G], xh[G];
#pragma unroll
  for (int g = 0; g < G; g++) {
    const int hg = min(h0 + g, a.heads - 1);
    const uint16_t* x = a.x + ((b * a.heads + hg) * a.len + tc) * D;
    xl[g] = *reinterpret_cast<const uint4*>(x + c);
    xh[g] = *reinterpret_cast<const uint4*>(x + H2 + c);
  }
#pragma unroll
  for (int i = 0; i < SV; i++)
    if (i * 256 + threadIdx.x < G * D) s_scale[i * 256 + threadIdx.x] = sv[i];
  __syncthreads();
  if (tok >= (PLANES ? a.len32 : a.len)) return;
  const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int g = 0; g < G; g++) {
    if (h0 + g >= a.heads) break;
    const int64_t bh = b * a.heads + h0 + g;
    if (!live) {  // padding key of a scale plane: zero scale bytes for both blocks
      if (PLANES && q < 2) a.scales[(bh * NB + j + q * NP) * a.len32 + tok] = 0;
      continue;
    }
    const int64_t row = bh * a.len + tok;
    float lo[8], hi[8];
    unpack8(xl[g], lo);
    unpack8(xh[g], hi);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float x0 = lo[i], x1 = hi[i];
      lo[i] = x0 * cs[i] - x1 * sn[i];  // RN32 of each product, then of the difference
      hi[i] = x1 * cs[i] + x0 * sn[i];
    }
    if (scaled) {
      const float* sc = s_scale + g * D + c;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo[i] = lo[i] * sc[i];
        hi[i] = hi[i] * sc[H2 + i];
      }
    }
    float ml = 0.0f, mh = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      ml = fmaxf(ml, fabsf(lo[i]));
      mh = fmaxf(mh, fabsf(hi[i]));
    }
    const int e_lo = mx_exponent(quad_max(ml)), e_hi = mx_exponent(quad_max(mh));
    uint8_t* crow = a.codes + row * (D / 2);
    *reinterpret_cast<uint32_t*>(crow + 16 * j + 4 * q) = pack8_fp4(lo, e8m0_as_float(e_lo));
    *reinterpret_cast<uint32_t*>(crow + 16 * (j + NP) + 4 * q) = pack8_fp4(hi, e8m0_as_float(e_hi));
    if (q < 2) {
      const uint8_t e8 = (uint8_t)((q == 0 ? e_lo : e_hi) + 127);
      if (PLANES) a.scales[(bh * NB + j + q * NP) * a.len32 + tok] = e8;
      else a.scales[row * NB + j + q * NP] = e8;
    }
  }
}

template <int D, bool PLANES>
__global__ __launch_bounds__(256) void quantize_rope_kernel(QuantRopeArgs a) {
  quantize_rope_block<D, PLANES>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Q-hat and K-hat with RoPE and V-hat in one launch: work-groups [0, nq) take the Q grid, the
// next nk the K grid (each flattened x fastest), the rest the V tiles (tile fastest), so no
// tensor waits for a kernel boundary.
template <int D>
__global__ __launch_bounds__(256) void quantize_qkv_rope_kernel(QuantRopeArgs qa, QuantRopeArgs ka, QuantVtArgs va,
                                                                dim3 qg, dim3 kg, int64_t v_tiles) {
  int64_t blk = blockIdx.x;
  const int64_t nq = (int64_t)qg.x * qg.y * qg.z;
  if (blk < nq) {
    quantize_rope_block<D, false>(qa, blk % qg.x, (int)((blk / qg.x) % qg.y), blk / ((int64_t)qg.x * qg.y));
    return;
  }
  blk -= nq;
  const int64_t nk = (int64_t)kg.x * kg.y * kg.z;
  if (blk < nk) {
    quantize_rope_block<D, true>(ka, blk % kg.x, (int)((blk / kg.x) % kg.y), blk / ((int64_t)kg.x * kg.y));
    return;
  }
  blk -= nk;
  quantize_vt_block<D>(va, blk % v_tiles, blk / v_tiles);
}

template <int D>
dim3 rope_grid(const QuantRopeArgs& a) {
  constexpr int p = rope_positions<D>();
  const int64_t n_tok = a.block_planes ? a.len32 : a.len;
  return dim3((uint32_t)((n_tok + p - 1) / p), (uint32_t)((a.heads + kRopeHeads - 1) / kRopeHeads), (uint32_t)a.batch);
}

template <int D>
static hipError_t quant_rope_d(QuantRopeArgs a, hipStream_t s) {
  const dim3 grid = rope_grid<D>(a);
  if (a.block_planes) hipLaunchKernelGGL((quantize_rope_kernel<D, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((quantize_rope_kernel<D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t quant_qkv_rope_d(const QuantRopeArgs& qa, const QuantRopeArgs& ka, const QuantVtArgs& va,
                                   hipStream_t s) {
  const dim3 qg = rope_grid<D>(qa), kg = rope_grid<D>(ka);
  const int64_t v_tiles = (va.len + vt_tokens<D>() - 1) / vt_tokens<D>();
  const int64_t blocks = (int64_t)qg.x * qg.y * qg.z + (int64_t)kg.x * kg.y * kg.z + v_tiles * va.bh;
  if (blocks >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_qkv_rope_kernel<D>, dim3((uint32_t)blocks), dim3(256), 0, s, qa, ka, va, qg, kg, v_tiles);
  return hipGetLastError();
}

hipError_t launch_quantize_qkv_rope(const QuantRopeArgs& qa, const QuantRopeArgs& ka, const QuantVtArgs& va,
                                    hipStream_t s) {
  if (qa.block_planes || !ka.block_planes || qa.d != ka.d || ka.d != va.d) return hipErrorInvalidValue;
  switch (qa.d) {
    case 64: return quant_qkv_rope_d<64>(qa, ka, va, s);
    case 128: return quant_qkv_rope_d<128>(qa, ka, va, s);
    case 256: return quant_qkv_rope_d<256>(qa, ka, va, s);
    default: return hipErrorInvalidValue;
  }
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
  constexpr int SI = kBlock * D / 256;  // stage elements per thread at most (256 threads)
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % a.heads_kv);
  const int64_t end = a.len0 + a.n;
  // K-hat: one thread per (new key, 32-channel block), on the threads the V-hat blocks leave
  // idle where there are any (d < 256), so the two parts' loads are in flight together
  constexpr int KT0 = D < 256 ? D : 0;
  if (threadIdx.x >= KT0) {
    for (int64_t it = threadIdx.x - KT0; it < a.n * NB; it += blockDim.x - KT0) {
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
  }
  // V-hat: every touched 32-key block, one thread per channel.  An element's source (the stage,
  // the new keys, or the zero padding past the last key) depends only on its position, the same
  // for every thread: the row is picked by uniform arithmetic, and the block's loads are in
  // flight together (padding inside a group of 8 reads the stage's first row and becomes 0)
  const int64_t open0 = a.len0 - a.len0 % kBlock;  // first key of the block that was open
  for (int64_t jb = a.len0 / kBlock; jb * kBlock < end; jb++) {
    for (int ch = threadIdx.x; ch < D; ch += blockDim.x) {
      uint32_t bits[32];
#pragma unroll
      for (int g8 = 0; g8 < 4; g8++) {
        if (jb * kBlock + 8 * g8 < end) {  // groups of 8 wholly past the last key are not read
#pragma unroll
          for (int i = 8 * g8; i < 8 * g8 + 8; i++) {
            const int64_t p = jb * kBlock + i;
            const uint16_t* src = p < a.len0 ? a.v_stage + (bh * kBlock + (p - open0)) * D
                                             : (p < end ? a.v_new + (bh * a.n + (p - a.len0)) * D
                                                        : a.v_stage + bh * kBlock * D);
            bits[i] = src[ch];
          }
        } else {
#pragma unroll
          for (int i = 8 * g8; i < 8 * g8 + 8; i++) bits[i] = 0u;
        }
      }
      // every value is needed here, so no conversion (and wait) moves into the branches above
#pragma unroll
      for (int i = 0; i < 32; i++) asm volatile("" ::"v"(bits[i]));
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; i++)
        v[i] = jb * kBlock + i < end ? (float)__builtin_bit_cast(_Float16, (uint16_t)bits[i]) : 0.0f;
      uint4 out;
      const uint32_t e8 = quantize_values32(v, &out);
      const int64_t blk_row = (bh * (a.rows32 / kBlock) + jb) * D;
      *reinterpret_cast<uint4*>(a.v_codes + (blk_row + ch) * 16) = out;
      a.v_scales[blk_row + (D / 16) * (ch % 16) + ch / 16] = (uint8_t)e8;
    }
  }
  // the block left open: its keys (FP16) go to the stage for the next append.  The new keys are
  // read before the barrier; the stage is written after it, once every read of the old stage is
  // done.  Keys before len0 are in the stage already, in the same slot.
  const int64_t open1 = end - end % kBlock;
  const int cnt = (int)((end - open1) * D);
  uint16_t sv[SI];
#pragma unroll
  for (int k = 0; k < SI; k++) {
    const int it = (int)threadIdx.x + 256 * k;
    const int64_t p = open1 + it / D;
    sv[k] = it < cnt && p >= a.len0 ? a.v_new[(bh * a.n + (p - a.len0)) * D + it % D] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < SI; k++) {
    const int it = (int)threadIdx.x + 256 * k;
    const int64_t p = open1 + it / D;
    if (it < cnt && p >= a.len0) a.v_stage[(bh * kBlock + (p - open1)) * D + it % D] = sv[k];
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

template <int D>
static hipError_t quant_kv_d(const QuantRowsArgs& ka, const QuantVtArgs& va, hipStream_t s) {
  const int64_t k_items = ka.rows / ka.len * ka.len32 * (D / kBlock);
  const int64_t k_blocks = (k_items + 255) / 256;
  const int64_t v_tiles = (va.len + vt_tokens<D>() - 1) / vt_tokens<D>();
  const int64_t blocks = k_blocks + v_tiles * va.bh;
  if (blocks >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_kv_kernel<D>, dim3((uint32_t)blocks), dim3(256), 0, s, ka, va, k_blocks, v_tiles);
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const QuantRowsArgs& ka, const QuantVtArgs& va, hipStream_t s) {
  if (!ka.block_planes || ka.d != va.d) return hipErrorInvalidValue;
  switch (ka.d) {
    case 64: return quant_kv_d<64>(ka, va, s);
    case 128: return quant_kv_d<128>(ka, va, s);
    case 256: return quant_kv_d<256>(ka, va, s);
    default: return hipErrorInvalidValue;
  }
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
