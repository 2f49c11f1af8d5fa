// K3: split-KV decode (one query token per sequence) and the FP16 (m, l, O) merge, gfx950.
//
// Decode is HBM-bound: every K-hat/V-hat byte is used by exactly one MFMA lane once, so the
// kernel skips LDS and loads each lane's MFMA operands straight from HBM into registers, one
// tile ahead of the computation (three when the grid leaves a SIMD at most one wave, where the
// bytes in flight per wave set the rate).  The query heads of a GQA group are the MFMA columns (the
// same S^T = K-hat Q-hat^T layout as the prefill kernel, see attn_prefill.hip), so a wave
// serves one (batch, KV head, split) and keeps its split's FP16 state in registers.
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace hifa4 {

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// The 4-bit K-hat and V-hat codes are read exactly once per call: their loads are marked
// non-temporal, so the stream does not displace the scale lines and the query in the caches
// (measured 12-14 % faster over a 2.3 GB cache; marking the scale loads too gained nothing).
__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int D>
struct TileOps {
  static constexpr int KSTEPS = D >= 128 ? D / 128 : 1;
  static constexpr int CB = D / 16;
  uint4 k[8][KSTEPS];   // K-hat A operands of the 8 score MFMAs (2 contraction steps for d = 256)
  uint2 ksc[KSTEPS];    // scale bytes of the 8 keys of the lane's MFMA row (byte t: MFMA t)
  uint4 v[CB];          // V-hat^T A operands of the channel blocks
  uint32_t vsc[CB / 4]; // scale bytes of the lane's CB channels (byte cb: channel 16 cb + col)
};

// HBM -> registers: this lane's MFMA operands of the tile at key k0 (see score_row_key and the
// channel map in device_common.h); keys past lk (or past the tile) read as code 0.
template <int D>
__device__ __forceinline__ void load_tile(TileOps<D>& t, const uint8_t* kc, const uint8_t* ks,
                                          const uint8_t* vc, const uint8_t* vs, int64_t k0,
                                          int64_t lk, int64_t lk32, int64_t plane, int bc, int col, int g) {
  constexpr int KSTEPS = TileOps<D>::KSTEPS;
  constexpr int CB = TileOps<D>::CB;
  const bool lane_k = D >= 128 || g < 2;
#pragma unroll
  for (int tt = 0; tt < 8; tt++) {
    const int kr = score_row_key(tt, col);
    const int64_t key = k0 + kr;
    const bool ok = kr < bc && key < lk && lane_k;
#pragma unroll
    for (int st = 0; st < KSTEPS; st++)
      t.k[tt][st] = ok ? load_nt16(kc + key * (D / 2) + 64 * st + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
  }
  // the 8 keys k0 + 32 (col/4) + 8 (col%4) + 0..7 lie in one 32-key block of the padded rows
  const int64_t kfirst = k0 + 32 * (col >> 2) + 8 * (col & 3);
#pragma unroll
  for (int st = 0; st < KSTEPS; st++)
    t.ksc[st] = (kfirst < lk32 && lane_k) ? *reinterpret_cast<const uint2*>(ks + (int64_t)(4 * st + g) * plane + kfirst)
                                          : make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  const bool okv = 32 * g < bc && k0 + 32 * g < lk32;
  const int64_t row = (k0 / kBlock + g) * D;  // block-major V-hat: cells (32-key block, channel)
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
    t.v[cb] = okv ? load_nt16(vc + (row + 16 * cb + col) * 16) : make_uint4(0u, 0u, 0u, 0u);
  if constexpr (CB == 4) {
    t.vsc[0] = okv ? *reinterpret_cast<const uint32_t*>(vs + row + CB * col) : 0x7F7F7F7Fu;
  } else if constexpr (CB == 8) {
    const uint2 w = okv ? *reinterpret_cast<const uint2*>(vs + row + CB * col) : make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    t.vsc[0] = w.x;
    t.vsc[1] = w.y;
  } else {
    const uint4 w = okv ? *reinterpret_cast<const uint4*>(vs + row + CB * col)
                        : make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
    t.vsc[0] = w.x;
    t.vsc[1] = w.y;
    t.vsc[2] = w.z;
    t.vsc[3] = w.w;
  }
}

// One tile of the split kernel: scores, masking, row step, P-hat, P-hat [V-hat | 1] and the FP16
// state update (o, l, m of the lane's query)
template <int D, int MODE, int PH>
__device__ __forceinline__ void decode_tile(const TileOps<D>& t_ops, int tile, int bc, int g, int64_t lk, int64_t shift,
                                            bool live_col, const uint4* qreg, const uint32_t* qsc, h2 (*o)[2],
                                            _Float16& l, float& m) {
  constexpr int KSTEPS = TileOps<D>::KSTEPS;
  constexpr int CB = TileOps<D>::CB;
  constexpr float C = SoftmaxC<D>::value;
  const int64_t k0 = (int64_t)tile * bc;
  float s[32];
#pragma unroll
  for (int tt = 0; tt < 8; tt++) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < KSTEPS; st++) {
      const uint32_t kw = tt < 4 ? t_ops.ksc[st].x : t_ops.ksc[st].y;
      switch (tt & 3) {
        case 0: acc = mfma_fp4_sel<0, 0>(t_ops.k[tt][st], kw, qreg[st], qsc[st], acc); break;
        case 1: acc = mfma_fp4_sel<1, 0>(t_ops.k[tt][st], kw, qreg[st], qsc[st], acc); break;
        case 2: acc = mfma_fp4_sel<2, 0>(t_ops.k[tt][st], kw, qreg[st], qsc[st], acc); break;
        default: acc = mfma_fp4_sel<3, 0>(t_ops.k[tt][st], kw, qreg[st], qsc[st], acc); break;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) s[4 * tt + i] = acc[i];
  }
  float bmax = -INFINITY;
#pragma unroll
  for (int k = 0; k < 32; k++) {
    const int64_t key = k0 + 32 * g + s_key(k);
    const bool vis = (32 * g + k < bc) && key < lk && key <= shift && live_col;
    s[k] = vis ? s[k] : -INFINITY;
    bmax = fmaxf(bmax, s[k]);
  }
  const float rmax = group_max4(bmax);
  // integer running max and FP16 rescale factor (all four lane groups hold the same row
  // maximum, so they agree); the P-hat scale of the lane's own 32-key block
  const RowStep rs = row_step(rmax, m, C);
  const PhatScale ps = phat_scale<PH == 2>(PH == 1 ? rmax : bmax, C, rs.mm);
  uint32_t p16[16];
  uint4 ph;
  if constexpr (PH == 2) ph = phat_codes_direct(s, C, ps.neg_big_m);
  else ph = phat_codes(s, C, ps.neg_big_m, p16);
  const uint32_t psc = (uint32_t)(int)(ps.e + 127.0f);
  const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
  v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
  lacc = mfma_fp4(ones, 127u, ph, psc, lacc);
  float lsum = lacc[0];
  if (MODE == 1) lsum = group_sum4(tree_sum32_h(p16) * e8m0_as_float((int)ps.e));
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    v4f pv = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t vw = t_ops.vsc[cb / 4];
    switch (cb & 3) {
      case 0: pv = mfma_fp4_sel<0, 0>(t_ops.v[cb], vw, ph, psc, pv); break;
      case 1: pv = mfma_fp4_sel<1, 0>(t_ops.v[cb], vw, ph, psc, pv); break;
      case 2: pv = mfma_fp4_sel<2, 0>(t_ops.v[cb], vw, ph, psc, pv); break;
      default: pv = mfma_fp4_sel<3, 0>(t_ops.v[cb], vw, ph, psc, pv); break;
    }
    state_update(o[cb], rs.alpha, pv);
  }
  l = __builtin_fmaf16(rs.alpha, l, (_Float16)lsum);
  m = rs.m_new;
}

// PH: the P-hat rule, as in the prefill kernel (0 = per 32-key block from the FP16 probabilities,
// 1 = per tile, 2 = Direct-P codes).  R: register sets of tile operands, so R - 1 tiles are in
// flight while one is computed: 2 when the grid fills the SIMDs with waves (registers allow two
// waves per SIMD), 4 when it leaves them at one wave or fewer (small batches), where the bytes
// in flight per wave set the rate.
template <int D, int MODE, int PH, int R>
__global__ __launch_bounds__(64) void attn_decode_split_kernel(AttnArgs a) {
  constexpr int KSTEPS = D >= 128 ? D / 128 : 1;
  constexpr int CB = D / 16;
  const int lane = threadIdx.x;
  const int g = lane >> 4, col = lane & 15;
  const int split = blockIdx.x;
  const int group = a.heads_q / a.heads_kv;
  const int hchunk = blockIdx.y % ((group + 15) / 16);
  const int kvh = blockIdx.y / ((group + 15) / 16);
  const int b = blockIdx.z;
  const int hl = 16 * hchunk + col;            // query head within the group (MFMA column)
  const bool live_col = hl < group;
  const int h = kvh * group + (live_col ? hl : 0);
  const int64_t lk = a.len_kv, lk32 = a.len_kv32;
  const int bc = a.kv_tile;

  const int t_lo = split * a.tiles_per_split;
  int t_hi = t_lo + a.tiles_per_split;
  if (t_hi > a.n_tiles) t_hi = a.n_tiles;

  // slices start at the buffers' strides (the rows allocated per (batch, KV head))
  const int64_t rows = a.kv_rows, rows32 = a.kv_rows32;
  const uint8_t* kc = a.k_codes + ((int64_t)b * a.heads_kv + kvh) * rows * (D / 2);
  const uint8_t* ks = a.k_scales + ((int64_t)b * a.heads_kv + kvh) * rows32 * (D / kBlock);
  const uint8_t* vc = a.v_codes + ((int64_t)b * a.heads_kv + kvh) * D * (rows32 / 2);
  const uint8_t* vs = a.v_scales + ((int64_t)b * a.heads_kv + kvh) * D * (rows32 / kBlock);
  // the first R - 1 tiles are put in flight before the query is loaded, so the latencies overlap
  TileOps<D> buf[R];
#pragma unroll
  for (int u = 0; u < R - 1; u++)
    if (t_lo + u < t_hi) load_tile<D>(buf[u], kc, ks, vc, vs, (int64_t)(t_lo + u) * bc, lk, lk32, rows32, bc, col, g);

  // Q-hat^T operand: column = query head, K-chunk g
  uint4 qreg[KSTEPS];
  uint32_t qsc[KSTEPS];
  if (a.q_fp16 != nullptr) {
    // FP16 Q: this lane quantizes its own 32-element block (4 st + g) of query head h
    const uint16_t* qx = a.q_fp16 + ((int64_t)b * a.heads_q + h) * D;
#pragma unroll
    for (int st = 0; st < KSTEPS; st++) {
      qreg[st] = make_uint4(0u, 0u, 0u, 0u);
      qsc[st] = 127u;
      if (live_col && (D >= 128 || g < 2)) {
        const int c0 = 128 * st + 32 * g;
        const float* sm = a.q_smooth ? a.q_smooth + (int64_t)kvh * D + c0 : nullptr;
        if (a.rope_cos != nullptr) {
          // FP16 query before RoPE, at position Lk - 1
          qsc[st] = quantize_block32_rope(qx, 4 * st + g, D, a.rope_cos + (lk - 1) * (D / 2),
                                          a.rope_sin + (lk - 1) * (D / 2), sm, &qreg[st]);
        } else {
          qsc[st] = quantize_block32(qx + c0, sm, &qreg[st]);
        }
      }
    }
  } else {
    const uint8_t* qc = a.q_codes + ((int64_t)b * a.heads_q + h) * (D / 2);
    const uint8_t* qs = a.q_scales + ((int64_t)b * a.heads_q + h) * (D / kBlock);
#pragma unroll
    for (int st = 0; st < KSTEPS; st++) {
      const bool ok = live_col && (D >= 128 || g < 2);
      qreg[st] = ok ? *reinterpret_cast<const uint4*>(qc + 64 * st + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
      qsc[st] = ok ? qs[4 * st + g] : 127u;
    }
  }

  constexpr float C = SoftmaxC<D>::value;  // equals a.c_log2 (checked by the launcher)
  const int64_t shift = lk - 1;

  h2 o[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; cb++) o[cb][0] = o[cb][1] = h2{(_Float16)0.0f, (_Float16)0.0f};
  _Float16 l = (_Float16)0.0f;
  float m = -INFINITY;

  if constexpr (R == 2) {
    // one tile ahead: the next tile loads into nxt, which then becomes cur.  The tile body is
    // decode_tile's, written out here: through the function this loop ran 2 % slower (register
    // allocation), while the ring below gains from it
    TileOps<D>& cur = buf[0];
    TileOps<D>& nxt = buf[1];
    for (int tile = t_lo; tile < t_hi; tile++) {
      if (tile + 1 < t_hi) load_tile<D>(nxt, kc, ks, vc, vs, (int64_t)(tile + 1) * bc, lk, lk32, rows32, bc, col, g);
      const int64_t k0 = (int64_t)tile * bc;
      float s[32];
#pragma unroll
      for (int tt = 0; tt < 8; tt++) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KSTEPS; st++) {
          const uint32_t kw = tt < 4 ? cur.ksc[st].x : cur.ksc[st].y;
          switch (tt & 3) {
            case 0: acc = mfma_fp4_sel<0, 0>(cur.k[tt][st], kw, qreg[st], qsc[st], acc); break;
            case 1: acc = mfma_fp4_sel<1, 0>(cur.k[tt][st], kw, qreg[st], qsc[st], acc); break;
            case 2: acc = mfma_fp4_sel<2, 0>(cur.k[tt][st], kw, qreg[st], qsc[st], acc); break;
            default: acc = mfma_fp4_sel<3, 0>(cur.k[tt][st], kw, qreg[st], qsc[st], acc); break;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) s[4 * tt + i] = acc[i];
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const int64_t key = k0 + 32 * g + s_key(k);
        const bool vis = (32 * g + k < bc) && key < lk && key <= shift && live_col;
        s[k] = vis ? s[k] : -INFINITY;
        bmax = fmaxf(bmax, s[k]);
      }
      const float rmax = group_max4(bmax);
      // integer running max and FP16 rescale factor (all four lane groups hold the same row
      // maximum, so they agree); the P-hat scale of the lane's own 32-key block
      const RowStep rs = row_step(rmax, m, C);
      const PhatScale ps = phat_scale<PH == 2>(PH == 1 ? rmax : bmax, C, rs.mm);
      uint32_t p16[16];
      uint4 ph;
      if constexpr (PH == 2) ph = phat_codes_direct(s, C, ps.neg_big_m);
      else ph = phat_codes(s, C, ps.neg_big_m, p16);
      const uint32_t psc = (uint32_t)(int)(ps.e + 127.0f);
      const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
      v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
      lacc = mfma_fp4(ones, 127u, ph, psc, lacc);
      float lsum = lacc[0];
      if (MODE == 1) lsum = group_sum4(tree_sum32_h(p16) * e8m0_as_float((int)ps.e));
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        v4f pv = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t vw = cur.vsc[cb / 4];
        switch (cb & 3) {
          case 0: pv = mfma_fp4_sel<0, 0>(cur.v[cb], vw, ph, psc, pv); break;
          case 1: pv = mfma_fp4_sel<1, 0>(cur.v[cb], vw, ph, psc, pv); break;
          case 2: pv = mfma_fp4_sel<2, 0>(cur.v[cb], vw, ph, psc, pv); break;
          default: pv = mfma_fp4_sel<3, 0>(cur.v[cb], vw, ph, psc, pv); break;
        }
        state_update(o[cb], rs.alpha, pv);
      }
      l = __builtin_fmaf16(rs.alpha, l, (_Float16)lsum);
      m = rs.m_new;
      if (tile + 1 < t_hi) cur = nxt;
    }
  } else {
    // ring of R operand sets: tile t uses set (t - t_lo) % R; before computing it, tile t + R - 1
    // is put in flight into the set tile t - 1 used
    for (int base = t_lo; base < t_hi; base += R) {
#pragma unroll
      for (int u = 0; u < R; u++) {
        const int tile = base + u;
        if (tile >= t_hi) break;
        if (tile + R - 1 < t_hi)
          load_tile<D>(buf[(u + R - 1) % R], kc, ks, vc, vs, (int64_t)(tile + R - 1) * bc, lk, lk32, rows32, bc, col, g);
        decode_tile<D, MODE, PH>(buf[u], tile, bc, g, lk, shift, live_col, qreg, qsc, o, l, m);
      }
    }
  }

  if (!live_col) return;
  const int64_t part = ((int64_t)b * a.heads_q + h) * a.num_splits + split;
  // register i of block cb holds channel 16 cb + 4 g + i: 4 adjacent channels per block
  uint16_t* po = a.part_o + part * D + 4 * g;
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
    *reinterpret_cast<uint2*>(po + 16 * cb) =
        make_uint2(__builtin_bit_cast(uint32_t, o[cb][0]), __builtin_bit_cast(uint32_t, o[cb][1]));
  if (g == 0) {
    a.part_ml[part * 2 + 0] = __builtin_bit_cast(uint16_t, (_Float16)m);
    a.part_ml[part * 2 + 1] = __builtin_bit_cast(uint16_t, (_Float16)l);
  }
}

// Sequential FP16 merge of the split states, one thread per (batch, head, channel).  The merge
// steps run in split order, but the partials of kMergeChunk splits are loaded together first, so
// a call waits one memory round trip per chunk instead of one per split (at B = 1 with 32 splits
// the one-per-split loop took 13 us, two thirds of the split kernel's time).
constexpr int kMergeChunk = 16;

template <int D>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(AttnArgs a) {
  const int64_t bh = blockIdx.x;
  const int ch = threadIdx.x;
  float m = -INFINITY, l = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < a.num_splits; s0 += kMergeChunk) {
    float msv[kMergeChunk], lsv[kMergeChunk], osv[kMergeChunk];
#pragma unroll
    for (int i = 0; i < kMergeChunk; i++) {
      const int64_t part = bh * a.num_splits + (s0 + i < a.num_splits ? s0 + i : a.num_splits - 1);
      const bool in = s0 + i < a.num_splits;
      const float ms = (float)__builtin_bit_cast(_Float16, a.part_ml[part * 2 + 0]);
      msv[i] = in ? ms : -INFINITY;
      lsv[i] = (float)__builtin_bit_cast(_Float16, a.part_ml[part * 2 + 1]);
      osv[i] = (float)__builtin_bit_cast(_Float16, a.part_o[part * D + ch]);
    }
    // all of the chunk's values are needed here, so none of their loads sinks into the
    // conditional merge step below (which would put one round trip per split back)
#pragma unroll
    for (int i = 0; i < kMergeChunk; i++) asm volatile("" ::"v"(msv[i]), "v"(lsv[i]), "v"(osv[i]));
#pragma unroll
    for (int i = 0; i < kMergeChunk; i++) {
      const float ms = msv[i];
      if (!(ms > -INFINITY)) continue;  // the split saw no key (or lies past the last split)
      const float mn = fmaxf(m, ms);
      const float a1 = (m == -INFINITY) ? 0.0f : __builtin_ldexpf(1.0f, (int)(m - mn));
      const float a2 = __builtin_ldexpf(1.0f, (int)(ms - mn));
      const float mo = a2 * osv[i];
      const float ml = a2 * lsv[i];
      // each fma is rounded to FP32 and then to FP16 (keep_f32: not fused into one FP16 rounding)
      o = (float)(_Float16)keep_f32(__builtin_fmaf(a1, o, mo));
      l = (float)(_Float16)keep_f32(__builtin_fmaf(a1, l, ml));
      m = mn;
    }
  }
  a.out[bh * D + ch] = __builtin_bit_cast(uint16_t, (_Float16)(o / l));
}

// compute units of the current device (cached per device)
int device_cus() {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static int cus[kDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
  }
  return cus[dev];
}

template <int D, int R>
void launch_split(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.normalizer == 1) hipLaunchKernelGGL((attn_decode_split_kernel<D, 1, 0, R>), grid, dim3(64), 0, s, a);
  else if (a.phat == 1) hipLaunchKernelGGL((attn_decode_split_kernel<D, 0, 1, R>), grid, dim3(64), 0, s, a);
  else if (a.phat == 2) hipLaunchKernelGGL((attn_decode_split_kernel<D, 0, 2, R>), grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((attn_decode_split_kernel<D, 0, 0, R>), grid, dim3(64), 0, s, a);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  if (a.c_log2 != SoftmaxC<D>::value) return hipErrorInvalidValue;  // the kernel's constant must be the caller's C
  const int group = a.heads_q / a.heads_kv;
  dim3 grid((uint32_t)a.num_splits, (uint32_t)(a.heads_kv * ((group + 15) / 16)), (uint32_t)a.batch);
  // one wave per work-group: with no more waves than SIMDs, each wave keeps three tiles in flight
  // (d <= 128; d = 256 operand sets do not fit four times in the registers)
  const int64_t waves = (int64_t)grid.x * grid.y * grid.z;
  if (D <= 128 && waves <= 4 * (int64_t)device_cus()) launch_split<D, D <= 128 ? 4 : 2>(a, grid, s);
  else launch_split<D, 2>(a, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((uint32_t)((int64_t)a.batch * a.heads_q)), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// ---- fixed device scratch for callers that cannot allocate (hifa4_attention_fwd_q16_noalloc)
//
// The split partials of one decode call live in this array instead of a caller workspace.  Each
// GPU the library runs on holds its own copy (at its own address) until the process ends.  In
// host code the name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current, and only that
// address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of scratch per device, nullptr until looked up
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace hifa4
