// K2: fused 4-bit attention forward (prefill, non-causal and causal) for gfx950.
//
// HiFA4 abstract: QK^T and PV run as 4-bit matrix products, the online-softmax state (m, l, O)
// is FP16, and the normalizer is accumulated from the same quantized P-hat that enters the PV
// product (P-Reordering), so it comes out of that product: P-hat times [V-hat | 1].
//
// Work decomposition.  A work-group serves one (batch, KV head) and BQ query positions of each
// of HW query heads of the group (HW * BQ / 32 = 8 waves); every K-hat/V-hat tile staged in LDS
// is shared by all of them (GQA).  A wave owns 32 query rows of one head, as two 16-column
// blocks of the 16x16x128 scaled FP4 MFMA.
//
// Layout trick.  Scores are computed transposed, S^T = K-hat Q-hat^T, so a query is an MFMA
// column and lives in lanes (l % 16) of all four 16-lane groups.  MFMA t (t = 0..7) takes key
// 32*(r/4) + 4t + (r%4) as its row r; its output register i of lane group g then holds key
// 32g + 4t + i.  After the 8 MFMAs each lane holds the 32 contiguous keys of one 32-key block of
// its query: exactly the per-lane slice the PV MFMA consumes as its B operand (P-hat^T), so
// P-hat is quantized and packed in registers without any data exchange; its scale (one per
// query and tile) needs only the row maximum, two shuffles.  O^T = V-hat^T P-hat^T then puts a
// query's outputs in its own lanes too, so the FP16 state update needs no shuffles either.
#include "device_common.h"
#include "launch.h"

namespace hifa4 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

template <int D>
struct Smem {
  static constexpr int KROW = D / 2;        // bytes of K-hat codes per key
  static constexpr int KSROW = D / kBlock;  // K-hat scale bytes per key
  uint8_t kc[kTileKeys * KROW];
  uint8_t ks[kTileKeys * KSROW];
  uint8_t vc[D * (kTileKeys / 2)];
  uint8_t vs[D * (kTileKeys / kBlock)];
};

__device__ __forceinline__ float wave_sum16(float x) {  // sum over the 16 lanes sharing l / 16
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <int D, bool CAUSAL, int MODE, bool STATS>
__global__ __launch_bounds__(kThreads) void attn_prefill_kernel(AttnArgs a) {
  constexpr int KSTEPS = D >= 128 ? D / 128 : 1;  // MFMA contractions over d
  constexpr int CB = D / 16;                      // 16-channel output blocks
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;   // lane group: K-chunk of the MFMA operands / key block of P-hat
  const int col = lane & 15; // MFMA column: query within a 16-column block

  const int group = a.heads_q / a.heads_kv;
  const int hw = group < kWaves ? group : kWaves;  // query heads per work-group
  const int bq = 32 * (kWaves / hw);               // query positions per head per work-group
  const int chunks = group / hw;
  const int kvh = blockIdx.y / chunks;
  const int h = kvh * group + (blockIdx.y % chunks) * hw + wave / (bq / 32);
  const int b = blockIdx.z;
  const int64_t q_wg = (int64_t)blockIdx.x * bq;
  const int64_t q_base = q_wg + 32 * (wave % (bq / 32));
  const int64_t lq = a.len_q, lk = a.len_kv;
  const int64_t shift = lk - lq;  // causal: key c visible to query r iff c <= r + shift
  const int bc = a.kv_tile;

  // ---- Q-hat^T operands (B operand of the score MFMA), kept in registers
  uint4 qreg[2][KSTEPS];
  uint32_t qsc[2][KSTEPS];
  const uint8_t* qc = a.q_codes + ((int64_t)b * a.heads_q + h) * lq * (D / 2);
  const uint8_t* qs = a.q_scales + ((int64_t)b * a.heads_q + h) * lq * (D / kBlock);
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int64_t q = q_base + 16 * qb + col;
#pragma unroll
    for (int s = 0; s < KSTEPS; s++) {
      qreg[qb][s] = make_uint4(0u, 0u, 0u, 0u);
      qsc[qb][s] = 127u;
      const bool has = q < lq && (D >= 128 || g < 2);
      if (has) {
        qreg[qb][s] = *reinterpret_cast<const uint4*>(qc + q * (D / 2) + 64 * s + 16 * g);
        qsc[qb][s] = qs[q * (D / kBlock) + 4 * s + g];
      }
    }
  }

  // ---- FP16 state (stored as FP16 values), running max m as an integer-valued float
  h2 o[2][CB][2];
  float l[2], m[2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    l[qb] = 0.0f;
    m[qb] = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      o[qb][cb][0] = h2{(_Float16)0.0f, (_Float16)0.0f};
      o[qb][cb][1] = h2{(_Float16)0.0f, (_Float16)0.0f};
    }
  }

  int64_t last_row = q_wg + bq - 1;
  if (last_row > lq - 1) last_row = lq - 1;
  int n_tiles = a.n_tiles;
  if (CAUSAL) {
    const int64_t kmax = last_row + shift;  // last key any row of this work-group sees
    const int need = (int)(kmax / bc) + 1;
    n_tiles = need < n_tiles ? need : n_tiles;
  }
  const int64_t nrb = (lq + 31) / 32;
  float* stats_row = nullptr;
  if (STATS && q_base < lq) {
    stats_row = a.stats + ((((int64_t)b * a.heads_q + h) * nrb) + q_base / 32) * a.n_tiles * 2;
    for (int i = lane; i < a.n_tiles * 2; i += 64) stats_row[i] = 0.0f;
  }

  const uint8_t* kc_g = a.k_codes + ((int64_t)b * a.heads_kv + kvh) * lk * (D / 2);
  const uint8_t* ks_g = a.k_scales + ((int64_t)b * a.heads_kv + kvh) * lk * (D / kBlock);
  const uint8_t* vc_g = a.v_codes + ((int64_t)b * a.heads_kv + kvh) * D * (a.len_kv32 / 2);
  const uint8_t* vs_g = a.v_scales + ((int64_t)b * a.heads_kv + kvh) * D * (a.len_kv32 / kBlock);
  const float C = a.c_log2;

  for (int tile = 0; tile < n_tiles; tile++) {
    const int64_t k0 = (int64_t)tile * bc;
    __syncthreads();  // previous tile's operands are no longer read
    // ---- stage K-hat (codes, scales) and V-hat^T (codes, scales) of keys [k0, k0 + bc)
    for (int c = threadIdx.x; c < kTileKeys * (D / 32); c += kThreads) {
      const int r = c / (D / 32), part = c % (D / 32);
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (r < bc && k0 + r < lk) val = *reinterpret_cast<const uint4*>(kc_g + (k0 + r) * (D / 2) + 16 * part);
      *reinterpret_cast<uint4*>(&sm.kc[r * (D / 2) + 16 * part]) = val;
    }
    for (int c = threadIdx.x; c < kTileKeys * (D / kBlock); c += kThreads) {
      const int r = c / (D / kBlock);
      uint8_t val = 127;
      if (r < bc && k0 + r < lk) val = ks_g[(k0 + r) * (D / kBlock) + c % (D / kBlock)];
      sm.ks[c] = val;
    }
    for (int c = threadIdx.x; c < D * 4; c += kThreads) {
      const int ch = c / 4, part = c % 4;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      uint8_t sval = 127;
      if (32 * part < bc && k0 + 32 * part < a.len_kv32) {
        val = *reinterpret_cast<const uint4*>(vc_g + (int64_t)ch * (a.len_kv32 / 2) + k0 / 2 + 16 * part);
        sval = vs_g[(int64_t)ch * (a.len_kv32 / kBlock) + k0 / kBlock + part];
      }
      *reinterpret_cast<uint4*>(&sm.vc[ch * 64 + 16 * part]) = val;
      sm.vs[ch * 4 + part] = sval;
    }
    __syncthreads();

    if (q_base >= lq) continue;
    if (CAUSAL && k0 > q_base + 31 + shift) continue;

    float sum_phat = 0.0f, sum_p = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      const int64_t q = q_base + 16 * qb + col;
      // ---- S^T = K-hat Q-hat^T: lane holds keys k0 + 32 g + (4 t + i)
      float s[32];
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const int kr = 32 * (col >> 2) + 4 * t + (col & 3);  // MFMA row -> key within the tile
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KSTEPS; st++) {
          uint4 ka = make_uint4(0u, 0u, 0u, 0u);
          uint32_t kscale = 127u;
          if (D >= 128 || g < 2) {
            ka = *reinterpret_cast<const uint4*>(&sm.kc[kr * (D / 2) + 64 * st + 16 * g]);
            kscale = sm.ks[kr * (D / kBlock) + 4 * st + g];
          }
          acc = mfma_fp4(ka, kscale, qreg[qb][st], qsc[qb][st], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) s[4 * t + i] = acc[i];
      }
      // ---- visibility
      float bmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const int64_t key = k0 + 32 * g + k;
        bool vis = (32 * g + k < bc) && key < lk && q < lq;
        if (CAUSAL) vis = vis && key <= q + shift;
        s[k] = vis ? s[k] : -INFINITY;
        bmax = fmaxf(bmax, s[k]);
      }
      float rmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      // ---- integer running max and the exact rescale factor
      const float m_old = m[qb];
      const float m_new = fmaxf(m_old, __builtin_ceilf(rmax * C));
      float alpha = 1.0f;
      if (m_new != m_old) alpha = (m_old == -INFINITY) ? 0.0f : __builtin_ldexpf(1.0f, (int)(m_old - m_new));
      const float negm = (m_new == -INFINITY) ? 0.0f : -m_new;
      // ---- P-tilde and P-hat (4-bit, block of the lane's 32 keys)
      // P-hat: one scale per (query, tile) from the tile's largest score (all four lane groups agree)
      int e = -127;
      if (rmax != -INFINITY) e = mx_exponent(exp2_x(__builtin_fmaf(rmax, C, negm), a.c1, a.c2, a.c3));
      const float scl = e8m0_as_float(e);
      float p[32];
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const float x = exp2_x(__builtin_fmaf(s[k], C, negm), a.c1, a.c2, a.c3);
        p[k] = s[k] == -INFINITY ? 0.0f : x;
      }
      uint4 ph;
      ph.x = pack8_fp4(p + 0, scl);
      ph.y = pack8_fp4(p + 8, scl);
      ph.z = pack8_fp4(p + 16, scl);
      ph.w = pack8_fp4(p + 24, scl);
      const uint32_t psc = (uint32_t)(e + 127);
      // ---- normalizer increment: rowsum(P-hat) from the ones column, or the FP32 tree sum
      const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
      v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
      lacc = mfma_fp4(ones, 127u, ph, psc, lacc);
      float lsum = lacc[0];
      float ptree = 0.0f;
      if (MODE == 1 || STATS) {
        float t16[16];
#pragma unroll
        for (int k = 0; k < 16; k++) t16[k] = p[k] + p[k + 16];
#pragma unroll
        for (int k = 0; k < 8; k++) t16[k] = t16[k] + t16[k + 8];
#pragma unroll
        for (int k = 0; k < 4; k++) t16[k] = t16[k] + t16[k + 4];
#pragma unroll
        for (int k = 0; k < 2; k++) t16[k] = t16[k] + t16[k + 2];
        const float sb = t16[0] + t16[1];
        const float s01 = sb + __shfl_xor(sb, 16);
        ptree = s01 + __shfl_xor(s01, 32);
        if (MODE == 1) lsum = ptree;
        if (STATS) {
          sum_p += sb;
          sum_phat += (g == 0) ? lacc[0] : 0.0f;
        }
      }
      // ---- O^T += V-hat^T P-hat^T per 16-channel block; FP16 state update
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const int ch = 16 * cb + col;
        const uint4 va = *reinterpret_cast<const uint4*>(&sm.vc[ch * 64 + 16 * g]);
        const uint32_t vsc = sm.vs[ch * 4 + g];
        v4f pv = {0.0f, 0.0f, 0.0f, 0.0f};
        pv = mfma_fp4(va, vsc, ph, psc, pv);
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const float o0 = __builtin_fmaf(alpha, (float)o[qb][cb][hh][0], pv[2 * hh]);
          const float o1 = __builtin_fmaf(alpha, (float)o[qb][cb][hh][1], pv[2 * hh + 1]);
          o[qb][cb][hh] = h2{(_Float16)o0, (_Float16)o1};
        }
      }
      l[qb] = (float)(_Float16)__builtin_fmaf(alpha, l[qb], lsum);
      m[qb] = m_new;
    }
    if (STATS) {
      // sum over the wave: P-tilde per lane block, P-hat once per query (lane group 0)
      float sp = sum_p, sh = sum_phat;
      sp += __shfl_xor(sp, 16);
      sp += __shfl_xor(sp, 32);
      sp = wave_sum16(sp);
      sh = wave_sum16(sh);
      if (lane == 0) {
        stats_row[tile * 2 + 0] = sh;
        stats_row[tile * 2 + 1] = sp;
      }
    }
  }

  // ---- epilogue: out = fp16(O / l); lane holds channels 16 cb + 4 g + i of its query
  if (q_base >= lq) return;
  uint16_t* out = a.out + ((int64_t)b * a.heads_q + h) * lq * D;
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int64_t q = q_base + 16 * qb + col;
    if (q >= lq) continue;
    const float lv = l[qb];
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      const _Float16 r0 = (_Float16)((float)o[qb][cb][0][0] / lv);
      const _Float16 r1 = (_Float16)((float)o[qb][cb][0][1] / lv);
      const _Float16 r2 = (_Float16)((float)o[qb][cb][1][0] / lv);
      const _Float16 r3 = (_Float16)((float)o[qb][cb][1][1] / lv);
      uint2 w;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16);
      *reinterpret_cast<uint2*>(out + q * D + 16 * cb + 4 * g) = w;
    }
  }
}

template <int D, bool CAUSAL, int MODE, bool STATS>
hipError_t launch4(const AttnArgs& a, hipStream_t s) {
  const int group = a.heads_q / a.heads_kv;
  const int hw = group < kWaves ? group : kWaves;
  const int bq = 32 * (kWaves / hw);
  const int64_t qblocks = (a.len_q + bq - 1) / bq;
  dim3 grid((uint32_t)qblocks, (uint32_t)(a.heads_kv * (group / hw)), (uint32_t)a.batch);
  hipLaunchKernelGGL((attn_prefill_kernel<D, CAUSAL, MODE, STATS>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch2(const AttnArgs& a, hipStream_t s) {
  const bool stats = a.stats != nullptr;
  if (a.normalizer == 1) return stats ? launch4<D, CAUSAL, 1, true>(a, s) : launch4<D, CAUSAL, 1, false>(a, s);
  return stats ? launch4<D, CAUSAL, 0, true>(a, s) : launch4<D, CAUSAL, 0, false>(a, s);
}

template <int D>
hipError_t launch1(const AttnArgs& a, hipStream_t s) {
  return a.causal ? launch2<D, true>(a, s) : launch2<D, false>(a, s);
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch1<64>(a, s);
    case 128: return launch1<128>(a, s);
    case 256: return launch1<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hifa4
