// K2: fused 4-bit attention forward (prefill, non-causal and causal) for gfx950.
//
// HiFA4 abstract: QK^T and PV run as 4-bit matrix products, the online-softmax state (m, l, O)
// is FP16, and the normalizer is accumulated from the same quantized P-hat that enters the PV
// product (P-Reordering), so it comes out of that product: P-hat times [V-hat | 1].
//
// Work decomposition.  A work-group serves one (batch, KV head) and BQ query positions of each
// of HW query heads of the group (HW * BQ / 32 = 8 waves); every K-hat/V-hat tile staged in LDS
// is shared by all of them (GQA).  A wave owns 32 query rows of one head, as two 16-column
// blocks of the 16x16x128 scaled FP4 MFMA, and loads each tile's MFMA operands from LDS once
// for both blocks.  Tiles are double-buffered: the next tile's bytes are fetched from HBM into
// registers while the current one is computed, so one barrier per tile remains.
//
// Layout trick.  Scores are computed transposed, S^T = K-hat Q-hat^T, so a query is an MFMA
// column and lives in lanes (l % 16) of all four 16-lane groups.  MFMA t (t = 0..7) takes key
// 32*(r/4) + 4t + (r%4) as its row r; its output register i of lane group g then holds key
// 32g + 4t + i.  After the 8 MFMAs each lane holds the 32 contiguous keys of one 32-key block of
// its query: exactly the per-lane slice the PV MFMA consumes as its B operand (P-hat^T), so
// P-hat is quantized and packed in registers without any data exchange; its scale (one per
// query and tile) needs only the row maximum, two shuffles.  O^T = V-hat^T P-hat^T then puts a
// query's outputs in its own lanes too, so the FP16 state update needs no shuffles either.
//
// Interior tiles (every key visible to every row of the 16-query block) take a path without
// any masking; only causal-diagonal and ragged tiles evaluate the visibility predicate.
#include "device_common.h"
#include "launch.h"

namespace hifa4 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

// One LDS buffer: K-hat codes [128 keys][D/2] (16-byte chunks XOR-swizzled, see kswz), K-hat
// scales transposed [D/32 blocks][128 keys], V-hat^T codes [D][64] (chunks swizzled, see vswz),
// V-hat scales [D][4].
template <int D>
struct Tile {
  uint8_t kc[kTileKeys * (D / 2)];
  uint8_t ks[kTileKeys * (D / kBlock)];
  uint8_t vc[D * (kTileKeys / 2)];
  uint8_t vs[D * (kTileKeys / kBlock)];
};

template <int D>
struct Prefetch {
  static constexpr int KCH = (kTileKeys * D / 2) / 16 / kThreads > 0 ? (kTileKeys * D / 2) / 16 / kThreads : 1;
  uint4 k[KCH];
  uint4 v[KCH];
  uint32_t ks;  // 4 K-hat scale bytes (threads < 128 * D / 32 / 4)
  uint32_t vs;  // 4 V-hat scale bytes of one channel (threads < D)
};

// XOR swizzles of the 16-byte chunks inside an LDS row.  One MFMA operand read touches, per
// 16-lane group, keys 32b + 4t + a (b = col/4, a = col%4) of K-hat, or channels 16cb + col of
// V-hat; the swizzle makes the 16-byte slots of any 8 consecutive lanes distinct modulo 128 bytes
// and of any 16 lanes distinct modulo 256 bytes, so the read is conflict-free whether the LDS
// serves it in 8-lane (32-bank) or 16-lane (64-bank) passes.  Both terms are fixed per lane.
template <int D>
__device__ __forceinline__ int kswz(int key, int chunk) {
  return D >= 128 ? chunk ^ (((key >> 5) & 3) ^ (((key >> 1) & 1) << 1)) : chunk ^ ((key >> 5) & 1);
}
__device__ __forceinline__ int vswz(int ch, int chunk) { return chunk ^ (((ch >> 2) & 3) ^ (((ch >> 1) & 1) << 1)); }

__device__ __forceinline__ float wave_sum16(float x) {  // sum over the 16 lanes sharing l / 16
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <int D>
__device__ __forceinline__ void fetch_tile(Prefetch<D>& pf, const uint8_t* kc_g, const uint8_t* ks_g,
                                           const uint8_t* vc_g, const uint8_t* vs_g, int k0, int lk,
                                           int lk32, int bc, int tid) {
  constexpr int CPR = D / 32;  // 16-byte chunks per key row
#pragma unroll
  for (int i = 0; i < Prefetch<D>::KCH; i++) {
    const int c = tid + i * kThreads;
    const int r = c / CPR, part = c % CPR;
    const bool ok = c < kTileKeys * CPR && r < bc && k0 + r < lk;
    pf.k[i] = ok ? *reinterpret_cast<const uint4*>(kc_g + (int64_t)(k0 + r) * (D / 2) + 16 * part) : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    // K-hat scales: 128 keys x D/32 bytes, 4 bytes per thread
    const int c = tid * 4;
    uint32_t w = 0x7F7F7F7Fu;
    if (c < kTileKeys * (D / kBlock)) {
      const int r = c / (D / kBlock);
      if (D >= 128) {
        if (r < bc && k0 + r < lk) w = *reinterpret_cast<const uint32_t*>(ks_g + (int64_t)(k0 + r) * (D / kBlock) + c % (D / kBlock));
      } else {  // D = 64: two keys per dword
        uint32_t lo = 0x7F7Fu, hi = 0x7F7Fu;
        if (r < bc && k0 + r < lk) lo = *reinterpret_cast<const uint16_t*>(ks_g + (int64_t)(k0 + r) * 2);
        if (r + 1 < bc && k0 + r + 1 < lk) hi = *reinterpret_cast<const uint16_t*>(ks_g + (int64_t)(k0 + r + 1) * 2);
        w = lo | (hi << 16);
      }
    }
    pf.ks = w;
  }
#pragma unroll
  for (int i = 0; i < Prefetch<D>::KCH; i++) {
    const int c = tid + i * kThreads;  // (channel, chunk) with 4 chunks of 16 bytes per channel
    const int ch = c >> 2, part = c & 3;
    const bool ok = ch < D && 32 * part < bc && k0 + 32 * part < lk32;
    pf.v[i] = ok ? *reinterpret_cast<const uint4*>(vc_g + (int64_t)ch * (lk32 / 2) + k0 / 2 + 16 * part) : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    uint32_t w = 0x7F7F7F7Fu;
    if (tid < D) {
      const uint8_t* src = vs_g + (int64_t)tid * (lk32 / kBlock) + k0 / kBlock;
      const int nb = (lk32 - k0) / kBlock;  // V-hat blocks left in the row
      if (bc == kTileKeys && nb >= 4 && (reinterpret_cast<uintptr_t>(src) & 3) == 0) {
        w = *reinterpret_cast<const uint32_t*>(src);
      } else {
        uint32_t b0 = 0x7F, b1 = 0x7F, b2 = 0x7F, b3 = 0x7F;
        if (nb > 0) b0 = src[0];
        if (nb > 1 && bc > 32) b1 = src[1];
        if (nb > 2 && bc > 64) b2 = src[2];
        if (nb > 3 && bc > 96) b3 = src[3];
        w = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      }
    }
    pf.vs = w;
  }
}

template <int D>
__device__ __forceinline__ void store_tile(Tile<D>& t, const Prefetch<D>& pf, int tid) {
  constexpr int CPR = D / 32;
#pragma unroll
  for (int i = 0; i < Prefetch<D>::KCH; i++) {
    const int c = tid + i * kThreads;
    if (c < kTileKeys * CPR) {
      const int r = c / CPR, part = c % CPR;
      const int sw = (part & ~3) | kswz<D>(r, part & 3);
      *reinterpret_cast<uint4*>(&t.kc[r * (D / 2) + 16 * sw]) = pf.k[i];
    }
  }
  if (tid * 4 < kTileKeys * (D / kBlock)) {  // 4 scale bytes -> transposed [block][key]
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int c = tid * 4 + j;
      const int key = D >= 128 ? c / (D / kBlock) : c / 2;
      const int blk = D >= 128 ? c % (D / kBlock) : c % 2;
      t.ks[blk * kTileKeys + key] = (uint8_t)(pf.ks >> (8 * j));
    }
  }
#pragma unroll
  for (int i = 0; i < Prefetch<D>::KCH; i++) {
    const int c = tid + i * kThreads;
    const int ch = c >> 2, part = c & 3;
    if (ch < D) *reinterpret_cast<uint4*>(&t.vc[ch * 64 + 16 * vswz(ch, part)]) = pf.v[i];
  }
  if (tid < D) *reinterpret_cast<uint32_t*>(&t.vs[tid * 4]) = pf.vs;
}

template <int D, bool CAUSAL, int MODE, bool STATS>
__global__ __launch_bounds__(kThreads) void attn_prefill_kernel(AttnArgs a) {
  constexpr int KSTEPS = D >= 128 ? D / 128 : 1;  // MFMA contractions over d
  constexpr int CB = D / 16;                      // 16-channel output blocks
  __shared__ Tile<D> tiles[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;    // lane group: K-chunk of the MFMA operands / key block of P-hat
  const int col = lane & 15;  // MFMA column: query within a 16-column block

  const int group = a.heads_q / a.heads_kv;
  const int hw = group < kWaves ? group : kWaves;  // query heads per work-group
  const int bq = 32 * (kWaves / hw);               // query positions per head per work-group
  const int chunks = group / hw;
  const int kvh = blockIdx.y / chunks;
  const int h = kvh * group + (blockIdx.y % chunks) * hw + wave / (bq / 32);
  const int b = blockIdx.z;
  // heaviest causal blocks first: they start while the short ones fill the tail
  const int qblk = CAUSAL ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int lq = (int)a.len_q, lk = (int)a.len_kv, lk32 = (int)a.len_kv32;
  const int q_wg = qblk * bq;
  const int q_base = q_wg + 32 * (wave % (bq / 32));
  const int shift = lk - lq;  // causal: key c visible to query r iff c <= r + shift
  const int bc = a.kv_tile;

  // ---- Q-hat^T operands (B operand of the score MFMA), kept in registers
  uint4 qreg[2][KSTEPS];
  uint32_t qsc[2][KSTEPS];
  {
    const uint8_t* qc = a.q_codes + ((int64_t)b * a.heads_q + h) * (int64_t)lq * (D / 2);
    const uint8_t* qs = a.q_scales + ((int64_t)b * a.heads_q + h) * (int64_t)lq * (D / kBlock);
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      const int q = q_base + 16 * qb + col;
#pragma unroll
      for (int s = 0; s < KSTEPS; s++) {
        const bool has = q < lq && (D >= 128 || g < 2);
        qreg[qb][s] = has ? *reinterpret_cast<const uint4*>(qc + (int64_t)q * (D / 2) + 64 * s + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
        qsc[qb][s] = has ? qs[(int64_t)q * (D / kBlock) + 4 * s + g] : 127u;
      }
    }
  }

  // ---- FP16 state; m is an integer-valued float
  h2 o[2][CB][2];
  _Float16 l[2];
  float m[2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    l[qb] = (_Float16)0.0f;
    m[qb] = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) o[qb][cb][0] = o[qb][cb][1] = h2{(_Float16)0.0f, (_Float16)0.0f};
  }

  int last_row = q_wg + bq - 1;
  if (last_row > lq - 1) last_row = lq - 1;
  int n_tiles = a.n_tiles;
  if (CAUSAL) {
    const int need = (last_row + shift) / bc + 1;  // tiles holding a key some row here sees
    n_tiles = need < n_tiles ? need : n_tiles;
  }
  const int nrb = (lq + 31) / 32;
  float* stats_row = nullptr;
  if (STATS && q_base < lq) {
    stats_row = a.stats + ((((int64_t)b * a.heads_q + h) * nrb) + q_base / 32) * (int64_t)a.n_tiles * 2;
    for (int i = lane; i < a.n_tiles * 2; i += 64) stats_row[i] = 0.0f;
  }

  const uint8_t* kc_g = a.k_codes + ((int64_t)b * a.heads_kv + kvh) * (int64_t)lk * (D / 2);
  const uint8_t* ks_g = a.k_scales + ((int64_t)b * a.heads_kv + kvh) * (int64_t)lk * (D / kBlock);
  const uint8_t* vc_g = a.v_codes + ((int64_t)b * a.heads_kv + kvh) * (int64_t)D * (lk32 / 2);
  const uint8_t* vs_g = a.v_scales + ((int64_t)b * a.heads_kv + kvh) * (int64_t)D * (lk32 / kBlock);
  const float C = a.c_log2;
  const bool wave_live = q_base < lq;
  const int wave_last = q_base + 31 < lq - 1 ? q_base + 31 : lq - 1;

  // per-lane LDS offsets of this lane's MFMA operands (see the loads in the tile loop)
  const int k_lane_off = (32 * (col >> 2) + (col & 3)) * (D / 2) + 16 * kswz<D>(32 * (col >> 2) + (col & 3), g);
  const int ks_lane_off = g * kTileKeys + 32 * (col >> 2) + (col & 3);
  const int v_lane_off = col * 64 + 16 * vswz(col, g);
  const int vs_lane_off = col * 4 + g;

  Prefetch<D> pf;
  fetch_tile<D>(pf, kc_g, ks_g, vc_g, vs_g, 0, lk, lk32, bc, tid);
  store_tile<D>(tiles[0], pf, tid);
  __syncthreads();

  for (int tile = 0; tile < n_tiles; tile++) {
    const int k0 = tile * bc;
    const Tile<D>& T = tiles[tile & 1];
    if (tile + 1 < n_tiles) fetch_tile<D>(pf, kc_g, ks_g, vc_g, vs_g, k0 + bc, lk, lk32, bc, tid);

    if (wave_live && !(CAUSAL && k0 > wave_last + shift)) {
      // ---- K-hat A operands of the 8 score MFMAs, shared by both query blocks.  MFMA t reads key
      // kr = 32 (col/4) + 4t + (col%4): the per-lane part is a fixed base, t and the contraction
      // step are immediate offsets (the swizzle term kr/32 = col/4 does not depend on t).
      const uint8_t* kbase = T.kc + k_lane_off;
      const uint8_t* ksbase = T.ks + ks_lane_off;
      uint4 ka[8][KSTEPS];
      uint32_t ksc[8][KSTEPS];
#pragma unroll
      for (int t = 0; t < 8; t++) {
#pragma unroll
        for (int st = 0; st < KSTEPS; st++) {
          if (D >= 128 || g < 2) {
            ka[t][st] = *reinterpret_cast<const uint4*>(kbase + 4 * t * (D / 2) + 64 * st);
            ksc[t][st] = ksbase[4 * t + 4 * st * kTileKeys];
          } else {
            ka[t][st] = make_uint4(0u, 0u, 0u, 0u);
            ksc[t][st] = 127u;
          }
        }
      }
      // ---- V-hat^T A operands of the PV MFMAs, shared by both query blocks
      const uint8_t* vbase = T.vc + v_lane_off;
      const uint8_t* vsbase = T.vs + vs_lane_off;
      uint4 va[CB];
      uint32_t vsc[CB];
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {  // channel 16 cb + col; the swizzle term (ch/4)%4 = col/4
        va[cb] = *reinterpret_cast<const uint4*>(vbase + 16 * 64 * cb);
        vsc[cb] = vsbase[16 * 4 * cb];
      }
      float sum_phat = 0.0f, sum_p = 0.0f;
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        // ---- S^T = K-hat Q-hat^T for this 16-query block: lane holds keys k0 + 32 g + (4 t + i)
        float s[32];
#pragma unroll
        for (int t = 0; t < 8; t++) {
          v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int st = 0; st < KSTEPS; st++) acc = mfma_fp4(ka[t][st], ksc[t][st], qreg[qb][st], qsc[qb][st], acc);
#pragma unroll
          for (int i = 0; i < 4; i++) s[4 * t + i] = acc[i];
        }
        const int qrow0 = q_base + 16 * qb;
        const int q = qrow0 + col;
        const bool full = bc == kTileKeys && k0 + kTileKeys <= lk && qrow0 + 15 < lq &&
                          (!CAUSAL || k0 + kTileKeys - 1 <= qrow0 + shift);
        float bmax = -INFINITY;
        if (full) {
#pragma unroll
          for (int k = 0; k < 32; k++) bmax = fmaxf(bmax, s[k]);
        } else {
          const int kb = k0 + 32 * g;
          int lim = lk - 1;  // last visible key of this row
          if (CAUSAL && q + shift < lim) lim = q + shift;
          if (k0 + bc - 1 < lim) lim = k0 + bc - 1;
          if (q >= lq) lim = -1;
#pragma unroll
          for (int k = 0; k < 32; k++) {
            s[k] = (kb + k <= lim) ? s[k] : -INFINITY;
            bmax = fmaxf(bmax, s[k]);
          }
        }
        const float rmax = group_max4(bmax);
        // ---- integer running max, FP16 rescale factor, P-hat scale of this row and tile
        const RowStep rs = row_step(rmax, m[qb], C);
        uint32_t p16[16];
        const uint4 ph = phat_codes(s, C, rs.neg_big_m, p16);
        const uint32_t psc = (uint32_t)(int)(rs.e + 127.0f);
        // ---- normalizer increment: rowsum(P-hat) from the ones column, or the FP32 tree sum
        const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
        v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
        lacc = mfma_fp4(ones, 127u, ph, psc, lacc);
        float lsum = lacc[0];
        if (MODE == 1 || STATS) {
          const float sb = tree_sum32_h(p16);
          const float ptree = group_sum4(sb) * e8m0_as_float((int)rs.e);
          if (MODE == 1) lsum = ptree;
          if (STATS) {
            sum_p += sb * e8m0_as_float((int)rs.e);
            sum_phat += (g == 0) ? lacc[0] : 0.0f;
          }
        }
        // ---- O^T += V-hat^T P-hat^T per 16-channel block; FP16 state update
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
          v4f pv = {0.0f, 0.0f, 0.0f, 0.0f};
          pv = mfma_fp4(va[cb], vsc[cb], ph, psc, pv);
          state_update(o[qb][cb], rs.alpha, pv);
        }
        l[qb] = __builtin_fmaf16(rs.alpha, l[qb], (_Float16)lsum);
        m[qb] = rs.m_new;
      }
      if (STATS) {
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

    if (tile + 1 < n_tiles) store_tile<D>(tiles[(tile + 1) & 1], pf, tid);
    __syncthreads();
  }

  // ---- epilogue: out = fp16(O / l); lane holds channels 16 cb + 4 g + i of its query
  if (!wave_live) return;
  uint16_t* out = a.out + ((int64_t)b * a.heads_q + h) * (int64_t)lq * D;
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int q = q_base + 16 * qb + col;
    if (q >= lq) continue;
    const float lv = (float)l[qb];
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      const h2 r01 = h2{(_Float16)((float)o[qb][cb][0][0] / lv), (_Float16)((float)o[qb][cb][0][1] / lv)};
      const h2 r23 = h2{(_Float16)((float)o[qb][cb][1][0] / lv), (_Float16)((float)o[qb][cb][1][1] / lv)};
      uint2 w;
      w.x = __builtin_bit_cast(uint32_t, r01);
      w.y = __builtin_bit_cast(uint32_t, r23);
      *reinterpret_cast<uint2*>(out + (int64_t)q * D + 16 * cb + 4 * g) = w;
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
