// K2: fused 4-bit attention forward (prefill, non-causal and causal) for gfx950.
//
// HiFA4 abstract: QK^T and PV run as 4-bit matrix products, the online-softmax state (m, l, O)
// is FP16, and the normalizer is accumulated from the same quantized P-hat that enters the PV
// product (P-Reordering), so it comes out of that product: P-hat times [V-hat | 1].
//
// Work decomposition.  A work-group serves one (batch, KV head) and BQ query positions of each
// of HW query heads of the GQA group; every K-hat/V-hat tile staged in LDS is shared by all of
// its waves.  A wave owns one block of 16 query rows of one head, the column block of the
// 16x16x128 scaled FP4 MFMA, so its registers hold one score tile at a time: 16 waves per
// work-group (4 per SIMD) for d <= 128 and 8 for d = 256, enough waves per SIMD for one wave's
// exponentials to run while another waits on its matrix products or LDS reads.  Tiles are
// double-buffered: the next tile is fetched from HBM into registers while the current one is
// computed, so one barrier per tile remains.
//
// Layout trick.  Scores are computed transposed, S^T = K-hat Q-hat^T, so a query is an MFMA
// column and lives in lanes (l % 16) of all four 16-lane groups.  MFMA t (t = 0..7) takes key
// 32*(r/4) + 4t + (r%4) as its row r; its output register i of lane group g then holds key
// 32g + 4t + i.  After the 8 MFMAs each lane holds the 32 contiguous keys of one 32-key block of
// its query: exactly the per-lane slice the PV MFMA consumes as its B operand (P-hat^T), so
// P-hat is quantized and packed in registers without any data exchange; its scale (one per
// query and tile) needs only the row maximum, two row-swap permutes.  O^T = V-hat^T P-hat^T
// then puts a query's outputs in its own lanes too, so the FP16 state update needs no exchange
// either.
//
// Interior tiles (every key visible to every row of the 16-query block) take a path without
// any masking; only causal-diagonal and ragged tiles evaluate the visibility predicate.
#include "device_common.h"
#include "launch.h"

namespace hifa4 {

namespace {

constexpr int kStatsRows = 16;  // query rows per tile-statistics block (one wave's rows)

template <int D>
struct Cfg {
  static constexpr int kWaves = D >= 256 ? 8 : 16;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKSteps = D >= 128 ? D / 128 : 1;  // MFMA contractions over d
  static constexpr int kCB = D / 16;                      // 16-channel output blocks
  // 16-byte chunks of one tile: K-hat codes (128 keys x D/2 bytes) then V-hat^T codes (D x 64)
  static constexpr int kKChunks = kTileKeys * (D / 32);
  static constexpr int kChunks = 2 * kKChunks;
  static constexpr int kChunksPerThread = (kChunks + kThreads - 1) / kThreads;
  // scale dwords of one tile: K-hat (128 x D/32 bytes) then V-hat (D x 4 bytes)
  static constexpr int kKScaleWords = kTileKeys * (D / kBlock) / 4;
  static constexpr int kScaleWords = kKScaleWords + D;
};

// Row stride in bytes of the V-hat scale rows in LDS: one row per 32-key block, padded so that the
// four lane groups of a wave (one block each) read four different bank ranges.
template <int D>
constexpr int vs_stride() { return D + 16; }

// One LDS buffer: K-hat codes [128 keys][D/2] (16-byte chunks XOR-swizzled, see kswz), K-hat
// scales transposed [D/32 blocks][128 keys], V-hat^T codes [D][64] (chunks swizzled, see vswz),
// V-hat scales [4 blocks][D] (rows vs_stride apart).
template <int D>
struct Tile {
  uint8_t kc[kTileKeys * (D / 2)];
  uint8_t ks[kTileKeys * (D / kBlock)];
  uint8_t vc[D * (kTileKeys / 2)];
  uint8_t vs[4 * vs_stride<D>()];
};

template <int D>
struct Prefetch {
  uint4 c[Cfg<D>::kChunksPerThread];
  uint32_t sw;  // one scale dword (threads < kScaleWords)
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

// HBM -> registers: this thread's code chunks and scale dword of the tile at key k0.  Keys at or
// past lk (and past bc for 64-key tiles) read as code 0 with scale byte 0x7F.
template <int D>
__device__ __forceinline__ void fetch_tile(Prefetch<D>& pf, const uint8_t* kc_g, const uint8_t* ks_g,
                                           const uint8_t* vc_g, const uint8_t* vs_g, int k0, int lk,
                                           int lk32, int bc, int tid) {
  using C = Cfg<D>;
  constexpr int CPR = D / 32;  // 16-byte chunks per K-hat key row
#pragma unroll
  for (int i = 0; i < C::kChunksPerThread; i++) {
    const int c = tid + i * C::kThreads;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (c < C::kKChunks) {
      const int r = c / CPR, part = c % CPR;
      if (r < bc && k0 + r < lk) w = *reinterpret_cast<const uint4*>(kc_g + (int64_t)(k0 + r) * (D / 2) + 16 * part);
    } else if (c < C::kChunks) {
      const int cv = c - C::kKChunks;  // (32-key block, channel): 16 bytes, contiguous in HBM
      const int part = cv / D, ch = cv % D;
      if (32 * part < bc && k0 + 32 * part < lk32)
        w = *reinterpret_cast<const uint4*>(vc_g + ((int64_t)(k0 / kBlock + part) * D + ch) * 16);
    }
    pf.c[i] = w;
  }
  uint32_t w = 0x7F7F7F7Fu;
  if (tid < C::kKScaleWords) {
    const int c = tid * 4;  // first scale byte of the dword: key c / (D/32), block c % (D/32)
    const int r = c / (D / kBlock);
    if (D >= 128) {
      if (r < bc && k0 + r < lk) w = *reinterpret_cast<const uint32_t*>(ks_g + (int64_t)(k0 + r) * (D / kBlock) + c % (D / kBlock));
    } else {  // D = 64: two keys per dword
      uint32_t lo = 0x7F7Fu, hi = 0x7F7Fu;
      if (r < bc && k0 + r < lk) lo = *reinterpret_cast<const uint16_t*>(ks_g + (int64_t)(k0 + r) * 2);
      if (r + 1 < bc && k0 + r + 1 < lk) hi = *reinterpret_cast<const uint16_t*>(ks_g + (int64_t)(k0 + r + 1) * 2);
      w = lo | (hi << 16);
    }
  } else if (tid < C::kScaleWords) {
    // V-hat scales of the tile: 4 blocks x D channels, contiguous in HBM; dword j holds channels
    // 4j % D .. +3 of block 4j / D
    const int j = tid - C::kKScaleWords;
    const int part = 4 * j / D;
    if (32 * part < bc && k0 + 32 * part < lk32)
      w = *reinterpret_cast<const uint32_t*>(vs_g + (int64_t)(k0 / kBlock) * D + 4 * j);
  }
  pf.sw = w;
}

// registers -> LDS buffer (swizzled codes, transposed K-hat scales)
template <int D>
__device__ __forceinline__ void store_tile(Tile<D>& t, const Prefetch<D>& pf, int tid) {
  using C = Cfg<D>;
  constexpr int CPR = D / 32;
#pragma unroll
  for (int i = 0; i < C::kChunksPerThread; i++) {
    const int c = tid + i * C::kThreads;
    if (c < C::kKChunks) {
      const int r = c / CPR, part = c % CPR;
      const int sw = (part & ~3) | kswz<D>(r, part & 3);
      *reinterpret_cast<uint4*>(&t.kc[r * (D / 2) + 16 * sw]) = pf.c[i];
    } else if (c < C::kChunks) {
      const int cv = c - C::kKChunks;
      const int part = cv / D, ch = cv % D;
      *reinterpret_cast<uint4*>(&t.vc[ch * 64 + 16 * vswz(ch, part)]) = pf.c[i];
    }
  }
  if (tid < C::kKScaleWords) {  // 4 scale bytes -> transposed [block][key]
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int c = tid * 4 + j;
      const int key = D >= 128 ? c / (D / kBlock) : c / 2;
      const int blk = D >= 128 ? c % (D / kBlock) : c % 2;
      t.ks[blk * kTileKeys + key] = (uint8_t)(pf.sw >> (8 * j));
    }
  } else if (tid < C::kScaleWords) {
    const int j = tid - C::kKScaleWords;
    *reinterpret_cast<uint32_t*>(&t.vs[(4 * j / D) * vs_stride<D>() + (4 * j) % D]) = pf.sw;
  }
}

template <int D, bool CAUSAL, int MODE, bool STATS>
__global__ __launch_bounds__(Cfg<D>::kThreads) void attn_prefill_kernel(AttnArgs a) {
  using Cf = Cfg<D>;
  constexpr int W = Cf::kWaves;
  constexpr int KSTEPS = Cf::kKSteps;
  constexpr int CB = Cf::kCB;
  __shared__ Tile<D> tiles[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;    // lane group: K-chunk of the MFMA operands / key block of P-hat
  const int col = lane & 15;  // MFMA column: query within the wave's 16-row block

  const int group = a.heads_q / a.heads_kv;
  const int hw = a.heads_per_wg;  // query heads per work-group (divides both group and W)
  const int wph = W / hw;         // waves per head
  const int bq = 16 * wph;        // query positions per head per work-group
  const int chunks = group / hw;
  const int kvh = blockIdx.y / chunks;
  const int h = kvh * group + (blockIdx.y % chunks) * hw + wave / wph;
  const int b = blockIdx.z;
  // heaviest causal blocks first: they start while the short ones fill the tail
  const int qblk = CAUSAL ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int lq = (int)a.len_q, lk = (int)a.len_kv, lk32 = (int)a.len_kv32;
  const int q_wg = qblk * bq;
  const int q0 = q_wg + 16 * (wave % wph);  // first query row of this wave
  const int shift = lk - lq;                // causal: key c visible to query r iff c <= r + shift
  const int bc = a.kv_tile;

  // ---- Q-hat^T operand (B operand of the score MFMA), kept in registers
  uint4 qreg[KSTEPS];
  uint32_t qsc[KSTEPS];
  {
    const uint8_t* qc = a.q_codes + ((int64_t)b * a.heads_q + h) * (int64_t)lq * (D / 2);
    const uint8_t* qs = a.q_scales + ((int64_t)b * a.heads_q + h) * (int64_t)lq * (D / kBlock);
    const int q = q0 + col;
#pragma unroll
    for (int s = 0; s < KSTEPS; s++) {
      const bool has = q < lq && (D >= 128 || g < 2);
      qreg[s] = has ? *reinterpret_cast<const uint4*>(qc + (int64_t)q * (D / 2) + 64 * s + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
      qsc[s] = has ? qs[(int64_t)q * (D / kBlock) + 4 * s + g] : 127u;
    }
  }

  // ---- FP16 state; m is an integer-valued float
  h2 o[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; cb++) o[cb][0] = o[cb][1] = h2{(_Float16)0.0f, (_Float16)0.0f};
  _Float16 l = (_Float16)0.0f;
  float m = -INFINITY;

  int last_row = q_wg + bq - 1;
  if (last_row > lq - 1) last_row = lq - 1;
  int n_tiles = a.n_tiles;
  if (CAUSAL) {
    const int need = (last_row + shift) / bc + 1;  // tiles holding a key some row here sees
    n_tiles = need < n_tiles ? need : n_tiles;
  }
  const bool wave_live = q0 < lq;
  const int wave_last = q0 + 15 < lq - 1 ? q0 + 15 : lq - 1;
  float* stats_row = nullptr;
  if (STATS && wave_live) {
    const int nrb = (lq + kStatsRows - 1) / kStatsRows;
    stats_row = a.stats + ((((int64_t)b * a.heads_q + h) * nrb) + q0 / kStatsRows) * (int64_t)a.n_tiles * 2;
    for (int i = lane; i < a.n_tiles * 2; i += 64) stats_row[i] = 0.0f;
  }

  const uint8_t* kc_g = a.k_codes + ((int64_t)b * a.heads_kv + kvh) * (int64_t)lk * (D / 2);
  const uint8_t* ks_g = a.k_scales + ((int64_t)b * a.heads_kv + kvh) * (int64_t)lk * (D / kBlock);
  const uint8_t* vc_g = a.v_codes + ((int64_t)b * a.heads_kv + kvh) * (int64_t)D * (lk32 / 2);
  const uint8_t* vs_g = a.v_scales + ((int64_t)b * a.heads_kv + kvh) * (int64_t)D * (lk32 / kBlock);
  // (both are the start of this (batch, KV head)'s block-major V-hat: lk32/32 blocks of D cells)
  const float C = a.c_log2;

  // per-lane LDS offsets of this lane's MFMA operands (see the loads in the tile loop)
  const int k_lane_off = (32 * (col >> 2) + (col & 3)) * (D / 2) + 16 * kswz<D>(32 * (col >> 2) + (col & 3), g);
  const int ks_lane_off = g * kTileKeys + 32 * (col >> 2) + (col & 3);
  const int v_lane_off = col * 64 + 16 * vswz(col, g);
  const int vs_lane_off = g * vs_stride<D>() + col;

  Prefetch<D> pf;
  fetch_tile<D>(pf, kc_g, ks_g, vc_g, vs_g, 0, lk, lk32, bc, tid);
  store_tile<D>(tiles[0], pf, tid);
  __syncthreads();

  for (int tile = 0; tile < n_tiles; tile++) {
    const int k0 = tile * bc;
    const Tile<D>& T = tiles[tile & 1];
    if (tile + 1 < n_tiles) fetch_tile<D>(pf, kc_g, ks_g, vc_g, vs_g, k0 + bc, lk, lk32, bc, tid);

    if (wave_live && !(CAUSAL && k0 > wave_last + shift)) {
      // ---- S^T = K-hat Q-hat^T: MFMA t reads key kr = 32 (col/4) + 4t + (col%4); the per-lane
      // part is a fixed base, t and the contraction step are immediate offsets (the swizzle term
      // kr/32 = col/4 does not depend on t).  Lane holds keys k0 + 32 g + (4 t + i).
      const uint8_t* kbase = T.kc + k_lane_off;
      const uint8_t* ksbase = T.ks + ks_lane_off;
      float s[32];
#pragma unroll
      for (int t = 0; t < 8; t++) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KSTEPS; st++) {
          uint4 ka = make_uint4(0u, 0u, 0u, 0u);
          uint32_t ksc = 127u;
          if (D >= 128 || g < 2) {
            ka = *reinterpret_cast<const uint4*>(kbase + 4 * t * (D / 2) + 64 * st);
            ksc = ksbase[4 * t + 4 * st * kTileKeys];
          }
          acc = mfma_fp4(ka, ksc, qreg[st], qsc[st], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) s[4 * t + i] = acc[i];
      }
      const int q = q0 + col;
      const bool full = bc == kTileKeys && k0 + kTileKeys <= lk && q0 + 15 < lq &&
                        (!CAUSAL || k0 + kTileKeys - 1 <= q0 + shift);
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
      const RowStep rs = row_step(rmax, m, C);
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
        const float two_e = e8m0_as_float((int)rs.e);
        if (MODE == 1) lsum = group_sum4(sb) * two_e;
        if (STATS) {
          float sp = sb * two_e;
          sp += __shfl_xor(sp, 16);
          sp += __shfl_xor(sp, 32);
          sp = wave_sum16(sp);
          const float sh = wave_sum16(lacc[0]);
          if (lane == 0) {
            stats_row[tile * 2 + 0] = sh;
            stats_row[tile * 2 + 1] = sp;
          }
        }
      }
      // ---- O^T += V-hat^T P-hat^T per 16-channel block (channel 16 cb + col; the swizzle term
      // (ch/4)%4 = col/4); FP16 state update
      const uint8_t* vbase = T.vc + v_lane_off;
      const uint8_t* vsbase = T.vs + vs_lane_off;
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const uint4 va = *reinterpret_cast<const uint4*>(vbase + 16 * 64 * cb);
        const uint32_t vsc = vsbase[16 * cb];
        v4f pv = {0.0f, 0.0f, 0.0f, 0.0f};
        pv = mfma_fp4(va, vsc, ph, psc, pv);
        state_update(o[cb], rs.alpha, pv);
      }
      l = __builtin_fmaf16(rs.alpha, l, (_Float16)lsum);
      m = rs.m_new;
    }

    if (tile + 1 < n_tiles) store_tile<D>(tiles[(tile + 1) & 1], pf, tid);
    __syncthreads();
  }

  // ---- epilogue: out = fp16(O / l); lane holds channels 16 cb + 4 g + i of its query
  const int q = q0 + col;
  if (!wave_live || q >= lq) return;
  uint16_t* out = a.out + ((int64_t)b * a.heads_q + h) * (int64_t)lq * D;
  const float lv = (float)l;
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    const h2 r01 = h2{(_Float16)((float)o[cb][0][0] / lv), (_Float16)((float)o[cb][0][1] / lv)};
    const h2 r23 = h2{(_Float16)((float)o[cb][1][0] / lv), (_Float16)((float)o[cb][1][1] / lv)};
    uint2 w;
    w.x = __builtin_bit_cast(uint32_t, r01);
    w.y = __builtin_bit_cast(uint32_t, r23);
    *reinterpret_cast<uint2*>(out + (int64_t)q * D + 16 * cb + 4 * g) = w;
  }
}

int gcd_int(int x, int y) {
  while (y) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

template <int D, bool CAUSAL, int MODE, bool STATS>
hipError_t launch4(AttnArgs a, hipStream_t s) {
  constexpr int W = Cfg<D>::kWaves;
  const int group = a.heads_q / a.heads_kv;
  const int hw = gcd_int(group, W);  // query heads per work-group
  const int bq = 16 * (W / hw);
  a.heads_per_wg = hw;
  const int64_t qblocks = (a.len_q + bq - 1) / bq;
  dim3 grid((uint32_t)qblocks, (uint32_t)(a.heads_kv * (group / hw)), (uint32_t)a.batch);
  hipLaunchKernelGGL((attn_prefill_kernel<D, CAUSAL, MODE, STATS>), grid, dim3(Cfg<D>::kThreads), 0, s, a);
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
