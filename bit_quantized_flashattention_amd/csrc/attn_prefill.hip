// K2: fused 4-bit attention forward (prefill, non-causal and causal) for gfx950.
//
// HiFA4 abstract: QK^T and PV run as 4-bit matrix products, the online-softmax state (m, l, O)
// is FP16, and the normalizer is accumulated from the same quantized P-hat that enters the PV
// product (P-Reordering), so it comes out of that product: P-hat times [V-hat | 1].
//
// Work decomposition.  A work-group serves one (batch, KV head) and BQ query positions of each
// of HW query heads of the GQA group; every K-hat/V-hat tile staged in LDS is shared by all of
// its waves.  A wave owns one block of 16 query rows of one head, the column block of the
// 16x16x128 scaled FP4 MFMA, so its registers hold one score tile at a time.  A work-group has 8
// waves; with registers capped at 80 (d <= 128) three work-groups share a CU, 6 waves per SIMD
// (4 at d = 256), enough for one wave's exponentials to run while another waits on its matrix
// products or LDS reads.  Causal grids that would fill the chip at most once run work-groups of 4
// waves instead (see launch4).  Tiles are double-buffered in LDS: the next tile is copied from HBM
// straight into LDS (buffer loads that write LDS) while the current one is computed, so one
// barrier per tile remains.
//
// Layout trick.  Scores are computed transposed, S^T = K-hat Q-hat^T, so a query is an MFMA
// column and lives in lanes (l % 16) of all four 16-lane groups.  MFMA t (t = 0..7) takes key
// 32*(r/4) + 8*(r%4) + t as its row r; its output register i of lane group g then holds key
// 32g + 8i + t.  After the 8 MFMAs each lane holds the 32 keys of one 32-key block of its query:
// exactly the per-lane slice the PV MFMA consumes as its B operand (P-hat^T), so P-hat is
// quantized and packed in registers without any data exchange, and its scale (one per query and
// 32-key block, the PV MFMA's per-lane B scale) comes from the lane's own maximum; the running
// max needs the row maximum, two row-swap permutes.  O^T = V-hat^T P-hat^T
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
#ifndef PREFILL_WAVES
#define PREFILL_WAVES 8  // waves per work-group: 8 x 16 query rows
#endif
#ifndef PREFILL_MIN_WAVES
#define PREFILL_MIN_WAVES 6  // waves per SIMD the P-Reordered kernels' registers must allow (3 work-groups per CU)
#endif
#ifndef PREFILL_STAGES
#define PREFILL_STAGES 2
#endif
#ifndef PREFILL_SMALL_GRID_WAVES
#define PREFILL_SMALL_GRID_WAVES 4  // waves per work-group of grids too small to fill the chip (0: off)
#endif
#ifndef PREFILL_SNAKE
#define PREFILL_SNAKE 1  // causal small-grid order: alternate direction every 32 work-groups of an XCD
#endif
constexpr int kCUsPerXCD = 32;
constexpr int kStages = PREFILL_STAGES;  // LDS ring depth (2: tile j+1 streams in while j is used)

template <int D, int WAVES = PREFILL_WAVES>
struct Cfg {
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKSteps = D >= 128 ? D / 128 : 1;  // MFMA contractions over d
  static constexpr int kCB = D / 16;                      // 16-channel output blocks
  static constexpr int kKRow = D / 2;                     // bytes of one K-hat key row
  static constexpr int kNB = D / kBlock;                  // scale blocks per key
  // byte offsets inside one LDS stage; the codes are stored in MFMA-operand order, 1 KB per
  // MFMA ([mfma][lane], 16 bytes per lane), so every operand read is a linear wave-wide read
  static constexpr int kKC = 0;                                   // K-hat: 8 x KSTEPS MFMAs
  static constexpr int kVC = kKC + 8 * kKSteps * 1024;            // V-hat^T: CB MFMAs
  static constexpr int kKS = kVC + kCB * 1024;                    // K-hat scales [D/32][128]
  static constexpr int kVS = kKS + kTileKeys * kNB;               // V-hat scales [4][D]
  static constexpr int kStageBytes = kVS + 4 * D;
  // wave-wide loads that fill one stage: codes at 16 bytes per lane (1 KB per load), scales at
  // 4 bytes per lane (256 bytes per load)
  static constexpr int kKCInstr = 8 * kKSteps;
  static constexpr int kVCInstr = kCB;
  static constexpr int kKSInstr = kTileKeys * kNB / 256;
  static constexpr int kVSInstr = 4 * D / 256;
  static constexpr int kInstr = kKCInstr + kVCInstr + kKSInstr + kVSInstr;
  static constexpr int kMaxLoadsPerWave = (kInstr + kWaves - 1) / kWaves;
};

__device__ __forceinline__ float wave_sum16(float x) {  // sum over the 16 lanes sharing l / 16
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

typedef int v4i __attribute__((ext_vector_type(4)));

// One wave-wide load of a stage: section (0 K-hat codes, 1 V-hat codes, 2 K-hat scales, 3 V-hat
// scales), its byte offset inside the stage (the same for all lanes: the hardware writes lane i
// at that offset + i * size) and this lane's byte offset inside the (batch, KV head) slice of
// its section at key 0.  Positions are inverted here: a lane loads whatever HBM bytes belong at
// its LDS position.  The code loads are exactly the operands of one MFMA: lane (g, col) of score
// MFMA t fetches chunk g of key score_row_key(t, col); lane (g, col) of PV MFMA cb fetches the
// 32-key block g of channel 16 cb + col.  The scale loads copy the block-plane K-hat rows and the
// V-hat block rows of the tile.
struct LoadOp {
  int sec;
  int lds;
  int voff;
};

template <int D>
__device__ __forceinline__ LoadOp load_op(int i, int lane, int plane) {
  using C = Cfg<D>;
  LoadOp op;
  const int g = lane >> 4, col = lane & 15;
  if (i < C::kKCInstr) {
    const int t = i / C::kKSteps, st = i % C::kKSteps;
    // d = 64 has two chunks per key: lanes g >= 2 fetch a duplicate that no MFMA reads
    const int chunk = D >= 128 ? 4 * st + g : (g & 1);
    op.sec = 0;
    op.lds = C::kKC + i * 1024;
    op.voff = score_row_key(t, col) * C::kKRow + 16 * chunk;
  } else if (i < C::kKCInstr + C::kVCInstr) {
    const int cb = i - C::kKCInstr;
    op.sec = 1;
    op.lds = C::kVC + cb * 1024;
    op.voff = (g * D + 16 * cb + col) * 16;  // block-major V-hat cells (32-key block g, channel 16 cb + col)
  } else if (i < C::kKCInstr + C::kVCInstr + C::kKSInstr) {
    const int q = i - C::kKCInstr - C::kVCInstr;
    const int pos = q * 256 + 4 * lane;  // [block][key] rows of 128 bytes
    op.sec = 2;
    op.lds = C::kKS + q * 256;
    op.voff = (pos / kTileKeys) * plane + pos % kTileKeys;  // plane: K-hat scale plane stride
  } else {
    const int q = i - C::kKCInstr - C::kVCInstr - C::kKSInstr;
    op.sec = 3;
    op.lds = C::kVS + q * 256;
    op.voff = q * 256 + 4 * lane;  // 4 blocks x D channels, contiguous
  }
  return op;
}

// Raw buffer descriptor (stride 0) of one (batch, KV head) slice of a section: a load past the
// end of the slice returns zeros (codes 0 and scale byte 0, i.e. 2^-127), which is what the
// ragged tail of the last tile needs.
__device__ __forceinline__ v4i make_desc(const void* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  v4i d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFFu));
  d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  d[3] = 0x00020000;
  return d;
}

struct Slices {
  v4i r[4];
};

// LDS byte address of a pointer into the work-group's shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// HBM -> LDS without registers: each lane's SIZE bytes at voff (+ the descriptor's base) land at
// LDS address m0 + lane * SIZE.  The load is tracked by the wave's vector-memory counter only;
// the kernel waits for it explicitly (wait_vmem) before the barrier that publishes the stage.
// It is written as inline assembly on purpose: with the compiler's buffer-to-LDS builtin the
// compiler cannot tell the stages apart and puts a wait for every outstanding load (the next
// tile's included) before the first LDS read of the current tile, which removes the overlap of
// loading and computing.  m0 is set inside the statement; the compiler uses m0 for nothing else
// in these kernels (checked in the generated code), so the clobber is safe.
template <int SIZE>
__device__ __forceinline__ void dma(const v4i& desc, uint32_t lds, int voff) {
  if (SIZE == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(desc)
                 : "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(desc)
                 : "m0");
}

// Section of stage load i (0 K-hat codes, 1 V-hat codes, 2 K-hat scales, 3 V-hat scales, 4 none)
// and its byte offset inside the stage: code loads fill 1 KB each, scale loads 256 bytes.
template <int D>
__host__ __device__ constexpr int load_section(int i) {
  using C = Cfg<D>;
  return i < C::kKCInstr ? 0 : i < C::kKCInstr + C::kVCInstr ? 1 : i < C::kKCInstr + C::kVCInstr + C::kKSInstr ? 2 : i < C::kInstr ? 3 : 4;
}
template <int D>
__device__ __forceinline__ int load_lds(int i) {
  using C = Cfg<D>;
  if (i < C::kKCInstr) return C::kKC + i * 1024;
  if (i < C::kKCInstr + C::kVCInstr) return C::kVC + (i - C::kKCInstr) * 1024;
  if (i < C::kKCInstr + C::kVCInstr + C::kKSInstr) return C::kKS + (i - C::kKCInstr - C::kVCInstr) * 256;
  return C::kVS + (i - C::kKCInstr - C::kVCInstr - C::kKSInstr) * 256;
}

template <int D>
__device__ __forceinline__ void issue_one(const Slices& sl, int sec, uint32_t dst, int voff, int k0) {
  using C = Cfg<D>;
  if (sec == 0) dma<16>(sl.r[0], dst, voff + k0 * C::kKRow);
  else if (sec == 1) dma<16>(sl.r[1], dst, voff + k0 * C::kKRow);
  else if (sec == 2) dma<4>(sl.r[2], dst, voff + k0);
  else dma<4>(sl.r[3], dst, voff + (k0 / kBlock) * D);
}

// Issue this wave's n loads of the tile starting at key k0 into the stage at LDS address stage.
// Load I of wave w is stage load w + W I; where all waves' loads I fall in one section, that
// section is known at compile time and the load needs no branch.  LDS addresses are computed
// from the (scalar) wave index, so they need no vector work.
template <int D, int WAVES, int I = 0>
__device__ __forceinline__ void issue_tile(const Slices& sl, const LoadOp* ops, int wave_u, int n, uint32_t stage,
                                           int k0) {
  using C = Cfg<D, WAVES>;
  constexpr int W = C::kWaves;
  if constexpr (I < C::kMaxLoadsPerWave) {
    const int j = wave_u + W * I;
    constexpr int s_lo = load_section<D>(W * I), s_hi = load_section<D>(W * I + W - 1);
    if constexpr (s_lo == s_hi && s_lo < 4) {
      issue_one<D>(sl, s_lo, stage + load_lds<D>(j), ops[I].voff, k0);
    } else {
      if (I >= n) return;
      issue_one<D>(sl, load_section<D>(j), stage + load_lds<D>(j), ops[I].voff, k0);
    }
    issue_tile<D, WAVES, I + 1>(sl, ops, wave_u, n, stage, k0);
  }
}

// s_waitcnt for "at most N vector-memory operations of this wave outstanding" (gfx9 encoding;
// the other counters are left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// the same for a wave-uniform n <= MAX (the waves of a work-group issue different numbers of loads)
template <int MAX>
__device__ __forceinline__ void wait_vmem_n(int n) {
  if constexpr (MAX > 0) {
    if (n >= MAX) {
      wait_vmem<MAX>();
      return;
    }
    wait_vmem_n<MAX - 1>(n);
  } else {
    wait_vmem<0>();
  }
}

// Smooth-QK scales of channels c0 .. c0+31 of KV head kvh, or nullptr for no rescale.
__device__ __forceinline__ const float* q_smooth_blk(const AttnArgs& a, int kvh, int d, int c0) {
  return a.q_smooth != nullptr ? a.q_smooth + (int64_t)kvh * d + c0 : nullptr;
}

// PH: the P-hat rule: 0 = one scale per (row, 32-key block), codes from the FP16 probabilities
// (the method); 1 = one scale per (row, tile) (accuracy variant); 2 = Direct-P codes, one scale
// per (row, 32-key block)
// The 8-wave instances keep their registers at the 6-waves-per-SIMD budget; the small-grid ones
// (4 waves per work-group) are held by LDS to 4 waves per SIMD, and their budget says so.
template <int D, bool CAUSAL, int MODE, bool STATS, int PH, int WAVES = PREFILL_WAVES>
__global__ __launch_bounds__(WAVES * 64, (MODE == 0 && !STATS && WAVES == PREFILL_WAVES) ? PREFILL_MIN_WAVES : 4) void attn_prefill_kernel(AttnArgs a) {
  using Cf = Cfg<D, WAVES>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * Cf::kStageBytes];
  constexpr int W = Cf::kWaves;
  constexpr int KSTEPS = Cf::kKSteps;
  constexpr int CB = Cf::kCB;

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
  // XCD-aware order: the hardware deals work-groups round-robin over the 8 XCDs, so hardware
  // index i runs on XCD i % 8.  Renumbering gives each XCD a contiguous range of logical
  // work-groups (x fastest: the query blocks of one (batch, KV head) together), so the K-hat /
  // V-hat tiles those work-groups share stay in that XCD's L2.
  // (64-bit: the grid's three dimensions may multiply past 2^32)
  const uint64_t gx = gridDim.x, gy = gridDim.y;
  const uint64_t nwg = gx * gy * gridDim.z;
  const uint64_t hwid = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const uint64_t per = nwg / 8, rem = nwg % 8, xcd = hwid % 8;
  uint64_t j = hwid / 8;  // dispatch position inside the XCD's range
  if constexpr (CAUSAL && PREFILL_SNAKE && WAVES == PREFILL_SMALL_GRID_WAVES) {
    // A small causal grid is resident all at once, and an XCD deals its work-groups over its 32
    // compute units in turn, so compute unit c would get positions c, c + 32, ...: with the
    // heaviest blocks first, the low units would get the heaviest of every round.  Reversing
    // every other round of 32 gives unit c blocks c, 63 - c, 64 + c, ... of the heaviest-first
    // order, whose lengths sum about equally.  (A bijection of the XCD's range, checked on the CPU.)
    const uint64_t n_x = per + (xcd < rem ? 1 : 0);
    const uint64_t r = j / kCUsPerXCD, c = j % kCUsPerXCD;
    if (r & 1) {
      const uint64_t m = n_x - kCUsPerXCD * r < (uint64_t)kCUsPerXCD ? n_x - kCUsPerXCD * r : (uint64_t)kCUsPerXCD;
      j = kCUsPerXCD * r + (m - 1 - c);
    }
  }
  const uint64_t lin = xcd * per + (xcd < rem ? xcd : rem) + j;
  const uint32_t bx = (uint32_t)(lin % gx), by = (uint32_t)((lin / gx) % gy), bz = (uint32_t)(lin / (gx * gy));
  const int kvh = by / chunks;
  const int h = kvh * group + (by % chunks) * hw + wave / wph;
  const int b = bz;
  // heaviest causal blocks first: they start while the short ones fill the tail
  const int qblk = CAUSAL ? (int)(gridDim.x - 1 - bx) : (int)bx;
  const int lq = (int)a.len_q, lk = (int)a.len_kv, lk32 = (int)a.len_kv32;
  const int64_t rows = a.kv_rows, rows32 = a.kv_rows32;  // strides of the K-hat / V-hat buffers
  const int q_wg = qblk * bq;
  const int q0 = q_wg + 16 * (wave % wph);  // first query row of this wave
  const int shift = lk - lq;                // causal: key c visible to query r iff c <= r + shift
  const int bc = a.kv_tile;

  // ---- Q-hat^T operand (B operand of the score MFMA), kept in registers
  uint4 qreg[KSTEPS];
  uint32_t qsc[KSTEPS];
  // FP16 Q (fused quantization): this lane's own 32-element block (4s + g) of query row q0 + col
  // is loaded here and quantized once the first K/V tile is in flight, so the two latencies overlap
  const bool fused_q = a.q_fp16 != nullptr;
  const bool q_has = q0 + col < lq && (D >= 128 || g < 2);
  Block32In qin[KSTEPS];
  {
    const int q = q0 + col;
    if (fused_q) {
      if (q_has) {
        const uint16_t* qx = a.q_fp16 + (((int64_t)b * a.heads_q + h) * lq + q) * D;
        // the channel scales are loaded with the values where registers allow (one K-step)
#pragma unroll
        for (int s = 0; s < KSTEPS; s++)
          load_block32(qx + 128 * s + 32 * g, KSTEPS == 1 ? q_smooth_blk(a, kvh, D, 128 * s + 32 * g) : nullptr, qin[s]);
      }
    } else {
      const uint8_t* qc = a.q_codes + ((int64_t)b * a.heads_q + h) * (int64_t)lq * (D / 2);
      const uint8_t* qs = a.q_scales + ((int64_t)b * a.heads_q + h) * (int64_t)lq * (D / kBlock);
#pragma unroll
      for (int s = 0; s < KSTEPS; s++) {
        const bool has = q < lq && (D >= 128 || g < 2);
        qreg[s] = has ? *reinterpret_cast<const uint4*>(qc + (int64_t)q * (D / 2) + 64 * s + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
        qsc[s] = has ? qs[(int64_t)q * (D / kBlock) + 4 * s + g] : 127u;
      }
    }
  }

  // the Q-hat loads complete here, so no wait for them lands inside the tile loop
  if (!fused_q) wait_vmem<0>();

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

  const int64_t slice = (int64_t)b * a.heads_kv + kvh;
  Slices sl;
  // slices start at the buffers' strides; the ranges cover the attended keys only, so loads past
  // them return zeros
  sl.r[0] = make_desc(a.k_codes + slice * rows * (D / 2), (int64_t)lk * (D / 2));
  sl.r[1] = make_desc(a.v_codes + slice * rows32 * (D / 2), (int64_t)lk32 * (D / 2));
  sl.r[2] = make_desc(a.k_scales + slice * (D / kBlock) * rows32, (int64_t)(D / kBlock) * rows32);
  sl.r[3] = make_desc(a.v_scales + slice * (rows32 / kBlock) * D, (int64_t)(lk32 / kBlock) * D);
  const uint32_t smem_lds = lds_addr(smem);
  // this wave's share of the stage loads: instructions wave, wave + W, ...
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n_loads = wave_u < Cf::kInstr ? (Cf::kInstr - wave_u + W - 1) / W : 0;
  LoadOp ops[Cf::kMaxLoadsPerWave];
#pragma unroll
  for (int i = 0; i < Cf::kMaxLoadsPerWave; i++) ops[i] = load_op<D>(wave_u + W * i, lane, (int)rows32);
  constexpr float C = SoftmaxC<D>::value;  // equals a.c_log2 (checked by the launcher)

  // per-lane LDS offsets of this lane's MFMA operands (see the reads in the tile loop)
  const int k_lane_off = Cf::kKC + 16 * lane;
  const int ks_lane_off = Cf::kKS + g * kTileKeys + 32 * (col >> 2) + 8 * (col & 3);
  const int v_lane_off = Cf::kVC + 16 * lane;
  const int vs_lane_off = Cf::kVS + g * D + CB * col;

  // prologue: tiles 0 .. kStages-2 in flight, wait for tile 0
#pragma unroll
  for (int p = 0; p < kStages - 1; p++)
    if (p < n_tiles) issue_tile<D, WAVES>(sl, ops, wave_u, n_loads, smem_lds + p * Cf::kStageBytes, p * bc);
  if (fused_q) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KSTEPS; s++) {
      qreg[s] = make_uint4(0u, 0u, 0u, 0u);
      qsc[s] = 127u;
      if (q_has) {
        if (KSTEPS > 1) load_block32(nullptr, q_smooth_blk(a, kvh, D, 128 * s + 32 * g), qin[s]);
        qsc[s] = quantize_loaded32(qin[s], a.q_smooth != nullptr, &qreg[s]);
      }
    }
  }
  if (kStages > 2 && n_tiles > 1) wait_vmem_n<Cf::kMaxLoadsPerWave>(n_loads);
  else wait_vmem<0>();
  __syncthreads();

  for (int tile = 0; tile < n_tiles; tile++) {
    const int k0 = tile * bc;
    const uint8_t* T = smem + (tile % kStages) * Cf::kStageBytes;
    const int ahead = tile + kStages - 1;
    if (ahead < n_tiles) issue_tile<D, WAVES>(sl, ops, wave_u, n_loads, smem_lds + (ahead % kStages) * Cf::kStageBytes, ahead * bc);

    if (wave_live && !(CAUSAL && k0 > wave_last + shift)) {
      // ---- S^T = K-hat Q-hat^T: MFMA t takes key score_row_key(t, r) as row r; its operands sit
      // in LDS in lane order.  Lane (g, col) then holds keys 32 g + 8 i + t in s[4 t + i].
      const uint8_t* kbase = T + k_lane_off;
      // the lane's 8 K-hat scale bytes of each contraction step (byte t serves MFMA t)
      uint2 ksw[KSTEPS];
#pragma unroll
      for (int st = 0; st < KSTEPS; st++) {
        ksw[st] = *reinterpret_cast<const uint2*>(T + ks_lane_off + 4 * kTileKeys * st);
        if (D < 128 && g >= 2) ksw[st] = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      }
      // operands read two MFMAs ahead into a double buffer, so LDS latency hides behind the
      // matrix pipe instead of stalling each MFMA
      constexpr int NK = 8 * KSTEPS;
      auto kop = [&](int j) -> uint4 {
        if (D < 128 && g >= 2) return make_uint4(0u, 0u, 0u, 0u);
        return *reinterpret_cast<const uint4*>(kbase + 1024 * j);
      };
      uint4 ka[2];
      ka[0] = kop(0);
      ka[1] = kop(1);
      float s[32];
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NK; j++) {
        const int t = j / KSTEPS, st = j % KSTEPS;
        if (st == 0) acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t kw = t < 4 ? ksw[st].x : ksw[st].y;
        switch (t & 3) {
          case 0: acc = mfma_fp4_sel<0, 0>(ka[j & 1], kw, qreg[st], qsc[st], acc); break;
          case 1: acc = mfma_fp4_sel<1, 0>(ka[j & 1], kw, qreg[st], qsc[st], acc); break;
          case 2: acc = mfma_fp4_sel<2, 0>(ka[j & 1], kw, qreg[st], qsc[st], acc); break;
          default: acc = mfma_fp4_sel<3, 0>(ka[j & 1], kw, qreg[st], qsc[st], acc); break;
        }
        if (j + 2 < NK) ka[j & 1] = kop(j + 2);
        if (st == KSTEPS - 1) {
#pragma unroll
          for (int i = 0; i < 4; i++) s[4 * t + i] = acc[i];
        }
        __builtin_amdgcn_sched_barrier(0);
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
        const int rel = lim - kb;  // key offset s_key(k) of the lane's block is visible iff <= rel
        // the mask as arithmetic (no compare and select, whose condition register costs wait
        // states): min(s, +inf) keeps a visible score, min(s, -inf) masks one; the sign of
        // rel - s_key(k) + 1/2 (never 0) tells which, and times +inf it is that bound
        const float relf = (float)(rel < -1 ? -1 : (rel > 31 ? 31 : rel));
#pragma unroll
        for (int k = 0; k < 32; k++) {
          const float lim_k = (relf + (0.5f - (float)s_key(k))) * INFINITY;
          s[k] = min_nn(s[k], lim_k);
          bmax = fmaxf(bmax, s[k]);
        }
      }
      const float rmax = group_max4(bmax);
      // ---- integer running max, FP16 rescale factor; P-hat scale of this lane's block (its own
      // maximum bmax: the lane holds one 32-key block of its row), or of the row's tile (PH = 1)
      RowStep rs;
      if constexpr (MODE == 2) rs = row_step_nearest16(rmax, m, C);
      else rs = row_step(rmax, m, C);
      const PhatScale ps = phat_scale<PH == 2>(PH == 1 ? rmax : bmax, C, rs.mm);
      uint32_t p16[16];
      uint4 ph;
      if constexpr (PH == 2) ph = phat_codes_direct(s, C, ps.neg_big_m);
      else ph = phat_codes(s, C, ps.neg_big_m, p16);
      const uint32_t psc = (uint32_t)(int)(ps.e + 127.0f);
      // ---- normalizer increment: rowsum(P-hat) from the ones column, or the FP32 tree sum
      const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
      v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
      lacc = mfma_fp4(ones, 127u, ph, psc, lacc);
      float lsum = lacc[0];
      if (MODE == 1 || STATS) {
        // the lane's block sum of FP16 probabilities times its block scale (exact)
        const float sb = tree_sum32_h(p16) * e8m0_as_float((int)ps.e);
        if (MODE == 1) lsum = group_sum4(sb);
        if (STATS) {
          float sp = sb;
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
      // ---- O^T += V-hat^T P-hat^T per channel block (PV MFMA cb takes channel 16 cb + r as row
      // r; operands in lane order); FP16 state update
      const uint8_t* vbase = T + v_lane_off;
      // the lane's CB V-hat scale bytes (byte cb: channel 16 cb + col, adjacent in the layout)
      uint32_t vsw[CB / 4];
      if constexpr (CB == 4) {
        vsw[0] = *reinterpret_cast<const uint32_t*>(T + vs_lane_off);
      } else if constexpr (CB == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(T + vs_lane_off);
        vsw[0] = w.x;
        vsw[1] = w.y;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(T + vs_lane_off);
        vsw[0] = w.x;
        vsw[1] = w.y;
        vsw[2] = w.z;
        vsw[3] = w.w;
      }
      // V-hat operands two MFMAs ahead; the state update of block cb - 1 follows MFMA cb, so the
      // matrix result latency is covered by the next MFMA
      uint4 va[2];
      va[0] = *reinterpret_cast<const uint4*>(vbase);
      va[1] = *reinterpret_cast<const uint4*>(vbase + 1024);
      v4f pv[2];
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const uint32_t vw = vsw[cb / 4];
        const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
        switch (cb & 3) {
          case 0: pv[cb & 1] = mfma_fp4_sel<0, 0>(va[cb & 1], vw, ph, psc, z); break;
          case 1: pv[cb & 1] = mfma_fp4_sel<1, 0>(va[cb & 1], vw, ph, psc, z); break;
          case 2: pv[cb & 1] = mfma_fp4_sel<2, 0>(va[cb & 1], vw, ph, psc, z); break;
          default: pv[cb & 1] = mfma_fp4_sel<3, 0>(va[cb & 1], vw, ph, psc, z); break;
        }
        // keeps the update of block cb - 1 behind MFMA cb: hoisted above it, the update waits
        // out the matrix latency of block cb - 1 with wait states (measured 1 % slower)
        __builtin_amdgcn_sched_barrier(0);
        if (cb + 2 < CB) va[cb & 1] = *reinterpret_cast<const uint4*>(vbase + 1024 * (cb + 2));
        if (cb >= 1) state_update(o[cb - 1], rs.alpha, pv[(cb - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      state_update(o[CB - 1], rs.alpha, pv[(CB - 1) & 1]);
      l = __builtin_fmaf16(rs.alpha, l, (_Float16)lsum);
      m = rs.m_new;
    }

    // tile + 1 must be resident before the barrier; the loads of tile + 2 may stay in flight
    if (kStages > 2 && tile + 2 < n_tiles) wait_vmem_n<Cf::kMaxLoadsPerWave>(n_loads);
    else wait_vmem<0>();
    __syncthreads();
  }

  // ---- epilogue: out = fp16(O / l); register i of block cb holds channel 16 cb + 4 g + i.  The
  // last barrier of the tile loop has freed the LDS ring: each wave stages its 16 x D output tile
  // there (rows padded by 16 bytes, so the 16 rows of a store do not share banks) and stores it
  // back row-contiguous, 1 KB per store instruction, instead of scattering 32-byte pieces of 16
  // rows from every store
  if (!wave_live) return;
  constexpr int kRowBytes = 2 * D + 16;
  static_assert(W * 16 * kRowBytes <= kStages * Cf::kStageBytes, "output staging fits the LDS ring");
  uint8_t* stile = smem + wave * 16 * kRowBytes;
  write_out_row<CB>(stile + col * kRowBytes + 8 * g, o, (float)l);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes have completed
  uint16_t* out = a.out + (((int64_t)b * a.heads_q + h) * (int64_t)lq + q0) * D;
  constexpr int kChunks = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < 16 * kChunks / 64; i++) {
    const int c = 64 * i + lane, r = c / kChunks, cc = c % kChunks;
    const uint4 val = *reinterpret_cast<const uint4*>(stile + r * kRowBytes + 16 * cc);
    if (q0 + r < lq) *reinterpret_cast<uint4*>(out + (int64_t)r * D + 8 * cc) = val;
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

// Grid of WAVES-wave work-groups: gcd(group, WAVES) query heads each, 16 * WAVES / heads rows of each
template <int D, int WAVES>
dim3 prefill_grid(AttnArgs& a) {
  const int group = a.heads_q / a.heads_kv;
  const int hw = gcd_int(group, WAVES);  // query heads per work-group
  const int bq = 16 * (WAVES / hw);
  a.heads_per_wg = hw;
  const int64_t qblocks = (a.len_q + bq - 1) / bq;
  return dim3((uint32_t)qblocks, (uint32_t)(a.heads_kv * (group / hw)), (uint32_t)a.batch);
}

// Work-groups of the default shape that fit on the chip at once: 256 compute units, each with
// room (registers and LDS) for three 8-wave work-groups at d <= 128.
constexpr int64_t kResidentWorkGroups = 256 * 3;

template <int D, bool CAUSAL, int MODE, bool STATS, int PH = 0>
hipError_t launch4(AttnArgs a, hipStream_t s) {
  // A causal grid of 8-wave work-groups that fills the chip at most once (short or
  // single-sequence prefill) leaves SIMDs idle, and its blocks, whose lengths differ by up to the
  // whole key range, finish unevenly.  The method's P-Reordered instance then runs 4-wave
  // work-groups: twice as many, each holding one wave per SIMD, so more SIMDs share the heavy
  // blocks (d128, Hq32/Hkv8: B1 L2048 33.8 -> 30.6 us, B1 L3072 57.4 -> 51.8 us, B2 L1024 26.6 ->
  // 22.7 us; at 1024 8-wave work-groups, B2 L2048, 8 waves stay 9 % faster).  A non-causal grid has
  // no such imbalance and keeps 8 waves, whose K/V tiles serve twice the rows (B1 L2048: 4 waves
  // 45.1 us, 8 waves 42.7 us).  Each wave computes the same 16 rows over the same tiles either
  // way, so the output is bit-identical.  opts.prefill_waves overrides the choice.
  if constexpr (PREFILL_SMALL_GRID_WAVES > 0 && MODE == 0 && !STATS && PH == 0) {
    AttnArgs big = a;
    const dim3 g = prefill_grid<D, PREFILL_WAVES>(big);
    // d = 256: LDS holds two work-groups per CU whatever their size, so 4-wave ones halve the
    // residency of any 8-wave grid with two per CU; they pay only where that grid leaves half the
    // CUs idle (Hq16/Hkv8: B1 L1024 22.5 -> 20.5 us; B1 L2048, 256 work-groups, even at 36.5-36.9;
    // B1 L4096 78.5 us with 8 waves, 92.0 with 4)
    const int64_t limit = D <= 128 ? kResidentWorkGroups : 128;
    const bool small = CAUSAL && (int64_t)g.x * g.y * g.z <= limit;
    if (a.wg_waves == PREFILL_SMALL_GRID_WAVES || (a.wg_waves == 0 && small)) {
      const dim3 gs = prefill_grid<D, PREFILL_SMALL_GRID_WAVES>(a);
      hipLaunchKernelGGL((attn_prefill_kernel<D, CAUSAL, MODE, STATS, PH, PREFILL_SMALL_GRID_WAVES>), gs,
                         dim3(PREFILL_SMALL_GRID_WAVES * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.wg_waves != 0 && a.wg_waves != PREFILL_WAVES) return hipErrorInvalidValue;  // checked by the API
  const dim3 g = prefill_grid<D, PREFILL_WAVES>(a);
  hipLaunchKernelGGL((attn_prefill_kernel<D, CAUSAL, MODE, STATS, PH>), g, dim3(Cfg<D>::kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch2(const AttnArgs& a, hipStream_t s) {
  const bool stats = a.stats != nullptr;
  // the variants run P-Reordered without tile statistics: the per-tile P-hat scale, Direct-P
  // codes, the round-to-nearest running max
  if (a.phat == 1) return launch4<D, CAUSAL, 0, false, 1>(a, s);
  if (a.phat == 2) return launch4<D, CAUSAL, 0, false, 2>(a, s);
  if (a.max_rule == 1) return launch4<D, CAUSAL, 2, false>(a, s);
  if (a.normalizer == 1) return stats ? launch4<D, CAUSAL, 1, true>(a, s) : launch4<D, CAUSAL, 1, false>(a, s);
  return stats ? launch4<D, CAUSAL, 0, true>(a, s) : launch4<D, CAUSAL, 0, false>(a, s);
}

template <int D>
hipError_t launch1(const AttnArgs& a, hipStream_t s) {
  if (a.c_log2 != SoftmaxC<D>::value) return hipErrorInvalidValue;  // the kernel's constant must be the caller's C
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
