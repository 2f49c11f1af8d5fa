// Internal launch interface between the C ABI (hifa4_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

struct QuantRowsArgs {
  const uint16_t* x;    // FP16 [rows, d]
  const float* scale;   // FP32 [Hs, d] or nullptr
  int64_t rows;         // B * H * L
  int64_t len;          // L
  int64_t len32;        // L rounded up to 32 (block-plane scales)
  int32_t heads;        // H
  int32_t heads_per_scale_row;  // query heads per KV head for Q (Hq/Hkv), 1 for K
  int32_t d;
  int32_t block_planes; // 0: scales [rows, d/32] (Q-hat); 1: [B*H, d/32, len32] (K-hat), tail 0
  uint8_t* codes;       // [rows, d/2]
  uint8_t* scales;
  int32_t scale_rule;   // 0: no-clip (the method); 1: OCP floor rule (accuracy variant)
};

struct QuantVtArgs {
  const uint16_t* v;    // FP16 [B*Hkv, L, d]
  int64_t bh;           // B * Hkv
  int64_t len;          // L
  int64_t len32;        // L rounded up to 32
  int32_t d;
  uint8_t* codes;       // [B*Hkv, len32/32, d, 16] (block-major)
  uint8_t* scales;      // [B*Hkv, len32/32, d]
  int32_t scale_rule;   // as in QuantRowsArgs
};

struct AttnArgs {
  const uint8_t* q_codes;   // Q-hat, or nullptr when q_fp16 is given
  const uint8_t* q_scales;
  const uint16_t* q_fp16;   // FP16 Q [B, Hq, Lq, d] quantized in the kernel prologue, or nullptr
  const float* q_smooth;    // Smooth-QK scales [Hkv, d] applied to q_fp16, or nullptr
  const float* rope_cos;    // FP32 [n_pos, d/2]: q_fp16 is before RoPE (query r at r + Lk - Lq), or nullptr
  const float* rope_sin;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  uint16_t* out;        // FP16 [B, Hq, Lq, d]
  float* stats;         // FP32 [B, Hq, ceil(Lq/16), n_tiles, 2] or nullptr
  uint16_t* part_o;     // decode: FP16 [B*Hq*S, d]
  uint16_t* part_ml;    // decode: FP16 [B*Hq*S, 2] (m, l)
  int32_t batch, heads_q, heads_kv, d;
  int64_t len_q, len_kv, len_kv32;
  int64_t kv_rows, kv_rows32;  // key rows allocated per (batch, KV head): the buffers' strides
  int32_t kv_tile;      // keys per tile (64 or 128)
  int32_t n_tiles;      // ceil(Lk / kv_tile)
  int32_t causal;
  int32_t normalizer;
  int32_t max_rule;     // 0: integer running max (the method's reading); 1: round-to-nearest FP16 (prefill)
  int32_t phat;         // P-hat rule: 0 per (row, 32-key block) from FP16 probabilities (the method's
                        // reading); 1 per (row, tile) (variant); 2 Direct-P codes per 32-key block
  int32_t num_splits;
  int32_t tiles_per_split;
  int32_t heads_per_wg;  // prefill: query heads served by one work-group (set by the launcher)
  int32_t wg_waves;      // prefill: requested waves per work-group (0 automatic, 4 or 8)
  float c_log2;         // fp32(log2(e) / sqrt(d)); the kernels use the same value as a constant per d
};

struct QuantRopeArgs {
  const uint16_t* x;    // FP16 [B, H, len, d], before RoPE
  const float* scale;   // Smooth-QK FP32 [Hs, d] or nullptr
  const float* rope_cos;  // FP32 [n_pos, d/2]
  const float* rope_sin;
  int64_t batch;
  int64_t len;          // L
  int64_t len32;        // L rounded up to 32 (block-plane scales)
  int64_t pos0;         // RoPE position of token 0 (Lk - Lq for Q, 0 for K)
  int32_t heads;        // H
  int32_t heads_per_scale_row;  // query heads per KV head for Q (Hq/Hkv), 1 for K
  int32_t scale_rows;   // Hs (rows of scale)
  int32_t d;
  int32_t block_planes; // 0: scales [rows, d/32] (Q-hat); 1: [B*H, d/32, len32] (K-hat), tail 0
  uint8_t* codes;       // [B*H*len, d/2]
  uint8_t* scales;
};
struct CacheAppendArgs {
  const uint16_t* k_new;  // FP16 [B*Hkv, n, d] (before RoPE when rope_cos is set)
  const uint16_t* v_new;  // FP16 [B*Hkv, n, d]
  const float* inv_s;     // Smooth-QK K factors [Hkv, d] or nullptr
  const float* rope_cos;  // FP32 [n_pos, d/2] or nullptr
  const float* rope_sin;
  int64_t bh;             // B * Hkv
  int32_t heads_kv;
  int32_t d;
  int64_t len0;           // keys already in the cache
  int64_t n;              // keys appended
  int64_t rows, rows32;   // capacity per (batch, KV head), and rounded up to 32
  uint8_t* k_codes;       // [B*Hkv, rows, d/2]
  uint8_t* k_scales;      // [B*Hkv, d/32, rows32]
  uint8_t* v_codes;       // [B*Hkv, rows32/32, d, 16]
  uint8_t* v_scales;      // [B*Hkv, rows32/32, d]
  uint16_t* v_stage;      // FP16 [B*Hkv, 32, d]: the keys of the open V-hat block
};
hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s);
hipError_t launch_cache_append(const CacheAppendArgs& a, hipStream_t s);
hipError_t launch_quantize_rope(QuantRopeArgs a, hipStream_t s);
// Q-hat (block_planes 0) and K-hat (block_planes 1) with RoPE and V-hat, one launch
hipError_t launch_quantize_qkv_rope(const QuantRopeArgs& qa, const QuantRopeArgs& ka, const QuantVtArgs& va,
                                    hipStream_t s);
hipError_t launch_quantize_vt(const QuantVtArgs& a, hipStream_t s);
// K-hat rows (block planes) and V-hat tiles of one (K, V) pair in one launch
hipError_t launch_quantize_kv(const QuantRowsArgs& ka, const QuantVtArgs& va, hipStream_t s);
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s);

// Bytes of the library's fixed decode scratch (one array per device, see decode_scratch).
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
// Device address of the current device's decode scratch (looked up once per device).
hipError_t decode_scratch(void** ptr);

}  // namespace hifa4
