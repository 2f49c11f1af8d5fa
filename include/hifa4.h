/*
 * hifa4.h -- C ABI of the MI355X (gfx950) 4-bit FlashAttention forward library (libhifa4.so).
 *
 * The operation follows "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for LLM
 * Inference" (arXiv 2607.04302v1), Abstract: Q and K get a calibration-static per-channel
 * Smooth-QK rescale after RoPE, Q, K, V are quantized to a 4-bit block format, and a tiled
 * attention kernel runs QK^T and PV as 4-bit matrix products while keeping the online-softmax
 * state (running max m, normalizer l, rescaled output O) in FP16.  The normalizer is accumulated
 * from the same quantized probabilities P-hat that enter the PV product (P-Reordering).
 *
 * 4-bit format (the HiFA4 abstract names it HIF4 without a bit layout; this library substitutes): E2M1
 * codes (sign, 2 exponent bits, 1 mantissa bit: 0, .5, 1, 1.5, 2, 3, 4, 6) with one
 * power-of-two E8M0 scale byte (2^(byte-127)) per block of 32 elements; two codes per byte,
 * the lower-index element in the low nibble.
 *
 * Memory layouts (all row-major, contiguous, no padding between rows):
 *   q        FP16 [B, Hq,  Lq, d]            k, v      FP16 [B, Hkv, Lk, d]
 *   q_codes  u8   [B, Hq,  Lq, d/2]          q_scales  u8   [B, Hq,  Lq, d/32]
 *   k_codes  u8   [B, Hkv, Lk, d/2]          k_scales  u8   [B, Hkv, d/32, Lk32]
 *                 (K-hat scales are block planes: for each 32-channel block, the scale bytes of
 *                 all keys; bytes of the padding keys Lk .. Lk32-1 are 0)
 *   v_codes  u8   [B, Hkv, Lk32/32, d, 16]   v_scales  u8   [B, Hkv, Lk32/32, d]
 *                 (V-hat is blocked along tokens and stored block-major: for each block of 32
 *                 tokens, the 16 code bytes of channel 0, then channel 1, ...; a key tile is one
 *                 contiguous run of bytes.  The scale bytes of a block are stored channel c at
 *                 position (d/16) * (c % 16) + c / 16.  Lk32 = Lk rounded up to 32, tail tokens
 *                 are 0)
 *   out      FP16 [B, Hq,  Lq, d]
 *   s, inv_s FP32 [Hkv, d]                   (query head h uses KV head h / (Hq/Hkv))
 *
 * Conventions: the caller owns every buffer; device pointers come from hipMalloc (or PyTorch's
 * allocator) and must be 16-byte aligned (the kernels move 16-byte vectors); device calls are asynchronous on the given HIP stream (NULL = default stream) and
 * never synchronize; no C++ exception crosses the ABI; a failed call launches nothing, returns a
 * status and leaves a description in hifa4_last_error() (thread-local).  The only global state
 * is that thread-local string, so calls from several threads are safe.
 * Supported: d in {64, 128, 256}; Hq % Hkv == 0 and (Hq/Hkv <= 8 or Hq/Hkv % 8 == 0);
 * Lq >= 1, Lk >= 1; causal requires Lq <= Lk (bottom-right aligned: key c is visible to query r
 * iff c <= r + Lk - Lq).  Scores must satisfy |S * log2(e)/sqrt(d)| < 2048 (the running max is
 * an FP16 integer).
 */
#ifndef HIFA4_H
#define HIFA4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HIFA4_OK = 0,
  HIFA4_ERR_NULL = 1,        /* a required pointer is NULL */
  HIFA4_ERR_SHAPE = 2,       /* inconsistent or out-of-range dimensions */
  HIFA4_ERR_UNSUPPORTED = 3, /* valid request this library does not implement */
  HIFA4_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  HIFA4_ERR_HIP = 5,         /* the HIP runtime reported an error (launch, device) */
  HIFA4_ERR_ALIGNMENT = 6    /* a device pointer is not 16-byte aligned */
} hifa4_status;

typedef struct {
  int32_t batch;    /* B   >= 1 */
  int32_t heads_q;  /* Hq  >= 1 */
  int32_t heads_kv; /* Hkv >= 1, divides Hq */
  int32_t head_dim; /* d in {64, 128, 256} */
  int64_t len_q;    /* Lq  >= 1 */
  int64_t len_kv;   /* Lk  >= 1 */
} hifa4_dims;

enum { HIFA4_P_REORDERED = 0, HIFA4_INCONSISTENT = 1 };

/* Running-max rules.  HIFA4_MAX_CEIL is the method as this library reads the HiFA4 abstract's
   FP16 online-softmax state: m = max over tiles of ceil(fp32(max S * C)), an integer, so every
   rescale 2^(m_old - m_new) is an exact power of two.  HIFA4_MAX_NEAREST16 is an accuracy
   variant: m = max over tiles of rn16(fp32(max S * C)), the rescale alpha = rn16(2^rn16(fp32(
   m_old - m_new))), and m + e (below) is rounded once to FP32; prefill, P-Reordered, without
   tile statistics. */
enum { HIFA4_MAX_CEIL = 0, HIFA4_MAX_NEAREST16 = 1 };

/* P-hat scale granularity.  HIFA4_PHAT_BLOCK32 is the method as this library reads the HiFA4
   abstract (P-hat is the 4-bit operand of the PV product, so it takes the 4-bit block format):
   one power-of-two scale per (query row, 32-key block).  HIFA4_PHAT_TILE is an accuracy variant
   with one scale per (query row, key tile), from the row's largest score in the tile. */
enum { HIFA4_PHAT_BLOCK32 = 0, HIFA4_PHAT_TILE = 1 };

/* P-hat code rule.  HIFA4_PHAT_EXP16 (the method): the E2M1 codes of the FP16 probabilities
   rn16(2^rn16(u)).  HIFA4_PHAT_DIRECT (Direct-P, after the "Hardware-Aware FP4 FlashAttention-4"
   abstract, which maps scores straight to FP4 probabilities): no exponential; the log2-domain score
   x = fma32(S, C, K), K = fp32(fp32(127 - (m + e)) + delta) - 127 with delta = fp32(1/4 -
   log2(1.5)/2), becomes 2^floor(x) (1 + frac(x)) (mantissa truncated to 23 bits), rounded to E2M1;
   the block exponent is e = max(-127, ceil(fp32(fma32(max S, C, -m) + fp32(delta - 2.5)))).
   Codes of value >= 1 then go to the E2M1 value nearest in the log2 domain. */
enum { HIFA4_PHAT_EXP16 = 0, HIFA4_PHAT_DIRECT = 1 };

typedef struct {
  int32_t causal;     /* 0 or 1 */
  int32_t normalizer; /* HIFA4_P_REORDERED: l from P-hat (the method); HIFA4_INCONSISTENT: l from
                         the FP32 probabilities before quantization (the conventional formulation
                         whose error Theorem 1 of the HiFA4 abstract describes) */
  int32_t kv_tile;    /* keys per tile, 64 or 128; part of the numerical definition (the FP16
                         state is rounded once per tile) */
  int32_t num_splits; /* Lq == 1 only: split-KV count; 0 = choose automatically (see
                         hifa4_decode_num_splits); part of the numerical definition */
  int64_t kv_capacity; /* key rows allocated per (batch, KV head) in the K-hat / V-hat buffers
                          (a cache filled by hifa4_cache_append); 0 = Lk.  The layouts above then
                          hold with Lk (Lk32) replaced by kv_capacity (rounded up to 32) for the
                          strides, while Lk keys are attended */
  int32_t max_rule;    /* HIFA4_MAX_CEIL (0) or HIFA4_MAX_NEAREST16 (1, prefill only) */
  int32_t phat_scale;  /* HIFA4_PHAT_BLOCK32 (0, the method) or HIFA4_PHAT_TILE (1) */
  int32_t phat_rule;   /* HIFA4_PHAT_EXP16 (0, the method) or HIFA4_PHAT_DIRECT (1, with
                          HIFA4_PHAT_BLOCK32 only) */
  int32_t prefill_waves; /* prefill work-group size in waves of 16 query rows: 0 = automatic (4 for
                            causal grids of at most 768 8-wave work-groups at d <= 128, all
                            resident at once, or at most 128 at d = 256; 8 otherwise), 4 or 8.  4 exists for HIFA4_P_REORDERED, HIFA4_MAX_CEIL, the method's P-hat
                            and no tile statistics (HIFA4_ERR_UNSUPPORTED otherwise).  Not part of
                            the numerical definition: every wave computes the same rows over the
                            same tiles, so the output is bit-identical.  Decode ignores it. */
} hifa4_attn_opts;

/*
 * Smooth-QK calibration (host, synchronous).  [HiFA4 Abstract: the per-channel Smooth-QK factors
 * are static, derived once offline from calibration data.]  q_cal FP16 bits [Hq, N, d], k_cal FP16 bits
 * [Hkv, N, d] (post-RoPE).  Per (KV head g, channel j): aK = max|k_cal[g, :, j]|, aQ = max over
 * the tokens and the query heads of group g of |q_cal|.  Gate: rho = max(aK) / median(aK) over
 * all (g, j); Smooth-QK is on iff rho >= gate_tau.  s = aK^alpha / aQ^(1-alpha) where on and both
 * maxima are non-zero, else 1; outputs s (FP32 of s) and inv_s (FP32 of 1/s computed in FP64),
 * both [Hkv, d] host arrays owned by the caller; *gate_on receives 0/1.
 * Errors: HIFA4_ERR_NULL, HIFA4_ERR_SHAPE (N < 1, Hq % Hkv != 0, d < 1, alpha outside [0, 1]).
 */
hifa4_status hifa4_calibrate(const uint16_t* q_cal, const uint16_t* k_cal, int64_t n_tokens,
                             int32_t heads_q, int32_t heads_kv, int32_t head_dim, float alpha,
                             float gate_tau, float* s, float* inv_s, int32_t* gate_on);

/*
 * Smooth-QK rescale + 4-bit quantization (device, async).  [HiFA4 Abstract: only a fusible
 * element-wise scaling remains at inference.]  Q' = fp32(Q * s[g(h)]), K' = fp32(K * inv_s[g]),
 * V' = V; each 32-element block (Q, K along d; V along tokens) gets the exponent
 * e = smallest with 6 * 2^e >= max|x| (clamped to [-127, 127], -127 for an all-zero block) and
 * codes = round-to-nearest-even(x / 2^e) on the E2M1 grid (ties to the even code, sign copied).
 * Any of q, k, v may be NULL to skip that tensor (its outputs are then not touched); s and inv_s
 * may be NULL for no rescale (both or neither).  Outputs use the layouts above.
 * Errors: HIFA4_ERR_NULL (an output of a present input is NULL), HIFA4_ERR_SHAPE,
 * HIFA4_ERR_UNSUPPORTED (d), HIFA4_ERR_ALIGNMENT, HIFA4_ERR_HIP.
 */
hifa4_status hifa4_quantize_qkv(const hifa4_dims* dims, const void* q, const void* k,
                                const void* v, const float* s, const float* inv_s,
                                void* q_codes, void* q_scales, void* k_codes, void* k_scales,
                                void* v_codes, void* v_scales, void* hip_stream);

/* Block scale rules of hifa4_quantize_qkv_rule. */
enum { HIFA4_SCALE_NO_CLIP = 0, HIFA4_SCALE_FLOOR = 1 };

/*
 * hifa4_quantize_qkv with a choice of block scale rule, for accuracy comparisons.
 * HIFA4_SCALE_NO_CLIP is the rule above (the method's: no element is clipped);
 * HIFA4_SCALE_FLOOR is the shared-exponent rule of the OCP microscaling format,
 * e = floor(log2 max|x|) - 2 clamped to [-127, 127] (-127 for a zero block), whose codes saturate
 * at 6 for magnitudes in (6, 8) * 2^e.  Errors: those of hifa4_quantize_qkv; HIFA4_ERR_SHAPE for
 * another rule.
 */
hifa4_status hifa4_quantize_qkv_rule(const hifa4_dims* dims, int32_t scale_rule, const void* q, const void* k,
                                     const void* v, const float* s, const float* inv_s, void* q_codes,
                                     void* q_scales, void* k_codes, void* k_scales, void* v_codes,
                                     void* v_scales, void* hip_stream);

/*
 * RoPE, Smooth-QK rescale and 4-bit quantization from pre-RoPE inputs, fused (device, async).
 * [HiFA4 Abstract: Smooth-QK rescales Q and K per channel after RoPE, and at inference only an
 * element-wise scaling remains, fusible into the preceding step.]  q, k hold FP16 values before
 * the rotary embedding; rope_cos, rope_sin are FP32 [rope_positions, d/2] device tables of the
 * rotate-half embedding (entry (p, i) rotates channels i and i + d/2 at position p).  Key t sits
 * at position t, query r at r + Lk - Lq.  Per pair, in FP32 with one rounding per product and per
 * sum: y_i = x_i c - x_{i+d/2} s, y_{i+d/2} = x_{i+d/2} c + x_i s; the rotated values are not
 * rounded to FP16; then Q' = fp32(y * s[g(h)]), K' = fp32(y * inv_s[g]) and the block
 * quantization of hifa4_quantize_qkv, with the same output layouts.  V is quantized as there.
 * Errors: those of hifa4_quantize_qkv; HIFA4_ERR_NULL for missing tables when q or k is given;
 * HIFA4_ERR_SHAPE when rope_positions < Lk or (q given) Lq > Lk.
 */
hifa4_status hifa4_quantize_qkv_rope(const hifa4_dims* dims, const void* q, const void* k, const void* v,
                                     const float* s, const float* inv_s, const float* rope_cos,
                                     const float* rope_sin, int64_t rope_positions, void* q_codes,
                                     void* q_scales, void* k_codes, void* k_scales, void* v_codes,
                                     void* v_scales, void* hip_stream);

/*
 * Append keys to a 4-bit K-hat / V-hat cache (device, async): in decoding, each new token's key
 * and value join the quantized cache before its attention.  dims->len_kv = keys already in the
 * cache (L0), dims->len_q = keys appended (n >= 1); heads_q is not used.  The cache buffers use
 * the layouts above with Lk replaced by kv_capacity (C >= L0 + n) for the strides:
 *   k_codes [B, Hkv, C, d/2], k_scales [B, Hkv, d/32, C32], v_codes [B, Hkv, C32/32, d, 16],
 *   v_scales [B, Hkv, C32/32, d];  v_stage FP16 [B, Hkv, 32, d] (caller-owned, keeps the FP16
 *   keys of the V-hat block that is still open between calls; contents undefined at L0 = 0).
 * k_new, v_new: FP16 [B, Hkv, n, d] (k_new before RoPE when the tables are given: key t at
 * position t).  K-hat rows are quantized as hifa4_quantize_qkv (or _rope) does; the V-hat blocks
 * the new keys touch are quantized again from FP16, zero-padded past L0 + n.  After any sequence
 * of appends the first L keys of the cache equal hifa4_quantize_qkv(_rope) of those L keys, byte
 * for byte (K-hat scale bytes past L are unspecified; attention masks them).  Read it with
 * hifa4_attention_fwd(_q16) and opts.kv_capacity = C.
 * Errors: HIFA4_ERR_NULL, HIFA4_ERR_SHAPE (L0 + n > C, short RoPE tables), HIFA4_ERR_UNSUPPORTED
 * (d), HIFA4_ERR_ALIGNMENT, HIFA4_ERR_HIP.
 */
hifa4_status hifa4_cache_append(const hifa4_dims* dims, int64_t kv_capacity, const void* k_new, const void* v_new,
                                const float* inv_s, const float* rope_cos, const float* rope_sin,
                                int64_t rope_positions, void* k_codes, void* k_scales, void* v_codes,
                                void* v_scales, void* v_stage, void* hip_stream);

/* Number of KV splits hifa4_attention_fwd uses for these dims and options (1 when Lq > 1). */
int32_t hifa4_decode_num_splits(const hifa4_dims* dims, const hifa4_attn_opts* opts);

/* Bytes of device workspace hifa4_attention_fwd needs (0 for prefill); 0 on invalid input. */
size_t hifa4_attention_workspace_bytes(const hifa4_dims* dims, const hifa4_attn_opts* opts);

/*
 * 4-bit attention forward (device, async).  [HiFA4 Abstract: QK^T and PV as 4-bit GEMMs,
 * online-softmax state in FP16, P-Reordering fused into the PV product.]
 * Per query row and per tile of kv_tile keys (ascending): S = Q-hat K-hat^T on the scaled FP4
 * matrix cores; m_new = max(m, ceil(fp32(max S * C))) with C = fp32(log2(e)/sqrt(d));
 * P-hat = E2M1 codes with one power-of-two scale 2^e per (query row, 32-key block) (P-hat is the
 * 4-bit operand of the PV product, so it takes the 4-bit block format), e = ceil(fp32(v - log2 6))
 * with v = fma(max over the block's visible S, C, -m_new) (-127 for a block without a visible
 * key), of the FP16 probabilities rn16(2^rn16(fma(S, C, -(m_new + e)))) (P-tilde = 2^e times
 * those); opts->phat_scale and opts->phat_rule select the variants above.  PV and the
 * l-increment = rowsum(P-hat) come from the same matrix-core pass; the state update is FP16
 * arithmetic, O = fma16(rn16(2^(m_old - m_new)), O, rn16(PV)), l likewise; out = fp16(O / l).
 * Lq == 1 runs split-KV decode (num_splits partial FP16 states in the workspace, merged in
 * split order); Lq > 1 runs the prefill kernel (workspace unused, may be NULL).
 * tile_stats: NULL, or FP32 [B, Hq, ceil(Lq/16), ceil(Lk/kv_tile), 2] receiving, per block of 16
 * query rows and key tile, (sum of P-hat, sum of P-tilde) over visible entries (zeros for tiles
 * a row block never visits); prefill only.
 * Under opts->max_rule = HIFA4_MAX_NEAREST16 the running max and the rescale follow that rule
 * (see the enum); Lq == 1, INCONSISTENT or tile_stats then return HIFA4_ERR_UNSUPPORTED.
 * HIFA4_PHAT_TILE and HIFA4_PHAT_DIRECT run P_REORDERED with HIFA4_MAX_CEIL and without
 * tile_stats (HIFA4_ERR_UNSUPPORTED otherwise; HIFA4_PHAT_DIRECT with HIFA4_PHAT_TILE too).
 * Errors: HIFA4_ERR_NULL, HIFA4_ERR_SHAPE, HIFA4_ERR_UNSUPPORTED, HIFA4_ERR_WORKSPACE,
 * HIFA4_ERR_ALIGNMENT, HIFA4_ERR_HIP.
 */
hifa4_status hifa4_attention_fwd(const hifa4_dims* dims, const hifa4_attn_opts* opts,
                                 const void* q_codes, const void* q_scales, const void* k_codes,
                                 const void* k_scales, const void* v_codes, const void* v_scales,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 float* tile_stats, void* hip_stream);

/*
 * The same forward pass with the Q quantization fused into the attention kernel.  [HiFA4
 * Abstract: the Smooth-QK rescale is element-wise and fusible.]  q is FP16 [B, Hq, Lq, d] and s
 * the Smooth-QK scales [Hkv, d] (device, or NULL for no rescale); each work-group rescales and
 * quantizes the query rows it serves exactly as hifa4_quantize_qkv would, in registers, so no
 * Q-hat is written to or read from memory.  Decode (Lq == 1) also takes rope_cos/rope_sin
 * (FP32 [rope_positions, d/2], both or neither): q is then taken before RoPE and rotated first,
 * exactly as hifa4_quantize_qkv_rope does (the query at position Lk - 1).  The output is
 * bit-identical to hifa4_quantize_qkv (or hifa4_quantize_qkv_rope) with the same arguments
 * followed by hifa4_attention_fwd; every other argument, the workspace rules and the errors are
 * those of hifa4_attention_fwd, plus HIFA4_ERR_SHAPE for tables shorter than Lk and
 * HIFA4_ERR_UNSUPPORTED for RoPE tables with Lq > 1 (prefill rotates Q faster as a streaming
 * pass: hifa4_quantize_qkv_rope, then hifa4_attention_fwd).
 */
hifa4_status hifa4_attention_fwd_q16(const hifa4_dims* dims, const hifa4_attn_opts* opts, const void* q,
                                     const float* s, const float* rope_cos, const float* rope_sin,
                                     int64_t rope_positions, const void* k_codes, const void* k_scales,
                                     const void* v_codes, const void* v_scales, void* out, void* workspace,
                                     size_t workspace_bytes, float* tile_stats, void* hip_stream);

/*
 * hifa4_attention_fwd_q16 without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Decode (Lq == 1) keeps its split partials in a fixed device array of the library, 8 MiB
 * (8388608 bytes) per GPU, held from the first call on that GPU until the process ends; prefill
 * needs no scratch.  The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); its first call on a device looks up the array's device address once.  Every other
 * argument, the output and the errors are those of hifa4_attention_fwd_q16, plus
 * HIFA4_ERR_WORKSPACE when hifa4_attention_workspace_bytes(dims, opts) exceeds 8 MiB.  The
 * partials are fully rewritten by every decode call before they are read, so nothing needs
 * clearing between calls; but all calls on one GPU share the one array, so calls that may
 * overlap on one GPU (on different streams, or from several threads) race and must be ordered
 * by the caller.
 */
hifa4_status hifa4_attention_fwd_q16_noalloc(const hifa4_dims* dims, const hifa4_attn_opts* opts, const void* q,
                                             const float* s, const float* rope_cos, const float* rope_sin,
                                             int64_t rope_positions, const void* k_codes, const void* k_scales,
                                             const void* v_codes, const void* v_scales, void* out,
                                             float* tile_stats, void* hip_stream);

/* Static description of a status code. */
const char* hifa4_status_string(hifa4_status status);

/* Detail of the last failure on the calling thread ("" if none); valid until the next call. */
const char* hifa4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HIFA4_H */
