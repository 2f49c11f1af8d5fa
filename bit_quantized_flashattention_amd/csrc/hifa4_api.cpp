// C ABI of libhifa4: argument validation, host-side Smooth-QK calibration, launch dispatch.
#include "hifa4.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

hifa4_status fail(hifa4_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

hifa4_status ok() {
  g_last_error.clear();
  return HIFA4_OK;
}

float half_bits_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const uint32_t ex = (h >> 10) & 0x1F;
  uint32_t man = h & 0x3FF;
  uint32_t bits;
  if (ex == 0) {
    if (man == 0) {
      bits = sign;
    } else {  // subnormal: normalize
      int e = -1;
      do {
        man <<= 1;
        e++;
      } while ((man & 0x400) == 0);
      bits = sign | ((uint32_t)(127 - 15 - e) << 23) | ((man & 0x3FF) << 13);
    }
  } else if (ex == 31) {
    bits = sign | 0x7F800000u | (man << 13);
  } else {
    bits = sign | ((ex - 15 + 127) << 23) | (man << 13);
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

int64_t round32(int64_t x) { return (x + 31) / 32 * 32; }

hifa4_status check_dims(const hifa4_dims* d) {
  if (d == nullptr) return fail(HIFA4_ERR_NULL, "dims is NULL");
  if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1 || d->len_q < 1 || d->len_kv < 1)
    return fail(HIFA4_ERR_SHAPE, "batch, heads and lengths must be >= 1");
  if (d->heads_q % d->heads_kv != 0) return fail(HIFA4_ERR_SHAPE, "heads_q must be a multiple of heads_kv");
  const int group = d->heads_q / d->heads_kv;
  if (group > 8 && group % 8 != 0)
    return fail(HIFA4_ERR_UNSUPPORTED, "heads_q / heads_kv must be <= 8 or a multiple of 8");
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(HIFA4_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (d->len_q >= (int64_t)1 << 31 || d->len_kv >= (int64_t)1 << 31)
    return fail(HIFA4_ERR_SHAPE, "lengths must be < 2^31");
  // the kernels address one (batch, KV head) slice of K-hat / V-hat codes with 32-bit offsets
  if (round32(d->len_kv) * (d->head_dim / 2) >= (int64_t)1 << 31)
    return fail(HIFA4_ERR_SHAPE, "len_kv * head_dim / 2 must stay below 2^31 bytes per (batch, KV head)");
  if (d->batch > 65535 || d->heads_q > 65535)
    return fail(HIFA4_ERR_SHAPE, "batch and heads_q must be <= 65535 (launch grid limits)");
  return HIFA4_OK;
}


int32_t auto_splits(const hifa4_dims* d, int kv_tile) {
  // enough (batch, KV head, split) waves to cover the 1024 SIMDs of the 256 compute units twice,
  // or once for up to 32 (batch, KV head) units, where each wave then keeps three tiles in flight
  // (the decode launcher's choice for grids of at most one wave per SIMD); at least 8 tiles per
  // split
  const int64_t tiles = (d->len_kv + kv_tile - 1) / kv_tile;
  const int64_t units = (int64_t)d->batch * d->heads_kv;
  const int64_t target = units <= 32 ? 1024 : 2048;
  int64_t s = (target + units - 1) / units;
  s = std::min<int64_t>(s, std::max<int64_t>(1, tiles / 8));
  s = std::max<int64_t>(1, std::min<int64_t>(s, 64));
  return (int32_t)s;
}

hifa4_status check_opts(const hifa4_dims* d, const hifa4_attn_opts* o) {
  if (o == nullptr) return fail(HIFA4_ERR_NULL, "opts is NULL");
  if (o->causal != 0 && o->causal != 1) return fail(HIFA4_ERR_SHAPE, "causal must be 0 or 1");
  if (o->normalizer != HIFA4_P_REORDERED && o->normalizer != HIFA4_INCONSISTENT)
    return fail(HIFA4_ERR_SHAPE, "normalizer must be HIFA4_P_REORDERED or HIFA4_INCONSISTENT");
  if (o->kv_tile != 64 && o->kv_tile != 128) return fail(HIFA4_ERR_UNSUPPORTED, "kv_tile must be 64 or 128");
  if (o->max_rule != HIFA4_MAX_CEIL && o->max_rule != HIFA4_MAX_NEAREST16)
    return fail(HIFA4_ERR_SHAPE, "max_rule must be HIFA4_MAX_CEIL or HIFA4_MAX_NEAREST16");
  if (o->phat_scale != HIFA4_PHAT_BLOCK32 && o->phat_scale != HIFA4_PHAT_TILE)
    return fail(HIFA4_ERR_SHAPE, "phat_scale must be HIFA4_PHAT_BLOCK32 or HIFA4_PHAT_TILE");
  if (o->phat_rule != HIFA4_PHAT_EXP16 && o->phat_rule != HIFA4_PHAT_DIRECT)
    return fail(HIFA4_ERR_SHAPE, "phat_rule must be HIFA4_PHAT_EXP16 or HIFA4_PHAT_DIRECT");
  if (o->phat_rule == HIFA4_PHAT_DIRECT && o->phat_scale != HIFA4_PHAT_BLOCK32)
    return fail(HIFA4_ERR_UNSUPPORTED, "HIFA4_PHAT_DIRECT takes one scale per 32-key block (HIFA4_PHAT_BLOCK32)");
  if ((o->phat_rule != HIFA4_PHAT_EXP16 || o->phat_scale != HIFA4_PHAT_BLOCK32) &&
      (o->normalizer != HIFA4_P_REORDERED || o->max_rule != HIFA4_MAX_CEIL))
    return fail(HIFA4_ERR_UNSUPPORTED, "the P-hat variants run P-Reordered with HIFA4_MAX_CEIL");
  if (o->num_splits < 0 || o->num_splits > 256) return fail(HIFA4_ERR_SHAPE, "num_splits must be in [0, 256]");
  if (o->prefill_waves != 0 && o->prefill_waves != 4 && o->prefill_waves != 8)
    return fail(HIFA4_ERR_SHAPE, "prefill_waves must be 0, 4 or 8");
  if (o->prefill_waves == 4 && d->len_q > 1 &&
      (o->normalizer != HIFA4_P_REORDERED || o->max_rule != HIFA4_MAX_CEIL ||
       o->phat_rule != HIFA4_PHAT_EXP16 || o->phat_scale != HIFA4_PHAT_BLOCK32))
    return fail(HIFA4_ERR_UNSUPPORTED, "prefill_waves = 4 runs the method's P-Reordered rules only");
  if (o->causal && d->len_q > d->len_kv) return fail(HIFA4_ERR_SHAPE, "causal attention needs len_q <= len_kv");
  if (o->kv_capacity != 0 &&
      (o->kv_capacity < d->len_kv || round32(o->kv_capacity) * (d->head_dim / 2) >= (int64_t(1) << 31)))
    return fail(HIFA4_ERR_SHAPE, "kv_capacity must be 0 or at least len_kv, with kv_capacity * head_dim / 2 below 2^31");
  return HIFA4_OK;
}

int32_t resolve_splits(const hifa4_dims* d, const hifa4_attn_opts* o) {
  if (d->len_q != 1) return 1;
  const int64_t tiles = (d->len_kv + o->kv_tile - 1) / o->kv_tile;
  int64_t s = o->num_splits > 0 ? o->num_splits : auto_splits(d, o->kv_tile);
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(s, tiles));
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// true when every non-NULL pointer of the list is 16-byte aligned
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (((uintptr_t)p & 15) != 0) return false;
  return true;
}

}  // namespace

extern "C" {

const char* hifa4_status_string(hifa4_status status) {
  switch (status) {
    case HIFA4_OK: return "ok";
    case HIFA4_ERR_NULL: return "null pointer";
    case HIFA4_ERR_SHAPE: return "invalid shape or argument";
    case HIFA4_ERR_UNSUPPORTED: return "unsupported configuration";
    case HIFA4_ERR_WORKSPACE: return "workspace missing or too small";
    case HIFA4_ERR_HIP: return "HIP runtime error";
    case HIFA4_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
  }
  return "unknown status";
}

const char* hifa4_last_error(void) { return g_last_error.c_str(); }

hifa4_status hifa4_calibrate(const uint16_t* q_cal, const uint16_t* k_cal, int64_t n_tokens,
                             int32_t heads_q, int32_t heads_kv, int32_t head_dim, float alpha,
                             float gate_tau, float* s, float* inv_s, int32_t* gate_on) {
  if (!q_cal || !k_cal || !s || !inv_s || !gate_on) return fail(HIFA4_ERR_NULL, "calibrate: NULL argument");
  if (n_tokens < 1 || heads_q < 1 || heads_kv < 1 || head_dim < 1 || heads_q % heads_kv != 0)
    return fail(HIFA4_ERR_SHAPE, "calibrate: need n_tokens, heads, head_dim >= 1 and heads_q % heads_kv == 0");
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(HIFA4_ERR_SHAPE, "calibrate: alpha must be in [0, 1]");
  const int group = heads_q / heads_kv;
  const int64_t d = head_dim;
  std::vector<double> aq((size_t)heads_kv * d, 0.0), ak((size_t)heads_kv * d, 0.0);
  for (int g = 0; g < heads_kv; g++) {
    for (int64_t t = 0; t < n_tokens; t++) {
      for (int64_t j = 0; j < d; j++) {
        const double v = std::fabs((double)half_bits_to_float(k_cal[((int64_t)g * n_tokens + t) * d + j]));
        double& dst = ak[(size_t)g * d + j];
        dst = std::max(dst, v);
      }
    }
    for (int hh = 0; hh < group; hh++) {
      const int h = g * group + hh;
      for (int64_t t = 0; t < n_tokens; t++) {
        for (int64_t j = 0; j < d; j++) {
          const double v = std::fabs((double)half_bits_to_float(q_cal[((int64_t)h * n_tokens + t) * d + j]));
          double& dst = aq[(size_t)g * d + j];
          dst = std::max(dst, v);
        }
      }
    }
  }
  std::vector<double> sorted = ak;
  std::sort(sorted.begin(), sorted.end());
  const size_t n = sorted.size();
  const double median = (n % 2) ? sorted[n / 2] : (sorted[n / 2 - 1] + sorted[n / 2]) / 2.0;
  const double kmax = sorted.back();
  const double rho = median > 0 ? kmax / median : INFINITY;
  const bool on = rho >= (double)gate_tau;
  *gate_on = on ? 1 : 0;
  for (size_t i = 0; i < n; i++) {
    double sv = 1.0;
    if (on && ak[i] > 0 && aq[i] > 0) sv = std::pow(ak[i], (double)alpha) / std::pow(aq[i], 1.0 - (double)alpha);
    const float s32 = (float)sv;
    s[i] = s32;
    inv_s[i] = (float)(1.0 / (double)s32);
  }
  return ok();
}

hifa4_status hifa4_quantize_qkv_rule(const hifa4_dims* dims, int32_t scale_rule, const void* q, const void* k,
                                     const void* v, const float* s, const float* inv_s, void* q_codes,
                                     void* q_scales, void* k_codes, void* k_scales, void* v_codes,
                                     void* v_scales, void* hip_stream) {
  hifa4_status st = check_dims(dims);
  if (st != HIFA4_OK) return st;
  if (scale_rule != HIFA4_SCALE_NO_CLIP && scale_rule != HIFA4_SCALE_FLOOR)
    return fail(HIFA4_ERR_SHAPE, "quantize: scale_rule must be HIFA4_SCALE_NO_CLIP or HIFA4_SCALE_FLOOR");
  if ((s == nullptr) != (inv_s == nullptr)) return fail(HIFA4_ERR_NULL, "quantize: pass both s and inv_s or neither");
  if (q && (!q_codes || !q_scales)) return fail(HIFA4_ERR_NULL, "quantize: q outputs are NULL");
  if (k && (!k_codes || !k_scales)) return fail(HIFA4_ERR_NULL, "quantize: k outputs are NULL");
  if (v && (!v_codes || !v_scales)) return fail(HIFA4_ERR_NULL, "quantize: v outputs are NULL");
  if (!aligned16({q, k, v, s, inv_s, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales}))
    return fail(HIFA4_ERR_ALIGNMENT, "quantize: device pointers must be 16-byte aligned");
  hipStream_t stream = (hipStream_t)hip_stream;
  const int group = dims->heads_q / dims->heads_kv;
  if (q) {
    hifa4::QuantRowsArgs a{(const uint16_t*)q, s, (int64_t)dims->batch * dims->heads_q * dims->len_q,
                           dims->len_q, round32(dims->len_q), dims->heads_q, group, dims->head_dim, 0,
                           (uint8_t*)q_codes, (uint8_t*)q_scales, scale_rule};
    hipError_t e = hifa4::launch_quantize_rows(a, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize q: ") + hipGetErrorString(e));
  }
  const hifa4::QuantRowsArgs ka{(const uint16_t*)k, inv_s, (int64_t)dims->batch * dims->heads_kv * dims->len_kv,
                                dims->len_kv, round32(dims->len_kv), dims->heads_kv, 1, dims->head_dim, 1,
                                (uint8_t*)k_codes, (uint8_t*)k_scales, scale_rule};
  const hifa4::QuantVtArgs va{(const uint16_t*)v, (int64_t)dims->batch * dims->heads_kv, dims->len_kv,
                              round32(dims->len_kv), dims->head_dim, (uint8_t*)v_codes, (uint8_t*)v_scales,
                              scale_rule};
  if (k && v) {
    hipError_t e = hifa4::launch_quantize_kv(ka, va, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize k, v: ") + hipGetErrorString(e));
    return ok();
  }
  if (k) {
    hipError_t e = hifa4::launch_quantize_rows(ka, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize k: ") + hipGetErrorString(e));
  }
  if (v) {
    hipError_t e = hifa4::launch_quantize_vt(va, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize v: ") + hipGetErrorString(e));
  }
  return ok();
}

hifa4_status hifa4_quantize_qkv(const hifa4_dims* dims, const void* q, const void* k, const void* v,
                                const float* s, const float* inv_s, void* q_codes, void* q_scales,
                                void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                                void* hip_stream) {
  return hifa4_quantize_qkv_rule(dims, HIFA4_SCALE_NO_CLIP, q, k, v, s, inv_s, q_codes, q_scales, k_codes,
                                 k_scales, v_codes, v_scales, hip_stream);
}

hifa4_status hifa4_quantize_qkv_rope(const hifa4_dims* dims, const void* q, const void* k, const void* v,
                                     const float* s, const float* inv_s, const float* rope_cos,
                                     const float* rope_sin, int64_t rope_positions, void* q_codes,
                                     void* q_scales, void* k_codes, void* k_scales, void* v_codes,
                                     void* v_scales, void* hip_stream) {
  hifa4_status st = check_dims(dims);
  if (st != HIFA4_OK) return st;
  if ((s == nullptr) != (inv_s == nullptr)) return fail(HIFA4_ERR_NULL, "quantize: pass both s and inv_s or neither");
  if ((q || k) && (!rope_cos || !rope_sin)) return fail(HIFA4_ERR_NULL, "quantize: RoPE tables are NULL");
  if (q && (!q_codes || !q_scales)) return fail(HIFA4_ERR_NULL, "quantize: q outputs are NULL");
  if (k && (!k_codes || !k_scales)) return fail(HIFA4_ERR_NULL, "quantize: k outputs are NULL");
  if (v && (!v_codes || !v_scales)) return fail(HIFA4_ERR_NULL, "quantize: v outputs are NULL");
  if (q && dims->len_q > dims->len_kv)
    return fail(HIFA4_ERR_SHAPE, "quantize: RoPE positions need len_q <= len_kv (query r sits at r + len_kv - len_q)");
  if ((q || k) && rope_positions < dims->len_kv)
    return fail(HIFA4_ERR_SHAPE, "quantize: the RoPE tables need at least len_kv positions");
  if (!aligned16({q, k, v, s, inv_s, rope_cos, rope_sin, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales}))
    return fail(HIFA4_ERR_ALIGNMENT, "quantize: device pointers must be 16-byte aligned");
  hipStream_t stream = (hipStream_t)hip_stream;
  const int group = dims->heads_q / dims->heads_kv;
  const hifa4::QuantRopeArgs qa{(const uint16_t*)q, s, rope_cos, rope_sin, dims->batch, dims->len_q,
                                round32(dims->len_q), dims->len_kv - dims->len_q, dims->heads_q, group,
                                dims->heads_kv, dims->head_dim, 0, (uint8_t*)q_codes, (uint8_t*)q_scales};
  const hifa4::QuantRopeArgs ka{(const uint16_t*)k, inv_s, rope_cos, rope_sin, dims->batch, dims->len_kv,
                                round32(dims->len_kv), 0, dims->heads_kv, 1, dims->heads_kv, dims->head_dim, 1,
                                (uint8_t*)k_codes, (uint8_t*)k_scales};
  const hifa4::QuantVtArgs va{(const uint16_t*)v, (int64_t)dims->batch * dims->heads_kv, dims->len_kv,
                              round32(dims->len_kv), dims->head_dim, (uint8_t*)v_codes, (uint8_t*)v_scales};
  if (q && k && v) {  // all three in one launch
    hipError_t e = hifa4::launch_quantize_qkv_rope(qa, ka, va, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize q, k, v: ") + hipGetErrorString(e));
    return ok();
  }
  if (q) {
    hipError_t e = hifa4::launch_quantize_rope(qa, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize q: ") + hipGetErrorString(e));
  }
  if (k) {
    hipError_t e = hifa4::launch_quantize_rope(ka, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize k: ") + hipGetErrorString(e));
  }
  if (v) {
    hipError_t e = hifa4::launch_quantize_vt(va, stream);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("quantize v: ") + hipGetErrorString(e));
  }
  return ok();
}

hifa4_status hifa4_cache_append(const hifa4_dims* dims, int64_t kv_capacity, const void* k_new, const void* v_new,
                                const float* inv_s, const float* rope_cos, const float* rope_sin,
                                int64_t rope_positions, void* k_codes, void* k_scales, void* v_codes,
                                void* v_scales, void* v_stage, void* hip_stream) {
  if (dims == nullptr) return fail(HIFA4_ERR_NULL, "dims is NULL");
  if (dims->batch < 1 || dims->heads_kv < 1 || dims->len_q < 1 || dims->len_kv < 0)
    return fail(HIFA4_ERR_SHAPE, "append: need batch, heads_kv, len_q (new keys) >= 1 and len_kv >= 0");
  if (dims->head_dim != 64 && dims->head_dim != 128 && dims->head_dim != 256)
    return fail(HIFA4_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (dims->len_kv + dims->len_q > kv_capacity || round32(kv_capacity) * (dims->head_dim / 2) >= (int64_t(1) << 31))
    return fail(HIFA4_ERR_SHAPE, "append: len_kv + len_q must not exceed kv_capacity (kv_capacity * head_dim / 2 < 2^31)");
  if (!k_new || !v_new || !k_codes || !k_scales || !v_codes || !v_scales || !v_stage)
    return fail(HIFA4_ERR_NULL, "append: a tensor pointer is NULL");
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return fail(HIFA4_ERR_NULL, "append: pass both RoPE tables or neither");
  if (rope_cos && rope_positions < dims->len_kv + dims->len_q)
    return fail(HIFA4_ERR_SHAPE, "append: the RoPE tables need len_kv + len_q positions");
  if (!aligned16({k_new, v_new, inv_s, rope_cos, rope_sin, k_codes, k_scales, v_codes, v_scales, v_stage}))
    return fail(HIFA4_ERR_ALIGNMENT, "append: device pointers must be 16-byte aligned");
  hifa4::CacheAppendArgs a{};
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.inv_s = inv_s;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.bh = (int64_t)dims->batch * dims->heads_kv;
  a.heads_kv = dims->heads_kv;
  a.d = dims->head_dim;
  a.len0 = dims->len_kv;
  a.n = dims->len_q;
  a.rows = kv_capacity;
  a.rows32 = round32(kv_capacity);
  a.k_codes = (uint8_t*)k_codes;
  a.k_scales = (uint8_t*)k_scales;
  a.v_codes = (uint8_t*)v_codes;
  a.v_scales = (uint8_t*)v_scales;
  a.v_stage = (uint16_t*)v_stage;
  hipError_t e = hifa4::launch_cache_append(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("append: ") + hipGetErrorString(e));
  return ok();
}

int32_t hifa4_decode_num_splits(const hifa4_dims* dims, const hifa4_attn_opts* opts) {
  if (check_dims(dims) != HIFA4_OK || check_opts(dims, opts) != HIFA4_OK) return 0;
  return resolve_splits(dims, opts);
}

size_t hifa4_attention_workspace_bytes(const hifa4_dims* dims, const hifa4_attn_opts* opts) {
  if (check_dims(dims) != HIFA4_OK || check_opts(dims, opts) != HIFA4_OK) return 0;
  if (dims->len_q != 1) return 0;
  const int64_t parts = (int64_t)dims->batch * dims->heads_q * resolve_splits(dims, opts);
  return align256((size_t)parts * dims->head_dim * 2) + align256((size_t)parts * 2 * 2);
}

}  // extern "C"

namespace {

// Shared tail of both attention entry points: a holds the tensor pointers; fills the sizes and
// launches the prefill or split-KV decode kernel.
hifa4_status attention_launch(hifa4::AttnArgs& a, const hifa4_dims* dims, const hifa4_attn_opts* opts,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  a.batch = dims->batch;
  a.heads_q = dims->heads_q;
  a.heads_kv = dims->heads_kv;
  a.d = dims->head_dim;
  a.len_q = dims->len_q;
  a.len_kv = dims->len_kv;
  a.len_kv32 = round32(dims->len_kv);
  a.kv_rows = opts->kv_capacity ? opts->kv_capacity : dims->len_kv;
  a.kv_rows32 = round32(a.kv_rows);
  a.kv_tile = opts->kv_tile;
  a.n_tiles = (int32_t)((dims->len_kv + opts->kv_tile - 1) / opts->kv_tile);
  a.causal = opts->causal;
  a.normalizer = opts->normalizer;
  a.max_rule = opts->max_rule;
  a.phat = opts->phat_rule == HIFA4_PHAT_DIRECT ? 2 : (opts->phat_scale == HIFA4_PHAT_TILE ? 1 : 0);
  a.wg_waves = opts->prefill_waves;
  a.c_log2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
  hipStream_t stream = (hipStream_t)hip_stream;
  hipError_t e;
  if (a.max_rule == HIFA4_MAX_NEAREST16) {
    if (dims->len_q == 1)
      return fail(HIFA4_ERR_UNSUPPORTED, "attention: HIFA4_MAX_NEAREST16 is prefill-only (the split merge assumes integer maxima)");
    if (a.stats || a.normalizer != HIFA4_P_REORDERED)
      return fail(HIFA4_ERR_UNSUPPORTED, "attention: HIFA4_MAX_NEAREST16 runs P-Reordered without tile statistics");
  }
  if (a.stats && a.phat != 0)
    return fail(HIFA4_ERR_UNSUPPORTED, "attention: the P-hat variants run without tile statistics");
  if (a.stats && a.wg_waves == 4 && dims->len_q > 1)
    return fail(HIFA4_ERR_UNSUPPORTED, "attention: prefill_waves = 4 runs without tile statistics");
  if (dims->len_q == 1) {
    if (a.stats) return fail(HIFA4_ERR_UNSUPPORTED, "attention: tile_stats is prefill-only");
    const size_t need = hifa4_attention_workspace_bytes(dims, opts);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(HIFA4_ERR_WORKSPACE, "attention: decode needs " + std::to_string(need) + " workspace bytes");
    a.num_splits = resolve_splits(dims, opts);
    a.tiles_per_split = (a.n_tiles + a.num_splits - 1) / a.num_splits;
    const int64_t parts = (int64_t)dims->batch * dims->heads_q * a.num_splits;
    a.part_o = (uint16_t*)workspace;
    a.part_ml = (uint16_t*)((char*)workspace + align256((size_t)parts * dims->head_dim * 2));
    e = hifa4::launch_attn_decode(a, stream);
  } else {
    a.num_splits = 1;
    a.tiles_per_split = a.n_tiles;
    e = hifa4::launch_attn_prefill(a, stream);
  }
  if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

hifa4_status hifa4_attention_fwd(const hifa4_dims* dims, const hifa4_attn_opts* opts,
                                 const void* q_codes, const void* q_scales, const void* k_codes,
                                 const void* k_scales, const void* v_codes, const void* v_scales,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 float* tile_stats, void* hip_stream) {
  hifa4_status st = check_dims(dims);
  if (st != HIFA4_OK) return st;
  st = check_opts(dims, opts);
  if (st != HIFA4_OK) return st;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales || !out)
    return fail(HIFA4_ERR_NULL, "attention: a tensor pointer is NULL");
  if (!aligned16({q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, out, workspace, tile_stats}))
    return fail(HIFA4_ERR_ALIGNMENT, "attention: device pointers must be 16-byte aligned");
  hifa4::AttnArgs a{};
  a.q_codes = (const uint8_t*)q_codes;
  a.q_scales = (const uint8_t*)q_scales;
  a.k_codes = (const uint8_t*)k_codes;
  a.k_scales = (const uint8_t*)k_scales;
  a.v_codes = (const uint8_t*)v_codes;
  a.v_scales = (const uint8_t*)v_scales;
  a.out = (uint16_t*)out;
  a.stats = tile_stats;
  return attention_launch(a, dims, opts, workspace, workspace_bytes, hip_stream);
}

hifa4_status hifa4_attention_fwd_q16(const hifa4_dims* dims, const hifa4_attn_opts* opts, const void* q,
                                     const float* s, const float* rope_cos, const float* rope_sin,
                                     int64_t rope_positions, const void* k_codes, const void* k_scales,
                                     const void* v_codes, const void* v_scales, void* out, void* workspace,
                                     size_t workspace_bytes, float* tile_stats, void* hip_stream) {
  hifa4_status st = check_dims(dims);
  if (st != HIFA4_OK) return st;
  st = check_opts(dims, opts);
  if (st != HIFA4_OK) return st;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !out)
    return fail(HIFA4_ERR_NULL, "attention: a tensor pointer is NULL");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(HIFA4_ERR_NULL, "attention: pass both RoPE tables or neither");
  if (rope_cos && dims->len_q != 1)
    return fail(HIFA4_ERR_UNSUPPORTED, "attention: in-kernel RoPE is for decode (len_q == 1); for prefill use "
                                       "hifa4_quantize_qkv_rope, then hifa4_attention_fwd");
  if (rope_cos && rope_positions < dims->len_kv)
    return fail(HIFA4_ERR_SHAPE, "attention: the RoPE tables need at least len_kv positions");
  if (!aligned16({q, s, rope_cos, rope_sin, k_codes, k_scales, v_codes, v_scales, out, workspace, tile_stats}))
    return fail(HIFA4_ERR_ALIGNMENT, "attention: device pointers must be 16-byte aligned");
  hifa4::AttnArgs a{};
  a.q_fp16 = (const uint16_t*)q;
  a.q_smooth = s;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.k_codes = (const uint8_t*)k_codes;
  a.k_scales = (const uint8_t*)k_scales;
  a.v_codes = (const uint8_t*)v_codes;
  a.v_scales = (const uint8_t*)v_scales;
  a.out = (uint16_t*)out;
  a.stats = tile_stats;
  return attention_launch(a, dims, opts, workspace, workspace_bytes, hip_stream);
}

hifa4_status hifa4_attention_fwd_q16_noalloc(const hifa4_dims* dims, const hifa4_attn_opts* opts, const void* q,
                                             const float* s, const float* rope_cos, const float* rope_sin,
                                             int64_t rope_positions, const void* k_codes, const void* k_scales,
                                             const void* v_codes, const void* v_scales, void* out,
                                             float* tile_stats, void* hip_stream) {
  hifa4_status st = check_dims(dims);
  if (st != HIFA4_OK) return st;
  st = check_opts(dims, opts);
  if (st != HIFA4_OK) return st;
  const size_t need = hifa4_attention_workspace_bytes(dims, opts);
  if (need > hifa4::kDecodeScratchBytes)
    return fail(HIFA4_ERR_WORKSPACE, "attention (no-alloc): decode partials need " + std::to_string(need) +
                                         " bytes, beyond the fixed scratch of " +
                                         std::to_string(hifa4::kDecodeScratchBytes) + " bytes");
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = hifa4::decode_scratch(&ws);
    if (e != hipSuccess) return fail(HIFA4_ERR_HIP, std::string("attention (no-alloc): scratch lookup: ") + hipGetErrorString(e));
  }
  return hifa4_attention_fwd_q16(dims, opts, q, s, rope_cos, rope_sin, rope_positions, k_codes, k_scales, v_codes,
                                 v_scales, out, ws, need, tile_stats, hip_stream);
}

}  // extern "C"
