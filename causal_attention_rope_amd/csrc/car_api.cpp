// C-ABI entry points (include/car.h): argument validation, RoPE frequency
// table, workspace sizing and dispatch to the HIP kernels.  Every check runs
// before any launch; a failed check returns its status with nothing
// enqueued.  The library keeps no state between calls.
#include <math.h>
#include <stdint.h>

#include "car.h"
#include "launch.hpp"

using namespace car;

namespace {

// Events recorded around the main kernel (both or neither).
TimedLaunch timed(hipEvent_t start, hipEvent_t stop) {
  if (start == nullptr || stop == nullptr) return TimedLaunch{nullptr, nullptr};
  return TimedLaunch{start, stop};
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(car_dtype dt) { return dt == CAR_DTYPE_F32 || dt == CAR_DTYPE_BF16; }
bool head_dim_ok(int D) { return D == 64 || D == 128; }
size_t elem_bytes(car_dtype dt) { return dt == CAR_DTYPE_F32 ? 4 : 2; }
bool positive_finite(float x) { return isfinite(x) && x > 0.f; }

car_status from_hip(hipError_t e) { return e == hipSuccess ? CAR_OK : CAR_ERR_HIP; }

// theta^(-2i/D) / (2 pi) (revolutions per position) for i < D/2, in double,
// split into float hi + lo.
bool pairing_ok(car_rope_pairing p) { return p == CAR_ROPE_ADJACENT || p == CAR_ROPE_HALF; }

RopeFreq make_freq(int D, float theta, car_rope_pairing pairing) {
  RopeFreq f{};
  f.half = pairing == CAR_ROPE_HALF;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < D / 2; ++i) {
    const double x = pow((double)theta, -2.0 * i / (double)D) / two_pi;
    f.hi[i] = (float)x;
    f.lo[i] = (float)(x - (double)f.hi[i]);
  }
  return f;
}

// Validates a cache description; fills the device view and its capacity.
car_status check_cache(const car_kv_cache* c, CacheArgs* out, int64_t* capacity) {
  if (c == nullptr || c->k == nullptr || c->v == nullptr) return CAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(c->k) || !aligned16(c->v)) return CAR_ERR_INVALID_ARGUMENT;
  if (c->format != CAR_CACHE_NATIVE && c->format != CAR_CACHE_INT8) return CAR_ERR_UNSUPPORTED;
  CacheArgs a{};
  a.k = c->k;
  a.v = c->v;
  a.table = c->block_table;
  if (c->format == CAR_CACHE_INT8) {
    if (c->k_scale == nullptr || c->v_scale == nullptr || !aligned16(c->k_scale) ||
        !aligned16(c->v_scale))
      return CAR_ERR_INVALID_ARGUMENT;
    a.k_scale = c->k_scale;
    a.v_scale = c->v_scale;
  }
  if (c->block_table != nullptr) {
    if (c->block_size != 16) return CAR_ERR_UNSUPPORTED;
    if (c->num_blocks <= 0 || c->max_blocks_per_seq <= 0) return CAR_ERR_INVALID_ARGUMENT;
    if ((int64_t)c->max_blocks_per_seq * 16 > INT32_MAX) return CAR_ERR_INVALID_ARGUMENT;
    a.num_blocks = c->num_blocks;
    a.mbps = c->max_blocks_per_seq;
    *capacity = (int64_t)c->max_blocks_per_seq * 16;
  } else {
    if (c->max_seq <= 0) return CAR_ERR_INVALID_ARGUMENT;
    a.max_seq = c->max_seq;
    *capacity = c->max_seq;
  }
  *out = a;
  return CAR_OK;
}

int64_t prefill_ws_bytes(car_dtype dt, int B, int Hkv, int S, int D) {
  return (int64_t)B * Hkv * S * D * (int64_t)elem_bytes(dt);
}

// bf16 into a contiguous native cache: prompts at consecutive slots keep
// their rotated keys in the cache only, and the attention reads them there
// (then no workspace is needed for prompts that fit the cache).
bool keys_go_to_cache(car_dtype dt, const car_kv_cache* c) {
  return dt == CAR_DTYPE_BF16 && c != nullptr && c->block_table == nullptr &&
         c->format == CAR_CACHE_NATIVE;
}

int decode_nsplit(int max_seq_len) { return (max_seq_len + DECODE_SPLIT - 1) / DECODE_SPLIT; }

bool is_int8(const car_kv_cache* c) { return c != nullptr && c->format == CAR_CACHE_INT8; }

// A chunk over an INT8 cache: bytes of one dequantized copy (K or V) of
// [B, Hkv, max_seq_len, D] in the call's dtype, rounded up to 256 bytes.
int64_t chunk_dequant_half_bytes(car_dtype dt, int B, int Hkv, int D, int max_seq_len) {
  const int64_t n = (int64_t)B * Hkv * max_seq_len * D * (int64_t)elem_bytes(dt);
  return (n + 255) / 256 * 256;
}

}  // namespace

extern "C" {

const char* car_status_string(car_status s) {
  switch (s) {
    case CAR_OK: return "CAR_OK";
    case CAR_ERR_INVALID_ARGUMENT: return "CAR_ERR_INVALID_ARGUMENT: invalid argument";
    case CAR_ERR_UNSUPPORTED: return "CAR_ERR_UNSUPPORTED: configuration not built";
    case CAR_ERR_WORKSPACE: return "CAR_ERR_WORKSPACE: workspace missing or too small";
    case CAR_ERR_HIP: return "CAR_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown car_status";
}

car_status car_rope_apply(void* x, car_dtype dtype, int B, int H, int S, int D,
                          const int32_t* positions, float theta, car_rope_pairing pairing,
                          hipStream_t stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || !pairing_ok(pairing)) return CAR_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || S < 0 || !positive_finite(theta)) return CAR_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * H * S == 0) return CAR_OK;
  if (x == nullptr || positions == nullptr || !aligned16(x)) return CAR_ERR_INVALID_ARGUMENT;
  return from_hip(launch_rope_apply(dtype == CAR_DTYPE_F32 ? F32 : BF16, D, x, B, H, S,
                                    positions, make_freq(D, theta, pairing), stream));
}

car_status car_kv_cache_append(const car_kv_cache* cache, car_dtype dtype, const void* k,
                               const void* v, int B, int Hkv, int S, int D,
                               const int32_t* positions, hipStream_t stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return CAR_ERR_UNSUPPORTED;
  if (B < 0 || Hkv < 0 || S < 0) return CAR_ERR_INVALID_ARGUMENT;
  if (cache != nullptr && cache->block_table != nullptr && cache->block_size != 16)
    return CAR_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * S == 0) return CAR_OK;
  if (k == nullptr || v == nullptr || positions == nullptr || !aligned16(k) || !aligned16(v))
    return CAR_ERR_INVALID_ARGUMENT;
  CacheArgs c;
  int64_t cap = 0;
  const car_status cs = check_cache(cache, &c, &cap);
  if (cs != CAR_OK) return cs;
  return from_hip(launch_kv_append(dtype == CAR_DTYPE_F32 ? F32 : BF16, D,
                                   cache->block_table != nullptr, is_int8(cache), c, k, v, B, Hkv,
                                   S, positions, stream));
}

car_status car_kv_int8_calibrate(const void* k, const void* v, car_dtype dtype, int B, int Hkv,
                                 int S, int D, const int32_t* positions, float theta,
                                 car_rope_pairing pairing, float* k_scale, float* v_scale,
                                 hipStream_t stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || !pairing_ok(pairing)) return CAR_ERR_UNSUPPORTED;
  if (B < 0 || Hkv < 0 || S < 0 || !positive_finite(theta)) return CAR_ERR_INVALID_ARGUMENT;
  if (Hkv == 0) return CAR_OK;
  if (k_scale == nullptr || v_scale == nullptr || !aligned16(k_scale) || !aligned16(v_scale))
    return CAR_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * S > 0) {
    if (k == nullptr || v == nullptr || positions == nullptr || !aligned16(k) || !aligned16(v))
      return CAR_ERR_INVALID_ARGUMENT;
  }
  if (Hkv > 65535) return CAR_ERR_UNSUPPORTED;  // one grid row per KV head
  return from_hip(launch_int8_calibrate(dtype == CAR_DTYPE_F32 ? F32 : BF16, D, k, v, B, Hkv, S,
                                        positions, make_freq(D, theta, pairing), k_scale,
                                        v_scale, stream));
}

size_t car_attn_prefill_workspace_bytes(car_dtype dtype, int B, int Hkv, int S, int D,
                                        const car_kv_cache* cache) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || B < 0 || Hkv < 0 || S < 0) return 0;
  if (keys_go_to_cache(dtype, cache) && S <= cache->max_seq) return 0;
  return (size_t)prefill_ws_bytes(dtype, B, Hkv, S, D);
}

car_status car_attn_prefill_timed(const void* q, const void* k, const void* v, void* out,
                                  car_dtype dtype, int B, int Hq, int Hkv, int S, int D,
                                  const int32_t* positions, const int32_t* seq_lens,
                                  float theta,
                                  car_rope_pairing pairing, float scale,
                                  const car_kv_cache* cache, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream,
                                  hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || !pairing_ok(pairing)) return CAR_ERR_UNSUPPORTED;
  if (cache != nullptr && cache->block_table != nullptr && cache->block_size != 16)
    return CAR_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 0 || Hkv < 0 || S < 0) return CAR_ERR_INVALID_ARGUMENT;
  if (!positive_finite(theta) || !positive_finite(scale)) return CAR_ERR_INVALID_ARGUMENT;
  if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return CAR_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * Hq * S == 0) return CAR_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || positions == nullptr)
    return CAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return CAR_ERR_INVALID_ARGUMENT;
  CacheArgs c{};
  int64_t cap = 0;
  if (cache != nullptr) {
    const car_status cs = check_cache(cache, &c, &cap);
    if (cs != CAR_OK) return cs;
  }
  // launch grids (fp32: Hq and B in grid y and z; bf16: query tiles x B x Hq
  // in x, at least 64 rows per tile) and 32-bit byte offsets within one
  // head's keys (the prompt's, or a contiguous cache's)
  if (B > 65535 || Hq > 65535 || (int64_t)B * Hq * ((S + 63) / 64) > INT32_MAX ||
      (S > cap ? (int64_t)S : cap) * D * 4 > (int64_t)UINT32_MAX)
    return CAR_ERR_UNSUPPORTED;
  // A workspace of the full size holds the rotated keys of every prompt;
  // without one (allowed when the keys go to a contiguous native cache) the
  // attention reads every prompt's keys back from the cache.
  const int64_t full = prefill_ws_bytes(dtype, B, Hkv, S, D);
  const bool keys_in_cache = keys_go_to_cache(dtype, cache);
  void* k_rot = workspace != nullptr && (int64_t)workspace_bytes >= full ? workspace : nullptr;
  if (k_rot == nullptr && (!keys_in_cache || S > cap)) return CAR_ERR_WORKSPACE;
  if (k_rot != nullptr && !aligned16(k_rot)) return CAR_ERR_WORKSPACE;

  const Dtype dt = dtype == CAR_DTYPE_F32 ? F32 : BF16;
  const RopeFreq fr = make_freq(D, theta, pairing);
  const bool paged = cache != nullptr && cache->block_table != nullptr;
  const bool values_by_attention =
      keys_in_cache && prefill_attention_stores_values(dt, B, Hq, S, &c);
  hipError_t e = launch_prefill_prep(dt, D, paged, is_int8(cache),
                                     cache != nullptr ? &c : nullptr, k, v, k_rot, B, Hkv,
                                     S, positions, seq_lens, fr, keys_in_cache,
                                     !values_by_attention, out, Hq / Hkv, stream);
  if (e != hipSuccess) return CAR_ERR_HIP;
  return from_hip(launch_prefill_attention(dt, D, q, k_rot, v, out, B, Hq, Hkv, S,
                                           positions, seq_lens, fr, scale,
                                           keys_in_cache ? &c : nullptr, stream,
                                           timed(kernel_start, kernel_stop)));
}

car_status car_attn_prefill(const void* q, const void* k, const void* v, void* out,
                            car_dtype dtype, int B, int Hq, int Hkv, int S, int D,
                            const int32_t* positions, const int32_t* seq_lens, float theta,
                            car_rope_pairing pairing, float scale, const car_kv_cache* cache,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return car_attn_prefill_timed(q, k, v, out, dtype, B, Hq, Hkv, S, D, positions, seq_lens,
                                theta, pairing, scale, cache, workspace, workspace_bytes, stream,
                                nullptr, nullptr);
}

size_t car_attn_prefill_cached_workspace_bytes(car_dtype dtype, int B, int Hkv, int D,
                                               int max_seq_len, const car_kv_cache* cache) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || B < 0 || Hkv < 0 || max_seq_len < 0) return 0;
  if (!is_int8(cache)) return 0;
  return 2 * (size_t)chunk_dequant_half_bytes(dtype, B, Hkv, D, max_seq_len);
}

car_status car_attn_prefill_cached_timed(const void* q, const void* k, const void* v,
                                         void* out, car_dtype dtype, int B, int Hq, int Hkv,
                                         int S, int D, const int32_t* seq_lens,
                                         const int32_t* chunk_lens, int max_seq_len,
                                         float theta, car_rope_pairing pairing, float scale,
                                         const car_kv_cache* cache, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream,
                                         hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || !pairing_ok(pairing)) return CAR_ERR_UNSUPPORTED;
  if (cache != nullptr && cache->block_table != nullptr && cache->block_size != 16)
    return CAR_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 0 || Hkv < 0 || S < 0) return CAR_ERR_INVALID_ARGUMENT;
  if (!positive_finite(theta) || !positive_finite(scale)) return CAR_ERR_INVALID_ARGUMENT;
  if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return CAR_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * Hq * S == 0) return CAR_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || seq_lens == nullptr)
    return CAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return CAR_ERR_INVALID_ARGUMENT;
  CacheArgs c;
  int64_t cap = 0;
  const car_status cs = check_cache(cache, &c, &cap);
  if (cs != CAR_OK) return cs;
  // every sequence's chunk fits: S tokens, or up to S with chunk_lens
  if (max_seq_len < (chunk_lens == nullptr ? S : 1) || max_seq_len > cap)
    return CAR_ERR_INVALID_ARGUMENT;
  // launch grids (fp32: B and Hq in grid y, z; bf16: query tiles of at least
  // 64 rows x B x Hq in x) and 32-bit byte offsets within one head of a
  // contiguous cache
  if (B > 65535 || Hq > 65535 || (int64_t)B * Hq * ((S + 63) / 64) > INT32_MAX ||
      cap * D * 4 > (int64_t)UINT32_MAX)
    return CAR_ERR_UNSUPPORTED;
  const bool i8 = is_int8(cache);
  if (i8) {
    const size_t need = car_attn_prefill_cached_workspace_bytes(dtype, B, Hkv, D, max_seq_len,
                                                                cache);
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
      return CAR_ERR_WORKSPACE;
  }

  const Dtype dt = dtype == CAR_DTYPE_F32 ? F32 : BF16;
  const RopeFreq fr = make_freq(D, theta, pairing);
  const bool paged = cache->block_table != nullptr;
  hipError_t e = launch_chunk_prep(dt, D, paged, i8, c, k, v, B, Hkv, S, seq_lens, chunk_lens,
                                   fr, stream);
  if (e != hipSuccess) return CAR_ERR_HIP;
  if (!i8)
    return from_hip(launch_prefill_cached(dt, D, paged, q, out, B, Hq, Hkv, S, c, seq_lens,
                                          chunk_lens, fr, scale, stream,
                                          timed(kernel_start, kernel_stop)));
  // INT8: the rows the chunk attends to, copied into the workspace and read
  // by the same attention kernel as a contiguous cache of max_seq_len slots:
  // dequantized values for fp32; for bf16 the codes, with the scales passed
  // on for the kernel to apply
  CacheArgs dq{};
  dq.k = workspace;
  dq.v = static_cast<char*>(workspace) + chunk_dequant_half_bytes(dtype, B, Hkv, D, max_seq_len);
  dq.max_seq = max_seq_len;
  if (dt == BF16) {
    dq.k_scale = c.k_scale;
    dq.v_scale = c.v_scale;
  }
  e = launch_int8_dequant(dt, D, paged, c, dq.k, dq.v, B, Hkv, S, max_seq_len, seq_lens,
                          chunk_lens, stream);
  if (e != hipSuccess) return CAR_ERR_HIP;
  return from_hip(launch_prefill_cached(dt, D, false, q, out, B, Hq, Hkv, S, dq, seq_lens,
                                        chunk_lens, fr, scale, stream,
                                        timed(kernel_start, kernel_stop)));
}

car_status car_attn_prefill_cached(const void* q, const void* k, const void* v, void* out,
                                   car_dtype dtype, int B, int Hq, int Hkv, int S, int D,
                                   const int32_t* seq_lens, const int32_t* chunk_lens,
                                   int max_seq_len, float theta, car_rope_pairing pairing,
                                   float scale, const car_kv_cache* cache, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return car_attn_prefill_cached_timed(q, k, v, out, dtype, B, Hq, Hkv, S, D, seq_lens,
                                       chunk_lens, max_seq_len, theta, pairing, scale, cache,
                                       workspace, workspace_bytes, stream, nullptr, nullptr);
}

size_t car_attn_decode_workspace_bytes(int B, int Hq, int D, int max_seq_len) {
  if (B < 0 || Hq < 0 || !head_dim_ok(D) || max_seq_len < 1) return 0;
  return (size_t)B * Hq * decode_nsplit(max_seq_len) * decode_partial_words(D) * sizeof(float);
}

car_status car_attn_decode_timed(const void* q, const void* k_new, const void* v_new,
                                 void* out, car_dtype dtype, int B, int Hq, int Hkv, int D,
                                 const int32_t* seq_lens, int max_seq_len, float theta,
                                 car_rope_pairing pairing, float scale,
                                 const car_kv_cache* cache, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  if (!dtype_ok(dtype) || !head_dim_ok(D) || !pairing_ok(pairing)) return CAR_ERR_UNSUPPORTED;
  if (cache != nullptr && cache->block_table != nullptr && cache->block_size != 16)
    return CAR_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 0 || Hkv < 0 || max_seq_len < 1) return CAR_ERR_INVALID_ARGUMENT;
  if (!positive_finite(theta) || !isfinite(scale)) return CAR_ERR_INVALID_ARGUMENT;
  if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return CAR_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * Hq == 0) return CAR_OK;
  const int group = Hq / Hkv;
  if (group != 1 && group != 2 && group != 4 && group != 8) return CAR_ERR_UNSUPPORTED;
  // launch grids: B * Hkv workgroups in x and one row per 256-token split in
  // y for the splits, B * Hq workgroups for the merge
  if ((int64_t)B * Hq > INT32_MAX || decode_nsplit(max_seq_len) > 65535) return CAR_ERR_UNSUPPORTED;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || out == nullptr ||
      seq_lens == nullptr)
    return CAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return CAR_ERR_INVALID_ARGUMENT;
  CacheArgs c;
  int64_t cap = 0;
  const car_status cs = check_cache(cache, &c, &cap);
  if (cs != CAR_OK) return cs;
  // a contiguous head's rows are addressed with 32-bit byte offsets
  if (cache->block_table == nullptr && cap * D * 4 > (int64_t)UINT32_MAX)
    return CAR_ERR_UNSUPPORTED;
  if (max_seq_len > cap) return CAR_ERR_INVALID_ARGUMENT;
  const size_t need = car_attn_decode_workspace_bytes(B, Hq, D, max_seq_len);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return CAR_ERR_WORKSPACE;
  const Dtype dt = dtype == CAR_DTYPE_F32 ? F32 : BF16;
  const bool paged = cache->block_table != nullptr;
  float* part = static_cast<float*>(workspace);
  const RopeFreq fr = make_freq(D, theta, pairing);
  const TimedLaunch tl = timed(kernel_start, kernel_stop);
  if (is_int8(cache))
    return from_hip(launch_decode_i8(dt, D, group, paged, q, k_new, v_new, out, B, Hq, Hkv,
                                     seq_lens, max_seq_len, c, part, fr, scale, stream, tl));
  return from_hip(launch_decode(dt, D, group, paged, q, k_new, v_new, out, B, Hq, Hkv, seq_lens,
                                max_seq_len, c, part, fr, scale, stream, tl));
}

car_status car_attn_decode(const void* q, const void* k_new, const void* v_new, void* out,
                           car_dtype dtype, int B, int Hq, int Hkv, int D,
                           const int32_t* seq_lens, int max_seq_len, float theta,
                           car_rope_pairing pairing, float scale, const car_kv_cache* cache,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return car_attn_decode_timed(q, k_new, v_new, out, dtype, B, Hq, Hkv, D, seq_lens,
                               max_seq_len, theta, pairing, scale, cache, workspace,
                               workspace_bytes, stream, nullptr, nullptr);
}

}  // extern "C"
