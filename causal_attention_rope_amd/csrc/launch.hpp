// Internal interface between the C-ABI shim (car_api.cpp) and the kernel
// translation units.  Plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace car {

// Per-pair RoPE frequency in revolutions per position, theta^(-2i/D) / (2 pi),
// as an unevaluated float sum hi + lo, and the pair layout: half == 0 pairs
// elements (2i, 2i+1), half == 1 pairs (i, i + D/2).
struct RopeFreq {
  float hi[64];
  float lo[64];
  int half;
};

// Device view of one layer's KV cache (see car_kv_cache in car.h).
struct CacheArgs {
  void* k;
  void* v;
  const int32_t* table;  // nullptr when contiguous
  int max_seq;           // contiguous: slots per sequence
  int num_blocks;        // paged: pool size in blocks
  int mbps;              // paged: row length of the block table
  const float* k_scale;  // INT8 cache: fp32 [Hkv, D]; value = code * scale
  const float* v_scale;
};

enum Dtype { F32 = 0, BF16 = 1 };

// Events recorded on the launch stream just before and just after the main
// kernel of a call (both null when the caller times nothing).
struct TimedLaunch {
  hipEvent_t start;
  hipEvent_t stop;
};

// Smallest number of tokens one decode workgroup handles (one split of the
// sequence; the launch may use a multiple of it).  It sizes the partials
// workspace.
constexpr int DECODE_SPLIT = 256;
// fp32 words per decode partial: running max, running sum, 2 pad, D values.
__host__ __device__ constexpr int decode_partial_words(int D) { return D + 4; }

// ---- rope_cache.hip -------------------------------------------------------
hipError_t launch_rope_apply(Dtype dt, int D, void* x, int B, int H, int S,
                             const int32_t* positions, const RopeFreq& fr, hipStream_t s);

// i8: the cache holds int8 codes (quantized with c.k_scale / c.v_scale).
hipError_t launch_kv_append(Dtype dt, int D, bool paged, bool i8, const CacheArgs& c,
                            const void* k, const void* v, int B, int Hkv, int S,
                            const int32_t* positions, hipStream_t s);

// Rotates k into k_rot (dense [B,Hkv,S,D]) and, if cache != nullptr, also
// stores the rotated keys and raw values into the cache (as int8 codes if i8).
// lens (nullable): tokens of each prompt; rows from there on are padding,
// neither rotated nor stored, and their rows of out ([B, Hkv*G, S, D]) are
// zeroed here.
// keys_in_cache (contiguous native cache only): sequences whose positions
// are consecutive cache slots (prompt_rows_in_cache) skip k_rot, and the
// attention must then be given the cache to read their keys from.
// store_v (only read with keys_in_cache): false when the attention kernel
// stores the values into the cache (prefill_attention_stores_values).
hipError_t launch_prefill_prep(Dtype dt, int D, bool paged, bool i8, const CacheArgs* cache,
                               const void* k, const void* v, void* k_rot, int B, int Hkv,
                               int S, const int32_t* positions, const int32_t* lens,
                               const RopeFreq& fr, bool keys_in_cache, bool store_v, void* out,
                               int G, hipStream_t s);

// Per-(KV head, channel) absmax / 127 of the rotated keys and of the values
// of a calibration batch, into k_scale / v_scale (fp32 [Hkv, D]).
hipError_t launch_int8_calibrate(Dtype dt, int D, const void* k, const void* v, int B, int Hkv,
                                 int S, const int32_t* positions, const RopeFreq& fr,
                                 float* k_scale, float* v_scale, hipStream_t s);

// A chunk continuing a cached prefix (P = seq_lens[b] tokens): rotates k at
// positions P..P+S-1 and stores the rotated keys and raw values there (as
// int8 codes if i8).
hipError_t launch_chunk_prep(Dtype dt, int D, bool paged, bool i8, const CacheArgs& c,
                             const void* k, const void* v, int B, int Hkv, int S,
                             const int32_t* seq_lens, const int32_t* chunk_lens,
                             const RopeFreq& fr, hipStream_t s);

// Rows 0..P+n-1 of each sequence of an INT8 cache, dequantized into dense
// [B, Hkv, max_seq, D] arrays dk, dv of the call's dtype, for the chunk
// attention to read as a contiguous cache of max_seq slots.
hipError_t launch_int8_dequant(Dtype dt, int D, bool paged, const CacheArgs& c, void* dk,
                               void* dv, int B, int Hkv, int S, int max_seq,
                               const int32_t* seq_lens, const int32_t* chunk_lens,
                               hipStream_t s);

// ---- prefill.hip -----------------------------------------------------------
// Whether launch_prefill_attention, given the contiguous native bf16 cache
// kcache of a prompt of this shape, stores the prompt's values into it (the
// paired form does; the K pass then stores only the keys).
bool prefill_attention_stores_values(Dtype dt, int B, int Hq, int S, const CacheArgs* kcache);

// kcache (nullable; bf16 only): the contiguous cache that the K pass filled
// with keys_in_cache; sequences whose positions are consecutive cache slots
// read their rotated keys from it instead of k_rot.  lens (nullable): tokens
// of each prompt; padding rows are written as zeros.
hipError_t launch_prefill_attention(Dtype dt, int D, const void* q, const void* k_rot,
                                    const void* v, void* out, int B, int Hq, int Hkv, int S,
                                    const int32_t* positions, const int32_t* lens,
                                    const RopeFreq& fr, float scale, const CacheArgs* kcache,
                                    hipStream_t s, const TimedLaunch& tl);

// Attention of a chunk over cache rows 0..P+S-1 (after launch_chunk_prep).
// chunk_lens (nullable): tokens of each sequence's chunk; the rest is padding.
// bf16 with a contiguous c whose k_scale is set: c holds INT8 codes as bf16
// (launch_int8_dequant) and the kernel applies the scales.
hipError_t launch_prefill_cached(Dtype dt, int D, bool paged, const void* q, void* out, int B,
                                 int Hq, int Hkv, int S, const CacheArgs& c,
                                 const int32_t* seq_lens, const int32_t* chunk_lens,
                                 const RopeFreq& fr, float scale, hipStream_t s,
                                 const TimedLaunch& tl);

// ---- decode.hip ------------------------------------------------------------
// Partials: [B, Hq, nsplit, decode_partial_words(D)] fp32 with nsplit =
// ceil(max_seq_len / split) <= ceil(max_seq_len / DECODE_SPLIT).
hipError_t launch_decode(Dtype dt, int D, int group, bool paged, const void* q,
                         const void* k_new, const void* v_new, void* out, int B, int Hq,
                         int Hkv, const int32_t* seq_lens, int max_seq_len, const CacheArgs& c,
                         float* partials, const RopeFreq& fr, float scale, hipStream_t s,
                         const TimedLaunch& tl);

// ---- decode_i8.hip ---------------------------------------------------------
// launch_decode over an INT8 cache (same partials workspace).
hipError_t launch_decode_i8(Dtype dt, int D, int group, bool paged, const void* q,
                            const void* k_new, const void* v_new, void* out, int B, int Hq,
                            int Hkv, const int32_t* seq_lens, int max_seq_len,
                            const CacheArgs& c, float* partials, const RopeFreq& fr,
                            float scale, hipStream_t s, const TimedLaunch& tl);

}  // namespace car
