/*
 * car.h -- causal attention with rotary position embedding (RoPE) and a KV
 * cache, as a C ABI over plain device pointers, for AMD MI355X (gfx950).
 *
 * What is computed is defined on these pages (titles as published):
 *   [Guide]     "手写LLM推理引擎：从黑盒到白盒的底层实现指南"
 *   [Intuition] "手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉"
 *   [Scratch]   "从零手搓AI推理引擎：告别调包思维，深入底层构建与优化"
 *   [NanoVLLM]  "以 Nano-vLLM 为例，深入理解 LLM 推理引擎（Part 2）"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Row-major, densely packed, head-major tensors ([Scratch] §3.1:
 *   the head split gives Q, K, V of shape (B, H, S, D); [Intuition] §5:
 *   a batch, head, sequence, dim order for the cache):
 *     q, out      [B, Hq,  S, D]      (decode: [B, Hq, D])
 *     k, v        [B, Hkv, S, D]      (decode: [B, Hkv, D])
 *     positions   int32 [B, S]        (decode uses seq_lens instead)
 *   Query head hq reads KV head hq / (Hq / Hkv) (contiguous GQA groups).
 * Element type.  CAR_DTYPE_F32 or CAR_DTYPE_BF16 for every float tensor of
 *   one call, caches included unless a cache is INT8 (car_cache_format).
 *   Arithmetic is fp32 (MFMA accumulation in fp32 for bf16); outputs are
 *   rounded to the element type, nearest-even.
 * Head dimension.  D must be 64 or 128; otherwise CAR_ERR_UNSUPPORTED.
 * RoPE ([Intuition] §4).  Each adjacent pair (x[2i], x[2i+1]) is rotated by
 *   the angle m * theta^(-2i/D), m the token's position:
 *   x'[2i] = x[2i] cos - x[2i+1] sin,  x'[2i+1] = x[2i] sin + x[2i+1] cos.
 *   V is never rotated.  `theta` is the base (10000 on the pages).
 * Positions and the cache.  A token's position equals its cache index
 *   ([Scratch] §3.2); positions are 0-based.
 * Ownership.  The caller owns every buffer.  The library never allocates,
 *   frees or keeps a pointer after a call returns, and holds no state
 *   between calls, with one exception: car_attn_decode_noalloc keeps its
 *   partials in a fixed device array per GPU (allocated when the library's
 *   code is loaded) and remembers that array's address per device.
 * Asynchrony.  Each call only enqueues kernels on `stream` (0 = the null
 *   stream) and returns; results are ready when the stream reaches them.
 * Errors.  Everything the host can check (null pointers, sizes, D, Hq/Hkv,
 *   16-byte alignment of every float tensor, block size, workspace size) is
 *   checked before any launch, and a failed check returns its status with
 *   nothing enqueued.  Nothing throws or aborts across the ABI.  Values in
 *   device memory (positions, seq_lens, block_table) cannot be checked by
 *   the host: the kernels clamp the indices they read, so that memory
 *   outside the given buffers is never touched, and store nothing at a cache
 *   index outside the cache (a position or seq_lens[b] outside [0, capacity),
 *   a chunk that does not fit), so that no other token's cached row is
 *   overwritten.  Outputs for such values are unspecified.
 */
#ifndef CAR_H_
#define CAR_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are int32 in C and in C++.  C++ sees them with a fixed
 * int32_t underlying type, so that any int32 a caller passes is a valid
 * value of the type: values not listed are rejected by the checks, never
 * undefined behaviour. */
#ifdef __cplusplus
#define CAR_ENUM(name) enum name : int32_t
#else
#define CAR_ENUM(name) enum name
#endif

typedef CAR_ENUM(car_dtype) {
  CAR_DTYPE_F32 = 0,
  CAR_DTYPE_BF16 = 1
} car_dtype;

/*
 * Which elements RoPE rotates together ([Intuition] §4 writes out the pairs
 * (q0,q1), (q2,q3), ...; checkpoints of the Llama/Qwen families the pages
 * name ([Guide] §6.1) pair each element of the first half with its twin in
 * the second).  Pair i has angle m * theta^(-2i/D) in both layouts.
 */
typedef CAR_ENUM(car_rope_pairing) {
  CAR_ROPE_ADJACENT = 0,  /* pair i = elements (2i, 2i+1) */
  CAR_ROPE_HALF = 1       /* pair i = elements (i, i + D/2) */
} car_rope_pairing;
/* Every entry point that rotates (car_rope_apply, car_attn_prefill,
 * car_attn_prefill_cached, car_attn_decode) takes the base theta (10000 on
 * the pages) and the pairing right after it; keys stored in a cache are
 * rotated in that layout, so one cache is read with one pairing.  Another
 * value returns CAR_ERR_UNSUPPORTED. */

/*
 * Element format of a KV cache.  [Intuition] §2 counts precision
 * compression of the cache, from 16-bit floats to INT8, among what a cache
 * has to support; [Scratch] §2.2 takes a channel's absolute maximum over 127
 * as its INT8 scale, computed once before inference and kept with the data,
 * and §5.3 divides by the scale and rounds to store, multiplying back to read.
 *   CAR_CACHE_NATIVE  elements of the call's dtype.
 *   CAR_CACHE_INT8    int8 codes, one fp32 scale per (KV head, channel):
 *     a value x of channel d, KV head hk is stored as
 *       code = clamp(round(x / s), -127, 127),  s = scale[hk][d],
 *     with x / s one IEEE fp32 division, ties rounded away from zero, and
 *     code 0 where s == 0; the cached value is code * s.  Keys are quantized
 *     from their fp32 rotated values.  car_kv_int8_calibrate computes the
 *     scales.  Every call that takes a cache accepts an INT8 one.
 */
typedef CAR_ENUM(car_cache_format) {
  CAR_CACHE_NATIVE = 0,
  CAR_CACHE_INT8 = 1
} car_cache_format;

typedef CAR_ENUM(car_status) {
  CAR_OK = 0,
  CAR_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, Hq % Hkv != 0,
                                   pointer not 16-byte aligned, bad cache shape */
  CAR_ERR_UNSUPPORTED = 2,      /* well formed but not built: D not in {64, 128},
                                   block_size != 16, Hq/Hkv not in {1, 2, 4, 8},
                                   unknown dtype, RoPE pairing or cache format */
  CAR_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  CAR_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} car_status;

/*
 * One layer's KV cache.  K and V are separate tensors ([NanoVLLM] §05, 5.2).
 *   contiguous (block_table == NULL): k, v are [B, Hkv, max_seq, D];
 *     token t of sequence b, head hk is row (b*Hkv + hk)*max_seq + t.
 *   paged (block_table != NULL): k, v are pools [num_blocks, Hkv, block_size, D]
 *     and block_table is int32 [B, max_blocks_per_seq]; token t of sequence b
 *     lives in physical block block_table[b][t / block_size] at offset
 *     t % block_size ([NanoVLLM] §05, 5.3; [Intuition] §5: pages of 16 tokens).
 *     block_size must be 16.
 * The caller keeps the table entries of every block a call touches in
 * [0, num_blocks) and distinct across sequences.
 * Element format (see car_cache_format): the call's dtype, or int8 codes in
 * the same shapes with fp32 scales k_scale, v_scale [Hkv, D] (device,
 * 16-byte aligned, read only).
 */
typedef struct car_kv_cache {
  void* k;
  void* v;
  const int32_t* block_table;
  int32_t max_seq;            /* contiguous: slots per sequence; ignored if paged */
  int32_t num_blocks;         /* paged only */
  int32_t block_size;         /* paged only; must be 16 */
  int32_t max_blocks_per_seq; /* paged only: row length of block_table */
  int32_t format;             /* car_cache_format; 0 (zero-initialised) is native */
  const float* k_scale;       /* CAR_CACHE_INT8 only */
  const float* v_scale;       /* CAR_CACHE_INT8 only */
} car_kv_cache;

/*
 * car_rope_apply -- rotate x in place by RoPE ([Intuition] §4).
 *   x          [B, H, S, D] device, read and written.
 *   positions  int32 [B, S] device: position m of token s of sequence b.
 * Every pair of every head and token is rotated by its own angle.
 */
car_status car_rope_apply(void* x, car_dtype dtype, int B, int H, int S, int D,
                          const int32_t* positions, float theta, car_rope_pairing pairing,
                          hipStream_t stream);

/*
 * car_kv_cache_append -- store already-rotated keys and raw values in the
 * cache at index == position ([Scratch] §3.2; [Guide] §2.5: K and V of a
 * token never change once computed, so they are written once and kept).
 *   k, v       [B, Hkv, S, D] device, read only.
 *   positions  int32 [B, S] device: cache index of each token; every index
 *              must lie below the cache capacity (max_seq, or
 *              max_blocks_per_seq * 16 when paged).
 *   cache      host pointer to the cache description; its k, v are written
 *              (as int8 codes for an INT8 cache).
 */
car_status car_kv_cache_append(const car_kv_cache* cache, car_dtype dtype,
                               const void* k, const void* v, int B, int Hkv, int S,
                               int D, const int32_t* positions, hipStream_t stream);

/*
 * car_kv_int8_calibrate -- the per-(KV head, channel) scales of an INT8 cache
 * from a calibration batch ([Scratch] §2.2: a channel's absolute maximum
 * divided by 127, computed once, before inference).  The keys are rotated at
 * their positions first, in fp32, because the cache holds rotated keys.
 *   k, v       [B, Hkv, S, D] device (k not rotated);  positions  int32 [B, S] device.
 *   k_scale, v_scale  fp32 [Hkv, D] device, 16-byte aligned, written:
 *              max over every (b, s) of |rotated key| (|value|) of the
 *              channel, divided by 127 (one fp32 division).
 * B * S == 0 writes zeros.  Inputs must be finite.
 */
car_status car_kv_int8_calibrate(const void* k, const void* v, car_dtype dtype, int B, int Hkv,
                                 int S, int D, const int32_t* positions, float theta,
                                 car_rope_pairing pairing, float* k_scale, float* v_scale,
                                 hipStream_t stream);

/*
 * Bytes of device workspace car_attn_prefill needs for these sizes: room for
 * the rotated keys [B, Hkv, S, D] in `dtype`, or 0 when they need none: bf16
 * into a contiguous native cache (`cache` non-NULL, no block table, format
 * native) with S at most its capacity.  Also 0 for invalid sizes.
 */
size_t car_attn_prefill_workspace_bytes(car_dtype dtype, int B, int Hkv, int S, int D,
                                        const car_kv_cache* cache);

/*
 * car_attn_prefill -- causal multi-head attention over a whole prompt.
 *   out[b, hq, i] = sum_j softmax_j(scale * q'[b,hq,i] . k'[b,hk,j]) v[b,hk,j]
 * over keys j with positions[b][j] <= positions[b][i], where q' and k' are q
 * and k rotated by RoPE at their positions ([Guide] §2.3 and §5.1: scaled
 * dot product, the upper-right triangle masked to -inf; [Scratch] §3.1 and
 * §3.3).  It runs as a tiled online softmax ([Scratch] §3.4: a running
 * maximum m and sum l per query row, the earlier accumulation corrected at
 * each key block) and never stores the S x S score matrix.
 *   q          [B, Hq, S, D] device;   k, v  [B, Hkv, S, D] device (k not rotated).
 *   out        [B, Hq, S, D] device, written.
 *   positions  int32 [B, S] device, strictly increasing along s over each
 *              prompt's tokens (so that the position order equals the index
 *              order); entries of padding rows are not read.
 *   seq_lens   NULL: every prompt has S tokens.  Otherwise int32 [B] device:
 *              prompt b is its first seq_lens[b] rows (0..S; values outside
 *              are clamped), a padded batch of prompts of different lengths
 *              ([Scratch] §3.3 names the padding mask).  Padding rows are
 *              neither attended to nor stored in the cache, and their output
 *              rows are written as zeros.
 *   scale      multiplies the scores before the softmax; 1/sqrt(D) on the
 *              pages ([Intuition] §4).
 *   cache      NULL: nothing is stored.  Otherwise every rotated key and raw
 *              value of a prompt token is also stored at index
 *              positions[b][s], as by
 *              car_kv_cache_append.  With an INT8 cache only the stored
 *              copy is quantized: the prompt attends to its own keys and
 *              values at full precision.
 *   workspace  device scratch for the rotated keys; its contents on entry are
 *              ignored and on exit unspecified.  With B*Hkv*S*D elements or
 *              more it is used.  Otherwise (NULL or smaller; allowed only when
 *              car_attn_prefill_workspace_bytes() is 0) the attention reads
 *              each prompt's rotated keys back from the cache rows p0.. where
 *              p0 is its first position: each prompt's positions must then be
 *              consecutive (p0, p0+1, ...) inside the cache, or its output is
 *              unspecified (the cache store stays correct, and no read leaves
 *              the cache).  With a workspace, prompts at consecutive slots
 *              read their keys from the cache too; others read the workspace.
 * S == 0 is a no-op returning CAR_OK.  Sizes one launch cannot cover (B or
 * Hq above 65535, B * Hq * ceil(S / 64) above 2^31 - 1, or S, or a cache's
 * capacity, times D * 4 bytes above 2^32 - 1) return CAR_ERR_UNSUPPORTED
 * before any work is queued.
 */
car_status car_attn_prefill(const void* q, const void* k, const void* v, void* out,
                            car_dtype dtype, int B, int Hq, int Hkv, int S, int D,
                            const int32_t* positions, const int32_t* seq_lens, float theta,
                            car_rope_pairing pairing,
                            float scale,
                            const car_kv_cache* cache, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * car_attn_prefill_cached -- a prompt chunk that continues a cached prefix
 * (chunked or continued prefill).  With P = seq_lens[b] tokens already in
 * the cache, the chunk's S tokens sit at positions P..P+S-1, which are also
 * their cache indices ([Scratch] §3.2).  q and k are rotated at those
 * positions; the rotated keys and raw values are stored at cache indices
 * P..P+S-1; chunk query i then attends over cache indices 0..P+i, the cached
 * prefix and the chunk up to itself ([Scratch] §3.3: a position sees itself
 * and earlier ones, the earlier ones read from the cache):
 *   out[b, hq, i] = sum_{j <= P+i} softmax_j(scale * q'[b,hq,i] . K[b,hk,j]) V[b,hk,j].
 * S = 1 is a decode step; P = 0 is a whole-prompt prefill that fills the cache.
 *   q            [B, Hq, S, D] device;  k, v  [B, Hkv, S, D] device (k not rotated).
 *   out          [B, Hq, S, D] device, written.
 *   seq_lens     int32 [B] device: tokens already cached; seq_lens[b] plus the
 *                chunk's length must not exceed max_seq_len.  (A value that
 *                would not fit is lowered until the chunk fits the cache.)
 *   chunk_lens   NULL: every chunk has S tokens.  Otherwise int32 [B] device:
 *                sequence b's chunk is its first chunk_lens[b] tokens (0..S),
 *                the rest of its S rows are padding ([Scratch] §3.3 names the
 *                padding mask): padding tokens are neither stored nor attended
 *                to, and their output rows are written as zeros.
 *   max_seq_len  host bound on seq_lens[b] + (chunk length) over the batch; at
 *                most the cache capacity, and at least S when chunk_lens is NULL.
 *   cache        contiguous or paged, native or INT8; rows 0..P-1 must hold the
 *                prefix (as written by earlier calls), rows P..P+S-1 are written.
 *                With an INT8 cache the chunk's keys and values are stored as
 *                codes first, and every key and value the chunk attends to,
 *                its own tokens included, is read back dequantized (code *
 *                scale), as a decode step reads its new token.
 *   workspace    native cache: unused (may be NULL).  INT8 cache: device scratch
 *                of at least car_attn_prefill_cached_workspace_bytes(), which
 *                receives the dequantized rows; contents on entry ignored, on
 *                exit unspecified.
 * S == 0 or an empty batch is a no-op returning CAR_OK.  Sizes one launch
 * cannot cover return CAR_ERR_UNSUPPORTED.
 */
car_status car_attn_prefill_cached(const void* q, const void* k, const void* v, void* out,
                                   car_dtype dtype, int B, int Hq, int Hkv, int S, int D,
                                   const int32_t* seq_lens, const int32_t* chunk_lens,
                                   int max_seq_len, float theta, car_rope_pairing pairing,
                                   float scale, const car_kv_cache* cache, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace car_attn_prefill_cached needs: 0 for a native
 * cache; for an INT8 cache two dense copies (K and V) of [B, Hkv,
 * max_seq_len, D] in `dtype`, each rounded up to 256 bytes.  Also 0 for
 * invalid sizes.
 */
size_t car_attn_prefill_cached_workspace_bytes(car_dtype dtype, int B, int Hkv, int D,
                                               int max_seq_len, const car_kv_cache* cache);

/*
 * Bytes of device workspace car_attn_decode needs: per (sequence, query head)
 * one partial (running max, running sum, D accumulators) in fp32 for every
 * 256-token split of max_seq_len tokens.  Returns 0 for invalid sizes.
 */
size_t car_attn_decode_workspace_bytes(int B, int Hq, int D, int max_seq_len);

/*
 * car_attn_decode -- one decode step: one new query token per sequence.
 * With L = seq_lens[b] tokens already cached, the new token's position is L
 * ([Scratch] §3.2).  q and k_new are rotated at position L; the rotated key
 * and raw value are written to cache index L; the query then attends over
 * cache indices 0..L, the cached tokens and itself ([Guide] §2.5: only the
 * new token's Q, K, V are computed; [Scratch] §3.3: with a cache the mask is
 * a single row, all visible).
 *   q           [B, Hq, D] device;  k_new, v_new  [B, Hkv, D] device (not rotated).
 *   out         [B, Hq, D] device, written.
 *   seq_lens    int32 [B] device; L + 1 must fit the cache capacity and
 *               must not exceed max_seq_len.
 *   max_seq_len host bound on seq_lens[b] + 1 over the batch; it sizes the
 *               launch (tokens beyond it are not read).
 *   cache       contiguous or paged, written at index L for every sequence.
 *               With an INT8 cache the new key and value are stored as codes
 *               and token L is attended to in that quantized form, like
 *               every cached token.
 *   workspace   device scratch of at least car_attn_decode_workspace_bytes();
 *               contents on entry ignored, on exit unspecified.
 * Calls that share a workspace must be ordered on one stream.
 * Sizes one launch cannot cover (B * Hq above 2^31 - 1, max_seq_len above
 * 65535 * 256 tokens, or a contiguous cache whose capacity times D * 4 bytes
 * is above 2^32 - 1) return CAR_ERR_UNSUPPORTED before any work is queued.
 */
car_status car_attn_decode(const void* q, const void* k_new, const void* v_new,
                           void* out, car_dtype dtype, int B, int Hq, int Hkv, int D,
                           const int32_t* seq_lens, int max_seq_len, float theta,
                           car_rope_pairing pairing,
                           float scale, const car_kv_cache* cache, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Timed variants: the same calls, with `kernel_start` recorded on `stream`
 * immediately before the call's attention kernel and `kernel_stop`
 * immediately after it, so that hipEventElapsedTime(kernel_start,
 * kernel_stop) is that one kernel's duration (a prefill's key-rotation
 * pass and any other kernel of the call fall outside).  Both events NULL:
 * exactly the untimed call.  Only one of the two NULL: nothing is recorded.
 */
car_status car_attn_prefill_timed(const void* q, const void* k, const void* v, void* out,
                                  car_dtype dtype, int B, int Hq, int Hkv, int S, int D,
                                  const int32_t* positions, const int32_t* seq_lens,
                                  float theta,
                                  car_rope_pairing pairing, float scale,
                                  const car_kv_cache* cache, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream,
                                  hipEvent_t kernel_start, hipEvent_t kernel_stop);
car_status car_attn_prefill_cached_timed(const void* q, const void* k, const void* v,
                                         void* out, car_dtype dtype, int B, int Hq, int Hkv,
                                         int S, int D, const int32_t* seq_lens,
                                         const int32_t* chunk_lens, int max_seq_len,
                                         float theta, car_rope_pairing pairing, float scale,
                                         const car_kv_cache* cache, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream,
                                         hipEvent_t kernel_start, hipEvent_t kernel_stop);
car_status car_attn_decode_timed(const void* q, const void* k_new, const void* v_new,
                                 void* out, car_dtype dtype, int B, int Hq, int Hkv, int D,
                                 const int32_t* seq_lens, int max_seq_len, float theta,
                                 car_rope_pairing pairing, float scale,
                                 const car_kv_cache* cache, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * car_attn_decode_noalloc -- car_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as car_attn_decode
 * without the workspace: the split partials live in a file-scope device array
 * of CAR_DECODE_NOALLOC_MAX_BYTES that every GPU the library runs on holds
 * until the process ends.  The call allocates and frees nothing.
 *   Limit: sizes with car_attn_decode_workspace_bytes(B, Hq, D, max_seq_len)
 *   above CAR_DECODE_NOALLOC_MAX_BYTES return CAR_ERR_WORKSPACE before any
 *   work is queued (48 MiB holds, e.g., 64 sequences of 32 query heads,
 *   D = 128, up to 11776 tokens).
 *   Device: the stream's (the current device for the null stream).  The first
 *   call on a device looks up the array's address there (hipGetSymbolAddress)
 *   and keeps it.
 *   Concurrency: every call on one GPU shares that GPU's array, so calls that
 *   overlap on a GPU (different streams or threads, unordered) race and must
 *   not be issued; calls ordered on one stream are safe.
 */
#define CAR_DECODE_NOALLOC_MAX_BYTES ((size_t)48 << 20)
car_status car_attn_decode_noalloc(const void* q, const void* k_new, const void* v_new,
                                   void* out, car_dtype dtype, int B, int Hq, int Hkv, int D,
                                   const int32_t* seq_lens, int max_seq_len, float theta,
                                   car_rope_pairing pairing, float scale,
                                   const car_kv_cache* cache, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* car_status_string(car_status status);

#ifdef __cplusplus
}
#endif

#endif /* CAR_H_ */
