// Device-side helpers shared by the kernels: element conversion, 16-byte
// vector access, the RoPE angle, DPP lane reductions.  gfx950 only.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.hpp"

namespace car {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats to packed bf16 (round to nearest even; gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a;
  const __bf16 hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Number of T elements in one 16-byte vector.
template <typename T> struct Vec16;
template <> struct Vec16<float> { static constexpr int N = 4; };
template <> struct Vec16<bf16_t> { static constexpr int N = 8; };

// 16-byte load into fp32 registers.
template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&f)[Vec16<T>::N]);

template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&f)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
}

template <>
__device__ __forceinline__ void load16<bf16_t>(const bf16_t* p, float (&f)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// Element e of a raw 16-byte vector of T, as fp32 (e a compile-time index).
template <typename T>
__device__ __forceinline__ float elem(const uint4& u, int e) {
  constexpr int PER_WORD = 4 / (int)sizeof(T);
  const int word = e / PER_WORD;
  const uint32_t w = word == 0 ? u.x : word == 1 ? u.y : word == 2 ? u.z : u.w;
  if constexpr (sizeof(T) == 4) return __uint_as_float(w);
  else return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// 16-byte store from fp32 registers (rounded to T).
template <typename T>
__device__ __forceinline__ void store16(T* p, const float (&f)[Vec16<T>::N]);

template <>
__device__ __forceinline__ void store16<float>(float* p, const float (&f)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

template <>
__device__ __forceinline__ void store16<bf16_t>(bf16_t* p, const float (&f)[8]) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]);
  u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]);
  u.w = pack_bf16x2(f[6], f[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// ---------------------------------------------------------------------------
// RoPE angle.  The angle of pair i at position m is m * theta_i with
// theta_i = base^(-2i/D).  It is handled in revolutions: the host supplies
// f_i = theta_i / (2 pi) as an unevaluated sum hi + lo of two floats (from a
// double), the product m * f_i is formed with an exact FMA residual, and its
// integer part is removed exactly, which leaves r in [-1/2, 1/2] revolutions
// with an absolute error near 2^-40.  cos and sin of 2 pi r come from the
// hardware v_cos_f32 / v_sin_f32, which take revolutions (measured max
// absolute error 1.24e-7 on [-1/2, 1/2)).  Branch free; valid for every
// position below 2^24.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cos_sin(int pos, float f_hi, float f_lo, float& c,
                                             float& s) {
  // No FMA contraction here: fusing m * f_hi into a - rint(a) would add the
  // product's rounding residual a second time.
#pragma clang fp contract(off)
  const float m = (float)pos;
  const float a = m * f_hi;
  const float e = fmaf(m, f_hi, -a) + m * f_lo;  // exact residual + low part
  const float r = (a - rintf(a)) + e;            // a - rint(a) is exact
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

// Rotate the adjacent pairs held in f[0..N) whose first pair index is p0.
template <int N>
__device__ __forceinline__ void rope_rotate_regs(float (&f)[N], int pos, int p0,
                                                 const RopeFreq& fr) {
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    float c, s;
    rope_cos_sin(pos, fr.hi[p0 + j], fr.lo[p0 + j], c, s);
    const float x0 = f[2 * j], x1 = f[2 * j + 1];
    f[2 * j] = x0 * c - x1 * s;
    f[2 * j + 1] = x0 * s + x1 * c;
  }
}

// Half-split layout (pair i = elements i and i + D/2): rotate the chunk
// f = elements d0..d0+N-1 of a row, given p = the partner elements d0 +- D/2
// (read from the unrotated row).  Elements of the first half take the first
// component of their pair's rotation, those of the second half the second.
template <int N>
__device__ __forceinline__ void rope_rotate_half_chunk(float (&f)[N], const float (&p)[N], int pos,
                                                       int d0, int D, const RopeFreq& fr) {
  const bool first = d0 < D / 2;
  const int i0 = first ? d0 : d0 - D / 2;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float c, s;
    rope_cos_sin(pos, fr.hi[i0 + j], fr.lo[i0 + j], c, s);
    f[j] = first ? f[j] * c - p[j] * s : p[j] * s + f[j] * c;
  }
}

// Element offset of the half-split partner of the chunk starting at d0.
__device__ __forceinline__ int rope_half_partner(int d0, int D) {
  return d0 < D / 2 ? d0 + D / 2 : d0 - D / 2;
}

// Rotate a chunk of a row that is only read: elements d0..d0+N-1 of `row`,
// already loaded into f, in either pair layout (HALF: 0 adjacent, 1 half
// split, -1 taken from fr.half at run time).
template <typename T, int N, int HALF = -1>
__device__ __forceinline__ void rope_rotate_chunk(float (&f)[N], const T* row, int d0, int D,
                                                  int pos, const RopeFreq& fr) {
  if (HALF == 1 || (HALF < 0 && fr.half)) {
    float p[N];
    load16<T>(row + rope_half_partner(d0, D), p);
    rope_rotate_half_chunk<N>(f, p, pos, d0, D, fr);
  } else {
    rope_rotate_regs<N>(f, pos, d0 / 2, fr);
  }
}

// The cos/sin a lane needs to rotate its chunk (elements d0..d0+N-1) at one
// position, computed once and applied to any number of rows at that
// position (the query heads and the new key of a decode step).
template <int N>
struct RopeChunk {
  float c[N], s[N];  // adjacent: N/2 pair angles; half split: one per element
  int d0;
};

template <int N, int HALF>  // HALF: 0 adjacent, 1 half split, -1 taken from fr.half
__device__ __forceinline__ RopeChunk<N> rope_prepare(int pos, int d0, int D, const RopeFreq& fr) {
  RopeChunk<N> r;
  r.d0 = d0;
  if (HALF == 1 || (HALF < 0 && fr.half)) {
    const int i0 = d0 < D / 2 ? d0 : d0 - D / 2;
#pragma unroll
    for (int j = 0; j < N; ++j) rope_cos_sin(pos, fr.hi[i0 + j], fr.lo[i0 + j], r.c[j], r.s[j]);
  } else {
#pragma unroll
    for (int j = 0; j < N / 2; ++j)
      rope_cos_sin(pos, fr.hi[d0 / 2 + j], fr.lo[d0 / 2 + j], r.c[j], r.s[j]);
  }
  return r;
}

// Rotate the chunk f (elements r.d0.. of `row`, already loaded) with the
// prepared angles; the half-split layout reads the partner chunk from `row`.
template <typename T, int N, int HALF>
__device__ __forceinline__ void rope_apply_prepared(float (&f)[N], const T* row, int D,
                                                    const RopeChunk<N>& r, const RopeFreq& fr) {
  if (HALF == 1 || (HALF < 0 && fr.half)) {
    float p[N];
    load16<T>(row + rope_half_partner(r.d0, D), p);
    const bool first = r.d0 < D / 2;
#pragma unroll
    for (int j = 0; j < N; ++j)
      f[j] = first ? f[j] * r.c[j] - p[j] * r.s[j] : p[j] * r.s[j] + f[j] * r.c[j];
  } else {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      const float x0 = f[2 * j], x1 = f[2 * j + 1];
      f[2 * j] = x0 * r.c[j] - x1 * r.s[j];
      f[2 * j + 1] = x0 * r.s[j] + x1 * r.c[j];
    }
  }
}

// ---------------------------------------------------------------------------
// INT8 cache codes ([Scratch] "从零手搓AI推理引擎" §2.2 and §5.3: a channel's
// scale is its absolute maximum over 127; a value is divided by its scale and
// rounded to store it, and multiplied by it to read it back).
// ---------------------------------------------------------------------------
// x / s as one IEEE fp32 division, rounded half away from zero, clamped to the
// symmetric range [-127, 127]; 0 when s == 0.  Returns the code's byte.
__device__ __forceinline__ uint32_t int8_code(float x, float s) {
  if (s == 0.f) return 0u;
  const float r = fminf(fmaxf(roundf(__fdiv_rn(x, s)), -127.f), 127.f);
  return (uint32_t)(int32_t)r & 0xffu;
}

// Codes of f[0..N) with the scales s[0..N) (16-byte aligned), four to a word,
// element 4w + j in byte j of word w (memory order).
template <int N>
__device__ __forceinline__ void int8_codes(const float (&f)[N], const float* s,
                                           uint32_t (&w)[N / 4]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const float4 sc = *reinterpret_cast<const float4*>(s + 4 * i);
    w[i] = int8_code(f[4 * i], sc.x) | (int8_code(f[4 * i + 1], sc.y) << 8) |
           (int8_code(f[4 * i + 2], sc.z) << 16) | (int8_code(f[4 * i + 3], sc.w) << 24);
  }
}

// Stores the N codes of f (N = 4, 8 or 16 bytes at p, aligned to N).
template <int N>
__device__ __forceinline__ void store_int8(int8_t* p, const float (&f)[N], const float* s) {
  uint32_t w[N / 4];
  int8_codes<N>(f, s, w);
  if constexpr (N == 4) *reinterpret_cast<uint32_t*>(p) = w[0];
  else if constexpr (N == 8) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  else *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Code j (0..3) of a word of four codes as fp32 (a sign-extended byte select
// folds into one conversion instruction).
__device__ __forceinline__ float int8_elem(uint32_t w, int j) {
  return (float)(int8_t)(w >> (8 * j));
}

// ---------------------------------------------------------------------------
// Cache addressing: element offset of row (sequence b, head hk, token t).
// ---------------------------------------------------------------------------
template <bool PAGED>
__device__ __forceinline__ int64_t cache_row(const CacheArgs& c, int b, int hk, int Hkv,
                                             int t);

template <>
__device__ __forceinline__ int64_t cache_row<false>(const CacheArgs& c, int b, int hk,
                                                    int Hkv, int t) {
  return ((int64_t)b * Hkv + hk) * c.max_seq + t;
}

template <>
__device__ __forceinline__ int64_t cache_row<true>(const CacheArgs& c, int b, int hk,
                                                   int Hkv, int t) {
  int blk = c.table[(int64_t)b * c.mbps + (t >> 4)];
  blk = min(max(blk, 0), c.num_blocks - 1);
  return (((int64_t)blk * Hkv + hk) << 4) + (t & 15);
}

// Largest token index a sequence can hold.
template <bool PAGED>
__device__ __forceinline__ int cache_last_slot(const CacheArgs& c) {
  return PAGED ? c.mbps * 16 - 1 : c.max_seq - 1;
}

// Whether the n >= 1 tokens of prompt b (positions rows of S entries) sit at
// positions p0, p0+1, ..., p0+n-1 with every one a slot of a contiguous cache
// of max_seq slots.  Positions strictly increase over a prompt's tokens, so
// the first and the last decide it.  Then the prompt's rotated keys, once
// stored at their positions, are rows p0..p0+n-1 of each head in the cache,
// and the attention reads them there.  An empty prompt (n = 0) gives false.
__device__ __forceinline__ bool prompt_rows_in_cache(const int32_t* positions, int b, int S,
                                                     int n, int max_seq, int* p0) {
  const int first = positions[(int64_t)b * S];
  const int last = positions[(int64_t)b * S + max(n, 1) - 1];
  *p0 = first;
  return n >= 1 && first >= 0 && last <= max_seq - 1 && last - first == n - 1;
}

// ---------------------------------------------------------------------------
// Lane exchange
// ---------------------------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int DPP_QUAD_XOR1 = 0xB1;
constexpr int DPP_QUAD_XOR2 = 0x4E;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LANES consecutive lanes (LANES in 1..64); every
// lane of a group receives the group's sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LANES >= 2) x += dpp_mov<DPP_QUAD_XOR1>(x);
  if constexpr (LANES >= 4) x += dpp_mov<DPP_QUAD_XOR2>(x);
  if constexpr (LANES >= 8) x += dpp_mov<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (LANES >= 16) x += dpp_mov<DPP_ROW_MIRROR>(x);
  if constexpr (LANES >= 32) x += __shfl_xor(x, 16);
  if constexpr (LANES >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Maximum over aligned groups of LANES consecutive lanes (LANES in 1..32).
template <int LANES>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (LANES >= 2) x = fmaxf(x, dpp_mov<DPP_QUAD_XOR1>(x));
  if constexpr (LANES >= 4) x = fmaxf(x, dpp_mov<DPP_QUAD_XOR2>(x));
  if constexpr (LANES >= 8) x = fmaxf(x, dpp_mov<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (LANES >= 16) x = fmaxf(x, dpp_mov<DPP_ROW_MIRROR>(x));
  if constexpr (LANES >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  return x;
}

// All-reduce over the lanes that share lane % STRIDE, STRIDE in {4, 8, 16, 32},
// without LDS traffic: rotations by 4 and 8 inside each row of 16 lanes (DPP
// row_ror), then the swaps of 16-lane rows and of 32-lane halves
// (v_permlane16_swap / v_permlane32_swap).
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;

// The two results of a permlane swap of x with itself hold, on every lane,
// the lane's own x and its partner's (lane ^ 16, resp. lane ^ 32), in an
// order that depends on the lane; a symmetric combine needs no select.
template <bool MAX>
__device__ __forceinline__ float combine16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return MAX ? fmaxf(a, b) : a + b;
}
template <bool MAX>
__device__ __forceinline__ float combine32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return MAX ? fmaxf(a, b) : a + b;
}

template <int STRIDE>
__device__ __forceinline__ float class_max(float x) {
  static_assert(STRIDE == 4 || STRIDE == 8 || STRIDE == 16 || STRIDE == 32, "stride");
  if constexpr (STRIDE <= 4) x = fmaxf(x, dpp_mov<DPP_ROW_ROR4>(x));
  if constexpr (STRIDE <= 8) x = fmaxf(x, dpp_mov<DPP_ROW_ROR8>(x));
  if constexpr (STRIDE <= 16) x = combine16<true>(x);
  return combine32<true>(x);
}

template <int STRIDE>
__device__ __forceinline__ float class_sum(float x) {
  static_assert(STRIDE == 4 || STRIDE == 8 || STRIDE == 16 || STRIDE == 32, "stride");
  if constexpr (STRIDE <= 4) x += dpp_mov<DPP_ROW_ROR4>(x);
  if constexpr (STRIDE <= 8) x += dpp_mov<DPP_ROW_ROR8>(x);
  if constexpr (STRIDE <= 16) x = combine16<false>(x);
  return combine32<false>(x);
}

// Reductions across the lanes that share lane % STRIDE (STRIDE a power of
// two dividing 64): combines lane, lane ^ STRIDE, lane ^ 2*STRIDE, ...
template <int STRIDE>
__device__ __forceinline__ float strided_max(float x) {
#pragma unroll
  for (int s = STRIDE; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}

template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
#pragma unroll
  for (int s = STRIDE; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Calls f(std::integral_constant<int, I>) for I = B .. E-1, so that array
// indices inside f are constants from the start (keeps small arrays in
// registers instead of stack memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace car
