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
// RoPE angle.  The angle of pair i at position m is m * f_i with
// f_i = theta^(-2i/D) supplied as an unevaluated sum hi + lo of two floats
// (computed once on the host in double precision).  The product is formed
// with an exact FMA residual, a = a_hi + a_lo.
//
// cos/sin use Cody and Waite's argument reduction: k = rint(a_hi * 2/pi),
// r = a_hi - k*(P1 + P2 + P3) + a_lo with pi/2 = P1 + P2 + P3 split into
// floats and each step an FMA; then Taylor polynomials on |r| <= pi/4
// (truncation below 3e-9) and the quadrant k mod 4.  Branch free.  The
// reduction keeps the absolute error near 1e-7 for |a| up to ~1e5 rad,
// i.e. every position a 32-bit cache index can hold at theta_0 = 1 up to
// 1e5 tokens; beyond that the error grows linearly with |a|.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cos_sin(int pos, float f_hi, float f_lo, float& c,
                                             float& s) {
  const float m = (float)pos;
  const float a = m * f_hi;
  const float a_lo = fmaf(m, f_hi, -a) + m * f_lo;
  constexpr float TWO_OVER_PI = 0.636619772367581343f;
  constexpr float P1 = 1.57079637050628662109e+00f;   // float(pi/2)
  constexpr float P2 = -4.37113882867379288655e-08f;  // float(pi/2 - P1)
  constexpr float P3 = -1.71512451000588187280e-15f;  // float(pi/2 - P1 - P2)
  const float k = rintf(a * TWO_OVER_PI);
  float r = fmaf(-k, P1, a);
  r = fmaf(-k, P2, r);
  r = fmaf(-k, P3, r);
  r += a_lo;
  const float r2 = r * r;
  // sin r = r - r^3/3! + r^5/5! - r^7/7! + r^9/9!
  float ps = fmaf(r2, 2.75573192239858906526e-06f, -1.98412698412698412526e-04f);
  ps = fmaf(r2, ps, 8.33333333333333321769e-03f);
  ps = fmaf(r2, ps, -1.66666666666666657415e-01f);
  const float sr = fmaf(r * r2, ps, r);
  // cos r = 1 - r^2/2! + r^4/4! - r^6/6! + r^8/8! - r^10/10!
  float pc = fmaf(r2, -2.75573192239858906526e-07f, 2.48015873015873015658e-05f);
  pc = fmaf(r2, pc, -1.38888888888888894189e-03f);
  pc = fmaf(r2, pc, 4.16666666666666643537e-02f);
  pc = fmaf(r2, pc, -0.5f);
  const float cr = fmaf(r2, pc, 1.0f);
  const int quadrant = ((int)k) & 3;
  const float s0 = (quadrant & 1) ? cr : sr;
  const float c0 = (quadrant & 1) ? sr : cr;
  s = (quadrant & 2) ? -s0 : s0;
  c = ((quadrant + 1) & 2) ? -c0 : c0;
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
