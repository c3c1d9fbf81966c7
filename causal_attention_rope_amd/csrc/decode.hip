// Decode attention: one new query token per sequence over its KV cache.
//
// What is computed ([Guide] "手写LLM推理引擎：从黑盒到白盒的底层实现指南" §2.5;
// [Scratch] "从零手搓AI推理引擎" §3.2-§3.3): with L tokens cached, the new token
// sits at position L; q and k_new are rotated there, k_new/v_new are stored at
// cache index L, and the query attends over indices 0..L.  Paged caches map
// index t to block_table[t / 16], offset t % 16 ([NanoVLLM] "以 Nano-vLLM 为例，
// 深入理解 LLM 推理引擎（Part 2）" §05, 5.3).
//
// How it maps to MI355X.  Decode reads every cached K/V row once and does
// ~1 flop per byte, so it is bound by HBM bandwidth.  The sequence is split
// into 256-token pieces; workgroup (split, kv head, sequence) streams its
// piece with 16-byte loads, LPR = D*sizeof(T)/16 lanes covering one row, so a
// wave load instruction moves 64/LPR whole rows (4 rows of 256 bytes for
// bf16, D = 128).  All G = Hq/Hkv query heads of a KV head are served from the
// same loads (GQA).  Dot products are reduced across the LPR lanes of a row
// with DPP moves; the softmax maximum and sums are combined across the rows
// of a wave with lane shuffles and across the 4 waves through LDS.  Each
// workgroup leaves one partial (max, sum, D accumulators) per query head; a
// second small kernel merges the partials of a sequence with the
// log-sum-exp rule of the online softmax ([Scratch] §3.4).  The workgroup
// whose piece holds index L also rotates k_new and stores it and v_new into
// the cache, and uses the new row from registers for its own score.
#include <math.h>

#include "common.hpp"

namespace car {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Rows per lane loaded at once: at most 16 (128 VGPRs of raw K/V) and at
// most 16 score registers across the G query heads, so that 2 waves fit per
// SIMD with the query and accumulator registers of all G heads.
constexpr int decode_steps(int all, int G) {
  const int s = all < 16 ? all : 16;
  return s < 16 / G ? s : 16 / G;
}

template <typename T, int D, int G, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ seq_lens, CacheArgs c, float* __restrict__ part, int Hkv,
    int nsplit, RopeFreq fr, float qk_scale) {
  constexpr int N = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = D / N;          // lanes per cache row
  constexpr int NG = 64 / LPR;        // rows per wave load instruction
  constexpr int TPW = DECODE_SPLIT / kWaves;  // tokens per wave
  constexpr int STEPS_ALL = TPW / NG;
  constexpr int STEPS = decode_steps(STEPS_ALL, G);
  constexpr int PASSES = STEPS_ALL / STEPS;
  constexpr int PW = decode_partial_words(D);
  static_assert(STEPS * PASSES == STEPS_ALL, "split must divide evenly");

  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_ml[kWaves][G][2];

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int L = min(max(seq_lens[b], 0), cache_last_slot<PAGED>(c));
  const int t0 = split * DECODE_SPLIT;
  if (t0 > L) return;  // uniform over the workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int grp = lane / LPR;
  const int col = (lane % LPR) * N;

  // Query heads of this KV head, rotated at position L, pre-scaled so that
  // exp2 of a score difference is the softmax weight.
  float qv[G][N];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load16<T>(q + ((int64_t)b * Hq + hk * G + g) * D + col, qv[g]);
    rope_rotate_regs<N>(qv[g], L, col / 2, fr);
#pragma unroll
    for (int e = 0; e < N; ++e) qv[g][e] *= qk_scale;
  }

  // The new token (index L) lives in this split's range only for one split.
  float kn[N], vn[N];
#pragma unroll
  for (int e = 0; e < N; ++e) kn[e] = vn[e] = 0.f;
  T* const Kc = static_cast<T*>(c.k);
  T* const Vc = static_cast<T*>(c.v);
  if (L < t0 + DECODE_SPLIT) {
    const int64_t src = ((int64_t)b * Hkv + hk) * D + col;
    load16<T>(k_new + src, kn);
    rope_rotate_regs<N>(kn, L, col / 2, fr);
    load16<T>(v_new + src, vn);
    if (wave == 0 && grp == 0) {
      const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, L) * D + col;
      store16<T>(Kc + dst, kn);
      *reinterpret_cast<uint4*>(Vc + dst) = *reinterpret_cast<const uint4*>(v_new + src);
    }
  }

  float m_run[G], l_run[G], acc[G][N];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) acc[g][e] = 0.f;
  }

  const int tw = t0 + wave * TPW;
  const int t_hi = L > 0 ? L - 1 : 0;  // last cached row (clamp target)
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    // Issue every K and V load of the pass first (memory-level parallelism);
    // rows are kept as raw 16-byte vectors and widened where they are used.
    uint4 kraw[STEPS], vraw[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int t = tw + (pass * STEPS + st) * NG + grp;
      const int64_t row = cache_row<PAGED>(c, b, hk, Hkv, min(t, t_hi));
      kraw[st] = *reinterpret_cast<const uint4*>(Kc + row * D + col);
      vraw[st] = *reinterpret_cast<const uint4*>(Vc + row * D + col);
    }
    float sc[STEPS][G];
    float mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = -INFINITY;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int t = tw + (pass * STEPS + st) * NG + grp;
      float kf[N];
#pragma unroll
      for (int e = 0; e < N; ++e) kf[e] = t < L ? elem<T>(kraw[st], e) : kn[e];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) p = fmaf(qv[g][e], kf[e], p);
        p = group_sum<LPR>(p);
        sc[st][g] = t <= L ? p : -INFINITY;
        mx[g] = fmaxf(mx[g], sc[st][g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m_new = fmaxf(m_run[g], strided_max<LPR>(mx[g]));
      // m_new is -inf only while no valid token has been seen by this wave.
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run[g] - m_new);
      l_run[g] *= alpha;
#pragma unroll
      for (int e = 0; e < N; ++e) acc[g][e] *= alpha;
      m_run[g] = m_new;
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int t = tw + (pass * STEPS + st) * NG + grp;
      float vf[N];
#pragma unroll
      for (int e = 0; e < N; ++e) vf[e] = t < L ? elem<T>(vraw[st], e) : (t == L ? vn[e] : 0.f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = t <= L ? fast_exp2(sc[st][g] - m_run[g]) : 0.f;
        l_run[g] += p;
#pragma unroll
        for (int e = 0; e < N; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
      }
    }
  }

  // Merge the rows of the wave (lanes that share the same columns).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = strided_sum<LPR>(l_run[g]);
#pragma unroll
    for (int e = 0; e < N; ++e) acc[g][e] = strided_sum<LPR>(acc[g][e]);
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < N; ++e) sm_acc[wave][g][col + e] = acc[g][e];
      if (lane == 0) {
        sm_ml[wave][g][0] = m_run[g];
        sm_ml[wave][g][1] = l_run[g];
      }
    }
  }
  __syncthreads();

  // Merge the waves and write one partial per query head.
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][g][0]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_ml[w][g][0];
      const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      a = fmaf(f, sm_acc[w][g][d], a);
      l = fmaf(f, sm_ml[w][g][1], l);
    }
    float* dst = part + (((int64_t)b * Hq + hk * G + g) * nsplit + split) * PW;
    dst[4 + d] = a;
    if (d == 0) {
      dst[0] = M;
      dst[1] = l;
    }
  }
}

// One wave per (sequence, query head): merge the partials of all splits that
// hold tokens 0..L and write the normalised output.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ seq_lens,
                                                            T* __restrict__ out, int Hq,
                                                            int nsplit, int last_slot) {
  constexpr int PW = decode_partial_words(D);
  constexpr int E = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int lane = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), last_slot);
  const int n = min(L / DECODE_SPLIT + 1, nsplit);
  const float* p = part + (int64_t)bh * nsplit * PW;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, p[(int64_t)s * PW]);
  float l = 0.f, a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = 0.f;
  for (int s = 0; s < n; ++s) {
    const float* ps = p + (int64_t)s * PW;
    const float f = fast_exp2(ps[0] - M);
    l = fmaf(f, ps[1], l);
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = fmaf(f, ps[4 + lane + 64 * e], a[e]);
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float o = a[e] * inv;
    if constexpr (sizeof(T) == 4) {
      out[(int64_t)bh * D + lane + 64 * e] = o;
    } else {
      const __bf16 h = (__bf16)o;
      out[(int64_t)bh * D + lane + 64 * e] = __builtin_bit_cast(uint16_t, h);
    }
  }
}

template <typename T, int D, int G, bool PAGED>
hipError_t decode_t(const void* q, const void* k_new, const void* v_new, void* out, int B,
                    int Hkv, const int32_t* seq_lens, int nsplit, const CacheArgs& c,
                    float* partials, const RopeFreq& fr, float scale, hipStream_t st,
                    const TimedLaunch& tl) {
  const float qk_scale = scale * 1.4426950408889634f;  // log2(e): softmax in base 2
  hipExtLaunchKernelGGL((decode_split_kernel<T, D, G, PAGED>), dim3(nsplit, Hkv, B),
                        dim3(kThreads), 0, st, tl.start, tl.stop, 0,
                        static_cast<const T*>(q), static_cast<const T*>(k_new),
                        static_cast<const T*>(v_new), seq_lens, c, partials, Hkv, nsplit, fr,
                        qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int last = PAGED ? c.mbps * 16 - 1 : c.max_seq - 1;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(B * Hkv * G), dim3(64), 0, st,
                     partials, seq_lens, static_cast<T*>(out), Hkv * G, nsplit, last);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t decode_paged(bool paged, const void* q, const void* kn, const void* vn, void* out,
                        int B, int Hkv, const int32_t* sl, int nsplit, const CacheArgs& c,
                        float* part, const RopeFreq& fr, float scale, hipStream_t st,
                        const TimedLaunch& tl) {
  return paged ? decode_t<T, D, G, true>(q, kn, vn, out, B, Hkv, sl, nsplit, c, part, fr, scale,
                                         st, tl)
               : decode_t<T, D, G, false>(q, kn, vn, out, B, Hkv, sl, nsplit, c, part, fr,
                                          scale, st, tl);
}

template <typename T, int D>
hipError_t decode_group(int group, bool paged, const void* q, const void* kn, const void* vn,
                        void* out, int B, int Hkv, const int32_t* sl, int nsplit,
                        const CacheArgs& c, float* part, const RopeFreq& fr, float scale,
                        hipStream_t st, const TimedLaunch& tl) {
  switch (group) {
    case 1: return decode_paged<T, D, 1>(paged, q, kn, vn, out, B, Hkv, sl, nsplit, c, part, fr, scale, st, tl);
    case 2: return decode_paged<T, D, 2>(paged, q, kn, vn, out, B, Hkv, sl, nsplit, c, part, fr, scale, st, tl);
    case 4: return decode_paged<T, D, 4>(paged, q, kn, vn, out, B, Hkv, sl, nsplit, c, part, fr, scale, st, tl);
    case 8: return decode_paged<T, D, 8>(paged, q, kn, vn, out, B, Hkv, sl, nsplit, c, part, fr, scale, st, tl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(Dtype dt, int D, int group, bool paged, const void* q,
                         const void* k_new, const void* v_new, void* out, int B, int Hq,
                         int Hkv, const int32_t* seq_lens, int nsplit, const CacheArgs& c,
                         float* partials, const RopeFreq& fr, float scale, hipStream_t s,
                         const TimedLaunch& tl) {
  (void)Hq;
  if (dt == F32)
    return D == 64 ? decode_group<float, 64>(group, paged, q, k_new, v_new, out, B, Hkv, seq_lens,
                                             nsplit, c, partials, fr, scale, s, tl)
                   : decode_group<float, 128>(group, paged, q, k_new, v_new, out, B, Hkv,
                                              seq_lens, nsplit, c, partials, fr, scale, s, tl);
  return D == 64 ? decode_group<bf16_t, 64>(group, paged, q, k_new, v_new, out, B, Hkv, seq_lens,
                                            nsplit, c, partials, fr, scale, s, tl)
                 : decode_group<bf16_t, 128>(group, paged, q, k_new, v_new, out, B, Hkv,
                                             seq_lens, nsplit, c, partials, fr, scale, s, tl);
}

}  // namespace car
