// Pieces shared by the decode kernels over native (bf16 / fp32) and INT8
// caches: the lazy-rescale threshold of the online softmax and the kernel
// that merges the per-split partials of a sequence ([Scratch]
// "从零手搓AI推理引擎" §3.4: running maxima and sums combined by the
// log-sum-exp rule).
#pragma once

#include "common.hpp"

namespace car {

namespace {

// Largest exp2 argument allowed before the running maximum is moved: weights
// stay at most 2^8, so the fp32 sums cannot overflow.
constexpr float kRescaleLog2 = 8.f;

// One wave per (sequence, query head): merge the partials of the splits that
// hold tokens 0..L (log-sum-exp rule) and write the normalised output.  The
// splits are taken 8 at a time with a running maximum, so that every load of
// a group (each split's maximum, sum and the lane's accumulators) is issued
// at once: one memory round trip per group instead of a pass for the maxima
// before the accumulators.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ seq_lens,
                                                            T* __restrict__ out, int Hq,
                                                            int nsplit, int split_tokens,
                                                            int last_slot) {
  constexpr int PW = decode_partial_words(D);
  constexpr int E = D / 64;
  constexpr int U = 8;  // splits per group
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int lane = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), last_slot);
  const int n = min(L / split_tokens + 1, nsplit);  // >= 1; every split holds a token
  const float* p = part + (int64_t)bh * nsplit * PW;

  float M = -INFINITY, l = 0.f, a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = 0.f;
  for (int s = 0; s < n; s += U) {
    float w[U], lw[U], v[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // splits past n read split n - 1 and weigh nothing
      const float* ps = p + (int64_t)min(s + u, n - 1) * PW;
      w[u] = s + u < n ? ps[0] : -INFINITY;
      lw[u] = ps[1];
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = ps[4 + lane + 64 * e];
    }
    float m_new = M;
#pragma unroll
    for (int u = 0; u < U; ++u) m_new = fmaxf(m_new, w[u]);  // finite: split s holds a token
    const float r = fast_exp2(M - m_new);  // 0 on the first group
    l *= r;
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] *= r;
    M = m_new;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = fast_exp2(w[u] - M);
      l = fmaf(f, lw[u], l);
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = fmaf(f, v[u][e], a[e]);
    }
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

}  // namespace

}  // namespace car
