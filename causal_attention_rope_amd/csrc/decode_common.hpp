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
// hold tokens 0..L (log-sum-exp rule) and write the normalised output.  Lane s
// reads split s's maximum and sum; the accumulators are read split by split,
// 4 splits at a time.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ seq_lens,
                                                            T* __restrict__ out, int Hq,
                                                            int nsplit, int split_tokens,
                                                            int last_slot) {
  constexpr int PW = decode_partial_words(D);
  constexpr int E = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int lane = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), last_slot);
  const int n = min(L / split_tokens + 1, nsplit);
  const float* p = part + (int64_t)bh * nsplit * PW;

  // max and weighted sum over splits, 64 splits per pass
  float M = -INFINITY;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, p[(int64_t)s * PW]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float l = 0.f;
  for (int s = lane; s < n; s += 64) l += fast_exp2(p[(int64_t)s * PW] - M) * p[(int64_t)s * PW + 1];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);

  float a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = 0.f;
  int s = 0;
  for (; s + 4 <= n; s += 4) {
    float w[4], v[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* ps = p + (int64_t)(s + u) * PW;
      w[u] = ps[0];
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = ps[4 + lane + 64 * e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float f = fast_exp2(w[u] - M);
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = fmaf(f, v[u][e], a[e]);
    }
  }
  for (; s < n; ++s) {
    const float* ps = p + (int64_t)s * PW;
    const float f = fast_exp2(ps[0] - M);
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

}  // namespace

}  // namespace car
