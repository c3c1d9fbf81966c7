// Prefill attention: causal softmax(scale * Q' K'^T) V over a whole prompt,
// as a tiled online softmax that never stores the S x S score matrix.
//
// What is computed: scaled dot-product attention with the upper triangle
// masked ([Guide] "手写LLM推理引擎：从黑盒到白盒的底层实现指南" §2.3, §5.1;
// [Scratch] "从零手搓AI推理引擎" §3.1, §3.3), Q rotated by RoPE at its
// position ([Intuition] "手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉"
// §4), evaluated block by block with a running maximum m and running sum l
// per query row that rescale the partial output whenever m grows ([Scratch]
// §3.4).  Keys arrive already rotated (one pass over K before this kernel).
//
// Two kernels:
//  * fp32: one thread per query row, key tiles staged in LDS; plain fp32
//    arithmetic for the 1e-4 accuracy of fp32 inputs.
//  * bf16: MFMA 32x32x16 bf16 with fp32 accumulation.  A workgroup owns 128
//    query rows (4 waves x 32) and walks key tiles of 64 (D = 128) or 128
//    (D = 64) keys up to the diagonal.  Each wave computes S^T = K Q^T so that
//    a lane holds one query's scores in its accumulator registers: the row
//    maximum and sum need only in-lane work plus one exchange with lane^32,
//    and the probabilities already sit in the operand layout of the second
//    product O^T = V^T P^T.  K tiles are staged row-major in LDS, V tiles
//    transposed (keys contiguous per head-dim row) with an XOR swizzle that
//    keeps both the transposing stores and the operand loads free of bank
//    conflicts; tiles are double-buffered so the next tile's global loads
//    overlap the current tile's MFMA work.  Workgroups of one head go to one
//    XCD (shared L2) and the longest (latest) query tiles start first.
#include <math.h>

#include "common.hpp"

namespace car {

namespace {

// ------------------------------------------------------------------ fp32 ---
constexpr int F32_ROWS = 64;  // query rows per workgroup (one per thread)
constexpr int F32_KT = 32;    // keys per LDS tile

template <int D>
__global__ __launch_bounds__(F32_ROWS) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kr, const float* __restrict__ v,
    float* __restrict__ out, const int32_t* __restrict__ positions, int Hq, int Hkv, int S,
    RopeFreq fr, float qk_scale) {
  __shared__ float4 sk[F32_KT][D / 4];
  __shared__ float4 sv[F32_KT][D / 4];
  const int b = blockIdx.z, hq = blockIdx.y;
  const int hk = hq / (Hq / Hkv);
  const int i0 = blockIdx.x * F32_ROWS;
  const int i = i0 + threadIdx.x;
  const int ic = min(i, S - 1);

  float qv[D];
  const float* qrow = q + (((int64_t)b * Hq + hq) * S + ic) * D;
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    float f[4];
    load16<float>(qrow + d, f);
    rope_rotate_regs<4>(f, positions[(int64_t)b * S + ic], d / 2, fr);
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[d + e] = f[e] * qk_scale;
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* kb = kr + ((int64_t)b * Hkv + hk) * S * D;
  const float* vb = v + ((int64_t)b * Hkv + hk) * S * D;
  const int jlast = min(S - 1, i0 + F32_ROWS - 1);
  for (int j0 = 0; j0 <= jlast; j0 += F32_KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < F32_KT * D / 4; idx += F32_ROWS) {
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      const int64_t row = min(j0 + r, S - 1);
      sk[r][c4] = *reinterpret_cast<const float4*>(kb + row * D + c4 * 4);
      sv[r][c4] = *reinterpret_cast<const float4*>(vb + row * D + c4 * 4);
    }
    __syncthreads();
    float s[F32_KT];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < F32_KT; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < D / 4; ++c4) {
        const float4 kk = sk[r][c4];
        dot = fmaf(qv[4 * c4], kk.x, dot);
        dot = fmaf(qv[4 * c4 + 1], kk.y, dot);
        dot = fmaf(qv[4 * c4 + 2], kk.z, dot);
        dot = fmaf(qv[4 * c4 + 3], kk.w, dot);
      }
      s[r] = (j0 + r <= ic) ? dot : -INFINITY;
      tmax = fmaxf(tmax, s[r]);
    }
    const float m_new = fmaxf(m, tmax);  // finite: key 0 is visible to every row
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int r = 0; r < F32_KT; ++r) {
      const float p = fast_exp2(s[r] - m_new);
      l += p;
#pragma unroll
      for (int c4 = 0; c4 < D / 4; ++c4) {
        const float4 vv = sv[r][c4];
        acc[4 * c4] = fmaf(p, vv.x, acc[4 * c4]);
        acc[4 * c4 + 1] = fmaf(p, vv.y, acc[4 * c4 + 1]);
        acc[4 * c4 + 2] = fmaf(p, vv.z, acc[4 * c4 + 2]);
        acc[4 * c4 + 3] = fmaf(p, vv.w, acc[4 * c4 + 3]);
      }
    }
    m = m_new;
  }
  if (i < S) {
    const float inv = 1.f / l;
    float* orow = out + (((int64_t)b * Hq + hq) * S + i) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      float f[4] = {acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
      store16<float>(orow + d, f);
    }
  }
}

// ------------------------------------------------------------ bf16 MFMA ---
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int D, int WAVES>
struct Tile {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;          // query rows per workgroup
  static constexpr int BN = D == 128 ? 64 : 128; // keys per tile
  static constexpr int KSTR = D + 8;             // K row stride in LDS (elements)
  static constexpr int VSTR = BN + 4;            // V^T row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CH = BN * D / (THREADS * 8);  // 16-byte chunks per thread per tensor
  static constexpr int NKB = BN / 32;            // 32-key blocks of S^T
  static constexpr int NDB = D / 32;             // 32-wide head-dim blocks of O^T
  static constexpr int QKS = D / 16;             // k-steps of Q K^T
  static constexpr int PKS = BN / 16;            // k-steps of P V
  static_assert(CH == 2 || CH == 4, "V is transposed 2 or 4 keys per thread");
};

// Physical key column of logical key `key` in V^T row d (XOR swizzle in
// groups of 4 keys, selected by d / 16).
__device__ __forceinline__ int vt_col(int d, int key) { return key ^ (((d >> 4) & 7) << 2); }

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // (a.lo16, b.lo16)
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a.hi16, b.hi16)
}

__device__ __forceinline__ uint32_t word_of(const u32x4_t& u, int w) { return u[w]; }

// Global -> register staging of the K and V tiles that start at key j0
// (rows past the sequence end are clamped to the last row; they are masked).
template <int D, int WAVES, int CH>
__device__ __forceinline__ void load_tile(u32x4_t (&kreg)[CH], u32x4_t (&vreg)[CH],
                                          const bf16_t* kbase, const bf16_t* vbase, int j0,
                                          int S, int tid) {
  using C = Tile<D, WAVES>;
  const int v_dc = tid % (D / 8), v_kg = tid / (D / 8);
  static_for<0, CH>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const int ch = tid + p * C::THREADS;
    const int key = ch / (D / 8), dc = ch % (D / 8);
    const int64_t krow = min(j0 + key, S - 1);
    kreg[p] = *reinterpret_cast<const u32x4_t*>(kbase + krow * D + dc * 8);
    const int64_t vrow = min(j0 + v_kg * CH + p, S - 1);
    vreg[p] = *reinterpret_cast<const u32x4_t*>(vbase + vrow * D + v_dc * 8);
  });
}

// Register -> LDS: K row-major, V transposed into V^T[d][key] (swizzled).
template <int D, int WAVES, int CH>
__device__ __forceinline__ void store_tile(const u32x4_t (&kreg)[CH], const u32x4_t (&vreg)[CH],
                                           bf16_t* ks, int tid) {
  using C = Tile<D, WAVES>;
  bf16_t* vs = ks + C::K_ELEMS;
  static_for<0, CH>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const int ch = tid + p * C::THREADS;
    const int key = ch / (D / 8), dc = ch % (D / 8);
    *reinterpret_cast<u32x4_t*>(ks + key * C::KSTR + dc * 8) = kreg[p];
  });
  const int v_dc = tid % (D / 8), v_kg = tid / (D / 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const int d = v_dc * 8 + e;
    bf16_t* dst = vs + d * C::VSTR + vt_col(d, v_kg * C::CH);
    if constexpr (C::CH == 4) {
      u32x2_t t;
      t[0] = (e & 1) ? perm_hi(word_of(vreg[0], w), word_of(vreg[1], w))
                     : perm_lo(word_of(vreg[0], w), word_of(vreg[1], w));
      t[1] = (e & 1) ? perm_hi(word_of(vreg[2], w), word_of(vreg[3], w))
                     : perm_lo(word_of(vreg[2], w), word_of(vreg[3], w));
      *reinterpret_cast<u32x2_t*>(dst) = t;
    } else {
      *reinterpret_cast<uint32_t*>(dst) =
          (e & 1) ? perm_hi(word_of(vreg[0], w), word_of(vreg[1], w))
                  : perm_lo(word_of(vreg[0], w), word_of(vreg[1], w));
    }
  }
}

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void prefill_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kr, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ out, const int32_t* __restrict__ positions, int Hq, int Hkv, int S,
    int nqt, RopeFreq fr, float sm_scale_log2) {
  using C = Tile<D, WAVES>;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * C::STAGE];

  // ---- work assignment: one head per XCD at a time, longest tiles first ----
  const int nbh = gridDim.x / nqt;
  const int bid = blockIdx.x;
  int bh, qt;
  if ((nbh & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    bh = (slot / nqt) * 8 + xcd;
    qt = nqt - 1 - slot % nqt;
  } else {
    bh = bid % nbh;
    qt = nqt - 1 - bid / nbh;
  }
  const int b = bh / Hq, hq = bh % Hq;
  const int hk = hq / (Hq / Hkv);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int l32 = lane & 31, g = lane >> 5;
  const int q0 = qt * C::BM;
  const int qw = q0 + wave * 32;             // first query row of this wave
  const int qrow = qw + l32;                 // this lane's query row
  const int qrc = min(qrow, S - 1);

  // ---- Q fragments (B operand of S^T = K Q^T), rotated, bf16 ----
  bf16x8_t qf[C::QKS];
  {
    const bf16_t* qp = q + ((int64_t)bh * S + qrc) * D;
    const int pos = positions[(int64_t)b * S + qrc];
#pragma unroll
    for (int ks = 0; ks < C::QKS; ++ks) {
      const int d0 = ks * 16 + g * 8;
      float f[8];
      load16<bf16_t>(qp + d0, f);
      rope_rotate_regs<8>(f, pos, d0 / 2, fr);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)f[e];
    }
  }

  const bf16_t* kbase = kr + ((int64_t)b * Hkv + hk) * S * D;
  const bf16_t* vbase = v + ((int64_t)b * Hkv + hk) * S * D;

  // ---- global -> register staging of one K tile and one V tile ----
  // K: chunk ch = tid + p*THREADS is (key ch / (D/8), dims (ch % (D/8))*8..+8).
  // V: thread holds keys (tid / (D/8))*CH .. +CH of dims (tid % (D/8))*8 .. +8,
  // transposed on the way into LDS.
  u32x4_t kreg[C::CH], vreg[C::CH];
  f32x16_t oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int q_end = min(q0 + C::BM, S);  // exclusive
  const int ntiles = (q_end + C::BN - 1) / C::BN;

  load_tile<D, WAVES>(kreg, vreg, kbase, vbase, 0, S, tid);
  store_tile<D, WAVES>(kreg, vreg, smem, tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * C::BN;
    if (t + 1 < ntiles) load_tile<D, WAVES>(kreg, vreg, kbase, vbase, j0 + C::BN, S, tid);

    if (j0 <= qw + 31) {  // some key of this tile is visible to this wave
      const bf16_t* ks = smem + (t & 1) * C::STAGE;
      const bf16_t* vs = ks + C::K_ELEMS;

      // S^T = K Q^T : lane holds keys kb*32 + 8*(r/4) + 4*g + r%4 of query qrow
      f32x16_t sacc[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < C::QKS; ++kk) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              ks + (kb * 32 + l32) * C::KSTR + kk * 16 + g * 8);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kb], 0, 0, 0);
        }
      }

      // causal mask, only where the tile reaches past this wave's first row
      if (j0 + C::BN - 1 > qw) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > qrow) sacc[kb][r] = -INFINITY;
          }
      }

      // online softmax update (base 2, scale folded into the exponent)
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float mc = m_new * sm_scale_log2;
      const float alpha = fast_exp2(m_run * sm_scale_log2 - mc);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

      bf16x8_t pf[C::PKS];
#pragma unroll
      for (int kk = 0; kk < C::PKS; ++kk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(fmaf(sacc[kk >> 1][8 * (kk & 1) + i], sm_scale_log2, -mc));
          l_run += p;
          pf[kk][i] = (__bf16)p;
        }
      }

      // O^T += V^T P^T : A operand = V^T rows d, keys {4g..4g+3, 8+4g..8+4g+3}
#pragma unroll
      for (int kk = 0; kk < C::PKS; ++kk) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int d = db * 32 + l32;
          const int key = kk * 16 + 4 * g;
          const u32x2_t lo =
              *reinterpret_cast<const u32x2_t*>(vs + d * C::VSTR + vt_col(d, key));
          const u32x2_t hi =
              *reinterpret_cast<const u32x2_t*>(vs + d * C::VSTR + vt_col(d, key + 8));
          const u32x4_t u = {lo[0], lo[1], hi[0], hi[1]};
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], oacc[db], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) store_tile<D, WAVES>(kreg, vreg, smem + ((t + 1) & 1) * C::STAGE, tid);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query qrow, dims db*32+8*(r/4)+4g+r%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < S) {
    const float inv = 1.f / l_tot;
    bf16_t* op = out + ((int64_t)bh * S + qrow) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 u;
        u.x = pack_bf16x2(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv);
        u.y = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * r4 + 4 * g) = u;
      }
  }
}

template <int D>
hipError_t prefill_f32_t(const void* q, const void* k_rot, const void* v, void* out, int B,
                         int Hq, int Hkv, int S, const int32_t* positions, const RopeFreq& fr,
                         float scale, hipStream_t st, const TimedLaunch& tl) {
  const dim3 grid((S + F32_ROWS - 1) / F32_ROWS, Hq, B);
  hipExtLaunchKernelGGL((prefill_f32_kernel<D>), grid, dim3(F32_ROWS), 0, st, tl.start, tl.stop,
                        0, static_cast<const float*>(q), static_cast<const float*>(k_rot),
                        static_cast<const float*>(v), static_cast<float*>(out), positions, Hq,
                        Hkv, S, fr, scale * 1.4426950408889634f);
  return hipGetLastError();
}

template <int D, int WAVES>
hipError_t prefill_bf16_launch(const void* q, const void* k_rot, const void* v, void* out,
                               int B, int Hq, int Hkv, int S, const int32_t* positions,
                               const RopeFreq& fr, float scale, hipStream_t st,
                               const TimedLaunch& tl) {
  using C = Tile<D, WAVES>;
  const int nqt = (S + C::BM - 1) / C::BM;
  hipExtLaunchKernelGGL((prefill_bf16_kernel<D, WAVES>), dim3(nqt * B * Hq), dim3(C::THREADS),
                        0, st, tl.start, tl.stop, 0, static_cast<const bf16_t*>(q),
                        static_cast<const bf16_t*>(k_rot), static_cast<const bf16_t*>(v),
                        static_cast<bf16_t*>(out), positions, Hq, Hkv, S, nqt, fr,
                        scale * 1.4426950408889634f);
  return hipGetLastError();
}

// 8-wave workgroups (256 query rows) when they alone fill the 256 CUs;
// otherwise 4-wave workgroups (128 rows) for more parallelism.
template <int D>
hipError_t prefill_bf16_t(const void* q, const void* k_rot, const void* v, void* out, int B,
                          int Hq, int Hkv, int S, const int32_t* positions, const RopeFreq& fr,
                          float scale, hipStream_t st, const TimedLaunch& tl) {
  const int64_t big = (int64_t)((S + 255) / 256) * B * Hq;
  if (big >= 256)
    return prefill_bf16_launch<D, 8>(q, k_rot, v, out, B, Hq, Hkv, S, positions, fr, scale, st,
                                     tl);
  return prefill_bf16_launch<D, 4>(q, k_rot, v, out, B, Hq, Hkv, S, positions, fr, scale, st,
                                   tl);
}

}  // namespace

hipError_t launch_prefill_attention(Dtype dt, int D, const void* q, const void* k_rot,
                                    const void* v, void* out, int B, int Hq, int Hkv, int S,
                                    const int32_t* positions, const RopeFreq& fr, float scale,
                                    hipStream_t s, const TimedLaunch& tl) {
  if (dt == F32)
    return D == 64 ? prefill_f32_t<64>(q, k_rot, v, out, B, Hq, Hkv, S, positions, fr, scale, s, tl)
                   : prefill_f32_t<128>(q, k_rot, v, out, B, Hq, Hkv, S, positions, fr, scale, s,
                                        tl);
  return D == 64 ? prefill_bf16_t<64>(q, k_rot, v, out, B, Hq, Hkv, S, positions, fr, scale, s, tl)
                 : prefill_bf16_t<128>(q, k_rot, v, out, B, Hq, Hkv, S, positions, fr, scale, s,
                                       tl);
}

}  // namespace car
