// Decode attention over an INT8 KV cache.
//
// What is computed: the decode step of [Guide] ("手写LLM推理引擎：从黑盒到白盒的底层实现指南")
// §2.5 and [Scratch] ("从零手搓AI推理引擎") §3.2-§3.3 -- q and k_new rotated at
// position L, the new key and value appended at cache index L, attention over
// indices 0..L -- with a cache whose rows are int8 codes and whose value is
// code * scale, one fp32 scale per (KV head, channel) ([Intuition]
// ("手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉") §2: the cache
// compressed from 16-bit floats to INT8; [Scratch] §2.2 and §5.3: per-channel
// absmax/127 scales, divide and round to store, multiply back to read).  The
// new key and value are quantized when appended and read in that form, like
// every other cached token.
//
// How it maps to MI355X.  The step streams every cached row once, now at one
// byte per element, so it stays bound by HBM bandwidth at half the bytes of a
// bf16 cache.  Because the scales are per channel they factor out of both
// contractions: q . (code_k * s_k) = (q * s_k) . code_k, folded into the query
// once per workgroup, and sum_j p_j (code_v * s_v) = s_v * sum_j p_j code_v,
// applied to the partial result once.  The inner loop is then one
// int8 -> fp32 conversion per element (a sign-extended byte select folds into
// the conversion instruction) and one fp32 FMA per element and query head;
// no dequantized copy of a row is ever formed.
//
// With several query heads per KV head (GQA) and bf16 inputs that FMA work
// grows G-fold per byte and would bound the kernel, so that case runs in
// decode_i8_mfma_kernel (below) with both contractions on the matrix cores.
// There a code c becomes the fp16 value 1152 + c with one byte permute per
// pair: the byte c XOR 0x80 = c + 128 is placed under the exponent byte 0x64
// (fp16 1024 + m for an 8-bit m), which is exact.  The constant 1152 adds the
// same amount to every score of a head (1152 times the sum of its query),
// which the softmax ignores; in P V it adds 1152 * l, removed once at the
// end.  Each head's query is scaled by a power of two so that its largest
// element lies in [0.5, 1) before rounding to fp16 (11 significant bits,
// against bf16's 8 in the native path), and the score is scaled back exactly.
//
// In decode_i8_split_kernel (one query head per KV head, or fp32 inputs)
// lanes hold E = 16 codes of a row (one 16-byte load), or 8 with eight query
// heads (registers for G query rows and accumulators), so LPR = D/E lanes
// cover a row and a load instruction moves 64/LPR rows.  The work split
// (splits of the sequence per workgroup, grid order, the online softmax with
// a lazy rescale, merging across rows, waves and workgroups) is that of the
// decode over a native cache.
#include <math.h>

#include "decode_common.hpp"

namespace car {

namespace {

template <int G>
constexpr int i8_waves() { return G > 1 ? 8 : 4; }

// Row steps per round: four (8 KB of K and V in flight per wave at D = 128)
// for bf16 with one query head and adjacent-pair RoPE, where the registers
// allow it; two otherwise (four would spill there).
template <typename T, int G, bool HALF>
constexpr int i8_round_steps() { return sizeof(T) == 2 && G == 1 && !HALF ? 4 : 2; }

template <int D, int G, int SPLIT, int RMAX>
struct I8Geom {
  static constexpr int WAVES = i8_waves<G>();
  static constexpr int TPW = SPLIT / WAVES;  // tokens per wave
  static constexpr int E = G >= 8 ? 8 : 16;  // codes per lane per row
  static constexpr int LPR = D / E;          // lanes per cache row
  static constexpr int NG = 64 / LPR;        // rows per load instruction
  static constexpr int STEPS = TPW / NG;
  static constexpr int R = STEPS < RMAX ? STEPS : RMAX;  // row steps per round
  static constexpr int ROUNDS = STEPS / R;
  static constexpr int W = E / 4;  // 32-bit words per lane per row
  static_assert(SPLIT % DECODE_SPLIT == 0 && TPW % 64 == 0, "whole 16-token blocks per wave");
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "lanes per row");
  static_assert(NG <= 16 && 16 % NG == 0, "a row step stays inside one 16-token block");
  static_assert(R % 2 == 0 && ROUNDS * R == STEPS, "rounds must tile the wave's tokens");
  static_assert(ROUNDS == 1 || ROUNDS % 2 == 0, "rounds are consumed in pairs");
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

// Two floats to packed fp16 (round to nearest even; one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2_t r;
  r.x = (_Float16)a;
  r.y = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}

constexpr float kCodeBias = 1152.f;          // fp16 value of code c is kCodeBias + c
constexpr uint32_t kOnePairF16 = 0x3C003C00u;  // (1.0, 1.0) in fp16

// Codes 2i, 2i+1 of a word as the fp16 pair (1152 + c, 1152 + c'): the bytes
// c ^ 0x80 under the exponent byte 0x64.
__device__ __forceinline__ uint32_t codes_f16_lo(uint32_t x80) {
  return __builtin_amdgcn_perm(0x64646464u, x80, 0x04010400u);
}
__device__ __forceinline__ uint32_t codes_f16_hi(uint32_t x80) {
  return __builtin_amdgcn_perm(0x64646464u, x80, 0x04030402u);
}
// Code j of row a and code j of row b as one fp16 pair (1152 + a_j, 1152 + b_j).
template <int J>
__device__ __forceinline__ uint32_t codes_f16_rows(uint32_t a, uint32_t b) {
  // byte 0 = a.byte J, byte 2 = b.byte J, bytes 1 and 3 zero; then the XOR
  // flips the code bytes to c + 128 and writes the exponent bytes
  return __builtin_amdgcn_perm(b, a, 0x0C000C00u | ((4u + J) << 16) | (uint32_t)J) ^ 0x64806480u;
}

template <int W> struct ChunkOf;
template <> struct ChunkOf<2> { typedef uint32_t type __attribute__((ext_vector_type(2))); };
template <> struct ChunkOf<4> { typedef uint32_t type __attribute__((ext_vector_type(4))); };

// Tokens per workgroup: 256 with one query head per KV head, as for the
// native cache; 2048 with several.  A code row is half a native row, so a
// split carries half the bytes per token and twice the tokens share each
// workgroup's setup and merge (measured on the GQA shapes: contiguous 42 ->
// 39 us, paged about 1% faster; 1024 and 4096 tokens slower).
template <int G>
constexpr int i8_split_tokens() { return G == 1 ? DECODE_SPLIT : 8 * DECODE_SPLIT; }

template <typename T, int D, int G, bool PAGED, int SPLIT, bool HALF>
__global__ __launch_bounds__(64 * i8_waves<G>())
__attribute__((amdgpu_waves_per_eu(G == 1 ? 4 : 2))) void decode_i8_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ seq_lens, CacheArgs c, float* __restrict__ part, int Hkv,
    int nsplit, RopeFreq fr, float qk_scale) {
  using Gm = I8Geom<D, G, SPLIT, i8_round_steps<T, G, HALF>()>;
  using Chunk = typename ChunkOf<Gm::W>::type;
  constexpr int E = Gm::E, W = Gm::W, LPR = Gm::LPR, NG = Gm::NG, R = Gm::R,
                ROUNDS = Gm::ROUNDS, TPW = Gm::TPW;
  constexpr int NT = Vec16<T>::N;  // input elements per 16-byte load
  constexpr int SUB = E / NT;      // input loads per lane chunk
  constexpr int PW = decode_partial_words(D);
  constexpr int kWaves = Gm::WAVES, kThreads = 64 * kWaves;
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_ml[kWaves][G][2];

  // Grid order as for the native cache: (sequence, KV head) fastest, splits
  // aligned to the last row so that the short last splits run last.
  const int hk = blockIdx.x % Hkv, b = blockIdx.x / Hkv;
  const int Hq = Hkv * G;
  const int L_in = seq_lens[b];  // outside the cache: clamped reads, no store
  const int L = min(max(L_in, 0), cache_last_slot<PAGED>(c));
  const bool store_new = L_in == L;
  const int nsb = min(L / SPLIT + 1, nsplit);
  const int split = (int)blockIdx.y - (nsplit - nsb);
  if (split < 0) return;  // uniform over the workgroup
  const int t0 = split * SPLIT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane / LPR;             // row of the step
  const int col = (lane % LPR) * E;       // first channel of the lane's codes
  const int tw = t0 + wave * TPW;         // first token of this wave
  const float* ks = c.k_scale + (int64_t)hk * D + col;

  // Query heads rotated at L, times the softmax scale (base 2) and the key
  // scale of each channel.  One set of angles serves all heads and k_new.
  RopeChunk<NT> rope[SUB];
#pragma unroll
  for (int j = 0; j < SUB; ++j) rope[j] = rope_prepare<NT, HALF>(L, col + j * NT, D, fr);
  float kscale[E];
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const float4 s4 = *reinterpret_cast<const float4*>(ks + e);
    kscale[e] = s4.x; kscale[e + 1] = s4.y; kscale[e + 2] = s4.z; kscale[e + 3] = s4.w;
  }
  float qf[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const T* qrow = q + ((int64_t)b * Hq + hk * G + g) * D;
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      float f[NT];
      load16<T>(qrow + col + j * NT, f);
      rope_apply_prepared<T, NT, HALF>(f, qrow, D, rope[j], fr);
#pragma unroll
      for (int e = 0; e < NT; ++e) qf[g][j * NT + e] = f[e] * qk_scale * kscale[j * NT + e];
    }
  }
  // The new token (index L): codes of the rotated key and of the value,
  // stored by the split that holds L and used from registers for token L.
  int8_t* const Kc = static_cast<int8_t*>(c.k);
  int8_t* const Vc = static_cast<int8_t*>(c.v);
  Chunk kn, vn;
#pragma unroll
  for (int w = 0; w < W; ++w) kn[w] = vn[w] = 0u;
  if (L < t0 + SPLIT) {
    const int64_t src = ((int64_t)b * Hkv + hk) * D;
    const float* vs = c.v_scale + (int64_t)hk * D + col;
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      float f[NT], g[NT];
      load16<T>(k_new + src + col + j * NT, f);
      rope_apply_prepared<T, NT, HALF>(f, k_new + src, D, rope[j], fr);
      load16<T>(v_new + src + col + j * NT, g);
      uint32_t kw[NT / 4], vw[NT / 4];
      int8_codes<NT>(f, ks + j * NT, kw);
      int8_codes<NT>(g, vs + j * NT, vw);
#pragma unroll
      for (int w = 0; w < NT / 4; ++w) {
        kn[j * NT / 4 + w] = kw[w];
        vn[j * NT / 4 + w] = vw[w];
      }
    }
    if (wave == 0 && grp == 0 && store_new) {
      const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, L) * D + col;
      *reinterpret_cast<Chunk*>(Kc + dst) = kn;
      *reinterpret_cast<Chunk*>(Vc + dst) = vn;
    }
  }

  float m_run[G], l_run[G], acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  if (tw <= L) {  // uniform per wave: this wave holds at least one token
    constexpr int NBLK = TPW / 16;
    static_assert(NBLK <= 64, "one block id per lane");
    int myblk = 0;
    if constexpr (PAGED) {
      const int32_t* trow = c.table + (int64_t)b * c.mbps;
      if (lane < NBLK)
        myblk = min(max(trow[min((tw >> 4) + lane, L >> 4)], 0), c.num_blocks - 1);
    }

    Chunk kb[2][R], vb[2][R];
    // Loads of round r into register buffer BUF.  Rows at or past L are only
    // ever replaced (consume), so they just stay inside the cache: paged
    // block ids are clamped to the sequence's last block, contiguous rows to L.
    const int64_t cbase = PAGED ? 0 : ((int64_t)b * Hkv + hk) * c.max_seq + tw;
    auto issue = [&](int r, auto BUF) {
      constexpr int buf = decltype(BUF)::value;
#pragma unroll
      for (int st = 0; st < R; ++st) {
        const int x = r * R + st;
        int64_t row0;
        int lrow = grp;
        if constexpr (PAGED) {
          const int blk = __builtin_amdgcn_readlane(myblk, (x * NG) >> 4);  // uniform index
          row0 = (((int64_t)blk * Hkv + hk) << 4) + ((x * NG) & 15);
        } else {
          row0 = cbase + x * NG;
          lrow = min(grp, L - tw - x * NG);
        }
        const int64_t off = row0 * D + lrow * D + col;
        // streamed once: non-temporal loads keep the rows out of the caches
        kb[buf][st] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(Kc + off));
        vb[buf][st] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(Vc + off));
      }
    };

    auto consume = [&](int r, auto BUF) {
      constexpr int buf = decltype(BUF)::value;
      const bool full = tw + (r + 1) * R * NG - 1 < L;
      if (!full) {
        // the round reaches index L: token L from registers, later rows zeroed
#pragma unroll
        for (int st = 0; st < R; ++st) {
          const int t = tw + (r * R + st) * NG + grp;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            kb[buf][st][w] = t < L ? kb[buf][st][w] : kn[w];
            vb[buf][st][w] = t < L ? vb[buf][st][w] : (t == L ? vn[w] : 0u);
          }
        }
      }
      float sc[R][G];
#pragma unroll
      for (int st = 0; st < R; ++st) {
        const int t = tw + (r * R + st) * NG + grp;
        float kf[E];
#pragma unroll
        for (int e = 0; e < E; ++e) kf[e] = int8_elem(kb[buf][st][e >> 2], e & 3);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float p0 = 0.f, p1 = 0.f;  // two chains for latency
#pragma unroll
          for (int e = 0; e < E; e += 2) {
            p0 = fmaf(qf[g][e], kf[e], p0);
            p1 = fmaf(qf[g][e + 1], kf[e + 1], p1);
          }
          const float sv = group_sum<LPR>(p0 + p1);
          sc[st][g] = (full || t <= L) ? sv : -INFINITY;
        }
      }
      // Lazy rescale, as for the native cache: the reference maximum of a
      // head moves only when a score exceeds it by more than kRescaleLog2.
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = sc[0][g];
#pragma unroll
        for (int st = 1; st < R; ++st) mx = fmaxf(mx, sc[st][g]);
        if (__builtin_amdgcn_ballot_w64(mx - m_run[g] > kRescaleLog2) != 0) {  // uniform
          const float m_new = fmaxf(m_run[g], class_max<LPR>(mx));
          const float alpha = fast_exp2(m_run[g] - m_new);
          m_run[g] = m_new;
          l_run[g] *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
        }
      }
#pragma unroll
      for (int st = 0; st < R; ++st) {
        float vf[E];
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = int8_elem(vb[buf][st][e >> 2], e & 3);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = fast_exp2(sc[st][g] - m_run[g]);
          l_run[g] += p;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
      }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    // The steady-state loop issues its loads unconditionally, so that each
    // wait covers only the round being consumed; the last two rounds follow.
    issue(0, B0{});
    if constexpr (ROUNDS == 1) {
      consume(0, B0{});
    } else {
#pragma unroll 1
      for (int r = 0; r < ROUNDS - 2; r += 2) {
        issue(r + 1, B1{});
        consume(r, B0{});
        issue(r + 2, B0{});
        consume(r + 1, B1{});
      }
      issue(ROUNDS - 1, B1{});
      consume(ROUNDS - 2, B0{});
      consume(ROUNDS - 1, B1{});
    }
  }

  // Merge the rows of the wave (lanes that share the same channels).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = class_sum<LPR>(l_run[g]);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = class_sum<LPR>(acc[g][e]);
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_acc[wave][g][col + e] = acc[g][e];
      if (lane == 0) {
        sm_ml[wave][g][0] = m_run[g];
        sm_ml[wave][g][1] = l_run[g];
      }
    }
  }
  __syncthreads();

  // Merge the waves; the value scale of each channel is applied here, once
  // (after removing the fp16 code bias, 1152 * l).
  const float* vsc = c.v_scale + (int64_t)hk * D;
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
    dst[4 + d] = a * vsc[d];
    if (d == 0) {
      dst[0] = M;
      dst[1] = l;
    }
  }
}

// ---------------------------------------- several heads: the matrix cores ---
// With G = Hq/Hkv query heads (2..8) per KV head and bf16 inputs, both
// contractions of a 16-token block run on the matrix cores, so the ALU does
// only the byte-to-fp16 conversion (one v_perm per two codes) and the
// softmax of the block:
//   scores S^T[t][n] = sum_d (1152 + K[t][d]) Q[n][d]  v_mfma_f32_16x16x32_f16
//   values O[n][d]  += sum_t P[n][t] (1152 + V[t][d])   v_mfma_f32_16x16x16_f16
// (the fp16 forms of the codes as in the packed-dot path; the constant 1152
// shifts every score of a head equally and adds 1152 * l to O, removed once).
// A wave streams 16-token blocks (one paged block, 2 KB per tensor at
// D = 128).  Lane l holds row r = l % 16 of the block and, at D = 128, the
// 32 codes of dims 16*(l/16) + [0, 16) and 64 + 16*(l/16) + [0, 16) (two
// 16-byte loads, each instruction reading 64 contiguous bytes of every row),
// which is the A operand of the score MFMAs with the contraction index
// permuted the same way in Q.  The score accumulator then holds S^T[token
// 4*(l/16) + i][head l % 16], which is exactly the A operand (P, heads x
// tokens) of the value MFMAs.  Their B operand (tokens x dims) needs the
// value codes transposed: each wave writes its block's rows to LDS and reads
// back, for dims 8c .. 8c+7 (c = l % 16), the four tokens 4*(l/16) + e; MFMA
// j then takes dim 8c + j of each.  Lanes with l % 16 >= G carry zero
// queries and their results are ignored.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct I8MfmaGeom {
  static constexpr int WAVES = 8;
  static constexpr int SPLIT = 8 * DECODE_SPLIT;  // tokens per workgroup (as i8_split_tokens)
  static constexpr int TPW = SPLIT / WAVES;       // tokens per wave
  static constexpr int NBLK = TPW / 16;           // 16-token blocks per wave
  static constexpr int KS = D / 32;               // score MFMAs (32 dims each)
  static constexpr int NL = D / 64;               // 16-byte loads per lane per row
  static constexpr int NJ = D / 16;               // value MFMAs (16 dims each)
  static constexpr int LROW = D + 16;             // LDS row stride of a value block (bytes)
  static_assert(NBLK <= 64, "one block id per lane");
};

// Dim of element e (0..7) of score k-step s for a lane of group g4 = l / 16.
template <int D>
__device__ __forceinline__ int i8m_dim(int s, int g4, int e) {
  return 64 * (s >> 1) + 16 * g4 + 8 * (s & 1) + e;
}

// Eight codes (two words) as the fp16 values 1152 + c.
__device__ __forceinline__ f16x8_t codes8_f16(uint32_t w0, uint32_t w1) {
  const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
  const u32x4_t u = {codes_f16_lo(x0), codes_f16_hi(x0), codes_f16_lo(x1), codes_f16_hi(x1)};
  return __builtin_bit_cast(f16x8_t, u);
}

template <int D, int G, bool PAGED, bool HALF>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void
decode_i8_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_new,
                      const bf16_t* __restrict__ v_new, const int32_t* __restrict__ seq_lens,
                      CacheArgs c, float* __restrict__ part, int Hkv, int nsplit, RopeFreq fr,
                      float qk_scale) {
  using Gm = I8MfmaGeom<D>;
  constexpr int WAVES = Gm::WAVES, SPLIT = Gm::SPLIT, TPW = Gm::TPW, NBLK = Gm::NBLK;
  constexpr int KS = Gm::KS, NL = Gm::NL, NJ = Gm::NJ, LROW = Gm::LROW;
  constexpr int PW = decode_partial_words(D);
  __shared__ __attribute__((aligned(16))) uint8_t sk[WAVES][16 * LROW];
  __shared__ __attribute__((aligned(16))) uint8_t sv[WAVES][16 * LROW];
  __shared__ __attribute__((aligned(16))) uint8_t snew[2][D];  // the new token's K and V codes
  __shared__ float sm_acc[WAVES][G][D];
  __shared__ float sm_ml[WAVES][G][2];

  // grid order, splits and the new token as in decode_i8_split_kernel
  const int hk = blockIdx.x % Hkv, b = blockIdx.x / Hkv;
  const int Hq = Hkv * G;
  const int L_in = seq_lens[b];  // outside the cache: clamped reads, no store
  const int L = min(max(L_in, 0), cache_last_slot<PAGED>(c));
  const bool store_new = L_in == L;
  const int nsb = min(L / SPLIT + 1, nsplit);
  const int split = (int)blockIdx.y - (nsplit - nsb);
  if (split < 0) return;  // uniform over the workgroup
  const int t0 = split * SPLIT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int tw = t0 + wave * TPW;  // first token of this wave
  const float* ksc = c.k_scale + (int64_t)hk * D;
  const float* vsc = c.v_scale + (int64_t)hk * D;

  // Q^T as the B operand: lane (g4, n = r16) holds, for k-step s, head n's
  // rotated query at dims i8m_dim(s, g4, 0..7) times qk_scale and the key
  // scale of each dim, divided by 2^ex (the power of two that brings the
  // head's largest element into [0.5, 1)); zero for n >= G.
  f16x8_t qb[KS];
  float qs;
  {
    float f[KS][8];
    if (r16 < G) {
      const bf16_t* qrow = q + ((int64_t)b * Hq + hk * G + r16) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = i8m_dim<D>(s, g4, 0);
        load16<bf16_t>(qrow + col, f[s]);
        rope_rotate_chunk<bf16_t, 8, HALF>(f[s], qrow, col, D, L, fr);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[s][e] *= qk_scale * ksc[col + e];
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[s][e] = 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[s][e]));
    int ex = 0;
    (void)frexpf(class_max<16>(mx), &ex);
    const float inv = ldexpf(1.f, -ex);
    qs = ldexpf(1.f, ex);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[s][e] = (_Float16)(f[s][e] * inv);
  }

  // The new token (index L): the codes of its rotated key and of its value,
  // computed by the lanes of wave 0 that hold row 0 (each its dims), stored
  // into the cache and into LDS, from where the lanes of row L take them in
  // place of the cached row.
  int8_t* const Kc = static_cast<int8_t*>(c.k);
  int8_t* const Vc = static_cast<int8_t*>(c.v);
  const bool has_new = L < t0 + SPLIT;  // uniform
  if (has_new && wave == 0 && r16 == 0) {
    const int64_t src = ((int64_t)b * Hkv + hk) * D;
    const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, L) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = i8m_dim<D>(s, g4, 0);
      float f[8], g[8];
      load16<bf16_t>(k_new + src + col, f);
      rope_rotate_chunk<bf16_t, 8, HALF>(f, k_new + src, col, D, L, fr);
      load16<bf16_t>(v_new + src + col, g);
      uint32_t kw[2], vw[2];
      int8_codes<8>(f, ksc + col, kw);
      int8_codes<8>(g, vsc + col, vw);
      if (store_new) {
        *reinterpret_cast<u32x2_t*>(Kc + dst + col) = u32x2_t{kw[0], kw[1]};
        *reinterpret_cast<u32x2_t*>(Vc + dst + col) = u32x2_t{vw[0], vw[1]};
      }
      *reinterpret_cast<u32x2_t*>(&snew[0][col]) = u32x2_t{kw[0], kw[1]};
      *reinterpret_cast<u32x2_t*>(&snew[1][col]) = u32x2_t{vw[0], vw[1]};
    }
  }
  if (has_new) __syncthreads();  // uniform over the workgroup

  f32x4_t o[NJ];  // O[head 4*g4 + i][dim 8*r16 + j] (D = 128; 4*r16 + j at D = 64)
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // head r16's reference maximum (log2 units)
  float l_run = 0.f;        // its sum over this lane's tokens

  if (tw <= L) {  // uniform per wave: this wave holds at least one token
    int myblk = 0;  // lane j: physical block of the wave's j-th block
    if constexpr (PAGED) {
      const int32_t* trow = c.table + (int64_t)b * c.mbps;
      if (lane < NBLK)
        myblk = min(max(trow[min((tw >> 4) + lane, L >> 4)], 0), c.num_blocks - 1);
    }
    const int64_t cbase = PAGED ? 0 : ((int64_t)b * Hkv + hk) * c.max_seq;
    const int nb = min(NBLK, ((L - tw) >> 4) + 1);  // blocks holding tokens <= L
    // Block bi's 16 rows of K and of V (streamed once), each load instruction
    // reading whole rows: load h of a lane covers row RPI*h + lrow, bytes
    // 16*lchunk .. 16*lchunk + 15.
    constexpr int CPR = D / 16, RPI = 64 / CPR;  // 16-byte chunks per row, rows per load
    const int lrow = lane / CPR, lchunk = lane % CPR;
    auto load_blk = [&](int bi, u32x4_t (&kb)[NL], u32x4_t (&vb)[NL]) {
      int64_t row0 = 0;
      if constexpr (PAGED) {
        const int blk = __builtin_amdgcn_readlane(myblk, bi);  // uniform index
        row0 = ((int64_t)blk * Hkv + hk) << 4;
      }
#pragma unroll
      for (int h = 0; h < NL; ++h) {
        const int r = RPI * h + lrow;
        // contiguous: rows past L stay inside the cache
        const int64_t row = PAGED ? row0 + r : cbase + min(tw + 16 * bi + r, L);
        const int64_t off = row * D + 16 * lchunk;
        // streamed once: non-temporal loads keep the rows out of the caches
        kb[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Kc + off));
        vb[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Vc + off));
      }
    };
    uint8_t* const skw = sk[wave];
    uint8_t* const svw = sv[wave];
    auto consume = [&](int bi, u32x4_t (&kb)[NL], u32x4_t (&vb)[NL]) {
      const int tb = tw + 16 * bi;  // first token of the block
      if (tb + 15 >= L) {  // the block reaches index L (uniform): token L from LDS
#pragma unroll
        for (int h = 0; h < NL; ++h) {
          if (tb + RPI * h + lrow == L) {
            kb[h] = *reinterpret_cast<const u32x4_t*>(&snew[0][16 * lchunk]);
            vb[h] = *reinterpret_cast<const u32x4_t*>(&snew[1][16 * lchunk]);
          }
        }
      }
      // the block's rows into LDS (row-major) for the reads of both operands
#pragma unroll
      for (int h = 0; h < NL; ++h) {
        const int o16 = (RPI * h + lrow) * LROW + 16 * lchunk;
        *reinterpret_cast<u32x4_t*>(skw + o16) = kb[h];
        *reinterpret_cast<u32x4_t*>(svw + o16) = vb[h];
      }
      // scores: S^T[token 4*g4 + i][head r16], log2 units; lane (r16, g4)
      // reads key row r16's bytes 64*h + 16*g4 .. + 15
      u32x4_t kr[NL];
#pragma unroll
      for (int h = 0; h < NL; ++h)
        kr[h] = *reinterpret_cast<const u32x4_t*>(skw + r16 * LROW + 64 * h + 16 * g4);
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4_t& w = kr[s >> 1];
        const f16x8_t a = codes8_f16(w[2 * (s & 1)], w[2 * (s & 1) + 1]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[s], sacc, 0, 0, 0);
      }
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tb + 4 * g4 + i;
        sc[i] = t <= L ? sacc[i] * qs : -INFINITY;
        mx = fmaxf(mx, sc[i]);
      }
      mx = class_max<16>(mx);  // the block's maximum of head r16
      // lazy rescale: the reference moves only when a score exceeds it by
      // more than kRescaleLog2; O's rows are heads 4*g4 + i, so each lane
      // takes the factors of those heads from the lanes that own them
      if (__builtin_amdgcn_ballot_w64(mx - m_run > kRescaleLog2) != 0) {  // uniform
        const float m_new = fmaxf(m_run, mx);  // finite: token tb <= L is visible
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        float ah[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a0 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), i);
          const int a1 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 4 + i);
          ah[i] = __builtin_bit_cast(float, g4 == 0 ? a0 : a1);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[j][i] *= ah[i];
      }
      // P (fp16) as the A operand of the value MFMAs; l sums the rounded P
      const uint32_t p01 = pack_f16x2(fast_exp2(sc[0] - m_run), fast_exp2(sc[1] - m_run));
      const uint32_t p23 = pack_f16x2(fast_exp2(sc[2] - m_run), fast_exp2(sc[3] - m_run));
      l_run = dot2_f16(p01, kOnePairF16, l_run);
      l_run = dot2_f16(p23, kOnePairF16, l_run);
      const f16x4_t pa = __builtin_bit_cast(f16x4_t, u32x2_t{p01, p23});
      // values: lane (g4, c = r16) reads dims NJ*c .. NJ*c + NJ-1 of tokens
      // 4*g4 + e; MFMA j takes dim NJ*c + j of each
      uint32_t vw[4][NJ / 4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint8_t* src = svw + (4 * g4 + e) * LROW + NJ * r16;
        if constexpr (NJ == 8) {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(src);
          vw[e][0] = x[0];
          vw[e][1] = x[1];
        } else {
          vw[e][0] = *reinterpret_cast<const uint32_t*>(src);
        }
      }
      static_for<0, NJ>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const uint32_t lo = codes_f16_rows<j % 4>(vw[0][j / 4], vw[1][j / 4]);
        const uint32_t hi = codes_f16_rows<j % 4>(vw[2][j / 4], vw[3][j / 4]);
        const f16x4_t vbm = __builtin_bit_cast(f16x4_t, u32x2_t{lo, hi});
        o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vbm, o[j], 0, 0, 0);
      });
    };

    // double-buffered blocks: block bi+1's loads are in flight while block
    // bi is consumed.  The steady-state loop issues its loads unconditionally
    // (so that each wait covers only the older block); the last one or two
    // blocks are consumed after it.
    u32x4_t kb0[NL], vb0[NL], kb1[NL], vb1[NL];
    load_blk(0, kb0, vb0);
    int bi = 0;
#pragma unroll 1
    for (; bi + 2 < nb; bi += 2) {
      load_blk(bi + 1, kb1, vb1);
      consume(bi, kb0, vb0);
      load_blk(bi + 2, kb0, vb0);
      consume(bi + 1, kb1, vb1);
    }
    if (bi + 1 < nb) {
      load_blk(bi + 1, kb1, vb1);
      consume(bi, kb0, vb0);
      consume(bi + 1, kb1, vb1);
    } else {
      consume(bi, kb0, vb0);
    }
  }

  // Merge the four lanes of each head column, then the waves (as the packed
  // path), removing the code bias 1152 * l and applying the value scales.
  l_run = class_sum<16>(l_run);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = 4 * g4 + i;
    if (hd < G) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) sm_acc[wave][hd][NJ * r16 + j] = o[j][i];
    }
  }
  if (g4 == 0 && r16 < G) {
    sm_ml[wave][r16][0] = m_run;
    sm_ml[wave][r16][1] = l_run;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += 64 * WAVES) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm_ml[w][g][0]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float mw = sm_ml[w][g][0];
      const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      a = fmaf(f, sm_acc[w][g][d], a);
      l = fmaf(f, sm_ml[w][g][1], l);
    }
    float* dst = part + (((int64_t)b * Hq + hk * G + g) * nsplit + split) * PW;
    dst[4 + d] = (a - kCodeBias * l) * vsc[d];
    if (d == 0) {
      dst[0] = M;
      dst[1] = l;
    }
  }
}

template <typename T, int D, int G, bool PAGED>
hipError_t decode_i8_t(const void* q, const void* k_new, const void* v_new, void* out, int B,
                       int Hkv, const int32_t* seq_lens, int max_seq_len, const CacheArgs& c,
                       float* partials, const RopeFreq& fr, float scale, hipStream_t st,
                       const TimedLaunch& tl) {
  constexpr int SPLIT = i8_split_tokens<G>();
  const int nsplit = (max_seq_len + SPLIT - 1) / SPLIT;  // <= the workspace's split count
  const float qk_scale = scale * 1.4426950408889634f;  // log2(e): softmax in base 2
  const dim3 grid(Hkv * B, nsplit), block(64 * i8_waves<G>());
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(k_new);
  const T* vv = static_cast<const T*>(v_new);
  if constexpr (sizeof(T) == 2 && G > 1) {  // bf16, several heads: the matrix-core kernel
    static_assert(SPLIT == I8MfmaGeom<D>::SPLIT, "both kernels split the sequence alike");
    if (fr.half)
      hipExtLaunchKernelGGL((decode_i8_mfma_kernel<D, G, PAGED, true>), grid, dim3(512), 0, st,
                            tl.start, tl.stop, 0, qq, kk, vv, seq_lens, c, partials, Hkv, nsplit,
                            fr, qk_scale);
    else
      hipExtLaunchKernelGGL((decode_i8_mfma_kernel<D, G, PAGED, false>), grid, dim3(512), 0, st,
                            tl.start, tl.stop, 0, qq, kk, vv, seq_lens, c, partials, Hkv, nsplit,
                            fr, qk_scale);
  } else if (fr.half)
    hipExtLaunchKernelGGL((decode_i8_split_kernel<T, D, G, PAGED, SPLIT, true>), grid, block,
                          0, st, tl.start, tl.stop, 0, qq, kk, vv, seq_lens, c, partials, Hkv,
                          nsplit, fr, qk_scale);
  else
    hipExtLaunchKernelGGL((decode_i8_split_kernel<T, D, G, PAGED, SPLIT, false>), grid, block,
                          0, st, tl.start, tl.stop, 0, qq, kk, vv, seq_lens, c, partials, Hkv,
                          nsplit, fr, qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int last = PAGED ? c.mbps * 16 - 1 : c.max_seq - 1;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(B * Hkv * G), dim3(64), 0, st,
                     partials, seq_lens, static_cast<T*>(out), Hkv * G, nsplit, SPLIT, last);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t decode_i8_paged(bool paged, const void* q, const void* kn, const void* vn, void* out,
                           int B, int Hkv, const int32_t* sl, int max_seq_len,
                           const CacheArgs& c, float* part, const RopeFreq& fr, float scale,
                           hipStream_t st, const TimedLaunch& tl) {
  return paged ? decode_i8_t<T, D, G, true>(q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part,
                                            fr, scale, st, tl)
               : decode_i8_t<T, D, G, false>(q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part,
                                             fr, scale, st, tl);
}

template <typename T, int D>
hipError_t decode_i8_group(int group, bool paged, const void* q, const void* kn, const void* vn,
                           void* out, int B, int Hkv, const int32_t* sl, int max_seq_len,
                           const CacheArgs& c, float* part, const RopeFreq& fr, float scale,
                           hipStream_t st, const TimedLaunch& tl) {
  switch (group) {
    case 1: return decode_i8_paged<T, D, 1>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    case 2: return decode_i8_paged<T, D, 2>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    case 4: return decode_i8_paged<T, D, 4>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    case 8: return decode_i8_paged<T, D, 8>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_i8(Dtype dt, int D, int group, bool paged, const void* q,
                            const void* k_new, const void* v_new, void* out, int B, int Hq,
                            int Hkv, const int32_t* seq_lens, int max_seq_len,
                            const CacheArgs& c, float* partials, const RopeFreq& fr,
                            float scale, hipStream_t s, const TimedLaunch& tl) {
  (void)Hq;
  if (dt == F32)
    return D == 64 ? decode_i8_group<float, 64>(group, paged, q, k_new, v_new, out, B, Hkv,
                                                seq_lens, max_seq_len, c, partials, fr, scale, s,
                                                tl)
                   : decode_i8_group<float, 128>(group, paged, q, k_new, v_new, out, B, Hkv,
                                                 seq_lens, max_seq_len, c, partials, fr, scale,
                                                 s, tl);
  return D == 64 ? decode_i8_group<bf16_t, 64>(group, paged, q, k_new, v_new, out, B, Hkv,
                                               seq_lens, max_seq_len, c, partials, fr, scale, s,
                                               tl)
                 : decode_i8_group<bf16_t, 128>(group, paged, q, k_new, v_new, out, B, Hkv,
                                                seq_lens, max_seq_len, c, partials, fr, scale, s,
                                                tl);
}

}  // namespace car
