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
// into pieces of 256 tokens (1024 when several query heads share a KV head);
// workgroup (kv head, sequence, split) streams its piece with 16-byte loads,
// LPR = D*sizeof(T)/16 lanes covering one row, so a
// wave load instruction moves 64/LPR whole rows (4 rows of 256 bytes for
// bf16, D = 128).  All G = Hq/Hkv query heads of a KV head are served from the
// same loads (GQA); with G > 1 the loads write straight into a per-wave LDS
// ring two rounds deep, so no registers wait on loads in flight.  Dot products are reduced across the LPR lanes of a row
// with DPP moves; the softmax maximum and sums are combined across the rows
// of a wave with lane shuffles and across the waves (4, or 8 with GQA)
// through LDS.  Each
// workgroup leaves one partial (max, sum, D accumulators) per query head; a
// second small kernel merges the partials of a sequence with the
// log-sum-exp rule of the online softmax ([Scratch] §3.4).  The workgroup
// whose piece holds index L also rotates k_new and stores it and v_new into
// the cache, and uses the new row from registers for its own score.
#include <math.h>

#include "decode_common.hpp"

namespace car {

namespace {

// Waves per workgroup: 4 with one query head per KV head; 8 with several,
// whose per-workgroup setup and merge (G heads each) are then shared by
// twice the tokens (measured on the paged GQA workload).
template <int G>
constexpr int decode_waves() { return G > 1 ? 8 : 4; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // (a.lo16, b.lo16)
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a.hi16, b.hi16)
}

constexpr uint32_t kOnePair = 0x3F803F80u;  // (1.0, 1.0) in bf16

// One non-temporal buffer -> LDS load: every lane moves the 16 bytes at
// rsrc.base + voff to lds_base + 16 * lane (lds_base uniform over the wave).
// Inline assembly without register outputs; the caller waits for it with an
// explicit vmcnt before reading the LDS it wrote.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                         void* lds_base) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(0u)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Buffer resource over `bytes` bytes at `base` (raw addressing, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Waits for all but N of this wave's vector memory operations (loads into
// LDS included), and keeps the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  static_assert(N == 0 || N == 4 || N == 8, "vmcnt values in use");
}

// Per-lane geometry of the decode split kernel.  A lane holds C chunks of
// 16 bytes of a cache row, chunks c*LPR + lane%LPR for c < C, so LPR =
// D*sizeof(T)/(16*C) lanes cover a row and each load instruction (one chunk
// per lane) moves 64/LPR rows.  C = 1 (measured faster than 2: it needs
// fewer registers per row step, so more rows are in flight).  A round is R
// row steps (two register buffers of R steps are live); R = 2 (more steps
// per round spilled or measured no faster).
constexpr int kDecodeChunks = 1;
constexpr int kDecodeRoundMax = 2;
template <typename T, int D, int G, int SPLIT = DECODE_SPLIT>
struct DecodeGeom {
  static constexpr int WAVES = decode_waves<G>();
  static constexpr int TPW = SPLIT / WAVES;    // tokens per wave
  static constexpr int N = Vec16<T>::N;        // elements per 16-byte chunk
  static constexpr int C = kDecodeChunks;      // chunks per lane per row
  static constexpr int LPR = D / N / C;        // lanes per cache row
  static constexpr int NG = 64 / LPR;          // rows per load instruction
  static constexpr int STEPS = TPW / NG;
  static_assert(SPLIT % DECODE_SPLIT == 0 && TPW % 64 == 0, "whole 16-token blocks per wave");
  static constexpr int R_MAX = kDecodeRoundMax;
  static constexpr int R = STEPS < R_MAX ? STEPS : R_MAX;  // steps per round
  static constexpr int ROUNDS = STEPS / R;
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "lanes per row");
  static_assert(NG <= 16 && 16 % NG == 0, "a row step stays inside one 16-token block");
  static_assert(R % 2 == 0 && ROUNDS * R == STEPS, "rounds must tile the wave's tokens");
  static_assert(ROUNDS == 1 || ROUNDS % 2 == 0, "rounds are consumed in pairs");
};

// Score of one row for one query head: the lane's part of q . k, reduced
// over the LPR lanes of the row.  bf16: packed dot2 on raw words.
template <typename T, int D, int C>
__device__ __forceinline__ float row_score(const uint32_t (&qw)[C][4], const u32x4_t (&k)[C]) {
  using Gm = DecodeGeom<T, D, 1>;
  float p = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2)
        p = dot2_bf16(qw[c][w], k[c][w], p);
      else
        p = fmaf(__uint_as_float(qw[c][w]), __uint_as_float(k[c][w]), p);
    }
  return group_sum<Gm::LPR>(p);
}

// HALF: RoPE pairs (i, i + D/2) instead of (2i, 2i+1), a compile-time choice
// so that the layout test stays out of the loop's register allocation.
template <typename T, int D, int G, bool PAGED, int SPLIT, bool HALF>
__global__ __launch_bounds__(64 * decode_waves<G>())
__attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2))) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ seq_lens, CacheArgs c, float* __restrict__ part, int Hkv,
    int nsplit, RopeFreq fr, float qk_scale) {
  using Gm = DecodeGeom<T, D, G, SPLIT>;
  constexpr int N = Gm::N, C = Gm::C, LPR = Gm::LPR, NG = Gm::NG, R = Gm::R,
                ROUNDS = Gm::ROUNDS, TPW = Gm::TPW;
  constexpr int PW = decode_partial_words(D);
  constexpr bool BF = sizeof(T) == 2;

  constexpr int kWaves = Gm::WAVES, kThreads = 64 * kWaves;
  // With several query heads (G > 1) the rows go from memory straight into a
  // per-wave LDS ring of two rounds, so that two rounds are in flight while
  // one is consumed from registers, and no registers wait for loads: at that
  // register count four waves per SIMD are all that fit, and the bytes in
  // flight per CU set the bandwidth.  A wave's partial sums later reuse its
  // own ring.
  constexpr bool DMA = G > 1;
  constexpr int NOPS = 2 * R * C;      // 1 KB wave loads per round (K and V)
  constexpr int ROUNDB = NOPS * 1024;  // bytes of one round
  constexpr int WAVEB = DMA ? 2 * ROUNDB : 16;
  static_assert(!DMA || (G * D * 4 <= WAVEB && ROUNDS >= 2), "ring geometry");
  __shared__ __align__(16) char ring[DMA ? kWaves * WAVEB : 16];
  __shared__ float sm_acc_w[DMA ? 1 : kWaves][DMA ? 1 : G][DMA ? 1 : D];
  auto sm_acc = [&](int w, int g, int d) -> float& {
    if constexpr (DMA)
      return reinterpret_cast<float*>(ring + w * WAVEB)[g * D + d];
    else
      return sm_acc_w[w][g][d];
  };
  __shared__ float sm_ml[kWaves][G][2];

  // Workgroups are numbered split-major with (sequence, KV head) fastest:
  // consecutive workgroup ids go to the 8 XCDs in turn, so every XCD gets
  // the same mix of sequences and splits and they all drain together.  The
  // splits of a sequence are aligned to the last row of the grid, so the
  // shorter last splits (0..L ends anywhere inside one) are dispatched last
  // and fill the end of the launch; rows before a sequence's first split
  // exit at once.
  const int hk = blockIdx.x % Hkv, b = blockIdx.x / Hkv;
  const int Hq = Hkv * G;
  // A length outside the cache is clamped for the reads (the output is then
  // unspecified) and the new token is not stored.
  const int L_in = seq_lens[b];
  const int L = min(max(L_in, 0), cache_last_slot<PAGED>(c));
  const bool store_new = L_in == L;
  const int nsb = min(L / SPLIT + 1, nsplit);  // splits that hold tokens 0..L
  const int split = (int)blockIdx.y - (nsplit - nsb);
  if (split < 0) return;  // uniform over the workgroup
  const int t0 = split * SPLIT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane / LPR;  // row of the step
  int col[C];                  // first element of the lane's chunks
#pragma unroll
  for (int ch = 0; ch < C; ++ch) col[ch] = (ch * LPR + lane % LPR) * N;
  const int tw = t0 + wave * TPW;  // first token of this wave

  // Query heads of this KV head, rotated at position L and pre-scaled so
  // that exp2 of a score difference is the softmax weight; as raw words
  // (packed bf16 pairs, or fp32 bit patterns), 4 per chunk.
  // The angles depend only on the position L and the lane's columns: one set
  // serves every query head of the group and the new key.
  RopeChunk<N> rope[C];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) rope[ch] = rope_prepare<N, HALF>(L, col[ch], D, fr);
  uint32_t qw[G][C][4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int ch = 0; ch < C; ++ch) {
      float f[N];
      const T* qrow = q + ((int64_t)b * Hq + hk * G + g) * D;
      load16<T>(qrow + col[ch], f);
      rope_apply_prepared<T, N, HALF>(f, qrow, D, rope[ch], fr);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (BF)
          qw[g][ch][w] = pack_bf16x2(f[2 * w] * qk_scale, f[2 * w + 1] * qk_scale);
        else
          qw[g][ch][w] = __float_as_uint(f[w] * qk_scale);
      }
    }

  // The new token (index L): rotated key and raw value, stored into the cache
  // by the split that holds L; in the cache's element type it is also the
  // row this split uses for token L.
  T* const Kc = static_cast<T*>(c.k);
  T* const Vc = static_cast<T*>(c.v);
  u32x4_t kn[C], vn[C];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) kn[ch] = vn[ch] = u32x4_t{0u, 0u, 0u, 0u};
  if (L < t0 + SPLIT) {
#pragma unroll
    for (int ch = 0; ch < C; ++ch) {
      const int64_t src = ((int64_t)b * Hkv + hk) * D + col[ch];
      float f[N];
      load16<T>(k_new + src, f);
      rope_apply_prepared<T, N, HALF>(f, k_new + (src - col[ch]), D, rope[ch], fr);
      T kt[N];
      store16<T>(kt, f);
      kn[ch] = *reinterpret_cast<const u32x4_t*>(kt);
      vn[ch] = *reinterpret_cast<const u32x4_t*>(v_new + src);
      if (wave == 0 && grp == 0 && store_new) {
        const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, L) * D + col[ch];
        *reinterpret_cast<u32x4_t*>(Kc + dst) = kn[ch];
        *reinterpret_cast<u32x4_t*>(Vc + dst) = vn[ch];
      }
    }
  }

  float m_run[G], l_run[G], acc[G][C][N];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int ch = 0; ch < C; ++ch)
#pragma unroll
      for (int e = 0; e < N; ++e) acc[g][ch][e] = 0.f;
  }

  if (tw <= L) {  // uniform per wave: this wave holds at least one token
    // Physical blocks of the wave's tokens: lane j holds the id of the wave's
    // j-th 16-token block, clamped to the sequence's last block so that the
    // table is never read past its row; a row step picks its id with a
    // wave-uniform lane read.
    constexpr int NBLK = TPW / 16;
    static_assert(NBLK <= 64, "one block id per lane");
    int myblk = 0;
    if constexpr (PAGED) {
      const int32_t* trow = c.table + (int64_t)b * c.mbps;
      if (lane < NBLK)
        myblk = min(max(trow[min((tw >> 4) + lane, L >> 4)], 0), c.num_blocks - 1);
    }

    u32x4_t kb[2][R][C], vb[2][R][C];
    // Loads of round r into register buffer BUF (a compile-time index).  The
    // NG rows of a step are consecutive cache rows (a step never straddles a
    // 16-token block), so each step needs one wave-uniform base and the lane's
    // chunk offset.  Rows at or past L are only ever replaced (consume), so
    // they just have to stay inside the cache: the paged block ids are
    // clamped to the sequence's last block, and contiguous rows to L.
    const int64_t cbase = PAGED ? 0 : ((int64_t)b * Hkv + hk) * c.max_seq + tw;
    auto issue = [&](int r, auto BUF) {
      constexpr int buf = decltype(BUF)::value;
#pragma unroll
      for (int st = 0; st < R; ++st) {
        const int x = r * R + st;
        int64_t row0;
        int lrow = grp;  // lane's row within the step
        if constexpr (PAGED) {
          const int blk = __builtin_amdgcn_readlane(myblk, (x * NG) >> 4);  // uniform index
          row0 = (((int64_t)blk * Hkv + hk) << 4) + ((x * NG) & 15);
        } else {
          row0 = cbase + x * NG;
          lrow = min(grp, L - tw - x * NG);  // never past row L (may be negative)
        }
        const T* kp = Kc + row0 * D;
        const T* vp = Vc + row0 * D;
#pragma unroll
        for (int ch = 0; ch < C; ++ch) {
          const int off = lrow * D + col[ch];
          // streamed once: non-temporal loads keep the rows out of the caches
          kb[buf][st][ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + off));
          vb[buf][st][ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp + off));
        }
      }
    };

    // Online-softmax update with the rows of round r held in buffer BUF.
    auto consume = [&](int r, auto BUF) {
      constexpr int buf = decltype(BUF)::value;
      const bool full = tw + (r + 1) * R * NG - 1 < L;
      if (!full) {
        // the round reaches index L: token L from registers, later rows zeroed
#pragma unroll
        for (int st = 0; st < R; ++st) {
          const int t = tw + (r * R + st) * NG + grp;
#pragma unroll
          for (int ch = 0; ch < C; ++ch)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              kb[buf][st][ch][w] = t < L ? kb[buf][st][ch][w] : kn[ch][w];
              vb[buf][st][ch][w] = t < L ? vb[buf][st][ch][w] : (t == L ? vn[ch][w] : 0u);
            }
        }
      }
      float sc[R][G];
#pragma unroll
      for (int st = 0; st < R; ++st) {
        const int t = tw + (r * R + st) * NG + grp;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sv = row_score<T, D, C>(qw[g], kb[buf][st]);
          sc[st][g] = (full || t <= L) ? sv : -INFINITY;
        }
      }
      // Lazy rescale: the reference maximum m_run of a head only moves when
      // a score exceeds it by more than kRescaleLog2 (weights up to 2^8); O
      // and l always share the reference, so the result is exact while the
      // cross-lane maximum, the exp and the rescale of O are skipped for most
      // rounds.  m_run is the same on every lane of the wave.
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = sc[0][g];
#pragma unroll
        for (int st = 1; st < R; ++st) mx = fmaxf(mx, sc[st][g]);
        if (__builtin_amdgcn_ballot_w64(mx - m_run[g] > kRescaleLog2) != 0) {  // uniform
          // round 0 always holds token tw <= L, so m_new is finite from here on
          const float m_new = fmaxf(m_run[g], class_max<LPR>(mx));
          const float alpha = fast_exp2(m_run[g] - m_new);
          m_run[g] = m_new;
          l_run[g] *= alpha;
#pragma unroll
          for (int ch = 0; ch < C; ++ch)
#pragma unroll
            for (int e = 0; e < N; ++e) acc[g][ch][e] *= alpha;
        }
      }
#pragma unroll
      for (int st = 0; st < R; st += 2) {
        if constexpr (BF) {
          // P V over a pair of rows with packed dot2: (p_a, p_b) . (v_a[e], v_b[e])
          uint32_t vp[C][N];
#pragma unroll
          for (int ch = 0; ch < C; ++ch)
#pragma unroll
            for (int e = 0; e < N; ++e)
              vp[ch][e] = (e & 1) ? perm_hi(vb[buf][st][ch][e >> 1], vb[buf][st + 1][ch][e >> 1])
                                  : perm_lo(vb[buf][st][ch][e >> 1], vb[buf][st + 1][ch][e >> 1]);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint32_t pp = pack_bf16x2(fast_exp2(sc[st][g] - m_run[g]),
                                            fast_exp2(sc[st + 1][g] - m_run[g]));
            l_run[g] = dot2_bf16(pp, kOnePair, l_run[g]);
#pragma unroll
            for (int ch = 0; ch < C; ++ch)
#pragma unroll
              for (int e = 0; e < N; ++e) acc[g][ch][e] = dot2_bf16(pp, vp[ch][e], acc[g][ch][e]);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float pr = fast_exp2(sc[st + h][g] - m_run[g]);
              l_run[g] += pr;
#pragma unroll
              for (int ch = 0; ch < C; ++ch)
#pragma unroll
                for (int e = 0; e < N; ++e)
                  acc[g][ch][e] = fmaf(pr, __uint_as_float(vb[buf][st + h][ch][e]), acc[g][ch][e]);
            }
          }
        }
      }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    if constexpr (DMA) {
      // Round r goes to ring slot r % 2 (its K rows, then its V rows, each
      // step's 1 KB loads in order); lane l's 16 bytes land at 16 * l of a
      // load's kilobyte and the lane reads them back from there.  The rows
      // are those of the register path: paged steps stay in one block (one
      // resource per block), contiguous rows are clamped to L.
      char* const wring = ring + wave * WAVEB;
      auto issue_dma = [&](int r, int slot) {
        char* const dst = wring + slot * ROUNDB;
#pragma unroll
        for (int st = 0; st < R; ++st) {
          const int x = r * R + st;
          int64_t e0;  // first element of the resource
          uint32_t bytes;
          int row;  // the lane's row within it
          if constexpr (PAGED) {
            const int blk = __builtin_amdgcn_readlane(myblk, (x * NG) >> 4);  // uniform index
            e0 = (((int64_t)blk * Hkv + hk) << 4) * D;
            bytes = 16 * D * sizeof(T);
            row = ((x * NG) & 15) + grp;
          } else {
            e0 = ((int64_t)b * Hkv + hk) * c.max_seq * D;
            bytes = (uint32_t)c.max_seq * D * sizeof(T);
            row = min(tw + x * NG + grp, L);
          }
          const __amdgpu_buffer_rsrc_t krs = raw_rsrc(Kc + e0, bytes);
          const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(Vc + e0, bytes);
#pragma unroll
          for (int ch = 0; ch < C; ++ch) {
            const uint32_t voff = (uint32_t)(row * D + col[ch]) * sizeof(T);
            dma16_nt(krs, voff, dst + (st * C + ch) * 2048);
            dma16_nt(vrs, voff, dst + (st * C + ch) * 2048 + 1024);
          }
        }
      };
      auto read_round = [&](int slot) {
        const char* const src = wring + slot * ROUNDB + lane * 16;
#pragma unroll
        for (int st = 0; st < R; ++st)
#pragma unroll
          for (int ch = 0; ch < C; ++ch) {
            kb[0][st][ch] = *reinterpret_cast<const u32x4_t*>(src + (st * C + ch) * 2048);
            vb[0][st][ch] = *reinterpret_cast<const u32x4_t*>(src + (st * C + ch) * 2048 + 1024);
          }
        // the slot is loaded again next: its reads must have returned
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      };
      issue_dma(0, 0);
      issue_dma(1, 1);
#pragma unroll 1
      for (int r = 0; r < ROUNDS - 2; ++r) {
        wait_vm<NOPS>();  // round r landed; round r + 1 may still be in flight
        read_round(r & 1);
        issue_dma(r + 2, r & 1);
        consume(r, B0{});
      }
      wait_vm<NOPS>();
      read_round(0);  // ROUNDS is even
      consume(ROUNDS - 2, B0{});
      wait_vm<0>();
      read_round(1);
      consume(ROUNDS - 1, B0{});
    } else {
    // Double-buffered rounds: round r+1's loads are in flight while round r
    // is consumed.
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
  }

  // Merge the rows of the wave (lanes that share the same columns).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = class_sum<LPR>(l_run[g]);
#pragma unroll
    for (int ch = 0; ch < C; ++ch)
#pragma unroll
      for (int e = 0; e < N; ++e) acc[g][ch][e] = class_sum<LPR>(acc[g][ch][e]);
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int ch = 0; ch < C; ++ch)
#pragma unroll
        for (int e = 0; e < N; ++e) sm_acc(wave, g, col[ch] + e) = acc[g][ch][e];
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
      a = fmaf(f, sm_acc(w, g, d), a);
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

// Tokens per workgroup: 256 with one query head per KV head (64 per wave);
// with several, 1024 (128 per wave of 8): each workgroup carries the
// per-head setup (rotated queries, partials) G times, and longer splits
// amortise it (measured on the paged GQA workload).
template <int G>
constexpr int split_tokens() { return G == 1 ? DECODE_SPLIT : 4 * DECODE_SPLIT; }

template <typename T, int D, int G, bool PAGED>
hipError_t decode_t(const void* q, const void* k_new, const void* v_new, void* out, int B,
                    int Hkv, const int32_t* seq_lens, int max_seq_len, const CacheArgs& c,
                    float* partials, const RopeFreq& fr, float scale, hipStream_t st,
                    const TimedLaunch& tl) {
  constexpr int SPLIT = split_tokens<G>();
  const int nsplit = (max_seq_len + SPLIT - 1) / SPLIT;  // <= the workspace's split count
  const float qk_scale = scale * 1.4426950408889634f;  // log2(e): softmax in base 2
  if (fr.half)
    hipExtLaunchKernelGGL((decode_split_kernel<T, D, G, PAGED, SPLIT, true>),
                          dim3(Hkv * B, nsplit), dim3(64 * decode_waves<G>()), 0, st, tl.start,
                          tl.stop, 0, static_cast<const T*>(q), static_cast<const T*>(k_new),
                          static_cast<const T*>(v_new), seq_lens, c, partials, Hkv, nsplit, fr,
                          qk_scale);
  else
    hipExtLaunchKernelGGL((decode_split_kernel<T, D, G, PAGED, SPLIT, false>),
                          dim3(Hkv * B, nsplit), dim3(64 * decode_waves<G>()), 0, st, tl.start,
                          tl.stop, 0, static_cast<const T*>(q), static_cast<const T*>(k_new),
                          static_cast<const T*>(v_new), seq_lens, c, partials, Hkv, nsplit, fr,
                          qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int last = PAGED ? c.mbps * 16 - 1 : c.max_seq - 1;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(B * Hkv * G), dim3(64), 0, st,
                     partials, seq_lens, static_cast<T*>(out), Hkv * G, nsplit, SPLIT, last);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t decode_paged(bool paged, const void* q, const void* kn, const void* vn, void* out,
                        int B, int Hkv, const int32_t* sl, int max_seq_len, const CacheArgs& c,
                        float* part, const RopeFreq& fr, float scale, hipStream_t st,
                        const TimedLaunch& tl) {
  return paged ? decode_t<T, D, G, true>(q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale,
                                         st, tl)
               : decode_t<T, D, G, false>(q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr,
                                          scale, st, tl);
}

template <typename T, int D>
hipError_t decode_group(int group, bool paged, const void* q, const void* kn, const void* vn,
                        void* out, int B, int Hkv, const int32_t* sl, int max_seq_len,
                        const CacheArgs& c, float* part, const RopeFreq& fr, float scale,
                        hipStream_t st, const TimedLaunch& tl) {
  switch (group) {
    case 1: return decode_paged<T, D, 1>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    case 2: return decode_paged<T, D, 2>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    case 4: return decode_paged<T, D, 4>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    case 8: return decode_paged<T, D, 8>(paged, q, kn, vn, out, B, Hkv, sl, max_seq_len, c, part, fr, scale, st, tl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(Dtype dt, int D, int group, bool paged, const void* q,
                         const void* k_new, const void* v_new, void* out, int B, int Hq,
                         int Hkv, const int32_t* seq_lens, int max_seq_len, const CacheArgs& c,
                         float* partials, const RopeFreq& fr, float scale, hipStream_t s,
                         const TimedLaunch& tl) {
  (void)Hq;
  if (dt == F32)
    return D == 64 ? decode_group<float, 64>(group, paged, q, k_new, v_new, out, B, Hkv, seq_lens,
                                             max_seq_len, c, partials, fr, scale, s, tl)
                   : decode_group<float, 128>(group, paged, q, k_new, v_new, out, B, Hkv,
                                              seq_lens, max_seq_len, c, partials, fr, scale, s, tl);
  return D == 64 ? decode_group<bf16_t, 64>(group, paged, q, k_new, v_new, out, B, Hkv, seq_lens,
                                            max_seq_len, c, partials, fr, scale, s, tl)
                 : decode_group<bf16_t, 128>(group, paged, q, k_new, v_new, out, B, Hkv,
                                             seq_lens, max_seq_len, c, partials, fr, scale, s, tl);
}

}  // namespace car
