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
//  * bf16: MFMA 32x32x16 bf16 with fp32 accumulation.  A workgroup of 8
//    waves (two per SIMD) owns 256 query rows (32 per wave) and walks key
//    tiles of 64 (D = 128) or 128 (D = 64) keys up to the diagonal.  Each
//    wave computes S^T = K Q^T so that a lane holds one query's scores in its
//    accumulator registers: the row maximum and sum need only in-lane work
//    plus one exchange between the two wave halves, and the probabilities
//    already sit in the operand layout of the second product O^T = V^T P^T.
//    K and V tiles are copied row-major from global memory straight into LDS
//    (buffer loads with an LDS destination), chunk-permuted so that the K
//    operand reads and the transposing V operand reads are free of bank
//    conflicts; tiles are double-buffered so the next tiles' loads overlap
//    the current tile's MFMA work.  A workgroup takes one long and one short
//    query tile of a head (equal work for every workgroup of the causal
//    triangle), and the heads are pinned to XCDs so that a KV head's tiles
//    stay in one L2.
#include <math.h>

#include "common.hpp"

namespace car {

namespace {

// Where the attention kernels read rotated keys and values.
constexpr int KEYS_PROMPT = 0;  // the prompt's own K' and V, [B, Hkv, S, D]
constexpr int KEYS_CONTIG = 1;  // a contiguous cache holding the prefix and the chunk
constexpr int KEYS_PAGED = 2;   // a paged cache holding the prefix and the chunk
// (bf16 only) a contiguous array of INT8 codes as bf16, the rows of an INT8
// cache, with the cache's per-(KV head, channel) scales in c.k_scale, c.v_scale
constexpr int KEYS_CODES = 3;

// Tokens of sequence b's prompt or chunk: S, or with per-sequence lengths
// (a padded batch of prompts or chunks of different lengths) lens[b]; rows
// from there on are padding.
template <int SRC>
__device__ __forceinline__ int chunk_len(const int32_t* lens, int b, int S) {
  return lens == nullptr ? S : min(max(lens[b], 0), S);
}

// Tokens cached before the chunk (0 for a prompt): seq_lens[b], kept small
// enough that the chunk's last key stays inside the cache.
template <int SRC>
__device__ __forceinline__ int chunk_start(const CacheArgs& c, const int32_t* seq_lens, int b,
                                           int S) {
  if constexpr (SRC == KEYS_PROMPT) {
    return 0;
  } else {
    const int P = min(max(seq_lens[b], 0), cache_last_slot<SRC == KEYS_PAGED>(c) + 1 - S);
    return max(P, 0);
  }
}

// ------------------------------------------------------------------ fp32 ---
constexpr int F32_ROWS = 64;  // query rows per workgroup (one per thread)
constexpr int F32_KT = 32;    // keys per LDS tile

template <int D, int SRC, int HALF>
__global__ __launch_bounds__(F32_ROWS) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kr, const float* __restrict__ v,
    float* __restrict__ out, const int32_t* __restrict__ positions, int Hq, int Hkv, int S,
    RopeFreq fr, float qk_scale, CacheArgs c, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ chunk_lens) {
  __shared__ float4 sk[F32_KT][D / 4];
  __shared__ float4 sv[F32_KT][D / 4];
  const int b = blockIdx.z, hq = blockIdx.y;
  const int hk = hq / (Hq / Hkv);
  const int i0 = blockIdx.x * F32_ROWS;
  const int i = i0 + threadIdx.x;
  const int Sb = chunk_len<SRC>(chunk_lens, b, S);   // rows i >= Sb are padding
  const int ic = min(i, max(Sb - 1, 0));
  const int P = chunk_start<SRC>(c, seq_lens, b, Sb);  // keys before the chunk
  const int nkeys = P + Sb;

  float qv[D];
  const float* qrow = q + (((int64_t)b * Hq + hq) * S + ic) * D;
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    float f[4];
    load16<float>(qrow + d, f);
    rope_rotate_chunk<float, 4, HALF>(f, qrow, d, D,
                                SRC == KEYS_PROMPT ? positions[(int64_t)b * S + ic] : P + ic, fr);
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[d + e] = f[e] * qk_scale;
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* kb = SRC == KEYS_PROMPT ? kr + ((int64_t)b * Hkv + hk) * S * D : nullptr;
  const float* vb = SRC == KEYS_PROMPT ? v + ((int64_t)b * Hkv + hk) * S * D : nullptr;
  const int jlast = min(nkeys - 1, P + i0 + F32_ROWS - 1);
  for (int j0 = 0; j0 <= jlast; j0 += F32_KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < F32_KT * D / 4; idx += F32_ROWS) {
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      const int j = min(j0 + r, nkeys - 1);
      int64_t off;  // element offset of key row j
      if constexpr (SRC == KEYS_PROMPT)
        off = (int64_t)j * D;
      else
        off = cache_row<SRC == KEYS_PAGED>(c, b, hk, Hkv, j) * D;
      const float* ksrc = SRC == KEYS_PROMPT ? kb : static_cast<const float*>(c.k);
      const float* vsrc = SRC == KEYS_PROMPT ? vb : static_cast<const float*>(c.v);
      sk[r][c4] = *reinterpret_cast<const float4*>(ksrc + off + c4 * 4);
      sv[r][c4] = *reinterpret_cast<const float4*>(vsrc + off + c4 * 4);
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
      s[r] = (j0 + r <= P + ic) ? dot : -INFINITY;
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
    const bool pad = i >= Sb;  // padding rows: zeros
    const float inv = 1.f / l;
    float* orow = out + (((int64_t)b * Hq + hq) * S + i) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = pad ? 0.f : acc[d + e] * inv;
      store16<float>(orow + d, f);
    }
  }
}

// ------------------------------------------------------------ bf16 MFMA ---
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kOnePair = 0x3F803F80u;  // (1.0, 1.0) in bf16
constexpr float kRescaleLog2 = 8.f;          // largest exp2 argument allowed before rescaling
constexpr float kFastMax = 16777216.f;       // 2^24: largest per-lane tile sum of P kept as is

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two floats to a packed bf16 pair with one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// One direct buffer -> LDS load: every lane moves the 16 bytes at
// rsrc.base + soff + voff to lds_base + 16 * lane (lds_base and soff uniform
// over the wave).  Issued from inline assembly (it has no register outputs):
// the compiler would count the builtin's load as a pending LDS write and
// wait for it before every later LDS read of the wave, which keeps loads
// issued in the middle of a step from overlapping that step's LDS work.
// Every wait for these loads is explicit (vmcnt before the step barriers).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                      void* lds_base) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Buffer resource over `bytes` bytes at `base` (raw addressing, no stride);
// the fourth descriptor word is the gfx9-family default data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Swap the two 32-lane halves of the wave: lane l receives x from lane l ^ 32.
__device__ __forceinline__ float swap_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  // lanes < 32 find the upper half's value in r[1], lanes >= 32 the lower half's in r[0]
  return __builtin_bit_cast(float, (__lane_id() < 32) ? r[1] : r[0]);
}

template <int D, int W>
struct Tile {
  static constexpr int WAVES = W;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;           // query rows per workgroup
  static constexpr int BN = D == 128 ? 64 : 128;  // keys per tile
  static constexpr int ROWB = D * 2;              // bytes per K or V row
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;         // bytes of one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;        // K tile then V tile
  static constexpr int RPI = 64 / CPR;            // rows per 1 KB direct-to-LDS load
  static constexpr int IPW = TILEB / 1024 / WAVES;  // such loads per wave per tensor
  static constexpr int NKB = BN / 32;             // 32-key blocks of S^T
  static constexpr int NDB = D / 32;              // 32-wide head-dim blocks of O^T
  static constexpr int QKS = D / 16;              // k-steps of Q K^T
  static constexpr int PKS = BN / 16;             // k-steps of P V
  static_assert(TILEB % (1024 * WAVES) == 0, "tiles split evenly into 1 KB loads");
};

// LDS layout of a K or V tile: rows of D bf16 in key order, the 16-byte
// chunk c of row r stored at chunk position phys(c, r), a permutation of the
// row's chunks.  LDS has 64 four-byte banks (256 bytes per cycle); a 16-byte
// read serves 16 lanes per cycle and an 8-byte read 32 lanes, so a read is
// conflict-free when those lanes cover each bank once.
//  * K operand reads (16 B, rows r..r+15 of one chunk c): D = 128 rows span
//    all banks, so phys must be one-to-one over r % 16; D = 64 rows fill half
//    the banks (r % 2 picks the half), so phys must be one-to-one over bits
//    1..3 of r.
//  * V transposing reads (8 B, 32 lanes = 4 rows x chunks c0..c0+3 of dims
//    0..31 of a 32-dim block): for D = 128, chunks c0, c0+1 (dims 0..15) and
//    c0+2, c0+3 (dims 16..31) must land in different bank halves, hence the
//    flip of chunk bit 3 by chunk bit 1; the row terms spread the 4 rows.
template <int CPR>
__device__ __forceinline__ int phys_chunk(int c, int r) {
  if constexpr (CPR == 16) {
    const int s = ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
    return (c ^ (((c >> 1) & 1) << 3)) ^ s;
  } else {
    return c ^ ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1));
  }
}

// Inverse of phys_chunk in c: the logical chunk stored at position p of row r.
template <int CPR>
__device__ __forceinline__ int logical_chunk(int p, int r) {
  if constexpr (CPR == 16) {
    const int y = p ^ (((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3));
    return y ^ (((y >> 1) & 1) << 3);
  } else {
    return p ^ ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1));
  }
}

// Workgroup forms, 8 waves (two per SIMD) either way:
//  * FORM_PAIR: 256 query rows (32 per wave) over the whole key range, and a
//    workgroup takes a long and a short query tile of a whole prompt;
//  * FORM_SPLIT: 128 query rows, one tile per workgroup, its key range split
//    over two groups of 4 waves (see KSPLIT below).  Chunks after a cached
//    prefix, whose tiles all cost about the same, and short prompts whose
//    pairs would leave most compute units idle take it: a 1024-token chunk
//    of 32 heads gets 256 workgroups, and B=4, H=12, S=512 gets 192, not 48.
constexpr int FORM_PAIR = 0;
constexpr int FORM_SPLIT = 1;

template <int D, int SRC, int HALF, int FORM>
__global__ __launch_bounds__((Tile<D, 8>::THREADS), 2) void prefill_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kr, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ out, const int32_t* __restrict__ positions, int Hq, int Hkv, int S,
    int nqt, RopeFreq fr, float sm_scale_log2, CacheArgs c, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ chunk_lens, int vstore) {
  constexpr bool PAIRED = FORM == FORM_PAIR;
  // FORM_SPLIT: waves 0..3 take the first half of the query tile's key tiles
  // and waves 4..7 the second, each group with its own double-buffered K and
  // V tiles; their partial results merge through LDS at the end.  The second
  // wave per SIMD hides the other's latency as in the paired form.
  constexpr bool KSPLIT = FORM == FORM_SPLIT;
  constexpr int NGRP = KSPLIT ? 2 : 1;
  using C = Tile<D, 8 / NGRP>;  // tile geometry of one group: BM query rows, its loads
  __shared__ __attribute__((aligned(1024))) char smem[NGRP * 2 * C::STAGEB];

  // ---- work assignment: balanced query-tile pairs, heads pinned to XCDs ----
  // Query tile i needs i+1 key-tile rows of the causal triangle, so a
  // workgroup takes the pair (nqt-1-p, p): every pair costs nqt+1 tile rows
  // (the middle tile of an odd nqt runs alone) and all workgroups of a launch
  // finish together.  Workgroups go to the 8 XCDs round-robin by id; when the
  // query head count is a multiple of 8, XCD x owns the consecutive heads
  // [x*hpx, (x+1)*hpx) of every sequence (else of the flattened batch), so
  // query heads of one KV group share its L2.
  // With a cached prefix every query tile costs about the same (the prefix
  // dominates), so a workgroup then takes a single tile: twice the workgroups.
  const int npair = PAIRED ? (nqt + 1) >> 1 : nqt;
  const int nbh = gridDim.x / npair;
  const int bid = blockIdx.x;
  int bh, pr;
  if ((Hq & 7) == 0) {
    // XCD x owns query heads [x*hpx, (x+1)*hpx) of every sequence, so that
    // sequences of different lengths load all XCDs alike
    const int hpx = Hq >> 3, nb = nbh / Hq;
    const int xcd = bid & 7, slot = bid >> 3;
    const int rest = slot / hpx;  // sequence fastest, then the pair
    bh = (rest % nb) * Hq + xcd * hpx + slot % hpx;
    pr = rest / nb;
  } else if ((nbh & 7) == 0) {
    const int hpx = nbh >> 3;
    const int xcd = bid & 7, slot = bid >> 3;
    bh = xcd * hpx + slot % hpx;
    pr = slot / hpx;
  } else {
    bh = bid % nbh;
    pr = bid / nbh;
  }
  const int b = bh / Hq, hq = bh % Hq;
  const int hk = hq / (Hq / Hkv);
  // Prompts of their own lengths (a padded batch): the pairs are formed over
  // each prompt's own query tiles (nqt_b of them), so that every working
  // workgroup of a prompt costs the same; workgroups past its pairs have
  // nothing to do (the K pass writes the padding rows' zeros), and the pair
  // index runs backwards, so that the highest pairs, which only the longest
  // prompts have, are dispatched first.
  int nqt_b = nqt;
  if constexpr (PAIRED && SRC == KEYS_PROMPT) {
    if (chunk_lens != nullptr) {
      nqt_b = (min(max(chunk_lens[b], 0), S) + C::BM - 1) / C::BM;
      pr = npair - 1 - pr;
      if (pr >= ((nqt_b + 1) >> 1)) return;  // uniform over the workgroup
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int grp = KSPLIT ? wave / C::WAVES : 0;  // key-range group
  const int wq = wave - grp * C::WAVES;           // wave within its group
  const int l32 = lane & 31, g = lane >> 5;
  // Keys: the prompt itself, or rows 0..P+S-1 of a cache that held P tokens
  // before this chunk; chunk query i sits at key index P+i.
  const int Sb = chunk_len<SRC>(chunk_lens, b, S);  // query rows >= Sb are padding
  const int P = chunk_start<SRC>(c, seq_lens, b, Sb);
  const int nkeys = P + Sb;
  // Keys and values that are INT8 codes: the key scales go into the query
  // and the value scales into the output, both in fp32.
  constexpr bool codes = SRC == KEYS_CODES;
  const bf16_t* kbase = nullptr;  // the head's key rows (paged: per block, below)
  const bf16_t* vbase = nullptr;
  if constexpr (SRC == KEYS_CONTIG || SRC == KEYS_CODES) {
    kbase = static_cast<const bf16_t*>(c.k) + ((int64_t)b * Hkv + hk) * c.max_seq * D;
    vbase = static_cast<const bf16_t*>(c.v) + ((int64_t)b * Hkv + hk) * c.max_seq * D;
  } else if constexpr (SRC == KEYS_PROMPT) {
    kbase = kr + ((int64_t)b * Hkv + hk) * S * D;
    vbase = v + ((int64_t)b * Hkv + hk) * S * D;
    // keys the K pass left in the cache only (at consecutive slots p0..), and
    // without k_rot every prompt's: rows p0.. of the cache, kept inside it
    // (positions that are not consecutive slots then give unspecified output)
    int p0;
    if (c.k != nullptr &&
        (prompt_rows_in_cache(positions, b, S, Sb, c.max_seq, &p0) || kr == nullptr)) {
      p0 = min(max(p0, 0), max(c.max_seq - Sb, 0));
      kbase = static_cast<const bf16_t*>(c.k) + (((int64_t)b * Hkv + hk) * c.max_seq + p0) * D;
    }
  }

  // ---- direct buffer -> LDS loads of K and V tiles ----
  // Load i of this wave fills LDS bytes [n KB, (n+1) KB) of a tile (n =
  // wave*IPW + i): lane l lands at chunk position l%CPR of tile row
  // n*RPI + l/CPR and so fetches that row's logical chunk stored there.  A
  // whole tile needs only the per-lane offsets within the tile plus the
  // tile's start as a scalar offset; in the last, partial tile the rows past
  // the end re-read the last key row (finite values; those keys are masked).
  // K and V have two buffers each: K holds tiles t+1 and t+2 while V holds t
  // and t+1 (the QK^T of tile t+1 is issued before the softmax of tile t).
  // In a paged cache each load's RPI rows lie in one 16-token block (tiles
  // and loads are aligned to RPI, which divides 16), so a load addresses that
  // block alone.  The block ids of a tile are read from the table one
  // pipeline step before its first load, into lanes (lane j: the tile's j-th
  // block), so the load takes its id with a v_readlane instead of waiting on
  // a scalar table read; the wait for that vector read is the per-step wait
  // for the tile loads.
  const uint32_t head_bytes = (uint32_t)nkeys * C::ROWB;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, head_bytes);
  uint32_t dma_off[C::IPW];
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    const int row = (wq * C::IPW + i) * C::RPI + lane / C::CPR;
    dma_off[i] = row * C::ROWB + (logical_chunk<C::CPR>(lane % C::CPR, row) << 4);
  }
  const int32_t* const trow = SRC == KEYS_PAGED ? c.table + (int64_t)b * c.mbps : nullptr;
  // lane j's block id of the tile starting at key j0 (clamped to the keys and the pool)
  auto block_ids = [&](int j0) -> int {
    if constexpr (SRC == KEYS_PAGED) {
      const int jb = min(j0 + 16 * (lane % (C::BN / 16)), nkeys - 1);
      return min(max(trow[jb >> 4], 0), c.num_blocks - 1);
    } else {
      return 0;
    }
  };
  auto issue = [&](__amdgpu_buffer_rsrc_t rs, const void* pool, int j0, char* dst, int ids) {
    if constexpr (SRC == KEYS_PAGED) {
      static_assert(16 % C::RPI == 0 && C::BN % 16 == 0, "a load stays inside one block");
#pragma unroll
      for (int i = 0; i < C::IPW; ++i) {
        const int r0 = (wq * C::IPW + i) * C::RPI;  // first tile row of this load
        const int row = r0 + lane / C::CPR;
        const int j = min(j0 + row, nkeys - 1);        // rows past the end: the last key
        // the load's block (uniform); rows past the end keep the last key's block
        const int blk = __builtin_amdgcn_readlane(ids, min(r0, nkeys - 1 - j0) >> 4);
        const bf16_t* bp = static_cast<const bf16_t*>(pool) + (((int64_t)blk * Hkv + hk) << 4) * D;
        const uint32_t off = (j & 15) * C::ROWB + (logical_chunk<C::CPR>(lane % C::CPR, row) << 4);
        dma16(make_rsrc(bp, 16 * C::ROWB), off, 0, dst + (wq * C::IPW + i) * 1024);
      }
    } else if (j0 + C::BN <= nkeys) {  // uniform
      (void)ids;
#pragma unroll
      for (int i = 0; i < C::IPW; ++i)
        dma16(rs, dma_off[i], (uint32_t)j0 * C::ROWB, dst + (wq * C::IPW + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < C::IPW; ++i) {
        const int row = (wq * C::IPW + i) * C::RPI + lane / C::CPR;
        const uint32_t off = min(j0 + row, nkeys - 1) * C::ROWB +
                             (logical_chunk<C::CPR>(lane % C::CPR, row) << 4);
        dma16(rs, off, 0, dst + (wq * C::IPW + i) * 1024);
      }
    }
  };
  char* const kbuf = smem + grp * 2 * C::STAGEB;  // [2][TILEB] of this group
  char* const vbuf = kbuf + 2 * C::TILEB;         // [2][TILEB]

  // ---- per-lane LDS read offsets (bytes within a tile) ----
  // K operand (S^T = K Q^T, A = K rows): row kb*32 + l32, chunk 2*kk + g.
  int koff[C::QKS];
#pragma unroll
  for (int kk = 0; kk < C::QKS; ++kk)
    koff[kk] = l32 * C::ROWB + (phys_chunk<C::CPR>(2 * kk + g, l32) << 4);
  // V operand (O^T = V^T P^T, A = V^T) by transposing reads: lane 16*qd + s
  // points at row kk*16 + 8h + 4*(lane/32) + s/4, dims db*32 + 16*(qd%2) + 4*(s%4)
  // (4 values); after the transpose the lane holds V[kk*16 + 8h + 4g + j][db*32 + l32].
  int voff[C::NDB][2];
  {
    const int qd = lane >> 4, s = lane & 15;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + 4 * g + (s >> 2);  // + kk*16 (phys_chunk ignores r >= 16)
        const int col = db * 32 + 16 * (qd & 1) + 4 * (s & 3);
        const int chunk = col >> 3;
        voff[db][h] = row * C::ROWB + (phys_chunk<C::CPR>(chunk, row) << 4) + ((col & 7) << 1);
      }
  }

  // ---- values into the cache (paired form, vstore != 0) ----
  // The K pass then stores only the keys: each 64- or 128-key value tile of
  // a KV head goes from LDS to the cache rows at the prompt's positions,
  // written by one workgroup, from the first query head of the KV group, in
  // its first (long) pass, while the tile sits in LDS anyway.  Pair p's long
  // pass reaches tiles [0, reach(p)), reach falling with p: tiles every pair
  // reaches go round-robin, and each higher tile to the last pair that still
  // reaches it, so that every pair stores about the same number.  Rows past
  // the prompt (padding, the clamped rows of a partial tile) and positions
  // outside the cache are not stored; prompts at consecutive slots p0.. need
  // no position reads.
  const int npair_b = PAIRED ? (nqt_b + 1) >> 1 : 1;
  const bool store_values = PAIRED && SRC == KEYS_PROMPT && vstore != 0 &&
                            hq % (Hq / Hkv) == 0;
  constexpr int TPQ = C::BM / C::BN;  // key tiles per query tile
  auto value_owner = [&](int t) {
    const int all = (nqt_b - npair_b + 1) * TPQ;  // tiles every pair's long pass reaches
    return t < all ? t % npair_b : nqt_b - 1 - t / TPQ;
  };
  int vp0 = 0;
  const bool v_consecutive = store_values && c.v != nullptr &&
                             prompt_rows_in_cache(positions, b, S, Sb, c.max_seq, &vp0);
  auto store_value_tile = [&](int t) {
    const char* vt = vbuf + (t & 1) * C::TILEB;
    bf16_t* const vc = static_cast<bf16_t*>(c.v) + ((int64_t)b * Hkv + hk) * c.max_seq * D;
    // the lane's chunk indices are formed here from a copy of the thread id
    // the compiler cannot see through, so that they hold no registers across
    // the key loop
    int tcopy = tid;
    asm volatile("" : "+v"(tcopy));
#pragma unroll
    for (int i = 0; i < C::TILEB / 16 / C::THREADS; ++i) {
      const int e = tcopy + i * C::THREADS;  // 16-byte chunk e of the tile
      const int r = e / C::CPR, ch = e % C::CPR;
      const int j = t * C::BN + r;
      if (j < Sb) {
        const int pos = v_consecutive ? vp0 + j : positions[(int64_t)b * S + j];
        if (pos >= 0 && pos < c.max_seq) {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(
              vt + r * C::ROWB + (phys_chunk<C::CPR>(ch, r) << 4));
          *reinterpret_cast<u32x4_t*>(vc + (int64_t)pos * D + ch * 8) = x;
        }
      }
    }
  };

  // ---- the pair's two query tiles, longest first ----
#pragma nounroll
  for (int pass = 0; pass < 2; ++pass) {
    const int qt = !PAIRED ? pr : (pass == 0 ? nqt_b - 1 - pr : pr);
    if (pass == 1) {
      if (!PAIRED || qt == nqt_b - 1 - pr) break;  // one tile, or no partner
      __syncthreads();                // every wave is done with the LDS tiles
    }
    const int q0 = qt * C::BM;
    const int qw = q0 + wq * 32;               // first query row of this wave
    const int qrow = qw + l32;                 // this lane's query row
    if (q0 >= Sb) {  // padding rows only (uniform): zeros
      if (grp == 0 && qrow < S) {
        bf16_t* op = out + ((int64_t)bh * S + qrow) * D;
  #pragma unroll
        for (int db = 0; db < C::NDB; ++db)
  #pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<u32x2_t*>(op + db * 32 + 8 * r4 + 4 * g) = u32x2_t{0u, 0u};
      }
      continue;
    }
    const int qrc = min(qrow, Sb - 1);

    // ---- Q rows, raw: their loads are issued before the first tiles' ----
    u32x4_t qraw[C::QKS];
    const bf16_t* qp = q + ((int64_t)bh * S + qrc) * D;
  #pragma unroll
    for (int ks = 0; ks < C::QKS; ++ks)
      qraw[ks] = *reinterpret_cast<const u32x4_t*>(qp + ks * 16 + g * 8);

    const int q_end = min(q0 + C::BM, Sb);  // exclusive
    const int ntiles = (P + q_end + C::BN - 1) / C::BN;
    // tiles 0..wlast hold keys visible to this wave (uniform per wave)
    const int wlast = min(ntiles - 1, (P + qw + 31) / C::BN);
    // this wave's group walks tiles tbeg .. tbeg+tcnt-1; the lambdas below
    // take the local index t - tbeg, which also picks the LDS buffers
    const int nt0 = KSPLIT ? (ntiles + 1) >> 1 : ntiles;  // steps of the launch
    const int tbeg = grp == 0 ? 0 : nt0;
    const int tcnt = grp == 0 ? nt0 : ntiles - nt0;
    const int ulast = min(wlast - tbeg, tcnt - 1);  // local index of the last visible tile

    int ids_v = 0, ids_k = 0;
    // first tiles K(0), V(0) and K(1), issued while the Q rows are in flight
    if (tcnt > 0) {
      const int ids0 = block_ids(tbeg * C::BN);
      issue(krs, c.k, tbeg * C::BN, kbuf, ids0);
      issue(vrs, c.v, tbeg * C::BN, vbuf, ids0);
      if (tcnt > 1) {
        ids_v = block_ids((tbeg + 1) * C::BN);
        issue(krs, c.k, (tbeg + 1) * C::BN, kbuf + C::TILEB, ids_v);
      }
      if (tcnt > 2) ids_k = block_ids((tbeg + 2) * C::BN);
    }

    // ---- Q fragments (B operand of S^T = K Q^T), rotated, bf16 ----
    bf16x8_t qf[C::QKS];
    {
      const int pos = SRC == KEYS_PROMPT ? positions[(int64_t)b * S + qrc] : P + qrc;
  #pragma unroll
      for (int ks = 0; ks < C::QKS; ++ks) {
        const int d0 = ks * 16 + g * 8;
        float f[8];
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = bf16_lo(qraw[ks][e]);
          f[2 * e + 1] = bf16_hi(qraw[ks][e]);
        }
        rope_rotate_chunk<bf16_t, 8, HALF>(f, qp, d0, D, pos, fr);
        if constexpr (codes) {  // keys are codes: q'.(code * s) = (q' * s).code
  #pragma unroll
          for (int e = 0; e < 8; ++e) f[e] *= c.k_scale[hk * D + d0 + e];
        }
        const u32x4_t u = {cvt_pk_bf16(f[0], f[1]), cvt_pk_bf16(f[2], f[3]),
                           cvt_pk_bf16(f[4], f[5]), cvt_pk_bf16(f[6], f[7])};
        qf[ks] = __builtin_bit_cast(bf16x8_t, u);
      }
    }

    f32x16_t oacc[C::NDB];
  #pragma unroll
    for (int db = 0; db < C::NDB; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t sacc[2][C::NKB];  // S^T of the tile being consumed and of the next one

    // S^T = K Q^T for the tile in K buffer kb_i: lane holds keys
    // kb*32 + 8*(r/4) + 4*g + r%4 of query qrow.  The two 32-key blocks are
    // interleaved so that consecutive MFMAs are independent.
    auto qk = [&](int kbi, auto SI) {
      constexpr int si = decltype(SI)::value;
      constexpr int NQ = C::QKS * C::NKB;
      const char* kt = kbuf + kbi * C::TILEB;
      // MFMA i: k-step i / NKB of 32-key block i % NKB; its K rows are read
      // two MFMAs ahead (a ring of three operand slots), in exactly this order
      auto load = [&](int i) {
        return *reinterpret_cast<const bf16x8_t*>(kt + (i % C::NKB) * 32 * C::ROWB +
                                                  koff[i / C::NKB]);
      };
      bf16x8_t ka[3];
      ka[0] = load(0);
      ka[1] = load(1);
      static_for<0, NQ>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i + 2 < NQ) ka[(i + 2) % 3] = load(i + 2);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int kk = i / C::NKB, kb = i % C::NKB;
        if constexpr (kk == 0)
          sacc[si][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf[0], f32x16_t{}, 0, 0, 0);
        else
          sacc[si][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf[kk], sacc[si][kb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // Online softmax of tile t (scores in sacc[si]) and O^T += V^T P^T with the
    // V tile in V buffer t&1.  The reference maximum m_run is only raised when
    // some row of the wave would otherwise see exp2 arguments above
    // kRescaleLog2 (weights up to 2^8): O and l always share the same
    // reference, so the result is exact while the rescale of O is skipped for
    // most tiles.
    auto softmax_pv = [&](int t, auto SI) {
      constexpr int si = decltype(SI)::value;
      const int j0 = (tbeg + t) * C::BN;
      if (j0 + C::BN - 1 > P + qw) {  // causal mask where the tile passes this wave's first row
  #pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > P + qrow) sacc[si][kb][r] = -INFINITY;
          }
      }
      // P (bf16) in the B-operand layout of O^T = V^T P^T against the
      // reference mc; lt sums the rounded P of this lane's keys
      bf16x8_t pf[C::PKS];
      float lt;
      auto make_p = [&](float mc) {
        lt = 0.f;
  #pragma unroll
        for (int kk = 0; kk < C::PKS; ++kk) {
          uint32_t pw[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = fast_exp2(fmaf(sacc[si][kk >> 1][8 * (kk & 1) + 2 * i], sm_scale_log2, -mc));
            const float p1 = fast_exp2(fmaf(sacc[si][kk >> 1][8 * (kk & 1) + 2 * i + 1], sm_scale_log2, -mc));
            pw[i] = cvt_pk_bf16(p0, p1);
            lt = dot2_bf16(pw[i], kOnePair, lt);
          }
          const u32x4_t u = {pw[0], pw[1], pw[2], pw[3]};
          pf[kk] = __builtin_bit_cast(bf16x8_t, u);
        }
      };
      // Fast path: P against the current reference m_run, kept unless some
      // lane's sum of it exceeds 2^kFastLog2 or is not finite (a score far
      // above m_run).  P up to that size is as exact in bf16 and as safe in
      // the fp32 sums as P up to 1, so the row maximum is only computed for
      // a wave's first tile and when the check fails.
      bool redo = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;  // first tile
      if (!redo) {
        make_p(m_run * sm_scale_log2);
        redo = __builtin_amdgcn_ballot_w64(!(lt <= kFastMax)) != 0;  // also NaN, inf
      }
      if (redo) {  // wave-uniform
        float mt = -INFINITY;
  #pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[si][kb][r]);
        mt = fmaxf(mt, swap_halves(mt));
        const bool grow = (mt - m_run) * sm_scale_log2 > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform branch
          const float m_new = fmaxf(m_run, mt);
          // (a row of key group 1 with no visible key so far keeps m = -inf and
          // alpha = 1 instead of exp2(-inf + inf))
          const float alpha = KSPLIT && m_new == -INFINITY
                                  ? 1.f
                                  : fast_exp2((m_run - m_new) * sm_scale_log2);
          m_run = m_new;
          l_run *= alpha;
  #pragma unroll
          for (int db = 0; db < C::NDB; ++db)
  #pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        // Such a row's P must be 0, not exp2(-inf + inf).
        make_p(KSPLIT && m_run == -INFINITY ? INFINITY : m_run * sm_scale_log2);
      }
      l_run += lt;

      // O^T += V^T P^T: operand i is k-step i / NDB (16 keys) of head-dim
      // block i % NDB, from two transposing reads.  At D = 128 the operands
      // are read two ahead (a ring of three slots) in exactly this order; at
      // D = 64 the compiler's order needs fewer registers.
      const char* vt = vbuf + (t & 1) * C::TILEB;
      constexpr int NP = C::PKS * C::NDB;
      auto load_v = [&](int i) {
        typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
        const char* base = vt + (i / C::NDB) * 16 * C::ROWB;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(base + voff[i % C::NDB][0]));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(base + voff[i % C::NDB][1]));
        const u32x2_t ul = __builtin_bit_cast(u32x2_t, lo);
        const u32x2_t uh = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t u = {ul[0], ul[1], uh[0], uh[1]};
        return __builtin_bit_cast(bf16x8_t, u);
      };
      auto mma_v = [&](bf16x8_t a, int i) {
        oacc[i % C::NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[i / C::NDB],
                                                                   oacc[i % C::NDB], 0, 0, 0);
      };
      if constexpr (D == 128) {
        bf16x8_t va[3];
        va[0] = load_v(0);
        va[1] = load_v(1);
        static_for<0, NP>([&](auto I) {
          constexpr int i = decltype(I)::value;
          if constexpr (i + 2 < NP) va[(i + 2) % 3] = load_v(i + 2);
          __builtin_amdgcn_sched_barrier(0);
          mma_v(va[i % 3], i);
          __builtin_amdgcn_sched_barrier(0);
        });
      } else {
  #pragma unroll
        for (int i = 0; i < NP; ++i) mma_v(load_v(i), i);
      }
    };

    // One pipeline step for tile t (S^T of tile t already issued into
    // sacc[SC]): make K(t+1) and V(t) visible, issue QK^T of tile t+1 into
    // sacc[SN], start the loads of K(t+2) and V(t+1), then softmax and P V of t.
    // Paged: block ids of tiles t+1 (V loads of step t), t+2 (K loads) and
    // t+3 (read during step t for the next step).
    // (t is the group's local tile index throughout.)
    auto step = [&](int t, auto SC, auto SN) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads landed
      __syncthreads();                     // everyone's loads landed; old buffers free
      if constexpr (PAIRED && SRC == KEYS_PROMPT) {
        if (store_values && pass == 0 && value_owner(t) == pr) store_value_tile(t);
      }
      // the next tiles' loads go out after the QK^T MFMAs: issued right
      // after the barrier, every wave's loads at once queue up in front of
      // the texture unit and stall the waves' issue
      if (t + 1 <= ulast) qk((t + 1) & 1, SN);
      if (t + 2 < tcnt)
        issue(krs, c.k, (tbeg + t + 2) * C::BN, kbuf + (t & 1) * C::TILEB, ids_k);
      if (t + 1 < tcnt)
        issue(vrs, c.v, (tbeg + t + 1) * C::BN, vbuf + ((t + 1) & 1) * C::TILEB, ids_v);
      if constexpr (SRC == KEYS_PAGED) {
        ids_v = ids_k;
        if (t + 3 < tcnt) ids_k = block_ids((tbeg + t + 3) * C::BN);
      }
      if (t <= ulast) softmax_pv(t, SC);
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // K(0) is visible; K(1) and V(0) may still be in flight (waited for in step 0)
    if (ulast >= 0) qk(0, S0{});
    for (int t = 0; t < nt0; t += 2) {
      step(t, S0{}, S1{});
      if (t + 1 < nt0) step(t + 1, S1{}, S0{});
    }

    if constexpr (KSPLIT) {
      // Group 1 hands its running maximum, sum and O to the wave of group 0
      // with the same query rows, lane by lane through LDS (the tile buffers
      // are free once every wave has passed the barrier); that wave merges
      // them by the online-softmax rule and stores the rows.  A wave of
      // group 1 that saw no visible key has m = -inf and contributes zero.
      constexpr int NV = C::NDB * 16 + 2;  // floats per lane
      float* const xo = reinterpret_cast<float*>(smem) + wq * NV * 64;
      __syncthreads();
      if (grp == 1) {
  #pragma unroll
        for (int db = 0; db < C::NDB; ++db)
  #pragma unroll
          for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = oacc[db][r];
        xo[(NV - 2) * 64 + lane] = m_run;
        xo[(NV - 1) * 64 + lane] = l_run;
      }
      __syncthreads();
      if (grp == 1) continue;  // (no later barrier: group 0 only merges and stores)
      const float m1 = xo[(NV - 2) * 64 + lane];
      const float m = fmaxf(m_run, m1);  // m_run is finite: key 0 is visible to every row
      const float a0 = fast_exp2((m_run - m) * sm_scale_log2);
      const float a1 = fast_exp2((m1 - m) * sm_scale_log2);
      l_run = l_run * a0 + xo[(NV - 1) * 64 + lane] * a1;
  #pragma unroll
      for (int db = 0; db < C::NDB; ++db)
  #pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[db][r] = oacc[db][r] * a0 + xo[(db * 16 + r) * 64 + lane] * a1;
    }

    // ---- normalise and store: lane holds query qrow, dims db*32+8*(r/4)+4g+r%4 ----
    const float l_tot = l_run + swap_halves(l_run);
    if (qrow < S) {
      const bool pad = qrow >= Sb;  // padding rows: zeros
      const float inv = 1.f / l_tot;
      bf16_t* op = out + ((int64_t)bh * S + qrow) * D;
  #pragma unroll
      for (int db = 0; db < C::NDB; ++db)
  #pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float o[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = oacc[db][4 * r4 + j] * inv;
          if constexpr (codes) {  // values are codes: sum p * (code * s) = s * sum p * code
  #pragma unroll
            for (int j = 0; j < 4; ++j) o[j] *= c.v_scale[hk * D + db * 32 + 8 * r4 + 4 * g + j];
          }
          u32x2_t u;
          u[0] = cvt_pk_bf16(o[0], o[1]);
          u[1] = cvt_pk_bf16(o[2], o[3]);
          if (pad) u = u32x2_t{0u, 0u};
          *reinterpret_cast<u32x2_t*>(op + db * 32 + 8 * r4 + 4 * g) = u;
        }
    }
  }
}

// Keys and values of one launch: the prompt's own (k_rot, v) or a cache.
struct KeySource {
  const void* k_rot;
  const void* v;
  CacheArgs c;
  const int32_t* seq_lens;
  const int32_t* chunk_lens;
  bool vstore;  // the paired form stores the values into c (contiguous, native bf16)
};

template <int D, int SRC, int HALF>
hipError_t prefill_f32_t(const void* q, const KeySource& ks, void* out, int B, int Hq, int Hkv,
                         int S, const int32_t* positions, const RopeFreq& fr, float scale,
                         hipStream_t st, const TimedLaunch& tl) {
  const dim3 grid((S + F32_ROWS - 1) / F32_ROWS, Hq, B);
  hipExtLaunchKernelGGL((prefill_f32_kernel<D, SRC, HALF>), grid, dim3(F32_ROWS), 0, st, tl.start,
                        tl.stop, 0, static_cast<const float*>(q),
                        static_cast<const float*>(ks.k_rot), static_cast<const float*>(ks.v),
                        static_cast<float*>(out), positions, Hq, Hkv, S, fr,
                        scale * 1.4426950408889634f, ks.c, ks.seq_lens, ks.chunk_lens);
  return hipGetLastError();
}

template <int D, int SRC, int HALF, int FORM>
hipError_t prefill_bf16_w(const void* q, const KeySource& ks, void* out, int B, int Hq, int Hkv,
                          int S, const int32_t* positions, const RopeFreq& fr, float scale,
                          hipStream_t st, const TimedLaunch& tl, bool vstore = false) {
  using C = Tile<D, FORM == FORM_SPLIT ? 4 : 8>;  // BM query rows per workgroup
  const int nqt = (S + C::BM - 1) / C::BM;
  const int npair = FORM == FORM_PAIR ? (nqt + 1) / 2 : nqt;  // workgroups per head
  hipExtLaunchKernelGGL((prefill_bf16_kernel<D, SRC, HALF, FORM>), dim3(npair * B * Hq), dim3(512), 0,
                        st, tl.start, tl.stop, 0, static_cast<const bf16_t*>(q),
                        static_cast<const bf16_t*>(ks.k_rot), static_cast<const bf16_t*>(ks.v),
                        static_cast<bf16_t*>(out), positions, Hq, Hkv, S, nqt, fr,
                        scale * 1.4426950408889634f, ks.c, ks.seq_lens, ks.chunk_lens,
                        vstore ? 1 : 0);
  return hipGetLastError();
}

// MI355X compute units: a whole prompt whose query-tile pairs number fewer
// than this runs in the split form instead.
constexpr int kComputeUnits = 256;

// Whether a bf16 prompt of this shape runs in the paired form.
bool paired_form(int B, int Hq, int S) {
  const int64_t pairs = (int64_t)((S + Tile<128, 8>::BM - 1) / Tile<128, 8>::BM + 1) / 2 * B * Hq;
  static_assert(Tile<128, 8>::BM == Tile<64, 8>::BM, "one query tile height");
  return pairs >= kComputeUnits;
}

template <int D, int SRC, int HALF>
hipError_t prefill_bf16_t(const void* q, const KeySource& ks, void* out, int B, int Hq, int Hkv,
                          int S, const int32_t* positions, const RopeFreq& fr, float scale,
                          hipStream_t st, const TimedLaunch& tl) {
  if constexpr (SRC == KEYS_PROMPT) {
    if (paired_form(B, Hq, S))
      return prefill_bf16_w<D, SRC, HALF, FORM_PAIR>(q, ks, out, B, Hq, Hkv, S, positions, fr,
                                                     scale, st, tl, ks.vstore);
  }
  return prefill_bf16_w<D, SRC, HALF, FORM_SPLIT>(q, ks, out, B, Hq, Hkv, S, positions, fr, scale,
                                                  st, tl);
}

template <int SRC, int HALF>
hipError_t prefill_dispatch_t(Dtype dt, int D, const void* q, const KeySource& ks, void* out,
                              int B, int Hq, int Hkv, int S, const int32_t* positions,
                              const RopeFreq& fr, float scale, hipStream_t s,
                              const TimedLaunch& tl) {
  if (dt == F32)
    return D == 64
               ? prefill_f32_t<64, SRC, HALF>(q, ks, out, B, Hq, Hkv, S, positions, fr, scale, s, tl)
               : prefill_f32_t<128, SRC, HALF>(q, ks, out, B, Hq, Hkv, S, positions, fr, scale, s,
                                               tl);
  return D == 64
             ? prefill_bf16_t<64, SRC, HALF>(q, ks, out, B, Hq, Hkv, S, positions, fr, scale, s, tl)
             : prefill_bf16_t<128, SRC, HALF>(q, ks, out, B, Hq, Hkv, S, positions, fr, scale, s,
                                              tl);
}

// The RoPE pair layout is a compile-time choice of the kernels, so that the
// layout test stays out of their register allocation.
template <int SRC>
hipError_t prefill_dispatch(Dtype dt, int D, const void* q, const KeySource& ks, void* out,
                            int B, int Hq, int Hkv, int S, const int32_t* positions,
                            const RopeFreq& fr, float scale, hipStream_t s,
                            const TimedLaunch& tl) {
  return fr.half ? prefill_dispatch_t<SRC, 1>(dt, D, q, ks, out, B, Hq, Hkv, S, positions, fr,
                                              scale, s, tl)
                 : prefill_dispatch_t<SRC, 0>(dt, D, q, ks, out, B, Hq, Hkv, S, positions, fr,
                                              scale, s, tl);
}

}  // namespace

bool prefill_attention_stores_values(Dtype dt, int B, int Hq, int S, const CacheArgs* kcache) {
  return dt == BF16 && kcache != nullptr && paired_form(B, Hq, S);
}

hipError_t launch_prefill_attention(Dtype dt, int D, const void* q, const void* k_rot,
                                    const void* v, void* out, int B, int Hq, int Hkv, int S,
                                    const int32_t* positions, const int32_t* lens,
                                    const RopeFreq& fr, float scale, const CacheArgs* kcache,
                                    hipStream_t s, const TimedLaunch& tl) {
  // the fp32 kernel always reads k_rot (its K pass never skips it)
  const KeySource ks{k_rot, v, kcache != nullptr && dt == BF16 ? *kcache : CacheArgs{}, nullptr,
                     lens, prefill_attention_stores_values(dt, B, Hq, S, kcache)};
  return prefill_dispatch<KEYS_PROMPT>(dt, D, q, ks, out, B, Hq, Hkv, S, positions, fr, scale, s,
                                       tl);
}

hipError_t launch_prefill_cached(Dtype dt, int D, bool paged, const void* q, void* out, int B,
                                 int Hq, int Hkv, int S, const CacheArgs& c,
                                 const int32_t* seq_lens, const int32_t* chunk_lens,
                                 const RopeFreq& fr, float scale, hipStream_t s,
                                 const TimedLaunch& tl) {
  const KeySource ks{nullptr, nullptr, c, seq_lens, chunk_lens, false};
  if (dt == BF16 && !paged && c.k_scale != nullptr) {  // a dense copy of INT8 codes
    if (D == 64)
      return fr.half ? prefill_bf16_t<64, KEYS_CODES, 1>(q, ks, out, B, Hq, Hkv, S, nullptr, fr,
                                                         scale, s, tl)
                     : prefill_bf16_t<64, KEYS_CODES, 0>(q, ks, out, B, Hq, Hkv, S, nullptr, fr,
                                                         scale, s, tl);
    return fr.half ? prefill_bf16_t<128, KEYS_CODES, 1>(q, ks, out, B, Hq, Hkv, S, nullptr, fr,
                                                        scale, s, tl)
                   : prefill_bf16_t<128, KEYS_CODES, 0>(q, ks, out, B, Hq, Hkv, S, nullptr, fr,
                                                        scale, s, tl);
  }
  return paged ? prefill_dispatch<KEYS_PAGED>(dt, D, q, ks, out, B, Hq, Hkv, S, nullptr, fr,
                                              scale, s, tl)
               : prefill_dispatch<KEYS_CONTIG>(dt, D, q, ks, out, B, Hq, Hkv, S, nullptr, fr,
                                               scale, s, tl);
}

}  // namespace car
