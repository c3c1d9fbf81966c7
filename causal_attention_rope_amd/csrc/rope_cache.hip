// RoPE and KV-cache stores: the bandwidth-bound elementwise kernels.
//
// Each thread moves 16-byte vectors (8 bf16 or 4 fp32 values, i.e. 4 or 2
// RoPE pairs) in a grid-stride loop; consecutive threads take consecutive
// vectors of a row, so every wave reads and writes whole 256-512 byte rows.
//
// RoPE follows [Intuition] ("手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉")
// §4: adjacent pairs (x[2i], x[2i+1]) rotated by m * theta^(-2i/D).  The cache
// store follows [Scratch] ("从零手搓AI推理引擎") §3.2: a token is written at the
// cache index equal to its position; paged caches resolve the index through
// the block table as in [NanoVLLM] ("以 Nano-vLLM 为例，深入理解 LLM 推理引擎（Part 2）")
// §05, 5.3.  An INT8 cache ([Intuition] §2: a cache compressed from 16-bit
// floats to INT8) stores codes with per-(KV head, channel) scales ([Scratch]
// §2.2, §5.3); its scales come from absmax_kernel over a calibration batch.
#include "common.hpp"

namespace car {

namespace {

constexpr int kThreads = 256;

inline int grid_for(int64_t nvec) {
  const int64_t blocks = (nvec + kThreads - 1) / kThreads;
  return (int)(blocks < 16384 ? (blocks > 0 ? blocks : 1) : 16384);
}

// HALF: pairs (i, i + D/2): a thread takes one 16-byte chunk of the first
// half of a row and its partner chunk in the second half (nvec counts those
// chunk pairs); otherwise one chunk of adjacent pairs (nvec counts chunks).
template <typename T, int D, bool HALF>
__global__ __launch_bounds__(kThreads) void rope_apply_kernel(T* __restrict__ x,
                                                              const int32_t* __restrict__ positions,
                                                              int H, int S, int64_t nvec,
                                                              RopeFreq fr) {
  constexpr int N = Vec16<T>::N;
  constexpr int VPR = HALF ? D / N / 2 : D / N;  // work items per row
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / VPR;
    const int col = (int)(i % VPR) * N;
    const int s = (int)(row % S);
    const int b = (int)(row / ((int64_t)S * H));
    const int pos = positions[(int64_t)b * S + s];
    T* p = x + row * D + col;
    float f[N];
    load16<T>(p, f);
    if constexpr (HALF) {
      float h[N], a[N];
      load16<T>(p + D / 2, h);
#pragma unroll
      for (int j = 0; j < N; ++j) a[j] = f[j];
      rope_rotate_half_chunk<N>(f, h, pos, col, D, fr);
      rope_rotate_half_chunk<N>(h, a, pos, col + D / 2, D, fr);
      store16<T>(p + D / 2, h);
    } else {
      rope_rotate_regs<N>(f, pos, col / 2, fr);
    }
    store16<T>(p, f);
  }
}

template <typename T, int D, bool PAGED, bool I8>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(CacheArgs c,
                                                             const T* __restrict__ k,
                                                             const T* __restrict__ v, int Hkv,
                                                             int S,
                                                             const int32_t* __restrict__ positions,
                                                             int64_t nvec) {
  constexpr int N = Vec16<T>::N;
  constexpr int VPR = D / N;
  const int last = cache_last_slot<PAGED>(c);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / VPR;
    const int col = (int)(i % VPR) * N;
    const int s = (int)(row % S);
    const int64_t bh = row / S;
    const int hk = (int)(bh % Hkv);
    const int b = (int)(bh / Hkv);
    const int pos = positions[(int64_t)b * S + s];
    if (pos < 0 || pos > last) continue;  // outside the cache: not stored
    const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, pos) * D + col;
    if constexpr (I8) {
      float kf[N], vf[N];
      load16<T>(k + row * D + col, kf);
      load16<T>(v + row * D + col, vf);
      store_int8<N>(static_cast<int8_t*>(c.k) + dst, kf, c.k_scale + hk * D + col);
      store_int8<N>(static_cast<int8_t*>(c.v) + dst, vf, c.v_scale + hk * D + col);
    } else {
      *reinterpret_cast<uint4*>(static_cast<T*>(c.k) + dst) =
          *reinterpret_cast<const uint4*>(k + row * D + col);
      *reinterpret_cast<uint4*>(static_cast<T*>(c.v) + dst) =
          *reinterpret_cast<const uint4*>(v + row * D + col);
    }
  }
}

// Rotate the prompt's keys once (dense copy for the attention kernel) and,
// with a cache, store rotated keys and raw values at their positions.
// KEYS_IN_CACHE (contiguous native cache): a prompt whose positions are
// consecutive slots of the cache gets no dense copy; the attention kernel
// reads its rotated keys from the cache rows instead.  store_v = 0 there:
// the attention kernel stores the values (it stages them in LDS anyway).
//
// Grid: (chunk blocks, groups of kPrepHeads KV heads, sequence).  A thread
// takes one 16-byte chunk of one token in each KV head of its group: the
// rotation angles depend only on the position and the chunk, so they are
// computed once for all those heads, and the row and chunk come from shifts
// instead of divisions by run-time sizes.
constexpr int kPrepHeads = 8;  // 2, 4 and 16 were slower at workload 3's shape
// chunk prep: a chunk has fewer tokens than a prompt, and one KV head per
// thread (more workgroups) measured faster than groups of 2, 4 or 8
constexpr int kChunkHeads = 1;
template <typename T, int D, bool PAGED, bool CACHE, bool I8, bool KEYS_IN_CACHE, int HALF>
__global__ __launch_bounds__(kThreads) void prefill_prep_kernel(
    CacheArgs c, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ k_rot,
    int Hkv, int S, const int32_t* __restrict__ positions, const int32_t* __restrict__ lens,
    RopeFreq fr, T* __restrict__ out, int G, int store_v) {
  constexpr int N = Vec16<T>::N;
  constexpr int VPR = D / N;
  const int hk0 = blockIdx.y * kPrepHeads, b = blockIdx.z;
  const int nh = min(kPrepHeads, Hkv - hk0);  // KV heads of this group
  const int n = lens == nullptr ? S : min(max(lens[b], 0), S);
  bool dense = k_rot != nullptr;  // the rotated keys also go to the dense copy
  if constexpr (KEYS_IN_CACHE) {
    int p0;
    if (dense && prompt_rows_in_cache(positions, b, S, n, c.max_seq, &p0)) dense = false;
  }
  const int items = S * VPR;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < items; i += gridDim.x * kThreads) {
    const int s = i / VPR;
    const int col = (i % VPR) * N;
    if (s >= n) {
      // padding: neither rotated nor stored; its output rows (the G query
      // heads of each KV head) are written as zeros here, since the attention
      // kernel visits only the query tiles that hold prompt tokens
#pragma unroll 1
      for (int g = 0; g < nh * G; ++g) {
        const int64_t hq = ((int64_t)b * Hkv + hk0) * G + g;
        *reinterpret_cast<uint4*>(out + (hq * S + s) * D + col) = make_uint4(0u, 0u, 0u, 0u);
      }
      continue;
    }
    const int pos = positions[(int64_t)b * S + s];
    // every head's chunk is loaded before any store (a store to the cache
    // could alias the next head's keys for all the compiler knows, which
    // would leave one load in flight per thread)
    uint4 raw[kPrepHeads], vraw[kPrepHeads];
    const bool in_cache = CACHE && pos >= 0 && pos <= cache_last_slot<PAGED>(c);
    const bool copy_v = in_cache && (I8 || store_v);  // the values are read here
#pragma unroll
    for (int j = 0; j < kPrepHeads; ++j) {  // (heads past the group's last read that one)
      const int64_t e0 = (((int64_t)b * Hkv + hk0 + min(j, nh - 1)) * S + s) * D + col;
      raw[j] = *reinterpret_cast<const uint4*>(k + e0);
      vraw[j] = copy_v ? *reinterpret_cast<const uint4*>(v + e0) : make_uint4(0u, 0u, 0u, 0u);
    }
    const RopeChunk<N> rot = rope_prepare<N, HALF>(pos, col, D, fr);
#pragma unroll
    for (int j = 0; j < kPrepHeads; ++j) {
      if (j >= nh) break;  // uniform over the block
      const int hk = hk0 + j;
      const int64_t row = ((int64_t)b * Hkv + hk) * S + s;
      float f[N];
#pragma unroll
      for (int e = 0; e < N; ++e) f[e] = elem<T>(raw[j], e);
      rope_apply_prepared<T, N, HALF>(f, k + row * D, D, rot, fr);
      if (dense) store16<T>(k_rot + row * D + col, f);
      if (in_cache) {  // else not stored
        const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, pos) * D + col;
        if constexpr (I8) {
          // the fp32 rotated key is quantized (not its rounded copy in k_rot)
          float vf[N];
#pragma unroll
          for (int e = 0; e < N; ++e) vf[e] = elem<T>(vraw[j], e);
          store_int8<N>(static_cast<int8_t*>(c.k) + dst, f, c.k_scale + hk * D + col);
          store_int8<N>(static_cast<int8_t*>(c.v) + dst, vf, c.v_scale + hk * D + col);
        } else {
          store16<T>(static_cast<T*>(c.k) + dst, f);
          if (store_v) *reinterpret_cast<uint4*>(static_cast<T*>(c.v) + dst) = vraw[j];
        }
      }
    }
  }
}

// A chunk continuing a cached prefix: token s of sequence b sits at position
// P + s, P = seq_lens[b]; its rotated key and raw value go to that index.  A
// chunk that does not fit the cache is not stored (the attention kernel then
// reads clamped rows and its output is unspecified).
// With chunk_lens, tokens s >= chunk_lens[b] are padding and are not stored.
// I8: an INT8 cache; the fp32 rotated key and the value are stored as codes.
template <typename T, int D, bool PAGED, bool I8, int HALF>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(
    CacheArgs c, const T* __restrict__ k, const T* __restrict__ v, int Hkv, int S,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ chunk_lens, RopeFreq fr) {
  // grid and per-thread work as prefill_prep_kernel: one chunk of one token
  // in each of kChunkHeads KV heads, with the angles computed once
  constexpr int N = Vec16<T>::N;
  constexpr int VPR = D / N;
  constexpr int kPrepHeads = kChunkHeads;
  const int hk0 = blockIdx.y * kPrepHeads, b = blockIdx.z;
  const int nh = min(kPrepHeads, Hkv - hk0);
  const int last = cache_last_slot<PAGED>(c);
  const int Sb = chunk_lens == nullptr ? S : min(max(chunk_lens[b], 0), S);
  const int P = seq_lens[b];
  if (P < 0 || P + Sb > last + 1) return;  // the chunk does not fit: not stored
  const int64_t items = (int64_t)Sb * VPR;  // padding rows s >= Sb are skipped
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * kThreads) {
    const int s = (int)(i / VPR);
    const int col = (int)(i % VPR) * N;
    const int pos = P + s;
    // every head's key and value chunks are loaded before any store
    uint4 raw[kPrepHeads], vraw[kPrepHeads];
#pragma unroll
    for (int j = 0; j < kPrepHeads; ++j) {  // (heads past the group's last read that one)
      const int64_t e0 = (((int64_t)b * Hkv + hk0 + min(j, nh - 1)) * S + s) * D + col;
      raw[j] = *reinterpret_cast<const uint4*>(k + e0);
      vraw[j] = *reinterpret_cast<const uint4*>(v + e0);
    }
    const RopeChunk<N> rot = rope_prepare<N, HALF>(pos, col, D, fr);
#pragma unroll
    for (int j = 0; j < kPrepHeads; ++j) {
      if (j >= nh) break;  // uniform over the block
      const int hk = hk0 + j;
      const int64_t row = ((int64_t)b * Hkv + hk) * S + s;
      float f[N];
#pragma unroll
      for (int e = 0; e < N; ++e) f[e] = elem<T>(raw[j], e);
      rope_apply_prepared<T, N, HALF>(f, k + row * D, D, rot, fr);
      const int64_t dst = cache_row<PAGED>(c, b, hk, Hkv, pos) * D + col;
      if constexpr (I8) {
        float vf[N];
#pragma unroll
        for (int e = 0; e < N; ++e) vf[e] = elem<T>(vraw[j], e);
        store_int8<N>(static_cast<int8_t*>(c.k) + dst, f, c.k_scale + hk * D + col);
        store_int8<N>(static_cast<int8_t*>(c.v) + dst, vf, c.v_scale + hk * D + col);
      } else {
        store16<T>(static_cast<T*>(c.k) + dst, f);
        *reinterpret_cast<uint4*>(static_cast<T*>(c.v) + dst) = vraw[j];
      }
    }
  }
}

// A chunk over an INT8 cache reads its keys and values through a dense copy:
// rows 0..P+n-1 of each sequence into contiguous [B, Hkv, max_seq, D] arrays
// dk, dv, which the chunk attention kernel then reads as its cache.  fp32:
// the dequantized values code * scale.  bf16: the codes themselves, exact in
// bf16 (integers of magnitude <= 127); the bf16 attention kernel applies the
// scales in fp32 instead (k_scale to the query, v_scale to the output), so
// that no dequantized value is rounded to bf16.  n is the chunk length
// (chunk_lens[b] or S) and P = seq_lens[b] lowered so that P + n <= max_seq:
// the same rows the attention kernel takes for a cache of max_seq slots.
// Rows from P+n on are not written (the attention never reads them).
template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void int8_dequant_rows_kernel(
    CacheArgs c, T* __restrict__ dk, T* __restrict__ dv, int Hkv, int S, int max_seq,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ chunk_lens,
    int64_t nvec) {
  constexpr int N = Vec16<T>::N;  // elements per 16 bytes of T (4 or 8 codes)
  constexpr int VPR = D / N;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / VPR;  // (b*Hkv + hk)*max_seq + t
    const int col = (int)(i % VPR) * N;
    const int t = (int)(row % max_seq);
    const int64_t bh = row / max_seq;
    const int hk = (int)(bh % Hkv);
    const int b = (int)(bh / Hkv);
    const int n = chunk_lens == nullptr ? S : min(max(chunk_lens[b], 0), S);
    const int P = max(min(max(seq_lens[b], 0), max_seq - n), 0);
    if (t >= P + n) continue;
    const int64_t src = cache_row<PAGED>(c, b, hk, Hkv, t) * D + col;
    uint32_t wk[N / 4], wv[N / 4];
    if constexpr (N == 4) {
      wk[0] = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(c.k) + src);
      wv[0] = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(c.v) + src);
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(c.k) + src);
      const uint2 e = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(c.v) + src);
      wk[0] = a.x, wk[1] = a.y, wv[0] = e.x, wv[1] = e.y;
    }
    float fk[N], fv[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      fk[j] = int8_elem(wk[j / 4], j % 4);
      fv[j] = int8_elem(wv[j / 4], j % 4);
      if constexpr (sizeof(T) == 4) {
        fk[j] *= c.k_scale[hk * D + col + j];
        fv[j] *= c.v_scale[hk * D + col + j];
      }
    }
    store16<T>(dk + row * D + col, fk);
    store16<T>(dv + row * D + col, fv);
  }
}

// Calibration of an INT8 cache ([Scratch] §2.2): per (KV head, channel), the
// absolute maximum over a batch of rotated keys and of values.  Workgroup
// (hk, y) scans a contiguous range of the B*S tokens of KV head hk, VPR lanes
// per row; the row groups are merged through LDS and each workgroup leaves
// one atomic maximum per channel on the fp32 bit patterns (ordered like the
// values, all being >= 0).  The arrays are zeroed before and divided by 127
// after (scale_finish_kernel).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const T* __restrict__ k,
                                                          const T* __restrict__ v, int Hkv,
                                                          int S,
                                                          const int32_t* __restrict__ positions,
                                                          int64_t rows, int64_t rows_per_block,
                                                          RopeFreq fr, uint32_t* __restrict__ kmax,
                                                          uint32_t* __restrict__ vmax) {
  constexpr int N = Vec16<T>::N;
  constexpr int VPR = D / N;          // lanes per row
  constexpr int RPI = kThreads / VPR;  // rows per pass of the workgroup
  __shared__ float red[2][RPI][D];
  const int hk = blockIdx.x;
  const int col = (int)(threadIdx.x % VPR) * N;
  const int rg = (int)(threadIdx.x / VPR);
  float km[N], vm[N];
#pragma unroll
  for (int j = 0; j < N; ++j) km[j] = vm[j] = 0.f;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  for (int64_t r = r0 + rg; r < r1; r += RPI) {
    const int b = (int)(r / S), s = (int)(r % S);
    const int64_t row = ((int64_t)b * Hkv + hk) * S + s;
    float f[N], g[N];
    load16<T>(k + row * D + col, f);
    rope_rotate_chunk<T, N>(f, k + row * D, col, D, positions[(int64_t)b * S + s], fr);
    load16<T>(v + row * D + col, g);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      km[j] = fmaxf(km[j], fabsf(f[j]));
      vm[j] = fmaxf(vm[j], fabsf(g[j]));
    }
  }
#pragma unroll
  for (int j = 0; j < N; ++j) {
    red[0][rg][col + j] = km[j];
    red[1][rg][col + j] = vm[j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * D; i += kThreads) {
    const int t = i / D, d = i % D;
    float m = 0.f;
#pragma unroll
    for (int g = 0; g < RPI; ++g) m = fmaxf(m, red[t][g][d]);
    atomicMax((t ? vmax : kmax) + (int64_t)hk * D + d, __float_as_uint(m));
  }
}

__global__ __launch_bounds__(kThreads) void scale_zero_kernel(uint32_t* __restrict__ a,
                                                              uint32_t* __restrict__ b, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) a[i] = b[i] = 0u;
}

// absmax bits -> absmax / 127 (one IEEE fp32 division)
__global__ __launch_bounds__(kThreads) void scale_finish_kernel(float* __restrict__ a,
                                                                float* __restrict__ b, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) {
    a[i] = __fdiv_rn(a[i], 127.f);
    b[i] = __fdiv_rn(b[i], 127.f);
  }
}

template <typename T, int D>
hipError_t int8_calibrate_t(const void* k, const void* v, int B, int Hkv, int S,
                            const int32_t* positions, const RopeFreq& fr, float* ks, float* vs,
                            hipStream_t st) {
  const int n = Hkv * D;
  const int gn = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(scale_zero_kernel, dim3(gn), dim3(kThreads), 0, st,
                     reinterpret_cast<uint32_t*>(ks), reinterpret_cast<uint32_t*>(vs), n);
  const int64_t rows = (int64_t)B * S;
  if (rows > 0) {
    const int64_t want = (rows + 255) / 256;  // >= 1
    const int64_t by = want < 1024 ? want : 1024;
    const int64_t rpb = (rows + by - 1) / by;
    const int gy = (int)((rows + rpb - 1) / rpb);
    hipLaunchKernelGGL((absmax_kernel<T, D>), dim3(Hkv, gy), dim3(kThreads), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), Hkv, S, positions,
                       rows, rpb, fr, reinterpret_cast<uint32_t*>(ks),
                       reinterpret_cast<uint32_t*>(vs));
  }
  hipLaunchKernelGGL(scale_finish_kernel, dim3(gn), dim3(kThreads), 0, st, ks, vs, n);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t rope_apply_t(void* x, int B, int H, int S, const int32_t* positions,
                        const RopeFreq& fr, hipStream_t st) {
  const int64_t rows = (int64_t)B * H * S;
  if (fr.half) {
    const int64_t nvec = rows * (D / Vec16<T>::N / 2);
    hipLaunchKernelGGL((rope_apply_kernel<T, D, true>), dim3(grid_for(nvec)), dim3(kThreads), 0,
                       st, static_cast<T*>(x), positions, H, S, nvec, fr);
  } else {
    const int64_t nvec = rows * (D / Vec16<T>::N);
    hipLaunchKernelGGL((rope_apply_kernel<T, D, false>), dim3(grid_for(nvec)), dim3(kThreads), 0,
                       st, static_cast<T*>(x), positions, H, S, nvec, fr);
  }
  return hipGetLastError();
}

template <typename T, int D, bool I8>
hipError_t kv_append_t(bool paged, const CacheArgs& c, const void* k, const void* v, int B,
                       int Hkv, int S, const int32_t* positions, hipStream_t st) {
  const int64_t nvec = (int64_t)B * Hkv * S * (D / Vec16<T>::N);
  const T* kk = static_cast<const T*>(k);
  const T* vv = static_cast<const T*>(v);
  if (paged)
    hipLaunchKernelGGL((kv_append_kernel<T, D, true, I8>), dim3(grid_for(nvec)), dim3(kThreads),
                       0, st, c, kk, vv, Hkv, S, positions, nvec);
  else
    hipLaunchKernelGGL((kv_append_kernel<T, D, false, I8>), dim3(grid_for(nvec)),
                       dim3(kThreads), 0, st, c, kk, vv, Hkv, S, positions, nvec);
  return hipGetLastError();
}

// (HALF: the pair layout, a compile-time choice of the prep kernels)
template <typename T, int D, bool I8, int HALF>
hipError_t prefill_prep_h(bool paged, const CacheArgs* cache, const void* k, const void* v,
                          void* k_rot, int B, int Hkv, int S, const int32_t* positions,
                          const int32_t* lens, const RopeFreq& fr, bool keys_in_cache,
                          bool store_v, void* out, int G, hipStream_t st) {
  T* const oo = static_cast<T*>(out);
  const T* kk = static_cast<const T*>(k);
  const T* vv = static_cast<const T*>(v);
  T* kr = static_cast<T*>(k_rot);
  if ((int64_t)B * Hkv * S == 0) return hipSuccess;
  // (B and Hkv <= Hq are at most 65535: the call checks them)
  const int64_t items = (int64_t)S * (D / Vec16<T>::N);
  const int64_t gx = (items + kThreads - 1) / kThreads;
  const dim3 grid((unsigned)(gx < 4096 ? gx : 4096), (Hkv + kPrepHeads - 1) / kPrepHeads, B);
  const dim3 block(kThreads);
  if (cache == nullptr) {
    CacheArgs none{};
    hipLaunchKernelGGL((prefill_prep_kernel<T, D, false, false, false, false, HALF>), grid, block, 0, st,
                       none, kk, vv, kr, Hkv, S, positions, lens, fr, oo, G, 1);
  } else if (paged) {
    hipLaunchKernelGGL((prefill_prep_kernel<T, D, true, true, I8, false, HALF>), grid, block, 0, st, *cache,
                       kk, vv, kr, Hkv, S, positions, lens, fr, oo, G, 1);
  } else if (!I8 && keys_in_cache) {
    hipLaunchKernelGGL((prefill_prep_kernel<T, D, false, true, false, true, HALF>), grid, block, 0, st,
                       *cache, kk, vv, kr, Hkv, S, positions, lens, fr, oo, G,
                       store_v ? 1 : 0);
  } else {
    hipLaunchKernelGGL((prefill_prep_kernel<T, D, false, true, I8, false, HALF>), grid, block, 0, st,
                       *cache, kk, vv, kr, Hkv, S, positions, lens, fr, oo, G, 1);
  }
  return hipGetLastError();
}

template <typename T, int D, bool I8>
hipError_t prefill_prep_t(bool paged, const CacheArgs* cache, const void* k, const void* v,
                          void* k_rot, int B, int Hkv, int S, const int32_t* positions,
                          const int32_t* lens, const RopeFreq& fr, bool keys_in_cache,
                          bool store_v, void* out, int G, hipStream_t st) {
  return fr.half ? prefill_prep_h<T, D, I8, 1>(paged, cache, k, v, k_rot, B, Hkv, S, positions,
                                                lens, fr, keys_in_cache, store_v, out, G, st)
                 : prefill_prep_h<T, D, I8, 0>(paged, cache, k, v, k_rot, B, Hkv, S, positions,
                                                lens, fr, keys_in_cache, store_v, out, G, st);
}

template <typename T, int D, int HALF>
hipError_t chunk_prep_h(bool paged, bool i8, const CacheArgs& c, const void* k, const void* v,
                        int B, int Hkv, int S, const int32_t* seq_lens,
                        const int32_t* chunk_lens, const RopeFreq& fr, hipStream_t st) {
  const T* kk = static_cast<const T*>(k);
  const T* vv = static_cast<const T*>(v);
  if ((int64_t)B * Hkv * S == 0) return hipSuccess;
  // (B and Hkv <= Hq are at most 65535: the call checks them)
  const int64_t gx = ((int64_t)S * (D / Vec16<T>::N) + kThreads - 1) / kThreads;
  const dim3 grid((unsigned)(gx < 4096 ? gx : 4096), (Hkv + kChunkHeads - 1) / kChunkHeads, B);
  const dim3 block(kThreads);
  if (i8) {
    if (paged)
      hipLaunchKernelGGL((chunk_prep_kernel<T, D, true, true, HALF>), grid, block, 0, st, c, kk, vv,
                         Hkv, S, seq_lens, chunk_lens, fr);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<T, D, false, true, HALF>), grid, block, 0, st, c, kk, vv,
                         Hkv, S, seq_lens, chunk_lens, fr);
  } else if (paged) {
    hipLaunchKernelGGL((chunk_prep_kernel<T, D, true, false, HALF>), grid, block, 0, st, c, kk, vv,
                       Hkv, S, seq_lens, chunk_lens, fr);
  } else {
    hipLaunchKernelGGL((chunk_prep_kernel<T, D, false, false, HALF>), grid, block, 0, st, c, kk, vv,
                       Hkv, S, seq_lens, chunk_lens, fr);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t chunk_prep_t(bool paged, bool i8, const CacheArgs& c, const void* k, const void* v,
                        int B, int Hkv, int S, const int32_t* seq_lens,
                        const int32_t* chunk_lens, const RopeFreq& fr, hipStream_t st) {
  return fr.half ? chunk_prep_h<T, D, 1>(paged, i8, c, k, v, B, Hkv, S, seq_lens, chunk_lens, fr, st)
                 : chunk_prep_h<T, D, 0>(paged, i8, c, k, v, B, Hkv, S, seq_lens, chunk_lens, fr, st);
}

template <typename T, int D>
hipError_t int8_dequant_t(bool paged, const CacheArgs& c, void* dk, void* dv, int B, int Hkv,
                          int S, int max_seq, const int32_t* seq_lens,
                          const int32_t* chunk_lens, hipStream_t st) {
  const int64_t nvec = (int64_t)B * Hkv * max_seq * (D / Vec16<T>::N);
  const dim3 grid(grid_for(nvec)), block(kThreads);
  if (paged)
    hipLaunchKernelGGL((int8_dequant_rows_kernel<T, D, true>), grid, block, 0, st, c,
                       static_cast<T*>(dk), static_cast<T*>(dv), Hkv, S, max_seq, seq_lens,
                       chunk_lens, nvec);
  else
    hipLaunchKernelGGL((int8_dequant_rows_kernel<T, D, false>), grid, block, 0, st, c,
                       static_cast<T*>(dk), static_cast<T*>(dv), Hkv, S, max_seq, seq_lens,
                       chunk_lens, nvec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_prep(Dtype dt, int D, bool paged, bool i8, const CacheArgs& c,
                             const void* k, const void* v, int B, int Hkv, int S,
                             const int32_t* seq_lens, const int32_t* chunk_lens,
                             const RopeFreq& fr, hipStream_t s) {
#define CAR_CHUNK(T, DD) \
  chunk_prep_t<T, DD>(paged, i8, c, k, v, B, Hkv, S, seq_lens, chunk_lens, fr, s)
  if (dt == F32) return D == 64 ? CAR_CHUNK(float, 64) : CAR_CHUNK(float, 128);
  return D == 64 ? CAR_CHUNK(bf16_t, 64) : CAR_CHUNK(bf16_t, 128);
#undef CAR_CHUNK
}

hipError_t launch_int8_dequant(Dtype dt, int D, bool paged, const CacheArgs& c, void* dk,
                               void* dv, int B, int Hkv, int S, int max_seq,
                               const int32_t* seq_lens, const int32_t* chunk_lens,
                               hipStream_t s) {
#define CAR_DEQ(T, DD) \
  int8_dequant_t<T, DD>(paged, c, dk, dv, B, Hkv, S, max_seq, seq_lens, chunk_lens, s)
  if (dt == F32) return D == 64 ? CAR_DEQ(float, 64) : CAR_DEQ(float, 128);
  return D == 64 ? CAR_DEQ(bf16_t, 64) : CAR_DEQ(bf16_t, 128);
#undef CAR_DEQ
}

hipError_t launch_rope_apply(Dtype dt, int D, void* x, int B, int H, int S,
                             const int32_t* positions, const RopeFreq& fr, hipStream_t s) {
  if (dt == F32)
    return D == 64 ? rope_apply_t<float, 64>(x, B, H, S, positions, fr, s)
                   : rope_apply_t<float, 128>(x, B, H, S, positions, fr, s);
  return D == 64 ? rope_apply_t<bf16_t, 64>(x, B, H, S, positions, fr, s)
                 : rope_apply_t<bf16_t, 128>(x, B, H, S, positions, fr, s);
}

hipError_t launch_kv_append(Dtype dt, int D, bool paged, bool i8, const CacheArgs& c,
                            const void* k, const void* v, int B, int Hkv, int S,
                            const int32_t* positions, hipStream_t s) {
  if (i8) {
    if (dt == F32)
      return D == 64 ? kv_append_t<float, 64, true>(paged, c, k, v, B, Hkv, S, positions, s)
                     : kv_append_t<float, 128, true>(paged, c, k, v, B, Hkv, S, positions, s);
    return D == 64 ? kv_append_t<bf16_t, 64, true>(paged, c, k, v, B, Hkv, S, positions, s)
                   : kv_append_t<bf16_t, 128, true>(paged, c, k, v, B, Hkv, S, positions, s);
  }
  if (dt == F32)
    return D == 64 ? kv_append_t<float, 64, false>(paged, c, k, v, B, Hkv, S, positions, s)
                   : kv_append_t<float, 128, false>(paged, c, k, v, B, Hkv, S, positions, s);
  return D == 64 ? kv_append_t<bf16_t, 64, false>(paged, c, k, v, B, Hkv, S, positions, s)
                 : kv_append_t<bf16_t, 128, false>(paged, c, k, v, B, Hkv, S, positions, s);
}

hipError_t launch_prefill_prep(Dtype dt, int D, bool paged, bool i8, const CacheArgs* cache,
                               const void* k, const void* v, void* k_rot, int B, int Hkv,
                               int S, const int32_t* positions, const int32_t* lens,
                               const RopeFreq& fr, bool keys_in_cache, bool store_v,
                               void* out, int G, hipStream_t s) {
#define CAR_PREP(T, DD, I)                                                             \
  prefill_prep_t<T, DD, I>(paged, cache, k, v, k_rot, B, Hkv, S, positions, lens, fr, \
                           keys_in_cache, store_v, out, G, s)
  if (i8 && cache != nullptr) {
    if (dt == F32) return D == 64 ? CAR_PREP(float, 64, true) : CAR_PREP(float, 128, true);
    return D == 64 ? CAR_PREP(bf16_t, 64, true) : CAR_PREP(bf16_t, 128, true);
  }
  if (dt == F32) return D == 64 ? CAR_PREP(float, 64, false) : CAR_PREP(float, 128, false);
  return D == 64 ? CAR_PREP(bf16_t, 64, false) : CAR_PREP(bf16_t, 128, false);
#undef CAR_PREP
}

hipError_t launch_int8_calibrate(Dtype dt, int D, const void* k, const void* v, int B, int Hkv,
                                 int S, const int32_t* positions, const RopeFreq& fr,
                                 float* k_scale, float* v_scale, hipStream_t s) {
  if (dt == F32)
    return D == 64 ? int8_calibrate_t<float, 64>(k, v, B, Hkv, S, positions, fr, k_scale, v_scale, s)
                   : int8_calibrate_t<float, 128>(k, v, B, Hkv, S, positions, fr, k_scale,
                                                  v_scale, s);
  return D == 64 ? int8_calibrate_t<bf16_t, 64>(k, v, B, Hkv, S, positions, fr, k_scale, v_scale, s)
                 : int8_calibrate_t<bf16_t, 128>(k, v, B, Hkv, S, positions, fr, k_scale,
                                                 v_scale, s);
}

}  // namespace car
