// car_attn_decode_noalloc (include/car.h): car_attn_decode with its split
// partials in a file-scope device array instead of a caller's workspace, for
// callers that cannot allocate device memory.  Same kernels, same results.
//
// Each GPU the library runs on holds its own copy of `scratch` (zero when the
// code object loads) until the process ends.  Its device address is looked up
// once per device, with that device current, on the first call that uses the
// device; kernels and every other host-side use take that address, never the
// array's host-side name.  Every call on one GPU shares the array: calls that
// overlap on a GPU (two streams, two threads) race on it.  Nothing in it has to
// start at zero: the split kernel writes every partial the merge reads.

#include <hip/hip_runtime.h>

#include <mutex>

#include "car.h"

namespace {

constexpr size_t kScratchBytes = CAR_DECODE_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, or null

// The device the call's work runs on: the stream's, or the current one for
// the null stream.
hipError_t call_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  *dev = static_cast<int>(d);
  return e;
}

// Address of `scratch` on `dev`, looked up on first use with `dev` current.
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" car_status car_attn_decode_noalloc(const void* q, const void* k_new,
                                              const void* v_new, void* out, car_dtype dtype,
                                              int B, int Hq, int Hkv, int D,
                                              const int32_t* seq_lens, int max_seq_len,
                                              float theta, car_rope_pairing pairing,
                                              float scale, const car_kv_cache* cache,
                                              hipStream_t stream) {
  // Sizes whose partials do not fit the array are refused before anything
  // else; invalid sizes (0 bytes) fall through to car_attn_decode's checks.
  if (car_attn_decode_workspace_bytes(B, Hq, D, max_seq_len) > kScratchBytes)
    return CAR_ERR_WORKSPACE;
  int dev = 0;
  if (call_device(stream, &dev) != hipSuccess) return CAR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CAR_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_on(dev, &ws) != hipSuccess) return CAR_ERR_HIP;
  return car_attn_decode(q, k_new, v_new, out, dtype, B, Hq, Hkv, D, seq_lens, max_seq_len,
                         theta, pairing, scale, cache, ws, kScratchBytes, stream);
}
