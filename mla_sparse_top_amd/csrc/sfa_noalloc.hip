// sfa_decode_noalloc: sfa_decode with its workspace in a fixed device array of this library
// instead of a caller buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in the code object: each GPU the library runs on holds its own copy, at its
// own address, until the process ends. Host code never passes the array's name to a kernel (on
// the host that name is only a stand-in, not a device address); the address comes from
// hipGetSymbolAddress, looked up once per device with that device current, and is cached.

#include <mutex>

#include <hip/hip_runtime.h>

#include "sfa.h"

namespace {

constexpr size_t kScratchBytes = SFA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, looked up on the first call for that device.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return SFA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SFA_ERR_HIP;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return SFA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev && hipSetDevice(prev) != hipSuccess) return SFA_ERR_HIP;
    if (e != hipSuccess || !p) return SFA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SFA_OK;
}

}  // namespace

extern "C" int sfa_decode_noalloc(const sfa_dims* dims, const void* query_nope, const void* query_rope,
                                  const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                                  const int32_t* topk_indices, const int32_t* block_table,
                                  const int32_t* kv_act_seqs, float softmax_scale, void* out, hipStream_t stream) {
  size_t need = 0;
  const int st = sfa_workspace_size(dims, 0, &need);
  if (st != SFA_OK) return st;
  if (need > kScratchBytes) return SFA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    // the stream's device, where the kernels run (the null stream belongs to the current one)
    if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
      return SFA_ERR_HIP;
    const int s2 = scratch_on(dev, &ws);
    if (s2 != SFA_OK) return s2;
  }
  return sfa_decode(dims, query_nope, query_rope, key_nope_2d, key_rope_2d, k_nope_scales, topk_indices,
                    block_table, kv_act_seqs, softmax_scale, out, ws, need, stream);
}
