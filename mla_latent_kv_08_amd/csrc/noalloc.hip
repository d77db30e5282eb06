// mla_decode_attn_noalloc: mla_decode_attn for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts that
// forbid allocation). Its scratch (split-KV partials, their lse, the run plan)
// is a file-scope device array of fixed size instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla.h"

namespace {

// Largest scratch the entry point serves (MLA_NOALLOC_SCRATCH_BYTES): the
// workspace mla_decode_attn needs at its default split on a 256-compute-unit
// GPU (about 33 MiB of partials for one workgroup per compute unit) with
// room to spare.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;

// One copy per GPU, held until the process ends. In host code this name is a
// host-side stand-in, never a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device with that device current. Returns null on an error.
void* scratch_ptr() {
  static std::once_flag once[kMaxDevices];
  static void* ptrs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
    ptrs[dev] = p;
  });
  return ptrs[dev];
}

}  // namespace

extern "C" {

MLA_API int mla_decode_attn_noalloc(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo,
                                    const void* q_pe, const mla_kv_cache* cache, const int32_t* seq_lens,
                                    int32_t max_seq_len, float softmax_scale, void* x_lat, float* lse,
                                    const mla_decode_opts* opts, void* stream) {
  size_t need = 0;
  int st = mla_decode_workspace_size(dims, dtype, max_seq_len, opts, &need);
  if (st) return st;
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return MLA_ERR_HIP;
  return mla_decode_attn(dims, dtype, q_lat, q_lat_lo, q_pe, cache, seq_lens, max_seq_len, softmax_scale, x_lat, lse,
                         ws, kScratchBytes, opts, stream);
}

}  // extern "C"
