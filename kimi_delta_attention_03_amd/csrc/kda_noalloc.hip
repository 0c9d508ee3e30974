// kda_chunk_fwd_noalloc: the forward of kda_chunk_fwd with its workspace
// taken from a static device array that the library holds on every GPU it
// runs on, for callers that cannot allocate device memory.
//
// The array `scratch` below is a file-scope device variable; on the host its
// name is only a stand-in for the symbol. Its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) on the
// first call on that device and kept in a per-device table; kernels only
// ever receive that address. Nothing here allocates or frees memory.
//
// Every call on one device uses that device's single array, which keeps the
// last call's contents. The forward needs nothing in it cleared: the chunk map
// rewrites every table entry and stage 1+2 rewrites every record before stage
// 3+4 reads it. Calls that overlap on one device (different streams, or
// different threads) race on the array; callers must serialise them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kda.h"
#include "kda_kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// device address of this device's array (looked up once per device)
kda_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kda::fail_msg(KDA_ERR_HIP, "no current HIP device");
  if (dev >= kMaxDevices) return kda::fail_msg(KDA_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return kda::fail_msg(KDA_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                                            const void* g, const void* beta, const float* initial_state,
                                            const int32_t* cu_seqlens, void* o, float* final_state,
                                            hipStream_t stream) {
  size_t need = 0;
  kda_status s = kda_chunk_fwd_workspace_bytes(p, &need);
  if (s != KDA_OK) return s;
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
    return kda::fail_msg(KDA_ERR_WORKSPACE,
                         "problem needs %zu bytes of workspace, more than the %zu-byte static scratch of "
                         "kda_chunk_fwd_noalloc; use kda_chunk_fwd with a caller workspace",
                         need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != KDA_OK) return s;
  return kda_chunk_fwd(p, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state, ws,
                       (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}
