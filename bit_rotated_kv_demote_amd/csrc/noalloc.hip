// oscar_step_noalloc: the fused decode step with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid device allocation).  The kernels are oscar_step's; only where the
// workspace lives differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/oscar.h"

namespace {

// One copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device is ever passed on.
__device__ __align__(256) unsigned char scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current.  Returns OSCAR_ERR_HIP if the runtime
// cannot resolve it.
oscar_status scratch_for(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return OSCAR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[device] == nullptr) {
    int current = 0;
    if (hipGetDevice(&current) != hipSuccess) return OSCAR_ERR_HIP;
    if (current != device && hipSetDevice(device) != hipSuccess) return OSCAR_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device) (void)hipSetDevice(current);
    if (e != hipSuccess || p == nullptr) return OSCAR_ERR_HIP;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return OSCAR_OK;
}

}  // namespace

extern "C" oscar_status oscar_step_noalloc(const oscar_layer_desc* desc, const oscar_pool* pool,
                                           const int32_t* seq_slot, const int32_t* position, const void* k_new,
                                           const void* v_new, const void* q, float* out, int32_t batch,
                                           int32_t max_seq_len, void* stream) {
  if (!desc || batch <= 0 || max_seq_len < 1) return OSCAR_ERR_INVALID;
  const size_t need = oscar_step_workspace_bytes(desc, batch, max_seq_len);
  if (need == 0) return OSCAR_ERR_UNSUPPORTED;
  if (need > (size_t)OSCAR_NOALLOC_SCRATCH_BYTES) return OSCAR_ERR_CAPACITY;
  // the stream's device (the current device for the null stream)
  int device = 0;
  if (stream != nullptr) {
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &device) != hipSuccess) return OSCAR_ERR_INVALID;
  } else if (hipGetDevice(&device) != hipSuccess) {
    return OSCAR_ERR_HIP;
  }
  void* ws = nullptr;
  const oscar_status st = scratch_for(device, &ws);
  if (st != OSCAR_OK) return st;
  // No byte of the workspace has to start at any value: the step's append
  // launch writes the rotated queries and lengths, and the decode's split
  // launch writes every partial record the merge reads.
  return oscar_step(desc, pool, seq_slot, position, k_new, v_new, q, out, ws, (size_t)OSCAR_NOALLOC_SCRATCH_BYTES,
                    batch, max_seq_len, stream);
}
