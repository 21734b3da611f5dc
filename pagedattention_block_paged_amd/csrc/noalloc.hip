// pa_step_noalloc: pa_step for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). Its workspace is a fixed array in the library's own device
// memory, one per GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address, so
// the array's address on each device is looked up once, with that device
// current, and only that pointer is handed to kernels.
#include <mutex>

#include "pa_internal.h"

namespace {

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// The device address of `scratch` on device `dev`, looked up on the first call
// for that device (with the device made current, the caller's device restored
// afterwards). Later calls return the kept pointer or the kept error.
hipError_t scratch_on(int dev, void** out) {
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    int cur = 0;
    d.err = hipGetDevice(&cur);
    if (d.err != hipSuccess) return;
    if (cur != dev && (d.err = hipSetDevice(dev)) != hipSuccess) return;
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess) d.ptr = p;
    if (cur != dev) {
      const hipError_t e = hipSetDevice(cur);
      if (d.err == hipSuccess) d.err = e;
    }
  });
  *out = d.ptr;
  return d.err;
}

}  // namespace

extern "C" pa_status pa_step_noalloc(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                                     const pa_tensor* key_cache, const pa_tensor* value_cache,
                                     const pa_tensor* slot_mapping, const pa_tensor* block_tables,
                                     const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                                     const pa_tensor* context_lens, float scale, pa_stream stream) {
  int dev = 0;
  const hipError_t ge = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
  if (ge != hipSuccess) return pa::report(PA_ERR_HIP, "pa_step_noalloc: stream device: %s", hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices) return pa::report(PA_ERR_HIP, "pa_step_noalloc: device %d out of range", dev);
  void* ws = nullptr;
  const hipError_t se = scratch_on(dev, &ws);
  if (se != hipSuccess || !ws)
    return pa::report(PA_ERR_HIP, "pa_step_noalloc: scratch address on device %d: %s", dev, hipGetErrorString(se));
  const pa_status st = pa::step_impl(out, q, k, v, key_cache, value_cache, slot_mapping, block_tables,
                                     query_start_loc, seq_lens, context_lens, scale, false, 1.f, 1.f, ws,
                                     PA_NOALLOC_SCRATCH_BYTES, stream, false);
  if (st == PA_ERR_WORKSPACE)
    return pa::report(PA_ERR_WORKSPACE,
                      "pa_step_noalloc: this step needs more scratch than the library's fixed %llu bytes (%s); "
                      "use pa_step with a workspace of pa_attention_workspace_size() bytes",
                      static_cast<unsigned long long>(PA_NOALLOC_SCRATCH_BYTES), pa_last_error());
  return st;
}
