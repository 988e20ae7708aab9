// sdkv_encode_pair_noalloc: the decode-step append encode (sdkv_encode_pair)
// for callers that cannot allocate device memory. Its scratch (the pursuit's
// residuals and per-workgroup winners, and OMP's state) lives in one
// file-scope device array per GPU instead of a caller workspace.
//
// `scratch` is a device symbol: in host code its name is only a stand-in,
// never a device address. Its address on each device is looked up once, with
// that device current, by hipGetSymbolAddress, kept per device, and only
// that pointer is handed to the kernels. Every call on a GPU shares that
// GPU's array (the kernels write every scratch word before reading it, so
// nothing needs clearing between calls); calls that overlap in time on one
// GPU race on it.
#include <mutex>

#include "sdkv_internal.h"

namespace sdkv {

constexpr size_t kNoallocScratchBytes = SDKV_NOALLOC_SCRATCH_BYTES;  // 4 MiB per GPU

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// This device's scratch address (looked up on the first call on the device).
static sdkv_status scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SDKV_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return SDKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SDKV_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SDKV_OK;
}

}  // namespace sdkv

using namespace sdkv;

extern "C" {

sdkv_status sdkv_encode_pair_noalloc(const sdkv_encode_args* key, const sdkv_encode_args* val,
                                     void* stream) {
  try {
    EncodePlan p0, p1;
    size_t off1 = 0, total = 0;
    sdkv_status s = plan_pair(key, val, &p0, &p1, &off1, &total);
    if (s != SDKV_OK) return s;
    if (total > kNoallocScratchBytes) return SDKV_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((s = scratch_for_current_device(&ws)) != SDKV_OK) return s;
    return launch_encode_pair(key, p0, (char*)ws, val, p1, (char*)ws + off1, (hipStream_t)stream);
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

}  // extern "C"
