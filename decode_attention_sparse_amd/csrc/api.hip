// Exported C ABI of libsdkv (declared in include/sdkv.h): argument
// validation, workspace sizing and dispatch. Validation is complete before
// anything is enqueued, so an error leaves every output untouched. No
// exception escapes: every entry point is wrapped in a catch-all.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "sdkv_internal.h"

using namespace sdkv;

namespace sdkv {

// The co-residency capacity of a (kernel, block size, device) never changes,
// so it is computed once and cached. This small mutex-guarded cache and the
// wait bounds below (changed only by the test hook) are the library's only
// process-wide state.
namespace {
struct CapEntry {
  const void* kernel;
  int dev, threads, cap;
};
std::mutex g_cap_mu;
std::vector<CapEntry> g_cap;
}  // namespace

// Bounds of the cross-workgroup waits. Normal: 2^24 polls (each after an
// s_sleep of 64 clocks, ~0.5 s), nothing added to the arrival targets.
// sdkv_test_set_wait replaces both, so that tests can make every wait give
// up on purpose while every kernel still exits normally.
namespace {
constexpr uint32_t kWaitPolls = 1u << 24;
std::atomic<uint32_t> g_wait_polls{kWaitPolls};
std::atomic<uint32_t> g_wait_extra{0};
}  // namespace

WaitCtl wait_ctl(uint32_t* err) {
  WaitCtl w;
  w.err = err;
  w.limit = g_wait_polls.load(std::memory_order_relaxed);
  w.extra = g_wait_extra.load(std::memory_order_relaxed);
  return w;
}

sdkv_status coresident_blocks(const void* kernel, int threads, size_t dyn_lds, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SDKV_ERR_DEVICE;
  if (dyn_lds == 0) {
    std::lock_guard<std::mutex> lk(g_cap_mu);
    for (const CapEntry& e : g_cap)
      if (e.kernel == kernel && e.dev == dev && e.threads == threads) {
        *out = e.cap;
        return SDKV_OK;
      }
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SDKV_ERR_DEVICE;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess)
    return SDKV_ERR_DEVICE;
  *out = cus * per_cu;
  if (dyn_lds == 0) {
    std::lock_guard<std::mutex> lk(g_cap_mu);
    g_cap.push_back(CapEntry{kernel, dev, threads, *out});
  }
  return SDKV_OK;
}

}  // namespace sdkv

static bool valid_dtype(int32_t t) { return t == SDKV_BF16 || t == SDKV_F32; }
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static sdkv_status check_encode(const sdkv_encode_args* a) {
  if (!a || !a->x || !a->dict || !a->codes) return SDKV_ERR_NULL;
  if (!valid_dtype(a->x_dtype) || !valid_dtype(a->dict_dtype)) return SDKV_ERR_DTYPE;
  if (a->n < 1 || (a->d != 64 && a->d != 128)) return SDKV_ERR_SHAPE;
  if (a->n_atoms < 1 || a->n_atoms > 65536) return SDKV_ERR_SHAPE;
  if (a->K < 1 || a->K > 32) return SDKV_ERR_SHAPE;
  if (a->low_plane && (a->klow < 1 || a->klow > a->K)) return SDKV_ERR_SHAPE;
  if (a->codes_ld != 0 && (a->codes_ld < a->K || a->codes_ld > ((int64_t)1 << 40)))
    return SDKV_ERR_SHAPE;
  if (a->low_plane && a->low_ld != 0 && (a->low_ld < a->klow || a->low_ld > ((int64_t)1 << 40)))
    return SDKV_ERR_SHAPE;
  if (a->n > ((int64_t)1 << 40)) return SDKV_ERR_UNSUPPORTED;
  if (!aligned16(a->x) || !aligned16(a->dict)) return SDKV_ERR_UNSUPPORTED;
  if (a->algorithm != SDKV_ENCODE_PURSUIT && a->algorithm != SDKV_ENCODE_OMP) return SDKV_ERR_SHAPE;
  if (a->algorithm == SDKV_ENCODE_OMP && (a->n > 64 || a->dict_dtype != SDKV_BF16))
    return SDKV_ERR_UNSUPPORTED;
  return SDKV_OK;
}

static sdkv_status check_attn(const sdkv_attn_args* a) {
  if (!a || !a->q || !a->dk || !a->dv || !a->key_codes || !a->val_codes || !a->out)
    return SDKV_ERR_NULL;
  if (!valid_dtype(a->q_dtype) || !valid_dtype(a->dict_dtype)) return SDKV_ERR_DTYPE;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0) return SDKV_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return SDKV_ERR_SHAPE;
  if (a->T < 1 || a->T > 0x7FFFFFFF) return SDKV_ERR_SHAPE;
  if (a->n_atoms < 1 || a->n_atoms > 65536) return SDKV_ERR_SHAPE;
  if (a->K < 1 || a->K > 32) return SDKV_ERR_SHAPE;
  if (a->code_stride != 0 && (a->code_stride < a->K || a->code_stride > 65536)) return SDKV_ERR_SHAPE;
  if (a->klow < 1 || a->klow > a->khigh || a->khigh > a->K) return SDKV_ERR_SHAPE;
  if (a->top_num < 1 || a->top_den < a->top_num || a->top_den > 0x7FFFFFFF) return SDKV_ERR_SHAPE;
  if (!isfinite(a->scale)) return SDKV_ERR_SHAPE;
  if (a->softmax_mode != SDKV_SOFTMAX_FLOAT && a->softmax_mode != SDKV_SOFTMAX_INT)
    return SDKV_ERR_SHAPE;
  if (a->select_mode != SDKV_SELECT_HEAD && a->select_mode != SDKV_SELECT_KV)
    return SDKV_ERR_SHAPE;
  if (a->reading != SDKV_READING_A && a->reading != SDKV_READING_B) return SDKV_ERR_SHAPE;
  if (a->n_atoms > kMaxAtomsDecode) return SDKV_ERR_UNSUPPORTED;
  if ((int64_t)a->B * a->Hq > 0x7FFFFFFF / 64) return SDKV_ERR_UNSUPPORTED;
  if (!aligned16(a->q) || !aligned16(a->dk) || !aligned16(a->dv)) return SDKV_ERR_UNSUPPORTED;
  if (a->reading == SDKV_READING_B && a->softmax_mode != SDKV_SOFTMAX_FLOAT)
    return SDKV_ERR_UNSUPPORTED;
  return SDKV_OK;
}

namespace sdkv {
sdkv_status plan_pair(const sdkv_encode_args* a0, const sdkv_encode_args* a1,
                      EncodePlan* p0, EncodePlan* p1, size_t* off1, size_t* total) {
  sdkv_status s = check_encode(a0);
  if (s != SDKV_OK) return s;
  s = check_encode(a1);
  if (s != SDKV_OK) return s;
  if (a0->n != a1->n || a0->d != a1->d || a0->n_atoms != a1->n_atoms || a0->K != a1->K ||
      a0->dict_dtype != a1->dict_dtype || a0->algorithm != a1->algorithm)
    return SDKV_ERR_SHAPE;
  if ((s = plan_encode(a0, p0)) != SDKV_OK || (s = plan_encode(a1, p1)) != SDKV_OK) return s;
  if (!p0->small || !p1->small) return SDKV_ERR_UNSUPPORTED;
  *off1 = align_up(p0->total, 256);
  *total = *off1 + p1->total;
  return SDKV_OK;
}
}  // namespace sdkv

extern "C" {

int32_t sdkv_abi_version(void) { return SDKV_ABI_VERSION; }

void sdkv_test_set_wait(uint32_t polls, uint32_t extra) {
  g_wait_polls.store(polls ? polls : kWaitPolls, std::memory_order_relaxed);
  g_wait_extra.store(extra, std::memory_order_relaxed);
}

const char* sdkv_status_str(sdkv_status s) {
  switch (s) {
    case SDKV_OK: return "ok";
    case SDKV_ERR_NULL: return "required pointer is NULL";
    case SDKV_ERR_SHAPE: return "size or count out of range";
    case SDKV_ERR_DTYPE: return "unknown dtype code";
    case SDKV_ERR_UNSUPPORTED: return "valid arguments outside the supported range";
    case SDKV_ERR_WORKSPACE: return "workspace too small";
    case SDKV_ERR_DEVICE: return "HIP runtime or launch error";
    case SDKV_ERR_WAIT: return "a cross-workgroup wait gave up (workgroups not co-resident)";
    default: return "unknown status";
  }
}

int64_t sdkv_selected_count(int64_t T, int64_t top_num, int64_t top_den) {
  if (T < 1 || top_num < 1 || top_den < top_num || T > 0x7FFFFFFF || top_den > 0x7FFFFFFF) return 0;
  const int64_t m = (T * top_num + top_den - 1) / top_den;
  return std::max<int64_t>(1, std::min<int64_t>(T, m));
}

sdkv_status sdkv_encode_workspace(const sdkv_encode_args* args, size_t* bytes) {
  try {
    if (!bytes) return SDKV_ERR_NULL;
    sdkv_status s = check_encode(args);
    if (s != SDKV_OK) return s;
    EncodePlan p;
    s = plan_encode(args, &p);
    if (s != SDKV_OK) return s;
    *bytes = p.total;
    return SDKV_OK;
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_encode(const sdkv_encode_args* args, void* ws, size_t ws_bytes, void* stream) {
  try {
    sdkv_status s = check_encode(args);
    if (s != SDKV_OK) return s;
    EncodePlan p;
    s = plan_encode(args, &p);
    if (s != SDKV_OK) return s;
    if (p.total > 0 && !ws) return SDKV_ERR_NULL;
    if (ws_bytes < p.total) return SDKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return SDKV_ERR_UNSUPPORTED;
    return launch_encode(args, p, ws, (hipStream_t)stream);
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_encode_pair_workspace(const sdkv_encode_args* a0, const sdkv_encode_args* a1,
                                       size_t* bytes) {
  try {
    if (!bytes) return SDKV_ERR_NULL;
    EncodePlan p0, p1;
    size_t off1 = 0, total = 0;
    const sdkv_status s = plan_pair(a0, a1, &p0, &p1, &off1, &total);
    if (s != SDKV_OK) return s;
    *bytes = total;
    return SDKV_OK;
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_encode_pair(const sdkv_encode_args* a0, const sdkv_encode_args* a1, void* ws,
                             size_t ws_bytes, void* stream) {
  try {
    EncodePlan p0, p1;
    size_t off1 = 0, total = 0;
    const sdkv_status s = plan_pair(a0, a1, &p0, &p1, &off1, &total);
    if (s != SDKV_OK) return s;
    if (!ws) return SDKV_ERR_NULL;
    if (ws_bytes < total) return SDKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return SDKV_ERR_UNSUPPORTED;
    return launch_encode_pair(a0, p0, (char*)ws, a1, p1, (char*)ws + off1, (hipStream_t)stream);
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_decode_attn_workspace(const sdkv_attn_args* args, size_t* bytes) {
  try {
    if (!bytes) return SDKV_ERR_NULL;
    sdkv_status s = check_attn(args);
    if (s != SDKV_OK) return s;
    DecodePlan p;
    s = plan_decode(args, &p);
    if (s != SDKV_OK) return s;
    *bytes = p.total;
    return SDKV_OK;
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_decode_attn(const sdkv_attn_args* args, void* ws, size_t ws_bytes, void* stream) {
  try {
    sdkv_status s = check_attn(args);
    if (s != SDKV_OK) return s;
    DecodePlan p;
    s = plan_decode(args, &p);
    if (s != SDKV_OK) return s;
    if (!ws) return SDKV_ERR_NULL;
    if (ws_bytes < p.total) return SDKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return SDKV_ERR_UNSUPPORTED;
    return launch_decode(args, p, ws, (hipStream_t)stream);
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_select_topk_workspace(int64_t rows, int64_t n, int64_t k, size_t* bytes) {
  try {
    if (!bytes) return SDKV_ERR_NULL;
    if (rows < 1 || n < 1 || k < 1 || k > n) return SDKV_ERR_SHAPE;
    if (n > ((int64_t)1 << 23) || rows > 0x7FFFFFFF) return SDKV_ERR_UNSUPPORTED;
    TopkPlan p;
    sdkv_status s = plan_topk(rows, n, k, &p);
    if (s != SDKV_OK) return s;
    *bytes = p.total;
    return SDKV_OK;
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

sdkv_status sdkv_select_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k,
                             int32_t* idx_out, float* thr_out, void* ws, size_t ws_bytes,
                             void* stream) {
  try {
    if (!scores || !idx_out) return SDKV_ERR_NULL;
    if (rows < 1 || n < 1 || k < 1 || k > n || ld < n) return SDKV_ERR_SHAPE;
    if (n > ((int64_t)1 << 23) || rows > 0x7FFFFFFF) return SDKV_ERR_UNSUPPORTED;
    TopkPlan p;
    sdkv_status s = plan_topk(rows, n, k, &p);
    if (s != SDKV_OK) return s;
    if (!ws) return SDKV_ERR_NULL;
    if (ws_bytes < p.total) return SDKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return SDKV_ERR_UNSUPPORTED;
    return launch_topk(scores, ld, idx_out, thr_out, p, ws, (hipStream_t)stream);
  } catch (...) {
    return SDKV_ERR_DEVICE;
  }
}

}  // extern "C"
