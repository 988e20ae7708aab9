// Host-side plans and launcher declarations inside libsdkv (not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/sdkv.h"
#include "sdkv_device.h"

namespace sdkv {

// Planning assumes an MI355X: 256 compute units. The same plan (and so the
// same workspace size) is used on any device.
constexpr int kPlanCUs = 256;
constexpr int kRowThreads = 1024;                             // select-bearing workgroups
constexpr int kMaxRowSPT = 32;                                // keys per thread
constexpr int64_t kMaxChunk = (int64_t)kRowThreads * kMaxRowSPT;  // 32768 tokens
// Rows split over several workgroups: at most 16 keys per thread. The row
// kernel with 32 keys per thread and the cross-workgroup select returned
// wrong selections on gfx950 (every row; correct at 16 keys per thread and
// with the single-workgroup select at 32), so it is not built.
constexpr int kMaxCoopSPT = 16;
constexpr int64_t kMaxCoopChunk = (int64_t)kRowThreads * kMaxCoopSPT;  // 16384 tokens
constexpr int kMaxRowP = 64;   // workgroups per decode row
constexpr int kMaxAtomsDecode = 32768;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct DecodePlan {
  int64_t rows = 0;      // B * Hq
  int64_t m = 0;         // selected tokens per row
  int P = 1;             // workgroups per row
  int64_t chunk = 0;     // tokens per workgroup
  int spt = 0;           // keys per thread (template instance)
  int fast = 0;          // K == 16, klow <= 4, khigh <= 16: vector code loads
  int wrt = 32;          // rows per W.Dv tile (32, or 64 for bf16 with > 32 rows)
  int nrt = 0;           // row tiles in the W.Dv kernel
  int nsub = 1;          // 128-atom sub-chunks per W.Dv workgroup
  int nchunks = 0;       // atom chunks in the W.Dv kernel
  // workspace byte offsets
  size_t off_u = 0, off_sel = 0, off_shigh = 0, off_wpart = 0, off_stats = 0;
  size_t off_zero = 0, zero_bytes = 0;  // [ghist | xchg | bar | err], cleared per call
  size_t off_ghist = 0, off_xchg = 0, off_bar = 0, off_err = 0, off_opart = 0;
  size_t off_cand = 0, off_ticket = 0, off_wtab = 0, off_ixchg = 0, off_ug = 0;
  size_t total = 0;
};

sdkv_status plan_decode(const sdkv_attn_args* a, DecodePlan* p);
sdkv_status launch_decode(const sdkv_attn_args* a, const DecodePlan& p, void* ws,
                          hipStream_t stream);

struct TopkPlan {
  int64_t rows = 0, n = 0, k = 0;
  int P = 1;
  int64_t chunk = 0;
  int spt = 0;
  size_t off_ghist = 0, off_xchg = 0, off_bar = 0, off_err = 0, zero_bytes = 0;
  size_t off_cand = 0, off_ticket = 0;
  size_t total = 0;
};
sdkv_status plan_topk(int64_t rows, int64_t n, int64_t k, TopkPlan* p);
sdkv_status launch_topk(const float* scores, int64_t ld, int32_t* idx, float* thr,
                        const TopkPlan& p, void* ws, hipStream_t stream);

struct EncodePlan {
  int64_t n = 0;
  int npad = 0;          // atoms padded to the sweep tile
  int rows_per_wg = 0;
  int64_t nwg = 0;
  size_t off_dh = 0, off_dn = 0, off_r = 0, off_rh = 0, off_scale = 0;
  int small = 0;         // n <= 64: fp32-accurate pursuit over the device
  int G = 0;             // small path: workgroups (atom slices)
  size_t off_part = 0;   // small path: per-workgroup winners [2][G][n]
  size_t off_omp = 0;    // small path, OMP: Q, R, z and support
  size_t total = 0;
};
sdkv_status plan_encode(const sdkv_encode_args* a, EncodePlan* p);
// Both problems on the small path, same n, d, n_atoms, K and dictionary dtype.
sdkv_status launch_encode_pair(const sdkv_encode_args* a0, const EncodePlan& p0, char* ws0,
                               const sdkv_encode_args* a1, const EncodePlan& p1, char* ws1,
                               hipStream_t stream);
sdkv_status launch_encode(const sdkv_encode_args* a, const EncodePlan& p, void* ws,
                          hipStream_t stream);
// Validation and plans of a paired small encode (sdkv_encode_pair): the
// second problem's scratch starts at byte off1, total bytes in *total.
sdkv_status plan_pair(const sdkv_encode_args* a0, const sdkv_encode_args* a1,
                      EncodePlan* p0, EncodePlan* p1, size_t* off1, size_t* total);

// Records caller-provided timing event i on `stream` (no-op without events).
inline bool record_stage(void* const* ev, int i, hipStream_t stream) {
  if (!ev) return true;
  return hipEventRecord((hipEvent_t)ev[i], stream) == hipSuccess;
}

// Bounds of the kernels' cross-workgroup waits, with `err` (workspace word
// 0) as the status word: the normal bound, or what sdkv_test_set_wait set.
WaitCtl wait_ctl(uint32_t* err);

// Largest number of co-resident workgroups for a kernel on the current device.
sdkv_status coresident_blocks(const void* kernel, int threads, size_t dyn_lds, int* out);

}  // namespace sdkv
