// Stand-alone exact top-k select over fp32 score rows (the "top 10%" step of
// the review page's Summary of "LLM Inference in a Flash!", exposed alone).
// Output: indices of the k largest scores per row, ties to the lower index,
// ascending; optionally the k-th largest score.
#include "select_core.h"
#include "sdkv_internal.h"

namespace sdkv {

constexpr int kTopkMaxP = 256;

struct TopkArgs {
  const float* s;
  int64_t ld, n, k, chunk;
  int P, row0, nrows;
  int32_t* idx;
  float* thr;
  uint32_t* ghist;  // [rows, 2048]
  uint32_t* cand;   // [rows, P, chunk]
  uint32_t* xchg;   // [rows, P, 2]
  uint32_t* bar;    // [rows, 2] barrier counters
  WaitCtl wait;     // status word (workspace word 0) and wait bounds
  uint32_t* ticket; // [8] workgroup start-order counters (see k_rows)
  int xcd_map;
};

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

template <int SPT>
__global__ __launch_bounds__(SB) void k_topk(TopkArgs a) {
  __shared__ SelShared sh;
  __shared__ uint32_t s_qcnt[5 * kTopkMaxP + 1];
  const int tid = threadIdx.x;
  // rows are assigned in workgroup start order, as in the decode row kernel
  __shared__ int s_tile;
  if (tid == 0) s_tile = ticket_tile(a.ticket, a.nrows * a.P, a.xcd_map != 0);
  __syncthreads();
  const int L = s_tile;
  const int p = L % a.P;
  const int64_t row = a.row0 + L / a.P;
  const int64_t t0 = (int64_t)p * a.chunk;
  const int64_t t1 = min(a.n, t0 + a.chunk);
  const float* src = a.s + row * a.ld;
  uint32_t key[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int64_t t = t0 + (int64_t)j * SB + tid;
    key[j] = (t < t1) ? float_key(src[t]) : 0u;
  }
  SelGroup grp;
  grp.P = a.P;
  grp.p = p;
  grp.ghist = a.ghist + row * 2048;
  grp.xchg = a.xchg + row * a.P * 2;
  grp.bar = a.bar + 2 * (int64_t)row;
  grp.local = a.xcd_map != 0;
  grp.wait = a.wait;
  grp.cand = a.cand + row * a.P * a.chunk;
  grp.cap = a.chunk;
  uint32_t offset, count, tau;
  const Mask sel = radix_select<SPT>(key, (uint32_t)a.k, sh, grp, &offset, &count, &tau, s_qcnt);
  int32_t* out = a.idx + row * a.k;
  ordered_ranks<SPT>(sel, sh, [&](int j, uint32_t r) {
    const int64_t pos = (int64_t)offset + r;
    if (pos < a.k) out[pos] = (int32_t)(t0 + (int64_t)j * SB + tid);
  });
  if (a.thr && p == 0 && tid == 0) a.thr[row] = key_float(tau);
}

static int topk_spt(int64_t chunk) {
  const int64_t need = (chunk + SB - 1) / SB;
  for (int s : {4, 16, 32})
    if (need <= s) return s;
  return 0;
}

sdkv_status plan_topk(int64_t rows, int64_t n, int64_t k, TopkPlan* p) {
  TopkPlan q;
  q.rows = rows;
  q.n = n;
  q.k = k;
  const int64_t p_min = (n + kMaxChunk - 1) / kMaxChunk;
  const int64_t p_par = std::max<int64_t>(1, kPlanCUs / std::max<int64_t>(1, rows));
  const int64_t p_cap = std::max<int64_t>(1, (n + 2047) / 2048);
  const int64_t P = std::max(p_min, std::min(p_par, p_cap));
  if (P > kTopkMaxP) return SDKV_ERR_UNSUPPORTED;
  q.P = (int)P;
  q.chunk = (n + P - 1) / P;
  q.spt = topk_spt(q.chunk);
  if (q.spt == 0) return SDKV_ERR_UNSUPPORTED;
  size_t off = 0;
  // cleared per call: the status word first (word 0 of the workspace)
  q.off_err = off;    off += 4;
  q.off_ticket = off; off += 8 * 4;
  q.off_bar = off;    off += (size_t)rows * 2 * 4;
  q.off_xchg = off;   off += (size_t)rows * q.P * 2 * 4;
  q.off_ghist = off;  off += (q.P > 1) ? (size_t)rows * 2048 * 4 : 0;
  q.zero_bytes = align_up(off, 256);
  q.off_cand = q.zero_bytes;
  q.total = q.off_cand + align_up(q.P > 1 ? (size_t)rows * q.P * q.chunk * 4 : 0, 256);
  *p = q;
  return SDKV_OK;
}

static const void* pick_topk_kernel(int spt) {
  if (spt == 4) return (const void*)&k_topk<4>;
  if (spt == 16) return (const void*)&k_topk<16>;
  if (spt == 32) return (const void*)&k_topk<32>;
  return nullptr;
}

sdkv_status launch_topk(const float* scores, int64_t ld, int32_t* idx, float* thr,
                        const TopkPlan& p, void* ws, hipStream_t stream) {
  char* base = (char*)ws;
  const int64_t zw = (int64_t)(p.zero_bytes / 4);
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)std::min<int64_t>(1024, (zw + 255) / 256)),
                     dim3(256), 0, stream, (uint32_t*)base, zw);
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  TopkArgs a;
  a.s = scores;
  a.ld = ld;
  a.n = p.n;
  a.k = p.k;
  a.chunk = p.chunk;
  a.P = p.P;
  a.idx = idx;
  a.thr = thr;
  a.ghist = (uint32_t*)(base + p.off_ghist);
  a.xchg = (uint32_t*)(base + p.off_xchg);
  a.bar = (uint32_t*)(base + p.off_bar);
  a.wait = wait_ctl((uint32_t*)(base + p.off_err));
  a.cand = (uint32_t*)(base + p.off_cand);
  const void* kfn = pick_topk_kernel(p.spt);
  if (!kfn) return SDKV_ERR_UNSUPPORTED;
  // per-XCD ticket classes (see k_rows): with P > 1 every class must hold
  // two rows' workgroups co-resident; each launch also needs whole rows per
  // class
  bool xcd_ok = true;
  if (p.P > 1) {
    int cap = 0;
    sdkv_status st = coresident_blocks(kfn, SB, 0, &cap);
    if (st != SDKV_OK) return st;
    if (cap < p.P) return SDKV_ERR_UNSUPPORTED;
    xcd_ok = 16 * p.P <= cap;
  }
  a.ticket = (uint32_t*)(base + p.off_ticket);
  // rows per launch bounded so the grid size fits an int; every launch gets
  // a fresh ticket range, so the ticket is cleared before each one
  const int64_t batch = std::max<int64_t>(1, std::min<int64_t>(p.rows, ((int64_t)1 << 30) / p.P));
  for (int64_t r0 = 0; r0 < p.rows; r0 += batch) {
    if (r0 > 0) {
      hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(64), 0, stream, a.ticket, (int64_t)8);
      if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
    }
    a.row0 = (int)r0;
    a.nrows = (int)std::min<int64_t>(batch, p.rows - r0);
    const int64_t nb = (int64_t)a.nrows * p.P;
    a.xcd_map = (xcd_ok && nb % 8 == 0 && (nb / 8) % p.P == 0) ? 1 : 0;
    void* args[] = {&a};
    const dim3 grid((unsigned)(a.nrows * p.P)), block(SB);
    if (hipLaunchKernel(kfn, grid, block, args, 0, stream) != hipSuccess) return SDKV_ERR_DEVICE;
  }
  return SDKV_OK;
}

}  // namespace sdkv
