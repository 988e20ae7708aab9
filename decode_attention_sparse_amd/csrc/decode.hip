// Hierarchical coded decode attention (one layer, one decode step) on gfx950.
//
// Method: "LLM Inference in a Flash!" -- review page, Summary (a cheap score
// from Klow atoms for every token, a Khigh-atom rescore for the best tenth)
// and FAQ on the 15x figure (a key/value is kept as atom indices plus
// coefficients; three atoms are enough to rank most tokens); abstract page
// (KV vectors are sums of fixed dictionary atoms, hence
// <q, k_t> = sum_j kappa_tj <q, d_{i_tj}>).
//
// Kernels, in launch order on the caller's stream:
//   k_utable_*   U = scale * Q Dk^T for every (batch, query head)   [MFMA bf16]
//   k_rows       per (batch, query head) and token chunk: U row staged in
//                LDS; s_low for every token of the chunk kept in registers;
//                exact top-m radix select (cooperative across the row's
//                chunks); Khigh rescore of the selected tokens; softmax
//                partials and per-atom value weights accumulated in LDS.
//   k_wdv_*      merge the per-chunk softmax partials and contract the value
//                weights with Dv: out = W Dv                       [MFMA bf16]
//   k_reduce_out sum of the per-atom-chunk output partials (fixed order).
#include "select_core.h"
#include "sdkv_internal.h"

namespace sdkv {

// ---------------------------------------------------------------------------
// U table
// ---------------------------------------------------------------------------
struct UArgs {
  const uint16_t* q;   // [rows, d] bf16
  const void* dk;      // [N, d]
  int rows, N, d;
  float scale;
  float* U;            // [rows, N] (workspace)
  float* u_dbg;        // optional copy
  uint32_t* zero;      // region cleared by this kernel
  int64_t zero_words;
};

__device__ __forceinline__ void clear_region(const UArgs& a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.zero_words; i += stride)
    a.zero[i] = 0u;
}

// bf16 dictionary: each wave owns 16 atoms; loops over 16-row query tiles.
__global__ __launch_bounds__(256) void k_utable_bf16(UArgs a) {
  clear_region(a);
  const int w = wave_id(), l = lane_id();
  const int a0 = (blockIdx.x * 4 + w) * 16;
  if (a0 >= a.N) return;
  const int atom = a0 + (l & 15);
  const int ks = a.d >> 5;
  const uint16_t* dk = (const uint16_t*)a.dk;
  u32x4 bf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf[s] = u32x4{0u, 0u, 0u, 0u};
    if (s < ks && atom < a.N)
      bf[s] = *(const u32x4*)(dk + (int64_t)atom * a.d + 32 * s + 8 * (l >> 4));
  }
  for (int r0 = 0; r0 < a.rows; r0 += 16) {
    const int row = r0 + (l & 15);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < ks) {
        u32x4 af = u32x4{0u, 0u, 0u, 0u};
        if (row < a.rows) af = *(const u32x4*)(a.q + (int64_t)row * a.d + 32 * s + 8 * (l >> 4));
        acc = mfma_bf16(af, bf[s], acc);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r0 + 4 * (l >> 4) + i;
      if (rr < a.rows && atom < a.N) {
        const float v = acc[i] * a.scale;
        a.U[(int64_t)rr * a.N + atom] = v;
        if (a.u_dbg) a.u_dbg[(int64_t)rr * a.N + atom] = v;
      }
    }
  }
}

// fp32 dictionary (small configurations): one thread per (row, atom).
__global__ __launch_bounds__(256) void k_utable_f32(UArgs a) {
  clear_region(a);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.rows * a.N) return;
  const int r = (int)(i / a.N), atom = (int)(i % a.N);
  const float* dk = (const float*)a.dk + (int64_t)atom * a.d;
  const uint16_t* q = a.q + (int64_t)r * a.d;
  float s = 0.f;
  for (int k = 0; k < a.d; ++k) s = fmaf(bf16_to_f32(q[k]), dk[k], s);
  const float v = s * a.scale;
  a.U[i] = v;
  if (a.u_dbg) a.u_dbg[i] = v;
}

// ---------------------------------------------------------------------------
// Row kernel: score -> select -> rescore -> softmax partial -> value weights
// ---------------------------------------------------------------------------
struct RowsArgs {
  const float* U;           // [rows, N]
  const uint32_t* low;      // low-plane source; `low_words` words per token
  int low_words;
  const uint32_t* kc;       // [B, Hkv, T, K]
  const uint32_t* vc;
  int N, K, klow, khigh, Hq, Hkv, G, P;
  int row0, nrows;
  int64_t T, m, chunk;
  float* s_low_out;         // optional [rows, T]
  int32_t* sel;             // [rows, m]
  float* s_high;            // [rows, m]
  float* wpart;             // [rows, P, N]
  float2* stats;            // [rows, P] (local max, local sum of exp)
  uint32_t* ghist;          // [rows, 3, 2048]
  uint32_t* xchg;           // [rows, P, 2]
  uint32_t* bar;            // [rows]
  uint32_t* err;
};

template <int SPT, int LPT>
__global__ __launch_bounds__(SB) void k_rows(RowsArgs a) {
  __shared__ float s_u[kMaxAtomsDecode];
  __shared__ SelShared sh;
  __shared__ float s_red[16];

  const int tid = threadIdx.x;
  const int L = xcd_tile(blockIdx.x, a.nrows * a.P);
  const int p = L % a.P;
  const int row = a.row0 + L / a.P;
  const int b = row / a.Hq, h = row % a.Hq, g = h / a.G;
  const int64_t kv = (int64_t)b * a.Hkv + g;
  const int64_t t0 = (int64_t)p * a.chunk;
  const int64_t t1 = min(a.T, t0 + a.chunk);

  // 1. stage this query head's U row in LDS
  {
    const float* src = a.U + (int64_t)row * a.N;
    const int n4 = a.N >> 2;
    for (int i = tid; i < n4; i += SB) ((float4*)s_u)[i] = ((const float4*)src)[i];
    for (int i = (n4 << 2) + tid; i < a.N; i += SB) s_u[i] = src[i];
  }
  __syncthreads();

  // 2. s_low of every token in the chunk -> order-preserving keys
  uint32_t key[SPT];
  {
    const uint32_t* lo = a.low + kv * a.T * a.low_words;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t t = t0 + (int64_t)j * SB + tid;
      key[j] = 0u;
      if (t < t1) {
        const uint32_t* wp = lo + t * a.low_words;
        float s = 0.f;
        for (int i = 0; i < a.klow; ++i) {
          const uint32_t wd = wp[i];
          s = fmaf(code_coef(wd), s_u[code_idx(wd) & (kMaxAtomsDecode - 1)], s);
        }
        key[j] = float_key(s);
        if (a.s_low_out) a.s_low_out[(int64_t)row * a.T + t] = s;
      }
    }
  }

  // 3. exact top-m selection across the row's P workgroups
  SelGroup grp;
  grp.P = a.P;
  grp.p = p;
  grp.ghist = a.ghist + (int64_t)row * 3 * 2048;
  grp.xchg = a.xchg + (int64_t)row * a.P * 2;
  grp.bar = a.bar + row;
  grp.err = a.err;
  uint32_t offset, count, tau;
  const uint64_t sel = radix_select<SPT>(key, (uint32_t)a.m, sh, grp, &offset, &count, &tau);

  int32_t* sel_row = a.sel + (int64_t)row * a.m;
  float* sh_row = a.s_high + (int64_t)row * a.m;
  ordered_ranks<SPT>(sel, sh, [&](int j, uint32_t r) {
    const int64_t pos = (int64_t)offset + r;
    if (pos < a.m) sel_row[pos] = (int32_t)(t0 + (int64_t)j * SB + tid);
  });
  const int64_t cnt = min((int64_t)count, a.m - (int64_t)offset);
  __threadfence_block();
  __syncthreads();

  // 4. Khigh rescore of this workgroup's selected tokens (LPT lanes per token)
  constexpr int TPW = 64 / LPT;  // tokens per wave per iteration
  const int w = wave_id(), lane = lane_id();
  const int jj = lane % LPT;
  const int64_t step = (int64_t)SNW * TPW;
  const int64_t my0 = (int64_t)w * TPW + lane / LPT;
  const int64_t wave0 = (int64_t)w * TPW;
  float lmax = -INFINITY;
  const uint32_t* kbase = a.kc + kv * a.T * a.K;
  for (int64_t base = 0; base + wave0 < cnt; base += step) {
    const int64_t i = base + my0;
    const bool valid = i < cnt;
    float v = 0.f;
    if (valid && jj < a.khigh) {
      const int64_t t = min(max((int64_t)sel_row[offset + i], (int64_t)0), a.T - 1);
      const uint32_t wd = kbase[t * a.K + jj];
      v = code_coef(wd) * s_u[code_idx(wd) & (kMaxAtomsDecode - 1)];
    }
    v = group_sum<LPT>(v);
    if (valid) {
      if (jj == 0) sh_row[offset + i] = v;
      lmax = fmaxf(lmax, v);
    }
  }
  const float M = block_max<SNW>(lmax, s_red);

  // 5. softmax partial + per-atom value weights (LDS float atomics)
  for (int i = tid; i < a.N; i += SB) s_u[i] = 0.f;
  __threadfence_block();
  __syncthreads();
  float lsum = 0.f;
  const uint32_t* vbase = a.vc + kv * a.T * a.K;
  for (int64_t base = 0; base + wave0 < cnt; base += step) {
    const int64_t i = base + my0;
    if (i < cnt) {
      const int64_t t = min(max((int64_t)sel_row[offset + i], (int64_t)0), a.T - 1);
      const float pt = __expf(sh_row[offset + i] - M);
      if (jj < a.K) {
        const uint32_t wd = vbase[t * a.K + jj];
        atomicAdd(&s_u[code_idx(wd) & (kMaxAtomsDecode - 1)], pt * code_coef(wd));
      }
      if (jj == 0) lsum += pt;
    }
  }
  const float lsum_all = block_sum<SNW>(lsum, s_red);
  __syncthreads();

  // 6. write the partial weights and the (max, sum) pair
  {
    float* dst = a.wpart + ((int64_t)row * a.P + p) * a.N;
    const int n4 = a.N >> 2;
    for (int i = tid; i < n4; i += SB) ((float4*)dst)[i] = ((const float4*)s_u)[i];
    for (int i = (n4 << 2) + tid; i < a.N; i += SB) dst[i] = s_u[i];
    if (tid == 0) a.stats[(int64_t)row * a.P + p] = make_float2(cnt > 0 ? M : -INFINITY, lsum_all);
  }
}

// ---------------------------------------------------------------------------
// W . Dv
// ---------------------------------------------------------------------------
struct WdvArgs {
  const float* wpart;     // [rows, P, N]
  const float2* stats;    // [rows, P]
  const void* dv;         // [N, d]
  int N, d, P, rows, nrt, nsub, nchunks;
  float* opart;           // [nchunks, rows, d]
  float* w_out;           // optional [rows, N]
};

constexpr int WPITCH = kWdvSub + 8;         // u16 elements per A row in LDS
constexpr int BPITCH = kWdvSub / 2 + 4;     // u32 words (atom pairs) per B row

// Fills s_coef[r][p] = exp(M_p - M_r) / L_r for the 16 rows of the tile.
__device__ __forceinline__ void wdv_coefs(const WdvArgs& a, int r0, float* s_coef) {
  const int tid = threadIdx.x;
  if (tid < 16) {
    const int row = r0 + tid;
    if (row < a.rows) {
      const float2* st = a.stats + (int64_t)row * a.P;
      float M = -INFINITY;
      for (int p = 0; p < a.P; ++p) M = fmaxf(M, st[p].x);
      float Lr = 0.f;
      for (int p = 0; p < a.P; ++p) {
        const float c = (st[p].y > 0.f) ? __expf(st[p].x - M) : 0.f;
        s_coef[tid * kMaxRowP + p] = c;
        Lr += c * st[p].y;
      }
      const float inv = 1.f / Lr;
      for (int p = 0; p < a.P; ++p) s_coef[tid * kMaxRowP + p] *= inv;
    } else {
      for (int p = 0; p < a.P; ++p) s_coef[tid * kMaxRowP + p] = 0.f;
    }
  }
}

// merged weight W[r][atom] for the tile's rows
__device__ __forceinline__ float wdv_weight(const WdvArgs& a, const float* s_coef, int r0, int r,
                                            int atom) {
  const int row = r0 + r;
  if (row >= a.rows || atom >= a.N) return 0.f;
  const float* src = a.wpart + (int64_t)row * a.P * a.N + atom;
  float acc = 0.f;
  for (int p = 0; p < a.P; ++p) acc = fmaf(s_coef[r * kMaxRowP + p], src[(int64_t)p * a.N], acc);
  return acc;
}

__global__ __launch_bounds__(256) void k_wdv_bf16(WdvArgs a) {
  __shared__ float s_coef[16 * kMaxRowP];
  __shared__ __attribute__((aligned(16))) uint16_t s_ahi[16 * WPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t s_alo[16 * WPITCH];
  __shared__ __attribute__((aligned(16))) uint32_t s_bt[128 * BPITCH];

  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int L = xcd_tile(blockIdx.x, a.nchunks * a.nrt);
  const int chunk = L / a.nrt, rt = L % a.nrt;
  const int r0 = rt * 16;
  wdv_coefs(a, r0, s_coef);
  __syncthreads();

  const uint16_t* dv = (const uint16_t*)a.dv;
  const int ncol = a.d >> 4;  // 16-wide output column tiles
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int sub = 0; sub < a.nsub; ++sub) {
    const int a0 = (chunk * a.nsub + sub) * kWdvSub;
    if (a0 >= a.N) break;
    // A: merged weights, split into bf16 hi + lo
    {
      const int atom = a0 + tid;  // kWdvSub == blockDim
      for (int r = 0; r < 16; ++r) {
        const float wv = wdv_weight(a, s_coef, r0, r, atom);
        if (a.w_out && r0 + r < a.rows && atom < a.N) a.w_out[(int64_t)(r0 + r) * a.N + atom] = wv;
        const uint32_t hi = f32_to_bf16_rne(wv);
        const uint32_t lo = f32_to_bf16_rne(wv - __uint_as_float(hi << 16));
        s_ahi[r * WPITCH + tid] = (uint16_t)hi;
        s_alo[r * WPITCH + tid] = (uint16_t)lo;
      }
    }
    // B: Dv rows a0 .. a0+255, transposed to [dim][atom pair]
    for (int it = tid; it < (kWdvSub / 2) * (a.d >> 3); it += 256) {
      const int ap = it % (kWdvSub / 2), sg = it / (kWdvSub / 2);
      const int atom = a0 + 2 * ap;
      u32x4 x0 = u32x4{0u, 0u, 0u, 0u}, x1 = u32x4{0u, 0u, 0u, 0u};
      if (atom < a.N) x0 = *(const u32x4*)(dv + (int64_t)atom * a.d + 8 * sg);
      if (atom + 1 < a.N) x1 = *(const u32x4*)(dv + (int64_t)(atom + 1) * a.d + 8 * sg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_bt[(8 * sg + 2 * i) * BPITCH + ap] = (x0[i] & 0xFFFFu) | (x1[i] << 16);
        s_bt[(8 * sg + 2 * i + 1) * BPITCH + ap] = (x0[i] >> 16) | (x1[i] & 0xFFFF0000u);
      }
    }
    __syncthreads();
    // MFMA: wave w owns output columns [32w, 32w+32)
    if (2 * w < ncol) {
#pragma unroll
      for (int ks = 0; ks < kWdvSub / 32; ++ks) {
        const int kk = ks * 32 + 8 * (l >> 4);
        const u32x4 ah = *(const u32x4*)(s_ahi + (l & 15) * WPITCH + kk);
        const u32x4 al = *(const u32x4*)(s_alo + (l & 15) * WPITCH + kk);
        const int n0 = 32 * w + (l & 15);
        const u32x4 b0 = *(const u32x4*)(s_bt + n0 * BPITCH + (kk >> 1));
        acc0 = mfma_bf16(ah, b0, acc0);
        acc0 = mfma_bf16(al, b0, acc0);
        if (2 * w + 1 < ncol) {
          const u32x4 b1 = *(const u32x4*)(s_bt + (n0 + 16) * BPITCH + (kk >> 1));
          acc1 = mfma_bf16(ah, b1, acc1);
          acc1 = mfma_bf16(al, b1, acc1);
        }
      }
    }
    __syncthreads();
  }
  if (2 * w < ncol) {
    float* dst = a.opart + (int64_t)chunk * a.rows * a.d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * (l >> 4) + i;
      if (row < a.rows) {
        dst[(int64_t)row * a.d + 32 * w + (l & 15)] = acc0[i];
        if (2 * w + 1 < ncol) dst[(int64_t)row * a.d + 32 * w + 16 + (l & 15)] = acc1[i];
      }
    }
  }
}

// fp32 value dictionary (small configurations): plain fp32 FMAs.
__global__ __launch_bounds__(256) void k_wdv_f32(WdvArgs a) {
  __shared__ float s_coef[16 * kMaxRowP];
  __shared__ float s_w[16 * kWdvSub];
  const int tid = threadIdx.x;
  const int L = xcd_tile(blockIdx.x, a.nchunks * a.nrt);
  const int chunk = L / a.nrt, rt = L % a.nrt;
  const int r0 = rt * 16;
  wdv_coefs(a, r0, s_coef);
  __syncthreads();
  const float* dv = (const float*)a.dv;
  const int r = tid >> 4;            // row within the tile
  const int c0 = (tid & 15) * 8;     // 8 output columns per thread
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int sub = 0; sub < a.nsub; ++sub) {
    const int a0 = (chunk * a.nsub + sub) * kWdvSub;
    if (a0 >= a.N) break;
    for (int rr = 0; rr < 16; ++rr) {
      const float wv = wdv_weight(a, s_coef, r0, rr, a0 + tid);
      s_w[rr * kWdvSub + tid] = wv;
      if (a.w_out && r0 + rr < a.rows && a0 + tid < a.N) a.w_out[(int64_t)(r0 + rr) * a.N + a0 + tid] = wv;
    }
    __syncthreads();
    const int na = min(kWdvSub, a.N - a0);
    if (c0 < a.d) {
      for (int k = 0; k < na; ++k) {
        const float wv = s_w[r * kWdvSub + k];
        const float* drow = dv + (int64_t)(a0 + k) * a.d + c0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wv, drow[i], acc[i]);
      }
    }
    __syncthreads();
  }
  const int row = r0 + r;
  if (row < a.rows && c0 < a.d) {
    float* dst = a.opart + ((int64_t)chunk * a.rows + row) * a.d + c0;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc[i];
  }
}

__global__ __launch_bounds__(256) void k_reduce_out(const float* opart, int nchunks, int64_t n,
                                                    float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int c = 0; c < nchunks; ++c) s += opart[(int64_t)c * n + i];
  out[i] = s;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int spt_for(int64_t chunk) {
  const int64_t need = (chunk + SB - 1) / SB;
  for (int s : {4, 8, 16, 32, 64})
    if (need <= s) return s;
  return 0;
}

sdkv_status plan_decode(const sdkv_attn_args* a, DecodePlan* p) {
  DecodePlan q;
  q.rows = (int64_t)a->B * a->Hq;
  q.m = sdkv_selected_count(a->T, a->top_num, a->top_den);
  const int64_t T = a->T;
  const int64_t p_min = (T + kMaxChunk - 1) / kMaxChunk;
  const int64_t p_par = std::max<int64_t>(1, kPlanCUs / std::max<int64_t>(1, q.rows));
  const int64_t p_cap = std::max<int64_t>(1, (T + 2047) / 2048);
  const int64_t P = std::max(p_min, std::min(p_par, p_cap));
  if (P > kMaxRowP) return SDKV_ERR_UNSUPPORTED;
  q.P = (int)P;
  q.chunk = (T + P - 1) / P;
  q.spt = spt_for(q.chunk);
  if (q.spt == 0) return SDKV_ERR_UNSUPPORTED;
  q.lpt = a->K <= 16 ? 16 : 32;
  q.nrt = (int)((q.rows + 15) / 16);
  const int nsub_total = (a->n_atoms + kWdvSub - 1) / kWdvSub;
  const int target = std::max(1, 512 / q.nrt);
  q.nsub = std::max(1, (nsub_total + target - 1) / target);
  q.nchunks = (nsub_total + q.nsub - 1) / q.nsub;

  const size_t A = 256;
  const int64_t N = a->n_atoms, rows = q.rows;
  size_t off = 0;
  q.off_u = off;      off = align_up(off + (size_t)rows * N * 4, A);
  q.off_sel = off;    off = align_up(off + (size_t)rows * q.m * 4, A);
  q.off_shigh = off;  off = align_up(off + (size_t)rows * q.m * 4, A);
  q.off_wpart = off;  off = align_up(off + (size_t)rows * q.P * N * 4, A);
  q.off_stats = off;  off = align_up(off + (size_t)rows * q.P * 8, A);
  q.off_zero = off;
  q.off_ghist = off;  off += (q.P > 1) ? (size_t)rows * 3 * 2048 * 4 : 0;
  q.off_xchg = off;   off += (size_t)rows * q.P * 2 * 4;
  q.off_bar = off;    off += (size_t)rows * 4;
  q.off_err = off;    off += 4;
  off = align_up(off, A);
  q.zero_bytes = off - q.off_zero;
  q.off_opart = off;  off = align_up(off + (size_t)q.nchunks * rows * a->d * 4, A);
  q.total = off;
  *p = q;
  return SDKV_OK;
}

template <int SPT, int LPT>
static const void* rows_kernel() {
  return (const void*)&k_rows<SPT, LPT>;
}

static const void* pick_rows_kernel(int spt, int lpt) {
#define SDKV_PICK(S)                                                   \
  if (spt == S) return lpt == 16 ? rows_kernel<S, 16>() : rows_kernel<S, 32>();
  SDKV_PICK(4)
  SDKV_PICK(8)
  SDKV_PICK(16)
  SDKV_PICK(32)
  SDKV_PICK(64)
#undef SDKV_PICK
  return nullptr;
}

sdkv_status launch_decode(const sdkv_attn_args* a, const DecodePlan& p, void* ws,
                          hipStream_t stream) {
  char* base = (char*)ws;
  const int64_t rows = p.rows;
  float* U = (float*)(base + p.off_u);
  int32_t* sel = a->sel ? a->sel : (int32_t*)(base + p.off_sel);
  float* shigh = a->s_high ? a->s_high : (float*)(base + p.off_shigh);
  float* wpart = (float*)(base + p.off_wpart);
  float2* stats = (float2*)(base + p.off_stats);
  uint32_t* ghist = (uint32_t*)(base + p.off_ghist);
  uint32_t* xchg = (uint32_t*)(base + p.off_xchg);
  uint32_t* bar = (uint32_t*)(base + p.off_bar);
  uint32_t* err = (uint32_t*)(base + p.off_err);
  float* opart = (float*)(base + p.off_opart);

  // 1. U table (+ clear the barrier / histogram region)
  UArgs ua;
  ua.q = (const uint16_t*)a->q;
  ua.dk = a->dk;
  ua.rows = (int)rows;
  ua.N = a->n_atoms;
  ua.d = a->d;
  ua.scale = a->scale;
  ua.U = U;
  ua.u_dbg = a->u;
  ua.zero = (uint32_t*)(base + p.off_zero);
  ua.zero_words = (int64_t)(p.zero_bytes / 4);
  void* const* ev = a->stage_events;
  if (!record_stage(ev, 0, stream)) return SDKV_ERR_DEVICE;
  if (a->dict_dtype == SDKV_BF16) {
    const int grid = (a->n_atoms + 63) / 64;
    hipLaunchKernelGGL(k_utable_bf16, dim3(grid), dim3(256), 0, stream, ua);
  } else {
    const int64_t n = rows * a->n_atoms;
    const int grid = (int)std::max<int64_t>(1, (n + 255) / 256);
    hipLaunchKernelGGL(k_utable_f32, dim3(grid), dim3(256), 0, stream, ua);
  }
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;

  // 2. row kernel, in row batches that fit co-resident when cooperative
  RowsArgs ra;
  ra.U = U;
  ra.low = a->key_low ? a->key_low : a->key_codes;
  ra.low_words = a->key_low ? a->klow : a->K;
  ra.kc = a->key_codes;
  ra.vc = a->val_codes;
  ra.N = a->n_atoms;
  ra.K = a->K;
  ra.klow = a->klow;
  ra.khigh = a->khigh;
  ra.Hq = a->Hq;
  ra.Hkv = a->Hkv;
  ra.G = a->Hq / a->Hkv;
  ra.P = p.P;
  ra.T = a->T;
  ra.m = p.m;
  ra.chunk = p.chunk;
  ra.s_low_out = a->s_low;
  ra.sel = sel;
  ra.s_high = shigh;
  ra.wpart = wpart;
  ra.stats = stats;
  ra.ghist = ghist;
  ra.xchg = xchg;
  ra.bar = bar;
  ra.err = err;
  const void* kfn = pick_rows_kernel(p.spt, p.lpt);
  if (!kfn) return SDKV_ERR_UNSUPPORTED;
  if (!record_stage(ev, 1, stream)) return SDKV_ERR_DEVICE;
  int64_t batch = rows;
  if (p.P > 1) {
    int cap = 0;
    sdkv_status st = coresident_blocks(kfn, SB, 0, &cap);
    if (st != SDKV_OK) return st;
    batch = std::min<int64_t>(rows, cap / p.P);
    if (batch < 1) return SDKV_ERR_UNSUPPORTED;
  }
  for (int64_t r0 = 0; r0 < rows; r0 += batch) {
    ra.row0 = (int)r0;
    ra.nrows = (int)std::min<int64_t>(batch, rows - r0);
    const dim3 grid((unsigned)(ra.nrows * p.P)), block(SB);
    void* args[] = {&ra};
    hipError_t e;
    if (p.P > 1)
      e = hipLaunchCooperativeKernel(kfn, grid, block, args, 0, stream);
    else
      e = hipLaunchKernel(kfn, grid, block, args, 0, stream);
    if (e != hipSuccess) return SDKV_ERR_DEVICE;
  }

  // 3. merge partials and contract with Dv
  WdvArgs wa;
  wa.wpart = wpart;
  wa.stats = stats;
  wa.dv = a->dv;
  wa.N = a->n_atoms;
  wa.d = a->d;
  wa.P = p.P;
  wa.rows = (int)rows;
  wa.nrt = p.nrt;
  wa.nsub = p.nsub;
  wa.nchunks = p.nchunks;
  wa.opart = opart;
  wa.w_out = a->w;
  const dim3 wgrid((unsigned)(p.nchunks * p.nrt));
  if (!record_stage(ev, 2, stream)) return SDKV_ERR_DEVICE;
  if (a->dict_dtype == SDKV_BF16)
    hipLaunchKernelGGL(k_wdv_bf16, wgrid, dim3(256), 0, stream, wa);
  else
    hipLaunchKernelGGL(k_wdv_f32, wgrid, dim3(256), 0, stream, wa);
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;

  const int64_t nout = rows * a->d;
  if (!record_stage(ev, 3, stream)) return SDKV_ERR_DEVICE;
  hipLaunchKernelGGL(k_reduce_out, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, stream,
                     (const float*)opart, p.nchunks, nout, a->out);
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  if (!record_stage(ev, 4, stream)) return SDKV_ERR_DEVICE;
  return SDKV_OK;
}

}  // namespace sdkv
