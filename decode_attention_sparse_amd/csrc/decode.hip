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
//                exact top-m select (one synchronisation of the row's
//                chunks around a shared sample's quantile window, or a
//                two-synchronisation radix select); Khigh rescore of the selected tokens; softmax
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
  const void* q;       // [rows, d] bf16, or fp32 when q_f32
  int q_f32;
  const void* dk;      // [N, d]
  int rows, N, d;
  float scale;
  float* U;            // [rows, N] (workspace)
  float* u_dbg;        // optional copy
  // shared selection: Ug[(b, g)] = scale * (sum_j q[b, g G + j]) Dk^T, the
  // group sums of U by linearity (bf16 dictionaries); ngroups = 0 otherwise
  float* Ug;           // [ngroups, N]
  int ngroups, Hq, Hkv, G;
  uint32_t* zero;      // region cleared by this kernel
  int64_t zero_words;
};

__device__ __forceinline__ void clear_region(const UArgs& a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.zero_words; i += stride)
    a.zero[i] = 0u;
}

// bf16 dictionary: each wave owns 16 atoms (its Dk fragments stay in
// registers); the workgroup stages the query rows in LDS, 64 at a time, so a
// query row is read from memory once per workgroup, not once per wave. bf16
// query rows go to the matrix cores as they are; fp32 query rows and the
// group rows of the shared selection (the group's query rows summed in fp32,
// head order) are split into three bf16 parts that hold them exactly, and
// run as three accumulating MFMAs.
constexpr int UQR = 64;          // query rows staged per pass
constexpr int UQP = 128 + 8;     // LDS pitch of a staged row (bf16 elements)
__global__ __launch_bounds__(256) void k_utable_bf16(UArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_qh[UQR * UQP];
  __shared__ __attribute__((aligned(16))) uint16_t s_qm[UQR * UQP];
  __shared__ __attribute__((aligned(16))) uint16_t s_ql[UQR * UQP];
  clear_region(a);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int a0 = (blockIdx.x * 4 + w) * 16;
  const int atom = a0 + (l & 15);
  const int ks = a.d >> 5;
  const int segs = a.d >> 3;  // 8-element segments per row
  const uint16_t* dk = (const uint16_t*)a.dk;
  u32x4 bf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf[s] = u32x4{0u, 0u, 0u, 0u};
    if (s < ks && atom < a.N)
      bf[s] = *(const u32x4*)(dk + (int64_t)atom * a.d + 32 * s + 8 * (l >> 4));
  }
  // pass kind 0: query rows [p0, p0 + 64) of [0, rows); kind 1: group rows
  for (int kind = 0; kind < 2; ++kind) {
    const int nrows = kind == 0 ? a.rows : a.ngroups;
    const bool split = kind == 1 || a.q_f32;
    for (int p0 = 0; p0 < nrows; p0 += UQR) {
      __syncthreads();  // the previous pass's fragments have been read
      if (!split) {
        // bf16 query rows: every item's 16 bytes requested before any is
        // stored (one round trip instead of one per item)
        constexpr int IT = UQR * 16 / 256;  // items per thread at d = 128
        u32x4 raw[IT];
#pragma unroll
        for (int k = 0; k < IT; ++k) {
          const int it = tid + 256 * k, r = it / segs, sg = it % segs, row = p0 + r;
          raw[k] = u32x4{0u, 0u, 0u, 0u};
          if (it < UQR * segs && row < nrows)
            raw[k] = *(const u32x4*)((const uint16_t*)a.q + (int64_t)row * a.d + 8 * sg);
        }
#pragma unroll
        for (int k = 0; k < IT; ++k) {
          const int it = tid + 256 * k, r = it / segs, sg = it % segs;
          if (it < UQR * segs) *(u32x4*)(s_qh + r * UQP + 8 * sg) = raw[k];
        }
      } else
      // stage: item = (row, 8-element segment), UQR * segs <= 1024 items
      for (int it = tid; it < UQR * segs; it += 256) {
        const int r = it / segs, sg = it % segs, row = p0 + r;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
        u32x4 raw = u32x4{0u, 0u, 0u, 0u};
        if (row < nrows) {
          if (kind == 0) {
            const int64_t off = (int64_t)row * a.d + 8 * sg;
            if (a.q_f32) {
              const float4* qp = (const float4*)((const float*)a.q + off);
              const float4 x0 = qp[0], x1 = qp[1];
              v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
              v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
            } else {
              raw = *(const u32x4*)((const uint16_t*)a.q + off);
            }
          } else {
            const int64_t q0 = (int64_t)(row / a.Hkv) * a.Hq + (int64_t)(row % a.Hkv) * a.G;
            for (int j = 0; j < a.G; ++j) {
              const int64_t off = (q0 + j) * a.d + 8 * sg;
              if (a.q_f32) {
                const float4* qp = (const float4*)((const float*)a.q + off);
                const float4 x0 = qp[0], x1 = qp[1];
                v[0] += x0.x; v[1] += x0.y; v[2] += x0.z; v[3] += x0.w;
                v[4] += x1.x; v[5] += x1.y; v[6] += x1.z; v[7] += x1.w;
              } else {
                const u32x4 q = *(const u32x4*)((const uint16_t*)a.q + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  v[2 * e] += bf16_lo(q[e]);
                  v[2 * e + 1] += bf16_hi(q[e]);
                }
              }
            }
          }
        }
        const int o = r * UQP + 8 * sg;
        if (split) {
          u32x4 hi, mid, lo;
          split3_bf16(v, hi, mid, lo);
          *(u32x4*)(s_qh + o) = hi;
          *(u32x4*)(s_qm + o) = mid;
          *(u32x4*)(s_ql + o) = lo;
        } else {
          *(u32x4*)(s_qh + o) = raw;
        }
      }
      __syncthreads();
      float* dst = kind == 0 ? a.U : a.Ug;
#pragma unroll
      for (int rt = 0; rt < UQR / 16; ++rt) {
        if (p0 + 16 * rt >= nrows) break;
        const int o = (16 * rt + (l & 15)) * UQP + 8 * (l >> 4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s < ks) {
            acc = mfma_bf16(*(const u32x4*)(s_qh + o + 32 * s), bf[s], acc);
            if (split) {
              acc = mfma_bf16(*(const u32x4*)(s_qm + o + 32 * s), bf[s], acc);
              acc = mfma_bf16(*(const u32x4*)(s_ql + o + 32 * s), bf[s], acc);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = p0 + 16 * rt + 4 * (l >> 4) + i;
          if (rr < nrows && atom < a.N) {
            const float v = acc[i] * a.scale;
            dst[(int64_t)rr * a.N + atom] = v;
            if (kind == 0 && a.u_dbg) a.u_dbg[(int64_t)rr * a.N + atom] = v;
          }
        }
      }
    }
  }
}

// Group sums of U for the shared selection: Ug[r][a] = sum_{j<G} U[r G + j][a]
// (query rows are (b, h) with h = g G + j, so group r = b Hkv + g), in j order.
__global__ __launch_bounds__(256) void k_usum(const float* U, float* Ug, int64_t n, int N, int G) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t r = i / N, at = i % N;
  const float* src = U + r * G * N + at;
  float s = src[0];
  for (int j = 1; j < G; ++j) s += src[(int64_t)j * N];
  Ug[i] = s;
}

// fp32 dictionary (small configurations): one thread per (row, atom).
__global__ __launch_bounds__(256) void k_utable_f32(UArgs a) {
  clear_region(a);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.rows * a.N) return;
  const int r = (int)(i / a.N), atom = (int)(i % a.N);
  const float* dk = (const float*)a.dk + (int64_t)atom * a.d;
  float s = 0.f;
  if (a.q_f32) {
    const float* q = (const float*)a.q + (int64_t)r * a.d;
    for (int k = 0; k < a.d; ++k) s = fmaf(q[k], dk[k], s);
  } else {
    const uint16_t* q = (const uint16_t*)a.q + (int64_t)r * a.d;
    for (int k = 0; k < a.d; ++k) s = fmaf(bf16_to_f32(q[k]), dk[k], s);
  }
  const float v = s * a.scale;
  a.U[i] = v;
  if (a.u_dbg) a.u_dbg[i] = v;
}

// ---------------------------------------------------------------------------
// Row kernel: score -> select -> rescore -> softmax -> value weights -> W
// ---------------------------------------------------------------------------
struct RowsArgs {
  const float* U;           // [rows, N]
  const uint32_t* low;      // low-plane source; `low_words` words per token
  int low_words;
  const uint32_t* kc;       // [B, Hkv, T] records of K words, `rs` words apart
  const uint32_t* vc;
  int64_t rs;
  int N, K, klow, khigh, Hq, Hkv, G, P;
  int row0, nrows;
  int64_t T, m, chunk;
  float* s_low_out;         // optional [rows, T]
  int32_t* sel_out;         // optional [rows, m]
  float* s_high_out;        // optional [rows, m]
  int32_t* sel;             // [rows, P, chunk] per-workgroup lists (when LDS is short)
  float* s_high;            // [rows, P, chunk]
  uint16_t* wpart;          // [rows, P, N] per-workgroup unnormalised weights, fp16
                            // bits scaled by 1 / stats.z
  float4* stats;            // [rows, P] (local max, local sum of exp, weight scale, 0)
  uint32_t* ghist;          // [rows, 2048]
  uint32_t* wtab;           // [rows, P, 2048] window tables: count | start << 16
  uint32_t* cand;           // [rows, P, chunk] threshold-bin candidates
  uint32_t* xchg;           // [rows, P, 2]
  uint32_t* bar;            // [rows, 2] barrier counters
  WaitCtl wait;             // status word (workspace word 0) and wait bounds
  uint32_t* ticket;         // [8] workgroup start-order counters, zeroed per call
  int xcd_map;              // per-XCD ticket classes (rows stay on one XCD)
  const float* Ug;          // [B * Hkv, N] group-summed U rows (shared selection)
  int shared;               // selection shared by the query heads of a KV head
  int readb;                // reading B: every token enters the softmax
  const uint32_t* vlow;     // optional [B, Hkv, T, klow] value low plane (reading B)
  int imode;                // integer-only softmax
  int32_t* p_int_out;       // optional [rows, m] integer probabilities
  uint32_t* ixchg;          // [rows, P, 4] integer-softmax exchange words
};

// --- integer-only softmax (review page, Summary and Strengths: token-wise
// INT16 requantization of the Softmax input, an integer polynomial exp, shift
// guards against INT32 overflow, fixed-point reciprocals). The polynomial is
// I-BERT's fit exp(p) ~ a (p + b)^2 + c on (-ln2, 0], a = 0.3585, b = 1.353,
// c = 0.344; the constants below are ln 2, b and c / a with 30 fractional
// bits (floor).
constexpr uint64_t kLN2_Q30 = 744261117ull;
constexpr int64_t kB_Q30 = 1452772687ll;
constexpr int64_t kCA_Q30 = 1030312935ll;

struct IntSoftmax {
  int k;      // requantization shift: q = rint(s 2^k), |q| <= 32767
  int qmax;   // the row's largest q
  int qb, g, qc;  // b 2^k; guard shift of the polynomial; (c/a) 2^(2(k-g))
  int h;      // guard shift of the exponentials before the INT32 sum
};

__device__ __forceinline__ int requant16(float s, int k) {
  return (int)fminf(fmaxf(rintf(ldexpf(s, k)), -32767.f), 32767.f);
}

// Row constants from the row's largest and smallest score and its size m.
__device__ __forceinline__ IntSoftmax int_softmax_consts(float smax, float smin, int64_t m) {
  IntSoftmax c;
  const float A = fmaxf(fabsf(smax), fabsf(smin));
  if (A == 0.f) {
    c.k = 30;
  } else {
    int E;
    frexpf(A, &E);  // A = f 2^E, f in [0.5, 1)
    c.k = min(30, max(1, 15 - E));
  }
  c.qmax = requant16(smax, c.k);
  c.qb = (int)(kB_Q30 >> (30 - c.k));
  c.g = max(0, c.k - 14);
  c.qc = (int)(kCA_Q30 >> (30 - 2 * (c.k - c.g)));
  const uint32_t tb = (uint32_t)(c.qb >> c.g);
  const uint32_t emax = tb * tb + (uint32_t)c.qc;
  c.h = max(0, (64 - __clzll((unsigned long long)m)) + (32 - __clz(emax)) - 30);
  return c;
}

// e' of one score: the range reduction x = -z ln2 + p at 30 fractional bits,
// p truncated to k bits, 2^-z times the polynomial, then the rounding guard
// shift by h.
__device__ __forceinline__ uint32_t int_exp_guarded(float s, const IntSoftmax& c) {
  const int qd = requant16(s, c.k) - c.qmax;  // <= 0
  const uint64_t X = (uint64_t)(-qd) << (30 - c.k);
  const uint64_t z = X / kLN2_Q30;
  if (z >= 31) return 0u;
  const int qp = -(int)((X - z * kLN2_Q30) >> (30 - c.k));
  const int t = (qp + c.qb) >> c.g;
  const uint32_t e = ((uint32_t)(t * t) + (uint32_t)c.qc) >> (int)z;
  return c.h > 0 ? (e + (1u << (c.h - 1))) >> c.h : e;
}

static_assert(kRowThreads == SB && kMaxRowSPT == kMaxSPT, "planner and kernels disagree");

struct Words3 {
  uint32_t x, y, z;
};

constexpr int kTokBatch = 2;   // selected tokens per thread per load batch
constexpr int kListCap = 3072; // selected tokens per workgroup kept in LDS

// Loads a 16-word code record, 64-byte aligned, as 4 x 16 bytes, into the
// first 16 words of w (32-word arrays: a register-allocation choice; with
// 16-word arrays the 32-key extension build spills far more).
__device__ __forceinline__ void load_record(const uint32_t* rec, uint32_t (&w)[32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = ((const u32x4*)rec)[q];
    w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
  }
}

// U row of `row` into LDS. All loads are issued before the first store
// (stores go to clamped indices: a duplicate store writes the same value).
__device__ __forceinline__ void stage_u(const RowsArgs& a, const float* src, float* s_u) {
  const int tid = threadIdx.x;
  const float4* src4 = (const float4*)src;
  const int n4 = a.N >> 2;
  constexpr int UPT = kMaxAtomsDecode / 4 / SB;
  if (n4 > 0) {
    float4 ub[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) ub[k] = src4[min(tid + k * SB, n4 - 1)];
#pragma unroll
    for (int k = 0; k < UPT; ++k) ((float4*)s_u)[min(tid + k * SB, n4 - 1)] = ub[k];
  }
  for (int i = (n4 << 2) + tid; i < a.N; i += SB) s_u[i] = src[i];
}

// U row staging and low scores of a chunk for records of 16 words whose
// first min(klow, 4) words score the token (klow <= 4). The U loads are
// issued with the first token batch; token batches are double-buffered (the
// next batch is requested before the current one is scored). LOW3: klow == 3,
// each token's three words are one 12-byte load.
template <int SPT, bool LOW3>
__device__ __forceinline__ void score_chunk(const RowsArgs& a, const float* usrc, const uint32_t* lo,
                                            int64_t t0, int64_t t1, float* s_u,
                                            uint32_t (&key)[SPT]) {
  const int tid = threadIdx.x;
  const int lw = a.low_words;
  constexpr int AMASK = kMaxAtomsDecode - 1;
  constexpr int JB = SPT < 8 ? SPT : 8;
  constexpr int NBATCH = SPT / JB;
  static_assert(SPT % JB == 0, "token batches must tile the chunk");
  uint32_t wb[2][JB][4];
  auto load_batch = [&](int jb, uint32_t (&w)[JB][4]) {
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int64_t t = min(t0 + (int64_t)(jb + jj) * SB + tid, a.T - 1);
      const uint32_t* wp = lo + t * lw;
      if (LOW3) {
        const Words3 v = *(const Words3*)wp;
        w[jj][0] = v.x; w[jj][1] = v.y; w[jj][2] = v.z; w[jj][3] = 0u;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[jj][i] = wp[min(i, a.klow - 1)];
      }
    }
  };
  load_batch(0, wb[0]);
  stage_u(a, usrc, s_u);
  __syncthreads();
  const int nk = LOW3 ? 3 : a.klow;
#pragma unroll
  for (int bt = 0; bt < NBATCH; ++bt) {
    if (bt + 1 < NBATCH) load_batch((bt + 1) * JB, wb[(bt + 1) & 1]);
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const uint32_t (&wd)[4] = wb[bt & 1][jj];
      const int64_t t = t0 + (int64_t)(bt * JB + jj) * SB + tid;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nk) s = fmaf(code_coef(wd[i]), s_u[code_idx(wd[i]) & AMASK], s);
      key[bt * JB + jj] = (t < t1) ? float_key(s) : 0u;
    }
  }
}

// EXT: the build that takes the attention flags (integer-only softmax, the
// selection shared by a KV head's query heads, reading B) from its arguments;
// the default build has them all off at compile time and keeps its registers.
template <int SPT, bool FAST, bool EXT>
__global__ __launch_bounds__(SB) void k_rows(RowsArgs a) {
  __shared__ float s_u[kMaxAtomsDecode];
  __shared__ SelShared sh;
  __shared__ float s_red[SNW];
  __shared__ uint16_t s_lt[kListCap];
  __shared__ float s_ls[kListCap];
  __shared__ uint32_t s_qcnt[5 * kMaxRowP + 1];

  const int tid = threadIdx.x;
  // Work is assigned in workgroup start order (tickets), not by block id, so
  // a row's P workgroups can wait on each other without a cooperative
  // launch (the host checks that the co-resident capacity covers a row).
  __shared__ int s_tile;
  if (tid == 0) s_tile = ticket_tile(a.ticket, a.nrows * a.P, a.xcd_map != 0);
  __syncthreads();
  const int L = s_tile;
  const int p = L % a.P;
  const int row = a.row0 + L / a.P;
  const int b = row / a.Hq, h = row % a.Hq, g = h / a.G;
  const int64_t kv = (int64_t)b * a.Hkv + g;
  const int64_t t0 = (int64_t)p * a.chunk;
  const int64_t t1 = min(a.T, t0 + a.chunk);
  constexpr int AMASK = kMaxAtomsDecode - 1;

  // 1. this query head's U row into LDS and 2. s_low of every token of the
  // chunk as order-preserving keys
  const uint32_t* lo = a.low + kv * a.T * a.low_words;
  const int lw = a.low_words;
  const bool low3 = FAST && a.klow == 3;
  uint32_t key[SPT];
  // the ranking table: this head's U row, or its group's summed row
  const bool im = EXT && a.imode, sh_sel = EXT && a.shared, rb = EXT && a.readb;
  const float* usrc = sh_sel ? a.Ug + kv * a.N : a.U + (int64_t)row * a.N;
  if (FAST) {
    if (low3) score_chunk<SPT, true>(a, usrc, lo, t0, t1, s_u, key);
    else score_chunk<SPT, false>(a, usrc, lo, t0, t1, s_u, key);
  } else {
    stage_u(a, usrc, s_u);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t t = t0 + (int64_t)j * SB + tid;
      key[j] = 0u;
      if (t < t1) {
        const uint32_t* wp = lo + t * lw;
        float s = 0.f;
        for (int i = 0; i < a.klow; ++i)
          s = fmaf(code_coef(wp[i]), s_u[code_idx(wp[i]) & AMASK], s);
        key[j] = float_key(s);
      }
    }
  }
  if (a.s_low_out) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t t = t0 + (int64_t)j * SB + tid;
      if (t < t1) a.s_low_out[(int64_t)row * a.T + t] = key_float(key[j]);
    }
  }

  // 3. exact top-m selection across the row's P workgroups
  SelGroup grp;
  grp.P = a.P;
  grp.p = p;
  grp.ghist = a.ghist + (int64_t)row * 2048;
  grp.xchg = a.xchg + (int64_t)row * a.P * 2;
  grp.bar = a.bar + 2 * (int64_t)row;
  grp.local = a.xcd_map != 0;
  grp.wait = a.wait;
  grp.cand = a.cand + (int64_t)row * a.P * a.chunk;
  grp.cap = a.chunk;
  // offset: this workgroup's first position in the row's selection (token
  // order); known from the radix selects, exchanged below when needed after
  // the window select. nbar: cross-workgroup barriers used so far.
  uint32_t offset = 0, count = 0, tau = 0, nbar = 0;
  bool need_offset = false;
  Mask sel = 0;
  if (SPT > kMaxCoopSPT || a.P == 1) {
    // single-workgroup rows (the only ones the host plans at SPT > kMaxCoopSPT)
    sel = radix_select_local<SPT>(key, (uint32_t)a.m, sh, &offset, &count, &tau);
  } else {
    // s_low of a fixed sample of the row's tokens (the same in every
    // workgroup of the row): all tokens if T <= kSampleN, else R = kSampleN /
    // 16 runs of 16 consecutive tokens, run g starting at floor(g T / R)
    // (inside the row: T > kSampleN = 16 R, so (R - 1) T / R + 15 < T)
    const int64_t ns = min((int64_t)kSampleN, a.T);
    const bool all = a.T <= kSampleN;
    uint32_t skey[kSamplePT];
    {
      uint32_t wd[kSamplePT][4];
      const uint32_t* wps[kSamplePT];
#pragma unroll
      for (int j = 0; j < kSamplePT; ++j) {
        const int64_t i = min((int64_t)(tid + j * SB), ns - 1);
        const int64_t t = all ? i : ((i >> 4) * a.T) / kSampleRuns + (i & 15);
        wps[j] = lo + t * lw;
        // (klow = 3 gets its own straight path: every instruction this kernel
        // runs is fetched from L2 once per compute unit, at a measured
        // ~0.3 us per KB, so shorter executed code is faster code)
        if (low3) {
#pragma unroll
          for (int c = 0; c < 3; ++c) wd[j][c] = wps[j][c];
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) wd[j][c] = wps[j][min(c, a.klow - 1)];
        }
      }
      if (low3) {
#pragma unroll
        for (int j = 0; j < kSamplePT; ++j) {
          float s = 0.f;
#pragma unroll
          for (int c = 0; c < 3; ++c) s = fmaf(code_coef(wd[j][c]), s_u[code_idx(wd[j][c]) & AMASK], s);
          skey[j] = (tid + j * SB < ns) ? float_key(s) : 0u;
        }
      } else
#pragma unroll
      for (int j = 0; j < kSamplePT; ++j) {
        const uint32_t* wp = wps[j];
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c < a.klow) s = fmaf(code_coef(wd[j][c]), s_u[code_idx(wd[j][c]) & AMASK], s);
        for (int c = 4; c < a.klow; ++c)
          s = fmaf(code_coef(wp[c]), s_u[code_idx(wp[c]) & AMASK], s);
        skey[j] = (tid + j * SB < ns) ? float_key(s) : 0u;
      }
    }
    nbar = 1;
    if (sample_window_select<SPT>(key, skey, (uint32_t)ns, (uint32_t)a.m, (uint32_t)a.T, sh, grp,
                                  a.wtab + (int64_t)row * a.P * 2048, &tau, &sel, s_qcnt)) {
      need_offset = a.sel_out != nullptr || a.s_high_out != nullptr || a.p_int_out != nullptr;
    } else {
      sel = radix_select_coop<SPT>(key, (uint32_t)a.m, sh, grp, &offset, &count, &tau, s_qcnt, 1u);
      nbar = 3;
    }
  }

  // 4. compaction: the selected tokens of this workgroup as offsets within
  // the chunk in LDS (this workgroup's region of the global list when they
  // do not fit), thread-major: thread t's tokens, in element order, follow
  // those of threads below t (one block scan of per-thread counts).
  int32_t* sel_g = a.sel + ((int64_t)row * a.P + p) * a.chunk;
  float* sh_g = a.s_high + ((int64_t)row * a.P + p) * a.chunk;
  uint32_t nsel;
  const uint32_t lbase = block_excl_scan<SNW>((uint32_t)__popc(sel), sh.tmp, &nsel);
  if (nsel <= (uint32_t)kListCap) {
    // (the usual case, no per-token test of the list's capacity)
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if ((sel >> j) & 1u) s_lt[lbase + (uint32_t)__popc(sel & ((1u << j) - 1u))] = (uint16_t)(j * SB + tid);
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      if ((sel >> j) & 1u) {
        const uint32_t r = lbase + (uint32_t)__popc(sel & ((1u << j) - 1u));
        if (r < (uint32_t)kListCap) s_lt[r] = (uint16_t)(j * SB + tid);
        else sel_g[r] = (int32_t)(t0 + (int64_t)j * SB + tid);
      }
    }
  }
  const int64_t cnt = nsel;
  const bool in_lds = cnt <= kListCap;
  __syncthreads();
  if (!in_lds) {
    // the whole list goes to the global region (entries below kListCap too)
    for (int64_t i = tid; i < min(cnt, (int64_t)kListCap); i += SB) sel_g[i] = (int32_t)(t0 + s_lt[i]);
    __threadfence_block();
    __syncthreads();
  }
  // debug outputs need the row-global position of this workgroup's entries
  if (need_offset) {
    if (tid == 0) st_agent(&grp.xchg[2 * p + 1], nsel);
    const bool ok = group_barrier(grp.bar, (uint32_t)a.P, ++nbar, grp.local, grp.wait);
    if (tid == 0) {
      uint32_t off = 0;
      for (int q = 0; q < p && ok; ++q) off += ld_agent(&grp.xchg[2 * q + 1]);
      sh.bcast[6] = off;
    }
    __syncthreads();
    offset = sh.bcast[6];
    __syncthreads();
  }
  int32_t* sel_dbg = a.sel_out ? a.sel_out + (int64_t)row * a.m : nullptr;
  float* sh_dbg = a.s_high_out ? a.s_high_out + (int64_t)row * a.m : nullptr;

  // shared selection: the rescore needs this head's own U row
  if (sh_sel) {
    __syncthreads();
    stage_u(a, a.U + (int64_t)row * a.N, s_u);
    __syncthreads();
  }

  // 5. Khigh rescore, one thread per selected token (entries i = tid + k*SB;
  // the same thread handles the same entries in every later loop). Value
  // records are fetched in the same pass; their |coefficient| sums bound the
  // value weights for the fixed-point accumulation below.
  const uint32_t* kbase = a.kc + kv * a.T * a.rs;
  const uint32_t* vbase = a.vc + kv * a.T * a.rs;
  const bool one_batch = cnt <= (int64_t)SB * kTokBatch;
  // (lmax, vb): running max of s_high and sum_t exp(s_t - lmax) sum_j |kappa^v_tj|
  float lmax = -INFINITY, vb = 0.f;
  float lmin = INFINITY, vmax = 0.f;  // integer mode: score range, largest sum_j |kappa^v|
  // (the 16-pair records are held in registers; other code lengths read
  // their words in the loops, so no register array is indexed at run time
  // and the kernel keeps no per-lane scratch)
  uint32_t vw[kTokBatch][32];
  for (int64_t base = 0; base < cnt; base += (int64_t)SB * kTokBatch) {
    int64_t tt[kTokBatch];
#pragma unroll
    for (int r = 0; r < kTokBatch; ++r) {
      const int64_t i = base + (int64_t)r * SB + tid;
      int64_t t = t0;
      if (i < cnt) t = in_lds ? t0 + s_lt[i] : (int64_t)sel_g[i];
      tt[r] = min(max(t, (int64_t)0), a.T - 1);
    }
    uint32_t kw[kTokBatch][32];
    if (FAST) {
#pragma unroll
      for (int r = 0; r < kTokBatch; ++r) {
        load_record(kbase + tt[r] * a.rs, kw[r]);
        load_record(vbase + tt[r] * a.rs, vw[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kTokBatch; ++r) {
      const int64_t i = base + (int64_t)r * SB + tid;
      float s = 0.f, va = 0.f;
      if (FAST && a.khigh == 16) {
        // (the usual khigh: no per-pair test, and the 16 table reads issue
        // together)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          s = fmaf(code_coef(kw[r][q]), s_u[code_idx(kw[r][q]) & AMASK], s);
          va += fabsf(code_coef(vw[r][q]));
        }
      } else if (FAST) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          if (q < a.khigh) s = fmaf(code_coef(kw[r][q]), s_u[code_idx(kw[r][q]) & AMASK], s);
          va += fabsf(code_coef(vw[r][q]));
        }
      } else {
        const uint32_t* kr = kbase + tt[r] * a.rs;
        const uint32_t* vr = vbase + tt[r] * a.rs;
        for (int q = 0; q < a.khigh; ++q)
          s = fmaf(code_coef(kr[q]), s_u[code_idx(kr[q]) & AMASK], s);
        for (int q = 0; q < a.K; ++q) va += fabsf(code_coef(vr[q]));
      }
      if (i < cnt) {
        if (in_lds) s_ls[i] = s;
        else sh_g[i] = s;
        if (im) {
          lmin = fminf(lmin, s);
          vmax = fmaxf(vmax, va);
        }
        if (s > lmax) {
          vb = vb * __expf(lmax - s) + va;
          lmax = s;
        } else {
          vb += __expf(s - lmax) * va;
        }
      }
    }
  }
  // reading B: this workgroup's unselected tokens enter with their s_low and
  // their first klow value words (value low plane, else the value records)
  const uint32_t* vlo = a.vlow ? a.vlow + kv * a.T * a.klow : vbase;
  const int64_t vlw = a.vlow ? a.klow : a.rs;
  if (rb) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t t = t0 + (int64_t)j * SB + tid;
      if (t < t1 && !((sel >> j) & 1u)) {
        float s = key_float(key[j]);
        if (sh_sel) {
          // the key holds the group's ranking score: this head's own s_low
          // (U_h is staged again by now), kept in the key for the weights
          const uint32_t* wp = lo + t * lw;
          s = 0.f;
          for (int c = 0; c < a.klow; ++c) s = fmaf(code_coef(wp[c]), s_u[code_idx(wp[c]) & AMASK], s);
          key[j] = float_key(s);
        }
        const uint32_t* vp = vlo + t * vlw;
        float va = 0.f;
        for (int c = 0; c < a.klow; ++c) va += fabsf(code_coef(vp[c]));
        if (s > lmax) {
          vb = vb * __expf(lmax - s) + va;
          lmax = s;
        } else {
          vb += __expf(s - lmax) * va;
        }
      }
    }
  }
  const float M = block_max<SNW>(lmax, s_red);
  // sum_t p_t sum_j |kappa^v_tj| over this workgroup's tokens (online-softmax
  // rescaling of each thread's running sum to the workgroup max)
  vb = (lmax > -INFINITY) ? vb * __expf(lmax - M) : 0.f;
  const float vsum = block_sum<SNW>(vb, s_red) * 1.0001f;

  // debug outputs: the selection in token order with its s_high
  if (sel_dbg || sh_dbg) {
    __threadfence_block();
    __syncthreads();
    ordered_ranks<SPT>(sel, sh, [&](int j, uint32_t r) {
      const int64_t i = (int64_t)offset + r;
      if (i < a.m) {
        const uint32_t lp = lbase + (uint32_t)__popc(sel & ((1u << j) - 1u));
        if (sel_dbg) sel_dbg[i] = (int32_t)(t0 + (int64_t)j * SB + tid);
        if (sh_dbg) sh_dbg[i] = in_lds ? s_ls[lp] : sh_g[lp];
      }
    });
  }

  // 5b. integer mode: the row's score range, every token's guarded integer
  // exponential e' (stored over its score), the row's sum of e' and the
  // 62-bit reciprocal. Two exchanges among the row's workgroups.
  uint64_t rcp = 0;
  if (im) {
    const float mn = -block_max<SNW>(-lmin, s_red);
    float smax = M, smin = mn;
    uint32_t* ix = a.ixchg + (int64_t)row * a.P * 4;
    if (a.P > 1) {
      if (tid == 0) {
        st_agent(&ix[4 * p], __float_as_uint(M));
        st_agent(&ix[4 * p + 1], __float_as_uint(mn));
      }
      const bool ok = group_barrier(grp.bar, (uint32_t)a.P, ++nbar, grp.local, grp.wait);
      if (wave_id() == 0) {
        // lane q reads workgroup q's pair: all P loads in one round trip
        const int l = lane_id();
        float qmax = smax, qmin = smin;
        if (ok && l < a.P) {
          qmax = __uint_as_float(ld_agent(&ix[4 * l]));
          qmin = __uint_as_float(ld_agent(&ix[4 * l + 1]));
        }
        qmax = fmaxf(wave_max(qmax), smax);
        qmin = fminf(-wave_max(-qmin), smin);
        if (l == 0) {
          sh.bcast[0] = __float_as_uint(qmax);
          sh.bcast[1] = __float_as_uint(qmin);
        }
      }
      __syncthreads();
      smax = __uint_as_float(sh.bcast[0]);
      smin = __uint_as_float(sh.bcast[1]);
    }
    const IntSoftmax ic = int_softmax_consts(smax, smin, a.m);
    uint32_t esum = 0;
    for (int64_t i = tid; i < cnt; i += SB) {
      float* slot = in_lds ? &s_ls[i] : &sh_g[i];
      const uint32_t e = int_exp_guarded(*slot, ic);
      *slot = __uint_as_float(e);
      esum += e;
    }
    __threadfence_block();
    uint32_t tot;
    (void)block_excl_scan<SNW>(esum, sh.tmp, &tot);
    if (a.P > 1) {
      if (tid == 0) st_agent(&ix[4 * p + 2], tot);
      const bool ok = group_barrier(grp.bar, (uint32_t)a.P, ++nbar, grp.local, grp.wait);
      if (wave_id() == 0) {
        const int l = lane_id();
        const uint32_t e = (ok && l < a.P) ? ld_agent(&ix[4 * l + 2]) : 0u;
        const uint32_t t = ok ? wave_sum_u32(e) : tot;
        if (l == 0) sh.bcast[2] = t;
      }
      __syncthreads();
      tot = sh.bcast[2];
    }
    rcp = tot ? (1ull << 62) / tot : 0ull;
    if (a.p_int_out) {
      int32_t* pd = a.p_int_out + (int64_t)row * a.m;
      ordered_ranks<SPT>(sel, sh, [&](int j, uint32_t r) {
        const int64_t i = (int64_t)offset + r;
        if (i < a.m) {
          const uint32_t lp = lbase + (uint32_t)__popc(sel & ((1u << j) - 1u));
          const uint32_t e = __float_as_uint(in_lds ? s_ls[lp] : sh_g[lp]);
          pd[i] = (int32_t)(((uint64_t)e * rcp) >> 32);
        }
      });
    }
  }
  // fixed-point scale bound: sum_t p_t sum_j |kappa^v_tj| <= the largest sum
  // when the p_t sum to at most 1 (integer mode)
  float vbound = vsum;
  if (im) vbound = block_max<SNW>(vmax, s_red) * 1.0001f;

  // 6. softmax weights and per-atom value weights. LDS integer atomics are
  // much faster than float ones on gfx950, so weights accumulate in int32
  // fixed point with a power-of-two scale S such that S * sum|p kappa| <=
  // 2^30: no bin can overflow, and each contribution is rounded to 2^-31
  // of the workgroup's total weight mass.
  const int sexp = (vbound > 0.f) ? 30 - ilogbf(vbound) - 1 : 0;
  const float S = ldexpf(1.f, min(sexp, 100));
  int32_t* s_w = (int32_t*)s_u;
  {
    const int n4 = a.N >> 2;
    for (int i = tid; i < n4; i += SB) ((int4*)s_w)[i] = make_int4(0, 0, 0, 0);
    for (int i = (n4 << 2) + tid; i < a.N; i += SB) s_w[i] = 0;
  }
  if (!in_lds) __threadfence_block();
  __syncthreads();
  float lsum = 0.f;
  for (int64_t base = 0; base < cnt; base += (int64_t)SB * kTokBatch) {
    float pt[kTokBatch];
    if (FAST && !one_batch) {
      int64_t tt[kTokBatch];
#pragma unroll
      for (int r = 0; r < kTokBatch; ++r) {
        const int64_t i = base + (int64_t)r * SB + tid;
        int64_t t = t0;
        if (i < cnt) t = in_lds ? t0 + s_lt[i] : (int64_t)sel_g[i];
        tt[r] = min(max(t, (int64_t)0), a.T - 1);
      }
#pragma unroll
      for (int r = 0; r < kTokBatch; ++r) load_record(vbase + tt[r] * a.rs, vw[r]);
    }
#pragma unroll
    for (int r = 0; r < kTokBatch; ++r) {
      const int64_t i = base + (int64_t)r * SB + tid;
      pt[r] = (i < cnt) ? (in_lds ? s_ls[i] : sh_g[i]) : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < kTokBatch; ++r) {
      const int64_t i = base + (int64_t)r * SB + tid;
      if (i < cnt) {
        const float pr = im ? (float)(((uint64_t)__float_as_uint(pt[r]) * rcp) >> 32) * 0x1p-30f
                            : __expf(pt[r] - M);
        lsum += pr;
        const float ps = pr * S;
        if (FAST) {
#pragma unroll
          for (int q = 0; q < 16; ++q)
            atomicAdd((uint32_t*)&s_w[code_idx(vw[r][q]) & AMASK],
                      (uint32_t)(int32_t)rintf(fmaf(code_coef(vw[r][q]), ps, 0.f)));
        } else {
          const int64_t t = in_lds ? t0 + s_lt[i] : (int64_t)sel_g[i];
          const uint32_t* vr = vbase + min(max(t, (int64_t)0), a.T - 1) * a.rs;
          for (int q = 0; q < a.K; ++q) {
            const uint32_t wv = vr[q];
            atomicAdd((uint32_t*)&s_w[code_idx(wv) & AMASK], (uint32_t)(int32_t)rintf(ps * code_coef(wv)));
          }
        }
      }
    }
  }
  if (rb) {
    // reading B: the unselected tokens' weights with their first klow value words
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t t = t0 + (int64_t)j * SB + tid;
      if (t < t1 && !((sel >> j) & 1u)) {
        const float pr = __expf(key_float(key[j]) - M);
        lsum += pr;
        const float ps = pr * S;
        const uint32_t* vp = vlo + t * vlw;
        for (int c = 0; c < a.klow; ++c)
          atomicAdd((uint32_t*)&s_w[code_idx(vp[c]) & AMASK],
                    (uint32_t)(int32_t)rintf(ps * code_coef(vp[c])));
      }
    }
  }
  const float lsum_all = block_sum<SNW>(lsum, s_red);
  __syncthreads();

  // 7. this workgroup's unnormalised weights and its (max, sum of exp) pair;
  // the W.Dv kernel merges the P partials of each row. The bins (|bin| <
  // 2^30) are stored as fp16 of bin * 2^-16 (below 2^14, so always finite):
  // a relative rounding of at most 2^-11 per weight. stats.z = 2^16 / S
  // turns a stored value back into a weight.
  uint16_t* dst = a.wpart + ((int64_t)row * a.P + p) * a.N;
  const int n8 = a.N >> 3;
  // (streaming stores: the partials are read once, by the next kernel)
  for (int i = tid; i < n8; i += SB) {
    const int4 v0 = ((const int4*)s_w)[2 * i], v1 = ((const int4*)s_w)[2 * i + 1];
    // (pairs converted together: one v_cvt_pk_f16_f32, round to nearest even)
    u32x4 h;
    h[0] = f32x2_to_f16x2_bits((float)v0.x * 0x1p-16f, (float)v0.y * 0x1p-16f);
    h[1] = f32x2_to_f16x2_bits((float)v0.z * 0x1p-16f, (float)v0.w * 0x1p-16f);
    h[2] = f32x2_to_f16x2_bits((float)v1.x * 0x1p-16f, (float)v1.y * 0x1p-16f);
    h[3] = f32x2_to_f16x2_bits((float)v1.z * 0x1p-16f, (float)v1.w * 0x1p-16f);
    __builtin_nontemporal_store(h, (u32x4*)(dst + 8 * i));
  }
  for (int i = (n8 << 3) + tid; i < a.N; i += SB)
    dst[i] = (uint16_t)f32_to_f16_bits((float)s_w[i] * 0x1p-16f);
  // (integer mode: the weights are already normalised; the merge adds them)
  if (tid == 0)
    a.stats[(int64_t)row * a.P + p] =
        make_float4(im ? 0.f : M, im ? 1.f : lsum_all, ldexpf(1.f, 16 - min(sexp, 100)), 0.f);
}

// ---------------------------------------------------------------------------
// out = W . Dv  (split-K over atom chunks, then a fixed-order sum)
// ---------------------------------------------------------------------------
struct WdvArgs {
  const uint16_t* wpart;  // [rows, P, N] unnormalised per-workgroup weights (fp16, scaled)
  const float4* stats;    // [rows, P] (max, sum of exp, weight scale, 0) per partial
  const void* dv;         // [N, d]
  int N, d, P, rows, nrt, nsub, nchunks;
  float* opart;           // [nchunks, rows, d]
  float* w_out;           // optional [rows, N] normalised weights
  int presum;             // partials already normalised (integer softmax): add them
};

constexpr int WSUB = 128;                 // atoms per MFMA sub-chunk
constexpr int WRT = 32;                   // rows per workgroup tile
constexpr int WPITCH = WSUB + 8;          // u16 per A row in LDS
constexpr int BPITCH = WSUB / 2 + 4;      // u32 (atom pairs) per B row in LDS

// s_coef[r][q] = g_q exp(M_q - max_q M_q) / sum_q exp(M_q - max M) l_q for
// the tile's rows: the softmax merge of the row's P partial results, with
// g_q the scale that turns partial q's stored fp16 values into weights.
__device__ __forceinline__ void wdv_coefs(const WdvArgs& a, int r0, float* s_coef) {
  const int w = wave_id(), l = lane_id();
  for (int r = w; r < WRT; r += 4) {
    const int row = r0 + r;
    float Mq = -INFINITY, lq = 0.f, gq = 0.f;
    if (row < a.rows && l < a.P) {
      const float4 st = a.stats[(int64_t)row * a.P + l];
      Mq = st.x;
      lq = st.y;
      gq = st.z;
    }
    const float Mx = wave_max(Mq);
    const float c = (lq > 0.f) ? __expf(Mq - Mx) : 0.f;
    const float Lr = wave_sum(c * lq);
    if (l < a.P) s_coef[r * kMaxRowP + l] = gq * (a.presum ? 1.f : (Lr > 0.f) ? c / Lr : 0.f);
  }
}

// 16 merged weights W[row][a0 .. a0+16) (zero outside the matrix)
__device__ __forceinline__ void wdv_merge16(const WdvArgs& a, const float* s_coef, int r, int row,
                                            int a0, float (&v)[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = 0.f;
  if (row >= a.rows) return;
  const uint16_t* src = a.wpart + (int64_t)row * a.P * a.N + a0;
  if (a0 + 16 <= a.N && (a.N & 7) == 0) {
#pragma unroll 4
    for (int q = 0; q < a.P; ++q) {
      const float c = s_coef[r * kMaxRowP + q];
      const u32x4* sp = (const u32x4*)(src + (int64_t)q * a.N);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4 x = sp[k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * k + 2 * j] = fmaf(c, f16_bits_to_f32(x[j] & 0xFFFFu), v[8 * k + 2 * j]);
          v[8 * k + 2 * j + 1] = fmaf(c, f16_bits_to_f32(x[j] >> 16), v[8 * k + 2 * j + 1]);
        }
      }
    }
  } else {
    for (int q = 0; q < a.P; ++q) {
      const float c = s_coef[r * kMaxRowP + q];
      for (int e = 0; e < 16 && a0 + e < a.N; ++e)
        v[e] = fmaf(c, f16_bits_to_f32(src[(int64_t)q * a.N + e]), v[e]);
    }
  }
  if (a.w_out) {
    float* wo = a.w_out + (int64_t)row * a.N + a0;
    for (int e = 0; e < 16 && a0 + e < a.N; ++e) wo[e] = v[e];
  }
}

// 512 threads: the A tile (RT = 32 or 64 rows x 128 atoms) is merged 8
// atoms per thread and row (RT / 32 rows per thread); wave w computes output
// columns [16w, 16w+16) for all RT / 16 row tiles. Taller tiles read each Dv
// sub-chunk for more rows (layers with many query rows). The loads of a
// sub-chunk (up to 8 weight partials per thread, and the Dv rows)
// are issued before anything waits on them; the first sub-chunk's loads go
// out before the softmax-merge coefficients are computed.
constexpr int WDV_PQ = 8;                 // partials per prefetched batch
template <int RT>
__global__ __launch_bounds__(512) void k_wdv_bf16(WdvArgs a) {
  static_assert(RT == 32 || RT == 64, "row tile height");
  constexpr int RPT = RT / 32;            // A rows per thread
  constexpr int NRT = RT / 16;            // 16-row MFMA tiles
  constexpr int PQ = WDV_PQ / RPT;        // partials per row prefetched
  __shared__ float s_coef[RT * kMaxRowP];
  __shared__ __attribute__((aligned(16))) uint16_t s_ahi[RT * WPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t s_alo[RT * WPITCH];
  __shared__ __attribute__((aligned(16))) uint32_t s_bt[128 * BPITCH];

  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int L = xcd_tile(blockIdx.x, a.nchunks * a.nrt);
  const int chunk = L / a.nrt, rt = L % a.nrt;
  const int r0 = rt * RT;
  const uint16_t* dv = (const uint16_t*)a.dv;
  const int ncol = a.d >> 4;
  // this thread's A slots (rows ar + 32 u, atoms c0 .. c0+8) and B items
  const int ar = tid >> 4, ac0 = (tid & 15) * 8;
  const bool a_fast = (a.N & 7) == 0;
  constexpr int BIT = (WSUB / 2) * (128 / 8) / 512;  // B items per thread (d = 128)
  u32x4 px[RPT][PQ];
  u32x4 bx[BIT][2];
  auto load_sub = [&](int a0) {
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int arow = r0 + ar + 32 * u;
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
        px[u][q] = u32x4{0u, 0u, 0u, 0u};
        if (q < a.P && arow < a.rows && a_fast && a0 + ac0 + 8 <= a.N)
          px[u][q] = *(const u32x4*)(a.wpart + ((int64_t)arow * a.P + q) * a.N + a0 + ac0);
      }
    }
#pragma unroll
    for (int k = 0; k < BIT; ++k) {
      const int it = tid + k * 512;
      const int ap = it % (WSUB / 2), sg = it / (WSUB / 2);
      const int atom = a0 + 2 * ap;
      bx[k][0] = u32x4{0u, 0u, 0u, 0u};
      bx[k][1] = bx[k][0];
      if (sg < (a.d >> 3)) {
        if (atom < a.N) bx[k][0] = *(const u32x4*)(dv + (int64_t)atom * a.d + 8 * sg);
        if (atom + 1 < a.N) bx[k][1] = *(const u32x4*)(dv + (int64_t)(atom + 1) * a.d + 8 * sg);
      }
    }
  };
  int a0 = chunk * a.nsub * WSUB;
  if (a0 < a.N) load_sub(a0);

  // softmax-merge coefficients of the tile's rows (all stats loads first)
  {
    float4 st[RT / 8];
#pragma unroll
    for (int k = 0; k < RT / 8; ++k) {
      const int row = r0 + w + 8 * k;
      st[k] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
      if (row < a.rows && l < a.P) st[k] = a.stats[(int64_t)row * a.P + l];
    }
#pragma unroll
    for (int k = 0; k < RT / 8; ++k) {
      const float Mq = st[k].x, lq = st[k].y;
      const float Mx = wave_max(Mq);
      const float c = (lq > 0.f) ? __expf(Mq - Mx) : 0.f;
      const float Lr = wave_sum(c * lq);
      if (l < a.P)
        s_coef[(w + 8 * k) * kMaxRowP + l] =
            st[k].z * (a.presum ? 1.f : (Lr > 0.f) ? c / Lr : 0.f);
    }
  }
  __syncthreads();
  f32x4 acc[NRT];
#pragma unroll
  for (int rr = 0; rr < NRT; ++rr) acc[rr] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int sub = 0; sub < a.nsub; ++sub) {
    a0 = (chunk * a.nsub + sub) * WSUB;
    if (a0 >= a.N) break;
    if (sub > 0) load_sub(a0);
    // A: merged weights of (row, atoms ac0 .. ac0+8), split into bf16 hi + lo
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int lr = ar + 32 * u, arow = r0 + lr;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
      if (arow < a.rows) {
        if (a_fast && a0 + ac0 + 8 <= a.N) {
#pragma unroll
          for (int q = 0; q < PQ; ++q) {
            if (q < a.P) {
              const float c = s_coef[lr * kMaxRowP + q];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                v[2 * j] = fmaf(c, f16_bits_to_f32(px[u][q][j] & 0xFFFFu), v[2 * j]);
                v[2 * j + 1] = fmaf(c, f16_bits_to_f32(px[u][q][j] >> 16), v[2 * j + 1]);
              }
            }
          }
          // partials beyond the prefetched batch
          for (int q = PQ; q < a.P; ++q) {
            const float c = s_coef[lr * kMaxRowP + q];
            const u32x4 x = *(const u32x4*)(a.wpart + ((int64_t)arow * a.P + q) * a.N + a0 + ac0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[2 * j] = fmaf(c, f16_bits_to_f32(x[j] & 0xFFFFu), v[2 * j]);
              v[2 * j + 1] = fmaf(c, f16_bits_to_f32(x[j] >> 16), v[2 * j + 1]);
            }
          }
        } else {
          const uint16_t* src = a.wpart + (int64_t)arow * a.P * a.N + a0 + ac0;
          for (int q = 0; q < a.P; ++q) {
            const float c = s_coef[lr * kMaxRowP + q];
            for (int e = 0; e < 8 && a0 + ac0 + e < a.N; ++e)
              v[e] = fmaf(c, f16_bits_to_f32(src[(int64_t)q * a.N + e]), v[e]);
          }
        }
        if (a.w_out) {
          float* wo = a.w_out + (int64_t)arow * a.N + a0 + ac0;
          for (int e = 0; e < 8 && a0 + ac0 + e < a.N; ++e) wo[e] = v[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t h0 = f32_to_bf16_rne(v[e]), h1 = f32_to_bf16_rne(v[e + 1]);
        const uint32_t l0 = f32_to_bf16_rne(v[e] - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_rne(v[e + 1] - __uint_as_float(h1 << 16));
        *(uint32_t*)&s_ahi[lr * WPITCH + ac0 + e] = h0 | (h1 << 16);
        *(uint32_t*)&s_alo[lr * WPITCH + ac0 + e] = l0 | (l1 << 16);
      }
    }
    // B: Dv rows a0..a0+127 transposed to [dim][atom pair]
#pragma unroll
    for (int k = 0; k < BIT; ++k) {
      const int it = tid + k * 512;
      const int ap = it % (WSUB / 2), sg = it / (WSUB / 2);
      if (sg < (a.d >> 3)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s_bt[(8 * sg + 2 * i) * BPITCH + ap] = (bx[k][0][i] & 0xFFFFu) | (bx[k][1][i] << 16);
          s_bt[(8 * sg + 2 * i + 1) * BPITCH + ap] = (bx[k][0][i] >> 16) | (bx[k][1][i] & 0xFFFF0000u);
        }
      }
    }
    __syncthreads();
    if (w < ncol) {
#pragma unroll
      for (int ks = 0; ks < WSUB / 32; ++ks) {
        const int kk = ks * 32 + 8 * (l >> 4);
        const u32x4 b0 = *(const u32x4*)(s_bt + (16 * w + (l & 15)) * BPITCH + (kk >> 1));
#pragma unroll
        for (int rr = 0; rr < NRT; ++rr) {
          const u32x4 ah = *(const u32x4*)(s_ahi + (rr * 16 + (l & 15)) * WPITCH + kk);
          const u32x4 al = *(const u32x4*)(s_alo + (rr * 16 + (l & 15)) * WPITCH + kk);
          acc[rr] = mfma_bf16(ah, b0, acc[rr]);
          acc[rr] = mfma_bf16(al, b0, acc[rr]);
        }
      }
    }
    __syncthreads();
  }
  if (w < ncol) {
    float* dst = a.opart + (int64_t)chunk * a.rows * a.d;
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + rr * 16 + 4 * (l >> 4) + i;
        if (row < a.rows) dst[(int64_t)row * a.d + 16 * w + (l & 15)] = acc[rr][i];
      }
  }
}

// fp32 value dictionary (small configurations): plain fp32 FMAs.
__global__ __launch_bounds__(256) void k_wdv_f32(WdvArgs a) {
  __shared__ float s_coef[WRT * kMaxRowP];
  __shared__ float s_w[WRT * WSUB];
  const int tid = threadIdx.x;
  const int L = xcd_tile(blockIdx.x, a.nchunks * a.nrt);
  const int chunk = L / a.nrt, rt = L % a.nrt;
  const int r0 = rt * WRT;
  wdv_coefs(a, r0, s_coef);
  __syncthreads();
  const float* dv = (const float*)a.dv;
  const int r = tid >> 3;            // row within the tile
  const int c0 = (tid & 7) * 16;     // 16 output columns per thread
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int sub = 0; sub < a.nsub; ++sub) {
    const int a0 = (chunk * a.nsub + sub) * WSUB;
    if (a0 >= a.N) break;
    {
      float v[16];
      const int rr = tid >> 3, c1 = (tid & 7) * 16;
      wdv_merge16(a, s_coef, rr, r0 + rr, a0 + c1, v);
#pragma unroll
      for (int e = 0; e < 16; ++e) s_w[rr * WSUB + c1 + e] = v[e];
    }
    __syncthreads();
    const int na = min(WSUB, a.N - a0);
    if (c0 < a.d) {
      for (int k = 0; k < na; ++k) {
        const float wv = s_w[r * WSUB + k];
        const float* drow = dv + (int64_t)(a0 + k) * a.d + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = fmaf(wv, drow[i], acc[i]);
      }
    }
    __syncthreads();
  }
  const int row = r0 + r;
  if (row < a.rows && c0 < a.d) {
    float* dst = a.opart + ((int64_t)chunk * a.rows + row) * a.d + c0;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = acc[i];
  }
}

// out[o] = sum_c opart[c][o] in a fixed order: 16 threads per output each
// sum every 16th chunk, then a fixed-order combine in LDS.
constexpr int RED_OUT = 64;   // outputs per workgroup
// Thread (o, q) sums chunks q, q+16, q+32, ... of output o; each block of 16
// such loads is issued before it is summed. Fixed order: deterministic.
__global__ __launch_bounds__(1024) void k_reduce_out(const float* opart, int nchunks, int64_t n,
                                                     float* out) {
  __shared__ float s_p[16][RED_OUT + 1];
  const int o = threadIdx.x % RED_OUT, q = threadIdx.x / RED_OUT;
  const int64_t i = (int64_t)blockIdx.x * RED_OUT + o;
  float s = 0.f;
  if (i < n) {
    for (int c0 = q; c0 < nchunks; c0 += 256) {
      float x[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int c = c0 + 16 * k;
        x[k] = (c < nchunks) ? opart[(int64_t)c * n + i] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) s += x[k];
    }
  }
  s_p[q][o] = s;
  __syncthreads();
  if (q == 0 && i < n) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += s_p[k][o];
    out[i] = t;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int spt_for(int64_t chunk) {
  const int64_t need = (chunk + SB - 1) / SB;
  for (int s : {4, 8, 16, 32})
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
  // a row is split only into chunks of at least 4096 tokens: below that the
  // cross-workgroup exchange costs more than the split saves
  const int64_t p_cap = std::max<int64_t>(1, (T + 4095) / 4096);
  int64_t P = std::max(p_min, std::min(p_par, p_cap));
  // rows split over several workgroups hold at most kMaxCoopSPT keys per
  // thread (the 32-key row kernel is built for single-workgroup rows only)
  if (P > 1) P = std::max(P, (T + kMaxCoopChunk - 1) / kMaxCoopChunk);
  if (P > kMaxRowP) return SDKV_ERR_UNSUPPORTED;
  q.P = (int)P;
  q.chunk = (T + P - 1) / P;
  q.spt = spt_for(q.chunk);
  if (q.spt == 0) return SDKV_ERR_UNSUPPORTED;
  q.fast = (a->K == 16 && a->klow <= 4 && a->khigh <= 16) ? 1 : 0;
  // W.Dv row tiles: 64 rows with a bf16 dictionary when there are more than
  // 32 query rows (each Dv sub-chunk is then read for twice the rows)
  q.wrt = (a->dict_dtype == SDKV_BF16 && q.rows > 32) ? 64 : WRT;
  q.nrt = (int)((q.rows + q.wrt - 1) / q.wrt);
  const int nsub_total = (a->n_atoms + WSUB - 1) / WSUB;
  // about one W.Dv workgroup per compute unit: more atom chunks would each
  // add an output partial for k_reduce_out to read
  const int target = std::max(1, kPlanCUs / q.nrt);
  q.nsub = std::max(1, (nsub_total + target - 1) / target);
  q.nchunks = (nsub_total + q.nsub - 1) / q.nsub;

  const size_t A = 256;
  const int64_t N = a->n_atoms, rows = q.rows;
  size_t off = 0;
  // cleared per call (by the U-table kernel): the status word first (word 0
  // of the workspace), tickets, barrier counters, exchange words, histograms
  q.off_zero = 0;
  q.off_err = off;    off += 4;
  q.off_ticket = off; off += 8 * 4;
  q.off_bar = off;    off += (size_t)rows * 2 * 4;
  q.off_xchg = off;   off += (size_t)rows * q.P * 2 * 4;
  q.off_ghist = off;  off += (q.P > 1) ? (size_t)rows * 2048 * 4 : 0;
  off = align_up(off, A);
  q.zero_bytes = off - q.off_zero;
  q.off_u = off;      off = align_up(off + (size_t)rows * N * 4, A);
  const size_t list = (size_t)rows * q.P * q.chunk * 4;  // per-workgroup regions
  q.off_sel = off;    off = align_up(off + list, A);
  q.off_shigh = off;  off = align_up(off + list, A);
  q.off_wpart = off;  off = align_up(off + (size_t)rows * q.P * N * 2, A);
  q.off_stats = off;  off = align_up(off + (size_t)rows * q.P * 16, A);
  q.off_opart = off;  off = align_up(off + (size_t)q.nchunks * rows * a->d * 4, A);
  q.off_cand = off;   off = align_up(off + (q.P > 1 ? (size_t)rows * q.P * q.chunk * 4 : 0), A);
  q.off_wtab = off;   off = align_up(off + (q.P > 1 ? (size_t)rows * q.P * 2048 * 4 : 0), A);
  q.off_ixchg = off;  off = align_up(off + (size_t)rows * q.P * 4 * 4, A);
  q.off_ug = off;     off = align_up(off + (a->select_mode == SDKV_SELECT_KV
                                            ? (size_t)a->B * a->Hkv * N * 4 : 0), A);
  q.total = off;
  *p = q;
  return SDKV_OK;
}

template <int S, bool EXT>
static const void* rows_kernel(bool fast) {
  return fast ? (const void*)&k_rows<S, true, EXT> : (const void*)&k_rows<S, false, EXT>;
}

static const void* pick_rows_kernel(int spt, bool fast, bool ext) {
#define SDKV_PICK(S) \
  if (spt == S) return ext ? rows_kernel<S, true>(fast) : rows_kernel<S, false>(fast);
  SDKV_PICK(4)
  SDKV_PICK(8)
  SDKV_PICK(16)
  SDKV_PICK(32)
#undef SDKV_PICK
  return nullptr;
}

sdkv_status launch_decode(const sdkv_attn_args* a, const DecodePlan& p, void* ws,
                          hipStream_t stream) {
  char* base = (char*)ws;
  const int64_t rows = p.rows;
  float* U = (float*)(base + p.off_u);
  int32_t* sel = (int32_t*)(base + p.off_sel);
  float* shigh = (float*)(base + p.off_shigh);
  uint16_t* wpart = (uint16_t*)(base + p.off_wpart);
  float4* stats = (float4*)(base + p.off_stats);
  uint32_t* ghist = (uint32_t*)(base + p.off_ghist);
  uint32_t* xchg = (uint32_t*)(base + p.off_xchg);
  uint32_t* bar = (uint32_t*)(base + p.off_bar);
  uint32_t* err = (uint32_t*)(base + p.off_err);
  float* opart = (float*)(base + p.off_opart);
  void* const* ev = a->stage_events;

  // 1. U table (+ clear the barrier / histogram region)
  UArgs ua;
  ua.q = a->q;
  ua.q_f32 = a->q_dtype == SDKV_F32 ? 1 : 0;
  ua.dk = a->dk;
  ua.rows = (int)rows;
  ua.N = a->n_atoms;
  ua.d = a->d;
  ua.scale = a->scale;
  ua.U = U;
  ua.u_dbg = a->u;
  ua.zero = (uint32_t*)(base + p.off_zero);
  ua.zero_words = (int64_t)(p.zero_bytes / 4);
  const bool shared = a->select_mode == SDKV_SELECT_KV;
  const bool ug_in_utable = shared && a->dict_dtype == SDKV_BF16;
  ua.Ug = (float*)(base + p.off_ug);
  ua.ngroups = ug_in_utable ? a->B * a->Hkv : 0;
  ua.Hq = a->Hq;
  ua.Hkv = a->Hkv;
  ua.G = a->Hq / a->Hkv;
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

  // shared selection with an fp32 dictionary: the group sums of U
  if (shared && !ug_in_utable) {
    const int64_t n = (int64_t)a->B * a->Hkv * a->n_atoms;
    hipLaunchKernelGGL(k_usum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, U,
                       (float*)(base + p.off_ug), n, a->n_atoms, a->Hq / a->Hkv);
    if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  }

  // 2. row kernel, in row batches that fit co-resident when cooperative
  RowsArgs ra;
  ra.U = U;
  ra.low = a->key_low ? a->key_low : a->key_codes;
  ra.rs = a->code_stride ? a->code_stride : a->K;
  ra.low_words = a->key_low ? a->klow : (int)ra.rs;
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
  ra.sel_out = a->sel;
  ra.s_high_out = a->s_high;
  ra.wpart = wpart;
  ra.stats = stats;
  ra.ghist = ghist;
  ra.wtab = (uint32_t*)(base + p.off_wtab);
  ra.cand = (uint32_t*)(base + p.off_cand);
  ra.xchg = xchg;
  ra.bar = bar;
  ra.wait = wait_ctl(err);
  ra.shared = a->select_mode == SDKV_SELECT_KV ? 1 : 0;
  ra.readb = a->reading == SDKV_READING_B ? 1 : 0;
  ra.vlow = a->val_low;
  ra.Ug = (const float*)(base + p.off_ug);
  ra.imode = a->softmax_mode == SDKV_SOFTMAX_INT ? 1 : 0;
  ra.p_int_out = ra.imode ? a->p_int : nullptr;
  ra.ixchg = (uint32_t*)(base + p.off_ixchg);
  const bool aligned = (((uintptr_t)a->key_codes | (uintptr_t)a->val_codes) & 15u) == 0 &&
                       ra.rs % 4 == 0;
  const void* kfn = pick_rows_kernel(p.spt, p.fast && aligned,
                                     ra.imode != 0 || ra.shared != 0 || ra.readb != 0);
  if (!kfn) return SDKV_ERR_UNSUPPORTED;
  ra.ticket = (uint32_t*)(base + p.off_ticket);
  // Per-XCD ticket classes need whole rows per class; with P > 1 every
  // class must also hold two rows' workgroups co-resident.
  const int64_t nb = rows * p.P;
  bool xcd = nb % 8 == 0 && (nb / 8) % p.P == 0;
  if (p.P > 1) {
    int cap = 0;
    sdkv_status st = coresident_blocks(kfn, SB, 0, &cap);
    if (st != SDKV_OK) return st;
    if (cap < p.P) return SDKV_ERR_UNSUPPORTED;
    xcd = xcd && 16 * p.P <= cap;
  }
  ra.xcd_map = xcd ? 1 : 0;
  if (!record_stage(ev, 1, stream)) return SDKV_ERR_DEVICE;
  {
    ra.row0 = 0;
    ra.nrows = (int)rows;
    const dim3 grid((unsigned)(rows * p.P)), block(SB);
    void* args[] = {&ra};
    if (hipLaunchKernel(kfn, grid, block, args, 0, stream) != hipSuccess) return SDKV_ERR_DEVICE;
  }

  // 3. contract the value weights with Dv
  WdvArgs wa;
  wa.wpart = wpart;
  wa.stats = stats;
  wa.presum = a->softmax_mode == SDKV_SOFTMAX_INT ? 1 : 0;
  wa.P = p.P;
  wa.w_out = a->w;
  wa.dv = a->dv;
  wa.N = a->n_atoms;
  wa.d = a->d;
  wa.rows = (int)rows;
  wa.nrt = p.nrt;
  wa.nsub = p.nsub;
  wa.nchunks = p.nchunks;
  wa.opart = opart;
  const dim3 wgrid((unsigned)(p.nchunks * p.nrt));
  if (!record_stage(ev, 2, stream)) return SDKV_ERR_DEVICE;
  if (a->dict_dtype == SDKV_BF16)
  {
    if (p.wrt == 64) hipLaunchKernelGGL(k_wdv_bf16<64>, wgrid, dim3(512), 0, stream, wa);
    else hipLaunchKernelGGL(k_wdv_bf16<32>, wgrid, dim3(512), 0, stream, wa);
  }
  else
    hipLaunchKernelGGL(k_wdv_f32, wgrid, dim3(256), 0, stream, wa);
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;

  const int64_t nout = rows * a->d;
  if (!record_stage(ev, 3, stream)) return SDKV_ERR_DEVICE;
  hipLaunchKernelGGL(k_reduce_out, dim3((unsigned)((nout + RED_OUT - 1) / RED_OUT)), dim3(1024), 0,
                     stream, (const float*)opart, p.nchunks, nout, a->out);
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  if (!record_stage(ev, 4, stream)) return SDKV_ERR_DEVICE;
  return SDKV_OK;
}

}  // namespace sdkv
