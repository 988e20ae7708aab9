// Greedy projection pursuit encode on gfx950 ("LLM Inference in a Flash!",
// review page, Summary and Strengths: one atom is projected out per step and,
// unlike OMP, no least-squares problem is ever re-solved; K atoms per
// key/value vector over a per-layer, per-stream dictionary).
//
// Per vector x:  r = x;  for k < K: a_k = argmax_a |<r, d_a>| (lowest index on
// ties), g_k = <r, d_{a_k}>, r -= g_k d_{a_k}.
//
// Structure (one workgroup = 4 waves = 256 vectors, all K steps inside; two
// workgroups share a compute unit, so one's chunk barriers do not stall the
// other's matrix work):
//   * screen: every step correlates the workgroup's residuals with all atoms
//     on the matrix cores (v_mfma_f32_16x16x32_f16). The residual rows are
//     scaled by a power of two and rounded to fp16; the dictionary is an fp16
//     copy (exact for bf16 atoms of unit-norm size). Each lane owns one atom
//     column (atoms = c mod 16) for the rows it holds and keeps the two
//     largest screened |c| of that column, each packed in one word: |c| with
//     its low 12 mantissa bits replaced by the complement of the 16-atom tile
//     index (and bit 31 marking a filled slot), so unsigned max / median
//     operations keep the larger values and, among equal truncated values,
//     the lower tile.
//   * exact pick: E bounds |exact - screened| for every atom (fp16 rounding
//     of the residual and, for fp32 dictionaries, of the atoms, plus the
//     truncation; derived below). Every kept value within 2E of the best is
//     recomputed in fp32 from the original dictionary; the largest exact |c|
//     wins, lowest atom index on ties. A column whose second value lies
//     within E of that winner may hide a third candidate: its atoms are then
//     all recomputed exactly by the whole wave (rare). Every atom that is not
//     recomputed is therefore exactly below the winner, so the pick is the
//     exact fp32 argmax.
//   * update: g = exact <r, d_a> (fp32), r -= g d_a in fp32.
#include "sdkv_device.h"
#include "sdkv_internal.h"

namespace sdkv {

constexpr int EB = 256;            // threads per workgroup (two per CU: <= 256 VGPRs)
constexpr int ENW = EB / 64;       // waves
constexpr int EROWS = ENW * 64;    // vectors per workgroup (64 per wave)
constexpr int ECH = 64;            // atoms per LDS chunk
constexpr int kPrepBlocks = 256;   // workgroups of the dictionary prep kernel

struct EncArgs {
  const void* x;
  int x_f32;
  const void* dict;
  int dict_f32;
  const uint16_t* dh;   // [npad, D] fp16 screen copy
  const float* dnorm;   // [kPrepBlocks] largest atom norm seen by each prep workgroup
  float* r;             // [n, D] residuals (workspace)
  int64_t n;
  int N, npad, K, klow;
  uint32_t* codes;
  int64_t codes_ld;
  float* coef_f32;
  float* resid_norm;
  uint32_t* low_plane;
  int64_t low_ld;
};

// fp16 screen copy of the dictionary (zero rows past N) and the largest atom
// norm: 8 consecutive elements per thread (one 16-byte store), the row's
// threads reduce its squared norm with lane shuffles, and each workgroup
// writes the largest norm it saw to dnorm[blockIdx.x].
__global__ __launch_bounds__(256) void k_prep_dict(const void* dict, int dict_f32, int N,
                                                   int npad, int D, uint16_t* dh, float* dnorm) {
  __shared__ float s_m[4];
  const int64_t groups = (int64_t)npad * D / 8;  // D / 8 groups per row (8 or 16 lanes)
  const int gpr = D / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  float mx = 0.f;
  // the trip count is the same for every lane of a row's lanes (rows never
  // straddle a stride: stride and gpr are powers of two with gpr | stride)
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const int a = (int)(g / gpr);
    float v[8];
    if (a < N) {
      if (dict_f32) {
        const float4* p = (const float4*)((const float*)dict + g * 8);
        const float4 x0 = p[0], x1 = p[1];
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      } else {
        const u32x4 u = *(const u32x4*)((const uint16_t*)dict + g * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[2 * e] = bf16_lo(u[e]); v[2 * e + 1] = bf16_hi(u[e]); }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    u32x4 o;
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = f32_to_f16_bits(v[2 * e]) | (f32_to_f16_bits(v[2 * e + 1]) << 16);
      s2 = fmaf(v[2 * e], v[2 * e], s2);
      s2 = fmaf(v[2 * e + 1], v[2 * e + 1], s2);
    }
    *(u32x4*)(dh + g * 8) = o;
    for (int off = gpr / 2; off > 0; off >>= 1) s2 += __shfl_xor(s2, off, 64);
    mx = fmaxf(mx, sqrtf(s2));
  }
  mx = wave_max(mx);
  if (lane_id() == 0) s_m[wave_id()] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    dnorm[blockIdx.x] = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
}

// median of three (v_med3_u32)
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}
// the same as one v_med3_u32 the optimiser cannot see into: next to
// max(a, max(b, c)), the min/max form shares max(a, b) with it and the
// maximum then takes two ops instead of one v_max3_u32
__device__ __forceinline__ uint32_t med3_u32_op(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int D>
__device__ __forceinline__ float exact_corr(const EncArgs& a, const float* rrow, int atom) {
  float s = 0.f;
  if (a.dict_f32) {
    const float4* dp = (const float4*)((const float*)a.dict + (int64_t)atom * D);
#pragma unroll 4
    for (int k = 0; k < D / 4; ++k) {
      const float4 dv = dp[k];
      const float4 rv = ((const float4*)rrow)[k];
      s = fmaf(rv.x, dv.x, s); s = fmaf(rv.y, dv.y, s);
      s = fmaf(rv.z, dv.z, s); s = fmaf(rv.w, dv.w, s);
    }
  } else {
    const u32x4* dp = (const u32x4*)((const uint16_t*)a.dict + (int64_t)atom * D);
#pragma unroll 4
    for (int k = 0; k < D / 8; ++k) {
      const u32x4 dv = dp[k];
      const float4 r0 = ((const float4*)rrow)[2 * k];
      const float4 r1 = ((const float4*)rrow)[2 * k + 1];
      s = fmaf(r0.x, bf16_lo(dv[0]), s); s = fmaf(r0.y, bf16_hi(dv[0]), s);
      s = fmaf(r0.z, bf16_lo(dv[1]), s); s = fmaf(r0.w, bf16_hi(dv[1]), s);
      s = fmaf(r1.x, bf16_lo(dv[2]), s); s = fmaf(r1.y, bf16_hi(dv[2]), s);
      s = fmaf(r1.z, bf16_lo(dv[3]), s); s = fmaf(r1.w, bf16_hi(dv[3]), s);
    }
  }
  return s;
}

template <int D>
__global__ __launch_bounds__(EB, 2) void k_encode(EncArgs a) {
  constexpr int KS = D / 32;           // MFMA k-steps per 16x16 tile
  constexpr int BP = D + 8;            // LDS row pitch (fp16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][ECH * BP];
  __shared__ uint32_t s_k1[EROWS * 16];  // per row and column: best screened key
  __shared__ uint32_t s_k2[EROWS * 16];  // and the second best (0: none)
  __shared__ float s_scale[EROWS];
  __shared__ float s_rnorm[EROWS];
  __shared__ float s_snorm[EROWS];       // |r * scale| from the fp32 residual
  __shared__ float s_dmax;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t row0 = (int64_t)blockIdx.x * EROWS;

  // largest atom norm (from the prep kernel's per-workgroup maxima)
  if (w == 0) {
    float dm = 0.f;
    for (int i = l; i < kPrepBlocks; i += 64) dm = fmaxf(dm, a.dnorm[i]);
    dm = wave_max(dm);
    if (l == 0) s_dmax = dm;
  }

  // --- init: r = x, |r| ---------------------------------------------------------
  {
    const int64_t rowg = row0 + tid;
    float nrm = 0.f;
    if (rowg < a.n) {
      float* rr = a.r + rowg * D;
      for (int k = 0; k < D; ++k) {
        const float v = a.x_f32 ? ((const float*)a.x)[rowg * D + k]
                                : bf16_to_f32(((const uint16_t*)a.x)[rowg * D + k]);
        rr[k] = v;
        nrm = fmaf(v, v, nrm);
      }
    }
    s_rnorm[tid] = sqrtf(nrm);
  }
  // residual rows are exchanged between waves of this workgroup through
  // global memory: workgroup-scope ordering (part of __syncthreads) suffices
  __syncthreads();

  const int nchunks = a.npad / ECH;
  for (int step = 0; step < a.K; ++step) {
    // --- A fragments: this wave's 64 residual rows, scaled fp16 ------------------
    u32x4 af[4][KS];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int rl = w * 64 + rt * 16 + (l & 15);
      const int64_t rowg = row0 + rl;
      float vals[KS][8];
      float mx = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
        if (rowg < a.n) {
          const float* src = a.r + rowg * D + 32 * s + 8 * (l >> 4);
          v0 = ((const float4*)src)[0];
          v1 = ((const float4*)src)[1];
        }
        vals[s][0] = v0.x; vals[s][1] = v0.y; vals[s][2] = v0.z; vals[s][3] = v0.w;
        vals[s][4] = v1.x; vals[s][5] = v1.y; vals[s][6] = v1.z; vals[s][7] = v1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(vals[s][e]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // power-of-two scale putting the row's largest |r| in [1, 2)
      const float sc = (mx > 0.f) ? ldexpf(1.f, min(-ilogbf(mx), 100)) : 1.f;
      // |r * sc| (0 exactly when r is zero, else >= 1)
      float s2 = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) s2 = fmaf(vals[s][e] * sc, vals[s][e] * sc, s2);
      s2 += __shfl_xor(s2, 16, 64);
      s2 += __shfl_xor(s2, 32, 64);
      if ((l >> 4) == 0) {
        s_scale[rl] = sc;
        s_snorm[rl] = sqrtf(s2);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pk[e] = f32_to_f16_bits(vals[s][2 * e] * sc) | (f32_to_f16_bits(vals[s][2 * e + 1] * sc) << 16);
        af[rt][s] = pk;
      }
    }

    // --- screen sweep over all atoms ------------------------------------------
    // the two largest keys per output row and atom column: |c| with its low
    // 12 mantissa bits replaced by the complement of the 16-atom tile index,
    // bit 31 set (0 = empty slot), so unsigned order is |c| order and, among
    // equal truncated values, the lower tile first
    uint32_t bkey[4][4], bkey2[4][4];
    // the mask lives in a register, so (x & mask) | code is one 3-input op
    uint32_t vmask = 0x7FFFF000u;
    asm volatile("" : "+v"(vmask));
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bkey[rt][i] = bkey2[rt][i] = 0u;

    constexpr int SEGS = D / 8;                  // 16-byte segments per atom row
    constexpr int LOADS = (ECH * SEGS) / EB;     // 16-byte loads per thread per chunk
    u32x4 pre[LOADS];
    auto load_chunk = [&](int c) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int e = tid + i * EB;
        const int at = e / SEGS, sg = e % SEGS;
        pre[i] = *(const u32x4*)(a.dh + ((int64_t)c * ECH + at) * D + sg * 8);
      }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int e = tid + i * EB;
        const int at = e / SEGS, sg = e % SEGS;
        *(u32x4*)(&s_b[buf][at * BP + sg * 8]) = pre[i];
      }
    };
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      const int buf = c & 1;
      if (c + 1 < nchunks) load_chunk(c + 1);
      // four tiles at a time: 16 independent accumulation chains, then per
      // output two 3-way maxima for the best and, for the second best, the
      // medians of (best, k0, k1) and (best', k2, k3) folded by one 3-way max
      // (9 VALU ops per four products)
      static_assert(ECH % 64 == 0, "chunks hold whole groups of four tiles");
#pragma unroll
      for (int tt = 0; tt < ECH / 16; tt += 4) {
        f32x4 acc[4][4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          u32x4 bfr[KS];
#pragma unroll
          for (int s = 0; s < KS; ++s)
            bfr[s] = *(const u32x4*)(&s_b[buf][((tt + h) * 16 + (l & 15)) * BP + 32 * s + 8 * (l >> 4)]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[h][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[h][rt] = mfma_f16(af[rt][s], bfr[s], acc[h][rt]);
        }
        const uint32_t tc0 = (~(uint32_t)(c * (ECH / 16) + tt) & 0xFFFu) | 0x80000000u;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k0 = (__float_as_uint(acc[0][rt][i]) & vmask) | tc0;
            const uint32_t k1 = (__float_as_uint(acc[1][rt][i]) & vmask) | (tc0 - 1u);
            const uint32_t k2 = (__float_as_uint(acc[2][rt][i]) & vmask) | (tc0 - 2u);
            const uint32_t k3 = (__float_as_uint(acc[3][rt][i]) & vmask) | (tc0 - 3u);
            const uint32_t b0 = bkey[rt][i];
            const uint32_t b1 = max(b0, max(k0, k1));
            // second largest of {b0, b2, k0..k3} (b0 >= b2): the largest of
            // b2, the median of (b0, k0, k1) and the median of (b1, k2, k3)
            bkey2[rt][i] = max(bkey2[rt][i], max(med3_u32_op(b0, k0, k1), med3_u32_op(b1, k2, k3)));
            bkey[rt][i] = max(b1, max(k2, k3));
          }
      }
      if (c + 1 < nchunks) store_chunk(buf ^ 1);
      __syncthreads();
    }

    // --- column winners -> LDS ----------------------------------------------
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = w * 64 + rt * 16 + 4 * (l >> 4) + i;
        s_k1[rl * 16 + (l & 15)] = bkey[rt][i];
        s_k2[rl * 16 + (l & 15)] = bkey2[rt][i];
      }
    __syncthreads();

    // --- exact pick + residual update: one thread per vector ----------------------
    // Error bound E (scaled units) of a kept key against the exact value:
    // fp16 rounding of r*sc (<= 2^-11 |r sc| |d|), of fp32 atoms (<= 2^-11
    // |r sc| |d|), truncation to 11 mantissa bits (<= 2^-11 |c|) and fp32
    // sums (~2^-17 |r sc| |d|): E = 2^-9 |r sc| dmax (bf16 atoms, twice the
    // bound) or 2^-8 |r sc| dmax (fp32 atoms, 2.6x), dmax >= 1 the largest
    // atom norm.
    {
      const int rl = tid;
      const int64_t rowg = row0 + rl;
      const bool live = rowg < a.n;
      float* rr = a.r + min(rowg, a.n - 1) * D;
      const float sc = s_scale[rl];
      const float E = ldexpf(s_snorm[rl] * fmaxf(s_dmax, 1.f), a.dict_f32 ? -8 : -9);
      float bc = 0.f, babs = -1.f;
      int ba = 0x7FFFFFFF;
      uint32_t fb = 0;  // columns to rescan: bit c
      if (live && s_snorm[rl] > 0.f) {
        float vmax = 0.f;
        for (int c = 0; c < 16; ++c) vmax = fmaxf(vmax, __uint_as_float(s_k1[rl * 16 + c] & 0x7FFFF000u));
        const float cut = vmax - 2.f * E;
        for (int c = 0; c < 16; ++c)
          for (int q = 0; q < 2; ++q) {
            const uint32_t k = q ? s_k2[rl * 16 + c] : s_k1[rl * 16 + c];
            const int atom = (int)((~k) & 0xFFFu) * 16 + c;
            if (k == 0u || atom >= a.N || __uint_as_float(k & 0x7FFFF000u) < cut) continue;
            const float cx = exact_corr<D>(a, rr, atom);
            const float ax = fabsf(cx);
            if (ax > babs || (ax == babs && atom < ba)) { babs = ax; bc = cx; ba = atom; }
          }
        // a column whose second key could be within E of the winner may hide
        // further candidates below it
        const float lim = babs * sc;
        for (int c = 0; c < 16; ++c) {
          const uint32_t k = s_k2[rl * 16 + c];
          if (k != 0u && __uint_as_float(k & 0x7FFFF000u) + E >= lim) fb |= 1u << c;
        }
      }
      // wave-cooperative rescans: every atom of the column, exact fp32
      for (uint64_t pend = __ballot(fb != 0u); pend; pend = __ballot(fb != 0u)) {
        const int ln = __builtin_ctzll(pend);
        const uint32_t fbl = (uint32_t)__builtin_amdgcn_readlane((int)fb, ln);
        const int c = __builtin_ctz(fbl);
        const float* rv = a.r + (row0 + w * 64 + ln) * D;
        uint64_t best = 0;
        for (int atom = c + 16 * l; atom < a.N; atom += 16 * 64) {
          const float ax = fabsf(exact_corr<D>(a, rv, atom));
          const uint64_t key = ((uint64_t)__float_as_uint(ax) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)atom);
          best = best > key ? best : key;
        }
        best = wave_max_u64(best);
        if (l == ln) {
          const float ax = __uint_as_float((uint32_t)(best >> 32));
          const int atom = (int)(0xFFFFFFFFu - (uint32_t)best);
          if (ax > babs || (ax == babs && atom < ba)) { babs = ax; ba = atom; bc = exact_corr<D>(a, rr, atom); }
          fb &= ~(1u << c);
        }
      }
      if (live) {
        // a zero residual: every correlation is 0, atom 0 wins the tie
        if (ba == 0x7FFFFFFF) { ba = 0; bc = exact_corr<D>(a, rr, 0); }
        // update with vector loads and stores, in element order
        float nrm = 0.f;
        if (a.dict_f32) {
          const float4* dp = (const float4*)((const float*)a.dict + (int64_t)ba * D);
#pragma unroll 4
          for (int k = 0; k < D / 4; ++k) {
            const float4 dv = dp[k];
            float4 v = ((const float4*)rr)[k];
            v.x = fmaf(-bc, dv.x, v.x); nrm = fmaf(v.x, v.x, nrm);
            v.y = fmaf(-bc, dv.y, v.y); nrm = fmaf(v.y, v.y, nrm);
            v.z = fmaf(-bc, dv.z, v.z); nrm = fmaf(v.z, v.z, nrm);
            v.w = fmaf(-bc, dv.w, v.w); nrm = fmaf(v.w, v.w, nrm);
            ((float4*)rr)[k] = v;
          }
        } else {
          const u32x4* dp = (const u32x4*)((const uint16_t*)a.dict + (int64_t)ba * D);
#pragma unroll 4
          for (int k = 0; k < D / 8; ++k) {
            const u32x4 dv = dp[k];
            float4 v0 = ((const float4*)rr)[2 * k], v1 = ((const float4*)rr)[2 * k + 1];
            v0.x = fmaf(-bc, bf16_lo(dv[0]), v0.x); nrm = fmaf(v0.x, v0.x, nrm);
            v0.y = fmaf(-bc, bf16_hi(dv[0]), v0.y); nrm = fmaf(v0.y, v0.y, nrm);
            v0.z = fmaf(-bc, bf16_lo(dv[1]), v0.z); nrm = fmaf(v0.z, v0.z, nrm);
            v0.w = fmaf(-bc, bf16_hi(dv[1]), v0.w); nrm = fmaf(v0.w, v0.w, nrm);
            v1.x = fmaf(-bc, bf16_lo(dv[2]), v1.x); nrm = fmaf(v1.x, v1.x, nrm);
            v1.y = fmaf(-bc, bf16_hi(dv[2]), v1.y); nrm = fmaf(v1.y, v1.y, nrm);
            v1.z = fmaf(-bc, bf16_lo(dv[3]), v1.z); nrm = fmaf(v1.z, v1.z, nrm);
            v1.w = fmaf(-bc, bf16_hi(dv[3]), v1.w); nrm = fmaf(v1.w, v1.w, nrm);
            ((float4*)rr)[2 * k] = v0;
            ((float4*)rr)[2 * k + 1] = v1;
          }
        }
        s_rnorm[rl] = sqrtf(nrm);
        a.codes[rowg * a.codes_ld + step] = (uint32_t)ba | (f32_to_f16_bits(bc) << 16);
        if (a.coef_f32) a.coef_f32[rowg * a.K + step] = bc;
      }
    }
    __syncthreads();
  }

  // --- final outputs ------------------------------------------------------------
  const int64_t rowg = row0 + tid;
  if (rowg < a.n) {
    if (a.resid_norm) a.resid_norm[rowg] = s_rnorm[tid];
    if (a.low_plane)
      for (int j = 0; j < a.klow; ++j) a.low_plane[rowg * a.low_ld + j] = a.codes[rowg * a.codes_ld + j];
  }
}

// ---------------------------------------------------------------------------
// Few vectors (n <= kSmallN, e.g. one decode step's new tokens): the same
// pursuit with the atoms spread over the device, one launch per step.
// Launch `step` (0 .. K) of k_small, for the problem blockIdx.y (a key and a
// value encode can share the launches):
//   * loads, all at once: its atom rows, r_{step-1} (x at step 0) and the
//     per-workgroup winners of step - 1;
//   * every workgroup reduces the same winners, so all agree on (g, a), and
//     forms r_step = r_{step-1} - g d_a; workgroup 0 stores r_step and the
//     code word of step - 1;
//   * step < K: correlates r_step with its ECHS atoms and stores its
//     per-vector winner;
//   * step == K: workgroup 0 writes the residual norms and the low plane.
// Residuals and winners alternate between two buffers by step parity. A
// winner is one 64-bit key, so every reduction is a plain maximum: |c| (fp32
// bits) above 0xFFFF - atom above the sign of c -- the larger |c| wins, then
// the lower atom, and c is recovered exactly.
// Each launch fetches its code anew, so the kernels keep their unrolled code
// small: NV (16 or kSmallN) bounds the vectors and PPL the winners per lane
// (G <= 64 * PPL) that a kernel is built for.
// ---------------------------------------------------------------------------
constexpr int kSmallN = 64;        // vectors per call on this path
constexpr int ECHS = 128;          // atoms per workgroup
constexpr int ESB = 256;           // threads per workgroup
constexpr int kSmallMaxG = 512;    // workgroups at 65,536 atoms
constexpr int kMaxK = 32;          // code length limit

struct SmallArgs {                 // one encode problem
  const void* x;
  const void* dict;
  float* r;                        // [2][n][D]
  uint64_t* part;                  // [2][n][G] winner keys
  uint32_t* codes;
  int64_t codes_ld;
  float* coef_f32;
  float* resid_norm;
  uint32_t* low_plane;
  int64_t low_ld;
  int x_f32;
  int klow;
  // OMP (comparison encoder) state, written by workgroup 0:
  float* Q;                        // [n][K][D] orthonormal directions of the support
  float* Rm;                       // [n][K][K] R of the support (R[i][k], i <= k)
  float* zq;                       // [n][K] coordinates <x, q_k>
  int* sup;                        // [n][K] support atoms in selection order
};

struct SmallLaunch {               // up to two problems of one shape
  SmallArgs p[2];
  int n, N, K, G;
};

__device__ __forceinline__ uint64_t win_key(float c, int atom) {
  const uint32_t u = __float_as_uint(c);
  return ((uint64_t)(u & 0x7FFFFFFFu) << 32) | ((uint32_t)(0xFFFF - atom) << 16) | (u >> 31);
}
__device__ __forceinline__ float key_coef(uint64_t k) {
  return __uint_as_float((uint32_t)(k >> 32) | ((uint32_t)k << 31));
}
__device__ __forceinline__ int key_atom(uint64_t k) { return 0xFFFF - (int)(((uint32_t)k >> 16) & 0xFFFFu); }
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ void split3_bf16x4(float4 v, uint2& hi, uint2& mid, uint2& lo) {
  const float a[8] = {v.x, v.y, v.z, v.w, 0.f, 0.f, 0.f, 0.f};
  u32x4 h, m, o;
  split3_bf16(a, h, m, o);
  hi = make_uint2(h[0], h[1]);
  mid = make_uint2(m[0], m[1]);
  lo = make_uint2(o[0], o[1]);
}

// Sum over the D/4 consecutive lanes that hold one vector (xor butterfly:
// every lane gets the same bits).
template <int D>
__device__ __forceinline__ float vec_sum(float x) {
#pragma unroll
  for (int o = D / 8; o > 0; o >>= 1) x += __shfl_xor(x, o, D / 4);
  return x;
}

// OMP, the last launch (step K + 1, one workgroup per vector): the
// coefficients of vector v from R g = z by back substitution, one lane per
// support slot, then the code words, fp32 coefficients and low plane.
template <int D>
__device__ __forceinline__ void omp_finish_one(const SmallArgs& a, const SmallLaunch& L, int v,
                                               int l, int K) {
  float rrow[kMaxK];
  const float* Rv = a.Rm + (int64_t)v * K * K;
  const int j = min(l, K - 1);
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) rrow[k] = (k < K) ? Rv[(int64_t)j * K + k] : 0.f;
  const float z = a.zq[(int64_t)v * K + j];
  float acc = 0.f, g = 0.f;
#pragma unroll
  for (int k = kMaxK - 1; k >= 0; --k) {
    if (k < K) {
      if (l == k) g = (z - acc) / rrow[k];
      const float gk = __shfl(g, k, 64);
      if (l < k) acc = fmaf(rrow[k], gk, acc);
    }
  }
  if (l < K) {
    const uint32_t word = (uint32_t)a.sup[(int64_t)v * K + l] | (f32_to_f16_bits(g) << 16);
    a.codes[(int64_t)v * a.codes_ld + l] = word;
    if (a.coef_f32) a.coef_f32[(int64_t)v * K + l] = g;
    if (a.low_plane && l < a.klow) a.low_plane[(int64_t)v * a.low_ld + l] = word;
  }
}


template <int D, bool F32D, int NV, int PPL, bool OMP>
__global__ __launch_bounds__(ESB) void k_small(SmallLaunch L, int step) {
  static_assert(ECHS * 2 == ESB && ECHS == 32 * (ESB / 64), "atom tiles per wave");
  static_assert(NV <= kSmallN && NV % 16 == 0 && 64 * PPL <= kSmallMaxG, "launch limits");
  constexpr int NW = ESB / 64;
  constexpr int RP = D + 4;                       // LDS row pitch of the residuals
  constexpr int NQ = NV * D / (4 * ESB);          // residual float4 groups per thread, at most
  constexpr int KS = D / 32;                      // MFMA k-steps over a row
  constexpr int RPB = D + 8;                      // pitch of the bf16 parts (elements)
  // fp32 dictionary: r_step in fp32; bf16 dictionary: its three bf16 parts
  __shared__ __attribute__((aligned(16))) float s_r[F32D ? NV * RP : 4];
  __shared__ __attribute__((aligned(16))) uint16_t s_p[F32D ? 8 : 3 * NV * RPB];
  __shared__ float s_c[F32D ? NV * ECHS : 1];
  __shared__ uint64_t s_key[NW * NV];
  __shared__ float s_g[NV];
  __shared__ int s_a[NV];
  const SmallArgs a = blockIdx.y ? L.p[1] : L.p[0];
  if constexpr (OMP) {
    if (step == L.K + 1) {
      if (blockIdx.x < L.n && threadIdx.x < 64) omp_finish_one<D>(a, L, blockIdx.x, lane_id(), L.K);
      return;
    }
  }
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int n = L.n, G = L.G, wg = blockIdx.x, nq = n * D / 4;
  const bool corr = step < L.K;

  // --- independent loads first: atom rows, residual, winners ----------------
  // bf16 dictionary: wave w owns atoms wg*ECHS + 32w .. +31 as two 16-atom
  // MFMA B tiles (lane: atom l & 15, eight k values from 8 * (l >> 4)).
  // fp32 dictionary: thread (atom tid % ECHS, half tid / ECHS) holds its row.
  // Indices past the end are clamped; what they load is never used.
  u32x4 bt[2][KS];
  float4 frow[F32D ? D / 4 : 1];
  if (corr) {
    if constexpr (!F32D) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int at = min(wg * ECHS + 32 * w + 16 * t + (l & 15), L.N - 1);
#pragma unroll
        for (int k = 0; k < KS; ++k)
          bt[t][k] = *(const u32x4*)((const uint16_t*)a.dict + (int64_t)at * D + 32 * k + 8 * (l >> 4));
      }
    } else {
      const int at = min(wg * ECHS + tid % ECHS, L.N - 1);
      const float4* dp = (const float4*)((const float*)a.dict + (int64_t)at * D);
#pragma unroll
      for (int q = 0; q < D / 4; ++q) frow[q] = dp[q];
    }
  }
  // residual: thread owns float4 groups tid + j * ESB (elements 4g .. 4g+3)
  float4 rr[NQ];
  if (step == 0) {
    if (a.x_f32) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) rr[j] = ((const float4*)a.x)[min(tid + j * ESB, nq - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const uint2 u = ((const uint2*)a.x)[min(tid + j * ESB, nq - 1)];
        rr[j] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
      }
    }
  } else {
    const float4* rp = (const float4*)(a.r + (int64_t)((step - 1) & 1) * n * D);
#pragma unroll
    for (int j = 0; j < NQ; ++j) rr[j] = rp[min(tid + j * ESB, nq - 1)];
    // winners of step - 1: a row of 16 lanes per vector, each lane the
    // maximum over every 16th workgroup, then over the row
    const uint64_t* pp = a.part + (int64_t)((step - 1) & 1) * n * G;
    for (int vb = 0; vb < n; vb += ESB / 16) {
      const int v = vb + (tid >> 4);
      const uint64_t* pv = pp + (int64_t)min(v, n - 1) * G;
      uint64_t e[4 * PPL];
#pragma unroll
      for (int t = 0; t < 4 * PPL; ++t) e[t] = pv[min((tid & 15) + 16 * t, G - 1)];
      uint64_t k = e[0];
#pragma unroll
      for (int t = 1; t < 4 * PPL; ++t) k = max_u64(k, e[t]);
      k = row_max_u64(k);
      if ((tid & 15) == 0 && v < n) { s_g[v] = key_coef(k); s_a[v] = key_atom(k); }
    }
  }
  __syncthreads();

  // --- OMP: the new atom joins the support. Its direction is orthogonalised
  // against the previous ones (modified Gram-Schmidt, coefficients R[i][k]),
  // normalised (R[k][k]; a direction in the support's span, possible only
  // when the residual is numerically zero, is dropped with R[k][k] = 1), and
  // r_step = r_{step-1} - z q_k with z = <r_{step-1}, q_k> = <x, q_k>: the
  // residual of the least-squares fit on the support. The coefficients come
  // from R g = z at the end. A vector's D/4 float4 groups sit in D/4
  // consecutive lanes.
  if constexpr (OMP) {
    if (step > 0) {
      const int k = step - 1;
      float4 q[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int i = 4 * min(tid + j * ESB, nq - 1);
        const uint2 u = *(const uint2*)((const uint16_t*)a.dict + (int64_t)s_a[i / D] * D + i % D);
        q[j] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
      }
      // previous directions QB at a time: their loads are issued together
      constexpr int QB = NQ <= 2 ? 4 : 1;
      for (int i0 = 0; i0 < k; i0 += QB) {
        float4 qi[QB][NQ];
#pragma unroll
        for (int u = 0; u < QB; ++u)
#pragma unroll
          for (int j = 0; j < NQ; ++j) {
            const int e = 4 * min(tid + j * ESB, nq - 1);
            qi[u][j] = *(const float4*)(a.Q + ((int64_t)(e / D) * L.K + min(i0 + u, k - 1)) * D + e % D);
          }
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          if (i0 + u < k) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
              float dot = q[j].x * qi[u][j].x;
              dot = fmaf(q[j].y, qi[u][j].y, dot); dot = fmaf(q[j].z, qi[u][j].z, dot);
              dot = fmaf(q[j].w, qi[u][j].w, dot);
              dot = vec_sum<D>(dot);
              q[j].x = fmaf(-dot, qi[u][j].x, q[j].x); q[j].y = fmaf(-dot, qi[u][j].y, q[j].y);
              q[j].z = fmaf(-dot, qi[u][j].z, q[j].z); q[j].w = fmaf(-dot, qi[u][j].w, q[j].w);
              const int gq = tid + j * ESB;
              if (wg == 0 && gq < nq && (4 * gq) % D == 0)
                a.Rm[((int64_t)(4 * gq / D) * L.K + i0 + u) * L.K + k] = dot;
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        float nn = q[j].x * q[j].x;
        nn = fmaf(q[j].y, q[j].y, nn); nn = fmaf(q[j].z, q[j].z, nn); nn = fmaf(q[j].w, q[j].w, nn);
        nn = vec_sum<D>(nn);
        const float rkk = sqrtf(nn);
        const bool ok = rkk > 1e-20f;
        const float inv = ok ? 1.f / rkk : 0.f;
        q[j].x *= inv; q[j].y *= inv; q[j].z *= inv; q[j].w *= inv;
        float z = rr[j].x * q[j].x;
        z = fmaf(rr[j].y, q[j].y, z); z = fmaf(rr[j].z, q[j].z, z); z = fmaf(rr[j].w, q[j].w, z);
        z = vec_sum<D>(z);
        rr[j].x = fmaf(-z, q[j].x, rr[j].x); rr[j].y = fmaf(-z, q[j].y, rr[j].y);
        rr[j].z = fmaf(-z, q[j].z, rr[j].z); rr[j].w = fmaf(-z, q[j].w, rr[j].w);
        const int gq = tid + j * ESB;
        if (wg == 0 && gq < nq) {
          const int v = 4 * gq / D, e = (4 * gq) % D;
          *(float4*)(a.Q + ((int64_t)v * L.K + k) * D + e) = q[j];
          if (e == 0) {
            a.Rm[((int64_t)v * L.K + k) * L.K + k] = ok ? rkk : 1.f;
            a.zq[(int64_t)v * L.K + k] = z;
            a.sup[(int64_t)v * L.K + k] = s_a[v];
          }
        }
      }
    }
  }

  // --- r_step = r_{step-1} - g d_a, one fmaf per element ---------------------
  if (!OMP && step > 0) {
    float4 dk[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int i = 4 * min(tid + j * ESB, nq - 1);
      const int64_t e = (int64_t)s_a[i / D] * D + i % D;
      if constexpr (F32D) {
        dk[j] = *(const float4*)((const float*)a.dict + e);
      } else {
        const uint2 u = *(const uint2*)((const uint16_t*)a.dict + e);
        dk[j] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
      }
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int i = 4 * min(tid + j * ESB, nq - 1);
      const float g = s_g[i / D];
      rr[j].x = fmaf(-g, dk[j].x, rr[j].x); rr[j].y = fmaf(-g, dk[j].y, rr[j].y);
      rr[j].z = fmaf(-g, dk[j].z, rr[j].z); rr[j].w = fmaf(-g, dk[j].w, rr[j].w);
    }
    if (wg == 0 && tid < n) {
      a.codes[(int64_t)tid * a.codes_ld + step - 1] = (uint32_t)s_a[tid] | (f32_to_f16_bits(s_g[tid]) << 16);
      if (a.coef_f32) a.coef_f32[(int64_t)tid * L.K + step - 1] = s_g[tid];
    }
  }
  float4* rq = (float4*)(a.r + (int64_t)(step & 1) * n * D);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int gq = tid + j * ESB;
    if (gq < nq) {
      const int v = 4 * gq / D, kk = (4 * gq) % D;
      if constexpr (F32D) {
        *(float4*)&s_r[v * RP + kk] = rr[j];
      } else {
        uint2 hi, mid, lo;
        split3_bf16x4(rr[j], hi, mid, lo);
        *(uint2*)&s_p[v * RPB + kk] = hi;
        *(uint2*)&s_p[(NV + v) * RPB + kk] = mid;
        *(uint2*)&s_p[(2 * NV + v) * RPB + kk] = lo;
      }
      if (wg == 0 && corr) rq[gq] = rr[j];
    }
  }
  __syncthreads();

  if (corr) {
    uint64_t* pq = a.part + (int64_t)(step & 1) * n * G;
    if constexpr (!F32D) {
      // --- correlations on the matrix cores: C[atom][vector] over 16-vector
      // tiles, r split exactly into three bf16 parts (every product exact,
      // fp32 accumulation); per wave the best of its 32 atoms per vector.
      // The matrix cores do not round a sum and its negation to the same
      // magnitude, so each atom is also run negated and its magnitude is
      // the larger of the two: an atom and its negated copy then get equal
      // magnitudes (exact ties, lowest index first), as do duplicates. The
      // coefficient keeps the sign of the atom's own correlation. --------
      for (int v0 = 0; v0 < n; v0 += 16) {
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 accn[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int vr = min(v0 + (l & 15), n - 1);  // columns past n are never stored
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const int off = vr * RPB + 32 * k + 8 * (l >> 4);
          const u32x4 hi = *(const u32x4*)&s_p[off];
          const u32x4 mid = *(const u32x4*)&s_p[NV * RPB + off];
          const u32x4 lo = *(const u32x4*)&s_p[2 * NV * RPB + off];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 ng = bt[t][k] ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            acc[t] = mfma_bf16(bt[t][k], hi, acc[t]);
            accn[t] = mfma_bf16(ng, hi, accn[t]);
            acc[t] = mfma_bf16(bt[t][k], mid, acc[t]);
            accn[t] = mfma_bf16(ng, mid, accn[t]);
            acc[t] = mfma_bf16(bt[t][k], lo, acc[t]);
            accn[t] = mfma_bf16(ng, lo, accn[t]);
          }
        }
        // lane holds vector v0 + (l & 15) against atoms 16t + 4 * (l >> 4) + i;
        // the four lanes of a vector (l ^ 16, l ^ 32) then combine
        uint64_t k = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int at = wg * ECHS + 32 * w + 16 * t + 4 * (l >> 4) + i;
            const float mag = fmaxf(fabsf(acc[t][i]), fabsf(accn[t][i]));
            const float c = __builtin_copysignf(mag, acc[t][i]);
            if (at < L.N) k = max_u64(k, win_key(c, at));
          }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, o, 64);
          const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), o, 64);
          k = max_u64(k, ((uint64_t)hi << 32) | lo);
        }
        const int v = v0 + l;
        if (l < 16 && v < n) s_key[w * NV + v] = k;
      }
      __syncthreads();
      // the workgroup's winner per vector: the best of the waves' winners
      if (tid < n) {
        uint64_t k = s_key[tid];
#pragma unroll
        for (int q = 1; q < NW; ++q) k = max_u64(k, s_key[q * NV + tid]);
        pq[(int64_t)tid * G + wg] = k;
      }
    } else {
      // --- correlations on the vector ALUs (fp32 dictionary): thread (atom,
      // half) takes the vectors of its half, each a sequential fp32 dot
      // product over k ---------------------------------------------------------
      const int al = tid % ECHS, half = tid / ECHS;
      const int nh = (n + 1) / 2;  // vectors [half * nh, min(n, half * nh + nh))
      const int v0 = half * nh, v1 = min(n, v0 + nh);
#pragma unroll
      for (int j = 0; j < NV / 2; ++j) {
        if (v0 + j < v1) {
          float sacc = 0.f;
#pragma unroll
          for (int q = 0; q < D / 4; ++q) {
            const float4 r4 = *(const float4*)&s_r[(v0 + j) * RP + 4 * q];
            sacc = fmaf(r4.x, frow[q].x, sacc); sacc = fmaf(r4.y, frow[q].y, sacc);
            sacc = fmaf(r4.z, frow[q].z, sacc); sacc = fmaf(r4.w, frow[q].w, sacc);
          }
          s_c[(v0 + j) * ECHS + al] = sacc;
        }
      }
      __syncthreads();
      // per vector: the best of this workgroup's atoms (wave w: vectors w, w+NW, ...)
      for (int v = w; v < n; v += NW) {
        uint64_t k = 0;
#pragma unroll
        for (int t = 0; t < ECHS / 64; ++t) {
          const int q = l + 64 * t, at = wg * ECHS + q;
          if (at < L.N) k = max_u64(k, win_key(s_c[v * ECHS + q], at));
        }
        k = wave_max_u64(k);
        if (l == 0) pq[(int64_t)v * G + wg] = k;
      }
    }
  } else if (wg == 0) {
    // --- final outputs -----------------------------------------------------------
    // |r_K|: a vector's D/4 groups sit in D/4 consecutive lanes of one pass
    if (a.resid_norm) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        float s2 = rr[j].x * rr[j].x;
        s2 = fmaf(rr[j].y, rr[j].y, s2); s2 = fmaf(rr[j].z, rr[j].z, s2); s2 = fmaf(rr[j].w, rr[j].w, s2);
#pragma unroll
        for (int o = D / 8; o > 0; o >>= 1) s2 += __shfl_xor(s2, o, 64);
        const int gq = tid + j * ESB;
        if (gq < nq && gq % (D / 4) == 0) a.resid_norm[4 * gq / D] = sqrtf(s2);
      }
    }
    // words of steps before K - 1 come from earlier launches; the last one
    // from this workgroup's own reduction (OMP: written by the last launch)
    if (!OMP && a.low_plane)
      for (int i = tid; i < n * a.klow; i += ESB) {
        const int v = i / a.klow, j = i % a.klow;
        a.low_plane[(int64_t)v * a.low_ld + j] =
            j == L.K - 1 ? (uint32_t)s_a[v] | (f32_to_f16_bits(s_g[v]) << 16)
                         : a.codes[(int64_t)v * a.codes_ld + j];
      }
  }
}

sdkv_status plan_encode(const sdkv_encode_args* a, EncodePlan* p) {
  EncodePlan q;
  q.n = a->n;
  if (a->n <= kSmallN) {
    q.small = 1;
    q.G = (a->n_atoms + ECHS - 1) / ECHS;
    size_t off = 0;
    q.off_r = off;     off = align_up(off + (size_t)2 * a->n * a->d * 4, 256);
    q.off_part = off;  off = align_up(off + (size_t)2 * q.G * a->n * 8, 256);
    if (a->algorithm == SDKV_ENCODE_OMP) {
      const size_t nK = (size_t)a->n * a->K;
      q.off_omp = off;  off = align_up(off + nK * a->d * 4 + nK * a->K * 4 + nK * 4 + nK * 4, 256);
    }
    q.total = off;
    *p = q;
    return SDKV_OK;
  }
  q.npad = (a->n_atoms + ECH - 1) / ECH * ECH;
  q.rows_per_wg = EROWS;
  q.nwg = (a->n + EROWS - 1) / EROWS;
  size_t off = 0;
  q.off_dh = off;  off = align_up(off + (size_t)q.npad * a->d * 2, 256);
  q.off_dn = off;  off = align_up(off + (size_t)kPrepBlocks * 4, 256);
  q.off_r = off;   off = align_up(off + (size_t)a->n * a->d * 4, 256);
  q.total = off;
  *p = q;
  return SDKV_OK;
}

static SmallArgs small_args(const sdkv_encode_args* a, const EncodePlan& p, char* base) {
  SmallArgs s;
  s.x = a->x;
  s.dict = a->dict;
  s.r = (float*)(base + p.off_r);
  s.part = (uint64_t*)(base + p.off_part);
  s.codes = a->codes;
  s.codes_ld = a->codes_ld ? a->codes_ld : a->K;
  s.coef_f32 = a->coef_f32;
  s.resid_norm = a->resid_norm;
  s.low_plane = a->low_plane;
  s.low_ld = a->low_ld ? a->low_ld : a->klow;
  s.x_f32 = a->x_dtype == SDKV_F32;
  s.klow = a->low_plane ? a->klow : 0;
  const size_t nK = (size_t)a->n * a->K;
  s.Q = (float*)(base + p.off_omp);
  s.Rm = s.Q + nK * a->d;
  s.zq = s.Rm + nK * a->K;
  s.sup = (int*)(s.zq + nK);
  return s;
}

template <int D, bool F32D, bool OMP = false>
static void launch_small_kernel(bool few, bool narrow, dim3 grid, hipStream_t stream,
                                const SmallLaunch& L, int step) {
  if (few && narrow)  hipLaunchKernelGGL((k_small<D, F32D, 16, 4, OMP>), grid, dim3(ESB), 0, stream, L, step);
  else if (few)       hipLaunchKernelGGL((k_small<D, F32D, 16, 8, OMP>), grid, dim3(ESB), 0, stream, L, step);
  else if (narrow)    hipLaunchKernelGGL((k_small<D, F32D, kSmallN, 4, OMP>), grid, dim3(ESB), 0, stream, L, step);
  else                hipLaunchKernelGGL((k_small<D, F32D, kSmallN, 8, OMP>), grid, dim3(ESB), 0, stream, L, step);
}

// The K + 1 launches of the small path for `count` (1 or 2) problems of one
// shape (n, d, n_atoms, K and dictionary dtype equal).
static sdkv_status launch_small(const sdkv_encode_args* const* a, const EncodePlan* const* p,
                                char* const* base, int count, hipStream_t stream) {
  SmallLaunch L;
  for (int i = 0; i < 2; ++i) L.p[i] = small_args(a[i < count ? i : 0], *p[i < count ? i : 0], base[i < count ? i : 0]);
  L.n = (int)a[0]->n;
  L.N = a[0]->n_atoms;
  L.K = a[0]->K;
  L.G = p[0]->G;
  const bool f32d = a[0]->dict_dtype == SDKV_F32;
  const dim3 grid((unsigned)L.G, (unsigned)count);
  const bool few = L.n <= 16, narrow = L.G <= 256;
  if (a[0]->algorithm == SDKV_ENCODE_OMP) {
    // (bf16 dictionaries only, checked by the caller) K + 2 launches
    for (int step = 0; step <= L.K + 1; ++step) {
      // the last launch finishes one vector per workgroup
      const dim3 g = step <= L.K ? grid : dim3((unsigned)L.n, (unsigned)count);
      if (a[0]->d == 128) launch_small_kernel<128, false, true>(few, narrow, g, stream, L, step);
      else                launch_small_kernel<64, false, true>(few, narrow, g, stream, L, step);
      if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
    }
    return SDKV_OK;
  }
  for (int step = 0; step <= L.K; ++step) {
    if (a[0]->d == 128) {
      if (f32d) launch_small_kernel<128, true>(few, narrow, grid, stream, L, step);
      else      launch_small_kernel<128, false>(few, narrow, grid, stream, L, step);
    } else {
      if (f32d) launch_small_kernel<64, true>(few, narrow, grid, stream, L, step);
      else      launch_small_kernel<64, false>(few, narrow, grid, stream, L, step);
    }
    if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  }
  return SDKV_OK;
}

sdkv_status launch_encode_pair(const sdkv_encode_args* a0, const EncodePlan& p0, char* ws0,
                               const sdkv_encode_args* a1, const EncodePlan& p1, char* ws1,
                               hipStream_t stream) {
  const sdkv_encode_args* a[2] = {a0, a1};
  const EncodePlan* p[2] = {&p0, &p1};
  char* base[2] = {ws0, ws1};
  return launch_small(a, p, base, 2, stream);
}

sdkv_status launch_encode(const sdkv_encode_args* a, const EncodePlan& p, void* ws,
                          hipStream_t stream) {
  char* base = (char*)ws;
  const int64_t codes_ld = a->codes_ld ? a->codes_ld : a->K;
  const int64_t low_ld = a->low_ld ? a->low_ld : a->klow;
  if (p.small) {
    void* const* ev = a->stage_events;
    if (!record_stage(ev, 0, stream) || !record_stage(ev, 1, stream)) return SDKV_ERR_DEVICE;
    const sdkv_encode_args* aa[1] = {a};
    const EncodePlan* pp[1] = {&p};
    char* bb[1] = {base};
    const sdkv_status st = launch_small(aa, pp, bb, 1, stream);
    if (st != SDKV_OK) return st;
    if (!record_stage(ev, 2, stream)) return SDKV_ERR_DEVICE;
    return SDKV_OK;
  }
  uint16_t* dh = (uint16_t*)(base + p.off_dh);
  const int dict_f32 = a->dict_dtype == SDKV_F32;
  void* const* ev = a->stage_events;
  if (!record_stage(ev, 0, stream)) return SDKV_ERR_DEVICE;
  hipLaunchKernelGGL(k_prep_dict, dim3(kPrepBlocks), dim3(256), 0, stream, a->dict, dict_f32,
                     a->n_atoms, p.npad, a->d, dh, (float*)(base + p.off_dn));
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  EncArgs e;
  e.x = a->x;
  e.x_f32 = a->x_dtype == SDKV_F32;
  e.dict = a->dict;
  e.dict_f32 = dict_f32;
  e.dh = dh;
  e.dnorm = (const float*)(base + p.off_dn);
  e.r = (float*)(base + p.off_r);
  e.n = a->n;
  e.N = a->n_atoms;
  e.npad = p.npad;
  e.K = a->K;
  e.klow = a->low_plane ? a->klow : 0;
  e.codes = a->codes;
  e.codes_ld = codes_ld;
  e.coef_f32 = a->coef_f32;
  e.resid_norm = a->resid_norm;
  e.low_plane = a->low_plane;
  e.low_ld = low_ld;
  const int64_t max_grid = 0x7FFFFFFF;
  if (p.nwg > max_grid) return SDKV_ERR_UNSUPPORTED;
  if (!record_stage(ev, 1, stream)) return SDKV_ERR_DEVICE;
  if (a->d == 128)
    hipLaunchKernelGGL(k_encode<128>, dim3((unsigned)p.nwg), dim3(EB), 0, stream, e);
  else
    hipLaunchKernelGGL(k_encode<64>, dim3((unsigned)p.nwg), dim3(EB), 0, stream, e);
  if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  if (!record_stage(ev, 2, stream)) return SDKV_ERR_DEVICE;
  return SDKV_OK;
}

}  // namespace sdkv
