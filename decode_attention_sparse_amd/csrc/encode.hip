// Greedy projection pursuit encode on gfx950 ("LLM Inference in a Flash!",
// review page, Summary and Strengths: one atom is projected out per step and,
// unlike OMP, no least-squares problem is ever re-solved; K atoms per
// key/value vector over a per-layer, per-stream dictionary).
//
// Per vector x:  r = x;  for k < K: a_k = argmax_a |<r, d_a>| (lowest index on
// ties), g_k = <r, d_{a_k}>, r -= g_k d_{a_k}.
//
// Structure (one workgroup = 8 waves = 512 vectors, all K steps inside):
//   * screen: every step correlates the workgroup's residuals with all atoms
//     on the matrix cores (v_mfma_f32_16x16x32_f16). The residual rows are
//     scaled by a power of two and rounded to fp16; the dictionary is an fp16
//     copy (exact for bf16 atoms of unit-norm size). Each lane keeps, per
//     output row it owns, the largest |c| seen in its atom column and that
//     atom's tile, packed in one word: |c| with its low 12 mantissa bits
//     replaced by the complement of the tile index, so a single unsigned
//     max keeps the larger value and, among equal truncated values, the
//     lower tile. (The truncation, at most 2^-11 of |c|, is well inside the
//     recheck window below.)
//   * exact pick: per vector, the 16 column winners whose screened |c| lie
//     within a window of the best are recomputed in fp32 from the original
//     dictionary; the largest exact |c| wins, lowest atom index on ties.
//     The window (2^-7 |r|) is 4x the worst-case screen error bound.
//   * update: g = exact <r, d_a> (fp32), r -= g d_a in fp32.
#include "sdkv_device.h"
#include "sdkv_internal.h"

namespace sdkv {

constexpr int EB = 512;            // threads per workgroup
constexpr int ENW = EB / 64;       // waves
constexpr int EROWS = ENW * 64;    // vectors per workgroup (64 per wave)
constexpr int ECH = 64;            // atoms per LDS chunk
constexpr int EWIN_SHIFT = 7;      // recheck window = |r| * 2^-7

struct EncArgs {
  const void* x;
  int x_f32;
  const void* dict;
  int dict_f32;
  const uint16_t* dh;   // [npad, D] fp16 screen copy
  float* r;             // [n, D] residuals (workspace)
  int64_t n;
  int N, npad, K, klow;
  uint32_t* codes;
  float* coef_f32;
  float* resid_norm;
  uint32_t* low_plane;
};

// fp16 screen copy of the dictionary, zero rows past N.
__global__ __launch_bounds__(256) void k_prep_dict(const void* dict, int dict_f32, int N,
                                                   int npad, int D, uint16_t* dh) {
  const int64_t total = (int64_t)npad * D;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int a = (int)(i / D);
    float v = 0.f;
    if (a < N)
      v = dict_f32 ? ((const float*)dict)[i] : bf16_to_f32(((const uint16_t*)dict)[i]);
    dh[i] = (uint16_t)f32_to_f16_bits(v);
  }
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
__global__ __launch_bounds__(EB) void k_encode(EncArgs a) {
  constexpr int KS = D / 32;           // MFMA k-steps per 16x16 tile
  constexpr int BP = D + 8;            // LDS row pitch (fp16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][ECH * BP];
  __shared__ float s_wv[EROWS * 16];
  __shared__ int32_t s_wi[EROWS * 16];
  __shared__ float s_scale[EROWS];
  __shared__ float s_rnorm[EROWS];

  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t row0 = (int64_t)blockIdx.x * EROWS;

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
      if ((l >> 4) == 0) s_scale[rl] = sc;
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
    // running best per output: |c| with its low 12 mantissa bits replaced by
    // the complement of the 16-atom tile index, so one unsigned max keeps the
    // larger |c| and, among equal truncated values, the lower tile
    uint32_t bkey[4][4];
    // the mask lives in a register, so (x & mask) | code is one 3-input op
    uint32_t vmask = 0x7FFFF000u;
    asm volatile("" : "+v"(vmask));
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bkey[rt][i] = 0u;

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
      // tiles in pairs: 8 independent accumulation chains, then one 3-way
      // max per output for the two tiles
#pragma unroll
      for (int tt = 0; tt < ECH / 16; tt += 2) {
        f32x4 acc[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
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
        const uint32_t tc0 = ~(uint32_t)(c * (ECH / 16) + tt) & 0xFFFu;
        const uint32_t tc1 = tc0 - 1u;  // the next tile's code
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k0 = (__float_as_uint(acc[0][rt][i]) & vmask) | tc0;
            const uint32_t k1 = (__float_as_uint(acc[1][rt][i]) & vmask) | tc1;
            bkey[rt][i] = max(bkey[rt][i], max(k0, k1));
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
        s_wv[rl * 16 + (l & 15)] = __uint_as_float(bkey[rt][i] & 0x7FFFF000u);
        s_wi[rl * 16 + (l & 15)] = (int)((~bkey[rt][i]) & 0xFFFu) * 16 + (l & 15);
      }
    __syncthreads();

    // --- exact pick + residual update: one thread per vector ----------------------
    {
      const int rl = tid;
      const int64_t rowg = row0 + rl;
      if (rowg < a.n) {
        float* rr = a.r + rowg * D;
        float vmax = 0.f;
        for (int c = 0; c < 16; ++c) vmax = fmaxf(vmax, s_wv[rl * 16 + c]);
        const float win = ldexpf(s_rnorm[rl] * s_scale[rl], -EWIN_SHIFT);
        float bc = 0.f, babs = -1.f;
        int ba = 0x7FFFFFFF;
        for (int c = 0; c < 16; ++c) {
          const int atom = s_wi[rl * 16 + c];
          if (atom >= a.N || s_wv[rl * 16 + c] < vmax - win) continue;
          const float cx = exact_corr<D>(a, rr, atom);
          const float ax = fabsf(cx);
          if (ax > babs || (ax == babs && atom < ba)) { babs = ax; bc = cx; ba = atom; }
        }
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
        a.codes[rowg * a.K + step] = (uint32_t)ba | (f32_to_f16_bits(bc) << 16);
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
      for (int j = 0; j < a.klow; ++j) a.low_plane[rowg * a.klow + j] = a.codes[rowg * a.K + j];
  }
}

sdkv_status plan_encode(const sdkv_encode_args* a, EncodePlan* p) {
  EncodePlan q;
  q.n = a->n;
  q.npad = (a->n_atoms + ECH - 1) / ECH * ECH;
  q.rows_per_wg = EROWS;
  q.nwg = (a->n + EROWS - 1) / EROWS;
  size_t off = 0;
  q.off_dh = off;  off = align_up(off + (size_t)q.npad * a->d * 2, 256);
  q.off_r = off;   off = align_up(off + (size_t)a->n * a->d * 4, 256);
  q.total = off;
  *p = q;
  return SDKV_OK;
}

sdkv_status launch_encode(const sdkv_encode_args* a, const EncodePlan& p, void* ws,
                          hipStream_t stream) {
  char* base = (char*)ws;
  uint16_t* dh = (uint16_t*)(base + p.off_dh);
  const int dict_f32 = a->dict_dtype == SDKV_F32;
  void* const* ev = a->stage_events;
  if (!record_stage(ev, 0, stream)) return SDKV_ERR_DEVICE;
  {
    const int64_t total = (int64_t)p.npad * a->d;
    const int grid = (int)std::min<int64_t>(2048, (total + 255) / 256);
    hipLaunchKernelGGL(k_prep_dict, dim3(grid), dim3(256), 0, stream, a->dict, dict_f32,
                       a->n_atoms, p.npad, a->d, dh);
    if (hipGetLastError() != hipSuccess) return SDKV_ERR_DEVICE;
  }
  EncArgs e;
  e.x = a->x;
  e.x_f32 = a->x_dtype == SDKV_F32;
  e.dict = a->dict;
  e.dict_f32 = dict_f32;
  e.dh = dh;
  e.r = (float*)(base + p.off_r);
  e.n = a->n;
  e.N = a->n_atoms;
  e.npad = p.npad;
  e.K = a->K;
  e.klow = a->low_plane ? a->klow : 0;
  e.codes = a->codes;
  e.coef_f32 = a->coef_f32;
  e.resid_norm = a->resid_norm;
  e.low_plane = a->low_plane;
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
