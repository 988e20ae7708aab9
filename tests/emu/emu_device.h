// Host emulation of the device primitives the select core and the decode
// row kernel use, so that their own source (select_core.h, the row kernel of
// decode.hip) can run on the CPU: every GPU thread is a fiber (ucontext),
// workgroup barriers, wave exchanges and the cross-workgroup barrier are
// cooperative waits. Test infrastructure only.
//
// The harness copies select_core.h next to this file under the name the
// header includes (sdkv_device.h resolves to this file), then compiles it
// with g++.
#pragma once
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#define __device__
#define __global__
#define __launch_bounds__(...)
#define __forceinline__ inline
#define __HIP_MEMORY_SCOPE_AGENT 0
#define __builtin_nontemporal_store(v, p) (*(p) = (v))

typedef uint32_t u32x4 __attribute__((vector_size(16)));
struct float2 {
  float x, y;
};
struct float4 {
  float x, y, z, w;
};
struct int4 {
  int x, y, z, w;
};
inline float2 make_float2(float x, float y) { return float2{x, y}; }
inline float4 make_float4(float x, float y, float z, float w) { return float4{x, y, z, w}; }
inline int4 make_int4(int x, int y, int z, int w) { return int4{x, y, z, w}; }
inline float __expf(float x) { return expf(x); }
inline int __clz(uint32_t x) { return x ? __builtin_clz(x) : 32; }
inline int __clzll(unsigned long long x) { return x ? __builtin_clzll(x) : 64; }
inline void __threadfence_block() {}

namespace emu {
struct D3 {
  unsigned x, y, z;
};
D3 tid3();
D3 bid3();
void block_barrier();
void wave_barrier();
uint64_t* wave_slots();       // 64 exchange slots of the calling thread's wave
uint32_t* wg_flag();          // one word of per-workgroup scratch
void spin_yield();
}  // namespace emu

#define threadIdx (::emu::tid3())
#define blockIdx (::emu::bid3())

inline void __syncthreads() { emu::block_barrier(); }
inline uint32_t __float_as_uint(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
inline float __uint_as_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
inline int __popcll(uint64_t x) { return __builtin_popcountll(x); }
inline int __popc(uint32_t x) { return __builtin_popcount(x); }
inline uint32_t __umulhi(uint32_t a, uint32_t b) { return (uint32_t)(((uint64_t)a * b) >> 32); }
// fibers never interleave inside one call: plain read-modify-write is atomic
template <class T>
inline T atomicAdd(T* p, T v) {
  const T o = *p;
  *p = o + v;
  return o;
}
template <class T>
inline T __hip_atomic_load(const T* p, int, int) {
  return *p;
}
template <class T, class U>
inline void __hip_atomic_store(T* p, U v, int, int) {
  *p = (T)v;
}
template <class T>
inline T __hip_atomic_fetch_add(T* p, T v, int, int) {
  const T o = *p;
  *p = o + v;
  return o;
}
using std::max;
using std::min;
inline int64_t min(int64_t a, int b) { return a < b ? a : (int64_t)b; }
inline int64_t min(int a, int64_t b) { return a < b ? (int64_t)a : b; }
inline int64_t max(int64_t a, int b) { return a > b ? a : (int64_t)b; }

// wave exchange: every lane deposits a value, then reads any lane's
inline uint64_t wave_xchg_read(uint64_t mine, int lane, int src) {
  uint64_t* s = emu::wave_slots();
  s[lane] = mine;
  emu::wave_barrier();
  const uint64_t v = s[src];
  emu::wave_barrier();
  return v;
}

namespace sdkv {
inline int lane_id() { return (int)(threadIdx.x & 63u); }
inline int wave_id() { return (int)(threadIdx.x >> 6); }
}  // namespace sdkv

inline uint64_t __ballot(int pred) {
  uint64_t* s = emu::wave_slots();
  const int lane = sdkv::lane_id();
  s[lane] = pred ? 1u : 0u;
  emu::wave_barrier();
  uint64_t b = 0;
  for (int i = 0; i < 64; ++i) b |= (s[i] ? 1ull : 0ull) << i;
  emu::wave_barrier();
  return b;
}
inline int __shfl(int v, int src, int) {
  return (int)(uint32_t)wave_xchg_read((uint32_t)v, sdkv::lane_id(), src & 63);
}

namespace sdkv {

// the device header's order-preserving float keys, restated
inline uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
inline float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// IEEE binary16 <-> binary32 from the formats' definitions (the device uses
// the hardware conversions, round to nearest even)
inline float f16_bits_to_f32(uint32_t b) {
  const uint32_t s = (b >> 15) & 1u, e = (b >> 10) & 31u, f = b & 1023u;
  float v;
  if (e == 0) v = ldexpf((float)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexpf((float)(f | 1024u), (int)e - 25);
  return s ? -v : v;
}
inline uint32_t f32_to_f16_bits(float x) {
  const uint32_t s = (__float_as_uint(x) >> 31) << 15;
  const float a = fabsf(x);
  if (a != a) return s | 0x7E00u;
  if (a >= 65520.f) return s | 0x7C00u;  // rounds to infinity
  if (a < 0x1p-14f) {                     // subnormal: multiples of 2^-24
    return s | (uint32_t)nearbyintf(a * 0x1p24f);  // round half even (default mode)
  }
  int e;
  frexpf(a, &e);                          // a = m 2^e, m in [0.5, 1)
  const float q = nearbyintf(ldexpf(a, 11 - e));  // 11 significant bits
  uint32_t m = (uint32_t)q, E = (uint32_t)(e - 1 + 15);
  if (m == 2048u) { m = 1024u; ++E; }
  if (E >= 31u) return s | 0x7C00u;
  return s | (E << 10) | (m - 1024u);
}
inline uint32_t f32x2_to_f16x2_bits(float lo, float hi) {
  return f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}
inline uint32_t code_idx(uint32_t w) { return w & 0xFFFFu; }
inline float code_coef(uint32_t w) { return f16_bits_to_f32(w >> 16); }

// wave reductions and scans by exchange (lane order, as the DPP versions)
template <class Op>
inline uint32_t wave_fold(uint32_t v, Op op, bool inclusive_scan) {
  uint64_t* s = emu::wave_slots();
  const int lane = lane_id();
  s[lane] = v;
  emu::wave_barrier();
  uint32_t r = (uint32_t)s[0];
  const int hi = inclusive_scan ? lane : 63;
  for (int i = 1; i <= hi; ++i) r = op(r, (uint32_t)s[i]);
  emu::wave_barrier();
  return r;
}
inline uint32_t wave_incl_scan(uint32_t v) {
  return wave_fold(v, [](uint32_t a, uint32_t b) { return a + b; }, true);
}
inline uint32_t wave_sum_u32(uint32_t v) {
  return wave_fold(v, [](uint32_t a, uint32_t b) { return a + b; }, false);
}
inline uint32_t wave_min_u32(uint32_t v) {
  return wave_fold(v, [](uint32_t a, uint32_t b) { return min(a, b); }, false);
}
inline uint32_t wave_max_u32(uint32_t v) {
  return wave_fold(v, [](uint32_t a, uint32_t b) { return max(a, b); }, false);
}

inline float wave_max(float v) {
  uint64_t* s = emu::wave_slots();
  s[lane_id()] = __float_as_uint(v);
  emu::wave_barrier();
  float r = __uint_as_float((uint32_t)s[0]);
  for (int i = 1; i < 64; ++i) r = fmaxf(r, __uint_as_float((uint32_t)s[i]));
  emu::wave_barrier();
  return r;
}
inline float wave_sum(float v) {
  uint64_t* s = emu::wave_slots();
  s[lane_id()] = __float_as_uint(v);
  emu::wave_barrier();
  float r = __uint_as_float((uint32_t)s[0]);
  for (int i = 1; i < 64; ++i) r += __uint_as_float((uint32_t)s[i]);
  emu::wave_barrier();
  return r;
}
template <int NW>
inline float block_max(float v, float* tmp) {
  v = wave_max(v);
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  float r = tmp[0];
  for (int i = 1; i < NW; ++i) r = fmaxf(r, tmp[i]);
  __syncthreads();
  return r;
}
template <int NW>
inline float block_sum(float v, float* tmp) {
  v = wave_sum(v);
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < NW; ++i) r += tmp[i];
  __syncthreads();
  return r;
}

template <int NW>
inline uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const uint32_t inc = wave_incl_scan(v);
  if (lane_id() == 63) tmp[wave_id()] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = tmp[i];
    base += (i < wave_id()) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

template <int NW>
inline uint32_t block_excl_scan_open(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const uint32_t inc = wave_incl_scan(v);
  if (lane_id() == 63) tmp[wave_id()] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = tmp[i];
    base += (i < wave_id()) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return base + inc - v;
}

struct WaitCtl {
  uint32_t* err;
  uint32_t limit;
  uint32_t extra;
};
inline uint32_t ld_agent(const uint32_t* p) { return *p; }
inline void st_agent(uint32_t* p, uint32_t v) { *p = v; }
// workgroup start order, as the device's tickets
inline int ticket_tile(uint32_t* tickets, int nb, bool xcd) {
  if (xcd) {
    const int c = (int)(blockIdx.x & 7u);
    return c * (nb >> 3) + (int)atomicAdd(&tickets[c], 1u);
  }
  return (int)atomicAdd(&tickets[0], 1u);
}

// arrival counter and bounded wait, as the device barrier (one thread
// arrives and waits; the workgroup meets before and after)
inline bool group_barrier(uint32_t* bar, uint32_t P, uint32_t round, bool, const WaitCtl& w) {
  __syncthreads();
  if (threadIdx.x == 0) {
    bar[0] += 1u;
    const uint32_t target = P * round + w.extra;
    uint32_t spins = 0;
    bool ok = true;
    while ((bar[0] & 0xFFFFu) < target) {
      emu::spin_yield();
      if (++spins > w.limit) {
        *w.err = 1u;
        ok = false;
        break;
      }
    }
    *emu::wg_flag() = ok ? 1u : 0u;
  }
  __syncthreads();
  return *emu::wg_flag() != 0u;
}

}  // namespace sdkv
