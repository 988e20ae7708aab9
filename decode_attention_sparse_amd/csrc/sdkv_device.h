// Device-side helpers shared by the libsdkv kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdkv {

// --- MFMA operand types (v_mfma_f32_16x16x32_{bf16,f16}) -------------------
// Lane layout (wave64) of the 16x16x32 shapes, as used throughout:
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) .. 8*(l/16)+7
//   B (32 x 16): lane l holds col l%16, k = 8*(l/16) .. 8*(l/16)+7
//   C (16 x 16): lane l holds rows 4*(l/16)+i (i < 4), col l%16
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// --- number formats ---------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// two fp32 values as packed binary16 (lo, hi), each rounded to nearest even
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2c __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_f16x2_bits(float lo, float hi) {
  const f32x2c v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v));
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
// code word: index in bits 0-15, binary16 coefficient in bits 16-31
__device__ __forceinline__ uint32_t code_idx(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ float code_coef(uint32_t w) { return f16_bits_to_f32(w >> 16); }

// Order-preserving map float -> uint32 (larger float -> larger key). Finite
// scores never map to 0, which marks "no token" in the select kernels.
// Adding +0 turns -0 into +0 (so both compare equal) and leaves every other
// non-NaN value as it is; negative values are then complemented and others
// get the top bit set, in three integer ops.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// fp32 values as hi + mid + lo bf16 parts, exactly: each part is the bf16
// rounding (v_cvt_pk_bf16_f32) of what the previous ones left, and the
// remainder after two 8-bit parts fits the third.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split3_bf16(const float (&v)[8], u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2v x = {v[2 * e], v[2 * e + 1]};
    const bf16x2v h = __builtin_convertvector(x, bf16x2v);
    const f32x2v r1 = x - __builtin_convertvector(h, f32x2v);
    const bf16x2v m = __builtin_convertvector(r1, bf16x2v);
    const f32x2v r2 = r1 - __builtin_convertvector(m, f32x2v);
    hi[e] = __builtin_bit_cast(uint32_t, h);
    mid[e] = __builtin_bit_cast(uint32_t, m);
    lo[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2v));
  }
}

// --- wave / block primitives ------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index as a scalar (uniform) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Inclusive scan over the 64 lanes of a wave with DPP moves (no LDS traffic):
// shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of
// row 0 (row 2) is added to row 1 (row 3) and lane 31 to rows 2 and 3.
// Lanes a move does not write keep `ident`, the operation's identity.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t ident, Op op) {
  const int id = (int)ident;
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  return wave_scan_dpp(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}
// reductions: the scan's last lane, returned to every lane as a scalar
__device__ __forceinline__ uint32_t wave_last(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_max(float v) {
  const uint32_t r = wave_scan_dpp(__float_as_uint(v), __float_as_uint(-INFINITY), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  });
  return __uint_as_float(wave_last(r));
}
__device__ __forceinline__ float wave_sum(float v) {
  const uint32_t r = wave_scan_dpp(__float_as_uint(v), 0u, [](uint32_t x, uint32_t y) {
    return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
  });
  return __uint_as_float(wave_last(r));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return wave_last(wave_incl_scan(v)); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_last(wave_scan_dpp(v, 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return min(x, y); }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_last(wave_scan_dpp(v, 0u, [](uint32_t x, uint32_t y) { return max(x, y); }));
}
// 64-bit maximum over each row of 16 lanes (row_ror 1, 2, 4, 8), in every lane
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  uint64_t t;
  t = dpp_u64<0x121>(v); v = t > v ? t : v;
  t = dpp_u64<0x122>(v); v = t > v ? t : v;
  t = dpp_u64<0x124>(v); v = t > v ? t : v;
  t = dpp_u64<0x128>(v); v = t > v ? t : v;
  return v;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}
// 64-bit maximum over the wave, returned to every lane as a scalar
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = row_max_u64(v);
  uint64_t r = lane_u64(v, 0), t;
  t = lane_u64(v, 16); r = t > r ? t : r;
  t = lane_u64(v, 32); r = t > r ? t : r;
  t = lane_u64(v, 48); r = t > r ? t : r;
  return r;
}

// sum within aligned groups of G lanes (G = 16 or 32)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive scan over each row of 16 lanes (row_shr 1, 2, 4, 8).
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  return v;
}
// Exclusive scan over the block (NW <= 16 waves) without its closing
// barrier: the caller passes a workgroup barrier before `tmp` (>= NW words of
// LDS) is written again. Returns the exclusive prefix; *total receives the
// block total. The wave totals are scanned across the 16 lanes of each row
// and read back with scalar lane reads (short code: this library's kernels
// are bound in part by fetching the instructions they execute).
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan_open(uint32_t v, uint32_t* tmp,
                                                         uint32_t* total) {
  static_assert(NW >= 1 && NW <= 16, "one row of lanes scans the wave totals");
  const uint32_t inc = wave_incl_scan(v);
  const int w = wave_id();
  if (lane_id() == 63) tmp[w] = inc;
  __syncthreads();
  const int r = lane_id() & 15;
  const uint32_t ws = row16_incl_scan(r < NW ? tmp[r] : 0u);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)ws, NW - 1);
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)ws, (w + 63) & 63);
  return (w > 0 ? base : 0u) + inc - v;
}
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const uint32_t ex = block_excl_scan_open<NW>(v, tmp, total);
  __syncthreads();
  return ex;
}
template <int NW>
__device__ __forceinline__ float block_max(float v, float* tmp) {
  v = wave_max(v);
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  float r = tmp[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, tmp[i]);
  __syncthreads();
  return r;
}
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* tmp) {
  v = wave_sum(v);
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += tmp[i];
  __syncthreads();
  return r;
}

// --- cross-workgroup barrier among the workgroups of one row -----------------
// The workgroups must be co-resident (the callers assign work by start-order
// tickets and check the capacity). MI355X has one L2 per XCD and the L2s are
// not coherent with each other. Cross-workgroup data is written and read with
// agent-scope atomic stores and loads (they bypass the per-CU L1), so
// workgroups on one XCD see each other's data in their shared L2; across XCDs
// an agent-scope release (write-back of the writer's L2, buffer_wbl2) and
// acquire (invalidation of the reader's L2, buffer_inv) are needed, and they
// are costly (about 6 us per barrier at the 128K layer step).
//
// `local`: the caller placed every workgroup of the row in one class of
// workgroup ids (id % 8, the XCD the dispatcher sends them to). Each
// workgroup checks this against the hardware XCC id. Arrival adds 1, plus
// 1 << 16 if the workgroup is not on its class's XCD (or `local` is false);
// such a workgroup releases before arriving. If, once all P have arrived,
// any workgroup of the row was not on the common XCD, every workgroup
// releases (if it has not), arrives at the row's second counter, waits for
// all P there and acquires: exact either way, fence-free when the placement
// holds. Without `local` every workgroup releases before arriving and
// acquires after the wait. `round` counts this row's barriers (1, 2, ...).
// bar[0] / bar[1] are the row's counters, zeroed before launch. Every thread
// first completes its own memory operations (s_waitcnt) and meets the others
// at the workgroup barrier; one thread does the rest. The spins are bounded:
// after w.limit polls the workgroup records the failure in *w.err (the
// status word the host reads after the call) and goes on, so no wave can
// wait forever; the barrier then returns false to every thread, and callers
// stop using exchanged data. w.extra raises every arrival target (0 in
// normal use: the host sets it only to exercise that path).
struct WaitCtl {
  uint32_t* err;     // status word: 1 once any wait gave up
  uint32_t limit;    // polls before giving up
  uint32_t extra;    // added to every arrival target
};
__device__ __forceinline__ uint32_t hw_xcc_id() {
  return (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID
}
// `seen`: the counter's value as this workgroup's own arrival left it (the
// arrival's returned value plus its increment): the last workgroup to arrive
// sees the target there and needs no poll.
__device__ __forceinline__ bool spin_until(uint32_t* ctr, uint32_t mask, uint32_t target,
                                           const WaitCtl& w, uint32_t* last, uint32_t seen) {
  uint32_t spins = 0, v = seen;
  bool ok = true;
  if ((v & mask) >= target) {
    *last = v;
    return true;
  }
  while (((v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & mask) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > w.limit) {
      __hip_atomic_store(w.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = false;
      break;
    }
  }
  *last = v;
  return ok;
}
__device__ __forceinline__ bool group_barrier(uint32_t* bar, uint32_t P, uint32_t round,
                                              bool local, const WaitCtl& w) {
  __shared__ uint32_t s_ok;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t target = P * round + w.extra;
  if (threadIdx.x == 0 && !local) {
    // rows spread over XCDs: everyone releases, arrives, waits, acquires
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t seen = __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    uint32_t v;
    const bool ok = spin_until(&bar[0], 0xFFFFu, target, w, &v, seen);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ok = ok;
  } else if (threadIdx.x == 0) {
    const bool remote = hw_xcc_id() != (blockIdx.x & 7u);
    if (remote) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t inc = 1u | ((uint32_t)remote << 16);
    const uint32_t seen = __hip_atomic_fetch_add(&bar[0], inc, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) + inc;
    uint32_t v;
    bool ok = spin_until(&bar[0], 0xFFFFu, target, w, &v, seen);
    if ((v >> 16) != 0u) {
      if (!remote) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t seen1 =
          __hip_atomic_fetch_add(&bar[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
      ok = spin_until(&bar[1], 0xFFFFFFFFu, target, w, &v, seen1) && ok;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0u;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup id -> logical tile mapping that keeps consecutive logical tiles on
// one XCD: the dispatcher hands workgroup ids to the 8 XCDs round-robin, so
// id i runs on XCD i % 8. When nb is a multiple of 8, XCD x gets the
// contiguous logical range [x*nb/8, (x+1)*nb/8). A bijection either way.
__device__ __forceinline__ int xcd_tile(int bid, int nb) {
  return (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
}

// Logical tile of this workgroup, handed out in start order by `tickets`
// (call from one thread). A workgroup holds a ticket only once it runs, so
// the holders of the lowest unfinished tickets are always resident: tiles
// that wait on each other (a row's workgroups) cannot deadlock as long as
// the co-resident capacity covers a row. With `xcd`, workgroup ids are split
// into 8 classes by id % 8 -- the XCD the dispatcher sends each id to -- and
// class c hands out the contiguous tiles [c nb/8, (c+1) nb/8) from its own
// counter, so tiles that share data stay on one XCD and share its L2. The
// caller guarantees nb % 8 == 0 for `xcd`.
__device__ __forceinline__ int ticket_tile(uint32_t* tickets, int nb, bool xcd) {
  if (xcd) {
    const int c = (int)(blockIdx.x & 7u);
    return c * (nb >> 3) + (int)atomicAdd(&tickets[c], 1u);
  }
  return (int)atomicAdd(&tickets[0], 1u);
}

}  // namespace sdkv
