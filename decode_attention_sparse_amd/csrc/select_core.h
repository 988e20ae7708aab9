// Exact top-m selection over register-resident keys, shared by the decode
// row kernel and the stand-alone top-k kernel.
//
// A row of n keys is split over P workgroups of SB threads; each thread holds
// SPT keys in registers, slot j of thread `tid` being element
// t0 + j*SB + tid of the row (so (j, wave, lane) order is element order).
// Keys are order-preserving uint32 images of fp32 scores; key 0 marks an
// empty slot.
//
// Selection = the m largest keys, ties broken toward the lower element index
// (the "top 10%" of the review page's Summary, with the tie rule read as
// lowest index first). Found by a 3-round MSD radix select over 11/11/10-bit
// digits; with P > 1 the per-workgroup digit histograms are merged through
// global atomics between cooperative barriers, and a final exchange of
// per-workgroup counts gives every workgroup its output offset and its share
// of the keys equal to the threshold.
#pragma once
#include "sdkv_device.h"

namespace sdkv {

constexpr int SB = 512;        // threads per block in select-bearing kernels
constexpr int SNW = SB / 64;   // waves per block

struct SelShared {
  uint32_t hist[2048];
  uint32_t scan[SB];
  uint32_t tmp[16];
  uint32_t bcast[8];
};

struct SelGroup {
  int P;              // workgroups sharing the row
  int p;              // this workgroup's position (element order)
  uint32_t* ghist;    // [3][2048] zeroed before launch (P > 1)
  uint32_t* xchg;     // [P][2]
  uint32_t* bar;      // barrier counter, zeroed before launch
  uint32_t* err;      // set to 1 if a barrier wait gave up
};

// Calls f(j, rank) for every set bit j of `bits`, where rank is the position
// of slot j among all set slots of the block in element order.
template <int SPT, class F>
__device__ __forceinline__ void ordered_ranks(uint64_t bits, SelShared& sh, F&& f) {
  static_assert(SPT * SNW <= SB, "rank table exceeds block");
  const int w = wave_id(), lane = lane_id();
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint64_t b = __ballot((bits >> j) & 1ull);
    if (lane == 0) sh.scan[j * SNW + w] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  const int e = threadIdx.x;
  const uint32_t v = (e < SPT * SNW) ? sh.scan[e] : 0u;
  uint32_t tot;
  const uint32_t ex = block_excl_scan<SNW>(v, sh.tmp, &tot);
  if (e < SPT * SNW) sh.scan[e] = ex;
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint64_t b = __ballot((bits >> j) & 1ull);
    if ((bits >> j) & 1ull) f(j, sh.scan[j * SNW + w] + (uint32_t)__popcll(b & lt));
  }
  __syncthreads();
}

// Returns this thread's selection bitmask; *offset / *count give the block's
// output range in the row's ascending selection list, *tau the threshold key.
template <int SPT>
__device__ uint64_t radix_select(const uint32_t (&key)[SPT], uint32_t m, SelShared& sh,
                                 const SelGroup& g, uint32_t* offset, uint32_t* count,
                                 uint32_t* tau_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0, need = m;
  for (int round = 0; round < 3; ++round) {
    const int shift = round == 0 ? 21 : (round == 1 ? 10 : 0);
    const int nbins = round == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += SB) sh.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const uint32_t k = key[j];
      if (k != 0u && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & (uint32_t)(nbins - 1)], 1u);
    }
    __syncthreads();
    if (g.P > 1) {
      uint32_t* gh = g.ghist + round * 2048;
      for (int i = tid; i < nbins; i += SB) {
        const uint32_t c = sh.hist[i];
        if (c) atomicAdd(&gh[i], c);
      }
      group_barrier(g.bar, (uint32_t)g.P * (round + 1), g.err);
      for (int i = tid; i < nbins; i += SB) sh.hist[i] = ld_agent(&gh[i]);
      __syncthreads();
    }
    // Find digit v with  #(digit > v) < need <= #(digit >= v).
    const int bpt = nbins / SB;
    uint32_t loc = 0;
    for (int i = 0; i < bpt; ++i) loc += sh.hist[tid * bpt + i];
    sh.scan[SB - 1 - tid] = loc;  // reversed order: a prefix scan gives suffix sums
    if (tid == 0) { sh.bcast[0] = 0u; sh.bcast[1] = 0u; sh.bcast[2] = 0u; }
    __syncthreads();
    const uint32_t rv = sh.scan[tid];
    uint32_t tot;
    const uint32_t above = block_excl_scan<SNW>(rv, sh.tmp, &tot);
    const int o = SB - 1 - tid;
    if (above < need && above + rv >= need) {
      uint32_t run = above;
      for (int i = bpt - 1; i >= 0; --i) {
        const uint32_t c = sh.hist[o * bpt + i];
        if (run + c >= need) {
          sh.bcast[0] = (uint32_t)(o * bpt + i);
          sh.bcast[1] = run;
          sh.bcast[2] = c;
          break;
        }
        run += c;
      }
    }
    __syncthreads();
    const uint32_t v = sh.bcast[0], gt = sh.bcast[1];
    __syncthreads();
    need -= min(need, gt);
    prefix |= v << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
  }
  const uint32_t tau = prefix;
  *tau_out = tau;

  uint64_t gt_bits = 0, eq_bits = 0;
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint32_t k = key[j];
    if (k > tau) { gt_bits |= 1ull << j; ++cg; }
    else if (k == tau && k != 0u) { eq_bits |= 1ull << j; ++ce; }
  }
  uint32_t tg, te;
  (void)block_excl_scan<SNW>(cg, sh.tmp, &tg);
  (void)block_excl_scan<SNW>(ce, sh.tmp, &te);
  uint32_t off_gt = 0, off_eq = 0;
  if (g.P > 1) {
    if (tid == 0) {
      st_agent(&g.xchg[2 * g.p], tg);
      st_agent(&g.xchg[2 * g.p + 1], te);
    }
    group_barrier(g.bar, (uint32_t)g.P * 4u, g.err);
    if (tid < 64) {
      uint32_t a = 0, b = 0;
      for (int q = tid; q < g.p; q += 64) {
        a += ld_agent(&g.xchg[2 * q]);
        b += ld_agent(&g.xchg[2 * q + 1]);
      }
      a = wave_sum_u32(a);
      b = wave_sum_u32(b);
      if (tid == 0) { sh.bcast[4] = a; sh.bcast[5] = b; }
    }
    __syncthreads();
    off_gt = sh.bcast[4];
    off_eq = sh.bcast[5];
    __syncthreads();
  }
  // Equal keys are handed out in element order: the blocks before this one
  // take min(need, off_eq) of them, this one takes the next min(rem, te).
  // Written without a subtraction guarded by a comparison: clang/LLVM tags
  // such a subtraction "no unsigned wrap" and has been seen to reuse that as
  // a global fact (need >= off_eq), folding min(need, off_eq) to off_eq.
  const uint32_t eq_before = min(need, off_eq);
  const uint32_t rem = need - eq_before;
  const uint32_t take = min(rem, te);
  *offset = off_gt + eq_before;
  *count = tg + take;
  uint64_t sel = gt_bits;
  if (take == te) {
    sel |= eq_bits;
  } else if (take > 0) {
    uint64_t keep = 0;
    ordered_ranks<SPT>(eq_bits, sh, [&](int j, uint32_t r) {
      if (r < take) keep |= 1ull << j;
    });
    sel |= keep;
  }
  return sel;
}

}  // namespace sdkv
