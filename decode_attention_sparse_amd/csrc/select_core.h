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
// lowest index first). Found by an MSD radix select over 11/11/10-bit digits.
// One workgroup per row: three local rounds. P > 1 workgroups per row: one
// global 11-bit histogram round, then an exchange of the keys in the
// threshold bin, after which every workgroup finishes the select and the
// per-workgroup counts locally (radix_select_coop) -- two cross-workgroup
// synchronisations in all.
#pragma once
#include "sdkv_device.h"

namespace sdkv {

constexpr int SB = 1024;       // threads per block in select-bearing kernels
constexpr int SNW = SB / 64;   // waves per block

struct SelShared {
  uint32_t hist[2048];
  uint32_t scan[SB];
  uint32_t tmp[2 * SB / 64];
  uint32_t bcast[8];
};

struct SelGroup {
  int P;              // workgroups sharing the row
  int p;              // this workgroup's position (element order)
  uint32_t* ghist;    // [2048] zeroed before launch (P > 1)
  uint32_t* xchg;     // [P][2]
  uint32_t* bar;      // [2] barrier counters, zeroed before launch
  bool local;         // all workgroups of the row are in one id % 8 class
  WaitCtl wait;       // status word and bounds of the barrier waits
  uint32_t* cand;     // [P][cap] candidate keys of each workgroup (P > 1)
  int64_t cap;        // candidate slots per workgroup (>= keys per workgroup)
};

constexpr int kCandPT = 16;  // candidates per thread kept in registers

// Per-thread element masks: bit j is element j of the thread's SPT <= 32.
using Mask = uint32_t;
constexpr int kMaxSPT = 32;

// Calls f(j, rank) for every set bit j of `bits`, where rank is the position
// of slot j among all set slots of the block in element order. Returns the
// number of set slots in the block.
template <int SPT, class F>
__device__ __forceinline__ uint32_t ordered_ranks(Mask bits, SelShared& sh, F&& f) {
  static_assert(SPT * SNW <= SB, "rank table exceeds block");
  static_assert(SPT <= kMaxSPT, "element masks are 32 bits");
  const int w = wave_id(), lane = lane_id();
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint64_t b = __ballot((bits >> j) & 1u);
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
    const uint64_t b = __ballot((bits >> j) & 1u);
    if ((bits >> j) & 1u) f(j, sh.scan[j * SNW + w] + (uint32_t)__popcll(b & lt));
  }
  __syncthreads();
  return tot;
}

// Finds, for each of NQ <= 2 ranks need[q], the digit v[q] of an
// nbins-bin histogram in sh.hist with #(digit > v) < need <= #(digit >= v);
// above[q] = #(digit > v[q]); *total (optional) = the histogram's total. All
// uniform across the block. (If fewer than need[q] keys exist, v[q] = 0 and
// above[q] = 0.) One prefix scan over the per-thread bin sums serves every
// rank: the count above thread t's bins is total - (inclusive prefix at t).
// zero_bins: every thread clears its own bins once it has read them, so the
// histogram is zero when the function returns.
template <int NQ>
__device__ __forceinline__ void find_digits(SelShared& sh, int nbins, const uint32_t (&need)[NQ],
                                            uint32_t (&v)[NQ], uint32_t (&above_out)[NQ],
                                            uint32_t* total = nullptr, bool zero_bins = false) {
  static_assert(NQ >= 1 && NQ <= 2, "bcast holds two (digit, above) pairs");
  const int tid = threadIdx.x;
  const int bpt = nbins / SB;
  uint32_t loc = 0;
  for (int i = 0; i < bpt; ++i) loc += sh.hist[tid * bpt + i];
  if (tid == 0)
    for (int q = 0; q < 2 * NQ; ++q) sh.bcast[q] = 0u;
  uint32_t tot;
  // (sh.tmp is next written after the barriers below)
  const uint32_t ex = block_excl_scan_open<SNW>(loc, sh.tmp, &tot);
  const uint32_t above = tot - ex - loc;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (above < need[q] && above + loc >= need[q]) {
      uint32_t run = above;
      for (int i = bpt - 1; i >= 0; --i) {
        const uint32_t c = sh.hist[tid * bpt + i];
        if (run + c >= need[q]) {
          sh.bcast[2 * q] = (uint32_t)(tid * bpt + i);
          sh.bcast[2 * q + 1] = run;
          break;
        }
        run += c;
      }
    }
  }
  if (zero_bins)
    for (int i = 0; i < bpt; ++i) sh.hist[tid * bpt + i] = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    v[q] = sh.bcast[2 * q];
    above_out[q] = sh.bcast[2 * q + 1];
  }
  if (total) *total = tot;
  __syncthreads();
}

// find_digits for one rank: returns v; *above_out = #(digit > v).
__device__ __forceinline__ uint32_t find_digit(SelShared& sh, int nbins, uint32_t need,
                                               uint32_t* above_out, uint32_t* total = nullptr) {
  const uint32_t nq[1] = {need};
  uint32_t v[1], ab[1];
  find_digits<1>(sh, nbins, nq, v, ab, total);
  *above_out = ab[0];
  return v[0];
}

// Multi-workgroup select with two cross-workgroup synchronisations:
//  1. a global histogram of the top 11 key bits gives the threshold bin v1;
//  2. each workgroup publishes the keys of its chunk that fall in bin v1
//     (a few percent of them) and its count of keys above the bin; every
//     workgroup then reads all candidates of the row and finishes the
//     remaining 21 bits of the radix select, and the per-workgroup counts
//     of keys above / equal to the threshold, locally.
template <int SPT>
__device__ __forceinline__ Mask radix_select_coop(const uint32_t (&key)[SPT], uint32_t m, SelShared& sh,
                                      const SelGroup& g, uint32_t* offset, uint32_t* count,
                                      uint32_t* tau_out, uint32_t* s_qcnt, uint32_t bar_base) {
  const int tid = threadIdx.x;
  // --- round 1: global histogram of the top 11 bits ----------------------------
  for (int i = tid; i < 2048; i += SB) sh.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if (key[j] != 0u) atomicAdd(&sh.hist[key[j] >> 21], 1u);
  __syncthreads();
  for (int i = tid; i < 2048; i += SB) {
    const uint32_t c = sh.hist[i];
    if (c) atomicAdd(&g.ghist[i], c);
  }
  if (!group_barrier(g.bar, (uint32_t)g.P, bar_base + 1u, g.local, g.wait)) {
    // a wait gave up (reported in the status word): select nothing
    *offset = 0; *count = 0; *tau_out = 0;
    return 0;
  }
  for (int i = tid; i < 2048; i += SB) sh.hist[i] = ld_agent(&g.ghist[i]);
  __syncthreads();
  uint32_t gt1;
  const uint32_t v1 = find_digit(sh, 2048, m, &gt1);
  const uint32_t need1 = m - min(m, gt1);

  // --- round 2: publish this workgroup's candidates (keys in bin v1) ----------
  Mask cbits = 0;
  uint32_t na = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint32_t k = key[j];
    const uint32_t dg = k >> 21;
    if (k != 0u && dg > v1) ++na;
    if (k != 0u && dg == v1) { cbits |= 1u << j; ++nc; }
  }
  uint32_t tna, tnc;
  (void)block_excl_scan<SNW>(na, sh.tmp, &tna);
  (void)block_excl_scan<SNW>(nc, sh.tmp, &tnc);
  uint32_t* mycand = g.cand + (int64_t)g.p * g.cap;
  ordered_ranks<SPT>(cbits, sh, [&](int j, uint32_t r) {
    if (r < g.cap) st_agent(&mycand[r], key[j]);
  });
  if (tid == 0) {
    st_agent(&g.xchg[2 * g.p], tna);
    st_agent(&g.xchg[2 * g.p + 1], tnc);
  }
  if (!group_barrier(g.bar, (uint32_t)g.P, bar_base + 2u, g.local, g.wait)) {
    *offset = 0; *count = 0; *tau_out = 0;
    return 0;
  }

  // --- every workgroup: counts per workgroup, then all candidates ------------
  // s_qcnt layout: [0,P) above-bin counts A_q, [P,2P) candidate counts c_q,
  // [2P,3P+1) candidate prefix, [3P+1,4P+1) #cand > tau, [4P+1,5P+1) #cand == tau
  const int P = g.P;
  if (tid < P) {
    s_qcnt[tid] = ld_agent(&g.xchg[2 * tid]);
    s_qcnt[P + tid] = min((uint32_t)g.cap, ld_agent(&g.xchg[2 * tid + 1]));
    s_qcnt[3 * P + 1 + tid] = 0u;
    s_qcnt[4 * P + 1 + tid] = 0u;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int q = 0; q < P; ++q) { s_qcnt[2 * P + q] = run; run += s_qcnt[P + q]; }
    s_qcnt[3 * P] = run;
  }
  __syncthreads();
  const uint32_t C = s_qcnt[3 * P];
  const uint32_t* cpre = s_qcnt + 2 * P;
  // candidate g_idx -> (workgroup q, slot) by binary search on the prefix
  auto cand_at = [&](uint32_t gi, int* qo) -> uint32_t {
    int lo = 0, hi = P - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cpre[mid] <= gi) lo = mid; else hi = mid - 1;
    }
    *qo = lo;
    return ld_agent(&g.cand[(int64_t)lo * g.cap + (gi - cpre[lo])]);
  };
  const bool in_regs = C <= (uint32_t)SB * kCandPT;
  uint32_t ck[kCandPT];
  uint32_t cq[kCandPT / 4];  // owning workgroup of each candidate, 8 bits each
  if (in_regs) {
    // this thread's candidates gi = tid + k*SB increase with k, so their
    // owning workgroup is found by advancing monotonically
    int q = 0;
#pragma unroll
    for (int k = 0; k < kCandPT; ++k) {
      const uint32_t gi = (uint32_t)(tid + k * SB);
      ck[k] = 0u;
      if (k % 4 == 0) cq[k / 4] = 0u;
      if ((uint32_t)(k * SB) < C && gi < C) {
        while (q + 1 < P && cpre[q + 1] <= gi) ++q;
        ck[k] = ld_agent(&g.cand[(int64_t)q * g.cap + (gi - cpre[q])]);
        cq[k / 4] |= (uint32_t)q << (8 * (k % 4));
      }
    }
  }
  // local rounds 2 and 3 over the candidates
  uint32_t prefix = v1 << 21, pmask = 0xFFE00000u, need = need1;
  for (int round = 1; round < 3; ++round) {
    const int shift = round == 1 ? 10 : 0;
    const int nbins = round == 1 ? 2048 : 1024;
    for (int i = tid; i < 2048; i += SB) sh.hist[i] = 0u;
    __syncthreads();
    if (in_regs) {
#pragma unroll
      for (int k = 0; k < kCandPT; ++k) {
        const uint32_t c = ck[k];
        if (c != 0u && (c & pmask) == prefix)
          atomicAdd(&sh.hist[(c >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
    } else {
      for (uint32_t gi = tid; gi < C; gi += SB) {
        int q;
        const uint32_t c = cand_at(gi, &q);
        if (c != 0u && (c & pmask) == prefix)
          atomicAdd(&sh.hist[(c >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
    }
    __syncthreads();
    uint32_t gt;
    const uint32_t v = find_digit(sh, nbins, need, &gt);
    need -= min(need, gt);
    prefix |= v << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
  }
  const uint32_t tau = prefix;
  *tau_out = tau;
  // Per-workgroup counts of candidates above / equal to tau. Candidates are
  // laid out in workgroup order, so the lanes of a wave see one or two
  // workgroups: aggregate with ballots, one LDS atomic per workgroup seen.
  auto tally = [&](int q, uint32_t c, bool valid) {
    const bool isgt = valid && c > tau, iseq = valid && c == tau;
    uint64_t pend = __ballot(isgt || iseq);
    while (pend) {
      const int leader = __builtin_ctzll(pend);
      const int qq = __shfl(q, leader, 64);
      const uint64_t same = __ballot((isgt || iseq) && q == qq);
      const uint32_t ngt = (uint32_t)__popcll(__ballot(isgt && q == qq));
      const uint32_t neq = (uint32_t)__popcll(__ballot(iseq && q == qq));
      if (lane_id() == leader) {
        if (ngt) atomicAdd(&s_qcnt[3 * P + 1 + qq], ngt);
        if (neq) atomicAdd(&s_qcnt[4 * P + 1 + qq], neq);
      }
      pend &= ~same;
    }
  };
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kCandPT; ++k) {
      const uint32_t gi = (uint32_t)(tid + k * SB);
      const int q = (int)((cq[k / 4] >> (8 * (k % 4))) & 0xFFu);
      if ((uint32_t)(k * SB) < C) tally(q, ck[k], gi < C && ck[k] >= tau);
    }
  } else {
    for (uint32_t base = 0; base < C; base += SB) {
      const uint32_t gi = base + tid;
      int q = 0;
      const uint32_t c = (gi < C) ? cand_at(gi, &q) : 0u;
      tally(q, c, gi < C && c >= tau);
    }
  }
  __syncthreads();
  uint32_t off_gt = 0, off_eq = 0;
  for (int q = 0; q < g.p; ++q) {
    off_gt += s_qcnt[q] + s_qcnt[3 * P + 1 + q];
    off_eq += s_qcnt[4 * P + 1 + q];
  }
  const uint32_t tg = tna + s_qcnt[3 * P + 1 + g.p];
  const uint32_t te = s_qcnt[4 * P + 1 + g.p];
  __syncthreads();

  Mask gt_bits = 0, eq_bits = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint32_t k = key[j];
    if (k > tau) gt_bits |= 1u << j;
    else if (k == tau && k != 0u) eq_bits |= 1u << j;
  }
  // see radix_select for why this is written without a guarded subtraction
  const uint32_t eq_before = min(need, off_eq);
  const uint32_t rem = need - eq_before;
  const uint32_t take = min(rem, te);
  *offset = off_gt + eq_before;
  *count = tg + take;
  Mask sel = gt_bits;
  if (take == te) {
    sel |= eq_bits;
  } else if (take > 0) {
    Mask keep = 0;
    ordered_ranks<SPT>(eq_bits, sh, [&](int j, uint32_t r) {
      if (r < take) keep |= 1u << j;
    });
    sel |= keep;
  }
  return sel;
}

// Returns this thread's selection bitmask; *offset / *count give the block's
// output range in the row's ascending selection list, *tau the threshold key.
// k-th largest (k >= 1) of the non-zero keys held by the block (N per
// thread) by an LDS radix select over 11/11/10-bit digits, starting at
// `round0` with every key known to carry the digits of `prefix` above it.
// Returns 0 if there are fewer than k keys.
template <int N>
__device__ __forceinline__ uint32_t local_kth(const uint32_t (&keys)[N], uint32_t k, SelShared& sh,
                                              int round0, uint32_t prefix) {
  const int tid = threadIdx.x;
  uint32_t pmask = round0 == 0 ? 0u : (round0 == 1 ? 0xFFE00000u : 0xFFFFFC00u);
  prefix &= pmask;
  uint32_t need = k;
  for (int round = round0; round < 3; ++round) {
    const int shift = round == 0 ? 21 : (round == 1 ? 10 : 0);
    const int nbins = round == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += SB) sh.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint32_t c = keys[j];
      if (c != 0u && (c & pmask) == prefix)
        atomicAdd(&sh.hist[(c >> shift) & (uint32_t)(nbins - 1)], 1u);
    }
    __syncthreads();
    uint32_t gt;
    const uint32_t v = find_digit(sh, nbins, need, &gt);
    need -= min(need, gt);
    prefix |= v << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
  }
  return prefix;
}

// Bin in [0, 2048) of a key's value on the linear scale (v - base) * inv,
// clamped. Monotone non-decreasing in the key for any base and any inv >= 0
// (IEEE rounding is monotone), so keys in a higher bin are always larger;
// identical wherever it is evaluated with the same base and inv.
__device__ __forceinline__ int value_bin(uint32_t k, float base, float inv) {
  const float x = (key_float(k) - base) * inv;
  return (int)fminf(fmaxf(x, 0.f), 2047.f);
}

constexpr int kSampleN = 4096;             // shared sample size (tokens)
constexpr int kSamplePT = kSampleN / SB;
constexpr int kSampleRuns = kSampleN / 16;  // runs of 16 consecutive tokens
static_assert(kSampleN % SB == 0 && (kSampleRuns & (kSampleRuns - 1)) == 0, "sample layout");

// Sample-window select with one cross-workgroup synchronisation.
//
// Every workgroup of the row holds the keys `skey` of the same fixed sample
// of ns of the row's T elements, so all derive the same window: the key
// range between the sample's order statistics of rank m ns / T -/+ (5
// standard deviations + 4), found with a linear 2048-bin histogram between
// the sample's smallest and largest value. The window [lo_key, hi_key) is
// split into 2048 fine bins, fine bin = (k - lo_key) * 2048 / span by a
// fixed-point multiply (monotone in the key, identical in every workgroup).
// Each workgroup
//   * counts its keys at or above hi_key (published in xchg[2p]),
//   * sorts its window keys by fine bin in LDS (a counting sort) and stores
//     them to its list `wl` (row slots [p * cap, p * cap + cap)), with its
//     2048-entry table `wt` of (count | start << 16) per bin.
// There are no global atomics. After the one barrier every workgroup sums
// the P count tables, finds the bin holding the threshold, and reads only
// that bin's keys from each workgroup's list. The threshold is their
// need-th largest key; their owners give each workgroup's count of keys
// equal to it (tie quota, lowest element index first). Keys above the
// threshold need no exchange: each workgroup selects its own. If the window
// misses the threshold, or the threshold's bin holds more than SB/2 keys,
// the function returns false having used one barrier, and the caller runs
// the two-barrier radix select; the result is exact either way. The
// selection's global output offset is not computed here.
template <int SPT>
__device__ __forceinline__ bool sample_window_select(const uint32_t (&key)[SPT],
                                                     const uint32_t (&skey)[kSamplePT],
                                                     uint32_t ns, uint32_t m, uint32_t T,
                                                     SelShared& sh, const SelGroup& g,
                                                     uint32_t* wt, uint32_t* tau_out,
                                                     Mask* sel_out, uint32_t* s_qcnt) {
  static_assert(SB * 2 == 2048, "two fine bins per thread");
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int P = g.P;
  // --- sample value range ------------------------------------------------------
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int j = 0; j < kSamplePT; ++j)
    if (skey[j] != 0u) { kmn = min(kmn, skey[j]); kmx = max(kmx, skey[j]); }
  kmn = wave_min_u32(kmn);
  kmx = wave_max_u32(kmx);
  if (lane == 0) { sh.tmp[w] = kmn; sh.tmp[SNW + w] = kmx; }
  if (tid == 0) { sh.bcast[5] = 0u; sh.bcast[7] = 0u; }
  for (int i = tid; i < 2048; i += SB) sh.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < SNW; ++i) { kmn = min(kmn, sh.tmp[i]); kmx = max(kmx, sh.tmp[SNW + i]); }
  const float base = key_float(kmn);
  const float span = key_float(kmx) - base;
  const float inv = (kmx > kmn && span > 0.f && span < INFINITY) ? 2048.f / span : 0.f;
  // --- window from the sample's rank estimates --------------------------------
  const float rho = (ns >= T) ? (float)m : (float)((double)m * ns / T);
  const float sd = sqrtf(fmaxf(rho * (1.f - rho / (float)ns), 0.f));
  const float wd = (ns >= T) ? 0.f : 5.f * sd + 4.f;
  const uint32_t r_hi = (uint32_t)fmaxf(1.f, floorf(rho - wd));
  const uint32_t r_lo = (uint32_t)fminf((float)ns, fmaxf((float)r_hi, ceilf(rho + wd)));
#pragma unroll
  for (int j = 0; j < kSamplePT; ++j)
    if (skey[j] != 0u) atomicAdd(&sh.hist[value_bin(skey[j], base, inv)], 1u);
  __syncthreads();  // also: every thread has read sh.tmp
  const uint32_t rr[2] = {r_hi, r_lo};
  uint32_t bb[2], gtx[2];
  find_digits<2>(sh, 2048, rr, bb, gtx, nullptr, true);  // leaves sh.hist zero
  const int b_hi = (int)bb[0], b_lo = (int)bb[1];
  // key thresholds at the edges of the coarse bins b_lo and b_hi
  uint32_t lo_key = 1u, hi_key = 0xFFFFFFFFu;
  if (inv > 0.f) {
    lo_key = max(1u, float_key(base + (float)b_lo / inv));
    hi_key = float_key(base + (float)(b_hi + 1) / inv);
  }
  if (hi_key <= lo_key) hi_key = lo_key + 1u;
  const uint32_t mulc =
      (uint32_t)fmin(4294967295.0, 2048.0 * 4294967296.0 / (double)(hi_key - lo_key));
  // --- publish: count above the window; window keys sorted by fine bin --------
  uint32_t na = 0;
  uint32_t pos[SPT];  // (fine bin << 16 | rank in bin) of window keys, else ~0
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint32_t k = key[j];
    na += (k >= hi_key) ? 1u : 0u;
    pos[j] = 0xFFFFFFFFu;
    if (k >= lo_key && k < hi_key) {
      const uint32_t fb = min(2047u, __umulhi(k - lo_key, mulc));
      pos[j] = (fb << 16) | atomicAdd(&sh.hist[fb], 1u);
    }
  }
  const uint32_t na_w = wave_sum_u32(na);
  if (lane == 0) atomicAdd(&sh.bcast[5], na_w);
  __syncthreads();
  // exclusive prefix over the 2048 bins, two per thread
  const uint32_t c0 = sh.hist[2 * tid], c1 = sh.hist[2 * tid + 1];
  uint32_t tot;
  // (sh.tmp is next written after the barrier below)
  const uint32_t ex = block_excl_scan_open<SNW>(c0 + c1, sh.tmp, &tot);
  uint32_t* mywt = wt + (int64_t)g.p * 2048;
  __hip_atomic_store((uint64_t*)(mywt + 2 * tid),
                     ((uint64_t)(c1 | ((ex + c0) << 16)) << 32) | (c0 | (ex << 16)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  sh.hist[2 * tid] = ex;
  sh.hist[2 * tid + 1] = ex + c0;
  if (tid == 0) st_agent(&g.xchg[2 * g.p], sh.bcast[5]);
  __syncthreads();
  uint32_t* mywl = g.cand + (int64_t)g.p * g.cap;
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if (pos[j] != 0xFFFFFFFFu) st_agent(&mywl[sh.hist[pos[j] >> 16] + (pos[j] & 0xFFFFu)], key[j]);
  if (!group_barrier(g.bar, (uint32_t)P, 1u, g.local, g.wait)) {
    // a wait gave up (reported in the status word): select nothing, and
    // report the select as done so that no further exchange is attempted
    *tau_out = 0;
    *sel_out = 0;
    return true;
  }
  // --- threshold bin from the counts above and the summed count tables --------
  if (tid < P) s_qcnt[tid] = ld_agent(&g.xchg[2 * tid]);
  {
    // eight tables' entries requested before any is added (one round trip
    // to L2 per eight workgroups instead of one per workgroup)
    uint32_t h0 = 0, h1 = 0;
    for (int q0 = 0; q0 < P; q0 += 8) {
      uint64_t e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        e[k] = __hip_atomic_load((const uint64_t*)(wt + (int64_t)min(q0 + k, P - 1) * 2048 + 2 * tid),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint64_t ek = (q0 + k < P) ? e[k] : 0ull;
        h0 += (uint32_t)ek & 0xFFFFu;
        h1 += (uint32_t)(ek >> 32) & 0xFFFFu;
      }
    }
    sh.hist[2 * tid] = h0;
    sh.hist[2 * tid + 1] = h1;
  }
  __syncthreads();
  uint32_t A = 0;
  for (int q = 0; q < P; ++q) A += s_qcnt[q];
  if (A >= m) {
    __syncthreads();
    return false;
  }
  const uint32_t need1 = m - A;
  uint32_t gt2, total;
  const int bstar = (int)find_digit(sh, 2048, need1, &gt2, &total);
  const uint32_t nc = sh.hist[bstar];
  if (total < need1 || nc > (uint32_t)(SB / 2)) {
    __syncthreads();
    return false;
  }
  const uint32_t need2 = need1 - gt2;  // 1 <= need2 <= nc
  // --- the threshold bin's keys from every workgroup --------------------------
  if (tid < P) {
    const uint32_t e = ld_agent(&wt[(int64_t)tid * 2048 + bstar]);
    s_qcnt[P + tid] = e & 0xFFFFu;   // count
    s_qcnt[2 * P + tid] = e >> 16;   // start
  }
  __syncthreads();
  if (tid < (int)nc) {
    int q = 0;
    uint32_t off = 0;
    while (q + 1 < P && off + s_qcnt[P + q] <= (uint32_t)tid) { off += s_qcnt[P + q]; ++q; }
    sh.scan[tid] = ld_agent(&g.cand[(int64_t)q * g.cap + s_qcnt[2 * P + q] + (tid - off)]);
    sh.scan[SB / 2 + tid] = (uint32_t)q;
  }
  __syncthreads();
  if (tid < (int)nc) {
    const uint32_t x = sh.scan[tid];
    uint32_t ngt = 0, nge = 0;
    for (uint32_t i = 0; i < nc; ++i) {
      const uint32_t y = sh.scan[i];
      ngt += y > x ? 1u : 0u;
      nge += y >= x ? 1u : 0u;
    }
    if (ngt < need2 && need2 <= nge) sh.bcast[7] = x;
  }
  __syncthreads();
  const uint32_t tau = sh.bcast[7];
  // keys of the bin above tau (all workgroups), equal to tau before / at this one
  uint32_t b_gt = 0, eq_before = 0, te = 0;
  for (uint32_t i = 0; i < nc; ++i) {
    const uint32_t y = sh.scan[i], q = sh.scan[SB / 2 + i];
    b_gt += y > tau ? 1u : 0u;
    eq_before += (y == tau && q < (uint32_t)g.p) ? 1u : 0u;
    te += (y == tau && q == (uint32_t)g.p) ? 1u : 0u;
  }
  __syncthreads();
  *tau_out = tau;
  // keys equal to tau to take, handed out in workgroup (element) order; see
  // radix_select_local for why this is written without a guarded subtraction
  const uint32_t need = need2 - min(need2, b_gt);
  const uint32_t eb = min(need, eq_before);
  const uint32_t rem = need - eb;
  const uint32_t take = min(rem, te);
  Mask gt_bits = 0, eq_bits = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint32_t k = key[j];
    if (k > tau) gt_bits |= 1u << j;
    else if (k == tau && k != 0u) eq_bits |= 1u << j;
  }
  Mask sel = gt_bits;
  if (take == te) {
    sel |= eq_bits;
  } else if (take > 0) {
    Mask keep = 0;
    ordered_ranks<SPT>(eq_bits, sh, [&](int j, uint32_t r) {
      if (r < take) keep |= 1u << j;
    });
    sel |= keep;
  }
  *sel_out = sel;
  return true;
}

// Exact top-m of the keys of one workgroup (the row is not split): three
// local radix rounds, then ties to the lowest element index.
template <int SPT>
__device__ __forceinline__ Mask radix_select_local(const uint32_t (&key)[SPT], uint32_t m,
                                                   SelShared& sh, uint32_t* offset,
                                                   uint32_t* count, uint32_t* tau_out) {
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
    uint32_t gt;
    const uint32_t v = find_digit(sh, nbins, need, &gt);
    need -= min(need, gt);
    prefix |= v << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
  }
  const uint32_t tau = prefix;
  *tau_out = tau;

  Mask gt_bits = 0, eq_bits = 0;
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const uint32_t k = key[j];
    if (k > tau) { gt_bits |= 1u << j; ++cg; }
    else if (k == tau && k != 0u) { eq_bits |= 1u << j; ++ce; }
  }
  uint32_t tg, te;
  (void)block_excl_scan<SNW>(cg, sh.tmp, &tg);
  (void)block_excl_scan<SNW>(ce, sh.tmp, &te);
  const uint32_t off_gt = 0, off_eq = 0;  // a single workgroup owns the row
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
  Mask sel = gt_bits;
  if (take == te) {
    sel |= eq_bits;
  } else if (take > 0) {
    Mask keep = 0;
    ordered_ranks<SPT>(eq_bits, sh, [&](int j, uint32_t r) {
      if (r < take) keep |= 1u << j;
    });
    sel |= keep;
  }
  return sel;
}

// Single- or multi-workgroup select (P > 1: radix_select_coop); s_qcnt is LDS
// scratch of >= 5P+1 words.
template <int SPT>
__device__ __forceinline__ Mask radix_select(const uint32_t (&key)[SPT], uint32_t m, SelShared& sh,
                                             const SelGroup& g, uint32_t* offset, uint32_t* count,
                                             uint32_t* tau_out, uint32_t* s_qcnt) {
  if (g.P > 1) return radix_select_coop<SPT>(key, m, sh, g, offset, count, tau_out, s_qcnt, 0u);
  return radix_select_local<SPT>(key, m, sh, offset, count, tau_out);
}

}  // namespace sdkv
