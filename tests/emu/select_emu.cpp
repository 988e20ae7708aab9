// Runs the select core (select_core.h) on the CPU for one row split over P
// workgroups of SB threads, every thread a fiber, and checks the selection:
// exactly m keys, every selected key >= every other, ties to the lower
// element. Test infrastructure only (see emu_device.h).
//
// usage: select_emu SPT P T m seed kind(normal|ties|plateau) [window(1)|radix(0)]
//                   [order: 0 ascending | 1 descending | 2 shuffled]
//
// The order is the one in which runnable fibers are resumed between their
// synchronisations. A result that depends on it means two threads touch the
// same location with no synchronisation between them (a race).
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <random>
#include <vector>

#include "sdkv_device.h"  // the emulation header, copied under this name
#include "emu_fibers.h"
#include "select_core.h"

using namespace sdkv;

struct Row {
  int P;
  int64_t T, m, chunk;
  std::vector<uint32_t> key;    // [T]
  std::vector<uint8_t> sel;     // [T] output
  std::vector<uint32_t> wt, xchg, bar, cand, ghist;
  uint32_t err = 0;
  std::vector<SelShared> sh;
  std::vector<std::vector<uint32_t>> qcnt;
  bool window = true;
  int fallbacks = 0;
};
static Row g_row;

template <int SPT>
static void thread_body() {
  Row& R = g_row;
  const int tid = (int)threadIdx.x, p = (int)blockIdx.x;
  const int64_t t0 = (int64_t)p * R.chunk, t1 = std::min<int64_t>(R.T, t0 + R.chunk);
  uint32_t key[SPT];
  for (int j = 0; j < SPT; ++j) {
    const int64_t t = t0 + (int64_t)j * SB + tid;
    key[j] = (t < t1) ? R.key[t] : 0u;
  }
  SelGroup grp;
  grp.P = R.P;
  grp.p = p;
  grp.ghist = R.ghist.data();
  grp.xchg = R.xchg.data();
  grp.bar = R.bar.data();
  grp.local = true;
  grp.wait = WaitCtl{&R.err, 1u << 22, 0u};
  grp.cand = R.cand.data();
  grp.cap = R.chunk;
  SelShared& sh = R.sh[p];
  uint32_t* s_qcnt = R.qcnt[p].data();
  uint32_t offset = 0, count = 0, tau = 0;
  Mask sel = 0;
  bool done = false;
  if (R.window) {
    // the row kernel's shared sample: all tokens if T <= kSampleN, else
    // kSampleRuns runs of 16 consecutive tokens, run g starting at g T / R
    const int64_t ns = std::min<int64_t>(kSampleN, R.T);
    const bool all = R.T <= kSampleN;
    uint32_t skey[kSamplePT];
    for (int j = 0; j < kSamplePT; ++j) {
      const int64_t i = std::min<int64_t>(tid + j * SB, ns - 1);
      const int64_t t = all ? i : ((i >> 4) * R.T) / kSampleRuns + (i & 15);
      skey[j] = (tid + j * SB < ns) ? R.key[t] : 0u;
    }
    done = sample_window_select<SPT>(key, skey, (uint32_t)ns, (uint32_t)R.m, (uint32_t)R.T, sh, grp,
                                     R.wt.data(), &tau, &sel, s_qcnt);
    if (!done && tid == 0) ++R.fallbacks;
    if (!done) sel = radix_select_coop<SPT>(key, (uint32_t)R.m, sh, grp, &offset, &count, &tau, s_qcnt, 1u);
  } else {
    sel = radix_select_coop<SPT>(key, (uint32_t)R.m, sh, grp, &offset, &count, &tau, s_qcnt, 0u);
  }
  for (int j = 0; j < SPT; ++j)
    if ((sel >> j) & 1u) R.sel[t0 + (int64_t)j * SB + tid] = 1;
}

template <int SPT>
static void fiber_entry() {
  thread_body<SPT>();
  emu::fiber_exit();
}

template <int SPT>
static int run(int P, int64_t T, int64_t m, uint32_t seed, const char* kind, bool window,
               int order) {
  Row& R = g_row;
  R.P = P;
  R.T = T;
  R.m = m;
  R.chunk = (T + P - 1) / P;
  R.window = window;
  if (R.chunk > (int64_t)SB * SPT) {
    fprintf(stderr, "chunk %lld exceeds %d keys per workgroup\n", (long long)R.chunk, SB * SPT);
    return 2;
  }
  std::mt19937_64 rng(seed);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::uniform_int_distribution<int> ui(-20, 20);
  R.key.resize(T);
  for (int64_t t = 0; t < T; ++t) {
    float v;
    if (!strcmp(kind, "ties")) v = (float)ui(rng);
    else if (!strcmp(kind, "plateau")) v = (t % 7 == 0) ? 1.0f : nd(rng);
    else v = nd(rng);
    R.key[t] = float_key(v);
  }
  R.sel.assign(T, 0);
  R.wt.assign((size_t)P * 2048, 0u);
  R.xchg.assign((size_t)P * 2, 0u);
  R.bar.assign(2, 0u);
  R.cand.assign((size_t)P * R.chunk, 0u);
  R.ghist.assign(2048, 0u);
  R.sh.assign(P, SelShared{});
  R.qcnt.assign(P, std::vector<uint32_t>(5 * 64 + 1, 0u));
  emu::run_fibers(P, SB, fiber_entry<SPT>, order, seed);

  // check: m selected; none unselected above a selected one; among keys
  // equal to the threshold, the lowest elements selected
  int64_t n = 0;
  uint32_t tau = 0xFFFFFFFFu;
  for (int64_t t = 0; t < T; ++t)
    if (R.sel[t]) { ++n; tau = std::min(tau, R.key[t]); }
  int bad = 0;
  bool seen_unselected_eq = false;
  for (int64_t t = 0; t < T; ++t) {
    if (!R.sel[t] && R.key[t] > tau) ++bad;
    if (R.key[t] == tau) {
      if (!R.sel[t]) seen_unselected_eq = true;
      else if (seen_unselected_eq) ++bad;
    }
  }
  const int64_t want = std::min<int64_t>(m, T);
  printf("SPT %d P %d T %lld m %lld %s %s order %d: selected %lld (want %lld), misplaced %d, window "
         "fallbacks %d, status %u\n",
         SPT, P, (long long)T, (long long)m, kind, window ? "window" : "radix", order, (long long)n,
         (long long)want, bad, R.fallbacks, R.err);
  return (n == want && bad == 0 && R.err == 0) ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc < 7) {
    fprintf(stderr, "usage: %s SPT P T m seed kind [window]\n", argv[0]);
    return 2;
  }
  const int spt = atoi(argv[1]), P = atoi(argv[2]);
  const int64_t T = atoll(argv[3]), m = atoll(argv[4]);
  const uint32_t seed = (uint32_t)atoi(argv[5]);
  const bool window = argc > 7 ? atoi(argv[7]) != 0 : true;
  const int order = argc > 8 ? atoi(argv[8]) : 0;
  if (spt == 16) return run<16>(P, T, m, seed, argv[6], window, order);
  if (spt == 32) return run<32>(P, T, m, seed, argv[6], window, order);
  if (spt == 8) return run<8>(P, T, m, seed, argv[6], window, order);
  fprintf(stderr, "SPT must be 8, 16 or 32\n");
  return 2;
}
