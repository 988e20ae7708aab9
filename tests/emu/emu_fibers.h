// Fiber scheduler for the host emulation (emu_device.h): every GPU thread of
// every workgroup is a ucontext fiber; workgroup and wave barriers are
// cooperative waits. run_fibers resumes the runnable fibers in ascending,
// descending or shuffled order between their synchronisations. Test
// infrastructure only.
#pragma once
#include <ucontext.h>

#include <algorithm>
#include <cstring>
#include <random>
#include <vector>

namespace emu {
struct Fiber {
  ucontext_t ctx;
  int tid = 0, wg = 0;
  bool done = false;
};
static ucontext_t g_main;
static Fiber* g_cur = nullptr;
static std::vector<Fiber*> g_fibers;
struct Wave {
  uint64_t slots[64];
  int count = 0;
  unsigned gen = 0;
};
struct Group {
  int count = 0;
  unsigned gen = 0;
  uint32_t flag = 0;
  std::vector<Wave> waves;
};
static std::vector<Group> g_groups;
static int g_sb = 0;

D3 tid3() { return D3{(unsigned)g_cur->tid, 0, 0}; }
D3 bid3() { return D3{(unsigned)g_cur->wg, 0, 0}; }
static void yield_now() {
  Fiber* f = g_cur;
  swapcontext(&f->ctx, &g_main);
}
void spin_yield() { yield_now(); }
void block_barrier() {
  Group& g = g_groups[g_cur->wg];
  const unsigned my = g.gen;
  if (++g.count == g_sb) {
    g.count = 0;
    ++g.gen;
  } else {
    while (g.gen == my) yield_now();
  }
}
void wave_barrier() {
  Wave& w = g_groups[g_cur->wg].waves[g_cur->tid >> 6];
  const unsigned my = w.gen;
  if (++w.count == 64) {
    w.count = 0;
    ++w.gen;
  } else {
    while (w.gen == my) yield_now();
  }
}
uint64_t* wave_slots() { return g_groups[g_cur->wg].waves[g_cur->tid >> 6].slots; }
uint32_t* wg_flag() { return &g_groups[g_cur->wg].flag; }
}  // namespace emu


namespace emu {
// nwg workgroups of sb fibers each running body(); order: 0 ascending,
// 1 descending, 2 shuffled (seeded)
inline void run_fibers(int nwg, int sb, void (*entry)(), int order, uint32_t seed,
                       size_t stack = 64 * 1024) {
  g_sb = sb;
  g_groups.assign(nwg, Group{});
  for (auto& g : g_groups) g.waves.assign(sb / 64, Wave{});
  std::vector<char> stacks((size_t)nwg * sb * stack);
  for (int p = 0; p < nwg; ++p)
    for (int t = 0; t < sb; ++t) {
      auto* f = new Fiber;
      f->tid = t;
      f->wg = p;
      getcontext(&f->ctx);
      f->ctx.uc_stack.ss_sp = &stacks[((size_t)p * sb + t) * stack];
      f->ctx.uc_stack.ss_size = stack;
      f->ctx.uc_link = nullptr;
      makecontext(&f->ctx, entry, 0);
      g_fibers.push_back(f);
    }
  std::vector<Fiber*> sweep(g_fibers);
  if (order == 1) std::reverse(sweep.begin(), sweep.end());
  std::mt19937 shuf(seed ^ 0x9E3779B9u);
  size_t live = sweep.size();
  while (live) {
    live = 0;
    if (order == 2) std::shuffle(sweep.begin(), sweep.end(), shuf);
    for (auto* f : sweep) {
      if (f->done) continue;
      g_cur = f;
      swapcontext(&g_main, &f->ctx);
      if (!f->done) ++live;
    }
  }
  for (auto* f : g_fibers) delete f;
  g_fibers.clear();
}
// to be called by a fiber's entry function when its body returns
inline void fiber_exit() {
  g_cur->done = true;
  swapcontext(&g_cur->ctx, &g_main);
}
}  // namespace emu
