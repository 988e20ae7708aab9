// Runs the decode row kernel (k_rows of decode.hip, its own source) on the
// CPU for one query row split over P workgroups of 1024 threads, every thread
// a fiber (emu_fibers.h, emu_device.h). The kernel's source is included as
// rows_kernel.inc, cut from decode.hip by the test with its __shared__
// declarations turned into per-workgroup storage. Test infrastructure only.
//
// usage: rows_emu SPT in.bin out.bin [order] [mode]
//   mode   : 0 the default build; the build that takes the attention flags
//            with 1 none set, 2 the integer-only softmax, 3 reading B
//   in.bin : int64 N T m P klow khigh, then f32 U[N], u32 low[T][3],
//            u32 kc[T][16], u32 vc[T][16]
//   out.bin: f32 s_low[T], i32 sel[m], f32 s_high[m], u16 wpart[P][N],
//            f32 stats[P][4], i32 p_int[m], u32 status, u32 cross-workgroup
//            barrier arrivals
#include <cstdio>
#include <cstdlib>
#include <map>
#include <utility>
#include <vector>

#include "sdkv_device.h"  // the emulation header, copied under this name
#include "emu_fibers.h"
#include "select_core.h"

namespace emu {
template <class T>
struct Box {
  T v;
};
// per-workgroup storage of one __shared__ declaration, filled with a byte
// pattern (LDS starts with unspecified contents)
template <class T>
T& wg_shared(int id) {
  static std::map<std::pair<unsigned, int>, Box<T>*> m;
  Box<T>*& b = m[{bid3().x, id}];
  if (!b) {
    b = new Box<T>;
    memset((void*)&b->v, 0xA5, sizeof(T));
  }
  return b->v;
}
}  // namespace emu

namespace sdkv {
// the planner's constants (sdkv_internal.h); the 32-key instance is built
// with the cross-workgroup select here
constexpr int kRowThreads = 1024;
constexpr int kMaxRowSPT = 32;
constexpr int kMaxCoopSPT = 32;
constexpr int kMaxRowP = 64;
constexpr int kMaxAtomsDecode = 32768;
#include "rows_kernel.inc"
}  // namespace sdkv

using namespace sdkv;

static RowsArgs g_args;
static int g_spt = 16;

template <int SPT, bool EXT>
static void fiber_entry() {
  k_rows<SPT, true, EXT>(g_args);
  emu::fiber_exit();
}

template <class T>
static void read_arr(FILE* f, std::vector<T>& v, size_t n) {
  v.resize(n);
  if (fread(v.data(), sizeof(T), n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
}

int main(int argc, char** argv) {
  if (argc < 4) {
    fprintf(stderr, "usage: %s SPT in.bin out.bin [order]\n", argv[0]);
    return 2;
  }
  g_spt = atoi(argv[1]);
  const int order = argc > 4 ? atoi(argv[4]) : 0;
  const int mode = argc > 5 ? atoi(argv[5]) : 0;
  FILE* fi = fopen(argv[2], "rb");
  if (!fi) return 2;
  int64_t h[6];
  if (fread(h, 8, 6, fi) != 6) return 2;
  const int N = (int)h[0], P = (int)h[3], klow = (int)h[4], khigh = (int)h[5];
  const int64_t T = h[1], m = h[2];
  std::vector<float> U;
  std::vector<uint32_t> low, kc, vc;
  read_arr(fi, U, N);
  read_arr(fi, low, (size_t)T * 3);
  read_arr(fi, kc, (size_t)T * 16);
  read_arr(fi, vc, (size_t)T * 16);
  fclose(fi);
  const int64_t chunk = (T + P - 1) / P;
  if (chunk > (int64_t)SB * g_spt) {
    fprintf(stderr, "chunk %lld exceeds %d keys per workgroup\n", (long long)chunk, SB * g_spt);
    return 2;
  }

  // workspace: words the launcher clears are zero, the rest hold a pattern
  std::vector<float> s_low(T), s_high_out(m);
  std::vector<int32_t> sel_out(m, -1), sel((size_t)P * chunk), p_int(m, 0);
  std::vector<float> s_high((size_t)P * chunk);
  std::vector<uint16_t> wpart((size_t)P * N, 0xA5A5u);
  std::vector<float4> stats(P);
  std::vector<uint32_t> ghist(2048, 0u), wtab((size_t)P * 2048, 0xA5A5A5A5u);
  std::vector<uint32_t> cand((size_t)P * chunk, 0xA5A5A5A5u), xchg(2 * P, 0u), bar(2, 0u);
  std::vector<uint32_t> ticket(8, 0u), ixchg(4 * P, 0u);
  uint32_t err = 0;

  RowsArgs& a = g_args;
  memset((void*)&a, 0, sizeof(a));
  a.U = U.data();
  a.low = low.data();
  a.low_words = 3;
  a.kc = kc.data();
  a.vc = vc.data();
  a.rs = 16;
  a.N = N;
  a.K = 16;
  a.klow = klow;
  a.khigh = khigh;
  a.Hq = a.Hkv = a.G = 1;
  a.P = P;
  a.row0 = 0;
  a.nrows = 1;
  a.T = T;
  a.m = m;
  a.chunk = chunk;
  a.s_low_out = s_low.data();
  a.sel_out = sel_out.data();
  a.s_high_out = s_high_out.data();
  a.sel = sel.data();
  a.s_high = s_high.data();
  a.wpart = wpart.data();
  a.stats = stats.data();
  a.ghist = ghist.data();
  a.wtab = wtab.data();
  a.cand = cand.data();
  a.xchg = xchg.data();
  a.bar = bar.data();
  a.wait = WaitCtl{&err, 1u << 22, 0u};
  a.ticket = ticket.data();
  a.xcd_map = 0;
  a.ixchg = ixchg.data();
  a.imode = mode == 2 ? 1 : 0;
  a.p_int_out = mode == 2 ? p_int.data() : nullptr;
  a.readb = mode == 3 ? 1 : 0;  // value low words from the value records

  void (*entry)() = nullptr;
  if (g_spt == 32) entry = mode ? fiber_entry<32, true> : fiber_entry<32, false>;
  if (g_spt == 16) entry = mode ? fiber_entry<16, true> : fiber_entry<16, false>;
  if (!entry) {
    fprintf(stderr, "SPT must be 16 or 32\n");
    return 2;
  }
  emu::run_fibers(P, SB, entry, order, 12345u);

  FILE* fo = fopen(argv[3], "wb");
  if (!fo) return 2;
  fwrite(s_low.data(), 4, T, fo);
  fwrite(sel_out.data(), 4, m, fo);
  fwrite(s_high_out.data(), 4, m, fo);
  fwrite(wpart.data(), 2, (size_t)P * N, fo);
  fwrite(stats.data(), 16, P, fo);
  fwrite(p_int.data(), 4, m, fo);
  const uint32_t rounds = bar[0] & 0xFFFFu;
  fwrite(&err, 4, 1, fo);
  fwrite(&rounds, 4, 1, fo);
  fclose(fo);
  printf("SPT %d P %d T %lld m %lld mode %d: status %u, barrier arrivals %u\n", g_spt, P,
         (long long)T, (long long)m, mode, err, rounds);
  return 0;
}
