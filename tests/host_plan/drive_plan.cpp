// Prints the inverse's launch plan for each d given on the command line, in
// the order prepare_perm_launch issues the launches: per panel at column c0
// a line "P d c0 items", then (unless it is the last panel) a line "B d c1
// items" for the band launch, then "R d d items" for each round after the
// chain.  items = (s,x,g0,cnt) groups.  Host code only.
#include <cstdio>
#include <cstdlib>

#include "inv_plan.h"

using namespace gptq;

static void put(const char* tag, int d, int c, const InvItems& it) {
  std::printf("%s %d %d", tag, d, c);
  for (int i = 0; i < it.n; ++i) std::printf(" %d,%d,%d,%d", it.s[i], it.x[i], it.g0[i], it.cnt[i]);
  std::printf("\n");
}

int main(int argc, char** argv) {
  for (int a = 1; a < argc; ++a) {
    const int d = std::atoi(argv[a]);
    InvPlan plan(d);
    for (int c0 = 0; c0 < d; c0 += INV_PW) {
      int rest = 0;
      if (c0 > 0 && c0 + INV_PW < d) {
        const int nt = (d - c0 - INV_PW + 127) / 128;
        rest = nt * (nt + 1) / 2;
      }
      put("P", d, c0, inv_panel_items(plan, c0, rest));
      const int c1 = std::min(d, c0 + INV_PW);
      if (c1 < d) put("B", d, c1, inv_band_items(plan, c1));
    }
    int rounds = 0;
    while (!plan.finished()) {
      const InvItems it = plan.take(d, -1.0);
      if (InvPlan::count(it) == 0 || ++rounds > 1000) {
        std::printf("STUCK %d\n", d);
        return 1;
      }
      put("R", d, d, it);
    }
  }
  return 0;
}
