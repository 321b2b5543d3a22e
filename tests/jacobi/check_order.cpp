// Host checker of the Jacobi pair order (csrc/jacobi_order.h) for every even
// number of columns up to 128: each round uses a column at most once, every
// pair of columns meets exactly once per sweep, round 0 holds every column
// (the kernel reads the final norms from the round-0 holders), a sweep has at
// most mp rounds (the kernel's schedule table holds mp * mp / 2 entries), and
// the columns that change units per round stay near one per unit for the
// widths the subspace iterations use.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "jacobi_order.h"

static int fails = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      std::fprintf(stderr, __VA_ARGS__);  \
      std::fprintf(stderr, "\n");         \
      ++fails;                            \
    }                                     \
  } while (0)

int main() {
  for (int mp = 2; mp <= 128; mp += 2) {
    const int h = mp / 2, R = ritz_rounds(mp);
    CHECK(R >= mp - 1 && R <= mp, "mp %d: %d rounds (table holds at most mp)", mp, R);
    std::vector<int> met((size_t)mp * mp, 0);
    long moves = 0, active = 0;
    for (int ri = 0; ri < R; ++ri) {
      std::vector<int> used(mp, 0);
      for (int u = 0; u < h; ++u) {
        int a, b;
        ritz_assign(mp, ri, u, a, b);
        if (a < 0) continue;
        if (a >= mp || b < 0 || b >= mp || a == b) {
          CHECK(false, "mp %d round %d unit %d: bad pair (%d, %d)", mp, ri, u, a, b);
          continue;
        }
        CHECK(!used[a] && !used[b], "mp %d round %d: column %d or %d used twice", mp, ri, a, b);
        used[a] = used[b] = 1;
        ++met[(size_t)(a < b ? a : b) * mp + (a < b ? b : a)];
        int na, nb;
        ritz_assign(mp, ri + 1 < R ? ri + 1 : 0, u, na, nb);
        moves += (na >= 0 && na != a && na != b) + (nb >= 0 && nb != a && nb != b);
        ++active;
      }
      if (ri == 0)
        for (int c = 0; c < mp; ++c) CHECK(used[c], "mp %d: column %d not held in round 0", mp, c);
    }
    for (int p = 0; p < mp; ++p)
      for (int q = p + 1; q < mp; ++q)
        CHECK(met[(size_t)p * mp + q] == 1, "mp %d: pair (%d, %d) met %d times", mp, p, q, met[(size_t)p * mp + q]);
    const double per = active ? (double)moves / active : 0.0;
    if (mp == 64 || mp == 96 || mp == 128) {
      CHECK(per <= 1.1, "mp %d: %.2f arriving columns per unit and round", mp, per);
      std::printf("mp %3d: %3d rounds, %.2f arriving columns per unit and round\n", mp, R, per);
    }
  }
  if (fails) {
    std::fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  std::printf("jacobi order checks passed\n");
  return 0;
}
