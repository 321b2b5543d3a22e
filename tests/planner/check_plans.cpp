// Host-only checks of the library's planner (csrc/planner.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_planner.py.
//
// Each plan is replayed against a model of what its launches compute, at the
// granularity the kernels work in:
//   - Hessian: every output tile's token slices partition the padded token
//     range, every 64x64 block of the output is reduced exactly once, from the
//     partials of its own tile;
//   - factor: every trailing update applies each panel's contribution to
//     each lower 64x64 block of L exactly once and only after that panel is
//     final, every panel step finds its blocks fully updated, and the same
//     for the blocked forward substitution that builds Y = L^{-1};
//   - quantise: every column receives the errors of all earlier columns
//     exactly once, in order, before its super-block is swept; the appended
//     (never rounded) columns end with all of them; error-buffer halves are
//     read only while they hold the super-block the update expects;
//   - streams: nothing on the main stream touches what a launch on the
//     second stream writes (or writes what it reads) between the fork that
//     starts it and the join that ends it.
// Tile counts (nwg) are checked against the shapes the kernels enumerate.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>
#include <vector>

#include "planner.h"

static int g_fail = 0;
static std::string g_case;
#define CHECK(cond, ...)                                                         \
  do {                                                                           \
    if (!(cond)) {                                                               \
      fprintf(stderr, "FAIL [%s] %s:%d: ", g_case.c_str(), __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                                              \
      fputc('\n', stderr);                                                       \
      if (++g_fail > 25) exit(1);                                                \
    }                                                                            \
  } while (0)

// ------------------------------------------------------------- streams -----
// An access to [lo, hi) of resource res of problem p.
struct Acc {
  int p, res;
  long long lo, hi;
  bool write;
};
static bool overlap(const Acc& a, const Acc& b) {
  return a.p == b.p && a.res == b.res && a.lo < b.hi && b.lo < a.hi;
}
struct Streams {
  std::vector<Acc> side;  // accesses of side launches since the last join
  bool forked = false;
  void fork() { forked = true; }
  void join() {
    side.clear();
    forked = false;
  }
  void launch(bool on_side, const std::vector<Acc>& acc, const char* what) {
    if (on_side) {
      CHECK(forked, "%s on the second stream without a fork", what);
      side.insert(side.end(), acc.begin(), acc.end());
      return;
    }
    for (const Acc& a : acc)
      for (const Acc& s : side)
        if ((a.write || s.write) && overlap(a, s)) {
          CHECK(false, "%s (main) %s res %d [%lld,%lld) of problem %d that a pending side launch %s", what,
                a.write ? "writes" : "reads", a.res, a.lo, a.hi, a.p, s.write ? "writes" : "reads");
          return;
        }
  }
};

// ------------------------------------------------------------- Hessian -----
static void check_hessian(const std::vector<HessJob>& jobs, bool use_xt) {
  std::vector<uint16_t> xt(use_xt ? std::max<size_t>(hess_xt_elems(jobs), 1) : 0);
  HessPlan P;
  plan_hessian(jobs, 256, 8, use_xt ? xt.data() : nullptr, P);
  const int np = (int)jobs.size();
  CHECK((int)P.probs.size() == np && (int)P.rprobs.size() == np && (int)P.xprobs.size() == np, "per-job records");
  CHECK(P.nparts == (int)P.tasks.size(), "nparts");
  for (size_t i = 0; i < P.tasks.size(); ++i) CHECK(P.tasks[i].part == (int)i, "task %zu writes partial %d", i,
                                                    P.tasks[i].part);
  // transposed copies: inside the buffer, one segment each
  size_t xt_end = 0;
  for (int p = 0; p < np; ++p) {
    const HessJob& J = jobs[p];
    const bool direct = hess_direct(J);
    CHECK(P.probs[p].direct == (direct ? 1 : 0), "job %d direct flag", p);
    if (!direct && J.tokens > 0) {
      CHECK(use_xt, "job %d needs a transposed copy", p);
      const XposeProb& x = P.xprobs[p];
      const size_t off = (size_t)(x.Xt - xt.data());
      CHECK(off >= xt_end && off + (size_t)x.n_pad * x.ldt <= xt.size(), "job %d copy outside the buffer", p);
      xt_end = off + (size_t)x.n_pad * x.ldt;
      CHECK(x.ldt >= x.t_pad && x.t_pad >= J.tokens && x.n_pad >= J.n, "job %d copy shape", p);
    }
  }
  int nx = 0;
  for (const Seg& s : P.xsegs) {
    const XposeProb& x = P.xprobs[s.prob];
    CHECK(s.nwg == (x.t_pad / 64) * (x.n_pad / 64), "copy segment of job %d: %d workgroups", s.prob, s.nwg);
    CHECK(s.wg0 == nx, "copy segment offsets");
    nx += s.nwg;
  }
  for (int p = 0; p < np; ++p) {
    const HessJob& J = jobs[p];
    const bool full = J.Y != nullptr;
    const int nt = cdiv(J.n, 256);
    const long long t_pad = cdiv64(J.tokens, 64) * 64;
    // tasks of this job, by tile
    std::vector<std::vector<std::pair<int, int>>> ranges(nt * nt);
    for (const SyrkTask& t : P.tasks) {
      if (t.prob != p) continue;
      CHECK(t.ti >= 0 && t.ti < nt && t.tj >= 0 && t.tj < nt && (full || t.ti <= t.tj), "job %d task tile (%d,%d)", p,
            t.ti, t.tj);
      CHECK(t.k0 % 32 == 0 && t.k1 % 32 == 0 && t.k0 < t.k1, "job %d task range [%d,%d)", p, t.k0, t.k1);
      ranges[t.ti * nt + t.tj].push_back({t.k0, t.k1});
    }
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = full ? 0 : ti; tj < nt; ++tj) {
        auto r = ranges[ti * nt + tj];
        std::sort(r.begin(), r.end());
        if (J.tokens == 0) {
          CHECK(r.empty(), "job %d: tasks without tokens", p);
          continue;
        }
        long long at = 0;
        for (auto& q : r) {
          CHECK(q.first == at, "job %d tile (%d,%d): token slices leave a gap or overlap at %lld", p, ti, tj, at);
          at = q.second;
        }
        CHECK(at == t_pad, "job %d tile (%d,%d): slices end at %lld, not %lld", p, ti, tj, at, t_pad);
      }
    // reductions: every 64-block of the output once
    const int nb = cdiv(J.n, 64);
    std::vector<int> seen(nb * nb, 0);
    for (const RedTask& r : P.rtasks) {
      if (r.prob != p) continue;
      CHECK(r.r0 % 64 == 0 && r.c0 % 64 == 0 && r.r0 < J.n && r.c0 < J.n && (full || r.r0 <= r.c0),
            "job %d reduction block (%d,%d)", p, r.r0, r.c0);
      seen[(r.r0 / 64) * nb + r.c0 / 64]++;
      long long covered = 0;
      for (int q = 0; q < r.nparts; ++q) {
        const int idx = r.part0 + q;
        CHECK(idx >= 0 && idx < (int)P.partlist.size(), "partial list index");
        const SyrkTask& t = P.tasks[P.partlist[idx]];
        CHECK(t.prob == p && t.ti == r.r0 / 256 && t.tj == r.c0 / 256, "job %d block (%d,%d) sums a foreign partial",
              p, r.r0, r.c0);
        covered += t.k1 - t.k0;
      }
      CHECK(covered == (J.tokens > 0 ? t_pad : 0), "job %d block (%d,%d) sums %lld of %lld tokens", p, r.r0, r.c0,
            covered, t_pad);
    }
    for (int i = 0; i < nb; ++i)
      for (int j = full ? 0 : i; j < nb; ++j) CHECK(seen[i * nb + j] == 1, "job %d block (%d,%d) reduced %d times", p,
                                                    i, j, seen[i * nb + j]);
  }
}

static void check_hessian64(int n, long long tokens) {
  Hess64Plan P;
  plan_hessian64(n, tokens, 256, P);
  const int nt = cdiv(n, 128), nb = cdiv(n, 64);
  const long long t_pad = cdiv64(tokens, 64) * 64;
  std::vector<int> seen(nb * nb, 0);
  for (const RedTask& r : P.rtasks) {
    CHECK(r.r0 <= r.c0 && r.r0 < n && r.c0 < n, "fp64 reduction block");
    seen[(r.r0 / 64) * nb + r.c0 / 64]++;
    long long covered = 0;
    for (int q = 0; q < r.nparts; ++q) {
      const SyrkTask& t = P.tasks[P.partlist[r.part0 + q]];
      CHECK(t.ti == r.r0 / 128 && t.tj == r.c0 / 128 && t.ti <= t.tj && t.tj < nt, "fp64 foreign partial");
      CHECK(t.part == P.partlist[r.part0 + q], "fp64 partial slot");
      covered += t.k1 - t.k0;
    }
    CHECK(covered == (tokens > 0 ? t_pad : 0), "fp64 block (%d,%d) sums %lld tokens", r.r0, r.c0, covered);
  }
  for (int i = 0; i < nb; ++i)
    for (int j = i; j < nb; ++j) CHECK(seen[i * nb + j] == 1, "fp64 block (%d,%d) reduced %d times", i, j,
                                       seen[i * nb + j]);
}

// -------------------------------------------------------------- factor -----
// L: lower 64-blocks (I >= J) with a count per contributing K-block t < J;
// Y: blocks (I > J) with a count per t in [J, I).  Resources for the stream
// check: 0 = L block I * nb + J, 1 = Y block I * nb + J, 2 = the problem's
// stored diagonal chain (k_chol_diag2 -> k_chol_panel2).
struct FacState {
  int n, nb;
  bool filled = false;
  std::vector<uint8_t> cl, cy;  // [I][J][t]
  std::vector<bool> finL, finY;
  int diag_k = -1;  // pair whose diagonal chain is stored (FK_DIAG2)
  explicit FacState(int n_) : n(n_), nb(cdiv(n_, 64)) {
    cl.assign((size_t)nb * nb * nb, 0);
    cy.assign((size_t)nb * nb * nb, 0);
    finL.assign(nb, false);
    finY.assign(nb, false);
  }
  uint8_t& L(int I, int J, int t) { return cl[((size_t)I * nb + J) * nb + t]; }
  uint8_t& Y(int I, int J, int t) { return cy[((size_t)I * nb + J) * nb + t]; }
};

static void add_blocks(std::vector<Acc>& acc, int p, int res, int nb, int I0, int I1, int J0, int J1, bool w) {
  for (int I = I0; I < I1; ++I) acc.push_back(Acc{p, res, (long long)I * nb + J0, (long long)I * nb + J1, w});
}

static void panel_step(FacState& F, int p, int k, bool pair, std::vector<Acc>& acc) {
  const int nb = F.nb, kk = pair ? 2 : 1;
  CHECK(F.filled, "problem %d panel before its matrix is filled", p);
  CHECK(!pair || k + 1 < nb, "problem %d pair step at the last block", p);
  for (int c = k; c < k + kk; ++c)
    for (int I = c; I < nb; ++I)
      for (int t = 0; t < c; ++t) {
        const int want = (pair && c == k + 1 && t == k) ? 0 : 1;
        CHECK(F.L(I, c, t) == want, "problem %d step %d: L(%d,%d) has panel %d applied %d times", p, k, I, c, t,
              F.L(I, c, t));
      }
  for (int r = k; r < k + kk; ++r)
    for (int J = 0; J < k; ++J)
      for (int t = J; t < r; ++t) {
        const int want = (pair && r == k + 1 && t == k) ? 0 : 1;
        CHECK(F.Y(r, J, t) == want, "problem %d step %d: Y(%d,%d) has term %d applied %d times", p, k, r, J, t,
              F.Y(r, J, t));
      }
  if (pair) {
    for (int I = k + 1; I < nb; ++I) F.L(I, k + 1, k) = 1;
    for (int J = 0; J < k; ++J) F.Y(k + 1, J, k) = 1;
  }
  for (int c = k; c < k + kk; ++c) F.finL[c] = true;
  for (int r = k; r < k + kk; ++r) F.finY[r] = true;
  const int P1b = std::min(cdiv(F.n, 64), ((k * 64) / 256 + 1) * 4);
  add_blocks(acc, p, 0, nb, k, nb, k, k + kk, true);
  add_blocks(acc, p, 1, nb, k, k + kk, 0, std::max(P1b, k + kk), true);  // with the zero fill to the outer panel
}

static void fac_gemm(FacState& F, int p, const Seg& s, int TS, std::vector<Acc>& acc) {
  const int n = F.n, nb = F.nb;
  if (s.a == GK_CHOL_TRAIL) {
    const int kb0 = s.b, kw = s.c, c0 = s.d, c1 = s.e;
    const int nrow = cdiv(n - c0, TS), ncol = cdiv(c1 - c0, TS);
    CHECK(s.nwg == nrow * ncol - ncol * (ncol - 1) / 2, "problem %d trailing update: %d tiles, expected %d", p, s.nwg,
          nrow * ncol - ncol * (ncol - 1) / 2);
    CHECK(kb0 % 64 == 0 && c0 % 64 == 0 && kb0 + kw <= c0 && c1 <= n, "problem %d trailing update ranges", p);
    const int t0 = kb0 / 64, t1 = cdiv(kb0 + kw, 64);
    for (int t = t0; t < t1; ++t) CHECK(F.finL[t], "problem %d update reads panel %d before it is final", p, t);
    for (int J = c0 / 64; J < cdiv(c1, 64); ++J)
      for (int I = J; I < nb; ++I)
        for (int t = t0; t < t1; ++t) {
          CHECK(F.L(I, J, t) == 0, "problem %d: panel %d applied twice to L(%d,%d)", p, t, I, J);
          F.L(I, J, t) = 1;
        }
    add_blocks(acc, p, 0, nb, c0 / 64, nb, c0 / 64, cdiv(c1, 64), true);
    add_blocks(acc, p, 0, nb, c0 / 64, nb, t0, t1, false);
  } else if (s.a == GK_ZUPD) {
    const int kb0 = s.b, kw = s.c, r0 = s.d, r1 = s.e;
    CHECK(s.nwg == cdiv(r1 - r0, TS) * cdiv(kb0 + kw, TS), "problem %d Y update: %d tiles", p, s.nwg);
    CHECK(kb0 % 64 == 0 && r0 % 64 == 0 && kb0 + kw <= r0 && r1 <= n, "problem %d Y update ranges", p);
    const int t0 = kb0 / 64, t1 = cdiv(kb0 + kw, 64);
    for (int t = t0; t < t1; ++t) CHECK(F.finL[t] && F.finY[t], "problem %d Y update reads block row %d early", p, t);
    for (int I = r0 / 64; I < cdiv(r1, 64); ++I)
      for (int J = 0; J < t1; ++J) {
        if (J >= t0)  // first write of these columns
          for (int t = 0; t < nb; ++t) CHECK(F.Y(I, J, t) == 0, "problem %d: Y(%d,%d) overwritten", p, I, J);
        for (int t = std::max(t0, J); t < t1; ++t) {
          CHECK(F.Y(I, J, t) == 0, "problem %d: term %d applied twice to Y(%d,%d)", p, t, I, J);
          F.Y(I, J, t) = 1;
        }
      }
    add_blocks(acc, p, 1, nb, r0 / 64, cdiv(r1, 64), 0, t1, true);
    add_blocks(acc, p, 0, nb, r0 / 64, cdiv(r1, 64), t0, t1, false);
    add_blocks(acc, p, 1, nb, t0, t1, 0, t1, false);
  } else {
    CHECK(false, "problem %d: unexpected product kind %d in the factor", p, s.a);
  }
}

static void check_factor(const std::vector<FacShape>& jobs, int ncu = 256) {
  const std::vector<PlanLaunch> L = plan_factor(jobs, ncu);
  std::vector<FacState> F;
  for (const FacShape& j : jobs) F.emplace_back(j.n);
  for (size_t p = 0; p < jobs.size(); ++p) F[p].filled = !jobs[p].fill;
  Streams st;
  bool made = false;
  for (const PlanLaunch& l : L) {
    if (l.kind == PL_FORK) {
      st.fork();
      continue;
    }
    if (l.kind == PL_JOIN) {
      st.join();
      continue;
    }
    int wg = 0;
    for (const Seg& s : l.segs) {
      CHECK(s.wg0 == wg && s.nwg > 0, "segment offsets");
      wg += s.nwg;
    }
    CHECK(wg == l.nwg, "launch workgroups");
    std::vector<Acc> acc;
    for (const Seg& s : l.segs) {
      FacState& f = F[s.prob];
      const int nb = f.nb;
      switch (l.kind) {
        case FK_FILL:
          CHECK(s.nwg == cdiv(f.n, 4), "fill tiles");
          f.filled = true;
          add_blocks(acc, s.prob, 0, nb, 0, nb, 0, nb, true);
          break;
        case FK_DIAG2: {
          // the pair's diagonal region must have every earlier update
          const int k = s.a;
          CHECK(s.nwg == 1 && k + 1 < nb, "problem %d diagonal chain launch", s.prob);
          for (int I = k; I < k + 2 && I < nb; ++I)
            for (int c = k; c <= I; ++c)
              for (int t = 0; t < c; ++t) {
                const int want = (c == k + 1 && t == k) ? 0 : 1;
                CHECK(f.L(I, c, t) == want, "problem %d diagonal chain %d: L(%d,%d) has panel %d applied %d times",
                      s.prob, k, I, c, t, f.L(I, c, t));
              }
          f.diag_k = k;
          add_blocks(acc, s.prob, 0, nb, k, std::min(k + 2, nb), k, std::min(k + 2, nb), false);
          acc.push_back(Acc{s.prob, 2, 0, 1, true});
          break;
        }
        case FK_PANEL:
        case FK_PANEL2:
          CHECK(s.nwg == nb, "panel workgroups");
          if (l.kind == FK_PANEL2 && s.b != 0) {
            CHECK(f.diag_k == s.a, "problem %d panel %d reads the diagonal chain of step %d", s.prob, s.a, f.diag_k);
            acc.push_back(Acc{s.prob, 2, 0, 1, false});
          }
          panel_step(f, s.prob, s.a, l.kind == FK_PANEL2, acc);
          break;
        case FK_GEMM64:
        case FK_RING64:
          fac_gemm(f, s.prob, s, 64, acc);
          CHECK(l.kind == FK_GEMM64 || f.n % 64 == 0, "ring product on n %% 64 != 0");
          break;
        case FK_RING128:
          fac_gemm(f, s.prob, s, 128, acc);
          CHECK(f.n % 64 == 0, "ring product on n %% 64 != 0");
          break;
        case FK_MAKEU:
          for (int b = 0; b < nb; ++b) CHECK(f.finL[b] && f.finY[b], "problem %d: U made before block %d is final",
                                             s.prob, b);
          add_blocks(acc, s.prob, 1, nb, 0, nb, 0, nb, false);
          made = true;
          break;
        default:
          CHECK(false, "unknown factor launch kind %d", l.kind);
      }
    }
    st.launch(l.side, acc, "factor launch");
  }
  CHECK(made && !st.forked, "factor ends with U made and the streams joined");
}

// ------------------------------------------------------------- quantise -----
// Resources: 0 = columns of the working weights, 1 = error-buffer half.
static void check_quantize(const std::vector<QuantShape>& jobs) {
  QuantLayout Ly;
  std::vector<PlanLaunch> L;
  plan_quantize(jobs, &Ly, &L);
  const int nl = (int)jobs.size();
  CHECK((int)Ly.sbk.size() == nl, "layout size");
  // buffer offsets: disjoint and inside the totals
  for (int p = 0; p < nl; ++p) {
    const QuantShape& J = jobs[p];
    const int sbw = Ly.sbk[p] * J.block;
    CHECK(J.group == 0 || sbw % J.group == 0 || J.group % sbw == 0 || Ly.sbk[p] == 1, "groups nest");
    CHECK(Ly.oE[p] + 2 * (size_t)J.out * sbw <= Ly.totE, "error buffer of layer %d", p);
    CHECK(J.ext_ww || Ly.oW[p] + (size_t)J.out * J.nt <= Ly.totW, "working weights of layer %d", p);
    CHECK(Ly.oO[p] + 2 * (size_t)J.out <= Ly.totO && Ly.oD[p] + (size_t)J.nt <= Ly.totD, "sums of layer %d", p);
    if (p > 0) CHECK(Ly.oE[p] >= Ly.oE[p - 1] + 2 * (size_t)jobs[p - 1].out * Ly.sbk[p - 1] * jobs[p - 1].block,
                     "error buffers overlap");
  }
  std::vector<std::vector<int>> applied(nl);  // per column: errors [0, applied) applied; -1 once swept
  std::vector<std::vector<bool>> swept(nl);
  std::vector<int> holder(2 * nl, -1);
  std::vector<bool> inited(nl, false), fitted(nl, false);
  for (int p = 0; p < nl; ++p) {
    applied[p].assign(jobs[p].nt, 0);
    swept[p].assign(jobs[p].n, false);
  }
  Streams st;
  for (const PlanLaunch& l : L) {
    if (l.kind == PL_FORK) {
      st.fork();
      continue;
    }
    if (l.kind == PL_JOIN) {
      st.join();
      continue;
    }
    int wg = 0;
    for (const Seg& s : l.segs) {
      CHECK(s.wg0 == wg && s.nwg > 0, "segment offsets");
      wg += s.nwg;
    }
    CHECK(wg == l.nwg, "launch workgroups");
    std::vector<Acc> acc;
    for (const Seg& s : l.segs) {
      const int p = s.prob;
      const QuantShape& J = jobs[p];
      const int sbw = Ly.sbk[p] * J.block;
      switch (l.kind) {
        case QK_INIT:
          CHECK(s.nwg == cdiv(J.out, 4), "init tiles");
          inited[p] = true;
          acc.push_back(Acc{p, 0, 0, J.nt, true});
          break;
        case QK_ROWFIT:
          CHECK(J.group == 0 && J.mode == 0 && s.nwg == cdiv(J.out, 4), "row fit");
          fitted[p] = true;
          break;
        case QK_SWEEP: {
          CHECK(l.block == J.block && l.mode == J.mode, "layer %d swept with block %d mode %d", p, l.block, l.mode);
          CHECK(s.nwg == cdiv(J.out, 16), "sweep tiles");
          CHECK(inited[p] && (J.group != 0 || J.mode != 0 || fitted[p]), "layer %d swept before its setup", p);
          const int sb0 = s.a * sbw, sb1 = std::min(sb0 + sbw, J.n);
          CHECK(sb0 < J.n, "layer %d super-block %d past the columns", p, s.a);
          for (int j = sb0; j < sb1; ++j) {
            CHECK(applied[p][j] == sb0, "layer %d column %d swept with errors [0,%d) applied, not [0,%d)", p, j,
                  applied[p][j], sb0);
            applied[p][j] = -1;
            swept[p][j] = true;
          }
          holder[2 * p + (s.a & 1)] = s.a;
          acc.push_back(Acc{p, 0, sb0, sb1, true});
          acc.push_back(Acc{p, 1, s.a & 1, (s.a & 1) + 1, true});
          break;
        }
        case QK_TRAIL: {
          const int TS = l.block, e0 = s.b, ew = s.c, c0 = s.d, c1 = s.e;
          CHECK(TS == 64 || TS == 128, "trail tile %d", TS);
          CHECK(s.nwg == cdiv(J.out, TS) * cdiv(c1 - c0, TS), "layer %d trail: %d tiles", p, s.nwg);
          const long long half_sz = (long long)J.out * sbw;
          CHECK(s.a % half_sz == 0 && s.a / half_sz < 2, "layer %d trail: error offset %d", p, s.a);
          const int half = (int)(s.a / half_sz);
          CHECK(e0 % sbw == 0 && ew == std::min(sbw, J.n - e0), "layer %d trail: errors [%d,+%d)", p, e0, ew);
          CHECK(holder[2 * p + half] == e0 / sbw, "layer %d trail reads half %d holding super-block %d, not %d", p,
                half, holder[2 * p + half], e0 / sbw);
          for (int j = e0; j < e0 + ew; ++j) CHECK(swept[p][j], "layer %d trail uses unswept column %d", p, j);
          CHECK(c0 >= e0 + ew && c1 <= J.nt && c0 < c1, "layer %d trail columns [%d,%d)", p, c0, c1);
          for (int j = c0; j < c1; ++j) {
            CHECK(applied[p][j] == e0, "layer %d column %d gets errors [%d,%d) after [0,%d)", p, j, e0, e0 + ew,
                  applied[p][j]);
            applied[p][j] = e0 + ew;
          }
          acc.push_back(Acc{p, 0, c0, c1, true});
          acc.push_back(Acc{p, 1, half, half + 1, false});
          break;
        }
        default:
          CHECK(false, "unknown quantise launch kind %d", l.kind);
      }
    }
    st.launch(l.side, acc, "quantise launch");
  }
  CHECK(!st.forked, "quantise ends with the streams joined");
  for (int p = 0; p < nl; ++p) {
    for (int j = 0; j < jobs[p].n; ++j) CHECK(swept[p][j], "layer %d column %d never swept", p, j);
    for (int j = jobs[p].n; j < jobs[p].nt; ++j)
      CHECK(applied[p][j] == jobs[p].n, "layer %d appended column %d ends with errors [0,%d)", p, j, applied[p][j]);
  }
}

// -------------------------------------------------------------- configs -----
struct Layer {
  const char* name;
  int out, n, tokens, bits, group, block;
};

static const uint16_t* fake_ptr(size_t off) {
  // an address used only for its alignment and as an opaque value
  static uint16_t base[64] __attribute__((aligned(256)));
  return base + off;
}

static void run_layer_set(const char* name, const std::vector<Layer>& layers, int r, bool shared_x) {
  g_case = name;
  std::vector<HessJob> hj;
  std::vector<FacShape> fj;
  std::vector<QuantShape> qj;
  for (size_t i = 0; i < layers.size(); ++i) {
    const Layer& y = layers[i];
    if (!(shared_x && i > 0)) {
      hj.push_back(HessJob{fake_ptr(0), y.tokens, y.n, y.n, nullptr, 0});
      fj.push_back(FacShape{y.n + r, r == 0});
    }
    qj.push_back(QuantShape{y.out, y.n, y.n + r, y.block, y.group, 0, r > 0});
  }
  check_hessian(hj, true);
  check_factor(fj);
  check_quantize(qj);
}

int main() {
  // the five workloads' shapes
  run_layer_set("single", {{"single", 256, 512, 1024, 4, 0, 128}}, 0, false);
  run_layer_set("square", {{"square", 4096, 4096, 262144, 4, 128, 128}}, 0, false);
  run_layer_set("mlp", {{"gate", 6144, 2048, 262144, 3, 128, 128}, {"up", 6144, 2048, 262144, 3, 128, 128}}, 0,
                true);
  run_layer_set("mlp-down", {{"down", 2048, 6144, 262144, 3, 128, 128}}, 0, false);
  run_layer_set("lora", {{"lora", 2048, 2048, 65536, 3, 0, 128}}, 64, false);
  {
    std::vector<Layer> vit;
    for (int b = 0; b < 12; ++b) {
      vit.push_back({"qkv", 2304, 768, 50176, 2, 64, 64});
      vit.push_back({"proj", 768, 768, 50176, 2, 64, 64});
      vit.push_back({"fc1", 3072, 768, 50176, 2, 64, 64});
      vit.push_back({"fc2", 768, 3072, 50176, 2, 64, 64});
    }
    run_layer_set("vit", vit, 0, false);
  }
  // ragged and edge shapes
  run_layer_set("ragged", {{"a", 203, 520, 3001, 4, 0, 128}, {"b", 77, 640, 6001, 4, 128, 16},
                           {"c", 96, 200, 2048, 3, 8, 32}, {"d", 5, 37, 700, 4, 0, 16}},
                0, false);
  run_layer_set("lora-ragged", {{"l96", 160, 400, 8192, 3, 0, 128}}, 96, false);
  run_layer_set("group-not-nesting", {{"g192", 64, 1152, 4096, 4, 192, 64}}, 0, false);
  run_layer_set("group-over-sb", {{"g1024", 64, 2048, 4096, 4, 1024, 128}}, 0, false);
  g_case = "bid-up";
  check_quantize({QuantShape{160, 384, 384, 128, 0, 1, false}, QuantShape{96, 200, 200, 16, 8, 1, false}});
  g_case = "hessian-layouts";
  check_hessian({HessJob{fake_ptr(1), 3001, 523, 520, nullptr, 0}, HessJob{fake_ptr(0), 0, 64, 64, nullptr, 1},
                 HessJob{fake_ptr(0), 999, 30, 30, nullptr, 0}, HessJob{fake_ptr(0), 2048, 304, 300, nullptr, 0}},
                true);
  check_hessian({HessJob{fake_ptr(0), 5000, 1000, 1000, nullptr, 0, fake_ptr(0)}}, true);  // cross Gram
  g_case = "hessian64";
  for (int n : {37, 64, 300, 2048, 4096})
    for (long long t : {0LL, 1LL, 999LL, 65536LL}) check_hessian64(n, t);
  g_case = "factor-mixed";
  check_factor({FacShape{4096, true}, FacShape{768, true}, FacShape{3072, true}, FacShape{200, true}});
  check_factor({FacShape{100, true}, FacShape{37, true}});
  // small chips: every pair step with more panel workgroups than CUs runs its
  // diagonal chains first
  g_case = "factor-diag-split";
  check_factor({FacShape{4096, true}, FacShape{768, true}, FacShape{3072, true}, FacShape{200, true}}, 8);
  check_factor({FacShape{4096, true}}, 32);
  check_factor({FacShape{100, true}, FacShape{37, true}, FacShape{520, false}}, 1);
  if (g_fail) {
    fprintf(stderr, "%d planner check(s) failed\n", g_fail);
    return 1;
  }
  printf("planner checks passed\n");
  return 0;
}
