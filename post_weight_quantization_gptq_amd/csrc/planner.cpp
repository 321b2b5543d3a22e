// Host planner (see planner.h): plain C++, no HIP calls.
#include "planner.h"

#include <algorithm>
#include <utility>

// ------------------------------------------------------------ Hessian plan --
// The tiles can read X directly (no transposed copy) when its rows are
// 16-byte aligned and n is a multiple of 8 (16-byte feature chunks never
// cross the end of a row).  A stage's per-lane byte offsets (32 rows of the
// pitch) are 32-bit, which bounds the pitch.
bool hess_direct(const HessJob& J) {
  return J.tokens > 0 && (J.ldx % 8) == 0 && (((uintptr_t)J.X) & 15) == 0 && (J.n % 8) == 0 &&
         J.ldx < (1LL << 25);
}

// Interleaved bit order of (i, j): tiles close in this order share rows of X.
static int morton2(int i, int j) {
  int m = 0;
  for (int b = 0; b < 10; ++b) m |= (((i >> b) & 1) << (2 * b + 1)) | (((j >> b) & 1) << (2 * b));
  return m;
}

// Number of token slices for one layer's tiles: whole rounds of the chip at
// one tile per CU, each task also paying for writing its partial (about ten
// 32-token steps of time), and the reduction reading every partial back
// (256 KB each, about 1/19 of a step of the chip's time at HBM speed).
// Depends on the layer alone, so a layer gets the same bits alone or batched.
static int hess_slices(int ntile, long long chunks, int ncu) {
  int best_s = 1;
  long long best = -1;
  for (int s = 1; s <= 64 && s <= std::max(1LL, chunks); ++s) {
    const long long rounds = cdiv((long long)ntile * s, (long long)ncu);
    // in 1/19 steps
    const long long cost = 19 * rounds * (cdiv(chunks, (long long)s) + 10) + (long long)s * ntile;
    if (best < 0 || cost < best) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

// Tasks of every layer: its upper 256x256 tiles times S token slices, slice
// by slice, so that the whole chip streams one window of tokens at a time and
// re-reads of X hit the L2/MALL.  Inside a slice the tiles go in Morton order,
// cut into 8 groups that are dealt out in turn: consecutive workgroups land
// on the 8 XCDs in turn, so each XCD works on one compact group of tiles that
// shares rows of X in its own L2.  The cut points of a layer depend on that
// layer alone, so a layer gets the same bits alone or in a batch.  The rows of
// the transposed copy are padded by 256 tokens so that rows at the same token
// offset spread over the L2 channels.
void plan_hessian(const std::vector<HessJob>& jobs, int ncu, int nxcd, uint16_t* xt, HessPlan& P) {
  for (size_t p = 0; p < jobs.size(); ++p) {
    const HessJob& J = jobs[p];
    const int vec = (J.ldx % 8 == 0) && (((uintptr_t)J.X & 15) == 0);
    const int nt = cdiv(J.n, 256);
    const long long chunks = cdiv(J.tokens, 64);
    const int n_pad = nt * 256, t_pad = (int)(chunks * 64);
    if (hess_direct(J)) {
      // the tiles read X itself (transposing LDS reads); no copy
      P.xprobs.push_back(XposeProb{J.X, J.ldx, nullptr, J.n, (int)J.tokens, n_pad, t_pad, vec, 0});
      P.probs.push_back(SyrkProb{J.X, J.ldx, 1, (int)J.tokens, J.n, 0, J.Y});
    } else {
      const int ldt = t_pad > 0 ? t_pad + 256 : 0;
      P.xprobs.push_back(XposeProb{J.X, J.ldx, xt, J.n, (int)J.tokens, n_pad, t_pad, vec, ldt});
      if (t_pad > 0) P.xsegs.push_back(Seg{(int)p, 0, (t_pad / 64) * (n_pad / 64), 0, 0, 0, 0, 0});
      P.probs.push_back(SyrkProb{xt, ldt, 0, (int)J.tokens, J.n, 0, nullptr});
      xt += (size_t)n_pad * ldt;
    }
    const bool full = J.Y != nullptr;
    P.rprobs.push_back(RedProb{J.H, J.n, J.accumulate, full ? 1 : 0, 0});
    if (J.n <= 0) continue;
    std::vector<std::pair<int, int>> tl;  // upper tiles, or every tile of a cross Gram
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = full ? 0 : ti; tj < nt; ++tj) tl.push_back({ti, tj});
    const int ntile = (int)tl.size();
    if (J.tokens > 0) {
      std::vector<std::pair<int, int>> mo = tl;
      std::stable_sort(mo.begin(), mo.end(), [](const std::pair<int, int>& x, const std::pair<int, int>& y) {
        return morton2(x.first, x.second) < morton2(y.first, y.second);
      });
      std::vector<int> ord;  // dealt order, indices into mo
      const int G = std::max(1, std::min(nxcd, ntile)), base = ntile / G, rem = ntile % G;
      for (int idx = 0; idx <= base; ++idx)
        for (int g = 0; g < G; ++g)
          if (idx < base + (g < rem ? 1 : 0)) ord.push_back(g * base + std::min(g, rem) + idx);
      const long long c32 = t_pad / 32;
      const int S = hess_slices(ntile, c32, ncu);
      const int first = (int)P.tasks.size();
      std::vector<int> pos(ntile);  // tile (canonical index) -> position inside a slice
      for (int q = 0; q < ntile; ++q) {
        const std::pair<int, int> t = mo[ord[q]];
        const int ci = full ? t.first * nt + t.second
                            : t.first * nt - t.first * (t.first - 1) / 2 + (t.second - t.first);
        pos[ci] = q;
      }
      for (int sl = 0; sl < S; ++sl) {
        const int k0 = (int)(32 * (c32 * sl / S)), k1 = (int)(32 * (c32 * (sl + 1) / S));
        for (int q = 0; q < ntile; ++q) {
          const std::pair<int, int> t = mo[ord[q]];
          P.tasks.push_back(SyrkTask{(int)p, t.first, t.second, k0, k1, (int)P.tasks.size(), 0, 0});
        }
      }
      for (int ci = 0; ci < ntile; ++ci) {
        const int ti = tl[ci].first, tj = tl[ci].second;
        const int part0 = (int)P.partlist.size();
        for (int sl = 0; sl < S; ++sl) P.partlist.push_back(first + sl * ntile + pos[ci]);
        for (int a = 0; a < 4; ++a)
          for (int b = 0; b < 4; ++b) {
            if (ti == tj && a > b && !full) continue;
            const int r0 = ti * 256 + 64 * a, c0 = tj * 256 + 64 * b;
            if (r0 >= J.n || c0 >= J.n) continue;
            P.rtasks.push_back(RedTask{(int)p, r0, c0, part0, S, 0, 0, 0});
          }
      }
    } else {
      // no tokens: every sub-block sums zero partials (H = 0, or H unchanged)
      for (int ci = 0; ci < ntile; ++ci) {
        const int ti = tl[ci].first, tj = tl[ci].second;
        for (int a = 0; a < 4; ++a)
          for (int b = 0; b < 4; ++b) {
            const int r0 = ti * 256 + 64 * a, c0 = tj * 256 + 64 * b;
            if ((ti == tj && a > b && !full) || r0 >= J.n || c0 >= J.n) continue;
            P.rtasks.push_back(RedTask{(int)p, r0, c0, 0, 0, 0, 0, 0});
          }
      }
    }
  }
  P.nparts = (int)P.tasks.size();
  int nxwg = 0;
  for (auto& sg : P.xsegs) {
    sg.wg0 = nxwg;
    nxwg += sg.nwg;
  }
}

size_t hess_xt_elems(const std::vector<HessJob>& jobs) {
  size_t e = 0;
  for (const HessJob& J : jobs)
    if (J.tokens > 0 && !hess_direct(J)) e += (size_t)cdiv(J.n, 256) * 256 * ((size_t)cdiv(J.tokens, 64) * 64 + 256);
  return e;
}

// One layer's Gram matrix accurate to float64 rounding: 128x128 upper tiles
// on float64 MFMA, each tile split over S token slices (S chosen so that the
// tasks fill whole rounds of the chip), partials summed in slice order.
void plan_hessian64(int n, long long tokens, int ncu, Hess64Plan& P) {
  const long long t_pad = cdiv64(tokens, 64) * 64;
  const int nt = cdiv(n, 128);
  const int ntile = nt * (nt + 1) / 2;
  const long long chunks = t_pad / 32;
  // slices: minimise rounds x slice length
  int S = 1;
  long long best = -1;
  for (int k = 1; k <= 64 && k <= std::max(1LL, chunks); ++k) {
    const long long rounds = cdiv((long long)ntile * k, (long long)ncu);
    const long long cost = rounds * cdiv(chunks, (long long)k);
    if (best < 0 || cost < best) {
      best = cost;
      S = k;
    }
  }
  std::vector<SyrkTask>& tasks = P.tasks;
  std::vector<int>& partlist = P.partlist;
  std::vector<RedTask>& rtasks = P.rtasks;
  if (chunks > 0) {
    for (int sl = 0; sl < S; ++sl) {
      const int k0 = (int)(32 * (chunks * sl / S)), k1 = (int)(32 * (chunks * (sl + 1) / S));
      int t = 0;
      for (int ti = 0; ti < nt; ++ti)
        for (int tj = ti; tj < nt; ++tj, ++t) tasks.push_back(SyrkTask{0, ti, tj, k0, k1, (int)tasks.size(), 0, 0});
    }
    int t = 0;
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = ti; tj < nt; ++tj, ++t) {
        const int part0 = (int)partlist.size();
        for (int sl = 0; sl < S; ++sl) partlist.push_back(sl * ntile + t);
        for (int a = 0; a < 2; ++a)
          for (int b = 0; b < 2; ++b) {
            if (ti == tj && a > b) continue;
            const int r0 = ti * 128 + 64 * a, c0 = tj * 128 + 64 * b;
            if (r0 >= n || c0 >= n) continue;
            rtasks.push_back(RedTask{0, r0, c0, part0, S, 0, 0, 0});
          }
      }
  } else {
    // no tokens: H = 0 (every sub-block sums zero partials)
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = ti; tj < nt; ++tj)
        for (int a = 0; a < 2; ++a)
          for (int b = 0; b < 2; ++b) {
            const int r0 = ti * 128 + 64 * a, c0 = tj * 128 + 64 * b;
            if ((ti == tj && a > b) || r0 >= n || c0 >= n) continue;
            rtasks.push_back(RedTask{0, r0, c0, 0, 0, 0, 0, 0});
          }
  }
}

// ------------------------------------------------------------- factor plan --
// Cholesky and Y = L^{-1}: outer panels of 256 columns, four 64-column steps
// each, taken in pairs (k, k+1) by one k_chol_panel2 launch (a last block
// without a partner takes the single-step k_chol_panel).  After a step, the
// updates of the rest of the outer panel (L columns [c0, P1) of every row
// below; Y rows [c0, P1)).  At the end of an outer panel the trailing updates
// with K = P1 - P0 split in two: the part the next outer panel reads (L
// columns [P1, S), S = P1 + 256; Y rows [P1, S)) on the main stream, and the
// rest (L's trailing triangle from S on; Y rows from S on) on the side
// stream, where it overlaps the next outer panel's steps (which neither read
// nor write it) and is joined before the next outer update.  With the
// general products (n % 64 != 0) everything stays on one stream.
std::vector<PlanLaunch> plan_factor(const std::vector<FacShape>& jobs, int ncu) {
  const int np = (int)jobs.size();
  std::vector<PlanLaunch> launches;
  auto add_launch = [&](int kind, std::vector<Seg>& segs, bool side = false) {
    int nwg = 0;
    for (auto& s : segs) {
      s.wg0 = nwg;
      nwg += s.nwg;
    }
    if (nwg == 0) return;
    launches.push_back(PlanLaunch{kind, 0, 0, side, segs, nwg});
  };
  auto add_sync = [&](int kind) { launches.push_back(PlanLaunch{kind, 0, 0, false, {}, 0}); };
  int maxnb = 0;
  for (const FacShape& J : jobs) maxnb = std::max(maxnb, cdiv(J.n, 64));
  // The ring-staged products need every K range and row pitch to be a
  // multiple of 64 (16-byte aligned chunks of 16 doubles).
  bool ring = true;
  for (const FacShape& J : jobs) ring = ring && (J.n % 64) == 0;
  {
    std::vector<Seg> s;
    for (int p = 0; p < np; ++p)
      if (jobs[p].fill) s.push_back(Seg{p, 0, cdiv(jobs[p].n, 4), 0, 0, 0, 0, 0});
    add_launch(FK_FILL, s);
  }
  bool side_busy = false;
  for (int k = 0; k < maxnb; k += 2) {
    std::vector<Seg> pan, pan2, inner, crit, bulk;
    int bulk_rows = 0;
    for (int p = 0; p < np; ++p) {
      const int n = jobs[p].n, nb = cdiv(n, 64);
      if (k >= nb) continue;
      const bool pair = k + 1 < nb;
      (pair ? pan2 : pan).push_back(Seg{p, 0, nb, k, 0, 0, 0, 0});
      const int k0 = 64 * k, pw = std::min(pair ? 128 : 64, n - k0);
      const int P0 = (k0 / 256) * 256, P1 = std::min(P0 + 256, n);
      const int c0 = k0 + pw;
      if (c0 < P1) {  // rest of the outer panel
        const int nrow = cdiv(n - c0, 64), ncol = cdiv(P1 - c0, 64);
        inner.push_back(Seg{p, 0, ncol * nrow - ncol * (ncol - 1) / 2, GK_CHOL_TRAIL, k0, pw, c0, P1});
        inner.push_back(Seg{p, 0, cdiv(P1 - c0, 64) * cdiv(c0, 64), GK_ZUPD, k0, pw, c0, P1});
      } else if (P1 < n) {  // end of the outer panel: trailing updates with K = P1 - P0
        const int S = ring ? std::min(P1 + 256, n) : n;
        {
          const int nrow = cdiv(n - P1, 64), ncol = cdiv(S - P1, 64);
          crit.push_back(Seg{p, 0, ncol * nrow - ncol * (ncol - 1) / 2, GK_CHOL_TRAIL, P0, P1 - P0, P1, S});
          crit.push_back(Seg{p, 0, cdiv(S - P1, 64) * cdiv(P1, 64), GK_ZUPD, P0, P1 - P0, P1, S});
        }
        if (S < n) {
          const int m = cdiv(n - S, 128);
          bulk.push_back(Seg{p, 0, m * (m + 1) / 2, GK_CHOL_TRAIL, P0, P1 - P0, S, n});
          bulk.push_back(Seg{p, 0, m * cdiv(P1, 128), GK_ZUPD, P0, P1 - P0, S, n});
          bulk_rows = std::max(bulk_rows, n - S);
        }
      }
    }
    int pan2_wg = 0;
    for (const Seg& sg : pan2) pan2_wg += sg.nwg;
    if (pan2_wg > ncu) {
      // more panel workgroups than CUs (batched layers): every workgroup
      // repeating its problem's diagonal chain would cost one chain per round
      // of the chip, so the chain runs once per problem first
      std::vector<Seg> dg;
      for (Seg& sg : pan2) {
        dg.push_back(Seg{sg.prob, 0, 1, sg.a, 0, 0, 0, 0});
        sg.b = 1;
      }
      add_launch(FK_DIAG2, dg);
    }
    add_launch(FK_PANEL2, pan2);
    add_launch(FK_PANEL, pan);
    add_launch(ring ? FK_RING64 : FK_GEMM64, inner);
    if (!crit.empty()) {
      if (side_busy) add_sync(PL_JOIN);  // the previous bulk update touches the columns updated now
      side_busy = false;
      if (!bulk.empty()) {
        if (bulk_rows < 1024) {  // small: 64-wide tiles, on the main stream
          for (Seg& sg : bulk) {
            const int n = jobs[sg.prob].n, m = cdiv(n - sg.d, 64);
            sg.nwg = (sg.a == GK_CHOL_TRAIL) ? m * (m + 1) / 2 : m * cdiv(sg.b + sg.c, 64);
          }
          for (Seg& sg : bulk) crit.push_back(sg);
        } else {
          add_sync(PL_FORK);
          add_launch(FK_RING128, bulk, true);
          side_busy = true;
        }
      }
      add_launch(ring ? FK_RING64 : FK_GEMM64, crit);
    }
  }
  if (side_busy) add_sync(PL_JOIN);
  {
    std::vector<Seg> s;
    for (int p = 0; p < np; ++p) s.push_back(Seg{p, 0, cdiv(jobs[p].n, 4), 0, 0, 0, 0, 0});
    add_launch(FK_MAKEU, s);
  }
  return launches;
}

// ----------------------------------------------------------- quantize plan --
// Super-blocks: each block's errors reach the rest of its super-block right
// away (inside the sweep kernel), the columns past it only at the
// super-block's end (one product with K = the super-block width), so the far
// columns of W are rewritten once per super-block instead of once per block.
// Groups must nest in it.  At a super-block's end, the next super-block's
// columns are updated on the main stream (its sweeps read them); the columns
// past it on the side stream, beside the next super-block's sweeps (which
// neither read nor write them; the errors sit in the other half of the
// two-super-block buffer), joined before the next far update.  Needs the
// groups to nest in a super-block (a group fit reads its whole group).
void plan_quantize(const std::vector<QuantShape>& jobs, QuantLayout* lay, std::vector<PlanLaunch>* out_launches) {
  const int nl = (int)jobs.size();
  QuantLayout& Ly = *lay;
  Ly = QuantLayout{};
  Ly.sbk.resize(nl);
  Ly.oW.resize(nl);
  Ly.oE.resize(nl);
  Ly.oO.resize(nl);
  Ly.oD.resize(nl);
  int maxblk = 0;
  for (int p = 0; p < nl; ++p) {
    const QuantShape& J = jobs[p];
    // 1024 columns for 128-wide blocks (more of the trailing update on the
    // sweep workgroups' own MFMAs, less beside the sweeps on the second
    // stream: faster while the sweep workgroups fit the chip in few rounds),
    // 512 for narrower blocks (K = B products, and batched small layers whose
    // sweep workgroups take many rounds, where the update kernels do better)
    int sb = std::max(1, (J.block >= 128 ? 1024 : 512) / J.block);
    const int sbw = sb * J.block;
    if (J.group && !(sbw % J.group == 0 || J.group % sbw == 0)) sb = 1;
    Ly.sbk[p] = sb;
    Ly.oW[p] = Ly.totW;
    if (!J.ext_ww) Ly.totW += (size_t)J.out * J.nt;
    Ly.oE[p] = Ly.totE;
    Ly.totE += 2 * (size_t)J.out * sb * J.block;  // two super-blocks: one swept while the other's far update runs
    Ly.oO[p] = Ly.totO;
    Ly.totO += (size_t)J.out * 2;
    Ly.oD[p] = Ly.totD;
    Ly.totD += (size_t)(J.nt + 63) / 64 * 64;
    maxblk = std::max(maxblk, cdiv(J.n, J.block));
  }
  std::vector<PlanLaunch>& launches = *out_launches;
  launches.clear();
  auto add_launch = [&](int kind, int block, std::vector<Seg>& segs, bool side = false, int mode = 0) {
    int nwg = 0;
    for (auto& s : segs) {
      s.wg0 = nwg;
      nwg += s.nwg;
    }
    if (nwg == 0) return;
    launches.push_back(PlanLaunch{kind, block, mode, side, segs, nwg});
  };
  auto add_sync = [&](int kind) { launches.push_back(PlanLaunch{kind, 0, 0, false, {}, 0}); };
  {
    std::vector<Seg> s, f;
    for (int p = 0; p < nl; ++p) {
      s.push_back(Seg{p, 0, cdiv(jobs[p].out, 4), 0, 0, 0, 0, 0});
      if (jobs[p].group == 0 && !jobs[p].mode) f.push_back(Seg{p, 0, cdiv(jobs[p].out, 4), 0, 0, 0, 0, 0});
    }
    add_launch(QK_INIT, 0, s);
    add_launch(QK_ROWFIT, 0, f);
  }
  std::vector<int> blocks;
  for (auto& J : jobs)
    if (std::find(blocks.begin(), blocks.end(), J.block) == blocks.end()) blocks.push_back(J.block);
  bool side_busy = false;
  // One sweep launch per super-block.
  for (int k = 0; k < maxblk; ++k) {
    for (int B : blocks)
      for (int mode = 0; mode < 2; ++mode) {
        std::vector<Seg> s;
        for (int p = 0; p < nl; ++p)
          if (jobs[p].block == B && jobs[p].mode == mode && k < cdiv(jobs[p].n, B) && k % Ly.sbk[p] == 0)
            s.push_back(Seg{p, 0, cdiv(jobs[p].out, 16), k / Ly.sbk[p], 0, 0, 0, 0});
        add_launch(QK_SWEEP, B, s, false, mode);
      }
    std::vector<Seg> crit, bulk;  // past the super-block (64 / 128 tiles)
    for (int p = 0; p < nl; ++p) {
      const int B = jobs[p].block, n = jobs[p].n, nt = jobs[p].nt, sb = Ly.sbk[p], sbw = sb * B;
      if (k >= cdiv(n, B)) continue;
      const int b0 = k * B, b1 = std::min(b0 + B, n);
      const int sb0 = (k / sb) * sbw, sb1 = std::min(sb0 + sbw, n);
      const int par = ((k / sb) & 1) * jobs[p].out * sbw;  // this super-block's half of the error buffer
      if (b1 == sb1 && sb1 < nt) {  // end of the super-block: all columns past it
        const bool nest = jobs[p].group == 0 || sbw % jobs[p].group == 0;
        const int S = nest ? std::min(sb1 + sbw, nt) : nt;
        crit.push_back(Seg{p, 0, cdiv(jobs[p].out, 64) * cdiv(S - sb1, 64), par, sb0, sb1 - sb0, sb1, S});
        if (S < nt) bulk.push_back(Seg{p, 0, cdiv(jobs[p].out, 128) * cdiv(nt - S, 128), par, sb0, sb1 - sb0, S, nt});
      }
    }
    if (!crit.empty()) {
      if (side_busy) add_sync(PL_JOIN);  // the previous far update covers the columns updated now
      side_busy = false;
      if (!bulk.empty()) {
        add_sync(PL_FORK);
        add_launch(QK_TRAIL, 128, bulk, true);
        side_busy = true;
      }
      add_launch(QK_TRAIL, 64, crit);
    }
  }
  if (side_busy) add_sync(PL_JOIN);
}
