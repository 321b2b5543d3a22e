// Host planner of the GPTQ library: the task tables and launch sequences of
// the Hessian, the factor and the quantise sweep, as plain C++ (no HIP
// calls), so the same code also builds into a host-only checker.  The C ABI
// (api.cpp) adds device pointers, uploads the tables and issues the launches.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "tables.h"

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
inline long long cdiv64(long long a, long long b) { return (a + b - 1) / b; }

// One grouped launch of a plan: its segments (wg0 = prefix sums of nwg) or,
// for the stream kinds, a fork (the second stream waits for the first) or a
// join (the first waits for the second).
struct PlanLaunch {
  int kind;
  int block;  // tile or block width of the kernel (quantise plans)
  int mode;   // sweeps: 0 GPTQ, 1 Bid-Up
  bool side;  // issued on the second stream
  std::vector<Seg> segs;
  int nwg;
};
constexpr int PL_FORK = 6, PL_JOIN = 7;

// ------------------------------------------------------------ Hessian -----
struct HessJob {
  const uint16_t* X;
  long long tokens, ldx;
  int n;
  float* H;
  int accumulate;
  // non-null: the cross Gram X^T Y (Y as X: [tokens][ldx]; direct layout
  // only), written in full
  const uint16_t* Y = nullptr;
};

struct HessPlan {
  std::vector<XposeProb> xprobs;
  std::vector<Seg> xsegs;
  std::vector<SyrkProb> probs;
  std::vector<SyrkTask> tasks;
  std::vector<RedProb> rprobs;
  std::vector<RedTask> rtasks;
  std::vector<int> partlist;
  int nparts = 0;
};

// X read in place by the tiles (no transposed copy).
bool hess_direct(const HessJob& J);
// Elements of the transposed copies the jobs need.
size_t hess_xt_elems(const std::vector<HessJob>& jobs);
// Tasks of every job on a chip of ncu CUs in nxcd XCDs; xt is the base of
// the transposed copies (may be null when no job needs one).
void plan_hessian(const std::vector<HessJob>& jobs, int ncu, int nxcd, uint16_t* xt, HessPlan& P);

// fp64 Gram of one layer: 128x128 upper tiles times S token slices over the
// transposed copy (t_pad = tokens rounded up to 64).
struct Hess64Plan {
  std::vector<SyrkTask> tasks;
  std::vector<RedTask> rtasks;
  std::vector<int> partlist;
};
void plan_hessian64(int n, long long tokens, int ncu, Hess64Plan& P);

// ------------------------------------------------------------- factor -----
enum FacKind {
  FK_FILL = 0,     // k_damp_fill: A from H (lower triangle, reversed, damped)
  FK_PANEL = 1,    // k_chol_panel: one 64-column step
  FK_GEMM64 = 2,   // k_gemm<64> (general n)
  FK_RING64 = 3,   // k_gemm_ring<64> (n % 64 == 0)
  FK_RING128 = 4,  // k_gemm_ring<128>
  FK_MAKEU = 5,    // k_make_u: U from Y
  FK_PANEL2 = 8,   // k_chol_panel2: two 64-column steps (segment b = 1: diagonal chain from FK_DIAG2)
  FK_DIAG2 = 9     // k_chol_diag2: a pair's diagonal chain, once per problem
};
struct FacShape {
  int n;
  bool fill;  // A is built from H by k_damp_fill (else assembled beforehand)
};
// ncu: CUs of the chip; a pair step whose panel workgroups exceed it runs
// its problems' diagonal chains once each first (FK_DIAG2).
std::vector<PlanLaunch> plan_factor(const std::vector<FacShape>& jobs, int ncu);

// ----------------------------------------------------------- quantise -----
enum QuantKind { QK_INIT = 0, QK_ROWFIT = 1, QK_SWEEP = 2, QK_TRAIL = 3 };
struct QuantShape {
  int out, n, nt, block, group, mode;
  bool ext_ww;  // the caller provides the working weights
};
// Per-layer super-block counts and the offsets (in elements) of each layer's
// working weights, two-super-block error buffer, per-row sums and error
// scales in their shared buffers.
struct QuantLayout {
  std::vector<int> sbk;
  std::vector<size_t> oW, oE, oO, oD;
  size_t totW = 0, totE = 0, totO = 0, totD = 0;
};
void plan_quantize(const std::vector<QuantShape>& jobs, QuantLayout* lay, std::vector<PlanLaunch>* launches);
