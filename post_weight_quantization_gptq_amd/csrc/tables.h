// Task-table records the host planner writes and the kernels read (plain
// data: no HIP types, so the planner also builds as ordinary C++).
#pragma once
#include <stdint.h>

// A grouped launch covers several problems (layers).  Each problem owns a
// contiguous range [wg0, wg0 + nwg) of the grid; a..d are kernel-specific.
struct Seg {
  int prob;
  int wg0;
  int nwg;
  int a, b, c, d, e;
};

// ---------------------------------------------------------------- Hessian --
// One 256x256 output tile of H over the token range [k0, k1) -> partial slot.
struct XposeProb {
  const uint16_t* X;
  long long ldx;
  uint16_t* Xt;  // [n_pad][ldt], tokens [0, t_pad) written
  int n, tokens, n_pad, t_pad;
  int vec;  // rows of X are 16-byte aligned (16-byte loads allowed)
  int ldt;  // row pitch of Xt in tokens (>= t_pad)
};
struct SyrkProb {
  // direct == 0: Xt is the feature-major copy [n_pad][ldt], zero-padded to
  // t_pad tokens.  direct == 1: Xt is X itself, token-major [tokens][ldt]
  // (16-byte aligned rows, n a multiple of 8); rows past `tokens` and
  // features past n are never read.
  const uint16_t* Xt;
  long long ldt;
  int direct;
  int tokens;
  int n;
  int pad0;
  // cross Gram X^T Y: the B operand's rows come from Yt (same layout and
  // pitch as Xt, direct mode only); null for X^T X
  const uint16_t* Yt;
};
struct SyrkTask {
  int prob, ti, tj, k0, k1, part, pad0, pad1;
};
// One 64x64 sub-block (r0 <= c0 region) of an upper tile: sum of its partials.
struct RedProb {
  float* H;
  int n;
  int accumulate;
  int full;  // 1: a cross Gram, every sub-block written as is (no mirror)
  int pad0;
};
struct RedTask {
  int prob, r0, c0, part0, nparts, pad0, pad1, pad2;
};
// GK_CHOL_TRAIL: A(i, j) -= sum_t L(i, t) L(j, t) on the lower tiles of rows
//   [d, n) x columns [d, e), t in [b, b + c).
// GK_ZUPD: Y(i, j) -= sum_t L(i, t) Y(t, j) on rows [d, e) x columns
//   [0, b + c), t in [b, b + c); columns from b on are written for the first
//   time (no accumulate).
// GK_NT: C(i, j) = sum_t A(i, t) B(j, t) with A = A [b][d], B = Y [c][d] and
//   C [b][c], all of pitch n (a plain product of two k-contiguous operands;
//   the flags info / nonfinite are not consulted); e = 1 or 2 declares B
//   upper or lower triangular, so a column tile skips the zero part of K
//   (K and the tile size multiples of 16).
enum GemmKind { GK_CHOL_TRAIL = 0, GK_ZUPD = 1, GK_NT = 2 };
