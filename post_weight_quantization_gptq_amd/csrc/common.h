// Internal definitions shared by the HIP kernels and the host planner of the
// GPTQ library (gfx950 / CDNA4).  Nothing here is part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef double f64x4 __attribute__((__vector_size__(4 * sizeof(double))));
typedef double f64x2 __attribute__((__vector_size__(2 * sizeof(double))));

#include "tables.h"

// fp64 Gram output (full symmetric [n][n]).
struct RedProb64 {
  double* H;
  int n;
  int pad0;
};

// ----------------------------------------------------------------- factor --
// Work matrices are fp64, row-major with leading dimension n.
//   A: damped, index-reversed matrix, overwritten by its Cholesky factor C
//   Y: C^{-1} (lower), T: scratch of the triangular inverse
struct FacProb {
  const float* H;  // input [n][ldh] fp32 (null when A was assembled elsewhere)
  double* A;       // [n][n]: P H_lam P (lower), overwritten by L
  double* Y;       // [n][n]: L^{-1}, built row block by row block
  float* U;        // output [n][ldu]
  double* C;       // GK_NT only: the product's output
  double* D;       // [3][64][64]: Y0, Y1, L10 of the current pair from k_chol_diag2 (batched plans)
  int n;
  int ldh;
  int ldu;
  int pad0;
  double lam_abs, lam_rel;
  double* lam;     // device slot: damping used
  int* info;       // device slot: 0 or 1 + failing column (H numbering)
  int* nonfinite;  // device slot
};



// -------------------------------------------------------- two-sided round --
// GPTQ-2D state (all [m][n] row-major unless noted); see round2d.hip.
struct R2dProb {
  const float* X;    // target
  const float* Lgt;  // [m][m]: UG[i][k] / UG[i][i] for k >= i (row i = column i of the unit lower Lg)
  const float* Uh1;  // [n][n]: UH[j][l] / UH[j][j] for l >= j
  const float* dG;   // [m] UG[i][i]
  const float* dH;   // [n] UH[j][j]
  float* C;          // pushes down the columns from the tiles above
  float* R;          // pushes along the rows from the tiles to the left
  float* D;          // delta = w - z
  float* Cf;         // C + delta, what a finished entry pushes right
  int* Z;            // the integers
  double* objp;      // [TM][TN] per-tile sums of squared scaled errors
  int m, n, qmin, qmax;
};

// Round-to-nearest of the low-rank factors: components 0..r-1 are the columns
// of L [n][r], r..2r-1 the rows of R [r][out]; each gets its own grid.
struct LrProb {
  const float* L;
  const float* R;
  uint8_t* Lc;  // [n][r]
  float* Ls;    // [r]
  uint8_t* Lz;  // [r]
  float* Lh;    // [n][r] dequantised (may be null)
  uint8_t* Rc;  // [r][out]
  float* Rs;
  uint8_t* Rz;
  float* Rh;    // [r][out] (may be null)
  int n, r, out, maxqL, maxqR;
  int pad0;
};

// Y[M][N] = X[M][K] What^T with What = s (q - z) from packed codes (4 bits,
// or 2, 3 and 8 in the general entry; the kernels take the width as a
// template parameter).
struct W4Prob {
  const uint16_t* X;  // bf16 bits, row pitch ldx
  const uint32_t* P;  // [N][K bits/32] row bitstreams (code k at stream bits [k bits, (k+1) bits))
  const float* S;     // [N][G]
  const uint8_t* Z;   // [N][G]
  float* Y;           // row pitch ldy
  long long ldx, ldy;
  int M, N, K, G;
  int gshift;  // group = 2^gshift (31: one group per row)
  int tiles_m, tiles_n;
};

// ------------------------------------------------------------------ sweep --
struct QLayer {
  const float* W;   // original weights [out][n]
  float* Ww;        // working weights [out][nt]
  const float* U;   // factor [nt][nt]
  uint8_t* codes;   // [out][n]
  float* scales;    // [out][ng]
  uint8_t* zeros;   // [out][ng]
  float* err;       // [out][n] or null
  float* Eb;        // errors of a super-block [2][out][ldE], by super-block parity
  const float* dinv;  // 1 / U_jj [nt], filled by k_init_work
  double* objp;     // per row: {sum E^2, sum D^2}, accumulated block by block
  double* obj;      // [2] {J, J_lam} (device)
  const double* lam;  // device slot holding the damping of U
  int out, n, nt, bits, group, block, nblk, ng;
  int ldE;          // width of the error buffer (one super-block of columns)
  int eoff_blk;     // column offset of one block inside it (= block)
  int sbk;          // blocks per super-block
  int mode;         // 0: GPTQ sweep; 1: Bid-Up pass (W = g, U = H, codes in/out, grid given)
};

typedef __attribute__((address_space(3))) void lds_void;
// Typed global and LDS views of generic pointers (for pointers read out of
// descriptors, which the compiler cannot prove global): accesses through a
// global view compile to global_* instructions, whose completion is counted
// by vmcnt alone, so waits for LDS results stay precise.
template <class T>
using gptr = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ gptr<T> glb(T* p) {
  return (gptr<T>)p;
}
template <class T>
using lptr = __attribute__((address_space(3))) T*;
template <class T>
__device__ __forceinline__ lptr<T> lds_view(T* p) {
  return (lptr<T>)p;
}

// global-memory views: loads through them count only against vmcnt (a
// generic pointer's flat loads also count against lgkmcnt, which LDS waits
// would then have to drain)
typedef const __attribute__((address_space(1))) double gdouble;
typedef const __attribute__((address_space(1))) float gfloat;

// s_waitcnt immediate that waits for vmcnt <= N only (gfx9 encoding).
template <int N>
struct VmWait {
  static constexpr int value = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
};

__device__ __forceinline__ int find_seg(const Seg* __restrict__ segs, int nseg, int wg) {
  int s = 0;
  while (s + 1 < nseg && segs[s + 1].wg0 <= wg) ++s;
  return s;
}
