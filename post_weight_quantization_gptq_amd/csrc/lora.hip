// GPTQ-intrinsic LoRA (GPTQ-intrinsic LoRA technical summary, method section
// 2): the calibration matrix is augmented to X~ = [X, X V_r] with V_r the top-r
// right singular vectors of X (= top-r eigenvectors of H = X^T X), and the
// GPTQ sweep runs on W~ = [W, 0]; the first n columns are rounded into Q and
// the r appended columns, never rounded, absorb the error and become R.
//
// X~ is never formed: its Gram matrix is H~ = [[H, H V], [V^T H, V^T H V]].
// H~ is singular (its last r columns are combinations of the first n), so the
// pages factor H~ + lam I by eigendecomposition and QR to allow a small lam;
// that gives the same U as a Cholesky of H~ + lam I, which is what is done
// here, in fp64 (the damped matrix stays positive definite, and fp64 keeps
// the condition number of ~1e6 at lam = 1e-4 mean(diag H) harmless).
//
// V_r comes from subspace iteration in fp64 on m >= r columns (Q <- orth(H Q)
// by one Cholesky-QR pass per step, from a fixed hash-generated block), with
// a Rayleigh-Ritz step every few steps that rotates Q onto the Ritz vectors
// and stops on a residual test (see top_subspace); a last Cholesky-QR pass
// on the r Ritz vectors makes V_r orthonormal to rounding.
// Only span(V_r) matters: Q and the product L R do not depend on the basis.
#include <algorithm>
#include <type_traits>
#include <utility>
#include <vector>

#include "../../include/gptq.h"
#include "blk64.h"
#include "jacobi_order.h"
#include "common.h"
#include "launch.h"
#include "plan.h"

namespace {

// Subspace iterations: a Rayleigh-Ritz check every kCheck steps, at most
// kMaxIters steps, stop when the top-r residual is below kTol ||theta_r||
// (about a hundred times the rounding floor of the fp64 products at n = 4096).
constexpr int kCheck = 4;
constexpr int kMaxIters = 600;
constexpr double kTol = 1e-11;

// C(i,j) = alpha * sum_k A(i,k) B(k,j) over the split's k range, written to
// P + z*M*N (split-K partial).  A(i,k) = A[i*sai + k*sak], B(k,j) = B[k*sbk + j*sbj].
struct DGemm {
  const double* A;
  long long sai, sak;
  const double* B;
  long long sbk, sbj;
  double* P;
  int M, N, K, ksplit;
};

// One 64x64 tile per workgroup over its split's k range, 4 waves of 32x32 on
// v_mfma_f64_16x16x4f64.  K chunks of 32 go through registers into a
// double-buffered LDS pair: the loads of chunk c+1 are in flight while chunk c
// is multiplied (the products here are thin and latency-bound).
__global__ __launch_bounds__(256) void k_dgemm(DGemm g) {
  constexpr int KC = 32;
  __shared__ double As[2][64][KC + 1];
  __shared__ double Bs[2][KC][65];
  const int tiles_n = (g.N + 63) / 64;
  const int i0 = 64 * (blockIdx.x / tiles_n), j0 = 64 * (blockIdx.x % tiles_n);
  const int z = blockIdx.y;
  const int kb = (int)((long long)g.K * z / g.ksplit), ke = (int)((long long)g.K * (z + 1) / g.ksplit);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;
  // this thread's 8 A and 8 B values of a chunk
  const bool ak = g.sak == 1, bj = g.sbj == 1;
  const int ar = ak ? tid >> 2 : tid & 63, akq = ak ? (tid & 3) * 8 : (tid >> 6) * 8;
  const int bk = bj ? tid >> 3 : (tid & 3) * 8, bjq = bj ? (tid & 7) * 8 : tid >> 2;
  const bool arow = i0 + ar < g.M;
  double ra[8], rb[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = k0 + akq + u;
      ra[u] = (arow && kk < ke) ? g.A[(long long)(i0 + ar) * g.sai + (long long)kk * g.sak] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = bj ? k0 + bk : k0 + bk + u, j = bj ? j0 + bjq + u : j0 + bjq;
      rb[u] = (kk < ke && j < g.N) ? g.B[(long long)kk * g.sbk + (long long)j * g.sbj] : 0.0;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 8; ++u) As[buf][ar][akq + u] = ra[u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (bj) Bs[buf][bk][bjq + u] = rb[u];
      else Bs[buf][bk + u][bjq] = rb[u];
    }
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][c][r] = 0.0;
  if (kb < ke) {
    load(kb);
    store(0);
  }
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += KC) {
    const bool more = k0 + KC < ke;
    if (more) load(k0 + KC);
#pragma unroll
    for (int kk = 0; kk < KC / 4; ++kk) {
      double av[2], bv[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) av[mi] = As[buf][32 * wr + 16 * mi + (lane & 15)][4 * kk + (lane >> 4)];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bv[ni] = Bs[buf][4 * kk + (lane >> 4)][32 * wc + 16 * ni + (lane & 15)];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  double* P = g.P + (size_t)z * g.M * g.N;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 32 * wr + 16 * mi + (lane >> 4) + 4 * r;
        const int j = j0 + 32 * wc + 16 * ni + (lane & 15);
        if (i < g.M && j < g.N) P[(size_t)i * g.N + j] = acc[mi][ni][r];
      }
}

// C[i][j] = sum_z P[z][i][j] in split order.
__global__ void k_dsum(const double* __restrict__ P, double* __restrict__ C, long long MN, int ksplit) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= MN) return;
  double s = 0.0;
  for (int z = 0; z < ksplit; ++z) s += P[z * MN + i];
  C[i] = s;
}

// Fixed start block: hash of (i, k) mapped to [-1, 1).
__global__ void k_start_block(double* __restrict__ V, int n, int r) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)n * r) return;
  unsigned long long x = (unsigned long long)i * 0x9E3779B97F4A7C15ull + 0x632BE59BD9B4E019ull;
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  V[i] = (double)(x >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

// ------------------------------------------------ Cholesky-QR pieces -----
// One Cholesky-QR pass turns Z (n x r, r <= 128) into V = Z L^{-T} with
// G = Z^T Z = L L^T, so V^T V = I.  Two kernels:
//   k_gram_chol: G by row chunks (each workgroup the Gram of its rows, 64 at
//     a time, on fp64 MFMA), then the last workgroup to finish sums the
//     partials in chunk order and factors G, as 64x64 blocks: the leaf
//     Cholesky and inverse of G00, L10 = G10 L00^{-T}, the leaf of
//     G11 - L10 L10^T and its inverse, Li10 = -Li11 L10 Li00; it writes
//     Li = L^{-1} (r x r row-major, zeros above the diagonal).
//   k_apply: V = Z Li^T, 64 rows per workgroup.
// A relative jitter of 1e-15 max diag(G) on the diagonal keeps a (nearly)
// rank-deficient G factorable; a pivot that still fails is replaced by 1, so
// the result stays finite (the second pass re-orthonormalises).
constexpr int kGramParts = 8;  // at most this many row chunks per Gram

// ZTb[c][t] = Z[i0 + t][64 b + c] for t < 64, zeros past n and r: the
// values go to registers first (zt_load), then to LDS transposed (zt_store),
// so the next chunk's loads can be in flight while this one is multiplied
__device__ __forceinline__ void zt_load(const double* __restrict__ Z, int n, int r, int i0, double (&v)[32]) {
  const int tid = threadIdx.x;
  const int rc = r > NB ? 2 * NB : NB;  // columns staged
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int e = tid + 256 * q, t = e / rc, c = e % rc;
    v[q] = (e < NB * rc && i0 + t < n && c < r) ? Z[(size_t)(i0 + t) * r + c] : 0.0;
  }
}

__device__ __forceinline__ void zt_store(int r, const double (&v)[32], double (*ZT0)[LDP], double (*ZT1)[LDP]) {
  const int tid = threadIdx.x;
  const int rc = r > NB ? 2 * NB : NB;
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int e = tid + 256 * q, t = e / rc, c = e % rc;
    if (e < NB * rc) {
      if (c < NB) ZT0[c][t] = v[q];
      else ZT1[c - NB][t] = v[q];
    }
  }
}

__global__ __launch_bounds__(256) void k_gram_chol(const double* __restrict__ Z, int n, int r, int rows_per,
                                                   double* __restrict__ Gp, double* __restrict__ Li,
                                                   unsigned* __restrict__ counter) {
  __shared__ __attribute__((aligned(16))) double LT[NB][LDP];   // Z^T chunk (cols 0-63), then leaf workspace
  __shared__ __attribute__((aligned(16))) double L10[NB][LDP];  // Z^T chunk (cols 64-127), then G10 / L10
  __shared__ __attribute__((aligned(16))) double Y0[NB][LDP];
  __shared__ __attribute__((aligned(16))) double Y1[NB][LDP];   // G11 until its leaf, then Li11
  __shared__ double Tm[32][33];
  __shared__ double lb[2 * NB];
  __shared__ double dv[NB];
  __shared__ double jit;
  __shared__ int flag, last;
  const int tid = threadIdx.x, nz = gridDim.x, z = blockIdx.x;
  const bool two = r > NB;
  const int nblk = two ? 3 : 1;
  {
    f64x4 g00[2][2], g10[2][2], g11[2][2];
    blk_zero(g00);
    blk_zero(g10);
    blk_zero(g11);
    const int ie = min(n, (z + 1) * rows_per);
    double v[32];
    zt_load(Z, n, r, z * rows_per, v);
    for (int i0 = z * rows_per; i0 < ie; i0 += NB) {
      zt_store(r, v, LT, L10);
      __syncthreads();
      if (i0 + NB < ie) zt_load(Z, n, r, i0 + NB, v);  // next chunk, in flight during the products
      blk_mma<true>(g00, LT, LT);
      if (two) {
        blk_mma<true>(g10, L10, LT);
        blk_mma<true>(g11, L10, L10);
      }
      __syncthreads();
    }
    double* P = Gp + (size_t)z * 3 * NB * NB;
    blk_each([&](int mi, int ni, int q, int rr, int c) {
      P[rr * NB + c] = g00[mi][ni][q];
      if (two) {
        P[NB * NB + rr * NB + c] = g10[mi][ni][q];
        P[2 * NB * NB + rr * NB + c] = g11[mi][ni][q];
      }
    });
  }
  // the last workgroup to finish reduces and factors
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(counter, 1u) == (unsigned)(nz - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  const int m0 = min(r, NB), m1 = r - m0;
  for (int b = 0; b < nblk; ++b) {
    double s[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) s[q] = 0.0;
    // in chunk order; four partials' loads in flight at a time
    int zz = 0;
    for (; zz + 4 <= nz; zz += 4) {
      double t4[4][16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double* P = Gp + ((size_t)(zz + u) * 3 + b) * NB * NB;
#pragma unroll
        for (int q = 0; q < 16; ++q) t4[u][q] = P[tid + 256 * q];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] += t4[u][q];
    }
    for (; zz < nz; ++zz) {
      const double* P = Gp + ((size_t)zz * 3 + b) * NB * NB;
#pragma unroll
      for (int q = 0; q < 16; ++q) s[q] += P[tid + 256 * q];
    }
    double (*D)[LDP] = b == 0 ? LT : b == 1 ? L10 : Y1;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      D[e >> 6][e & 63] = s[q];
    }
  }
  __syncthreads();
  if (tid < 64) {
    double d = tid < m0 ? LT[tid][tid] : 0.0;
    if (tid < m1) d = fmax(d, Y1[tid][tid]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) d = fmax(d, __shfl_xor(d, o));
    if (tid == 0) jit = 1e-15 * d;
  }
  __syncthreads();
  if (tid < 64) {
    LT[tid][tid] = tid < m0 ? LT[tid][tid] + jit : 1.0;
    if (two) Y1[tid][tid] += jit;
  }
  __syncthreads();
  chol64_blocked(LT, dv, lb, &flag);  // a failed pivot is replaced by 1
  inv64_waves(LT, dv, Y0, Tm);
  f64x4 acc[2][2];
  if (two) {
    // L10 = G10 Li00^T
    blk_zero(acc);
    blk_mma<true>(acc, L10, Y0);
    __syncthreads();
    blk_each([&](int mi, int ni, int q, int rr, int c) { L10[rr][c] = acc[mi][ni][q]; });
    f64x4 d1[2][2];
    blk_each([&](int mi, int ni, int q, int rr, int c) { d1[mi][ni][q] = Y1[rr][c]; });
    __syncthreads();
    // G11 - L10 L10^T, padded with the identity past m1
    blk_neg(d1);
    blk_mma<true>(d1, L10, L10);
    blk_neg(d1);
    blk_each([&](int mi, int ni, int q, int rr, int c) {
      LT[rr][c] = (rr < m1 && c < m1) ? d1[mi][ni][q] : ((rr == c) ? 1.0 : 0.0);
    });
    __syncthreads();
    chol64_blocked(LT, dv, lb, &flag);
    inv64_waves(LT, dv, Y1, Tm);
    // Li10 = -Li11 (L10 Li00)
    blk_zero(acc);
    blk_mma<false>(acc, L10, Y0);
    blk_each([&](int mi, int ni, int q, int rr, int c) { LT[rr][c] = acc[mi][ni][q]; });
    __syncthreads();
    blk_zero(acc);
    blk_mma<false>(acc, Y1, LT);
    blk_each([&](int mi, int ni, int q, int rr, int c) {
      if (rr < m1) {
        Li[(size_t)(NB + rr) * r + c] = -acc[mi][ni][q];
        if (c < m1) Li[(size_t)(NB + rr) * r + NB + c] = Y1[rr][c];
      }
    });
  }
  blk_each([&](int mi, int ni, int q, int rr, int c) {
    if (rr < m0 && c < m0) Li[(size_t)rr * r + c] = Y0[rr][c];
    if (rr < m0 && c < m1) Li[(size_t)rr * r + NB + c] = 0.0;
  });
  if (tid == 0) *counter = 0u;  // ready for the next launch
}

// V[i][c] = sum_t Z[i][t] Li[c][t] (V = Z Li^T), rows [64 blockIdx.x, +64)
__global__ __launch_bounds__(256) void k_apply(const double* __restrict__ Z, int n, int r,
                                               const double* __restrict__ Li, double* __restrict__ V) {
  __shared__ __attribute__((aligned(16))) double Zs0[NB][LDP];
  __shared__ __attribute__((aligned(16))) double Zs1[NB][LDP];
  __shared__ __attribute__((aligned(16))) double Lb0[NB][LDP];
  __shared__ __attribute__((aligned(16))) double Lb1[NB][LDP];
  const int tid = threadIdx.x, i0 = NB * blockIdx.x;
  const bool two = r > NB;
  auto load = [&](double (*D)[LDP], const double* S, int ld, int r0, int c0, int rmax, int cmax) {
    double v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q, rr = e >> 6, c = e & 63;
      v[q] = (r0 + rr < rmax && c0 + c < cmax) ? S[(size_t)(r0 + rr) * ld + c0 + c] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      D[e >> 6][e & 63] = v[q];
    }
  };
  load(Zs0, Z, r, i0, 0, n, r);
  load(Lb0, Li, r, 0, 0, r, r);
  if (two) {
    load(Zs1, Z, r, i0, NB, n, r);
    load(Lb1, Li, r, NB, 0, r, r);
  }
  __syncthreads();
  f64x4 acc0[2][2], acc1[2][2];
  blk_zero(acc0);
  blk_mma<true>(acc0, Zs0, Lb0);
  if (two) {
    blk_zero(acc1);
    blk_mma<true>(acc1, Zs0, Lb1);
    __syncthreads();
    load(Lb0, Li, r, NB, NB, r, r);
    __syncthreads();
    blk_mma<true>(acc1, Zs1, Lb0);
  }
  blk_each([&](int mi, int ni, int q, int rr, int c) {
    if (i0 + rr < n) {
      if (c < r) V[(size_t)(i0 + rr) * r + c] = acc0[mi][ni][q];
      if (two && NB + c < r) V[(size_t)(i0 + rr) * r + NB + c] = acc1[mi][ni][q];
    }
  });
}

// --------------------------------------------- Rayleigh-Ritz pieces -----
// The subspace iterations run on m >= r columns; every few steps the basis Q
// (orthonormal, dim x m) is rotated onto the Ritz vectors of the operator A
// in span(Q): with M = Q^T A Q = Y diag(theta) Y^T (theta descending), Q <- Q Y
// and Z = A Q <- Z Y.  The first r columns then hold the current estimate of
// the top-r eigenvectors, and the iteration stops once their residual
// ||A Q_r - Q_r diag(theta_r)||_F falls below a tolerance relative to
// ||theta_r||: by the sin-theta theorem the distance of span(Q_r) from the
// top-r eigenspace is at most that residual over the gap theta_r - lambda_{r+1}.
// The extra m - r columns make the subspace converge at the rate
// lambda_{m+1} / lambda_r instead of lambda_{r+1} / lambda_r.

constexpr int kRitzMax = 128;  // widest subspace
// LDS pitch of a column: even (16-byte aligned row pairs) and 64 bytes off
// a multiple of 128, so two 4-lane units reading 64 bytes of two columns in
// one 8-lane phase of a 16-byte read hit disjoint banks
constexpr int kRitzPitch = kRitzMax + 8;

// 1/x, 1/sqrt(x) and sqrt(x) for x > 0 from the hardware estimates and two
// Newton steps each (the estimates are good to about 2^-23), double precision
// to a few ulp without the long IEEE sequences on the rotation's serial path
__device__ __forceinline__ double rcp_f64(double x) {
  double y = __builtin_amdgcn_rcp(x);
  y = fma(y, fma(-x, y, 1.0), y);
  return fma(y, fma(-x, y, 1.0), y);
}
__device__ __forceinline__ double rsq_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x * y, y, 1.5);
  return y * fma(-0.5 * x * y, y, 1.5);
}
__device__ __forceinline__ double sqrt_f64(double x) { return x * rsq_f64(x); }

// Sum over the L (4, 8 or 16) lanes of an aligned group, the same bits on
// every lane (pairwise sums: lane pairs, quads, the two quads of a group of 8,
// then the two halves of a group of 16).
template <int L>
__device__ __forceinline__ double lane_sum(double x) {
  auto mv = [](double v, auto ctrl) {
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)b, decltype(ctrl)::value, 0xF, 0xF, true);
    const unsigned hi =
        (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), decltype(ctrl)::value, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
  };
  x += mv(x, std::integral_constant<int, 0xB1>{});  // quad_perm [1,0,3,2]
  x += mv(x, std::integral_constant<int, 0x4E>{});  // quad_perm [2,3,0,1]
  if constexpr (L >= 8) x += mv(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
  if constexpr (L == 16) x += mv(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

// This lane's part of ||x||^2 over its T row pairs (even and odd rows
// summed apart, then added).
template <int T>
__device__ __forceinline__ double sqnorm(const f64x2 (&x)[T]) {
  double s0 = 0.0, s1 = 0.0;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    s0 = fma(x[t][0], x[t][0], s0);
    s1 = fma(x[t][1], x[t][1], s1);
  }
  return s0 + s1;
}

// Eigenpairs of a symmetric positive semidefinite m x m matrix (m <= 128) by
// one-sided (Hestenes) Jacobi on B = M: rotations of column pairs until all
// columns are mutually orthogonal, B J = U diag(sigma); for M = M^T >= 0 the
// singular values are the eigenvalues and U holds the eigenvectors, so no
// rotation needs to be accumulated.  Each unit of L lanes holds its two
// columns in registers (lane sub: rows 2 sub + 2 L t and the next, t < T);
// between rounds a column that changes units goes through its home slot in
// LDS, written only when it was rotated since it was read, and the schedule
// above keeps that to about one column per unit and round (one barrier per
// round).  A pair is rotated when |b_p . b_q| > 1e-15 ||b_p|| ||b_q||
// (p < q); sweeps stop when none is (at most 40).  Writes Y[i][k] (m x m
// row-major, column k the eigenvector of the k-th largest eigenvalue) and
// theta[k].  One workgroup of L lanes per column pair (at most 64 L).
constexpr int kRitzSweeps = 40;
template <int L, int T>
__global__ __launch_bounds__(L * 64) void k_ritz(const double* __restrict__ M, int m, double* __restrict__ Y,
                                              double* __restrict__ theta) {
  __shared__ __attribute__((aligned(16))) double Bc[kRitzMax][kRitzPitch];  // Bc[c][i] = B[i][c]
  __shared__ double sig[kRitzMax];
  __shared__ int rank_of[kRitzMax];
  __shared__ int rotated[kRitzSweeps];
  // the sweep's schedule, [round][unit] = a | b << 8 (0xffff: idle); at most
  // mp <= kRitzMax rounds of mp / 2 units
  __shared__ unsigned short sched[kRitzMax * kRitzMax / 2];
  const int tid = threadIdx.x, nth = blockDim.x;
  const int mp = (m + 1) & ~1;  // even number of columns (a zero column pads)
  const int h = mp / 2, R = ritz_rounds(mp);
  for (int e = tid; e < mp * kRitzMax; e += nth) {
    const int c = e / kRitzMax, i = e % kRitzMax;
    Bc[c][i] = (c < m && i < m) ? 0.5 * (M[(size_t)i * m + c] + M[(size_t)c * m + i]) : 0.0;
  }
  for (int e = tid; e < R * h; e += nth) {
    int sa, sb;
    ritz_assign(mp, e / h, e % h, sa, sb);
    sched[e] = sa < 0 ? 0xffff : (unsigned short)(sa | sb << 8);
  }
  if (tid < kRitzSweeps) rotated[tid] = 0;
  __syncthreads();
  const int u = tid / L, sub = tid % L;
  f64x2 x0[T] = {}, x1[T] = {};  // the unit's columns a (x0) and b (x1)
  auto slot = [&](int ri, int& sa, int& sb) {
    const unsigned v = u < h ? sched[ri * h + u] : 0xffffu;
    sa = v == 0xffffu ? -1 : (int)(v & 0xff);
    sb = v == 0xffffu ? -1 : (int)(v >> 8);
  };
  int a, b;
  slot(0, a, b);
  bool d0 = false, d1 = false;  // the column differs from its home copy
  if (a >= 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      x0[t] = *(const f64x2*)&Bc[a][2 * sub + 2 * L * t];
      x1[t] = *(const f64x2*)&Bc[b][2 * sub + 2 * L * t];
    }
  }
  double n0 = 0.0;     // ||x0||^2, carried into the next round when x0 stays
  bool n0ok = false;
  for (int sweep = 0; sweep < kRitzSweeps; ++sweep) {
    for (int ri = 0; ri < R; ++ri) {
      if (a >= 0) {
        // two accumulators per sum (rows 2 sub + 2 L t and the next) halve
        // the dependent chain
        double n1a = 0.0, n1b = 0.0, gaa = 0.0, gab = 0.0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          n1a = fma(x1[t][0], x1[t][0], n1a);
          n1b = fma(x1[t][1], x1[t][1], n1b);
          gaa = fma(x0[t][0], x1[t][0], gaa);
          gab = fma(x0[t][1], x1[t][1], gab);
        }
        if (!n0ok) n0 = lane_sum<L>(sqnorm<T>(x0));
        const double n1 = lane_sum<L>(n1a + n1b);
        const double ga = lane_sum<L>(gaa + gab);
        if (ga * ga > 1e-30 * n0 * n1) {  // |ga| > 1e-15 ||b_a|| ||b_b||
          // rotation of (p, q) = (min, max) of (a, b): b_p' = c b_p - s b_q,
          // b_q' = s b_p + c b_q, with tan = t zeroing their product
          // t = 2 ga sign(d) / (|d| + sqrt(d^2 + 4 ga^2)), d = be - al: the
          // smaller root of t^2 + 2 zeta t - 1 = 0, zeta = d / (2 ga).  t needs
          // only near double precision (a slightly-off angle is fixed by the
          // next sweep); c = 1/sqrt(1 + t^2) is exact to rounding, so (c, s)
          // stays an orthogonal rotation and no column is rescaled.
          const bool ap = a < b;
          const double d = ap ? n1 - n0 : n0 - n1, g2 = 2.0 * ga;
          const double rr = fma(d, d, g2 * g2);
          double y = __builtin_amdgcn_rsq(rr);
          y = y * fma(-0.5 * rr * y, y, 1.5);
          const double den = fabs(d) + rr * y;
          double w = __builtin_amdgcn_rcp(den);
          w = fma(w, fma(-den, w, 1.0), w);
          const double tn = (d >= 0.0 ? g2 : -g2) * w;
          const double cs = rsq_f64(fma(tn, tn, 1.0)), sn = cs * tn, s0 = ap ? sn : -sn;
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
              const double p = x0[t][v], q = x1[t][v];
              x0[t][v] = cs * p - s0 * q;
              x1[t][v] = cs * q + s0 * p;
            }
          d0 = d1 = true;
          n0ok = false;
          if (sub == 0) rotated[sweep] = 1;
        }
      }
      // hand over: changed columns leaving the unit go home, then the
      // arrivals are read.  Inside a cross level a unit keeps x0 and swaps
      // x1 (the common case, no selects); level changes take the general way.
      int na, nb;
      slot(ri + 1 < R ? ri + 1 : 0, na, nb);
      const bool same0 = a >= 0 && na == a && nb != b;
      if (same0) {
        if (d1)
#pragma unroll
          for (int t = 0; t < T; ++t) *(f64x2*)&Bc[b][2 * sub + 2 * L * t] = x1[t];
        if (!n0ok) n0 = lane_sum<L>(sqnorm<T>(x0));  // overlaps the wait below
        n0ok = true;
      } else if (a >= 0) {
        const bool keep0 = a == na || a == nb, keep1 = b == na || b == nb;
        if (!keep0 && d0)
#pragma unroll
          for (int t = 0; t < T; ++t) *(f64x2*)&Bc[a][2 * sub + 2 * L * t] = x0[t];
        if (!keep1 && d1)
#pragma unroll
          for (int t = 0; t < T; ++t) *(f64x2*)&Bc[b][2 * sub + 2 * L * t] = x1[t];
      }
      __syncthreads();
      if (same0) {
#pragma unroll
        for (int t = 0; t < T; ++t) x1[t] = *(const f64x2*)&Bc[nb][2 * sub + 2 * L * t];
        d1 = false;
      } else if (na >= 0) {
        // new x0 = column na, new x1 = column nb, each kept or read
        const bool s0a = na == a, s1a = na == b, s0b = nb == a, s1b = nb == b;
        const bool e0 = s0a ? d0 : s1a && d1, e1 = s0b ? d0 : s1b && d1;
        d0 = e0;
        d1 = e1;
        n0ok = false;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const f64x2 o0 = x0[t], o1 = x1[t];
          x0[t] = s0a ? o0 : s1a ? o1 : *(const f64x2*)&Bc[na][2 * sub + 2 * L * t];
          x1[t] = s0b ? o0 : s1b ? o1 : *(const f64x2*)&Bc[nb][2 * sub + 2 * L * t];
        }
      }
      a = na;
      b = nb;
    }
    if (rotated[sweep] == 0) break;  // read after the last round's barrier; set before it
  }
  // the units hold every column (round 0 pairs them all): norms and home copies
  if (a >= 0) {
    double n0 = 0.0, n1 = 0.0;
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        n0 = fma(x0[t][v], x0[t][v], n0);
        n1 = fma(x1[t][v], x1[t][v], n1);
      }
      if (d0) *(f64x2*)&Bc[a][2 * sub + 2 * L * t] = x0[t];
      if (d1) *(f64x2*)&Bc[b][2 * sub + 2 * L * t] = x1[t];
    }
    n0 = lane_sum<L>(n0);
    n1 = lane_sum<L>(n1);
    if (sub == 0) {
      if (a < m) sig[a] = sqrt(n0);
      if (b < m) sig[b] = sqrt(n1);
    }
  }
  __syncthreads();
  if (tid < m) {
    const double sc = sig[tid];
    int rank = 0;
    for (int d = 0; d < m; ++d) rank += (sig[d] > sc || (sig[d] == sc && d < tid)) ? 1 : 0;
    rank_of[tid] = rank;
    theta[rank] = sc;
  }
  __syncthreads();
  for (int e = tid; e < m * m; e += nth) {
    const int i = e / m, c = e % m;
    const double sc = sig[c];
    Y[(size_t)i * m + rank_of[c]] = sc > 0.0 ? Bc[c][i] / sc : 0.0;
  }
}

// part[b] = this block's share of sum over i < dim, c < r of
// (Z[i][c] - theta[c] Q[i][c])^2 (Q, Z of pitch m), fixed order per block
__global__ __launch_bounds__(256) void k_ritz_resid(const double* __restrict__ Q, const double* __restrict__ Z,
                                                    const double* __restrict__ theta, int dim, int m, int r,
                                                    double* __restrict__ part) {
  __shared__ double red[256];
  const long long cnt = (long long)dim * r, stride = (long long)gridDim.x * 256;
  double acc = 0.0;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < cnt; e += stride) {
    const long long i = e / r;
    const int c = (int)(e % r);
    const double v = Z[i * m + c] - theta[c] * Q[i * m + c];
    acc = fma(v, v, acc);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// conv[0] = 1 if the residual meets the tolerance (else 0), conv[1] = the
// squared residual, conv[2] = ||theta_r||^2
__global__ __launch_bounds__(256) void k_ritz_conv(const double* __restrict__ part, int np,
                                                   const double* __restrict__ theta, int r, double tol,
                                                   double* __restrict__ conv) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < np; i += 256) acc += part[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double t2 = 0.0;
    for (int c = 0; c < r; ++c) t2 = fma(theta[c], theta[c], t2);
    conv[0] = red[0] <= tol * tol * t2 ? 1.0 : 0.0;
    conv[1] = red[0];
    conv[2] = t2;
  }
}

// V[i][c] = Q[i][c] for c < r (Q of pitch m, V of pitch r)
__global__ void k_cols(const double* __restrict__ Q, int dim, int m, int r, double* __restrict__ V) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long long)dim * r) return;
  const long long i = e / r;
  V[e] = Q[i * m + (int)(e % r)];
}

// lam = lam_abs + lam_rel * mean(diag H); clears the slot's flags and the
// Gram kernels' arrival counter.
__global__ __launch_bounds__(256) void k_lora_lambda(const double* __restrict__ H, int n, double lam_abs,
                                                     double lam_rel, Slot* __restrict__ slot,
                                                     unsigned* __restrict__ counter) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += H[(size_t)i * n + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    slot->lam = lam_abs + lam_rel * red[0] / (double)n;
    slot->info = 0;
    slot->nonfinite = 0;
    *counter = 0u;
  }
}

// A[i][j] (j <= i) = Ht[nt-1-i][nt-1-j] + lam delta_ij with
// Ht = [[H, HV], [V^T H, M]], M = V^T H V.  4 rows per workgroup.
__global__ __launch_bounds__(256) void k_lora_assemble(const double* __restrict__ H64, const double* __restrict__ HV,
                                                       const double* __restrict__ M, int n, int r,
                                                       double* __restrict__ A, Slot* __restrict__ slot) {
  const int nt = n + r;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= nt) return;
  const double lam = slot->lam;
  const int I = nt - 1 - i;
  bool bad = false;
  for (int j = threadIdx.x & 63; j <= i; j += 64) {
    const int J = nt - 1 - j;  // J >= I
    double v;
    if (J < n) v = H64[(size_t)I * n + J];
    else if (I < n) v = HV[(size_t)I * r + (J - n)];
    else v = M[(size_t)(I - n) * r + (J - n)];
    bad |= !__builtin_isfinite(v);
    A[(size_t)i * nt + j] = v + (i == j ? lam : 0.0);
  }
  if (bad) atomicOr(&slot->nonfinite, 1);
}

// L[n][r] = V (fp32); R[k][row] = Ww[row][n + k].
__global__ void k_lora_extract(const double* __restrict__ V, const float* __restrict__ Ww, int out, int n, int r,
                               float* __restrict__ L, float* __restrict__ R) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (long long)n * r) L[i] = (float)V[i];
  if (i < (long long)r * out) {
    const long long k = i / out, row = i % out;
    R[i] = Ww[row * (n + r) + n + k];
  }
}

inline int cdivl(long long a, long long b) { return (int)((a + b - 1) / b); }

#define LLAUNCH(name, ...)                                                                          \
  do {                                                                                              \
    if ((rc = hk.launch(name, [&] { hipLaunchKernelGGL(__VA_ARGS__); return hipGetLastError(); }))) \
      return rc;                                                                                    \
  } while (0)

// C = the product; split-K partials go to scratch and are summed by k_dsum
int dgemm(hipStream_t st, const LoraHooks& hk, const DGemm& g0, double* C, double* scratch) {
  DGemm g = g0;
  const int tiles = cdivl(g.M, 64) * cdivl(g.N, 64);
  if (g.ksplit < 1) g.ksplit = 1;
  g.P = (g.ksplit == 1) ? C : scratch;
  int rc;
  LLAUNCH("k_dgemm", k_dgemm, dim3(tiles, g.ksplit), dim3(256), 0, st, g);
  if (g.ksplit == 1) return 0;
  const long long MN = (long long)g.M * g.N;
  LLAUNCH("k_dsum", k_dsum, dim3(cdivl(MN, 256)), dim3(256), 0, st, (const double*)scratch, C, MN, g.ksplit);
  return 0;
}

// split-K: about 128 of K per workgroup (4 chunks), at most 16 partials
inline int ksplit_for(int K) { return std::max(1, std::min(16, K / 128)); }

// one Cholesky-QR pass over nrows x r: Vout = Zin L^{-T}, Zin^T Zin = L L^T
int orth(hipStream_t st, const LoraHooks& hk, const double* Zin, double* Vout, int nrows, int r, double* Gp,
         double* Li, unsigned* cnt) {
  const int nrb = cdivl(nrows, 64), rows_per = 64 * cdivl(nrb, std::min(kGramParts, nrb));
  const int nparts = cdivl(nrows, rows_per);
  int rc;
  LLAUNCH("k_gram_chol", k_gram_chol, dim3(nparts), dim3(256), 0, st, Zin, nrows, r, rows_per, Gp, Li, cnt);
  LLAUNCH("k_apply", k_apply, dim3(nrb), dim3(256), 0, st, Zin, nrows, r, (const double*)Li, Vout);
  return 0;
}

// k_ritz<L, T> for m <= kRitzMax: L lanes per column pair, T = ceil(m / 2L)
// row pairs per lane.
template <int L, int T>
int ritz_launch(hipStream_t st, const LoraHooks& hk, const double* M, int m, double* Y, double* theta, int t) {
  if constexpr (T > kRitzMax / (2 * L)) {
    return GPTQ_ERR_UNSUPPORTED;
  } else {
    if (t != T) return ritz_launch<L, T + 1>(st, hk, M, m, Y, theta, t);
    const int nth = 64 * cdivl(L * ((m + 1) / 2), 64);
    const auto kern = k_ritz<L, T>;
    int rc;
    LLAUNCH("k_ritz", kern, dim3(1), dim3(nth), 0, st, M, m, Y, theta);
    return 0;
  }
}
// 8 lanes per pair: 4 and 16 measured within a few percent, neither faster
constexpr int kRitzLanes = 8;
int ritz(hipStream_t st, const LoraHooks& hk, const double* M, int m, double* Y, double* theta) {
  constexpr int L = kRitzLanes;
  return ritz_launch<L, 1>(st, hk, M, m, Y, theta, cdivl(m, 2 * L));
}

// Width of the iterated subspace for the top-r eigenvectors in dimension dim.
inline int sub_width(int dim, int r) { return std::max(r, std::min({kRitzMax, dim, std::max(r + 32, 64)})); }

// Buffers of one top-subspace computation (dim x m unless noted).
struct SubBufs {
  double *Q, *Z, *Qn, *Zn;
  double *M, *Y, *theta;  // m x m, m x m, m
  double *parts, *conv;   // kParts, 4
  double *S;              // split-K partials: ksplit_for(dim) * m * m at least
  double *Gp, *Li;
  unsigned* cnt;
};

constexpr int kResidParts = 256;

// Orthonormal V[dim][r] spanning the top-r eigenvectors of the symmetric
// positive semidefinite operator op (op(Q, Z): Z = A Q for dim x m blocks),
// by subspace iteration with Cholesky-QR on m columns from a fixed start, a
// Rayleigh-Ritz check every kCheck steps (see k_ritz), and a final
// Cholesky-QR pass on the r Ritz vectors.  *converged = whether the residual
// test passed before kMaxIters; V holds the last Ritz vectors either way.
// Vtmp: dim x r scratch.  Each check reads one flag back (a host wait).
int top_subspace(hipStream_t st, const LoraHooks& hk, const std::function<int(const double*, double*)>& op, int dim,
                 int m, int r, const SubBufs& b, double* V, double* Vtmp, bool* converged) {
  int rc;
  double *Q = b.Q, *Z = b.Z, *Qn = b.Qn, *Zn = b.Zn;
  LLAUNCH("k_start_block", k_start_block, dim3(cdivl((long long)dim * m, 256)), dim3(256), 0, st, Q, dim, m);
  *converged = false;
  for (int it = 0; it < kMaxIters; ++it) {
    if ((rc = op(Q, Z))) return rc;
    const bool last = it == kMaxIters - 1;
    if (it >= 1 && (it % kCheck == kCheck - 1 || last)) {  // Q is orthonormal from step 1 on
      DGemm g{Q, 1, m, Z, m, 1, nullptr, m, m, dim, ksplit_for(dim)};  // M = Q^T Z
      if ((rc = dgemm(st, hk, g, b.M, b.S))) return rc;
      if ((rc = ritz(st, hk, b.M, m, b.Y, b.theta))) return rc;
      DGemm gq{Q, m, 1, b.Y, m, 1, nullptr, dim, m, m, 1};  // Qn = Q Y
      if ((rc = dgemm(st, hk, gq, Qn, b.S))) return rc;
      DGemm gz{Z, m, 1, b.Y, m, 1, nullptr, dim, m, m, 1};  // Zn = Z Y
      if ((rc = dgemm(st, hk, gz, Zn, b.S))) return rc;
      LLAUNCH("k_ritz_resid", k_ritz_resid, dim3(kResidParts), dim3(256), 0, st, (const double*)Qn,
              (const double*)Zn, (const double*)b.theta, dim, m, r, b.parts);
      LLAUNCH("k_ritz_conv", k_ritz_conv, dim3(1), dim3(256), 0, st, (const double*)b.parts, kResidParts,
              (const double*)b.theta, r, kTol, b.conv);
      double hc[3];
      if ((rc = hk.read(b.conv, hc, sizeof(hc)))) return rc;
      std::swap(Q, Qn);
      std::swap(Z, Zn);
      if (hc[0] != 0.0) {
        *converged = true;
        break;
      }
      if (last) break;
    }
    if ((rc = orth(st, hk, Z, Q, dim, m, b.Gp, b.Li, b.cnt))) return rc;
  }
  LLAUNCH("k_cols", k_cols, dim3(cdivl((long long)dim * r, 256)), dim3(256), 0, st, (const double*)Q, dim, m, r,
          Vtmp);
  return orth(st, hk, Vtmp, V, dim, r, b.Gp, b.Li, b.cnt);
}

// Lays a SubBufs out with take(bytes) -> pointer.
template <class Take>
void sub_layout(int dim, int m, Take&& take, SubBufs* b) {
  const size_t dm = (size_t)dim * m * 8;
  b->Q = (double*)take(dm);
  b->Z = (double*)take(dm);
  b->Qn = (double*)take(dm);
  b->Zn = (double*)take(dm);
  b->M = (double*)take((size_t)m * m * 8);
  b->Y = (double*)take((size_t)m * m * 8);
  b->theta = (double*)take((size_t)m * 8);
  b->parts = (double*)take((size_t)kResidParts * 8);
  b->conv = (double*)take(4 * 8);
}

// ----------------------------------------------- refinement: OLrC, Bid-Up -----
// (GPTQ-intrinsic LoRA technical summary, section 4: OLrC re-fits L, R for a
// fixed Q, Bid-Up moves Q on its fixed grid for fixed L, R; they alternate
// and the layer objective never increases.)
//
// OLrC: with E = W - What, the rank-r correction C minimising
// tr((E - C) H (E - C)^T) is C = P P^T E, P the top-r eigenvectors of
// E H E^T (Eckart-Young on E F for any H = F F^T), so no square root or
// inverse of H is needed.  P comes from the same checked subspace iteration
// as V_r, on the operator Q -> EH (E^T Q) with EH = E H formed once; then
// L = E^T P, R = P^T (C = R^T L^T).  Its objective is
// J = sum(g * E) with g = (E - C) H = EH - P (P^T EH), which is also the
// gradient Bid-Up starts from.
// Bid-Up: one pass of the column sweep in its Bid-Up mode, on g (fp32) with
// U = H (fp32): the sweep's lazy block updates carry the moves forward.

// E = W - What - C (C may be null); What = s (q - z) in fp32 as stored
__global__ void k_resid(const float* __restrict__ W, const uint8_t* __restrict__ codes,
                        const float* __restrict__ scales, const uint8_t* __restrict__ zeros, int out, int n,
                        int group, const double* __restrict__ C, double* __restrict__ E) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)out * n) return;
  const int row = (int)(i / n), col = (int)(i % n);
  const int ng = group ? n / group : 1;
  const size_t gi = (size_t)row * ng + (group ? col / group : 0);
  const float s = scales[gi], z = (float)zeros[gi];
  const float wh = s * ((float)codes[i] - z);
  E[i] = (double)W[i] - (double)wh - (C ? C[i] : 0.0);
}

// g = EH - Y (Y may be null), g32 = fl32(g); part[b] = this block's share of
// sum(g * E), each thread over a fixed stride of the elements (fixed order)
__global__ __launch_bounds__(256) void k_gfinal(const double* __restrict__ EH, const double* __restrict__ Y,
                                                const double* __restrict__ E, long long cnt,
                                                float* __restrict__ g32, double* __restrict__ part) {
  __shared__ double red[256];
  const long long stride = (long long)gridDim.x * 256;
  double acc = 0.0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < cnt; i += stride) {
    const double g = EH[i] - (Y ? Y[i] : 0.0);
    g32[i] = (float)g;
    acc += g * E[i];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// dst[0] = sum of part[0..np) (fixed order) + (add ? add[0] : 0)
__global__ __launch_bounds__(256) void k_sum_parts(const double* __restrict__ part, int np,
                                                   const double* __restrict__ add, double* __restrict__ dst) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < np; i += 256) acc += part[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) dst[0] = red[0] + (add ? add[0] : 0.0);
}

__global__ void k_f64_to_f32(const double* __restrict__ a, float* __restrict__ b, long long cnt) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cnt) b[i] = (float)a[i];
}

__global__ void k_f32_to_f64(const float* __restrict__ a, double* __restrict__ b, long long cnt) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cnt) b[i] = (double)a[i];
}

// L[n][r] = T (fp32); R[k][i] = P[i][k]
__global__ void k_olrc_out(const double* __restrict__ T, const double* __restrict__ P, int n, int out, int r,
                           float* __restrict__ L, float* __restrict__ R) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (long long)n * r) L[i] = (float)T[i];
  if (i < (long long)r * out) {
    const long long k = i / out, row = i % out;
    R[i] = (float)P[row * r + k];
  }
}

// the arrival counter of the Gram kernels and the device constant 0
__global__ void k_ref_init(unsigned* __restrict__ cnt, double* __restrict__ dev) {
  if (threadIdx.x == 0) {
    *cnt = 0u;
    dev[0] = 0.0;
  }
}

constexpr int kParts = 512;  // partial sums of the objective dot product

struct RefBufs {
  double *E, *EH, *Y, *P, *Pt, *T, *X, *S, *Gp, *Li, *parts, *Ld, *Rd, *dev;
  unsigned* cnt;
  float *g32, *H32;
  SubBufs sb;  // the top-r subspace of E H E^T (dimension out)
};

// Lay the refinement buffers out from offset off of base (base may be null
// to size them); returns the end offset.
size_t ref_layout(int out, int n, int r, uint8_t* base, size_t off, RefBufs* b) {
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return base ? base + o : nullptr;
  };
  const size_t on = (size_t)out * n;
  const int ks = std::max(ksplit_for(n), ksplit_for(out));
  const int m = sub_width(out, r);
  b->E = (double*)take(on * 8);
  b->EH = (double*)take(on * 8);
  b->Y = (double*)take(on * 8);
  b->P = (double*)take((size_t)out * r * 8);
  b->Pt = (double*)take((size_t)out * r * 8);
  b->T = (double*)take((size_t)n * m * 8);
  b->X = (double*)take((size_t)r * n * 8);
  b->S = (double*)take((size_t)ks * std::max(out, n) * m * 8);
  b->Gp = (double*)take((size_t)kGramParts * 3 * 64 * 64 * 8);
  b->Li = (double*)take((size_t)m * m * 8);
  b->parts = (double*)take((size_t)kParts * 8);
  b->Ld = (double*)take((size_t)n * r * 8);
  b->Rd = (double*)take((size_t)r * out * 8);
  b->dev = (double*)take(8 * 8);
  b->cnt = (unsigned*)take(sizeof(unsigned));
  b->g32 = (float*)take(on * 4);
  b->H32 = (float*)take((size_t)n * n * 4);
  sub_layout(out, m, take, &b->sb);
  b->sb.S = b->S;
  b->sb.Gp = b->Gp;
  b->sb.Li = b->Li;
  b->sb.cnt = b->cnt;
  return off;
}

// EH[out][n] = E[out][n] H[n][n] (H symmetric, so E H = E H^T: both operands
// k-contiguous) on the fp64 MFMA ring when the shapes allow, else k_dgemm
int e_times_h(hipStream_t st, const LoraHooks& hk, const double* E, const double* H, double* EH, double* S, int out,
              int n) {
  const bool ring = n % 16 == 0 && ((uintptr_t)E & 15) == 0 && ((uintptr_t)H & 15) == 0 && ((uintptr_t)EH & 15) == 0;
  if (ring) return hk.gemm_nt(E, H, EH, out, n, n, n);
  DGemm g{E, n, 1, H, n, 1, nullptr, out, n, n, 1};
  return dgemm(st, hk, g, EH, S);
}

int run_gfinal(hipStream_t st, const LoraHooks& hk, const RefBufs& b, const double* EH, const double* Y,
               const double* E, long long cnt, const double* add, double* J) {
  int rc;
  LLAUNCH("k_gfinal", k_gfinal, dim3(kParts), dim3(256), 0, st, EH, Y, E, cnt, b.g32, b.parts);
  LLAUNCH("k_sum_parts", k_sum_parts, dim3(1), dim3(256), 0, st, (const double*)b.parts, kParts, add, J);
  return 0;
}

// OLrC for the current codes: leaves g (fp32) for a Bid-Up pass in b.g32,
// J in *J (device), and (if L, R are given) the factors.
int olrc(hipStream_t st, const RefineIO& io, const LoraHooks& hk, const RefBufs& b, double* J, float* L, float* R) {
  const int out = io.out, n = io.n, r = io.r;
  const long long on = (long long)out * n;
  int rc;
  LLAUNCH("k_resid", k_resid, dim3(cdivl(on, 256)), dim3(256), 0, st, io.W, io.codes, io.scales, io.zeros, out, n,
          io.group, (const double*)nullptr, b.E);
  if ((rc = e_times_h(st, hk, b.E, io.H64, b.EH, b.S, out, n))) return rc;  // EH = E H
  const int m = sub_width(out, r);
  // A = E H E^T applied as EH (E^T Q)
  auto op = [&](const double* Q, double* Z) -> int {
    int rc2;
    DGemm t{b.E, 1, n, Q, m, 1, nullptr, n, m, out, ksplit_for(out)};  // T = E^T Q
    if ((rc2 = dgemm(st, hk, t, b.T, b.S))) return rc2;
    DGemm z{b.EH, n, 1, b.T, m, 1, nullptr, out, m, n, ksplit_for(n)};  // Z = EH T
    return dgemm(st, hk, z, Z, b.S);
  };
  double* P = b.P;
  bool conv = false;
  if ((rc = top_subspace(st, hk, op, out, m, r, b.sb, P, b.Pt, &conv))) return rc;
  if (!conv) hk.not_converged();
  {
    DGemm t{b.E, 1, n, P, r, 1, nullptr, n, r, out, ksplit_for(out)};  // L = E^T P
    if ((rc = dgemm(st, hk, t, b.T, b.S))) return rc;
    DGemm x{P, 1, r, b.EH, n, 1, nullptr, r, n, out, ksplit_for(out)};  // X = P^T EH
    if ((rc = dgemm(st, hk, x, b.X, b.S))) return rc;
    DGemm y{P, r, 1, b.X, n, 1, nullptr, out, n, r, 1};  // Y = P X
    if ((rc = dgemm(st, hk, y, b.Y, b.S))) return rc;
  }
  if ((rc = run_gfinal(st, hk, b, b.EH, b.Y, b.E, on, nullptr, J))) return rc;
  if (L && R) {
    const long long ne = std::max((long long)n * r, (long long)r * out);
    LLAUNCH("k_olrc_out", k_olrc_out, dim3(cdivl(ne, 256)), dim3(256), 0, st, (const double*)b.T, (const double*)P, n,
            out, r, L, R);
  }
  return 0;
}

// One Bid-Up pass from b.g32 (g of the current codes) with H in b.H32;
// *J = *J0 + the summed objective change of the moves (device values).
int bid_up_pass(hipStream_t st, const RefineIO& io, const LoraHooks& hk, const RefBufs& b, const double* J0,
                double* J) {
  QuantJob q{b.g32, io.out, io.n, io.n, b.H32, io.bits, io.group, io.block, io.codes, io.scales, io.zeros,
             nullptr, b.dev, b.dev + 2, nullptr};
  q.mode = 1;
  int rc = hk.quantize(q);
  if (rc) return rc;
  LLAUNCH("k_sum_parts", k_sum_parts, dim3(1), dim3(256), 0, st, (const double*)(b.dev + 2), 1, J0, J);
  return 0;
}

int check_refine(const RefineIO& io, const LoraHooks& hk) {
  if (io.r < 1 || io.r > 128 || io.r > io.out || io.r > io.n)
    return hk.set_err(GPTQ_ERR_UNSUPPORTED, "rank must be in 1..min(128, out, n)");
  return 0;
}

}  // namespace

int run_olrc(hipStream_t st, const RefineIO& io, const LoraHooks& hk, double* J) {
  int rc = check_refine(io, hk);
  if (rc) return rc;
  RefBufs b;
  const size_t bytes = ref_layout(io.out, io.n, io.r, nullptr, 0, &b);
  uint8_t* base = (uint8_t*)hk.ensure(bytes);
  if (!base) return GPTQ_ERR_NO_MEMORY;
  ref_layout(io.out, io.n, io.r, base, 0, &b);
  LLAUNCH("k_ref_init", k_ref_init, dim3(1), dim3(64), 0, st, b.cnt, b.dev);
  return olrc(st, io, hk, b, J, io.L, io.R);
}

int run_bid_up(hipStream_t st, const RefineIO& io, const LoraHooks& hk, double* J) {
  int rc = check_refine(io, hk);
  if (rc) return rc;
  const int out = io.out, n = io.n, r = io.r;
  const long long on = (long long)out * n;
  RefBufs b;
  const size_t bytes = ref_layout(out, n, r, nullptr, 0, &b);
  uint8_t* base = (uint8_t*)hk.ensure(bytes);
  if (!base) return GPTQ_ERR_NO_MEMORY;
  ref_layout(out, n, r, base, 0, &b);
  LLAUNCH("k_ref_init", k_ref_init, dim3(1), dim3(64), 0, st, b.cnt, b.dev);
  // C = R^T L^T in fp64, D = W - What - C, g = D H, J0 = sum(g * D)
  LLAUNCH("k_f32_to_f64", k_f32_to_f64, dim3(cdivl((long long)n * r, 256)), dim3(256), 0, st, (const float*)io.L,
          b.Ld, (long long)n * r);
  LLAUNCH("k_f32_to_f64", k_f32_to_f64, dim3(cdivl((long long)r * out, 256)), dim3(256), 0, st, (const float*)io.R,
          b.Rd, (long long)r * out);
  {
    DGemm c{b.Rd, 1, out, b.Ld, 1, r, nullptr, out, n, r, 1};
    if ((rc = dgemm(st, hk, c, b.Y, b.S))) return rc;
  }
  LLAUNCH("k_resid", k_resid, dim3(cdivl(on, 256)), dim3(256), 0, st, io.W, io.codes, io.scales, io.zeros, out, n,
          io.group, (const double*)b.Y, b.E);
  if ((rc = e_times_h(st, hk, b.E, io.H64, b.EH, b.S, out, n))) return rc;  // g = D H
  if ((rc = run_gfinal(st, hk, b, b.EH, nullptr, b.E, on, nullptr, b.dev + 4))) return rc;
  LLAUNCH("k_f64_to_f32", k_f64_to_f32, dim3(cdivl((long long)n * n, 256)), dim3(256), 0, st, io.H64, b.H32,
          (long long)n * n);
  return bid_up_pass(st, io, hk, b, b.dev + 4, J);
}

int run_lora(hipStream_t st, const LoraIO& io, const LoraHooks& hk) {
  const int n = io.n, r = io.r, nt = n + r, out = io.out;
  if (r > 128) return hk.set_err(GPTQ_ERR_UNSUPPORTED, "rank above 128 is not supported");
  if (io.rounds > 0 && r > out) return hk.set_err(GPTQ_ERR_UNSUPPORTED, "refinement needs rank <= out");
  // workspace layout
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const int ks_n = ksplit_for(n);  // split-K for K = n products
  const int m = sub_width(n, r);    // columns of the subspace iteration
  const size_t oH64 = take((size_t)n * n * 8), oV = take((size_t)n * r * 8),
               oZ = take((size_t)n * r * 8), oLi = take((size_t)m * m * 8),
               oM = take((size_t)r * r * 8), oHV = take((size_t)n * r * 8),
               oS = take((size_t)ks_n * n * m * 8),
               oGp = take((size_t)kGramParts * 3 * 64 * 64 * 8), oCnt = take(sizeof(unsigned)),
               oA = take((size_t)nt * nt * 8), oU = take((size_t)nt * nt * 4), oW = take((size_t)out * nt * 4);
  SubBufs sb;
  std::vector<size_t> sub_off;
  sub_layout(n, m, [&](size_t bytes) { sub_off.push_back(take(bytes)); return (void*)nullptr; }, &sb);
  RefBufs rb;
  const size_t oRef = off;
  if (io.rounds > 0) off = ref_layout(out, n, r, nullptr, off, &rb);
  uint8_t* base = (uint8_t*)hk.ensure(off);
  if (!base) return GPTQ_ERR_NO_MEMORY;
  if (io.rounds > 0) ref_layout(out, n, r, base, oRef, &rb);
  // slots: the call's Slot, then the refinement trace
  Slot* slot = (Slot*)hk.slots(sizeof(Slot) + (size_t)(2 * std::max(io.rounds, 0) + 2) * sizeof(double));
  if (!slot) return GPTQ_ERR_NO_MEMORY;
  double* trace = (double*)(slot + 1);
  double *H64 = (double*)(base + oH64), *V = (double*)(base + oV), *Z = (double*)(base + oZ),
         *Li = (double*)(base + oLi), *M = (double*)(base + oM), *HV = (double*)(base + oHV),
         *S = (double*)(base + oS), *Gp = (double*)(base + oGp), *A = (double*)(base + oA);
  unsigned* cnt = (unsigned*)(base + oCnt);
  float* U = (float*)(base + oU);
  float* Ww = (float*)(base + oW);
  {
    size_t k = 0;
    sub_layout(n, m, [&](size_t) { return (void*)(base + sub_off[k++]); }, &sb);
    sb.S = S;
    sb.Gp = Gp;
    sb.Li = Li;
    sb.cnt = cnt;
  }

  // H accurate to float64 rounding: the Schur complement below cancels the
  // top-r eigen-directions of H against a damping far below their size
  int rc = hk.hessian64(io.X, io.tokens, io.ldx, n, H64);
  if (rc) return rc;
  LLAUNCH("k_lora_lambda", k_lora_lambda, dim3(1), dim3(256), 0, st, (const double*)H64, n, io.lam_abs, io.lam_rel,
          slot, cnt);
  {
    auto op = [&](const double* Q, double* Zq) -> int {
      DGemm g{H64, n, 1, Q, m, 1, nullptr, n, m, n, ks_n};  // Zq = H Q
      return dgemm(st, hk, g, Zq, S);
    };
    bool conv = false;
    if ((rc = top_subspace(st, hk, op, n, m, r, sb, V, Z, &conv))) return rc;
    if (!conv) hk.not_converged();
  }
  {
    DGemm g{H64, n, 1, V, r, 1, nullptr, n, r, n, ks_n};  // HV = H V
    if ((rc = dgemm(st, hk, g, HV, S))) return rc;
    DGemm m{V, 1, r, HV, r, 1, nullptr, r, r, n, ks_n};  // M = V^T H V
    if ((rc = dgemm(st, hk, m, M, S))) return rc;
  }
  LLAUNCH("k_lora_assemble", k_lora_assemble, dim3(cdivl(nt, 4)), dim3(256), 0, st, (const double*)H64,
          (const double*)HV, (const double*)M, n, r, A, slot);
  if ((rc = hk.factor(A, nt, U, slot))) return rc;
  QuantJob J{io.W, out, n, nt, U, io.bits, io.group, io.block, io.codes, io.scales, io.zeros, nullptr,
             &slot->lam, slot->obj, Ww};
  if ((rc = hk.quantize(J))) return rc;
  if (io.rounds <= 0) {
    const long long ne = std::max((long long)n * r, (long long)r * out);
    LLAUNCH("k_lora_extract", k_lora_extract, dim3(cdivl(ne, 256)), dim3(256), 0, st, (const double*)V,
            (const float*)Ww, out, n, r, io.L, io.R);
    return 0;
  }
  // refinement: rounds of OLrC then Bid-Up, and a last OLrC for L, R
  RefineIO ri{io.W, out, n, H64, r, io.bits, io.group, io.block, io.codes, io.scales, io.zeros, io.L, io.R};
  LLAUNCH("k_ref_init", k_ref_init, dim3(1), dim3(64), 0, st, rb.cnt, rb.dev);
  LLAUNCH("k_sum_parts", k_sum_parts, dim3(1), dim3(256), 0, st, (const double*)slot->obj, 1,
          (const double*)nullptr, trace);
  LLAUNCH("k_f64_to_f32", k_f64_to_f32, dim3(cdivl((long long)n * n, 256)), dim3(256), 0, st,
          (const double*)H64, rb.H32, (long long)n * n);
  for (int t = 0; t < io.rounds; ++t) {
    if ((rc = olrc(st, ri, hk, rb, trace + 1 + 2 * t, nullptr, nullptr))) return rc;
    if ((rc = bid_up_pass(st, ri, hk, rb, trace + 1 + 2 * t, trace + 2 + 2 * t))) return rc;
  }
  return olrc(st, ri, hk, rb, trace + 1 + 2 * io.rounds, io.L, io.R);
}
#undef LLAUNCH
