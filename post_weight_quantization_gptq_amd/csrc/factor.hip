// Damping and the upper Cholesky factor of the inverse damped Hessian, in fp64.
//
// lam = lam_abs + lam_rel * mean(diag H) and H_lam = H + lam I (Lattice
// Geometry of NN Quantization, technical overview section 3.1).  The sweep
// needs U upper with H_lam^{-1} = U^T U: the unit-upper factor of the LDL of
// the inverse Gram matrix is diag(U)^{-1} U (GPTQ-2D technical summary,
// sections 2 and 4).  With P the index reversal and C = chol(P H_lam P),
// U = P C^{-1} P, so one Cholesky and one triangular inverse suffice
// (2n^3/3 flops instead of 4n^3/3 for Cholesky -> inverse -> Cholesky).
//
// Cholesky: right-looking over 256-wide outer panels, each factored as two
// pairs of 64-wide steps (k_chol_panel2; k_chol_panel for an unpaired last
// block).  A pair launch factors both 64x64 diagonal blocks with the
// four-wave blocked leaf and inverts them (blk64.h), then each workgroup
// computes its panel rows below as A_ik L_kk^{-T} on fp64 MFMA.  Between the
// pairs, a narrow update brings the second pair's columns up to date; after
// the outer panel, one update with K = 256 reaches the next outer panel's
// columns on the main stream and the rest of the trailing lower triangle on
// the second stream (four times less traffic over the trailing matrix than
// updating it after every 64 columns).  When a pair's panel launch would
// outnumber the CUs (batched layers), k_chol_diag2 first runs the pair's
// diagonal chain once per problem and the panel workgroups load it.
// Inverse: Y = L^{-1} by blocked forward substitution of L Y = I run in step
// with the factorization.  Step k finishes block row k of Y
// (Y_kj = L_kk^{-1} B_kj, B_kj = -sum_{t<k} L_kt Y_tj) in the same launch as
// the panel, and B_ik -= L_ik Y_k: joins the Cholesky updates: the rows of
// the outer panel right away, the rows past it in the outer update (K = 256
// again).  So the inverse adds no serial steps and no long-K products, and
// its n^3/3 flops ride in launches that are there anyway.
#include "blk64.h"
#include "common.h"
#include "launch.h"


// ------------------------------------------------------------ damping -----
__global__ __launch_bounds__(256) void k_damp_lambda(const FacProb* __restrict__ probs, int nprob) {
  __shared__ double red[256];
  const int p = blockIdx.x;
  if (p >= nprob) return;
  const FacProb pb = probs[p];
  if (pb.H == nullptr) return;  // assembled elsewhere (lam already set)
  // each thread sums its entries in index order; unrolled so that the loads
  // of several entries are in flight at once
  double s = 0.0;
#pragma unroll 8
  for (int i = threadIdx.x; i < pb.n; i += 256) s += (double)glb(pb.H)[(size_t)i * pb.ldh + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = pb.n > 0 ? red[0] / (double)pb.n : 0.0;
    *pb.lam = pb.lam_abs + pb.lam_rel * mean;
    *pb.info = 0;
    *pb.nonfinite = 0;
  }
}

// A[i][j] = H[n-1-i][n-1-j] + lam delta_ij, lower triangle only (j <= i).
// Segment: one workgroup per 4 rows, one wave per row.  With 16-byte aligned
// rows each lane moves 4 entries per step (a reversed float4 in, two double2
// out), several steps in flight at once; otherwise one entry per lane.
__global__ __launch_bounds__(256) void k_damp_fill(const FacProb* __restrict__ probs,
                                                   const Seg* __restrict__ segs, int nseg) {
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const FacProb pb = probs[sg.prob];
  const int n = pb.n;
  const int i = (blockIdx.x - sg.wg0) * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  const int lane = threadIdx.x & 63;
  const double lam = *pb.lam;
  gptr<const float> hrow = glb(pb.H) + (size_t)(n - 1 - i) * pb.ldh;
  gptr<double> arow = glb(pb.A) + (size_t)i * n;
  bool bad = false;
  const bool vec = (n % 4) == 0 && (pb.ldh % 4) == 0 && (((uintptr_t)pb.H) & 15) == 0 && (((uintptr_t)pb.A) & 15) == 0;
  if (vec) {
#pragma unroll 4
    for (int j4 = 4 * lane; j4 <= i; j4 += 256) {
      // columns j4 .. j4+3 of A are columns n-1-j4 .. n-4-j4 of H
      const f32x4 v = *(gptr<const f32x4>)(hrow + (n - 4 - j4));
      double d[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float h = v[3 - t];
        bad |= (j4 + t <= i) && !__builtin_isfinite(h);
        d[t] = (double)h + (i == j4 + t ? lam : 0.0);
      }
      if (j4 + 3 <= i) {
        *(gptr<f64x2>)(arow + j4) = f64x2{d[0], d[1]};
        *(gptr<f64x2>)(arow + j4 + 2) = f64x2{d[2], d[3]};
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (j4 + t <= i) arow[j4 + t] = d[t];
      }
    }
  } else {
    for (int j = lane; j <= i; j += 64) {
      const float h = hrow[n - 1 - j];
      bad |= !__builtin_isfinite(h);
      arow[j] = (double)h + (i == j ? lam : 0.0);
    }
  }
  if (bad) atomicOr(pb.nonfinite, 1);
}

// Panel step k (64 columns starting at k0), one workgroup per 64-block of
// the problem.  Every group factors the diagonal block the same way and
// inverts it; then
//   - group for row block i > k: its rows of the panel, L_ik = A_ik L_kk^{-T};
//   - group for row block k: writes L_kk^{-1} as Y_kk and zeros the rest of
//     its rows of the 256-wide diagonal block of Y (read as a whole by the
//     products of the outer step);
//   - group for column block j < k: Y_kj = L_kk^{-1} B_kj, where B_kj holds
//     -sum_{t<k} L_kt Y_tj from the updates of the earlier steps (forward
//     substitution of L Y = I, one block row per step).
// The products run on fp64 MFMA, 4 waves of 32 x 32.
__global__ __launch_bounds__(256) void k_chol_panel(const FacProb* __restrict__ probs,
                                                    const Seg* __restrict__ segs, int nseg) {
  __shared__ __attribute__((aligned(16))) double LT[NB][LDP];  // the diagonal block, then L (row-major)
  __shared__ __attribute__((aligned(16))) double Ys[NB][LDP];  // L^{-1}, row-major
  __shared__ __attribute__((aligned(16))) double Rs[NB][LDP];  // this group's panel rows, or B_kj
  __shared__ double Tm[32][33];
  __shared__ double lb[2 * NB];
  __shared__ double dv[NB];
  __shared__ int flag;
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const FacProb pb = probs[sg.prob];
  if (*pb.info != 0 || *pb.nonfinite != 0) return;
  const int n = pb.n, k = sg.a, nb = (n + NB - 1) / NB, g = blockIdx.x - sg.wg0;
  const int k0 = k * NB, m = min(NB, n - k0);
  const bool yrole = g >= nb - k;                 // Y_kj for column block j
  const int i = yrole ? k : k + g, j = yrole ? g - (nb - k) : 0;
  const int tid = threadIdx.x;
  gptr<double> A = glb(pb.A);
  const int r0 = i * NB, mr = yrole ? m : ((i == k) ? 0 : min(NB, n - r0));
  {
    // both 64x64 blocks: 16 + 16 loads per thread, all in flight together
    double ta[16], tr[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q, r = e >> 6, c = e & 63;  // coalesced over c
      ta[q] = (r < m && c <= r) ? A[(size_t)(k0 + r) * n + k0 + c] : 0.0;
      if (yrole)
        tr[q] = (r < m) ? glb(pb.Y)[(size_t)(k0 + r) * n + NB * j + c] : 0.0;
      else
        tr[q] = (r < mr && c < m) ? A[(size_t)(r0 + r) * n + k0 + c] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q, r = e >> 6, c = e & 63;
      LT[r][c] = (r < m && c < m) ? ta[q] : ((r == c) ? 1.0 : 0.0);
      Rs[r][c] = tr[q];
    }
  }
  __syncthreads();
  const int bad = chol64_blocked(LT, dv, lb, &flag);
  if (bad >= 0) {
    if (tid == 0 && g == 0) atomicMax(pb.info, n - (k0 + bad));
    return;
  }
  inv64_waves(LT, dv, Ys, Tm);
  if (!yrole && i == k) {
    // Only L_kk^{-1} is kept: nothing reads the diagonal block of L again (the
    // updates read the panel rows below it), and the other groups of this
    // launch are still reading A_kk, so A_kk stays as is.  The whole block,
    // zeros above the diagonal included, then zeros up to the end of the
    // 256-wide diagonal block.
    const int P1 = min((k0 / 256) * 256 + 256, n);
    const int wz = P1 - k0;  // 64 .. 256 columns
    for (int e = tid; e < NB * wz; e += 256) {
      const int r = e / wz, c = e % wz;
      if (r < m) glb(pb.Y)[(size_t)(k0 + r) * n + k0 + c] = (c < m && c <= r) ? Ys[r][c] : 0.0;
    }
    return;
  }
  // yrole: Out(r, c) = sum_t Ys[r][t] Rs[t][c]   (Y_kj = L_kk^{-1} B_kj)
  // else:  Out(r, c) = sum_t Rs[r][t] Ys[c][t]   (L_ik = A_ik L_kk^{-T})
  const int lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;
  f64x4 acc[2][2];
  blk_zero(acc);
  if (yrole)
    blk_mma<false>(acc, Ys, Rs);
  else
    blk_mma<true>(acc, Rs, Ys);
  gptr<double> out = yrole ? glb(pb.Y) + (size_t)k0 * n + NB * j : A + (size_t)r0 * n + k0;
  const int mc = yrole ? NB : m;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * wr + 16 * mi + (lane >> 4) + 4 * q;
        const int c = 32 * wc + 16 * ni + (lane & 15);
        if (r < mr && c < mc) out[(size_t)r * n + c] = acc[mi][ni][q];
      }
}

// The diagonal chain of the pair of 64-column steps k, k+1: the leaf
// Cholesky and inverse of D0 = A_kk (Y0 = L_kk^{-1}), L10 = A_{k+1,k} Y0^T,
// D1 = A_{k+1,k+1} - L10 L10^T, its leaf and inverse (Y1 = L_{k+1,k+1}^{-1}).
// In: LT = A_kk (lower), L10 = A_{k+1,k}, d1 = A_{k+1,k+1} (lower, in the
// product accumulator layout, zero past m1).  Out: Y0, Y1, L10 in LDS; LT is
// free.  Returns false (after recording the failing pivot) when a leaf fails.
__device__ __forceinline__ bool pair_diag(const FacProb& pb, int k0, int m1, bool report,
                                          double (&LT)[NB][LDP], double (&Y0)[NB][LDP], double (&Y1)[NB][LDP],
                                          double (&L10)[NB][LDP], double (&Tm)[32][33], double* lb, double* dv,
                                          int* flag, f64x4 (&d1)[2][2]) {
  const int n = pb.n, k1 = k0 + NB;
  int bad = chol64_blocked(LT, dv, lb, flag);
  if (bad >= 0) {
    if (report && threadIdx.x == 0) atomicMax(pb.info, n - (k0 + bad));
    return false;
  }
  inv64_waves(LT, dv, Y0, Tm);
  f64x4 acc[2][2];
  // L10 = A_{k+1,k} Y0^T
  blk_zero(acc);
  blk_mma<true>(acc, L10, Y0);
  __syncthreads();
  blk_each([&](int mi, int ni, int q, int r, int c) { L10[r][c] = acc[mi][ni][q]; });
  __syncthreads();
  // D1 - L10 L10^T, padded with the identity past m1
  blk_neg(d1);
  blk_mma<true>(d1, L10, L10);
  blk_neg(d1);
  blk_each([&](int mi, int ni, int q, int r, int c) {
    LT[r][c] = (r < m1 && c < m1) ? d1[mi][ni][q] : ((r == c) ? 1.0 : 0.0);
  });
  __syncthreads();
  bad = chol64_blocked(LT, dv, lb, flag);
  if (bad >= 0) {
    if (report && threadIdx.x == 0) atomicMax(pb.info, n - (k1 + bad));
    return false;
  }
  inv64_waves(LT, dv, Y1, Tm);
  return true;
}

// Loads of the pair's diagonal region for pair_diag: A_kk and A_{k+1,k} into
// LT and L10 (row-major), A_{k+1,k+1} into d1.
__device__ __forceinline__ void pair_diag_loads(gptr<double> A, int n, int k0, int m1, double (&LT)[NB][LDP],
                                                double (&L10)[NB][LDP], f64x4 (&d1)[2][2]) {
  const int tid = threadIdx.x, k1 = k0 + NB;
  double ta[16], tb[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, r = e >> 6, c = e & 63;
    ta[q] = (c <= r) ? A[(size_t)(k0 + r) * n + k0 + c] : 0.0;
    tb[q] = (r < m1) ? A[(size_t)(k1 + r) * n + k0 + c] : 0.0;
  }
  blk_each([&](int mi, int ni, int q, int r, int c) {
    d1[mi][ni][q] = (r < m1 && c <= r) ? A[(size_t)(k1 + r) * n + k1 + c] : 0.0;
  });
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, r = e >> 6, c = e & 63;
    LT[r][c] = ta[q];
    L10[r][c] = tb[q];
  }
}

// Batched problems: the diagonal chain of pair k once per problem (one
// workgroup per segment), Y0, Y1 and L10 stored to the problem's D
// (3 x 64 x 64, row-major) for k_chol_panel2's rows, instead of every one of
// its workgroups repeating it.  Same code and order as the repeated chain,
// so the results are the same bits.
__global__ __launch_bounds__(256) void k_chol_diag2(const FacProb* __restrict__ probs,
                                                    const Seg* __restrict__ segs, int nseg) {
  __shared__ __attribute__((aligned(16))) double LT[NB][LDP];
  __shared__ __attribute__((aligned(16))) double Y0[NB][LDP];
  __shared__ __attribute__((aligned(16))) double Y1[NB][LDP];
  __shared__ __attribute__((aligned(16))) double L10[NB][LDP];
  __shared__ double Tm[32][33];
  __shared__ double lb[2 * NB];
  __shared__ double dv[NB];
  __shared__ int flag;
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const FacProb pb = probs[sg.prob];
  if (*pb.info != 0 || *pb.nonfinite != 0) return;
  const int n = pb.n, k0 = sg.a * NB, m1 = min(NB, n - k0 - NB);
  f64x4 d1[2][2];
  pair_diag_loads(glb(pb.A), n, k0, m1, LT, L10, d1);
  __syncthreads();
  if (!pair_diag(pb, k0, m1, true, LT, Y0, Y1, L10, Tm, lb, dv, &flag, d1)) return;
  gptr<double> D = glb(pb.D);
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int r = e >> 6, c = e & 63;
    D[e] = Y0[r][c];
    D[NB * NB + e] = Y1[r][c];
    D[2 * NB * NB + e] = L10[r][c];
  }
}

// Two 64-column steps k, k+1 of one outer panel in a single launch.  Every
// workgroup first runs the pair's diagonal chain itself (pair_diag), or, when
// the segment's b is 1, loads its results from k_chol_diag2; then its own
// part:
//   - row block i >= k+2: L_ik = A_ik L_kk^{-T}, then
//     L_{i,k+1} = (A_{i,k+1} - L_ik L10^T) L_{k+1,k+1}^{-T};
//   - row block k: writes Y_kk = L_kk^{-1}, Y_{k+1,k} = -Y_{k+1,k+1} L10 Y_kk,
//     Y_{k+1,k+1}, and zeros to the end of the 256-wide diagonal block;
//   - row block k+1: nothing (L10 is read by no later step, and writing it
//     would race with the other groups' loads of A_{k+1,k});
//   - column block j < k: Y_kj = Y_kk B_kj, then
//     Y_{k+1,j} = Y_{k+1,k+1} (B_{k+1,j} - L10 Y_kj).
// This replaces two panel launches and the narrow update between them; the
// repeated diagonal work is parallel and costs less than the launches while
// the workgroups fit the chip in one round.
// Needs k + 1 < nb (block k is then full; block k+1 may be partial).
__global__ __launch_bounds__(256) void k_chol_panel2(const FacProb* __restrict__ probs,
                                                     const Seg* __restrict__ segs, int nseg) {
  __shared__ __attribute__((aligned(16))) double LT[NB][LDP];   // leaf workspace (D0, then D1), then the operand stage
  __shared__ __attribute__((aligned(16))) double Y0[NB][LDP];   // L_kk^{-1}
  __shared__ __attribute__((aligned(16))) double Y1[NB][LDP];   // L_{k+1,k+1}^{-1}
  __shared__ __attribute__((aligned(16))) double L10[NB][LDP];  // A_{k+1,k}, then L10
  __shared__ double Tm[32][33];
  __shared__ double lb[2 * NB];
  __shared__ double dv[NB];
  __shared__ int flag;
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const FacProb pb = probs[sg.prob];
  if (*pb.info != 0 || *pb.nonfinite != 0) return;
  const int n = pb.n, k = sg.a, nb = (n + NB - 1) / NB, g = blockIdx.x - sg.wg0;
  const bool pre = sg.b != 0;  // the diagonal chain's results are in pb.D
  const int k0 = k * NB, k1 = k0 + NB, m1 = min(NB, n - k1);
  const bool yrole = g >= nb - k;
  const int i = yrole ? k : k + g, j = yrole ? g - (nb - k) : 0;
  const int tid = threadIdx.x;
  gptr<double> A = glb(pb.A);
  gptr<double> Y = glb(pb.Y);
  const int r0 = i * NB, mr = min(NB, n - r0);
  const bool own = yrole || i >= k + 2;
  // this group's two blocks (A_ik or B_kj in tx, row-major by thread; the
  // second in x1, accumulator layout), loaded with the diagonal region's
  f64x4 x1[2][2];
  double tx[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, r = e >> 6, c = e & 63;
    tx[q] = !own ? 0.0 : yrole ? Y[(size_t)(k0 + r) * n + NB * j + c]
                               : ((r < mr) ? A[(size_t)(r0 + r) * n + k0 + c] : 0.0);
  }
  blk_each([&](int mi, int ni, int q, int r, int c) {
    x1[mi][ni][q] = !own ? 0.0 : yrole ? ((r < m1) ? Y[(size_t)(k1 + r) * n + NB * j + c] : 0.0)
                                       : ((r < mr && c < m1) ? A[(size_t)(r0 + r) * n + k1 + c] : 0.0);
  });
  if (pre) {
    gptr<const double> D = glb((const double*)pb.D);
    for (int e = tid; e < NB * NB; e += 256) {
      const int r = e >> 6, c = e & 63;
      Y0[r][c] = D[e];
      Y1[r][c] = D[NB * NB + e];
      L10[r][c] = D[2 * NB * NB + e];
    }
    __syncthreads();
  } else {
    f64x4 d1[2][2];
    pair_diag_loads(A, n, k0, m1, LT, L10, d1);
    __syncthreads();
    if (!pair_diag(pb, k0, m1, g == 0, LT, Y0, Y1, L10, Tm, lb, dv, &flag, d1)) return;
  }
  f64x4 acc[2][2];
  const int P1 = min((k0 / 256) * 256 + 256, n);
  if (!yrole && i == k) {
    // Y rows of the pair: Y_kk, Y_{k+1,k} = -Y1 (L10 Y0), Y_{k+1,k+1}, zeros
    // to the end of the outer panel's diagonal block
    for (int e = tid; e < NB * (P1 - k0); e += 256) {
      const int r = e / (P1 - k0), c = e % (P1 - k0);
      Y[(size_t)(k0 + r) * n + k0 + c] = (c < NB && c <= r) ? Y0[r][c] : 0.0;
    }
    for (int e = tid; e < NB * (P1 - k1); e += 256) {
      const int r = e / (P1 - k1), c = e % (P1 - k1);
      if (r < m1) Y[(size_t)(k1 + r) * n + k1 + c] = (c < m1 && c <= r) ? Y1[r][c] : 0.0;
    }
    blk_zero(acc);
    blk_mma<false>(acc, L10, Y0);
    blk_each([&](int mi, int ni, int q, int r, int c) { LT[r][c] = acc[mi][ni][q]; });
    __syncthreads();
    blk_zero(acc);
    blk_mma<false>(acc, Y1, LT);
    blk_neg(acc);
    blk_each([&](int mi, int ni, int q, int r, int c) {
      if (r < m1) Y[(size_t)(k1 + r) * n + k0 + c] = acc[mi][ni][q];
    });
    return;
  }
  // Row block k+1 keeps A_{k+1,k} as it is: every group of this launch
  // loads it at its start, and nothing after this launch reads L10 (the
  // next updates read L's rows from k+2 on).
  if (!yrole && i == k + 1) return;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    LT[e >> 6][e & 63] = tx[q];
  }
  __syncthreads();
  blk_zero(acc);
  if (!yrole) {
    // L_ik = A_ik Y0^T
    blk_mma<true>(acc, LT, Y0);
    blk_each([&](int mi, int ni, int q, int r, int c) {
      if (r < mr) A[(size_t)(r0 + r) * n + k0 + c] = acc[mi][ni][q];
    });
    __syncthreads();
    blk_each([&](int mi, int ni, int q, int r, int c) { LT[r][c] = acc[mi][ni][q]; });
    __syncthreads();
    // A_{i,k+1} - L_ik L10^T, then times Y1^T
    blk_neg(x1);
    blk_mma<true>(x1, LT, L10);
    blk_neg(x1);
    __syncthreads();
    blk_each([&](int mi, int ni, int q, int r, int c) { LT[r][c] = x1[mi][ni][q]; });
    __syncthreads();
    blk_zero(acc);
    blk_mma<true>(acc, LT, Y1);
    blk_each([&](int mi, int ni, int q, int r, int c) {
      if (r < mr && c < m1) A[(size_t)(r0 + r) * n + k1 + c] = acc[mi][ni][q];
    });
  } else {
    // Y_kj = Y0 B_kj
    blk_mma<false>(acc, Y0, LT);
    blk_each([&](int mi, int ni, int q, int r, int c) { Y[(size_t)(k0 + r) * n + NB * j + c] = acc[mi][ni][q]; });
    __syncthreads();
    blk_each([&](int mi, int ni, int q, int r, int c) { LT[r][c] = acc[mi][ni][q]; });
    __syncthreads();
    // B_{k+1,j} - L10 Y_kj, then Y1 times it
    blk_neg(x1);
    blk_mma<false>(x1, L10, LT);
    blk_neg(x1);
    __syncthreads();
    blk_each([&](int mi, int ni, int q, int r, int c) { LT[r][c] = x1[mi][ni][q]; });
    __syncthreads();
    blk_zero(acc);
    blk_mma<false>(acc, Y1, LT);
    blk_each([&](int mi, int ni, int q, int r, int c) {
      if (r < m1) Y[(size_t)(k1 + r) * n + NB * j + c] = acc[mi][ni][q];
    });
  }
}

// --------------------------------------------------- fp64 MFMA products ---
// General form (any n): one 64 x 64 output tile per workgroup, 4 waves of
// 32 x 32, v_mfma_f64_16x16x4.
//   C(i, j) = beta C(i, j) + alpha sum_{t in [kb, ke)} Aop(i, t) Bop(t, j)
// Aop(i, t) = A[i * lda + t]; Bop(t, j) = B[t * sbk + j * sbj] (one of sbk,
// sbj is 1).  The kind decides the operands from the problem's matrices.
// K chunks of 32 are staged through registers into a double-buffered LDS
// pair: the loads of chunk c+1 are in flight while chunk c is multiplied.
// Problems with n % 64 == 0 take k_gemm_ring below instead.
template <int TS>
__global__ __launch_bounds__(256) void k_gemm(const FacProb* __restrict__ probs, const Seg* __restrict__ segs,
                                              int nseg) {
  constexpr int KC = (TS == 64) ? 32 : 16;  // k per chunk
  constexpr int MB = TS / 32;               // 16x16 blocks per wave side
  constexpr int TPR = 256 / TS;             // threads per row of a k-contiguous operand
  constexpr int TPK = 256 / KC;             // threads per k row of a j-contiguous operand
  constexpr int V = KC * TS / 256;          // values per thread per operand (8)
  __shared__ double As[2][TS][KC + 1];
  __shared__ double Bs[2][KC][TS + 1];
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const FacProb pb = probs[sg.prob];
  if (*pb.info != 0 || *pb.nonfinite != 0) return;
  const int n = pb.n;
  const int t = blockIdx.x - sg.wg0;
  gptr<const double> A;
  gptr<const double> B;
  gptr<double> C;
  long long lda, sbk, sbj, ldc;
  int mt, nt, kb, ke;
  double alpha, beta;
  if (sg.a == GK_CHOL_TRAIL) {
    // A[i][j] -= sum_{t in [kb, kb+kw)} A[i][t] A[j][t] for the lower tiles of
    // rows [c0, n) x columns [c0, c1)
    const int kb0 = sg.b, kw = sg.c, c0 = sg.d, c1 = sg.e;
    const int nrow = (n - c0 + TS - 1) / TS, ncol = (c1 - c0 + TS - 1) / TS;
    int b = 0, tt = t;
    while (b < ncol && tt >= nrow - b) {
      tt -= nrow - b;
      ++b;
    }
    const int a = b + tt;
    const int i0 = c0 + TS * a, j0 = c0 + TS * b;
    A = glb((const double*)pb.A) + (size_t)i0 * n + kb0;
    lda = n;
    B = glb((const double*)pb.A) + (size_t)j0 * n + kb0;
    sbk = 1;
    sbj = n;
    C = glb(pb.A) + (size_t)i0 * n + j0;
    ldc = n;
    mt = min(TS, n - i0);
    nt = min(TS, c1 - j0);
    kb = 0;
    ke = kw;
    alpha = -1.0;
    beta = 1.0;
  } else {
    // Y(i, j) -= sum_t L(i, t) Y(t, j): rows [r0, r1) x columns [0, kb0 + kw)
    const int kb0 = sg.b, kw = sg.c, r0 = sg.d, r1 = sg.e;
    const int ncol = (kb0 + kw + TS - 1) / TS;
    const int i0 = r0 + TS * (t / ncol), j0 = TS * (t % ncol);
    A = glb((const double*)pb.A) + (size_t)i0 * n + kb0;
    lda = n;
    B = glb((const double*)pb.Y) + (size_t)kb0 * n + j0;
    sbk = n;
    sbj = 1;
    C = glb(pb.Y) + (size_t)i0 * n + j0;
    ldc = n;
    mt = min(TS, r1 - i0);
    nt = min(TS, kb0 + kw - j0);
    kb = 0;
    ke = kw;
    alpha = -1.0;
    beta = j0 < kb0 ? 1.0 : 0.0;  // columns from kb0 on: first write
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1;
  f64x4 acc[MB][MB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0;

  double ra[V], rb[V];
  // k-contiguous operands: thread -> row tid / TPR, V/4 quads of k at a
  // stride of KC/(V/4); j-contiguous: k row tid / TPK, V/4 quads of j at a
  // stride of TS/(V/4).  Loads never branch: an out-of-range element reads a
  // valid address of the same operand and is replaced by zero.
  constexpr int NQ = V / 4;
  const int lr = tid / TPR, lq = (tid % TPR) * 4;
  const int kr = tid / TPK, jq = (tid % TPK) * 4;
  auto load = [&](int k0) {
    const bool rok = lr < mt;
    gptr<const double> ap = A + (size_t)(rok ? lr : 0) * lda;
#pragma unroll
    for (int h = 0; h < NQ; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + lq + (KC / NQ) * h + u;
        const bool ok = rok && kk < ke;
        const double v = ap[ok ? kk : kb];
        ra[4 * h + u] = ok ? v : 0.0;
      }
    if (sbj == 1) {
      const int kk = k0 + kr;
      const bool kok = kk < ke;
      gptr<const double> bp = B + (size_t)(kok ? kk : kb) * sbk;
#pragma unroll
      for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = jq + (TS / NQ) * h + u;
          const bool ok = kok && j < nt;
          const double v = bp[ok ? j : 0];
          rb[4 * h + u] = ok ? v : 0.0;
        }
    } else {
      const bool jok = lr < nt;
      gptr<const double> bp = B + (size_t)(jok ? lr : 0) * sbj;
#pragma unroll
      for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kk = k0 + lq + (KC / NQ) * h + u;
          const bool ok = jok && kk < ke;
          const double v = bp[ok ? kk : kb];
          rb[4 * h + u] = ok ? v : 0.0;
        }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < NQ; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u) As[buf][lr][lq + (KC / NQ) * h + u] = ra[4 * h + u];
    if (sbj == 1) {
#pragma unroll
      for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) Bs[buf][kr][jq + (TS / NQ) * h + u] = rb[4 * h + u];
    } else {
#pragma unroll
      for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) Bs[buf][lq + (KC / NQ) * h + u][lr] = rb[4 * h + u];
    }
  };
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
      double a[MB], b[MB];
#pragma unroll
      for (int mi = 0; mi < MB; ++mi) a[mi] = As[buf][(TS / 2) * wr + 16 * mi + (lane & 15)][4 * kk + (lane >> 4)];
#pragma unroll
      for (int ni = 0; ni < MB; ++ni) b[ni] = Bs[buf][4 * kk + (lane >> 4)][(TS / 2) * wc + 16 * ni + (lane & 15)];
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int ni = 0; ni < MB; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // every load of C before any store (one memory round trip, not one per element)
  double cur[MB][MB][4];
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int ni = 0; ni < MB; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (TS / 2) * wr + 16 * mi + (lane >> 4) + 4 * r;
        const int j = (TS / 2) * wc + 16 * ni + (lane & 15);
        cur[mi][ni][r] = (beta != 0.0 && i < mt && j < nt) ? C[(size_t)i * ldc + j] : 0.0;
      }
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int ni = 0; ni < MB; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (TS / 2) * wr + 16 * mi + (lane >> 4) + 4 * r;
        const int j = (TS / 2) * wc + 16 * ni + (lane & 15);
        if (i < mt && j < nt) C[(size_t)i * ldc + j] = cur[mi][ni][r] + alpha * acc[mi][ni][r];
      }
}


// Products of the factor when n % 64 == 0 (every K range, row offset and
// pitch is then a multiple of 64): one TS x TS tile per workgroup (TS = 128
// on 8 waves of 64 x 32, or TS = 64 on 4 waves of 32 x 32), fp64 MFMA
// 16x16x4.  K chunks of 16 go from global memory straight into an LDS ring
// (global_load_lds, 16 B per lane; 3 stages), so no register staging and no
// load latency on the critical path.
//   - k-contiguous operands (L always, and L again as B in the Cholesky
//     update) sit row-major, 128 B per row and chunk, the 16-byte k-pairs
//     XOR-swizzled by (row / 2) % 8: a lane reads its two k values with one
//     ds_read_b128 and 16 lanes on 16 rows hit 16 distinct bank groups;
//   - j-contiguous B (Y in the inverse's updates) sits k-major, the j-pairs
//     of a row XOR-swizzled by 8 ((k / 2) % 2).
// K order: MFMA lane group g holds k = 8p + 2g + u in sub-step u of pair
// step p, the same for both operands, so each pair step sums the 8 k's of
// its range once.  Rows past the tile's edge read a valid row whose
// results are never stored.
// s_waitcnt vmcnt(ahead * PER) for a runtime ahead in [0, NST - 2]
template <int NST, int PER>
__device__ __forceinline__ void ring_wait(int ahead) {
  if constexpr (NST > 2) {
    if (ahead >= NST - 2) {
      __builtin_amdgcn_s_waitcnt(VmWait<(NST - 2) * PER>::value);
      return;
    }
    ring_wait<NST - 1, PER>(ahead);
  } else {
    __builtin_amdgcn_s_waitcnt(VmWait<0>::value);
  }
}

template <int TS>
struct RingCfg {
  static constexpr int NW = TS == 128 ? 8 : 4;  // waves
  static constexpr int WGC = NW / 2;            // wave grid 2 x WGC
  static constexpr int WM = TS / 2, WN = TS / WGC;
  static constexpr int MI = WM / 16, NI = WN / 16;
  // three stages (two in flight): for 64-wide tiles that is 48 KB of LDS, so
  // two workgroups share a CU and cover each other's waits (measured faster
  // than one workgroup with six stages)
  static constexpr int KC = 16, NST = 3;
  static constexpr int OPB = TS * KC * 8;       // bytes per operand per stage
  static constexpr int STB = 2 * OPB;
  static constexpr int NQ = OPB / 1024 / NW;    // global_load_lds per operand per wave per stage
};

template <int TS>
__device__ __forceinline__ void ring_tile(const FacProb* __restrict__ probs, const Seg* __restrict__ segs, int nseg,
                                          int vt, uint8_t* lds) {
  using C_ = RingCfg<TS>;
  constexpr int NW = C_::NW, MI = C_::MI, NI = C_::NI, KC = C_::KC, NST = C_::NST;
  constexpr int OPB = C_::OPB, STB = C_::STB, NQ = C_::NQ;
  static_assert(NQ >= 1 && NQ * NW * 1024 == OPB, "load split");
  const Seg sg = segs[find_seg(segs, nseg, vt)];
  const FacProb pb = probs[sg.prob];
  if (sg.a != GK_NT && (*pb.info != 0 || *pb.nonfinite != 0)) return;
  const int n = pb.n;
  const int t = vt - sg.wg0;
  const double* A;
  const double* B;
  gptr<double> C;  // a global view: its accesses stay off lgkmcnt
  long long lda, ldb, ldc;  // ldb: pitch between B's k-contiguous rows (j) or k rows
  bool bkc;                 // B k-contiguous
  int mt, nt, kb, ke;
  double alpha, beta;
  if (sg.a == GK_CHOL_TRAIL) {
    const int kb0 = sg.b, kw = sg.c, c0 = sg.d, c1 = sg.e;
    const int nrow = (n - c0 + TS - 1) / TS, ncol = (c1 - c0 + TS - 1) / TS;
    int b = 0, tt = t;
    while (b < ncol && tt >= nrow - b) {
      tt -= nrow - b;
      ++b;
    }
    const int i0 = c0 + TS * (b + tt), j0 = c0 + TS * b;
    A = pb.A + (size_t)i0 * n + kb0;
    B = pb.A + (size_t)j0 * n + kb0;
    lda = ldb = n;
    bkc = true;
    C = glb(pb.A) + (size_t)i0 * n + j0;
    ldc = n;
    mt = min(TS, n - i0);
    nt = min(TS, c1 - j0);
    kb = 0;
    ke = kw;
    alpha = -1.0;
    beta = 1.0;
  } else if (sg.a == GK_NT) {
    const int M = sg.b, N = sg.c, K = sg.d;
    const int ncol = (N + TS - 1) / TS;
    const int i0 = TS * (t / ncol), j0 = TS * (t % ncol);
    A = pb.A + (size_t)i0 * n;
    B = pb.Y + (size_t)j0 * n;
    lda = ldb = n;
    bkc = true;
    C = glb(pb.C) + (size_t)i0 * n + j0;
    ldc = n;
    mt = min(TS, M - i0);
    nt = min(TS, N - j0);
    // e = 1: B upper triangular (B[j][t] = 0 for t < j): t from j0;
    // e = 2: B lower triangular (B[j][t] = 0 for t > j): t below j0 + TS
    kb = sg.e == 1 ? j0 : 0;
    ke = sg.e == 2 ? min(K, j0 + TS) : K;
    alpha = 1.0;
    beta = 0.0;
  } else {
    // Y(i, j) -= sum_t L(i, t) Y(t, j): rows [r0, r1) x columns [0, kb0 + kw)
    const int kb0 = sg.b, kw = sg.c, r0 = sg.d, r1 = sg.e;
    const int ncol = (kb0 + kw + TS - 1) / TS;
    const int i0 = r0 + TS * (t / ncol), j0 = TS * (t % ncol);
    A = pb.A + (size_t)i0 * n + kb0;
    lda = n;
    B = pb.Y + (size_t)kb0 * n + j0;
    ldb = n;
    bkc = false;
    C = glb(pb.Y) + (size_t)i0 * n + j0;
    ldc = n;
    mt = min(TS, r1 - i0);
    nt = min(TS, kb0 + kw - j0);
    kb = 0;
    ke = kw;
    alpha = -1.0;
    beta = j0 < kb0 ? 1.0 : 0.0;  // columns from kb0 on: first write
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = w / C_::WGC, wc = w % C_::WGC;
  const int nst = (ke - kb) / KC;

  // global sources of this lane, per instruction q (k offset added per stage)
  const double* asrc[NQ];
  const double* bsrc[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const int slot = (NW * qi + w) * 64 + lane;  // 16-byte slot of the stage
    const int r = slot >> 3, p = slot & 7;       // k-contiguous: row, pair slot
    const int kp = p ^ ((r >> 1) & 7);
    asrc[qi] = A + (size_t)(r < mt ? r : 0) * lda + kb + 2 * kp;
    if (bkc) {
      bsrc[qi] = B + (size_t)(r < nt ? r : 0) * ldb + kb + 2 * kp;
    } else {
      const int k = slot / (TS / 2), jp = (slot % (TS / 2)) ^ (8 * ((k >> 1) & 1));
      bsrc[qi] = B + (size_t)(kb + k) * ldb + (2 * jp < nt ? 2 * jp : 0);
    }
  }
  auto issue = [&](int st, int buf) {
    uint8_t* base = lds + buf * STB;
    const size_t ka = (size_t)st * KC, kbo = bkc ? (size_t)st * KC : (size_t)st * KC * ldb;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      __builtin_amdgcn_global_load_lds((const void*)(asrc[qi] + ka), (lds_void*)(base + (NW * qi + w) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[qi] + kbo), (lds_void*)(base + OPB + (NW * qi + w) * 1024),
                                       16, 0, 0);
    }
  };

  f64x4 acc[MI][NI];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < NI; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0;

  const int li = lane & 15, g = lane >> 4;
  // C's current values, loaded first so their latency hides behind the
  // ring's (vector loads complete in issue order, so the waits below, which
  // count only the ring's loads, are only stricter for them), and all of them
  // before any store: one round trip, not one per element
  double cur[MI][NI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = wr * C_::WM + 16 * mi + g + 4 * r;
        const int j = wc * C_::WN + 16 * ni + li;
        cur[mi][ni][r] = (beta != 0.0 && i < mt && j < nt) ? C[(size_t)i * ldc + j] : 0.0;
      }
#pragma unroll
  for (int q = 0; q < NST - 1; ++q)
    if (q < nst) issue(q, q);
  for (int st = 0; st < nst; ++st) {
    // stage st has landed once at most (stages issued after it) x 2 NQ loads remain
    ring_wait<NST, 2 * NQ>(min(NST - 2, nst - 1 - st));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (st + NST - 1 < nst) issue(st + NST - 1, (st + NST - 1) % NST);
    const uint8_t* sa = lds + (st % NST) * STB;
    const uint8_t* sb = sa + OPB;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      double av[MI][2], bv[NI][2];
      const int kp = 4 * ps + g;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wr * C_::WM + 16 * mi + li;
        const f64x2 v = *(const f64x2*)(sa + r * 128 + ((kp ^ ((r >> 1) & 7)) << 4));
        av[mi][0] = v[0];
        av[mi][1] = v[1];
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int j = wc * C_::WN + 16 * ni + li;
        if (bkc) {
          const f64x2 v = *(const f64x2*)(sb + j * 128 + ((kp ^ ((j >> 1) & 7)) << 4));
          bv[ni][0] = v[0];
          bv[ni][1] = v[1];
        } else {
          const int k = 2 * kp;  // and k + 1: same swizzle
          const int off = (((j >> 1) ^ (8 * ((k >> 1) & 1))) << 4) + 8 * (j & 1);
          bv[ni][0] = *(const double*)(sb + k * (TS * 8) + off);
          bv[ni][1] = *(const double*)(sb + (k + 1) * (TS * 8) + off);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mi][u], bv[ni][u], acc[mi][ni], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = wr * C_::WM + 16 * mi + g + 4 * r;
        const int j = wc * C_::WN + 16 * ni + li;
        if (i < mt && j < nt) C[(size_t)i * ldc + j] = cur[mi][ni][r] + alpha * acc[mi][ni][r];
      }
}

// Tiles vt = blockIdx.x, blockIdx.x + gridDim.x, ... < ntot: a grid smaller
// than the tile count makes the launch persistent, so it can run beside the
// factorization's serial chain without taking every CU.
template <int TS>
__global__ __launch_bounds__(RingCfg<TS>::NW * 64) void k_gemm_ring(const FacProb* __restrict__ probs,
                                                                     const Seg* __restrict__ segs, int nseg,
                                                                     int ntot) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[RingCfg<TS>::NST * RingCfg<TS>::STB];
  for (int vt = blockIdx.x; vt < ntot; vt += gridDim.x) {
    ring_tile<TS>(probs, segs, nseg, vt, lds);
    __syncthreads();  // the next tile refills the ring
  }
}

// U[i][j] = Y[n-1-i][n-1-j] for j >= i (upper), 0 below; fp32.  4 rows per WG.
__global__ __launch_bounds__(256) void k_make_u(const FacProb* __restrict__ probs,
                                                const Seg* __restrict__ segs, int nseg) {
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const FacProb pb = probs[sg.prob];
  if (*pb.info != 0 || *pb.nonfinite != 0) return;
  const int n = pb.n;
  const int i = (blockIdx.x - sg.wg0) * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  const double* yrow = pb.Y + (size_t)(n - 1 - i) * n;
  float* urow = pb.U + (size_t)i * pb.ldu;
  for (int j = threadIdx.x & 63; j < n; j += 64) urow[j] = (j >= i) ? (float)yrow[n - 1 - j] : 0.f;
}

hipError_t launch_damp_lambda(const FacProb* probs, int nprob, hipStream_t st) {
  if (nprob <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_damp_lambda, dim3(nprob), dim3(256), 0, st, probs, nprob);
  return hipGetLastError();
}

#define SEG_LAUNCH(name, kern, threads)                                                   \
  hipError_t name(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st) { \
    if (nwg <= 0) return hipSuccess;                                                      \
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(threads), 0, st, probs, segs, nseg);         \
    return hipGetLastError();                                                             \
  }

SEG_LAUNCH(launch_damp_fill, k_damp_fill, 256)
SEG_LAUNCH(launch_chol_panel, k_chol_panel, 256)
SEG_LAUNCH(launch_chol_panel2, k_chol_panel2, 256)
SEG_LAUNCH(launch_chol_diag2, k_chol_diag2, 256)
SEG_LAUNCH(launch_gemm64, k_gemm<64>, 256)
hipError_t launch_gemm_ring(int ts, const FacProb* probs, const Seg* segs, int nseg, int ntot, int maxwg,
                            hipStream_t st) {
  if (ntot <= 0) return hipSuccess;
  const int grid = (maxwg > 0 && maxwg < ntot) ? maxwg : ntot;
  if (ts == 128)
    hipLaunchKernelGGL(k_gemm_ring<128>, dim3(grid), dim3(512), 0, st, probs, segs, nseg, ntot);
  else
    hipLaunchKernelGGL(k_gemm_ring<64>, dim3(grid), dim3(256), 0, st, probs, segs, nseg, ntot);
  return hipGetLastError();
}
SEG_LAUNCH(launch_make_u, k_make_u, 256)
