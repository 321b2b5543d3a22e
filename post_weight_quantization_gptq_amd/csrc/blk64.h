// 64x64 fp64 block kernels for one 256-thread workgroup (four waves), shared
// by the factorization and the small Gram factorizations of the LoRA path:
// a blocked Cholesky of a diagonal block, the inverse of its factor, and
// 64x64x64 block products on fp64 MFMA, all with operands in LDS.
#pragma once
#include "common.h"

#define NB 64
// LDS pitch of a 64x64 fp64 block: rows 16-byte aligned (one ds_read_b128
// gives a lane two k values) and 16 rows of a column read hit distinct banks
#define LDP (NB + 2)

// ----------------------------------------------------------- Cholesky -----
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), l);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Cholesky of the 64x64 diagonal block by the workgroup's four waves,
// blocked by 16 columns.  For each 16-column sub-panel, wave 0 runs the
// column steps with lane r holding row r's 16 entries of the sub-panel (at
// most 15 FMAs per step), then the four waves apply the rank-16 update to the
// lower 16x16 tiles right of it on fp64 MFMA.
// Column step j: 1/sqrt of the pivot by the hardware estimate and one Newton
// step (the estimate is good to about 2^-26, so one step reaches double
// precision), l = a_j * rs on every lane (lane j: sqrt of the pivot; lanes
// below: the multipliers; lanes above: values above the diagonal that
// nothing reads).  The multipliers of the next two rows reach every lane by
// readlane and lane j+1's updated entry is the next pivot (also by
// readlane), so the serial chain never waits for LDS; the other multipliers
// go through LDS (two alternating rows of broadcast reads) and their part of
// the update lands one step later.
// The steps contain no branch: a failed pivot (not positive or not finite) is
// recorded and replaced by 1, so the rest stays finite and is discarded.  A
// scheduling fence ends every step, so the compiler interleaves the next
// pivot's chain with the step's FMAs and no more.
// In: M[r][c] row-major, lower triangle valid (padded with the identity).
// Out: M lower = L (entries above the diagonal are don't-care), dv[r] =
// 1 / L[r][r].  Returns the first failing pivot or -1, the same on every
// thread.  lb: 2 NB doubles of LDS; flag: one int of LDS.
struct PanelWave {
  double a[16];
  double dvr;
  int fail;
  double pl;       // the previous step's multiplier
  double plk[16];  // its broadcast multipliers of columns >= its column + 3
};

// Column step C of the sub-panel at c0.  The rank-1 update of columns C+1 and
// C+2 takes the multipliers of rows J+1 and J+2 by readlane, so the next
// pivot (lane J+1's updated a[C+1], also by readlane) and the next step's
// multipliers never wait for LDS.  Columns from C+3 on take theirs through
// LDS, and that part of the update is applied one step later (the column is
// first read two steps on), so the LDS latency stays off the serial chain.
template <int C>
__device__ __forceinline__ double sub_step(PanelWave& st, double* lb, int r, int c0, double rs) {
  const int J = c0 + C;
  const double l = st.a[C] * rs;
  st.a[C] = l;
  st.dvr = (r == J) ? rs : st.dvr;
  double rsn = 0.0;
  double lk[16];
  if constexpr (C + 1 < 16) {
    st.a[C + 1] -= l * readlane_f64(l, J + 1);
    if constexpr (C + 2 < 16) st.a[C + 2] -= l * readlane_f64(l, J + 2);
    const double dn = readlane_f64(st.a[C + 1], J + 1);
    const bool ok = dn > 0.0 && __builtin_isfinite(dn);
    st.fail = (st.fail < 0 && !ok) ? J + 1 : st.fail;
    const double dd = ok ? dn : 1.0;
    rsn = __builtin_amdgcn_rsq(dd);
    rsn = rsn * (1.5 - 0.5 * dd * rsn * rsn);
    if constexpr (C + 3 < 16) {
      double* row = lb + NB * (C & 1);
      row[r] = l;
#pragma unroll
      for (int t = C + 3; t < 16; ++t) lk[t] = row[c0 + t];
    }
  }
  // the deferred part of the previous step's update (columns >= C + 2)
  if constexpr (C >= 1 && C + 2 < 16) {
#pragma unroll
    for (int t = C + 2; t < 16; ++t) st.a[t] -= st.pl * st.plk[t];
  }
  if constexpr (C + 3 < 16) {
    st.pl = l;
#pragma unroll
    for (int t = C + 3; t < 16; ++t) st.plk[t] = lk[t];
  }
  __builtin_amdgcn_sched_barrier(0);
  return rsn;
}

template <int C>
struct SubSteps {
  __device__ __forceinline__ static void run(PanelWave& st, double* lb, int r, int c0, double rs) {
    const double rsn = sub_step<C>(st, lb, r, c0, rs);
    SubSteps<C + 1>::run(st, lb, r, c0, rsn);
  }
};
template <>
struct SubSteps<16> {
  __device__ __forceinline__ static void run(PanelWave&, double*, int, int, double) {}
};

__device__ __forceinline__ int chol64_blocked(double (*M)[LDP], double* dv, double* lb, int* flag) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  PanelWave st;
  st.dvr = 0.0;
  st.fail = -1;
#pragma unroll 1
  for (int p = 0; p < 4; ++p) {
    const int c0 = 16 * p;
    if (w == 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) st.a[t] = M[lane][c0 + t];
      const double d = readlane_f64(st.a[0], c0);
      const bool ok = d > 0.0 && __builtin_isfinite(d);
      st.fail = (st.fail < 0 && !ok) ? c0 : st.fail;
      const double dd = ok ? d : 1.0;
      double rs = __builtin_amdgcn_rsq(dd);
      rs = rs * (1.5 - 0.5 * dd * rs * rs);
      SubSteps<0>::run(st, lb, lane, c0, rs);
#pragma unroll
      for (int t = 0; t < 16; ++t) M[lane][c0 + t] = st.a[t];
    }
    __syncthreads();
    if (p < 3) {
      // M[i][j] -= sum_{t<16} M[i][c0+t] M[j][c0+t] on the lower 16x16 tiles
      // of rows / columns [c0 + 16, 64)
      const int nt = 3 - p, ntiles = nt * (nt + 1) / 2;
      const int i16 = lane & 15, k4 = lane >> 4;
      for (int tile = w; tile < ntiles; tile += 4) {
        int ti = 0, rem = tile;
        while (rem > ti) {
          rem -= ti + 1;
          ++ti;
        }
        const int i0 = c0 + 16 + 16 * ti, j0 = c0 + 16 + 16 * rem;
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(M[i0 + i16][c0 + 4 * s4 + k4], M[j0 + i16][c0 + 4 * s4 + k4], acc, 0,
                                                    0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) M[i0 + k4 + 4 * q][j0 + i16] -= acc[q];
      }
      __syncthreads();
    }
  }
  if (w == 0) {
    dv[lane] = st.dvr;
    if (lane == 0) *flag = st.fail;
  }
  __syncthreads();
  return *flag;
}

// Y = L^{-1} of the 64x64 lower block by the four waves: the diagonal 16x16
// inverses by forward substitution (wave w, lane = column), then two doubling
// levels [[A,0],[B,C]]^{-1} = [[A^-1,0],[-C^-1 B A^-1, C^-1]] on fp64 MFMA
// (16 -> 32: waves 0 and 1; 32 -> 64: one 16x16 output block per wave).
// Ys is row-major with zeros above the diagonal; Tm is scratch [32][33].
__device__ __forceinline__ void inv64_waves(double (*Ls)[LDP], const double* dv, double (*Ys)[LDP],
                                            double (*Tm)[33]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  {
    const int c = lane & 15, o = 16 * w;
    double y[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      double s = (rr == c) ? 1.0 : 0.0;
#pragma unroll
      for (int kk = 0; kk < rr; ++kk) s -= Ls[o + rr][o + kk] * y[kk];
      y[rr] = s * dv[o + rr];
    }
    if (lane < 16) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) Ys[o + rr][o + c] = y[rr];
    }
    // zeros above the diagonal blocks (read by the products below and by callers)
    for (int e = lane; e < 16 * (NB - o - 16); e += 64) Ys[o + (e & 15)][o + 16 + (e >> 4)] = 0.0;
  }
  __syncthreads();
  const int i16 = lane & 15, k4 = lane >> 4;
  if (w < 2) {
    // pair (2w, 2w+1): Y[b1][b0] = -Y[b1][b1] L[b1][b0] Y[b0][b0]
    const int b0 = 32 * w, b1 = b0 + 16;
    double (*T)[33] = Tm + 16 * w;  // rows 16w..16w+15 of the scratch, 16 columns used
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(Ls[b1 + i16][b0 + 4 * s + k4], Ys[b0 + 4 * s + k4][b0 + i16], acc, 0,
                                                0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) T[k4 + 4 * q][i16] = acc[q];
    __builtin_amdgcn_wave_barrier();
    f64x4 acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(Ys[b1 + i16][b1 + 4 * s + k4], T[4 * s + k4][i16], acc2, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) Ys[b1 + k4 + 4 * q][b0 + i16] = -acc2[q];
  }
  __syncthreads();
  {
    // Y[32:64][0:32] = -Y22 (L21 Y11); wave w owns output block (p, q)
    const int p = w >> 1, q = w & 1;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb < q) continue;  // Y11 is lower triangular
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(Ls[32 + 16 * p + i16][16 * kb + 4 * s + k4],
                                                  Ys[16 * kb + 4 * s + k4][16 * q + i16], acc, 0, 0, 0);
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) Tm[16 * p + k4 + 4 * qq][16 * q + i16] = acc[qq];
    __syncthreads();
    f64x4 acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb > p) continue;  // Y22 is lower triangular
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(Ys[32 + 16 * p + i16][32 + 16 * kb + 4 * s + k4],
                                                   Tm[16 * kb + 4 * s + k4][16 * q + i16], acc2, 0, 0, 0);
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) Ys[32 + 16 * p + k4 + 4 * qq][16 * q + i16] = -acc2[qq];
  }
  __syncthreads();
}

// 64x64x64 block products on the four waves (each wave a 32x32 quarter of
// the result, fp64 MFMA 16x16x4), operands in LDS:
//   acc += sum_t Aop(r, t) Bop(t, c),  Aop(r, t) = A[r][t],
//   Bop(t, c) = B[t][c] (BT = false) or B[c][t] (BT = true).
// K order: in pair step p, lane group g holds t = 8p + 2g + u in sub-step u
// (the same for both operands), so a row operand is one ds_read_b128.
// The accumulator layout: wave w holds rows 32 (w / 2) + 16 mi + (lane / 16)
// + 4 q and columns 32 (w % 2) + 16 ni + lane % 16.
template <bool BT>
__device__ __forceinline__ void blk_mma(f64x4 (&acc)[2][2], const double (*A)[LDP], const double (*B)[LDP]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wr = w >> 1, wc = w & 1;
  const int li = lane & 15, g = lane >> 4;
  // fully unrolled: a loop back-edge makes the compiler move the
  // accumulators between AGPRs and VGPRs (and drain the MFMA pipe) each trip
#pragma unroll
  for (int ps = 0; ps < NB / 8; ++ps) {
    const int t = 8 * ps + 2 * g;
    f64x2 av[2], bv[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) av[mi] = *(const f64x2*)&A[32 * wr + 16 * mi + li][t];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int c = 32 * wc + 16 * ni + li;
      if (BT) {
        bv[ni] = *(const f64x2*)&B[c][t];
      } else {
        bv[ni][0] = B[t][c];
        bv[ni][1] = B[t + 1][c];
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mi][u], bv[ni][u], acc[mi][ni], 0, 0, 0);
  }
}

__device__ __forceinline__ void blk_neg(f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[mi][ni][q] = -acc[mi][ni][q];
}

// visit the accumulator's elements: f(mi, ni, q, row, col)
template <class F>
__device__ __forceinline__ void blk_each(F&& f) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wr = w >> 1, wc = w & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f(mi, ni, q, 32 * wr + 16 * mi + (lane >> 4) + 4 * q, 32 * wc + 16 * ni + (lane & 15));
}

__device__ __forceinline__ void blk_zero(f64x4 (&acc)[2][2]) {
  blk_each([&](int mi, int ni, int q, int, int) { acc[mi][ni][q] = 0.0; });
}
