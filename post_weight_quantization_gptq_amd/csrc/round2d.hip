// Two-sided adaptive rounding, GPTQ-2D (GPTQ-2D technical summary).
//
// Problem (section 1): integers Z minimising ||A (Z - X) B||_F^2, i.e. the
// one-sided sweep over vec(X) with the Gram H kron G (G = A^T A, H = B B^T),
// whose feedback factor is UH kron UG (G^{-1} = UG^T UG, H^{-1} = UH^T UH).
// Rounding entry (i, j) with delta = w_ij - z_ij changes w_kl by
// -Lg[k][i] delta Uh[j][l] on the lower-right rectangle k >= i, l >= j, with
// the unit factors Lg[k][i] = UG[i][k] / UG[i][i] and Uh[j][l] = UH[j][l] /
// UH[j][j] (section 2: Kronecker feedback, rank-1 updates).  Entry (k, l) is
// reached after every (i, j) with i <= k, j <= l, so its value is
// x_kl - R_kl - C_kl with the lazy buffers (section 2: C = L E pushed down
// the columns, then to the right along the rows)
//   C_kl = sum_{i<k} Lg[k][i] delta_il,
//   R_kl = sum_{j<l} Cf_kj Uh[j][l],   Cf_kj = C_kj + delta_kj,
// and every entry is pushed once down its column and once along its row:
// O(mn max(m, n)) work.  Entries on one anti-diagonal are independent.
//
// On the GPU the matrix is cut into 64 x 64 tiles processed by anti-diagonals
// of tiles (the blocked form of section 2 / Algorithm 4: groups of
// anti-diagonals, the rest of the matrix updated by products):
//   k_r2d_tile: one workgroup per tile of the stage, four lanes per row of
//     the tile; the workgroup walks the tile's own anti-diagonals, pushing
//     inside the tile only;
//   k_r2d_push: the stage's deltas pushed down to every tile below
//     (C += Lg Delta) and its final C to every tile on the right
//     (R += Cf Uh), one 64 x 64 output tile per workgroup on fp32 MFMA.
//     The pushes into the next row block and the next column block (all the
//     next stage's tiles read) run on the main stream; the rest runs on a
//     second stream beside the next stage's tiles, which neither read nor
//     write those blocks, and is joined before the next stage's near pushes
//     (which update blocks it also updates).
// Tiles of one stage write disjoint column blocks of C and disjoint row
// blocks of R, so nothing within a push races.
#include "common.h"
#include "launch.h"

#define T2 64
#define T2P (T2 + 1)

// U1[i][k] = U[i][k] / U[i][i] for k >= i, 0 below; d[i] = U[i][i]
__global__ __launch_bounds__(256) void k_r2d_unit(const float* __restrict__ U, int n, float* __restrict__ U1,
                                                  float* __restrict__ d) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)n * n) return;
  const int i = (int)(e / n), k = (int)(e % n);
  const float di = U[(size_t)i * n + i];
  U1[e] = k >= i ? U[e] / di : 0.f;
  if (k == i) d[i] = di;
}

__global__ __launch_bounds__(256) void k_r2d_fill(float* __restrict__ a, float* __restrict__ b, long long cnt) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < cnt) {
    a[e] = 0.f;
    b[e] = 0.f;
  }
}

// In-tile layout: the four lanes of row group k own row k of the tile.  At
// inner stage s the row processes column l = s - k (anti-diagonal order).
// What only row k reads stays in its registers: lane p holds the row's R
// for columns p + 4u and the row's column-push multipliers Lg[r0 + k2][r0 +
// k] for k2 = k + 1 + p + 4u.  What passes between rows sits in LDS: the
// column buffer C (column-major, Ct[l][k]), the target and row l of Uh.  All
// LDS arrays have a pitch of 69 words: along an anti-diagonal the addresses
// step by 68 = 4 * 17 words, which spreads a wave's 16 rows x 4 lanes over
// the banks (a pitch of 65 would put all 16 rows on one bank).  Indices past
// a ragged tile are clamped to column 64, the padding, which no decision
// reads, so the pushes are branch-free.
#define T2L 69

__global__ __launch_bounds__(256) void k_r2d_tile(R2dProb p, int S, int Ibeg) {
  __shared__ float Xs[T2][T2L], Ct[T2][T2L], Uk[T2][T2L];
  // the tile's results stay in LDS until the walk ends (measured: stores
  // from inside the walk cost a quarter more time per stage)
  __shared__ float Qs[T2][T2L], Ds[T2][T2L], Fs[T2][T2L];
  __shared__ double red[256];
  const int TN = (p.n + T2 - 1) / T2;
  const int I = Ibeg + blockIdx.x, J = S - I;
  const int r0 = I * T2, c0 = J * T2;
  const int mt = min(T2, p.m - r0), nt = min(T2, p.n - c0);
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < T2 * T2; e += 256) {
    const int a = e >> 6, b = e & 63;
    const bool in = a < mt && b < nt;
    const size_t g = (size_t)(r0 + a) * p.n + c0 + b;
    Xs[a][b] = in ? p.X[g] : 0.f;
    Ct[b][a] = in ? p.C[g] : 0.f;
    Uk[a][b] = (a < nt && b < nt) ? p.Uh1[(size_t)(c0 + a) * p.n + c0 + b] : 0.f;
  }
  const int k = tid >> 2, part = tid & 3;
  double se = 0.0;
  float rrow[16], lrow[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int c = part + 4 * u, k2 = k + 1 + part + 4 * u;
    rrow[u] = (k < mt && c < nt) ? p.R[(size_t)(r0 + k) * p.n + c0 + c] : 0.f;
    lrow[u] = (k < mt && k2 < mt) ? p.Lgt[(size_t)(r0 + k) * p.m + r0 + k2] : 0.f;
  }
  __syncthreads();
  const float qmin = (float)p.qmin, qmax = (float)p.qmax;
  for (int s = 0; s < mt + nt - 1; ++s) {
    const int l = s - k;
    if (k < mt && l >= 0 && l < nt) {
      // R_kl from the owner lane (l % 4) of the row group
      float rs = rrow[0];
#pragma unroll
      for (int u = 1; u < 16; ++u) rs = (u == (l >> 2)) ? rrow[u] : rs;
      const float r = __shfl(rs, (lane & ~3) | (l & 3), 64);
      const float c = Ct[l][k];
      const float wv = Xs[k][l] - (r + c);
      const float q = fminf(fmaxf(rintf(wv), qmin), qmax);
      const float d = wv - q;
      const float cf = c + d;
      // column push: C[k2][l] += Lg[k2][k] d for the rows below
      float cv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) cv[u] = Ct[l][min(k + 1 + part + 4 * u, T2)];
#pragma unroll
      for (int u = 0; u < 16; ++u) Ct[l][min(k + 1 + part + 4 * u, T2)] = fmaf(lrow[u], d, cv[u]);
      // row push: R[k][c] += Cf_kl Uh[l][c] for the columns right of l.
      // Applied to every column of the row: Uh[l][c] is 0 left of l, and
      // column l itself (Uh[l][l] = 1) has just been read for the last time.
#pragma unroll
      for (int u = 0; u < 16; ++u) rrow[u] = fmaf(cf, Uk[l][part + 4 * u], rrow[u]);
      if (part == 0) {
        Qs[k][l] = q;
        Ds[k][l] = d;
        Fs[k][l] = cf;
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < T2 * T2; e += 256) {
    const int a = e >> 6, b = e & 63;
    if (a < mt && b < nt) {
      const size_t g = (size_t)(r0 + a) * p.n + c0 + b;
      const float d = Ds[a][b];
      p.Z[g] = (int)Qs[a][b];
      p.D[g] = d;
      p.Cf[g] = Fs[a][b];
      const double es = (double)d / ((double)p.dG[r0 + a] * (double)p.dH[c0 + b]);
      se += es * es;
    }
  }
  red[tid] = se;
  __syncthreads();
  for (int kk = 128; kk > 0; kk >>= 1) {
    if (tid < kk) red[tid] += red[tid + kk];
    __syncthreads();
  }
  if (tid == 0) p.objp[(size_t)I * TN + J] = red[0];
}

// Push items of tile (I, J) on the near (far = false) or far side: the
// next row block / column block only, or every block past it.
__host__ __device__ inline int r2d_items(int TM, int TN, int I, int J, bool far, int* nc, int* nr) {
  *nc = far ? max(0, TM - I - 2) : (I + 1 < TM ? 1 : 0);
  *nr = far ? max(0, TN - J - 2) : (J + 1 < TN ? 1 : 0);
  return *nc + *nr;
}

// One 64 x 64 output tile of a push of stage S:
//   kind 0, tile (I, J), row block K > I:    C[K][J] += Lg[K][I] D[I][J]
//   kind 1, tile (I, J), column block L > J: R[I][L] += Cf[I][J] Uh[J][L]
// near: K = I + 1 and L = J + 1 (what the next stage's tiles read); far:
// the blocks past those (read two or more stages later).
// K = 64 on v_mfma_f32_32x32x2f32, 4 waves of 32 x 32.
// Items vt = blockIdx.x, blockIdx.x + gridDim.x, ... < ntot: a grid smaller
// than the item count makes the launch persistent, so the far pushes leave
// CUs free for the next stage's tiles.
__global__ __launch_bounds__(256) void k_r2d_push(R2dProb p, int S, int Ibeg, int Iend, int far, int ntot) {
  __shared__ float As[T2][T2P];  // [t][r]
  __shared__ float Bs[T2][T2P];  // [t][c]
  const int TM = (p.m + T2 - 1) / T2, TN = (p.n + T2 - 1) / T2;
  const int skip = far ? 2 : 1;
  for (int vt = blockIdx.x; vt < ntot; vt += gridDim.x) {
  int item = vt, I = Ibeg, kind = 0, blk = 0;
  for (; I <= Iend; ++I) {
    int nc, nr;
    r2d_items(TM, TN, I, S - I, far != 0, &nc, &nr);
    if (item < nc) {
      kind = 0;
      blk = I + skip + item;
      break;
    }
    item -= nc;
    if (item < nr) {
      kind = 1;
      blk = S - I + skip + item;
      break;
    }
    item -= nr;
  }
  if (I > Iend) return;  // never: vt < ntot
  const int J = S - I;
  const int r0 = I * T2, c0 = J * T2;
  const int mtI = min(T2, p.m - r0), ntJ = min(T2, p.n - c0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;
  float* out;
  int orows, ocols;  // output tile extent
  if (kind == 0) {
    const int k0 = blk * T2;
    orows = min(T2, p.m - k0);
    ocols = ntJ;
    // A(r, t) = Lg[k0 + r][r0 + t] = Lgt[r0 + t][k0 + r]; B(t, c) = D[r0 + t][c0 + c]
    for (int e = tid; e < T2 * T2; e += 256) {
      const int t = e >> 6, x = e & 63;
      As[t][x] = (t < mtI && x < orows) ? p.Lgt[(size_t)(r0 + t) * p.m + k0 + x] : 0.f;
      Bs[t][x] = (t < mtI && x < ocols) ? p.D[(size_t)(r0 + t) * p.n + c0 + x] : 0.f;
    }
    out = p.C + (size_t)k0 * p.n + c0;
  } else {
    const int l0 = blk * T2;
    orows = mtI;
    ocols = min(T2, p.n - l0);
    // A(r, t) = Cf[r0 + r][c0 + t]; B(t, c) = Uh[c0 + t][l0 + c]
    for (int e = tid; e < T2 * T2; e += 256) {
      const int a = e >> 6, b = e & 63;
      As[b][a] = (a < orows && b < ntJ) ? p.Cf[(size_t)(r0 + a) * p.n + c0 + b] : 0.f;
      Bs[a][b] = (a < ntJ && b < ocols) ? p.Uh1[(size_t)(c0 + a) * p.n + l0 + b] : 0.f;
    }
    out = p.R + (size_t)r0 * p.n + l0;
  }
  __syncthreads();
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll 8
  for (int kk = 0; kk < T2 / 2; ++kk) {
    const float a = As[2 * kk + (lane >> 5)][32 * wr + (lane & 31)];
    const float b = Bs[2 * kk + (lane >> 5)][32 * wc + (lane & 31)];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
  float cur[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 32 * wr + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int j = 32 * wc + (lane & 31);
    cur[r] = (i < orows && j < ocols) ? out[(size_t)i * p.n + j] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 32 * wr + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int j = 32 * wc + (lane & 31);
    if (i < orows && j < ocols) out[(size_t)i * p.n + j] = cur[r] + acc[r];
  }
  __syncthreads();  // the next item refills As, Bs
  }
}

// J = sum of the tiles' partial sums, in tile order
__global__ __launch_bounds__(256) void k_r2d_obj(const double* __restrict__ objp, int nt, double* __restrict__ J) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < nt; i += 256) s += objp[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) *J = red[0];
}

hipError_t launch_r2d_unit(const float* U, int n, float* U1, float* d, hipStream_t st) {
  const long long cnt = (long long)n * n;
  if (cnt == 0) return hipSuccess;
  hipLaunchKernelGGL(k_r2d_unit, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, U, n, U1, d);
  return hipGetLastError();
}

hipError_t launch_r2d_fill(float* a, float* b, long long cnt, hipStream_t st) {
  if (cnt == 0) return hipSuccess;
  hipLaunchKernelGGL(k_r2d_fill, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, a, b, cnt);
  return hipGetLastError();
}

hipError_t launch_r2d_tile(const R2dProb& p, int S, int Ibeg, int ntiles, hipStream_t st) {
  if (ntiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_r2d_tile, dim3(ntiles), dim3(256), 0, st, p, S, Ibeg);
  return hipGetLastError();
}

int r2d_push_items(int m, int n, int S, bool far) {
  const int TM = (m + T2 - 1) / T2, TN = (n + T2 - 1) / T2;
  const int Ib = max(0, S - TN + 1), Ie = min(TM - 1, S);
  int total = 0, nc, nr;
  for (int I = Ib; I <= Ie; ++I) total += r2d_items(TM, TN, I, S - I, far, &nc, &nr);
  return total;
}

hipError_t launch_r2d_push(const R2dProb& p, int S, int Ibeg, int Iend, bool far, int maxwg, hipStream_t st) {
  const int nitems = r2d_push_items(p.m, p.n, S, far);
  if (nitems <= 0) return hipSuccess;
  const int grid = (maxwg > 0 && maxwg < nitems) ? maxwg : nitems;
  hipLaunchKernelGGL(k_r2d_push, dim3(grid), dim3(256), 0, st, p, S, Ibeg, Iend, far ? 1 : 0, nitems);
  return hipGetLastError();
}

hipError_t launch_r2d_obj(const double* objp, int nt, double* J, hipStream_t st) {
  hipLaunchKernelGGL(k_r2d_obj, dim3(1), dim3(256), 0, st, objp, nt, J);
  return hipGetLastError();
}
