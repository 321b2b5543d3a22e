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
// V_r comes from subspace iteration in fp64 (V <- orth(H V), orthonormalised
// by Cholesky-QR applied twice), started from a fixed hash-generated block.
// Only span(V_r) matters: Q and the product L R do not depend on the basis.
#include <algorithm>
#include <utility>
#include <vector>

#include "../../include/gptq.h"
#include "common.h"
#include "launch.h"
#include "plan.h"

namespace {

constexpr int kIters = 12;

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

__global__ __launch_bounds__(256) void k_dgemm(DGemm g) {
  __shared__ double As[64][17];
  __shared__ double Bs[16][65];
  const int tiles_n = (g.N + 63) / 64;
  const int i0 = 64 * (blockIdx.x / tiles_n), j0 = 64 * (blockIdx.x % tiles_n);
  const int z = blockIdx.y;
  const int kb = (int)((long long)g.K * z / g.ksplit), ke = (int)((long long)g.K * (z + 1) / g.ksplit);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0;
  for (int k0 = kb; k0 < ke; k0 += 16) {
    if (g.sak == 1) {
      const int r = tid >> 2, kq = (tid & 3) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + kq + u, i = i0 + r;
        As[r][kq + u] = (i < g.M && kk < ke) ? g.A[i * g.sai + kk] : 0.0;
      }
    } else {
      const int r = tid & 63, kq = (tid >> 6) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + kq + u, i = i0 + r;
        As[r][kq + u] = (i < g.M && kk < ke) ? g.A[i * g.sai + kk * g.sak] : 0.0;
      }
    }
    if (g.sbj == 1) {
      const int kr = tid >> 4, jq = (tid & 15) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + kr, j = j0 + jq + u;
        Bs[kr][jq + u] = (kk < ke && j < g.N) ? g.B[kk * g.sbk + j] : 0.0;
      }
    } else {
      const int jl = tid >> 2, kq = (tid & 3) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + kq + u, j = j0 + jl;
        Bs[kq + u][jl] = (kk < ke && j < g.N) ? g.B[kk * g.sbk + j * g.sbj] : 0.0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      double a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) a[mi] = As[32 * wr + 16 * mi + (lane & 15)][4 * kk + (lane >> 4)];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) b[ni] = Bs[4 * kk + (lane >> 4)][32 * wc + 16 * ni + (lane & 15)];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
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

// G (r x r, symmetric PD) = L L^T -> Linv = L^{-1} (lower); then Z L^{-T} has
// orthonormal columns.  One workgroup, r <= 128 (L in LDS, the inverse is
// built column by column in global memory, one thread per column).
__global__ __launch_bounds__(256) void k_chol_inv_small(const double* __restrict__ G, double* __restrict__ Linv, int r) {
  __shared__ double Ls[128 * 128];
  const int tid = threadIdx.x;
  double dmax = 0.0;
  for (int i = 0; i < r; ++i) dmax = fmax(dmax, G[i * r + i]);
  for (int e = tid; e < r * r; e += 256) {
    const int i = e / r, j = e % r;
    Ls[e] = (j <= i) ? G[e] + (i == j ? 1e-15 * dmax : 0.0) : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < r; ++j) {
    const double d = Ls[j * r + j];
    const double sd = sqrt(d > 0.0 ? d : 1e-300);
    __syncthreads();
    if (tid == 0) Ls[j * r + j] = sd;
    for (int i = j + 1 + tid; i < r; i += 256) Ls[i * r + j] /= sd;
    __syncthreads();
    const int w = r - j - 1;
    for (int e = tid; e < w * w; e += 256) {
      const int i = j + 1 + e / w, k = j + 1 + e % w;
      if (k <= i) Ls[i * r + k] -= Ls[i * r + j] * Ls[k * r + j];
    }
    __syncthreads();
  }
  for (int j = tid; j < r; j += 256) {
    for (int i = 0; i < j; ++i) Linv[i * r + j] = 0.0;
    Linv[j * r + j] = 1.0 / Ls[j * r + j];
    for (int i = j + 1; i < r; ++i) {
      double s = 0.0;
      for (int t = j; t < i; ++t) s += Ls[i * r + t] * Linv[t * r + j];
      Linv[i * r + j] = -s / Ls[i * r + i];
    }
  }
}

// lam = lam_abs + lam_rel * mean(diag H); clears the slot's flags.
__global__ __launch_bounds__(256) void k_lora_lambda(const double* __restrict__ H, int n, double lam_abs,
                                                     double lam_rel, Slot* __restrict__ slot) {
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

hipError_t dgemm(hipStream_t st, const DGemm& g0, double* C, double* scratch) {
  DGemm g = g0;
  const int tiles = cdivl(g.M, 64) * cdivl(g.N, 64);
  if (g.ksplit < 1) g.ksplit = 1;
  g.P = (g.ksplit == 1) ? C : scratch;
  hipLaunchKernelGGL(k_dgemm, dim3(tiles, g.ksplit), dim3(256), 0, st, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.ksplit == 1) return e;
  const long long MN = (long long)g.M * g.N;
  hipLaunchKernelGGL(k_dsum, dim3(cdivl(MN, 256)), dim3(256), 0, st, (const double*)scratch, C, MN, g.ksplit);
  return hipGetLastError();
}

}  // namespace

int run_lora(hipStream_t st, const LoraIO& io, const LoraHooks& hk) {
  const int n = io.n, r = io.r, nt = n + r, out = io.out;
  if (r > 128) return hk.set_err(GPTQ_ERR_UNSUPPORTED, "rank above 128 is not supported");
  // workspace layout
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const int ks_n = std::max(1, std::min(16, n / 256));   // split-K for K = n products
  const size_t oH64 = take((size_t)n * n * 8), oV = take((size_t)n * r * 8),
               oZ = take((size_t)n * r * 8), oG = take((size_t)r * r * 8), oLi = take((size_t)r * r * 8),
               oM = take((size_t)r * r * 8), oHV = take((size_t)n * r * 8),
               oS = take((size_t)std::max(ks_n * n * r, ks_n * r * r) * 8), oA = take((size_t)nt * nt * 8),
               oU = take((size_t)nt * nt * 4), oW = take((size_t)out * nt * 4);
  uint8_t* base = (uint8_t*)hk.ensure(off);
  if (!base) return GPTQ_ERR_NO_MEMORY;
  Slot* slot = (Slot*)hk.slots(sizeof(Slot));
  if (!slot) return GPTQ_ERR_NO_MEMORY;
  double *H64 = (double*)(base + oH64), *V = (double*)(base + oV), *Z = (double*)(base + oZ),
         *G = (double*)(base + oG), *Li = (double*)(base + oLi), *M = (double*)(base + oM),
         *HV = (double*)(base + oHV), *S = (double*)(base + oS), *A = (double*)(base + oA);
  float* U = (float*)(base + oU);
  float* Ww = (float*)(base + oW);

  // H accurate to float64 rounding: the Schur complement below cancels the
  // top-r eigen-directions of H against a damping far below their size
  int rc = hk.hessian64(io.X, io.tokens, io.ldx, n, H64);
  if (rc) return rc;
  hipError_t e;
#define LCHK(x)                                                        \
  do {                                                                 \
    e = (x);                                                           \
    if (e != hipSuccess) return hk.set_err(GPTQ_ERR_HIP, hipGetErrorString(e)); \
  } while (0)
  hipLaunchKernelGGL(k_lora_lambda, dim3(1), dim3(256), 0, st, (const double*)H64, n, io.lam_abs, io.lam_rel, slot);
  LCHK(hipGetLastError());
  hipLaunchKernelGGL(k_start_block, dim3(cdivl((long long)n * r, 256)), dim3(256), 0, st, V, n, r);
  LCHK(hipGetLastError());
  auto orth = [&](const double* Zin, double* Vout) -> hipError_t {
    // G = Z^T Z ; Z L^{-T} -> Vout
    DGemm g{Zin, 1, r, Zin, r, 1, nullptr, r, r, n, ks_n};
    hipError_t e2 = dgemm(st, g, G, S);
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL(k_chol_inv_small, dim3(1), dim3(256), 0, st, (const double*)G, Li, r);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    DGemm h{Zin, r, 1, Li, 1, r, nullptr, n, r, r, 1};
    return dgemm(st, h, Vout, S);
  };
  for (int it = 0; it < kIters; ++it) {
    DGemm g{H64, n, 1, V, r, 1, nullptr, n, r, n, ks_n};  // Z = H V
    LCHK(dgemm(st, g, Z, S));
    LCHK(orth(Z, V));  // Cholesky-QR, twice
    LCHK(orth(V, Z));
    std::swap(V, Z);
  }
  {
    DGemm g{H64, n, 1, V, r, 1, nullptr, n, r, n, ks_n};  // HV = H V
    LCHK(dgemm(st, g, HV, S));
    DGemm m{V, 1, r, HV, r, 1, nullptr, r, r, n, ks_n};  // M = V^T H V
    LCHK(dgemm(st, m, M, S));
  }
  hipLaunchKernelGGL(k_lora_assemble, dim3(cdivl(nt, 4)), dim3(256), 0, st, (const double*)H64, (const double*)HV,
                     (const double*)M, n, r, A, slot);
  LCHK(hipGetLastError());
  if ((rc = hk.factor(A, nt, U, slot))) return rc;
  QuantJob J{io.W, out, n, nt, U, io.bits, io.group, io.block, io.codes, io.scales, io.zeros, nullptr,
             &slot->lam, slot->obj, Ww};
  if ((rc = hk.quantize(J))) return rc;
  const long long cnt = std::max((long long)n * r, (long long)r * out);
  hipLaunchKernelGGL(k_lora_extract, dim3(cdivl(cnt, 256)), dim3(256), 0, st, (const double*)V, (const float*)Ww,
                     out, n, r, io.L, io.R);
  LCHK(hipGetLastError());
#undef LCHK
  return 0;
}
