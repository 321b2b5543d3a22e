// Quantised-input calibration target (Lattice Geometry of NN Quantization,
// section 5.1: in a network whose earlier layers are already quantised, the
// layer sees inputs Xq instead of X; from Babai's point of view only the
// target changes).  For every row w of W the rounding minimises
//   ||Xq q - X w||^2 + lam ||q - w||^2
// (damping as a ridge towards w), i.e. (q - w*)^T Hq_lam (q - w*) + const with
//   Hq_lam = Xq^T Xq + lam I,  w* = Hq_lam^{-1} (G + lam I) w,  G = Xq^T X,
// so the GPTQ sweep runs unchanged on the target W* = W (G + lam I)^T
// Hq_lam^{-1} = ((W (G + lam I)^T) U^T) U with Hq_lam^{-1} = U^T U.  With
// Xq = X the target is W itself.  The three products run in fp64 (the
// inverse amplifies product rounding by the condition number of Hq_lam);
// these kernels widen the operands and narrow the result.
#include "common.h"
#include "launch.h"

// Wd = W, Gd = G + lam I, Ud = U, UdT = U^T (fp32 -> fp64)
__global__ __launch_bounds__(256) void k_qr_prep(const float* __restrict__ W, const float* __restrict__ G,
                                                 const float* __restrict__ U, const double* __restrict__ lam,
                                                 int out, int n, double* __restrict__ Wd, double* __restrict__ Gd,
                                                 double* __restrict__ Ud, double* __restrict__ UdT) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long nn = (long long)n * n;
  if (e < (long long)out * n) Wd[e] = (double)W[e];
  if (e < nn) {
    const int i = (int)(e / n), j = (int)(e % n);
    Gd[e] = (double)G[e] + (i == j ? *lam : 0.0);
    Ud[e] = (double)U[e];
    UdT[(size_t)j * n + i] = (double)U[e];
  }
}

__global__ __launch_bounds__(256) void k_qr_out(const double* __restrict__ a, float* __restrict__ b, long long cnt) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < cnt) b[e] = (float)a[e];
}

hipError_t launch_qr_prep(const float* W, const float* G, const float* U, const double* lam, int out, int n,
                          double* Wd, double* Gd, double* Ud, double* UdT, hipStream_t st) {
  const long long cnt = std::max((long long)out * n, (long long)n * n);
  if (cnt <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_qr_prep, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, W, G, U, lam, out, n, Wd, Gd,
                     Ud, UdT);
  return hipGetLastError();
}

hipError_t launch_qr_out(const double* a, float* b, long long cnt, hipStream_t st) {
  if (cnt <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_qr_out, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, a, b, cnt);
  return hipGetLastError();
}
