// Calibration Hessian H = X^T X on bf16 MFMA (gfx950).
//
// The Gram matrix of the calibration inputs (Lattice Geometry of NN
// Quantization, technical overview section 3.1; GPTQ-2D technical summary
// section 1) is a dense contraction over tokens with both operands stored
// feature-contiguous ([tokens, n] rows).  The MFMA wants 8 consecutive tokens
// per lane, so every 8x8 (token x feature) patch a thread loads is transposed
// in registers with byte permutes and written to LDS feature-major.
//
// Work split: one workgroup = one 256x256 upper tile of H over a token range;
// the planner gives each XCD its own slice of tokens, so the workgroups that
// run together on one XCD stream the same rows of X through that XCD's L2.
// Partials are summed afterwards in a fixed order (deterministic, no atomics).
#include "common.h"
#include "launch.h"

#define SYK_ROW 144              // LDS bytes per feature row: 64 tokens + 16 B pad
#define SYK_OPB (256 * SYK_ROW)  // LDS bytes per operand tile

// Load this thread's 8 tokens x 8 features patch (zero outside the data).
__device__ __forceinline__ void syk_load(u32x4 (&r)[8], const uint16_t* __restrict__ X,
                                         long long ldx, int n, int vec, int f, int krow, int k1) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = krow + t;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < k1) {
      const uint16_t* p = X + (long long)row * ldx + f;
      if (vec && f + 8 <= n) {
        v = *(const u32x4*)p;
      } else if (f < n) {
        unsigned h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const int m = min(8, n - f);
        for (int e = 0; e < m; ++e) h[e] = p[e];
        v.x = h[0] | (h[1] << 16);
        v.y = h[2] | (h[3] << 16);
        v.z = h[4] | (h[5] << 16);
        v.w = h[6] | (h[7] << 16);
      }
    }
    r[t] = v;
  }
}

// Transpose the 8x8 patch (token-major in r[t]) and store feature-major:
// feature row (8c + e), tokens [8g, 8g + 8).
__device__ __forceinline__ void syk_store(uint8_t* lds, const u32x4 (&r)[8], int c, int g) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // low halves of an even/odd token pair for even e, high halves for odd e
    const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
    o.x = __builtin_amdgcn_perm(r[1][e >> 1], r[0][e >> 1], sel);
    o.y = __builtin_amdgcn_perm(r[3][e >> 1], r[2][e >> 1], sel);
    o.z = __builtin_amdgcn_perm(r[5][e >> 1], r[4][e >> 1], sel);
    o.w = __builtin_amdgcn_perm(r[7][e >> 1], r[6][e >> 1], sel);
    *(u32x4*)(lds + (8 * c + e) * SYK_ROW + 16 * g) = o;
  }
}

__global__ __launch_bounds__(256, 1) void k_syrk(const SyrkProb* __restrict__ probs,
                                                 const SyrkTask* __restrict__ tasks,
                                                 float* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * SYK_OPB];
  const SyrkTask tk = tasks[blockIdx.x];
  if (tk.part < 0) return;
  const SyrkProb pb = probs[tk.prob];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = tid & 7, c = tid >> 3;
  const int fa = tk.ti * 256 + 8 * c, fb = tk.tj * 256 + 8 * c;
  const bool diag = tk.ti == tk.tj;
  const int nsteps = (tk.k1 - tk.k0 + 63) >> 6;

  u32x4 ra[8], rb[8];
  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][q][r] = 0.f;

  syk_load(ra, pb.X, pb.ldx, pb.n, pb.vec, fa, tk.k0 + 8 * g, tk.k1);
  if (!diag) syk_load(rb, pb.X, pb.ldx, pb.n, pb.vec, fb, tk.k0 + 8 * g, tk.k1);
  syk_store(lds, ra, c, g);
  if (!diag) syk_store(lds + SYK_OPB, rb, c, g);
  __syncthreads();

  const int arow = 128 * (w >> 1) + (lane & 31);
  const int brow = 128 * (w & 1) + (lane & 31);
  const int koff = 16 * (lane >> 5);
  for (int s = 0; s < nsteps; ++s) {
    const uint8_t* cur = lds + (s & 1) * 2 * SYK_OPB;
    uint8_t* nxt = lds + ((s + 1) & 1) * 2 * SYK_OPB;
    const bool more = s + 1 < nsteps;
    if (more) {
      const int kr = tk.k0 + (s + 1) * 64 + 8 * g;
      syk_load(ra, pb.X, pb.ldx, pb.n, pb.vec, fa, kr, tk.k1);
      if (!diag) syk_load(rb, pb.X, pb.ldx, pb.n, pb.vec, fb, kr, tk.k1);
    }
    const uint8_t* As = cur;
    const uint8_t* Bs = diag ? cur : cur + SYK_OPB;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        a[m] = *(const bf16x8*)(As + (arow + 32 * m) * SYK_ROW + ks * 32 + koff);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        b[q] = *(const bf16x8*)(Bs + (brow + 32 * q) * SYK_ROW + ks * 32 + koff);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[m][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b[q], acc[m][q], 0, 0, 0);
    }
    if (more) {
      syk_store(nxt, ra, c, g);
      if (!diag) syk_store(nxt + SYK_OPB, rb, c, g);
    }
    __syncthreads();
  }

  float* P = partials + (size_t)tk.part * 65536;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * (w >> 1) + 32 * m + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = 128 * (w & 1) + 32 * q + (lane & 31);
        P[row * 256 + col] = acc[m][q][r];
      }
}

// Sum the partials of one 64x64 sub-block of an upper tile in list order,
// write it to H (upper part) and mirror it into the lower part, so H is
// exactly symmetric.  With accumulate, the previous upper value is added.
__global__ __launch_bounds__(256) void k_syrk_reduce(const RedProb* __restrict__ probs,
                                                     const RedTask* __restrict__ tasks,
                                                     const int* __restrict__ partlist,
                                                     const float* __restrict__ partials) {
  __shared__ float S[64][65];
  const RedTask tk = tasks[blockIdx.x];
  const RedProb pb = probs[tk.prob];
  const int tid = threadIdx.x, n = pb.n;
  const int lr0 = tk.r0 & 255, lc0 = tk.c0 & 255;
  const int cc = tid & 63;
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    float s = 0.f;
    for (int p = 0; p < tk.nparts; ++p)
      s += partials[(size_t)partlist[tk.part0 + p] * 65536 + (lr0 + rr) * 256 + lc0 + cc];
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    if (pb.accumulate && i < n && j < n && i <= j) s += pb.H[(size_t)i * n + j];
    S[rr][cc] = s;
  }
  __syncthreads();
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    if (i < n && j < n && i <= j) pb.H[(size_t)i * n + j] = S[rr][cc];
  }
  // mirror: H[j][i] = S[i][j] for i < j, written along contiguous rows of H
  for (int q = 0; q < 16; ++q) {
    const int ci = (tid >> 6) + 4 * q;  // column index inside the sub-block
    const int ri = tid & 63;            // row index inside the sub-block
    const int i = tk.r0 + ri, j = tk.c0 + ci;
    if (i < n && j < n && i < j) pb.H[(size_t)j * n + i] = S[ri][ci];
  }
}

__global__ void k_zero_f32(float* __restrict__ p, long long count) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (; i < count; i += stride) p[i] = 0.f;
}

hipError_t launch_syrk(const SyrkProb* probs, const SyrkTask* tasks, int ntasks, float* partials,
                       hipStream_t st) {
  if (ntasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_syrk, dim3(ntasks), dim3(256), 0, st, probs, tasks, partials);
  return hipGetLastError();
}

hipError_t launch_syrk_reduce(const RedProb* probs, const RedTask* tasks, int ntasks,
                              const int* partlist, const float* partials, hipStream_t st) {
  if (ntasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_syrk_reduce, dim3(ntasks), dim3(256), 0, st, probs, tasks, partlist, partials);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, long long count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  long long blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, count);
  return hipGetLastError();
}
