// Calibration Hessian H = X^T X on bf16 MFMA (gfx950).
//
// The Gram matrix of the calibration inputs (Lattice Geometry of NN
// Quantization, technical overview section 3.1; GPTQ-2D technical summary
// section 1) is a dense contraction over tokens with both operands stored
// feature-contiguous ([tokens, n] rows).  The MFMA wants 8 consecutive tokens
// per lane, so X is first copied once, transposed and zero-padded, into a
// feature-major workspace (one bandwidth-bound pass); every tile of the
// contraction then moves 16-byte rows straight into LDS in the order the
// MFMA reads them, with no per-tile transposition or bounds checks.
//
// Work split: one workgroup = one 256x256 upper tile of H over a token range;
// the planner gives each XCD its own slice of tokens, so the workgroups that
// run together on one XCD stream the same rows of X through that XCD's L2.
// Partials are summed afterwards in a fixed order (deterministic, no atomics).
#include "common.h"
#include "launch.h"


// Transposed, zero-padded copy of X: Xt[f][t] for f < n_pad, t < t_pad (a
// multiple of 64 tokens).  One 64 x 64 (token x feature) tile per group: rows
// of X come in with 16-byte loads, go out feature-major with 16-byte stores.
__global__ __launch_bounds__(256) void k_xpose(const XposeProb* __restrict__ probs,
                                               const Seg* __restrict__ segs, int nseg) {
  __shared__ uint16_t T[64][64 + 8];
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const XposeProb pb = probs[sg.prob];
  const int t = blockIdx.x - sg.wg0;
  const int fblocks = pb.n_pad / 64;
  const int t0 = 64 * (t / fblocks), f0 = 64 * (t % fblocks);
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + 256 * q;
    const int r = idx >> 3, c8 = (idx & 7) * 8;  // token row r, features c8..c8+7
    const int tok = t0 + r, f = f0 + c8;
    unsigned h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (tok < pb.tokens && f < pb.n) {
      const uint16_t* src = pb.X + (long long)tok * pb.ldx + f;
      if (pb.vec && f + 8 <= pb.n) {
        const u32x4 v = *(const u32x4*)src;
        h[0] = v.x & 0xffff; h[1] = v.x >> 16; h[2] = v.y & 0xffff; h[3] = v.y >> 16;
        h[4] = v.z & 0xffff; h[5] = v.z >> 16; h[6] = v.w & 0xffff; h[7] = v.w >> 16;
      } else {
        for (int e = 0; e < 8 && f + e < pb.n; ++e) h[e] = src[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) T[c8 + e][r] = (uint16_t)h[e];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + 256 * q;
    const int f = idx >> 3, r8 = (idx & 7) * 8;  // feature f, tokens r8..r8+7
    const u32x4 o = *(const u32x4*)&T[f][r8];
    *(u32x4*)(pb.Xt + (size_t)(f0 + f) * pb.t_pad + t0 + r8) = o;
  }
}

// One 256x256 upper tile of H over the token range [k0, k1) of Xt (both
// multiples of 64; the copy is zero-padded, so no bounds are checked).
// Per 64-token step each operand is a 256-row x 128-byte tile in LDS.  The
// rows travel from L2 straight into LDS (global_load_lds, 16 B per lane, no
// registers in between) while the previous step is multiplied; inside a row
// the 16-byte token chunks are stored XOR-swizzled by (row % 8), so the
// fragment reads of 32 consecutive rows hit all LDS banks.
#define SYK_STAGE (2 * 256 * 128)  // bytes per stage (two operands)

typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_syrk(const SyrkProb* __restrict__ probs,
                                                 const SyrkTask* __restrict__ tasks,
                                                 float* __restrict__ partials) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * SYK_STAGE];
  const SyrkTask tk = tasks[blockIdx.x];
  if (tk.part < 0) return;
  const SyrkProb pb = probs[tk.prob];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool diag = tk.ti == tk.tj;
  const int nsteps = (tk.k1 - tk.k0) >> 6;
  const size_t tp = (size_t)pb.t_pad;
  // Load slot of this lane: instruction q of wave w fills LDS rows
  // 8(4q+w) .. 8(4q+w)+7; lane -> row 8(4q+w) + lane/8, chunk position lane%8,
  // holding token chunk (lane%8) ^ (row%8).
  const int lrow = 8 * w + (lane >> 3);
  const int tchunk = (lane & 7) ^ ((lane >> 3) & 7);
  const uint16_t* ga = pb.Xt + (size_t)(tk.ti * 256 + lrow) * tp + tk.k0 + 8 * tchunk;
  const uint16_t* gb = pb.Xt + (size_t)(tk.tj * 256 + lrow) * tp + tk.k0 + 8 * tchunk;

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][q][r] = 0.f;

  auto issue = [&](int step, int stage) {
    uint8_t* base = lds + stage * SYK_STAGE;
    const size_t off = (size_t)step * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(ga + (size_t)(32 * q) * tp + off),
                                       (lds_void*)(base + (4 * q + w) * 1024), 16, 0, 0);
    if (!diag) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(gb + (size_t)(32 * q) * tp + off),
                                         (lds_void*)(base + 256 * 128 + (4 * q + w) * 1024), 16, 0, 0);
    }
  };
  const int arow = 128 * (w >> 1) + (lane & 31);
  const int brow = 128 * (w & 1) + (lane & 31);
  const int sw = lane & 7;  // = row % 8 for every fragment row of this lane

  if (nsteps > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) issue(s + 1, (s + 1) & 1);
    const uint8_t* As = lds + (s & 1) * SYK_STAGE;
    const uint8_t* Bs = diag ? As : As + 256 * 128;
    // fragments of sub-step ks+1 are requested before the MFMAs of ks
    bf16x8 fa[2][4], fb[2][4];
#pragma unroll
    for (int ks = 0; ks < 5; ++ks) {
      if (ks < 4) {
        const int ch = ((2 * ks + (lane >> 5)) ^ sw) * 16;
#pragma unroll
        for (int m = 0; m < 4; ++m) fa[ks & 1][m] = *(const bf16x8*)(As + (arow + 32 * m) * 128 + ch);
#pragma unroll
        for (int q = 0; q < 4; ++q) fb[ks & 1][q] = *(const bf16x8*)(Bs + (brow + 32 * q) * 128 + ch);
      }
      if (ks > 0) {
        const int u = (ks - 1) & 1;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[m][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[u][m], fb[u][q], acc[m][q], 0, 0, 0);
      }
    }
    // keep the order: reads of sub-step 0; then (reads of k+1, MFMAs of k)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of step s+1 have landed
    __syncthreads();                // ... and everybody's; stage s&1 is free again
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
  float sum[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) sum[q] = 0.f;
  for (int p = 0; p < tk.nparts; ++p) {  // parts in list order, 16 loads in flight
    const float* src = partials + (size_t)partlist[tk.part0 + p] * 65536 + (lr0 + (tid >> 6)) * 256 + lc0 + cc;
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = src[4 * q * 256];
#pragma unroll
    for (int q = 0; q < 16; ++q) sum[q] += v[q];
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    float s = sum[q];
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

hipError_t launch_xpose(const XposeProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st) {
  if (nwg <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_xpose, dim3(nwg), dim3(256), 0, st, probs, segs, nseg);
  return hipGetLastError();
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
