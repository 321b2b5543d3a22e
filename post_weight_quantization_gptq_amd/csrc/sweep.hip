// The GPTQ column sweep with lazy block updates, on gfx950.
//
// For each output row independently (Lattice Geometry of NN Quantization,
// technical overview section 2: the layer problem splits into one problem per
// neuron) and each column j in natural order: round w_j onto the row's (or
// group's) min-max grid, scale the rounding error by the Cholesky diagonal,
// E_j = (w_j - what_j)/U_jj, and feed it forward, w_k -= E_j U_jk (GPTQ
// encyclopedia entry, technical approach: closed-form compensation of the
// remaining weights; GPTQ-2D technical summary section 1: fixed order and a
// triangular feedback matrix).  Inside a block of B columns the feedback is
// applied column by column; the block's errors reach the later columns as one
// product W[:, b1:] -= E_blk U[blk, b1:] (GPTQ-2D section 2, GPTQ's lazy block
// update), done on fp32 MFMA.
//
// Sweep layout: 16 lanes per row, each lane owning B/16 consecutive columns of
// the block in registers; the B x B block of U sits in LDS and every lane
// reads its own slice of row j of it.  The value w_j is broadcast from its
// owner lane inside the 16-lane group; every lane of the group repeats the
// scalar rounding step, so no further exchange is needed before the update.
#include "common.h"
#include "launch.h"

struct Grid {
  float s, r, z;
};

// Asymmetric min-max grid over values with minimum mn and maximum mx; every
// step in fp32 exactly as specified (0 always inside the range).
__device__ __forceinline__ Grid grid_from(float mn, float mx, float maxq) {
  const float lo = fminf(mn, 0.f), hi = fmaxf(mx, 0.f);
  Grid g;
  if (hi == lo) {
    g.s = 1.f;
    g.r = 1.f;
    g.z = 0.f;
    return g;
  }
  g.s = (hi - lo) / maxq;
  g.r = 1.f / g.s;
  const float zr = __fadd_rn(__fmul_rn(-lo, g.r), 0.f);
  g.z = fminf(fmaxf(rintf(zr), 0.f), maxq);
  return g;
}

// Working copy of W (and zero columns n..nt-1 for the augmented variant).
__global__ __launch_bounds__(256) void k_init_work(const QLayer* __restrict__ L,
                                                   const Seg* __restrict__ segs, int nseg) {
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const QLayer ly = L[sg.prob];
  const int row = (blockIdx.x - sg.wg0) * 4 + (threadIdx.x >> 6);
  if (row >= ly.out) return;
  for (int c = threadIdx.x & 63; c < ly.nt; c += 64)
    ly.Ww[(size_t)row * ly.nt + c] = c < ly.n ? ly.W[(size_t)row * ly.n + c] : 0.f;
}

// One grid per row on the original row (group == 0).  One wave per row.
__global__ __launch_bounds__(256) void k_rowfit(const QLayer* __restrict__ L,
                                                const Seg* __restrict__ segs, int nseg) {
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const QLayer ly = L[sg.prob];
  const int row = (blockIdx.x - sg.wg0) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  if (row < ly.out)
    for (int c = lane; c < ly.n; c += 64) {
      const float v = ly.W[(size_t)row * ly.n + c];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if (row < ly.out && lane == 0) {
    const Grid g = grid_from(mn, mx, (float)((1 << ly.bits) - 1));
    ly.scales[(size_t)row * ly.ng] = g.s;
    ly.zeros[(size_t)row * ly.ng] = (uint8_t)g.z;
  }
}

template <int CPL>
__global__ __launch_bounds__(256) void k_sweep(const QLayer* __restrict__ L,
                                               const Seg* __restrict__ segs, int nseg) {
  constexpr int B = 16 * CPL;
  __shared__ __attribute__((aligned(16))) float Us[B * B];
  __shared__ float dinv[B];
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const QLayer ly = L[sg.prob];
  const int blk = sg.a;
  const int b0 = blk * B, b1 = min(b0 + B, ly.n), bw = b1 - b0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15;
  const int row = (blockIdx.x - sg.wg0) * 16 + w * 4 + (lane >> 4);
  const bool rv = row < ly.out;
  const int nt = ly.nt, G = ly.group;
  const float maxq = (float)((1 << ly.bits) - 1);

  for (int e = tid; e < B * B; e += 256) {
    const int j = e / B, k = e % B;
    Us[e] = (j < bw && k < bw) ? ly.U[(size_t)(b0 + j) * nt + b0 + k] : 0.f;
  }
  for (int j = tid; j < B; j += 256) dinv[j] = j < bw ? 1.f / ly.U[(size_t)(b0 + j) * nt + b0 + j] : 0.f;

  float wv[CPL], wo[CPL], qv[CPL], ev[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int lc = CPL * l16 + c;
    const bool in = rv && lc < bw;
    wv[c] = in ? ly.Ww[(size_t)row * nt + b0 + lc] : 0.f;
    wo[c] = in ? ly.W[(size_t)row * ly.n + b0 + lc] : 0.f;
    qv[c] = 0.f;
    ev[c] = 0.f;
  }
  Grid g = {1.f, 1.f, 0.f};
  if (rv && (G == 0 || (b0 % G) != 0)) {
    // the row's grid, or the grid of a group that began in an earlier block
    const size_t gi = (size_t)row * ly.ng + (G ? b0 / G : 0);
    g.s = ly.scales[gi];
    g.r = 1.f / g.s;
    g.z = (float)ly.zeros[gi];
  }
  __syncthreads();

  double se = 0.0, sd = 0.0;
  for (int o = 0; o < 16; ++o) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = o * CPL + c;
      if (j < bw) {
        if (G != 0 && ((b0 + j) % G) == 0) {
          // fit the group's grid on its current values [b0+j, b0+j+G)
          float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
          for (int c2 = 0; c2 < CPL; ++c2) {
            const int lc = CPL * l16 + c2;
            if (lc >= j && lc < j + G && lc < bw) {
              mn = fminf(mn, wv[c2]);
              mx = fmaxf(mx, wv[c2]);
            }
          }
          if (j + G > B && rv)  // group extends past this block (group > block)
            for (int cc = B + l16; cc < j + G; cc += 16) {
              const float v = ly.Ww[(size_t)row * nt + b0 + cc];
              mn = fminf(mn, v);
              mx = fmaxf(mx, v);
            }
#pragma unroll
          for (int m = 8; m > 0; m >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, m, 16));
            mx = fmaxf(mx, __shfl_xor(mx, m, 16));
          }
          g = grid_from(mn, mx, maxq);
          if (rv && l16 == 0) {
            const size_t gi = (size_t)row * ly.ng + (b0 + j) / G;
            ly.scales[gi] = g.s;
            ly.zeros[gi] = (uint8_t)g.z;
          }
        }
        const float wj = __shfl(wv[c], o, 16);
        const float x = __fadd_rn(__fmul_rn(wj, g.r), g.z);
        const float q = fminf(fmaxf(rintf(x), 0.f), maxq);
        const float what = g.s * (q - g.z);
        const float e = (wj - what) * dinv[j];
        if (l16 == o) {
          qv[c] = q;
          ev[c] = e;
          const float d = wo[c] - what;
          sd += (double)d * (double)d;
          se += (double)e * (double)e;
        }
        const float* urow = Us + j * B + CPL * l16;
#pragma unroll
        for (int c2 = 0; c2 < CPL; ++c2) wv[c2] = fmaf(-e, urow[c2], wv[c2]);
      }
    }
  }

#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int lc = CPL * l16 + c;
    if (rv && lc < bw) {
      ly.codes[(size_t)row * ly.n + b0 + lc] = (uint8_t)qv[c];
      ly.Eb[(size_t)row * B + lc] = ev[c];
      if (ly.err) ly.err[(size_t)row * ly.n + b0 + lc] = ev[c];
    }
  }
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) {
    se += __shfl_xor(se, m, 16);
    sd += __shfl_xor(sd, m, 16);
  }
  if (rv && l16 == 0) {
    double* op = ly.objp + ((size_t)row * ly.nblk + blk) * 2;
    op[0] = se;
    op[1] = sd;
  }
}

// W[:, b1:nt] -= E[:, 0:K] U[b0:b1, b1:nt] for one 64x64 tile, K <= 128,
// on v_mfma_f32_32x32x2f32 (4 waves of 32x32).
__global__ __launch_bounds__(256) void k_trail(const QLayer* __restrict__ L,
                                               const Seg* __restrict__ segs, int nseg) {
  __shared__ float As[64][129];
  __shared__ float Bs[128][65];
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const QLayer ly = L[sg.prob];
  const int blk = sg.a, B = ly.block;
  const int b0 = blk * B, b1 = min(b0 + B, ly.n), K = b1 - b0;
  const int nt = ly.nt;
  const int tiles_j = (nt - b1 + 63) / 64;
  const int t = blockIdx.x - sg.wg0;
  const int i0 = 64 * (t / tiles_j), j0 = b1 + 64 * (t % tiles_j);
  const int mt = min(64, ly.out - i0), ntc = min(64, nt - j0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < 64 * 128; e += 256) {
    const int r = e >> 7, k = e & 127;
    As[r][k] = (r < mt && k < K) ? ly.Eb[(size_t)(i0 + r) * B + k] : 0.f;
  }
  for (int e = tid; e < 128 * 64; e += 256) {
    const int k = e >> 6, j = e & 63;
    Bs[k][j] = (k < K && j < ntc) ? ly.U[(size_t)(b0 + k) * nt + j0 + j] : 0.f;
  }
  __syncthreads();
  const int wr = w >> 1, wc = w & 1;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int ksteps = (K + 1) >> 1;
  for (int kk = 0; kk < ksteps; ++kk) {
    const float a = As[32 * wr + (lane & 31)][2 * kk + (lane >> 5)];
    const float b = Bs[2 * kk + (lane >> 5)][32 * wc + (lane & 31)];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 32 * wr + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int j = 32 * wc + (lane & 31);
    if (i < mt && j < ntc) ly.Ww[(size_t)(i0 + i) * nt + j0 + j] -= acc[r];
  }
}

// J_lam = sum E^2, ||D||^2 (plus the appended columns, whose final values are
// the compensation R), J = J_lam - lam ||D||^2; fixed-order reduction.
__global__ __launch_bounds__(256) void k_objective(const QLayer* __restrict__ L, int nl) {
  __shared__ double r0[256], r1[256];
  const int p = blockIdx.x;
  if (p >= nl) return;
  const QLayer ly = L[p];
  const int tid = threadIdx.x;
  double se = 0.0, sd = 0.0;
  const long long np = (long long)ly.out * ly.nblk;
  for (long long i = tid; i < np; i += 256) {
    se += ly.objp[2 * i];
    sd += ly.objp[2 * i + 1];
  }
  const int ne = ly.nt - ly.n;
  if (ne > 0) {
    const long long nx = (long long)ly.out * ne;
    for (long long i = tid; i < nx; i += 256) {
      const long long r = i / ne, c = ly.n + i % ne;
      const double v = ly.Ww[r * ly.nt + c];
      sd += v * v;
    }
  }
  r0[tid] = se;
  r1[tid] = sd;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (tid < k) {
      r0[tid] += r0[tid + k];
      r1[tid] += r1[tid + k];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double lam = *ly.lam;
    ly.obj[0] = r0[0] - lam * r1[0];
    ly.obj[1] = r0[0];
  }
}

#define QSEG_LAUNCH(name, kern, threads)                                                  \
  hipError_t name(const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st) {  \
    if (nwg <= 0) return hipSuccess;                                                      \
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(threads), 0, st, L, segs, nseg);             \
    return hipGetLastError();                                                             \
  }

QSEG_LAUNCH(launch_init_work, k_init_work, 256)
QSEG_LAUNCH(launch_rowfit, k_rowfit, 256)
QSEG_LAUNCH(launch_trail, k_trail, 256)

hipError_t launch_sweep(int block, const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st) {
  if (nwg <= 0) return hipSuccess;
  switch (block) {
    case 16: hipLaunchKernelGGL(k_sweep<1>, dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    case 32: hipLaunchKernelGGL(k_sweep<2>, dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    case 64: hipLaunchKernelGGL(k_sweep<4>, dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    case 128: hipLaunchKernelGGL(k_sweep<8>, dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_objective(const QLayer* L, int nl, hipStream_t st) {
  if (nl <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_objective, dim3(nl), dim3(256), 0, st, L, nl);
  return hipGetLastError();
}
