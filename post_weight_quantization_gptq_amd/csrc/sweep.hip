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
#include "grid.h"
#include "launch.h"

// Working copy of W (and zero columns n..nt-1 for the augmented variant),
// and 1 / U_jj for every column (the sweep's error scale), once per layer.
__global__ __launch_bounds__(256) void k_init_work(const QLayer* __restrict__ L,
                                                   const Seg* __restrict__ segs, int nseg) {
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const QLayer ly = L[sg.prob];
  const int wi = blockIdx.x - sg.wg0;
  for (int c = wi * 256 + threadIdx.x; c < ly.nt; c += sg.nwg * 256)
    ((float*)ly.dinv)[c] = 1.f / ly.U[(size_t)c * ly.nt + c];
  const int row = wi * 4 + (threadIdx.x >> 6);
  if (row >= ly.out) return;
  const int lane = threadIdx.x & 63;
  gptr<const float> src = glb(ly.W) + (size_t)row * ly.n;
  gptr<float> dst = glb(ly.Ww) + (size_t)row * ly.nt;
  if ((ly.n % 4) == 0 && (ly.nt % 4) == 0 && ((((uintptr_t)ly.W) | ((uintptr_t)ly.Ww)) & 15) == 0) {
    // 16 bytes per lane per step, several steps in flight
#pragma unroll 4
    for (int c = 4 * lane; c < ly.nt; c += 256)
      *(gptr<f32x4>)(dst + c) = c < ly.n ? *(gptr<const f32x4>)(src + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int c = lane; c < ly.nt; c += 64) dst[c] = c < ly.n ? src[c] : 0.f;
  }
  if (lane < 2) ly.objp[(size_t)row * 2 + lane] = 0.0;
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

// Broadcast lane SRC of each 16-lane row to the whole row (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ float bcast16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + SRC, 0xF, 0xF, false));
}

template <int CPL>
struct SweepState {
  float wv[CPL];  // current weights of this lane's columns
  float dv[CPL];  // 1/U_jj of this lane's columns
  float qv[CPL];  // codes
  float hv[CPL];  // dequantised values
  float ev[CPL];  // scaled errors
  Grid g;
  int nextg;      // next group start inside the block (or a large number)
};

struct SweepCtx {
  lptr<const float> Us;     // LDS U block
  gptr<const float> Wwrow;  // working row (global), columns past the super-block
  lptr<const float> Wsrow;  // the row's columns of the super-block in LDS, indexed by column - sb0
  float maxq;
  int B, bw, b0, G, l16, rv;
  int sb0, sb1;        // the super-block's columns [sb0, sb1)
  gptr<float> scales;
  gptr<uint8_t> zeros;
  size_t grow;  // row offset into scales/zeros
};

// Fit the grid of the group starting at in-block column j on the current
// values of columns [j, j+G): registers for the block, the super-block's
// rows in LDS past it, the working row in global memory past the
// super-block.
template <int CPL>
__device__ __forceinline__ void fit_group(SweepState<CPL>& st, const SweepCtx& cx, int j) {
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
  for (int c2 = 0; c2 < CPL; ++c2) {
    const int lc = CPL * cx.l16 + c2;
    if (lc >= j && lc < j + cx.G && lc < cx.bw) {
      mn = fminf(mn, st.wv[c2]);
      mx = fmaxf(mx, st.wv[c2]);
    }
  }
  if (j + cx.G > cx.B && cx.rv)  // group extends past this block
    for (int cc = cx.B + cx.l16; cc < j + cx.G; cc += 16) {
      const int col = cx.b0 + cc;
      const float v = col < cx.sb1 ? cx.Wsrow[col - cx.sb0] : cx.Wwrow[col];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 16));
    mx = fmaxf(mx, __shfl_xor(mx, m, 16));
  }
  st.g = grid_from(mn, mx, cx.maxq);
  if (cx.rv && cx.l16 == 0) {
    const size_t gi = cx.grow + (cx.b0 + j) / cx.G;
    cx.scales[gi] = st.g.s;
    cx.zeros[gi] = (uint8_t)st.g.z;
  }
}

// Bid-Up: the grid of the group starting at in-block column j, as given.
template <int CPL>
__device__ __forceinline__ void load_group(SweepState<CPL>& st, const SweepCtx& cx, int j) {
  const size_t gi = cx.grow + (cx.b0 + j) / cx.G;
  st.g.s = cx.scales[gi];
  st.g.r = 1.f / st.g.s;
  st.g.z = (float)cx.zeros[gi];
}

// The CPL columns owned by lane O of every row group.
// Groups are multiples of 8 >= CPL columns, so a group can only start at the
// first column of an owner lane: the check runs once per owner.
// Columns past the end of a ragged block need no test: their weights, U rows
// and 1/U_jj are zero, so they produce e = 0 and change nothing (their codes
// are never written).  Each step loads the next column's U row before its
// own chain starts, so the LDS latency stays off the serial path.
//
// Bid-Up (BID): the working row holds g = d H (d = w - c - what) and "U" is
// H itself.  Column j moves its code to the grid point nearest
// t = what_j + g_j / H_jj when that is strictly nearer (in the rounded
// coordinate x) than the current code; the move e = what_new - what_old is
// fed forward exactly as the sweep's error (g_k -= e H_jk), and the owner
// keeps the objective change e (e H_jj - 2 g_j) where the sweep keeps what.
// H_jj is the owner's own entry of row j of the block (ucur[c]).
template <int O, int CPL, bool BID>
__device__ __forceinline__ void sweep_owner(SweepState<CPL>& st, const SweepCtx& cx, float (&ucur)[CPL]) {
  constexpr int B = 16 * CPL;
  if (O * CPL == st.nextg && O * CPL < cx.bw) {
    if constexpr (BID)
      load_group<CPL>(st, cx, O * CPL);
    else
      fit_group<CPL>(st, cx, O * CPL);
    st.nextg += cx.G;
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = O * CPL + c;
    float unext[CPL];
    if (j + 1 < B) {
      lptr<const float> un = cx.Us + (j + 1) * B + CPL * cx.l16;
#pragma unroll
      for (int v = 0; v < CPL; ++v) unext[v] = un[v];
    }
    const float wj = bcast16<O>(st.wv[c]);
    float e;
    if constexpr (BID) {
      // dequantised values rounded as stored (__fmul_rn: no fusion into the
      // subtraction), so a code that stays put moves by exactly 0
      const float qo = bcast16<O>(st.qv[c]);
      const float ho = __fmul_rn(st.g.s, qo - st.g.z);
      const float t = fmaf(wj, bcast16<O>(st.dv[c]), ho);
      const float x = __fadd_rn(__fmul_rn(t, st.g.r), st.g.z);
      const float qs = fminf(fmaxf(rintf(x), 0.f), cx.maxq);
      const float qn = (fabsf(x - qs) < fabsf(x - qo)) ? qs : qo;
      e = __fmul_rn(st.g.s, qn - st.g.z) - ho;
      if (cx.l16 == O) {
        st.qv[c] = qn;
        st.hv[c] = e * fmaf(e, ucur[c], -2.f * wj);
        st.ev[c] = e;
      }
    } else {
      const float x = __fadd_rn(__fmul_rn(wj, st.g.r), st.g.z);
      const float q = fminf(fmaxf(rintf(x), 0.f), cx.maxq);
      const float what = __fmul_rn(st.g.s, q - st.g.z);  // as stored, not fused into the error
      e = (wj - what) * bcast16<O>(st.dv[c]);
      if (cx.l16 == O) {
        st.qv[c] = q;
        st.hv[c] = what;
        st.ev[c] = e;
      }
    }
    // take the owner's values now (an empty asm pins them), so the 16 owners'
    // candidates do not all stay live to the end of the block: 138 registers
    // instead of 439, which lets other kernels share the CU
    __asm__ volatile("" : "+v"(st.qv[c]), "+v"(st.hv[c]), "+v"(st.ev[c]));
#pragma unroll
    for (int c2 = 0; c2 < CPL; ++c2) st.wv[c2] = fmaf(-e, ucur[c2], st.wv[c2]);
    if (j + 1 < B) {
#pragma unroll
      for (int v = 0; v < CPL; ++v) ucur[v] = unext[v];
    }
  }
}

template <int O, int CPL, bool BID>
struct SweepAll {
  __device__ __forceinline__ static void run(SweepState<CPL>& st, const SweepCtx& cx, float (&ucur)[CPL]) {
    sweep_owner<O, CPL, BID>(st, cx, ucur);
    SweepAll<O + 1, CPL, BID>::run(st, cx, ucur);
  }
};
template <int CPL, bool BID>
struct SweepAll<16, CPL, BID> {
  __device__ __forceinline__ static void run(SweepState<CPL>&, const SweepCtx&, float (&)[CPL]) {}
};

// One super-block of sbk consecutive blocks for 16 rows per workgroup (4
// rows per wave, 16 lanes per row).  The rows' columns of the super-block
// stay in LDS for the whole launch; the errors of each swept block reach the
// rest of the super-block, W[rows, b1:sb1] -= E[rows, blk] U[blk, b1:sb1], on
// the workgroup's own fp32 MFMAs (v_mfma_f32_16x16x4f32, 64-column tiles,
// U read from L2 one work item ahead).  Columns past the super-block get one
// product per super-block afterwards (k_trail), from the errors stored in the
// super-block's half of the error buffer.
//
// 128-wide blocks take eight waves: four sweep, and four apply the updates.
// Right after a block is swept, the update waves apply its errors to the next
// block's columns only; the rest of that product (the columns past the next
// block) runs while the next block is swept, beside the sweeping waves on the
// same SIMDs, with the errors double-buffered by block parity.  Every column
// still takes the blocks' products in block order, each summed in the same
// order as by one pass per block.  A group fit reads columns past its block,
// which that overlapped product may still be writing, so layers whose groups
// do not nest in a block keep one pass per block.  Narrower blocks: four
// waves, which sweep and then apply each block's product.
//
// BID: one Bid-Up pass instead of the GPTQ sweep (codes are read as the
// starting point, the grid is the one given, and the per-row sums are the
// objective changes of the moves).
// Widest super-block for blocks of B columns (the planner keeps to it):
// 1024 columns at B = 128 (138 KB of LDS, one workgroup per CU either way),
// 512 below (at B = 64, 53 KB: three workgroups per CU, which the batched
// small layers need)
template <int B>
constexpr int sweep_sbw() {
  return B >= 128 ? 1024 : 512;
}
template <int B>
struct SweepLds {
  static constexpr int WP = sweep_sbw<B>() + 4;
  static constexpr int EP = B + 4;
  float us[B * B];   // the diagonal block of U
  float ws[16 * WP];  // the rows' columns of the super-block
  // the errors of a block (by block parity for the 128-wide blocks, whose
  // far update runs during the next block's sweep)
  static constexpr int NE = B >= 128 ? 2 : 1;
  float es[NE][16 * EP];
};

template <int CPL, bool BID>
__global__ __launch_bounds__(CPL == 8 ? 512 : 256) void k_sweep(const QLayer* __restrict__ L,
                                                                const Seg* __restrict__ segs, int nseg) {
  constexpr int B = 16 * CPL;
  // 128-wide blocks: four more waves apply the previous block's errors to the
  // super-block's far columns while the first four sweep the current block
  constexpr bool SPLIT = CPL == 8;
  constexpr int NTH = SPLIT ? 512 : 256;
  using LD = SweepLds<B>;
  __shared__ __attribute__((aligned(16))) LD lds;
  float* Us = lds.us;
  const Seg sg = segs[find_seg(segs, nseg, blockIdx.x)];
  const QLayer ly = L[sg.prob];
  const int sbi = sg.a;  // super-block index
  const int kb0 = sbi * ly.sbk, kb1 = min(kb0 + ly.sbk, ly.nblk);
  const int sb0 = kb0 * B, sb1 = min(kb1 * B, ly.n), sbw = sb1 - sb0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool chain = w < 4;             // sweeps the rows (all waves unless SPLIT)
  const int uw = SPLIT ? (w & 3) : w;   // index among the waves that apply updates
  const int l16 = lane & 15, rr = (w & 3) * 4 + (lane >> 4);
  const int r0 = (blockIdx.x - sg.wg0) * 16;
  const int row = r0 + rr;
  const bool rv = chain && row < ly.out;
  const int nt = ly.nt, G = ly.group;
  // overlap the far update with the next block's sweep only where no group
  // fit reads past its block (a fit reads columns the overlapped update is
  // still writing): Bid-Up, per-row grids, or groups that nest in a block
  const bool ovl = SPLIT && (BID || G == 0 || (B % G) == 0);

  // the diagonal block U[b0r:b0r+bwr, c0:c0+cw] (c0 = b0r, cw = bwr) -> LDS at
  // pitch B, zero past the ragged edge; all loads of a thread in flight at once
  auto load_u = [&](int b0r, int bwr, int c0, int cw, int pitch) {
    constexpr int PER = B * B / 4 / 256 > 0 ? B * B / 4 / 256 : 1;
    const bool vec = (nt % 4) == 0 && (c0 % 4) == 0 && cw == B;
    f32x4 tmp[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = tid + 256 * q;
      const int j = idx / (B / 4), k4 = (idx % (B / 4)) * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (idx < B * B / 4 && j < bwr) {
        gptr<const float> src = glb(ly.U) + (size_t)(b0r + j) * nt + c0 + k4;
        if (vec) {
          v = *(gptr<const f32x4>)src;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = (k4 + u < cw) ? src[u] : 0.f;
        }
      }
      tmp[q] = v;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = tid + 256 * q;
      const int j = idx / (B / 4), k4 = (idx % (B / 4)) * 4;
      if (idx < B * B / 4) *(f32x4*)&Us[j * pitch + k4] = tmp[q];
    }
  };

  // the rows' super-block columns -> LDS (zeros for rows past the end), the
  // first diagonal block of U, and the rows' objective sums so far
  {
    const bool vec = (nt % 4) == 0 && (sbw % 4) == 0;
    const int per_row = (sbw + 3) / 4;
    for (int e = tid; e < 16 * per_row; e += NTH) {
      const int r = e / per_row, c4 = (e % per_row) * 4;
      const int gr = r0 + r;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (gr < ly.out) {
        gptr<const float> src = glb((const float*)ly.Ww) + (size_t)gr * nt + sb0 + c4;
        if (vec) {
          v = *(gptr<const f32x4>)src;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = (c4 + u < sbw) ? src[u] : 0.f;
        }
      }
      *(f32x4*)&lds.ws[r * LD::WP + c4] = v;
    }
  }
  if (tid < 256) load_u(sb0, min(B, ly.n - sb0), sb0, min(B, ly.n - sb0), B);
  double obj_e = 0.0, obj_d = 0.0;
  if (rv && l16 == 0) {
    obj_e = glb(ly.objp)[(size_t)row * 2];
    obj_d = glb(ly.objp)[(size_t)row * 2 + 1];
  }
  SweepState<CPL> st;
  st.g = Grid{1.f, 1.f, 0.f};
  if (rv && (G == 0 || (sb0 % G) != 0)) {
    // the row's grid, or the grid of a group that began in an earlier super-block
    const size_t gi = (size_t)row * ly.ng + (G ? sb0 / G : 0);
    st.g.s = glb(ly.scales)[gi];
    st.g.r = 1.f / st.g.s;
    st.g.z = (float)glb(ly.zeros)[gi];
  }
  SweepCtx cx;
  cx.Us = lds_view((const float*)Us);
  cx.Wwrow = glb((const float*)ly.Ww) + (size_t)(rv ? row : 0) * nt;
  cx.Wsrow = lds_view((const float*)lds.ws) + rr * LD::WP;
  cx.maxq = (float)((1 << ly.bits) - 1);
  cx.B = B;
  cx.G = G;
  cx.l16 = l16;
  cx.rv = rv;
  cx.sb0 = sb0;
  cx.sb1 = sb1;
  cx.scales = glb(ly.scales);
  cx.zeros = glb(ly.zeros);
  cx.grow = (size_t)(rv ? row : 0) * ly.ng;
  double se = 0.0, sd = 0.0;  // this lane's sums over the super-block, in block order
  // the next block's per-column inputs, loaded ahead (their latency hides
  // behind the previous block's update)
  float pdv[CPL], pwo[CPL], pqv[CPL];
  auto prefetch = [&](int blk) {
    const int b0 = blk * B, bw = min(B, ly.n - b0);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int lc = CPL * l16 + c;
      const bool in = rv && lc < bw;
      pdv[c] = (lc < bw) ? glb(ly.dinv)[b0 + lc] : 0.f;
      pwo[c] = (in && !BID) ? glb(ly.W)[(size_t)row * ly.n + b0 + lc] : 0.f;
      pqv[c] = (in && BID) ? (float)glb(ly.codes)[(size_t)row * ly.n + b0 + lc] : 0.f;
    }
  };
  // a whole B x B diagonal block of U straight into LDS (pitch B), 1 KB per
  // instruction, without registers; in flight during the update
  const bool u_dma = (nt % 4) == 0 && (((uintptr_t)ly.U) & 15) == 0;
  auto dma_u = [&](int nb0) {
    constexpr int NINST = B * B / 256;  // 1 KB instructions for the block
    constexpr int RPI = 256 / B;        // rows per instruction
    const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int q = 0; q < (NINST + 3) / 4; ++q) {
      const int inst = 4 * q + wu;
      if (inst < NINST) {
        const int r = inst * RPI + (4 * lane) / B, cc = (4 * lane) % B;
        __builtin_amdgcn_global_load_lds((const void*)(ly.U + (size_t)(nb0 + r) * nt + nb0 + cc),
                                         (lds_void*)(Us + inst * 256), 16, 0, 0);
      }
    }
  };
  if (chain) prefetch(kb0);

  // W[rows, b1:sb1) -= E U[b0:b0+B, b1:sb1) with the errors of the block at
  // b0 (error buffer eb), by the update waves (index uw of four)
    // The block's errors reach the rest of the super-block:
    // W[rows, b1:sb1] -= E[rows, blk] U[blk, b1:sb1] on v_mfma_f32_16x16x4f32,
    // one tile of 16 rows x 64 columns per wave at a time.  K order: lane
    // group g = lane / 16 takes k = (B / 4) g + kk at step kk (the same in
    // both operands), so a lane's E values are contiguous in LDS; the four
    // MFMAs of a step take columns 4 (lane % 16) + u, u = 0..3, of the tile,
    // so a lane's U values are one 16-byte load per step.  bw == B whenever
    // columns follow the block (only the layer's last block is ragged).
  auto apply = [&](int eb, int b0, int b1, int sb1) {
      constexpr int KQ = B / 4;
      constexpr int KH = KQ > 8 ? 8 : KQ;  // K steps per work item
      constexpr int NH = KQ / KH;          // items per 64-column tile
      const int li = lane & 15, g = lane >> 4;
      const bool uvec = (nt % 4) == 0 && (((uintptr_t)ly.U) & 15) == 0;
      // this wave's work items: tiles c0 = b1 + 64 (uw + 4 i), each in NH
      // K-halves; the U loads of item it+1 are in flight while item it is
      // multiplied
      const int ntile = (sb1 - b1 + 63) / 64;
      const int myt = ntile > uw ? (ntile - uw + 3) / 4 : 0;
      const int nitem = myt * NH;
      auto load_item = [&](int it, f32x4 (&ub)[KH]) {
        const int c0 = b1 + 64 * (uw + 4 * (it / NH)), h = it % NH;
        const int col = c0 + 4 * li;
        const bool full = uvec && col + 4 <= sb1;
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) {
          gptr<const float> src = glb(ly.U) + (size_t)(b0 + KQ * g + KH * h + kk) * nt + col;
          if (full) {
            ub[kk] = *(gptr<const f32x4>)src;
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) ub[kk][u] = (col + u < sb1) ? src[u] : 0.f;
          }
        }
      };
      f32x4 ubA[KH], ubB[KH];
      f32x4 acc[4];
      if (nitem > 0) load_item(0, ubA);
      for (int it = 0; it < nitem; it += 2) {
        // two items per trip (register sets A and B alternate)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int cur = it + half;
          if (cur >= nitem) break;
          f32x4 (&ubc)[KH] = half ? ubB : ubA;
          f32x4 (&ubn)[KH] = half ? ubA : ubB;
          if (cur + 1 < nitem) load_item(cur + 1, ubn);
          const int c0 = b1 + 64 * (uw + 4 * (cur / NH)), h = cur % NH;
          const int col = c0 + 4 * li;
          if (h == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          float ea[KH];
#pragma unroll
          for (int k4 = 0; k4 < KH / 4; ++k4) {
            const f32x4 v = *(const f32x4*)&lds.es[eb][li * LD::EP + KQ * g + KH * h + 4 * k4];
            ea[4 * k4] = v[0];
            ea[4 * k4 + 1] = v[1];
            ea[4 * k4 + 2] = v[2];
            ea[4 * k4 + 3] = v[3];
          }
#pragma unroll
          for (int kk = 0; kk < KH; ++kk)
#pragma unroll
            for (int u = 0; u < 4; ++u)
              acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[kk], ubc[kk][u], acc[u], 0, 0, 0);
          if (h == NH - 1) {
            // lane: rows 4 g + q, columns col + u
            const bool full = col + 4 <= sb1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float* wr = &lds.ws[(4 * g + q) * LD::WP + col - sb0];
              if (full) {
                f32x4 v = *(f32x4*)wr;
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] -= acc[u][q];
                *(f32x4*)wr = v;
              } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  if (col + u < sb1) wr[u] -= acc[u][q];
              }
            }
          }
        }
      }
    };
  __syncthreads();
  for (int blk = kb0; blk < kb1; ++blk) {
    const int b0 = blk * B, b1 = min(b0 + B, ly.n), bw = b1 - b0;
    if (chain) {
    cx.bw = bw;
    cx.b0 = b0;
    float wo[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int lc = CPL * l16 + c;
      st.wv[c] = lc < bw ? lds.ws[rr * LD::WP + b0 - sb0 + lc] : 0.f;
      st.dv[c] = pdv[c];
      wo[c] = pwo[c];
      st.qv[c] = pqv[c];
      st.hv[c] = 0.f;
      st.ev[c] = 0.f;
    }
    st.nextg = (G == 0) ? (1 << 30) : ((b0 % G) == 0 ? 0 : G - (b0 % G));

    float ucur[CPL];
#pragma unroll
    for (int v = 0; v < CPL; ++v) ucur[v] = Us[CPL * l16 + v];
    SweepAll<0, CPL, BID>::run(st, cx, ucur);

#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int lc = CPL * l16 + c;
      lds.es[(blk & 1) % LD::NE][rr * LD::EP + lc] = st.ev[c];  // zero past bw (the sweep leaves ev = 0 there)
      if (rv && lc < bw) {
        glb(ly.codes)[(size_t)row * ly.n + b0 + lc] = (uint8_t)st.qv[c];
        glb(ly.Eb)[((size_t)((blk / ly.sbk) & 1) * ly.out + row) * ly.ldE + ly.eoff_blk * (blk % ly.sbk) + lc] = st.ev[c];
        if (ly.err) glb(ly.err)[(size_t)row * ly.n + b0 + lc] = st.ev[c];
        if (BID) {
          se += (double)st.hv[c];
        } else {
          const double d = (double)wo[c] - (double)st.hv[c];
          sd += d * d;
          se += (double)st.ev[c] * (double)st.ev[c];
        }
      }
    }
    } else if (ovl && blk > kb0) {
      // the previous block's errors on the columns past this block (this
      // block's own columns took them before its sweep)
      apply(((blk - 1) & 1) % LD::NE, b0 - B, b1, sb1);
    }
    __syncthreads();  // the errors are in LDS; the diagonal U block is free
    const bool more = blk + 1 < kb1;
    const int nb0 = b1, nbw = more ? min(B, ly.n - nb0) : 0;
    const bool dma = more && u_dma && nbw == B;
    if (more && chain) {
      prefetch(blk + 1);
      if (dma) dma_u(nb0);
    }
    // this block's errors: on the next block's columns only when the far ones
    // are left to the update waves during the next sweep, else on every
    // column past the block
    if (!SPLIT || !chain) apply((blk & 1) % LD::NE, b0, b1, ovl ? min(b1 + B, sb1) : sb1);
    if (more && !dma && tid < 256) load_u(nb0, nbw, nb0, nbw, B);
    __builtin_amdgcn_s_waitcnt(0);  // the next diagonal block has landed
    __syncthreads();                // the updated columns and that block are visible
  }

#pragma unroll
  for (int m = 8; m > 0; m >>= 1) {
    se += __shfl_xor(se, m, 16);
    sd += __shfl_xor(sd, m, 16);
  }
  if (rv && l16 == 0) {
    // per-row sums, accumulated over the super-blocks in order
    gptr<double> op = glb(ly.objp) + (size_t)row * 2;
    op[0] = obj_e + se;
    op[1] = obj_d + sd;
  }
}

// W[:, j0:j1] -= E[:, eoff:eoff+K] U[kb:kb+K, j0:j1] for one TS x TS tile
// (TS = 128 for the products past a super-block, 64 for the narrow ones
// inside it), on v_mfma_f32_32x32x2f32 (4 waves of TS/2 x TS/2).  K chunks of
// 32 go through registers into a double-buffered LDS pair, so the loads of
// chunk c+1 are in flight while chunk c is multiplied.  The tile's W is read
// after the K loop, which keeps the 128-wide tile within 256 registers, so
// two workgroups share a CU and cover each other's stalls.
template <int TS>
__global__ __launch_bounds__(256, 2) void k_trail(const QLayer* __restrict__ L, const Seg* __restrict__ segs, int nseg,
                                               int ntot) {
  constexpr int KC = 32;
  constexpr int MB = TS / 64;        // 32x32 blocks per wave side
  constexpr int TPR = 256 / TS;      // threads per E row
  constexpr int VA = KC / TPR;       // E values per thread (multiple of 4)
  constexpr int TPK = 256 / KC;      // threads per U row (k)
  constexpr int VB = TS / TPK;       // U values per thread (multiple of 4)
  static_assert(VA % 4 == 0 && VB % 4 == 0 && VB >= 4, "load split");
  __shared__ float As[2][TS][KC + 1];
  __shared__ __attribute__((aligned(16))) float Bs[2][KC][TS + 4];
  // tiles vt = blockIdx.x, blockIdx.x + gridDim.x, ... < ntot (persistent when
  // the grid is smaller than the tile count)
  for (int vt = blockIdx.x; vt < ntot; vt += gridDim.x) {
  const Seg sg = segs[find_seg(segs, nseg, vt)];
  const QLayer ly = L[sg.prob];
  const int eoff = sg.a, kb = sg.b, K = sg.c, j0 = sg.d, j1 = sg.e;
  const int nt = ly.nt;
  const int tiles_j = (j1 - j0 + TS - 1) / TS;
  const int t = vt - sg.wg0;
  const int i0 = TS * (t / tiles_j), jj0 = j0 + TS * (t % tiles_j);
  const int mt = min(TS, ly.out - i0), ntc = min(TS, j1 - jj0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1;
  f32x16 acc[MB][MB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int ar = tid / TPR, ak = (tid % TPR) * VA;  // E: row, first k
  // U: k row; the thread's 16-byte chunks are 4 (tid % TPK) + 4 TPK q, so the
  // TPK threads of a row write consecutive chunks (no bank conflicts)
  const int bk = tid / TPK, bj = (tid % TPK) * 4;
  const bool arow_ok = ar < mt;
  gptr<const float> ap = glb((const float*)ly.Eb) + (size_t)(i0 + (arow_ok ? ar : 0)) * ly.ldE + eoff;
  const bool evec = (ly.ldE % 4) == 0 && (eoff % 4) == 0;
  const bool uvec = (nt % 4) == 0 && (jj0 % 4) == 0 && (((uintptr_t)ly.U) & 15) == 0;
  // The tile's W, loaded first so its latency hides behind the K loop, and
  // all of it before any store (the stores could alias the loads as far as
  // the compiler knows, so interleaving them would cost one memory round
  // trip per element).  Every global access goes through a global view: a
  // generic pointer's flat accesses also count against lgkmcnt, so the LDS
  // waits of the K loop would drain the next chunk's loads with them.
  gptr<float> wbase = glb(ly.Ww) + (size_t)i0 * nt + jj0;
  f32x4 ra[VA / 4], rb[VB / 4];
  auto load = [&](int kc) {
#pragma unroll
    for (int q = 0; q < VA / 4; ++q) {
      const int k = kc + ak + 4 * q;
      if (evec && arow_ok && k + 4 <= K) {
        ra[q] = *(gptr<const f32x4>)(ap + k);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool ok = arow_ok && k + u < K;
          const float v = ap[ok ? k + u : 0];
          ra[q][u] = ok ? v : 0.f;
        }
      }
    }
    const int k = kc + bk;
    const bool kok = k < K;
    gptr<const float> bp = glb(ly.U) + (size_t)(kb + (kok ? k : 0)) * nt + jj0;
#pragma unroll
    for (int q = 0; q < VB / 4; ++q) {
      const int j = bj + 4 * TPK * q;
      if (uvec && kok && j + 4 <= ntc) {
        rb[q] = *(gptr<const f32x4>)(bp + j);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool ok = kok && j + u < ntc;
          const float v = bp[ok ? j + u : 0];
          rb[q][u] = ok ? v : 0.f;
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < VA / 4; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) As[buf][ar][ak + 4 * q + u] = ra[q][u];
#pragma unroll
    for (int q = 0; q < VB / 4; ++q) *(f32x4*)&Bs[buf][bk][bj + 4 * TPK * q] = rb[q];
  };
  if (K > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  int buf = 0;
  for (int kc = 0; kc < K; kc += KC) {
    const bool more = kc + KC < K;
    if (more) load(kc + KC);
#pragma unroll
    for (int kk = 0; kk < KC / 2; ++kk) {
      float av[MB], bv[MB];
#pragma unroll
      for (int mi = 0; mi < MB; ++mi) av[mi] = As[buf][(TS / 2) * wr + 32 * mi + (lane & 31)][2 * kk + (lane >> 5)];
#pragma unroll
      for (int ni = 0; ni < MB; ++ni) bv[ni] = Bs[buf][2 * kk + (lane >> 5)][(TS / 2) * wc + 32 * ni + (lane & 31)];
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int ni = 0; ni < MB; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int ni = 0; ni < MB; ++ni) {
      float cur[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (TS / 2) * wr + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int j = (TS / 2) * wc + 32 * ni + (lane & 31);
        cur[r] = (i < mt && j < ntc) ? wbase[(size_t)i * nt + j] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (TS / 2) * wr + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int j = (TS / 2) * wc + 32 * ni + (lane & 31);
        if (i < mt && j < ntc) wbase[(size_t)i * nt + j] = cur[r] - acc[mi][ni][r];
      }
    }
  __syncthreads();  // the next tile refills the LDS pair
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
  for (long long i = tid; i < ly.out; i += 256) {
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
hipError_t launch_trail(int ts, const QLayer* L, const Seg* segs, int nseg, int nwg, int maxwg, hipStream_t st) {
  if (nwg <= 0) return hipSuccess;
  const int grid = (maxwg > 0 && maxwg < nwg) ? maxwg : nwg;
  if (ts == 64)
    hipLaunchKernelGGL(k_trail<64>, dim3(grid), dim3(256), 0, st, L, segs, nseg, nwg);
  else
    hipLaunchKernelGGL(k_trail<128>, dim3(grid), dim3(256), 0, st, L, segs, nseg, nwg);
  return hipGetLastError();
}

template <bool BID>
hipError_t launch_sweep_t(int block, const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st) {
  switch (block) {
    case 16: hipLaunchKernelGGL((k_sweep<1, BID>), dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    case 32: hipLaunchKernelGGL((k_sweep<2, BID>), dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    case 64: hipLaunchKernelGGL((k_sweep<4, BID>), dim3(nwg), dim3(256), 0, st, L, segs, nseg); break;
    case 128: hipLaunchKernelGGL((k_sweep<8, BID>), dim3(nwg), dim3(512), 0, st, L, segs, nseg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sweep(int block, int mode, const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st) {
  if (nwg <= 0) return hipSuccess;
  return mode ? launch_sweep_t<true>(block, L, segs, nseg, nwg, st) : launch_sweep_t<false>(block, L, segs, nseg, nwg, st);
}

hipError_t launch_objective(const QLayer* L, int nl, hipStream_t st) {
  if (nl <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_objective, dim3(nl), dim3(256), 0, st, L, nl);
  return hipGetLastError();
}
