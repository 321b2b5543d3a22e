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
    *(u32x4*)(pb.Xt + (size_t)(f0 + f) * pb.ldt + t0 + r8) = o;
  }
}

// One 256x256 upper tile of H over the token range [k0, k1) of Xt (both
// multiples of 64; the copy is zero-padded, so no bounds are checked).
//
// Pipeline: a ring of 4 LDS stages of 32 tokens (each operand a 256-row x
// 64-byte tile, 16 KB); rows travel from L2 straight into LDS
// (global_load_lds, 16 B per lane, no registers in between) three stages
// ahead of the stage being multiplied.  Inside a row the 16-byte token chunks
// are stored XOR-swizzled by (row / 4) % 4, so a fragment read of 16
// consecutive rows covers all LDS banks.  Each wave owns a 128x128 quarter of
// the tile (4 x 4 MFMA 32x32x16 accumulators, 256 AGPRs); the fragment reads
// of the next 16-token sub-step are interleaved with the MFMAs of the current
// one, across the stage boundary too.
#define SYK_KT 32                   // tokens per stage
#define SYK_OPB (256 * SYK_KT * 2)  // bytes of one operand tile in a stage
#define SYK_STB (2 * SYK_OPB)       // bytes of a stage
#define SYK_NST 4                   // stages in the ring

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// TR = false: operands from the feature-major copy Xt, one 16-byte row chunk
// per MFMA lane.  TR = true: operands straight from X (token-major).  A stage
// then holds 32 token rows of 256 features (512 B each, 16-byte chunks
// XOR-swizzled by 4 (row % 4)), and the fragments come out of LDS with the
// transposing read ds_read_b64_tr_b16: in each 16-lane group, lane i points
// at 4 features of token (i / 4) and receives 4 tokens of one feature, so
// two such reads give a lane the 8 consecutive tokens of its feature that
// the 32x32x16 MFMA wants, with no copy of X.
template <bool DIAG, bool TR, int NW>
__device__ __forceinline__ void syrk_tile(const SyrkProb& pb, const SyrkTask& tk, uint8_t* lds,
                                          float* __restrict__ partials) {
  constexpr int NI = 16 / NW;                 // global_load_lds per operand per lane per stage
  constexpr int L = DIAG ? NI : 2 * NI;       // ... for both operands
  constexpr int WC = NW / 2;                  // waves across the tile's columns (2 down)
  constexpr int NBF = 8 / WC;                 // 32-column B fragments per wave
  constexpr int NTH = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nsteps = (tk.k1 - tk.k0) / SYK_KT;
  const size_t tp = (size_t)pb.ldt;
  const uint16_t* ga;
  const uint16_t* gb;
  size_t gstep, gq;  // element offsets per step and per instruction
  int tok0 = 0, trow = 0;
  if (!TR) {
    // Load slot: instruction q of wave w fills the 16 LDS rows 16(NW q+w) ..
    // 16(NW q+w)+15 (1 KB); lane -> row 16(NW q+w) + lane/4 at chunk
    // position lane%4, holding token chunk (lane%4) ^ ((row/4)%4) =
    // (lane%4) ^ (lane/16).
    const int lrow = 16 * w + (lane >> 2);
    const int tchunk = (lane & 3) ^ (lane >> 4);
    ga = pb.Xt + (size_t)(tk.ti * 256 + lrow) * tp + tk.k0 + 8 * tchunk;
    gb = (pb.Yt ? pb.Yt : pb.Xt) + (size_t)(tk.tj * 256 + lrow) * tp + tk.k0 + 8 * tchunk;
    gstep = SYK_KT;
    gq = 16 * NW * tp;
  } else {
    // instruction q of wave w fills token rows 2(NW q+w), 2(NW q+w)+1 (1 KB);
    // lane -> row 2(NW q+w) + lane/32 at chunk position lane%32, holding
    // feature chunk (lane%32) ^ 4 (row % 4).  Chunks past n read chunk 0.
    trow = 2 * w + (lane >> 5);
    const int chunk = (lane & 31) ^ (4 * (trow & 3));
    const int fa = tk.ti * 256 + 8 * chunk, fb = tk.tj * 256 + 8 * chunk;
    ga = pb.Xt + (fa < pb.n ? fa : tk.ti * 256);
    gb = (pb.Yt ? pb.Yt : pb.Xt) + (fb < pb.n ? fb : tk.tj * 256);
    tok0 = tk.k0;
    gstep = 0;
    gq = 0;
  }
  auto issue = [&](int step, int stage) {
    uint8_t* base = lds + stage * SYK_STB;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      size_t off;
      if (!TR) {
        off = (size_t)q * gq + (size_t)step * gstep;
      } else {
        // token row of this lane; rows past the end read the last row (the
        // stage's tail is zeroed in LDS before use)
        int t = tok0 + step * SYK_KT + 2 * NW * q + trow;
        t = t < pb.tokens ? t : pb.tokens - 1;
        off = (size_t)t * tp;
      }
      __builtin_amdgcn_global_load_lds((const void*)(ga + off), (lds_void*)(base + (NW * q + w) * 1024), 16, 0, 0);
      if (!DIAG)
        __builtin_amdgcn_global_load_lds((const void*)(gb + off), (lds_void*)(base + SYK_OPB + (NW * q + w) * 1024),
                                         16, 0, 0);
    }
  };
  // Fragment rows of this lane: arow + 32m (A), brow + 32q (B); all have
  // (row/4)%4 == (lane/4)%4.  Wave w: rows 128 (w / WC), columns
  // (256 / WC) (w % WC) of the tile.
  const int arow = 128 * (w / WC) + (lane & 31);
  const int brow = (256 / WC) * (w % WC) + (lane & 31);
  const int sw = (lane >> 2) & 3;
  // TR: 16-lane group g = lane/16, i = lane%16: features 16(g%2) + 4(i%4) of
  // the 32-feature block, tokens 8(g/2) + i/4 (+4 for the second read)
  const int tg = lane >> 4, ti4 = lane & 15;
  const int tr_tok = 8 * (tg >> 1) + (ti4 >> 2);
  const int tr_f = 16 * (tg & 1) + 4 * (ti4 & 3);
  auto tr_addr = [&](const uint8_t* st, int f, int tok) -> const lds_v4i16* {
    const int c = f >> 3, half = (f >> 2) & 1;
    return (const lds_v4i16*)(st + tok * 512 + ((c ^ (4 * (tok & 3))) << 4) + 8 * half);
  };
  auto rd = [&](const uint8_t* st, int ks, bf16x8* fa, bf16x8* fb) {
    const uint8_t* sb = DIAG ? st : st + SYK_OPB;
    if (!TR) {
      const int ch = ((2 * ks + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int m = 0; m < 4; ++m) fa[m] = *(const bf16x8*)(st + (arow + 32 * m) * 64 + ch);
#pragma unroll
      for (int q = 0; q < NBF; ++q) fb[q] = *(const bf16x8*)(sb + (brow + 32 * q) * 64 + ch);
    } else {
      const int tok = 16 * ks + tr_tok;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int f = 128 * (w / WC) + 32 * m + tr_f;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tr_addr(st, f, tok));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tr_addr(st, f, tok + 4));
        const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        fa[m] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int q = 0; q < NBF; ++q) {
        const int f = (256 / WC) * (w % WC) + 32 * q + tr_f;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tr_addr(sb, f, tok));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tr_addr(sb, f, tok + 4));
        const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        fb[q] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  // TR: zero the token rows of stage `stage` (step `step`) past the end of X
  auto zero_tail = [&](int step, int stage) {
    const int t0 = tok0 + step * SYK_KT;
    if (!TR || t0 + SYK_KT <= pb.tokens) return;  // uniform
    const int valid = pb.tokens - t0;  // may be <= 0
    uint8_t* base = lds + stage * SYK_STB;
    for (int e = tid; e < (DIAG ? 1 : 2) * SYK_KT * 32; e += NTH) {
      const int op = e / (SYK_KT * 32), row = (e / 32) % SYK_KT, c = e % 32;
      if (row >= valid) *(u32x4*)(base + op * SYK_OPB + row * 512 + c * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[4][NBF];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < NBF; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][q][r] = 0.f;
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < NBF; ++q)
        acc[m][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[q], acc[m][q], 0, 0, 0);
  };

  // Three stages in flight from the start; past the last step the copies
  // repeat the last step into stages nobody reads again (keeps the count of
  // copies in flight uniform).
  const int last = nsteps - 1;
  issue(0, 0);
  issue(min(1, last), 1);
  issue(min(2, last), 2);
  __builtin_amdgcn_s_waitcnt(VmWait<2 * L>::value);  // stage 0 has landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (TR && tok0 + SYK_KT > pb.tokens) {  // uniform: a tail already in stage 0
    zero_tail(0, 0);
    __syncthreads();
  }
  bf16x8 a0[4], b0[NBF], a1[4], b1[NBF];
  constexpr int NRD = (4 + NBF) * (TR ? 2 : 1);  // LDS reads per sub-step
  constexpr int NMF = 4 * NBF;                   // MFMAs per sub-step
  constexpr int NIL = NRD < NMF ? NRD : NMF;     // interleaved pairs
  rd(lds, 0, a0, b0);
  for (int s = 0; s < nsteps; ++s) {
    rd(lds + (s & 3) * SYK_STB, 1, a1, b1);
    mma(a0, b0);

    // stage s+1 has landed (only stage s+2 may still be in flight) for this
    // wave, and after the barrier for every wave; stage s-1 is free
    __builtin_amdgcn_s_waitcnt(VmWait<L>::value);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (TR && s + 1 < nsteps && tok0 + (s + 2) * SYK_KT > pb.tokens) {  // uniform
      zero_tail(s + 1, (s + 1) & 3);
      __syncthreads();
    }
    issue(min(s + 3, last), (s + 3) & 3);
    rd(lds + ((s + 1) & 3) * SYK_STB, 0, a0, b0);
    mma(a1, b1);

  }
  __builtin_amdgcn_s_waitcnt(VmWait<0>::value);  // no copy into LDS outlives the group

  float* P = partials + (size_t)tk.part * 65536;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < NBF; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * (w / WC) + 32 * m + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = (256 / WC) * (w % WC) + 32 * q + (lane & 31);
        P[row * 256 + col] = acc[m][q][r];
      }
}

#define SYK_NW 8  // waves per workgroup (2 per SIMD)
__global__ __launch_bounds__(64 * SYK_NW, 1) void k_syrk(const SyrkProb* __restrict__ probs,
                                                         const SyrkTask* __restrict__ tasks,
                                                         float* __restrict__ partials) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SYK_NST * SYK_STB];
  const SyrkTask tk = tasks[blockIdx.x];
  if (tk.part < 0) return;
  const SyrkProb pb = probs[tk.prob];
  const bool diag = tk.ti == tk.tj && !pb.Yt;  // one operand serves both sides
  if (pb.direct) {
    if (diag)
      syrk_tile<true, true, SYK_NW>(pb, tk, lds, partials);
    else
      syrk_tile<false, true, SYK_NW>(pb, tk, lds, partials);
  } else {
    if (diag)
      syrk_tile<true, false, SYK_NW>(pb, tk, lds, partials);
    else
      syrk_tile<false, false, SYK_NW>(pb, tk, lds, partials);
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
    if (pb.accumulate && i < n && j < n && (i <= j || pb.full)) s += pb.H[(size_t)i * n + j];
    S[rr][cc] = s;
  }
  __syncthreads();
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    if (i < n && j < n && (i <= j || pb.full)) pb.H[(size_t)i * n + j] = S[rr][cc];
  }
  if (pb.full) return;  // a cross Gram has no mirror
  // mirror: H[j][i] = S[i][j] for i < j, written along contiguous rows of H
  for (int q = 0; q < 16; ++q) {
    const int ci = (tid >> 6) + 4 * q;  // column index inside the sub-block
    const int ri = tid & 63;            // row index inside the sub-block
    const int i = tk.r0 + ri, j = tk.c0 + ci;
    if (i < n && j < n && i < j) pb.H[(size_t)j * n + i] = S[ri][ci];
  }
}

// ---------------------------------------------------------------------------
// Gram matrix accurate to float64 rounding, for callers whose later steps
// cancel most of H (the intrinsic-LoRA Schur complement loses the top
// eigen-directions of H against a damping of 1e-4 of its mean diagonal, so a
// float32 accumulation error of H is amplified beyond the codes' tolerance).
// bf16 values are exact in float64, so are their products; the sums run in
// float64 on v_mfma_f64_16x16x4.  One 128x128 upper tile per workgroup over
// a token range (multiple of 32), 4 waves of 64x64 (4 x 4 MFMA blocks).  The
// MFMA's four k-slots of step s take tokens 8k + s of a 32-token stage, so a
// lane reads its row's 8 consecutive tokens with one 16-byte LDS read and
// uses them over the stage's 8 steps (A and B use the same token order).
#define S64_ROWB 64                 // bytes per LDS row (32 tokens)
#define S64_OPB (128 * S64_ROWB)    // one operand tile per stage (8 KB)

__device__ __forceinline__ double bf16_to_f64(unsigned h) {
  return (double)__uint_as_float(h << 16);
}

template <bool DIAG>
__device__ __forceinline__ void syrk64_tile(const SyrkProb& pb, const SyrkTask& tk, uint8_t* lds,
                                            double* __restrict__ partials) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nsteps = (tk.k1 - tk.k0) / 32;
  const size_t tp = (size_t)pb.ldt;
  // instruction q of wave w fills LDS rows 16(4q+w)..+15 (1 KB): lane ->
  // row 16(4q+w) + lane/4 at chunk position lane%4 holding token chunk
  // (lane%4) ^ ((row/4)%4) = (lane%4) ^ (lane/16)
  const int lrow = 16 * w + (lane >> 2);
  const int tchunk = (lane & 3) ^ (lane >> 4);
  const uint16_t* ga = pb.Xt + (size_t)(tk.ti * 128 + lrow) * tp + tk.k0 + 8 * tchunk;
  const uint16_t* gb = pb.Xt + (size_t)(tk.tj * 128 + lrow) * tp + tk.k0 + 8 * tchunk;
  auto issue = [&](int step, int stage) {
    uint8_t* base = lds + stage * 2 * S64_OPB;
    const size_t off = (size_t)step * 32;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(ga + (size_t)(64 * q) * tp + off),
                                       (lds_void*)(base + (4 * q + w) * 1024), 16, 0, 0);
    if (!DIAG) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(gb + (size_t)(64 * q) * tp + off),
                                         (lds_void*)(base + S64_OPB + (4 * q + w) * 1024), 16, 0, 0);
    }
  };
  // fragment rows: 64(w/2) + 16 mb + lane%16 (A), 64(w%2) + 16 nb + lane%16 (B);
  // the lane reads token chunk lane/16, stored at chunk position
  // (lane/16) ^ ((row/4)%4) = (lane/16) ^ ((lane/4)%4)
  const int arow = 64 * (w >> 1) + (lane & 15);
  const int brow = 64 * (w & 1) + (lane & 15);
  const int ch = ((lane >> 4) ^ ((lane >> 2) & 3)) * 16;

  f64x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][q][r] = 0.0;

  if (nsteps > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) issue(s + 1, (s + 1) & 1);
    const uint8_t* As = lds + (s & 1) * 2 * S64_OPB;
    const uint8_t* Bs = DIAG ? As : As + S64_OPB;
    u32x4 fa[4], fb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) fa[m] = *(const u32x4*)(As + (arow + 16 * m) * S64_ROWB + ch);
#pragma unroll
    for (int q = 0; q < 4; ++q) fb[q] = *(const u32x4*)(Bs + (brow + 16 * q) * S64_ROWB + ch);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      double av[4], bv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const unsigned word = fa[m][st >> 1];
        av[m] = bf16_to_f64((st & 1) ? (word >> 16) : (word & 0xffffu));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned word = fb[q][st >> 1];
        bv[q] = bf16_to_f64((st & 1) ? (word >> 16) : (word & 0xffffu));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[m][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[m], bv[q], acc[m][q], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  double* P = partials + (size_t)tk.part * 16384;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 64 * (w >> 1) + 16 * m + (lane >> 4) + 4 * r;
        const int col = 64 * (w & 1) + 16 * q + (lane & 15);
        P[row * 128 + col] = acc[m][q][r];
      }
}

__global__ __launch_bounds__(256, 1) void k_syrk64(const SyrkProb* __restrict__ probs,
                                                   const SyrkTask* __restrict__ tasks,
                                                   double* __restrict__ partials) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * 2 * S64_OPB];
  const SyrkTask tk = tasks[blockIdx.x];
  if (tk.part < 0) return;
  const SyrkProb pb = probs[tk.prob];
  if (tk.ti == tk.tj)
    syrk64_tile<true>(pb, tk, lds, partials);
  else
    syrk64_tile<false>(pb, tk, lds, partials);
}

// Sum the float64 partials of one 64x64 sub-block of a 128x128 upper tile in
// list order; write the upper part and its mirror (exactly symmetric H).
__global__ __launch_bounds__(256) void k_syrk64_reduce(const RedProb64* __restrict__ probs,
                                                       const RedTask* __restrict__ tasks,
                                                       const int* __restrict__ partlist,
                                                       const double* __restrict__ partials) {
  __shared__ double S[64][65];
  const RedTask tk = tasks[blockIdx.x];
  const RedProb64 pb = probs[tk.prob];
  const int tid = threadIdx.x, n = pb.n;
  const int lr0 = tk.r0 & 127, lc0 = tk.c0 & 127;
  const int cc = tid & 63;
  double sum[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) sum[q] = 0.0;
  for (int p = 0; p < tk.nparts; ++p) {
    const double* src = partials + (size_t)partlist[tk.part0 + p] * 16384 + (lr0 + (tid >> 6)) * 128 + lc0 + cc;
    double v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = src[4 * q * 128];
#pragma unroll
    for (int q = 0; q < 16; ++q) sum[q] += v[q];
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) S[(tid >> 6) + 4 * q][cc] = sum[q];
  __syncthreads();
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    if (i < n && j < n && i <= j) pb.H[(size_t)i * n + j] = S[rr][cc];
  }
  for (int q = 0; q < 16; ++q) {
    const int ci = (tid >> 6) + 4 * q;
    const int ri = tid & 63;
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
  hipLaunchKernelGGL(k_syrk, dim3(ntasks), dim3(64 * SYK_NW), 0, st, probs, tasks, partials);
  return hipGetLastError();
}

hipError_t launch_syrk_reduce(const RedProb* probs, const RedTask* tasks, int ntasks,
                              const int* partlist, const float* partials, hipStream_t st) {
  if (ntasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_syrk_reduce, dim3(ntasks), dim3(256), 0, st, probs, tasks, partlist, partials);
  return hipGetLastError();
}

hipError_t launch_syrk64(const SyrkProb* probs, const SyrkTask* tasks, int ntasks, double* partials,
                         hipStream_t st) {
  if (ntasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_syrk64, dim3(ntasks), dim3(256), 0, st, probs, tasks, partials);
  return hipGetLastError();
}

hipError_t launch_syrk64_reduce(const RedProb64* probs, const RedTask* tasks, int ntasks, const int* partlist,
                                const double* partials, hipStream_t st) {
  if (ntasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_syrk64_reduce, dim3(ntasks), dim3(256), 0, st, probs, tasks, partlist, partials);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, long long count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  long long blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, count);
  return hipGetLastError();
}
