// Calibration Hessian H = X^T X on bf16 MFMA (gfx950).
//
// The Gram matrix of the calibration inputs (Lattice Geometry of NN
// Quantization, technical overview section 3.1; GPTQ-2D technical summary
// section 1) is a dense contraction over tokens with both operands stored
// feature-contiguous ([tokens, n] rows).  The MFMA wants 8 consecutive tokens
// per lane.  When X's rows are 16-byte aligned the tiles read X in place and
// transpose in the LDS read (ds_read_b64_tr_b16); otherwise X is first copied
// once, transposed and zero-padded, into a feature-major workspace (k_xpose)
// whose rows the tiles read directly.
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

// One 256x256 upper tile of H over the token range [k0, k1) (a multiple of
// 32 tokens; TR mode clamps and zeroes rows past the end of X).
//
// Four waves, one per SIMD; wave w owns the 128x128 quarter at rows
// 128 (w / 2), columns 128 (w % 2) of the tile: 4 x 4 accumulators of
// v_mfma_f32_32x32x16_bf16 (256 AGPRs).  A 128x128 block per wave is the
// largest the register file allows and needs the fewest LDS bytes per MFMA:
// each 16-token sub-step reads 8 operand fragments (16 transposing reads of
// 512 B) for 16 MFMAs, against 12 reads for 8 MFMAs with 128x64 blocks.
//
// Pipeline: a ring of 4 LDS stages of 32 tokens (each operand a 256-feature
// x 32-token tile, 16 KB); rows travel from L2 straight into LDS
// (global_load_lds, 16 B per lane) three stages ahead of the stage being
// multiplied.  The fragments of sub-step j+1 are read while the MFMAs of
// sub-step j run, one read issued after each MFMA, so the LDS port and the
// matrix pipe work side by side; a stage's copies are issued between the
// MFMAs of its second sub-step.
//
// TR = false: operands from the feature-major copy Xt ([feature][token]),
// one 16-byte row chunk per MFMA lane.  A stage holds 256 rows of 64 B, the
// 16-byte token chunks XOR-swizzled by (row / 4) % 4.
// TR = true: operands straight from X (token-major).  A stage holds 32 token
// rows of 256 features (512 B each, 16-byte chunks XOR-swizzled by
// 4 (row % 4)), and the fragments come out of LDS with the transposing read
// ds_read_b64_tr_b16: in each 16-lane group, lane i points at 4 features of
// token (i / 4) and receives 4 tokens of one feature, so two such reads give
// a lane the 8 consecutive tokens of its feature that the 32x32x16 MFMA
// wants, with no copy of X.
#define SYK_KT 32                   // tokens per stage
#define SYK_OPB (256 * SYK_KT * 2)  // bytes of one operand tile in a stage
#define SYK_STB (2 * SYK_OPB)       // bytes of a stage
#define SYK_NST 4                   // stages in the ring
#define SYK_NW 4                    // waves per workgroup (one per SIMD)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
#define SG_MFMA 0x008
#define SG_VMEM_RD 0x020
#define SG_DS_RD 0x100

template <bool DIAG, bool TR>
__device__ __forceinline__ void syrk_tile(const SyrkProb& pb, const SyrkTask& tk, uint8_t* lds,
                                          float* __restrict__ partials) {
  constexpr int NI = 4;                  // global_load_lds per operand per wave per stage (16 KB / 4 / 1 KB)
  constexpr int L = DIAG ? NI : 2 * NI;  // ... for both operands
  constexpr int NTH = 64 * SYK_NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets on the scalar unit
  const int nsteps = (tk.k1 - tk.k0) / SYK_KT;
  const size_t tp = (size_t)pb.ldt;
  const uint16_t* ga;
  const uint16_t* gb;
  size_t gstep, gq;  // element offsets per step and per instruction
  int tok0 = 0, trow = 0;
  if (!TR) {
    // instruction q of wave w fills the 16 LDS rows 16(4q+w) .. +15 (1 KB);
    // lane -> row 16(4q+w) + lane/4 at chunk position lane%4, holding token
    // chunk (lane%4) ^ ((row/4)%4) = (lane%4) ^ (lane/16)
    const int lrow = 16 * w + (lane >> 2);
    const int tchunk = (lane & 3) ^ (lane >> 4);
    ga = pb.Xt + (size_t)(tk.ti * 256 + lrow) * tp + tk.k0 + 8 * tchunk;
    gb = (pb.Yt ? pb.Yt : pb.Xt) + (size_t)(tk.tj * 256 + lrow) * tp + tk.k0 + 8 * tchunk;
    gstep = SYK_KT;
    gq = 16 * SYK_NW * tp;
  } else {
    // instruction q of wave w fills token rows 2(4q+w), 2(4q+w)+1 (1 KB);
    // lane -> row 2(4q+w) + lane/32 at chunk position lane%32, holding
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
  // TR copies: a stage's rows start at a uniform (scalar) address, and each
  // lane adds a 32-bit byte offset: its row 8q + trow and its feature chunk.
  // Rows past the end of X take the last row's offset instead (the stage's
  // tail is zeroed in LDS before use); cur[] holds the offsets of the stage
  // being copied.
  const unsigned rowb = (unsigned)pb.ldt * 2u;
  const unsigned lbA = TR ? 2u * (unsigned)(ga - pb.Xt) : 0u;
  const unsigned lbB = TR ? 2u * (unsigned)(gb - (pb.Yt ? pb.Yt : pb.Xt)) : 0u;
  const char* xa = (const char*)pb.Xt;
  const char* xb = (const char*)(pb.Yt ? pb.Yt : pb.Xt);
  unsigned curA[NI], curB[NI];
  // A stage that starts past the end of X (the last 32-token stage of a
  // 64-token chunk) reads row tokens-1 throughout; its rows are all zeroed.
  auto stage_row0 = [&](int step) {  // uniform: first token row read by the stage
    const int t0 = tok0 + step * SYK_KT;
    return t0 < pb.tokens ? t0 : pb.tokens - 1;
  };
  auto prep = [&](int step) {
    const int valid = pb.tokens - stage_row0(step);  // uniform; >= 1
    const unsigned lastrow = (unsigned)(valid - 1) * rowb;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int r = 2 * SYK_NW * q + trow;
      const unsigned ro = r < valid ? (unsigned)r * rowb : lastrow;
      curA[q] = ro + lbA;
      curB[q] = ro + lbB;
    }
  };
  auto issue_one = [&](int step, int stage, int q, bool bop) {
    uint8_t* base = lds + stage * SYK_STB + (bop ? SYK_OPB : 0);
    const void* src;
    if (!TR) {
      src = (bop ? gb : ga) + (size_t)q * gq + (size_t)step * gstep;
    } else {
      const size_t t0b = (size_t)stage_row0(step) * rowb;  // uniform
      src = (bop ? xb : xa) + t0b + (bop ? curB[q] : curA[q]);
    }
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + (SYK_NW * q + w) * 1024), 16, 0, 0);
  };
  auto issue = [&](int step, int stage) {
    if (TR) prep(step);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      issue_one(step, stage, q, false);
      if (!DIAG) issue_one(step, stage, q, true);
    }
  };
  // Fragment rows of this lane: 128 (w/2) + 32 m + lane%32 (A) and
  // 128 (w%2) + 32 q + lane%32 (B); all have (row/4)%4 == (lane/4)%4.
  const int arow = 128 * (w >> 1) + (lane & 31);
  const int brow = 128 * (w & 1) + (lane & 31);
  const int sw = (lane >> 2) & 3;
  // TR: 16-lane group g = lane/16, i = lane%16: features 16(g%2) + 4(i%4) of
  // the 32-feature block, tokens 8(g/2) + i/4 (+4 for the second read)
  const int tg = lane >> 4, ti4 = lane & 15;
  const int tr_tok = 8 * (tg >> 1) + (ti4 >> 2);
  const int tr_f = 16 * (tg & 1) + 4 * (ti4 & 3);
  // byte offset inside a stage of fragment k's first read (k < 4: A block m = k,
  // else B block q = k - 4), for token sub-step 0; sub-step 1 adds 16 token rows
  // (TR) or 32 bytes (!TR), the second TR read 4 token rows
  int foff[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int bop = k >= 4 && !DIAG;
    const int r = (k < 4 ? arow + 32 * k : brow + 32 * (k - 4));
    if (!TR) {
      foff[k] = bop * SYK_OPB + r * 64 + (((lane >> 5) ^ sw) << 4);
    } else {
      const int f = (k < 4 ? 128 * (w >> 1) + 32 * k : 128 * (w & 1) + 32 * (k - 4)) + tr_f;
      const int c = f >> 3, half = (f >> 2) & 1;
      foff[k] = bop * SYK_OPB + tr_tok * 512 + ((c ^ (4 * (tr_tok & 3))) << 4) + 8 * half;
    }
  }
  (void)arow;
  (void)brow;
  // The two reads (TR) or the one read (!TR) of fragment k of sub-step ks in
  // the stage at st.
  auto rd_lo = [&](const uint8_t* st, int ks, int k) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + foff[k] + ks * 16 * 512));
  };
  auto rd_hi = [&](const uint8_t* st, int ks, int k) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + foff[k] + ks * 16 * 512 + 4 * 512));
  };
  auto rd_b128 = [&](const uint8_t* st, int ks, int k) -> bf16x8 {
    // sub-step ks: token chunk 2 ks + lane/32, stored at (2 ks + lane/32) ^ sw
    const int off = foff[k] ^ ((2 * ks) << 4);
    return *(const bf16x8*)(st + off);
  };
  auto join = [](v4i16 lo, v4i16 hi) -> bf16x8 {
    const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][q][r] = 0.f;

  // MFMA order of a sub-step: new fragments come in gradually, in the order
  // they are read (A0 B0 B1 A1 B2 A2 B3 A3).
  constexpr int MORD[16][2] = {{0, 0}, {0, 1}, {1, 0}, {1, 1}, {0, 2}, {1, 2}, {2, 0}, {2, 1},
                               {2, 2}, {0, 3}, {1, 3}, {2, 3}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};
  constexpr int RORD[8] = {0, 4, 5, 1, 6, 2, 7, 3};  // fragment read order (k: A m = k, B q = k - 4)

  // One sub-step: the 16 MFMAs on cur[] with the 8 fragments of the next
  // sub-step (stage nst, sub-step nks) read into nxt[] in between; with
  // `loads`, the copies of stage `lstep` into slot `lslot` go between the
  // MFMAs too.  The reads are issued behind the first 12 MFMAs (two behind
  // each of the first four), so that they have landed when the next
  // sub-step starts: its first MFMA waits for every LDS read of this one.
  // The copies go behind the last 8 MFMAs.
  auto substep = [&](const bf16x8* cur, bf16x8* nxt, const uint8_t* nst, int nks, bool loads, int lstep,
                     int lslot) {
    const bf16x8* ca = cur;
    const bf16x8* cb = cur + 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = MORD[i][0], q = MORD[i][1];
      acc[m][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[m], cb[q], acc[m][q], 0, 0, 0);
      if ((i & 1) == 0) {
        const int k = RORD[i >> 1];
        if (TR) {
          const v4i16 lo = rd_lo(nst, nks, k);
          const v4i16 hi = rd_hi(nst, nks, k);
          nxt[k] = join(lo, hi);
        } else {
          nxt[k] = rd_b128(nst, nks, k);
        }
      }
      if (loads && i >= 8 && (!DIAG || (i & 1) == 0)) {
        issue_one(lstep, lslot, (i - 8) >> 1, !DIAG && (i & 1));
      }
    }
    // TR: 16 reads of 8 bytes per lane; !TR: 8 reads of 16 bytes
    constexpr int NR = TR ? 16 : 8;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      // TR: two reads behind MFMAs 0-3, one behind 4-11; !TR: one behind 0-7
      const int nr = NR == 16 ? (i < 4 ? 2 : (i < 12 ? 1 : 0)) : (i < 8 ? 1 : 0);
      if (nr == 2) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 2, 0);
      if (nr == 1) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
      if (loads && i >= 8 && (!DIAG || (i & 1) == 0)) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
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
  bf16x8 f0[8], f1[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f0[k] = TR ? join(rd_lo(lds, 0, k), rd_hi(lds, 0, k)) : rd_b128(lds, 0, k);
  }
  for (int s = 0; s < nsteps; ++s) {
    const uint8_t* st = lds + (s & 3) * SYK_STB;
    // sub-step 2s on f0, reading sub-step 2s+1 (same stage) into f1
    substep(f0, f1, st, 1, false, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // stage s+1 has landed (only stage s+2 may still be in flight) for this
    // wave, and after the barrier for every wave; stage s-1 is free
    __builtin_amdgcn_s_waitcnt(VmWait<L>::value);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (TR && s + 1 < nsteps && tok0 + (s + 2) * SYK_KT > pb.tokens) {  // uniform
      zero_tail(s + 1, (s + 1) & 3);
      __syncthreads();
    }
    // sub-step 2s+1 on f1, reading sub-step 2s+2 (stage s+1) into f0; the
    // copies of stage s+3 go into the slot of stage s-1
    if (TR) prep(min(s + 3, last));
    substep(f1, f0, lds + ((s + 1) & 3) * SYK_STB, 0, true, min(s + 3, last), (s + 3) & 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(VmWait<0>::value);  // no copy into LDS outlives the group

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
      syrk_tile<true, true>(pb, tk, lds, partials);
    else
      syrk_tile<false, true>(pb, tk, lds, partials);
  } else {
    if (diag)
      syrk_tile<true, false>(pb, tk, lds, partials);
    else
      syrk_tile<false, false>(pb, tk, lds, partials);
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
  const gptr<float> Hg = glb(pb.H);  // global view: H's accesses stay off lgkmcnt
  const int tid = threadIdx.x, n = pb.n;
  const int lr0 = tk.r0 & 255, lc0 = tk.c0 & 255;
  const int cc = tid & 63;
  // summing: thread t takes rows 4 (t / 16) .. +3 at columns 4 (t % 16) .. +3,
  // one 16-byte load per row and part (parts in list order)
  const int sr = 4 * (tid >> 4), sc = 4 * (tid & 15);
  f32x4 sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // four parts per trip: their list entries, then their 16 loads, all in
  // flight together; the sums still run part by part in list order
  const float* base = partials + (lr0 + sr) * 256 + lc0 + sc;
  for (int p0 = 0; p0 < tk.nparts; p0 += 4) {
    const int np = min(4, tk.nparts - p0);
    int pid[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pid[k] = k < np ? partlist[tk.part0 + p0 + k] : 0;
    f32x4 v[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      gptr<const f32x4> src = (gptr<const f32x4>)(base + (size_t)pid[k] * 65536);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[k][u] = k < np ? src[u * 64] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < np)
#pragma unroll
        for (int u = 0; u < 4; ++u) sum[u] += v[k][u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) S[sr + u][sc + w] = sum[u][w];
  __syncthreads();
  if (pb.accumulate) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rr = (tid >> 6) + 4 * q;
      const int i = tk.r0 + rr, j = tk.c0 + cc;
      if (i < n && j < n && (i <= j || pb.full)) S[rr][cc] += Hg[(size_t)i * n + j];
    }
    __syncthreads();
  }
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    if (i < n && j < n && (i <= j || pb.full)) Hg[(size_t)i * n + j] = S[rr][cc];
  }
  if (pb.full) return;  // a cross Gram has no mirror
  // mirror: H[j][i] = S[i][j] for i < j, written along contiguous rows of H
  for (int q = 0; q < 16; ++q) {
    const int ci = (tid >> 6) + 4 * q;  // column index inside the sub-block
    const int ri = tid & 63;            // row index inside the sub-block
    const int i = tk.r0 + ri, j = tk.c0 + ci;
    if (i < n && j < n && i < j) Hg[(size_t)j * n + i] = S[ri][ci];
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
  const gptr<double> Hg = glb(pb.H);  // global view: H's accesses stay off lgkmcnt
  const int tid = threadIdx.x, n = pb.n;
  const int lr0 = tk.r0 & 127, lc0 = tk.c0 & 127;
  // summing: thread t takes rows 4 (t / 16) .. +3 at columns 4 (t % 16) .. +3,
  // two 16-byte loads per row and part (parts in list order)
  const int sr = 4 * (tid >> 4), sc = 4 * (tid & 15);
  f64x2 sum[4][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u][0] = sum[u][1] = f64x2{0.0, 0.0};
  // two parts per trip: their list entries, then their 16 loads, all in
  // flight together; the sums still run part by part in list order
  const double* base = partials + (lr0 + sr) * 128 + lc0 + sc;
  for (int p0 = 0; p0 < tk.nparts; p0 += 2) {
    const int np = min(2, tk.nparts - p0);
    int pid[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) pid[k] = k < np ? partlist[tk.part0 + p0 + k] : 0;
    f64x2 v[2][4][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      gptr<const f64x2> src = (gptr<const f64x2>)(base + (size_t)pid[k] * 16384);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[k][u][0] = k < np ? src[u * 64] : f64x2{0.0, 0.0};
        v[k][u][1] = k < np ? src[u * 64 + 1] : f64x2{0.0, 0.0};
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (k < np)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sum[u][0] += v[k][u][0];
          sum[u][1] += v[k][u][1];
        }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) S[sr + u][sc + w] = sum[u][w >> 1][w & 1];
  __syncthreads();
  const int cc = tid & 63;
  for (int q = 0; q < 16; ++q) {
    const int rr = (tid >> 6) + 4 * q;
    const int i = tk.r0 + rr, j = tk.c0 + cc;
    if (i < n && j < n && i <= j) Hg[(size_t)i * n + j] = S[rr][cc];
  }
  for (int q = 0; q < 16; ++q) {
    const int ci = (tid >> 6) + 4 * q;
    const int ri = tid & 63;
    const int i = tk.r0 + ri, j = tk.c0 + ci;
    if (i < n && j < n && i < j) Hg[(size_t)j * n + i] = S[ri][ci];
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
