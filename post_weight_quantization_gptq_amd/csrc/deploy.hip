// Deployable outputs of a quantised layer (gfx950): packed code words, the
// low-rank factors on low-precision grids, and the product of bf16
// activations with 4-bit weights (W4A16).
//
// GPTQ encyclopedia entry, technical approach (the quantised weights are used
// through GPU matrix kernels at inference) and performance and accuracy
// (4-bit weights take a quarter of the fp32 memory); GPTQ-intrinsic LoRA
// technical summary, results: L and R themselves stored at low precision (4
// and 8 bits).  The pages fix no storage format; ours is stated per kernel.
#include "common.h"
#include "grid.h"
#include "launch.h"

typedef const __attribute__((address_space(1))) uint32_t gu32;
typedef const __attribute__((address_space(1))) u32x4 gu32x4;
typedef const __attribute__((address_space(1))) uint8_t gu8;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------- packing --
// Rows of codes as little-endian bitstreams in 32-bit words: code k of a row
// occupies stream bits [k bits, (k + 1) bits), stream bit b sits in word b/32
// at position b%32, and the row ends in zero bits up to a whole word.  One
// thread per output word; bits of a code above `bits` are ignored.
__global__ __launch_bounds__(256) void k_pack(const uint8_t* __restrict__ codes, int rows, int n, int bits,
                                              int words, uint32_t* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * words) return;
  const int i = (int)(idx / words), w = (int)(idx % words);
  const uint8_t* c = codes + (size_t)i * n;
  const int b0 = 32 * w;
  const int kend = min(n, (b0 + 31) / bits + 1);
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t v = 0;
  for (int k = b0 / bits; k < kend; ++k) {
    const int off = k * bits - b0;  // negative for a code begun in the previous word
    const uint32_t q = c[k] & mask;
    v |= off >= 0 ? (q << off) : (q >> -off);
  }
  out[idx] = v;
}

// The inverse: one thread per code.
__global__ __launch_bounds__(256) void k_unpack(const uint32_t* __restrict__ packed, int rows, int n, int bits,
                                                int words, uint8_t* __restrict__ codes) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * n) return;
  const int i = (int)(idx / n), k = (int)(idx % n);
  const uint32_t* p = packed + (size_t)i * words;
  const int b = k * bits, w = b >> 5, off = b & 31;
  uint32_t v = p[w] >> off;
  if (off + bits > 32) v |= p[w + 1] << (32 - off);
  codes[idx] = (uint8_t)(v & ((1u << bits) - 1u));
}

// ------------------------------------------------- low-rank factors --
// One workgroup per rank component (a column of L, then a row of R): the
// min-max grid of the sweep over the component, then round-to-nearest with
// the sweep's fp32 steps, x = fl32(fl32(v r) + z), q = clamp(rne(x)),
// vhat = fl32(s (q - z)).
__global__ __launch_bounds__(256) void k_lr_quant(const LrProb p) {
  __shared__ float red[2][4];
  const int c = blockIdx.x, tid = threadIdx.x;
  const bool isL = c < p.r;
  const int comp = isL ? c : c - p.r;
  const int len = isL ? p.n : p.out;
  const size_t stride = isL ? (size_t)p.r : 1;
  const size_t base = isL ? (size_t)comp : (size_t)comp * p.out;
  const float* src = (isL ? p.L : p.R) + base;
  float mn = INFINITY, mx = -INFINITY;
  for (int i = tid; i < len; i += 256) {
    const float v = src[i * stride];
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = mn;
    red[1][tid >> 6] = mx;
  }
  __syncthreads();
  mn = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
  mx = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const float maxq = (float)(isL ? p.maxqL : p.maxqR);
  const Grid g = grid_from(mn, mx, maxq);
  uint8_t* codes = (isL ? p.Lc : p.Rc) + base;
  float* hat = isL ? p.Lh : p.Rh;
  if (tid == 0) {
    (isL ? p.Ls : p.Rs)[comp] = g.s;
    (isL ? p.Lz : p.Rz)[comp] = (uint8_t)g.z;
  }
  for (int i = tid; i < len; i += 256) {
    const float v = src[i * stride];
    const float x = __fadd_rn(__fmul_rn(v, g.r), g.z);
    const float q = fminf(fmaxf(rintf(x), 0.f), maxq);
    codes[i * stride] = (uint8_t)q;
    if (hat) hat[base + i * stride] = __fmul_rn(g.s, q - g.z);
  }
}

// ------------------------------------------------------ W4A16 product --
// Y = X What^T, X [M][K] bf16, What = s (q - z) per (row, group) from the
// packed 4-bit codes, on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// The matrix unit multiplies bf16 by bf16, so each weight enters as
// bf16(fl32(s (q - z))) (round to nearest even); the activations are exact.
//
// Tile: BM rows of X x BN rows of the codes per workgroup, one wave per
// 128 x 64 block of it (4 x 2 MFMA accumulators); K in steps of 32.  The
// large-M shape is 512 x 128 (8 waves): each dequantised code tile then
// feeds twice the MFMAs of a 256-row tile.
//   A: X rows go from L2 straight into LDS (global_load_lds, 16 B per lane)
//      three steps ahead, in a ring of four stages.  Each 64-byte LDS row
//      holds its four 16-byte k-chunks XOR-swizzled by (row / 4) % 4, so a
//      fragment read of 16 consecutive rows covers all 64 banks.
//   B: every thread loads WPT code words one step ahead into registers,
//      dequantises them with the group's s, z (reloaded only where a group
//      starts) and writes the bf16 values into a double-buffered LDS stage in
//      the same swizzled layout; the MFMA lanes then read A and B alike.
// One barrier per step.  The fragments of the first 16-k sub-step of a step
// are read right after the barrier, beside the previous step's last MFMAs;
// the second sub-step's are read beside the first sub-step's MFMAs, which
// also hide the dequantisation of the next step.  Code rows past N and X
// rows past M are read clamped (valid memory) and never stored.
#define W4_KS 32
#define W4_NA 4

// eight codes of one word -> eight bf16 of fl32(s (q - z)), codes in order
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s, float z) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2 v;
    v.x = __fmul_rn((float)((w >> (8 * j)) & 15u) - z, s);
    v.y = __fmul_rn((float)((w >> (8 * j + 4)) & 15u) - z, s);
    o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// The same for BITS-bit codes: code i of the eight at bits BITS i of v (the
// chunk's stretch of the row's bitstream, shifted down to bit 0).
template <int BITS>
__device__ __forceinline__ u32x4 dequant8b(uint64_t v, float s, float z) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2 t;
    t.x = __fmul_rn((float)((uint32_t)(v >> (BITS * (2 * j))) & mask) - z, s);
    t.y = __fmul_rn((float)((uint32_t)(v >> (BITS * (2 * j + 1))) & mask) - z, s);
    o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2));
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// Chunk cu (codes 8 cu .. 8 cu + 7) of a 32-code step of a BITS-bit row
// stream starts at bit 8 BITS cu of the step's BITS words: word (BITS cu) / 4,
// bit 8 ((BITS cu) % 4).  It reaches into the next word only when it does not
// fit in the rest of its own, and that word is then still one of the step's.
template <int BITS>
__device__ __forceinline__ uint64_t chunk_bits(const __attribute__((address_space(1))) uint32_t* step_words, int cu) {
  const int wi = (BITS * cu) >> 2, sh = 8 * ((BITS * cu) & 3);
  const bool two = sh + 8 * BITS > 32;
  const uint32_t lo = step_words[wi];
  const uint32_t hi = step_words[two ? wi + 1 : wi];
  return (((uint64_t)hi << 32) | lo) >> sh;
}

template <int BM, int BN, int BITS>
__global__ __launch_bounds__(BM * BN / 8192 * 64, 1) void k_gemm_w4a16(const W4Prob p) {
  constexpr int WN = BN / 64;               // waves across the codes (each 128 x 64)
  constexpr int NW = (BM / 128) * WN;       // waves
  constexpr int AST = BM * W4_KS * 2;       // bytes of an A stage
  constexpr int BST = BN * W4_KS * 2;       // bytes of a B stage
  constexpr int NQ = BM / 16 / NW;          // global_load_lds per lane per stage
  constexpr int WPT = BN * 4 / (64 * NW);   // code words per thread per step
  constexpr int TPR = 4 / WPT;              // threads per code row
  __shared__ __attribute__((aligned(1024))) uint8_t lds[W4_NA * AST + 2 * BST];
  uint8_t* const As = lds;
  uint8_t* const Bs = lds + W4_NA * AST;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets on the scalar unit
  // Consecutive workgroups go to the eight XCDs in turn; give XCD x a
  // contiguous run of tiles (row-panel major), so the workgroups resident on
  // one XCD share the X panel through its L2.
  const int nt = p.tiles_m * p.tiles_n;
  const int xcd = blockIdx.x & 7;
  const int T = xcd * (nt >> 3) + min(xcd, nt & 7) + (blockIdx.x >> 3);
  const int m0 = (T / p.tiles_n) * BM, n0 = (T % p.tiles_n) * BN;
  const int nsteps = p.K / W4_KS, last = nsteps - 1;

  // A copy: instruction q of wave w fills LDS rows 16 (NW q + w) .. +15 of a
  // stage; lane -> row 16 (NW q + w) + lane / 4 at chunk position lane % 4,
  // holding k-chunk (lane % 4) ^ (lane / 16).
  const uint16_t* ga[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int row = min(m0 + 16 * (NW * q + w) + (lane >> 2), p.M - 1);
    ga[q] = p.X + (size_t)row * p.ldx + 8 * ((lane & 3) ^ (lane >> 4));
  }
  auto issue_a = [&](int step, int stage) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(ga[q] + step * W4_KS),
                                       (lds_void*)(As + stage * AST + (NW * q + w) * 1024), 16, 0, 0);
  };
  // B: thread -> code row n0 + tid / TPR, words WPT (tid % TPR) .. +WPT-1 of
  // each step (k-chunks of the same numbers).  Groups are powers of two of
  // at least 8 codes (or the whole row), so one (s, z) serves a word.
  const int nl = tid / TPR, c0 = WPT * (tid % TPR);
  const int nrow = min(n0 + nl, p.N - 1);
  gu32* gb = (gu32*)(p.P + (size_t)nrow * (p.K >> 3) + c0);
  gu32* grow = (gu32*)(p.P + (size_t)nrow * ((p.K >> 5) * BITS));  // BITS != 4: the row's stream
  gfloat* gs = (gfloat*)(p.S + (size_t)nrow * p.G);
  gu8* gz = (gu8*)(p.Z + (size_t)nrow * p.G);
  const int bsw = (nl >> 2) & 3;
  uint32_t bw[WPT];  // BITS == 4: one word per chunk
  uint64_t bv[WPT];  // other BITS: the chunk's bits
  float bsc[WPT], bzp[WPT];
  // s, z are reloaded only where a group starts (every step for groups
  // shorter than a step); they stay in registers in between
  const unsigned gmask = (1u << p.gshift) - 1u;
  auto load_b = [&](int step) {
    const bool fresh = p.gshift < 5 || ((unsigned)(step * W4_KS) & gmask) == 0;  // uniform
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      if constexpr (BITS == 4)
        bw[u] = gb[4 * step + u];
      else
        bv[u] = chunk_bits<BITS>(grow + (size_t)BITS * step, c0 + u);
      if (fresh) {
        const int g = (step * W4_KS + 8 * (c0 + u)) >> p.gshift;
        bsc[u] = gs[g];
        bzp[u] = (float)gz[g];
      }
    }
  };
  auto store_b = [&](int stage) {
#pragma unroll
    for (int u = 0; u < WPT; ++u)
      *(u32x4*)(Bs + stage * BST + nl * 64 + (((c0 + u) ^ bsw) << 4)) =
          BITS == 4 ? dequant8(bw[u], bsc[u], bzp[u]) : dequant8b<BITS>(bv[u], bsc[u], bzp[u]);
  };

  // fragments: wave w owns rows 128 (w / WN) and columns 64 (w % WN) of the
  // tile; lane -> fragment row lane % 32, k-chunk 2 ks + lane / 32
  const int sw = (lane >> 2) & 3, hh = lane >> 5, r31 = lane & 31;
  const int wm0 = 128 * (w / WN), wn0 = 64 * (w % WN);
  auto rd = [&](int sa, int sb, int ks, bf16x8* fa, bf16x8* fb) {
    const int ch = ((2 * ks + hh) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8*)(As + sa * AST + (wm0 + 32 * i + r31) * 64 + ch);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *(const bf16x8*)(Bs + sb * BST + (wn0 + 32 * j + r31) * 64 + ch);
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  // Prologue: step 0 in LDS (A copied, B dequantised), steps 1 and 2 in
  // flight, the first sub-step's fragments read.  Past the last step the
  // copies repeat the last step into stages nobody reads again, so copies
  // keep flowing at the same rate to the end.
  load_b(0);
  __builtin_amdgcn_sched_barrier(0);
  issue_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  store_b(0);
  __builtin_amdgcn_sched_barrier(0);
  load_b(min(1, last));
  __builtin_amdgcn_sched_barrier(0);
  issue_a(min(1, last), 1);
  issue_a(min(2, last), 2);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(VmWait<2 * NQ>::value);  // A(0) (only A(1), A(2) may be in flight)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
  rd(0, 0, 0, fa0, fb0);
  // Step s: the second sub-step's fragments are read while the first
  // sub-step's MFMAs run beside the dequantisation of step s + 1; then the
  // code words of step s + 2 and the X copy of step s + 3 go out, the
  // barrier publishes step s + 1, and the next step's first fragments are
  // read while the second sub-step's MFMAs run.  Before the barrier every
  // wave has its own LDS reads back (lgkmcnt 0), so the stages it read may be
  // overwritten after it.
  for (int s = 0; s < nsteps; ++s) {
    const int sa = s % W4_NA, sb = s & 1;
    rd(sa, sb, 1, fa1, fb1);
    mma(fa0, fb0);
    store_b(sb ^ 1);  // at the last step: rewrites the stage of step s - 1, read by no one
    __builtin_amdgcn_sched_barrier(0);
    load_b(min(s + 2, last));
    __builtin_amdgcn_sched_barrier(0);
    issue_a(min(s + 3, last), (s + 3) % W4_NA);
    __builtin_amdgcn_sched_barrier(0);
    // A(s + 1) has landed: at least the NQ copies of each of A(s + 2),
    // A(s + 3) and the code-word load of step s + 2 were issued after it
    // (vmcnt counts loads in issue order)
    __builtin_amdgcn_s_waitcnt(VmWait<2 * NQ + 1>::value & ~(15 << 8));  // and lgkmcnt == 0
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (s < last) rd((s + 1) % W4_NA, sb ^ 1, 0, fa0, fb0);
    mma(fa1, fb1);
  }
  __builtin_amdgcn_s_waitcnt(VmWait<0>::value);  // no copy into LDS outlives the group

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn0 + 32 * j + r31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < p.M && col < p.N) p.Y[(size_t)row * p.ldy + col] = acc[i][j][r];
      }
    }
}

// ------------------------------------------------ W4A16 product, few rows --
// The same product for few rows of X (decode-sized batches), where the tiled
// kernel would run almost empty: the work is reading the codes.  One
// workgroup of 8 waves per 16 rows of the codes (16 columns of Y) and 16 rows
// of X (grid y; more rows of X re-read the codes from L2); the waves split K
// in eight.  Lane (j = lane % 16, c = lane / 16) dequantises code
// words of row n0 + j into its B operand and takes the same k of X[j] (row j
// clamped to M - 1) as its A operand, and v_mfma_f32_16x16x32_bf16
// accumulates the 16 x 16 block of Y.  The eight partial blocks are summed in
// LDS in a fixed order.  The arithmetic per entry is that of the tiled kernel
// (bf16 weights, exact products, fp32 sums); only the order of the sums
// differs.
#define W4V_NW 8
template <int BITS>
__global__ __launch_bounds__(64 * W4V_NW) void k_gemv_w4a16(const W4Prob p) {
  __shared__ f32x4 red[W4V_NW][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;  // code rows; rows of X
  const int j = lane & 15, c = lane >> 4;
  const int nrow = min(n0 + j, p.N - 1);
  const uint32_t* crow = p.P + (size_t)nrow * (BITS == 4 ? (p.K >> 3) : (p.K >> 5) * BITS);
  gfloat* gs = (gfloat*)(p.S + (size_t)nrow * p.G);
  gu8* gz = (gu8*)(p.Z + (size_t)nrow * p.G);
  const uint16_t* xrow = p.X + (size_t)min(m0 + j, p.M - 1) * p.ldx;
  const unsigned gmask = (1u << p.gshift) - 1u;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const u32x4& xa, const u32x4& bq) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa), __builtin_bit_cast(bf16x8, bq), acc,
                                                  0, 0, 0);
  };
  // Blocks of 128 k, split among the waves.  In block t the lane loads the
  // four code words of k = 128 t + 32 c .. +31 at once (16 bytes); its 16-k
  // sub-step u multiplies the 8 of them at 128 t + 32 c + 8 u with the same
  // k of X (the 32 k of one MFMA are then {128 t + 32 c' + 8 u + e}, every
  // k of the block once over u).  Groups of 128 codes or more hold one (s, z)
  // per block for every lane, reloaded only where a group starts (a uniform
  // test); smaller groups load theirs per sub-step.
  const int nblk = p.K >> 7;
  const int t0 = (int)((long long)nblk * w / W4V_NW), t1 = (int)((long long)nblk * (w + 1) / W4V_NW);
  const bool big = p.gshift >= 7;
  float sc = 0.f, zp = 0.f;
  for (int t = t0; t < t1; ++t) {
    const int kb = 128 * t + 32 * c;
    // the 32 codes of k = kb .. kb + 31: BITS words; chunk u = the 8 at kb + 8 u
    u32x4 wq = {0u, 0u, 0u, 0u};
    uint64_t cv[4] = {0, 0, 0, 0};
    if constexpr (BITS == 4) {
      wq = *(const gu32x4*)(crow + (kb >> 3));
    } else {
      gu32* sw = (gu32*)(crow + (size_t)BITS * (kb >> 5));
      uint32_t wv[BITS];
#pragma unroll
      for (int e = 0; e < BITS; ++e) wv[e] = sw[e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int wi = (BITS * u) >> 2, sh = 8 * ((BITS * u) & 3);
        const uint32_t hi = (sh + 8 * BITS > 32) ? wv[wi + 1 < BITS ? wi + 1 : wi] : wv[wi];
        cv[u] = (((uint64_t)hi << 32) | wv[wi]) >> sh;
      }
    }
    auto deq = [&](int u, float s_, float z_) {
      return BITS == 4 ? dequant8(wq[u], s_, z_) : dequant8b<BITS>(cv[u], s_, z_);
    };
    u32x4 xa[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) xa[u] = *(const u32x4*)(xrow + kb + 8 * u);
    if (big) {
      if (t == t0 || ((unsigned)(128 * t) & gmask) == 0) {  // uniform
        const int g = (128 * t) >> p.gshift;
        sc = gs[g];
        zp = (float)gz[g];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) mma(xa[u], deq(u, sc, zp));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = (kb + 8 * u) >> p.gshift;
        mma(xa[u], deq(u, gs[g], (float)gz[g]));
      }
    }
  }
  // K % 128: up to three 32-k steps left, one per wave, in the layout of a
  // 32-k MFMA step (lane k-chunk c)
  const int s_tail = 4 * nblk + w;
  if (s_tail < (p.K >> 5)) {  // uniform
    const int k = 32 * s_tail + 8 * c;
    const int g = k >> p.gshift;
    const u32x4 wt = BITS == 4 ? dequant8(((const gu32*)crow)[k >> 3], gs[g], (float)gz[g])
                               : dequant8b<BITS>(chunk_bits<BITS>((gu32*)crow + (size_t)BITS * s_tail, c), gs[g],
                                                 (float)gz[g]);
    mma(*(const u32x4*)(xrow + k), wt);
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 t = red[0][lane];
#pragma unroll
    for (int q = 1; q < W4V_NW; ++q) t += red[q][lane];
    // lane holds rows 4 (lane / 16) + r of the block, column lane % 16
    const int col = n0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 4 * (lane >> 4) + r;
      if (row < p.M && col < p.N) p.Y[(size_t)row * p.ldy + col] = t[r];
    }
  }
}

// ------------------------------------------------------------ launchers --
hipError_t launch_pack(const uint8_t* codes, int rows, int n, int bits, uint32_t* out, hipStream_t st) {
  const int words = (int)(((long long)n * bits + 31) / 32);
  const long long cnt = (long long)rows * words;
  if (cnt == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, codes, rows, n, bits, words,
                     out);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* packed, int rows, int n, int bits, uint8_t* codes, hipStream_t st) {
  const int words = (int)(((long long)n * bits + 31) / 32);
  const long long cnt = (long long)rows * n;
  if (cnt == 0) return hipSuccess;
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, packed, rows, n, bits,
                     words, codes);
  return hipGetLastError();
}

hipError_t launch_lr_quant(const LrProb& p, hipStream_t st) {
  hipLaunchKernelGGL(k_lr_quant, dim3(2 * p.r), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int BITS>
static void gemv_bits(const W4Prob& p, hipStream_t st) {
  hipLaunchKernelGGL(k_gemv_w4a16<BITS>, dim3(p.tiles_n, p.tiles_m), dim3(64 * W4V_NW), 0, st, p);
}

hipError_t launch_gemv_w4a16(W4Prob p, int bits, hipStream_t st) {
  p.tiles_m = (p.M + 15) / 16;
  p.tiles_n = (p.N + 15) / 16;
  switch (bits) {
    case 2: gemv_bits<2>(p, st); break;
    case 3: gemv_bits<3>(p, st); break;
    case 8: gemv_bits<8>(p, st); break;
    default: gemv_bits<4>(p, st); break;
  }
  return hipGetLastError();
}

template <int BITS>
static void gemm_bits(const W4Prob& p, int shape, hipStream_t st) {
  const dim3 grid(p.tiles_m * p.tiles_n);
  if (shape == 1)
    hipLaunchKernelGGL((k_gemm_w4a16<512, 128, BITS>), grid, dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemm_w4a16<256, 128, BITS>), grid, dim3(256), 0, st, p);
}

hipError_t launch_gemm_w4a16(W4Prob p, int shape, int bits, hipStream_t st) {
  const int bm = shape == 1 ? 512 : 256, bn = 128;
  p.tiles_m = (p.M + bm - 1) / bm;
  p.tiles_n = (p.N + bn - 1) / bn;
  switch (bits) {
    case 2: gemm_bits<2>(p, shape, st); break;
    case 3: gemm_bits<3>(p, shape, st); break;
    case 8: gemm_bits<8>(p, shape, st); break;
    default: gemm_bits<4>(p, shape, st); break;
  }
  return hipGetLastError();
}
