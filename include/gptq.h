/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library.
 *
 * The library computes, for one linear layer with weight W [out, n] (stored as
 * a Linear weight: rows = output neurons, columns = input dimensions) and a
 * calibration matrix X [tokens, n], integer codes Q, per-group scales and zero
 * points minimising the layer-wise reconstruction error ||X (W - What)^T||_F^2
 * (GPTQ-intrinsic LoRA technical summary, "problem statement"; Lattice Geometry
 * of NN Quantization, technical overview section 2, where the problem splits
 * into one closest-vector problem per output row).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every
 *     input and output buffer; the library never frees or keeps them.
 *   - Row-major throughout.  X holds bfloat16 values as their uint16 bit
 *     patterns.  Matrices of size [rows, cols] have leading dimension cols
 *     unless an ld argument is given.
 *   - A context owns its device workspace (grown on demand, kept until
 *     gptq_destroy) and the HIP stream it was created with.  Calls are
 *     asynchronous on that stream except those marked SYNC, which wait for the
 *     stream before returning.  The context also owns a second stream (default
 *     priority) on which the factor runs part of its trailing updates; every
 *     call joins it back into the context's stream by event before its last
 *     launch, so work later enqueued on the context's stream sees all results.
 *     A context is not thread-safe: one context per host thread/stream.
 *   - Every call returns a gptq_status.  Argument errors are detected on the
 *     host before anything is launched.  After GPTQ_ERR_HIP the HIP error text
 *     is available from gptq_last_error().
 *   - Results are deterministic: repeated calls on the same inputs give the
 *     same bytes (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad bits/group/block */
  GPTQ_ERR_NOT_PD = 2,      /* damped Hessian not positive definite (see info) */
  GPTQ_ERR_NONFINITE = 3,   /* non-finite entry in H */
  GPTQ_ERR_UNSUPPORTED = 4, /* valid but unsupported shape or alignment */
  GPTQ_ERR_HIP = 5,         /* HIP runtime error (text in gptq_last_error) */
  GPTQ_ERR_NO_MEMORY = 6,   /* workspace allocation failed */
  GPTQ_ERR_NOT_CONVERGED = 7 /* a subspace iteration stopped at its step cap; every
                                output is written, from its last iterate */
} gptq_status;

typedef struct gptq_ctx_s* gptq_ctx;

/* Create a context on HIP device `device`, issuing work on `stream` (a
 * hipStream_t; NULL = the device's null stream).  *ctx [host] receives the
 * handle.  Creates the context's second stream and two events; device
 * workspace is allocated by the first call that needs it. */
int gptq_create(gptq_ctx* ctx, int device, void* stream);

/* Wait for the context's streams, free its workspace and the context. */
int gptq_destroy(gptq_ctx ctx);

/* Static text for a status code. */
const char* gptq_strerror(int status);

/* Text of the last error recorded in ctx (empty string if none). */
const char* gptq_last_error(gptq_ctx ctx);

/* Calibration Hessian (GPTQ-2D technical summary section 1, Gram G = A^T A;
 * Lattice Geometry section 3.1, X^T X):
 *   H[n][n] (fp32, full symmetric) = (accumulate ? H : 0) + X^T X
 * X[tokens][ldx] bf16 bit patterns; only the first n columns are read.
 * The sum is unscaled.  bf16 products are exact in fp32; accumulation is fp32
 * in a fixed order (split over tokens, partials summed in a fixed order), and
 * H is exactly symmetric.  Requires ldx >= n; rows are read with 16-byte
 * loads when ldx % 8 == 0 and X is 16-byte aligned, element by element
 * otherwise.  tokens == 0 leaves H (accumulate) or zeroes it.
 * Asynchronous. */
int gptq_hessian(gptq_ctx ctx, const uint16_t* X, int64_t tokens, int32_t n, int64_t ldx,
                 float* H, int accumulate);

/* Damping and factor (Lattice Geometry section 3.1: X^T X + lam I; GPTQ-2D
 * sections 2 and 4: the feedback factors are the unit-triangular factors of
 * the inverse Gram matrix):
 *   lam = lam_abs + lam_rel * mean(diag H)
 *   U[n][n] fp32, upper triangular with positive diagonal, zero below it, with
 *   (H + lam I)^{-1} = U^T U.
 * Computed in fp64 by Cholesky of the index-reversed damped matrix and a
 * triangular inverse (U = P chol(P H_lam P)^{-1} P, P the reversal), so pivots
 * are eliminated from column n-1 down to 0.
 * SYNC.  *info [host] = 0 on success, else 1 + the column (in H's numbering)
 * of the first non-positive pivot met in that order, and GPTQ_ERR_NOT_PD is
 * returned (U is then undefined).  *lam_used [host] (may be NULL) = lam.
 * H is not modified.  Non-finite H -> GPTQ_ERR_NONFINITE. */
int gptq_factor(gptq_ctx ctx, const float* H, int32_t n, double lam_abs, double lam_rel,
                float* U, int32_t* info, double* lam_used);

/* Blocked column sweep (GPTQ encyclopedia entry, technical approach: quantise
 * a column, update the remaining weights in closed form, groups with their own
 * scale; GPTQ-2D sections 1-2: fixed order, triangular feedback, GPTQ's lazy
 * block update).  For every row, columns j = 0..n-1 in natural order:
 *   at a group start (or once per row when group == 0, on the original row)
 *     fit lo = min(min v, 0), hi = max(max v, 0), s = (hi-lo)/maxq (s = 1 if
 *     hi == lo), r = 1/s, z = rne(-lo*r) on the current weights v of the group;
 *   x = fl32(fl32(w_j*r) + z), q = clamp(rne(x), 0, maxq), what = s (q - z),
 *   E_j = (w_j - what)/U_jj, and w_k -= E_j U_jk for k > j
 * with the in-block part done per column and the rest, after each block of
 * `block` columns, as W[:, b1:] -= E[:, b0:b1] U[b0:b1, b1:].
 * Inputs: W[out][n] fp32 (not modified), U[n][n] from gptq_factor, lam (the
 * damping used for U, for the objective).  Outputs: codes[out][n] uint8 in
 * [0, 2^bits-1]; scales[out][ng] fp32 and zeros[out][ng] uint8 with
 * ng = group ? n/group : 1; err[out][n] fp32 the scaled errors E (may be NULL);
 * obj[2] [host] = {J, J_lam}: J_lam = sum E^2 = tr(D (H+lam I) D^T) and
 * J = J_lam - lam ||D||^2 = ||X D^T||^2 with D = W - What.
 * Requirements: 2 <= bits <= 8; group == 0 or (group % 8 == 0, n % group == 0,
 * and group % block == 0 or block % group == 0); block in {16,32,64,128}.
 * SYNC (objective read back). */
int gptq_quantize(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const float* U,
                  int32_t bits, int32_t group, int32_t block, double lam,
                  uint8_t* codes, float* scales, uint8_t* zeros, float* err, double* obj);

/* GPTQ-intrinsic LoRA (GPTQ-intrinsic LoRA technical summary, method section 2):
 * X~ = [X, X V_r] with V_r the top-r eigenvectors of H = X^T X; the sweep runs
 * on W~ = [W, 0] against the factor of X~^T X~ + lam I (lam = lam_abs +
 * lam_rel * mean(diag H)), rounding only the first n columns; the r appended
 * columns absorb the error.  Outputs codes/scales/zeros as gptq_quantize (W^T
 * ~ Q + L R in the pages' convention, i.e. W ~ What + R^T L^T):
 *   L[n][r] fp32: an orthonormal basis of the top-r eigenspace of H (found by
 *                 subspace iteration in fp64 on min(128, n, max(r + 32, 64))
 *                 columns with a Rayleigh-Ritz check every 4 steps, stopping
 *                 when ||H L - L diag(theta)||_F <= 1e-11 ||theta||; any basis
 *                 gives the same Q and the same product L R);
 *   R[r][out] fp32;
 *   obj[2] [host] = {J, J_lam}, J = ||X (W - What - R^T L^T)^T||^2.
 * X as gptq_hessian; 1 <= r <= min(128, n); requirements on bits/group/block as
 * gptq_quantize.  SYNC.  *info semantics as gptq_factor (may be NULL).
 * GPTQ_ERR_NOT_CONVERGED: the iteration reached its cap of 600 steps (the
 * r-th and (r+1)-th eigenvalues too close for it); every output is written,
 * from the last Ritz vectors. */
int gptq_lora(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const uint16_t* X,
              int64_t tokens, int64_t ldx, int32_t r, int32_t bits, int32_t group,
              int32_t block, double lam_abs, double lam_rel, uint8_t* codes, float* scales,
              uint8_t* zeros, float* L, float* R, double* obj, int32_t* info);

/* gptq_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, checks, kernels and results (codes, scales, zeros, err
 * and obj bit-identical to gptq_quantize on the same inputs), but every
 * intermediate lives in a fixed array of about 12.7 MB of device memory that
 * the library holds for the process's lifetime, one copy per device, and
 * the pinned host staging it uses is made when the context is created.  The
 * call performs no hipMalloc, hipFree, hipHostMalloc or event creation.
 * Limits: out <= 1024, n <= 4096, out * n <= 2^20; beyond them
 * GPTQ_ERR_UNSUPPORTED with a message.  All contexts on one device share its array, whose
 * contents persist from call to call (the parts that must start at zero are
 * cleared by the call's own kernels): calls that overlap on one device race
 * and give undefined results; serialise them.  Per-kernel timing is off for
 * this call.  SYNC (objective read back). */
int gptq_quantize_noalloc(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const float* U,
                          int32_t bits, int32_t group, int32_t block, double lam,
                          uint8_t* codes, float* scales, uint8_t* zeros, float* err, double* obj);

/* Gram matrix accurate to float64 rounding, H = X^T X in fp64 (the products
 * of bf16 values are exact in fp64 and the sums run in fp64 on fp64 MFMA).  X
 * as gptq_hessian; H[n][n] fp64, device, caller-owned, fully written.  The
 * Hessian the refinement steps below take.  ASYNC on the context's stream. */
int gptq_hessian64(gptq_ctx ctx, const uint16_t* X, int64_t tokens, int32_t n, int64_t ldx, double* H);

/* Refinement after the intrinsic LoRA (GPTQ-intrinsic LoRA technical summary,
 * section 4, Bid-Up refinement: OLrC fits L, R for a fixed Q, Bid-Up moves Q
 * on its fixed grid for fixed L, R, the two alternate and the layer objective
 * never increases).  Objective: J = tr(D H D^T), D = W - What - R^T L^T,
 * What = s (q - z) per group (fp32 as stored), H from gptq_hessian64.
 *
 * gptq_olrc: for the given codes, the rank-r correction C minimising J is
 * C = P P^T E with E = W - What and P the top-r eigenvectors of E H E^T
 * (found by the checked subspace iteration gptq_lora uses for L, in
 * dimension out; GPTQ_ERR_NOT_CONVERGED, with every output written, when it
 * reaches its cap).  Writes L[n][r] = E^T P and R[r][out] = P^T (fp32, device) and
 * J (host, the objective with that correction).  codes/scales/zeros as
 * gptq_quantize's outputs (read only); bits is checked only.
 *
 * gptq_bid_up: one pass over the columns j = 0..n-1 of every row: with
 * g = D H (gradient of the row objective up to the factor -2), the code
 * moves to q* = clamp(rne(x)), x = fl32(fl32(t / s) + z) (t / s as
 * t * fl32(1/s)), t = fl32(what_j + g_j / H_jj), only when that is strictly
 * nearer, |x - q*| < |x - q_j|; the move updates g for the later columns.
 * codes [out][n] are read and rewritten in place (device); L, R as written by
 * gptq_olrc; J (host) = the objective after the pass (its value before plus
 * the summed change of the moves).  The moves run on fp32 with the sweep's
 * lazy block updates (block as gptq_quantize).
 *
 * Both: W[out][n] fp32 and H[n][n] fp64 device; 1 <= r <= min(128, out, n);
 * requirements on bits/group/block as gptq_quantize.  SYNC. */
int gptq_olrc(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const double* H, int32_t r,
              int32_t bits, int32_t group, const uint8_t* codes, const float* scales,
              const uint8_t* zeros, float* L, float* R, double* J);
int gptq_bid_up(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const double* H, int32_t r,
                const float* L, const float* R, int32_t bits, int32_t group, int32_t block,
                uint8_t* codes, const float* scales, const uint8_t* zeros, double* J);

/* gptq_lora followed by `rounds` >= 1 rounds of gptq_olrc then gptq_bid_up,
 * and a last gptq_olrc, all on the fp64 Hessian the LoRA computes (shared,
 * not recomputed).  Outputs codes/scales/zeros (the grid stays the sweep's),
 * L, R from the last OLrC, and trace[2 rounds + 2] (host): J after the
 * sweep, then after every step (non-increasing up to rounding).  Arguments
 * otherwise as gptq_lora (also r <= out).  SYNC. */
int gptq_lora_refine(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const uint16_t* X,
                     int64_t tokens, int64_t ldx, int32_t r, int32_t bits, int32_t group,
                     int32_t block, double lam_abs, double lam_rel, int32_t rounds, uint8_t* codes,
                     float* scales, uint8_t* zeros, float* L, float* R, double* trace, int32_t* info);

/* Cross Gram G = X^T Y (sum over tokens of x_t^T y_t), fp32 [n][n] written in
 * full (not symmetric), on the same bf16 MFMA tiles as gptq_hessian.  X and
 * Y are [tokens][ldx] bf16 bits with the same tokens and pitch; rows 16-byte
 * aligned and n % 8 == 0 (else GPTQ_ERR_UNSUPPORTED).  tokens == 0 writes
 * zeros.  ASYNC on the context's stream. */
int gptq_cross_gram(gptq_ctx ctx, const uint16_t* X, const uint16_t* Y, int64_t tokens, int32_t n,
                    int64_t ldx, float* G);

/* GPTQ with the quantised-input target (Lattice Geometry of NN Quantization,
 * section 5.1: when the layer's inputs come from already-quantised layers,
 * Xq instead of X, only the target of the nearest-plane problem changes).
 * Every row minimises ||Xq q - X w||^2 + lam ||q - w||^2 (damping as a ridge
 * towards w), which is the GPTQ sweep of gptq_quantize on the target
 *   W* = W (G + lam I)^T Hq_lam^{-1},  G = Xq^T X,  Hq_lam = Xq^T Xq + lam I,
 * lam = lam_abs + lam_rel * mean(diag(Xq^T Xq)), with the factor of Hq_lam.
 * With Xq = X the target is W.  The Grams run as gptq_hessian (fp32, bf16
 * MFMA; G over all tiles), the three products forming W* in fp64.
 * Inputs: W[out][n] fp32; X, Xq [tokens][ldx] bf16 bits (device), the same
 * tokens and pitch, rows 16-byte aligned, n % 16 == 0.  Outputs as
 * gptq_quantize (codes, scales, zeros; the grid is fitted on W*'s
 * error-updated values), Wt[out][n] fp32 the target W* (may be NULL), obj[2]
 * [host] = {J, J_lam} of the sweep relative to W* and Hq (J = tr((W* - What)
 * Hq (W* - What)^T); ||Xq What^T - X W^T||^2 differs from it by a constant of
 * W).  *info as gptq_factor.  Requirements on bits/group/block as
 * gptq_quantize.  SYNC. */
int gptq_quantize_qronos(gptq_ctx ctx, const float* W, int32_t out, int32_t n, const uint16_t* X,
                         const uint16_t* Xq, int64_t tokens, int64_t ldx, int32_t bits, int32_t group,
                         int32_t block, double lam_abs, double lam_rel, uint8_t* codes, float* scales,
                         uint8_t* zeros, float* Wt, double* obj, int32_t* info);

/* Two-sided adaptive rounding, GPTQ-2D (GPTQ-2D technical summary): integers
 * Z minimising ||A (Z - X) B||_F^2 greedily, with exactly the trajectory of
 * the one-sided sweep over vec(X) (column-major) under the Gram H kron G,
 * G = A^T A, H = B B^T (section 1; Theorem 2: same result in any order that
 * respects the dependencies, here anti-diagonals).  Rounding entry (i, j)
 * with delta = w_ij - z_ij, z_ij = clamp(rne(fl32(w_ij)), qmin, qmax), feeds
 * -Lg[k][i] delta Uh[j][l] to the entries k >= i, l >= j, with the unit
 * factors Lg[k][i] = UG[i][k] / UG[i][i], Uh[j][l] = UH[j][l] / UH[j][j]
 * (section 2: Kronecker feedback, rank-1 updates, the lazy buffer C = L E).
 * Inputs (device, fp32, row-major): X[m][n] the real target; UG[m][m] and
 * UH[n][n] upper with G^{-1} = UG^T UG, H^{-1} = UH^T UH (gptq_factor of G
 * and of H, with or without damping).  Outputs: Z[m][n] int32 in [qmin,
 * qmax]; delta[m][n] fp32 the rounding residuals w - z (may be NULL);
 * J [host] = sum of (delta_ij / (UG_ii UH_jj))^2 = ||A (Z - X) B||_F^2 for
 * the G, H the factors belong to.  The rounding decisions are taken in fp32
 * and the feedback accumulates in fp32.  SYNC. */
int gptq_round_2d(gptq_ctx ctx, const float* X, int32_t m, int32_t n, const float* UG, const float* UH,
                  int32_t qmin, int32_t qmax, int32_t* Z, float* delta, double* J);

/* One layer of a batch.  X may be NULL: then H must already hold the layer's
 * Hessian (several layers may point at the same H and X == NULL to share it).
 * H and U are caller-provided [n][n] fp32 buffers (H is written when X != NULL).
 * obj and info are outputs written by the call. */
typedef struct {
  const uint16_t* X;
  int64_t tokens;
  int64_t ldx;
  const float* W;
  int32_t out, n;
  int32_t bits, group, block;
  int32_t pad0;
  double lam_abs, lam_rel;
  float* H;
  float* U;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* err;      /* may be NULL */
  double obj[2];   /* out: {J, J_lam} */
  int32_t info;    /* out: as gptq_factor */
  int32_t pad1;
} gptq_layer;

/* Quantise many independent layers at once (Hessians, factors, sweeps and
 * trailing updates each run as one grouped launch over all layers per step).
 * layers [host] array of nlayers descriptors; results equal those of calling
 * gptq_hessian, gptq_factor and gptq_quantize per layer.  SYNC.  Returns the
 * first error met; per-layer info/obj are filled in for every layer. */
int gptq_quantize_batched(gptq_ctx ctx, int32_t nlayers, gptq_layer* layers);

/* Deployable outputs (GPTQ encyclopedia entry, technical approach: the
 * quantised weights are used through GPU matrix kernels at inference;
 * performance and accuracy: 4-bit weights take a quarter of the fp32 memory;
 * GPTQ-intrinsic LoRA technical summary, results: L and R themselves at low
 * precision, 4 and 8 bits).  The pages fix no storage format; ours follows.
 * All ASYNC on the context's stream; device buffers, caller-owned.
 *
 * gptq_pack_codes: codes[rows][n] uint8 -> packed[rows][words], words =
 * ceil(n bits / 32) uint32: each row is a little-endian bitstream, code k at
 * stream bits [k bits, (k + 1) bits), stream bit b in word b / 32 at position
 * b % 32, zero bits up to the end of the last word (at 4 bits: code k is the
 * nibble 4 (k % 8) of word k / 8; at 8 bits: byte k).  Code bits above `bits`
 * are ignored.  1 <= bits <= 8.  gptq_unpack_codes is the inverse (codes
 * written in [0, 2^bits - 1]). */
int gptq_pack_codes(gptq_ctx ctx, const uint8_t* codes, int32_t rows, int32_t n, int32_t bits,
                    uint32_t* packed);
int gptq_unpack_codes(gptq_ctx ctx, const uint32_t* packed, int32_t rows, int32_t n, int32_t bits,
                      uint8_t* codes);

/* Round-to-nearest of the low-rank factors of gptq_lora / gptq_olrc (L[n][r],
 * R[r][out] fp32), L at bits_L and R at bits_R (each 2..8): every rank
 * component, a column of L and a row of R, gets its own grid fitted as in
 * gptq_quantize (lo = min(min v, 0), hi = max(max v, 0), s = (hi - lo)/maxq,
 * z = rne(-lo/s) in [0, maxq], maxq = 2^bits - 1 of its factor),
 * then q = clamp(rne(fl32(fl32(v * fl32(1/s)) + z))), vhat = fl32(s (q - z)).
 * Outputs: Lcodes[n][r], Lscales[r], Lzeros[r], Rcodes[r][out], Rscales[r],
 * Rzeros[r]; Lhat[n][r] and Rhat[r][out] the dequantised factors (each may
 * be NULL).  r == 0 writes nothing. */
int gptq_quantize_lowrank(gptq_ctx ctx, const float* L, const float* R, int32_t n, int32_t r, int32_t out,
                          int32_t bits_L, int32_t bits_R, uint8_t* Lcodes, float* Lscales, uint8_t* Lzeros,
                          float* Lhat, uint8_t* Rcodes, float* Rscales, uint8_t* Rzeros, float* Rhat);

/* W4A16 product Y = X What^T of a 4-bit layer: X[M][ldx] bf16 bits (16-byte
 * aligned rows), packed[N][K/8] from gptq_pack_codes at 4 bits, scales[N][G]
 * fp32 and zeros[N][G] uint8 as gptq_quantize writes them (G = K/group, or 1
 * for group 0), What = s (q - z) per group.  Every weight enters the bf16
 * matrix unit as bf16(fl32(s (q - z))) (nearest, ties to even); products are
 * exact and summed in fp32 (for M <= 128 a split-K kernel sums in another
 * order).  Y[M][ldy] fp32, fully written in its M x N part.
 * K == 0 writes zeros.  Requirements: K % 32 == 0; group 0, K, or a power of
 * two >= 8 dividing K; ldx % 8 == 0, X and packed 16-byte aligned (else
 * GPTQ_ERR_UNSUPPORTED). */
int gptq_gemm_w4a16(gptq_ctx ctx, const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* packed,
                    const float* scales, const uint8_t* zeros, int32_t N, int32_t K, int32_t group, float* Y,
                    int64_t ldy);

/* The same product for the other widths the layers are quantised at (GPTQ
 * encyclopedia entry, technical approach and performance and accuracy: 2 to
 * 4 bits; GPTQ-intrinsic LoRA technical summary, results: 3-bit layers, L
 * and R at 4 and 8 bits): bits in {2, 3, 4, 8}, packed[N][K bits/32] from
 * gptq_pack_codes at that width (each row one bitstream, so 32 codes fill
 * `bits` whole words).  Everything else, rounding and requirements included,
 * as gptq_gemm_w4a16, which is this call with bits = 4.  Other widths:
 * GPTQ_ERR_UNSUPPORTED. */
int gptq_gemm_wqa16(gptq_ctx ctx, const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* packed,
                    const float* scales, const uint8_t* zeros, int32_t N, int32_t K, int32_t group, int32_t bits,
                    float* Y, int64_t ldy);

/* Measurement support (not part of the method).  gptq_timing(ctx, kernels)
 * clears the totals and from then on brackets each launch of the named
 * kernels with a pair of HIP events on the context's stream.  kernels [host]
 * is a comma-separated list of kernel names (e.g. "k_syrk,k_sweep"), "*" for
 * every kernel the context launches, or NULL to stop recording (totals are
 * kept until the next gptq_timing call).  Kernel names: k_xpose, k_syrk,
 * k_syrk_reduce, k_syrk64, k_syrk64_reduce, k_damp_lambda, k_damp_fill,
 * k_chol_panel, k_chol_panel2, k_gemm64, k_gemm_ring64, k_gemm_ring128,
 * k_make_u, k_init_work, k_rowfit, k_sweep, k_trail, k_objective, and for the
 * LoRA and refinement paths k_lora_lambda, k_start_block, k_dgemm, k_dsum,
 * k_gram_chol, k_apply, k_lora_assemble, k_lora_extract, k_ref_init, k_resid,
 * k_gfinal, k_sum_parts, k_f32_to_f64, k_f64_to_f32, k_olrc_out, and for the
 * two-sided rounding k_r2d_unit, k_r2d_fill, k_r2d_tile, k_r2d_push, k_r2d_obj,
 * and for the quantised-input target k_qr_prep, k_qr_out, and for the
 * deployable outputs k_pack, k_unpack, k_lr_quant, k_gemm_w4a16,
 * k_gemv_w4a16 (4-bit codes), k_gemm_wqa16, k_gemv_wqa16 (other widths).
 * gptq_kernel_time
 * waits for the recorded events and returns the summed elapsed milliseconds
 * and the number of timed launches of kernel `name` (0 and 0 if none).  Each
 * timed launch costs two event records on the stream. */
int gptq_timing(gptq_ctx ctx, const char* kernels);
int gptq_kernel_time(gptq_ctx ctx, const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
