// Host-side planning types shared by the C ABI and the intrinsic-LoRA driver
// (internal to the library).
#pragma once
#include <functional>

#include "common.h"

// Per-call device slot of one factor/quantise job.
struct Slot {
  double lam;
  int info;
  int nonfinite;
  double obj[2];
};

struct QuantJob {
  const float* W;
  int out, n, nt;  // nt = n + appended (never rounded) columns
  const float* U;  // [nt][nt]
  int bits, group, block;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* err;
  const double* lam;  // device pointer to the damping of U
  double* obj;        // device [2]
  float* Ww_ext;      // optional caller-owned working buffer [out][nt]
  // 0: GPTQ sweep.  1: one Bid-Up pass: W holds g = (W - C - What) H, U holds
  // H, codes are read and rewritten on the given grid (scales, zeros), obj[0]
  // receives the summed objective change of the moves.
  int mode = 0;
};

struct LoraIO {
  const float* W;
  int out, n;
  const uint16_t* X;
  long long tokens, ldx;
  int r, bits, group, block;
  double lam_abs, lam_rel;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* L;
  float* R;
  int rounds = 0;  // refinement rounds (OLrC then Bid-Up) after the sweep
};

// One refinement step's operands: the layer, H in fp64 [n][n] (device), the
// current codes on their fixed grid, and L [n][r], R [r][out] (OLrC writes
// them; Bid-Up reads them).
struct RefineIO {
  const float* W;
  int out, n;
  const double* H64;
  int r, bits, group, block;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* L;
  float* R;
};

// Services the C ABI lends to the LoRA driver (workspace, the shared stages).
struct LoraHooks {
  std::function<int(const uint16_t*, long long, long long, int, double*)> hessian64;
  std::function<void*(size_t)> ensure;  // LoRA workspace of at least n bytes
  std::function<void*(size_t)> slots;   // device slots of at least n bytes
  std::function<int(double*, int, float*, Slot*)> factor;  // factor an assembled A
  std::function<int(const QuantJob&)> quantize;
  std::function<int(int, const char*)> set_err;
  // issue one launch (the function) on the context's stream under the given
  // kernel name (a string literal), timed when timing is on
  std::function<int(const char*, const std::function<hipError_t()>&)> launch;
  // C[M][N] = A[M][K] B[N][K]^T in fp64, all of pitch ld, on the factor's
  // fp64 MFMA ring (needs K % 16 == 0, even ld and 16-byte aligned bases)
  std::function<int(const double*, const double*, double*, int, int, int, int)> gemm_nt;
  // copy bytes from device to host after the context's stream has drained
  std::function<int(const void*, void*, size_t)> read;
  // note that a subspace iteration stopped at its cap (reported by the call)
  std::function<void()> not_converged;
};

// With io.rounds > 0 the slots hold, after the Slot, the objective trace
// (2 rounds + 2 doubles: after the sweep, then after every step).
int run_lora(hipStream_t st, const LoraIO& io, const LoraHooks& hooks);
// OLrC for the given codes: L, R and the objective into *J (device).
int run_olrc(hipStream_t st, const RefineIO& io, const LoraHooks& hooks, double* J);
// One Bid-Up pass for the given L, R: codes rewritten, objective into *J (device).
int run_bid_up(hipStream_t st, const RefineIO& io, const LoraHooks& hooks, double* J);
