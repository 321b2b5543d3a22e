// Host-side launchers of the kernels (internal to the library).
#pragma once
#include "common.h"

// Hessian
hipError_t launch_xpose(const XposeProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);
hipError_t launch_syrk(const SyrkProb* probs, const SyrkTask* tasks, int ntasks, float* partials,
                       hipStream_t st);
hipError_t launch_syrk_reduce(const RedProb* probs, const RedTask* tasks, int ntasks,
                              const int* partlist, const float* partials, hipStream_t st);
hipError_t launch_zero_f32(float* p, long long count, hipStream_t st);
hipError_t launch_syrk64(const SyrkProb* probs, const SyrkTask* tasks, int ntasks, double* partials,
                         hipStream_t st);
hipError_t launch_syrk64_reduce(const RedProb64* probs, const RedTask* tasks, int ntasks, const int* partlist,
                                const double* partials, hipStream_t st);

// Factor
hipError_t launch_damp_lambda(const FacProb* probs, int nprob, hipStream_t st);
hipError_t launch_damp_fill(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);
hipError_t launch_chol_panel(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);
hipError_t launch_chol_panel2(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);
hipError_t launch_chol_diag2(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);
hipError_t launch_gemm64(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);
// ts = 64 or 128; at most maxwg workgroups (0: one per tile), persistent over the ntot tiles
hipError_t launch_gemm_ring(int ts, const FacProb* probs, const Seg* segs, int nseg, int ntot, int maxwg,
                            hipStream_t st);
hipError_t launch_make_u(const FacProb* probs, const Seg* segs, int nseg, int nwg, hipStream_t st);

// Sweep
hipError_t launch_init_work(const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st);
hipError_t launch_rowfit(const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st);
// mode 0: the GPTQ sweep; mode 1: one Bid-Up pass (see the QLayer mode field)
hipError_t launch_sweep(int block, int mode, const QLayer* L, const Seg* segs, int nseg, int nwg, hipStream_t st);
// at most maxwg workgroups (0: one per tile), persistent over the nwg tiles
hipError_t launch_trail(int ts, const QLayer* L, const Seg* segs, int nseg, int nwg, int maxwg, hipStream_t st);
hipError_t launch_objective(const QLayer* L, int nl, hipStream_t st);

// two-sided rounding (round2d.hip)
hipError_t launch_r2d_unit(const float* U, int n, float* U1, float* d, hipStream_t st);
hipError_t launch_r2d_fill(float* a, float* b, long long cnt, hipStream_t st);
hipError_t launch_r2d_tile(const R2dProb& p, int S, int Ibeg, int ntiles, hipStream_t st);
// far = false: the pushes into the next row / column block; true: the rest
// (at most maxwg workgroups, 0: one per item; persistent over the items)
hipError_t launch_r2d_push(const R2dProb& p, int S, int Ibeg, int Iend, bool far, int maxwg, hipStream_t st);
hipError_t launch_r2d_obj(const double* objp, int nt, double* J, hipStream_t st);

// quantised-input target (qronos.hip)
hipError_t launch_qr_prep(const float* W, const float* G, const float* U, const double* lam, int out, int n,
                          double* Wd, double* Gd, double* Ud, double* UdT, hipStream_t st);
hipError_t launch_qr_out(const double* a, float* b, long long cnt, hipStream_t st);

// deployable outputs (deploy.hip)
hipError_t launch_pack(const uint8_t* codes, int rows, int n, int bits, uint32_t* out, hipStream_t st);
hipError_t launch_unpack(const uint32_t* packed, int rows, int n, int bits, uint8_t* codes, hipStream_t st);
hipError_t launch_lr_quant(const LrProb& p, hipStream_t st);
// sets the tile counts itself; K % 32 == 0; codes of 2, 3, 4 or 8 bits
// tile shape 0: 256 x 128 (4 waves), 1: 512 x 128 (8 waves)
hipError_t launch_gemm_w4a16(W4Prob p, int shape, int bits, hipStream_t st);
// few rows of X (up to 128): split-K product on 16 x 16 MFMA blocks
hipError_t launch_gemv_w4a16(W4Prob p, int bits, hipStream_t st);
