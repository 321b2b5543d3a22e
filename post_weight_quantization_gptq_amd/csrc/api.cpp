// C ABI of the GPTQ library: argument checks, the launch planner and the
// context's workspace.  The planner turns the shapes of a call into per-launch
// task tables (packed in one buffer, uploaded with one copy per call) and then
// issues every kernel on the context's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <mutex>
#include <vector>

#include "../../include/gptq.h"
#include "common.h"
#include "launch.h"
#include "plan.h"
#include "planner.h"

#define GPTQ_API extern "C" __attribute__((visibility("default")))

namespace {

struct DevBuf {
  void* p = nullptr;
  size_t cap = 0;
};

}  // namespace

struct gptq_ctx_s {
  int device = 0;
  hipStream_t stream = nullptr;
  int ncu = 256;
  int nxcd = 8;
  std::string err;
  DevBuf partials, xt, facA, facY, work, eblk, objp, dinv, slots, blob, lora, r2d, qr;
  void* hblob = nullptr;  // pinned staging for the task tables
  size_t hblob_cap = 0;
  void* hsmall = nullptr;  // pinned read-back area
  size_t hsmall_cap = 0;
  hipEvent_t blob_ev = nullptr;
  bool blob_pending = false;
  // this device's copy of the no-allocation scratch array (device address)
  uint8_t* na_base = nullptr;
  // set when a subspace iteration of the current call stopped at its cap
  bool not_converged = false;
  // second stream (default priority) for the factor's trailing updates that
  // run beside its serial chain; fork / join events order it against stream
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  // per-kernel timing (off unless gptq_timing enabled it)
  struct Timed {
    const char* name;
    hipEvent_t a, b;
  };
  bool timing = false;
  std::string tfilter;  // "*" or ",name,name,"
  std::vector<Timed> tpend;
  std::vector<hipEvent_t> tpool;
  std::vector<std::string> tname;
  std::vector<double> tms;
  std::vector<long long> tcount;
};

namespace {

int set_err(gptq_ctx c, int status, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return status;
}

#define HIPCHK(c, expr)                                                                       \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return set_err((c), GPTQ_ERR_HIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                     __LINE__);                                                               \
  } while (0)

hipError_t timer_event(gptq_ctx c, hipEvent_t* e) {
  if (!c->tpool.empty()) {
    *e = c->tpool.back();
    c->tpool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Fold the finished event pairs into the per-name totals.
int timer_collect(gptq_ctx c) {
  for (const auto& t : c->tpend) {
    HIPCHK(c, hipEventSynchronize(t.b));
    float ms = 0.f;
    HIPCHK(c, hipEventElapsedTime(&ms, t.a, t.b));
    size_t k = 0;
    while (k < c->tname.size() && c->tname[k] != t.name) ++k;
    if (k == c->tname.size()) {
      c->tname.push_back(t.name);
      c->tms.push_back(0.0);
      c->tcount.push_back(0);
    }
    c->tms[k] += ms;
    c->tcount[k] += 1;
    c->tpool.push_back(t.a);
    c->tpool.push_back(t.b);
  }
  c->tpend.clear();
  return GPTQ_OK;
}

bool timer_wants(gptq_ctx c, const char* name) {
  if (!c->timing) return false;
  if (c->tfilter == "*") return true;
  return c->tfilter.find(std::string(",") + name + ",") != std::string::npos;
}

// Issue one kernel launch on stream st; with timing on, bracket it by an
// event pair on that stream.
#define LAUNCH_ON(c, st, name, expr)                           \
  do {                                                         \
    hipEvent_t ea_ = nullptr, eb_ = nullptr;                   \
    const bool timed_ = timer_wants(c, name);                  \
    if (timed_) {                                              \
      HIPCHK(c, timer_event(c, &ea_));                         \
      HIPCHK(c, timer_event(c, &eb_));                         \
      HIPCHK(c, hipEventRecord(ea_, st));                      \
    }                                                          \
    HIPCHK(c, expr);                                           \
    if (timed_) {                                              \
      HIPCHK(c, hipEventRecord(eb_, st));                      \
      (c)->tpend.push_back(gptq_ctx_s::Timed{name, ea_, eb_}); \
    }                                                          \
  } while (0)
#define LAUNCH(c, name, expr) LAUNCH_ON(c, (c)->stream, name, expr)

int ensure(gptq_ctx c, DevBuf& b, size_t bytes) {
  if (bytes == 0) bytes = 256;
  if (b.cap >= bytes) return GPTQ_OK;
  if (b.p) {
    HIPCHK(c, hipStreamSynchronize(c->stream));
    HIPCHK(c, hipFree(b.p));
    b.p = nullptr;
    b.cap = 0;
  }
  const size_t want = (bytes + (2u << 20) - 1) & ~((size_t)(2u << 20) - 1);
  if (hipMalloc(&b.p, want) != hipSuccess) {
    (void)hipGetLastError();
    return set_err(c, GPTQ_ERR_NO_MEMORY, "device allocation of %zu bytes failed", want);
  }
  b.cap = want;
  return GPTQ_OK;
}

int ensure_pinned(gptq_ctx c, void*& p, size_t& cap, size_t bytes) {
  if (cap >= bytes) return GPTQ_OK;
  if (p) {
    HIPCHK(c, hipStreamSynchronize(c->stream));
    HIPCHK(c, hipHostFree(p));
    p = nullptr;
    cap = 0;
  }
  const size_t want = std::max<size_t>(bytes, 1 << 16);
  if (hipHostMalloc(&p, want, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    return set_err(c, GPTQ_ERR_NO_MEMORY, "pinned allocation of %zu bytes failed", want);
  }
  cap = want;
  return GPTQ_OK;
}

// Packed task tables of one call.
struct Blob {
  std::vector<uint8_t> h;
  template <class T>
  size_t add(const T* p, size_t n) {
    size_t off = (h.size() + 63) & ~(size_t)63;
    h.resize(off + sizeof(T) * std::max<size_t>(n, 1));
    if (n) memcpy(h.data() + off, p, sizeof(T) * n);
    return off;
  }
  template <class T>
  size_t add(const std::vector<T>& v) {
    return add(v.data(), v.size());
  }
};

// Upload a blob; returns the device base pointer in *dbase.
int upload(gptq_ctx c, const Blob& b, uint8_t** dbase) {
  const size_t bytes = b.h.size();
  int rc = ensure(c, c->blob, bytes);
  if (rc) return rc;
  if (c->blob_pending) {
    HIPCHK(c, hipEventSynchronize(c->blob_ev));
    c->blob_pending = false;
  }
  rc = ensure_pinned(c, c->hblob, c->hblob_cap, bytes);
  if (rc) return rc;
  memcpy(c->hblob, b.h.data(), bytes);
  HIPCHK(c, hipMemcpyAsync(c->blob.p, c->hblob, bytes, hipMemcpyHostToDevice, c->stream));
  HIPCHK(c, hipEventRecord(c->blob_ev, c->stream));
  c->blob_pending = true;
  *dbase = (uint8_t*)c->blob.p;
  return GPTQ_OK;
}

// ------------------------------------------- no-allocation scratch ------
// gptq_quantize_noalloc works entirely inside this array (one copy per
// device, held until the process ends): the device slot, the task tables, the
// working weights, the errors of two super-blocks, the per-row sums and the
// error scales.  Limits: out <= NA_MAX_OUT, n <= NA_MAX_N, out * n <= NA_MAX_ELEMS.
constexpr int NA_MAX_OUT = 1024;
constexpr int NA_MAX_N = 4096;
constexpr long long NA_MAX_ELEMS = 1LL << 20;
constexpr size_t NA_SLOT = 256;
constexpr size_t NA_BLOB = 64 << 10;
constexpr size_t NA_WW = (size_t)NA_MAX_ELEMS * sizeof(float);
constexpr size_t NA_EB = (size_t)2 * NA_MAX_OUT * 1024 * sizeof(float);  // two 1024-column super-blocks
constexpr size_t NA_OBJP = (size_t)NA_MAX_OUT * 2 * sizeof(double);
constexpr size_t NA_DINV = (size_t)(NA_MAX_N + 64) * sizeof(float);
constexpr size_t NA_BYTES = NA_SLOT + NA_BLOB + NA_WW + NA_EB + NA_OBJP + NA_DINV;

// Pointers into the scratch array of one device.
struct NoAlloc {
  Slot* slot;
  uint8_t* blob;
  float* ww;
  float* eb;
  double* objp;
  float* dinv;
};
NoAlloc noalloc_view(uint8_t* base) {
  NoAlloc v;
  v.slot = (Slot*)base;
  v.blob = base + NA_SLOT;
  v.ww = (float*)(v.blob + NA_BLOB);
  v.eb = (float*)((uint8_t*)v.ww + NA_WW);
  v.objp = (double*)((uint8_t*)v.eb + NA_EB);
  v.dinv = (float*)((uint8_t*)v.objp + NA_OBJP);
  return v;
}

// Upload a blob into the scratch array through the context's pinned staging
// (allocated when the context was created); never allocates.
int upload_noalloc(gptq_ctx c, const Blob& b, uint8_t* dst, uint8_t** dbase) {
  const size_t bytes = b.h.size();
  if (bytes > NA_BLOB || bytes > c->hblob_cap)
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "task tables of %zu bytes exceed the no-allocation limit", bytes);
  if (c->blob_pending) {
    HIPCHK(c, hipEventSynchronize(c->blob_ev));
    c->blob_pending = false;
  }
  memcpy(c->hblob, b.h.data(), bytes);
  HIPCHK(c, hipMemcpyAsync(dst, c->hblob, bytes, hipMemcpyHostToDevice, c->stream));
  HIPCHK(c, hipEventRecord(c->blob_ev, c->stream));
  c->blob_pending = true;
  *dbase = dst;
  return GPTQ_OK;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int d) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != d) (void)hipSetDevice(d);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};


// ------------------------------------------------------------ Hessian plan --
int run_hessian(gptq_ctx c, const std::vector<HessJob>& jobs) {
  const size_t xt_elems = hess_xt_elems(jobs);
  int rc = ensure(c, c->xt, xt_elems * sizeof(uint16_t));
  if (rc) return rc;
  HessPlan P;
  plan_hessian(jobs, c->ncu, c->nxcd, (uint16_t*)c->xt.p, P);
  if ((rc = ensure(c, c->partials, (size_t)std::max(P.nparts, 1) * 65536 * sizeof(float)))) return rc;
  int nxwg = 0;
  for (const auto& sg : P.xsegs) nxwg += sg.nwg;
  Blob b;
  const size_t o_xprobs = b.add(P.xprobs), o_xsegs = b.add(P.xsegs);
  const size_t o_probs = b.add(P.probs), o_tasks = b.add(P.tasks), o_rprobs = b.add(P.rprobs),
               o_rtasks = b.add(P.rtasks), o_plist = b.add(P.partlist);
  uint8_t* d = nullptr;
  rc = upload(c, b, &d);
  if (rc) return rc;
  if (nxwg > 0)  // no transposed copy when every X is read in place
    LAUNCH(c, "k_xpose", launch_xpose((const XposeProb*)(d + o_xprobs), (const Seg*)(d + o_xsegs), (int)P.xsegs.size(),
                                      nxwg, c->stream));
  LAUNCH(c, "k_syrk", launch_syrk((const SyrkProb*)(d + o_probs), (const SyrkTask*)(d + o_tasks),
                        (int)P.tasks.size(), (float*)c->partials.p, c->stream));
  LAUNCH(c, "k_syrk_reduce", launch_syrk_reduce((const RedProb*)(d + o_rprobs), (const RedTask*)(d + o_rtasks),
                               (int)P.rtasks.size(), (const int*)(d + o_plist),
                               (const float*)c->partials.p, c->stream));
  return GPTQ_OK;
}

// One layer's Gram matrix accurate to float64 rounding ([n][n] doubles, full
// symmetric): the same transposed copy of X, 128x128 upper tiles on float64
// MFMA, each tile split over S token slices (S chosen so that the tasks fill
// whole rounds of the chip), partials summed in slice order.
int run_hessian64(gptq_ctx c, const uint16_t* X, long long tokens, long long ldx, int n, double* H) {
  if (n <= 0) return GPTQ_OK;
  const int n_pad = cdiv(n, 256) * 256;
  const long long t_pad = cdiv(tokens, 64) * 64;
  int rc = ensure(c, c->xt, (size_t)n_pad * (size_t)std::max(t_pad, 64LL) * sizeof(uint16_t));
  if (rc) return rc;
  uint16_t* xt = (uint16_t*)c->xt.p;
  const int vec = (ldx % 8 == 0) && (((uintptr_t)X & 15) == 0);
  std::vector<XposeProb> xprobs{XposeProb{X, ldx, xt, n, (int)tokens, n_pad, (int)t_pad, vec, (int)t_pad}};
  std::vector<Seg> xsegs;
  if (t_pad > 0) xsegs.push_back(Seg{0, 0, (int)(t_pad / 64) * (n_pad / 64), 0, 0, 0, 0, 0});
  const int nwx = xsegs.empty() ? 0 : xsegs[0].nwg;
  std::vector<SyrkProb> probs{SyrkProb{xt, t_pad, 0, (int)tokens, n, 0}};
  std::vector<RedProb64> rprobs{RedProb64{H, n, 0}};
  Hess64Plan P;
  plan_hessian64(n, tokens, c->ncu, P);
  const std::vector<SyrkTask>& tasks = P.tasks;
  const std::vector<RedTask>& rtasks = P.rtasks;
  const std::vector<int>& partlist = P.partlist;
  if ((rc = ensure(c, c->partials, std::max<size_t>(tasks.size(), 1) * 16384 * sizeof(double)))) return rc;
  Blob b;
  const size_t o_xprobs = b.add(xprobs), o_xsegs = b.add(xsegs), o_probs = b.add(probs), o_tasks = b.add(tasks),
               o_rprobs = b.add(rprobs), o_rtasks = b.add(rtasks), o_plist = b.add(partlist);
  uint8_t* d = nullptr;
  if ((rc = upload(c, b, &d))) return rc;
  LAUNCH(c, "k_xpose", launch_xpose((const XposeProb*)(d + o_xprobs), (const Seg*)(d + o_xsegs), (int)xsegs.size(),
                                    nwx, c->stream));
  LAUNCH(c, "k_syrk64", launch_syrk64((const SyrkProb*)(d + o_probs), (const SyrkTask*)(d + o_tasks),
                                      (int)tasks.size(), (double*)c->partials.p, c->stream));
  LAUNCH(c, "k_syrk64_reduce", launch_syrk64_reduce((const RedProb64*)(d + o_rprobs), (const RedTask*)(d + o_rtasks),
                                                    (int)rtasks.size(), (const int*)(d + o_plist),
                                                    (const double*)c->partials.p, c->stream));
  return GPTQ_OK;
}

// ------------------------------------------------------------- factor plan --
struct FacJob {
  const float* H;  // null: A (and lam) prepared by an earlier kernel
  int n, ldh, ldu;
  double lam_abs, lam_rel;
  float* U;
};

// Enqueue the factor of every job.  A/Y offsets (in doubles) into facA/facY.
int run_factor(gptq_ctx c, const std::vector<FacJob>& jobs, Slot* dslots, bool assembled_A = false,
               double** A_out = nullptr) {
  const int np = (int)jobs.size();
  std::vector<size_t> oA(np);
  size_t totA = 0;
  for (int p = 0; p < np; ++p) {
    oA[p] = totA;
    totA += (size_t)jobs[p].n * jobs[p].n;
  }
  int rc;
  if (!assembled_A) {
    rc = ensure(c, c->facA, totA * sizeof(double));
    if (rc) return rc;
  }
  // Y matrices, then one 3 x 64 x 64 block per problem for the pair chains
  // of batched plans
  if ((rc = ensure(c, c->facY, (totA + (size_t)np * 3 * 64 * 64) * sizeof(double)))) return rc;
  std::vector<FacProb> probs(np);
  for (int p = 0; p < np; ++p) {
    const FacJob& J = jobs[p];
    FacProb f;
    f.H = J.H;
    f.A = (double*)c->facA.p + oA[p];
    f.Y = (double*)c->facY.p + oA[p];
    f.D = (double*)c->facY.p + totA + (size_t)p * 3 * 64 * 64;
    f.U = J.U;
    f.n = J.n;
    f.ldh = J.ldh;
    f.ldu = J.ldu;
    f.pad0 = 0;
    f.lam_abs = J.lam_abs;
    f.lam_rel = J.lam_rel;
    f.lam = &dslots[p].lam;
    f.info = &dslots[p].info;
    f.nonfinite = &dslots[p].nonfinite;
    probs[p] = f;
    if (A_out) A_out[p] = f.A;
  }
  Blob b;
  const size_t o_probs = b.add(probs);
  std::vector<FacShape> shapes(np);
  for (int p = 0; p < np; ++p) shapes[p] = FacShape{jobs[p].n, jobs[p].H != nullptr};
  const std::vector<PlanLaunch> launches = plan_factor(shapes, c->ncu);
  std::vector<size_t> offs(launches.size());
  for (size_t i = 0; i < launches.size(); ++i)
    if (!launches[i].segs.empty()) offs[i] = b.add(launches[i].segs);
  uint8_t* d = nullptr;
  if ((rc = upload(c, b, &d))) return rc;
  const FacProb* dp = (const FacProb*)(d + o_probs);
  LAUNCH(c, "k_damp_lambda", launch_damp_lambda(dp, np, c->stream));
  // the side stream's updates take at most this many CUs (one workgroup per
  // CU, whose registers fill the CU), leaving about 96 to the serial chain:
  // the 64 panel workgroups of a 4096-wide problem and its narrow updates
  // (measured best at n = 4096 among caps of 128 to 256 CUs).  Batched plans,
  // whose panel launches outnumber the CUs anyway (they run the diagonal
  // chains first), give the updates all but 64 CUs: there the updates set the
  // pace, and the 64 keep the diagonal chains from waiting for them (ViT:
  // caps of 160, 192, 208 and 256 measured; 192 best, within about 1%).
  bool batched = false;
  for (const PlanLaunch& l : launches) batched = batched || l.kind == FK_DIAG2;
  const int side_wg = batched ? std::max(1, c->ncu - std::min(64, c->ncu / 2))
                              : std::max(1, c->ncu - std::min(96, c->ncu / 2));
  for (size_t i = 0; i < launches.size(); ++i) {
    const PlanLaunch& l = launches[i];
    const Seg* sg = (const Seg*)(d + offs[i]);
    const int nseg = (int)l.segs.size();
    hipStream_t st = l.side ? c->side : c->stream;
    switch (l.kind) {
      case FK_FILL: LAUNCH(c, "k_damp_fill", launch_damp_fill(dp, sg, nseg, l.nwg, c->stream)); break;
      case FK_PANEL: LAUNCH(c, "k_chol_panel", launch_chol_panel(dp, sg, nseg, l.nwg, c->stream)); break;
      case FK_PANEL2: LAUNCH(c, "k_chol_panel2", launch_chol_panel2(dp, sg, nseg, l.nwg, c->stream)); break;
      case FK_DIAG2: LAUNCH(c, "k_chol_diag2", launch_chol_diag2(dp, sg, nseg, l.nwg, c->stream)); break;
      case FK_GEMM64: LAUNCH(c, "k_gemm64", launch_gemm64(dp, sg, nseg, l.nwg, c->stream)); break;
      case FK_RING64: LAUNCH_ON(c, st, "k_gemm_ring64", launch_gemm_ring(64, dp, sg, nseg, l.nwg, 0, st)); break;
      case FK_RING128:
        LAUNCH_ON(c, st, "k_gemm_ring128", launch_gemm_ring(128, dp, sg, nseg, l.nwg, l.side ? side_wg : 0, st));
        break;
      case FK_MAKEU: LAUNCH(c, "k_make_u", launch_make_u(dp, sg, nseg, l.nwg, c->stream)); break;
      case PL_FORK:
        HIPCHK(c, hipEventRecord(c->fork_ev, c->stream));
        HIPCHK(c, hipStreamWaitEvent(c->side, c->fork_ev, 0));
        break;
      case PL_JOIN:
        HIPCHK(c, hipEventRecord(c->join_ev, c->side));
        HIPCHK(c, hipStreamWaitEvent(c->stream, c->join_ev, 0));
        break;
    }
  }
  return GPTQ_OK;
}

// ----------------------------------------------------------- quantize plan --
// na: run inside the no-allocation scratch array (single layer within the
// limits, checked by the caller); nothing is allocated.
int run_quantize(gptq_ctx c, const std::vector<QuantJob>& jobs, std::vector<float*>* Ww_out = nullptr,
                 const NoAlloc* na = nullptr) {
  const int nl = (int)jobs.size();
  std::vector<QuantShape> shapes(nl);
  for (int p = 0; p < nl; ++p) {
    const QuantJob& J = jobs[p];
    shapes[p] = QuantShape{J.out, J.n, J.nt, J.block, J.group, J.mode, J.Ww_ext != nullptr};
  }
  QuantLayout QLy;
  std::vector<PlanLaunch> launches;
  plan_quantize(shapes, &QLy, &launches);
  const std::vector<int>& sbk = QLy.sbk;
  // the sweep keeps a super-block's columns of its rows in LDS: at most 1024
  // columns for 128-wide blocks, 512 for narrower ones
  for (size_t p = 0; p < shapes.size(); ++p)
    if (sbk[p] * shapes[p].block > (shapes[p].block >= 128 ? 1024 : 512))
      return set_err(c, GPTQ_ERR_UNSUPPORTED, "super-block wider than the sweep's LDS row buffer");
  const size_t totW = QLy.totW, totE = QLy.totE, totO = QLy.totO, totD = QLy.totD;
  const std::vector<size_t>&oW = QLy.oW, &oE = QLy.oE, &oO = QLy.oO, &oD = QLy.oD;
  int rc;
  float* work_p;
  float* eblk_p;
  double* objp_p;
  float* dinv_p;
  if (na) {
    if (totW * sizeof(float) > NA_WW || totE * sizeof(float) > NA_EB || totO * sizeof(double) > NA_OBJP ||
        totD * sizeof(float) > NA_DINV)
      return set_err(c, GPTQ_ERR_UNSUPPORTED, "layer exceeds the no-allocation limits");
    work_p = na->ww;
    eblk_p = na->eb;
    objp_p = na->objp;
    dinv_p = na->dinv;
  } else {
    if ((rc = ensure(c, c->work, totW * sizeof(float)))) return rc;
    if ((rc = ensure(c, c->eblk, totE * sizeof(float)))) return rc;
    if ((rc = ensure(c, c->objp, totO * sizeof(double)))) return rc;
    if ((rc = ensure(c, c->dinv, totD * sizeof(float)))) return rc;
    work_p = (float*)c->work.p;
    eblk_p = (float*)c->eblk.p;
    objp_p = (double*)c->objp.p;
    dinv_p = (float*)c->dinv.p;
  }
  std::vector<QLayer> L(nl);
  for (int p = 0; p < nl; ++p) {
    const QuantJob& J = jobs[p];
    QLayer q;
    q.W = J.W;
    q.Ww = J.Ww_ext ? J.Ww_ext : work_p + oW[p];
    q.U = J.U;
    q.codes = J.codes;
    q.scales = J.scales;
    q.zeros = J.zeros;
    q.err = J.err;
    q.Eb = eblk_p + oE[p];
    q.objp = objp_p + oO[p];
    q.dinv = dinv_p + oD[p];
    q.obj = J.obj;
    q.lam = J.lam;
    q.out = J.out;
    q.n = J.n;
    q.nt = J.nt;
    q.bits = J.bits;
    q.group = J.group;
    q.block = J.block;
    q.nblk = cdiv(J.n, J.block);
    q.ng = J.group ? J.n / J.group : 1;
    q.ldE = sbk[p] * J.block;
    q.eoff_blk = J.block;
    q.sbk = sbk[p];
    q.mode = J.mode;
    L[p] = q;
    if (Ww_out) Ww_out->push_back(q.Ww);
  }
  Blob b;
  const size_t o_L = b.add(L);
  std::vector<size_t> offs(launches.size());
  for (size_t i = 0; i < launches.size(); ++i)
    if (!launches[i].segs.empty()) offs[i] = b.add(launches[i].segs);
  uint8_t* d = nullptr;
  if ((rc = na ? upload_noalloc(c, b, na->blob, &d) : upload(c, b, &d))) return rc;
  const QLayer* dL = (const QLayer*)(d + o_L);
  for (size_t i = 0; i < launches.size(); ++i) {
    const PlanLaunch& l = launches[i];
    const Seg* sg = (const Seg*)(d + offs[i]);
    const int nseg = (int)l.segs.size();
    hipStream_t st = l.side ? c->side : c->stream;
    switch (l.kind) {
      case QK_INIT: LAUNCH(c, "k_init_work", launch_init_work(dL, sg, nseg, l.nwg, c->stream)); break;
      case QK_ROWFIT: LAUNCH(c, "k_rowfit", launch_rowfit(dL, sg, nseg, l.nwg, c->stream)); break;
      case QK_SWEEP: LAUNCH(c, "k_sweep", launch_sweep(l.block, l.mode, dL, sg, nseg, l.nwg, c->stream)); break;
      case QK_TRAIL:  // beside the sweeps: a persistent grid of two workgroups per CU
        LAUNCH_ON(c, st, "k_trail", launch_trail(l.block, dL, sg, nseg, l.nwg, l.side ? 2 * c->ncu : 0, st));
        break;
      case PL_FORK:
        HIPCHK(c, hipEventRecord(c->fork_ev, c->stream));
        HIPCHK(c, hipStreamWaitEvent(c->side, c->fork_ev, 0));
        break;
      case PL_JOIN:
        HIPCHK(c, hipEventRecord(c->join_ev, c->side));
        HIPCHK(c, hipStreamWaitEvent(c->stream, c->join_ev, 0));
        break;
    }
  }
  LAUNCH(c, "k_objective", launch_objective(dL, nl, c->stream));
  return GPTQ_OK;
}

int check_quant_args(gptq_ctx c, int out, int n, int bits, int group, int block) {
  if (out < 0 || n < 0) return set_err(c, GPTQ_ERR_INVALID_ARG, "negative size");
  if (bits < 2 || bits > 8) return set_err(c, GPTQ_ERR_INVALID_ARG, "bits must be in 2..8");
  if (!(block == 16 || block == 32 || block == 64 || block == 128))
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
  if (group < 0) return set_err(c, GPTQ_ERR_INVALID_ARG, "negative group");
  if (group) {
    if (group % 8) return set_err(c, GPTQ_ERR_UNSUPPORTED, "group must be a multiple of 8");
    if (n % group) return set_err(c, GPTQ_ERR_INVALID_ARG, "group must divide n");
    if (group % block && block % group)
      return set_err(c, GPTQ_ERR_UNSUPPORTED, "group and block must divide one another");
  }
  return GPTQ_OK;
}

int check_x(gptq_ctx c, const uint16_t* X, long long tokens, int n, long long ldx) {
  if (tokens < 0 || n < 0 || ldx < n) return set_err(c, GPTQ_ERR_INVALID_ARG, "bad X sizes");
  if (tokens > 0 && n > 0 && !X) return set_err(c, GPTQ_ERR_INVALID_ARG, "X is null");
  if ((uintptr_t)X & 1) return set_err(c, GPTQ_ERR_INVALID_ARG, "X is not 2-byte aligned");
  if (tokens > 0x7fffffffLL) return set_err(c, GPTQ_ERR_UNSUPPORTED, "tokens > 2^31-1");
  return GPTQ_OK;
}

int ensure_small(gptq_ctx c, size_t bytes) { return ensure_pinned(c, c->hsmall, c->hsmall_cap, bytes); }

}  // namespace

// The no-allocation scratch array (see NoAlloc) and each device's address of
// its copy, looked up once per device (with that device current) when the
// first context on it is created.  Host code must use these addresses, never
// the array's name (a host-side stand-in).
static __device__ __align__(256) uint8_t scratch[NA_BYTES];
static std::mutex g_na_mu;
static uint8_t* g_na_ptr[64];
static int g_na_state[64];  // 0: not looked up, 1: found, 2: lookup failed

// ================================================================ C ABI ====
GPTQ_API const char* gptq_strerror(int status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_NOT_PD: return "damped Hessian is not positive definite";
    case GPTQ_ERR_NONFINITE: return "non-finite value in the Hessian";
    case GPTQ_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case GPTQ_ERR_HIP: return "HIP runtime error";
    case GPTQ_ERR_NO_MEMORY: return "out of device memory";
    case GPTQ_ERR_NOT_CONVERGED: return "subspace iteration stopped at its cap; outputs are from the last iterate";
    default: return "unknown status";
  }
}

GPTQ_API const char* gptq_last_error(gptq_ctx ctx) { return ctx ? ctx->err.c_str() : ""; }

GPTQ_API int gptq_create(gptq_ctx* ctx, int device, void* stream) {
  if (!ctx) return GPTQ_ERR_INVALID_ARG;
  *ctx = nullptr;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return GPTQ_ERR_INVALID_ARG;
  gptq_ctx c = new gptq_ctx_s();
  c->device = device;
  c->stream = (hipStream_t)stream;
  DeviceGuard g(device);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
    c->ncu = prop.multiProcessorCount;
  if (hipEventCreateWithFlags(&c->blob_ev, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming) != hipSuccess ||
      hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess) {
    if (c->blob_ev) (void)hipEventDestroy(c->blob_ev);
    if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
    if (c->join_ev) (void)hipEventDestroy(c->join_ev);
    delete c;
    return GPTQ_ERR_HIP;
  }
  {
    // this device's copy of the no-allocation scratch array
    std::lock_guard<std::mutex> lk(g_na_mu);
    if (device < 64 && g_na_state[device] == 0) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) (void)hipGetLastError();
      g_na_state[device] = (e == hipSuccess && ptr) ? 1 : 2;
      g_na_ptr[device] = (uint8_t*)ptr;
    }
    c->na_base = (device < 64 && g_na_state[device] == 1) ? g_na_ptr[device] : nullptr;
  }
  // pinned host staging that gptq_quantize_noalloc uses (it allocates nothing itself)
  (void)ensure_pinned(c, c->hblob, c->hblob_cap, NA_BLOB);
  (void)ensure_pinned(c, c->hsmall, c->hsmall_cap, 4096);
  c->err.clear();
  *ctx = c;
  return GPTQ_OK;
}

GPTQ_API int gptq_destroy(gptq_ctx c) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  {
    DeviceGuard g(c->device);
    (void)hipStreamSynchronize(c->stream);
    if (c->side) (void)hipStreamSynchronize(c->side);
    DevBuf* bufs[] = {&c->partials, &c->xt, &c->facA, &c->facY, &c->work, &c->eblk, &c->dinv,
                      &c->objp, &c->slots, &c->blob, &c->lora, &c->r2d, &c->qr};
    for (DevBuf* b : bufs)
      if (b->p) (void)hipFree(b->p);
    if (c->hblob) (void)hipHostFree(c->hblob);
    if (c->hsmall) (void)hipHostFree(c->hsmall);
    if (c->blob_ev) (void)hipEventDestroy(c->blob_ev);
    if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
    if (c->join_ev) (void)hipEventDestroy(c->join_ev);
    if (c->side) (void)hipStreamDestroy(c->side);
    for (const auto& t : c->tpend) {
      (void)hipEventDestroy(t.a);
      (void)hipEventDestroy(t.b);
    }
    for (hipEvent_t e : c->tpool) (void)hipEventDestroy(e);
  }
  delete c;
  return GPTQ_OK;
}

GPTQ_API int gptq_timing(gptq_ctx c, const char* kernels) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  DeviceGuard g(c->device);
  int rc = timer_collect(c);
  if (rc) return rc;
  c->tname.clear();
  c->tms.clear();
  c->tcount.clear();
  c->timing = kernels != nullptr;
  c->tfilter.clear();
  if (kernels) {
    std::string k(kernels);
    k.erase(std::remove(k.begin(), k.end(), ' '), k.end());
    c->tfilter = (k == "*") ? k : "," + k + ",";
  }
  return GPTQ_OK;
}

GPTQ_API int gptq_kernel_time(gptq_ctx c, const char* name, double* total_ms, int64_t* launches) {
  if (!c || !name || !total_ms || !launches) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  DeviceGuard g(c->device);
  int rc = timer_collect(c);
  if (rc) return rc;
  *total_ms = 0.0;
  *launches = 0;
  for (size_t k = 0; k < c->tname.size(); ++k)
    if (c->tname[k] == name) {
      *total_ms = c->tms[k];
      *launches = c->tcount[k];
    }
  return GPTQ_OK;
}

GPTQ_API int gptq_hessian(gptq_ctx c, const uint16_t* X, int64_t tokens, int32_t n, int64_t ldx,
                          float* H, int accumulate) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  int rc = check_x(c, X, tokens, n, ldx);
  if (rc) return rc;
  if (n > 0 && !H) return set_err(c, GPTQ_ERR_INVALID_ARG, "H is null");
  if (n == 0) return GPTQ_OK;
  DeviceGuard g(c->device);
  return run_hessian(c, {HessJob{X, tokens, ldx, n, H, accumulate ? 1 : 0}});
}

GPTQ_API int gptq_cross_gram(gptq_ctx c, const uint16_t* X, const uint16_t* Y, int64_t tokens, int32_t n,
                             int64_t ldx, float* G) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  int rc = check_x(c, X, tokens, n, ldx);
  if (rc) return rc;
  if ((rc = check_x(c, Y, tokens, n, ldx))) return rc;
  if (n > 0 && !G) return set_err(c, GPTQ_ERR_INVALID_ARG, "G is null");
  if (n == 0) return GPTQ_OK;
  HessJob J{X, tokens, ldx, n, G, 0};
  J.Y = Y;
  if (tokens > 0 && !(hess_direct(J) && ((uintptr_t)Y & 15) == 0))
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "cross Gram needs 16-byte aligned rows and n % 8 == 0");
  DeviceGuard g(c->device);
  return run_hessian(c, {J});
}

GPTQ_API int gptq_factor(gptq_ctx c, const float* H, int32_t n, double lam_abs, double lam_rel,
                         float* U, int32_t* info, double* lam_used) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (info) *info = 0;
  if (n < 0 || (n > 0 && (!H || !U)) || !info) return set_err(c, GPTQ_ERR_INVALID_ARG, "bad factor arguments");
  if (!std::isfinite(lam_abs) || !std::isfinite(lam_rel)) return set_err(c, GPTQ_ERR_INVALID_ARG, "non-finite damping");
  if (n == 0) return GPTQ_OK;
  DeviceGuard g(c->device);
  int rc = ensure(c, c->slots, sizeof(Slot));
  if (rc) return rc;
  Slot* ds = (Slot*)c->slots.p;
  if ((rc = run_factor(c, {FacJob{H, n, n, n, lam_abs, lam_rel, U}}, ds))) return rc;
  if ((rc = ensure_small(c, sizeof(Slot)))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, ds, sizeof(Slot), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  const Slot s = *(const Slot*)c->hsmall;
  if (lam_used) *lam_used = s.lam;
  if (s.nonfinite) return set_err(c, GPTQ_ERR_NONFINITE, "non-finite entry in H");
  *info = s.info;
  if (s.info) return set_err(c, GPTQ_ERR_NOT_PD, "not positive definite at column %d", s.info - 1);
  return GPTQ_OK;
}

GPTQ_API int gptq_quantize(gptq_ctx c, const float* W, int32_t out, int32_t n, const float* U,
                           int32_t bits, int32_t group, int32_t block, double lam, uint8_t* codes,
                           float* scales, uint8_t* zeros, float* err, double* obj) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  int rc = check_quant_args(c, out, n, bits, group, block);
  if (rc) return rc;
  if (!obj) return set_err(c, GPTQ_ERR_INVALID_ARG, "obj is null");
  obj[0] = obj[1] = 0.0;
  if (out == 0 || n == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros) return set_err(c, GPTQ_ERR_INVALID_ARG, "null pointer");
  DeviceGuard g(c->device);
  if ((rc = ensure(c, c->slots, sizeof(Slot)))) return rc;
  Slot* ds = (Slot*)c->slots.p;
  Slot hs{};
  hs.lam = lam;
  HIPCHK(c, hipMemcpyAsync(ds, &hs, sizeof(Slot), hipMemcpyHostToDevice, c->stream));
  QuantJob J{W, out, n, n, U, bits, group, block, codes, scales, zeros, err, &ds->lam, ds->obj, nullptr};
  if ((rc = run_quantize(c, {J}))) return rc;
  if ((rc = ensure_small(c, sizeof(Slot)))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, ds, sizeof(Slot), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  const Slot s = *(const Slot*)c->hsmall;
  obj[0] = s.obj[0];
  obj[1] = s.obj[1];
  return GPTQ_OK;
}

GPTQ_API int gptq_quantize_noalloc(gptq_ctx c, const float* W, int32_t out, int32_t n, const float* U,
                                   int32_t bits, int32_t group, int32_t block, double lam, uint8_t* codes,
                                   float* scales, uint8_t* zeros, float* err, double* obj) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  int rc = check_quant_args(c, out, n, bits, group, block);
  if (rc) return rc;
  if (!obj) return set_err(c, GPTQ_ERR_INVALID_ARG, "obj is null");
  obj[0] = obj[1] = 0.0;
  if (out == 0 || n == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros) return set_err(c, GPTQ_ERR_INVALID_ARG, "null pointer");
  if (out > NA_MAX_OUT || n > NA_MAX_N || (long long)out * n > NA_MAX_ELEMS)
    return set_err(c, GPTQ_ERR_UNSUPPORTED,
                   "layer %d x %d exceeds the no-allocation limits (out <= %d, n <= %d, out * n <= %lld)", out, n,
                   NA_MAX_OUT, NA_MAX_N, NA_MAX_ELEMS);
  if (!c->na_base) return set_err(c, GPTQ_ERR_HIP, "the no-allocation scratch array is unavailable on device %d", c->device);
  if (c->hblob_cap < NA_BLOB || c->hsmall_cap < 2 * sizeof(Slot))
    return set_err(c, GPTQ_ERR_NO_MEMORY, "the context's pinned staging was not allocated");
  DeviceGuard g(c->device);
  const NoAlloc na = noalloc_view(c->na_base);
  // per-kernel timing would create event pairs: off for this call
  struct TimingOff {
    gptq_ctx c;
    bool was;
    ~TimingOff() { c->timing = was; }
  } toff{c, c->timing};
  c->timing = false;
  Slot* hs = (Slot*)c->hsmall;  // [0]: the slot sent, [1]: the slot read back
  if (c->blob_pending) {  // an earlier upload may still read the pinned staging
    HIPCHK(c, hipEventSynchronize(c->blob_ev));
    c->blob_pending = false;
  }
  hs[0] = Slot{};
  hs[0].lam = lam;
  HIPCHK(c, hipMemcpyAsync(na.slot, &hs[0], sizeof(Slot), hipMemcpyHostToDevice, c->stream));
  QuantJob J{W, out, n, n, U, bits, group, block, codes, scales, zeros, err, &na.slot->lam, na.slot->obj, nullptr};
  if ((rc = run_quantize(c, {J}, nullptr, &na))) return rc;
  HIPCHK(c, hipMemcpyAsync(&hs[1], na.slot, sizeof(Slot), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  obj[0] = hs[1].obj[0];
  obj[1] = hs[1].obj[1];
  return GPTQ_OK;
}

GPTQ_API int gptq_quantize_batched(gptq_ctx c, int32_t nlayers, gptq_layer* layers) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (nlayers < 0 || (nlayers > 0 && !layers)) return set_err(c, GPTQ_ERR_INVALID_ARG, "bad layer list");
  if (nlayers == 0) return GPTQ_OK;
  for (int i = 0; i < nlayers; ++i) {
    gptq_layer& l = layers[i];
    l.info = 0;
    l.obj[0] = l.obj[1] = 0.0;
    int rc = check_quant_args(c, l.out, l.n, l.bits, l.group, l.block);
    if (rc) return rc;
    if (l.n <= 0 || l.out <= 0) return set_err(c, GPTQ_ERR_INVALID_ARG, "layer %d: empty", i);
    if (!l.W || !l.H || !l.U || !l.codes || !l.scales || !l.zeros)
      return set_err(c, GPTQ_ERR_INVALID_ARG, "layer %d: null pointer", i);
    if (l.X && (rc = check_x(c, l.X, l.tokens, l.n, l.ldx))) return rc;
  }
  DeviceGuard g(c->device);
  int rc;
  std::vector<HessJob> hj;
  for (int i = 0; i < nlayers; ++i)
    if (layers[i].X) hj.push_back(HessJob{layers[i].X, layers[i].tokens, layers[i].ldx, layers[i].n, layers[i].H, 0});
  if (!hj.empty() && (rc = run_hessian(c, hj))) return rc;
  // one factor per distinct (H, U, damping)
  std::vector<int> fac_of(nlayers, -1);
  std::vector<FacJob> fj;
  for (int i = 0; i < nlayers; ++i) {
    for (int j = 0; j < i; ++j)
      if (layers[j].H == layers[i].H && layers[j].U == layers[i].U && layers[j].n == layers[i].n &&
          layers[j].lam_abs == layers[i].lam_abs && layers[j].lam_rel == layers[i].lam_rel) {
        fac_of[i] = fac_of[j];
        break;
      }
    if (fac_of[i] < 0) {
      fac_of[i] = (int)fj.size();
      fj.push_back(FacJob{layers[i].H, layers[i].n, layers[i].n, layers[i].n, layers[i].lam_abs, layers[i].lam_rel, layers[i].U});
    }
  }
  const int nf = (int)fj.size();
  if ((rc = ensure(c, c->slots, sizeof(Slot) * (nf + nlayers)))) return rc;
  Slot* ds = (Slot*)c->slots.p;
  if ((rc = run_factor(c, fj, ds))) return rc;
  std::vector<QuantJob> qj;
  for (int i = 0; i < nlayers; ++i) {
    const gptq_layer& l = layers[i];
    qj.push_back(QuantJob{l.W, l.out, l.n, l.n, l.U, l.bits, l.group, l.block, l.codes, l.scales, l.zeros,
                          l.err, &ds[fac_of[i]].lam, ds[nf + i].obj, nullptr});
  }
  if ((rc = run_quantize(c, qj))) return rc;
  const size_t bytes = sizeof(Slot) * (nf + nlayers);
  if ((rc = ensure_small(c, bytes))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, ds, bytes, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  const Slot* hs = (const Slot*)c->hsmall;
  int first = GPTQ_OK;
  for (int i = 0; i < nlayers; ++i) {
    const Slot& f = hs[fac_of[i]];
    layers[i].info = f.info;
    layers[i].obj[0] = hs[nf + i].obj[0];
    layers[i].obj[1] = hs[nf + i].obj[1];
    if (!first && f.nonfinite) first = set_err(c, GPTQ_ERR_NONFINITE, "layer %d: non-finite H", i);
    if (!first && f.info) first = set_err(c, GPTQ_ERR_NOT_PD, "layer %d: not positive definite", i);
  }
  return first;
}

namespace {

// C[M][N] = A[M][K] B[N][K]^T (pitch ld) on the fp64 MFMA ring, 128 tiles;
// tri = 1 / 2: B upper / lower triangular (zero part of K skipped).
int run_gemm_nt(gptq_ctx c, const double* A, const double* B, double* C, int M, int N, int K, int ld, int tri = 0) {
  FacProb p{};
  p.A = (double*)A;
  p.Y = (double*)B;
  p.C = C;
  p.n = ld;
  const int ntiles = cdiv(M, 128) * cdiv(N, 128);
  std::vector<Seg> segs{Seg{0, 0, ntiles, GK_NT, M, N, K, tri}};
  Blob b;
  const size_t op = b.add(&p, 1), os = b.add(segs);
  uint8_t* d = nullptr;
  int rc = upload(c, b, &d);
  if (rc) return rc;
  LAUNCH(c, "k_gemm_ring128",
         launch_gemm_ring(128, (const FacProb*)(d + op), (const Seg*)(d + os), 1, ntiles, 0, c->stream));
  return GPTQ_OK;
}

// Services the LoRA and refinement drivers borrow from the context.
LoraHooks lora_hooks(gptq_ctx c) {
  LoraHooks hooks;
  hooks.hessian64 = [c](const uint16_t* X_, long long t_, long long ld_, int n_, double* H_) {
    return run_hessian64(c, X_, t_, ld_, n_, H_);
  };
  hooks.ensure = [c](size_t bytes) -> void* {
    if (ensure(c, c->lora, bytes)) return nullptr;
    return c->lora.p;
  };
  hooks.factor = [c](double* A, int nt, float* U, Slot* slot) {
    // A was assembled (damped, reversed, lower) by the LoRA kernels
    std::vector<FacJob> fj{FacJob{nullptr, nt, nt, nt, 0.0, 0.0, U}};
    DevBuf save = c->facA;
    c->facA.p = A;
    c->facA.cap = (size_t)nt * nt * sizeof(double);
    int rc2 = run_factor(c, fj, slot, true);
    c->facA = save;
    return rc2;
  };
  hooks.quantize = [c](const QuantJob& j) { return run_quantize(c, {j}); };
  hooks.slots = [c](size_t bytes) -> void* {
    if (ensure(c, c->slots, bytes)) return nullptr;
    return c->slots.p;
  };
  hooks.set_err = [c](int st, const char* msg) { return set_err(c, st, "%s", msg); };
  hooks.launch = [c](const char* name, const std::function<hipError_t()>& f) -> int {
    LAUNCH(c, name, f());
    return GPTQ_OK;
  };
  hooks.gemm_nt = [c](const double* A, const double* B, double* C, int M, int N, int K, int ld) {
    return run_gemm_nt(c, A, B, C, M, N, K, ld);
  };
  hooks.read = [c](const void* dev, void* host, size_t bytes) -> int {
    int rc2 = ensure_small(c, bytes);
    if (rc2) return rc2;
    HIPCHK(c, hipMemcpyAsync(c->hsmall, dev, bytes, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
    memcpy(host, c->hsmall, bytes);
    return GPTQ_OK;
  };
  hooks.not_converged = [c]() { c->not_converged = true; };
  return hooks;
}

// gptq_lora and gptq_lora_refine: the sweep on the augmented Hessian, then
// `rounds` refinement rounds; obj (rounds == 0: {J, J_lam}) or the trace
// (rounds > 0: 2 rounds + 2 values) is copied to res.
int lora_impl(gptq_ctx c, const float* W, int32_t out, int32_t n, const uint16_t* X, int64_t tokens, int64_t ldx,
              int32_t r, int32_t bits, int32_t group, int32_t block, double lam_abs, double lam_rel, int32_t rounds,
              uint8_t* codes, float* scales, uint8_t* zeros, float* L, float* R, double* res, int32_t* info) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (info) *info = 0;
  int rc = check_quant_args(c, out, n, bits, group, block);
  if (rc) return rc;
  if ((rc = check_x(c, X, tokens, n, ldx))) return rc;
  if (r < 1 || r > 128 || r > n) return set_err(c, GPTQ_ERR_UNSUPPORTED, "rank must be in 1..min(128, n)");
  if (!res || !W || !codes || !scales || !zeros || !L || !R || out <= 0 || n <= 0)
    return set_err(c, GPTQ_ERR_INVALID_ARG, "null pointer or empty layer");
  if (rounds > 0 && r > out) return set_err(c, GPTQ_ERR_UNSUPPORTED, "refinement needs rank <= out");
  const int nres = rounds > 0 ? 2 * rounds + 2 : 2;
  for (int k = 0; k < nres; ++k) res[k] = 0.0;
  DeviceGuard g(c->device);
  LoraIO io{W, out, n, X, tokens, ldx, r, bits, group, block, lam_abs, lam_rel, codes, scales, zeros, L, R};
  io.rounds = rounds;
  const LoraHooks hooks = lora_hooks(c);
  c->not_converged = false;
  rc = run_lora(c->stream, io, hooks);
  if (rc) return rc;
  const size_t bytes = sizeof(Slot) + (rounds > 0 ? (size_t)nres * sizeof(double) : 0);
  if ((rc = ensure_small(c, bytes))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, c->slots.p, bytes, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  const Slot s = *(const Slot*)c->hsmall;
  if (s.nonfinite) return set_err(c, GPTQ_ERR_NONFINITE, "non-finite entry in H");
  if (info) *info = s.info;
  if (s.info) return set_err(c, GPTQ_ERR_NOT_PD, "augmented Hessian not positive definite");
  if (rounds > 0) {
    const double* tr = (const double*)((const Slot*)c->hsmall + 1);
    for (int k = 0; k < nres; ++k) res[k] = tr[k];
  } else {
    res[0] = s.obj[0];
    res[1] = s.obj[1];
  }
  if (c->not_converged)
    return set_err(c, GPTQ_ERR_NOT_CONVERGED, "a top-%d subspace iteration stopped at its cap", (int)r);
  return GPTQ_OK;
}

// gptq_olrc / gptq_bid_up: one refinement step on caller-held state.
int refine_step(gptq_ctx c, bool bid, const float* W, int32_t out, int32_t n, const double* H, int32_t r,
                int32_t bits, int32_t group, int32_t block, uint8_t* codes, float* scales, uint8_t* zeros, float* L,
                float* R, double* J) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  int rc = check_quant_args(c, out, n, bits, group, block);
  if (rc) return rc;
  if (!J || !W || !H || !codes || !scales || !zeros || !L || !R || out <= 0 || n <= 0)
    return set_err(c, GPTQ_ERR_INVALID_ARG, "null pointer or empty layer");
  if (r < 1 || r > 128 || r > n || r > out)
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "rank must be in 1..min(128, out, n)");
  *J = 0.0;
  DeviceGuard g(c->device);
  if ((rc = ensure(c, c->slots, sizeof(double)))) return rc;
  double* dJ = (double*)c->slots.p;
  RefineIO io{W, out, n, H, r, bits, group, block, codes, scales, zeros, L, R};
  const LoraHooks hooks = lora_hooks(c);
  c->not_converged = false;
  rc = bid ? run_bid_up(c->stream, io, hooks, dJ) : run_olrc(c->stream, io, hooks, dJ);
  if (rc) return rc;
  if ((rc = ensure_small(c, sizeof(double)))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, dJ, sizeof(double), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  *J = *(const double*)c->hsmall;
  if (c->not_converged)
    return set_err(c, GPTQ_ERR_NOT_CONVERGED, "the top-%d subspace iteration stopped at its cap", (int)r);
  return GPTQ_OK;
}

}  // namespace

GPTQ_API int gptq_round_2d(gptq_ctx c, const float* X, int32_t m, int32_t n, const float* UG, const float* UH,
                           int32_t qmin, int32_t qmax, int32_t* Z, float* delta, double* J) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (J) *J = 0.0;
  if (m < 0 || n < 0 || !J || (m > 0 && n > 0 && (!X || !UG || !UH || !Z)))
    return set_err(c, GPTQ_ERR_INVALID_ARG, "bad two-sided rounding arguments");
  if (qmin > qmax) return set_err(c, GPTQ_ERR_INVALID_ARG, "qmin > qmax");
  if (m == 0 || n == 0) return GPTQ_OK;
  DeviceGuard g(c->device);
  const int TM = cdiv(m, 64), TN = cdiv(n, 64);
  const size_t mn = (size_t)m * n;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t oL = take((size_t)m * m * 4), oU = take((size_t)n * n * 4), odG = take((size_t)m * 4),
               odH = take((size_t)n * 4), oC = take(mn * 4), oR = take(mn * 4), oD = take(mn * 4), oCf = take(mn * 4),
               oO = take((size_t)TM * TN * 8), oJ = take(8);
  int rc = ensure(c, c->r2d, off);
  if (rc) return rc;
  uint8_t* base = (uint8_t*)c->r2d.p;
  R2dProb p;
  p.X = X;
  p.Lgt = (const float*)(base + oL);
  p.Uh1 = (const float*)(base + oU);
  p.dG = (const float*)(base + odG);
  p.dH = (const float*)(base + odH);
  p.C = (float*)(base + oC);
  p.R = (float*)(base + oR);
  p.D = delta ? delta : (float*)(base + oD);
  p.Cf = (float*)(base + oCf);
  p.Z = Z;
  p.objp = (double*)(base + oO);
  p.m = m;
  p.n = n;
  p.qmin = qmin;
  p.qmax = qmax;
  double* dJ = (double*)(base + oJ);
  LAUNCH(c, "k_r2d_unit", launch_r2d_unit(UG, m, (float*)p.Lgt, (float*)p.dG, c->stream));
  LAUNCH(c, "k_r2d_unit", launch_r2d_unit(UH, n, (float*)p.Uh1, (float*)p.dH, c->stream));
  LAUNCH(c, "k_r2d_fill", launch_r2d_fill(p.C, p.R, (long long)mn, c->stream));
  // anti-diagonals of 64 x 64 tiles: the stage's tiles, the pushes into the
  // next row / column block on the main stream, the rest on the side stream
  // beside the next stage's tiles (joined before the next near pushes)
  bool side_busy = false;
  for (int S = 0; S < TM + TN - 1; ++S) {
    const int Ib = std::max(0, S - TN + 1), Ie = std::min(TM - 1, S);
    LAUNCH(c, "k_r2d_tile", launch_r2d_tile(p, S, Ib, Ie - Ib + 1, c->stream));
    if (side_busy) {
      HIPCHK(c, hipEventRecord(c->join_ev, c->side));
      HIPCHK(c, hipStreamWaitEvent(c->stream, c->join_ev, 0));
    }
    LAUNCH(c, "k_r2d_push", launch_r2d_push(p, S, Ib, Ie, false, 0, c->stream));
    HIPCHK(c, hipEventRecord(c->fork_ev, c->stream));
    HIPCHK(c, hipStreamWaitEvent(c->side, c->fork_ev, 0));
    LAUNCH_ON(c, c->side, "k_r2d_push", launch_r2d_push(p, S, Ib, Ie, true, 0, c->side));
    side_busy = true;
  }
  if (side_busy) {
    HIPCHK(c, hipEventRecord(c->join_ev, c->side));
    HIPCHK(c, hipStreamWaitEvent(c->stream, c->join_ev, 0));
  }
  LAUNCH(c, "k_r2d_obj", launch_r2d_obj(p.objp, TM * TN, dJ, c->stream));
  if ((rc = ensure_small(c, sizeof(double)))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, dJ, sizeof(double), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  *J = *(const double*)c->hsmall;
  return GPTQ_OK;
}

GPTQ_API int gptq_quantize_qronos(gptq_ctx c, const float* W, int32_t out, int32_t n, const uint16_t* X,
                                  const uint16_t* Xq, int64_t tokens, int64_t ldx, int32_t bits, int32_t group,
                                  int32_t block, double lam_abs, double lam_rel, uint8_t* codes, float* scales,
                                  uint8_t* zeros, float* Wt, double* obj, int32_t* info) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (info) *info = 0;
  int rc = check_quant_args(c, out, n, bits, group, block);
  if (rc) return rc;
  if ((rc = check_x(c, X, tokens, n, ldx))) return rc;
  if ((rc = check_x(c, Xq, tokens, n, ldx))) return rc;
  if (!obj || !W || !codes || !scales || !zeros || out <= 0 || n <= 0)
    return set_err(c, GPTQ_ERR_INVALID_ARG, "null pointer or empty layer");
  if (n % 16 || ldx % 8 || ((uintptr_t)X & 15) || ((uintptr_t)Xq & 15) || tokens <= 0)
    return set_err(c, GPTQ_ERR_UNSUPPORTED,
                   "quantised-input target needs n % 16 == 0, 16-byte aligned rows of X and Xq, tokens > 0");
  if (!std::isfinite(lam_abs) || !std::isfinite(lam_rel)) return set_err(c, GPTQ_ERR_INVALID_ARG, "non-finite damping");
  obj[0] = obj[1] = 0.0;
  DeviceGuard g(c->device);
  const size_t nn = (size_t)n * n, on = (size_t)out * n;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t oH = take(nn * 4), oG = take(nn * 4), oU = take(nn * 4), oWd = take(on * 8), oGd = take(nn * 8),
               oUd = take(nn * 8), oUt = take(nn * 8), oT1 = take(on * 8), oT2 = take(on * 8),
               oWs = take(Wt ? 0 : on * 4);
  if ((rc = ensure(c, c->qr, off))) return rc;
  uint8_t* base = (uint8_t*)c->qr.p;
  float *Hq = (float*)(base + oH), *G = (float*)(base + oG), *U = (float*)(base + oU);
  double *Wd = (double*)(base + oWd), *Gd = (double*)(base + oGd), *Ud = (double*)(base + oUd),
         *UdT = (double*)(base + oUt), *T1 = (double*)(base + oT1), *T2 = (double*)(base + oT2);
  float* Ws = Wt ? Wt : (float*)(base + oWs);
  // Hq = Xq^T Xq and G = Xq^T X in one grouped Hessian launch
  std::vector<HessJob> hj{HessJob{Xq, tokens, ldx, n, Hq, 0}, HessJob{Xq, tokens, ldx, n, G, 0}};
  hj[1].Y = X;
  if ((rc = run_hessian(c, hj))) return rc;
  if ((rc = ensure(c, c->slots, sizeof(Slot)))) return rc;
  Slot* ds = (Slot*)c->slots.p;
  if ((rc = run_factor(c, {FacJob{Hq, n, n, n, lam_abs, lam_rel, U}}, ds))) return rc;
  // W* = ((W (G + lam I)^T) U^T) U in fp64
  LAUNCH(c, "k_qr_prep", launch_qr_prep(W, G, U, &ds->lam, out, n, Wd, Gd, Ud, UdT, c->stream));
  if ((rc = run_gemm_nt(c, Wd, Gd, T1, out, n, n, n))) return rc;
  if ((rc = run_gemm_nt(c, T1, Ud, T2, out, n, n, n, 1))) return rc;   // T1 U^T: U upper
  if ((rc = run_gemm_nt(c, T2, UdT, Wd, out, n, n, n, 2))) return rc;  // T2 U = T2 (U^T)^T: U^T lower
  LAUNCH(c, "k_qr_out", launch_qr_out(Wd, Ws, (long long)on, c->stream));
  QuantJob J{Ws, out, n, n, U, bits, group, block, codes, scales, zeros, nullptr, &ds->lam, ds->obj, nullptr};
  if ((rc = run_quantize(c, {J}))) return rc;
  if ((rc = ensure_small(c, sizeof(Slot)))) return rc;
  HIPCHK(c, hipMemcpyAsync(c->hsmall, ds, sizeof(Slot), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  const Slot s = *(const Slot*)c->hsmall;
  if (s.nonfinite) return set_err(c, GPTQ_ERR_NONFINITE, "non-finite entry in the quantised-input Gram");
  if (info) *info = s.info;
  if (s.info) return set_err(c, GPTQ_ERR_NOT_PD, "damped quantised-input Gram not positive definite");
  obj[0] = s.obj[0];
  obj[1] = s.obj[1];
  return GPTQ_OK;
}

GPTQ_API int gptq_lora(gptq_ctx c, const float* W, int32_t out, int32_t n, const uint16_t* X,
                       int64_t tokens, int64_t ldx, int32_t r, int32_t bits, int32_t group,
                       int32_t block, double lam_abs, double lam_rel, uint8_t* codes, float* scales,
                       uint8_t* zeros, float* L, float* R, double* obj, int32_t* info) {
  return lora_impl(c, W, out, n, X, tokens, ldx, r, bits, group, block, lam_abs, lam_rel, 0, codes, scales, zeros,
                   L, R, obj, info);
}

GPTQ_API int gptq_lora_refine(gptq_ctx c, const float* W, int32_t out, int32_t n, const uint16_t* X,
                              int64_t tokens, int64_t ldx, int32_t r, int32_t bits, int32_t group,
                              int32_t block, double lam_abs, double lam_rel, int32_t rounds, uint8_t* codes,
                              float* scales, uint8_t* zeros, float* L, float* R, double* trace, int32_t* info) {
  if (rounds < 1) return set_err(c, GPTQ_ERR_INVALID_ARG, "rounds must be at least 1");
  return lora_impl(c, W, out, n, X, tokens, ldx, r, bits, group, block, lam_abs, lam_rel, rounds, codes, scales,
                   zeros, L, R, trace, info);
}

GPTQ_API int gptq_hessian64(gptq_ctx c, const uint16_t* X, int64_t tokens, int32_t n, int64_t ldx, double* H) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  int rc = check_x(c, X, tokens, n, ldx);
  if (rc) return rc;
  if (n > 0 && !H) return set_err(c, GPTQ_ERR_INVALID_ARG, "H is null");
  if (n == 0) return GPTQ_OK;
  DeviceGuard g(c->device);
  return run_hessian64(c, X, tokens, ldx, n, H);
}

GPTQ_API int gptq_olrc(gptq_ctx c, const float* W, int32_t out, int32_t n, const double* H, int32_t r,
                       int32_t bits, int32_t group, const uint8_t* codes, const float* scales,
                       const uint8_t* zeros, float* L, float* R, double* J) {
  return refine_step(c, false, W, out, n, H, r, bits, group, 128, (uint8_t*)codes, (float*)scales,
                     (uint8_t*)zeros, L, R, J);
}

GPTQ_API int gptq_bid_up(gptq_ctx c, const float* W, int32_t out, int32_t n, const double* H, int32_t r,
                         const float* L, const float* R, int32_t bits, int32_t group, int32_t block,
                         uint8_t* codes, const float* scales, const uint8_t* zeros, double* J) {
  return refine_step(c, true, W, out, n, H, r, bits, group, block, codes, (float*)scales, (uint8_t*)zeros,
                     (float*)L, (float*)R, J);
}

// ------------------------------------------------------ deployable outputs --
GPTQ_API int gptq_pack_codes(gptq_ctx c, const uint8_t* codes, int32_t rows, int32_t n, int32_t bits,
                             uint32_t* packed) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (rows < 0 || n < 0 || bits < 1 || bits > 8) return set_err(c, GPTQ_ERR_INVALID_ARG, "bad packing arguments");
  if ((int64_t)n * bits > INT32_MAX - 32) return set_err(c, GPTQ_ERR_UNSUPPORTED, "row too long to pack");
  if (rows == 0 || n == 0) return GPTQ_OK;
  if (!codes || !packed) return set_err(c, GPTQ_ERR_INVALID_ARG, "null buffer");
  DeviceGuard g(c->device);
  LAUNCH(c, "k_pack", launch_pack(codes, rows, n, bits, packed, c->stream));
  return GPTQ_OK;
}

GPTQ_API int gptq_unpack_codes(gptq_ctx c, const uint32_t* packed, int32_t rows, int32_t n, int32_t bits,
                               uint8_t* codes) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (rows < 0 || n < 0 || bits < 1 || bits > 8) return set_err(c, GPTQ_ERR_INVALID_ARG, "bad packing arguments");
  if ((int64_t)n * bits > INT32_MAX - 32) return set_err(c, GPTQ_ERR_UNSUPPORTED, "row too long to pack");
  if (rows == 0 || n == 0) return GPTQ_OK;
  if (!codes || !packed) return set_err(c, GPTQ_ERR_INVALID_ARG, "null buffer");
  DeviceGuard g(c->device);
  LAUNCH(c, "k_unpack", launch_unpack(packed, rows, n, bits, codes, c->stream));
  return GPTQ_OK;
}

GPTQ_API int gptq_quantize_lowrank(gptq_ctx c, const float* L, const float* R, int32_t n, int32_t r, int32_t out,
                                   int32_t bits_L, int32_t bits_R, uint8_t* Lcodes, float* Lscales, uint8_t* Lzeros,
                                   float* Lhat, uint8_t* Rcodes, float* Rscales, uint8_t* Rzeros, float* Rhat) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (n < 0 || r < 0 || out < 0 || bits_L < 2 || bits_L > 8 || bits_R < 2 || bits_R > 8)
    return set_err(c, GPTQ_ERR_INVALID_ARG, "bad low-rank quantisation arguments");
  if (r == 0) return GPTQ_OK;
  if (n == 0 || out == 0) return set_err(c, GPTQ_ERR_INVALID_ARG, "empty factor with r > 0");
  if (!L || !R || !Lcodes || !Lscales || !Lzeros || !Rcodes || !Rscales || !Rzeros)
    return set_err(c, GPTQ_ERR_INVALID_ARG, "null buffer");
  DeviceGuard g(c->device);
  LrProb p{L, R, Lcodes, Lscales, Lzeros, Lhat, Rcodes, Rscales, Rzeros, Rhat, n, r, out, (1 << bits_L) - 1,
           (1 << bits_R) - 1, 0};
  LAUNCH(c, "k_lr_quant", launch_lr_quant(p, c->stream));
  return GPTQ_OK;
}

static int gemm_wq(gptq_ctx c, const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* packed,
                   const float* scales, const uint8_t* zeros, int32_t N, int32_t K, int32_t group, int32_t bits,
                   float* Y, int64_t ldy) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (M < 0 || N < 0 || K < 0 || group < 0) return set_err(c, GPTQ_ERR_INVALID_ARG, "negative size");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "the product takes codes of 2, 3, 4 or 8 bits");
  if (M > INT32_MAX - 512) return set_err(c, GPTQ_ERR_UNSUPPORTED, "M too large");
  if (M == 0 || N == 0) return GPTQ_OK;
  if (!Y || (K > 0 && (!X || !packed || !scales || !zeros))) return set_err(c, GPTQ_ERR_INVALID_ARG, "null buffer");
  if (ldx < K || ldy < N) return set_err(c, GPTQ_ERR_INVALID_ARG, "pitch smaller than the row");
  if (K == 0) {  // an empty sum: Y = 0 (the other operands are not read)
    DeviceGuard g(c->device);
    HIPCHK(c, hipMemset2DAsync(Y, (size_t)ldy * sizeof(float), 0, (size_t)N * sizeof(float), (size_t)M, c->stream));
    return GPTQ_OK;
  }
  if (K % 32 != 0 || ldx % 8 != 0 || ((uintptr_t)X & 15) != 0 || ((uintptr_t)packed & 15) != 0)
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "the product needs K %% 32 == 0 and 16-byte aligned rows of X and codes");
  if ((long long)cdiv64(M, 256) * cdiv64(N, 128) > INT32_MAX)
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "product too large for one launch");
  int gshift = 31;
  if (group != 0 && group != K) {
    if (group < 8 || (group & (group - 1)) != 0 || K % group != 0)
      return set_err(c, GPTQ_ERR_UNSUPPORTED, "the product needs group 0 or a power of two >= 8 dividing K");
    gshift = __builtin_ctz((unsigned)group);
  }
  DeviceGuard g(c->device);
  W4Prob p{};
  p.X = X;
  p.P = packed;
  p.S = scales;
  p.Z = zeros;
  p.Y = Y;
  p.ldx = ldx;
  p.ldy = ldy;
  p.M = (int)M;
  p.N = N;
  p.K = K;
  p.G = gshift == 31 ? 1 : K / group;
  p.gshift = gshift;
  if (M <= 128) {  // decode-sized: split K over 16 x 16 blocks, bound by reading the codes
    LAUNCH(c, bits == 4 ? "k_gemv_w4a16" : "k_gemv_wqa16", launch_gemv_w4a16(p, bits, c->stream));
    return GPTQ_OK;
  }
  // 512-row tiles (8 waves: each dequantised code tile feeds twice the
  // MFMAs) once X has more than 256 rows, else 256 x 128 (4 waves)
  LAUNCH(c, bits == 4 ? "k_gemm_w4a16" : "k_gemm_wqa16", launch_gemm_w4a16(p, M > 256 ? 1 : 0, bits, c->stream));
  return GPTQ_OK;
}

GPTQ_API int gptq_gemm_w4a16(gptq_ctx c, const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* packed,
                             const float* scales, const uint8_t* zeros, int32_t N, int32_t K, int32_t group,
                             float* Y, int64_t ldy) {
  return gemm_wq(c, X, M, ldx, packed, scales, zeros, N, K, group, 4, Y, ldy);
}

GPTQ_API int gptq_gemm_wqa16(gptq_ctx c, const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* packed,
                             const float* scales, const uint8_t* zeros, int32_t N, int32_t K, int32_t group,
                             int32_t bits, float* Y, int64_t ldy) {
  return gemm_wq(c, X, M, ldx, packed, scales, zeros, N, K, group, bits, Y, ldy);
}
