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
constexpr size_t NA_EB = (size_t)2 * NA_MAX_OUT * 512 * sizeof(float);
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

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
inline long long cdiv64(long long a, long long b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ Hessian plan --
struct HessJob {
  const uint16_t* X;
  long long tokens, ldx;
  int n;
  float* H;
  int accumulate;
  // non-null: the cross Gram X^T Y (Y as X: [tokens][ldx]; direct layout
  // only), written in full
  const uint16_t* Y = nullptr;
};

struct HessPlan {
  std::vector<XposeProb> xprobs;
  std::vector<Seg> xsegs;
  std::vector<SyrkProb> probs;
  std::vector<SyrkTask> tasks;
  std::vector<RedProb> rprobs;
  std::vector<RedTask> rtasks;
  std::vector<int> partlist;
  int nparts = 0;
};

// The tiles can read X directly (no transposed copy) when its rows are
// 16-byte aligned and n is a multiple of 8 (16-byte feature chunks never
// cross the end of a row).  A stage's per-lane byte offsets (32 rows of the
// pitch) are 32-bit, which bounds the pitch.
static bool hess_direct(const HessJob& J) {
  return J.tokens > 0 && (J.ldx % 8) == 0 && (((uintptr_t)J.X) & 15) == 0 && (J.n % 8) == 0 &&
         J.ldx < (1LL << 25);
}

// Interleaved bit order of (i, j): tiles close in this order share rows of X.
static int morton2(int i, int j) {
  int m = 0;
  for (int b = 0; b < 10; ++b) m |= (((i >> b) & 1) << (2 * b + 1)) | (((j >> b) & 1) << (2 * b));
  return m;
}

// Number of token slices for one layer's tiles: whole rounds of the chip at
// one tile per CU, each task also paying for writing its partial (about ten
// 32-token steps of time).  Depends on the layer alone.
static int hess_slices(int ntile, long long chunks, int ncu) {
  int best_s = 1;
  long long best = -1;
  for (int s = 1; s <= 64 && s <= std::max(1LL, chunks); ++s) {
    const long long rounds = cdiv((long long)ntile * s, (long long)ncu);
    const long long cost = rounds * (cdiv(chunks, (long long)s) + 10);
    if (best < 0 || cost < best) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

// Tasks of every layer: its upper 256x256 tiles times S token slices, slice
// by slice, so that the whole chip streams one window of tokens at a time and
// re-reads of X hit the L2/MALL.  Inside a slice the tiles go in Morton order,
// cut into 8 groups that are dealt out in turn: consecutive workgroups land
// on the 8 XCDs in turn, so each XCD works on one compact group of tiles that
// shares rows of X in its own L2.  The cut points of a layer depend on that
// layer alone, so a layer gets the same bits alone or in a batch.  The rows of
// the transposed copy are padded by 256 tokens so that rows at the same token
// offset spread over the L2 channels.
void plan_hessian(const std::vector<HessJob>& jobs, int ncu, int nxcd, uint16_t* xt, HessPlan& P) {
  for (size_t p = 0; p < jobs.size(); ++p) {
    const HessJob& J = jobs[p];
    const int vec = (J.ldx % 8 == 0) && (((uintptr_t)J.X & 15) == 0);
    const int nt = cdiv(J.n, 256);
    const long long chunks = cdiv(J.tokens, 64);
    const int n_pad = nt * 256, t_pad = (int)(chunks * 64);
    if (hess_direct(J)) {
      // the tiles read X itself (transposing LDS reads); no copy
      P.xprobs.push_back(XposeProb{J.X, J.ldx, nullptr, J.n, (int)J.tokens, n_pad, t_pad, vec, 0});
      P.probs.push_back(SyrkProb{J.X, J.ldx, 1, (int)J.tokens, J.n, 0, J.Y});
    } else {
      const int ldt = t_pad > 0 ? t_pad + 256 : 0;
      P.xprobs.push_back(XposeProb{J.X, J.ldx, xt, J.n, (int)J.tokens, n_pad, t_pad, vec, ldt});
      if (t_pad > 0) P.xsegs.push_back(Seg{(int)p, 0, (t_pad / 64) * (n_pad / 64), 0, 0, 0, 0, 0});
      P.probs.push_back(SyrkProb{xt, ldt, 0, (int)J.tokens, J.n, 0, nullptr});
      xt += (size_t)n_pad * ldt;
    }
    const bool full = J.Y != nullptr;
    P.rprobs.push_back(RedProb{J.H, J.n, J.accumulate, full ? 1 : 0, 0});
    if (J.n <= 0) continue;
    std::vector<std::pair<int, int>> tl;  // upper tiles, or every tile of a cross Gram
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = full ? 0 : ti; tj < nt; ++tj) tl.push_back({ti, tj});
    const int ntile = (int)tl.size();
    if (J.tokens > 0) {
      std::vector<std::pair<int, int>> mo = tl;
      std::stable_sort(mo.begin(), mo.end(), [](const std::pair<int, int>& x, const std::pair<int, int>& y) {
        return morton2(x.first, x.second) < morton2(y.first, y.second);
      });
      std::vector<int> ord;  // dealt order, indices into mo
      const int G = std::max(1, std::min(nxcd, ntile)), base = ntile / G, rem = ntile % G;
      for (int idx = 0; idx <= base; ++idx)
        for (int g = 0; g < G; ++g)
          if (idx < base + (g < rem ? 1 : 0)) ord.push_back(g * base + std::min(g, rem) + idx);
      const long long c32 = t_pad / 32;
      const int S = hess_slices(ntile, c32, ncu);
      const int first = (int)P.tasks.size();
      std::vector<int> pos(ntile);  // tile (canonical index) -> position inside a slice
      for (int q = 0; q < ntile; ++q) {
        const std::pair<int, int> t = mo[ord[q]];
        const int ci = full ? t.first * nt + t.second
                            : t.first * nt - t.first * (t.first - 1) / 2 + (t.second - t.first);
        pos[ci] = q;
      }
      for (int sl = 0; sl < S; ++sl) {
        const int k0 = (int)(32 * (c32 * sl / S)), k1 = (int)(32 * (c32 * (sl + 1) / S));
        for (int q = 0; q < ntile; ++q) {
          const std::pair<int, int> t = mo[ord[q]];
          P.tasks.push_back(SyrkTask{(int)p, t.first, t.second, k0, k1, (int)P.tasks.size(), 0, 0});
        }
      }
      for (int ci = 0; ci < ntile; ++ci) {
        const int ti = tl[ci].first, tj = tl[ci].second;
        const int part0 = (int)P.partlist.size();
        for (int sl = 0; sl < S; ++sl) P.partlist.push_back(first + sl * ntile + pos[ci]);
        for (int a = 0; a < 4; ++a)
          for (int b = 0; b < 4; ++b) {
            if (ti == tj && a > b && !full) continue;
            const int r0 = ti * 256 + 64 * a, c0 = tj * 256 + 64 * b;
            if (r0 >= J.n || c0 >= J.n) continue;
            P.rtasks.push_back(RedTask{(int)p, r0, c0, part0, S, 0, 0, 0});
          }
      }
    } else {
      // no tokens: every sub-block sums zero partials (H = 0, or H unchanged)
      for (int ci = 0; ci < ntile; ++ci) {
        const int ti = tl[ci].first, tj = tl[ci].second;
        for (int a = 0; a < 4; ++a)
          for (int b = 0; b < 4; ++b) {
            const int r0 = ti * 256 + 64 * a, c0 = tj * 256 + 64 * b;
            if ((ti == tj && a > b && !full) || r0 >= J.n || c0 >= J.n) continue;
            P.rtasks.push_back(RedTask{(int)p, r0, c0, 0, 0, 0, 0, 0});
          }
      }
    }
  }
  P.nparts = (int)P.tasks.size();
}

int run_hessian(gptq_ctx c, const std::vector<HessJob>& jobs) {
  size_t xt_elems = 0;
  for (const HessJob& J : jobs)
    if (J.tokens > 0 && !hess_direct(J)) xt_elems += (size_t)cdiv(J.n, 256) * 256 * ((size_t)cdiv(J.tokens, 64) * 64 + 256);
  int rc = ensure(c, c->xt, xt_elems * sizeof(uint16_t));
  if (rc) return rc;
  HessPlan P;
  plan_hessian(jobs, c->ncu, c->nxcd, (uint16_t*)c->xt.p, P);
  if ((rc = ensure(c, c->partials, (size_t)std::max(P.nparts, 1) * 65536 * sizeof(float)))) return rc;
  int nxwg = 0;
  for (auto& sg : P.xsegs) {
    sg.wg0 = nxwg;
    nxwg += sg.nwg;
  }
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
  const int nt = cdiv(n, 128);
  const int ntile = nt * (nt + 1) / 2;
  const long long chunks = t_pad / 32;
  // slices: minimise rounds x slice length
  int S = 1;
  long long best = -1;
  for (int k = 1; k <= 64 && k <= std::max(1LL, chunks); ++k) {
    const long long rounds = cdiv((long long)ntile * k, (long long)c->ncu);
    const long long cost = rounds * cdiv(chunks, (long long)k);
    if (best < 0 || cost < best) {
      best = cost;
      S = k;
    }
  }
  std::vector<SyrkTask> tasks;
  std::vector<int> partlist;
  std::vector<RedTask> rtasks;
  if (chunks > 0) {
    for (int sl = 0; sl < S; ++sl) {
      const int k0 = (int)(32 * (chunks * sl / S)), k1 = (int)(32 * (chunks * (sl + 1) / S));
      int t = 0;
      for (int ti = 0; ti < nt; ++ti)
        for (int tj = ti; tj < nt; ++tj, ++t) tasks.push_back(SyrkTask{0, ti, tj, k0, k1, (int)tasks.size(), 0, 0});
    }
    int t = 0;
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = ti; tj < nt; ++tj, ++t) {
        const int part0 = (int)partlist.size();
        for (int sl = 0; sl < S; ++sl) partlist.push_back(sl * ntile + t);
        for (int a = 0; a < 2; ++a)
          for (int b = 0; b < 2; ++b) {
            if (ti == tj && a > b) continue;
            const int r0 = ti * 128 + 64 * a, c0 = tj * 128 + 64 * b;
            if (r0 >= n || c0 >= n) continue;
            rtasks.push_back(RedTask{0, r0, c0, part0, S, 0, 0, 0});
          }
      }
  } else {
    // no tokens: H = 0 (every sub-block sums zero partials)
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = ti; tj < nt; ++tj)
        for (int a = 0; a < 2; ++a)
          for (int b = 0; b < 2; ++b) {
            const int r0 = ti * 128 + 64 * a, c0 = tj * 128 + 64 * b;
            if ((ti == tj && a > b) || r0 >= n || c0 >= n) continue;
            rtasks.push_back(RedTask{0, r0, c0, 0, 0, 0, 0, 0});
          }
  }
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
  if ((rc = ensure(c, c->facY, totA * sizeof(double)))) return rc;
  std::vector<FacProb> probs(np);
  int maxnb = 0, maxn = 0;
  for (int p = 0; p < np; ++p) {
    const FacJob& J = jobs[p];
    FacProb f;
    f.H = J.H;
    f.A = (double*)c->facA.p + oA[p];
    f.Y = (double*)c->facY.p + oA[p];
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
    maxnb = std::max(maxnb, cdiv(J.n, 64));
    maxn = std::max(maxn, J.n);
    if (A_out) A_out[p] = f.A;
  }
  Blob b;
  const size_t o_probs = b.add(probs);
  struct L {
    int kind;  // 0 fill, 1 panel, 2 gemm (general, 64 tiles), 3 ring gemm 64, 4 ring gemm 128, 5 makeu,
               // 6 fork (side stream waits for the main stream), 7 join (main waits for the side stream),
               // 8 panel pair
    bool side;  // launch on the side stream
    size_t off;
    int nseg, nwg;
  };
  std::vector<L> launches;
  auto add_launch = [&](int kind, std::vector<Seg>& segs, bool side = false) {
    int nwg = 0;
    for (auto& s : segs) {
      s.wg0 = nwg;
      nwg += s.nwg;
    }
    if (nwg == 0) return;
    launches.push_back(L{kind, side, b.add(segs), (int)segs.size(), nwg});
  };
  auto add_sync = [&](int kind) { launches.push_back(L{kind, false, 0, 0, 0}); };
  // The ring-staged products need every K range and row pitch to be a
  // multiple of 64 (16-byte aligned chunks of 16 doubles).
  bool ring = true;
  for (const FacJob& J : jobs) ring = ring && (J.n % 64) == 0;
  {
    std::vector<Seg> s;
    for (int p = 0; p < np; ++p)
      if (jobs[p].H) s.push_back(Seg{p, 0, cdiv(jobs[p].n, 4), 0, 0, 0, 0, 0});
    add_launch(0, s);
  }
  // Cholesky and Y = L^{-1}: outer panels of 256 columns, four 64-column
  // steps each.  Step k: the panel launch (every 64-block of the problem),
  // then the updates of the rest of the outer panel (L columns [c0, P1) of
  // every row below; Y rows [c0, P1)).  At the end of an outer panel the
  // trailing updates with K = P1 - P0 split in two: the part the next outer
  // panel reads (L columns [P1, S), S = P1 + 256; Y rows [P1, S)) on the main
  // stream, and the rest (L's trailing triangle from S on; Y rows from S on)
  // on the side stream, where it overlaps the next outer panel's steps (which
  // neither read nor write it) and is joined before the next outer update.
  // With the general products (n % 64 != 0) everything stays on one stream.
  bool side_busy = false;
  // Steps go in pairs (k, k+1) inside an outer panel: one launch of
  // k_chol_panel2 (kind 8) does both; a last block without a partner takes
  // the single-step k_chol_panel.
  for (int k = 0; k < maxnb; k += 2) {
    std::vector<Seg> pan, pan2, inner, crit, bulk;
    int bulk_rows = 0;
    for (int p = 0; p < np; ++p) {
      const int n = jobs[p].n, nb = cdiv(n, 64);
      if (k >= nb) continue;
      const bool pair = k + 1 < nb;
      (pair ? pan2 : pan).push_back(Seg{p, 0, nb, k, 0, 0, 0, 0});
      const int k0 = 64 * k, pw = std::min(pair ? 128 : 64, n - k0);
      const int P0 = (k0 / 256) * 256, P1 = std::min(P0 + 256, n);
      const int c0 = k0 + pw;
      if (c0 < P1) {  // rest of the outer panel
        const int nrow = cdiv(n - c0, 64), ncol = cdiv(P1 - c0, 64);
        inner.push_back(Seg{p, 0, ncol * nrow - ncol * (ncol - 1) / 2, GK_CHOL_TRAIL, k0, pw, c0, P1});
        inner.push_back(Seg{p, 0, cdiv(P1 - c0, 64) * cdiv(c0, 64), GK_ZUPD, k0, pw, c0, P1});
      } else if (P1 < n) {  // end of the outer panel: trailing updates with K = P1 - P0
        const int S = ring ? std::min(P1 + 256, n) : n;
        {
          const int nrow = cdiv(n - P1, 64), ncol = cdiv(S - P1, 64);
          crit.push_back(Seg{p, 0, ncol * nrow - ncol * (ncol - 1) / 2, GK_CHOL_TRAIL, P0, P1 - P0, P1, S});
          crit.push_back(Seg{p, 0, cdiv(S - P1, 64) * cdiv(P1, 64), GK_ZUPD, P0, P1 - P0, P1, S});
        }
        if (S < n) {
          const int m = cdiv(n - S, 128);
          bulk.push_back(Seg{p, 0, m * (m + 1) / 2, GK_CHOL_TRAIL, P0, P1 - P0, S, n});
          bulk.push_back(Seg{p, 0, m * cdiv(P1, 128), GK_ZUPD, P0, P1 - P0, S, n});
          bulk_rows = std::max(bulk_rows, n - S);
        }
      }
    }
    add_launch(8, pan2);
    add_launch(1, pan);
    add_launch(ring ? 3 : 2, inner);
    if (!crit.empty()) {
      if (side_busy) add_sync(7);  // the previous bulk update touches the columns updated now
      side_busy = false;
      if (!bulk.empty()) {
        if (bulk_rows < 1024) {  // small: 64-wide tiles, on the main stream
          for (Seg& sg : bulk) {
            const int n = jobs[sg.prob].n, m = cdiv(n - sg.d, 64);
            sg.nwg = (sg.a == GK_CHOL_TRAIL) ? m * (m + 1) / 2 : m * cdiv(sg.b + sg.c, 64);
          }
          for (Seg& sg : bulk) crit.push_back(sg);
        } else {
          add_sync(6);
          add_launch(4, bulk, true);
          side_busy = true;
        }
      }
      add_launch(ring ? 3 : 2, crit);
    }
  }
  if (side_busy) add_sync(7);
  {
    std::vector<Seg> s;
    for (int p = 0; p < np; ++p) s.push_back(Seg{p, 0, cdiv(jobs[p].n, 4), 0, 0, 0, 0, 0});
    add_launch(5, s);
  }
  uint8_t* d = nullptr;
  if ((rc = upload(c, b, &d))) return rc;
  const FacProb* dp = (const FacProb*)(d + o_probs);
  LAUNCH(c, "k_damp_lambda", launch_damp_lambda(dp, np, c->stream));
  // the side stream's updates take at most this many CUs (one workgroup per
  // CU, whose registers fill the CU), leaving about 96 to the serial chain:
  // the 64 panel workgroups of a 4096-wide problem and its narrow updates
  // (measured best at n = 4096 among caps of 128 to 256 CUs)
  const int side_wg = std::max(1, c->ncu - std::min(96, c->ncu / 2));
  for (const L& l : launches) {
    const Seg* sg = (const Seg*)(d + l.off);
    hipStream_t st = l.side ? c->side : c->stream;
    switch (l.kind) {
      case 0: LAUNCH(c, "k_damp_fill", launch_damp_fill(dp, sg, l.nseg, l.nwg, c->stream)); break;
      case 1: LAUNCH(c, "k_chol_panel", launch_chol_panel(dp, sg, l.nseg, l.nwg, c->stream)); break;
      case 8: LAUNCH(c, "k_chol_panel2", launch_chol_panel2(dp, sg, l.nseg, l.nwg, c->stream)); break;
      case 2: LAUNCH(c, "k_gemm64", launch_gemm64(dp, sg, l.nseg, l.nwg, c->stream)); break;
      case 3: LAUNCH_ON(c, st, "k_gemm_ring64", launch_gemm_ring(64, dp, sg, l.nseg, l.nwg, 0, st)); break;
      case 4:
        LAUNCH_ON(c, st, "k_gemm_ring128", launch_gemm_ring(128, dp, sg, l.nseg, l.nwg, l.side ? side_wg : 0, st));
        break;
      case 5: LAUNCH(c, "k_make_u", launch_make_u(dp, sg, l.nseg, l.nwg, c->stream)); break;
      case 6:
        HIPCHK(c, hipEventRecord(c->fork_ev, c->stream));
        HIPCHK(c, hipStreamWaitEvent(c->side, c->fork_ev, 0));
        break;
      case 7:
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
  // Super-blocks: each block's errors reach the rest of its super-block right
  // away, the columns past it only at the super-block's end (one product with
  // K = the super-block width), so the far columns of W are rewritten once
  // per super-block instead of once per block.  Groups must nest in it.
  std::vector<int> sbk(nl);
  size_t totW = 0, totE = 0, totO = 0, totD = 0;
  std::vector<size_t> oW(nl), oE(nl), oO(nl), oD(nl);
  for (int p = 0; p < nl; ++p) {
    const QuantJob& J = jobs[p];
    int sb = std::max(1, 512 / J.block);
    const int sbw = sb * J.block;
    if (J.group && !(sbw % J.group == 0 || J.group % sbw == 0)) sb = 1;
    sbk[p] = sb;
    oW[p] = totW;
    if (!J.Ww_ext) totW += (size_t)J.out * J.nt;
    oE[p] = totE;
    totE += 2 * (size_t)J.out * sb * J.block;  // two super-blocks: one swept while the other's far update runs
    oO[p] = totO;
    totO += (size_t)J.out * 2;
    oD[p] = totD;
    totD += (size_t)(J.nt + 63) / 64 * 64;
  }
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
  int maxblk = 0;
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
    maxblk = std::max(maxblk, q.nblk);
    if (Ww_out) Ww_out->push_back(q.Ww);
  }
  Blob b;
  const size_t o_L = b.add(L);
  struct Lc {
    int kind;  // 0 init, 1 rowfit, 2 sweep, 3 trail, 6 fork, 7 join (as in the factor)
    int block;
    bool side;
    size_t off;
    int nseg, nwg;
    int mode;  // sweeps: 0 GPTQ, 1 Bid-Up
  };
  std::vector<Lc> launches;
  auto add_launch = [&](int kind, int block, std::vector<Seg>& segs, bool side = false, int mode = 0) {
    int nwg = 0;
    for (auto& s : segs) {
      s.wg0 = nwg;
      nwg += s.nwg;
    }
    if (nwg == 0) return;
    launches.push_back(Lc{kind, block, side, b.add(segs), (int)segs.size(), nwg, mode});
  };
  auto add_sync = [&](int kind) { launches.push_back(Lc{kind, 0, false, 0, 0, 0, 0}); };
  {
    std::vector<Seg> s, f;
    for (int p = 0; p < nl; ++p) {
      s.push_back(Seg{p, 0, cdiv(jobs[p].out, 4), 0, 0, 0, 0, 0});
      if (jobs[p].group == 0 && !jobs[p].mode) f.push_back(Seg{p, 0, cdiv(jobs[p].out, 4), 0, 0, 0, 0, 0});
    }
    add_launch(0, 0, s);
    add_launch(1, 0, f);
  }
  std::vector<int> blocks;
  for (auto& J : jobs)
    if (std::find(blocks.begin(), blocks.end(), J.block) == blocks.end()) blocks.push_back(J.block);
  // At a super-block's end, the next super-block's columns are updated on
  // the main stream (its sweeps read them); the columns past it on the side
  // stream, beside the next super-block's sweeps (which neither read nor
  // write them; the errors sit in the other half of the two-super-block
  // buffer), joined before the next far update.  Needs the groups to nest in
  // a super-block (a group fit reads its whole group).
  bool side_busy = false;
  // One sweep launch per super-block (the sweep kernel applies each block's
  // errors to the rest of its super-block itself).
  for (int k = 0; k < maxblk; ++k) {
    for (int B : blocks)
      for (int mode = 0; mode < 2; ++mode) {
        std::vector<Seg> s;
        for (int p = 0; p < nl; ++p)
          if (jobs[p].block == B && jobs[p].mode == mode && k < L[p].nblk && k % sbk[p] == 0)
            s.push_back(Seg{p, 0, cdiv(jobs[p].out, 16), k / sbk[p], 0, 0, 0, 0});
        add_launch(2, B, s, false, mode);
      }
    std::vector<Seg> crit, bulk;  // past the super-block (64 / 128 tiles)
    for (int p = 0; p < nl; ++p) {
      if (k >= L[p].nblk) continue;
      const int B = jobs[p].block, n = jobs[p].n, nt = jobs[p].nt, sb = sbk[p], sbw = sb * B;
      const int b0 = k * B, b1 = std::min(b0 + B, n);
      const int sb0 = (k / sb) * sbw, sb1 = std::min(sb0 + sbw, n);
      const int par = ((k / sb) & 1) * jobs[p].out * L[p].ldE;  // this super-block's half of the error buffer
      if (b1 == sb1 && sb1 < nt) {  // end of the super-block: all columns past it
        const bool nest = jobs[p].group == 0 || sbw % jobs[p].group == 0;
        const int S = nest ? std::min(sb1 + sbw, nt) : nt;
        crit.push_back(Seg{p, 0, cdiv(jobs[p].out, 64) * cdiv(S - sb1, 64), par, sb0, sb1 - sb0, sb1, S});
        if (S < nt) bulk.push_back(Seg{p, 0, cdiv(jobs[p].out, 128) * cdiv(nt - S, 128), par, sb0, sb1 - sb0, S, nt});
      }
    }
    if (!crit.empty()) {
      if (side_busy) add_sync(7);  // the previous far update covers the columns updated now
      side_busy = false;
      if (!bulk.empty()) {
        add_sync(6);
        add_launch(3, 128, bulk, true);
        side_busy = true;
      }
      add_launch(3, 64, crit);
    }
  }
  if (side_busy) add_sync(7);
  uint8_t* d = nullptr;
  if ((rc = na ? upload_noalloc(c, b, na->blob, &d) : upload(c, b, &d))) return rc;
  const QLayer* dL = (const QLayer*)(d + o_L);
  for (const Lc& l : launches) {
    const Seg* sg = (const Seg*)(d + l.off);
    hipStream_t st = l.side ? c->side : c->stream;
    switch (l.kind) {
      case 0: LAUNCH(c, "k_init_work", launch_init_work(dL, sg, l.nseg, l.nwg, c->stream)); break;
      case 1: LAUNCH(c, "k_rowfit", launch_rowfit(dL, sg, l.nseg, l.nwg, c->stream)); break;
      case 2: LAUNCH(c, "k_sweep", launch_sweep(l.block, l.mode, dL, sg, l.nseg, l.nwg, c->stream)); break;
      case 3:  // beside the sweeps: one workgroup per CU, which leaves room on each CU for a sweep's
        LAUNCH_ON(c, st, "k_trail", launch_trail(l.block, dL, sg, l.nseg, l.nwg, l.side ? c->ncu : 0, st));
        break;
      case 6:
        HIPCHK(c, hipEventRecord(c->fork_ev, c->stream));
        HIPCHK(c, hipStreamWaitEvent(c->side, c->fork_ev, 0));
        break;
      case 7:
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

GPTQ_API int gptq_gemm_w4a16(gptq_ctx c, const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* packed,
                             const float* scales, const uint8_t* zeros, int32_t N, int32_t K, int32_t group,
                             float* Y, int64_t ldy) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  c->err.clear();
  if (M < 0 || N < 0 || K < 0 || group < 0) return set_err(c, GPTQ_ERR_INVALID_ARG, "negative size");
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
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "W4A16 needs K %% 32 == 0 and 16-byte aligned rows of X and codes");
  if ((long long)cdiv64(M, 256) * cdiv64(N, 128) > INT32_MAX)
    return set_err(c, GPTQ_ERR_UNSUPPORTED, "W4A16 product too large for one launch");
  int gshift = 31;
  if (group != 0 && group != K) {
    if (group < 8 || (group & (group - 1)) != 0 || K % group != 0)
      return set_err(c, GPTQ_ERR_UNSUPPORTED, "W4A16 needs group 0 or a power of two >= 8 dividing K");
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
    LAUNCH(c, "k_gemv_w4a16", launch_gemv_w4a16(p, c->stream));
    return GPTQ_OK;
  }
  // 512-row tiles (8 waves: each dequantised code tile feeds twice the
  // MFMAs) once X has more than 256 rows, else 256 x 128 (4 waves)
  LAUNCH(c, "k_gemm_w4a16", launch_gemm_w4a16(p, M > 256 ? 1 : 0, c->stream));
  return GPTQ_OK;
}
