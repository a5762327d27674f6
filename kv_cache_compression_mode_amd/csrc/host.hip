// C ABI of the JoLT codec: argument checks, workspace layout, host algorithms
// (counter-based RNG, Haar rotation, Lagrangian-dual allocation) and the
// orchestration of the HIP kernels.  See include/jolt.h for the contract.
#include "../../include/jolt.h"

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "plan.hpp"

using namespace jolt;

// ------------------------------------------------------------- profiling
namespace jolt {
namespace {
struct ProfRec {
  std::vector<std::pair<int, int>> ev;   // indices into the event pool
  double bytes = 0, flops = 0;           // host-side accounting
};
std::mutex g_prof_mu;
std::string g_prof_sel;                  // "" off, "*" every kernel, else ",name,name,"
std::map<std::string, ProfRec> g_prof;
std::vector<hipEvent_t> g_pool;          // created once, reused after every enable
size_t g_pool_used = 0;

int pool_event() {
  if (g_pool_used == g_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    g_pool.push_back(e);
  }
  return static_cast<int>(g_pool_used++);
}

void prof_release() {
  g_prof.clear();
  g_pool_used = 0;
}
}  // namespace

bool prof_enabled(const char* name) {
  if (g_prof_sel.empty()) return false;
  return g_prof_sel == "*" || g_prof_sel.find("," + std::string(name) + ",") != std::string::npos;
}

void prof_add_work(const char* name, double bytes, double flops) {
  if (!prof_enabled(name)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec& r = g_prof[name];
  r.bytes += bytes;
  r.flops += flops;
}

ProfScope::ProfScope(const char* n, hipStream_t s) : name(n), stream(s), e0(-1), e1(-1) {
  if (!prof_enabled(name)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  e0 = pool_event();
  e1 = pool_event();
  if (e0 < 0 || e1 < 0) { e0 = e1 = -1; return; }
  (void)hipEventRecord(g_pool[e0], stream);
}

ProfScope::~ProfScope() {
  if (e0 < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_pool[e1], stream);
  g_prof[name].ev.emplace_back(e0, e1);
}
}  // namespace jolt

namespace {

constexpr uint32_t kMagic = 0x544C4F4Au;      // "JOLT", little-endian
constexpr uint32_t kVersion = 1;
constexpr uint64_t kTagRotation = 0x4A4F4C54524F5431ull;   // "JOLTROT1"
constexpr uint64_t kTagSketch = 0x4A4F4C54534B5431ull;     // "JOLTSKT1"
struct HipFail {};
inline void ck(hipError_t e) {
  if (e != hipSuccess) throw HipFail{};
}


// ------------------------------------------------------------- host RNG
uint64_t mix64h(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

double normal_h(uint64_t key, uint64_t i) {
  const uint64_t k = i >> 1;
  const uint64_t w1 = mix64h(key + (2 * k + 1) * 0x9E3779B97F4A7C15ull);
  const uint64_t w2 = mix64h(key + (2 * k + 2) * 0x9E3779B97F4A7C15ull);
  const double u1 = (static_cast<double>(w1 >> 11) + 0.5) * 0x1p-53;
  const double u2 = (static_cast<double>(w2 >> 11) + 0.5) * 0x1p-53;
  const double rad = std::sqrt(-2.0 * std::log(u1));
  const double ang = 2.0 * 3.141592653589793 * u2;
  return (i & 1) ? rad * std::sin(ang) : rad * std::cos(ang);
}

// Haar rotation: Householder QR (fp64) of the seeded Gaussian matrix, Q with diag(R) > 0.
void rotation_host(uint64_t seed, int D, double* Q) {
  const uint64_t key = mix64h(seed ^ kTagRotation);
  std::vector<double> A(static_cast<size_t>(D) * D), tau(D), sgn(D);
  for (int i = 0; i < D * D; ++i) A[i] = normal_h(key, static_cast<uint64_t>(i));
  auto at = [&](int r, int c) -> double& { return A[static_cast<size_t>(r) * D + c]; };
  for (int j = 0; j < D; ++j) {
    double sigma = 0.0;
    for (int i = j + 1; i < D; ++i) sigma += at(i, j) * at(i, j);
    const double alpha = at(j, j);
    double beta = alpha, t = 0.0;
    if (sigma > 0.0) {
      const double nrm = std::sqrt(alpha * alpha + sigma);
      beta = alpha >= 0.0 ? -nrm : nrm;
      t = (beta - alpha) / beta;
      const double sc = 1.0 / (alpha - beta);
      for (int i = j + 1; i < D; ++i) at(i, j) *= sc;
      for (int c = j + 1; c < D; ++c) {
        double w = at(j, c);
        for (int i = j + 1; i < D; ++i) w += at(i, j) * at(i, c);
        at(j, c) -= t * w;
        for (int i = j + 1; i < D; ++i) at(i, c) -= t * at(i, j) * w;
      }
    }
    tau[j] = t;
    sgn[j] = beta < 0.0 ? -1.0 : 1.0;
    at(j, j) = beta;
  }
  // Q = H_0 ... H_{D-1}: apply reflectors back to front to the identity
  std::vector<double> M(static_cast<size_t>(D) * D, 0.0);
  for (int i = 0; i < D; ++i) M[static_cast<size_t>(i) * D + i] = 1.0;
  for (int j = D - 1; j >= 0; --j) {
    if (tau[j] == 0.0) continue;
    for (int c = 0; c < D; ++c) {
      double w = M[static_cast<size_t>(j) * D + c];
      for (int i = j + 1; i < D; ++i) w += at(i, j) * M[static_cast<size_t>(i) * D + c];
      M[static_cast<size_t>(j) * D + c] -= tau[j] * w;
      for (int i = j + 1; i < D; ++i) M[static_cast<size_t>(i) * D + c] -= tau[j] * at(i, j) * w;
    }
  }
  for (int r = 0; r < D; ++r)
    for (int c = 0; c < D; ++c) Q[static_cast<size_t>(r) * D + c] = M[static_cast<size_t>(r) * D + c] * sgn[c];
}


// The head of a record: header words and the padding after each section.
RecordHead record_head(int64_t H, int64_t T, int64_t D, int32_t dtype, jolt_choice c, uint64_t seed) {
  const BlobLayout L = blob_layout(H, T, D, c);
  RecordHead h{};
  const uint32_t w[16] = {kMagic, kVersion, static_cast<uint32_t>(H), static_cast<uint32_t>(T),
                          static_cast<uint32_t>(D), static_cast<uint32_t>(dtype),
                          static_cast<uint32_t>(c.r_T), static_cast<uint32_t>(c.r_D),
                          static_cast<uint32_t>(c.bits), static_cast<uint32_t>(kGroup),
                          static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), 0, 0, 0, 0};
  std::memcpy(h.w, w, sizeof(w));
  const size_t groups = static_cast<size_t>(H * T * D / kGroup);
  const size_t ends[5] = {L.ut + 2ull * T * c.r_T, L.ud + 2ull * D * c.r_D, L.g + 2ull * H * c.r_T * c.r_D,
                          L.sc + 4ull * groups, L.cd + 4ull * c.bits * groups};
  const size_t next[5] = {L.ud, L.g, L.sc, L.cd, L.total};
  for (int j = 0; j < 5; ++j) {
    h.pad[2 * j] = static_cast<uint32_t>(ends[j]);
    h.pad[2 * j + 1] = static_cast<uint32_t>(next[j] - ends[j]);
  }
  return h;
}

// --------------------------------------------------- allocate workspace
struct Carver {
  size_t off = 0;
  char* base = nullptr;
  template <typename T> T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += a256(count * sizeof(T));
    return p;
  }
};

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

struct AllocWS {
  // persistent
  float* UT; float* UD; double* lamT; double* lamD; double* frob2;
  const void** xptrs; uint64_t* tags;
  int* status;         // device word: bit 0 set when a bounded wait of the eigensolver gave up
  bool x16;            // every input tensor is 16-byte aligned
  // scratch (chunk tensors)
  float* G; float* V;
  float* GDpart;
  void* syev;
  void* syevD;
  float* GD; float* GDc;
  float* Ucm; float* Vr; float* P; double* lam_tmp; float* qtau; int* perm; float* sgn;
  float* Om; float* Y; float* Z; float* Bm; float* Wr; float* Wd;
  // the feature-mode factor's own scratch (it runs beside the token path)
  float* qtauD; double* lamDt; int* permD; float* sgnD;
  // CholeskyQR: a second buffer of the token factor and of the feature factor, and their work
  float* Ucm2; float* cq; float* Vr2; float* cqD;
  bool householder;    // re-orthonormalize by Householder QR only (after a CholeskyQR breakdown)
  size_t bytes;
  int chunk;
  int nlanes;          // scratch sets, one per stream (chunks alternate between them)
  hipEvent_t band_done;  // recorded once the token eigensolver's band reduction is queued
  // early read-back (exact path, one chunk): the token eigenvalues, feature
  // spectra and ||X||^2 copied to this pinned host buffer ([batch][R] | [batch][D]
  // | [batch]) as soon as they are final, early_done recorded after the copies
  double* early; hipEvent_t eig_done, early_done;
};

struct Dims {
  int64_t H, T, D, HD, nT, R, n_pad, ell, ell_pad;
  bool dual, flash;
};

// Split-K factor of the feature Gram sum_h X_h^T X_h when it is one product
// over K = H * T rows (direct and randomized paths): chunks of about 4096
// rows keep every fp32 accumulation short, and the partial sums are added in
// a fixed order.  The dual path gets it from the token Gram's diagonal blocks.
int gram_d_ksplit(const Dims& d) {
  if (d.dual && !d.flash) return 1;
  const int64_t K = d.H * d.T;
  return static_cast<int>(std::min<int64_t>(32, std::max<int64_t>(1, (K + 4095) / 4096)));
}

Dims dims_of(const jolt_alloc_req* r) {
  Dims d{};
  d.H = r->shape.H; d.T = r->shape.T; d.D = r->shape.D; d.HD = d.H * d.D;
  d.nT = std::min(d.T, d.HD);
  d.R = cap_of(r);
  d.flash = r->method == JOLT_FLASH;
  d.dual = d.T > d.HD;
  d.n_pad = pad64(d.nT);
  d.ell = std::min<int64_t>(d.R + r->oversample, d.nT);
  d.ell_pad = pad64(d.ell);
  return d;
}

// Persistent outputs, the pointer and tag arrays of every tensor, then one
// or two sets of chunk scratch (lanes): with two, consecutive chunks of half
// the size alternate between two streams, so one chunk's single-CU-per-tensor
// chase overlaps the other's matrix-core stages.
AllocWS carve_alloc(const jolt_alloc_req* r, void* base, AllocWS* lane1 = nullptr) {
  const Dims d = dims_of(r);
  const int nt = 2 * r->n_layers;
  AllocWS w{};
  // scratch per tensor drives the chunk size (bounded by 4 GiB of scratch)
  size_t per = 0;
  if (!d.flash) per = 3 * static_cast<size_t>(d.n_pad) * d.n_pad * 4;
  else per = static_cast<size_t>(d.T) * d.ell * 4 * 2 + static_cast<size_t>(d.HD) * d.ell * 12 +
             static_cast<size_t>(d.ell_pad) * d.ell_pad * 12;
  per += static_cast<size_t>(std::max(d.T, d.HD)) * std::max<int64_t>(d.R, 1) * 8 + (1 << 20);
  per += static_cast<size_t>(gram_d_ksplit(d)) * d.D * d.D * 4;
  per += syev_top_work_bytes(d.D, static_cast<int>(d.D), 1);
  per += (static_cast<size_t>(d.T) * std::max<int64_t>(d.R, 1) + d.D * d.D) * 4 +
         (cholesky_qr_work_floats(d.T, std::max<int64_t>(d.R, 1), 1) + cholesky_qr_work_floats(d.D, d.D, 1)) * 4;
  if (d.R > 0) per += syev_top_work_bytes(d.flash ? d.ell_pad : d.n_pad, static_cast<int>(d.R), 1);
  // up to 64 tensors (24 GiB of scratch) in flight.  Token eigenproblems of
  // n >= 2048 go in two lanes of half chunks: there the stages around the
  // chase are throughput-bound and overlap it; at smaller n they are
  // latency-bound, and halving the batch only doubles their count (the
  // randomized path keeps one lane).
  int chunk = static_cast<int>(std::max<size_t>(1, std::min<size_t>(64, (24ull << 30) / per)));
  chunk = std::min(chunk, nt);
  const int nlanes = (chunk >= 2 && !d.flash && d.R > 0 && d.n_pad >= 2048) ? 2 : 1;
  chunk = (chunk + nlanes - 1) / nlanes;
  w.chunk = chunk;
  w.nlanes = nlanes;
  Carver c;
  c.base = static_cast<char*>(base);
  const int64_t R = std::max<int64_t>(d.R, 1);
  w.UT = c.take<float>(static_cast<size_t>(nt) * d.T * R);
  w.UD = c.take<float>(static_cast<size_t>(nt) * d.D * d.D);
  w.lamT = c.take<double>(static_cast<size_t>(nt) * R);
  w.lamD = c.take<double>(static_cast<size_t>(nt) * d.D);
  // lamT .. status is one span, read back in one copy; xptrs and tags
  // another, uploaded in one copy
  w.frob2 = c.take<double>(nt);
  w.status = c.take<int>(1);
  w.xptrs = c.take<const void*>(nt);
  w.tags = c.take<uint64_t>(nt);
  const int64_t n = d.flash ? d.ell_pad : d.n_pad;
  auto carve_scratch = [&](AllocWS& w) {
    w.G = c.take<float>(static_cast<size_t>(chunk) * n * n);
    w.V = c.take<float>(static_cast<size_t>(chunk) * n * n);
    w.GDpart = c.take<float>(static_cast<size_t>(chunk) * gram_d_ksplit(d) * d.D * d.D);
    w.syevD = c.take<char>(syev_top_work_bytes(d.D, static_cast<int>(d.D), chunk));
    w.syev = d.R > 0 ? static_cast<void*>(c.take<char>(syev_top_work_bytes(n, static_cast<int>(d.R), chunk)))
                     : nullptr;
    w.GD = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.GDc = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.Ucm = c.take<float>(static_cast<size_t>(chunk) * d.T * R);
    w.Vr = c.take<float>(static_cast<size_t>(chunk) * std::max(d.nT, d.D) * std::max<int64_t>(R, d.D));
    w.P = c.take<float>(static_cast<size_t>(chunk) * R * d.HD);
    w.lam_tmp = c.take<double>(static_cast<size_t>(chunk) * std::max<int64_t>(R, d.D));
    w.qtau = c.take<float>(householder_qr_work_floats(std::max(d.T, d.HD),
                                                       std::max<int64_t>(std::max(R, d.ell), d.D), chunk));
    w.perm = c.take<int>(static_cast<size_t>(chunk) * std::max<int64_t>(R, d.D));
    w.sgn = c.take<float>(static_cast<size_t>(chunk) * std::max<int64_t>(R, d.D));
    if (d.flash) {
      w.Om = c.take<float>(static_cast<size_t>(chunk) * d.HD * d.ell);
      w.Y = c.take<float>(static_cast<size_t>(chunk) * d.T * d.ell);
      w.Z = c.take<float>(static_cast<size_t>(chunk) * d.HD * d.ell);
      w.Bm = c.take<float>(static_cast<size_t>(chunk) * d.ell * d.HD);
      w.Wr = c.take<float>(static_cast<size_t>(chunk) * d.ell * R);
    }
    w.Wd = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.qtauD = c.take<float>(householder_qr_work_floats(d.D, d.D, chunk));
    w.lamDt = c.take<double>(static_cast<size_t>(chunk) * d.D);
    w.permD = c.take<int>(static_cast<size_t>(chunk) * d.D);
    w.sgnD = c.take<float>(static_cast<size_t>(chunk) * d.D);
    w.Ucm2 = c.take<float>(static_cast<size_t>(chunk) * d.T * R);
    w.cq = c.take<float>(cholesky_qr_work_floats(d.T, R, chunk));
    w.Vr2 = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.cqD = c.take<float>(cholesky_qr_work_floats(d.D, d.D, chunk));
  };
  carve_scratch(w);
  if (nlanes > 1) {
    AllocWS w1 = w;
    carve_scratch(w1);
    if (lane1) *lane1 = w1;
  }
  w.bytes = c.off;
  if (lane1) lane1->bytes = c.off;
  return w;
}

// ------------------------------------------------- factor pipeline pieces
GemmArgs gemm0() {
  GemmArgs g{};
  g.am = g.ak = g.bk = g.bn = plain(1);
  g.alpha = 1.f;
  g.a_dtype = g.b_dtype = g.c_dtype = kF32;
  return g;
}

// Host-side HIP objects of one call.  Auxiliary streams (non-blocking,
// default priority) are leased from a per-device pool and handed back when the
// call ends, so concurrent calls never share one; events are created for the
// call alone and destroyed with it, so no call can wait on another's record.
// The pool is guarded by a mutex.  Device memory is never allocated here.
struct StreamPool {
  std::mutex mu;
  std::map<int, std::vector<hipStream_t>> idle;   // device -> streams not leased
};
StreamPool& stream_pool() {
  static StreamPool p;
  return p;
}

// Pinned host staging buffers for the small uploads and read-backs of a call
// (pointer tables, launch arguments, spectra): copies from and to them are
// plain DMA that never makes the host wait, where a pageable copy stages
// through the runtime and blocks.  A buffer is leased like a stream and goes
// back with an event recorded after the last copy that touches it; the next
// lease waits on that event, so a copy still in flight never sees its memory
// rewritten.  Buffers come from hipHostMalloc on first need and are kept until
// the process ends.
struct PinnedBuf {
  void* p = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;   // recorded after the buffer's last copy
  bool armed = false;          // `done` has been recorded at least once
};
struct PinnedPool {
  std::mutex mu;
  std::map<int, std::vector<PinnedBuf>> idle;   // device -> buffers not leased
};
PinnedPool& pinned_pool() {
  static PinnedPool p;
  return p;
}

class CallHip {
 public:
  CallHip() = default;
  CallHip(const CallHip&) = delete;
  CallHip& operator=(const CallHip&) = delete;
  ~CallHip() {
    for (hipEvent_t e : events_) (void)hipEventDestroy(e);
    if (!leased_.empty()) {
      StreamPool& p = stream_pool();
      std::lock_guard<std::mutex> lk(p.mu);
      auto& v = p.idle[dev_];
      v.insert(v.end(), leased_.begin(), leased_.end());
    }
    if (!pinned_.empty()) {
      PinnedPool& p = pinned_pool();
      std::lock_guard<std::mutex> lk(p.mu);
      auto& v = p.idle[pdev_];
      v.insert(v.end(), pinned_.begin(), pinned_.end());
    }
  }
  // Pinned host memory of at least `bytes` that no other call holds until
  // this one ends; a copy that uses it is followed by copied(ptr, stream).
  void* pinned(size_t bytes) {
    if (pinned_.empty()) ck(hipGetDevice(&pdev_));
    PinnedBuf b;
    {
      PinnedPool& p = pinned_pool();
      std::lock_guard<std::mutex> lk(p.mu);
      auto& v = p.idle[pdev_];
      int best = -1;
      for (int i = 0; i < static_cast<int>(v.size()); ++i)
        if (v[i].bytes >= bytes && (best < 0 || v[i].bytes < v[best].bytes)) best = i;
      if (best >= 0) {
        b = v[best];
        v.erase(v.begin() + best);
      }
    }
    if (b.p) {
      if (b.armed) ck(hipEventSynchronize(b.done));
    } else {
      size_t sz = 64 << 10;
      while (sz < bytes) sz *= 2;
      ck(hipHostMalloc(&b.p, sz, hipHostMallocDefault));
      b.bytes = sz;
      ck(hipEventCreateWithFlags(&b.done, hipEventDisableTiming));
    }
    pinned_.push_back(b);
    return b.p;
  }
  // Marks the end of the copies queued so far on s that touch buffer p.
  void copied(const void* p, hipStream_t s) {
    for (PinnedBuf& b : pinned_)
      if (b.p == p) {
        ck(hipEventRecord(b.done, s));
        b.armed = true;
        return;
      }
  }
  // A stream no other call holds until this one ends.
  hipStream_t lease() {
    if (leased_.empty()) ck(hipGetDevice(&dev_));
    hipStream_t st = nullptr;
    {
      StreamPool& p = stream_pool();
      std::lock_guard<std::mutex> lk(p.mu);
      auto& v = p.idle[dev_];
      if (!v.empty()) {
        st = v.back();
        v.pop_back();
      }
    }
    if (!st) ck(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
    leased_.push_back(st);
    return st;
  }
  hipEvent_t event() {
    hipEvent_t e = nullptr;
    ck(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    events_.push_back(e);
    return e;
  }

 private:
  int dev_ = 0, pdev_ = 0;
  std::vector<hipStream_t> leased_;
  std::vector<hipEvent_t> events_;
  std::vector<PinnedBuf> pinned_;
};

// Runs the feature-mode factor on an auxiliary stream of the call after the
// work queued on s so far; join() makes s wait for it.
struct FeatureFork {
  CallHip& hip;
  hipStream_t s;
  hipStream_t aux = nullptr;
  hipEvent_t join_ev = nullptr;
  FeatureFork(CallHip& h, hipStream_t s_) : hip(h), s(s_) {}
  hipStream_t start() {
    aux = hip.lease();
    const hipEvent_t fork = hip.event();
    ck(hipEventRecord(fork, s));
    ck(hipStreamWaitEvent(aux, fork, 0));
    return aux;
  }
  void done() {
    if (!aux) return;
    join_ev = hip.event();
    ck(hipEventRecord(join_ev, aux));
  }
  void join() {
    if (join_ev) ck(hipStreamWaitEvent(s, join_ev, 0));
    aux = nullptr;
    join_ev = nullptr;
  }
};

// Orthonormal columns spanning the leading columns of the nearly orthonormal
// column-major src (m x k, ld m, unit-norm columns up to a few percent) into
// dst, nested spans kept: one CholeskyQR pass, or Householder QR where k is too
// wide for it or after it broke down (w.householder; src is then overwritten).
void orthonormalize(float* src, float* dst, int64_t m, int64_t k, int batch, float* hwork, float* cwork,
                    const AllocWS& w, hipStream_t s) {
  if (!w.householder && k <= cholesky_qr_max_k() && m >= k) {
    ck(cholesky_qr(src, dst, m, k, m, m * k, batch, cwork, w.status, s));
  } else {
    ck(householder_qr(src, m, k, m, m * k, batch, hwork, s));
    ck(hipMemcpyAsync(dst, src, sizeof(float) * batch * m * k, hipMemcpyDeviceToDevice, s));
  }
}

// Feature-mode factor of `batch` tensors from their D x D Grams in w.GD.
void feature_factor(const Dims& d, int batch, int t0, const AllocWS& w, hipStream_t s) {
  const int64_t D = d.D;
  ck(hipMemcpyAsync(w.GDc, w.GD, sizeof(float) * batch * D * D, hipMemcpyDeviceToDevice, s));
  ck(syev_top(w.GD, D, batch, static_cast<int>(D), w.Vr2, nullptr, w.syevD, s, w.status));
  orthonormalize(w.Vr2, w.Vr, D, D, batch, w.qtauD, w.cqD, w, s);
  // Rayleigh quotients diag(U^T G U): W = G U (column-major), then column dots
  GemmArgs g = gemm0();
  g.M = D; g.N = D; g.K = D;
  g.A = w.GDc; g.am = plain(D); g.ak = plain(1); g.a_batch = D * D;
  g.B = w.Vr; g.bk = plain(1); g.bn = plain(D); g.b_batch = D * D;
  g.C = w.Wd; g.c_m = 1; g.c_n = D; g.c_batch = D * D;
  ck(launch_gemm(g, batch, s));
  ck(launch_col_dot(w.Vr, w.Wd, D, D, D, D * D, batch, w.lamDt, D, s));
  ck(finalize_factor_ws(w.Vr, D, D, D, D * D, w.lamDt, D, w.UD + static_cast<size_t>(t0) * D * D, D,
                        D * D, w.lamD + static_cast<size_t>(t0) * D, D, batch, w.permD, w.sgnD, s));
}

// Token-mode eigenvalues as Rayleigh quotients ||X_(T)^T u_j||^2 of the
// orthonormal column-major U (T x R), then sort/sign/emit (the randomized
// path, whose small eigenproblem only approximates the captured energies).
void token_finalize(const Dims& d, int batch, int t0, const AllocWS& w, int xdt, hipStream_t s) {
  const int64_t T = d.T, HD = d.HD, D = d.D, R = d.R;
  GemmArgs g = gemm0();
  g.M = R; g.N = HD; g.K = T;
  g.A = w.Ucm; g.am = plain(T); g.ak = plain(1); g.a_batch = T * R;
  g.b_ptrs = reinterpret_cast<const void* const*>(w.xptrs); g.b_dtype = xdt; g.ptr_align16 = w.x16;
  g.bk = plain(D); g.bn = segmented(D, T * D, 1);
  g.C = w.P; g.c_m = HD; g.c_n = 1; g.c_batch = R * HD;
  ck(launch_gemm(g, batch, s));
  ck(launch_row_sumsq(w.P, R, HD, R * HD, batch, w.lam_tmp, R, s));
  ck(finalize_factor_ws(w.Ucm, T, R, T, T * R, w.lam_tmp, R, w.UT + static_cast<size_t>(t0) * T * R, R,
                        T * R, w.lamT + static_cast<size_t>(t0) * R, R, batch, w.perm, w.sgn, s));
}

void analyze_exact(const Dims& d, int batch, int t0, const AllocWS& w, int xdt, CallHip& hip, hipStream_t s) {
  const int64_t T = d.T, D = d.D, HD = d.HD, n = d.n_pad, R = d.R;
  const void* const* xp = reinterpret_cast<const void* const*>(w.xptrs);
  ck(hipMemsetAsync(w.G, 0, sizeof(float) * batch * n * n, s));
  GemmArgs g = gemm0();
  g.a_ptrs = xp; g.b_ptrs = xp; g.a_dtype = g.b_dtype = xdt; g.ptr_align16 = w.x16;
  if (d.dual) {   // C = X_(T)^T X_(T), HD x HD
    g.M = HD; g.N = HD; g.K = T;
    g.am = segmented(D, T * D, 1); g.ak = plain(D);
    g.bk = plain(D); g.bn = segmented(D, T * D, 1);
  } else {        // G_T = X_(T) X_(T)^T, T x T
    g.M = T; g.N = T; g.K = HD;
    g.am = plain(D); g.ak = segmented(D, T * D, 1);
    g.bk = segmented(D, T * D, 1); g.bn = plain(D);
  }
  // column-major; the tridiagonal path reads the lower triangle only
  g.C = w.G; g.c_m = 1; g.c_n = n; g.c_batch = n * n;
  g.c_lower = 1;
  ck(launch_gemm(g, batch, s, "gram"));
  if (d.dual) {
    ck(launch_sum_diag_blocks(w.G, d.H, D, w.GD, batch, s));   // n == HD here
  } else {
    GemmArgs gd = gemm0();
    gd.a_ptrs = xp; gd.b_ptrs = xp; gd.a_dtype = gd.b_dtype = xdt; gd.ptr_align16 = w.x16;
    gd.M = D; gd.N = D; gd.K = d.H * T;
    gd.am = plain(1); gd.ak = plain(D); gd.bk = plain(D); gd.bn = plain(1);
    gd.C = w.GD; gd.c_m = D; gd.c_n = 1; gd.c_batch = D * D;
    gd.ksplit = gram_d_ksplit(d); gd.partial = w.GDpart;
    ck(launch_gemm(gd, batch, s, "gram"));
  }
  // the feature path runs on a stream of its own, forked here (its Gram is
  // complete in stream order); its kernels are enqueued after the token
  // path's, so that their launches on the host do not hold back the token
  // path's first kernels
  FeatureFork ff(hip, s);
  const hipStream_t fs = ff.start();
  // the band reduction's end, recorded on s by the eigensolver below
  const hipEvent_t band_done = R > 0 ? (w.band_done ? w.band_done : hip.event()) : nullptr;
  auto feature = [&] {
    // the feature factor, then ||X||^2 of every tensor, off the token path's
    // critical path: once the token band reduction (latency-bound launches)
    // is done, beside the token bulge chase and eigenpair solve (a few CUs
    // per tensor, HBM idle)
    if (band_done) ck(hipStreamWaitEvent(fs, band_done, 0));
    feature_factor(d, batch, t0, w, fs);
    ck(launch_sumsq(xp, batch, d.H * T * D, xdt, w.frob2 + t0, fs));
    if (w.early) {
      // everything the allocation reads is final here: to the host while the
      // token path forms its factors
      ck(hipStreamWaitEvent(fs, w.eig_done, 0));
      ck(hipMemcpyAsync(w.early, w.lam_tmp, sizeof(double) * batch * R, hipMemcpyDeviceToHost, fs));
      ck(hipMemcpyAsync(w.early + batch * R, w.lamD + static_cast<size_t>(t0) * D, sizeof(double) * batch * D,
                        hipMemcpyDeviceToHost, fs));
      ck(hipMemcpyAsync(w.early + batch * (R + D), w.frob2 + t0, sizeof(double) * batch, hipMemcpyDeviceToHost, fs));
      ck(hipEventRecord(w.early_done, fs));
    }
    ff.done();
    ff.join();
  };
  if (R == 0) {
    feature();
    return;
  }
  // leading eigenvectors V_R of the token Gram: the first R columns of w.V
  // (column-major, leading dimension n)
  // (dual: each column scaled by 1 / sqrt(lambda), so that X_(T) v / sqrt(lambda)
  // has unit norm and the recovered factor is nearly orthonormal)
  const SyevSide side{hip.lease(), hip.event(), hip.event()};
  ck(syev_top(w.G, n, batch, static_cast<int>(R), w.V, w.lam_tmp, w.syev, s, w.status, band_done, d.dual, &side));
  if (w.early) ck(hipEventRecord(w.eig_done, s));   // w.lam_tmp final (the eigensolver copies it in stream order)
  if (d.dual) {
    // U' = X_(T) V_R Lambda^{-1/2} (T x R, column-major)
    GemmArgs gu = gemm0();
    gu.a_ptrs = xp; gu.a_dtype = xdt; gu.ptr_align16 = w.x16;
    gu.M = T; gu.N = R; gu.K = HD;
    gu.am = plain(D); gu.ak = segmented(D, T * D, 1);
    gu.B = w.V; gu.bk = plain(1); gu.bn = plain(n); gu.b_batch = n * n;
    gu.C = w.Ucm2; gu.c_m = 1; gu.c_n = T; gu.c_batch = T * R;
    ck(launch_gemm(gu, batch, s));
  } else {
    ck(copy_cols(w.V, n, n * n, w.Ucm2, T, T * R, T, R, batch, s));
  }
  orthonormalize(w.Ucm2, w.Ucm, T, R, batch, w.qtau, w.cq, w, s);
  // the token spectrum: the eigensolver's eigenvalues of the token Gram
  // (fp64, descending; the dual Gram shares the nonzero ones)
  ck(finalize_factor_ws(w.Ucm, T, R, T, T * R, w.lam_tmp, R, w.UT + static_cast<size_t>(t0) * T * R, R, T * R,
                        w.lamT + static_cast<size_t>(t0) * R, R, batch, w.perm, w.sgn, s));
  feature();
}

void analyze_flash(const Dims& d, int batch, int t0, const AllocWS& w, int xdt, int q, uint64_t seed,
                   CallHip& hip, hipStream_t s) {
  const int64_t T = d.T, D = d.D, HD = d.HD, R = d.R, ell = d.ell, ep = d.ell_pad;
  const void* const* xp = reinterpret_cast<const void* const*>(w.xptrs);
  // feature mode: exact Gram path (a sketch of width D spans all of R^D)
  {
    GemmArgs gd = gemm0();
    gd.a_ptrs = xp; gd.b_ptrs = xp; gd.a_dtype = gd.b_dtype = xdt; gd.ptr_align16 = w.x16;
    gd.M = D; gd.N = D; gd.K = d.H * T;
    gd.am = plain(1); gd.ak = plain(D); gd.bk = plain(D); gd.bn = plain(1);
    gd.C = w.GD; gd.c_m = D; gd.c_n = 1; gd.c_batch = D * D;
    gd.ksplit = gram_d_ksplit(d); gd.partial = w.GDpart;
    ck(launch_gemm(gd, batch, s, "gram"));
  }
  // the feature path runs on a stream of its own, forked here (its Gram is
  // complete in stream order); its kernels are enqueued after the token
  // path's, so that their launches on the host do not hold back the token
  // path's first kernels
  FeatureFork ff(hip, s);
  const hipStream_t fs = ff.start();
  auto feature = [&] {
    // ||X||^2 of every tensor, off the token path's critical path
    ck(launch_sumsq(xp, batch, d.H * T * D, xdt, w.frob2 + t0, fs));
    feature_factor(d, batch, t0, w, fs);
    ff.done();
    ff.join();
  };
  if (R == 0) {
    feature();
    return;
  }
  ck(launch_sketch(w.Om, HD, ell, seed, w.tags, batch, s));
  auto AY = [&](const float* Bsrc, int64_t ldb, bool b_rowmajor, float* out) {
    // out (T x ell, column-major) = X_(T) B, B is HD x ell
    GemmArgs g = gemm0();
    g.a_ptrs = xp; g.a_dtype = xdt; g.ptr_align16 = w.x16;
    g.M = T; g.N = ell; g.K = HD;
    g.am = plain(D); g.ak = segmented(D, T * D, 1);
    g.B = Bsrc;
    if (b_rowmajor) { g.bk = plain(ldb); g.bn = plain(1); }
    else { g.bk = plain(1); g.bn = plain(ldb); }
    g.b_batch = HD * ell;
    g.C = out; g.c_m = 1; g.c_n = T; g.c_batch = T * ell;
    ck(launch_gemm(g, batch, s));
  };
  AY(w.Om, HD, false, w.Y);                 // the sketch is column-major (k contiguous)
  ck(householder_qr(w.Y, T, ell, T, T * ell, batch, w.qtau, s));
  for (int it = 0; it < q; ++it) {
    GemmArgs g = gemm0();                       // Z = X_(T)^T Q (HD x ell, column-major)
    g.a_ptrs = xp; g.a_dtype = xdt; g.ptr_align16 = w.x16;
    g.M = HD; g.N = ell; g.K = T;
    g.am = segmented(D, T * D, 1); g.ak = plain(D);
    g.B = w.Y; g.bk = plain(1); g.bn = plain(T); g.b_batch = T * ell;
    g.C = w.Z; g.c_m = 1; g.c_n = HD; g.c_batch = HD * ell;
    ck(launch_gemm(g, batch, s));
    ck(householder_qr(w.Z, HD, ell, HD, HD * ell, batch, w.qtau, s));
    AY(w.Z, HD, false, w.Y);
    ck(householder_qr(w.Y, T, ell, T, T * ell, batch, w.qtau, s));
  }
  {
    GemmArgs g = gemm0();                       // B = Q^T X_(T) (ell x HD, row-major)
    g.M = ell; g.N = HD; g.K = T;
    g.A = w.Y; g.am = plain(T); g.ak = plain(1); g.a_batch = T * ell;
    g.b_ptrs = xp; g.b_dtype = xdt; g.bk = plain(D); g.bn = segmented(D, T * D, 1); g.ptr_align16 = w.x16;
    g.C = w.Bm; g.c_m = HD; g.c_n = 1; g.c_batch = ell * HD;
    ck(launch_gemm(g, batch, s));
  }
  ck(hipMemsetAsync(w.G, 0, sizeof(float) * batch * ep * ep, s));
  {
    GemmArgs g = gemm0();                       // M = B B^T (ell x ell, padded)
    g.M = ell; g.N = ell; g.K = HD;
    g.A = w.Bm; g.am = plain(HD); g.ak = plain(1); g.a_batch = ell * HD;
    g.B = w.Bm; g.bk = plain(1); g.bn = plain(HD); g.b_batch = ell * HD;
    g.C = w.G; g.c_m = ep; g.c_n = 1; g.c_batch = ep * ep;
    ck(launch_gemm(g, batch, s));
  }
  // top R eigenvectors of the ell x ell (zero-padded) B B^T, by the same
  // tridiagonal solver as the exact path, then their first ell rows
  ck(syev_top(w.G, ep, batch, static_cast<int>(R), w.V, nullptr, w.syev, s, w.status));
  ck(copy_cols(w.V, ep, ep * ep, w.Wr, ell, ell * R, ell, R, batch, s));
  {
    GemmArgs g = gemm0();                       // U = Q W_R (T x R, column-major)
    g.M = T; g.N = R; g.K = ell;
    g.A = w.Y; g.am = plain(1); g.ak = plain(T); g.a_batch = T * ell;
    g.B = w.Wr; g.bk = plain(1); g.bn = plain(ell); g.b_batch = ell * R;
    g.C = w.Ucm2; g.c_m = 1; g.c_n = T; g.c_batch = T * R;
    ck(launch_gemm(g, batch, s));
  }
  orthonormalize(w.Ucm2, w.Ucm, T, R, batch, w.qtau, w.cq, w, s);
  token_finalize(d, batch, t0, w, xdt, s);
  feature();
}

// Algorithmic work of the residual path of one tensor (encode or decode):
// the Tucker reconstruction in its cheaper product order, 2 min(r_T,
// r_T r_D / D + r_D) flops per element, and the rotation, 2 D; the bytes are
// the input (or output) once, the codes and scales once, and the record's
// factors and core once.
struct PathWork {
  double bytes, flops;
};
PathWork residual_work(int64_t H, int64_t T, int64_t D, jolt_choice c, int elem_bytes) {
  const double N = static_cast<double>(H * T * D);
  const double rT = c.r_T, rD = c.r_D;
  const double rec = c.r_T > 0 ? 2.0 * std::min(rT, rT * rD / static_cast<double>(D) + rD) : 0.0;
  const double codes = N * (c.bits + 1) / 8.0;          // b-bit codes + bf16 (offset, step) per 32
  const double facs = 2.0 * (T * rT + D * rD + H * rT * rD);
  return {N * elem_bytes + codes + facs, N * (rec + 2.0 * D)};
}

int64_t rtp_of(int r_T) { return (static_cast<int64_t>(r_T) + 31) / 32 * 32; }
// the encoder's W parts: k padded to whole 64-value chunks
int64_t enc_rtp(int r_T) { return (static_cast<int64_t>(r_T) + 63) / 64 * 64; }

size_t decode_ws_one(const jolt_shape* s, jolt_choice c) {
  if (c.r_T == 0) return 0;
  return 2 * a256(2ull * s->H * s->D * rtp_of(c.r_T));
}

// ------------------------------------------------- allocation-free decode
// Scratch of jolt_decode_many_static: the W planes of the records of one
// launch pair.  A file-scope device array, one copy per GPU, held until the
// process ends; host code uses the address hipGetSymbolAddress gives for the
// current device, never the array's name.
constexpr size_t kStaticScratchBytes = size_t{32} << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device (under a lock) and kept.
constexpr int kMaxDevices = 64;
void* static_scratch() {
  static std::mutex mu;
  static void* per_dev[kMaxDevices] = {};
  int dev = 0;
  ck(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) throw HipFail{};
  std::lock_guard<std::mutex> lk(mu);
  if (!per_dev[dev]) {
    void* p = nullptr;
    ck(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    per_dev[dev] = p;
  }
  return per_dev[dev];
}

// Decode n records of one shape, up to kDecBatch per launch pair (W
// prologue + decode).  The W planes of the records of one launch pair are
// carved in order from ws; ws_cap bounds that carve: when the next record's
// planes do not fit, the pair launched so far is issued and the carve starts
// again at ws (the next pair's prologue runs after the previous decode on
// the stream, so reusing the bytes is ordered).  The caller guarantees that
// one record's planes fit ws_cap.
size_t decode_w_bytes(int64_t H, int64_t D, jolt_choice c) {
  return c.r_T ? 2 * a256(2ull * H * D * rtp_of(c.r_T)) : 0;
}

// The decode's view of one record: its sections, the W planes at wsp (the
// record's decode_w_bytes), its first W tile.
DecRec dec_rec(int64_t H, int64_t T, int64_t D, jolt_choice c, const void* blob_dev, void* out, char* wsp,
               int wtile0) {
  const BlobLayout L = blob_layout(H, T, D, c);
  DecRec R{};
  R.blob = static_cast<const char*>(blob_dev);
  R.out = out;
  R.H = static_cast<int32_t>(H); R.T = static_cast<int32_t>(T);
  R.r_T = c.r_T; R.r_D = c.r_D; R.bits = c.bits;
  R.r_Tp = static_cast<int32_t>(rtp_of(c.r_T));
  R.Whi = reinterpret_cast<uint16_t*>(wsp);
  // the device addresses the sections from the record's base: the same layout
  if (D != 128 || L.ut != 256 || L.ud != R.off_ud() || L.g != R.off_g() || L.sc != R.off_sc() ||
      L.cd != R.off_cd() || reinterpret_cast<char*>(R.Wlo()) != wsp + decode_w_bytes(H, D, c) / 2)
    throw HipFail{};
  R.wtile0 = wtile0;
  return R;
}

void decode_records(int n, const jolt_shape* shape, const jolt_choice* ch, const void* const* blobs,
                    const void* rot_dev, void* const* outs, void* ws, size_t ws_cap, hipStream_t s) {
  const int64_t H = shape->H, T = shape->T, D = shape->D;
  const size_t n2 = static_cast<size_t>(D) * D;
  const uint16_t* Qt16 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(rot_dev) + 2 * a256(4 * n2));
  DecBatch b{};
  size_t used = 0;
  int wtiles = 0, first = 0;
  auto issue = [&]() {
    if (b.n == 0) return;
    b.H = static_cast<int32_t>(H);
    b.T = static_cast<int32_t>(T);
    b.out_dtype = shape->dtype == JOLT_BF16 ? kBF16 : kF32;
    b.Qt16 = Qt16;
    b.out16 = 1;
    for (int j = 0; j < b.n; ++j) b.out16 &= (reinterpret_cast<uintptr_t>(b.rec[j].out) & 15) == 0 ? 1 : 0;
    b.wtiles_total = wtiles;
    if (prof_enabled("decode")) {
      double by = 0.0, fl = 0.0;
      for (int j = 0; j < b.n; ++j) {
        const PathWork pw = residual_work(H, T, D, ch[first + j], shape->dtype == JOLT_BF16 ? 2 : 4);
        by += pw.bytes;
        fl += pw.flops;
      }
      prof_add_work("decode", by, fl);
    }
    ck(launch_decode_batch(b, s));
    b = DecBatch{};
    used = 0;
    wtiles = 0;
  };
  for (int i = 0; i < n; ++i) {
    const jolt_choice c = ch[i];
    const size_t wneed = decode_w_bytes(H, D, c);
    if (b.n == kDecBatch || (b.n > 0 && used + wneed > ws_cap)) issue();
    if (b.n == 0) first = i;
    DecRec& R = b.rec[b.n++];
    R = dec_rec(H, T, D, c, blobs[i], outs[i], static_cast<char*>(ws) + used, wtiles);
    used += wneed;
    wtiles += static_cast<int>(H * (R.r_Tp / 32));
  }
  issue();
}

// The prepared rotation buffer from a D x D orthogonal Q (fp64, row-major,
// host): fp32 Q, fp32 Q^T, bf16 Q^T and the three exact bf16 parts of the
// fp32 Q in the encoder's matrix-core fragment order.  Synchronizes s.
void upload_rotation(const double* Q, int D, void* q_dev, hipStream_t s) {
  const size_t n = static_cast<size_t>(D) * D;
  std::vector<float> buf(2 * n);
  std::vector<uint16_t> b16(n);
  for (size_t i = 0; i < n; ++i) {
    const size_t r = i / D, c = i % D;
    buf[i] = static_cast<float>(Q[i]);
    buf[n + c * D + r] = static_cast<float>(Q[i]);       // Q^T
    // bf16 (nearest-even, via the fp32 value) of Q^T: b16[c][r] = Q[r][c]
    float f = static_cast<float>(Q[i]);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    b16[c * D + r] = static_cast<uint16_t>(u >> 16);
  }
  // exact three-part bf16 split of the fp32 Q: hi = rne(f), mid = rne(f - hi),
  // lo = f - hi - mid (a bf16 value), stored in matrix-core fragment order
  // [part][cb][ds][lane][e] = part of Q[32 cb + lane % 32][16 ds + 8 (lane / 32) + e]
  std::vector<uint16_t> q3(3 * n);
  auto rne = [](float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  };
  auto widen = [](uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  };
  for (size_t i = 0; i < n; ++i) {
    const size_t c = i / D, d = i % D;               // buf[i] = Q[c][d]
    const size_t o = ((c / 32 * (D / 16) + d / 16) * 64 + (d / 8 % 2) * 32 + c % 32) * 8 + d % 8;
    const float f = buf[i];
    const uint16_t h = rne(f);
    const float r1 = f - widen(h);
    const uint16_t m = rne(r1);
    const float r2 = r1 - widen(m);
    uint32_t u;
    std::memcpy(&u, &r2, 4);
    q3[o] = h;
    q3[n + o] = m;
    q3[2 * n + o] = static_cast<uint16_t>(u >> 16);
  }
  char* base = static_cast<char*>(q_dev);
  ck(hipMemcpyAsync(base, buf.data(), 4 * n, hipMemcpyHostToDevice, s));
  ck(hipMemcpyAsync(base + a256(4 * n), buf.data() + n, 4 * n, hipMemcpyHostToDevice, s));
  ck(hipMemcpyAsync(base + 2 * a256(4 * n), b16.data(), 2 * n, hipMemcpyHostToDevice, s));
  ck(hipMemcpyAsync(base + 2 * a256(4 * n) + a256(2 * n), q3.data(), 6 * n, hipMemcpyHostToDevice, s));
  ck(hipStreamSynchronize(s));
}

template <typename F>
jolt_status guard(F&& f) {
  try {
    return f();
  } catch (const HipFail&) {
    return JOLT_EHIP;
  } catch (...) {
    return JOLT_EHIP;
  }
}

}  // namespace

// ================================================================== ABI
// split-K of the encode's U~_T^T X product (K = T tokens)
int encode_ksplit(int64_t T) { return static_cast<int>(std::min<int64_t>(16, std::max<int64_t>(1, T / 256))); }

// ---- encode of many tensors of one shape: the per-tensor steps of jolt_encode,
// batched over the tensors of each (r_T, r_D) and over all tensors for the
// residual kernel and the headers (the same kernels and arithmetic).
struct EncManyLayout {
  std::vector<int> order;                  // Tucker tensors grouped by (r_T, r_D), input order kept
  std::vector<std::pair<int, int>> groups; // [begin, end) into order
  std::vector<size_t> w_off, p_off, part_off;   // per group, bytes into the workspace
  size_t arr_off, total;
  size_t n_ptrs;                           // pointer slots
};
EncManyLayout enc_many_layout(int n, const jolt_shape* shape, const jolt_choice* ch) {
  EncManyLayout L;
  const int64_t H = shape->H, T = shape->T, D = shape->D, HD = H * D;
  std::vector<int> idx;
  for (int i = 0; i < n; ++i)
    if (ch[i].r_T > 0) idx.push_back(i);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
    return ch[a].r_T != ch[b].r_T ? ch[a].r_T < ch[b].r_T : ch[a].r_D < ch[b].r_D;
  });
  L.order = idx;
  size_t off = 0;
  for (size_t b = 0; b < idx.size();) {
    size_t e = b;
    while (e < idx.size() && ch[idx[e]].r_T == ch[idx[b]].r_T && ch[idx[e]].r_D == ch[idx[b]].r_D) ++e;
    const size_t m = e - b, rT = ch[idx[b]].r_T;
    L.groups.emplace_back(static_cast<int>(b), static_cast<int>(e));
    L.w_off.push_back(off);
    off += a256(4ull * m * H * D * enc_rtp(static_cast<int>(rT)));
    L.p_off.push_back(off);
    off += a256(4ull * m * rT * HD);
    L.part_off.push_back(off);
    off += a256(4ull * m * rT * HD * encode_ksplit(T));
    b = e;
  }
  // pointers: casts 4 per Tucker tensor, P 2 per, G2 3 and G3 2 per (tensor, head);
  // blobs 1 per tensor
  const size_t nt = idx.size();
  L.n_ptrs = 4 * nt + 2 * nt + 5 * nt * H + static_cast<size_t>(n);
  L.arr_off = off;
  off += a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n) + a256(sizeof(RecordHead) * n);
  L.total = off + 256;
  return L;
}

extern "C" {

size_t jolt_blob_bytes(const jolt_shape* shape, jolt_choice choice) {
  if (!shape_ok(shape) || !choice_ok(shape, choice)) return 0;
  return blob_layout(shape->H, shape->T, shape->D, choice).total;
}

size_t jolt_workspace_bytes(const jolt_alloc_req* req) {
  if (!req_ok(req)) return 0;
  return carve_alloc(req, nullptr).bytes;
}

int32_t jolt_spectrum_len(const jolt_alloc_req* req) {
  if (!req_ok(req)) return 0;
  return cap_of(req);
}


size_t jolt_encode_workspace_bytes(const jolt_shape* shape, jolt_choice c) {
  if (!shape_ok(shape) || !choice_ok(shape, c)) return 0;
  const size_t w = a256(4ull * shape->H * c.r_T * shape->D);
  return a256(4ull * shape->H * shape->D * enc_rtp(c.r_T)) + w + a256(w * encode_ksplit(shape->T)) + 256;
}

size_t jolt_decode_workspace_bytes(const jolt_shape* shape, jolt_choice c) {
  if (!shape_ok(shape) || !choice_ok(shape, c)) return 0;
  return decode_ws_one(shape, c);
}

size_t jolt_decode_many_workspace_bytes(int32_t n, const jolt_shape* shape, const jolt_choice* choices) {
  if (n < 0 || !shape_ok(shape) || (n > 0 && !choices)) return 0;
  size_t tot = 256;
  for (int i = 0; i < n; ++i) {
    if (!choice_ok(shape, choices[i])) return 0;
    tot += decode_ws_one(shape, choices[i]);
  }
  return tot;
}

size_t jolt_rotation_bytes(int32_t D) {
  if (D != kD) return 0;
  return a256(4ull * D * D) * 2 + a256(2ull * D * D) + a256(6ull * D * D);
}

jolt_status jolt_plan_from_spectra(const jolt_alloc_req* req, const double* spectra_T, int32_t len_T,
                                   const double* spectra_D, const double* frob2, jolt_plan* plan) {
  if (!req_ok(req) || !spectra_T || !spectra_D || !frob2 || !plan || !plan->choice) return JOLT_EINVAL;
  if (len_T < cap_of(req)) return JOLT_EINVAL;
  const int nt = 2 * req->n_layers;
  for (int i = 0; i < nt; ++i)
    if (!std::isfinite(frob2[i])) return JOLT_ERANGE;
  return plan_dual(req, spectra_T, len_T, spectra_D, frob2, plan);
}

jolt_status jolt_rotation_host(uint64_t seed, int32_t D, double* Q) {
  if (D < 1 || D > 4096 || !Q) return JOLT_EINVAL;
  rotation_host(seed, D, Q);
  return JOLT_OK;
}

double jolt_rng_normal(uint64_t seed, uint64_t tag, uint64_t index) {
  return normal_h(mix64h(seed ^ tag), index);
}

jolt_status jolt_rotation(uint64_t seed, int32_t D, void* q_dev, size_t q_bytes, void* stream) {
  if (D != kD || !q_dev) return JOLT_EINVAL;
  if (q_bytes < jolt_rotation_bytes(D)) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    std::vector<double> Q(static_cast<size_t>(D) * D);
    rotation_host(seed, D, Q.data());
    upload_rotation(Q.data(), D, q_dev, static_cast<hipStream_t>(stream));
    return JOLT_OK;
  });
}

jolt_status jolt_rotation_from(const double* Q, int32_t D, void* q_dev, size_t q_bytes, void* stream) {
  if (D != kD || !q_dev || !Q) return JOLT_EINVAL;
  if (q_bytes < jolt_rotation_bytes(D)) return JOLT_ENOSPACE;
  // orthogonal to fp64 working accuracy: |Q^T Q - I| entrywise below 1e-12
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) {
      double s = 0.0;
      for (int k = 0; k < D; ++k) s += Q[static_cast<size_t>(k) * D + i] * Q[static_cast<size_t>(k) * D + j];
      if (!(std::fabs(s - (i == j ? 1.0 : 0.0)) <= 1e-12)) return JOLT_EINVAL;
    }
  return guard([&]() -> jolt_status {
    upload_rotation(Q, D, q_dev, static_cast<hipStream_t>(stream));
    return JOLT_OK;
  });
}

jolt_status jolt_allocate(const jolt_alloc_req* req, const void* const* x_dev, void* ws_dev,
                          size_t ws_bytes, void* stream, jolt_plan* plan) {
  if (!req_ok(req) || !x_dev || !ws_dev || !plan || !plan->choice) return JOLT_EINVAL;
  const int nt = 2 * req->n_layers;
  for (int i = 0; i < nt; ++i)
    if (!x_dev[i]) return JOLT_EINVAL;
  AllocWS w1{};
  AllocWS w = carve_alloc(req, ws_dev, &w1);
  if (ws_bytes < w.bytes) return JOLT_ENOSPACE;
  w.x16 = true;
  for (int i = 0; i < nt; ++i) w.x16 = w.x16 && (reinterpret_cast<uintptr_t>(x_dev[i]) & 15) == 0;
  w1.x16 = w.x16;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Dims d = dims_of(req);
    const int xdt = req->shape.dtype == JOLT_BF16 ? kBF16 : kF32;
    ck(hipMemsetAsync(w.frob2, 0, sizeof(double) * nt, s));
    ck(hipMemsetAsync(w.status, 0, sizeof(int), s));
    CallHip stage;                                // pinned staging of the upload and the read-back
    // every tensor's pointer and sketch tag, uploaded once (one span of the workspace)
    {
      const size_t up = reinterpret_cast<const char*>(w.tags + nt) - reinterpret_cast<const char*>(w.xptrs);
      char* img = static_cast<char*>(stage.pinned(up));
      std::memcpy(img, x_dev, sizeof(void*) * nt);
      uint64_t* tags = reinterpret_cast<uint64_t*>(img + (reinterpret_cast<char*>(w.tags) - reinterpret_cast<char*>(w.xptrs)));
      for (int t = 0; t < nt; ++t)
        tags[t] = kTagSketch ^ ((static_cast<uint64_t>(t / 2) << 8) | static_cast<uint64_t>(t % 2));
      ck(hipMemcpyAsync(w.xptrs, img, up, hipMemcpyHostToDevice, s));
      stage.copied(img, s);
    }
    const int R = static_cast<int>(d.R);
    // the read-back span: lamT [nt][max(R, 1)], lamD [nt][D], frob2 [nt], status
    const size_t rb = reinterpret_cast<const char*>(w.status + 1) - reinterpret_cast<const char*>(w.lamT);
    char* back = static_cast<char*>(stage.pinned(rb));
    auto host_of = [&](const void* dev) { return back + (static_cast<const char*>(dev) - reinterpret_cast<const char*>(w.lamT)); };
    const double* lt = reinterpret_cast<const double*>(host_of(w.lamT));
    const double* ld = reinterpret_cast<const double*>(host_of(w.lamD));
    const double* f2 = reinterpret_cast<const double*>(host_of(w.frob2));
    // The exact path on one chunk reads its spectra back early and forms the
    // plan on the host while the token factors are still being formed; the
    // plan is kept when the final read-back holds the same values.
    const bool early = !d.flash && R > 0 && nt <= w.chunk;
    double* early_host = nullptr;
    jolt_status early_rc = JOLT_EINVAL;
    bool early_ok = false;
    // the whole analysis; returns the status word
    auto analyze_all = [&](bool householder) -> int {
      w.householder = w1.householder = householder;
      w.early = nullptr;
      // chunks alternate between the lanes: lane 0 on s, lane 1 on a second
      // stream of this call, forked from s and joined back into it
      CallHip hip;
      hipStream_t ls = nullptr;
      if (w.nlanes > 1 && nt > w.chunk) {
        ls = hip.lease();
        const hipEvent_t fork = hip.event();
        ck(hipEventRecord(fork, s));
        ck(hipStreamWaitEvent(ls, fork, 0));
      }
      // a chunk on the second lane starts once the previous chunk's band
      // reduction is queued ahead of it, so that chunk's chase (one CU per
      // tensor) runs beside this chunk's matrix-core stages
      if (early && !householder) {
        early_host = static_cast<double*>(stage.pinned(sizeof(double) * nt * (R + d.D + 1)));
        w.early = early_host;
        w.eig_done = hip.event();
        w.early_done = hip.event();
      }
      std::vector<hipEvent_t> marks;
      if (ls)
        for (int c = 0; c * w.chunk < nt; ++c) marks.push_back(hip.event());
      for (int t0 = 0, c = 0; t0 < nt; t0 += w.chunk, ++c) {
        const int batch = std::min(w.chunk, nt - t0);
        const bool second = ls && (c & 1);
        AllocWS wl = second ? w1 : w;
        hipStream_t sl = second ? ls : s;
        wl.xptrs = w.xptrs + t0;
        wl.tags = w.tags + t0;
        wl.band_done = ls ? marks[c] : nullptr;
        if (ls && c > 0) ck(hipStreamWaitEvent(sl, marks[c - 1], 0));
        if (d.flash) analyze_flash(d, batch, t0, wl, xdt, req->power_iters, req->seed, hip, sl);
        else analyze_exact(d, batch, t0, wl, xdt, hip, sl);
      }
      if (ls) {
        const hipEvent_t join = hip.event();
        ck(hipEventRecord(join, ls));
        ck(hipStreamWaitEvent(s, join, 0));
      }
      ck(hipMemcpyAsync(back, w.lamT, rb, hipMemcpyDeviceToHost, s));
      stage.copied(back, s);
      if (w.early) {
        stage.copied(early_host, s);                 // s has joined the stream of the early copies
        ck(hipEventSynchronize(w.early_done));
        const double* ef = early_host + nt * (R + d.D);
        bool fin = true;
        for (int i = 0; i < nt; ++i) fin = fin && std::isfinite(ef[i]);
        if (fin) {
          early_rc = plan_dual(req, early_host, R, early_host + nt * R, ef, plan);
          early_ok = true;
        }
        w.early = nullptr;
      }
      ck(hipStreamSynchronize(s));
      int status = 0;
      std::memcpy(&status, host_of(w.status), sizeof(int));
      return status;
    };
    int status = analyze_all(false);
    bool status_first_pass_only = true;
    if (status == 2) {
      status_first_pass_only = false;
      // a CholeskyQR pass met a nearly dependent column (rank-deficient
      // input): the same analysis again with Householder QR throughout
      ck(hipMemsetAsync(w.frob2, 0, sizeof(double) * nt, s));
      ck(hipMemsetAsync(w.status, 0, sizeof(int), s));
      status = analyze_all(true);
    }
    if (status != 0) return JOLT_EHIP;          // an eigensolver wait gave up: the factors are not valid
    for (int i = 0; i < nt; ++i)
      if (!std::isfinite(f2[i])) return JOLT_ERANGE;
    if (R == 0) std::memset(host_of(w.lamT), 0, sizeof(double) * nt);   // no token spectra: zero placeholders
    if (plan->spectra_T && R > 0) std::memcpy(plan->spectra_T, lt, sizeof(double) * nt * R);
    if (plan->spectra_D) std::memcpy(plan->spectra_D, ld, sizeof(double) * nt * d.D);
    if (plan->frob2) std::memcpy(plan->frob2, f2, sizeof(double) * nt);
    // the early plan stands when it was formed from exactly the values read back
    // at the end (a repeated analysis or any difference forms it again)
    if (early_ok && status_first_pass_only &&
        std::memcmp(lt, early_host, sizeof(double) * nt * R) == 0 &&
        std::memcmp(ld, early_host + nt * R, sizeof(double) * nt * d.D) == 0 &&
        std::memcmp(f2, early_host + nt * (R + d.D), sizeof(double) * nt) == 0)
      return early_rc;
    return plan_dual(req, lt, std::max(R, 1), ld, f2, plan);
  });
}

jolt_status jolt_factors(const jolt_alloc_req* req, void* ws_dev, int32_t tensor, const float** U_T,
                         int32_t* ld_T, const float** U_D) {
  if (!req_ok(req) || !ws_dev || tensor < 0 || tensor >= 2 * req->n_layers) return JOLT_EINVAL;
  const AllocWS w = carve_alloc(req, ws_dev);
  const Dims d = dims_of(req);
  const int64_t R = std::max<int64_t>(d.R, 1);
  if (U_T) *U_T = w.UT + static_cast<size_t>(tensor) * d.T * R;
  if (ld_T) *ld_T = static_cast<int32_t>(R);
  if (U_D) *U_D = w.UD + static_cast<size_t>(tensor) * d.D * d.D;
  return JOLT_OK;
}

jolt_status jolt_factors_many(const jolt_alloc_req* req, void* ws_dev, int32_t first, int32_t n, const float** U_T,
                              int32_t* ld_T, const float** U_D) {
  if (!req_ok(req) || !ws_dev || first < 0 || n < 0 || first + n > 2 * req->n_layers) return JOLT_EINVAL;
  if (n > 0 && (!U_T || !ld_T || !U_D)) return JOLT_EINVAL;
  const AllocWS w = carve_alloc(req, ws_dev);
  const Dims d = dims_of(req);
  const int64_t R = std::max<int64_t>(d.R, 1);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t t = first + i;
    U_T[i] = w.UT + static_cast<size_t>(t) * d.T * R;
    ld_T[i] = static_cast<int32_t>(R);
    U_D[i] = w.UD + static_cast<size_t>(t) * d.D * d.D;
  }
  return JOLT_OK;
}

jolt_status jolt_encode(const jolt_shape* shape, const void* x_dev, jolt_choice c, const float* U_T_dev,
                        int32_t ld_T, const float* U_D_dev, int32_t ld_D, const void* rot_dev, uint64_t seed,
                        void* blob_dev, size_t blob_bytes, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!shape_ok(shape) || !choice_ok(shape, c) || !x_dev || !rot_dev || !blob_dev) return JOLT_EINVAL;
  const bool tucker = c.r_T > 0;
  if (tucker && (!U_T_dev || !U_D_dev || ld_T < c.r_T || ld_D < c.r_D || !ws_dev)) return JOLT_EINVAL;
  const BlobLayout L = blob_layout(shape->H, shape->T, shape->D, c);
  if (blob_bytes < L.total) return JOLT_ENOSPACE;
  if (tucker && ws_bytes < jolt_encode_workspace_bytes(shape, c)) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t H = shape->H, T = shape->T, D = shape->D, rT = c.r_T, rD = c.r_D;
    const int xdt = shape->dtype == JOLT_BF16 ? kBF16 : kF32;
    char* blob = static_cast<char*>(blob_dev);
    uint16_t* Ut = reinterpret_cast<uint16_t*>(blob + L.ut);
    uint16_t* Ud = reinterpret_cast<uint16_t*>(blob + L.ud);
    uint16_t* G = reinterpret_cast<uint16_t*>(blob + L.g);
    const int64_t rTp = enc_rtp(c.r_T);
    uint16_t* W2 = static_cast<uint16_t*>(ws_dev);
    float* P = reinterpret_cast<float*>(static_cast<char*>(ws_dev) + a256(4ull * H * D * rTp));
    const size_t n = static_cast<size_t>(D) * D;
    const uint16_t* Q3 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(rot_dev) + 2 * a256(4 * n) +
                                                           a256(2 * n));
    if (tucker) {
      ck(launch_to_bf16(U_T_dev, ld_T, Ut, T, rT, s));
      ck(launch_to_bf16(U_D_dev, ld_D, Ud, D, rD, s));
      // P = U~_T^T X_(T): P[j][h*D + d] = (U~_T^T X_h)[j][d], all heads in one
      // product (r_T x HD, K = T tokens), split along K for parallelism
      GemmArgs g = gemm0();
      g.M = rT; g.N = H * D; g.K = T;
      g.A = Ut; g.a_dtype = kBF16; g.am = plain(1); g.ak = plain(rT);
      g.B = x_dev; g.b_dtype = xdt; g.bk = plain(D); g.bn = segmented(D, T * D, 1);
      g.C = P; g.c_m = H * D; g.c_n = 1;
      g.ksplit = encode_ksplit(T);
      g.partial = P + a256(4ull * H * rT * D) / 4;
      ck(launch_gemm(g, 1, s));
      GemmArgs g2 = gemm0();                     // G~_h = bf16(P_h U~_D)  (r_T x r_D)
      g2.M = rT; g2.N = rD; g2.K = D;
      g2.A = P; g2.am = plain(H * D); g2.ak = plain(1); g2.a_batch = D;
      g2.B = Ud; g2.b_dtype = kBF16; g2.bk = plain(rD); g2.bn = plain(1); g2.b_batch = 0;
      g2.C = G; g2.c_dtype = kBF16; g2.c_m = rD; g2.c_n = 1; g2.c_batch = rT * rD;
      ck(launch_gemm(g2, static_cast<int>(H), s));
      // W_h = G~_h U~_D^T in two bf16 parts (hi, lo), [part][h][d][k]
      ck(launch_enc_w(nullptr, nullptr, G, Ud, W2, 0, 1, static_cast<int>(H), static_cast<int>(rT),
                      static_cast<int>(rD), static_cast<int>(rTp), s));
    }
    EncodeArgs ea{};
    ea.X = x_dev; ea.x_dtype = xdt; ea.H = H; ea.T = T;
    ea.Ut = tucker ? Ut : nullptr; ea.W2 = tucker ? W2 : nullptr; ea.r_T = rT; ea.r_Tp = tucker ? rTp : 0;
    ea.Q3 = Q3; ea.bits = c.bits;
    ea.scales = reinterpret_cast<uint16_t*>(blob + L.sc);
    ea.codes = reinterpret_cast<uint8_t*>(blob + L.cd);
    if (prof_enabled("encode_residual")) {
      const PathWork pw = residual_work(H, T, D, c, xdt == kBF16 ? 2 : 4);
      prof_add_work("encode_residual", pw.bytes - 2.0 * (D * rD + H * rT * rD), pw.flops);
    }
    ck(launch_encode_residual(ea, s));
    ck(launch_write_header(blob, record_head(H, T, D, shape->dtype, c, seed), s));
    return JOLT_OK;
  });
}

size_t jolt_encode_many_workspace_bytes(int32_t n, const jolt_shape* shape, const jolt_choice* choices) {
  if (n < 0 || !shape_ok(shape) || (n > 0 && !choices)) return 0;
  for (int i = 0; i < n; ++i)
    if (!choice_ok(shape, choices[i])) return 0;
  return enc_many_layout(n, shape, choices).total;
}

jolt_status jolt_encode_many(int32_t n, const jolt_shape* shape, const jolt_choice* choices,
                             const void* const* x_dev, const float* const* U_T_dev, const int32_t* ld_T,
                             const float* const* U_D_dev, const int32_t* ld_D, const void* rot_dev, uint64_t seed,
                             void* const* blob_dev, const size_t* blob_bytes, void* ws_dev, size_t ws_bytes,
                             void* stream) {
  if (n < 0 || !shape_ok(shape) || !rot_dev) return JOLT_EINVAL;
  if (n == 0) return JOLT_OK;
  if (!choices || !x_dev || !blob_dev || !blob_bytes) return JOLT_EINVAL;
  for (int i = 0; i < n; ++i) {
    const jolt_choice c = choices[i];
    if (!choice_ok(shape, c) || !x_dev[i] || !blob_dev[i]) return JOLT_EINVAL;
    if (c.r_T > 0 && (!U_T_dev || !U_D_dev || !ld_T || !ld_D || !U_T_dev[i] || !U_D_dev[i] || ld_T[i] < c.r_T ||
                      ld_D[i] < c.r_D))
      return JOLT_EINVAL;
    if (blob_bytes[i] < blob_layout(shape->H, shape->T, shape->D, c).total) return JOLT_ENOSPACE;
  }
  const EncManyLayout L = enc_many_layout(n, shape, choices);
  if (!ws_dev || ws_bytes < L.total) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t H = shape->H, T = shape->T, D = shape->D, HD = H * D;
    const int xdt = shape->dtype == JOLT_BF16 ? kBF16 : kF32;
    char* ws = static_cast<char*>(ws_dev);
    const size_t nq = static_cast<size_t>(D) * D;
    const uint16_t* Q3 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(rot_dev) + 2 * a256(4 * nq) +
                                                           a256(2 * nq));
    bool al16 = true;
    for (int i = 0; i < n; ++i)
      al16 = al16 && (reinterpret_cast<uintptr_t>(x_dev[i]) & 15) == 0 && (reinterpret_cast<uintptr_t>(blob_dev[i]) & 15) == 0;
    auto blob = [&](int i) { return static_cast<char*>(blob_dev[i]); };
    auto lay = [&](int i) { return blob_layout(H, T, D, choices[i]); };
    // host images of the pointer arrays, the residual arguments and the header words
    std::vector<const void*> ptr(L.n_ptrs, nullptr);
    std::vector<EncodeArgs> args(n);
    std::vector<RecordHead> heads(n);
    void** dptr = reinterpret_cast<void**>(ws + L.arr_off);
    EncodeArgs* dargs = reinterpret_cast<EncodeArgs*>(ws + L.arr_off + a256(8 * L.n_ptrs));
    RecordHead* dheads = reinterpret_cast<RecordHead*>(ws + L.arr_off + a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n));
    size_t np = 0;
    auto slots = [&](size_t k) { const size_t o = np; np += k; return o; };
    struct GroupPtrs { size_t ut_in, ut_out, ud_in, ud_out, pa, pb, g2a, g2b, g2c, g3a, g3b; };
    std::vector<GroupPtrs> gp(L.groups.size());
    std::vector<uint16_t*> Wslot(n, nullptr);
    for (size_t g = 0; g < L.groups.size(); ++g) {
      const int b0 = L.groups[g].first, e0 = L.groups[g].second, m = e0 - b0;
      const jolt_choice c = choices[L.order[b0]];
      const int64_t rT = c.r_T, rD = c.r_D;
      GroupPtrs& q = gp[g];
      q.ut_in = slots(m); q.ut_out = slots(m); q.ud_in = slots(m); q.ud_out = slots(m);
      q.pa = slots(m); q.pb = slots(m);
      q.g2a = slots(m * H); q.g2b = slots(m * H); q.g2c = slots(m * H);
      q.g3a = slots(m * H); q.g3b = slots(m * H);
      float* P = reinterpret_cast<float*>(ws + L.p_off[g]);
      uint16_t* W = reinterpret_cast<uint16_t*>(ws + L.w_off[g]);
      const int64_t rTp = enc_rtp(static_cast<int>(rT));
      for (int j = 0; j < m; ++j) {
        const int i = L.order[b0 + j];
        const BlobLayout B = lay(i);
        ptr[q.ut_in + j] = U_T_dev[i];
        ptr[q.ut_out + j] = blob(i) + B.ut;
        ptr[q.ud_in + j] = U_D_dev[i];
        ptr[q.ud_out + j] = blob(i) + B.ud;
        ptr[q.pa + j] = blob(i) + B.ut;
        ptr[q.pb + j] = x_dev[i];
        for (int64_t h = 0; h < H; ++h) {
          const size_t k = static_cast<size_t>(j) * H + h;
          ptr[q.g2a + k] = P + static_cast<size_t>(j) * rT * HD + h * D;
          ptr[q.g2b + k] = blob(i) + B.ud;
          ptr[q.g2c + k] = blob(i) + B.g + 2ull * h * rT * rD;
          ptr[q.g3a + k] = blob(i) + B.g + 2ull * h * rT * rD;
          ptr[q.g3b + k] = blob(i) + B.ud;
        }
        Wslot[i] = W + static_cast<size_t>(j) * 2 * H * D * rTp;
      }
    }
    const size_t blob_slot = slots(n);
    for (int i = 0; i < n; ++i) {
      const jolt_choice c = choices[i];
      const BlobLayout B = lay(i);
      ptr[blob_slot + i] = blob(i);
      EncodeArgs& ea = args[i];
      ea = EncodeArgs{};
      ea.X = x_dev[i]; ea.x_dtype = xdt; ea.H = H; ea.T = T;
      ea.Ut = c.r_T > 0 ? reinterpret_cast<const uint16_t*>(blob(i) + B.ut) : nullptr;
      ea.W2 = Wslot[i]; ea.r_T = c.r_T; ea.r_Tp = c.r_T > 0 ? enc_rtp(c.r_T) : 0;
      ea.Q3 = Q3; ea.bits = c.bits;
      ea.scales = reinterpret_cast<uint16_t*>(blob(i) + B.sc);
      ea.codes = reinterpret_cast<uint8_t*>(blob(i) + B.cd);
      heads[i] = record_head(H, T, D, shape->dtype, c, seed);
    }
    // one upload of the host images, staged in pinned memory (the copy runs
    // ahead of the launches below without holding the host)
    CallHip stage;
    {
      const size_t nb = a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n) + a256(sizeof(RecordHead) * n);
      char* img = static_cast<char*>(stage.pinned(nb));
      std::memcpy(img, ptr.data(), 8 * L.n_ptrs);
      std::memcpy(img + a256(8 * L.n_ptrs), args.data(), sizeof(EncodeArgs) * n);
      std::memcpy(img + a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n), heads.data(), sizeof(RecordHead) * n);
      ck(hipMemcpyAsync(dptr, img, nb, hipMemcpyHostToDevice, s));
      stage.copied(img, s);
    }
    auto dp = [&](size_t slot) { return dptr + slot; };
    for (size_t g = 0; g < L.groups.size(); ++g) {
      const int b0 = L.groups[g].first, e0 = L.groups[g].second, m = e0 - b0;
      const int i0 = L.order[b0];
      const jolt_choice c = choices[i0];
      const int64_t rT = c.r_T, rD = c.r_D;
      const GroupPtrs& q = gp[g];
      // one ld per group is required by the batched casts: tensors of a group share it or go one by one
      bool same_ld = true;
      for (int j = 0; j < m; ++j)
        same_ld = same_ld && ld_T[L.order[b0 + j]] == ld_T[i0] && ld_D[L.order[b0 + j]] == ld_D[i0];
      if (same_ld) {
        ck(launch_to_bf16_many(reinterpret_cast<const float* const*>(dp(q.ut_in)), ld_T[i0],
                               reinterpret_cast<uint16_t* const*>(dp(q.ut_out)), T, rT, m, s));
        ck(launch_to_bf16_many(reinterpret_cast<const float* const*>(dp(q.ud_in)), ld_D[i0],
                               reinterpret_cast<uint16_t* const*>(dp(q.ud_out)), D, rD, m, s));
      } else {
        for (int j = 0; j < m; ++j) {
          const int i = L.order[b0 + j];
          ck(launch_to_bf16(U_T_dev[i], ld_T[i], reinterpret_cast<uint16_t*>(blob(i) + lay(i).ut), T, rT, s));
          ck(launch_to_bf16(U_D_dev[i], ld_D[i], reinterpret_cast<uint16_t*>(blob(i) + lay(i).ud), D, rD, s));
        }
      }
      float* P = reinterpret_cast<float*>(ws + L.p_off[g]);
      GemmArgs g1 = gemm0();                    // P = U~_T^T X_(T) per tensor (as in jolt_encode)
      g1.M = rT; g1.N = HD; g1.K = T;
      g1.a_ptrs = reinterpret_cast<const void* const*>(dp(q.pa)); g1.a_dtype = kBF16;
      g1.am = plain(1); g1.ak = plain(rT);
      g1.b_ptrs = reinterpret_cast<const void* const*>(dp(q.pb)); g1.b_dtype = xdt;
      g1.bk = plain(D); g1.bn = segmented(D, T * D, 1);
      g1.ptr_align16 = al16 ? 1 : 0;
      g1.C = P; g1.c_m = HD; g1.c_n = 1; g1.c_batch = rT * HD;
      g1.ksplit = encode_ksplit(T);
      g1.partial = reinterpret_cast<float*>(ws + L.part_off[g]);
      // many tensors give enough tiles: the split's chunks are summed inside
      // each workgroup (the same arithmetic as jolt_encode's split launch)
      g1.split_seq = 1;
      ck(launch_gemm(g1, m, s));
      GemmArgs g2 = gemm0();                    // G~_h = bf16(P_h U~_D) per (tensor, head)
      g2.M = rT; g2.N = rD; g2.K = D;
      g2.a_ptrs = reinterpret_cast<const void* const*>(dp(q.g2a)); g2.am = plain(HD); g2.ak = plain(1);
      g2.b_ptrs = reinterpret_cast<const void* const*>(dp(q.g2b)); g2.b_dtype = kBF16;
      g2.bk = plain(rD); g2.bn = plain(1);
      g2.c_ptrs = reinterpret_cast<void* const*>(dp(q.g2c)); g2.c_dtype = kBF16; g2.c_m = rD; g2.c_n = 1;
      g2.ptr_align16 = al16 ? 1 : 0;
      ck(launch_gemm(g2, static_cast<int>(m * H), s));
      // W_h = G~_h U~_D^T per (tensor, head), in two bf16 parts (hi, lo)
      const int64_t rTp = enc_rtp(static_cast<int>(rT));
      ck(launch_enc_w(reinterpret_cast<const uint16_t* const*>(dp(q.g3a)),
                      reinterpret_cast<const uint16_t* const*>(dp(q.g3b)), nullptr, nullptr,
                      reinterpret_cast<uint16_t*>(ws + L.w_off[g]), 2 * H * D * rTp, m, static_cast<int>(H),
                      static_cast<int>(rT), static_cast<int>(rD), static_cast<int>(rTp), s));
    }
    if (prof_enabled("encode_residual")) {
      // the residual kernel reads X and U~_T and writes codes and scales (the
      // core and U~_D enter through W, formed beforehand)
      double by = 0.0, fl = 0.0;
      for (int i = 0; i < n; ++i) {
        const PathWork pw = residual_work(H, T, D, choices[i], xdt == kBF16 ? 2 : 4);
        by += pw.bytes - 2.0 * (D * choices[i].r_D + H * choices[i].r_T * choices[i].r_D);
        fl += pw.flops;
      }
      prof_add_work("encode_residual", by, fl);
    }
    ck(launch_encode_residual_many(dargs, n, H, T, xdt, s));
    ck(launch_write_headers(reinterpret_cast<uint32_t* const*>(dp(blob_slot)), dheads, n, s));
    return JOLT_OK;
  });
}

jolt_status jolt_decode(const jolt_shape* shape, jolt_choice c, const void* blob_dev, size_t blob_bytes,
                        const void* rot_dev, void* xhat_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!shape_ok(shape) || !choice_ok(shape, c) || !blob_dev || !rot_dev || !xhat_dev) return JOLT_EINVAL;
  if (blob_bytes < blob_layout(shape->H, shape->T, shape->D, c).total) return JOLT_ENOSPACE;
  const size_t need = decode_ws_one(shape, c);
  if (need > 0 && (!ws_dev || ws_bytes < need)) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    decode_records(1, shape, &c, &blob_dev, rot_dev, &xhat_dev, ws_dev, need, static_cast<hipStream_t>(stream));
    return JOLT_OK;
  });
}

jolt_status jolt_decode_many(int32_t n, const jolt_shape* shape, const jolt_choice* choices,
                             const void* const* blobs, const size_t* blob_bytes, const void* rot_dev,
                             void* const* outs, void* ws_dev, size_t ws_bytes, void* stream) {
  if (n < 0 || !shape_ok(shape) || !rot_dev) return JOLT_EINVAL;
  if (n == 0) return JOLT_OK;
  if (!choices || !blobs || !blob_bytes || !outs) return JOLT_EINVAL;
  for (int i = 0; i < n; ++i) {
    if (!choice_ok(shape, choices[i]) || !blobs[i] || !outs[i]) return JOLT_EINVAL;
    if (blob_bytes[i] < blob_layout(shape->H, shape->T, shape->D, choices[i]).total) return JOLT_ENOSPACE;
  }
  const size_t need = jolt_decode_many_workspace_bytes(n, shape, choices);
  if (!ws_dev || ws_bytes < need) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    decode_records(n, shape, choices, blobs, rot_dev, outs, ws_dev, need, static_cast<hipStream_t>(stream));
    return JOLT_OK;
  });
}

// ---------------------------------------------- cross-layer SVD baseline
// Workspace: per-tensor feature Grams and their split-K partials, the summed
// Gram, its eigenvectors, the eigensolver's scratch, eigenvalues, status.
struct XlLayout {
  size_t gram, part, gsum, Z, syev, lam, status, total;
  int ksplit;
};
XlLayout xl_layout(int n, const jolt_shape* sh, int r) {
  XlLayout L{};
  const int64_t D = sh->D, K = static_cast<int64_t>(sh->H) * sh->T;
  L.ksplit = static_cast<int>(std::min<int64_t>(32, std::max<int64_t>(1, (K + 4095) / 4096)));
  size_t off = 0;
  L.gram = off; off += a256(4ull * n * D * D);
  L.part = off; off += a256(4ull * n * L.ksplit * D * D);
  L.gsum = off; off += a256(4ull * D * D);
  L.Z = off; off += a256(4ull * D * D);
  L.syev = off; off += a256(syev_top_work_bytes(D, r, 1));
  L.lam = off; off += a256(8ull * r);
  L.status = off; off += 256;
  L.total = off;
  return L;
}

size_t jolt_xl_workspace_bytes(int32_t n, const jolt_shape* shape, int32_t r) {
  if (n < 1 || !shape_ok(shape) || r < 1 || r > shape->D) return 0;
  return xl_layout(n, shape, r).total;
}

jolt_status jolt_xl_encode(int32_t n, const jolt_shape* shape, const void* const* x_dev, int32_t r,
                           void* basis_dev, void* const* coeff_dev, double* lam_host, void* ws_dev,
                           size_t ws_bytes, void* stream) {
  if (n < 1 || !shape_ok(shape) || r < 1 || r > shape->D || !x_dev || !basis_dev || !coeff_dev || !ws_dev)
    return JOLT_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!x_dev[i] || !coeff_dev[i]) return JOLT_EINVAL;
  const XlLayout L = xl_layout(n, shape, r);
  if (ws_bytes < L.total) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t H = shape->H, T = shape->T, D = shape->D;
    const int xdt = shape->dtype == JOLT_BF16 ? kBF16 : kF32;
    char* ws = static_cast<char*>(ws_dev);
    float* gram = reinterpret_cast<float*>(ws + L.gram);
    float* gsum = reinterpret_cast<float*>(ws + L.gsum);
    float* Z = reinterpret_cast<float*>(ws + L.Z);
    double* lam = reinterpret_cast<double*>(ws + L.lam);
    int* status = reinterpret_cast<int*>(ws + L.status);
    uint16_t* basis = static_cast<uint16_t*>(basis_dev);
    ck(hipMemsetAsync(status, 0, sizeof(int), s));
    for (int i = 0; i < n; ++i) {           // feature Gram of tensor i: X_(D) X_(D)^T over H T rows
      GemmArgs g = gemm0();
      g.A = x_dev[i]; g.B = x_dev[i]; g.a_dtype = g.b_dtype = xdt;
      g.M = D; g.N = D; g.K = H * T;
      g.am = plain(1); g.ak = plain(D); g.bk = plain(D); g.bn = plain(1);
      g.C = gram + static_cast<size_t>(i) * D * D; g.c_m = D; g.c_n = 1;
      g.ksplit = L.ksplit;
      g.partial = reinterpret_cast<float*>(ws + L.part) + static_cast<size_t>(i) * L.ksplit * D * D;
      ck(launch_gemm(g, 1, s, "gram"));
    }
    ck(launch_sum_batch(gram, D * D, n, gsum, s));
    ck(syev_top(gsum, D, 1, r, Z, lam, ws + L.syev, s, status));
    // basis bf16 [r][D]: row j = eigenvector j (column j of the column-major Z)
    ck(launch_to_bf16(Z, D, basis, r, D, s));
    for (int i = 0; i < n; ++i) {           // C_i = bf16(X_i U~)  ([H T][r])
      GemmArgs g = gemm0();
      g.A = x_dev[i]; g.a_dtype = xdt; g.am = plain(D); g.ak = plain(1);
      g.B = basis; g.b_dtype = kBF16; g.bk = plain(1); g.bn = plain(D);
      g.M = H * T; g.N = r; g.K = D;
      g.C = coeff_dev[i]; g.c_dtype = kBF16; g.c_m = r; g.c_n = 1;
      ck(launch_gemm(g, 1, s));
    }
    std::vector<double> lh(r);
    int st = 0;
    ck(hipMemcpyAsync(lh.data(), lam, sizeof(double) * r, hipMemcpyDeviceToHost, s));
    ck(hipMemcpyAsync(&st, status, sizeof(int), hipMemcpyDeviceToHost, s));
    ck(hipStreamSynchronize(s));
    if (st != 0) return JOLT_EHIP;
    if (lam_host) std::memcpy(lam_host, lh.data(), sizeof(double) * r);
    return JOLT_OK;
  });
}

jolt_status jolt_xl_decode(int32_t n, const jolt_shape* shape, int32_t r, const void* basis_dev,
                           const void* const* coeff_dev, void* const* out_dev, void* stream) {
  if (n < 0 || !shape_ok(shape) || r < 1 || r > shape->D) return JOLT_EINVAL;
  if (n == 0) return JOLT_OK;
  if (!basis_dev || !coeff_dev || !out_dev) return JOLT_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!coeff_dev[i] || !out_dev[i]) return JOLT_EINVAL;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t H = shape->H, T = shape->T, D = shape->D;
    for (int i = 0; i < n; ++i) {           // X^_i = C_i U~^T, in the input dtype
      GemmArgs g = gemm0();
      g.A = coeff_dev[i]; g.a_dtype = kBF16; g.am = plain(r); g.ak = plain(1);
      g.B = basis_dev; g.b_dtype = kBF16; g.bk = plain(D); g.bn = plain(1);
      g.M = H * T; g.N = D; g.K = r;
      g.C = out_dev[i]; g.c_dtype = shape->dtype == JOLT_BF16 ? kBF16 : kF32; g.c_m = D; g.c_n = 1;
      ck(launch_gemm(g, 1, s));
    }
    return JOLT_OK;
  });
}

// -------------------------------------------------- appended tokens (fold-in)
// Workspace: W fp32 [r_T][H D], M = W W^T (padded to rp = ceil32(r_T)), its
// eigenvectors Z [rp][rp] (column-major), eigenvalues fp64, pseudo-inverse
// scales fp32, B = X_new W^T and P = B Z diag(1/lambda) [dT][rp], U_new fp32
// [dT][r_T], the eigensolver's scratch, the encoder's W parts, status.
struct AppendLayout {
  size_t W, M, Z, lam, inv, B, P, U, syev, W2, status, total;
  int64_t rp;
};
AppendLayout append_layout(const jolt_shape* sh, int32_t dT, jolt_choice c) {
  AppendLayout L{};
  const int64_t HD = static_cast<int64_t>(sh->H) * sh->D;
  L.rp = (static_cast<int64_t>(c.r_T) + 31) / 32 * 32;
  size_t off = 0;
  L.W = off; off += a256(4ull * c.r_T * HD);
  L.M = off; off += a256(4ull * L.rp * L.rp);
  L.Z = off; off += a256(4ull * L.rp * L.rp);
  L.lam = off; off += a256(8ull * L.rp);
  L.inv = off; off += a256(4ull * L.rp);
  L.B = off; off += a256(4ull * dT * L.rp);
  L.P = off; off += a256(4ull * dT * L.rp);
  L.U = off; off += a256(4ull * dT * c.r_T);
  L.syev = off; off += a256(syev_top_work_bytes(L.rp, static_cast<int>(L.rp), 1));
  L.W2 = off; off += a256(4ull * sh->H * sh->D * enc_rtp(c.r_T));
  L.status = off; off += 256;
  L.total = off;
  return L;
}

size_t jolt_append_workspace_bytes(const jolt_shape* base, jolt_choice choice, int32_t n_new) {
  if (!shape_ok(base) || !choice_ok(base, choice) || choice.r_T < 1 || n_new < 1) return 0;
  return append_layout(base, n_new, choice).total;
}

jolt_status jolt_append(const jolt_shape* base, jolt_choice choice, const void* base_blob, size_t base_bytes,
                        const void* x_new_dev, int32_t n_new, const void* rot_dev, uint64_t seed, void* blob_dev,
                        size_t blob_bytes, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!shape_ok(base) || !choice_ok(base, choice) || choice.r_T < 1 || n_new < 1) return JOLT_EINVAL;
  if (!base_blob || !x_new_dev || !rot_dev || !blob_dev || !ws_dev) return JOLT_EINVAL;
  const int64_t H = base->H, T = base->T, D = base->D, HD = H * D, dT = n_new;
  const int64_t rT = choice.r_T, rD = choice.r_D;
  const BlobLayout B0 = blob_layout(H, T, D, choice), B1 = blob_layout(H, dT, D, choice);
  if (base_bytes < B0.total || blob_bytes < B1.total) return JOLT_ENOSPACE;
  const AppendLayout L = append_layout(base, n_new, choice);
  if (ws_bytes < L.total) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int xdt = base->dtype == JOLT_BF16 ? kBF16 : kF32;
    char* ws = static_cast<char*>(ws_dev);
    const char* b0 = static_cast<const char*>(base_blob);
    char* b1 = static_cast<char*>(blob_dev);
    float* W = reinterpret_cast<float*>(ws + L.W);
    float* M = reinterpret_cast<float*>(ws + L.M);
    float* Z = reinterpret_cast<float*>(ws + L.Z);
    double* lam = reinterpret_cast<double*>(ws + L.lam);
    float* inv = reinterpret_cast<float*>(ws + L.inv);
    float* Bm = reinterpret_cast<float*>(ws + L.B);
    float* P = reinterpret_cast<float*>(ws + L.P);
    float* U = reinterpret_cast<float*>(ws + L.U);
    int* status = reinterpret_cast<int*>(ws + L.status);
    const int64_t rp = L.rp;
    uint16_t* Ut1 = reinterpret_cast<uint16_t*>(b1 + B1.ut);
    uint16_t* Ud1 = reinterpret_cast<uint16_t*>(b1 + B1.ud);
    uint16_t* G1 = reinterpret_cast<uint16_t*>(b1 + B1.g);
    ck(hipMemsetAsync(status, 0, sizeof(int), s));
    // the new record keeps the base's stored U~_D and G~
    ck(hipMemcpyAsync(Ud1, b0 + B0.ud, 2ull * D * rD, hipMemcpyDeviceToDevice, s));
    ck(hipMemcpyAsync(G1, b0 + B0.g, 2ull * H * rT * rD, hipMemcpyDeviceToDevice, s));
    {                                         // W[:, h D ..] = G~_h U~_D^T  (r_T x D per head)
      GemmArgs g = gemm0();
      g.M = rT; g.N = D; g.K = rD;
      g.A = G1; g.a_dtype = kBF16; g.am = plain(rD); g.ak = plain(1); g.a_batch = rT * rD;
      g.B = Ud1; g.b_dtype = kBF16; g.bk = plain(1); g.bn = plain(rD); g.b_batch = 0;
      g.C = W; g.c_m = HD; g.c_n = 1; g.c_batch = D;
      ck(launch_gemm(g, static_cast<int>(H), s));
    }
    ck(hipMemsetAsync(M, 0, 4ull * rp * rp, s));
    {                                         // M = W W^T (r_T x r_T inside rp x rp zeros)
      GemmArgs g = gemm0();
      g.M = rT; g.N = rT; g.K = HD;
      g.A = W; g.am = plain(HD); g.ak = plain(1);
      g.B = W; g.bk = plain(1); g.bn = plain(HD);
      g.C = M; g.c_m = rp; g.c_n = 1;
      ck(launch_gemm(g, 1, s));
    }
    {                                         // B = X_new,(T) W^T  (dT x r_T, row stride rp)
      GemmArgs g = gemm0();
      g.M = dT; g.N = rT; g.K = HD;
      g.A = x_new_dev; g.a_dtype = xdt; g.am = plain(D); g.ak = segmented(D, dT * D, 1);
      g.B = W; g.bk = plain(1); g.bn = plain(HD);
      g.C = Bm; g.c_m = rp; g.c_n = 1;
      ck(launch_gemm(g, 1, s));
    }
    // M = Z diag(lambda) Z^T, its padding to rp a diagonal block at the top
    // of the spectrum (B has zeros there, so it adds nothing); 1/lambda,
    // guarding only non-positive eigenvalues: the normal equations in fp32
    // resolve the smallest eigenvalues of these systems (a few 1e-6 of the
    // largest) to well under 1%, and the error each direction adds scales
    // with the new tokens' small projection on it
    ck(launch_pad_diag(M, rT, rp, s));
    ck(syev_top(M, rp, 1, static_cast<int>(rp), Z, lam, ws + L.syev, s, status));
    ck(launch_pinv_scale(lam, rp, 0x1p-40, inv, s));
    {                                         // P = B Z diag(inv)
      GemmArgs g = gemm0();
      g.M = dT; g.N = rp; g.K = rT;
      g.A = Bm; g.am = plain(rp); g.ak = plain(1);
      g.B = Z; g.bk = plain(1); g.bn = plain(rp);
      g.col_scale = inv;
      g.C = P; g.c_m = rp; g.c_n = 1;
      ck(launch_gemm(g, 1, s));
    }
    {                                         // U_new = P Z^T restricted to r_T columns
      GemmArgs g = gemm0();
      g.M = dT; g.N = rT; g.K = rp;
      g.A = P; g.am = plain(rp); g.ak = plain(1);
      g.B = Z; g.bk = plain(rp); g.bn = plain(1);
      g.C = U; g.c_m = rT; g.c_n = 1;
      ck(launch_gemm(g, 1, s));
    }
    ck(launch_to_bf16(U, rT, Ut1, dT, rT, s));
    // the residual against the stored parts, rotated and quantized
    const int64_t rTp = enc_rtp(choice.r_T);
    uint16_t* W2 = reinterpret_cast<uint16_t*>(ws + L.W2);
    ck(launch_enc_w(nullptr, nullptr, G1, Ud1, W2, 0, 1, static_cast<int>(H), static_cast<int>(rT),
                    static_cast<int>(rD), static_cast<int>(rTp), s));
    const size_t n = static_cast<size_t>(D) * D;
    EncodeArgs ea{};
    ea.X = x_new_dev; ea.x_dtype = xdt; ea.H = H; ea.T = dT;
    ea.Ut = Ut1; ea.W2 = W2; ea.r_T = rT; ea.r_Tp = rTp;
    ea.Q3 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(rot_dev) + 2 * a256(4 * n) + a256(2 * n));
    ea.bits = choice.bits;
    ea.scales = reinterpret_cast<uint16_t*>(b1 + B1.sc);
    ea.codes = reinterpret_cast<uint8_t*>(b1 + B1.cd);
    ck(launch_encode_residual(ea, s));
    ck(launch_write_header(b1, record_head(H, dT, D, base->dtype, choice, seed), s));
    int st = 0;
    ck(hipMemcpyAsync(&st, status, sizeof(int), hipMemcpyDeviceToHost, s));
    ck(hipStreamSynchronize(s));
    return st != 0 ? JOLT_EHIP : JOLT_OK;
  });
}

// ------------------------------------------------- decode fused into attention
struct AttnLayout {
  size_t wk, wv, part, total;
  int n_blk, nq;
};
AttnLayout attn_layout(const jolt_shape* sh, jolt_choice ck, jolt_choice cv, int G, int n_new) {
  AttnLayout L{};
  L.nq = G * n_new;
  L.n_blk = static_cast<int>((static_cast<int64_t>(sh->T) + 255) / 256);
  size_t off = 0;
  L.wk = off; off += a256(decode_w_bytes(sh->H, sh->D, ck));
  L.wv = off; off += a256(decode_w_bytes(sh->H, sh->D, cv));
  L.part = off; off += a256(4ull * sh->H * L.nq * L.n_blk * (sh->D + 2));
  L.total = off + 256;
  return L;
}

bool attn_args_ok(const jolt_shape* sh, jolt_choice ck, jolt_choice cv, int G, int n_new) {
  return shape_ok(sh) && choice_ok(sh, ck) && choice_ok(sh, cv) && G >= 1 && n_new >= 1 &&
         static_cast<int64_t>(G) * n_new <= kAttnMaxQ;
}

size_t jolt_attend_workspace_bytes(const jolt_shape* shape, jolt_choice choice_k, jolt_choice choice_v, int32_t G,
                                   int32_t n_new) {
  if (!attn_args_ok(shape, choice_k, choice_v, G, n_new)) return 0;
  return attn_layout(shape, choice_k, choice_v, G, n_new).total;
}

jolt_status jolt_attend(const jolt_shape* shape, jolt_choice choice_k, const void* blob_k, size_t blob_k_bytes,
                        jolt_choice choice_v, const void* blob_v, size_t blob_v_bytes, const void* rot_dev,
                        const float* q_dev, int32_t G, int32_t n_new, float* out_dev, void* ws_dev,
                        size_t ws_bytes, void* stream) {
  if (!attn_args_ok(shape, choice_k, choice_v, G, n_new)) return JOLT_EINVAL;
  if (!blob_k || !blob_v || !rot_dev || !q_dev || !out_dev || !ws_dev) return JOLT_EINVAL;
  const int64_t H = shape->H, T = shape->T, D = shape->D;
  if (blob_k_bytes < blob_layout(H, T, D, choice_k).total || blob_v_bytes < blob_layout(H, T, D, choice_v).total)
    return JOLT_ENOSPACE;
  const AttnLayout L = attn_layout(shape, choice_k, choice_v, G, n_new);
  if (ws_bytes < L.total) return JOLT_ENOSPACE;
  return guard([&]() -> jolt_status {
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(ws_dev);
    const size_t n2 = static_cast<size_t>(D) * D;
    DecBatch b{};
    b.n = 2;
    b.H = static_cast<int32_t>(H);
    b.T = static_cast<int32_t>(T);
    b.rec[0] = dec_rec(H, T, D, choice_k, blob_k, nullptr, ws + L.wk, 0);
    b.rec[1] = dec_rec(H, T, D, choice_v, blob_v, nullptr, ws + L.wv,
                       static_cast<int>(H * (b.rec[0].r_Tp / 32)));
    b.wtiles_total = static_cast<int>(H * (b.rec[0].r_Tp / 32 + b.rec[1].r_Tp / 32));
    ck(launch_make_w(b, s));
    AttnArgs a{};
    a.k = b.rec[0];
    a.v = b.rec[1];
    a.Qt16 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(rot_dev) + 2 * a256(4 * n2));
    a.q = q_dev;
    a.out = out_dev;
    a.part = reinterpret_cast<float*>(ws + L.part);
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(D)));
    a.H = static_cast<int32_t>(H); a.T = static_cast<int32_t>(T);
    a.G = G; a.n_new = n_new; a.nq = L.nq; a.n_blk = L.n_blk;
    if (prof_enabled("attend")) {
      // the two records read once, the queries read and the outputs written
      // once; the two reconstructions and 4 D flops per (query vector, token)
      const int e = shape->dtype == JOLT_BF16 ? 2 : 4;
      const PathWork pk = residual_work(H, T, D, choice_k, e), pv = residual_work(H, T, D, choice_v, e);
      const double xbytes = 2.0 * static_cast<double>(H * T * D) * e;    // the inputs / outputs counted there
      prof_add_work("attend", pk.bytes + pv.bytes - xbytes + 8.0 * H * L.nq * D,
                    pk.flops + pv.flops + 4.0 * H * L.nq * static_cast<double>(T) * D);
    }
    ck(launch_attn_decode(a, s));
    return JOLT_OK;
  });
}

size_t jolt_decode_static_scratch_bytes(void) { return kStaticScratchBytes; }

jolt_status jolt_decode_many_static(int32_t n, const jolt_shape* shape, const jolt_choice* choices,
                                    const void* const* blobs, const size_t* blob_bytes, const void* rot_dev,
                                    void* const* outs, void* stream) {
  if (n < 0 || !shape_ok(shape) || !rot_dev) return JOLT_EINVAL;
  if (n == 0) return JOLT_OK;
  if (!choices || !blobs || !blob_bytes || !outs) return JOLT_EINVAL;
  for (int i = 0; i < n; ++i) {
    if (!choice_ok(shape, choices[i]) || !blobs[i] || !outs[i]) return JOLT_EINVAL;
    if (blob_bytes[i] < blob_layout(shape->H, shape->T, shape->D, choices[i]).total) return JOLT_ENOSPACE;
    if (decode_w_bytes(shape->H, shape->D, choices[i]) > kStaticScratchBytes) return JOLT_ENOSPACE;
  }
  return guard([&]() -> jolt_status {
    decode_records(n, shape, choices, blobs, rot_dev, outs, static_scratch(), kStaticScratchBytes,
                   static_cast<hipStream_t>(stream));
    return JOLT_OK;
  });
}

jolt_status jolt_quantize(const float* y_dev, int64_t rows, int32_t D, int32_t bits, void* scales_dev,
                          void* codes_dev, void* stream) {
  if (rows < 0 || D != kD || bits < 1 || bits > 4) return JOLT_EINVAL;
  if (rows == 0) return JOLT_OK;                       // nothing to do; pointers may be NULL
  if (!y_dev || !scales_dev || !codes_dev) return JOLT_EINVAL;
  return guard([&]() -> jolt_status {
    // fp32 rows read once, b-bit codes and the bf16 (offset, step) pair per group written once
    prof_add_work("quantize", static_cast<double>(rows) * D * (4.0 + (bits + 1) / 8.0), 0.0);
    ck(launch_quantize(y_dev, rows, bits, static_cast<uint16_t*>(scales_dev),
                       static_cast<uint8_t*>(codes_dev), static_cast<hipStream_t>(stream)));
    return JOLT_OK;
  });
}

jolt_status jolt_header_parse(const void* header, size_t bytes, jolt_shape* shape, jolt_choice* choice,
                              uint64_t* seed) {
  if (!header || bytes < 64) return JOLT_EINVAL;
  uint32_t w[16];
  std::memcpy(w, header, 64);
  if (w[0] != kMagic || w[1] != kVersion || w[9] != static_cast<uint32_t>(kGroup)) return JOLT_EFORMAT;
  jolt_shape s{static_cast<int32_t>(w[2]), static_cast<int32_t>(w[3]), static_cast<int32_t>(w[4]),
               static_cast<int32_t>(w[5])};
  jolt_choice c{static_cast<int32_t>(w[6]), static_cast<int32_t>(w[7]), static_cast<int32_t>(w[8])};
  if (!shape_ok(&s) || !choice_ok(&s, c)) return JOLT_EFORMAT;
  if (shape) *shape = s;
  if (choice) *choice = c;
  if (seed) *seed = static_cast<uint64_t>(w[10]) | (static_cast<uint64_t>(w[11]) << 32);
  return JOLT_OK;
}

const char* jolt_status_str(jolt_status s) {
  switch (s) {
    case JOLT_OK: return "ok";
    case JOLT_EINVAL: return "invalid argument";
    case JOLT_ENOSPACE: return "buffer too small";
    case JOLT_EBUDGET: return "byte budget below the cheapest plan";
    case JOLT_ERANGE: return "non-finite input";
    case JOLT_EFORMAT: return "bad record header";
    case JOLT_EHIP: return "HIP runtime error";
    case JOLT_ENODEV: return "no usable device";
  }
  return "unknown status";
}

int32_t jolt_version(void) { return static_cast<int32_t>(kVersion); }

void jolt_debug_chase_wait_limit(int32_t polls) { set_chase_spin_limit(polls < 0 ? (1 << 22) : polls); }

jolt_status jolt_profile_enable(const char* kernels) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (hipDeviceSynchronize() != hipSuccess) return JOLT_EHIP;   // no recorded event in flight
  prof_release();
  if (!kernels || !*kernels) {
    g_prof_sel.clear();
  } else if (std::strcmp(kernels, "*") == 0) {
    g_prof_sel = "*";
  } else {
    g_prof_sel = std::string(",") + kernels + ",";
    g_prof_sel.erase(std::remove(g_prof_sel.begin(), g_prof_sel.end(), ' '), g_prof_sel.end());
  }
  return JOLT_OK;
}

jolt_status jolt_profile_query(const char* kernel, jolt_kernel_stats* out) {
  if (!kernel || !out) return JOLT_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess) return JOLT_EHIP;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  auto it = g_prof.find(kernel);
  jolt_kernel_stats st{0, 0.0, 0.0, 0.0};
  if (it != g_prof.end()) {
    const ProfRec& r = it->second;
    st.launches = static_cast<int64_t>(r.ev.size());
    for (const auto& e : r.ev) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_pool[e.first], g_pool[e.second]) != hipSuccess) return JOLT_EHIP;
      st.total_ms += ms;
    }
    st.bytes = r.bytes;
    st.flops = r.flops;
  }
  *out = st;
  return JOLT_OK;
}

}  // extern "C"
