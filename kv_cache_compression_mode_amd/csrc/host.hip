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

using namespace jolt;

// ------------------------------------------------------------- profiling
namespace jolt {
namespace {
struct ProfRec {
  std::vector<std::pair<int, int>> ev;   // indices into the event pool
  double bytes = 0, flops = 0;           // host-side accounting
  std::vector<std::pair<unsigned long long*, int64_t>> slots;   // device [count][2] counters
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
  for (auto& kv : g_prof)
    for (auto& sl : kv.second.slots) (void)hipFree(sl.first);
  g_prof.clear();
  g_pool_used = 0;
}
}  // namespace

bool prof_enabled(const char* name) {
  if (g_prof_sel.empty()) return false;
  return g_prof_sel == "*" || g_prof_sel.find("," + std::string(name) + ",") != std::string::npos;
}

unsigned long long* prof_slots(const char* name, int64_t count) {
  if (!prof_enabled(name) || count <= 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec& r = g_prof[name];
  if (r.slots.empty() || r.slots.back().second < count) {
    unsigned long long* p = nullptr;
    const size_t bytes = static_cast<size_t>(count) * 2 * sizeof(unsigned long long);
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    if (hipMemset(p, 0, bytes) != hipSuccess) { (void)hipFree(p); return nullptr; }
    r.slots.emplace_back(p, count);
  }
  return r.slots.back().first;
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
constexpr int kGroup = 32;
constexpr int kD = 128;
// E[(max - min)^2] of 32 iid N(0, 1), by numerical quadrature.
constexpr double kKappa32 = 17.60642599755;
constexpr uint64_t kTagRotation = 0x4A4F4C54524F5431ull;   // "JOLTROT1"
constexpr uint64_t kTagSketch = 0x4A4F4C54534B5431ull;     // "JOLTSKT1"
// Jacobi thresholds: rotate when |a_pq| > max(tau_abs_rel * trace, tau_rel * sqrt(|a_pp a_qq|)).
// An absolute floor near fp32 noise (1e-9 of the trace) keeps the noise-bulk
// eigenvectors accurate: the truncation residual sits in that bulk.
constexpr float kTauRel = 2e-6f;
constexpr float kTauAbsRel = 1e-9f;
constexpr int kMaxSweeps = 30;
// A matrix of the block-Jacobi batch is done once its relative off-diagonal
// Frobenius mass off/fro is below 2^-19, or once it has stopped falling (a
// sweep removes less than 10% of it) after reaching 2^-12: what is left then
// sits in entries below the rotation thresholds (about n * kTauAbsRel * trace
// in total), and further sweeps only rotate pairs at the threshold, which no
// longer moves the leading invariant subspaces or their captured energy.
constexpr double kOffRel = 1.0 / (1 << 19);
constexpr double kOffStall = 1.0 / (1 << 12);
constexpr double kOffStallRatio = 0.9;

struct HipFail {};
inline void ck(hipError_t e) {
  if (e != hipSuccess) throw HipFail{};
}

size_t a256(size_t n) { return (n + 255) / 256 * 256; }

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

// ------------------------------------------------------------ byte model
struct BlobLayout {
  size_t ut, ud, g, sc, cd, total;
};
BlobLayout blob_layout(int64_t H, int64_t T, int64_t D, jolt_choice c) {
  const size_t groups = static_cast<size_t>(H * T * D / kGroup);
  BlobLayout L{};
  L.ut = 256;
  L.ud = L.ut + a256(2ull * T * c.r_T);
  L.g = L.ud + a256(2ull * D * c.r_D);
  L.sc = L.g + a256(2ull * H * c.r_T * c.r_D);
  L.cd = L.sc + a256(4ull * groups);
  L.total = L.cd + a256(4ull * c.bits * groups);
  return L;
}

bool shape_ok(const jolt_shape* s) {
  return s && s->H >= 1 && s->T >= 1 && s->D == kD && (s->dtype == JOLT_BF16 || s->dtype == JOLT_F32);
}
bool choice_ok(const jolt_shape* s, jolt_choice c) {
  if (c.bits < 1 || c.bits > 4) return false;
  if (c.r_T == 0 && c.r_D == 0) return true;
  const int64_t nT = std::min<int64_t>(s->T, static_cast<int64_t>(s->H) * s->D);
  return c.r_T >= 1 && c.r_T <= nT && c.r_D >= 1 && c.r_D <= s->D;
}

// ---------------------------------------------------------- the dual
int rank_cap_T(int64_t H, int64_t T, int64_t D, double ratio, int step) {
  const double N = static_cast<double>(H * T * D);
  const double bbar = 2.0 * N / ratio;
  const int64_t q = static_cast<int64_t>(std::floor(bbar / (4.0 * static_cast<double>(T))));
  return static_cast<int>(std::min<int64_t>(std::min<int64_t>(T, H * D), (q / step) * step));
}
int numerical_rank(const double* lam, int len, int64_t n) {
  if (len <= 0 || !(lam[0] > 0.0)) return 0;
  const double thr = static_cast<double>(n) * 0x1p-52 * lam[0];
  int c = 0;
  for (int i = 0; i < len; ++i) c += lam[i] > thr;
  return c;
}
double rho(int bits) {
  const int L = (1 << bits) - 1;
  return kKappa32 / (12.0 * static_cast<double>(L * L));
}

struct Pt {
  int64_t bytes;
  double dist;
  int idx;
};
struct Seg {
  double slope;
  int unit;
  int64_t start;
  int k;
};

int steps_T(const jolt_alloc_req* r) { return r->step_T > 0 ? r->step_T : 32; }
int steps_D(const jolt_alloc_req* r) { return r->step_D > 0 ? r->step_D : 16; }
int cap_of(const jolt_alloc_req* r) {
  const jolt_shape& s = r->shape;
  return r->r_T_cap > 0 ? r->r_T_cap : rank_cap_T(s.H, s.T, s.D, r->budget_ratio, steps_T(r));
}

bool req_ok(const jolt_alloc_req* r) {
  if (!r || !shape_ok(&r->shape) || r->n_layers < 1 || r->group_layers < 1) return false;
  if (!(r->budget_ratio > 0.0) || !std::isfinite(r->budget_ratio)) return false;
  if (r->n_bits < 1 || r->n_bits > 4) return false;
  for (int i = 0; i < r->n_bits; ++i)
    if (r->bit_menu[i] < 1 || r->bit_menu[i] > 4) return false;
  if (r->method != JOLT_EXACT && r->method != JOLT_FLASH) return false;
  if (r->method == JOLT_FLASH && (r->oversample < 0 || r->power_iters < 0)) return false;
  const int64_t nT = std::min<int64_t>(r->shape.T, static_cast<int64_t>(r->shape.H) * r->shape.D);
  const int cap = cap_of(r);
  return cap >= 0 && cap <= nT && cap <= 2048;
}

jolt_status plan_dual(const jolt_alloc_req* req, const double* spT, int lenT, const double* spD,
                      const double* frob2, jolt_plan* plan) {
  const jolt_shape& s = req->shape;
  const int L = req->n_layers, G = req->group_layers;
  const int64_t N = static_cast<int64_t>(s.H) * s.T * s.D;
  const int64_t n_total = N * 2 * L;
  const int64_t budget = static_cast<int64_t>(std::floor(2.0 * static_cast<double>(n_total) / req->budget_ratio));
  const int cap = cap_of(req);
  const int64_t nT = std::min<int64_t>(s.T, static_cast<int64_t>(s.H) * s.D);
  const int sT = steps_T(req), sD = steps_D(req);
  const int n_groups = (L + G - 1) / G;
  // prefix sums of every tensor's spectra, accumulated in index order from
  // 0.0: the residual energy max(0, ||X||^2 - sum_{i<r} lambda_i) in O(1) per choice
  const int ntens = 2 * L;
  std::vector<double> preT(static_cast<size_t>(ntens) * (lenT + 1)), preD(static_cast<size_t>(ntens) * (s.D + 1));
  for (int t = 0; t < ntens; ++t) {
    double* pt = preT.data() + static_cast<size_t>(t) * (lenT + 1);
    double* pd = preD.data() + static_cast<size_t>(t) * (s.D + 1);
    pt[0] = 0.0;
    for (int i = 0; i < lenT; ++i) pt[i + 1] = pt[i] + spT[static_cast<size_t>(t) * lenT + i];
    pd[0] = 0.0;
    for (int i = 0; i < s.D; ++i) pd[i + 1] = pd[i] + spD[static_cast<size_t>(t) * s.D + i];
  }
  auto tail_T = [&](int t, double f2, int r) {
    return std::max(0.0, f2 - preT[static_cast<size_t>(t) * (lenT + 1) + std::min(r, lenT)]);
  };
  auto tail_D = [&](int t, double f2, int r) {
    return std::max(0.0, f2 - preD[static_cast<size_t>(t) * (s.D + 1) + std::min(r, static_cast<int>(s.D))]);
  };
  struct Unit {
    int first, last;
    std::vector<jolt_choice> menu;
    std::vector<Pt> hull;
  };
  std::vector<Unit> units;
  for (int g = 0; g < n_groups; ++g) {
    for (int kind = 0; kind < 2; ++kind) {
      Unit u;
      u.first = g * G;
      u.last = std::min(L, (g + 1) * G);
      int RT = cap, RD = s.D;
      for (int l = u.first; l < u.last; ++l) {
        const int t = l * 2 + kind;
        RT = std::min(RT, numerical_rank(spT + static_cast<size_t>(t) * lenT, lenT, nT));
        RD = std::min(RD, numerical_rank(spD + static_cast<size_t>(t) * s.D, s.D, s.D));
      }
      for (int b = 0; b < req->n_bits; ++b) u.menu.push_back({0, 0, req->bit_menu[b]});
      for (int rt = sT; rt <= RT; rt += sT)
        for (int rd = sD; rd <= RD; rd += sD)
          for (int b = 0; b < req->n_bits; ++b) u.menu.push_back({rt, rd, req->bit_menu[b]});
      std::vector<Pt> pts;
      for (int i = 0; i < static_cast<int>(u.menu.size()); ++i) {
        const jolt_choice c = u.menu[i];
        const int64_t nb = static_cast<int64_t>(u.last - u.first) *
                           static_cast<int64_t>(blob_layout(s.H, s.T, s.D, c).total);
        double dist = 0.0;
        for (int l = u.first; l < u.last; ++l) {
          const int t = l * 2 + kind;
          const double f2 = frob2[t];
          if (!(f2 > 0.0)) continue;
          const double e = (tail_T(t, f2, c.r_T) + tail_D(t, f2, c.r_D)) / f2;
          dist += rho(c.bits) * std::min(1.0, e);
        }
        pts.push_back({nb, dist, i});
      }
      std::sort(pts.begin(), pts.end(), [](const Pt& a, const Pt& b) {
        if (a.bytes != b.bytes) return a.bytes < b.bytes;
        if (a.dist != b.dist) return a.dist < b.dist;
        return a.idx < b.idx;
      });
      for (const Pt& p : pts) {
        if (!u.hull.empty() && p.dist >= u.hull.back().dist) continue;
        while (u.hull.size() >= 2) {
          const Pt& a = u.hull[u.hull.size() - 2];
          const Pt& b = u.hull.back();
          const double cross = static_cast<double>(b.bytes - a.bytes) * (p.dist - a.dist) -
                               (b.dist - a.dist) * static_cast<double>(p.bytes - a.bytes);
          if (cross <= 0.0) u.hull.pop_back();
          else break;
        }
        u.hull.push_back(p);
      }
      units.push_back(std::move(u));
    }
  }
  std::vector<int> pos(units.size(), 0);
  int64_t total = 0;
  for (const Unit& u : units) total += u.hull[0].bytes;
  if (total > budget) return JOLT_EBUDGET;
  std::vector<Seg> segs;
  for (int ui = 0; ui < static_cast<int>(units.size()); ++ui) {
    const auto& h = units[ui].hull;
    for (int k = 0; k + 1 < static_cast<int>(h.size()); ++k) {
      const double dB = static_cast<double>(h[k + 1].bytes - h[k].bytes);
      const double dD = h[k].dist - h[k + 1].dist;
      segs.push_back({dD / dB, ui, h[k].bytes, k});
    }
  }
  std::sort(segs.begin(), segs.end(), [](const Seg& a, const Seg& b) {
    if (a.slope != b.slope) return a.slope > b.slope;
    if (a.unit != b.unit) return a.unit < b.unit;
    return a.start < b.start;
  });
  for (const Seg& sg : segs) {
    const auto& h = units[sg.unit].hull;
    if (pos[sg.unit] != sg.k) break;   // cannot happen on a strictly convex hull
    const int64_t step = h[sg.k + 1].bytes - h[sg.k].bytes;
    if (total + step > budget) break;
    total += step;
    pos[sg.unit] = sg.k + 1;
  }
  double obj = 0.0;
  for (int ui = 0; ui < static_cast<int>(units.size()); ++ui) {
    const Unit& u = units[ui];
    const Pt& p = u.hull[pos[ui]];
    const jolt_choice c = u.menu[p.idx];
    plan->choice[ui] = c;
    obj += p.dist;
    if (plan->tensor_bytes)
      for (int l = u.first; l < u.last; ++l)
        plan->tensor_bytes[l * 2 + (ui & 1)] = blob_layout(s.H, s.T, s.D, c).total;
  }
  plan->objective = obj;
  plan->total_bytes = static_cast<uint64_t>(total);
  plan->budget_bytes = static_cast<uint64_t>(budget);
  plan->r_T_cap = cap;
  return JOLT_OK;
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
  bool x16;            // every input tensor is 16-byte aligned
  // scratch (chunk tensors)
  float* G; float* V; float* J; int* active; int* rot; float* tauabs; double* offp;
  float* GDpart;
  void* syev;
  void* syevD;
  float* GD; float* GDc; float* VD;
  int* order; float* Ucm; float* Vr; float* P; double* lam_tmp; float* qtau; int* perm; float* sgn;
  float* Om; float* Y; float* Z; float* Bm; float* Wr; float* Wd;
  // the feature-mode factor's own scratch (it runs beside the token path)
  float* qtauD; double* lamDt; int* permD; float* sgnD;
  size_t bytes;
  int chunk;
  int nlanes;          // scratch sets, one per stream (chunks alternate between them)
  hipEvent_t band_done;  // recorded once the token eigensolver's band reduction is queued
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

bool eig_jacobi();

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
  if (!d.flash && d.R > 0) per += syev_top_work_bytes(d.n_pad, static_cast<int>(d.R), 1);
  // up to 64 tensors (24 GiB of scratch) in flight.  Token eigenproblems of
  // n >= 2048 go in two lanes of half chunks: there the stages around the
  // chase are throughput-bound and overlap it; at smaller n they are
  // latency-bound, and halving the batch only doubles their count (the
  // Jacobi and randomized paths keep one lane).
  int chunk = static_cast<int>(std::max<size_t>(1, std::min<size_t>(64, (24ull << 30) / per)));
  chunk = std::min(chunk, nt);
  const int nlanes = (chunk >= 2 && !eig_jacobi() && !d.flash && d.R > 0 && d.n_pad >= 2048) ? 2 : 1;
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
  w.frob2 = c.take<double>(nt);
  w.xptrs = c.take<const void*>(nt);
  w.tags = c.take<uint64_t>(nt);
  const int64_t n = d.flash ? d.ell_pad : d.n_pad;
  auto scratch = [&](AllocWS& w) {
    w.G = c.take<float>(static_cast<size_t>(chunk) * n * n);
    w.V = c.take<float>(static_cast<size_t>(chunk) * n * n);
    w.J = c.take<float>(static_cast<size_t>(chunk) * (n / 64) * 64 * 64);
    w.active = c.take<int>(static_cast<size_t>(chunk) * (n / 64));
    w.rot = c.take<int>(chunk);
    w.tauabs = c.take<float>(chunk);
    w.offp = c.take<double>(static_cast<size_t>(chunk) * kOffBlocks * 2);
    w.GDpart = c.take<float>(static_cast<size_t>(chunk) * gram_d_ksplit(d) * d.D * d.D);
    w.syevD = c.take<char>(syev_top_work_bytes(d.D, static_cast<int>(d.D), chunk));
    w.syev = (!d.flash && d.R > 0)
                 ? static_cast<void*>(c.take<char>(syev_top_work_bytes(d.n_pad, static_cast<int>(d.R), chunk)))
                 : nullptr;
    w.GD = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.GDc = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.VD = c.take<float>(static_cast<size_t>(chunk) * d.D * d.D);
    w.order = c.take<int>(static_cast<size_t>(chunk) * std::max<int64_t>(R, d.D));
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
  };
  scratch(w);
  if (nlanes > 1) {
    AllocWS w1 = w;
    scratch(w1);
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

// Jacobi to convergence on `batch` n x n matrices in w.G (V -> w.V); host loop
// over sweeps, stopping when a sweep applies no rotation.
// The token Gram's eigensolver: two-stage tridiagonal reduction by default,
// block Jacobi with JOLT_EIG=jacobi.
bool eig_jacobi() {
  static const bool on = [] {
    const char* e = std::getenv("JOLT_EIG");
    return e && std::strcmp(e, "jacobi") == 0;
  }();
  return on;
}

bool trace_on() {
  static const bool on = [] {
    const char* e = std::getenv("JOLT_TRACE");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

void run_jacobi(float* A, float* V, int64_t n, int batch, const AllocWS& w, hipStream_t s) {
  JacobiWork jw{A, V, n, batch, w.J, w.active, w.rot, w.tauabs};
  ck(jacobi_init(jw, kTauAbsRel, s));
  const int nb = static_cast<int>(n / 32);
  std::vector<int> cnt(batch);
  std::vector<float> tau(batch);
  std::vector<double> part(static_cast<size_t>(batch) * kOffBlocks * 2);
  std::vector<char> done(batch, 0);
  std::vector<double> prev(batch, INFINITY);
  ck(hipMemcpyAsync(tau.data(), w.tauabs, sizeof(float) * batch, hipMemcpyDeviceToHost, s));
  auto t_prev = std::chrono::steady_clock::now();
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    ck(hipMemsetAsync(w.rot, 0, sizeof(int) * batch, s));
    for (int r = 0; r < nb - 1; ++r) ck(jacobi_round(jw, r, kTauRel, s));
    ck(jacobi_offnorm(A, n, batch, w.offp, s));
    ck(hipMemcpyAsync(cnt.data(), w.rot, sizeof(int) * batch, hipMemcpyDeviceToHost, s));
    ck(hipMemcpyAsync(part.data(), w.offp, sizeof(double) * part.size(), hipMemcpyDeviceToHost, s));
    ck(hipStreamSynchronize(s));
    int64_t tot = 0;
    int busy = 0, newly = 0;
    double worst = 0.0;
    for (int z = 0; z < batch; ++z) {
      tot += cnt[z];
      busy += cnt[z] != 0;
      double off2 = 0.0, dia2 = 0.0;
      for (int b = 0; b < kOffBlocks; ++b) {
        off2 += part[(static_cast<size_t>(z) * kOffBlocks + b) * 2];
        dia2 += part[(static_cast<size_t>(z) * kOffBlocks + b) * 2 + 1];
      }
      const double rel = off2 > 0.0 ? std::sqrt(off2 / (off2 + dia2)) : 0.0;
      worst = std::max(worst, rel);
      const bool stalled = rel <= kOffStall && rel >= kOffStallRatio * prev[z];
      prev[z] = rel;
      if (!done[z] && (rel <= kOffRel || stalled)) {
        done[z] = 1;
        tau[z] = INFINITY;          // no pair of this matrix rotates again
        ++newly;
      }
    }
    if (trace_on()) {
      const auto now = std::chrono::steady_clock::now();
      std::fprintf(stderr,
                   "[jolt] jacobi n=%lld batch=%d sweep %d: %lld rotations, %d matrices busy, "
                   "max off/fro %.3e, %.3f ms\n",
                   static_cast<long long>(n), batch, sweep, static_cast<long long>(tot), busy, worst,
                   std::chrono::duration<double, std::milli>(now - t_prev).count());
      t_prev = now;
    }
    if (!tot || std::all_of(done.begin(), done.end(), [](char c) { return c != 0; })) break;
    if (newly) ck(hipMemcpyAsync(w.tauabs, tau.data(), sizeof(float) * batch, hipMemcpyHostToDevice, s));
  }
}

// A second stream per device (default priority) for the feature-mode factor,
// which depends only on the feature Gram and runs beside the token path; fork
// and join through events.  Created on first use, kept for the process.
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
AuxStream& aux_stream() {
  static std::vector<AuxStream> per_dev;
  int dev = 0;
  ck(hipGetDevice(&dev));
  if (static_cast<int>(per_dev.size()) <= dev) per_dev.resize(dev + 1);
  AuxStream& a = per_dev[dev];
  if (!a.s) {
    ck(hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking));
    ck(hipEventCreateWithFlags(&a.fork, hipEventDisableTiming));
    ck(hipEventCreateWithFlags(&a.join, hipEventDisableTiming));
  }
  return a;
}
// The second lane's stream (non-blocking, default priority) and its fork / join events.
AuxStream& lane_stream() {
  static std::vector<AuxStream> per_dev;
  int dev = 0;
  ck(hipGetDevice(&dev));
  if (static_cast<int>(per_dev.size()) <= dev) per_dev.resize(dev + 1);
  AuxStream& a = per_dev[dev];
  if (!a.s) {
    ck(hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking));
    ck(hipEventCreateWithFlags(&a.fork, hipEventDisableTiming));
    ck(hipEventCreateWithFlags(&a.join, hipEventDisableTiming));
  }
  return a;
}
// Events marking each chunk's band reduction (grown on demand, kept per device).
hipEvent_t* lane_marks(int count) {
  static std::vector<std::vector<hipEvent_t>> per_dev;
  int dev = 0;
  ck(hipGetDevice(&dev));
  if (static_cast<int>(per_dev.size()) <= dev) per_dev.resize(dev + 1);
  std::vector<hipEvent_t>& v = per_dev[dev];
  while (static_cast<int>(v.size()) < count) {
    hipEvent_t e;
    ck(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    v.push_back(e);
  }
  return v.data();
}
// Runs the feature-mode factor on the auxiliary stream after the work queued
// on s so far (the tridiagonal path; the Jacobi path shares scratch and stays
// on s); join() makes s wait for it.
struct FeatureFork {
  AuxStream* a = nullptr;
  hipStream_t s;
  explicit FeatureFork(hipStream_t s_) : s(s_) {}
  hipStream_t start() {
    if (eig_jacobi()) return s;
    a = &aux_stream();
    ck(hipEventRecord(a->fork, s));
    ck(hipStreamWaitEvent(a->s, a->fork, 0));
    return a->s;
  }
  void done() {
    if (a) ck(hipEventRecord(a->join, a->s));
  }
  void join() {
    if (a) ck(hipStreamWaitEvent(s, a->join, 0));
    a = nullptr;
  }
};

// Feature-mode factor of `batch` tensors from their D x D Grams in w.GD.
void feature_factor(const Dims& d, int batch, int t0, const AllocWS& w, hipStream_t s) {
  const int64_t D = d.D;
  ck(hipMemcpyAsync(w.GDc, w.GD, sizeof(float) * batch * D * D, hipMemcpyDeviceToDevice, s));
  if (eig_jacobi()) {
    ck(jacobi_small128(w.GD, w.VD, batch, kTauRel, kTauAbsRel, kMaxSweeps, s));
    ck(topk_diag(w.GD, D, batch, static_cast<int>(D), w.order, s));
    ck(launch_gather_cols(w.VD, D, D * D, w.order, D, w.Vr, D, D * D, D, D, batch, s));
  } else {
    ck(syev_top(w.GD, D, batch, static_cast<int>(D), w.Vr, nullptr, w.syevD, s));
  }
  ck(householder_qr(w.Vr, D, D, D, D * D, batch, w.qtauD, s));
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
// orthonormal column-major U (T x R), then sort/sign/emit.
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

void analyze_exact(const Dims& d, int batch, int t0, const AllocWS& w, int xdt, hipStream_t s) {
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
  g.c_lower = eig_jacobi() ? 0 : 1;
  ck(launch_gemm(g, batch, s));
  if (d.dual) {
    ck(launch_sum_diag_blocks(w.G, d.H, D, w.GD, batch, s));   // n == HD here
  } else {
    GemmArgs gd = gemm0();
    gd.a_ptrs = xp; gd.b_ptrs = xp; gd.a_dtype = gd.b_dtype = xdt; gd.ptr_align16 = w.x16;
    gd.M = D; gd.N = D; gd.K = d.H * T;
    gd.am = plain(1); gd.ak = plain(D); gd.bk = plain(D); gd.bn = plain(1);
    gd.C = w.GD; gd.c_m = D; gd.c_n = 1; gd.c_batch = D * D;
    gd.ksplit = gram_d_ksplit(d); gd.partial = w.GDpart;
    ck(launch_gemm(gd, batch, s));
  }
  FeatureFork ff(s);
  feature_factor(d, batch, t0, w, ff.start());
  ff.done();
  if (R == 0) {
    ff.join();
    return;
  }
  // leading eigenvectors V_R of the token Gram, column-major with leading dimension ldv
  const float* VR;
  int64_t ldv, vr_batch;
  bool in_ucm = false;
  if (eig_jacobi()) {
    run_jacobi(w.G, w.V, n, batch, w, s);
    ck(topk_diag(w.G, n, batch, static_cast<int>(R), w.order, s));
    if (d.dual) {     // n == HD
      ck(launch_gather_cols(w.V, n, n * n, w.order, R, w.Vr, HD, HD * R, HD, R, batch, s));
    } else {
      ck(launch_gather_cols(w.V, n, n * n, w.order, R, w.Ucm, T, T * R, T, R, batch, s));
      in_ucm = true;
    }
    VR = w.Vr; ldv = HD; vr_batch = HD * R;
  } else {
    ck(syev_top(w.G, n, batch, static_cast<int>(R), w.V, nullptr, w.syev, s, w.band_done));
    VR = w.V; ldv = n; vr_batch = n * n;
  }
  if (in_ucm) {
  } else if (d.dual) {
    // U' = X_(T) V_R (T x R, column-major)
    GemmArgs gu = gemm0();
    gu.a_ptrs = xp; gu.a_dtype = xdt; gu.ptr_align16 = w.x16;
    gu.M = T; gu.N = R; gu.K = HD;
    gu.am = plain(D); gu.ak = segmented(D, T * D, 1);
    gu.B = VR; gu.bk = plain(1); gu.bn = plain(ldv); gu.b_batch = vr_batch;
    gu.C = w.Ucm; gu.c_m = 1; gu.c_n = T; gu.c_batch = T * R;
    ck(launch_gemm(gu, batch, s));
  } else {
    ck(copy_cols(VR, ldv, vr_batch, w.Ucm, T, T * R, T, R, batch, s));
  }
  ck(householder_qr(w.Ucm, T, R, T, T * R, batch, w.qtau, s));
  token_finalize(d, batch, t0, w, xdt, s);
  ff.join();
}

void analyze_flash(const Dims& d, int batch, int t0, const AllocWS& w, int xdt, int q, uint64_t seed,
                   hipStream_t s) {
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
    ck(launch_gemm(gd, batch, s));
  }
  FeatureFork ff(s);
  feature_factor(d, batch, t0, w, ff.start());
  ff.done();
  if (R == 0) {
    ff.join();
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
  AY(w.Om, ell, true, w.Y);
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
  run_jacobi(w.G, w.V, ep, batch, w, s);
  ck(topk_diag(w.G, ep, batch, static_cast<int>(R), w.order, s));
  ck(launch_gather_cols(w.V, ep, ep * ep, w.order, R, w.Wr, ell, ell * R, ell, R, batch, s));
  {
    GemmArgs g = gemm0();                       // U = Q W_R (T x R, column-major)
    g.M = T; g.N = R; g.K = ell;
    g.A = w.Y; g.am = plain(1); g.ak = plain(T); g.a_batch = T * ell;
    g.B = w.Wr; g.bk = plain(1); g.bn = plain(ell); g.b_batch = ell * R;
    g.C = w.Ucm; g.c_m = 1; g.c_n = T; g.c_batch = T * R;
    ck(launch_gemm(g, batch, s));
  }
  ck(householder_qr(w.Ucm, T, R, T, T * R, batch, w.qtau, s));
  token_finalize(d, batch, t0, w, xdt, s);
  ff.join();
}

int64_t rtp_of(int r_T) { return (static_cast<int64_t>(r_T) + 31) / 32 * 32; }
// the encoder's W parts: k padded to whole 64-value chunks
int64_t enc_rtp(int r_T) { return (static_cast<int64_t>(r_T) + 63) / 64 * 64; }

size_t decode_ws_one(const jolt_shape* s, jolt_choice c) {
  if (c.r_T == 0) return 0;
  return 2 * a256(2ull * s->H * s->D * rtp_of(c.r_T));
}

// Decode n records of one shape, kDecBatch per launch pair (W prologue + decode).
void decode_records(int n, const jolt_shape* shape, const jolt_choice* ch, const void* const* blobs,
                    const void* rot_dev, void* const* outs, void* ws, hipStream_t s) {
  const int64_t H = shape->H, T = shape->T, D = shape->D;
  const size_t n2 = static_cast<size_t>(D) * D;
  const uint16_t* Qt16 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(rot_dev) + 2 * a256(4 * n2));
  char* wsp = static_cast<char*>(ws);
  for (int i0 = 0; i0 < n; i0 += kDecBatch) {
    DecBatch b{};
    b.n = std::min(kDecBatch, n - i0);
    b.H = static_cast<int32_t>(H);
    b.T = static_cast<int32_t>(T);
    b.out_dtype = shape->dtype == JOLT_BF16 ? kBF16 : kF32;
    b.Qt16 = Qt16;
    int wtiles = 0;
    for (int j = 0; j < b.n; ++j) {
      const jolt_choice c = ch[i0 + j];
      const BlobLayout L = blob_layout(H, T, D, c);
      const char* blob = static_cast<const char*>(blobs[i0 + j]);
      DecRec& R = b.rec[j];
      R.Ut = reinterpret_cast<const uint16_t*>(blob + L.ut);
      R.Ud = reinterpret_cast<const uint16_t*>(blob + L.ud);
      R.G = reinterpret_cast<const uint16_t*>(blob + L.g);
      R.scales = reinterpret_cast<const uint32_t*>(blob + L.sc);
      R.codes = reinterpret_cast<const uint32_t*>(blob + L.cd);
      R.out = outs[i0 + j];
      R.r_T = c.r_T; R.r_D = c.r_D; R.bits = c.bits;
      R.r_Tp = static_cast<int32_t>(rtp_of(c.r_T));
      const size_t wb = a256(2ull * H * D * R.r_Tp);
      R.Whi = reinterpret_cast<uint16_t*>(wsp);
      R.Wlo = reinterpret_cast<uint16_t*>(wsp + (c.r_T ? wb : 0));
      wsp += c.r_T ? 2 * wb : 0;
      R.wtile0 = wtiles;
      wtiles += static_cast<int>(H * (R.r_Tp / 32));
    }
    b.out16 = 1;
    for (int j = 0; j < b.n; ++j) b.out16 &= (reinterpret_cast<uintptr_t>(b.rec[j].out) & 15) == 0 ? 1 : 0;
    b.wtiles_total = wtiles;
    ck(launch_decode_batch(b, s));
  }
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
    off += a256(6ull * m * H * D * enc_rtp(static_cast<int>(rT)));
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
  off += a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n) + a256(4ull * 16 * n);
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
  return a256(6ull * shape->H * shape->D * enc_rtp(c.r_T)) + w + a256(w * encode_ksplit(shape->T)) + 256;
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(q_dev);
    ck(hipMemcpyAsync(base, buf.data(), 4 * n, hipMemcpyHostToDevice, s));
    ck(hipMemcpyAsync(base + a256(4 * n), buf.data() + n, 4 * n, hipMemcpyHostToDevice, s));
    ck(hipMemcpyAsync(base + 2 * a256(4 * n), b16.data(), 2 * n, hipMemcpyHostToDevice, s));
    ck(hipMemcpyAsync(base + 2 * a256(4 * n) + a256(2 * n), q3.data(), 6 * n, hipMemcpyHostToDevice, s));
    ck(hipStreamSynchronize(s));
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
    const int64_t N = d.H * d.T * d.D;
    ck(hipMemsetAsync(w.frob2, 0, sizeof(double) * nt, s));
    // every tensor's pointer and sketch tag, uploaded once
    std::vector<const void*> ptrs(x_dev, x_dev + nt);
    std::vector<uint64_t> tags(nt);
    for (int t = 0; t < nt; ++t)
      tags[t] = kTagSketch ^ ((static_cast<uint64_t>(t / 2) << 8) | static_cast<uint64_t>(t % 2));
    ck(hipMemcpyAsync(w.xptrs, ptrs.data(), sizeof(void*) * nt, hipMemcpyHostToDevice, s));
    ck(hipMemcpyAsync(w.tags, tags.data(), sizeof(uint64_t) * nt, hipMemcpyHostToDevice, s));
    ck(hipStreamSynchronize(s));
    // chunks alternate between the lanes: lane 0 on s, lane 1 on a second
    // stream forked from s and joined back into it
    AuxStream* ls = nullptr;
    if (w.nlanes > 1 && nt > w.chunk) {
      ls = &lane_stream();
      ck(hipEventRecord(ls->fork, s));
      ck(hipStreamWaitEvent(ls->s, ls->fork, 0));
    }
    // a chunk on the second lane starts once the previous chunk's band
    // reduction is queued ahead of it, so that chunk's chase (one CU per
    // tensor) runs beside this chunk's matrix-core stages
    hipEvent_t* marks = ls ? lane_marks(nt / w.chunk + 1) : nullptr;
    for (int t0 = 0, c = 0; t0 < nt; t0 += w.chunk, ++c) {
      const int batch = std::min(w.chunk, nt - t0);
      const bool second = ls && (c & 1);
      AllocWS wl = second ? w1 : w;
      hipStream_t sl = second ? ls->s : s;
      wl.xptrs = w.xptrs + t0;
      wl.tags = w.tags + t0;
      wl.band_done = marks ? marks[c] : nullptr;
      if (marks && c > 0) ck(hipStreamWaitEvent(sl, marks[c - 1], 0));
      ck(launch_sumsq(reinterpret_cast<const void* const*>(wl.xptrs), batch, N, xdt, w.frob2 + t0, sl));
      if (d.flash) analyze_flash(d, batch, t0, wl, xdt, req->power_iters, req->seed, sl);
      else analyze_exact(d, batch, t0, wl, xdt, sl);
    }
    if (ls) {
      ck(hipEventRecord(ls->join, ls->s));
      ck(hipStreamWaitEvent(s, ls->join, 0));
    }
    const int R = static_cast<int>(d.R);
    std::vector<double> lt(static_cast<size_t>(nt) * std::max(R, 1)), ld(static_cast<size_t>(nt) * d.D), f2(nt);
    if (R > 0) ck(hipMemcpyAsync(lt.data(), w.lamT, sizeof(double) * nt * R, hipMemcpyDeviceToHost, s));
    ck(hipMemcpyAsync(ld.data(), w.lamD, sizeof(double) * nt * d.D, hipMemcpyDeviceToHost, s));
    ck(hipMemcpyAsync(f2.data(), w.frob2, sizeof(double) * nt, hipMemcpyDeviceToHost, s));
    ck(hipStreamSynchronize(s));
    for (int i = 0; i < nt; ++i)
      if (!std::isfinite(f2[i])) return JOLT_ERANGE;
    if (plan->spectra_T && R > 0) std::memcpy(plan->spectra_T, lt.data(), sizeof(double) * nt * R);
    if (plan->spectra_D) std::memcpy(plan->spectra_D, ld.data(), sizeof(double) * nt * d.D);
    if (plan->frob2) std::memcpy(plan->frob2, f2.data(), sizeof(double) * nt);
    return plan_dual(req, lt.data(), std::max(R, 1), ld.data(), f2.data(), plan);
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
    uint16_t* W3 = static_cast<uint16_t*>(ws_dev);
    float* P = reinterpret_cast<float*>(static_cast<char*>(ws_dev) + a256(6ull * H * D * rTp));
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
      // W_h = G~_h U~_D^T in three bf16 parts, [part][h][d][k]
      ck(launch_enc_w(nullptr, nullptr, G, Ud, W3, 0, 1, static_cast<int>(H), static_cast<int>(rT),
                      static_cast<int>(rD), static_cast<int>(rTp), s));
    }
    EncodeArgs ea{};
    ea.X = x_dev; ea.x_dtype = xdt; ea.H = H; ea.T = T;
    ea.Ut = tucker ? Ut : nullptr; ea.W3 = tucker ? W3 : nullptr; ea.r_T = rT; ea.r_Tp = tucker ? rTp : 0;
    ea.Q3 = Q3; ea.bits = c.bits;
    ea.scales = reinterpret_cast<uint16_t*>(blob + L.sc);
    ea.codes = reinterpret_cast<uint8_t*>(blob + L.cd);
    ck(launch_encode_residual(ea, s));
    const uint32_t hdr[16] = {kMagic, kVersion, static_cast<uint32_t>(H), static_cast<uint32_t>(T),
                              static_cast<uint32_t>(D), static_cast<uint32_t>(shape->dtype),
                              static_cast<uint32_t>(rT), static_cast<uint32_t>(rD),
                              static_cast<uint32_t>(c.bits), static_cast<uint32_t>(kGroup),
                              static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), 0, 0, 0, 0};
    ck(launch_write_header(blob, hdr, s));
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
    std::vector<uint32_t> words(static_cast<size_t>(16) * n);
    void** dptr = reinterpret_cast<void**>(ws + L.arr_off);
    EncodeArgs* dargs = reinterpret_cast<EncodeArgs*>(ws + L.arr_off + a256(8 * L.n_ptrs));
    uint32_t* dwords = reinterpret_cast<uint32_t*>(ws + L.arr_off + a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n));
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
        Wslot[i] = W + static_cast<size_t>(j) * 3 * H * D * rTp;
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
      ea.W3 = Wslot[i]; ea.r_T = c.r_T; ea.r_Tp = c.r_T > 0 ? enc_rtp(c.r_T) : 0;
      ea.Q3 = Q3; ea.bits = c.bits;
      ea.scales = reinterpret_cast<uint16_t*>(blob(i) + B.sc);
      ea.codes = reinterpret_cast<uint8_t*>(blob(i) + B.cd);
      const uint32_t hdr[16] = {kMagic, kVersion, static_cast<uint32_t>(H), static_cast<uint32_t>(T),
                                static_cast<uint32_t>(D), static_cast<uint32_t>(shape->dtype),
                                static_cast<uint32_t>(c.r_T), static_cast<uint32_t>(c.r_D),
                                static_cast<uint32_t>(c.bits), static_cast<uint32_t>(kGroup),
                                static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), 0, 0, 0, 0};
      std::memcpy(&words[static_cast<size_t>(16) * i], hdr, sizeof(hdr));
    }
    // one upload of the host images (pageable memory: the call copies before returning)
    {
      std::vector<char> img(a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n) + a256(4ull * 16 * n), 0);
      std::memcpy(img.data(), ptr.data(), 8 * L.n_ptrs);
      std::memcpy(img.data() + a256(8 * L.n_ptrs), args.data(), sizeof(EncodeArgs) * n);
      std::memcpy(img.data() + a256(8 * L.n_ptrs) + a256(sizeof(EncodeArgs) * n), words.data(), 4ull * 16 * n);
      ck(hipMemcpyAsync(dptr, img.data(), img.size(), hipMemcpyHostToDevice, s));
      ck(hipStreamSynchronize(s));
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
      // W_h = G~_h U~_D^T per (tensor, head), in three bf16 parts
      const int64_t rTp = enc_rtp(static_cast<int>(rT));
      ck(launch_enc_w(reinterpret_cast<const uint16_t* const*>(dp(q.g3a)),
                      reinterpret_cast<const uint16_t* const*>(dp(q.g3b)), nullptr, nullptr,
                      reinterpret_cast<uint16_t*>(ws + L.w_off[g]), 3 * H * D * rTp, m, static_cast<int>(H),
                      static_cast<int>(rT), static_cast<int>(rD), static_cast<int>(rTp), s));
    }
    ck(launch_encode_residual_many(dargs, n, H, T, xdt, s));
    ck(launch_write_headers(reinterpret_cast<uint32_t* const*>(dp(blob_slot)), dwords, n, s));
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
    decode_records(1, shape, &c, &blob_dev, rot_dev, &xhat_dev, ws_dev, static_cast<hipStream_t>(stream));
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
    decode_records(n, shape, choices, blobs, rot_dev, outs, ws_dev, static_cast<hipStream_t>(stream));
    return JOLT_OK;
  });
}

jolt_status jolt_quantize(const float* y_dev, int64_t rows, int32_t D, int32_t bits, void* scales_dev,
                          void* codes_dev, void* stream) {
  if (rows < 0 || D != kD || bits < 1 || bits > 4) return JOLT_EINVAL;
  if (rows == 0) return JOLT_OK;                       // nothing to do; pointers may be NULL
  if (!y_dev || !scales_dev || !codes_dev) return JOLT_EINVAL;
  return guard([&]() -> jolt_status {
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
    for (const auto& sl : r.slots) {
      std::vector<unsigned long long> c(static_cast<size_t>(sl.second) * 2);
      if (hipMemcpy(c.data(), sl.first, c.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) !=
          hipSuccess)
        return JOLT_EHIP;
      for (size_t i = 0; i < c.size(); i += 2) {
        st.bytes += static_cast<double>(c[i]);
        st.flops += static_cast<double>(c[i + 1]);
      }
    }
  }
  *out = st;
  return JOLT_OK;
}

}  // extern "C"
