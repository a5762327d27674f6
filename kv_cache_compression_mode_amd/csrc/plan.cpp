// The byte model and the Lagrangian-dual allocation (host C++ only, so that
// it also builds with a host compiler and its sanitizers).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <vector>

namespace jolt {
namespace {
// E[(max - min)^2] of 32 iid N(0, 1), by numerical quadrature.
constexpr double kKappa32 = 17.60642599755;
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
}  // namespace

size_t a256(size_t n) { return (n + 255) / 256 * 256; }

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
// r_T is bounded by H D (the token factor's columns span at most the H D
// columns of the token unfolding); a record may hold fewer tokens than r_T
// (tokens appended to an encoded tensor keep its choice).
bool choice_ok(const jolt_shape* s, jolt_choice c) {
  if (c.bits < 1 || c.bits > 4) return false;
  if (c.r_T == 0 && c.r_D == 0) return true;
  return c.r_T >= 1 && c.r_T <= static_cast<int64_t>(s->H) * s->D && c.r_D >= 1 && c.r_D <= s->D;
}

// ---------------------------------------------------------- the dual
int rank_cap_T(int64_t H, int64_t T, int64_t D, double ratio, int step) {
  const double N = static_cast<double>(H * T * D);
  const double bbar = 2.0 * N / ratio;
  const int64_t q = static_cast<int64_t>(std::floor(bbar / (4.0 * static_cast<double>(T))));
  return static_cast<int>(std::min<int64_t>(std::min<int64_t>(T, H * D), (q / step) * step));
}
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
      // the menu runs over (r_T, r_D) with the bit widths innermost: each
      // layer's clipped relative tail is formed once per rank pair and
      // weighted per width, summed over the layers in order
      std::vector<Pt> pts;
      pts.reserve(u.menu.size());
      std::vector<double> clip(static_cast<size_t>(u.last - u.first));
      std::vector<char> live(clip.size());
      for (int i0 = 0; i0 < static_cast<int>(u.menu.size()); i0 += req->n_bits) {
        const jolt_choice c0 = u.menu[i0];
        for (int l = u.first; l < u.last; ++l) {
          const int t = l * 2 + kind;
          const double f2 = frob2[t];
          live[l - u.first] = f2 > 0.0;
          if (f2 > 0.0) clip[l - u.first] = std::min(1.0, (tail_T(t, f2, c0.r_T) + tail_D(t, f2, c0.r_D)) / f2);
        }
        for (int i = i0; i < i0 + req->n_bits; ++i) {
          const jolt_choice c = u.menu[i];
          const int64_t nb = static_cast<int64_t>(u.last - u.first) *
                             static_cast<int64_t>(blob_layout(s.H, s.T, s.D, c).total);
          const double w = rho(c.bits);
          double dist = 0.0;
          for (size_t l = 0; l < clip.size(); ++l)
            if (live[l]) dist += w * clip[l];
          pts.push_back({nb, dist, i});
        }
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

}  // namespace jolt
