// Host-only driver of the allocation planner (plan.cpp) for a build with the
// host compiler's address and undefined-behaviour sanitizers.
//
// usage: plan_driver H T dtype L G ratio nbits b0 b1 b2 b3 method oversample
//                    r_T_cap step_T step_D lenT spectra.bin
// spectra.bin: fp64 [2L][lenT] token spectra, [2L][128] feature spectra,
// [2L] squared norms.  Prints the status, then (status 0) the plan: total,
// budget, cap, objective (%a, exact), one line per group and kind, the
// bytes of every tensor.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "plan.hpp"

int main(int argc, char** argv) {
  if (argc != 19) {
    std::fprintf(stderr, "expected 18 arguments\n");
    return 2;
  }
  jolt_alloc_req r{};
  r.shape.H = std::atoi(argv[1]);
  r.shape.T = std::atoi(argv[2]);
  r.shape.D = 128;
  r.shape.dtype = std::atoi(argv[3]);
  r.n_layers = std::atoi(argv[4]);
  r.group_layers = std::atoi(argv[5]);
  r.budget_ratio = std::atof(argv[6]);
  r.n_bits = std::atoi(argv[7]);
  for (int i = 0; i < 4; ++i) r.bit_menu[i] = std::atoi(argv[8 + i]);
  r.method = std::atoi(argv[12]);
  r.oversample = std::atoi(argv[13]);
  r.power_iters = 1;
  r.r_T_cap = std::atoi(argv[14]);
  r.step_T = std::atoi(argv[15]);
  r.step_D = std::atoi(argv[16]);
  const int lenT = std::atoi(argv[17]);
  if (!jolt::req_ok(&r) || lenT < 1) {
    std::printf("status %d\n", static_cast<int>(JOLT_EINVAL));
    return 0;
  }
  const int nt = 2 * r.n_layers;
  std::vector<double> sT(static_cast<size_t>(nt) * lenT), sD(static_cast<size_t>(nt) * 128), f2(nt);
  FILE* f = std::fopen(argv[18], "rb");
  if (!f) return 2;
  const bool ok = std::fread(sT.data(), sizeof(double), sT.size(), f) == sT.size() &&
                  std::fread(sD.data(), sizeof(double), sD.size(), f) == sD.size() &&
                  std::fread(f2.data(), sizeof(double), f2.size(), f) == f2.size();
  std::fclose(f);
  if (!ok) return 2;
  const int ng = (r.n_layers + r.group_layers - 1) / r.group_layers;
  std::vector<jolt_choice> choice(static_cast<size_t>(ng) * 2);
  std::vector<uint64_t> tb(nt);
  jolt_plan plan{};
  plan.choice = choice.data();
  plan.tensor_bytes = tb.data();
  const jolt_status st = jolt::plan_dual(&r, sT.data(), lenT, sD.data(), f2.data(), &plan);
  std::printf("status %d\n", static_cast<int>(st));
  if (st != JOLT_OK) return 0;
  std::printf("total %llu budget %llu cap %d objective %a\n", static_cast<unsigned long long>(plan.total_bytes),
              static_cast<unsigned long long>(plan.budget_bytes), plan.r_T_cap, plan.objective);
  for (const jolt_choice& c : choice) std::printf("choice %d %d %d\n", c.r_T, c.r_D, c.bits);
  for (uint64_t b : tb) std::printf("bytes %llu\n", static_cast<unsigned long long>(b));
  return 0;
}
