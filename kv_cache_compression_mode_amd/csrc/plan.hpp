// The codec's byte model and the Lagrangian-dual allocation of ranks and
// bit widths (host C++, no device code): the record layout every entry point
// sizes buffers with, the request and shape checks, and the planner that
// turns spectra into a plan.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/jolt.h"

namespace jolt {

constexpr int kGroup = 32;        // values per quantization group
constexpr int kD = 128;           // head dimension

size_t a256(size_t n);

// Byte offsets of a record's sections (header 256 B, then U~_T, U~_D, G~,
// scales, codes, each 256-aligned) and its total size.
struct BlobLayout {
  size_t ut, ud, g, sc, cd, total;
};
BlobLayout blob_layout(int64_t H, int64_t T, int64_t D, jolt_choice c);

bool shape_ok(const jolt_shape* s);
bool choice_ok(const jolt_shape* s, jolt_choice c);
bool req_ok(const jolt_alloc_req* r);
int cap_of(const jolt_alloc_req* r);
int rank_cap_T(int64_t H, int64_t T, int64_t D, double ratio, int step);

// The plan from per-tensor spectra (lenT token eigenvalues and D feature
// eigenvalues per tensor, fp64, descending) and squared norms.
jolt_status plan_dual(const jolt_alloc_req* req, const double* spT, int lenT, const double* spD,
                      const double* frob2, jolt_plan* plan);

}  // namespace jolt
