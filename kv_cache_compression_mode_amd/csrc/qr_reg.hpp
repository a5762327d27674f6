// The register panel QR (Householder, one workgroup of RT threads per
// panel of up to kLeaf rows x 32 columns), shared by the QR routines and the
// band reduction, which runs it inside a fused launch.
#pragma once

#include "device.hpp"

namespace jolt {
namespace {

constexpr int kLeaf = 1024;      // rows of one register panel
constexpr int RT = kLeaf / 2, RW = RT / 64;
struct QrRegLds {
  float xs[kLeaf] __attribute__((aligned(16)));   // column j, rows > j
  float rowj[2][32];                              // row j, by the parity of j
  float red[2][RW][32];                           // per-wave partial dots, by the parity of j
  float St[32][33];                               // St[j][l] = v_l^T v_j (l < j)
  float Tl[32][33];
  float Rl[32][33];                               // rows of R
  float tau_s[32], sgn[32];
};

// The column loop of the register panel QR below on the thread's column
// c = t & 31, rows 64 (t >> 5) .. + 63 in p (mr rows, nb columns); leaves
// column c's unscaled x below the diagonal in p and returns its scale, R in
// L.Rl, v_l^T v_j in L.St, tau and sign(beta) in L.tau_s / L.sgn, and T in
// L.Tl (rows written by threads t < 32; visible after a barrier).
__device__ float qr_reg_factor(float (&p)[64], int mr, int nb, QrRegLds& L) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = t & 31, g = t >> 5, rb = 64 * g;
  const bool live = 128 * wave < mr;
  if (!live && lane < 32) L.red[0][wave][c] = L.red[1][wave][c] = 0.f;   // waves past the panel add nothing
  float vscale = 0.f;                                          // scale of this column's reflector
#pragma clang loop unroll(disable)
  for (int j = 0; j < nb; ++j) {
    const int par = j & 1;
    if (c == j) {                                              // publish column j
#pragma unroll
      for (int r = 0; r < 64; r += 4)
        *reinterpret_cast<float4*>(&L.xs[rb + r]) = make_float4(p[r], p[r + 1], p[r + 2], p[r + 3]);
    }
    // rows <= j of x are zero: written by lanes 0 .. j of wave 0 after the
    // publishing lane j of the same wave (one wave's LDS writes land in order)
    if (t <= j) L.xs[t] = 0.f;
    if (g == 0) {                                              // publish row j (row block 0)
      float a[16];                                             // p[j] by the bits of j (j < 32)
#pragma unroll
      for (int q = 0; q < 16; ++q) {               // values first: a select of two loads keeps p in registers
        const float lo = p[2 * q], hi = p[2 * q + 1];
        a[q] = (j & 1) ? hi : lo;
      }
#pragma unroll
      for (int w = 2, n2 = 8; n2 >= 1; w <<= 1, n2 >>= 1) {
#pragma unroll
        for (int q = 0; q < n2; ++q) {
          const float lo = a[2 * q], hi = a[2 * q + 1];
          a[q] = (j & w) ? hi : lo;
        }
      }
      L.rowj[par][c] = a[0];
    }
    // x sits in the wave's own rows (its two row blocks), published by its
    // own lanes: a wave-level sync orders it.  Row j and the partial dots
    // cross waves and are read after the barrier below; both are kept by
    // the parity of j, so a wave that runs ahead into column j + 1 writes
    // the other copy while slower waves still read column j's.
    wave_lds_sync();
    float x[64];
    if (live) {
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int r = 0; r < 64; r += 4) {
        const float4 q = *reinterpret_cast<const float4*>(&L.xs[rb + r]);
        x[r] = q.x; x[r + 1] = q.y; x[r + 2] = q.z; x[r + 3] = q.w;
        s0 += q.x * p[r];
        s1 += q.y * p[r + 1];
        s2 += q.z * p[r + 2];
        s3 += q.w * p[r + 3];
      }
      const float part = half_sum((s0 + s1) + (s2 + s3));
      if (lane < 32) L.red[par][wave][c] = part;
    }
    __syncthreads();
    float raw = 0.f, sigma = 0.f;
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      raw += L.red[par][w][c];
      sigma += L.red[par][w][j];
    }
    const float alpha = L.rowj[par][j];
    float tau = 0.f, beta = alpha, scale = 0.f;
    if (sigma > 0.f) {
      // hardware square root and reciprocals (about 1 ulp): the column's
      // critical path, and the reflector needs no correctly rounded quotient
      const float nrm = __builtin_amdgcn_sqrtf(fmaf(alpha, alpha, sigma));
      beta = alpha >= 0.f ? -nrm : nrm;
      tau = (beta - alpha) * __builtin_amdgcn_rcpf(beta);
      scale = __builtin_amdgcn_rcpf(alpha - beta);
    }
    const float d = L.rowj[par][c] + scale * raw;                // v^T P[:, c]
    if (c == j) vscale = scale;
    // rows > j right of j: P -= x (scale tau d)
    const float e = c > j ? scale * tau * d : 0.f;
    if (live) {
#pragma unroll
      for (int r = 0; r < 64; ++r) p[r] -= x[r] * e;
    }
    // Row j is final after this step and only R reads it: it goes to LDS,
    // its registers keep a stale value that later steps multiply by x = 0.
    if (g == 0) {
      L.Rl[j][c] = c == j ? beta : (c > j ? L.rowj[par][c] - tau * d : 0.f);
      if (c < j) L.St[j][c] = vscale * d;
      if (c == j) {
        L.tau_s[j] = tau;
        L.sgn[j] = beta < 0.f ? -1.f : 1.f;
      }
    }
  }
  __syncthreads();
  if (t < 32) {                                                // row t of T, in registers
    float tr[32];                                              // tr[l] = 0 for l < t
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float u[4] = {0.f, 0.f, 0.f, 0.f};                   // four interleaved chains
#pragma unroll
      for (int l = 0; l < j; ++l) u[l & 3] = fmaf(tr[l], L.St[j][l], u[l & 3]);
      const float tj = L.tau_s[j];
      tr[j] = (j >= nb || j < t) ? 0.f : (j == t ? tj : -tj * ((u[0] + u[1]) + (u[2] + u[3])));
      L.Tl[t][j] = tr[j];
    }
  }
  return vscale;
}

// Householder QR of one panel (mp = m - c0 <= kLeaf rows, nb <= 32 columns)
// in registers: thread t holds column c = t & 31, rows 64 g .. 64 g + 63 with
// g = t >> 5, so a wave holds 128 rows of all 32 columns.  Column j: the
// threads of column j publish it below the diagonal (x) and the threads of
// row block 0 publish row j; every thread forms its column's dot x^T P[:, c]
// over its 64 rows, the two row blocks of a wave are added by one lane swap
// and the eight waves through LDS, and every thread then has sigma = x^T x,
// alpha = P[j][j], tau, beta and d_c = v^T P[:, c] = P[j][c] + scale x^T
// P[:, c] for its own column.  Columns right of j take P -= tau v d^T; column
// j keeps x below the diagonal (v = scale_j x, scaled when V is written) and
// beta on it, so for c < j, v_c^T v_j = scale_c d_c is kept for T.  One
// barrier per column (x reaches the threads of its own wave only); waves
// whose rows all lie past the panel skip the arithmetic.  T follows the factorization by the forward
// recurrence, T[t][j] = -tau_j sum_{t <= l < j} T[t][l] (v_l^T v_j), T[j][j]
// = tau_j.  Outputs are those of k_qr_block mode 0, plus (write_r) R in the
// panel's top rows.
__device__ void qr_reg_run(float* A, int64_t m, int64_t ld, int64_t bstride, int64_t c0, int nb, float* Vp,
                           int64_t vstride, float* Tp, int64_t tstride, float* taus_g, int64_t k, int write_r,
                           int64_t z, QrRegLds& L) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = t & 31, g = t >> 5, rb = 64 * g;               // column, first row
  const int mr = static_cast<int>(m - c0);
  float* Az = A + z * bstride;
  // The panel (columns c0.., rows c0.., column stride ld) through a buffer
  // resource; offsets of rows past the panel or columns past nb start at 2^31
  // (past any panel: ld <= 32768), which reads 0 and drops stores.
  constexpr uint32_t kOff = 0x80000000u;
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(Az + c0 * ld + c0, 0, static_cast<int>(((nb - 1) * ld + mr) * 4), 0x00020000);
  const uint32_t cb = static_cast<uint32_t>(c) * static_cast<uint32_t>(ld) * 4u + 4u * rb;
  auto off = [&](int r) -> int {
    return static_cast<int>(c < nb && rb + r < mr ? cb + 4u * r : kOff);
  };
  // 16-byte loads where the thread's 64 rows all lie in the panel, single
  // words in the block that straddles its end
  float p[64];
  const bool full = rb + 64 <= mr;
  if (full) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(pr, off(4 * q), 0, 0);
      p[4 * q] = __uint_as_float(v[0]);
      p[4 * q + 1] = __uint_as_float(v[1]);
      p[4 * q + 2] = __uint_as_float(v[2]);
      p[4 * q + 3] = __uint_as_float(v[3]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 64; ++r) p[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pr, off(r), 0, 0));
  }
  const float vscale = qr_reg_factor(p, mr, nb, L);
  // V (explicit, zero above row c0, unit diagonal), tau / sign(beta)
  float* V = Vp + z * vstride;
  for (int64_t r = t; r < c0; r += RT)
#pragma unroll
    for (int q = 0; q < 32; ++q) V[q * m + r] = 0.f;
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(V + c0, 0, static_cast<int>((31 * m + mr) * 4), 0x00020000);
  const uint32_t vb = static_cast<uint32_t>(c) * static_cast<uint32_t>(m) * 4u + 4u * rb;
  auto vval = [&](int r) -> float {
    const int i = rb + r;
    return (c >= nb || i < c) ? 0.f : (i == c ? 1.f : vscale * p[r]);
  };
  if (full) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float w0 = vval(4 * q), w1 = vval(4 * q + 1), w2 = vval(4 * q + 2), w3 = vval(4 * q + 3);
      const __attribute__((ext_vector_type(4))) uint32_t w = {__float_as_uint(w0), __float_as_uint(w1),
                                                               __float_as_uint(w2), __float_as_uint(w3)};
      __builtin_amdgcn_raw_buffer_store_b128(w, vr, static_cast<int>(vb + 16u * q), 0, 0);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 64; ++r)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vval(r)), vr,
                                            static_cast<int>(rb + r < mr ? vb + 4u * r : kOff), 0, 0);
  }
  if (t < nb) {
    taus_g[z * 2 * k + c0 + t] = L.tau_s[t];
    taus_g[z * 2 * k + k + c0 + t] = L.sgn[t];
  }
  if (write_r && g == 0) {                                     // R: rows <= c of row block 0
#pragma unroll
    for (int r = 0; r < 32; ++r)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L.Rl[r][c]), pr, r <= c && r < nb ? off(r) : static_cast<int>(kOff),
                                            0, 0);
  }
  __syncthreads();
  for (int idx = t; idx < 1024; idx += RT) Tp[z * tstride + idx] = L.Tl[idx >> 5][idx & 31];
}

}  // namespace
}  // namespace jolt
