// Householder thin QR of tall column-major panels, one workgroup per panel,
// and the factor finalization (sort by eigenvalue, sign convention, layout).
//
// Used to orthonormalize the Tucker factors and, in FlashJoLT, every sketch
// product of the randomized range finder (JoLT abstract, last sentence: a
// randomized-SVD variant; the QR is Householder, computed on the GPU).
//
// Panel A (m x k, column j at A + j*ld, m >= k).  Factorization: for each
// column j the reflector H_j = I - tau_j v_j v_j^T (v_j[j] = 1) maps
// A[j:, j] to beta_j e_1 with beta_j = -sign(alpha) * ||A[j:, j]||; the
// panel columns are updated in chunks of 16 (one block reduction per chunk).
// Blocked in panels of 32 columns (compact WY, I - V T V^T): a panel is
// factored by one workgroup, the trailing columns are updated with two
// matrix-core products, and Q = H_0 ... H_{k-1} [I; 0] is formed in place,
// back to front, the same way; column j is then multiplied by sign(beta_j) so
// that diag(R) >= 0.  Threads run along rows: every panel access is a
// coalesced column read.
#include "device.hpp"
#include <algorithm>
#include <utility>
#include "kernels.hpp"
#include "qr_reg.hpp"

namespace jolt {
namespace {

constexpr int QT = 1024;         // threads per panel
constexpr int QW = QT / 64;      // waves
constexpr int CH = 16;           // columns per reduction chunk

__device__ __forceinline__ float block_sum(float v, float* red, float* bcast) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int i = 0; i < QW; ++i) s += red[i];
    *bcast = s;
  }
  __syncthreads();
  return *bcast;
}

// w_c = sum_{i > j} v_i A[i][c] (+ A[j][c] * vj) for the chunk's columns,
// reduced over the workgroup into wsum[0..nc).
__device__ __forceinline__ void chunk_dots(const float* a, int64_t m, int64_t ld, int64_t j,
                                           int64_t c0, int nc, float vj_coef, float (*red)[CH],
                                           float* wsum) {
  float part[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) part[c] = 0.f;
  const float* v = a + j * ld;
  for (int64_t i = j + 1 + threadIdx.x; i < m; i += QT) {
    const float vi = v[i];
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nc) part[c] += vi * a[(c0 + c) * ld + i];
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const float s = wave_sum(part[c]);
    if (lane == 0) red[w][c] = s;
  }
  __syncthreads();
  if (threadIdx.x < nc) {
    float s = vj_coef * a[(c0 + threadIdx.x) * ld + j];
    for (int i = 0; i < QW; ++i) s += red[i][threadIdx.x];
    wsum[threadIdx.x] = s;
  }
  __syncthreads();
}

// Householder factorization of the panel columns [c0, c0 + nb) (rows c0..m-1),
// one workgroup per matrix.  Reflector vectors stay below the diagonal of A
// (beta on the diagonal); the explicit unit-lower V panel, the compact-WY
// factor T (I - V T V^T = H_c0 ... H_{c0+nb-1}) and tau / sign(beta) are
// written out for the blocked updates.
__global__ __launch_bounds__(QT) void k_hqr_panel(float* A, int64_t m, int64_t k, int64_t ld,
                                                  int64_t bstride, int64_t c0, int nb, float* Vp,
                                                  int64_t vstride, float* Tp, int64_t tstride,
                                                  float* taus_g) {
  __shared__ float red[QW][CH];
  __shared__ float red1[QW];
  __shared__ float bc;
  __shared__ float wsum[CH];
  __shared__ float S[32][33];
  __shared__ float Ts[32][33];
  const int64_t z = blockIdx.x;
  float* a = A + z * bstride;
  float* taus = taus_g + z * 2 * k;
  float* V = Vp + z * vstride;         // column-major m x 32 (this panel's slot)
  float* T = Tp + z * tstride;         // row-major 32 x 32
  for (int j = 0; j < nb; ++j) {
    const int64_t r0 = c0 + j;
    float* col = a + r0 * ld;
    float s = 0.f;
    for (int64_t i = r0 + 1 + threadIdx.x; i < m; i += QT) s += col[i] * col[i];
    const float sigma = block_sum(s, red1, &bc);
    const float alpha = col[r0];
    float tau = 0.f, beta = alpha;
    if (sigma > 0.f) {
      const float nrm = sqrtf(alpha * alpha + sigma);
      beta = alpha >= 0.f ? -nrm : nrm;
      tau = (beta - alpha) / beta;
      const float scale = 1.f / (alpha - beta);
      for (int64_t i = r0 + 1 + threadIdx.x; i < m; i += QT) col[i] *= scale;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      col[r0] = beta;
      taus[r0] = tau;
      taus[k + r0] = beta < 0.f ? -1.f : 1.f;
      Ts[j][j] = tau;
    }
    __syncthreads();
    if (tau != 0.f) {
      for (int64_t cc = r0 + 1; cc < c0 + nb; cc += CH) {
        const int nc = static_cast<int>(c0 + nb - cc < CH ? c0 + nb - cc : CH);
        chunk_dots(a, m, ld, r0, cc, nc, 1.f, red, wsum);
        for (int64_t i = r0 + threadIdx.x; i < m; i += QT) {
          const float vi = (i == r0) ? 1.f : col[i];
#pragma unroll
          for (int c = 0; c < CH; ++c)
            if (c < nc) a[(cc + c) * ld + i] -= tau * vi * wsum[c];
        }
        __syncthreads();
      }
    }
  }
  // S[i][j] = v_i . v_j for i < j  (v_j starts at row c0 + j with a unit entry)
  for (int j = 1; j < nb; ++j) {
    for (int c0c = 0; c0c < j; c0c += CH) {
      const int nc = j - c0c < CH ? j - c0c : CH;
      chunk_dots(a, m, ld, c0 + j, c0 + c0c, nc, 1.f, red, wsum);
      if (threadIdx.x < nc) S[c0c + threadIdx.x][j] = wsum[threadIdx.x];
      __syncthreads();
    }
  }
  // T[0:j, j] = -tau_j T[0:j, 0:j] S[0:j, j]  (upper triangular, column by column)
  if (threadIdx.x == 0) {
    for (int j = 0; j < nb; ++j) {
      for (int i = 0; i < j; ++i) {
        float acc = 0.f;
        for (int l = i; l < j; ++l) acc += Ts[i][l] * S[l][j];
        Ts[i][j] = -Ts[j][j] * acc;
      }
      for (int i = j + 1; i < 32; ++i) Ts[i][j] = 0.f;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 32; idx += QT) {
    const int r = idx / 32, c = idx % 32;
    T[idx] = (r < nb && c < nb) ? Ts[r][c] : 0.f;
  }
  // explicit V panel (zeros above, unit diagonal); columns past nb are zero
  for (int j = 0; j < 32; ++j) {
    const float* col = a + (c0 + j) * ld;
    for (int64_t i = threadIdx.x; i < m; i += QT) {
      float v = 0.f;
      if (j < nb) v = i < c0 + j ? 0.f : (i == c0 + j ? 1.f : col[i]);
      V[j * m + i] = v;
    }
  }
}

// ---- Register panels and tall-skinny QR (TSQR) with Householder
// reconstruction.  A panel block of up to kLeaf rows x 32 columns lives in
// the registers of one workgroup (64 rows of one column per thread) and is
// factored there.  Taller panels are split into row leaves factored
// independently; their stacked R factors
// are factored once more (the TSQR tree), the panel's orthonormal factor is
// assembled as diag(Q_i) Q_top, and the compact-WY form I - V T V^T of the
// panel is recovered from it by a sign-chosen LU of Q - S (Ballard, Demmel,
// Grigori, Jacobsen, Knight, Nguyen, "Reconstructing Householder vectors from
// tall-skinny QR", 2015): V = L, T = -U S L_1^{-T}, and the Householder R is
// S R, so sign(beta_j) = s_j when diag(R) >= 0.  The blocked updates that
// follow use V and T exactly as for a panel factored in place.
constexpr int LT = 1024;         // threads of the reconstruction's LU kernel
constexpr int kStack = 32 * 32 * 32;   // per matrix: up to 32 leaves x 32 rows x 32 (Rs, Qt)

// k_qr_reg: the register panel QR (qr_reg.hpp) of panel blockIdx.y.
__global__ __launch_bounds__(RT) void k_qr_reg(float* A, int64_t m, int64_t ld, int64_t bstride, int64_t c0,
                                               int nb, float* Vp, int64_t vstride, float* Tp, int64_t tstride,
                                               float* taus_g, int64_t k, int write_r) {
  __shared__ QrRegLds L;
  qr_reg_run(A, m, ld, bstride, c0, nb, Vp, vstride, Tp, tstride, taus_g, k, write_r, blockIdx.y, L);
}

// TSQR leaves and top level in registers, the factorization of k_qr_reg
// followed by the explicit Q = E - V (T V_1^T) (V_1: the first 32 rows of
// V).  Mode 1: leaf blockIdx.x (rows row0 .. row0 + rl of the panel) ->
// Q_i into Qb (column-major, leading dimension m - c0) and R_i into rows
// 32 i .. 32 i + 31 of the stack Rs (row-major, zero below the diagonal).
// Mode 2: the stack (nl * 32 rows, row-major) -> Q_top into Qt (row-major,
// 32 wide), column j times sign(beta_j) so that diag(R) >= 0.  Q's rows
// are formed on the fp32 matrix cores, each wave transposing its own rows
// of V through a private LDS tile, 64 rows at a time.
__global__ __launch_bounds__(RT) void k_qr_leaf(const float* A, int64_t m, int64_t ld, int64_t bstride,
                                                int64_t c0, int nb, int mode, int nl, int64_t rl, float* Qb,
                                                float* Rs, float* Qt, int64_t aux_stride) {
  __shared__ QrRegLds L;
  __shared__ float Ms[32][33];                                 // M = T V_1^T
  extern __shared__ float leaf_vw[];                           // [RW][64][33]: per-wave V rows
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, rl32 = lane & 31, hf = lane >> 5;
  const int c = t & 31, g = t >> 5, rb = 64 * g;
  const int64_t z = blockIdx.y;
  const int64_t mp = m - c0;
  const int64_t row0 = mode == 1 ? blockIdx.x * rl : 0;
  const int mr = mode == 1 ? static_cast<int>(mp - row0 < rl ? mp - row0 : rl) : nl * 32;
  float p[64];
  if (mode == 1) {
    const float* a = A + z * bstride + (c0 + c) * ld + c0 + row0;
#pragma unroll
    for (int r = 0; r < 64; ++r) p[r] = (c < nb && rb + r < mr) ? a[rb + r] : 0.f;
  } else {
    const float* rs = Rs + z * kStack;
#pragma unroll
    for (int r = 0; r < 64; ++r) p[r] = (c < nb && rb + r < mr) ? rs[(rb + r) * 32 + c] : 0.f;
  }
  const float vscale = qr_reg_factor(p, mr, nb, L);
  auto vval = [&](int r) -> float {                            // V at row rb + r, column c
    const int i = rb + r;
    return (c >= nb || i < c) ? 0.f : (i == c ? 1.f : vscale * p[r]);
  };
  __syncthreads();                                             // T complete
  if (g == 0) {
#pragma unroll
    for (int r = 0; r < 32; ++r) L.St[r][c] = vval(r);         // V_1 (St is free after T)
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {                                // M[a][b] = sum_k T[a][k] V_1[b][k]
    const int e = t + RT * q, a = e >> 5, b = e & 31;
    float u = 0.f;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) u += L.Tl[a][kk] * L.St[b][kk];
    Ms[a][b] = u;
  }
  if (mode == 1) {                                             // R_i into the stack
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = t + RT * q, a = e >> 5, b = e & 31;
      Rs[z * kStack + (blockIdx.x * 32 + a) * 32 + b] = (a < nb && b < nb && a <= b) ? L.Rl[a][b] : 0.f;
    }
  }
  __syncthreads();
  if (128 * wave >= mr) return;                                // no rows of the panel in this wave
  float* vw = leaf_vw + wave * 64 * 33;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int base = 128 * wave + 64 * h2;                     // this round's rows
    if (hf == h2) {
#pragma unroll
      for (int r = 0; r < 64; ++r) vw[r * 33 + c] = vval(r);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < 32; kk += 2) {
        const int k = kk + hf;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(vw[(32 * blk + rl32) * 33 + k], Ms[k][rl32], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = base + 32 * blk + (e >> 2) * 8 + hf * 4 + (e & 3);
        if (i < mr) {
          const float qv = (i == rl32 ? 1.f : 0.f) - acc[e];
          if (mode == 1) {
            Qb[z * aux_stride + static_cast<int64_t>(rl32) * mp + row0 + i] = qv;
          } else {
            const float sg = rl32 < nb ? L.sgn[rl32] : 1.f;   // beta_c = R_cc: flip so diag(R) >= 0
            Qt[z * kStack + static_cast<int64_t>(i) * 32 + rl32] = sg * qv;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

constexpr int kQrSplit = 16;     // row chunks of a tall block-reflector application

// Block reflector on a tall block: Z <- (I - V op(T) V^T) Z, Z mr x nc
// (column-major, leading dimension ldz), V mr x 32 (leading dimension ldv,
// rows aligned with Z's), op(T) = T or T^T.  The rows split into chunks of
// rch rows (a multiple of 64) and the columns into tiles of 64:
// k_wy_part: W_c = V_c^T Z_c for row chunk c and one column tile;
// k_wy_mid: W2 = op(T) (sum over c of W_c), summed in chunk order;
// k_wy_upd: Z_c -= V_c W2.
// Inside a chunk the rows stream in blocks of 64, the next block loaded into
// registers while the current one is multiplied on the fp32 matrix cores.
struct WyTile {
  float Zs[64][65];
  float Vs[64][33];
};

__device__ __forceinline__ void wy_load(const float* Z, int64_t ldz, int64_t mr, int nc, int j0, const float* V,
                                        int64_t ldv, int64_t r0, float (&rz)[16], float (&rv)[8]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = tid + 256 * q, c = idx >> 6, rr = idx & 63;
    rz[q] = (r0 + rr < mr && j0 + c < nc) ? Z[static_cast<int64_t>(j0 + c) * ldz + r0 + rr] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q, c = idx >> 6, rr = idx & 63;
    rv[q] = r0 + rr < mr ? V[static_cast<int64_t>(c) * ldv + r0 + rr] : 0.f;
  }
}

__device__ __forceinline__ void wy_store(WyTile& L, const float (&rz)[16], const float (&rv)[8]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = tid + 256 * q;
    L.Zs[idx & 63][idx >> 6] = rz[q];
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q;
    L.Vs[idx & 63][idx >> 6] = rv[q];
  }
}

__global__ __launch_bounds__(256) void k_wy_part(const float* Z_g, int64_t ldz, int64_t z_batch, int64_t mr, int nc,
                                                 const float* V_g, int64_t ldv, int64_t v_batch, int64_t rch,
                                                 float* Wp) {
  __shared__ WyTile L;
  __shared__ float Wh[2][32][65];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, hf = lane >> 5;
  const int64_t z = blockIdx.z;
  const int ch = blockIdx.x, nch = gridDim.x, j0 = 64 * blockIdx.y;
  const float* Z = Z_g + z * z_batch;
  const float* V = V_g + z * v_batch;
  const int64_t rbeg = ch * rch, rend = rbeg + rch < mr ? rbeg + rch : mr;
  const int cb = 32 * (wave & 1), kb = 32 * (wave >> 1);
  float rz[16], rv[8];
  f32x16 acc = {};
  if (rbeg < rend) wy_load(Z, ldz, rend, nc, j0, V, ldv, rbeg, rz, rv);
  for (int64_t r0 = rbeg; r0 < rend; r0 += 64) {
    wy_store(L, rz, rv);
    __syncthreads();
    if (r0 + 64 < rend) wy_load(Z, ldz, rend, nc, j0, V, ldv, r0 + 64, rz, rv);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 2) {
      const int k = kb + kk + hf;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(L.Vs[k][rl], L.Zs[k][cb + rl], acc, 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) Wh[wave >> 1][(e >> 2) * 8 + hf * 4 + (e & 3)][cb + rl] = acc[e];
  __syncthreads();
  float* wp = Wp + (z * nch + ch) * 32 * static_cast<int64_t>(nc);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q, a = idx >> 6, j = idx & 63;
    if (j0 + j < nc) wp[a * static_cast<int64_t>(nc) + j0 + j] = Wh[0][a][j] + Wh[1][a][j];
  }
}

__global__ __launch_bounds__(256) void k_wy_mid(int nc, int nch, const float* Wp, const float* T_g, int64_t t_batch,
                                                int trans, float* W2) {
  __shared__ float Ws[32][65];
  __shared__ float Ts[32][33];
  const int tid = threadIdx.x;
  const int64_t z = blockIdx.y;
  const int j0 = 64 * blockIdx.x;
  {
    float rt[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rt[q] = T_g[z * t_batch + tid + 256 * q];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      if (trans) Ts[idx & 31][idx >> 5] = rt[q];
      else Ts[idx >> 5][idx & 31] = rt[q];
    }
  }
  const float* wp = Wp + z * nch * 32 * static_cast<int64_t>(nc);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q, a = idx >> 6, j = idx & 63;
    // the chunks' shares added in chunk order, all loads in flight (nch <= kQrSplit)
    float v[kQrSplit];
#pragma unroll
    for (int c = 0; c < kQrSplit; ++c)
      v[c] = (c < nch && j0 + j < nc) ? wp[(c * 32 + a) * static_cast<int64_t>(nc) + j0 + j] : 0.f;
    float u = 0.f;
#pragma unroll
    for (int c = 0; c < kQrSplit; ++c) u += v[c];
    Ws[a][j] = u;
  }
  __syncthreads();
  float* w2 = W2 + z * 32 * static_cast<int64_t>(nc);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q, a = idx >> 6, j = idx & 63;
    float u = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) u += Ts[a][m] * Ws[m][j];
    if (j0 + j < nc) w2[a * static_cast<int64_t>(nc) + j0 + j] = u;
  }
}

__global__ __launch_bounds__(256) void k_wy_upd(float* Z_g, int64_t ldz, int64_t z_batch, int64_t mr, int nc,
                                                const float* V_g, int64_t ldv, int64_t v_batch, int64_t rch,
                                                const float* W2) {
  __shared__ WyTile L;
  __shared__ float Ws[32][65];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, hf = lane >> 5;
  const int64_t z = blockIdx.z;
  const int ch = blockIdx.x, j0 = 64 * blockIdx.y;
  float* Z = Z_g + z * z_batch;
  const float* V = V_g + z * v_batch;
  const int64_t rbeg = ch * rch, rend = rbeg + rch < mr ? rbeg + rch : mr;
  const float* w2 = W2 + z * 32 * static_cast<int64_t>(nc);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q, a = idx >> 6, j = idx & 63;
    Ws[a][j] = j0 + j < nc ? w2[a * static_cast<int64_t>(nc) + j0 + j] : 0.f;
  }
  const int cb = 32 * (wave & 1), kb = 32 * (wave >> 1);
  float rz[16], rv[8];
  if (rbeg < rend) wy_load(Z, ldz, rend, nc, j0, V, ldv, rbeg, rz, rv);
  for (int64_t r0 = rbeg; r0 < rend; r0 += 64) {
    __syncthreads();                     // W2 visible; the previous block's Zs / Vs reads done
    wy_store(L, rz, rv);
    __syncthreads();
    if (r0 + 64 < rend) wy_load(Z, ldz, rend, nc, j0, V, ldv, r0 + 64, rz, rv);
    f32x16 d = {};
#pragma unroll
    for (int kk = 0; kk < 32; kk += 2) {
      const int k = kk + hf;
      d = __builtin_amdgcn_mfma_f32_32x32x2f32(L.Vs[kb + rl][k], Ws[k][cb + rl], d, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Zs[kb + (e >> 2) * 8 + hf * 4 + (e & 3)][cb + rl] -= d[e];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q, c = idx >> 6, rr = idx & 63;
      if (r0 + rr < rend && j0 + c < nc) Z[static_cast<int64_t>(j0 + c) * ldz + r0 + rr] = L.Zs[rr][c];
    }
  }
}

// Top block of the panel's Q (leaf 0's first nb rows times Q_top's first
// block), its sign-chosen LU, and T = -U S L_1^{-T}; U and L_1 -> UL for the
// tall part.
__global__ __launch_bounds__(LT) void k_hr_lu(int64_t m, int64_t c0, int nb, const float* Qb, const float* Qt,
                                              int64_t aux_stride, float* Tp, int64_t tstride, float* taus_g,
                                              int64_t k, float* UL) {
  __shared__ float B[32][33];
  __shared__ float Xi[32][33];
  __shared__ float sg[32];
  const int i = threadIdx.x, r = i / 32, c = i % 32;
  const int64_t z = blockIdx.x;
  const int64_t mp = m - c0;
  {
    float t = 0.f;
    if (r < nb && c < nb) {
      const float* qb = Qb + z * aux_stride;
      const float* qt = Qt + z * kStack;
      for (int a = 0; a < nb; ++a) t += qb[a * mp + r] * qt[a * 32 + c];
    }
    B[r][c] = t;
  }
  __syncthreads();
  for (int j = 0; j < nb; ++j) {
    if (i == 0) {
      const float s = B[j][j] >= 0.f ? -1.f : 1.f;
      sg[j] = s;
      B[j][j] -= s;
    }
    __syncthreads();
    if (c == 0 && r > j && r < nb) B[r][j] /= B[j][j];
    __syncthreads();
    if (r > j && r < nb && c > j && c < nb) B[r][c] -= B[r][j] * B[j][c];
    __syncthreads();
  }
  // Xi = L_1^{-1} (unit lower), one column per thread
  if (i < 32) {
    for (int rr = 0; rr < 32; ++rr) Xi[rr][i] = 0.f;
    if (i < nb) {
      Xi[i][i] = 1.f;
      for (int rr = i + 1; rr < nb; ++rr) {
        float t = 0.f;
        for (int qq = i; qq < rr; ++qq) t += B[rr][qq] * Xi[qq][i];
        Xi[rr][i] = -t;
      }
    }
  }
  __syncthreads();
  // T[r][c] = -sum_q U[r][q] s_q Xi[c][q]
  float t = 0.f;
  if (r < nb && c < nb && r <= c) {
    for (int qq = r; qq <= c; ++qq) t -= B[r][qq] * sg[qq] * Xi[c][qq];
  }
  Tp[z * tstride + i] = t;
  if (i < nb) {
    float d = 0.f;
    for (int qq = i; qq <= i; ++qq) d -= B[i][qq] * sg[qq] * Xi[i][qq];
    taus_g[z * 2 * k + c0 + i] = d;
    taus_g[z * 2 * k + k + c0 + i] = sg[i];
  }
  UL[z * 1024 + i] = (r < nb && c < nb) ? B[r][c] : 0.f;      // U upper, L_1 strict lower
}

// Explicit V of a tall panel: rows above c0 are zero, the top nb rows are
// L_1, every other row is (Q_i row . Q_top block) U^{-1}.
__global__ __launch_bounds__(256) void k_hr_tall(int64_t m, int64_t c0, int nb, int64_t rl, const float* Qb,
                                                 const float* Qt, int64_t aux_stride, const float* UL,
                                                 float* Vp, int64_t vstride) {
  __shared__ float U[32][33];          // U on and above the diagonal, L_1 below
  __shared__ float Qs[2][32][33];
  const int64_t z = blockIdx.y;
  const int64_t g0 = blockIdx.x * 256ll;
  const int64_t mp = m - c0;
  const int64_t lo = g0 - c0 > 0 ? g0 - c0 : 0;
  const int64_t leaf0 = lo / rl;
  {
    // every load in flight before the LDS writes
    float ru[4], rq[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) ru[q] = UL[z * 1024 + threadIdx.x + 256 * q];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = threadIdx.x + 256 * q, s = idx / 1024, a = (idx % 1024) / 32, c = idx % 32;
      const int64_t leaf = leaf0 + s;
      rq[q] = leaf * rl < mp ? Qt[z * kStack + (leaf * 32 + a) * 32 + c] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = threadIdx.x + 256 * q;
      U[idx / 32][idx % 32] = ru[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = threadIdx.x + 256 * q, s = idx / 1024, a = (idx % 1024) / 32, c = idx % 32;
      Qs[s][a][c] = rq[q];
    }
  }
  __syncthreads();
  const int64_t g = g0 + threadIdx.x;
  if (g >= m) return;
  float* V = Vp + z * vstride;
  const int64_t r = g - c0;
  float x[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) x[c] = 0.f;
  if (r >= 0 && r < nb) {
#pragma unroll
    for (int c = 0; c < 32; ++c) x[c] = c < r ? U[r][c] : (c == r ? 1.f : 0.f);
  } else if (r >= nb) {
    const int s = static_cast<int>(r / rl - leaf0);
    const float* qb = Qb + z * aux_stride;
    float q[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) q[c] = 0.f;
    for (int a = 0; a < nb; ++a) {
      const float qa = qb[a * mp + r];
#pragma unroll
      for (int c = 0; c < 32; ++c) q[c] += qa * Qs[s][a][c];
    }
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      if (c < nb) {
        float t = q[c];
        for (int a = 0; a < c; ++a) t -= x[a] * U[a][c];
        x[c] = t / U[c][c];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 32; ++c) V[c * m + g] = x[c];
}

// Q[:, c0 .. c0+nb) <- columns of the identity (rows 0..m-1).
__global__ __launch_bounds__(256) void k_eye_cols(float* A, int64_t m, int64_t ld, int64_t bstride,
                                                   int64_t c0, int nb) {
  float* a = A + blockIdx.y * bstride;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < m * nb; idx += 256ll * gridDim.x) {
    const int64_t j = idx / m, i = idx % m;
    a[(c0 + j) * ld + i] = (i == c0 + j) ? 1.f : 0.f;
  }
}

// diag(R) >= 0: column j times sign(beta_j).
__global__ __launch_bounds__(256) void k_col_signs(float* A, int64_t m, int64_t k, int64_t ld,
                                                    int64_t bstride, const float* taus_g) {
  float* a = A + blockIdx.y * bstride;
  const float* sg = taus_g + blockIdx.y * 2 * k + k;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < m * k; idx += 256ll * gridDim.x) {
    const int64_t j = idx / m, i = idx % m;
    if (sg[j] < 0.f) a[j * ld + i] = -a[j * ld + i];
  }
}

// perm: eigenvalues descending, ties to the lower index (bitonic, one workgroup).
__global__ __launch_bounds__(1024) void k_sort_desc(const double* lam, int64_t R, int64_t lam_batch,
                                                    int* perm) {
  __shared__ double key[2048];
  __shared__ int ix[2048];
  const int tid = threadIdx.x;
  int n2 = 1;
  while (n2 < R) n2 <<= 1;
  const double* l = lam + blockIdx.x * lam_batch;
  for (int i = tid; i < n2; i += 1024) {
    key[i] = i < R ? l[i] : -INFINITY;
    ix[i] = i;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool fwd = (i & size) == 0;
          const double ki = key[i], kj = key[j];
          const int ii = ix[i], ij = ix[j];
          const bool i_first = ki > kj || (ki == kj && ii < ij);
          if (fwd != i_first) {
            key[i] = kj; key[j] = ki; ix[i] = ij; ix[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < R; i += 1024) perm[blockIdx.x * R + i] = ix[i];
}

// sign of output column j: the largest-|.| entry of source column perm[j]
// (lowest row on ties) made positive.
__global__ __launch_bounds__(256) void k_col_sign(const float* U, int64_t m, int64_t ld, int64_t bstride,
                                                  const int* perm, int64_t R, float* sign) {
  const int64_t z = blockIdx.y, j = blockIdx.x;
  const float* col = U + z * bstride + static_cast<int64_t>(perm[z * R + j]) * ld;
  float best = -1.f;
  int64_t bi = 0;
  if (m % 4 == 0 && ld % 4 == 0 && bstride % 4 == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0) {
    // 16-byte loads, each thread's four rows scanned in order
    for (int64_t i = 4 * static_cast<int64_t>(threadIdx.x); i < m; i += 1024) {
      const float4 q = *reinterpret_cast<const float4*>(col + i);
      const float v[4] = {fabsf(q.x), fabsf(q.y), fabsf(q.z), fabsf(q.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v[e] > best) { best = v[e]; bi = i + e; }
    }
  } else {
    for (int64_t i = threadIdx.x; i < m; i += 256) {
      const float v = fabsf(col[i]);
      if (v > best) { best = v; bi = i; }
    }
  }
  __shared__ float bv[256];
  __shared__ int64_t bx[256];
  bv[threadIdx.x] = best;
  bx[threadIdx.x] = bi;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      const float o = bv[threadIdx.x + s];
      const int64_t oi = bx[threadIdx.x + s];
      if (o > bv[threadIdx.x] || (o == bv[threadIdx.x] && oi < bx[threadIdx.x])) {
        bv[threadIdx.x] = o;
        bx[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) sign[z * R + j] = col[bx[0]] < 0.f ? -1.f : 1.f;
}

// U_out[i][j] = sign[j] * U_cm[perm[j]][i] (row-major out); lam_out[j] = lam[perm[j]].
// 128 rows x 32 columns per workgroup through an LDS transpose: 16-byte loads
// along the source columns and 16-byte stores along the output rows where the
// layouts are 16-byte aligned, single words otherwise.
__global__ __launch_bounds__(256) void k_emit(const float* U, int64_t m, int64_t ld, int64_t bstride,
                                              const int* perm, const float* sign, int64_t R,
                                              const double* lam, int64_t lam_batch, float* out,
                                              int64_t ld_out, int64_t out_batch, double* lam_out,
                                              int64_t lam_out_batch) {
  __shared__ float tile[32][132];                 // [column][row]
  const int64_t z = blockIdx.z;
  const int64_t i0 = blockIdx.x * 128ll, j0 = blockIdx.y * 32ll;
  const int tid = threadIdx.x;
  // loads: thread -> column jj = tid / 8, rows 4 (tid % 8) + 32 q
  {
    const int jj = tid >> 3;
    const int64_t j = j0 + jj;
    const bool vin = ld % 4 == 0 && bstride % 4 == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0;
    const float* src = j < R ? U + z * bstride + static_cast<int64_t>(perm[z * R + j]) * ld : nullptr;
    const float sg = j < R ? sign[z * R + j] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int il = 4 * (tid & 7) + 32 * q;
      const int64_t i = i0 + il;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (src) {
        if (vin && i + 3 < m) {
          const float4 x = *reinterpret_cast<const float4*>(src + i);
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = i + e < m ? src[i + e] : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[jj][il + e] = sg * v[e];
    }
  }
  __syncthreads();
  // stores: thread -> row ii = tid / 2, columns 16 (tid % 2) .. + 15
  {
    const int ii = tid >> 1;
    const int64_t i = i0 + ii;
    if (i < m) {
      float* orow = out + z * out_batch + i * ld_out;
      const bool vout = ld_out % 4 == 0 && out_batch % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jl = 16 * (tid & 1) + 4 * q;
        const int64_t jg = j0 + jl;
        const float v[4] = {tile[jl][ii], tile[jl + 1][ii], tile[jl + 2][ii], tile[jl + 3][ii]};
        if (vout && jg + 3 < R) {
          *reinterpret_cast<float4*>(orow + jg) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (jg + e < R) orow[jg + e] = v[e];
        }
      }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < 32) {
    const int64_t j = j0 + threadIdx.x;
    if (j < R) lam_out[z * lam_out_batch + j] = lam[z * lam_batch + perm[z * R + j]];
  }
}

// ---------------------------------------------------------------- CholeskyQR
// The thin QR factorization U = Q R of a full-rank tall U (m x k, k <= 256)
// from its Gram: G = U^T U = L L^T (Cholesky, L lower with positive
// diagonal), Q = U L^{-T}, R = L^T.  In exact arithmetic this is the
// factorization with diag(R) > 0, so span(Q[:, :j]) = span(U[:, :j]) for
// every j.
//
// k_chol_inv computes L^{-1} in one pass over the columns.  Element form,
// step j (the rows above j already final, d = A[j][j] the Schur
// complement's pivot, s = 1 / sqrt(d)):
//   rows i > j, columns k != j:  A[i][k] -= A[i][j] b[k] s^2
//   rows i > j, column j:        A[i][j]  = -A[i][j] s^2
//   row j, columns k < j:        A[j][k] *= s,   A[j][j] = s,
// with b[k] = A[k][j] for k > j (column j: the Cholesky update) and A[j][k]
// for k < j (row j of the inverse so far: its forward substitution); after
// the last step the lower triangle holds L^{-1}.  Blocked by 32: step J
// factors the diagonal block, W = L_JJ^{-1} (the element form, one wave, in
// LDS), then with 32 x 32 fp32 matrix-core products
//   L_IJ = S_IJ W^T (I > J),  block (I, J) <- -L_IJ W,
//   X_JK = W Y_JK (K < J: row block J of the inverse, final),
//   S_IK -= L_IJ L_KJ^T (J < K <= I),  Y_IK -= L_IJ X_JK (K < J < I),
// each block held in one wave's registers (matrix-core accumulator layout).
// A pivot not above pivot_rel times its column's original diagonal (a
// column nearly in the span of the earlier ones) sets bit 1 of *status; the
// step then continues with the original diagonal, so the results stay
// finite but are not a factorization.  With minus_identity the output is
// L^{-1} - I (a correction, for a nearly orthonormal U).  k is padded to a
// multiple of 32 with an identity block.
constexpr int kCholMaxK = 256;
constexpr int CB = 32, CBP = CB + 1, CNB = kCholMaxK / CB;
constexpr int kCholBlocks = CNB * (CNB + 1) / 2;   // 36 lower blocks, over 8 waves
constexpr int CW = 8;                                // waves of k_chol_inv
struct CholLds {
  float col[CNB][CB][CBP];   // block column J: S_IJ staged, then L_IJ
  float row[CNB][CB][CBP];   // block row J of the inverse: X_JK (K < J), W = X_JJ
  float d0[kCholMaxK];       // original diagonal
};

// row of register i of lane l in the accumulator layout, column l % 32
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
__device__ __forceinline__ void acc_to_tile(const f32x16& a, float (*t)[CBP], int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) t[acc_row(i, lane)][lane & 31] = a[i];
}
__device__ __forceinline__ f32x16 tile_to_acc(const float (*t)[CBP], int lane) {
  f32x16 a;
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = t[acc_row(i, lane)][lane & 31];
  return a;
}
// c + sA A B over one 32-block of k; A(m, k) = ta[m][k], B(k, n) = tb[k][n] or (tbt) tb[n][k]
template <bool TB>
__device__ __forceinline__ f32x16 mm32(f32x16 c, float sA, const float (*ta)[CBP], const float (*tb)[CBP],
                                       int lane) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < CB; kk += 2) {
    const float a = sA * ta[r][kk + h];
    const float b = TB ? tb[r][kk + h] : tb[kk + h][r];
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  return c;
}
__device__ __forceinline__ void chol_block_of(int bi, int& I, int& K) {
  I = 0;
  while ((I + 1) * (I + 2) / 2 <= bi) ++I;
  K = bi - I * (I + 1) / 2;
}

// W <- L^{-1} for the 32 x 32 block W = L L^T (lower triangle read; the
// upper triangle is zeroed), by one wave: the element form above.  Lane
// (h, c) owns the elements (2 t + h, c).  A wave's LDS operations execute in
// program order, so at each step every read (the pivot, row j and column j,
// the lane's own elements) is issued before any write.  Row pairs above j
// are final and skipped; the upper triangle is never read for a lower
// element, so it takes whatever the update gives and is zeroed at the end.
// The pivot's reciprocal square root is the hardware one (about 1 ulp: a
// relative perturbation of the factor near 2^-23, below the Gram's own rounding).
__device__ void chol_inv_block(float (*W)[CBP], const float* d0, float pivot_rel, int lane, bool& bad) {
  const int c = lane & 31, h = lane >> 5;
  for (int j = 0; j < CB; ++j) {
    wave_lds_sync();
    float d = W[j][j];
    const float dj0 = d0[j];
    const float* pb = c > j ? &W[c][j] : &W[j][c];      // b[c]: column j below the pivot, row j left of it
    const float bc = c == j ? 0.f : *pb;
    float bi[CB / 2], v[CB / 2];
#pragma unroll
    for (int t = 0; t < CB / 2; ++t) {
      if (2 * t + 1 < j) continue;                    // both rows above j
      bi[t] = W[2 * t + h][j];
      v[t] = W[2 * t + h][c];
    }
    if (!(d > pivot_rel * dj0)) {
      bad = true;
      d = dj0 > 0.f ? dj0 : 1.f;
    }
    const float sj = __builtin_amdgcn_rsqf(d), s2 = sj * sj;
    const float g = -bc * s2;
    const bool cj = c == j;
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < CB / 2; ++t) {
      if (2 * t + 1 < j) continue;
      const int i = 2 * t + h;
      const float w_gt = cj ? -bi[t] * s2 : fmaf(bi[t], g, v[t]);
      if (2 * t > j) {
        W[i][c] = w_gt;                               // both rows below j
      } else {
        const float w_eq = cj ? sj : v[t] * sj;
        W[i][c] = i > j ? w_gt : (i == j ? w_eq : v[t]);
      }
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int t = 0; t < CB / 2; ++t) {
    const int i = 2 * t + h;
    if (c > i) W[i][c] = 0.f;
  }
  wave_lds_sync();
}

__global__ __launch_bounds__(CW * 64) void k_chol_inv(const float* G, int64_t g_batch, int k, float pivot_rel,
                                                   float* Linv, int64_t l_batch, int minus_identity, int* status) {
  __shared__ CholLds sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t z = blockIdx.x;
  const float* Gz = G + z * g_batch;
  const int nb = (k + CB - 1) / CB, nblk = nb * (nb + 1) / 2;
  constexpr int NS = (kCholBlocks + CW - 1) / CW;
  f32x16 acc[NS];
  int bI[NS], bK[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int bi = wave + CW * s;
    bI[s] = bK[s] = -1;
    if (bi >= nblk) continue;
    chol_block_of(bi, bI[s], bK[s]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int gi = CB * bI[s] + acc_row(i, lane), gk = CB * bK[s] + (lane & 31);
      acc[s][i] = (gi < k && gk < k) ? Gz[static_cast<int64_t>(gi) * k + gk] : (gi == gk ? 1.f : 0.f);
      if (bI[s] == bK[s] && gi == gk) sm.d0[gi] = acc[s][i];
    }
  }
  __syncthreads();
  bool bad = false;
  for (int J = 0; J < nb; ++J) {
    float(*W)[CBP] = sm.row[J];
    // ---- A: the diagonal block's owner factors it: W = L_JJ^{-1}
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (bI[s] != J || bK[s] != J) continue;
      acc_to_tile(acc[s], W, lane);
      chol_inv_block(W, sm.d0 + CB * J, pivot_rel, lane, bad);
      acc[s] = tile_to_acc(W, lane);           // X_JJ = W, final
    }
    __syncthreads();
    // ---- B: block column J of L, its blocks' inverse values; row block J of the inverse
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int I = bI[s], K = bK[s];
      if (I > J && K == J) {
        float(*C)[CBP] = sm.col[I];
        acc_to_tile(acc[s], C, lane);          // S_IJ
        wave_lds_sync();
        const f32x16 L = mm32<true>(f32x16{}, 1.f, C, W, lane);   // S_IJ W^T
        wave_lds_sync();
        acc_to_tile(L, C, lane);
        wave_lds_sync();
        acc[s] = mm32<false>(f32x16{}, -1.f, C, W, lane);          // -L_IJ W
      } else if (I == J && K < J) {
        float(*Y)[CBP] = sm.row[K];
        acc_to_tile(acc[s], Y, lane);          // Y_JK
        wave_lds_sync();
        acc[s] = mm32<false>(f32x16{}, 1.f, W, Y, lane);           // X_JK = W Y_JK, final
        wave_lds_sync();
        acc_to_tile(acc[s], Y, lane);
      }
    }
    __syncthreads();
    // ---- C: trailing blocks
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int I = bI[s], K = bK[s];
      if (I <= J || K == J) continue;
      if (K > J) acc[s] = mm32<true>(acc[s], -1.f, sm.col[I], sm.col[K], lane);   // S_IK -= L_IJ L_KJ^T
      else acc[s] = mm32<false>(acc[s], -1.f, sm.col[I], sm.row[K], lane);       // Y_IK -= L_IJ X_JK
    }
    __syncthreads();
  }
  float* Lz = Linv + z * l_batch;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int I = bI[s], K = bK[s];
    if (I < 0) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int gi = CB * I + acc_row(i, lane), gk = CB * K + (lane & 31);
      if (gi < k && gk < k) {
        Lz[static_cast<int64_t>(gi) * k + gk] = acc[s][i] - (minus_identity && gi == gk ? 1.f : 0.f);
        if (I != K) Lz[static_cast<int64_t>(gk) * k + gi] = 0.f;    // the mirrored block above the diagonal
      }
    }
  }
  if (bad) __hip_atomic_fetch_or(status, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace


size_t householder_qr_work_floats(int64_t m, int64_t k, int batch) {
  const int64_t P = (k + 31) / 32;
  // V panels (m x 32 each), T factors (32 x 32 each), W / W2 (32 x k), tau + signs (2k),
  // TSQR: leaf Q (m x 32), stacked R and Q_top (kStack each), LU (32 x 32); split-K partials
  return static_cast<size_t>(batch) * (P * m * 32 + P * 32 * 32 + 2 * 32 * k + 2 * k + 64 + m * 32 +
                                       2 * kStack + 1024 + static_cast<int64_t>(kQrSplit) * 32 * k);
}


size_t panel_factor_scratch_floats(int64_t m, int batch) {
  return static_cast<size_t>(batch) * (m * 32 + 2 * kStack + 1024);
}

int64_t panel_block_rows() { return kLeaf; }

hipError_t panel_factor(float* A, int64_t m, int64_t ld, int64_t bstride, int64_t c0, int nb, int batch,
                        float* Vp, int64_t vstride, float* Tp, int64_t tstride, float* taus, int64_t k,
                        float* scratch, hipStream_t s, int write_r) {
  static const hipError_t lds_attr =   // once per process (thread-safe initialization)
      hipFuncSetAttribute(reinterpret_cast<const void*>(k_qr_leaf), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(RW * 64 * 33 * sizeof(float)));
  if (lds_attr != hipSuccess) return lds_attr;
  float* Qb = scratch;                                            // [batch][m][32]
  float* Rs = Qb + static_cast<size_t>(batch) * m * 32;           // [batch][kStack]
  float* Qt = Rs + static_cast<size_t>(batch) * kStack;           // [batch][kStack]
  float* UL = Qt + static_cast<size_t>(batch) * kStack;           // [batch][1024]
  ProfScope ps("qr_panel", s);
  const int64_t mp = m - c0;
  const int64_t nl = (mp + kLeaf - 1) / kLeaf;
  hipError_t e;
  if (nl <= 1) {
    k_qr_reg<<<dim3(1, batch), RT, 0, s>>>(A, m, ld, bstride, c0, nb, Vp, vstride, Tp, tstride, taus, k, write_r);
  } else if (nl <= 32) {
    const int64_t rl = (mp + nl - 1) / nl;
    const size_t vw_lds = static_cast<size_t>(RW) * 64 * 33 * sizeof(float);
    k_qr_leaf<<<dim3(static_cast<unsigned>(nl), batch), RT, vw_lds, s>>>(A, m, ld, bstride, c0, nb, 1,
                                                                         static_cast<int>(nl), rl, Qb, Rs, Qt,
                                                                         m * 32);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_qr_leaf<<<dim3(1, batch), RT, vw_lds, s>>>(A, m, ld, bstride, c0, nb, 2, static_cast<int>(nl), rl, Qb, Rs,
                                                 Qt, m * 32);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_hr_lu<<<batch, LT, 0, s>>>(m, c0, nb, Qb, Qt, m * 32, Tp, tstride, taus, k, UL);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_hr_tall<<<dim3(static_cast<unsigned>((m + 255) / 256), batch), 256, 0, s>>>(m, c0, nb, rl, Qb, Qt, m * 32,
                                                                                  UL, Vp, vstride);
  } else {
    k_hqr_panel<<<batch, QT, 0, s>>>(A, m, k, ld, bstride, c0, nb, Vp, vstride, Tp, tstride, taus);
  }
  return hipGetLastError();
}

hipError_t apply_wy_tall(float* Z, int64_t ldz, int64_t z_batch, int64_t mr, int nc, const float* V, int64_t ldv,
                         int64_t v_batch, const float* T, int64_t t_batch, int trans, int batch, float* Wp,
                         float* W2, hipStream_t s) {
  if (mr <= 0 || nc <= 0) return hipSuccess;
  ProfScope ps("qr_update", s);
  // algorithmic work: Z read and written once, V read once; 4 mr nc 32 flops
  // (V^T Z and V W2) + 2 32^2 nc (op(T) W)
  prof_add_work("qr_update", static_cast<double>(batch) * 4.0 * (2.0 * mr * nc + mr * 32.0),
                static_cast<double>(batch) * (4.0 * mr * nc * 32.0 + 2.0 * 1024.0 * nc));
  const int64_t blocks = (mr + 63) / 64;
  const int nch = static_cast<int>(blocks < kQrSplit ? blocks : kQrSplit);
  const int64_t rch = 64 * ((blocks + nch - 1) / nch);
  const int nct = (nc + 63) / 64;
  k_wy_part<<<dim3(nch, nct, batch), 256, 0, s>>>(Z, ldz, z_batch, mr, nc, V, ldv, v_batch, rch, Wp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_wy_mid<<<dim3(nct, batch), 256, 0, s>>>(nc, nch, Wp, T, t_batch, trans, W2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_wy_upd<<<dim3(nch, nct, batch), 256, 0, s>>>(Z, ldz, z_batch, mr, nc, V, ldv, v_batch, rch, W2);
  return hipGetLastError();
}

hipError_t householder_qr(float* A, int64_t m, int64_t k, int64_t ld, int64_t bstride, int batch,
                          float* work, hipStream_t s) {
  constexpr int NB = 32;
  const int64_t P = (k + NB - 1) / NB;
  float* Vall = work;                                        // [batch][P][m][32]
  float* Tall = Vall + static_cast<size_t>(batch) * P * m * NB;   // [batch][P][32][32]
  float* W2 = Tall + static_cast<size_t>(batch) * P * NB * NB;    // [batch][32][k] (two such slots)
  float* taus = W2 + static_cast<size_t>(batch) * 2 * NB * k;     // [batch][2k]
  float* Qb = taus + static_cast<size_t>(batch) * (2 * k + 64);    // [batch][m][32]
  float* part = Qb + panel_factor_scratch_floats(m, batch);       // [batch][kQrSplit][32][k]
  const int64_t vstride = P * m * NB, tstride = P * NB * NB;
  auto Vp = [&](int64_t p) { return Vall + p * m * NB; };
  auto Tp = [&](int64_t p) { return Tall + p * NB * NB; };
  hipError_t e;
  // ---- factorization
  for (int64_t p = 0; p < P; ++p) {
    const int64_t c0 = p * NB;
    const int nb = static_cast<int>(k - c0 < NB ? k - c0 : NB);
    if ((e = panel_factor(A, m, ld, bstride, c0, nb, batch, Vp(p), vstride, Tp(p), tstride, taus, k, Qb, s)) !=
        hipSuccess)
      return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n2 = k - c0 - nb, mr = m - c0;
    if (n2 <= 0) continue;
    // A2 <- (I - V T^T V^T) A2 (rows c0.., the columns right of the panel)
    if ((e = apply_wy_tall(A + (c0 + nb) * ld + c0, ld, bstride, mr, static_cast<int>(n2), Vp(p) + c0, m,
                           vstride, Tp(p), tstride, 1, batch, part, W2, s)) != hipSuccess)
      return e;
  }
  // ---- explicit Q, back to front: the panel's columns start as identity
  // columns, then Q[c0:, c0:] <- (I - V T V^T) Q[c0:, c0:]
  for (int64_t p = P - 1; p >= 0; --p) {
    const int64_t c0 = p * NB;
    const int nb = static_cast<int>(k - c0 < NB ? k - c0 : NB);
    int64_t blocks = (m * nb + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    k_eye_cols<<<dim3(blocks, batch), 256, 0, s>>>(A, m, ld, bstride, c0, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = apply_wy_tall(A + c0 * ld + c0, ld, bstride, m - c0, static_cast<int>(k - c0), Vp(p) + c0, m, vstride,
                           Tp(p), tstride, 0, batch, part, W2, s)) != hipSuccess)
      return e;
  }
  int64_t blocks = (m * k + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_col_signs<<<dim3(blocks, batch), 256, 0, s>>>(A, m, k, ld, bstride, taus);
  return hipGetLastError();
}

int cholesky_qr_ksplit(int64_t m) {
  // the Gram's fp32 sums run over chunks of at most 512 rows, added in a fixed order
  return static_cast<int>(std::min<int64_t>(16, std::max<int64_t>(1, (m + 511) / 512)));
}

int64_t cholesky_qr_max_k() { return kCholMaxK; }

size_t cholesky_qr_work_floats(int64_t m, int64_t k, int batch) {
  return static_cast<size_t>(batch) * (2 + cholesky_qr_ksplit(m)) * k * k;
}

hipError_t cholesky_qr(const float* U, float* Q, int64_t m, int64_t k, int64_t ld, int64_t bstride, int batch,
                       float* work, int* status, hipStream_t s) {
  if (k < 1 || k > kCholMaxK || m < k) return hipErrorInvalidValue;
  const int ks = cholesky_qr_ksplit(m);
  float* G = work;                                               // [batch][k][k], lower triangle
  float* Li = G + static_cast<size_t>(batch) * k * k;            // [batch][k][k], L^{-1} - I
  float* part = Li + static_cast<size_t>(batch) * k * k;         // [batch][ks][k][k]
  ProfScope ps("cholqr", s);
  // algorithmic work: U read twice (Gram, product), Q written once; k (k + 1) m
  // flops for the Gram's triangle, m k (k + 1) for the triangular product,
  // k^3 / 3 for the factorization and inverse
  prof_add_work("cholqr", batch * (3.0 * 4.0 * m * k), batch * (2.0 * k * (k + 1.0) * m + k * k * (k / 3.0)));
  hipError_t e;
  // G = U^T U (row-major, rows m >= columns n).  U is nearly orthonormal, so
  // G departs from I by little and that departure is what L carries: the
  // Gram takes fp32-grade products (three bf16 planes) even for columns
  // concentrated on a few rows.
  GemmArgs g{};
  g.alpha = 1.f;
  g.a_dtype = g.b_dtype = g.c_dtype = kF32;
  g.M = k; g.N = k; g.K = m;
  g.A = U; g.am = plain(ld); g.ak = plain(1); g.a_batch = bstride;
  g.B = U; g.bk = plain(1); g.bn = plain(ld); g.b_batch = bstride;
  g.C = G; g.c_m = k; g.c_n = 1; g.c_batch = k * k;
  g.c_lower = 1;
  g.split_f32 = 2;
  if (ks > 1) { g.ksplit = ks; g.partial = part; }
  if ((e = launch_gemm(g, batch, s, "cholqr_gemm")) != hipSuccess) return e;
  // a pivot below half its column's original diagonal (the column's part
  // outside the span of the earlier ones under sqrt(1/2) of its norm) is
  // more departure from orthonormality than one pass removes to fp32
  // accuracy: the caller falls back to Householder QR
  k_chol_inv<<<batch, CW * 64, 0, s>>>(G, k * k, static_cast<int>(k), 0x1p-1f, Li, k * k, 1, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // Q = U + U (L^{-T} - I), B(j, n) = (L^{-1} - I)[n][j]: U's fp32 values pass
  // through exactly (the identity's term, read in the product's epilogue) and
  // only the small correction carries the split products' rounding (lo x lo,
  // 2^-18 of a correction under 1e-2, left out)
  GemmArgs q{};
  q.alpha = 1.f;
  q.beta = 1.f;
  q.c_in = U;
  q.a_dtype = q.b_dtype = q.c_dtype = kF32;
  q.M = m; q.N = k; q.K = k;
  q.A = U; q.am = plain(1); q.ak = plain(ld); q.a_batch = bstride;
  q.B = Li; q.bk = plain(1); q.bn = plain(k); q.b_batch = k * k;
  q.C = Q; q.c_m = 1; q.c_n = ld; q.c_batch = bstride;
  q.split_f32 = 3;
  q.b_upper = 1;
  return launch_gemm(q, batch, s, "cholqr_gemm");
}

hipError_t finalize_factor_ws(const float* U_cm, int64_t m, int64_t R, int64_t ld_cm, int64_t cm_batch,
                              const double* lam, int64_t lam_batch, float* U_out, int64_t ld_out,
                              int64_t out_batch, double* lam_out, int64_t lam_out_batch, int batch,
                              int* perm, float* sign, hipStream_t s) {
  k_sort_desc<<<batch, 1024, 0, s>>>(lam, R, lam_batch, perm);
  k_col_sign<<<dim3(R, batch), 256, 0, s>>>(U_cm, m, ld_cm, cm_batch, perm, R, sign);
  dim3 grid((m + 127) / 128, (R + 31) / 32, batch);
  k_emit<<<grid, 256, 0, s>>>(U_cm, m, ld_cm, cm_batch, perm, sign, R, lam, lam_batch, U_out, ld_out,
                              out_batch, lam_out, lam_out_batch);
  return hipGetLastError();
}

}  // namespace jolt
