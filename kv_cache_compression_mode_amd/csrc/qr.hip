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
#include "kernels.hpp"

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
  for (int64_t i = threadIdx.x; i < m; i += 256) {
    const float v = fabsf(col[i]);
    if (v > best) { best = v; bi = i; }
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
__global__ __launch_bounds__(256) void k_emit(const float* U, int64_t m, int64_t ld, int64_t bstride,
                                              const int* perm, const float* sign, int64_t R,
                                              const double* lam, int64_t lam_batch, float* out,
                                              int64_t ld_out, int64_t out_batch, double* lam_out,
                                              int64_t lam_out_batch) {
  __shared__ float tile[32][33];
  const int64_t z = blockIdx.z;
  const int64_t i0 = blockIdx.x * 32ll, j0 = blockIdx.y * 32ll;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int jj = ty; jj < 32; jj += 8) {
    const int64_t j = j0 + jj, i = i0 + tx;
    float v = 0.f;
    if (j < R && i < m) {
      const int src = perm[z * R + j];
      v = sign[z * R + j] * U[z * bstride + static_cast<int64_t>(src) * ld + i];
    }
    tile[jj][tx] = v;
  }
  __syncthreads();
  for (int ii = ty; ii < 32; ii += 8) {
    const int64_t i = i0 + ii, j = j0 + tx;
    if (i < m && j < R) out[z * out_batch + i * ld_out + j] = tile[tx][ii];
  }
  if (blockIdx.x == 0 && threadIdx.x < 32) {
    const int64_t j = j0 + threadIdx.x;
    if (j < R) lam_out[z * lam_out_batch + j] = lam[z * lam_batch + perm[z * R + j]];
  }
}

}  // namespace

size_t householder_qr_work_floats(int64_t m, int64_t k, int batch) {
  const int64_t P = (k + 31) / 32;
  // V panels (m x 32 each), T factors (32 x 32 each), W / W2 (32 x k), tau + signs (2k)
  return static_cast<size_t>(batch) * (P * m * 32 + P * 32 * 32 + 2 * 32 * k + 2 * k + 64);
}

hipError_t householder_qr(float* A, int64_t m, int64_t k, int64_t ld, int64_t bstride, int batch,
                          float* work, hipStream_t s) {
  constexpr int NB = 32;
  const int64_t P = (k + NB - 1) / NB;
  float* Vall = work;                                        // [batch][P][m][32]
  float* Tall = Vall + static_cast<size_t>(batch) * P * m * NB;   // [batch][P][32][32]
  float* W = Tall + static_cast<size_t>(batch) * P * NB * NB;     // [batch][32][k]
  float* W2 = W + static_cast<size_t>(batch) * NB * k;            // [batch][32][k]
  float* taus = W2 + static_cast<size_t>(batch) * NB * k;         // [batch][2k]
  const int64_t vstride = P * m * NB, tstride = P * NB * NB;
  auto Vp = [&](int64_t p) { return Vall + p * m * NB; };
  auto Tp = [&](int64_t p) { return Tall + p * NB * NB; };
  auto gemm = [&](int64_t M, int64_t N, int64_t K, const float* Ab, GemmDim am, GemmDim ak, int64_t ab,
                  const float* Bb, GemmDim bk, GemmDim bn, int64_t bb, float* Cb, int64_t cm, int64_t cn,
                  int64_t cb, float alpha, float beta) -> hipError_t {
    if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = Ab; g.a_dtype = kF32; g.am = am; g.ak = ak; g.a_batch = ab;
    g.B = Bb; g.b_dtype = kF32; g.bk = bk; g.bn = bn; g.b_batch = bb;
    g.C = Cb; g.c_dtype = kF32; g.c_m = cm; g.c_n = cn; g.c_batch = cb;
    g.alpha = alpha; g.beta = beta;
    return launch_gemm(g, batch, s);
  };
  hipError_t e;
  // ---- factorization
  for (int64_t p = 0; p < P; ++p) {
    const int64_t c0 = p * NB;
    const int nb = static_cast<int>(k - c0 < NB ? k - c0 : NB);
    {
      ProfScope ps("qr_panel", s);
      k_hqr_panel<<<batch, QT, 0, s>>>(A, m, k, ld, bstride, c0, nb, Vp(p), vstride, Tp(p), tstride, taus);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n2 = k - c0 - nb, mr = m - c0;
    if (n2 <= 0) continue;
    // W = V^T A2  (nb x n2, K = m - c0)
    if ((e = gemm(nb, n2, mr, Vp(p) + c0, plain(m), plain(1), vstride, A + (c0 + nb) * ld + c0, plain(1),
                  plain(ld), bstride, W, k, 1, NB * k, 1.f, 0.f)) != hipSuccess) return e;
    // W2 = T^T W
    if ((e = gemm(nb, n2, nb, Tp(p), plain(1), plain(NB), tstride, W, plain(k), plain(1), NB * k, W2, k,
                  1, NB * k, 1.f, 0.f)) != hipSuccess) return e;
    // A2 -= V W2
    if ((e = gemm(mr, n2, nb, Vp(p) + c0, plain(1), plain(m), vstride, W2, plain(k), plain(1), NB * k,
                  A + (c0 + nb) * ld + c0, 1, ld, bstride, -1.f, 1.f)) != hipSuccess) return e;
  }
  // ---- explicit Q, back to front
  for (int64_t p = P - 1; p >= 0; --p) {
    const int64_t c0 = p * NB;
    const int nb = static_cast<int>(k - c0 < NB ? k - c0 : NB);
    const int64_t n2 = k - c0 - nb, mr = m - c0;
    if (n2 > 0) {
      // Q[c0:, right] -= V (T (V^T Q[c0:, right]))
      if ((e = gemm(nb, n2, mr, Vp(p) + c0, plain(m), plain(1), vstride, A + (c0 + nb) * ld + c0,
                    plain(1), plain(ld), bstride, W, k, 1, NB * k, 1.f, 0.f)) != hipSuccess) return e;
      if ((e = gemm(nb, n2, nb, Tp(p), plain(NB), plain(1), tstride, W, plain(k), plain(1), NB * k, W2,
                    k, 1, NB * k, 1.f, 0.f)) != hipSuccess) return e;
      if ((e = gemm(mr, n2, nb, Vp(p) + c0, plain(1), plain(m), vstride, W2, plain(k), plain(1), NB * k,
                    A + (c0 + nb) * ld + c0, 1, ld, bstride, -1.f, 1.f)) != hipSuccess) return e;
    }
    // panel columns: E - V (T V_top^T), V_top = rows c0 .. c0+nb of V
    int64_t blocks = (m * nb + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    k_eye_cols<<<dim3(blocks, batch), 256, 0, s>>>(A, m, ld, bstride, c0, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = gemm(nb, nb, nb, Tp(p), plain(NB), plain(1), tstride, Vp(p) + c0, plain(m), plain(1), vstride,
                  W2, k, 1, NB * k, 1.f, 0.f)) != hipSuccess) return e;
    if ((e = gemm(mr, nb, nb, Vp(p) + c0, plain(1), plain(m), vstride, W2, plain(k), plain(1), NB * k,
                  A + c0 * ld + c0, 1, ld, bstride, -1.f, 1.f)) != hipSuccess) return e;
  }
  int64_t blocks = (m * k + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_col_signs<<<dim3(blocks, batch), 256, 0, s>>>(A, m, k, ld, bstride, taus);
  return hipGetLastError();
}

hipError_t finalize_factor_ws(const float* U_cm, int64_t m, int64_t R, int64_t ld_cm, int64_t cm_batch,
                              const double* lam, int64_t lam_batch, float* U_out, int64_t ld_out,
                              int64_t out_batch, double* lam_out, int64_t lam_out_batch, int batch,
                              int* perm, float* sign, hipStream_t s) {
  k_sort_desc<<<batch, 1024, 0, s>>>(lam, R, lam_batch, perm);
  k_col_sign<<<dim3(R, batch), 256, 0, s>>>(U_cm, m, ld_cm, cm_batch, perm, R, sign);
  dim3 grid((m + 31) / 32, (R + 31) / 32, batch);
  k_emit<<<grid, 256, 0, s>>>(U_cm, m, ld_cm, cm_batch, perm, sign, R, lam, lam_batch, U_out, ld_out,
                              out_batch, lam_out, lam_out_batch);
  return hipGetLastError();
}

}  // namespace jolt
