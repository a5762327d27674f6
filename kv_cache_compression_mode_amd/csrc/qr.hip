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
// trailing columns are updated in chunks of 16 (one block reduction per
// chunk).  Then Q = H_0 ... H_{k-1} [I; 0] is formed in place, back to front,
// and column j is multiplied by sign(beta_j) so that diag(R) >= 0.
// Threads run along rows, so every access is a coalesced column read.
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

__global__ __launch_bounds__(QT) void k_hqr(float* A, int64_t m, int64_t k, int64_t ld, int64_t bstride,
                                            float* tau_g) {
  __shared__ float red[QW][CH];
  __shared__ float red1[QW];
  __shared__ float bc;
  __shared__ float wsum[CH];
  float* a = A + blockIdx.x * bstride;
  float* taus = tau_g + blockIdx.x * 2 * k;       // [tau_j ..., sign(beta_j) ...]
  // ---- factorization
  for (int64_t j = 0; j < k; ++j) {
    float* col = a + j * ld;
    float s = 0.f;
    for (int64_t i = j + 1 + threadIdx.x; i < m; i += QT) s += col[i] * col[i];
    const float sigma = block_sum(s, red1, &bc);
    const float alpha = col[j];
    float tau = 0.f, beta = alpha;
    if (sigma > 0.f) {
      const float nrm = sqrtf(alpha * alpha + sigma);
      beta = alpha >= 0.f ? -nrm : nrm;
      tau = (beta - alpha) / beta;
      const float scale = 1.f / (alpha - beta);
      for (int64_t i = j + 1 + threadIdx.x; i < m; i += QT) col[i] *= scale;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      col[j] = beta;
      taus[j] = tau;
      taus[k + j] = beta < 0.f ? -1.f : 1.f;
    }
    __syncthreads();
    if (tau != 0.f) {
      for (int64_t c0 = j + 1; c0 < k; c0 += CH) {
        const int nc = static_cast<int>(k - c0 < CH ? k - c0 : CH);
        chunk_dots(a, m, ld, j, c0, nc, 1.f, red, wsum);
        // A[i][c] -= tau v_i w_c  (v_j = 1)
        for (int64_t i = j + threadIdx.x; i < m; i += QT) {
          const float vi = (i == j) ? 1.f : col[i];
#pragma unroll
          for (int c = 0; c < CH; ++c)
            if (c < nc) a[(c0 + c) * ld + i] -= tau * vi * wsum[c];
        }
        __syncthreads();
      }
    }
  }
  // ---- form Q in place, back to front
  for (int64_t j = k - 1; j >= 0; --j) {
    const float tau = taus[j];
    float* col = a + j * ld;
    if (tau != 0.f) {
      for (int64_t c0 = j + 1; c0 < k; c0 += CH) {
        const int nc = static_cast<int>(k - c0 < CH ? k - c0 : CH);
        // row j of the formed columns is zero here: w_c = sum_{i>j} v_i Q[i][c]
        chunk_dots(a, m, ld, j, c0, nc, 0.f, red, wsum);
        for (int64_t i = j + threadIdx.x; i < m; i += QT) {
          const float vi = (i == j) ? 1.f : col[i];
#pragma unroll
          for (int c = 0; c < CH; ++c)
            if (c < nc) a[(c0 + c) * ld + i] -= tau * vi * wsum[c];
        }
        __syncthreads();
      }
    }
    for (int64_t i = threadIdx.x; i < m; i += QT) {
      float q;
      if (i < j) q = 0.f;
      else if (i == j) q = 1.f - tau;
      else q = -tau * col[i];
      col[i] = q;
    }
    __syncthreads();
  }
  // ---- diag(R) >= 0
  for (int64_t j = 0; j < k; ++j) {
    if (taus[k + j] < 0.f) {
      float* col = a + j * ld;
      for (int64_t i = threadIdx.x; i < m; i += QT) col[i] = -col[i];
    }
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

hipError_t householder_qr(float* A, int64_t m, int64_t k, int64_t ld, int64_t batch_stride, int batch,
                          float* tau_work, hipStream_t s) {
  k_hqr<<<batch, QT, 0, s>>>(A, m, k, ld, batch_stride, tau_work);
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
