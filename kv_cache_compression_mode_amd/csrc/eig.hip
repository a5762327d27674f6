// Symmetric eigensolver for the codec's Gram matrices: parallel block Jacobi.
//
// The factors of the partial Tucker decomposition are leading eigenvectors of
// the token- and feature-mode Grams (JoLT abstract: partial Tucker on the token
// and feature axes; the solver is not named on the pages).  Jacobi suits the
// hardware: every step is a batch of independent plane rotations (no
// sequential Householder chain), clusters of equal eigenvalues need no special
// care, and the block form turns the rotations into dense 64x64x64 products on
// the fp32 matrix cores.
//
// Block form (n = 32 * nb):  a "round" pairs the nb blocks of 32 indices with
// the circle method; every pair (p, q) is a 64 x 64 sub-problem solved by one
// workgroup in LDS (one cyclic sweep of scalar rotations, accumulated into
// J_pq); then A <- J^T A J and V <- V J are applied with matrix-core products,
// in place, each workgroup owning disjoint blocks.  Rotations use the
// threshold |a_pq| > max(tau_abs, tau_rel * sqrt(|a_pp a_qq|)); a sub-problem
// with nothing above threshold leaves J = I and its updates are skipped.  A
// sweep is nb - 1 rounds; the host stops when a sweep rotates nothing.
#include "device.hpp"
#include "kernels.hpp"

namespace jolt {
namespace {

constexpr int SB = 32;       // block edge
constexpr int NS = 64;       // sub-problem edge (a pair of blocks)
constexpr int LP = NS + 1;   // padded LDS row

// One round of the scalar cyclic Jacobi on an ns x ns matrix in LDS (S, with
// row stride ld) accumulating into Jl.  Returns (in threads < ns/2) 1 if a
// rotation was applied.
template <int ns, int ld, int NT>
__device__ __forceinline__ int jacobi_scalar_round(float (*S)[ld], float (*Jl)[ld], float* rc, float* rs,
                                                    int* ru, int* rv, int ir, float tau_rel,
                                                    float tau_abs) {
  const int tid = threadIdx.x;
  int rot = 0;
  if (tid < ns / 2) {
    int u, v;
    rr_pair(tid, ir, ns, &u, &v);
    const float apq = S[u][v], app = S[u][u], aqq = S[v][v];
    float c = 1.f, s = 0.f;
    if (fabsf(apq) > tau_abs && fabsf(apq) > tau_rel * sqrtf(fabsf(app * aqq))) {
      const float theta = (aqq - app) / (2.f * apq);
      const float t = (theta >= 0.f ? 1.f : -1.f) / (fabsf(theta) + sqrtf(theta * theta + 1.f));
      c = 1.f / sqrtf(t * t + 1.f);
      s = t * c;
      rot = 1;
    }
    rc[tid] = c; rs[tid] = s; ru[tid] = u; rv[tid] = v;
  }
  __syncthreads();
  // two-sided update, one 2x2 block (pair i rows x pair j cols) per item
  for (int idx = tid; idx < (ns / 2) * (ns / 2); idx += NT) {
    const int i = idx / (ns / 2), j = idx % (ns / 2);
    const int ui = ru[i], vi = rv[i], uj = ru[j], vj = rv[j];
    const float ci = rc[i], si = rs[i], cj = rc[j], sj = rs[j];
    const float a = S[ui][uj], b = S[ui][vj], c = S[vi][uj], d = S[vi][vj];
    const float a1 = ci * a - si * c, b1 = ci * b - si * d;
    const float c1 = si * a + ci * c, d1 = si * b + ci * d;
    S[ui][uj] = a1 * cj - b1 * sj;
    S[ui][vj] = a1 * sj + b1 * cj;
    S[vi][uj] = c1 * cj - d1 * sj;
    S[vi][vj] = c1 * sj + d1 * cj;
  }
  for (int idx = tid; idx < ns * (ns / 2); idx += NT) {
    const int r = idx / (ns / 2), j = idx % (ns / 2);
    const int uj = ru[j], vj = rv[j];
    const float cj = rc[j], sj = rs[j];
    const float x = Jl[r][uj], y = Jl[r][vj];
    Jl[r][uj] = x * cj - y * sj;
    Jl[r][vj] = x * sj + y * cj;
  }
  __syncthreads();
  return rot;
}

__device__ __forceinline__ int slot_index(int u, int p, int q) {
  return u < SB ? p * SB + u : q * SB + (u - SB);
}

__global__ __launch_bounds__(256) void k_trace_init(float* A, float* V, int64_t n, float tau_abs_rel,
                                                    float* tau_abs) {
  const int64_t z = blockIdx.y;
  float* v = V + z * n * n;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n * n; i += 256ll * gridDim.x)
    v[i] = (i / n == i % n) ? 1.f : 0.f;
  if (blockIdx.x == 0) {
    const float* a = A + z * n * n;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += a[i * n + i];
    s = wave_sum(s);
    __shared__ double part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0)
      tau_abs[z] = tau_abs_rel * static_cast<float>(part[0] + part[1] + part[2] + part[3]);
  }
}

// Sub-problem solve: one workgroup per (pair, matrix).  The scalar rounds are
// latency-bound (two barriers each), so four waves share every round.
constexpr int ST = 256;
__global__ __launch_bounds__(ST) void k_jac_solve(const float* A, int64_t n, float* J, int* active,
                                                  int* rot_count, const float* tau_abs_g, int round,
                                                  float tau_rel) {
  __shared__ float S[NS][LP];
  __shared__ float Jl[NS][LP];
  __shared__ float rc[NS / 2], rs[NS / 2];
  __shared__ int ru[NS / 2], rv[NS / 2];
  const int tid = threadIdx.x;
  const int nb = static_cast<int>(n / SB);
  const int pair = blockIdx.x;
  const int64_t z = blockIdx.y;
  int p, q;
  rr_pair(pair, round, nb, &p, &q);
  const float* a = A + z * n * n;
  // rows of the four 32 x 32 blocks, 16-byte loads
  for (int idx = tid; idx < NS * (NS / 4); idx += ST) {
    const int u = idx / (NS / 4), v4 = (idx % (NS / 4)) * 4;
    const float4 x = *reinterpret_cast<const float4*>(a + static_cast<int64_t>(slot_index(u, p, q)) * n +
                                                      slot_index(v4, p, q));
    S[u][v4] = x.x; S[u][v4 + 1] = x.y; S[u][v4 + 2] = x.z; S[u][v4 + 3] = x.w;
  }
  for (int idx = tid; idx < NS * NS; idx += ST) Jl[idx / NS][idx % NS] = (idx / NS == idx % NS) ? 1.f : 0.f;
  __syncthreads();
  const float tau_abs = tau_abs_g[z];
  int any = 0;
  for (int idx = tid; idx < NS * NS; idx += ST) {
    const int u = idx / NS, v = idx % NS;
    if (u < v) {
      const float apq = S[u][v];
      if (fabsf(apq) > tau_abs && fabsf(apq) > tau_rel * sqrtf(fabsf(S[u][u] * S[v][v]))) any = 1;
    }
  }
  const int64_t aidx = z * (nb / 2) + pair;
  __shared__ int flag;
  if (tid == 0) flag = 0;
  __syncthreads();
  if (any) atomicOr(&flag, 1);
  __syncthreads();
  if (!flag) {
    if (tid == 0) active[aidx] = 0;
    return;
  }
  int nrot = 0;
  for (int ir = 0; ir < NS - 1; ++ir)
    nrot += jacobi_scalar_round<NS, LP, ST>(S, Jl, rc, rs, ru, rv, ir, tau_rel, tau_abs);
  float* jo = J + aidx * NS * NS;
  for (int idx = tid; idx < NS * (NS / 4); idx += ST) {
    const int u = idx / (NS / 4), v4 = (idx % (NS / 4)) * 4;
    *reinterpret_cast<float4*>(jo + u * NS + v4) = make_float4(Jl[u][v4], Jl[u][v4 + 1], Jl[u][v4 + 2],
                                                               Jl[u][v4 + 3]);
  }
  if (nrot) atomicAdd(rot_count + z, nrot);
  if (tid == 0) active[aidx] = 1;
}

// 64x64 += over K=64 on fp32 matrix cores: quadrant (wm, wn) of this wave.
// Aop(m, k) and Bop(k, n) are LDS reads.
#define MFMA_64(ACC, AEXPR, BEXPR)                                              \
  _Pragma("unroll") for (int kk = 0; kk < NS; kk += 2) {                        \
    const int k = kk + (lane >> 5);                                             \
    const int mm = wm + (lane & 31), nn = wn + (lane & 31);                     \
    ACC = __builtin_amdgcn_mfma_f32_32x32x2f32(AEXPR, BEXPR, ACC, 0, 0, 0);     \
  }

// Apply the round's rotations: A super-blocks (i <= j) then V row chunks.
__global__ __launch_bounds__(256) void k_jac_update(float* A, float* V, int64_t n, const float* J,
                                                    const int* active, int round,
                                                    unsigned long long* work) {
  __shared__ float M[NS][LP];
  __shared__ float Ji[NS][LP];
  __shared__ float Jj[NS][LP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int nb = static_cast<int>(n / SB), np = nb / 2;
  const int nA = np * (np + 1) / 2;
  const int64_t z = blockIdx.y;
  const int* act = active + z * np;
  if (static_cast<int>(blockIdx.x) < nA) {
    // linear index -> (i, j), i <= j, row-major over the upper triangle
    int rem = blockIdx.x, i = 0;
    while (rem >= np - i) { rem -= np - i; ++i; }
    const int j = i + rem;
    const int ai = act[i], aj = act[j];
    if (!ai && !aj) return;
    if (work && tid == 0) {   // bytes of A moved (mirror write off the diagonal), MFMA flops
      unsigned long long* w = work + 2 * (blockIdx.y * gridDim.x + blockIdx.x);
      w[0] += static_cast<unsigned long long>(NS * NS * 4 * (i == j ? 2 : 3));
      w[1] += static_cast<unsigned long long>(4 * NS * NS * NS);
    }
    int pi, qi, pj, qj;
    rr_pair(i, round, nb, &pi, &qi);
    rr_pair(j, round, nb, &pj, &qj);
    float* a = A + z * n * n;
    const float* Jpi = J + (z * np + i) * NS * NS;
    const float* Jpj = J + (z * np + j) * NS * NS;
    for (int idx = tid; idx < NS * (NS / 4); idx += 256) {
      const int u = idx / (NS / 4), v4 = (idx % (NS / 4)) * 4;
      const float4 x = *reinterpret_cast<const float4*>(a + static_cast<int64_t>(slot_index(u, pi, qi)) * n +
                                                        slot_index(v4, pj, qj));
      M[u][v4] = x.x; M[u][v4 + 1] = x.y; M[u][v4 + 2] = x.z; M[u][v4 + 3] = x.w;
      const float4 ji = ai ? *reinterpret_cast<const float4*>(Jpi + u * NS + v4)
                           : make_float4(u == v4, u == v4 + 1, u == v4 + 2, u == v4 + 3);
      const float4 jj = aj ? *reinterpret_cast<const float4*>(Jpj + u * NS + v4)
                           : make_float4(u == v4, u == v4 + 1, u == v4 + 2, u == v4 + 3);
      Ji[u][v4] = ji.x; Ji[u][v4 + 1] = ji.y; Ji[u][v4 + 2] = ji.z; Ji[u][v4 + 3] = ji.w;
      Jj[u][v4] = jj.x; Jj[u][v4 + 1] = jj.y; Jj[u][v4 + 2] = jj.z; Jj[u][v4 + 3] = jj.w;
    }
    __syncthreads();
    f32x16 acc = {};
    MFMA_64(acc, Ji[k][mm], M[k][nn]);                   // T = Ji^T M
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r)                         // T overwrites M
      M[wm + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)][wn + (lane & 31)] = acc[r];
    __syncthreads();
    f32x16 acc2 = {};
    MFMA_64(acc2, M[mm][k], Jj[k][nn]);                  // O = T Jj
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r)                         // O overwrites M
      M[wm + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)][wn + (lane & 31)] = acc2[r];
    __syncthreads();
    if (i == j) {
      for (int idx = tid; idx < NS * NS; idx += 256) {
        const int u = idx / NS, v = idx % NS;
        if (u < v) {
          const float s = 0.5f * (M[u][v] + M[v][u]);
          M[u][v] = s;
          M[v][u] = s;
        }
      }
      __syncthreads();
    }
    for (int idx = tid; idx < NS * (NS / 4); idx += 256) {
      const int u = idx / (NS / 4), v4 = (idx % (NS / 4)) * 4;
      *reinterpret_cast<float4*>(a + static_cast<int64_t>(slot_index(u, pi, qi)) * n + slot_index(v4, pj, qj)) =
          make_float4(M[u][v4], M[u][v4 + 1], M[u][v4 + 2], M[u][v4 + 3]);
    }
    if (i != j) {
      for (int idx = tid; idx < NS * NS; idx += 256) {
        const int v = idx / NS, u = idx % NS;
        a[slot_index(v, pj, qj) * n + slot_index(u, pi, qi)] = M[u][v];
      }
    }
  } else {
    const int idx0 = blockIdx.x - nA;
    const int i = idx0 % np;
    const int64_t r0 = static_cast<int64_t>(idx0 / np) * NS;
    if (!act[i]) return;
    if (work && tid == 0) {   // the V block read and written, one product
      unsigned long long* w = work + 2 * (blockIdx.y * gridDim.x + blockIdx.x);
      w[0] += static_cast<unsigned long long>(NS * NS * 4 * 2);
      w[1] += static_cast<unsigned long long>(2 * NS * NS * NS);
    }
    int pi, qi;
    rr_pair(i, round, nb, &pi, &qi);
    float* v = V + z * n * n;
    const float* Jpi = J + (z * np + i) * NS * NS;
    for (int idx = tid; idx < NS * (NS / 4); idx += 256) {
      const int u = idx / (NS / 4), w4 = (idx % (NS / 4)) * 4;
      const float4 x = *reinterpret_cast<const float4*>(v + (r0 + u) * n + slot_index(w4, pi, qi));
      M[u][w4] = x.x; M[u][w4 + 1] = x.y; M[u][w4 + 2] = x.z; M[u][w4 + 3] = x.w;
      const float4 ji = *reinterpret_cast<const float4*>(Jpi + u * NS + w4);
      Ji[u][w4] = ji.x; Ji[u][w4 + 1] = ji.y; Ji[u][w4 + 2] = ji.z; Ji[u][w4 + 3] = ji.w;
    }
    __syncthreads();
    f32x16 acc = {};
    MFMA_64(acc, M[mm][k], Ji[k][nn]);                   // O = M Ji
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      v[(r0 + m) * n + slot_index(wn + (lane & 31), pi, qi)] = acc[r];
    }
  }
}

// Off-diagonal and diagonal sums of squares, rows strided over kOffBlocks
// workgroups per matrix; one partial pair per workgroup (no atomics).
__global__ __launch_bounds__(256) void k_offnorm(const float* A, int64_t n, double* part) {
  const int64_t z = blockIdx.y;
  const float* a = A + z * n * n;
  double off = 0.0, dia = 0.0;
  for (int64_t i = blockIdx.x; i < n; i += kOffBlocks) {
    const float* row = a + i * n;
    for (int64_t j = threadIdx.x; j < n; j += 256) {
      const double v = row[j];
      if (j == i) dia += v * v;
      else off += v * v;
    }
  }
  off = wave_sum(off);
  dia = wave_sum(dia);
  __shared__ double po[4], pd[4];
  if ((threadIdx.x & 63) == 0) { po[threadIdx.x >> 6] = off; pd[threadIdx.x >> 6] = dia; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* p = part + (z * kOffBlocks + blockIdx.x) * 2;
    p[0] = (po[0] + po[1]) + (po[2] + po[3]);
    p[1] = (pd[0] + pd[1]) + (pd[2] + pd[3]);
  }
}

// Scalar cyclic Jacobi to convergence on one 128 x 128 matrix per workgroup.
__global__ __launch_bounds__(512) void k_jacobi128(float* A, float* V, float tau_rel,
                                                   float tau_abs_rel, int max_sweeps) {
  constexpr int N = 128, L = N + 1;
  extern __shared__ float smem[];
  float (*S)[L] = reinterpret_cast<float (*)[L]>(smem);
  float (*Jl)[L] = reinterpret_cast<float (*)[L]>(smem + N * L);
  __shared__ float rc[N / 2], rs[N / 2];
  __shared__ int ru[N / 2], rv[N / 2];
  __shared__ int cnt;
  __shared__ float tr;
  const int tid = threadIdx.x;
  const int64_t z = blockIdx.x;
  float* a = A + z * N * N;
  for (int idx = tid; idx < N * N; idx += 512) {
    S[idx / N][idx % N] = a[idx];
    Jl[idx / N][idx % N] = (idx / N == idx % N) ? 1.f : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int i = 0; i < N; ++i) s += S[i][i];
    tr = static_cast<float>(s);
  }
  __syncthreads();
  const float tau_abs = tau_abs_rel * tr;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    if (tid == 0) cnt = 0;
    __syncthreads();
    int nrot = 0;
    for (int ir = 0; ir < N - 1; ++ir)
      nrot += jacobi_scalar_round<N, L, 512>(S, Jl, rc, rs, ru, rv, ir, tau_rel, tau_abs);
    if (nrot) atomicAdd(&cnt, nrot);
    __syncthreads();
    if (cnt == 0) break;
    __syncthreads();
  }
  float* vv = V + z * N * N;
  for (int idx = tid; idx < N * N; idx += 512) {
    a[idx] = S[idx / N][idx % N];
    vv[idx] = Jl[idx / N][idx % N];
  }
}

// Bitonic sort of (key desc, index asc) in LDS; writes the first R indices.
__global__ __launch_bounds__(1024) void k_topk_diag(const float* A, int64_t n, int R, int* out) {
  __shared__ float key[4096];
  __shared__ int ix[4096];
  const int tid = threadIdx.x;
  const int64_t z = blockIdx.x;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  const float* a = A + z * n * n;
  for (int i = tid; i < n2; i += 1024) {
    key[i] = i < n ? a[static_cast<int64_t>(i) * n + i] : -INFINITY;
    ix[i] = i;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool fwd = (i & size) == 0;
          const float ki = key[i], kj = key[j];
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
  for (int i = tid; i < R; i += 1024) out[z * R + i] = ix[i];
}

}  // namespace

hipError_t jacobi_init(const JacobiWork& w, float tau_abs_rel, hipStream_t s) {
  int64_t blocks = (w.n * w.n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  k_trace_init<<<dim3(blocks, w.batch), 256, 0, s>>>(w.A, w.V, w.n, tau_abs_rel, w.tau_abs);
  return hipGetLastError();
}

hipError_t jacobi_round(const JacobiWork& w, int round, float tau_rel, hipStream_t s) {
  const int nb = static_cast<int>(w.n / SB), np = nb / 2;
  {
    ProfScope ps("jacobi_solve", s);
    k_jac_solve<<<dim3(np, w.batch), ST, 0, s>>>(w.A, w.n, w.J, w.active, w.rot_count, w.tau_abs,
                                                 round, tau_rel);
  }
  const int nA = np * (np + 1) / 2;
  const int nV = np * static_cast<int>(w.n / NS);
  {
    unsigned long long* work = prof_slots("jacobi_update", static_cast<int64_t>(nA + nV) * w.batch);
    ProfScope ps("jacobi_update", s);
    k_jac_update<<<dim3(nA + nV, w.batch), 256, 0, s>>>(w.A, w.V, w.n, w.J, w.active, round, work);
  }
  return hipGetLastError();
}

hipError_t jacobi_offnorm(const float* A, int64_t n, int batch, double* part, hipStream_t s) {
  k_offnorm<<<dim3(kOffBlocks, batch), 256, 0, s>>>(A, n, part);
  return hipGetLastError();
}

hipError_t jacobi_small128(float* A, float* V, int batch, float tau_rel, float tau_abs_rel,
                           int max_sweeps, hipStream_t s) {
  const size_t lds = 2 * 128 * 129 * sizeof(float);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_jacobi128),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr = true;
  }
  ProfScope ps("jacobi128", s);
  k_jacobi128<<<batch, 512, lds, s>>>(A, V, tau_rel, tau_abs_rel, max_sweeps);
  return hipGetLastError();
}

hipError_t topk_diag(const float* A, int64_t n, int batch, int R, int* idx, hipStream_t s) {
  k_topk_diag<<<batch, 1024, 0, s>>>(A, n, R, idx);
  return hipGetLastError();
}

}  // namespace jolt
