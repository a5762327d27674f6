// Strided, batched fp32-accumulating GEMM on CDNA4 matrix cores, plus the
// small streaming kernels the factor pipeline needs (sum of squares, casts,
// Gaussian sketch, column gathers).
//
// The GEMM serves the codec's dense contractions whose operands are views of
// a [H][T][D] tensor: the token unfolding X_(T)[t][h*D+d] and its transpose
// are not plain strided matrices, so every dimension carries a two-level
// ("segmented") stride: offset(i) = (i / len) * seg + (i % len) * stride.
// Segment lengths are multiples of the tile edge, so a tile never straddles
// a segment and the per-tile base is computed once.
#include "device.hpp"
#include "kernels.hpp"

namespace jolt {

namespace {

constexpr int BM = 64, BN = 64, BK = 16, PAD = 4;

__device__ __forceinline__ int64_t dim_off(const GemmDim& d, int64_t i) {
  return (i / d.len) * d.seg + (i % d.len) * d.stride;
}

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return load_as_f32<T>(static_cast<const T*>(p), i);
}

// One 64x64 output tile per workgroup, 4 waves of 32x32, fp32 MFMA 32x32x2.
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  __shared__ float As[BK][BM + PAD];
  __shared__ float Bs[BK][BN + PAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int64_t zz = blockIdx.z;
  const int64_t z = zz / g.ksplit, kz = zz % g.ksplit;
  const int64_t kbeg = kz * g.kchunk;
  const int64_t kend = (kbeg + g.kchunk < g.K) ? kbeg + g.kchunk : g.K;
  const char* Ab = g.a_ptrs ? static_cast<const char*>(g.a_ptrs[z])
                           : static_cast<const char*>(g.A) + z * g.a_batch * static_cast<int64_t>(sizeof(TA));
  const char* Bb = g.b_ptrs ? static_cast<const char*>(g.b_ptrs[z])
                           : static_cast<const char*>(g.B) + z * g.b_batch * static_cast<int64_t>(sizeof(TB));
  const int64_t a_mbase = dim_off(g.am, m0);
  const int64_t b_nbase = dim_off(g.bn, n0);
  const bool a_mcontig = g.am.stride == 1;
  const bool b_ncontig = g.bn.stride == 1;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  f32x16 acc = {};
  if (g.c_lower && m0 + BM <= n0) return;          // tile wholly above the diagonal

  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const int64_t a_kbase = dim_off(g.ak, k0);
    const int64_t b_kbase = dim_off(g.bk, k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int mm, kk;
      if (a_mcontig) { kk = tid >> 4; mm = ((tid & 15) << 2) + j; }
      else           { mm = tid >> 2; kk = ((tid & 3) << 2) + j; }
      float v = 0.f;
      if (m0 + mm < g.M && k0 + kk < kend) {
        if (g.a_sym && m0 + mm < k0 + kk)
          v = ld<TA>(Ab, (k0 + kk) * g.am.stride + (m0 + mm) * g.ak.stride);
        else
          v = ld<TA>(Ab, a_mbase + mm * g.am.stride + a_kbase + kk * g.ak.stride);
      }
      As[kk][mm] = v;
      int nn, kb;
      if (b_ncontig) { kb = tid >> 4; nn = ((tid & 15) << 2) + j; }
      else           { nn = tid >> 2; kb = ((tid & 3) << 2) + j; }
      float w = 0.f;
      if (n0 + nn < g.N && k0 + kb < kend)
        w = ld<TB>(Bb, b_nbase + nn * g.bn.stride + b_kbase + kb * g.bk.stride);
      Bs[kb][nn] = w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const float a = As[kk + (lane >> 5)][wm + (lane & 31)];
      const float b = Bs[kk + (lane >> 5)][wn + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }

  if (g.ksplit > 1) {   // partial sums, reduced in a fixed order by k_splitk_reduce
    float* Pp = g.partial + (z * g.ksplit + kz) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = m0 + wm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      const int64_t n = n0 + wn + (lane & 31);
      if (m < g.M && n < g.N) Pp[m * g.N + n] = acc[i];
    }
    return;
  }
  char* Cb = static_cast<char*>(g.C);
  const int64_t cz = z * g.c_batch;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t m = m0 + wm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    const int64_t n = n0 + wn + (lane & 31);
    if (m < g.M && n < g.N && (!g.c_lower || m >= n)) {
      float v = g.alpha * acc[i];
      if (g.col_scale) v *= g.col_scale[z * g.col_scale_batch + n];
      const int64_t off = cz + m * g.c_m + n * g.c_n;
      if (g.c_dtype == kF32) {
        float* C = reinterpret_cast<float*>(Cb);
        if (g.beta != 0.f) v += g.beta * C[off];
        C[off] = v;
      } else {
        uint16_t* C = reinterpret_cast<uint16_t*>(Cb);
        C[off] = f32_to_bf16_rne(v);
      }
    }
  }
}

// Both operands bf16: bf16 matrix cores (32x32x16, fp32 accumulation).  A
// product of two bf16 values is exact in fp32, so the result carries the same
// fp32 accumulation as the fp32 path.  LDS holds the tiles k-contiguous per
// row (As[m][k], Bs[n][k]) so that an MFMA operand (8 consecutive k of one
// row) is one 16-byte read; tiles are filled with 16-byte global loads along
// whichever dimension is contiguous.
constexpr int BK16 = 32, KP = BK16 + 8;

__device__ __forceinline__ void fill_tile_bf16(uint16_t (*S)[KP], const uint16_t* base, int64_t rbase,
                                               int64_t rstride, bool rcontig, int64_t kbase, int64_t kstride,
                                               bool kcontig, int64_t r0, int64_t rlim, int64_t k0, int64_t klim,
                                               int tid) {
  // 64 rows x 32 k = 2048 elements, 8 per thread
  if (kcontig) {
    const int r = tid >> 2, kq = (tid & 3) * 8;
    const uint16_t* p = base + rbase + r * rstride + kbase + kq;
    uint16_t v[8];
    if (r0 + r < rlim && k0 + kq + 8 <= klim && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      const uint4 raw = *reinterpret_cast<const uint4*>(p);
      *reinterpret_cast<uint4*>(v) = raw;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (r0 + r < rlim && k0 + kq + i < klim) ? p[i] : static_cast<uint16_t>(0);
    }
    *reinterpret_cast<uint4*>(&S[r][kq]) = *reinterpret_cast<uint4*>(v);
  } else if (rcontig) {
    const int k = tid >> 3, rq = (tid & 7) * 8;
    const uint16_t* p = base + rbase + rq + kbase + k * kstride;
    uint16_t v[8];
    if (r0 + rq + 8 <= rlim && k0 + k < klim && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      const uint4 raw = *reinterpret_cast<const uint4*>(p);
      *reinterpret_cast<uint4*>(v) = raw;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (r0 + rq + i < rlim && k0 + k < klim) ? p[i] : static_cast<uint16_t>(0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) S[rq + i][k] = v[i];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = tid * 8 + j, r = e >> 5, k = e & 31;
      S[r][k] = (r0 + r < rlim && k0 + k < klim) ? base[rbase + r * rstride + kbase + k * kstride]
                                                 : static_cast<uint16_t>(0);
    }
  }
}

__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][KP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN][KP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int64_t zz = blockIdx.z;
  const int64_t z = zz / g.ksplit, kz = zz % g.ksplit;
  const int64_t kbeg = kz * g.kchunk;
  const int64_t kend = (kbeg + g.kchunk < g.K) ? kbeg + g.kchunk : g.K;
  const uint16_t* Ab = g.a_ptrs ? static_cast<const uint16_t*>(g.a_ptrs[z])
                                : static_cast<const uint16_t*>(g.A) + z * g.a_batch;
  const uint16_t* Bb = g.b_ptrs ? static_cast<const uint16_t*>(g.b_ptrs[z])
                                : static_cast<const uint16_t*>(g.B) + z * g.b_batch;
  const int64_t a_mbase = dim_off(g.am, m0);
  const int64_t b_nbase = dim_off(g.bn, n0);
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int r = lane & 31, half = lane >> 5;
  f32x16 acc = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK16) {
    fill_tile_bf16(As, Ab, a_mbase, g.am.stride, g.am.stride == 1, dim_off(g.ak, k0), g.ak.stride,
                   g.ak.stride == 1, m0, g.M, k0, kend, tid);
    fill_tile_bf16(Bs, Bb, b_nbase, g.bn.stride, g.bn.stride == 1, dim_off(g.bk, k0), g.bk.stride,
                   g.bk.stride == 1, n0, g.N, k0, kend, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK16; kk += 16) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[wm + r][kk + 8 * half]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&Bs[wn + r][kk + 8 * half]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  if (g.ksplit > 1) {
    float* Pp = g.partial + (z * g.ksplit + kz) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = m0 + wm + (i >> 2) * 8 + half * 4 + (i & 3);
      const int64_t n = n0 + wn + r;
      if (m < g.M && n < g.N) Pp[m * g.N + n] = acc[i];
    }
    return;
  }
  char* Cb = static_cast<char*>(g.C);
  const int64_t cz = z * g.c_batch;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t m = m0 + wm + (i >> 2) * 8 + half * 4 + (i & 3);
    const int64_t n = n0 + wn + r;
    if (m < g.M && n < g.N) {
      float v = g.alpha * acc[i];
      if (g.col_scale) v *= g.col_scale[z * g.col_scale_batch + n];
      const int64_t off = cz + m * g.c_m + n * g.c_n;
      if (g.c_dtype == kF32) {
        float* C = reinterpret_cast<float*>(Cb);
        if (g.beta != 0.f) v += g.beta * C[off];
        C[off] = v;
      } else {
        uint16_t* C = reinterpret_cast<uint16_t*>(Cb);
        C[off] = f32_to_bf16_rne(v);
      }
    }
  }
}

// C = alpha * sum_kz partial[z][kz] (+ beta C), split order fixed: deterministic.
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs g) {
  const int64_t z = blockIdx.y, MN = g.M * g.N;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < MN; i += 256ll * gridDim.x) {
    const float* p = g.partial + z * g.ksplit * MN + i;
    float acc = 0.f;
    for (int kz = 0; kz < g.ksplit; ++kz) acc += p[kz * MN];
    const int64_t m = i / g.N, n = i % g.N;
    if (g.c_lower && m < n) continue;
    float v = g.alpha * acc;
    if (g.col_scale) v *= g.col_scale[z * g.col_scale_batch + n];
    const int64_t off = z * g.c_batch + m * g.c_m + n * g.c_n;
    if (g.c_dtype == kF32) {
      float* C = static_cast<float*>(g.C);
      if (g.beta != 0.f) v += g.beta * C[off];
      C[off] = v;
    } else {
      static_cast<uint16_t*>(g.C)[off] = f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------- misc
// Sum of squares in fp64, one accumulator per tensor (blockIdx.y).
template <typename T>
__global__ __launch_bounds__(256) void k_sumsq(const void* const* xs, int64_t n, double* out) {
  const T* x = static_cast<const T*>(xs[blockIdx.y]);
  double s = 0.0;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const double v = load_as_f32<T>(x, i);
    s += v * v;
  }
  s = wave_sum(s);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(out + blockIdx.y, part[0] + part[1] + part[2] + part[3]);
}

// Gaussian sketch: out[z][i][j] = N(seed, tag ^ (layer<<8|kind), i*cols + j), fp32.
__global__ __launch_bounds__(256) void k_sketch(float* out, int64_t rows, int64_t cols,
                                                 uint64_t seed, const uint64_t* tags) {
  const int64_t n = rows * cols;
  const uint64_t key = mix64(seed ^ tags[blockIdx.y]);
  float* o = out + blockIdx.y * n;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x)
    o[i] = static_cast<float>(rng_normal(key, static_cast<uint64_t>(i)));
}

// fp32 [rows][ld_in] (first `cols` columns) -> bf16 [rows][cols], RNE.
__global__ __launch_bounds__(256) void k_to_bf16(const float* in, int64_t ld_in, uint16_t* out,
                                                  int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const int64_t r = i / cols, c = i % cols;
    out[i] = f32_to_bf16_rne(in[r * ld_in + c]);
  }
}

// out[z][r + j*ld_out] = in[z][r*ld_in + idx[z][j]] (gather columns, emit column-major).
__global__ __launch_bounds__(256) void k_gather_cols(const float* in, int64_t ld_in, int64_t in_batch,
                                                      const int* idx, int64_t idx_batch,
                                                      float* out, int64_t ld_out, int64_t out_batch,
                                                      int64_t rows, int64_t ncols) {
  const int64_t z = blockIdx.y;
  const int64_t n = rows * ncols;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const int64_t j = i / rows, r = i % rows;
    out[z * out_batch + j * ld_out + r] = in[z * in_batch + r * ld_in + idx[z * idx_batch + j]];
  }
}

// Sum of squares of each row of P [rows][cols] (fp64 accumulation).
__global__ __launch_bounds__(256) void k_row_sumsq(const float* P, int64_t rows, int64_t cols,
                                                    int64_t batch, double* out, int64_t out_batch) {
  const int64_t z = blockIdx.y, r = blockIdx.x;
  const float* p = P + z * batch + r * cols;
  double s = 0.0;
  for (int64_t c = threadIdx.x; c < cols; c += 256) { const double v = p[c]; s += v * v; }
  s = wave_sum(s);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[z * out_batch + r] = part[0] + part[1] + part[2] + part[3];
}

// out[z][j] = sum_i A[z][j*ld + i] * B[z][j*ld + i] (column-major dots, fp64 accumulation).
__global__ __launch_bounds__(256) void k_col_dot(const float* A, const float* B, int64_t m, int64_t ld,
                                                  int64_t bs, double* out, int64_t out_batch) {
  const int64_t z = blockIdx.y, j = blockIdx.x;
  const float* a = A + z * bs + j * ld;
  const float* b = B + z * bs + j * ld;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < m; i += 256) s += static_cast<double>(a[i]) * b[i];
  s = wave_sum(s);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[z * out_batch + j] = part[0] + part[1] + part[2] + part[3];
}

// Copy an n x n fp32 matrix into an n_pad x n_pad zero-padded one (batched).
__global__ __launch_bounds__(256) void k_pad_copy(const float* in, int64_t n, int64_t in_batch,
                                                   float* out, int64_t n_pad) {
  const int64_t z = blockIdx.y, tot = n_pad * n_pad;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < tot; i += 256ll * gridDim.x) {
    const int64_t r = i / n_pad, c = i % n_pad;
    out[z * tot + i] = (r < n && c < n) ? in[z * in_batch + r * n + c] : 0.f;
  }
}

// G_D = sum over heads of the D x D diagonal blocks of the dual Gram C (HD x HD).
__global__ __launch_bounds__(256) void k_sum_diag_blocks(const float* C, int64_t H, int64_t D,
                                                          float* GD) {
  const int64_t z = blockIdx.y, HD = H * D;
  const float* c = C + z * HD * HD;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < D * D; i += 256ll * gridDim.x) {
    const int64_t r = i / D, k = i % D;
    float s = 0.f;
    for (int64_t h = 0; h < H; ++h) s += c[(h * D + r) * HD + h * D + k];
    GD[z * D * D + i] = s;
  }
}

int grid1(int64_t n, int cap = 4096) {
  int64_t b = (n + 255) / 256;
  return static_cast<int>(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g0, int batch, hipStream_t s) {
  GemmArgs g = g0;
  if (g.ksplit < 1 || !g.partial) g.ksplit = 1;
  // bf16 x bf16 on bf16 matrix cores when every segmented dimension keeps a
  // 32-wide k tile inside one segment
  auto seg_ok = [](const GemmDim& d) { return d.len == INT64_MAX || d.len % BK16 == 0; };
  const bool bf = g.a_dtype == kBF16 && g.b_dtype == kBF16 && seg_ok(g.ak) && seg_ok(g.bk) && seg_ok(g.am) &&
                  seg_ok(g.bn) && !g.a_sym && !g.c_lower;
  const int kt = bf ? BK16 : BK;
  g.kchunk = (g.K + g.ksplit - 1) / g.ksplit;
  g.kchunk = (g.kchunk + kt - 1) / kt * kt;            // chunks start on tile edges
  dim3 grid((g.M + BM - 1) / BM, (g.N + BN - 1) / BN, batch * g.ksplit);
  ProfScope ps("gemm", s);
  if (prof_enabled("gemm")) {   // dense flops; operands once, C written (and read when beta != 0) once
    const double ea = g.a_dtype == kBF16 ? 2 : 4, eb = g.b_dtype == kBF16 ? 2 : 4;
    const double ec = g.c_dtype == kBF16 ? 2 : 4;
    prof_add_work("gemm",
                  batch * (g.M * g.K * ea + g.K * g.N * eb + g.M * g.N * ec * (g.beta != 0.f ? 2 : 1)),
                  2.0 * g.M * g.N * g.K * batch);
  }
  if (bf) k_gemm_bf16<<<grid, 256, 0, s>>>(g);
  else if (g.a_dtype == kBF16 && g.b_dtype == kBF16) k_gemm<uint16_t, uint16_t><<<grid, 256, 0, s>>>(g);
  else if (g.a_dtype == kBF16) k_gemm<uint16_t, float><<<grid, 256, 0, s>>>(g);
  else if (g.b_dtype == kBF16) k_gemm<float, uint16_t><<<grid, 256, 0, s>>>(g);
  else k_gemm<float, float><<<grid, 256, 0, s>>>(g);
  if (g.ksplit > 1) {
    k_splitk_reduce<<<dim3(grid1(g.M * g.N), batch), 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_sumsq(const void* const* xs_dev, int ntensors, int64_t n, int dtype, double* out,
                        hipStream_t s) {
  dim3 grid(grid1(n, 1024), ntensors);
  if (dtype == kBF16) k_sumsq<uint16_t><<<grid, 256, 0, s>>>(xs_dev, n, out);
  else k_sumsq<float><<<grid, 256, 0, s>>>(xs_dev, n, out);
  return hipGetLastError();
}

hipError_t launch_sketch(float* out, int64_t rows, int64_t cols, uint64_t seed, const uint64_t* tags,
                         int ntensors, hipStream_t s) {
  k_sketch<<<dim3(grid1(rows * cols), ntensors), 256, 0, s>>>(out, rows, cols, seed, tags);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* in, int64_t ld_in, uint16_t* out, int64_t rows, int64_t cols,
                          hipStream_t s) {
  k_to_bf16<<<grid1(rows * cols), 256, 0, s>>>(in, ld_in, out, rows, cols);
  return hipGetLastError();
}

hipError_t launch_gather_cols(const float* in, int64_t ld_in, int64_t in_batch, const int* idx,
                              int64_t idx_batch, float* out, int64_t ld_out, int64_t out_batch,
                              int64_t rows, int64_t ncols, int batch, hipStream_t s) {
  k_gather_cols<<<dim3(grid1(rows * ncols), batch), 256, 0, s>>>(in, ld_in, in_batch, idx, idx_batch,
                                                                 out, ld_out, out_batch, rows, ncols);
  return hipGetLastError();
}

hipError_t launch_row_sumsq(const float* P, int64_t rows, int64_t cols, int64_t batch_stride,
                            int batch, double* out, int64_t out_batch, hipStream_t s) {
  k_row_sumsq<<<dim3(rows, batch), 256, 0, s>>>(P, rows, cols, batch_stride, out, out_batch);
  return hipGetLastError();
}

hipError_t launch_col_dot(const float* A, const float* B, int64_t m, int64_t ncols, int64_t ld,
                          int64_t batch_stride, int batch, double* out, int64_t out_batch, hipStream_t s) {
  k_col_dot<<<dim3(ncols, batch), 256, 0, s>>>(A, B, m, ld, batch_stride, out, out_batch);
  return hipGetLastError();
}

hipError_t launch_pad_copy(const float* in, int64_t n, int64_t in_batch, float* out, int64_t n_pad,
                           int batch, hipStream_t s) {
  k_pad_copy<<<dim3(grid1(n_pad * n_pad), batch), 256, 0, s>>>(in, n, in_batch, out, n_pad);
  return hipGetLastError();
}

hipError_t launch_sum_diag_blocks(const float* C, int64_t H, int64_t D, float* GD, int batch,
                                  hipStream_t s) {
  k_sum_diag_blocks<<<dim3(grid1(D * D), batch), 256, 0, s>>>(C, H, D, GD);
  return hipGetLastError();
}

}  // namespace jolt
