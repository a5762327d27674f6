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

#include <utility>

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
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t h) { return bf16_bits_to_f32(h); }

// One 64x64 output tile per workgroup, 4 waves of 32x32, fp32 MFMA 32x32x2,
// K tiles of 32.  Each thread loads fixed positions of every tile (four rows
// by two k, or one row by eight k, along whichever dimension is contiguous);
// the next tile's loads are issued before the current tile's MFMAs, and the
// K position advances with segment counters (no divisions in the loop).
constexpr int FK = 32;
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  __shared__ float As[FK][BM + PAD];
  __shared__ float Bs[FK][BN + PAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int64_t zz = blockIdx.z;
  const int64_t z = zz / g.ksplit, kz = zz % g.ksplit;
  const int64_t kbeg = kz * g.kchunk;
  const int64_t kend = (kbeg + g.kchunk < g.K) ? kbeg + g.kchunk : g.K;
  // tile wholly outside the kept triangle (c_lower > 0: m >= n; < 0: m <= n)
  if (g.c_lower > 0 ? m0 + BM <= n0 : (g.c_lower < 0 && n0 + BN <= m0)) return;
  const char* Ab = g.a_ptrs ? static_cast<const char*>(g.a_ptrs[z])
                           : static_cast<const char*>(g.A) + z * g.a_batch * static_cast<int64_t>(sizeof(TA));
  const char* Bb = g.b_ptrs ? static_cast<const char*>(g.b_ptrs[z])
                           : static_cast<const char*>(g.B) + z * g.b_batch * static_cast<int64_t>(sizeof(TB));
  const bool a_mcontig = g.am.stride == 1;
  const bool b_ncontig = g.bn.stride == 1;
  // this thread's tile positions: element e = 0..7 at row pr(e), k pk(e), four
  // rows by two k along a contiguous row dimension, else one row by eight k
  auto pr = [&](bool rc, int e) { return rc ? ((tid & 15) << 2) + (e & 3) : tid >> 2; };
  auto pk = [&](bool rc, int e) { return rc ? (tid >> 4) + 16 * (e >> 2) : ((tid & 3) << 3) + e; };
  // element offsets inside one batch entry fit in 32 bits (checked at launch)
  const TA* Ap = reinterpret_cast<const TA*>(Ab);
  const TB* Bp = reinterpret_cast<const TB*>(Bb);
  const int a_mbase = static_cast<int>(dim_off(g.am, m0));
  const int b_nbase = static_cast<int>(dim_off(g.bn, n0));
  const int ams = static_cast<int>(g.am.stride), aks = static_cast<int>(g.ak.stride);
  const int bns = static_cast<int>(g.bn.stride), bks = static_cast<int>(g.bk.stride);
  int64_t a_kseg = 0, a_kin = kbeg, b_kseg = 0, b_kin = kbeg;
  if (g.ak.len != INT64_MAX) { a_kseg = kbeg / g.ak.len; a_kin = kbeg % g.ak.len; }
  if (g.bk.len != INT64_MAX) { b_kseg = kbeg / g.bk.len; b_kin = kbeg % g.bk.len; }
  float ra[8], rb[8];
  auto load = [&](int64_t k0) {
    const int a_kbase = static_cast<int>(a_kseg * g.ak.seg + a_kin * g.ak.stride);
    const int b_kbase = static_cast<int>(b_kseg * g.bk.seg + b_kin * g.bk.stride);
    const int kl = static_cast<int>(kend - k0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ar = pr(a_mcontig, e), ak = pk(a_mcontig, e);
      const int64_t m = m0 + ar;
      float v = 0.f;
      if (m < g.M && ak < kl) {
        if (g.a_sym && m < k0 + ak)
          v = to_f32(Ap[static_cast<int>(k0 + ak) * ams + static_cast<int>(m) * aks]);
        else
          v = to_f32(Ap[a_mbase + ar * ams + a_kbase + ak * aks]);
      }
      ra[e] = v;
      const int br = pr(b_ncontig, e), bk = pk(b_ncontig, e);
      rb[e] = (n0 + br < g.N && bk < kl) ? to_f32(Bp[b_nbase + br * bns + b_kbase + bk * bks]) : 0.f;
    }
  };
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  f32x16 acc = {};
  // C (when accumulated, beta != 0) is read before the K loop
  char* Cb = g.c_ptrs ? static_cast<char*>(g.c_ptrs[z]) : static_cast<char*>(g.C);
  const int64_t cz = g.c_ptrs ? 0 : z * g.c_batch;
  auto kept = [&](int64_t m, int64_t n) {
    return m < g.M && n < g.N && (g.c_lower == 0 || (g.c_lower > 0 ? m >= n : m <= n));
  };
  float cold[16];
  const bool rd_c = g.ksplit == 1 && g.beta != 0.f && g.c_dtype == kF32;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t m = m0 + wm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    const int64_t n = n0 + wn + (lane & 31);
    const float* Cr = g.c_in ? g.c_in : reinterpret_cast<const float*>(Cb);
    cold[i] = (rd_c && kept(m, n)) ? Cr[cz + m * g.c_m + n * g.c_n] : 0.f;
  }
  if (kbeg < kend) load(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += FK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      As[pk(a_mcontig, e)][pr(a_mcontig, e)] = ra[e];
      Bs[pk(b_ncontig, e)][pr(b_ncontig, e)] = rb[e];
    }
    __syncthreads();
    if (k0 + FK < kend) {
      a_kin += FK; if (a_kin == g.ak.len) { a_kin = 0; ++a_kseg; }
      b_kin += FK; if (b_kin == g.bk.len) { b_kin = 0; ++b_kseg; }
      load(k0 + FK);
    }
#pragma unroll
    for (int kk = 0; kk < FK; kk += 2) {
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
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t m = m0 + wm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    const int64_t n = n0 + wn + (lane & 31);
    if (kept(m, n)) {
      float v = g.alpha * acc[i];
      if (g.col_scale) v *= g.col_scale[z * g.col_scale_batch + n];
      const int64_t off = cz + m * g.c_m + n * g.c_n;
      if (g.c_dtype == kF32) {
        if (rd_c) v += g.beta * cold[i];
        reinterpret_cast<float*>(Cb)[off] = v;
      } else {
        reinterpret_cast<uint16_t*>(Cb)[off] = f32_to_bf16_rne(v);
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
  char* Cb = g.c_ptrs ? static_cast<char*>(g.c_ptrs[z]) : static_cast<char*>(g.C);
  const int64_t cz = g.c_ptrs ? 0 : z * g.c_batch;
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
        if (g.beta != 0.f) v += g.beta * (g.c_in ? g.c_in : C)[off];
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
    if (g.c_lower > 0 ? m < n : (g.c_lower < 0 && m > n)) continue;
    float v = g.alpha * acc;
    if (g.col_scale) v *= g.col_scale[z * g.col_scale_batch + n];
    void* Cz = g.c_ptrs ? g.c_ptrs[z] : g.C;
    const int64_t off = (g.c_ptrs ? 0 : z * g.c_batch) + m * g.c_m + n * g.c_n;
    if (g.c_dtype == kF32) {
      float* C = static_cast<float*>(Cz);
      if (g.beta != 0.f) v += g.beta * (g.c_in ? g.c_in : C)[off];
      C[off] = v;
    } else {
      static_cast<uint16_t*>(Cz)[off] = f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------- 128 x 128 tiles
// Large products on bf16 matrix cores: 128 x 128 output tiles, K tiles of 64,
// four waves of 64 x 64 (2 x 2 blocks of MFMA 32x32x16).  LDS keeps each
// operand tile k-contiguous per row ([row][k], 144-byte rows) with the
// 16-byte chunk index XOR-swizzled by (row / 16) % 8.  The fragment reads
// (one chunk per lane, sixteen consecutive rows per sixteen lanes) then see
// one swizzle and the odd 144-byte stride alone, which puts sixteen rows on
// sixteen distinct 16-byte bank groups; the transposing writes (rows 8 apart
// across lanes) are spread by the swizzle.  Operands in memory:
//   kOpBfK   bf16, k contiguous: 16-byte loads along k;
//   kOpBfM   bf16, rows contiguous: 16-byte loads along the rows, transposed
//            in registers (four k by eight rows per thread) on the way to LDS;
//   kOpF32K  fp32, k contiguous: split into bf16 planes hi = rne(x),
//            lo = rne(x - hi), so x = hi + lo to 2^-17 relative; the product
//            takes hi B + lo B (or A hi + A lo): exact bf16 products summed in
//            fp32, ~2^-17 relative error per term (fp32 operands: 2^-24);
//   kOpF32M  fp32, rows contiguous: 16-byte loads of four rows at one k,
//            split the same way and transposed in registers (four rows by
//            four k per thread) on the way to LDS.
// Both operands fp32 (split_f32): all four products hi hi + lo hi + hi lo +
// lo lo (lo is about 2^-8 of x, so lo lo is a 2^-16 term, and one of a
// fixed sign in a Gram's diagonal: it is kept), or (split_f32 = 3, a product
// that forms a small correction) the first three.
// The next K tile's global loads are issued before the current tile's MFMAs.
constexpr int XT = 128, XK = 64, XKP = XK + 8;
enum { kOpBfK = 0, kOpBfM = 1, kOpF32K = 2, kOpF32M = 3 };

__device__ __forceinline__ int xswz(int row, int chunk) { return chunk ^ ((row >> 4) & 7); }

template <int MODE> struct XRegs { uint4 v[4]; };
template <> struct XRegs<kOpF32K> { float4 v[8]; };
template <> struct XRegs<kOpF32M> { float4 v[8]; };

// One operand's addressing: a buffer resource on its batch entry, this
// thread's byte offsets (rows and in-tile k; kXOut for rows past the end,
// which read as zero) and the K tile's byte offset, advanced per tile with
// scalar segment counters.  Every offset fits in 31 bits (checked at launch).
constexpr uint32_t kXOut = 0x80000000u;
struct XAddr {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo[8];
  int64_t kseg, kin;
};

__device__ __forceinline__ int64_t x_koff(const GemmDim& kd, const XAddr& a) {
  return a.kseg * kd.seg + a.kin * kd.stride;
}

template <int MODE>
__device__ __forceinline__ void x_addr(XAddr& a, const char* base, const GemmDim& rd, const GemmDim& kd,
                                       int64_t r0, int64_t rows, int64_t kbeg, int tid) {
  a.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, static_cast<int>(kXOut), 0x00020000);
  if (kd.len == INT64_MAX) { a.kseg = 0; a.kin = kbeg; }
  else { a.kseg = kbeg / kd.len; a.kin = kbeg % kd.len; }
  if constexpr (MODE == kOpBfM) {
    const int64_t r = r0 + 8 * (tid & 15);
    const int64_t rb = dim_off(rd, r0) + 8 * (tid & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a.vo[i] = r < rows ? static_cast<uint32_t>(2 * (rb + (4 * (tid >> 4) + i) * kd.stride)) : kXOut;
  } else if constexpr (MODE == kOpF32M) {
    // rows 4 (tid % 32) .. + 3 (rows is a multiple of 4), k = 4 (tid / 32) + 32 h + j, load 4 h + j
    const int64_t r = r0 + 4 * (tid & 31);
    const int64_t rb = dim_off(rd, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t k = 4 * (tid >> 5) + 32 * (i >> 2) + (i & 3);
      a.vo[i] = r < rows ? static_cast<uint32_t>(4 * (rb + k * kd.stride)) : kXOut;
    }
  } else {
    constexpr int NR = MODE == kOpBfK ? 4 : 8, SH = MODE == kOpBfK ? 3 : 4;
    constexpr int64_t E = MODE == kOpBfK ? 2 : 4;
    const int64_t kl = MODE == kOpBfK ? 8 * (tid & 7) : 4 * (tid & 15);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t r = r0 + (tid >> SH) + (XT / NR) * i;
      a.vo[i] = r < rows ? static_cast<uint32_t>(E * (dim_off(rd, r) + kl)) : kXOut;
    }
  }
}

__device__ __forceinline__ void x_next(XAddr& a, const GemmDim& kd) {
  a.kin += XK;
  if (a.kin == kd.len) { a.kin = 0; ++a.kseg; }
}

template <int MODE>
__device__ __forceinline__ void x_load(XRegs<MODE>& R, const XAddr& a, const GemmDim& kd) {
  constexpr int64_t E = MODE == kOpF32K || MODE == kOpF32M ? 4 : 2;
  // the K tile's offset is the same in every lane: a scalar operand
  const int so = __builtin_amdgcn_readfirstlane(static_cast<int>(E * x_koff(kd, a)));
  if constexpr (MODE == kOpF32K || MODE == kOpF32M) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(a.rs, static_cast<int>(a.vo[i]), so, 0);
      R.v[i] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                           __uint_as_float(v[3]));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(a.rs, static_cast<int>(a.vo[i]), so, 0);
      R.v[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
}

__device__ __forceinline__ uint32_t x_half(const uint4& v, int e) {    // 16-bit element e of eight
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ void x_split(float x, uint32_t& hi, uint32_t& lo) {
  const uint16_t h = f32_to_bf16_rne(x);
  hi = h;
  lo = f32_to_bf16_rne(x - bf16_bits_to_f32(h));
}
// three planes: x = hi + mid + lo to 2^-24 relative (the fp32 significand)
__device__ __forceinline__ void x_split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint16_t h = f32_to_bf16_rne(x);
  const float r = x - bf16_bits_to_f32(h);
  const uint16_t m = f32_to_bf16_rne(r);
  hi = h;
  mid = m;
  lo = f32_to_bf16_rne(r - bf16_bits_to_f32(m));
}

template <int MODE, int NP = 2>
__device__ __forceinline__ void x_store(const XRegs<MODE>& R, uint16_t (*Sh)[XKP], uint16_t (*Sl)[XKP],
                                        uint16_t (*S3)[XKP], int tid) {
  if constexpr (MODE == kOpBfK) {
    const int kc = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(&Sh[row][xswz(row, kc) * 8]) = R.v[i];
    }
  } else if constexpr (MODE == kOpBfM) {
    const int mc = tid & 15, kg = tid >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 8 * mc + e;
      uint2 w;
      w.x = x_half(R.v[0], e) | (x_half(R.v[1], e) << 16);
      w.y = x_half(R.v[2], e) | (x_half(R.v[3], e) << 16);
      *reinterpret_cast<uint2*>(&Sh[row][xswz(row, kg >> 1) * 8 + (kg & 1) * 4]) = w;
    }
  } else if constexpr (MODE == kOpF32M) {
    const int rg = tid & 31, kq = tid >> 5;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = 4 * kq + 32 * h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * rg + e;
        uint32_t hh[4], ll[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 v = R.v[4 * h + j];
          x_split(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w, hh[j], ll[j]);
        }
        const int col = xswz(row, kb >> 3) * 8 + (kb & 7);
        *reinterpret_cast<uint2*>(&Sh[row][col]) = make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
        *reinterpret_cast<uint2*>(&Sl[row][col]) = make_uint2(ll[0] | (ll[1] << 16), ll[2] | (ll[3] << 16));
      }
    }
  } else {
    const int kc4 = tid & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 4) + 16 * i;
      uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
      const int col = xswz(row, kc4 >> 1) * 8 + (kc4 & 1) * 4;
      if constexpr (NP == 3) {
        uint32_t t0, t1, t2, t3;
        x_split3(R.v[i].x, h0, l0, t0); x_split3(R.v[i].y, h1, l1, t1);
        x_split3(R.v[i].z, h2, l2, t2); x_split3(R.v[i].w, h3, l3, t3);
        *reinterpret_cast<uint2*>(&S3[row][col]) = make_uint2(t0 | (t1 << 16), t2 | (t3 << 16));
      } else {
        x_split(R.v[i].x, h0, l0); x_split(R.v[i].y, h1, l1);
        x_split(R.v[i].z, h2, l2); x_split(R.v[i].w, h3, l3);
      }
      *reinterpret_cast<uint2*>(&Sh[row][col]) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      *reinterpret_cast<uint2*>(&Sl[row][col]) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
    }
  }
}

// NP = 3 (both operands fp32, k contiguous): three planes each, and the six
// products down to 2^-16 (hi hi, mid hi, hi mid, mid mid, lo hi, hi lo),
// fp32-grade products for sums whose rounding must not exceed fp32's.
template <int AM, int BMODE, int NP = 2>
__global__ __launch_bounds__(256, 2) void k_gemm_x(GemmArgs g) {
  constexpr bool AS = AM == kOpF32K || AM == kOpF32M, BS = BMODE == kOpF32K || BMODE == kOpF32M;
  static_assert(NP == 2 || (AM == kOpF32K && BMODE == kOpF32K), "three planes: fp32 k-contiguous operands");
  __shared__ __attribute__((aligned(16))) uint16_t As[AS ? NP : 1][XT][XKP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BS ? NP : 1][XT][XKP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups are dispatched round-robin over the 8 XCDs by linear id; when
  // the batch dimension is a multiple of 8 the id is remapped so that every
  // tile of one batch entry runs on the same XCD (its operands stream through
  // one L2 together rather than through all eight).  A bijection of the ids.
  uint32_t bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (gridDim.z % 8 == 0) {
    const uint32_t G = gridDim.x * gridDim.y;
    const uint32_t L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t xcd = L % 8, j = L / 8, tile = j % G;
    bz = xcd + 8 * (j / G);
    bx = tile % gridDim.x;
    by = tile / gridDim.x;
  }
  const int64_t m0 = static_cast<int64_t>(bx) * XT;
  const int64_t n0 = static_cast<int64_t>(by) * XT;
  // tile wholly outside the kept triangle (c_lower > 0: m >= n; < 0: m <= n)
  if (g.c_lower > 0 ? m0 + XT <= n0 : (g.c_lower < 0 && n0 + XT <= m0)) return;
  const int64_t zz = bz;
  const int64_t z = zz / g.ksplit, kz = zz % g.ksplit;
  const int64_t kbeg = kz * g.kchunk;
  int64_t kend = (kbeg + g.kchunk < g.K) ? kbeg + g.kchunk : g.K;
  if (g.a_lower && m0 + XT < kend) kend = m0 + XT;
  if (g.b_upper && n0 + XT < kend) kend = n0 + XT;
  const size_t ea = AS ? 4 : 2, eb = BS ? 4 : 2;
  const char* Ab = g.a_ptrs ? static_cast<const char*>(g.a_ptrs[z])
                            : static_cast<const char*>(g.A) + z * g.a_batch * static_cast<int64_t>(ea);
  const char* Bb = g.b_ptrs ? static_cast<const char*>(g.b_ptrs[z])
                            : static_cast<const char*>(g.B) + z * g.b_batch * static_cast<int64_t>(eb);
  XAddr pa, pb;
  x_addr<AM>(pa, Ab, g.am, g.ak, m0, g.M, kbeg, tid);
  x_addr<BMODE>(pb, Bb, g.bn, g.bk, n0, g.N, kbeg, tid);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int r = lane & 31, half = lane >> 5;
  // in-order chunk sums (seq_len > 0) only where A is bf16: the launcher
  // never asks them of an fp32 A, whose kernels keep those 64 registers
  constexpr bool SEQ = !AS;
  f32x16 acc[2][2] = {};
  f32x16 sum[SEQ ? 2 : 1][SEQ ? 2 : 1] = {};   // the finished chunks, added in order
  // K tiles in flight: two register stages where the registers allow (a
  // stage is 16 registers per bf16 operand, 32 per fp32 one), so that a
  // tile's global loads have two tiles of matrix-core work to arrive in
  constexpr int PF = !BS ? 2 : 1;
  XRegs<AM> ra[PF];
  XRegs<BMODE> rb[PF];
  // Every tile issues its stage's loads: past the last tile the address
  // stays on the last one (a harmless reload), so that the loads and their
  // waits follow one pattern on every path through the loop.
  if (kbeg < kend) {
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      if (st > 0 && kbeg + st * XK < kend) { x_next(pa, g.ak); x_next(pb, g.bk); }
      x_load<AM>(ra[st], pa, g.ak);
      x_load<BMODE>(rb[st], pb, g.bk);
    }
  }
  int64_t seq_left = g.seq_len;   // K left in the current chunk
  auto tile = [&](XRegs<AM>& ra_, XRegs<BMODE>& rb_, int64_t k0) {
    x_store<AM, NP>(ra_, As[0], As[AS ? 1 : 0], As[AS ? NP - 1 : 0], tid);
    x_store<BMODE, NP>(rb_, Bs[0], Bs[BS ? 1 : 0], Bs[BS ? NP - 1 : 0], tid);
    __syncthreads();
    if (k0 + PF * XK < kend) {
      x_next(pa, g.ak);
      x_next(pb, g.bk);
    }
    x_load<AM>(ra_, pa, g.ak);
    x_load<BMODE>(rb_, pb, g.bk);
#pragma unroll
    for (int kk = 0; kk < XK / 16; ++kk) {
      const int ch = 2 * kk + half;
      bf16x8 a[2], b[2], al[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra_r = wm + 32 * i + r, rb_r = wn + 32 * i + r;
        a[i] = *reinterpret_cast<const bf16x8*>(&As[0][ra_r][xswz(ra_r, ch) * 8]);
        b[i] = *reinterpret_cast<const bf16x8*>(&Bs[0][rb_r][xswz(rb_r, ch) * 8]);
        if constexpr (AS) al[i] = *reinterpret_cast<const bf16x8*>(&As[AS ? 1 : 0][ra_r][xswz(ra_r, ch) * 8]);
        if constexpr (BS) bl[i] = *reinterpret_cast<const bf16x8*>(&Bs[BS ? 1 : 0][rb_r][xswz(rb_r, ch) * 8]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
          if constexpr (AS) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], b[j], acc[i][j], 0, 0, 0);
          if constexpr (BS) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bl[j], acc[i][j], 0, 0, 0);
          if constexpr (AS && BS)
            if (g.split_f32 != 3)                  // 3: lo x lo left out (a small correction's product)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bl[j], acc[i][j], 0, 0, 0);
          if constexpr (NP == 3) {
            const int ra_r = wm + 32 * i + r, rb_r = wn + 32 * j + r;
            const bf16x8 a3 = *reinterpret_cast<const bf16x8*>(&As[NP - 1][ra_r][xswz(ra_r, ch) * 8]);
            const bf16x8 b3 = *reinterpret_cast<const bf16x8*>(&Bs[NP - 1][rb_r][xswz(rb_r, ch) * 8]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b3, acc[i][j], 0, 0, 0);
          }
        }
    }
    if (SEQ && g.seq_len > 0) {
      seq_left -= XK;
      if (seq_left == 0 || k0 + XK >= kend) {
        // a chunk done: sum = ((0 + c0) + c1) + ..., the order of the split-K reduction
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            sum[SEQ ? i : 0][SEQ ? j : 0] += acc[i][j];
            acc[i][j] = f32x16{};
          }
        seq_left = g.seq_len;
      }
    }
    __syncthreads();
  };
  int64_t k0 = kbeg;
  if constexpr (PF == 2)
    for (; k0 + XK < kend; k0 += 2 * XK) {
      tile(ra[0], rb[0], k0);
      tile(ra[PF - 1], rb[PF - 1], k0 + XK);
    }
  for (; k0 < kend; k0 += XK) tile(ra[0], rb[0], k0);
  if (SEQ && g.seq_len > 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = sum[SEQ ? i : 0][SEQ ? j : 0];
  }
  if (g.ksplit > 1) {   // partial sums, reduced in a fixed order by k_splitk_reduce
    float* Pp = g.partial + (z * g.ksplit + kz) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + wm + 32 * i + (e >> 2) * 8 + half * 4 + (e & 3);
          const int64_t n = n0 + wn + 32 * j + r;
          if (m < g.M && n < g.N) Pp[m * g.N + n] = acc[i][j][e];
        }
    return;
  }
  char* Cb = g.c_ptrs ? static_cast<char*>(g.c_ptrs[z]) : static_cast<char*>(g.C);
  const int64_t cz = g.c_ptrs ? 0 : z * g.c_batch;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm + 32 * i + (e >> 2) * 8 + half * 4 + (e & 3);
        const int64_t n = n0 + wn + 32 * j + r;
        if (m < g.M && n < g.N && (g.c_lower == 0 || (g.c_lower > 0 ? m >= n : m <= n))) {
          float v = g.alpha * acc[i][j][e];
          if (g.col_scale) v *= g.col_scale[z * g.col_scale_batch + n];
          const int64_t off = cz + m * g.c_m + n * g.c_n;
          if (g.c_dtype == kF32) {
            float* C = reinterpret_cast<float*>(Cb);
            if (g.beta != 0.f) v += g.beta * (g.c_in ? g.c_in : C)[off];
            C[off] = v;
          } else {
            reinterpret_cast<uint16_t*>(Cb)[off] = f32_to_bf16_rne(v);
          }
        }
      }
}

// ---------------------------------------------------------------- misc
// Sum of squares in fp64, one accumulator per tensor (blockIdx.y).
// 16-byte loads, four in flight per thread, where the tensor is 16-byte
// aligned and a multiple of 16 bytes long; element loads otherwise.
template <typename T>
__global__ __launch_bounds__(256) void k_sumsq(const void* const* xs, int64_t n, double* out) {
  const T* x = static_cast<const T*>(xs[blockIdx.y]);
  constexpr int E = 16 / sizeof(T);                     // elements per 16 bytes
  double s = 0.0;
  const int64_t stride = 256ll * gridDim.x;
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0 && n % E == 0) {
    const int64_t nv = n / E;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    for (int64_t i0 = blockIdx.x * 256ll + threadIdx.x; i0 < nv; i0 += 4 * stride) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = i0 + u * stride < nv ? xv[i0 + u * stride] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const double d = load_as_f32<T>(e, k);
          s += d * d;
        }
      }
    }
  } else {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += stride) {
      const double v = load_as_f32<T>(x, i);
      s += v * v;
    }
  }
  s = wave_sum(s);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(out + blockIdx.y, part[0] + part[1] + part[2] + part[3]);
}

// Gaussian sketch, stored column-major: element (i, j) of the rows x cols
// matrix is N(seed, tag ^ (layer<<8|kind), i*cols + j) at out[z][j][i], fp32
// (its product with the token unfolding then reads it k-contiguous).
__global__ __launch_bounds__(256) void k_sketch(float* out, int64_t rows, int64_t cols,
                                                 uint64_t seed, const uint64_t* tags) {
  const int64_t n = rows * cols;
  const uint64_t key = mix64(seed ^ tags[blockIdx.y]);
  float* o = out + blockIdx.y * n;
  for (int64_t o_idx = blockIdx.x * 256ll + threadIdx.x; o_idx < n; o_idx += 256ll * gridDim.x) {
    const int64_t j = o_idx / rows, i = o_idx - j * rows;
    o[o_idx] = static_cast<float>(rng_normal(key, static_cast<uint64_t>(i * cols + j)));
  }
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

// out[z] = bf16(in[z]) for rows x cols of row stride ld_in, per-tensor pointers.
__global__ __launch_bounds__(256) void k_to_bf16_many(const float* const* ins, int64_t ld_in, uint16_t* const* outs,
                                                       int64_t rows, int64_t cols) {
  const float* in = ins[blockIdx.y];
  uint16_t* out = outs[blockIdx.y];
  const int64_t n = rows * cols;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const int64_t r = i / cols, c = i % cols;
    out[i] = f32_to_bf16_rne(in[r * ld_in + c]);
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

// G_D = sum over heads of the D x D diagonal blocks of the dual Gram C (HD x HD,
// symmetric, column-major; only its lower triangle is read).
__global__ __launch_bounds__(256) void k_sum_diag_blocks(const float* C, int64_t H, int64_t D,
                                                          float* GD) {
  const int64_t z = blockIdx.y, HD = H * D;
  const float* c = C + z * HD * HD;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < D * D; i += 256ll * gridDim.x) {
    const int64_t r = i / D, k = i % D, lo = r < k ? r : k, hi = r < k ? k : r;
    float s = 0.f;
    for (int64_t h = 0; h < H; ++h) s += c[(h * D + lo) * HD + h * D + hi];
    GD[z * D * D + i] = s;
  }
}

// out[i] = sum over the batch of in[j][i], in batch order (deterministic).
__global__ __launch_bounds__(256) void k_sum_batch(const float* in, int64_t count, int n, float* out) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < count; i += 256ll * gridDim.x) {
    float s = 0.f;
    for (int j = 0; j < n; ++j) s += in[j * count + i];
    out[i] = s;
  }
}

int grid1(int64_t n, int cap = 4096) {
  int64_t b = (n + 255) / 256;
  return static_cast<int>(b < 1 ? 1 : (b > cap ? cap : b));
}

// Largest element offset of indices [0, n) along d (strides non-negative).
int64_t dim_span(const GemmDim& d, int64_t n) {
  if (n <= 0) return 0;
  const int64_t i = n - 1;
  return d.len == INT64_MAX ? i * d.stride : (i / d.len) * d.seg + (i % d.len) * d.stride;
}
// Largest |offset| of indices [0, n) along d (any signs).
int64_t dim_reach(const GemmDim& d, int64_t n) {
  if (n <= 0) return 0;
  auto ab = [](int64_t v) { return v < 0 ? -v : v; };
  if (d.len == INT64_MAX) return ab((n - 1) * d.stride);
  const int64_t nseg = (n + d.len - 1) / d.len, inner = (n < d.len ? n : d.len) - 1;
  return ab((nseg - 1) * d.seg) + ab(inner * d.stride);
}

// Operand mode for the 128 x 128 kernel (rows rd, contraction kd), or -1.
int x_mode(int dtype, const GemmDim& rd, const GemmDim& kd, int64_t rows, int64_t kext, bool use_ptrs,
           bool ptrs_aligned, const void* base, int64_t batch_stride) {
  const int64_t q = dtype == kBF16 ? 8 : 4;     // elements per 16 bytes
  auto mult = [](int64_t v, int64_t m) { return v % m == 0; };
  auto within = [](const GemmDim& d, int64_t t) { return d.len == INT64_MAX || d.len % t == 0; };
  auto seg16 = [&](const GemmDim& d) { return d.len == INT64_MAX || mult(d.seg, q); };
  if (use_ptrs ? !ptrs_aligned : ((reinterpret_cast<uintptr_t>(base) & 15) != 0 || !mult(batch_stride, q)))
    return -1;
  // every byte offset inside one batch entry below 2^31 (buffer addressing)
  if (rd.stride < 0 || kd.stride < 0 || rd.seg < 0 || kd.seg < 0 ||
      (dim_span(rd, rows + XT) + dim_span(kd, kext) + 8) * (dtype == kBF16 ? 2 : 4) >= (int64_t{1} << 31))
    return -1;
  if (kd.stride == 1 && within(kd, XK) && seg16(kd) && mult(rd.stride, q) && seg16(rd))
    return dtype == kBF16 ? kOpBfK : kOpF32K;
  if (dtype == kBF16 && rd.stride == 1 && within(rd, XT) && seg16(rd) && mult(rows, 8) && within(kd, XK) &&
      mult(kd.stride, q) && seg16(kd))
    return kOpBfM;
  if (dtype == kF32 && rd.stride == 1 && within(rd, XT) && seg16(rd) && mult(rows, 4) && within(kd, XK) &&
      mult(kd.stride, q) && seg16(kd))
    return kOpF32M;
  return -1;
}

template <int AM>
void launch_x_b(const GemmArgs& g, int xb, dim3 grid, hipStream_t s) {
  if (xb == kOpBfK) k_gemm_x<AM, kOpBfK><<<grid, 256, 0, s>>>(g);
  else if (xb == kOpBfM) k_gemm_x<AM, kOpBfM><<<grid, 256, 0, s>>>(g);
  else if (xb == kOpF32K) k_gemm_x<AM, kOpF32K><<<grid, 256, 0, s>>>(g);
  else k_gemm_x<AM, kOpF32M><<<grid, 256, 0, s>>>(g);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g0, int batch, hipStream_t s, const char* scope) {
  GemmArgs g = g0;
  if (g.c_in && (g.c_ptrs || g.c_dtype != kF32)) return hipErrorInvalidValue;
  if (g.ksplit < 1 || !g.partial) g.ksplit = 1;
  // algorithmic work: operands read once, C written (and read when beta != 0)
  // once; 2 M N K flops, or for a triangle-only output (a symmetric product
  // such as a Gram) its half: M (M + 1) K flops and M (M + 1) / 2 outputs
  auto account = [&](const char* name) {
    if (!prof_enabled(name)) return;
    const double ea = g.a_dtype == kBF16 ? 2 : 4, eb = g.b_dtype == kBF16 ? 2 : 4;
    const double ec = g.c_dtype == kBF16 ? 2 : 4;
    const bool tri = g.c_lower != 0 && g.M == g.N;
    const double outs = tri ? 0.5 * g.M * (g.M + 1.0) : 1.0 * g.M * g.N;
    const double fl = tri ? 1.0 * g.M * (g.M + 1.0) * g.K : 2.0 * g.M * g.N * g.K;
    // a Gram reads its one operand once (A and B are the same tensor)
    const bool same = (g.A && g.A == g.B) || (g.a_ptrs && g.a_ptrs == g.b_ptrs);
    const double in = same ? g.M * g.K * ea : g.M * g.K * ea + g.K * g.N * eb;
    prof_add_work(name, batch * (in + outs * ec * (g.beta != 0.f ? 2 : 1)), fl * batch);
  };
  // 128 x 128 bf16 matrix-core tiles when the operands allow 16-byte loads
  // (at least one of them bf16); a column-major C is produced as the
  // row-major C^T = B^T A^T so that its stores run along rows
  if (!g.a_sym && g.K % XK == 0 && (g.a_dtype == kBF16 || g.b_dtype == kBF16 || g.split_f32)) {
    GemmArgs x = g;
    if (x.c_m == 1 && x.c_n != 1 && !x.col_scale) {
      std::swap(x.M, x.N); std::swap(x.A, x.B); std::swap(x.a_dtype, x.b_dtype);
      std::swap(x.am, x.bn); std::swap(x.ak, x.bk); std::swap(x.a_batch, x.b_batch);
      std::swap(x.a_ptrs, x.b_ptrs); std::swap(x.c_m, x.c_n);
      std::swap(x.a_lower, x.b_upper);                 // B^T lower <=> B upper
      x.c_lower = -x.c_lower;                          // m >= n of C is m <= n of C^T
    }
    const int xa = x_mode(x.a_dtype, x.am, x.ak, x.M, x.K, x.a_ptrs != nullptr, x.ptr_align16 != 0, x.A, x.a_batch);
    const int xb = x_mode(x.b_dtype, x.bn, x.bk, x.N, x.K, x.b_ptrs != nullptr, x.ptr_align16 != 0, x.B, x.b_batch);
    // two fp32 operands (split_f32) need one of them k contiguous
    const bool fa = xa == kOpF32K || xa == kOpF32M, fb = xb == kOpF32K || xb == kOpF32M;
    const bool pair_ok = xa >= 0 && xb >= 0 && (!(fa && fb) || ((xa == kOpF32K || xb == kOpF32K) && g.split_f32));
    if (pair_ok) {
      x.kchunk = (x.K + x.ksplit - 1) / x.ksplit;
      x.kchunk = (x.kchunk + XK - 1) / XK * XK;
      x.seq_len = 0;
      // the chunks in one workgroup, summed in order (kernels with a bf16 A)
      if (x.split_seq && x.ksplit > 1 && (xa == kOpBfK || xa == kOpBfM)) {
        x.seq_len = x.kchunk;
        x.ksplit = 1;
        x.kchunk = x.K;
      }
      dim3 grid((x.M + XT - 1) / XT, (x.N + XT - 1) / XT, batch * x.ksplit);
      const char* name = scope ? scope : "gemm_bf16";
      ProfScope ps(name, s);
      account(name);
      if (xa == kOpBfK) launch_x_b<kOpBfK>(x, xb, grid, s);
      else if (xa == kOpBfM) launch_x_b<kOpBfM>(x, xb, grid, s);
      else if (xa == kOpF32K && xb == kOpF32K && x.split_f32 == 2) k_gemm_x<kOpF32K, kOpF32K, 3><<<grid, 256, 0, s>>>(x);
      else if (xa == kOpF32K) launch_x_b<kOpF32K>(x, xb, grid, s);
      else if (xb == kOpBfK) k_gemm_x<kOpF32M, kOpBfK><<<grid, 256, 0, s>>>(x);
      else if (xb == kOpBfM) k_gemm_x<kOpF32M, kOpBfM><<<grid, 256, 0, s>>>(x);
      else k_gemm_x<kOpF32M, kOpF32K><<<grid, 256, 0, s>>>(x);
      if (x.ksplit > 1) k_splitk_reduce<<<dim3(grid1(x.M * x.N), batch), 256, 0, s>>>(x);
      return hipGetLastError();
    }
  }
  // the 64 x 64 kernels address each batch entry with 32-bit element offsets
  {
    const int64_t lim = int64_t{1} << 31;
    auto ab = [](int64_t v) { return v < 0 ? -v : v; };
    const int64_t sa = dim_reach(g.am, g.M + BM) + dim_reach(g.ak, g.K + BK16);
    const int64_t ssym = g.a_sym ? ab((g.K + FK) * g.am.stride) + ab((g.M + BM) * g.ak.stride) : 0;
    const int64_t sb = dim_reach(g.bn, g.N + BN) + dim_reach(g.bk, g.K + BK16);
    if (sa >= lim || ssym >= lim || sb >= lim) return hipErrorInvalidValue;
  }
  // bf16 x bf16 on bf16 matrix cores when every segmented dimension keeps a
  // 32-wide k tile inside one segment
  auto seg_ok = [](const GemmDim& d) { return d.len == INT64_MAX || d.len % BK16 == 0; };
  const bool bf = g.a_dtype == kBF16 && g.b_dtype == kBF16 && seg_ok(g.ak) && seg_ok(g.bk) && seg_ok(g.am) &&
                  seg_ok(g.bn) && !g.a_sym && !g.c_lower;
  const int kt = bf ? BK16 : FK;
  if (!bf && !g.a_sym && g.c_m == 1 && g.c_n != 1 && !g.col_scale) {
    // column-major C as the row-major C^T = B^T A^T: stores and the C read run along rows
    std::swap(g.M, g.N); std::swap(g.A, g.B); std::swap(g.a_dtype, g.b_dtype);
    std::swap(g.am, g.bn); std::swap(g.ak, g.bk); std::swap(g.a_batch, g.b_batch);
    std::swap(g.a_ptrs, g.b_ptrs); std::swap(g.c_m, g.c_n);
    g.c_lower = -g.c_lower;
  }
  g.kchunk = (g.K + g.ksplit - 1) / g.ksplit;
  g.kchunk = (g.kchunk + kt - 1) / kt * kt;            // chunks start on tile edges
  dim3 grid((g.M + BM - 1) / BM, (g.N + BN - 1) / BN, batch * g.ksplit);
  const char* name = scope ? scope : "gemm";
  ProfScope ps(name, s);
  account(name);
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
  // at most 128 workgroups per tensor, each thread looping over its share:
  // few atomic additions per output (they serialize on one address)
  dim3 grid(grid1(n, 128), ntensors);
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

hipError_t launch_to_bf16_many(const float* const* ins_dev, int64_t ld_in, uint16_t* const* outs_dev, int64_t rows,
                               int64_t cols, int n, hipStream_t s) {
  if (n <= 0 || rows * cols <= 0) return hipSuccess;
  k_to_bf16_many<<<dim3(grid1(rows * cols), n), 256, 0, s>>>(ins_dev, ld_in, outs_dev, rows, cols);
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

// inv[i] = 1 / lam[i] when lam[i] > rel * max_j lam[j], else 0 (one workgroup).
__global__ __launch_bounds__(256) void k_pinv_scale(const double* lam, int64_t n, double rel, float* inv) {
  __shared__ double red[256];
  double m = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) m = fmax(m, lam[i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  const double thr = rel * red[0];
  for (int64_t i = threadIdx.x; i < n; i += 256) inv[i] = lam[i] > thr ? static_cast<float>(1.0 / lam[i]) : 0.f;
}

// M[j][j] = max_{i < n} M[i][i] for n <= j < np (M: np x np, row stride np,
// zero outside the leading n x n block): the padding becomes a block of
// eigenvalues at the top of the spectrum, away from the leading block's.
__global__ __launch_bounds__(256) void k_pad_diag(float* M, int64_t n, int64_t np) {
  __shared__ float red[256];
  float m = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 256) m = fmaxf(m, M[i * np + i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  for (int64_t j = n + threadIdx.x; j < np; j += 256) M[j * np + j] = red[0];
}

hipError_t launch_pad_diag(float* M, int64_t n, int64_t np, hipStream_t s) {
  if (np <= n) return hipSuccess;
  k_pad_diag<<<1, 256, 0, s>>>(M, n, np);
  return hipGetLastError();
}

hipError_t launch_pinv_scale(const double* lam, int64_t n, double rel, float* inv, hipStream_t s) {
  k_pinv_scale<<<1, 256, 0, s>>>(lam, n, rel, inv);
  return hipGetLastError();
}

hipError_t launch_sum_batch(const float* in, int64_t count, int n, float* out, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  k_sum_batch<<<grid1(count), 256, 0, s>>>(in, count, n, out);
  return hipGetLastError();
}

hipError_t launch_sum_diag_blocks(const float* C, int64_t H, int64_t D, float* GD, int batch,
                                  hipStream_t s) {
  k_sum_diag_blocks<<<dim3(grid1(D * D), batch), 256, 0, s>>>(C, H, D, GD);
  return hipGetLastError();
}

}  // namespace jolt
