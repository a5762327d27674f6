// Leading eigenpairs of a batch of symmetric n x n matrices (the token Gram)
// by two-stage tridiagonal reduction:
//
//  1. dense -> band (half-bandwidth 32): per 32-column panel, a Householder
//     QR of the panel below the band (the LDS / TSQR panel kernels) and the
//     two-sided update A22 <- H^T A22 H as matrix-core products,
//     H = I - V T V^T:  X = A22 V T,  W = X - V (T^T V^T X) / 2,
//     A22 <- A22 - V W^T - W V^T;
//  2. band -> tridiagonal by bulge chasing: sweep j annihilates column j
//     below the subdiagonal with a reflector of length <= 32 and chases the
//     bulge it creates down the band one 32-row block per step; sweeps are
//     pipelined (sweep j step s runs at tick S j + s, one wave per sweep in
//     flight; S >= 4 keeps the rows of concurrent steps, and of each step and
//     the next step's prefetch, disjoint);
//  3. the top R eigenvalues of the tridiagonal by bisection on Sturm counts
//     and their eigenvectors by inverse iteration on T - lambda I = L D L^T,
//     both in fp64;
//  4. back-transformation: the chase reflectors in reverse order, grouped
//     into blocks of 32 sweeps at one step (compact WY, matrix cores) applied
//     in a wavefront of launches, then the panel reflectors as matrix-core
//     products.
//
// The factors the codec needs are the leading eigenvectors of the Gram
// (JoLT abstract: Tucker factors from the leading singular vectors of the
// mode unfoldings); every Householder step is the textbook one (beta =
// -sign(alpha) ||x||, tau = (beta - alpha) / beta).
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"
#include "qr_reg.hpp"

#include <cfloat>
#include <vector>

namespace jolt {
namespace {

constexpr int SBW = 32;           // half-bandwidth after stage 1 (= panel width)
constexpr int BWS = 2 * SBW;      // band storage width: the bulge stays within 2b - 1
constexpr int RFS = SBW + 1;      // stored floats per chase reflector: v[0..31], tau

__host__ __device__ inline int64_t sweep_steps(int64_t n, int64_t j) {
  return (n - 1 - j < 2) ? 0 : (n - 3 - j) / SBW + 1;
}
__host__ __device__ inline int64_t floor_sum(int64_t M) {       // sum_{m=0}^{M} floor(m / SBW)
  if (M < 0) return 0;
  const int64_t q = M / SBW, r = M % SBW;
  return SBW * q * (q - 1) / 2 + q * (r + 1);
}
// index of the first reflector of sweep j (sweeps in order, steps in order)
__host__ __device__ inline int64_t sweep_offset(int64_t n, int64_t j) {
  if (j > n - 2) j = n - 2;
  if (j <= 0) return 0;
  return j + floor_sum(n - 3) - floor_sum(n - 3 - j);
}

// Band storage: Bw[i * BWS + k] = A[i][i - k], 0 <= k < BWS.
__global__ __launch_bounds__(256) void k_band_init(const float* A, int64_t n, float* Bw) {
  const int64_t z = blockIdx.y;
  const float* a = A + z * n * n;
  float* b = Bw + z * n * BWS;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < n * BWS; idx += 256ll * gridDim.x) {
    const int64_t i = idx / BWS, k = idx % BWS;
    b[idx] = (k <= SBW && i - k >= 0) ? a[(i - k) * n + i] : 0.f;   // column-major (row i, column i - k)
  }
}

// n <= 32768, so every band offset fits in 32 bits
__device__ __forceinline__ int bidx(int r, int c) { return r * BWS + (r - c); }

// Stage 2: one workgroup of NW waves per matrix; sweep j runs on wave j % NW.
// Every block of a step moves between the band and registers along its rows
// (row r of the band holds A[r][r - k], k = 0..63, contiguous), so each
// access of a wave covers two 128-byte row segments; a wave's private LDS
// tiles provide the transposed views the step needs.  Per wave:
//  * the below block of step s is kept in LDS: it is the left block of step
//    s + 1 of the same sweep, which writes it back to the band (the last step
//    of a sweep writes it itself);
//  * the diagonal block, the below block and (step 0) the column being
//    annihilated of the wave's next step are loaded one tick ahead, into
//    registers.
// With S >= 4 ticks between consecutive sweeps every value a prefetch reads
// was written at least two ticks earlier, and no concurrent step touches it.
// The band is addressed through a buffer resource of the matrix's n rows:
// rows past the last read as zero and writes to them are dropped, which
// covers the ragged last block of every sweep without per-row masks.
constexpr int TLD = SBW + 1;      // LDS tile row stride (conflict-free transposes)
constexpr uint32_t kOut = 0x80000000u;   // a byte offset past any band (n <= 32768)
struct ChaseLds {
  float tile[2][SBW * TLD];       // ping-pong: carried left block / staged below block
  float x[SBW];                   // the column annihilated by the next step
};
constexpr int kChaseLdsClaim = 160 * 1024 - 1024;   // a CU's LDS less the static part
struct ChaseStep {
  int j, s, r0, L, r1, hi;
  bool last;
  int64_t ref0;                   // index of the sweep's first reflector
};
// sweeps of one wave: j = wave, wave + nw, ...; sweep j runs its steps at
// ticks S j .. S j + steps(j) - 1 (S nw >= steps(0), so they never overlap)
struct ChaseClock {
  int j, start, K;
  int64_t ref0;
  __device__ void init(int wave, int S, int n) {
    j = wave; start = S * j; K = static_cast<int>(sweep_steps(n, j)); ref0 = sweep_offset(n, j);
  }
  // the step at tick t (ticks visited in increasing order)
  __device__ bool at(int t, int nw, int S, int n, ChaseStep& g) {
    if (t - start >= K && K > 0) {
      j += nw; start = S * j; K = static_cast<int>(sweep_steps(n, j)); ref0 = sweep_offset(n, j);
    }
    const int s = t - start;
    if (s < 0 || s >= K) return false;
    g.j = j; g.s = s; g.last = (s == K - 1); g.ref0 = ref0;
    g.r0 = j + 1 + s * SBW;
    g.L = min(n - g.r0, SBW);
    g.r1 = g.r0 + g.L;
    g.hi = min(g.r1 + SBW, n);
    return true;
  }
};
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), 0, 0);
}

// row of register ii in a 32x32 fp32 matrix-core accumulator, less 4 (lane / 32)
__device__ __forceinline__ constexpr int rofs(int ii) { return (ii >> 2) * 8 + (ii & 3); }
// the sum of p over each half (32 lanes) of the wave, in every lane of the half:
// a butterfly within rows of 16 (DPP: lane xor 1, xor 2, rotate by 4 and 8)
// and a swap of odd and even rows (v_permlane16_swap).  The association of
// the additions depends on the lane, so callers take one lane's value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum32(float p) {
  p += dpp_f<0xB1>(p);            // quad_perm [1, 0, 3, 2]
  p += dpp_f<0x4E>(p);            // quad_perm [2, 3, 0, 1]
  p += dpp_f<0x124>(p);           // row_ror 4
  p += dpp_f<0x128>(p);           // row_ror 8
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);     // even row's sum + odd row's
}
// sum of a[i] b[i], i < 16, as four interleaved chains (short dependency chain)
template <typename A, typename B>
__device__ __forceinline__ float dot16(const A& a, const B& b) {
  float s0 = a[0] * b[0], s1 = a[1] * b[1], s2 = a[2] * b[2], s3 = a[3] * b[3];
#pragma unroll
  for (int i = 4; i < 16; i += 4) {
    s0 = fmaf(a[i], b[i], s0);
    s1 = fmaf(a[i + 1], b[i + 1], s1);
    s2 = fmaf(a[i + 2], b[i + 2], s2);
    s3 = fmaf(a[i + 3], b[i + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_chase(float* Bw_g, int n, float* Rf_g, int64_t rf_stride, int S,
                                                   int* status, int spin_limit) {
  extern __shared__ float chase_lds_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31, h4 = 4 * h;
  ChaseLds& sm = reinterpret_cast<ChaseLds*>(chase_lds_raw)[wave];
  float* Bw = Bw_g + static_cast<int64_t>(blockIdx.x) * n * BWS;
  const __amdgpu_buffer_rsrc_t band = __builtin_amdgcn_make_buffer_rsrc(Bw, 0, n * BWS * 4, 0x00020000);
  float* Rf = Rf_g + blockIdx.x * rf_stride;
  const int last = n - 3;
  const int ticks = last >= 0 ? S * last + static_cast<int>(sweep_steps(n, last)) : 0;
  // Lane (h, l32) holds column l32 of a 32 x 32 block at rows h4 + rofs(ii),
  // ii < 16: the accumulator layout of the fp32 matrix cores, so the block
  // updates (rank one or two) are single 32x32x2 products.  Byte offsets of
  // this lane's element in row h4 of a block; row r adds 65 floats.
  constexpr uint32_t RS = 4 * (BWS + 1);
  f32x16 pd;                        // the diagonal block of the next step (used in place)
  float pb[16], px = 0.f;           // next step: below block rows, the column it annihilates
  auto prefetch = [&](const ChaseStep& q) {
    const uint32_t od = 4u * static_cast<uint32_t>(q.r0 * BWS + h4 * (BWS + 1) - l32);  // (r0 + a, r0 + l32)
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) pd[ii] = bload(band, od + rofs(ii) * RS);
    if (q.r1 < q.hi) {
      const uint32_t ob = 4u * static_cast<uint32_t>(q.r1 * BWS + h4 * (BWS + 1) + q.L - l32);  // (r1 + a, r0 + l32)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) pb[ii] = bload(band, ob + rofs(ii) * RS);
    } else {
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) pb[ii] = 0.f;
    }
    if (q.s == 0) px = bload(band, 4u * static_cast<uint32_t>(q.r0 * BWS + 1 + l32 * (BWS + 1)));  // (r0 + l32, j)
  };
  // Progress ring instead of a workgroup barrier per tick: the band values a
  // prefetch at tick t reads were last written by the previous sweep (the
  // previous wave, one tick behind at most) at tick t - 1 or earlier, and
  // older sweeps only earlier still; so wave w publishes each finished tick
  // (after its stores) and waits, before prefetching at tick t, for its
  // predecessor to have finished tick t - 1.  Waits point to strictly
  // earlier ticks of other waves, so they always end; the spin is bounded
  // all the same (spin_limit polls): a wait that gives up sets bit 0 of
  // *status (a vector atomic, read back by the host) and the wave carries
  // on, so the kernel still ends and the caller sees the failure.
  __shared__ int tick_done[NW];
  if ((threadIdx.x & 63) == 0) tick_done[wave] = -1;
  __syncthreads();
  const int pred = (wave + NW - 1) % NW;
  auto wait_pred = [&](int t_need) {
    for (int spin = 0;; ++spin) {
      if (__hip_atomic_load(&tick_done[pred], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= t_need) break;
      if (spin >= spin_limit) {
        if (lane == 0) __hip_atomic_fetch_or(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };
  // row a = h4 + rofs(ii) of a block against this lane's column l32: a <= l32, a >= l32
  uint32_t m_le[16], m_ge[16];
#pragma unroll
  for (int ii = 0; ii < 16; ++ii) {
    m_le[ii] = h4 + rofs(ii) <= l32 ? ~0u : 0u;
    m_ge[ii] = h4 + rofs(ii) >= l32 ? ~0u : 0u;
    // opaque to the optimizer: kept as vector registers and combined with
    // v_bfi, rather than turned back into per-row lane masks in scalar registers
    asm volatile("" : "+v"(m_le[ii]), "+v"(m_ge[ii]));
  }
  ChaseClock ck, ckn;
  ck.init(wave, S, n);
  ckn.init(wave, S, n);
  {
    ChaseStep g0;
    if (ckn.at(0, NW, S, n, g0)) prefetch(g0);
  }
  int cur = 0;                      // tile holding the carried left block
  for (int t = 0; t < ticks; ++t) {
    ChaseStep g, gn;
    const bool act = ck.at(t, NW, S, n, g);
    const bool actn = ckn.at(t + 1, NW, S, n, gn);
    float* Lt = sm.tile[cur];
    float* Ft = sm.tile[cur ^ 1];
    if (act) {
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) Ft[(h4 + rofs(ii)) * TLD + l32] = pb[ii];   // below block, row-major
      if (g.s == 0 && lane < SBW) sm.x[lane] = px;
    }
    // the next step's loads are issued once this step has used the diagonal
    // block (pd), just before the block below; the step's values and the
    // wait that orders them are as before
    float tau = 0.f, vo = 0.f;
    float vh[16];
    if (act) {
      const int L = g.L, r0 = g.r0;
      wave_lds_sync();
      // reflector (I - tau v v^T) x = beta e_1 from x = sm.x (zero past L)
      float xh[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x4 = *reinterpret_cast<const float4*>(&sm.x[8 * q4 + h4]);   // rows h4 + rofs(4 q4 ..)
        xh[4 * q4] = x4.x; xh[4 * q4 + 1] = x4.y; xh[4 * q4 + 2] = x4.z; xh[4 * q4 + 3] = x4.w;
      }
      const float xo = sm.x[l32];
      const float alpha = sm.x[0];
      const float x0 = xh[0];
      xh[0] = h ? x0 : 0.f;                        // row 0 (alpha) is not in sigma
      float sig = dot16(xh, xh);
      xh[0] = x0;
      sig = half_sum(sig);
      float beta = alpha, scale = 0.f;
      if (sig > 0.f) {
        // hardware square root and reciprocals (about 1 ulp): the reflector
        // needs no correctly rounded quotient, and the chain is the step's
        // critical path
        const float nrm = __builtin_amdgcn_sqrtf(fmaf(alpha, alpha, sig));
        beta = alpha >= 0.f ? -nrm : nrm;
        tau = (beta - alpha) * __builtin_amdgcn_rcpf(beta);
        scale = __builtin_amdgcn_rcpf(alpha - beta);
      }
      // the same value in every lane: made wave-uniform, so the branches on it are scalar
      tau = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tau)));
      // v_i, i = h4 + rofs(ii)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) vh[ii] = xh[ii] * scale;
      if (h == 0) vh[0] = 1.f;
      vo = (l32 == 0) ? 1.f : xo * scale;          // v_{l32}
      const int64_t ridx = g.ref0 + g.s;
      if (lane < SBW) Rf[ridx * RFS + lane] = vo;
      if (lane == 0) Rf[ridx * RFS + SBW] = tau;
      // left block (rows r0.., columns r0-32 .. r0-1) from the left; written back
      if (g.s == 0) {
        if (h == 0) bstore(band, 4u * static_cast<uint32_t>(r0 * BWS + 1 + l32 * (BWS + 1)),
                           l32 == 0 ? beta : 0.f);
      } else {
        f32x16 li;
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) li[ii] = Lt[(h4 + rofs(ii)) * TLD + l32];
        const float y = half_sum(dot16(vh, li));
        // L - tau v y^T: A = [v 0], B = [-tau y^T; 0].  Column 0 (lane l32 = 0)
        // is the annihilated column, zeroed in the tile by the previous step,
        // so it stays exactly zero; its top entry becomes beta.
        li = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 0.f : vo, h ? 0.f : -tau * y, li, 0, 0, 0);
        if (lane == 0) li[0] = beta;
        const uint32_t ol = 4u * static_cast<uint32_t>(r0 * BWS + h4 * (BWS + 1) + SBW - l32);
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) bstore(band, ol + rofs(ii) * RS, li[ii]);
      }
      if (tau != 0.f) {
        // diagonal block: pd holds column l32 of its lower triangle (rows
        // a >= l32; the rest of the column is other band data).  Row l32 of
        // the block is D[l32][c] = the tile's (l32, c) for c <= l32 (written by
        // lane c) and D[c][l32] = pd for c > l32: selected bitwise with the
        // lane's row masks.
        float* Ds = Lt;
        wave_lds_sync();
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) Ds[(h4 + rofs(ii)) * TLD + l32] = pd[ii];
        wave_lds_sync();
        float drow[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          const uint32_t tv = __float_as_uint(Ds[l32 * TLD + h4 + rofs(ii)]);
          drow[ii] = __uint_as_float((m_le[ii] & tv) | (~m_le[ii] & __float_as_uint(pd[ii])));
        }
        const float wo = half_sum(dot16(drow, vh));     // w = D v (lane: row l32)
        // gamma = v^T w over the 32 rows, one value for the whole wave
        const float gam = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sum32(vo * wo))));
        // D <- H D H = D - tau (v w^T + w v^T) + tau^2 (v^T w) v v^T  (lane: column l32)
        // as one rank-two product: A = [v w], B = [(tau^2 gam v - tau w)^T; -tau v^T]
        const f32x16 dm = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? wo : vo, h ? -tau * vo : tau * tau * gam * vo - tau * wo,
                                                               pd, 0, 0, 0);
        // lower triangle only: the other rows go to an offset past the band (dropped)
        const uint32_t od = 4u * static_cast<uint32_t>(r0 * BWS + h4 * (BWS + 1) - l32);
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          const uint32_t base = ii < 8 ? od : od + 16 * RS;
          bstore(band, ((m_ge[ii] & base) | (~m_ge[ii] & kOut)) + (rofs(ii) - (ii < 8 ? 0 : 16)) * RS, dm[ii]);
        }
      }
    }
    if (actn) {
      if (t > 0) wait_pred(t - 1);
      prefetch(gn);
    }
    if (act) {
      if (g.r1 < g.hi) {
        // below block (rows r1 .., columns r0 .. r1-1) from the right (lane: row l32)
        f32x16 bi;                                 // the block's transpose: lane = its row l32
        wave_lds_sync();
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) bi[ii] = Ft[l32 * TLD + h4 + rofs(ii)];
        if (tau != 0.f) {
          const float zr = half_sum(dot16(bi, vh));
          // B^T - tau v z^T: A = [v 0], B = [-tau z^T; 0]
          bi = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 0.f : vo, h ? 0.f : -tau * zr, bi, 0, 0, 0);
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) Ft[l32 * TLD + h4 + rofs(ii)] = bi[ii];
        }
        if (h == 0) {
          sm.x[l32] = bi[0];                       // the next step's column (zero past hi)
          // which that step annihilates: zero in the carried tile (its left block)
          if (!g.last) Ft[l32 * TLD] = 0.f;
        }
        if (g.last) {
          wave_lds_sync();
          const uint32_t ob = 4u * static_cast<uint32_t>(g.r1 * BWS + h4 * (BWS + 1) + SBW - l32);
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) bstore(band, ob + rofs(ii) * RS, Ft[(h4 + rofs(ii)) * TLD + l32]);
        }
      }
      cur ^= 1;
    }
    // this tick's band stores complete, then published
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_store(&tick_done[wave], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// d[i] = T[i][i], e[i] = T[i+1][i] (fp64), from the band after the chase.
__global__ __launch_bounds__(256) void k_tri_out(const float* Bw, int64_t n, double* d, double* e) {
  const int64_t z = blockIdx.y;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    d[z * n + i] = Bw[z * n * BWS + i * BWS];
    e[z * n + i] = (i + 1 < n) ? Bw[z * n * BWS + (i + 1) * BWS + 1] : 0.0;
  }
}

// Number of eigenvalues of the tridiagonal (d, e2 = e^2) below x (Sturm
// count): by Sylvester's law of inertia, the negative pivots q_i = (d_i - x)
// - e2_{i-1} / q_{i-1} of L D L^T = T - x I, a vanishing pivot counted as
// negative.  The pivots are ratios of the leading principal minors, q_i =
// P_i / P_{i-1} with P_i = (d_i - x) P_{i-1} - e2_{i-1} P_{i-2} (P_{-1} = 1),
// so q_i < 0 exactly where the signs of P_i and P_{i-1} differ; the minors
// leave no division on the dependency chain, one fused multiply-add per row
// (the e2 P_{i-2} term is formed a row earlier).  d, e2 and x come scaled by
// powers of two so that |d_i - x| < 2 and e2_i < 4: |P| grows at most 6x a
// row, and every 8 rows both minors are rescaled by a power of two (exact).
// Each minor takes -pv times its predecessor, pv = max(2^-900, pivmin / 2^ex)
// (the pivot floor of the unscaled count, far below any pivot that matters
// unless the whole matrix is at the fp64 floor): a vanishing pivot becomes a
// tiny negative one, and a zero does not propagate where e2 vanishes.
__device__ __forceinline__ int sturm_count_minors(const double* d, const double* e2, int64_t n, double x,
                                                  double kPv) {
  double pm2 = 1.0;
  double pm1 = __builtin_fma(-kPv, 1.0, d[0] - x);
  bool neg = pm1 < 0.0;
  int cnt = neg;
  auto row = [&](int64_t i) {
    const double t = e2[i - 1] * pm2;
    double p = __builtin_fma(d[i] - x, pm1, -t);
    p = __builtin_fma(-kPv, pm1, p);
    const bool ng = p < 0.0;
    cnt += ng != neg;
    neg = ng;
    pm2 = pm1;
    pm1 = p;
  };
  int64_t i = 1;
  for (; i + 8 <= n; i += 8) {                      // whole blocks of 8 rows, then a rescale
#pragma unroll
    for (int u = 0; u < 8; ++u) row(i + u);
    const int ex = max(__builtin_amdgcn_frexp_exp(pm1), __builtin_amdgcn_frexp_exp(pm2));
    pm1 = __builtin_amdgcn_ldexp(pm1, -ex);
    pm2 = __builtin_amdgcn_ldexp(pm2, -ex);
  }
  for (; i < n; ++i) row(i);                        // at most 7 rows: no rescale needed
  return cnt;
}

// Top R eigenvalues, descending: lam[q] is the (n-1-q)-th smallest, by
// bisection to fp64 resolution inside the Gershgorin interval.
constexpr int BSL = 4;           // threads per eigenvalue (a power of two <= 64)
__global__ __launch_bounds__(256) void k_bisect(const double* d_g, const double* e_g, int64_t n, int R,
                                               double* lam) {
  extern __shared__ double sh[];
  double* d = sh;
  double* e2 = sh + n;
  __shared__ double gl_s, gu_s, piv_s, tol_s;
  __shared__ int ex_s;
  __shared__ int grid_cnt[256];
  const int64_t z = blockIdx.y;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    d[i] = d_g[z * n + i];
    const double ei = (i + 1 < n) ? e_g[z * n + i] : 0.0;
    e2[i] = ei * ei;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double gl = INFINITY, gu = -INFINITY, emax = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      const double el = i > 0 ? fabs(e_g[z * n + i - 1]) : 0.0;
      const double er = i + 1 < n ? fabs(e_g[z * n + i]) : 0.0;
      gl = fmin(gl, d[i] - el - er);
      gu = fmax(gu, d[i] + el + er);
      emax = fmax(emax, e2[i]);
    }
    const double span = fmax(fabs(gl), fabs(gu));
    gl_s = gl - 2.0 * DBL_EPSILON * span - DBL_MIN;
    gu_s = gu + 2.0 * DBL_EPSILON * span + DBL_MIN;
    piv_s = DBL_MIN * fmax(1.0, emax);
    // brackets narrower than 1e-12 of the spectrum's span are not refined
    // further: the tridiagonal itself carries fp32 rounding (~1e-7 of its
    // norm), and the eigenvalues feed the allocation's energies and the
    // inverse-iteration shifts, neither of which sees a difference that small
    tol_s = 1e-12 * (gu - gl);
    // the counts run on T / 2^ex with 2^ex >= max |x| over the interval
    // (powers of two: the scaled values and every x are exact)
    ex_s = __builtin_amdgcn_frexp_exp(fmax(fabs(gl_s), fabs(gu_s)));
  }
  __syncthreads();
  const int ex = ex_s;
  const double pv = fmax(0x1p-900, __builtin_amdgcn_ldexp(piv_s, -ex));
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    d[i] = __builtin_amdgcn_ldexp(d[i], -ex);
    e2[i] = __builtin_amdgcn_ldexp(e2[i], -2 * ex);
  }
  __syncthreads();
  // a shared first pass: counts at 256 interior points x_i = gl + (gu - gl) (i + 1) / 257
  // of the whole interval, one per thread, from which every eigenvalue takes
  // its starting bracket (one count per thread, as a multisection step, but a
  // 257-way split)
  const double g0 = gl_s, gw = gu_s - gl_s;
  grid_cnt[threadIdx.x] =
      sturm_count_minors(d, e2, n, __builtin_amdgcn_ldexp(g0 + gw * (threadIdx.x + 1) * (1.0 / 257.0), -ex), pv);
  __syncthreads();
  // BSL threads per eigenvalue (multisection): each evaluates one of BSL
  // interior points of the bracket, which then shrinks to 1 / (BSL + 1)
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int q = gid / BSL, sub = gid % BSL;
  if (q >= R) return;                             // whole groups leave together
  const int64_t k = n - 1 - q;                    // wanted: the k-th smallest (0-based)
  // the first grid point whose count exceeds k (256 if none); counts rise with x
  int f = 0;
  for (int span = 256; span > 0; span >>= 1)
    if (f + span <= 256 && grid_cnt[f + span - 1] <= k) f += span;
  double lo = f > 0 ? g0 + gw * f * (1.0 / 257.0) : gl_s;            // x_{f-1}
  double hi = f < 256 ? g0 + gw * (f + 1) * (1.0 / 257.0) : gu_s;     // x_f
  for (int it = 0; it < 100; ++it) {
    if (hi - lo <= fmax(2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)), tol_s) + piv_s) break;
    const double w = hi - lo;
    const double x = lo + w * (sub + 1) * (1.0 / (BSL + 1));
    const int cnt = sturm_count_minors(d, e2, n, __builtin_amdgcn_ldexp(x, -ex), pv);
    double nlo = lo, nhi = hi;
    bool found = false;
#pragma unroll
    for (int t = 0; t < BSL; ++t) {
      const int ct = __shfl(cnt, (threadIdx.x & 63 & ~(BSL - 1)) + t);
      const double xt = lo + w * (t + 1) * (1.0 / (BSL + 1));
      if (!found) {
        if (ct > k) { nhi = xt; found = true; }
        else nlo = xt;
      }
    }
    if (!(nlo > lo || nhi < hi)) break;           // no progress at fp64 resolution
    lo = nlo;
    hi = nhi;
  }
  if (sub == 0) lam[z * R + q] = 0.5 * (lo + hi);
}

// Eigenvector of eigenvalue lam[q] by inverse iteration (two solves with
// T - lam I = L D L^T from a fixed pseudo-random start; the factorization
// and the first forward substitution share one pass), normalized, fp32
// out as column q of Z (column-major, ld n).  With lam within a few ulps of
// ||T|| of the eigenvalue, each solve shrinks the other eigenvectors'
// components relative to this one's by about eps ||T|| / gap (under 1e-7 for
// the gaps these spectra have): two solves reach fp64 level from a random
// start, past what the fp32 output keeps.  The factorization keeps the
// reciprocal pivots, so each solve is multiply-only; intermediate vectors
// are rescaled on the fly.  Scratch rp / y: [i][q] interleaved (coalesced
// across q).
constexpr int IVW = 64;          // threads (eigenvectors) per inverse-iteration workgroup
constexpr int IVC = 16;          // solve steps per register chunk (n is a multiple of 32)
__device__ __forceinline__ double invit_start(int q, int64_t i) {   // uniform in [0.5, 1.5)
  const uint64_t hsh = mix64(0x9E3779B97F4A7C15ull * static_cast<uint64_t>(q + 1) + static_cast<uint64_t>(i));
  return 0.5 + static_cast<double>(hsh >> 11) * 0x1p-53;
}
// One thread per eigenvector: the solves run over [i][q] scratch (coalesced
// over the eigenvectors) in chunks of IVC steps whose loads are issued
// together; the normalized vector is written by k_invit_out.
__global__ __launch_bounds__(IVW) void k_invit(const double* d_g, const double* e_g, int64_t n, int R,
                                              const double* lam, double* rp_g, double* y_g, double* nrm_g) {
  const int64_t z = blockIdx.y;
  const double* d = d_g + z * n;
  const double* e = e_g + z * n;
  double tn = 0.0;                                  // infinity norm of T
  for (int64_t i = threadIdx.x; i < n; i += IVW)
    tn = fmax(tn, fabs(d[i]) + fabs(e[i]) + (i ? fabs(e[i - 1]) : 0.0));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tn = fmax(tn, __shfl_xor(tn, o));
  const int q = blockIdx.x * IVW + threadIdx.x;
  if (q >= R) return;
  double* rp = rp_g + z * n * R;
  double* y = y_g + z * n * R;
  const double lm = lam[z * R + q];
  const double tiny = fmax(tn, DBL_MIN) * DBL_EPSILON;
  // L D L^T of T - lam I: pivots p_i = (d_i - lam) - e_{i-1}^2 / p_{i-1},
  // kept as 1 / p_i, in the same pass as the first forward solve L u = y0
  // (l_i = e_{i-1} / p_{i-1}: it needs only the previous pivot)
  {
    double r = 0.0, u = 0.0;
    for (int64_t i0 = 0; i0 < n; i0 += IVC) {
      double rr[IVC], yy[IVC];
#pragma unroll
      for (int c = 0; c < IVC; ++c) {
        const int64_t i = i0 + c;
        u = invit_start(q, i) - (i ? e[i - 1] * r * u : 0.0);
        yy[c] = u;
        double p = (d[i] - lm) - (i ? e[i - 1] * e[i - 1] * r : 0.0);
        if (fabs(p) < tiny) p = tiny;
        r = __builtin_amdgcn_rcp(p);                 // 1 / p: reciprocal + one Newton step (~2e-15)
        r = __builtin_fma(__builtin_fma(-p, r, 1.0), r, r);
        rr[c] = r;
      }
#pragma unroll
      for (int c = 0; c < IVC; ++c) {
        rp[(i0 + c) * R + q] = rr[c];
        y[(i0 + c) * R + q] = yy[c];
      }
    }
  }
  double sc = 1.0, s2 = 0.0;
  for (int it = 0; it < 2; ++it) {
    if (it > 0) {
      // forward: L u = sc * y   (L unit lower, l_i = e_{i-1} / p_{i-1})
      double u = 0.0, rprev = 0.0;
      for (int64_t i0 = 0; i0 < n; i0 += IVC) {
        double yy[IVC], rr[IVC];
#pragma unroll
        for (int c = 0; c < IVC; ++c) {
          const int64_t i = i0 + c;
          yy[c] = y[i * R + q];
          rr[c] = rp[i * R + q];
        }
#pragma unroll
        for (int c = 0; c < IVC; ++c) {
          const int64_t i = i0 + c;
          u = yy[c] * sc - (i ? e[i - 1] * rprev * u : 0.0);
          yy[c] = u;
          rprev = rr[c];
        }
#pragma unroll
        for (int c = 0; c < IVC; ++c) y[(i0 + c) * R + q] = yy[c];
      }
    }
    // D L^T x = u:  x_i = (u_i - e_i x_{i+1}) / p_i; the last pass also sums x^2
    double xs = 0.0, mx = 0.0;
    s2 = 0.0;
    for (int64_t i0 = n - IVC; i0 >= 0; i0 -= IVC) {
      double yy[IVC], rr[IVC];
#pragma unroll
      for (int c = 0; c < IVC; ++c) {
        yy[c] = y[(i0 + c) * R + q];
        rr[c] = rp[(i0 + c) * R + q];
      }
#pragma unroll
      for (int c = IVC - 1; c >= 0; --c) {
        const int64_t i = i0 + c;
        xs = (yy[c] - (i + 1 < n ? e[i] * xs : 0.0)) * rr[c];
        yy[c] = xs;
        mx = fmax(mx, fabs(xs));
        s2 = fma(xs, xs, s2);
      }
#pragma unroll
      for (int c = 0; c < IVC; ++c) y[(i0 + c) * R + q] = yy[c];
    }
    sc = mx > 0.0 ? 1.0 / mx : 1.0;
  }
  // the last solve's x, normalized
  nrm_g[z * R + q] = s2 > 0.0 ? 1.0 / sqrt(s2) : 0.0;
}

// Z[:, q] = y[:, q] * nrm[q] as fp32, through a 32 x 32 LDS transpose ([i][q]
// scratch to column-major Z).
// With lam_scale, column q is also multiplied by 1 / sqrt(lam_scale[q]) where
// that eigenvalue is positive (in fp64, before the rounding to fp32).
__global__ __launch_bounds__(256) void k_invit_out(const double* y_g, const double* nrm_g, int64_t n, int R,
                                                   float* Z, int64_t z_batch, const double* lam_scale) {
  __shared__ float tile[32][33];
  const int64_t z = blockIdx.z;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int q0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const double* y = y_g + z * n * R;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = i0 + ty + 8 * k;
    const int q = q0 + tx;
    double f = 0.0;
    if (q < R) {
      f = nrm_g[z * R + q];
      if (lam_scale && lam_scale[z * R + q] > 0.0) f /= sqrt(lam_scale[z * R + q]);
    }
    tile[ty + 8 * k][tx] = (i < n && q < R) ? static_cast<float>(y[i * R + q] * f) : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = q0 + ty + 8 * k;
    const int64_t i = i0 + tx;
    if (i < n && q < R) Z[z * z_batch + static_cast<int64_t>(q) * n + i] = tile[tx][ty + 8 * k];
  }
}

// Stage 2 back-transformation in blocks.  Block (G, s) gathers the step-s
// reflectors of the 32 sweeps j = 32G .. 32G + 31: reflector i acts on rows
// rb + i .. rb + i + 31 (rb = 32G + 1 + 32s), so the block is I - V T V^T
// with V a 63 x 32 staircase and T the upper-triangular factor of the
// product H_{32G} ... H_{32G+31} (forward accumulation: T[i][i] = tau_i,
// T[0:i, i] = -tau_i T[0:i, 0:i] V[:, 0:i]^T v_i).  Applying the sweeps in
// reverse order equals applying, for the groups in reverse order, their
// blocks in increasing s: a block only overlaps its neighbours in s within
// its group and blocks of adjacent groups, which the wavefront t = 2 g' + s
// (g' = 0 for the last group) orders; blocks of one t touch disjoint rows.
constexpr int CBR = 2 * SBW;      // staircase rows (63) padded to 64

// V T of every block: one wave per (G, s).  S = V^T V on fp32 matrix cores
// (the 64 x 32 staircase), then the recurrence with row `lane` of T in
// registers (lanes 0..31), unrolled so that every S read is independent;
// the block is stored as V T (64 x 32, row-major), which its application
// multiplies by V^T Z (so that T is applied once per block, not once per
// block and column chunk).
__global__ __launch_bounds__(64) void k_cb_tfac(const float* Rf_g, int64_t rf_stride, int n, int K0, float* Tg,
                                                int64_t t_stride) {
  __shared__ float Vs[CBR][SBW + 1];     // staircase V[r][i]
  __shared__ float S[SBW][SBW + 1];      // S[l][i] = v_l^T v_i
  __shared__ float tau[SBW];
  const int lane = threadIdx.x, rl = lane & 31, hf = lane >> 5, blk = blockIdx.x, G = blk / K0, s = blk % K0;
  const int64_t z = blockIdx.y;
  const float* Rf = Rf_g + z * rf_stride;
  const int jg = G * SBW, last = n - 3;
  // every load in flight before the LDS writes; zeros off the staircase
  float rv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = lane + 64 * q, i = idx / SBW, r = idx % SBW, j = jg + i;
    rv[q] = (j <= last && s < sweep_steps(n, j)) ? Rf[(sweep_offset(n, j) + s) * RFS + r] : 0.f;
  }
  float tl = 0.f;
  if (lane < SBW) {
    const int j = jg + lane;
    tl = (j <= last && s < sweep_steps(n, j)) ? Rf[(sweep_offset(n, j) + s) * RFS + SBW] : 0.f;
  }
  for (int idx = lane; idx < CBR * SBW; idx += 64) {
    const int row = idx / SBW, i = idx % SBW;
    if (row < i || row >= i + SBW) Vs[row][i] = 0.f;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = lane + 64 * q, i = idx / SBW, r = idx % SBW;
    Vs[i + r][i] = rv[q];
  }
  if (lane < SBW) tau[lane] = tl;
  __syncthreads();
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < CBR; kk += 2) {
    const int k = kk + hf;
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[k][rl], Vs[k][rl], acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) S[(e >> 2) * 8 + hf * 4 + (e & 3)][rl] = acc[e];
  __syncthreads();
  float tr[SBW];
  if (lane < SBW) {
    // T[lane][i] = -tau_i sum_{lane <= p < i} T[lane][p] S[p][i] (T[lane][p] = 0
    // for p < lane), the sum in four interleaved chains
#pragma unroll
    for (int i = 0; i < SBW; ++i) {
      float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < i; ++p) u[p & 3] = fmaf(tr[p], S[p][i], u[p & 3]);
      const float us = (u[0] + u[1]) + (u[2] + u[3]);
      tr[i] = i < lane ? 0.f : (i == lane ? tau[i] : -tau[i] * us);
    }
  }
  // V T (64 x 32), the product the blocks are applied with: T through LDS
  // (row `lane` from its lane), then two 32 x 32 tiles on fp32 matrix cores
  __syncthreads();                                 // every read of S done
  if (lane < SBW) {
#pragma unroll
    for (int i = 0; i < SBW; ++i) S[lane][i] = tr[i];
  }
  __syncthreads();
  float* VTb = Tg + z * t_stride + static_cast<int64_t>(blk) * CBR * SBW;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16 vt = {};
#pragma unroll
    for (int kk = 0; kk < SBW; kk += 2) {
      const int k = kk + hf;
      vt = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[32 * t + rl][k], S[k][rl], vt, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) VTb[(32 * t + (e >> 2) * 8 + hf * 4 + (e & 3)) * SBW + rl] = vt[e];
  }
}

// Wavefront steps 2u and 2u + 1 in one launch, one workgroup per (group,
// 64 columns of Z): the group's blocks s0 = 2u - 2 g' and s0 + 1 (those that
// exist), applied in that order to the 95 rows they span, kept in LDS.  The
// blocks of group g' - 1 that overlap them have s' <= s0 + 1, so they ran
// in launches u' < u; the row spans of one launch are disjoint.  Per block:
// W = V^T Z_rows (K split over two wave pairs), Z_rows -= (V T) W, on fp32
// matrix cores (32x32x2) from LDS.
constexpr int CBW = CBR + SBW;    // window rows of a block pair (95, padded to 96)
__global__ __launch_bounds__(256) void k_cb_apply(int u, int glo, int nchunk, float* Z, int n, int R,
                                                  int64_t z_batch, const float* Rf_g, int64_t rf_stride,
                                                  const float* Tg, int64_t t_stride, int ng, int K0) {
  __shared__ float Vs[2][CBR][SBW + 1];  // staircases V[r][i] of the two blocks
  __shared__ float VTs[2][CBR][SBW + 1]; // V T of the two blocks
  __shared__ float Zs[CBW][65];          // window rows x 64 columns
  __shared__ float Wp[2][SBW][65];       // W partial sums (two halves of the rows)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, hf = lane >> 5;
  uint32_t bx, by;
  xcd_group_2d(bx, by);                            // the blocks of one matrix on one XCD
  const int bi = static_cast<int>(bx) / nchunk, ch = static_cast<int>(bx) % nchunk;
  const int gp = glo + bi, G = ng - 1 - gp, jg = G * SBW;
  if (gp >= ng) return;
  const int smax = min(K0, static_cast<int>(sweep_steps(n, jg)));
  const int s0 = 2 * u - 2 * gp;
  const bool has0 = s0 >= 0 && s0 < smax, has1 = s0 + 1 >= 0 && s0 + 1 < smax;
  if (!has0 && !has1) return;
  const int rw = jg + 1 + s0 * SBW;                // window row 0 (block s0's first row)
  // rows the applied blocks span: [lo, hi) of the window
  const int lo = has0 ? 0 : SBW;
  const int hi = min(has1 ? CBW - 1 : CBR - 1, n - rw);
  const int c0 = ch * 64, nc = min(64, R - c0);
  const int64_t z = by;
  const float* Rf = Rf_g + z * rf_stride;
  float* Zz = Z + z * z_batch;
  const int last = n - 3;
  // one phase of loads, every load in flight before the first LDS write: the
  // blocks' V T, Z, the staircases V[i + r][i] = v_r of sweep jg + i; zeros
  // off the staircases (disjoint positions)
  float rt[2][8], rz[24], rv[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int sb = s0 + b;
    const bool ok = b == 0 ? has0 : has1;
    const float* tb = Tg + z * t_stride + (static_cast<int64_t>(G) * K0 + (ok ? sb : 0)) * CBR * SBW;
#pragma unroll
    for (int q = 0; q < 8; ++q) rt[b][q] = ok ? tb[tid + 256 * q] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, i = idx / SBW, r = idx % SBW, j = jg + i;
      rv[b][q] = (ok && j <= last && sb < sweep_steps(n, j)) ? Rf[(sweep_offset(n, j) + sb) * RFS + r] : 0.f;
    }
  }
  // the window: thread -> row 32 j + (tid & 31), column 8 q + (tid >> 5)
  // (q < 8, j < 3): 32 consecutive rows of a column per 32 lanes, and the
  // offsets step by constants
  const int zr = tid & 31, zc = tid >> 5;
  const float* zsrc = Zz + static_cast<int64_t>(c0 + zc) * n + rw + zr;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int r = zr + 32 * j;
      rz[3 * q + j] = (r >= lo && r < hi && zc + 8 * q < nc) ? zsrc[static_cast<int64_t>(8 * q) * n + 32 * j] : 0.f;
    }
  for (int idx = tid; idx < 2 * CBR * SBW; idx += 256) {
    const int b = idx / (CBR * SBW), row = (idx / SBW) % CBR, i = idx % SBW;
    if (row < i || row >= i + SBW) Vs[b][row][i] = 0.f;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = tid + 256 * q;
      VTs[b][idx / SBW][idx % SBW] = rt[b][q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      const int i = idx / SBW, r = idx % SBW;
      Vs[b][i + r][i] = rv[b][q];
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 3; ++j) Zs[zr + 32 * j][zc + 8 * q] = rz[3 * q + j];
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b == 0 ? !has0 : !has1) continue;          // uniform over the workgroup
    const int off = b * SBW;                       // the block's rows: window rows off .. off + 63
    // W = V^T Z: wave w -> columns 32 (w & 1) .., rows of V 32 (w >> 1) ..
    {
      const int cb = 32 * (wave & 1), kb = 32 * (wave >> 1);
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < SBW; kk += 2) {
        const int k = kb + kk + hf;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[b][k][rl], Zs[off + k][cb + rl], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) Wp[wave >> 1][(e >> 2) * 8 + hf * 4 + (e & 3)][cb + rl] = acc[e];
    }
    __syncthreads();
    // Z_rows -= (V T) W: wave w -> rows 32 (w >> 1) .., columns 32 (w & 1) ..
    {
      const int rbk = 32 * (wave >> 1), cb = 32 * (wave & 1);
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < SBW; kk += 2) {
        const int k = kk + hf;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(VTs[b][rbk + rl][k], Wp[0][k][cb + rl] + Wp[1][k][cb + rl], acc,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = off + rbk + (e >> 2) * 8 + hf * 4 + (e & 3);
        Zs[r][cb + rl] -= acc[e];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 3; ++j) rz[3 * q + j] = Zs[zr + 32 * j][zc + 8 * q];
  float* zdst = Zz + static_cast<int64_t>(c0 + zc) * n + rw + zr;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int r = zr + 32 * j;
      if (r >= lo && r < hi && zc + 8 * q < nc) zdst[static_cast<int64_t>(8 * q) * n + 32 * j] = rz[3 * q + j];
    }
}

// Panel back-transformation, K consecutive panels per launch: Z rows r_q ..
// <- (I - V_q T_q V_q^T) Z rows r_q .. for q = p_hi, p_hi - 1, .., p_hi - K + 1
// (r_q = 32 (q + 1); panel q's V is m_q x 32, m_q = n - r_q), one workgroup
// per 64 columns of Z and matrix.  Pass 0 accumulates W = V_{p_hi}^T Z over
// 64-row chunks; pass i streams the chunks again, subtracts V_q W2_q (W2 =
// T W) and, from the updated chunk, accumulates the next panel's W: K + 1
// passes over Z for K panels.  fp32 matrix cores; the next chunk is loaded
// into registers during the current one.
__device__ __forceinline__ int64_t panel_voff(int64_t n, int64_t q) {   // panels 0 .. q-1 stacked
  return SBW * (q * n - SBW * q * (q + 1) / 2);
}
__global__ __launch_bounds__(256) void k_apply_wy(float* Z, int64_t n, int64_t z_batch, int R, const float* Vst,
                                                  int64_t v_batch, const float* Tst, int64_t t_batch, int p_hi,
                                                  int K) {
  __shared__ float Vs[2][64][SBW + 1];   // chunk rows of V: [0] the panel applied, [1] the next one
  __shared__ float Zs[64][65];           // Z rows of a chunk x 64 columns
  __shared__ float Wp[2][SBW][65];       // W partial sums (two row halves)
  __shared__ float W2s[SBW][65];         // W2 = T W of the panel applied
  __shared__ float Ts[SBW][SBW + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, hf = lane >> 5;
  uint32_t bx, by;
  xcd_group_2d(bx, by);                            // the column blocks of one matrix on one XCD
  const int64_t z = by;
  const int c0 = static_cast<int>(bx) * 64, nc = min(64, R - c0);
  float* Zz = Z + z * z_batch;
  const int cb = 32 * (wave & 1), kb = 32 * (wave >> 1);
  float rz[16], rv[2][8];
  // chunk loader: Z rows k0 .. k0 + 63 (16 per thread); V rows of panel qa
  // (applied) and qn (next), zero outside a panel's rows (or qa / qn < 0)
  auto load = [&](int64_t k0, int64_t zlo, int qa, int qn) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q, c = idx >> 6, rr = idx & 63;
      const int64_t row = k0 + rr;
      rz[q] = (row >= zlo && row < n && c < nc) ? Zz[static_cast<int64_t>(c0 + c) * n + row] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int pq = b == 0 ? qa : qn;
      const int64_t rq = SBW * (pq + 1), mq = n - rq;
      const float* V = Vst + z * v_batch + (pq >= 0 ? panel_voff(n, pq) : 0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int idx = tid + 256 * q, c = idx >> 6, rr = idx & 63;
        const int64_t row = k0 + rr;
        rv[b][q] = (pq >= 0 && row >= rq && row < n) ? V[static_cast<int64_t>(c) * mq + (row - rq)] : 0.f;
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q;
      Zs[idx & 63][idx >> 6] = rz[q];
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int idx = tid + 256 * q;
        Vs[b][idx & 63][idx >> 6] = rv[b][q];
      }
  };
  // W2s = T_q (W partial sums); every wave then sees it after the barrier
  auto form_w2 = [&](const f32x16& wacc, int q) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Wp[wave >> 1][(e >> 2) * 8 + hf * 4 + (e & 3)][cb + rl] = wacc[e];
    {
      float rt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rt[i] = Tst[z * t_batch + static_cast<int64_t>(q) * 1024 + tid + 256 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i) Ts[(tid + 256 * i) / SBW][(tid + 256 * i) % SBW] = rt[i];
    }
    __syncthreads();
    if (wave < 2) {
      f32x16 w2 = {};
#pragma unroll
      for (int kk = 0; kk < SBW; kk += 2) {
        const int k = kk + hf;
        w2 = __builtin_amdgcn_mfma_f32_32x32x2f32(Ts[rl][k], Wp[0][k][32 * wave + rl] + Wp[1][k][32 * wave + rl],
                                                   w2, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) W2s[(e >> 2) * 8 + hf * 4 + (e & 3)][32 * wave + rl] = w2[e];
    }
    __syncthreads();
  };
  // pass 0: W of panel p_hi (V in slot 1 of the loader, as "next")
  {
    const int64_t rq = SBW * (p_hi + 1);
    f32x16 acc = {};
    const int64_t k0s = rq;
    load(k0s, rq, -1, p_hi);
    for (int64_t k0 = k0s; k0 < n; k0 += 64) {
      stage();
      __syncthreads();
      if (k0 + 64 < n) load(k0 + 64, rq, -1, p_hi);
#pragma unroll
      for (int kk = 0; kk < SBW; kk += 2) {
        const int k = kb + kk + hf;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[1][k][rl], Zs[k][cb + rl], acc, 0, 0, 0);
      }
      __syncthreads();
    }
    form_w2(acc, p_hi);
  }
  // passes 1 .. K: apply panel qa = p_hi - i + 1, accumulate W of qn = qa - 1
  for (int i = 1; i <= K; ++i) {
    const int qa = p_hi - i + 1, qn = i < K ? qa - 1 : -1;
    const int64_t ra = SBW * (qa + 1);
    const int64_t k0s = qn >= 0 ? SBW * (qn + 1) : ra;       // stream from the lower panel's first row
    f32x16 acc = {};
    load(k0s, k0s, qa, qn);
    for (int64_t k0 = k0s; k0 < n; k0 += 64) {
      stage();
      __syncthreads();
      if (k0 + 64 < n) load(k0 + 64, k0s, qa, qn);
      // Z -= V_qa W2: wave w -> chunk rows 32 (w >> 1) .., columns 32 (w & 1) ..
      f32x16 d = {};
#pragma unroll
      for (int kk = 0; kk < SBW; kk += 2) {
        const int k = kk + hf;
        d = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[0][kb + rl][k], W2s[k][cb + rl], d, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = kb + (e >> 2) * 8 + hf * 4 + (e & 3);
        Zs[rr][cb + rl] -= d[e];
      }
      __syncthreads();
      if (qn >= 0) {
#pragma unroll
        for (int kk = 0; kk < SBW; kk += 2) {
          const int k = kb + kk + hf;
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[1][k][rl], Zs[k][cb + rl], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int idx = tid + 256 * q, c = idx >> 6, rr = idx & 63;
        const int64_t row = k0 + rr;
        if (row >= ra && row < n && c < nc) Zz[static_cast<int64_t>(c0 + c) * n + row] = Zs[rr][c];
      }
      __syncthreads();
    }
    if (qn >= 0) form_w2(acc, qn);
  }
}

// ---- stage 1 of the band reduction: one panel's two-sided update
//
// With the panel's reflectors I - V T V^T (V: mp x 32, column-major, leading
// dimension mp) and the trailing block A22 (mp x mp, the lower triangle is
// stored, column-major with leading dimension n):
//   Y = A22 V, X = Y T, S = V^T X, W = X - V (T^T S) / 2,
//   A22 <- A22 - V W^T - W V^T (lower triangle).
// k_symm_v forms Y for 64 rows of A22 per workgroup, streaming A22 in 64 x
// 64 chunks read from the stored triangle (mirrored right of the diagonal),
// then X = Y T for its rows and its rows' share of S; k_w_form sums the
// shares and writes [V W]; k_syr2k updates one 64 x 64 tile of the lower
// triangle from [V W] [W V]^T.  Rows and columns are multiples of 4, so
// 16-byte accesses never straddle the end of a column.
constexpr int SY = 64;    // rows of a stage-1 block

__global__ __launch_bounds__(256) void k_symm_v(const float* A, int64_t n, int64_t a_batch, int mp,
                                                const float* V_g, int64_t v_batch, const float* T_g,
                                                int64_t t_batch, float* VW_g, int64_t vw_batch, float* SP) {
  __shared__ float Ls[SY][SY + 1];       // chunk of A22 as stored: Ls[c][r] = column c, row r
  __shared__ float Vs[SBW][SY + 1];      // rows of V: Vs[col][row]
  __shared__ float Ys[SY][SBW + 1];      // Y, then X (row-major)
  __shared__ float Ts[SBW][SBW + 1];
  __shared__ float Vb[SBW][SY + 1];      // V rows of this block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, hf = lane >> 5;
  uint32_t bx, by;
  xcd_group_2d(bx, by);                            // the blocks of one matrix on one XCD
  const int64_t z = by;
  const int ib = static_cast<int>(bx), i0 = SY * ib, nb = (mp + SY - 1) / SY;
  const float* a = A + z * a_batch;
  const float* V = V_g + z * v_batch;
  {
    float rt[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rt[q] = T_g[z * t_batch + tid + 256 * q];
#pragma unroll
    for (int q = 0; q < 4; ++q) Ts[(tid + 256 * q) >> 5][(tid + 256 * q) & 31] = rt[q];
  }
  float4 ra[4], rv[2];
  auto load = [&](int jc) {
    const int j0 = SY * jc;
    const int rs = jc > ib ? j0 : i0, cs = jc > ib ? i0 : j0;   // stored block: rows rs.., columns cs..
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
      ra[q] = (rs + r4 < mp && cs + c < mp)
                  ? *reinterpret_cast<const float4*>(a + static_cast<int64_t>(cs + c) * n + rs + r4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
      rv[q] = j0 + r4 < mp ? *reinterpret_cast<const float4*>(V + static_cast<int64_t>(c) * mp + j0 + r4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  const int wi = wave & 1, kh = wave >> 1;
  f32x16 acc = {};
  load(0);
  for (int jc = 0; jc < nb; ++jc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
      Ls[c][r4] = ra[q].x; Ls[c][r4 + 1] = ra[q].y; Ls[c][r4 + 2] = ra[q].z; Ls[c][r4 + 3] = ra[q].w;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
      Vs[c][r4] = rv[q].x; Vs[c][r4 + 1] = rv[q].y; Vs[c][r4 + 2] = rv[q].z; Vs[c][r4 + 3] = rv[q].w;
      if (jc == ib) { Vb[c][r4] = rv[q].x; Vb[c][r4 + 1] = rv[q].y; Vb[c][r4 + 2] = rv[q].z; Vb[c][r4 + 3] = rv[q].w; }
    }
    __syncthreads();
    if (jc + 1 < nb) load(jc + 1);
    const int i = SY / 2 * wi + rl;
    if (jc < ib) {                       // A(i, k) = Ls[k][i]
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int k = 32 * kh + 2 * s + hf;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ls[k][i], Vs[rl][k], acc, 0, 0, 0);
      }
    } else if (jc > ib) {                // A(i, k) = Ls[i][k]
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int k = 32 * kh + 2 * s + hf;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ls[i][k], Vs[rl][k], acc, 0, 0, 0);
      }
    } else {                             // diagonal chunk: the lower triangle, mirrored
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int k = 32 * kh + 2 * s + hf;
        const float lo = Ls[k][i], up = Ls[i][k];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(i >= k ? lo : up, Vs[rl][k], acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // Y = the two k halves
  if (kh == 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Ys[SY / 2 * wi + (e >> 2) * 8 + hf * 4 + (e & 3)][rl] = acc[e];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Ys[SY / 2 * wi + (e >> 2) * 8 + hf * 4 + (e & 3)][rl] += acc[e];
  }
  __syncthreads();
  // X = Y T (waves 0, 1: 32 rows each)
  f32x16 xa = {};
  if (wave < 2) {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int k = 2 * s + hf;
      xa = __builtin_amdgcn_mfma_f32_32x32x2f32(Ys[32 * wave + rl][k], Ts[k][rl], xa, 0, 0, 0);
    }
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Ys[32 * wave + (e >> 2) * 8 + hf * 4 + (e & 3)][rl] = xa[e];
  }
  __syncthreads();
  // X -> the W half of [V W] (column-major, leading dimension mp)
  float* Wd = VW_g + z * vw_batch + static_cast<int64_t>(SBW) * mp;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
    if (i0 + r4 < mp)
      *reinterpret_cast<float4*>(Wd + static_cast<int64_t>(c) * mp + i0 + r4) =
          make_float4(Ys[r4][c], Ys[r4 + 1][c], Ys[r4 + 2][c], Ys[r4 + 3][c]);
  }
  // this block's share of S = V^T X (wave 0, K = 64 rows)
  if (wave == 0) {
    f32x16 sa = {};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int k = 2 * s + hf;
      sa = __builtin_amdgcn_mfma_f32_32x32x2f32(Vb[rl][k], Ys[k][rl], sa, 0, 0, 0);
    }
    float* sp = SP + (z * nb + ib) * 1024;
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[((e >> 2) * 8 + hf * 4 + (e & 3)) * 32 + rl] = sa[e];
  }
}

// [V W] for 64 rows: S = sum of the blocks' shares, S2 = T^T S, W = X - V S2 / 2
__global__ __launch_bounds__(256) void k_w_form(int mp, const float* V_g, int64_t v_batch, const float* T_g,
                                                int64_t t_batch, float* VW_g, int64_t vw_batch, const float* SP) {
  __shared__ float Ss[SBW][SBW + 1], Ts[SBW][SBW + 1], S2[SBW][SBW + 1];
  __shared__ float Vr[SY][SBW + 1];
  const int tid = threadIdx.x;
  uint32_t bx, by;
  xcd_group_2d(bx, by);                            // the blocks of one matrix on one XCD
  const int64_t z = by;
  const int ib = static_cast<int>(bx), i0 = SY * ib, nb = (mp + SY - 1) / SY;
  const float* V = V_g + z * v_batch;
  float* VW = VW_g + z * vw_batch;
  const float* sp = SP + z * nb * 1024;
  {
    // elements 4 tid .. 4 tid + 3, the shares added in block order, eight loads in flight
    const int e = 4 * tid;
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b0 = 0; b0 < nb; b0 += 8) {
      float4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = b0 + q < nb ? *reinterpret_cast<const float4*>(sp + (b0 + q) * 1024 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < 8; ++q) { u.x += v[q].x; u.y += v[q].y; u.z += v[q].z; u.w += v[q].w; }
    }
    const float4 t4 = *reinterpret_cast<const float4*>(T_g + z * t_batch + e);
    const int a = e >> 5, b = e & 31;
    Ss[a][b] = u.x; Ss[a][b + 1] = u.y; Ss[a][b + 2] = u.z; Ss[a][b + 3] = u.w;
    Ts[a][b] = t4.x; Ts[a][b + 1] = t4.y; Ts[a][b + 2] = t4.z; Ts[a][b + 3] = t4.w;
  }
  // V rows of this block: to LDS and to the V half of [V W]
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
    if (i0 + r4 < mp) {
      const float4 v = *reinterpret_cast<const float4*>(V + static_cast<int64_t>(c) * mp + i0 + r4);
      *reinterpret_cast<float4*>(VW + static_cast<int64_t>(c) * mp + i0 + r4) = v;
      Vr[r4][c] = v.x; Vr[r4 + 1][c] = v.y; Vr[r4 + 2][c] = v.z; Vr[r4 + 3][c] = v.w;
    } else {
      Vr[r4][c] = 0.f; Vr[r4 + 1][c] = 0.f; Vr[r4 + 2][c] = 0.f; Vr[r4 + 3][c] = 0.f;
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int q = 0; q < 4; ++q) {                  // S2 = T^T S
    const int e = tid + 256 * q, a = e >> 5, b = e & 31;
    float u = 0.f;
#pragma unroll
    for (int m = 0; m < SBW; ++m) u += Ts[m][a] * Ss[m][b];
    S2[a][b] = 0.5f * u;
  }
  __syncthreads();
  float* Wd = VW + static_cast<int64_t>(SBW) * mp;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
    if (i0 + r4 < mp) {
      float* w = Wd + static_cast<int64_t>(c) * mp + i0 + r4;
      float4 x = *reinterpret_cast<const float4*>(w);
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll 4
      for (int a2 = 0; a2 < SBW; ++a2) {
        const float s2 = S2[a2][c];
        d0 += Vr[r4][a2] * s2;
        d1 += Vr[r4 + 1][a2] * s2;
        d2 += Vr[r4 + 2][a2] * s2;
        d3 += Vr[r4 + 3][a2] * s2;
      }
      x.x -= d0; x.y -= d1; x.z -= d2; x.w -= d3;
      *reinterpret_cast<float4*>(w) = x;
    }
  }
}

// A22 -= [V W] [W V]^T on the 64 x 64 tile (bi, bj), bi >= bj, of the lower
// triangle of matrix z; the diagonal tiles keep their upper part.  256
// threads (tid < 256, four waves); an inactive caller issues no memory
// operation but takes the same three barriers as an active one.
__device__ __forceinline__ void syr2k_tile(float* A, int64_t n, int64_t a_batch, int mp, const float* VW_g,
                                           int64_t vw_batch, int64_t z, int bi, int bj, int tid, bool active,
                                           float (*As)[SY + 1], float (*Bs)[SY + 1]) {
  const int lane = tid & 63, wave = tid >> 6, rl = lane & 31, hf = lane >> 5;
  const int i0 = SY * bi, j0 = SY * bj;
  float* a = A + z * a_batch;
  const float* VW = VW_g + z * vw_batch;
  float4 rc[4], ra[4], rb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
    rc[q] = (active && i0 + r4 < mp && j0 + c < mp)
                ? *reinterpret_cast<const float4*>(a + static_cast<int64_t>(j0 + c) * n + i0 + r4)
                : make_float4(0.f, 0.f, 0.f, 0.f);
    // operand column k = c: [V W] column c at rows i0.., [W V] column c = [V W] column c ^ 32 at rows j0..
    ra[q] = (active && i0 + r4 < mp) ? *reinterpret_cast<const float4*>(VW + static_cast<int64_t>(c) * mp + i0 + r4)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
    rb[q] = (active && j0 + r4 < mp)
                ? *reinterpret_cast<const float4*>(VW + static_cast<int64_t>(c ^ SBW) * mp + j0 + r4)
                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
    As[c][r4] = ra[q].x; As[c][r4 + 1] = ra[q].y; As[c][r4 + 2] = ra[q].z; As[c][r4 + 3] = ra[q].w;
    Bs[c][r4] = rb[q].x; Bs[c][r4 + 1] = rb[q].y; Bs[c][r4 + 2] = rb[q].z; Bs[c][r4 + 3] = rb[q].w;
  }
  __syncthreads();
  const int wi = wave & 1, wj = wave >> 1;
  f32x16 acc = {};
  if (!(bi == bj && wi < wj)) {          // sub-blocks above the diagonal are not needed
#pragma unroll
    for (int s = 0; s < SBW; ++s) {
      const int k = 2 * s + hf;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[k][32 * wi + rl], Bs[k][32 * wj + rl], acc, 0, 0, 0);
    }
  }
  __syncthreads();
  // the product, column-major through LDS (As reused: As[c][r] = product at row r, column c)
#pragma unroll
  for (int e = 0; e < 16; ++e) As[32 * wj + rl][32 * wi + (e >> 2) * 8 + hf * 4 + (e & 3)] = acc[e];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + 256 * q, c = idx >> 4, r4 = (idx & 15) * 4;
    if (active && i0 + r4 < mp && j0 + c < mp) {
      const int gc = j0 + c;
      float4 v = rc[q];
      if (i0 + r4 >= gc) v.x -= As[c][r4];
      if (i0 + r4 + 1 >= gc) v.y -= As[c][r4 + 1];
      if (i0 + r4 + 2 >= gc) v.z -= As[c][r4 + 2];
      if (i0 + r4 + 3 >= gc) v.w -= As[c][r4 + 3];
      *reinterpret_cast<float4*>(a + static_cast<int64_t>(gc) * n + i0 + r4) = v;
    }
  }
}

// tile (bi, bj), bi >= bj, of the lower triangle from its linear index x = bi (bi + 1) / 2 + bj
__device__ __forceinline__ void tri_tile(int x, int& bi, int& bj) {
  bi = static_cast<int>((sqrtf(8.f * x + 1.f) - 1.f) * 0.5f);
  while (bi * (bi + 1) / 2 > x) --bi;
  while ((bi + 1) * (bi + 2) / 2 <= x) ++bi;
  bj = x - bi * (bi + 1) / 2;
}

// Every tile of the lower triangle (col0_only: the tiles (bi, 0) of the first
// block column, one per workgroup).
__global__ __launch_bounds__(256) void k_syr2k(float* A, int64_t n, int64_t a_batch, int mp, const float* VW_g,
                                               int64_t vw_batch, int col0_only) {
  __shared__ float As[2 * SBW][SY + 1];  // [V W] rows of the tile's rows: As[k][r]
  __shared__ float Bs[2 * SBW][SY + 1];  // [W V] rows of the tile's columns: Bs[k][r]
  uint32_t bx, by;
  xcd_group_2d(bx, by);                            // the tiles of one matrix on one XCD
  int bi, bj;
  if (col0_only) { bi = static_cast<int>(bx); bj = 0; }
  else tri_tile(static_cast<int>(bx), bi, bj);
  syr2k_tile(A, n, a_batch, mp, VW_g, vw_batch, by, bi, bj, threadIdx.x, true, As, Bs);
}

// One launch for the tail of panel p's update and the next panel's QR, which
// do not touch each other's data: workgroups 0 .. batch-1 factor panel p + 1
// (its columns, the first block column of A22, were updated by k_syr2k's
// col0_only launch before), the others update the tiles (bi, bj), bj >= 1,
// two tiles per workgroup (a tile per 256 threads).  The QR workgroups come
// first in dispatch order, so they start at once and the tiles fill the
// rest of the chip beside them.
constexpr size_t kTileLds = 2 * sizeof(float) * 2 * SBW * (SY + 1);   // As + Bs of one tile
constexpr size_t kBandStepLds = 2 * kTileLds > sizeof(QrRegLds) ? 2 * kTileLds : sizeof(QrRegLds);
__global__ __launch_bounds__(RT) void k_band_step(float* A, int64_t n, int64_t a_batch, int mp, const float* VW_g,
                                                  int64_t vw_batch, int ntiles, int npairs, int batch,
                                                  float* panel, int mp_next, float* Vn, int64_t vstride, float* Tn,
                                                  int64_t tstride, float* taus) {
  static_assert(RT == 512, "two 256-thread tiles per workgroup");
  __shared__ __align__(16) char raw[kBandStepLds];
  const uint32_t L = blockIdx.x;
  if (L < static_cast<uint32_t>(batch)) {
    qr_reg_run(panel, mp_next, n, a_batch, 0, SBW, Vn, vstride, Tn, tstride, taus, SBW, 1, L,
               *reinterpret_cast<QrRegLds*>(raw));
    return;
  }
  uint32_t z, pair;
  xcd_group(L - static_cast<uint32_t>(batch), static_cast<uint32_t>(npairs), static_cast<uint32_t>(batch), z, pair);
  const int half = threadIdx.x >> 8;
  const int ti = 2 * static_cast<int>(pair) + half;
  const bool active = ti < ntiles;
  int bi = 1, bj = 1;
  if (active) {                                    // the triangle of tiles with bj >= 1, shifted by one
    tri_tile(ti, bi, bj);
    ++bi; ++bj;
  }
  float* base = reinterpret_cast<float*>(raw + half * kTileLds);
  auto As = reinterpret_cast<float (*)[SY + 1]>(base);
  auto Bs = reinterpret_cast<float (*)[SY + 1]>(base + 2 * SBW * (SY + 1));
  syr2k_tile(A, n, a_batch, mp, VW_g, vw_batch, z, bi, bj, threadIdx.x & 255, active, As, Bs);
}

__global__ __launch_bounds__(256) void k_copy_cols(const float* in, int64_t ld_in, int64_t in_batch, float* out,
                                                  int64_t ld_out, int64_t out_batch, int64_t rows, int64_t cols) {
  const int64_t z = blockIdx.y;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < rows * cols; idx += 256ll * gridDim.x) {
    const int64_t c = idx / rows, r = idx % rows;
    out[z * out_batch + c * ld_out + r] = in[z * in_batch + c * ld_in + r];
  }
}

struct SyevLayout {
  int64_t P, vtot, nref;
  size_t v_off, t_off, tau_off, y_off, x_off, s1_off, s2_off, s3_off, wb_off, wb2_off, part_off, pscr_off,
      bw_off, rf_off, d_off, e_off, lam_off, dp_off, yv_off, nrm_off, cbt_off, sp_off, total;
  int64_t ng, K0;                 // chase groups of 32 sweeps, steps of sweep 0
};

SyevLayout syev_layout(int64_t n, int R, int batch) {
  SyevLayout L{};
  L.P = n / SBW - 1;
  L.vtot = 0;
  for (int64_t p = 0; p < L.P; ++p) L.vtot += (n - (p + 1) * SBW) * SBW;
  L.nref = sweep_offset(n, n - 2);
  const size_t B = static_cast<size_t>(batch);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const int64_t Rm = R > SBW ? R : SBW;
  L.v_off = take(B * L.vtot * 4);
  L.t_off = take(B * (L.P > 0 ? L.P : 1) * 1024 * 4);
  L.tau_off = take(B * 2 * SBW * 4);
  L.y_off = take(B * n * SBW * 4);
  L.x_off = take(B * n * 2 * SBW * 4);
  L.s1_off = take(B * 1024 * 4);
  L.s2_off = take(B * 1024 * 4);
  L.s3_off = take(B * 1024 * 4);
  L.wb_off = take(B * SBW * Rm * 4);
  L.wb2_off = take(B * SBW * Rm * 4);
  L.part_off = take(B * 16 * SBW * Rm * 4);
  L.pscr_off = take(panel_factor_scratch_floats(n, batch) * 4);
  L.bw_off = take(B * n * BWS * 4);
  L.rf_off = take(B * (L.nref > 0 ? L.nref : 1) * RFS * 4);
  L.d_off = take(B * n * 8);
  L.e_off = take(B * n * 8);
  L.lam_off = take(B * R * 8);
  L.dp_off = take(B * n * R * 8);
  L.yv_off = take(B * n * R * 8);
  L.nrm_off = take(B * R * 8);
  L.ng = (n - 2 + SBW - 1) / SBW;
  L.K0 = sweep_steps(n, 0);
  L.cbt_off = take(B * (L.ng > 0 ? L.ng : 1) * (L.K0 > 0 ? L.K0 : 1) * CBR * SBW * 4);
  L.sp_off = take(B * ((n + SY - 1) / SY) * 1024 * 4);
  L.total = off;
  return L;
}

// split-K for the products with a 32-row output and a long K (a workgroup per
// output tile would otherwise walk K alone): chunks of at least 256
int ksplit_for(int64_t K) {
  const int64_t s = K / 256;
  return static_cast<int>(s < 1 ? 1 : (s > 16 ? 16 : s));
}

}  // namespace

size_t syev_top_work_bytes(int64_t n, int R, int batch) { return syev_layout(n, R, batch).total; }

namespace {
std::atomic<int> g_chase_spin_limit{1 << 22};
}  // namespace

void set_chase_spin_limit(int polls) { g_chase_spin_limit.store(polls < 0 ? 0 : polls); }

hipError_t syev_top(float* A, int64_t n, int batch, int R, float* Z, double* lam_out, void* work,
                    hipStream_t s, int* status, hipEvent_t band_done, bool inv_sqrt_scale,
                    const SyevSide* side) {
  if (n % SBW != 0 || n > 32768 || R < 1 || R > n || !status) return hipErrorInvalidValue;
  const SyevLayout Lw = syev_layout(n, R, batch);
  char* wb = static_cast<char*>(work);
  float* Vst = reinterpret_cast<float*>(wb + Lw.v_off);
  float* Tst = reinterpret_cast<float*>(wb + Lw.t_off);
  float* taus = reinterpret_cast<float*>(wb + Lw.tau_off);
  float* Yb = reinterpret_cast<float*>(wb + Lw.y_off);
  float* VW = reinterpret_cast<float*>(wb + Lw.x_off);     // [V | W], mp x 64 column-major
  float* S1 = reinterpret_cast<float*>(wb + Lw.s1_off);
  float* S2 = reinterpret_cast<float*>(wb + Lw.s2_off);
  float* Wb = reinterpret_cast<float*>(wb + Lw.wb_off);
  float* Wb2 = reinterpret_cast<float*>(wb + Lw.wb2_off);
  float* part = reinterpret_cast<float*>(wb + Lw.part_off);
  float* pscr = reinterpret_cast<float*>(wb + Lw.pscr_off);
  float* SP = reinterpret_cast<float*>(wb + Lw.sp_off);
  float* Bw = reinterpret_cast<float*>(wb + Lw.bw_off);
  float* Rf = reinterpret_cast<float*>(wb + Lw.rf_off);
  double* dd = reinterpret_cast<double*>(wb + Lw.d_off);
  double* ee = reinterpret_cast<double*>(wb + Lw.e_off);
  double* lam = reinterpret_cast<double*>(wb + Lw.lam_off);
  double* dp = reinterpret_cast<double*>(wb + Lw.dp_off);
  double* yv = reinterpret_cast<double*>(wb + Lw.yv_off);
  const int64_t nn = n * n;
  hipError_t e;
  auto gemm = [&](int64_t M, int64_t N, int64_t K, const float* Ab, GemmDim am, GemmDim ak, int64_t ab,
                  const float* Bb, GemmDim bk, GemmDim bn, int64_t bb, float* Cb, int64_t cm, int64_t cn,
                  int64_t cb, float alpha, float beta, int ksplit = 1, int a_sym = 0,
                  int c_lower = 0) -> hipError_t {
    if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
    GemmArgs g{};
    g.a_sym = a_sym; g.c_lower = c_lower;
    g.M = M; g.N = N; g.K = K;
    g.A = Ab; g.a_dtype = kF32; g.am = am; g.ak = ak; g.a_batch = ab;
    g.B = Bb; g.b_dtype = kF32; g.bk = bk; g.bn = bn; g.b_batch = bb;
    g.C = Cb; g.c_dtype = kF32; g.c_m = cm; g.c_n = cn; g.c_batch = cb;
    g.alpha = alpha; g.beta = beta;
    if (ksplit > 1) { g.ksplit = ksplit; g.partial = part; }
    return launch_gemm(g, batch, s);
  };
  // ---- stage 1: dense -> band
  std::vector<int64_t> voff(Lw.P > 0 ? Lw.P : 1);
  {
    int64_t o = 0;
    for (int64_t p = 0; p < Lw.P; ++p) { voff[p] = o; o += (n - (p + 1) * SBW) * SBW; }
  }
  {
  ProfScope ps_band("band", s);
  {
    // algorithmic work per panel: the lower triangle of A22 read by the
    // symmetric product and read and written by the rank-64 update (3 passes),
    // the panel read and written; 2 mp^2 b (A22 V) + 2 mp^2 (2 b) / 2 (the
    // lower half of [V W][W V]^T) + 4 mp b^2 (panel QR) flops
    double by = 0.0, fl = 0.0;
    for (int64_t p = 0; p < Lw.P; ++p) {
      const double mp = static_cast<double>(n - (p + 1) * SBW);
      by += 3.0 * 4.0 * mp * (mp + 1) / 2 + 2.0 * 4.0 * mp * SBW;
      fl += 2.0 * mp * mp * SBW + 2.0 * mp * mp * SBW + 4.0 * mp * SBW * SBW;
    }
    prof_add_work("band", batch * by, batch * fl);
  }
  bool qr_done = false;   // panel p was factored inside the previous panel's band step
  for (int64_t p = 0; p < Lw.P; ++p) {
    const int64_t c = p * SBW, r = c + SBW, mp = n - r;
    float* panel = A + c * n + r;                  // column-major mp x 32 (ld n)
    float* V = Vst + voff[p];
    float* T = Tst + p * 1024;
    const int64_t vs = Lw.vtot, ts = Lw.P * 1024;
    // R into the panel's top rows: by the panel kernel when the panel is one
    // block, else as panel_top -= V_top (T^T (V^T panel))
    const bool r_in = mp <= panel_block_rows();
    if (!qr_done && (e = panel_factor(panel, mp, n, nn, 0, SBW, batch, V, vs, T, ts, taus, SBW, pscr, s,
                                      r_in ? 1 : 0)) != hipSuccess)
      return e;
    qr_done = false;
    if (!r_in) {
      if ((e = gemm(SBW, SBW, mp, V, plain(mp), plain(1), vs, panel, plain(1), plain(n), nn, S1, SBW, 1, 1024, 1.f,
                    0.f, ksplit_for(mp))) != hipSuccess) return e;
      if ((e = gemm(SBW, SBW, SBW, T, plain(1), plain(SBW), ts, S1, plain(SBW), plain(1), 1024, S2, SBW, 1, 1024,
                    1.f, 0.f)) != hipSuccess) return e;
      if ((e = gemm(SBW, SBW, SBW, V, plain(1), plain(mp), vs, S2, plain(SBW), plain(1), 1024, panel, 1, n, nn,
                    -1.f, 1.f)) != hipSuccess) return e;
    }
    // Y = A22 V, X = Y T and the shares of V^T X; [V W]; A22 -= [V W] [W V]^T
    float* A22 = A + r * n + r;
    const int64_t vwb = n * 2 * SBW;
    const int nbk = static_cast<int>((mp + SY - 1) / SY);
    k_symm_v<<<dim3(nbk, batch), 256, 0, s>>>(A22, n, nn, static_cast<int>(mp), V, vs, T, ts, VW, vwb, SP);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_w_form<<<dim3(nbk, batch), 256, 0, s>>>(static_cast<int>(mp), V, vs, T, ts, VW, vwb, SP);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the next panel (the first block column of A22 below its first 32 rows)
    // is factored beside the rest of this update when it is one register
    // block: its block column first, then one launch for both
    const int64_t mpn = mp - SBW;
    if (p + 1 < Lw.P && mpn > 0 && mpn <= panel_block_rows()) {
      k_syr2k<<<dim3(static_cast<unsigned>(nbk), batch), 256, 0, s>>>(A22, n, nn, static_cast<int>(mp), VW, vwb, 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      const int ntiles = nbk * (nbk - 1) / 2, npairs = (ntiles + 1) / 2;
      const unsigned grid = static_cast<unsigned>(batch) * static_cast<unsigned>(1 + npairs);
      k_band_step<<<grid, RT, 0, s>>>(A22, n, nn, static_cast<int>(mp), VW, vwb, ntiles, npairs, batch,
                                      A + r * n + r + SBW, static_cast<int>(mpn), Vst + voff[p + 1], vs,
                                      Tst + (p + 1) * 1024, ts, taus);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      qr_done = true;
    } else {
      k_syr2k<<<dim3(static_cast<unsigned>(nbk * (nbk + 1) / 2), batch), 256, 0, s>>>(A22, n, nn,
                                                                                    static_cast<int>(mp), VW, vwb, 0);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  }
  if (band_done && (e = hipEventRecord(band_done, s)) != hipSuccess) return e;
  // ---- stage 2: band -> tridiagonal
  {
    int64_t blocks = (n * BWS + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    k_band_init<<<dim3(static_cast<unsigned>(blocks), batch), 256, 0, s>>>(A, n, Bw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // sweeps in flight: 8 waves up to 32 steps per sweep (n <= 1026), else 16
    const int64_t K0 = sweep_steps(n, 0);
    const int nw = K0 > 32 ? 16 : 8;
    int S = static_cast<int>((K0 + nw - 1) / nw);
    if (S < 4) S = 4;
    // With 8 waves the chase asks for all of a CU's LDS (its waves use
    // 8 * sizeof(ChaseLds) of it) so that no other workgroup is placed beside
    // it: its ticks are bound by the CU's memory pipeline, which a neighbour on
    // the CU (the feature path runs beside the token chase) would share.  The
    // 16-wave chase of the larger matrices runs beside the other lane's
    // stages, which need those CUs (claiming them cost 20% of that step).
    const size_t lds = nw == 8 ? static_cast<size_t>(kChaseLdsClaim) : static_cast<size_t>(nw) * sizeof(ChaseLds);
    static_assert(16 * sizeof(ChaseLds) <= kChaseLdsClaim, "the chase's tiles fit its claim");
    static const hipError_t attr = [] {   // once per process (thread-safe initialization)
      hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(k_chase<8>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kChaseLdsClaim);
      if (r == hipSuccess)
        r = hipFuncSetAttribute(reinterpret_cast<const void*>(k_chase<16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kChaseLdsClaim);
      return r;
    }();
    if (attr != hipSuccess) return attr;
    {
      ProfScope ps("chase", s);
      const int spin = g_chase_spin_limit.load();
      if (nw == 8) k_chase<8><<<batch, 8 * 64, lds, s>>>(Bw, static_cast<int>(n), Rf, Lw.nref * RFS, S, status, spin);
      else k_chase<16><<<batch, 16 * 64, lds, s>>>(Bw, static_cast<int>(n), Rf, Lw.nref * RFS, S, status, spin);
      // algorithmic work: the band read and written once, every reflector
      // written once; per step (b = 32) the reflector's two-sided action on the
      // diagonal block (w = D v, D - v w^T - w v^T + c v v^T: 5 b^2 flops), its
      // left action on the left block (4 b^2) and right action on the block
      // below (4 b^2)
      prof_add_work("chase", static_cast<double>(batch) * (2.0 * n * BWS * 4 + Lw.nref * RFS * 4.0),
                    static_cast<double>(batch) * Lw.nref * 13.0 * SBW * SBW);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the block factors V T of the chase back-transformation need only the
    // reflectors: on the side stream, beside the tridiagonal eigenpairs
    if (side && Lw.ng > 0 && Lw.K0 > 0) {
      if ((e = hipEventRecord(side->chase_done, s)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side->s, side->chase_done, 0)) != hipSuccess) return e;
      {
        ProfScope ps("chase_back", side->s);
        k_cb_tfac<<<dim3(static_cast<unsigned>(Lw.ng * Lw.K0), batch), 64, 0, side->s>>>(
            Rf, Lw.nref * RFS, static_cast<int>(n), static_cast<int>(Lw.K0),
            reinterpret_cast<float*>(wb + Lw.cbt_off), Lw.ng * Lw.K0 * CBR * SBW);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(side->tfac_done, side->s)) != hipSuccess) return e;
    }
    int64_t tb = (n + 255) / 256;
    k_tri_out<<<dim3(static_cast<unsigned>(tb), batch), 256, 0, s>>>(Bw, n, dd, ee);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // ---- stage 3: top R eigenpairs of the tridiagonal (fp64)
  {
    const size_t lds = static_cast<size_t>(2 * n) * sizeof(double);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bisect),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 65536);
    if (attr != hipSuccess) return attr;
    if (lds > 65536) return hipErrorInvalidValue;
    const unsigned gx = static_cast<unsigned>((R + IVW - 1) / IVW);
    double* nrm = reinterpret_cast<double*>(wb + Lw.nrm_off);
    {
      ProfScope ps("tri_eig", s);
      k_bisect<<<dim3(static_cast<unsigned>((BSL * R + 255) / 256), batch), 256, lds, s>>>(dd, ee, n, R, lam);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      k_invit<<<dim3(gx, batch), IVW, 0, s>>>(dd, ee, n, R, lam, dp, yv, nrm);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      k_invit_out<<<dim3(static_cast<unsigned>((n + 31) / 32), static_cast<unsigned>((R + 31) / 32), batch), 256, 0,
                    s>>>(yv, nrm, n, R, Z, n * n, inv_sqrt_scale ? lam : nullptr);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (lam_out) {
      if ((e = hipMemcpyAsync(lam_out, lam, sizeof(double) * batch * R, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return e;
    }
  }
  // ---- stage 4: back-transformation (chase reflectors in blocks, then panel reflectors)
  {
    float* Tcb = reinterpret_cast<float*>(wb + Lw.cbt_off);
    const int ng = static_cast<int>(Lw.ng), K0 = static_cast<int>(Lw.K0);
    const int64_t tstr = Lw.ng * Lw.K0 * CBR * SBW;
    if (ng > 0 && K0 > 0) {
      ProfScope ps("chase_back", s);
      // algorithmic work: Z (n x R) read and written once, every reflector
      // read once; each 32-long reflector applied to R columns (4 b R flops)
      prof_add_work("chase_back", static_cast<double>(batch) * (2.0 * n * R * 4 + Lw.nref * RFS * 4.0),
                    static_cast<double>(batch) * Lw.nref * 4.0 * SBW * R);
      if (side) {
        if ((e = hipStreamWaitEvent(s, side->tfac_done, 0)) != hipSuccess) return e;
      } else {
        k_cb_tfac<<<dim3(static_cast<unsigned>(ng * K0), batch), 64, 0, s>>>(Rf, Lw.nref * RFS,
                                                                           static_cast<int>(n), K0, Tcb, tstr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      const int nchunk = (R + 63) / 64;
      const int tmax = 2 * (ng - 1) + K0 - 1;
      // wavefront steps 2u and 2u + 1 per launch: groups g' with a block at either
      for (int u = 0; 2 * u <= tmax; ++u) {
        const int x = 2 * u - K0 + 1;                // g' >= x / 2, rounded up
        const int glo = x > 0 ? (x + 1) / 2 : 0;
        const int ghi = u < ng - 1 ? u : ng - 1;
        if (ghi < glo) continue;
        k_cb_apply<<<dim3(static_cast<unsigned>((ghi - glo + 1) * nchunk), batch), 256, 0, s>>>(
            u, glo, nchunk, Z, static_cast<int>(n), R, n * n, Rf, Lw.nref * RFS, Tcb, tstr, ng, K0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
    ProfScope ps_bb("band_back", s);
    {
      // algorithmic work: per panel, Z rows r.. (mp x R) read and written,
      // V read; 4 mp b R flops
      double by = 0.0, fl = 0.0;
      for (int64_t p = 0; p < Lw.P; ++p) {
        const double mp = static_cast<double>(n - (p + 1) * SBW);
        by += 4.0 * (2.0 * mp * R + mp * SBW);
        fl += 4.0 * mp * SBW * R;
      }
      prof_add_work("band_back", batch * by, batch * fl);
    }
    // K panels per launch, from the last panel down
    constexpr int KBB = 8;
    for (int64_t p = Lw.P - 1; p >= 0; p -= KBB) {
      const int K = static_cast<int>(p + 1 < KBB ? p + 1 : KBB);
      k_apply_wy<<<dim3(static_cast<unsigned>((R + 63) / 64), batch), 256, 0, s>>>(
          Z, n, nn, R, Vst, Lw.vtot, Tst, Lw.P * 1024, static_cast<int>(p), K);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t copy_cols(const float* in, int64_t ld_in, int64_t in_batch, float* out, int64_t ld_out,
                     int64_t out_batch, int64_t rows, int64_t cols, int batch, hipStream_t s) {
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_copy_cols<<<dim3(static_cast<unsigned>(blocks), batch), 256, 0, s>>>(in, ld_in, in_batch, out, ld_out,
                                                                       out_batch, rows, cols);
  return hipGetLastError();
}

}  // namespace jolt
