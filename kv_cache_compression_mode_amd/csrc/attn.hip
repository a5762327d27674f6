// Decode fused into an attention consumer (D = 128).
//
// The KV cache is the cost the codec exists to cut (JoLT abstract, first
// sentence); a consumer that reads the compressed records directly never
// writes the reconstructed cache to memory.  For one layer, per KV head h and
// its query vectors q_j (the G query heads of a GQA group times the new
// tokens), attention over the T cached tokens:
//     out_j = softmax(q_j K^_h^T / sqrt(D)) V^_h,
// with K^_h and V^_h reconstructed tile by tile from their records exactly as
// the decode does (U~_T W + Y^ Q on bf16 matrix cores, W = G~ U~_D^T as a
// bf16 hi + lo pair, dequantization fused), kept in registers.
//
// One workgroup of 4 waves per (256 tokens, KV head); a wave owns 64 tokens.
//  1. K^ tile computed transposed (features as the product's rows): each lane
//     holds one token's 64 features of its half, so a score is a dot over the
//     lane's values plus one swap of the wave's halves.
//  2. Per-wave softmax statistics (max, sum of exp) and weights p.
//  3. V^ tile computed with tokens as rows: each lane holds one feature of 16
//     tokens, so P V is a dot over the lane's values plus one swap of halves.
//  4. The 4 waves' partials (m, l, o) merged in LDS into the block's partial;
//     a second kernel merges the blocks of each (head, query) in order.
#include "device.hpp"
#include "kernels.hpp"

namespace jolt {
namespace {

constexpr int D = 128;
constexpr int kRows = 256;                  // tokens per workgroup

struct AttnLds {
  // W's k steps (hi, lo planes, 4 column tiles), two steps per stage,
  // double-buffered: [buf][step][plane][ct][lane][8]; reused for the merge
  uint16_t wl[2][2][2 * 4 * 64 * 8];
  uint16_t ql[4 * 8 * 64 * 8];              // Q^T bf16 in fragment order [ct][d / 16][lane][8]
  float q[kAttnMaxQ][D];                    // the head's query vectors
  float p[4][kAttnMaxQ][64];                // per-wave softmax weights, token-major in the wave
};
static_assert(sizeof(float) * 4 * kAttnMaxQ * (D + 2) <= sizeof(uint16_t) * 2 * 2 * 2 * 4 * 64 * 8,
              "the merge fits the W staging area");

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0));
  return v;
}

__device__ __forceinline__ bf16x8 load8(const uint16_t* base, int64_t idx, int64_t limit, bool aligned) {
  bf16x8 v;
  if (aligned && idx + 8 <= limit) {
    const uint4 raw = ldg16(base + idx);
    v = *reinterpret_cast<const bf16x8*>(&raw);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t b = idx + i < limit ? ldg_u16(base + idx + i) : static_cast<uint16_t>(0);
      v[i] = __builtin_bit_cast(__bf16, b);
    }
  }
  return v;
}

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The reconstruction of one record's rows t0 .. t0+63 of head h (this wave),
// all 4 waves of the block in step (block barriers inside).  ROWS = false:
// acc[rt][ct][i] = X^[t0 + 32 rt + lane % 32][32 ct + 8 (i / 4) + 4 half + i % 4]
// (features as the product's rows); ROWS = true: acc[rt][ct][i] =
// X^[t0 + 32 rt + 8 (i / 4) + 4 half + i % 4][32 ct + lane % 32].  The same
// operand registers serve both: a matrix-core operand holds one row (or
// column) and 8 consecutive k per lane, so swapping the operands transposes
// the product.  Rows past T come out zero.
template <bool ROWS>
__device__ __forceinline__ void reconstruct(const DecRec& R, int64_t h, int64_t t0, int T, AttnLds& sm,
                                            f32x16 (&acc)[2][4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 31, half = lane >> 5;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x16{};
  const bool ua = (R.r_T % 8) == 0;
  const int nks = R.r_Tp / 16, nst = nks / 2;
  bf16x8 a[2][2];   // [step][rt]: U~_T rows of this wave
  auto load_k = [&](int st) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kk = 32 * st + 16 * sub + 8 * half;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int64_t t = t0 + 32 * rt + r;
        a[sub][rt] = t < T ? load8(R.Ut() + t * R.r_T, kk, R.r_T, ua) : zero8();
      }
    }
  };
  uint4 wh[2], wlo[2];
  auto load_w = [&](int st) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int64_t o = ((h * 4 + wave) * nks + 2 * st + sub) * 512 + lane * 8;
      wh[sub] = ldg16(R.Whi + o);
      wlo[sub] = ldg16(R.Wlo() + o);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      *reinterpret_cast<uint4*>(&sm.wl[buf][sub][(wave * 64 + lane) * 8]) = wh[sub];
      *reinterpret_cast<uint4*>(&sm.wl[buf][sub][((4 + wave) * 64 + lane) * 8]) = wlo[sub];
    }
  };
  if (nst > 0) {
    load_w(0);
    load_k(0);
    store_w(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bf16x8 ca[2][2] = {{a[0][0], a[0][1]}, {a[1][0], a[1][1]}};
    if (st + 1 < nst) {
      load_w(st + 1);
      load_k(st + 1);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 ch = *reinterpret_cast<const bf16x8*>(&sm.wl[buf][sub][(ct * 64 + lane) * 8]);
        const bf16x8 cl = *reinterpret_cast<const bf16x8*>(&sm.wl[buf][sub][((4 + ct) * 64 + lane) * 8]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          if constexpr (ROWS) {
            acc[rt][ct] = mma(ca[sub][rt], ch, acc[rt][ct]);
            acc[rt][ct] = mma(ca[sub][rt], cl, acc[rt][ct]);
          } else {
            acc[rt][ct] = mma(ch, ca[sub][rt], acc[rt][ct]);
            acc[rt][ct] = mma(cl, ca[sub][rt], acc[rt][ct]);
          }
        }
      }
    }
    // the other buffer was last read in the previous stage, before its barrier
    if (st + 1 < nst) store_w(buf ^ 1);
    __syncthreads();
  }
  // the dequantized, rotated-back residual: + Y^ Q (K = 128 features)
  const int bits = R.bits;
  for (int d0 = 0; d0 < D; d0 += 16) {
    const int dd = d0 + 8 * half;               // this lane's 8 features
    const int g = dd >> 5, bitpos = (dd & 31) * bits;
    bf16x8 y[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t t = t0 + 32 * rt + r;
      uint32_t sw = 0u, w0 = 0u, w1 = 0u;       // rows past T: m16 = s16 = 0 gives y = 0
      if (t < T) {
        const int64_t gi = (h * T + t) * 4 + g;
        sw = ldg32(R.scales() + gi);
        const uint32_t* cw = R.codes() + gi * bits;
        w0 = ldg32(cw + (bitpos >> 5));
        if ((bitpos & 31) + 8 * bits > 32) w1 = ldg32(cw + (bitpos >> 5) + 1);
      }
      y[rt] = dequant8<bf16x8>(sw, w0, w1, static_cast<uint32_t>(bitpos & 31), static_cast<uint32_t>(bits));
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&sm.ql[((ct * 8 + (d0 >> 4)) * 64 + lane) * 8]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if constexpr (ROWS) acc[rt][ct] = mma(y[rt], bq, acc[rt][ct]);
        else acc[rt][ct] = mma(bq, y[rt], acc[rt][ct]);
      }
    }
  }
}

__device__ __forceinline__ float max32(float v) {   // max over the 32 lanes of a half
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float sum32(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__global__ __launch_bounds__(256, 2) void k_attn_decode(AttnArgs a) {
  __shared__ __align__(16) AttnLds sm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 31, half = lane >> 5;
  uint32_t blk = blockIdx.x, hh = blockIdx.y;
  xcd_group_2d(blk, hh);                         // a head's blocks on one XCD (its W in one L2)
  const int64_t h = hh;
  const int T = a.T, nq = a.nq;
  const int64_t t0 = static_cast<int64_t>(blk) * kRows + 64 * wave;
  // Q^T (bf16, fragment order) and the head's query vectors into LDS
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = threadIdx.x + 256 * j, l = c & 63;
    *reinterpret_cast<uint4*>(&sm.ql[c * 8]) =
        ldg16(a.Qt16 + (32 * (c >> 9) + (l & 31)) * D + 16 * ((c >> 6) & 7) + 8 * (l >> 5));
  }
  for (int i = threadIdx.x; i < nq * D; i += 256) {
    const int j = i / D, d = i % D;
    // vector j = g * n_new + s of KV head h is query head h G + g, new token s
    const int g = j / a.n_new, s = j % a.n_new;
    sm.q[j][d] = a.q[((h * a.G + g) * a.n_new + s) * D + d];
  }
  __syncthreads();
  f32x16 acc[2][4];
  // ---- 1. K^ (features as rows): lane = token, 64 features of its half
  reconstruct<false>(a.k, h, t0, T, sm, acc);
  float m_w[kAttnMaxQ], l_w[kAttnMaxQ];
#pragma unroll
  for (int j = 0; j < kAttnMaxQ; ++j) {
    if (j >= nq) break;
    float sc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float part = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          part = fmaf(acc[rt][ct][i], sm.q[j][32 * ct + 8 * (i >> 2) + 4 * half + (i & 3)], part);
      const float s = half_sum(part) * a.scale;
      sc[rt] = t0 + 32 * rt + r < T ? s : -INFINITY;
    }
    // 2. the wave's softmax statistics over its 64 tokens
    const float m = max32(fmaxf(sc[0], sc[1]));
    const bool none = m == -INFINITY;                  // every token of the wave past T
    float pe[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) pe[rt] = none ? 0.f : __expf(sc[rt] - m);
    m_w[j] = m;
    l_w[j] = sum32(pe[0] + pe[1]);
    if (half == 0) {
      sm.p[wave][j][r] = pe[0];
      sm.p[wave][j][32 + r] = pe[1];
    }
  }
  // (the barriers inside the next reconstruction order the p stores before their reads)
  // ---- 3. V^ (tokens as rows): lane = feature 32 ct + r of 16 tokens per tile
  reconstruct<true>(a.v, h, t0, T, sm, acc);
  // all waves are past the staging loop (its last barrier): the W area is free
  float* mrg = reinterpret_cast<float*>(&sm.wl[0][0][0]);      // [wave][j][D + 2]
#pragma unroll
  for (int j = 0; j < kAttnMaxQ; ++j) {
    if (j >= nq) break;
    float o[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      float part = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          part = fmaf(sm.p[wave][j][32 * rt + 8 * (i >> 2) + 4 * half + (i & 3)], acc[rt][ct][i], part);
      o[ct] = half_sum(part);
    }
    float* dst = mrg + (wave * kAttnMaxQ + j) * (D + 2);
    if (half == 0) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dst[32 * ct + r] = o[ct];
    }
    if (lane == 0) {
      dst[D] = m_w[j];
      dst[D + 1] = l_w[j];
    }
  }
  __syncthreads();
  // ---- 4. the block's partial: merge the 4 waves (in wave order)
  for (int i = threadIdx.x; i < nq * D; i += 256) {
    const int j = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[(w * kAttnMaxQ + j) * (D + 2) + D]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* src = mrg + (w * kAttnMaxQ + j) * (D + 2);
      const float f = src[D] == -INFINITY ? 0.f : __expf(src[D] - M);
      L = fmaf(src[D + 1], f, L);
      O = fmaf(src[d], f, O);
    }
    float* out = a.part + ((h * nq + j) * static_cast<int64_t>(a.n_blk) + blk) * (D + 2);
    out[d] = O;
    if (d == 0) {
      out[D] = M;
      out[D + 1] = L;
    }
  }
}

// out[hq][s][d] = sum_b o_b[d] e^{m_b - M} / sum_b l_b e^{m_b - M}, blocks in
// order; one workgroup of D threads per (KV head, query vector).
__global__ __launch_bounds__(128) void k_attn_merge(AttnArgs a) {
  const int64_t h = blockIdx.y;
  const int j = blockIdx.x, d = threadIdx.x;
  const float* p = a.part + (h * a.nq + j) * static_cast<int64_t>(a.n_blk) * (D + 2);
  float M = -INFINITY;
  for (int b = 0; b < a.n_blk; ++b) M = fmaxf(M, p[b * (D + 2) + D]);
  float L = 0.f, O = 0.f;
  for (int b = 0; b < a.n_blk; ++b) {
    const float mb = p[b * (D + 2) + D];
    const float f = mb == -INFINITY ? 0.f : __expf(mb - M);
    L = fmaf(p[b * (D + 2) + D + 1], f, L);
    O = fmaf(p[b * (D + 2) + d], f, O);
  }
  const int g = j / a.n_new, s = j % a.n_new;
  a.out[((h * a.G + g) * a.n_new + s) * D + d] = O / L;
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.nq < 1 || a.nq > kAttnMaxQ || a.T < 1 || a.H < 1) return hipErrorInvalidValue;
  if (a.n_blk != (a.T + kRows - 1) / kRows) return hipErrorInvalidValue;
  {
    ProfScope ps("attend", s);
    k_attn_decode<<<dim3(a.n_blk, a.H), 256, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  k_attn_merge<<<dim3(a.nq, a.H), D, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace jolt
