// Residual, rotation, group quantization and decode kernels (D = 128).
//
// JoLT abstract (arXiv 2607.12550v2), method sentence: after the partial
// Tucker truncation, the energy it drops is restored by the residual, rotated
// by a random orthogonal matrix and then quantized to few bits; news article
// paragraph 4: the rotation
// whitens the residual so the quantization error is close to independent and
// uniform.  Groups are 32 consecutive rotated features of one (head, token)
// row; each group stores a bf16 offset (min rounded toward -inf) and a bf16
// step ((max - offset) / (2^b - 1) rounded toward +inf), codes are
// rint((y - offset) / step) clamped to [0, 2^b - 1], all in IEEE fp32 with a
// correctly rounded divide, packed as a little-endian bit stream (code k at
// bits [k*b, (k+1)*b) of the group's 4b bytes).  One thread quantizes one
// group, so the group's reductions and its bit stream stay in registers.
#include "device.hpp"
#include "kernels.hpp"

namespace jolt {
namespace {

constexpr int D = 128;

// The group of 32 values y (one thread): scale word (offset | step << 16)
// and the B code words.
template <int B>
__device__ __forceinline__ void quantize_group(const float (&y)[32], bool store, uint32_t* scale_word,
                                               uint32_t* code_words) {
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int c = 1; c < 32; ++c) {
    mn = fminf(mn, y[c]);
    mx = fmaxf(mx, y[c]);
  }
  const uint16_t m16b = bf16_round_down(mn);
  const float m16 = bf16_bits_to_f32(m16b);
  const float L = static_cast<float>((1 << B) - 1);
  const uint16_t s16b = bf16_round_up(__fdiv_rn(mx - m16, L));
  const float s16 = bf16_bits_to_f32(s16b);
  uint32_t w[B];
#pragma unroll
  for (int k = 0; k < B; ++k) w[k] = 0u;
  if (s16 != 0.f) {
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const float t = fminf(fmaxf(rintf(__fdiv_rn(y[c] - m16, s16)), 0.f), L);
      const uint32_t code = static_cast<uint32_t>(t);
      const int pos = c * B, wi = pos >> 5, sh = pos & 31;
      w[wi] |= code << sh;
      if (sh + B > 32) w[wi + 1] |= code >> (32 - sh);
    }
  }
  if (!store) return;
  *scale_word = static_cast<uint32_t>(m16b) | (static_cast<uint32_t>(s16b) << 16);
  if constexpr (B == 4) {
    *reinterpret_cast<uint4*>(code_words) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (B == 2) {
    *reinterpret_cast<uint2*>(code_words) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int k = 0; k < B; ++k) code_words[k] = w[k];
  }
}

__device__ __forceinline__ void quantize_any(const float (&y)[32], int bits, bool store, uint32_t* scale_word,
                                             uint32_t* code_words) {
  switch (bits) {
    case 1: quantize_group<1>(y, store, scale_word, code_words); break;
    case 2: quantize_group<2>(y, store, scale_word, code_words); break;
    case 3: quantize_group<3>(y, store, scale_word, code_words); break;
    default: quantize_group<4>(y, store, scale_word, code_words); break;
  }
}

// Standalone quantizer: one group per thread.
__global__ __launch_bounds__(256) void k_quantize(const float* Y, int64_t ngroups, int bits, uint32_t* scales,
                                                  uint32_t* codes) {
  const int64_t g = blockIdx.x * 256ll + threadIdx.x;
  if (g >= ngroups) return;
  const float* src = Y + g * 32;
  float y[32];
  if ((reinterpret_cast<uintptr_t>(Y) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = reinterpret_cast<const float4*>(src)[q];
      y[4 * q] = v.x; y[4 * q + 1] = v.y; y[4 * q + 2] = v.z; y[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) y[c] = src[c];
  }
  quantize_any(y, bits, true, scales + g, codes + g * bits);
}

__device__ __forceinline__ bf16x8 load8_bf16(const uint16_t* base, int64_t idx, int64_t limit,
                                             bool aligned) {
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

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0));
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 raw) { return *reinterpret_cast<const bf16x8*>(&raw); }

// ------------------------------------------------------------------ encode
// Both products of the encoder run on bf16 matrix cores (32x32x16, fp32
// accumulate) over two-part splits of their fp32 operands: f = hi + lo + r
// with hi = rne_bf16(f), lo = rne_bf16(f - hi) and |r| <= 2^-18 |f|.  Every
// product of two bf16 values is exact in fp32; the reconstruction U~_T (hi +
// lo) of exact bf16 U~_T and the rotation's hi hi + hi lo + lo hi leave out
// terms below 2^-17 relative per product (lo lo and the remainders r), and
// the fp32 accumulation keeps the large hi x hi terms in an accumulator of
// their own and adds the small ones in a second.  That error is some 10^4
// times below the quantization step the residual then takes.

__device__ __forceinline__ uint16_t rne_bits(float f) {   // finite f
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ void split2(float f, uint16_t& h, uint16_t& l) {
  h = rne_bits(f);
  l = rne_bits(f - bf16_bits_to_f32(h));           // the difference is exact
}

// W_h = G~_h U~_D^T in two bf16 parts, stored in matrix-core fragment
// order: W2[p][h][cb][ks][lane][e] (cb < 4 blocks of 32 features, ks < r_Tp/16
// steps of 16 values of k, lane = 32 half + r) holds part p of W_h[k][d] for
// d = 32 cb + r, k = 16 ks + 8 half + e, so the B operand of one k step of one
// wave is 1 KB of consecutive bytes; k >= r_T is zero, r_Tp a multiple of 64
// (whole staged chunks of U~_T in the encoder).
// One wave per (tensor, head, 32 values of k), K = r_D in steps of 16 on bf16
// matrix cores (the factors are bf16, so the products are exact and only the
// fp32 sum rounds).  Tensor j of a launch reads G~_h from Gp[j H + h] and
// U~_D from Udp[j H + h] (or G0 + h r_T r_D and Ud0 when Gp is null) and
// writes W2 + j w2_batch.
__global__ __launch_bounds__(64) void k_enc_w(const uint16_t* const* Gp, const uint16_t* const* Udp,
                                              const uint16_t* G0, const uint16_t* Ud0, uint16_t* W2,
                                              int64_t w2_batch, int H, int r_T, int r_D, int r_Tp) {
  const int lane = threadIdx.x, r = lane & 31, half = lane >> 5;
  const int k0 = blockIdx.x * 32, h = blockIdx.y, j = blockIdx.z;
  const uint16_t* G = Gp ? Gp[static_cast<int64_t>(j) * H + h] : G0 + static_cast<int64_t>(h) * r_T * r_D;
  const uint16_t* Ud = Udp ? Udp[static_cast<int64_t>(j) * H + h] : Ud0;
  uint16_t* out = W2 + j * w2_batch;
  const bool ga = (r_D % 8) == 0 && (reinterpret_cast<uintptr_t>(G) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(Ud) & 15) == 0;
  const int k = k0 + r;
  f32x16 acc[4] = {};
  for (int j0 = 0; j0 < r_D; j0 += 16) {
    const int jj = j0 + 8 * half;
    const bf16x8 b = k < r_T ? load8_bf16(G + static_cast<int64_t>(k) * r_D, jj, r_D, ga) : zero8();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 a = load8_bf16(Ud + static_cast<int64_t>(32 * ct + r) * r_D, jj, r_D, ga);
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[ct], 0, 0, 0);
    }
  }
  const int64_t part = static_cast<int64_t>(H) * D * r_Tp;
  const int KS = r_Tp / 16, ks = k >> 4, fl = ((k >> 3) & 1) * 32, e = k & 7;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int64_t fb = ((static_cast<int64_t>(h) * 4 + ct) * KS + ks) * 512 + e;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dr = (i >> 2) * 8 + half * 4 + (i & 3);     // feature 32 ct + dr
      uint16_t hb, lb;
      split2(acc[ct][i], hb, lb);
      const int64_t off = fb + (fl + dr) * 8;
      out[off] = hb;
      out[part + off] = lb;
    }
  }
}

// One workgroup (4 waves) per 64-row tile of one head.
//  1. recon = U~_T[t0 .. t0+64) W_h: wave w computes features [32w, 32w+32)
//     of both 32-row blocks.  U~_T is staged in LDS in chunks of 64 values
//     of k (whole 128-byte rows of the chunk, double-buffered, shared by the
//     waves); the two W parts stream from memory in fragment order, two k
//     steps ahead; hi in one accumulator, lo in another.
//  2. recon is staged in LDS; thread (m, g) = (tid / 4, tid % 4) takes its
//     32 features of group g of row m, forms R = X - recon and stores R's
//     two bf16 parts in LDS as [part][row][feature].
//  3. Y = R Q^T with A = the R parts from LDS and B = the first two Q parts
//     (bf16, in fragment order like W, in cache), three products per step
//     (hi hi, hi lo, lo hi).
//  4. Y is staged in LDS and thread (m, g) quantizes group g of row m.
constexpr int ER = 64;                         // rows per workgroup
constexpr int EYS = 144;                       // fp32 row stride of staged recon / Y (group g at 36 g)
constexpr int ERS = 136;                       // bf16 row stride of the staged R parts
constexpr int kEncLds = ER * EYS * 4;          // 36864 bytes: staged recon / Y
constexpr int EUC = 64;                        // k per staged U~_T chunk
constexpr int EUS = EUC + 8;                   // bf16 row stride of a staged U~_T chunk
static_assert(2 * ER * EUS * 2 <= kEncLds, "U~_T chunks fit the staging area");
static_assert(2 * ER * ERS * 2 <= kEncLds, "the R parts fit the staging area");

// UV: rows of U~_T are 16-byte aligned (r_T % 8 == 0 and an aligned base), so
// a chunk is read with 16-byte loads; otherwise element by element.
template <typename TX, bool UV>
__device__ __forceinline__ void encode_tile(const EncodeArgs& a, float* lds_f, uint32_t tile, uint32_t head) {
  float* st = lds_f;                                          // recon, then Y
  uint16_t* rp = reinterpret_cast<uint16_t*>(lds_f);          // R parts
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, half = lane >> 5;
  const int64_t h = head, t0 = static_cast<int64_t>(tile) * ER;
  const int col = wave * 32 + rl;
  const int qm = tid >> 2, qg = tid & 3;
  const int64_t qt = t0 + qm;
  const bool qvalid = qt < a.T;
  // 1. reconstruction
  f32x16 hi0 = {}, hi1 = {}, lo0 = {}, lo1 = {};
  if (a.r_T > 0) {
    const int64_t rT = a.r_T;
    const int KS = static_cast<int>(a.r_Tp / 16);
    const int64_t part = a.H * D * a.r_Tp;
    const uint16_t* wb = a.W2 + ((h * 4 + wave) * KS) * 512 + lane * 8;
    // U~_T chunk loader: row ur = tid / 4, k = 16 (tid % 4) .. +16 of the chunk
    const int ur = tid >> 2, uk = 16 * (tid & 3);
    const int64_t ut = t0 + ur;
    const bool urv = ut < a.T;
    const uint16_t* urow = a.Ut + (urv ? ut : 0) * rT;      // rows past T read row 0, then zero
    uint4 ru[2];
    bool uok[2];
    // branch-free: out-of-range loads read a valid address and are zeroed by a
    // select when stored (so the loads stay in flight until then)
    auto load_u = [&](int64_t k0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t k = k0 + uk + 8 * q;
        if constexpr (UV) {
          uok[q] = urv && k < rT;
          ru[q] = ldg16(urow + (uok[q] ? k : 0));
        } else {
          uok[q] = true;
          uint32_t v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool ok = urv && k + e < rT;
            const uint32_t b = ldg_u16(urow + (ok ? k + e : 0));
            v[e] = ok ? b : 0u;
          }
          ru[q] = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
        }
      }
    };
    auto store_u = [&](int buf) {
      uint16_t* dst = rp + (buf * ER + ur) * EUS + uk;
#pragma unroll
      for (int q = 0; q < 2; ++q) {     // a mask per word (a select of uint4 values goes through memory)
        const uint32_t m = uok[q] ? ~0u : 0u;
        *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(ru[q].x & m, ru[q].y & m, ru[q].z & m, ru[q].w & m);
      }
    };
    const int nks = KS;                            // a multiple of 4 (r_Tp of the encoder: 64 k)
    // W fragments in a ring of four k steps, loaded two steps ahead (a slot
    // is refilled only after its step's products are issued)
    uint4 wf[4][2];
    auto load_w = [&](int slot, int ks) {         // steps past the end reload the last one (unused)
      const uint16_t* src = wb + static_cast<int64_t>(ks < nks ? ks : nks - 1) * 512;
      wf[slot][0] = ldg16(src);
      wf[slot][1] = ldg16(src + part);
    };
    load_u(0);
    load_w(0, 0);
    load_w(1, 1);
    store_u(0);
    __syncthreads();
    for (int c0 = 0; c0 < nks; c0 += EUC / 16) {   // every chunk holds EUC / 16 whole k steps
      const int buf = (c0 / (EUC / 16)) & 1;
      const bool more = c0 + EUC / 16 < nks;
      if (more) load_u(static_cast<int64_t>(c0) * 16 + EUC);
      const uint16_t* ua = rp + (buf * ER + rl) * EUS + 8 * half;
#pragma unroll
      for (int s4 = 0; s4 < EUC / 16; ++s4) {
        const int ks = c0 + s4;
        {                                             // ks % 4 == s4: chunks start at multiples of 4
          const bf16x8 bh = as_bf16x8(wf[s4][0]), bl = as_bf16x8(wf[s4][1]);
          load_w((s4 + 2) & 3, ks + 2);
          const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const uint4*>(ua + 16 * s4));
          const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const uint4*>(ua + 32 * EUS + 16 * s4));
          hi0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bh, hi0, 0, 0, 0);
          hi1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bh, hi1, 0, 0, 0);
          lo0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bl, lo0, 0, 0, 0);
          lo1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bl, lo1, 0, 0, 0);
        }
      }
      if (more) store_u(buf ^ 1);
      __syncthreads();
    }
  }
  // this thread's 32 X values (row qt, features 32 qg ..)
  float x[32];
  {
    // rows past T read row 0 and are zeroed below (no divergent loads)
    const int64_t base = (h * a.T + (qvalid ? qt : 0)) * D + 32 * qg;
    const TX* src = static_cast<const TX*>(a.X) + base;
    const bool xv = (reinterpret_cast<uintptr_t>(a.X) & 15) == 0;
    if constexpr (sizeof(TX) == 2) {
      if (xv) {
        uint4 raw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) raw[q] = ldg16(src + 8 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wv[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[8 * q + 2 * e] = __uint_as_float(wv[e] << 16);
            x[8 * q + 2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) x[c] = bf16_bits_to_f32(ldg_u16(src + c));
      }
    } else {
      if (xv) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint4 v = ldg16(src + 4 * q);
          x[4 * q] = __uint_as_float(v.x); x[4 * q + 1] = __uint_as_float(v.y);
          x[4 * q + 2] = __uint_as_float(v.z); x[4 * q + 3] = __uint_as_float(v.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) x[c] = __uint_as_float(ldg32(src + c));
      }
    }
  }
  if (!qvalid) {
#pragma unroll
    for (int c = 0; c < 32; ++c) x[c] = 0.f;
  }
  if (a.r_T > 0) {
    // 2. stage recon; thread (m, g) forms its part of R
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = (i >> 2) * 8 + half * 4 + (i & 3);
      st[m * EYS + wave * 36 + rl] = hi0[i] + lo0[i];
      st[(32 + m) * EYS + wave * 36 + rl] = hi1[i] + lo1[i];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(st + qm * EYS + qg * 36 + 4 * q);
      x[4 * q] -= v.x; x[4 * q + 1] -= v.y; x[4 * q + 2] -= v.z; x[4 * q + 3] -= v.w;
    }
    __syncthreads();                              // the R parts overwrite the staged recon
  }
  {
    uint32_t wh[16], wl[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      uint16_t h0, l0, h1, l1;
      split2(x[2 * e], h0, l0);
      split2(x[2 * e + 1], h1, l1);
      wh[e] = h0 | (static_cast<uint32_t>(h1) << 16);
      wl[e] = l0 | (static_cast<uint32_t>(l1) << 16);
    }
    uint16_t* row = rp + qm * ERS + 32 * qg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint4*>(row + 8 * q) = make_uint4(wh[4 * q], wh[4 * q + 1], wh[4 * q + 2], wh[4 * q + 3]);
      *reinterpret_cast<uint4*>(row + ER * ERS + 8 * q) =
          make_uint4(wl[4 * q], wl[4 * q + 1], wl[4 * q + 2], wl[4 * q + 3]);
    }
  }
  __syncthreads();
  // 3. rotation
  f32x16 yh0 = {}, yh1 = {}, yl0 = {}, yl1 = {};
  {
    // Q parts in fragment order: [p][cb][ds][lane][e] = part p of Q[32 cb + r][16 ds + 8 half + e]
    const uint16_t* qb = a.Q3 + wave * (D / 16) * 512 + lane * 8;
    uint4 qf[4][2];                               // ring of four d steps, two ahead
    auto load_q = [&](int slot, int ds) {
      if (ds < D / 16) {
        const uint16_t* src = qb + ds * 512;
        qf[slot][0] = ldg16(src);
        qf[slot][1] = ldg16(src + D * D);
      }
    };
    load_q(0, 0);
    load_q(1, 1);
    const uint16_t* ra = rp + rl * ERS + 8 * half;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const int d0 = 16 * ds, slot = ds & 3;
      const bf16x8 qh = as_bf16x8(qf[slot][0]), ql = as_bf16x8(qf[slot][1]);
      load_q((ds + 2) & 3, ds + 2);
      const bf16x8 h0 = as_bf16x8(*reinterpret_cast<const uint4*>(ra + d0));
      const bf16x8 h1 = as_bf16x8(*reinterpret_cast<const uint4*>(ra + 32 * ERS + d0));
      const bf16x8 l0 = as_bf16x8(*reinterpret_cast<const uint4*>(ra + ER * ERS + d0));
      const bf16x8 l1 = as_bf16x8(*reinterpret_cast<const uint4*>(ra + (ER + 32) * ERS + d0));
      yh0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h0, qh, yh0, 0, 0, 0);
      yh1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h1, qh, yh1, 0, 0, 0);
      yl0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h0, ql, yl0, 0, 0, 0);
      yl1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h1, ql, yl1, 0, 0, 0);
      yl0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l0, qh, yl0, 0, 0, 0);
      yl1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l1, qh, yl1, 0, 0, 0);
    }
  }
  __syncthreads();                                // Y overwrites the R parts
  // 4. stage Y; thread (m, g) quantizes group g of row m
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = (i >> 2) * 8 + half * 4 + (i & 3);
    st[m * EYS + wave * 36 + rl] = yh0[i] + yl0[i];
    st[(32 + m) * EYS + wave * 36 + rl] = yh1[i] + yl1[i];
  }
  __syncthreads();
  float y[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(st + qm * EYS + qg * 36 + 4 * q);
    y[4 * q] = v.x; y[4 * q + 1] = v.y; y[4 * q + 2] = v.z; y[4 * q + 3] = v.w;
  }
  const int64_t gi = (h * a.T + qt) * 4 + qg;
  quantize_any(y, a.bits, qvalid, reinterpret_cast<uint32_t*>(a.scales) + gi,
               reinterpret_cast<uint32_t*>(a.codes) + gi * a.bits);
}

template <typename TX>
__device__ __forceinline__ void encode_any(const EncodeArgs& a, uint32_t tile, uint32_t head) {
  __shared__ __attribute__((aligned(16))) float lds_f[kEncLds / 4];
  if (a.r_T % 8 == 0 && (reinterpret_cast<uintptr_t>(a.Ut) & 15) == 0) encode_tile<TX, true>(a, lds_f, tile, head);
  else encode_tile<TX, false>(a, lds_f, tile, head);
}
template <typename TX>
__global__ __launch_bounds__(256, 4) void k_encode_residual(EncodeArgs a) {
  uint32_t tile, head;
  xcd_group_2d(tile, head);                        // the row tiles of one head on one XCD
  encode_any<TX>(a, tile, head);
}
// Tensors of one shape in one launch: grid (row tiles, heads, tensors); all
// the tiles of one tensor run on one XCD, whose L2 then holds the tensor's W
// parts and U~_T rows (each used by many tiles).
template <typename TX>
__global__ __launch_bounds__(256, 4) void k_encode_residual_many(const EncodeArgs* list) {
  uint32_t tensor, idx;
  xcd_group(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gridDim.x * gridDim.y, gridDim.z, tensor,
            idx);
  const EncodeArgs a = list[tensor];
  encode_any<TX>(a, idx % gridDim.x, idx / gridDim.x);
}

// ------------------------------------------------------------------ decode
// bf16 matrix cores (32x32x16, fp32 accumulate).  Stored factors and core are
// bf16, so U~_T x W is exact per product once W = G~_h U~_D^T is carried as a
// hi + lo pair of bf16 (relative error 2^-17); the dequantized residual and Q
// enter in bf16 (relative 2^-9 each, far below the quantization error they
// ride on).  Every MFMA operand is one 16-byte load per lane: lane l holds
// row l%32 and k = 8*(l/32) .. +8 of A, column l%32 and the same k of B.

// W_h = G~_h U~_D^T as bf16 hi + lo planes in matrix-core fragment order,
// [h][d / 32][k / 16][32 ((k / 8) % 2) + d % 32][k % 8] (k < r_Tp, r_Tp a
// multiple of 32), so that one k step of one column tile is 1 KB of
// consecutive bytes for the decoding wave.  One wave per (record, head, 32
// rows of r_T).
__global__ __launch_bounds__(256) void k_make_w(DecBatch b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= b.wtiles_total) return;
  // the record holding this tile: the last with first tile <= tile (records
  // are in order, so a binary search)
  int ri = 0;
  for (int hi = b.n - 1; ri < hi;) {
    const int mid = (ri + hi + 1) >> 1;
    if (b.rec[mid].wtile0 <= tile) ri = mid;
    else hi = mid - 1;
  }
  const DecRec& R = b.rec[ri];
  const int local = tile - R.wtile0;
  const int ktiles = R.r_Tp / 32;
  const int h = local / ktiles, k0 = (local % ktiles) * 32;
  const int r = lane & 31, half = lane >> 5;
  f32x16 acc[4] = {};
  const int k = k0 + r;
  const bool arow = k < R.r_T;
  const bool ga = (R.r_D % 8) == 0;
  for (int j0 = 0; j0 < R.r_D; j0 += 16) {
    const int jj = j0 + 8 * half;
    const bf16x8 a = arow ? load8_bf16(R.G() + (static_cast<int64_t>(h) * R.r_T + k) * R.r_D, jj, R.r_D, ga)
                          : zero8();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bb = load8_bf16(R.Ud() + static_cast<int64_t>(32 * ct + r) * R.r_D, jj, R.r_D, ga);
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[ct], 0, 0, 0);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = (i >> 2) * 8 + half * 4 + (i & 3);   // k = k0 + m, feature 32 ct + r
      const float w = acc[ct][i];
      const uint16_t hi = f32_to_bf16_rne(w);
      const uint16_t lo = f32_to_bf16_rne(w - bf16_bits_to_f32(hi));
      const int k = k0 + m;
      const int64_t off = ((static_cast<int64_t>(h) * 4 + ct) * (R.r_Tp / 16) + (k >> 4)) * 512 +
                          (((k >> 3) & 1) * 32 + r) * 8 + (k & 7);
      R.Whi[off] = hi;
      R.Wlo()[off] = lo;
    }
  }
}

// One wave per (record, head, 64 rows): X^ rows = U~_T W (hi + lo) + Yhat Q,
// computed transposed (features as the product's rows, tokens as its
// columns) so that each lane ends with runs of 4 consecutive features of one
// token; a swap of the wave's halves makes them runs of 8, stored 16 bytes at
// a time.
template <typename TO>
__global__ __launch_bounds__(256, 2) void k_decode(DecBatch b) {
  // two k steps of W (hi, lo planes, 4 column tiles) per buffer,
  // [step][plane][ct][lane][8]
  __shared__ __align__(16) uint16_t wl[2][2][2 * 4 * 64 * 8];
  // Q^T bf16 in fragment order [ct][d / 16][lane][8], read by every wave
  __shared__ __align__(16) uint16_t ql[4 * 8 * 64 * 8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // a block = 256 rows (4 waves of 64) of one (record, head); the blocks of
  // one (record, head) share its W and run on one XCD
  uint32_t xb = blockIdx.x, grp = blockIdx.y;
  xcd_group_2d(xb, grp);
  const DecRec& R = b.rec[grp / b.H];
  const int64_t h = grp % b.H, t0 = static_cast<int64_t>(xb) * 256 + 64 * wave;
  const int r = lane & 31, half = lane >> 5;
  f32x16 acc[2][4] = {};
  const bool ua = (R.r_T % 8) == 0;
  // a stage = two k steps (32 of r_T; r_Tp is a multiple of 32): U~_T rows
  // streamed from memory and W staged through LDS, both one stage ahead of
  // the MFMAs; each thread moves the hi and lo 16 bytes of (column tile = its
  // wave, its lane) of both steps
  bf16x8 a[2][2];   // [step][rt]
  auto load_k = [&](int st) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kk = 32 * st + 16 * sub + 8 * half;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int64_t t = t0 + 32 * rt + r;
        a[sub][rt] = t < b.T ? load8_bf16(R.Ut() + t * R.r_T, kk, R.r_T, ua) : zero8();
      }
    }
  };
  const int nks = R.r_Tp / 16, nst = nks / 2;
  uint4 wh[2], wlo[2];
  auto load_w = [&](int st) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int64_t o = ((h * 4 + wave) * nks + 2 * st + sub) * 512 + lane * 8;   // fragment order
      wh[sub] = ldg16(R.Whi + o);
      wlo[sub] = ldg16(R.Wlo() + o);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      *reinterpret_cast<uint4*>(&wl[buf][sub][(wave * 64 + lane) * 8]) = wh[sub];
      *reinterpret_cast<uint4*>(&wl[buf][sub][((4 + wave) * 64 + lane) * 8]) = wlo[sub];
    }
  };
  // thread i moves the 16-byte fragments i + 256 j of Q^T
  uint4 qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = threadIdx.x + 256 * j, l = c & 63;
    qv[j] = ldg16(b.Qt16 + (32 * (c >> 9) + (l & 31)) * D + 16 * ((c >> 6) & 7) + 8 * (l >> 5));
  }
  if (nst > 0) {
    load_w(0);
    load_k(0);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(&ql[(threadIdx.x + 256 * j) * 8]) = qv[j];
  if (nst > 0) store_w(0);
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
      bf16x8 ch[4], cl[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        ch[ct] = *reinterpret_cast<const bf16x8*>(&wl[buf][sub][(ct * 64 + lane) * 8]);
        cl[ct] = *reinterpret_cast<const bf16x8*>(&wl[buf][sub][((4 + ct) * 64 + lane) * 8]);
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch[ct], ca[sub][rt], acc[rt][ct], 0, 0, 0);
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cl[ct], ca[sub][rt], acc[rt][ct], 0, 0, 0);
        }
      }
    }
    // the other buffer was last read in the previous stage, before its barrier
    if (st + 1 < nst) store_w(buf ^ 1);
    __syncthreads();
  }
  const int bits = R.bits;
  // the streamed words of one d step (scales, code words), the next step's
  // loaded during this one's dequantization and MFMAs (Q^T from LDS)
  uint32_t sw[2], w0[2], w1[2];
  auto load_d = [&](int d0) {
    const int dd = d0 + 8 * half;               // this lane's 8 features
    const int g = dd >> 5, bitpos = (dd & 31) * bits;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t t = t0 + 32 * rt + r;
      sw[rt] = 0u; w0[rt] = 0u; w1[rt] = 0u;
      if (t < b.T) {
        const int64_t gi = (h * b.T + t) * 4 + g;
        sw[rt] = ldg32(R.scales() + gi);
        const uint32_t* cw = R.codes() + gi * bits;
        w0[rt] = ldg32(cw + (bitpos >> 5));
        if ((bitpos & 31) + 8 * bits > 32) w1[rt] = ldg32(cw + (bitpos >> 5) + 1);
      }
    }
  };
  load_d(0);
  for (int d0 = 0; d0 < D; d0 += 16) {
    const int dd = d0 + 8 * half;
    const int bitpos = (dd & 31) * bits;
    const uint32_t csw[2] = {sw[0], sw[1]}, cw0[2] = {w0[0], w0[1]}, cw1[2] = {w1[0], w1[1]};
    uint4 cq[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) cq[ct] = *reinterpret_cast<const uint4*>(&ql[((ct * 8 + (d0 >> 4)) * 64 + lane) * 8]);
    if (d0 + 16 < D) load_d(d0 + 16);
    bf16x8 y[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      y[rt] = dequant8<bf16x8>(csw[rt], cw0[rt], cw1[rt], static_cast<uint32_t>(bitpos & 31),
                               static_cast<uint32_t>(bits));
    // rows past T: scale word 0 gives m16 = s16 = 0, so y = 0
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&cq[ct]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq, y[rt], acc[rt][ct], 0, 0, 0);
    }
  }
  // acc[rt][ct][i] is feature 32 ct + 8 (i / 4) + 4 half + i % 4 of token
  // t0 + 32 rt + r
  TO* out = static_cast<TO*>(R.out);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t t = t0 + 32 * rt + r;
    if (t >= b.T) continue;
    TO* orow = out + (h * b.T + t) * D;
    if (!b.out16) {   // an output not 16-byte aligned: one element per store
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * ct + 8 * (i >> 2) + 4 * half + (i & 3);
          if constexpr (sizeof(TO) == 2) orow[c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[rt][ct][i]));
          else orow[c] = acc[rt][ct][i];
        }
      continue;
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if constexpr (sizeof(TO) == 2) {
        // groups 2j and 2j + 1 of 8 features: the lower half gathers group 2j
        // (its own 4 + the upper half's 4), the upper half group 2j + 1
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t p[2][2];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const int i = (2 * j + g) * 4 + 2 * w;
              p[g][w] = pack_bf16x2(acc[rt][ct][i], acc[rt][ct][i + 1]);
            }
          const auto s0 = __builtin_amdgcn_permlane32_swap(p[0][0], p[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(p[0][1], p[1][1], false, false);
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          stg16(orow + 32 * ct + 8 * (2 * j + half), v);
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 v = {__float_as_uint(acc[rt][ct][4 * g]), __float_as_uint(acc[rt][ct][4 * g + 1]),
                           __float_as_uint(acc[rt][ct][4 * g + 2]), __float_as_uint(acc[rt][ct][4 * g + 3])};
          stg16(orow + 32 * ct + 8 * g + 4 * half, v);
        }
      }
    }
  }
}


}  // namespace

hipError_t launch_quantize(const float* Y, int64_t rows, int bits, uint16_t* scales, uint8_t* codes,
                           hipStream_t s) {
  const int64_t ng = rows * (D / 32);
  if (ng == 0) return hipSuccess;
  ProfScope ps("quantize", s);
  k_quantize<<<(ng + 255) / 256, 256, 0, s>>>(Y, ng, bits, reinterpret_cast<uint32_t*>(scales),
                                              reinterpret_cast<uint32_t*>(codes));
  return hipGetLastError();
}

hipError_t launch_enc_w(const uint16_t* const* Gp, const uint16_t* const* Udp, const uint16_t* G0,
                        const uint16_t* Ud0, uint16_t* W2, int64_t w2_batch, int n, int H, int r_T, int r_D,
                        int r_Tp, hipStream_t s) {
  if (n <= 0 || r_T <= 0) return hipSuccess;
  if (r_Tp % 64 != 0 || r_Tp < r_T) return hipErrorInvalidValue;
  ProfScope ps("encode_w", s);
  k_enc_w<<<dim3(r_Tp / 32, H, n), 64, 0, s>>>(Gp, Udp, G0, Ud0, W2, w2_batch, H, r_T, r_D, r_Tp);
  return hipGetLastError();
}

hipError_t launch_encode_residual(const EncodeArgs& a, hipStream_t s) {
  dim3 grid((a.T + ER - 1) / ER, a.H);
  ProfScope ps("encode_residual", s);
  if (a.x_dtype == kBF16) k_encode_residual<uint16_t><<<grid, 256, 0, s>>>(a);
  else k_encode_residual<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_encode_residual_many(const EncodeArgs* list_dev, int n, int64_t H, int64_t T, int x_dtype,
                                       hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((T + ER - 1) / ER, H, n);
  ProfScope ps("encode_residual", s);
  if (x_dtype == kBF16) k_encode_residual_many<uint16_t><<<grid, 256, 0, s>>>(list_dev);
  else k_encode_residual_many<float><<<grid, 256, 0, s>>>(list_dev);
  return hipGetLastError();
}

hipError_t launch_make_w(const DecBatch& b, hipStream_t s) {
  if (b.wtiles_total <= 0) return hipSuccess;
  ProfScope ps("decode_w", s);
  k_make_w<<<(b.wtiles_total + 3) / 4, 256, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_decode_batch(const DecBatch& b, hipStream_t s) {
  {
    const hipError_t e = launch_make_w(b, s);
    if (e != hipSuccess) return e;
  }
  ProfScope ps("decode", s);
  const dim3 grid((b.T + 255) / 256, b.n * b.H);
  if (b.out_dtype == kBF16) k_decode<uint16_t><<<grid, 256, 0, s>>>(b);
  else k_decode<float><<<grid, 256, 0, s>>>(b);
  return hipGetLastError();
}

// One workgroup of 64 threads per record: words 0..63 of the head (header,
// then zeros), then the section paddings, one byte per thread.
__device__ __forceinline__ void write_head(uint32_t* blob, const RecordHead& h) {
  const int t = threadIdx.x;
  blob[t] = t < 16 ? h.w[t] : 0u;
  uint8_t* b = reinterpret_cast<uint8_t*>(blob);
#pragma unroll
  for (int j = 0; j < 5; ++j)
    for (uint32_t k = t; k < h.pad[2 * j + 1]; k += 64) b[h.pad[2 * j] + k] = 0;
}
__global__ __launch_bounds__(64) void k_header_many(uint32_t* const* blobs, const RecordHead* heads) {
  write_head(blobs[blockIdx.x], heads[blockIdx.x]);
}
__global__ __launch_bounds__(64) void k_header(uint32_t* blob, RecordHead head) { write_head(blob, head); }

hipError_t launch_write_headers(uint32_t* const* blobs_dev, const RecordHead* heads_dev, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_header_many<<<n, 64, 0, s>>>(blobs_dev, heads_dev);
  return hipGetLastError();
}
hipError_t launch_write_header(void* blob, const RecordHead& head, hipStream_t s) {
  k_header<<<1, 64, 0, s>>>(static_cast<uint32_t*>(blob), head);
  return hipGetLastError();
}

}  // namespace jolt
