// Residual, rotation, group quantization and decode kernels (D = 128).
//
// JoLT abstract (arXiv 2607.12550v2), method sentence: after the partial
// Tucker truncation the residual is restored by "a random orthogonal rotation
// followed by low-bit quantization"; news article paragraph 4: the rotation
// whitens the residual so the quantization error is close to independent and
// uniform.  Groups are 32 consecutive rotated features of one (head, token)
// row; each group stores a bf16 offset (min rounded toward -inf) and a bf16
// step ((max - offset) / (2^b - 1) rounded toward +inf), codes are
// rint((y - offset) / step) clamped to [0, 2^b - 1], all in IEEE fp32 with a
// correctly rounded divide, packed as a little-endian bit stream (code k at
// bits [k*b, (k+1)*b) of the group's 4b bytes).
//
// Layout of one workgroup (256 threads, 4 waves) over a 32-row tile: wave w
// owns features [32w, 32w + 32) = quantization group w.  In the 32x32 fp32
// matrix-core accumulator, register i of lane l holds row
// (i/4)*8 + (l/32)*4 + i%4 and column l%32, so one register across a
// half-wave is exactly one group: min/max are 5 xor-shuffles and the bit
// stream is assembled from ballots.
#include "device.hpp"
#include "kernels.hpp"

namespace jolt {
namespace {

constexpr int D = 128;
constexpr int TM = 32;        // rows per tile
constexpr int KC = 64;        // K chunk of the reconstruction product

__device__ __forceinline__ float half_min(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Quantize the group held by this half-wave (one value per lane) and write
// its (offset, step) pair and 4*bits code bytes.  Every lane of the wave must
// call it (ballots); `valid` masks rows past the tensor end.
__device__ __forceinline__ void quantize_group(float y, int bits, bool valid, uint32_t* scale_word,
                                               uint32_t* code_words) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const float mn = half_min(y), mx = half_max(y);
  const uint16_t m16b = bf16_round_down(mn);
  const float m16 = bf16_bits_to_f32(m16b);
  const float L = static_cast<float>((1 << bits) - 1);
  const float s32 = __fdiv_rn(mx - m16, L);
  const uint16_t s16b = bf16_round_up(s32);
  const float s16 = bf16_bits_to_f32(s16b);
  uint32_t code = 0;
  if (s16 != 0.f) {
    float t = rintf(__fdiv_rn(y - m16, s16));
    t = fminf(fmaxf(t, 0.f), L);
    code = static_cast<uint32_t>(t);
  }
  uint32_t mask[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned long long b = __ballot(j < bits ? ((code >> j) & 1u) : 0u);
    mask[j] = static_cast<uint32_t>(b >> (32 * half));
  }
  if (!valid) return;
  if (k == 0) *scale_word = static_cast<uint32_t>(m16b) | (static_cast<uint32_t>(s16b) << 16);
  if (k < bits) {
    // word k holds stream bits 32k .. 32k+31; stream bit s = bit (s % bits) of code s / bits
    uint32_t w = 0;
    for (int i = 0; i < 32; ++i) {
      const int s = 32 * k + i;
      const int cidx = s / bits, bj = s - cidx * bits;
      w |= ((mask[bj] >> cidx) & 1u) << i;
    }
    code_words[k] = w;
  }
}

// Standalone quantizer: one group per half-wave, 8 groups per workgroup.
__global__ __launch_bounds__(256) void k_quantize(const float* Y, int64_t ngroups, int bits,
                                                  uint32_t* scales, uint32_t* codes) {
  const int64_t g = blockIdx.x * 8ll + (threadIdx.x >> 5);
  const bool valid = g < ngroups;
  const float y = valid ? Y[g * 32 + (threadIdx.x & 31)] : 0.f;
  quantize_group(y, bits, valid, scales + g, codes + g * bits);
}

template <typename TX>
__device__ __forceinline__ float load_x(const void* X, int64_t i) {
  return load_as_f32<TX>(static_cast<const TX*>(X), i);
}

// acc += Ut[t0 .. t0+32)[0 .. r_T) * W[0 .. r_T)[32w .. 32w+32), fp32 matrix cores.
__device__ __forceinline__ void recon_tile(f32x16& acc, const uint16_t* Ut, const float* W, int64_t r_T,
                                           int64_t T, int64_t t0, float (*Us)[TM + 1]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t k0 = 0; k0 < r_T; k0 += KC) {
    __syncthreads();
    for (int idx = tid; idx < KC * TM; idx += 256) {
      const int m = idx / KC, kk = idx % KC;
      const int64_t t = t0 + m, k = k0 + kk;
      Us[kk][m] = (t < T && k < r_T) ? bf16_bits_to_f32(Ut[t * r_T + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; kk += 2) {
      const int kr = kk + (lane >> 5);
      const int64_t k = k0 + kr;
      const float a = Us[kr][lane & 31];
      const float b = k < r_T ? W[k * D + wave * 32 + (lane & 31)] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
  }
}

template <typename TX>
__global__ __launch_bounds__(256) void k_encode_residual(EncodeArgs a) {
  __shared__ float Us[KC][TM + 1];
  __shared__ float Rs[TM][D + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t h = blockIdx.y, t0 = static_cast<int64_t>(blockIdx.x) * TM;
  f32x16 acc = {};
  if (a.r_T > 0) recon_tile(acc, a.Ut, a.W + h * a.r_T * D, a.r_T, a.T, t0, Us);
  // residual R = X - recon, staged in LDS as [row][feature]
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    const int c = wave * 32 + (lane & 31);
    const int64_t t = t0 + m;
    const float x = t < a.T ? load_x<TX>(a.X, (h * a.T + t) * D + c) : 0.f;
    Rs[m][c] = x - acc[i];
  }
  __syncthreads();
  // Y = R Q^T: Y[m][c] = sum_d R[m][d] Q[c][d] = sum_d R[m][d] Qt[d][c]
  f32x16 y = {};
#pragma unroll 8
  for (int kk = 0; kk < D; kk += 2) {
    const int d = kk + (lane >> 5);
    y = __builtin_amdgcn_mfma_f32_32x32x2f32(Rs[lane & 31][d], a.Qt[d * D + wave * 32 + (lane & 31)], y,
                                             0, 0, 0);
  }
  uint32_t* sc = reinterpret_cast<uint32_t*>(a.scales);
  uint32_t* cd = reinterpret_cast<uint32_t*>(a.codes);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    const int64_t t = t0 + m;
    const int64_t g = (h * a.T + t) * 4 + wave;          // group index
    quantize_group(y[i], a.bits, t < a.T, sc + g, cd + g * a.bits);
  }
}

// ------------------------------------------------------------------ decode
// bf16 matrix cores (32x32x16, fp32 accumulate).  Stored factors and core are
// bf16, so U~_T x W is exact per product once W = G~_h U~_D^T is carried as a
// hi + lo pair of bf16 (relative error 2^-17); the dequantized residual and Q
// enter in bf16 (relative 2^-9 each, far below the quantization error they
// ride on).  Every MFMA operand is one 16-byte load per lane: lane l holds
// row l%32 and k = 8*(l/32) .. +8 of A, column l%32 and the same k of B.

__device__ __forceinline__ bf16x8 load8_bf16(const uint16_t* base, int64_t idx, int64_t limit,
                                             bool aligned) {
  bf16x8 v;
  if (aligned && idx + 8 <= limit) {
    const uint4 raw = *reinterpret_cast<const uint4*>(base + idx);
    v = *reinterpret_cast<const bf16x8*>(&raw);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t b = idx + i < limit ? base[idx + i] : static_cast<uint16_t>(0);
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

// W_h^T = (G~_h U~_D^T)^T as bf16 hi + lo, [h][d][k] with row stride r_Tp.
// One wave per (record, head, 32 rows of r_T).
__global__ __launch_bounds__(256) void k_make_w(DecBatch b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= b.wtiles_total) return;
  int ri = 0;
  while (ri + 1 < b.n && b.rec[ri + 1].wtile0 <= tile) ++ri;
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
    const bf16x8 a = arow ? load8_bf16(R.G + (static_cast<int64_t>(h) * R.r_T + k) * R.r_D, jj, R.r_D, ga)
                          : zero8();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bb = load8_bf16(R.Ud + static_cast<int64_t>(32 * ct + r) * R.r_D, jj, R.r_D, ga);
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[ct], 0, 0, 0);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = (i >> 2) * 8 + half * 4 + (i & 3);
      const int d = 32 * ct + r;
      const float w = acc[ct][i];
      const uint16_t hi = f32_to_bf16_rne(w);
      const uint16_t lo = f32_to_bf16_rne(w - bf16_bits_to_f32(hi));
      const int64_t off = (static_cast<int64_t>(h) * D + d) * R.r_Tp + k0 + m;
      R.Whi[off] = hi;
      R.Wlo[off] = lo;
    }
  }
}

// One wave per (record, head, 64 rows): X^ rows = U~_T W (hi + lo) + Yhat Q.
template <typename TO>
__global__ __launch_bounds__(256) void k_decode(DecBatch b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= b.tiles_total) return;
  int ri = 0;
  while (ri + 1 < b.n && b.rec[ri + 1].tile0 <= tile) ++ri;
  const DecRec& R = b.rec[ri];
  const int local = tile - R.tile0;
  const int tilesT = (b.T + 63) / 64;
  const int64_t h = local / tilesT, t0 = static_cast<int64_t>(local % tilesT) * 64;
  const int r = lane & 31, half = lane >> 5;
  f32x16 acc[2][4] = {};
  const bool ua = (R.r_T % 8) == 0;
  for (int k0 = 0; k0 < R.r_Tp; k0 += 16) {
    const int kk = k0 + 8 * half;
    bf16x8 a[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t t = t0 + 32 * rt + r;
      a[rt] = t < b.T ? load8_bf16(R.Ut + t * R.r_T, kk, R.r_T, ua) : zero8();
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t wo = (h * D + 32 * ct + r) * R.r_Tp + kk;
      const uint4 rh = *reinterpret_cast<const uint4*>(R.Whi + wo);
      const uint4 rl = *reinterpret_cast<const uint4*>(R.Wlo + wo);
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&rh);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&rl);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rt], bh, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rt], bl, acc[rt][ct], 0, 0, 0);
      }
    }
  }
  const int bits = R.bits;
  const uint32_t qmask = (1u << bits) - 1u;
  for (int d0 = 0; d0 < D; d0 += 16) {
    const int dd = d0 + 8 * half;               // this lane's 8 features
    const int g = dd >> 5, bitpos = (dd & 31) * bits;
    bf16x8 y[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t t = t0 + 32 * rt + r;
      if (t < b.T) {
        const int64_t gi = (h * b.T + t) * 4 + g;
        const uint32_t sw = R.scales[gi];
        const float m16 = bf16_bits_to_f32(static_cast<uint16_t>(sw & 0xffffu));
        const float s16 = bf16_bits_to_f32(static_cast<uint16_t>(sw >> 16));
        const uint32_t* cw = R.codes + gi * bits;
        uint64_t stream = cw[bitpos >> 5];
        if ((bitpos & 31) + 8 * bits > 32) stream |= static_cast<uint64_t>(cw[(bitpos >> 5) + 1]) << 32;
        stream >>= (bitpos & 31);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t q = static_cast<uint32_t>(stream >> (i * bits)) & qmask;
          y[rt][i] = static_cast<__bf16>(fmaf(static_cast<float>(q), s16, m16));
        }
      } else {
        y[rt] = zero8();
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint4 rq = *reinterpret_cast<const uint4*>(b.Qt16 + (32 * ct + r) * D + dd);
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&rq);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y[rt], bq, acc[rt][ct], 0, 0, 0);
    }
  }
  TO* out = static_cast<TO*>(R.out);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t t = t0 + 32 * rt + (i >> 2) * 8 + half * 4 + (i & 3);
        if (t < b.T) {
          const int64_t off = (h * b.T + t) * D + 32 * ct + r;
          if constexpr (sizeof(TO) == 2) out[off] = f32_to_bf16_rne(acc[rt][ct][i]);
          else out[off] = acc[rt][ct][i];
        }
      }
    }
  }
}

__global__ void k_header(uint32_t* blob, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t w4,
                         uint32_t w5, uint32_t w6, uint32_t w7, uint32_t w8, uint32_t w9, uint32_t w10,
                         uint32_t w11, uint32_t w12, uint32_t w13, uint32_t w14, uint32_t w15) {
  const uint32_t w[16] = {w0, w1, w2, w3, w4, w5, w6, w7, w8, w9, w10, w11, w12, w13, w14, w15};
  if (threadIdx.x < 16) blob[threadIdx.x] = w[threadIdx.x];
}

}  // namespace

hipError_t launch_quantize(const float* Y, int64_t rows, int bits, uint16_t* scales, uint8_t* codes,
                           hipStream_t s) {
  const int64_t ng = rows * (D / 32);
  k_quantize<<<(ng + 7) / 8, 256, 0, s>>>(Y, ng, bits, reinterpret_cast<uint32_t*>(scales),
                                          reinterpret_cast<uint32_t*>(codes));
  return hipGetLastError();
}

hipError_t launch_encode_residual(const EncodeArgs& a, hipStream_t s) {
  dim3 grid((a.T + TM - 1) / TM, a.H);
  ProfScope ps("encode_residual", s);
  if (a.x_dtype == kBF16) k_encode_residual<uint16_t><<<grid, 256, 0, s>>>(a);
  else k_encode_residual<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_batch(const DecBatch& b, hipStream_t s) {
  if (b.wtiles_total > 0) {
    ProfScope ps("decode_w", s);
    k_make_w<<<(b.wtiles_total + 3) / 4, 256, 0, s>>>(b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("decode", s);
  if (b.out_dtype == kBF16) k_decode<uint16_t><<<(b.tiles_total + 3) / 4, 256, 0, s>>>(b);
  else k_decode<float><<<(b.tiles_total + 3) / 4, 256, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_write_header(void* blob, const uint32_t* w, hipStream_t s) {
  k_header<<<1, 64, 0, s>>>(static_cast<uint32_t*>(blob), w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7],
                            w[8], w[9], w[10], w[11], w[12], w[13], w[14], w[15]);
  return hipGetLastError();
}

}  // namespace jolt
