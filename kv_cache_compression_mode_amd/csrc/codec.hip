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
// Layout of one workgroup (256 threads, 4 waves) over a 64-row tile: wave w
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

// Bit interleaves: bit i of x moves to bit 2i (16 bits), 4i (8 bits), 3i (12 bits).
__device__ __forceinline__ uint32_t spread2_16(uint32_t x) {
  x &= 0xFFFFu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return (x | (x << 1)) & 0x55555555u;
}
__device__ __forceinline__ uint32_t spread4_8(uint32_t x) {
  x &= 0xFFu;
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  return (x | (x << 3)) & 0x11111111u;
}
__device__ __forceinline__ uint64_t spread3_12(uint64_t x) {
  x &= 0xFFFull;
  x = (x | (x << 16)) & 0x00000000FF0000FFull;
  x = (x | (x << 8)) & 0x000000F00F00F00Full;
  x = (x | (x << 4)) & 0x00000C30C30C30C3ull;
  return (x | (x << 2)) & 0x0000249249249249ull;
}
// Word k (k < bits) of a group's code stream (stream bit s = bit s % bits of
// code s / bits, word k = stream bits [32k, 32k + 32)) from the per-bit masks
// m[j] (bit c = bit j of code c).
__device__ __forceinline__ uint32_t pack_word(const uint32_t (&m)[4], int bits, int k) {
  switch (bits) {
    case 1: return m[0];
    case 2: return spread2_16(m[0] >> (16 * k)) | (spread2_16(m[1] >> (16 * k)) << 1);
    case 3: {   // codes c0 .. c0 + 11 cover the word; c0 = floor(32k / 3)
      const int c0 = (32 * k) / 3, sh = 32 * k - 3 * c0;
      const uint64_t w = spread3_12(m[0] >> c0) | (spread3_12(m[1] >> c0) << 1) | (spread3_12(m[2] >> c0) << 2);
      return static_cast<uint32_t>(w >> sh);
    }
    default:
      return spread4_8(m[0] >> (8 * k)) | (spread4_8(m[1] >> (8 * k)) << 1) |
             (spread4_8(m[2] >> (8 * k)) << 2) | (spread4_8(m[3] >> (8 * k)) << 3);
  }
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
  if (k < bits) code_words[k] = pack_word(mask, bits, k);
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

// One workgroup per 64-row tile of one head (two 32-row blocks).  The
// reconstruction Ut[t0 .. t0+64) W_h and the rotation R Q^T run on fp32
// matrix cores (32x32x2, k in increasing order), their B operands (W_h, then
// Q^T) staged through LDS in chunks of 32 k with the next chunk's loads issued
// before the current chunk's MFMAs; wave w keeps the two 32x32 blocks of
// features [32w, 32w + 32), i.e. quantization group w of every row.
constexpr int ER = 64;        // rows per workgroup
constexpr int EK = 32;        // K chunk
constexpr int EWP = D + 4;    // LDS row stride of a staged B chunk (16-byte rows)

template <typename TX>
__device__ __forceinline__ void encode_tile(const EncodeArgs& a) {
  __shared__ float Us[EK][ER + 1];                               // Ut chunk, [k][row]
  __shared__ __attribute__((aligned(16))) float Bs[EK][EWP];     // W_h or Q^T chunk, [k][feature]
  __shared__ float Rs[ER][D + 1];                                // residual rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rl = lane & 31, half = lane >> 5;
  const int64_t h = blockIdx.y, t0 = static_cast<int64_t>(blockIdx.x) * ER;
  const int col = wave * 32 + rl;
  // B chunk loader: 32 rows x 128 floats, rows kb = (tid >> 5) + 8 i, float4 column 4 (tid & 31)
  const int bk = tid >> 5, bc = 4 * (tid & 31);
  float4 rb[4];
  auto load_b = [&](const float* src, int64_t k0, int64_t kmax) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k = k0 + bk + 8 * i;
      rb[i] = k < kmax ? *reinterpret_cast<const float4*>(src + k * D + bc) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_b = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<float4*>(&Bs[bk + 8 * i][bc]) = rb[i];
  };
  f32x16 acc0 = {}, acc1 = {};
  if (a.r_T > 0) {
    const float* Wh = a.W + h * a.r_T * D;
    // Ut chunk loader: row ur = tid >> 2, k = 8 (tid & 3) .. +8
    const int ur = tid >> 2, uk = 8 * (tid & 3);
    const int64_t ut = t0 + ur;
    float ru[8];
    auto load_u = [&](int64_t k0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t k = k0 + uk + i;
        ru[i] = (ut < a.T && k < a.r_T) ? bf16_bits_to_f32(a.Ut[ut * a.r_T + k]) : 0.f;
      }
    };
    load_u(0);
    load_b(Wh, 0, a.r_T);
    for (int64_t k0 = 0; k0 < a.r_T; k0 += EK) {
#pragma unroll
      for (int i = 0; i < 8; ++i) Us[uk + i][ur] = ru[i];
      store_b();
      __syncthreads();
      if (k0 + EK < a.r_T) {
        load_u(k0 + EK);
        load_b(Wh, k0 + EK, a.r_T);
      }
#pragma unroll
      for (int kk = 0; kk < EK; kk += 2) {
        const int k = kk + half;
        const float b = Bs[k][col];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(Us[k][rl], b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(Us[k][32 + rl], b, acc1, 0, 0, 0);
      }
      __syncthreads();
    }
  }
  // residual R = X - recon, staged in LDS as [row][feature]
  load_b(a.Qt, 0, D);                            // first Q^T chunk, in flight meanwhile
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = (i >> 2) * 8 + half * 4 + (i & 3);
    const int64_t ta = t0 + m, tb = t0 + 32 + m;
    const float xa = ta < a.T ? load_x<TX>(a.X, (h * a.T + ta) * D + col) : 0.f;
    const float xb = tb < a.T ? load_x<TX>(a.X, (h * a.T + tb) * D + col) : 0.f;
    Rs[m][col] = xa - acc0[i];
    Rs[32 + m][col] = xb - acc1[i];
  }
  // Y = R Q^T: Y[m][c] = sum_d R[m][d] Qt[d][c]
  f32x16 y0 = {}, y1 = {};
  for (int d0 = 0; d0 < D; d0 += EK) {
    store_b();
    __syncthreads();
    if (d0 + EK < D) load_b(a.Qt, d0 + EK, D);
#pragma unroll
    for (int kk = 0; kk < EK; kk += 2) {
      const int k = kk + half;
      const float b = Bs[k][col];
      y0 = __builtin_amdgcn_mfma_f32_32x32x2f32(Rs[rl][d0 + k], b, y0, 0, 0, 0);
      y1 = __builtin_amdgcn_mfma_f32_32x32x2f32(Rs[32 + rl][d0 + k], b, y1, 0, 0, 0);
    }
    __syncthreads();
  }
  uint32_t* sc = reinterpret_cast<uint32_t*>(a.scales);
  uint32_t* cd = reinterpret_cast<uint32_t*>(a.codes);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = (i >> 2) * 8 + half * 4 + (i & 3);
    const int64_t ta = t0 + m, tb = t0 + 32 + m;
    const int64_t ga = (h * a.T + ta) * 4 + wave, gb = (h * a.T + tb) * 4 + wave;   // group indices
    quantize_group(y0[i], a.bits, ta < a.T, sc + ga, cd + ga * a.bits);
    quantize_group(y1[i], a.bits, tb < a.T, sc + gb, cd + gb * a.bits);
  }
}

template <typename TX>
__global__ __launch_bounds__(256, 2) void k_encode_residual(EncodeArgs a) {
  encode_tile<TX>(a);
}
// Tensors of one shape in one launch: blockIdx.z selects the tensor's arguments.
template <typename TX>
__global__ __launch_bounds__(256, 2) void k_encode_residual_many(const EncodeArgs* list) {
  const EncodeArgs a = list[blockIdx.z];
  encode_tile<TX>(a);
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
__global__ __launch_bounds__(256, 2) void k_decode(DecBatch b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= b.tiles_total) return;
  // the record holding this tile: the last with first tile <= tile (records
  // are in order, so a binary search)
  int ri = 0;
  for (int hi = b.n - 1; ri < hi;) {
    const int mid = (ri + hi + 1) >> 1;
    if (b.rec[mid].tile0 <= tile) ri = mid;
    else hi = mid - 1;
  }
  const DecRec& R = b.rec[ri];
  const int local = tile - R.tile0;
  const int tilesT = (b.T + 63) / 64;
  const int64_t h = local / tilesT, t0 = static_cast<int64_t>(local % tilesT) * 64;
  const int r = lane & 31, half = lane >> 5;
  f32x16 acc[2][4] = {};
  const bool ua = (R.r_T % 8) == 0;
  // U~_T rows of one k step (16 of r_T) streamed from memory, the next
  // step's loaded during this one's MFMAs; W (hi, lo) is shared by all row
  // tiles of the head and stays in cache
  bf16x8 a[2];
  auto load_k = [&](int k0) {
    const int kk = k0 + 8 * half;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t t = t0 + 32 * rt + r;
      a[rt] = t < b.T ? load8_bf16(R.Ut + t * R.r_T, kk, R.r_T, ua) : zero8();
    }
  };
  if (R.r_Tp > 0) load_k(0);
  for (int k0 = 0; k0 < R.r_Tp; k0 += 16) {
    const int kk = k0 + 8 * half;
    const bf16x8 ca[2] = {a[0], a[1]};
    bf16x8 ch[4], cl[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t wo = (h * D + 32 * ct + r) * R.r_Tp + kk;
      const uint4 rh = *reinterpret_cast<const uint4*>(R.Whi + wo);
      const uint4 rlo = *reinterpret_cast<const uint4*>(R.Wlo + wo);
      ch[ct] = *reinterpret_cast<const bf16x8*>(&rh);
      cl[ct] = *reinterpret_cast<const bf16x8*>(&rlo);
    }
    if (k0 + 16 < R.r_Tp) load_k(k0 + 16);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[rt], ch[ct], acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[rt], cl[ct], acc[rt][ct], 0, 0, 0);
      }
    }
  }
  const int bits = R.bits;
  const uint32_t qmask = (1u << bits) - 1u;
  // the streamed words of one d step (scales, code words), the next step's
  // loaded during this one's dequantization and MFMAs (Q^T stays in cache)
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
        sw[rt] = R.scales[gi];
        const uint32_t* cw = R.codes + gi * bits;
        w0[rt] = cw[bitpos >> 5];
        if ((bitpos & 31) + 8 * bits > 32) w1[rt] = cw[(bitpos >> 5) + 1];
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
    for (int ct = 0; ct < 4; ++ct) cq[ct] = *reinterpret_cast<const uint4*>(b.Qt16 + (32 * ct + r) * D + dd);
    if (d0 + 16 < D) load_d(d0 + 16);
    bf16x8 y[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float m16 = bf16_bits_to_f32(static_cast<uint16_t>(csw[rt] & 0xffffu));
      const float s16 = bf16_bits_to_f32(static_cast<uint16_t>(csw[rt] >> 16));
      const uint64_t stream = (static_cast<uint64_t>(cw0[rt]) | (static_cast<uint64_t>(cw1[rt]) << 32)) >>
                              (bitpos & 31);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t q = static_cast<uint32_t>(stream >> (i * bits)) & qmask;
        y[rt][i] = static_cast<__bf16>(fmaf(static_cast<float>(q), s16, m16));
      }
    }
    // rows past T: scale word 0 gives m16 = s16 = 0, so y = 0
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&cq[ct]);
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

__global__ void k_header_many(uint32_t* const* blobs, const uint32_t* words) {
  if (threadIdx.x < 16) blobs[blockIdx.x][threadIdx.x] = words[blockIdx.x * 16 + threadIdx.x];
}
hipError_t launch_write_headers(uint32_t* const* blobs_dev, const uint32_t* words_dev, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_header_many<<<n, 64, 0, s>>>(blobs_dev, words_dev);
  return hipGetLastError();
}
hipError_t launch_write_header(void* blob, const uint32_t* w, hipStream_t s) {
  k_header<<<1, 64, 0, s>>>(static_cast<uint32_t*>(blob), w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7],
                            w[8], w[9], w[10], w[11], w[12], w[13], w[14], w[15]);
  return hipGetLastError();
}

}  // namespace jolt
