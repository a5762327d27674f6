// Device-side helpers shared by the codec's HIP kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jolt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>(u >> 16);  // inf/nan
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 values as a packed bf16 pair (lo in the low half), round to
// nearest even: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// The 8 dequantized values y = m16 + q * s16 (fp32 fma, then bf16 nearest
// even) of one lane's 8 consecutive codes: the group's scale word sw
// (offset | step << 16), the code words w0 (and w1 when the 8 b-bit codes
// cross a word) holding them from bit sh on.  One funnel shift, then one
// bit-field extract per code.
template <typename V8>
__device__ __forceinline__ V8 dequant8(uint32_t sw, uint32_t w0, uint32_t w1, uint32_t sh, uint32_t bits) {
  const float m16 = __uint_as_float(sw << 16);
  const float s16 = __uint_as_float(sw & 0xffff0000u);
  const uint32_t w = __builtin_amdgcn_alignbit(w1, w0, sh);
  V8 y;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    y[i] = static_cast<__bf16>(fmaf(static_cast<float>(__builtin_amdgcn_ubfe(w, i * bits, bits)), s16, m16));
  return y;
}

// Largest bf16 <= f: truncation rounds toward zero, so a negative inexact
// value takes one more unit of magnitude.
__device__ __forceinline__ uint16_t bf16_round_down(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t hi = u >> 16;
  if ((u & 0xffffu) != 0u && (u >> 31) != 0u) hi += 1u;
  return static_cast<uint16_t>(hi);
}

// Smallest bf16 >= f.
__device__ __forceinline__ uint16_t bf16_round_up(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t hi = u >> 16;
  if ((u & 0xffffu) != 0u && (u >> 31) == 0u) hi += 1u;
  return static_cast<uint16_t>(hi);
}

// 16-byte load and store through the global address space: global_load /
// global_store are counted by vmcnt alone, while the flat instructions that a
// generic pointer gives also count in lgkmcnt, so an LDS wait would hold on
// them too.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const void* p) {
  // a plain vector type: copying HIP's uint4 struct would go through a generic reference
  const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ldg32(const void* p) {
  return *(const __attribute__((address_space(1))) uint32_t*)(p);
}
__device__ __forceinline__ uint16_t ldg_u16(const void* p) {
  return *(const __attribute__((address_space(1))) uint16_t*)(p);
}
__device__ __forceinline__ void stg32(void* p, uint32_t v) { *(__attribute__((address_space(1))) uint32_t*)(p) = v; }
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *(__attribute__((address_space(1))) u32x4*)(p) = v; }

template <typename T> __device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2) by linear id.  For a grid of nb groups of gsize ids each (group-major:
// a group's ids consecutive), xcd_group gives the group and the index in it
// of linear id L such that, when nb is a multiple of 8, every id of a group
// runs on one XCD (a group's shared operands go through one L2); otherwise
// the plain decomposition.  A bijection either way.
__device__ __forceinline__ void xcd_group(uint32_t L, uint32_t gsize, uint32_t nb, uint32_t& grp, uint32_t& idx) {
  if (nb % 8 == 0) {
    const uint32_t j = L / 8;
    grp = L % 8 + 8 * (j / gsize);
    idx = j % gsize;
  } else {
    grp = L / gsize;
    idx = L % gsize;
  }
}
// the same for a 2-D grid: x = the index in a group, y = the group
__device__ __forceinline__ void xcd_group_2d(uint32_t& x, uint32_t& y) {
  xcd_group(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x, gridDim.y, y, x);
}

// orders one wave's LDS accesses (LDS executes a wave's operations in order)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// v(lane l) + v(lane l ^ 32), the same value in both halves of the wave: one
// lane swap of the halves (v_permlane32_swap, gfx950) instead of a trip
// through LDS.  Both halves add the lower half's value to the upper half's.
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ----------------------------------------------------- counter-based RNG
// SplitMix64 (Steele, Lea & Flood 2014): word i of the stream keyed by
// key = mix64(seed ^ tag) is mix64(key + (i + 1) * GAMMA); normals come from
// Box-Muller pairs of uniforms ((w >> 11) + 0.5) * 2^-53, in fp64.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ double rng_normal(uint64_t key, uint64_t i) {
  const uint64_t k = i >> 1;
  const uint64_t w1 = mix64(key + (2 * k + 1) * kGamma);
  const uint64_t w2 = mix64(key + (2 * k + 2) * kGamma);
  const double u1 = (static_cast<double>(w1 >> 11) + 0.5) * 0x1p-53;
  const double u2 = (static_cast<double>(w2 >> 11) + 0.5) * 0x1p-53;
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 2.0 * 3.141592653589793 * u2;
  return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

// ------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace jolt
