// Device helpers shared by the MTLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Storage types: fp32 is stored as float, bf16 as its 16-bit pattern.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Store<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16_bits(v);
  }
};

// Eight consecutive stored elements (16-byte aligned for bf16, 32 for fp32)
// as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// ---------------------------------------------------------------------------
// Slot arithmetic and the stride-aware mask (integers, exact).
//   Token t (1-based) lives in slot ceil(t/s) (1-based).  Query i attends key
//   j iff j == i, or s | j and j/s < ceil(i/s).  In slot terms: query i sees
//   the completed slots b = 1..floor((i-1)/s) plus its own partial slot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int slot_of(int t, int s) { return (t + s - 1) / s; }
__device__ __forceinline__ int completed_slots(int i, int s) { return (i - 1) / s; }
__device__ __forceinline__ bool stride_visible(int i, int j, int s) {
  return (j == i) || ((j % s) == 0 && (j / s) < slot_of(i, s));
}

// ---------------------------------------------------------------------------
// Wave64 reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace mtla
