// Measurement kernels: the achievable rates of this GPU, against which the
// MTLA kernels' roofline fractions are also reported.  None of them computes
// any part of the method.
//   calib_read_kernel : streaming read of a buffer (HBM read bandwidth when
//                       the buffer is larger than the last-level caches);
//   calib_mfma_kernel : independent chains of 32x32x16 MFMAs on registers
//                       (the matrix cores' issue rate, no memory traffic);
//   calib_empty_kernel: a kernel that does nothing (the launch floor).
#include "common.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadInFlight = 8;

// Thread i reads 16-byte chunks i, i + G, i + 2G, ... (G = threads in the
// grid), kReadInFlight of them per round, all loads of a round issued before
// any is used; the chunks are xor-folded and each wave writes one word, so
// no load is dead.
__global__ __launch_bounds__(kReadThreads) void calib_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                  uint32_t* __restrict__ sink) {
  const size_t G = static_cast<size_t>(gridDim.x) * kReadThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadInFlight - 1) * G < n16; i += kReadInFlight * G) {
    u32x4 v[kReadInFlight];
#pragma unroll
    for (int k = 0; k < kReadInFlight; ++k) v[k] = __builtin_nontemporal_load(src + i + k * G);
#pragma unroll
    for (int k = 0; k < kReadInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += G) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[(static_cast<size_t>(blockIdx.x) * kReadThreads + threadIdx.x) / 64] = acc;
}

// Each wave runs kChains independent accumulation chains of `iters`
// 32x32x16 MFMAs (bf16 or fp16 operands, fp32 accumulators) on register
// operands; the accumulators are summed and written, one float per lane.
constexpr int kChains = 4;

template <bool F16>
__global__ __launch_bounds__(256) void calib_mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  u16x8 a, b;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    // small distinct values (the rate does not depend on them)
    a[r] = F16 ? f32_to_f16_bits(0.001f * (lane + r)) : f32_to_bf16_bits(0.001f * (lane + r));
    b[r] = F16 ? f32_to_f16_bits(0.002f * (r - lane)) : f32_to_bf16_bits(0.002f * (r - lane));
  }
  f32x16 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[k][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      if constexpr (F16)
        c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c[k], 0, 0, 0);
      else
        c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c[k], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ void calib_empty_kernel() {}

}  // namespace

hipError_t launch_calib_read(const void* src, size_t bytes, int workgroups, uint32_t* sink, hipStream_t st) {
  calib_read_kernel<<<workgroups, kReadThreads, 0, st>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(bool f16, int workgroups, int iters, float* out, hipStream_t st) {
  if (f16)
    calib_mfma_kernel<true><<<workgroups, 256, 0, st>>>(iters, out);
  else
    calib_mfma_kernel<false><<<workgroups, 256, 0, st>>>(iters, out);
  return hipGetLastError();
}

double calib_mfma_flops(int workgroups, int iters) {
  // waves x chains x iterations x (2 x 32 x 32 x 16) flops
  return 4.0 * workgroups * kChains * static_cast<double>(iters) * (2.0 * 32 * 32 * 16);
}

hipError_t launch_calib_empty(hipStream_t st) {
  calib_empty_kernel<<<1, 64, 0, st>>>();
  return hipGetLastError();
}

}  // namespace mtla
