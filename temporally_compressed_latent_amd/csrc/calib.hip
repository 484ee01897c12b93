// Measurement kernels: the achievable rates of this GPU, against which the
// MTLA kernels' roofline fractions are also reported.  None of them computes
// any part of the method.
//   calib_read_kernel : streaming read of a buffer (HBM read bandwidth when
//                       the buffer is larger than the last-level caches);
//   calib_mfma_kernel : independent chains of 32x32x16 MFMAs on registers
//                       (the matrix cores' issue rate, no memory traffic);
//   calib_empty_kernel: a kernel that does nothing (the launch floor);
//   calib_tile_stream_kernel: the long-cache decode attention's load
//                       schedule with no arithmetic (the ceiling of that
//                       access pattern);
//   calib_load_pattern_kernel: a compute unit's issue cost of one 16-byte-
//                       per-lane load instruction from L2-resident data, for
//                       a contiguous kilobyte or for 16 rows x 64 bytes (the
//                       MFMA operand layout of row-major rows).
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

// One workgroup of 8 waves per compute unit; every wave issues kPatLoads
// 16-byte-per-lane loads before using any, twice over the same addresses
// (the first pass brings them into L2), and thread 0 records the second
// pass's s_memtime cycles from the barrier before its loads to the barrier
// after their use.  Pattern 0: load i of a wave reads 1,024 contiguous bytes
// (lane l at 16 l + 1024 i, eight whole 128-byte lines); pattern 1: 16 rows of
// 64 bytes at a 576-byte row pitch (lane l at row l % 16, byte 16 (l / 16),
// + 64 i: sixteen half lines).  Each wave starts at its own 4 KB offset; the
// buffer resource ends at `bytes`, so no access leaves the buffer.
constexpr int kPatLoads = 32;
template <int P>
__global__ __launch_bounds__(512) void calib_load_pattern_kernel(const uint8_t* __restrict__ buf, uint32_t bytes,
                                                                 uint32_t* __restrict__ cycles) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), static_cast<short>(0),
                                                    static_cast<int>(bytes), kBufferRsrcWord3);
  const uint32_t span = bytes > 131072u ? bytes - 65536u : 65536u;
  const int base = static_cast<int>((static_cast<uint32_t>(blockIdx.x * 8 + wave) * 4096u) % span);
  const int off = base + (P == 0 ? 16 * lane : (lane & 15) * 576 + (lane >> 4) * 16);
  constexpr int step = P == 0 ? 1024 : 64;
  uint32_t acc = 0;
  uint64_t t0 = 0, t1 = 0;
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    t0 = __builtin_amdgcn_s_memtime();
    u32x4 v[kPatLoads];
#pragma unroll
    for (int i = 0; i < kPatLoads; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + i * step, 0, 0);
#pragma unroll
    for (int i = 0; i < kPatLoads; ++i) acc ^= v[i][0] ^ v[i][3];
    __syncthreads();
    t1 = __builtin_amdgcn_s_memtime();
  }
  if (tid == 0) cycles[blockIdx.x] = static_cast<uint32_t>(t1 - t0);
  // (never true for the data used: keeps the loads alive)
  if (acc == 0x9e3779b9u) cycles[gridDim.x + (tid & 63)] = acc;
}

// The load schedule of the long-cache decode attention without its
// arithmetic: one workgroup of 8 waves per (split, sequence) streams 64-row
// tiles of 1,152-byte rows (576 bf16) straight into LDS, two tile buffers,
// the loads of the split's tile after next issued once every wave is done
// with the current one.  IL: split k takes tiles k, k + S, ... (else a
// contiguous range); NT: non-temporal loads.  Each wave folds one LDS word
// per tile and writes it if it matches a pattern no input here produces, so
// no load is dead.
constexpr int kTileRowBytes = 1152, kTileRows = 64, kTileChunks = kTileRows * kTileRowBytes / 16;
constexpr int kTileLoadsPerWave = kTileChunks / (8 * 64);  // 9
template <bool NT>
__device__ __forceinline__ void tile_load16(i32x4_t rsrc, uint32_t lds_base, int voff, int soff) {
  if (NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
template <bool IL, bool NT>
__global__ __launch_bounds__(512) void calib_tile_stream_kernel(const uint8_t* __restrict__ rows, int rows_per_seq,
                                                                uint32_t* __restrict__ sink) {
  constexpr int TS = kTileRows, LPW = kTileLoadsPerWave, CPR = kTileRowBytes / 16;
  static_assert(LPW * 8 * 64 == kTileChunks, "tile shape");
  __shared__ __align__(16) uint8_t kb0[kTileChunks * 16];
  __shared__ __align__(16) uint8_t kb1[kTileChunks * 16];
  const int split = blockIdx.x, b = blockIdx.y, nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = rows_per_seq;
  const int lo = IL ? split * TS : static_cast<int>(static_cast<long long>(split) * n / nsplit);
  const int hi = IL ? n : static_cast<int>(static_cast<long long>(split + 1) * n / nsplit);
  const int step = IL ? nsplit * TS : TS;
  const i32x4_t rs = make_rsrc_words(rows + static_cast<size_t>(b) * n * kTileRowBytes, hi * kTileRowBytes);
  int voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int slot = (wave * LPW + i) * 64 + lane;
    const int r = slot / CPR, c = (slot % CPR) ^ ((r >> 1) & 7);
    voff[i] = r * kTileRowBytes + c * 16;
  }
  auto issue = [&](int j0, uint8_t* dst) {
    const uint32_t base = lds_addr(dst + wave * LPW * 64 * 16);
    const int so = __builtin_amdgcn_readfirstlane(j0 * kTileRowBytes);
#pragma unroll
    for (int i = 0; i < LPW; ++i) tile_load16<NT>(rs, base + i * 64 * 16, voff[i], so);
  };
  uint32_t acc = 0;
  if (lo < hi) issue(lo, kb0);
  if (lo + step < hi) issue(lo + step, kb1);
  auto tile = [&](int j0, uint8_t* kt) {
    if (j0 + step < hi)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    acc ^= reinterpret_cast<const uint32_t*>(kt)[(tid * 7 + j0) % (kTileChunks * 4)];
    lds_barrier();
    if (j0 + 2 * step < hi) issue(j0 + 2 * step, kt);
  };
  for (int j0 = lo; j0 < hi; j0 += 2 * step) {
    tile(j0, kb0);
    if (j0 + step < hi) tile(j0 + step, kb1);
  }
  if (acc == 0x9e3779b9u && (tid & 63) == 0) sink[(static_cast<size_t>(b) * nsplit + split) * 8 + wave] = acc;
}

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

hipError_t launch_calib_tile_stream(const void* rows, int seqs, int rows_per_seq, int splits, bool interleave,
                                    bool nt, uint32_t* sink, hipStream_t st) {
  const dim3 grid(splits, seqs);
  const uint8_t* r = static_cast<const uint8_t*>(rows);
  if (interleave && nt) calib_tile_stream_kernel<true, true><<<grid, 512, 0, st>>>(r, rows_per_seq, sink);
  else if (interleave) calib_tile_stream_kernel<true, false><<<grid, 512, 0, st>>>(r, rows_per_seq, sink);
  else if (nt) calib_tile_stream_kernel<false, true><<<grid, 512, 0, st>>>(r, rows_per_seq, sink);
  else calib_tile_stream_kernel<false, false><<<grid, 512, 0, st>>>(r, rows_per_seq, sink);
  return hipGetLastError();
}

hipError_t launch_calib_empty(hipStream_t st) {
  calib_empty_kernel<<<1, 64, 0, st>>>();
  return hipGetLastError();
}

hipError_t launch_calib_load_pattern(int pattern, int workgroups, const void* buf, size_t bytes, uint32_t* cycles,
                                     hipStream_t st) {
  const auto* b = static_cast<const uint8_t*>(buf);
  const auto n = static_cast<uint32_t>(bytes);
  if (pattern == 0)
    calib_load_pattern_kernel<0><<<workgroups, 512, 0, st>>>(b, n, cycles);
  else
    calib_load_pattern_kernel<1><<<workgroups, 512, 0, st>>>(b, n, cycles);
  return hipGetLastError();
}

}  // namespace mtla
