// Gate + temporal merge into the slot cache: the launches ("Multi-head
// Temporal Latent Attention", Key claims: paper Sec. 4.1 Eq. 13; Method (1);
// Sec. 4.3 Eq. 17).  The per-workgroup work is merge_blocks (merge_body.hpp).
#include "merge_body.hpp"

namespace mtla {

namespace {

// XMAP: a one-dimensional grid of 8 * cpx * B workgroups in which XCD x
// (workgroups are dealt to the 8 XCDs round-robin by linear id) takes runs
// x*cpx .. x*cpx + cpx - 1 of every sequence, so the pe rows of those tokens
// are fetched into one L2; otherwise grid (runs, B).
template <typename T, bool STAGE, bool XMAP>
__global__ __launch_bounds__(kMergeThreads) __attribute__((amdgpu_waves_per_eu(4))) void merge_kernel(MergeArgs a, int blocks_per_wg, int write_open,
                                                              int chunks, int cpx) {
  if constexpr (XMAP) {
    const int L = blockIdx.x, k = L >> 3;
    const int chunk = (L & 7) * cpx + k / a.B, b = k % a.B;
    if (chunk >= chunks) return;
    merge_blocks<T, false, STAGE>(a, b, chunk, blocks_per_wg, write_open);
  } else {
    merge_blocks<T, false, STAGE>(a, blockIdx.y, blockIdx.x, blocks_per_wg, write_open);
  }
}

// When one call spans several workgroups per sequence, the open-slot state is
// written afterwards by this kernel (one workgroup per sequence): it redoes
// the last block's fp32 sum with the same operation order, so that the first
// workgroup's read of the old state never races with the new write.
template <typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_tail_kernel(MergeArgs a) {
  __shared__ float gw[kMaxChunkTokens];
  const int b = blockIdx.x;
  const SeqRange r = seq_range(a, b);
  if (!r.ok) return;
  const int W = a.d_c + a.d_r;
  const int ts = r.bk1 * a.s + 1;
  const int t0 = max(ts, r.p0);
  merge_gates<T>(a, b, r.p0, t0, r.t_last - t0 + 1, gw);
  __syncthreads();
  const int ch = threadIdx.x;
  if (ch >= W / 8) return;
  const int e = ch * 8;
  float acc[8];
  if (t0 > ts) {
    const float* oa = a.open_acc + (static_cast<size_t>(b) * 2 + (r.p0 - 1) % 2) * W + e;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = oa[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  }
  for (int t = t0; t <= r.t_last; ++t) {
    float x[8];
    token_chunk<T>(a, b, t - r.p0, e, x);
    const float w = gw[t - t0];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, x[j], acc[j]);
  }
  store8(a.open_acc + (static_cast<size_t>(b) * 2 + r.t_last % 2) * W + e, acc);
}

// Beam reorder ([MTLA-repo]: evaluation by Fairseq-style parallel beam
// search; a kept hypothesis b continues hypothesis src[b]).  One workgroup
// per (destination b, run of kReorderSlots slots); 16-byte units (d_c and d_r
// are multiples of 8, so a row is), four units in flight per thread.  The
// x == 0 workgroup also copies the open-slot state and the token count.  A
// destination whose parent index is out of range is left untouched.
constexpr int kReorderSlots = 64;

template <typename U>
__global__ __launch_bounds__(256) void reorder_kernel(ReorderArgs a) {
  const int b = blockIdx.y;
  const int parent = a.src[b];
  if (parent < 0 || parent >= a.B) return;
  const int p = a.pos[parent];
  int n = p >= 1 ? slot_of(p, a.s) : 0;
  if (n > a.max_slots) n = a.max_slots;
  const int r0 = blockIdx.x * kReorderSlots;
  const int r1 = min(n, r0 + kReorderSlots);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < a.open_floats; i += blockDim.x)
      a.open_out[static_cast<size_t>(b) * a.open_floats + i] = a.open_in[static_cast<size_t>(parent) * a.open_floats + i];
    if (a.pos_out && threadIdx.x == 0) a.pos_out[b] = p;
  }
  if (r0 >= r1) return;
  const size_t seq_bytes = static_cast<size_t>(a.max_slots) * a.row_bytes;
  const U* in = reinterpret_cast<const U*>(static_cast<const char*>(a.cache_in) + parent * seq_bytes +
                                           static_cast<size_t>(r0) * a.row_bytes);
  U* out = reinterpret_cast<U*>(static_cast<char*>(a.cache_out) + b * seq_bytes +
                                static_cast<size_t>(r0) * a.row_bytes);
  const int units = (r1 - r0) * (a.row_bytes / static_cast<int>(sizeof(U)));
  constexpr int K = 4;
  for (int i0 = threadIdx.x; i0 < units; i0 += K * 256) {
    U v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = min(i0 + k * 256, units - 1);
      v[k] = in[i];
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (i0 + k * 256 < units) out[i0 + k * 256] = v[k];
  }
}

__global__ void pe_kernel(int rows, int d, float* pe) {
  const size_t n = static_cast<size_t>(rows) * d;
  for (size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; idx < n;
       idx += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int p = static_cast<int>(idx / d);
    const int e = static_cast<int>(idx % d);
    const int k = e / 2;
    const double ang = static_cast<double>(p) * pow(10000.0, -2.0 * k / d);
    pe[idx] = static_cast<float>((e % 2 == 0) ? sin(ang) : cos(ang));
  }
}

__global__ void debug_mask_kernel(int n, int s, uint8_t* mask) {
  const size_t total = static_cast<size_t>(n) * n;
  for (size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int i = static_cast<int>(idx / n) + 1;
    const int j = static_cast<int>(idx % n) + 1;
    mask[idx] = stride_visible(i, j, s) ? 1 : 0;
  }
}

__global__ void debug_limits_kernel(int n, int s, int32_t* hi) {
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
  if (i0 < n) hi[i0] = completed_slots(i0 + 1, s);
}

int grid_for(size_t n, int threads) {
  size_t g = (n + threads - 1) / threads;
  if (g > 65535) g = 65535;
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int dtype, hipStream_t st) {
  // Blocks one call can touch: ceil((T-1)/s) + 1 (a block may continue).
  const long long max_blocks = (static_cast<long long>(a.T) - 1 + a.s - 1) / a.s + 1;
  // Blocks per workgroup: enough workgroups (~2048) to fill the chip, at most
  // 32 tokens of gates per workgroup (one pass of the gate loads) unless one
  // block is longer.
  const int cap = a.s >= 32 ? 1 : 32 / a.s;
  long long per = (max_blocks * a.B + 2047) / 2048;
  const int blocks_per_wg = static_cast<int>(per < 1 ? 1 : (per > cap ? cap : per));
  const long long chunks = (max_blocks + blocks_per_wg - 1) / blocks_per_wg;
  // The merge kernel writes the open-slot state itself when no block of the
  // call continues one that began before it (nothing reads the old state:
  // every appended token starts or extends a block of this call; the host
  // knows this when all sequences start at one position), or for a one-token
  // call: the thread that reads the old state (a continued block) is then the
  // thread that writes the new one, after its read.  Otherwise the continued
  // block and the last block may belong to threads of different waves with
  // no barrier between them, and for an even token count the read and the
  // write address the same half of open_acc, so merge_tail_kernel writes the
  // state after the merge kernel has finished.
  const bool fresh = a.pos0 == nullptr && (a.p0_all - 1) % a.s == 0;
  const int write_open = fresh || (chunks == 1 && max_blocks == 1) ? 1 : 0;
  // The c rows of a workgroup's tokens stay in LDS from the gate pass to the
  // merge (bf16, at most kStageTokens tokens per workgroup).
  const bool stage = dtype == 1 && blocks_per_wg * a.s <= kStageTokens;
  const int cpx = static_cast<int>((chunks + 7) / 8);
  const bool xmap = chunks >= 8;
  const dim3 grid = xmap ? dim3(static_cast<unsigned>(8 * cpx * a.B)) : dim3(static_cast<unsigned>(chunks), a.B);
  auto go = [&](auto kern) {
    kern<<<grid, kMergeThreads, 0, st>>>(a, blocks_per_wg, write_open, static_cast<int>(chunks), cpx);
  };
  if (dtype == 0) {
    if (xmap) go(merge_kernel<float, false, true>); else go(merge_kernel<float, false, false>);
    if (!write_open) merge_tail_kernel<float><<<a.B, kMergeThreads, 0, st>>>(a);
  } else {
    if (stage && xmap) go(merge_kernel<uint16_t, true, true>);
    else if (stage) go(merge_kernel<uint16_t, true, false>);
    else if (xmap) go(merge_kernel<uint16_t, false, true>);
    else go(merge_kernel<uint16_t, false, false>);
    if (!write_open) merge_tail_kernel<uint16_t><<<a.B, kMergeThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_reorder(const ReorderArgs& a, hipStream_t st) {
  if (a.row_bytes % 16 != 0) return hipErrorInvalidValue;
  dim3 grid((a.max_slots + kReorderSlots - 1) / kReorderSlots, a.B);
  reorder_kernel<uint4><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_sinusoidal_pe(int rows, int d, float* pe, hipStream_t st) {
  pe_kernel<<<grid_for(static_cast<size_t>(rows) * d, 256), 256, 0, st>>>(rows, d, pe);
  return hipGetLastError();
}

hipError_t launch_debug_mask(int n, int s, uint8_t* mask, hipStream_t st) {
  debug_mask_kernel<<<grid_for(static_cast<size_t>(n) * n, 256), 256, 0, st>>>(n, s, mask);
  return hipGetLastError();
}

hipError_t launch_debug_limits(int n, int s, int32_t* hi, hipStream_t st) {
  debug_limits_kernel<<<(n + 255) / 256, 256, 0, st>>>(n, s, hi);
  return hipGetLastError();
}

}  // namespace mtla
