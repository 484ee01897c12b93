// Gate + temporal merge into the slot cache ("Multi-head Temporal Latent
// Attention", Key claims: paper Sec. 4.1 Eq. 13; Method (1); Sec. 4.3 Eq. 17
// for the cumulative in-block partial merges used by prefill).
//
// Work split: one workgroup per (sequence, run of consecutive blocks).  The
// gates of the run's tokens are computed first (a wave takes four tokens at a
// time, a d_c dot product each), then every (block, 8-column chunk) pair is
// independent: a thread walks its block's tokens in order, carrying the fp32
// block sum.  Every stored value is rounded once from that fp32 sum.  The fp32
// state of the open slot after token t lives at open_acc[b, t % 2].
#include "common.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMaxChunkTokens = 256;

struct SeqRange {
  int p0;       // first appended token (1-based)
  int t_last;   // last appended token
  int bk0, bk1; // first/last touched block (0-based slot rows)
  bool ok;
};

__device__ __forceinline__ SeqRange seq_range(const MergeArgs& a, int b) {
  SeqRange r;
  r.p0 = a.pos0 ? a.pos0[b] : a.p0_all;
  const long long tl = static_cast<long long>(r.p0) + a.T - 1;
  r.ok = r.p0 >= 1 && tl <= a.pe_rows;
  r.t_last = static_cast<int>(tl);
  r.bk0 = r.ok ? (r.p0 - 1) / a.s : 0;
  r.bk1 = r.ok ? (r.t_last - 1) / a.s : 0;
  r.ok = r.ok && r.bk1 < a.max_slots;
  return r;
}

// Gates of tokens ta..ta+ntok-1 of sequence b into gw[0..ntok): each wave
// takes kGateTok tokens at a time (independent streams, loads in flight
// together).
constexpr int kGateTok = 4;

template <typename T>
__device__ void compute_gates(const MergeArgs& a, int b, int p0, int ta, int ntok, float* gw) {
  const T* c = static_cast<const T*>(a.c);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int k0 = wave * kGateTok; k0 < ntok; k0 += nwaves * kGateTok) {
    const T* rows[kGateTok];
    const float* pes[kGateTok];
    const float* whs[kGateTok];
#pragma unroll
    for (int k = 0; k < kGateTok; ++k) {
      const int t = ta + k0 + k;
      const bool in = k0 + k < ntok;
      rows[k] = in ? c + (static_cast<size_t>(b) * a.T + (t - p0)) * a.d_c : nullptr;
      pes[k] = in ? a.pe + static_cast<size_t>(t - 1) * a.d_c : a.pe;
      whs[k] = in ? a.w_hyp + static_cast<size_t>((t - 1) % a.s) * a.wh_stride : a.w_hyp;
    }
    float w[kGateTok];
    gates_of_tokens<kGateTok, T>(rows, pes, whs, a.d_c, lane, w);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kGateTok; ++k) {
        if (k0 + k < ntok) {
          gw[k0 + k] = w[k];
          if (a.gate_out) a.gate_out[static_cast<size_t>(b) * a.T + (ta + k0 + k - p0)] = w[k];
        }
      }
    }
  }
}

// The same gates with every load of a pass in flight together, for
// d_c = 64 GE: wave w takes tokens w, w + nwaves, ... (NTOK of them per pass),
// lane l holds elements l + 64 j of c_t, pe_t and W_hyp, and the sum runs in
// the order of gate_from_lane_values (the same bits as gates_of_tokens and
// the decode-step kernels).  Token indices past the last are clamped (their
// gates are computed and dropped), so the loads are unconditional.  PP: one
// W_hyp row per place in the block, loaded with each token.
template <typename T, int GE, int NTOK, bool PP>
__device__ void compute_gates_lanes(const MergeArgs& a, int b, int p0, int ta, int ntok, float* gw) {
  const T* c = static_cast<const T*>(a.c);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  float wh[PP ? NTOK : 1][GE];
  if constexpr (!PP) {
#pragma unroll
    for (int j = 0; j < GE; ++j) wh[0][j] = a.w_hyp[lane + 64 * j];
  }
  for (int k0 = wave; k0 < ntok; k0 += nwaves * NTOK) {
    float x[NTOK][GE], pv[NTOK][GE];
#pragma unroll
    for (int k = 0; k < NTOK; ++k) {
      const int t = ta + min(k0 + k * nwaves, ntok - 1);
      const T* row = c + (static_cast<size_t>(b) * a.T + (t - p0)) * a.d_c;
      const float* per = a.pe + static_cast<size_t>(t - 1) * a.d_c;
      const float* whr = a.w_hyp + static_cast<size_t>((t - 1) % a.s) * a.wh_stride;
#pragma unroll
      for (int j = 0; j < GE; ++j) {
        x[k][j] = Store<T>::load(row, lane + 64 * j);
        pv[k][j] = per[lane + 64 * j];
        if constexpr (PP) wh[k][j] = whr[lane + 64 * j];
      }
    }
#pragma unroll
    for (int k = 0; k < NTOK; ++k) {
      const float w = gate_from_lane_values<GE>(x[k], pv[k], wh[PP ? k : 0]);
      const int kk = k0 + k * nwaves;
      if (lane == 0 && kk < ntok) {
        gw[kk] = w;
        if (a.gate_out) a.gate_out[static_cast<size_t>(b) * a.T + (ta + kk - p0)] = w;
      }
    }
  }
}

template <typename T>
__device__ void merge_gates(const MergeArgs& a, int b, int p0, int ta, int ntok, float* gw) {
  if (a.d_c == 256 && a.wh_stride == 0)
    compute_gates_lanes<T, 4, 8, false>(a, b, p0, ta, ntok, gw);
  else if (a.d_c == 256)
    compute_gates_lanes<T, 4, 8, true>(a, b, p0, ta, ntok, gw);
  else if (a.d_c == 512 && a.wh_stride == 0)
    compute_gates_lanes<T, 8, 4, false>(a, b, p0, ta, ntok, gw);
  else if (a.d_c == 512)
    compute_gates_lanes<T, 8, 4, true>(a, b, p0, ta, ntok, gw);
  else
    compute_gates<T>(a, b, p0, ta, ntok, gw);
}

// Eight elements of x_t = [c_t ; k^R_t] starting at column e (e % 8 == 0, and
// d_c % 8 == 0, so a chunk never straddles c and k^R).
template <typename T>
__device__ __forceinline__ void token_chunk(const MergeArgs& a, int b, int tok, int e, float* x) {
  const size_t row = static_cast<size_t>(b) * a.T + tok;
  if (e < a.d_c)
    load8(static_cast<const T*>(a.c) + row * a.d_c + e, x);
  else
    load8(static_cast<const T*>(a.k_r) + row * a.d_r + (e - a.d_c), x);
}

// One workgroup per (sequence, run of blocks_per_wg consecutive blocks).
// After the gates, thread t takes 8-column chunk ch of block blo + bb for
// (bb, ch) = (t / CPB, t % CPB), CPB = W / 8 (and further blocks in steps of
// 256 / CPB), and walks that block's tokens in order carrying the fp32 sums.
template <typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a, int blocks_per_wg,
                                                              int write_open) {
  __shared__ float gw[kMaxChunkTokens];
  const int b = blockIdx.y;
  const SeqRange r = seq_range(a, b);
  if (!r.ok) return;
  const int s = a.s;
  const int W = a.d_c + a.d_r;
  const int blo = r.bk0 + static_cast<int>(blockIdx.x) * blocks_per_wg;
  if (blo > r.bk1) return;
  const int bhi = min(r.bk1, blo + blocks_per_wg - 1);
  const int ta = max(r.p0, blo * s + 1);
  const int tb = min(r.t_last, bhi * s + s);
  merge_gates<T>(a, b, r.p0, ta, tb - ta + 1, gw);
  __syncthreads();

  T* cache = static_cast<T*>(a.cache);
  T* P = static_cast<T*>(a.partials);
  const int CPB = W / 8;
  const int bpp = kMergeThreads / CPB;  // blocks per pass
  const int ch = threadIdx.x % CPB, bb0 = threadIdx.x / CPB;
  if (bb0 >= bpp) return;
  const int e = ch * 8;
  for (int blk = blo + bb0; blk <= bhi; blk += bpp) {
    const int ts = blk * s + 1;
    const int t0 = max(ts, r.p0);
    const int t1 = min(ts + s - 1, r.t_last);
    float acc[8];
    if (t0 > ts) {  // a block that began before this call continues the open slot
      const float* oa = a.open_acc + (static_cast<size_t>(b) * 2 + (r.p0 - 1) % 2) * W + e;
      const float4 lo = *reinterpret_cast<const float4*>(oa);
      const float4 hi = *reinterpret_cast<const float4*>(oa + 4);
      acc[0] = lo.x; acc[1] = lo.y; acc[2] = lo.z; acc[3] = lo.w;
      acc[4] = hi.x; acc[5] = hi.y; acc[6] = hi.z; acc[7] = hi.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    }
    // four tokens' chunks in flight at a time (indices clamped to the block)
    for (int t = t0; t <= t1; t += 4) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) token_chunk<T>(a, b, min(t + u, t1) - r.p0, e, x[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t + u <= t1) {
          const float w = gw[t + u - ta];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, x[u][j], acc[j]);
          if (P) store8(P + (static_cast<size_t>(b) * a.T + (t + u - r.p0)) * W + e, acc);
        }
      }
    }
    store8(cache + (static_cast<size_t>(b) * a.max_slots + blk) * W + e, acc);
    if (write_open && blk == r.bk1) store8(a.open_acc + (static_cast<size_t>(b) * 2 + r.t_last % 2) * W + e, acc);
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
  const int write_open = chunks == 1 ? 1 : 0;
  dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.B));
  if (dtype == 0) {
    merge_kernel<float><<<grid, kMergeThreads, 0, st>>>(a, blocks_per_wg, write_open);
    if (!write_open) merge_tail_kernel<float><<<a.B, kMergeThreads, 0, st>>>(a);
  } else {
    merge_kernel<uint16_t><<<grid, kMergeThreads, 0, st>>>(a, blocks_per_wg, write_open);
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
