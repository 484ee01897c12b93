// Gate + temporal merge, device side ("Multi-head Temporal Latent Attention",
// Key claims: paper Sec. 4.1 Eq. 13; Method (1); Sec. 4.3 Eq. 17 for the
// cumulative in-block partial merges used by prefill).  The merge kernels and
// the decode step's merge-and-absorb kernel run this same code, so a token
// merges to the same bits whichever entry point appends it.
//
// Work split: one workgroup per (sequence, run of consecutive blocks).  The
// gates of the run's tokens are computed first (a wave takes four tokens at a
// time, a d_c dot product each), then every (block, 8-column chunk) pair is
// independent: a thread walks its block's tokens in order, carrying the fp32
// block sum.  Every stored value is rounded once from that fp32 sum.  The fp32
// state of the open slot after token t lives at open_acc[b, t % 2].
#pragma once
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
// stage (optional, LDS): row k of it receives c of token ta + k, for the
// merge that follows (the values as loaded, so the merge's bits do not change).
template <typename T, int GE, int NTOK, bool PP>
__device__ void compute_gates_lanes(const MergeArgs& a, int b, int p0, int ta, int ntok, float* gw,
                                    T* stage = nullptr) {
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
      const int kc = min(k0 + k * nwaves, ntok - 1);
      const int t = ta + kc;
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
    // (after every token's loads are issued, so that they stay in flight
    // together)
    if (stage) {
#pragma unroll
      for (int k = 0; k < NTOK; ++k) {
        const int kc = min(k0 + k * nwaves, ntok - 1);
#pragma unroll
        for (int j = 0; j < GE; ++j) Store<T>::store(stage, static_cast<size_t>(kc) * a.d_c + lane + 64 * j, x[k][j]);
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

// ONE: a single token (the gate loads of one pass shrink to one token's;
// the gate's arithmetic, and so its bits, do not change).
// stage: see compute_gates_lanes; only the d_c = 256 and 512 paths fill it
// (gates_stage_c says which).
__device__ __forceinline__ bool gates_stage_c(const MergeArgs& a) { return a.d_c == 256 || a.d_c == 512; }

template <typename T, bool ONE = false>
__device__ void merge_gates(const MergeArgs& a, int b, int p0, int ta, int ntok, float* gw, T* stage = nullptr) {
  if (a.d_c == 256 && a.wh_stride == 0)
    compute_gates_lanes<T, 4, ONE ? 1 : 8, false>(a, b, p0, ta, ntok, gw, stage);
  else if (a.d_c == 256)
    compute_gates_lanes<T, 4, ONE ? 1 : 8, true>(a, b, p0, ta, ntok, gw, stage);
  else if (a.d_c == 512 && a.wh_stride == 0)
    compute_gates_lanes<T, 8, ONE ? 1 : 4, false>(a, b, p0, ta, ntok, gw, stage);
  else if (a.d_c == 512)
    compute_gates_lanes<T, 8, ONE ? 1 : 4, true>(a, b, p0, ta, ntok, gw, stage);
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

// The work of one workgroup (kMergeThreads threads) of the merge: sequence b,
// run `chunk` of blocks_per_wg consecutive blocks.  After the gates, thread t
// takes 8-column chunk ch of block blo + bb for (bb, ch) = (t / CPB, t % CPB),
// CPB = W / 8 (and further blocks in steps of 256 / CPB), and walks that
// block's tokens in order carrying the fp32 sums.  The open-slot state is
// written only if write_open (see launch_merge).  ONE: a.T == 1.  STAGE: the
// workgroup's tokens are at most kStageTokens, and the gate pass leaves their
// c rows in LDS (d_c = 256 or 512), so the merge reads them from there
// instead of from memory a second time.
constexpr int kStageTokens = 32;
template <typename T, bool ONE = false, bool STAGE = false>
__device__ void merge_blocks(const MergeArgs& a, int b, int chunk, int blocks_per_wg, int write_open) {
  __shared__ float gw[kMaxChunkTokens];
  __shared__ __align__(16) T xs[STAGE ? kStageTokens * 512 : 1];
  const SeqRange r = seq_range(a, b);
  if (!r.ok) return;
  const int s = a.s;
  const int W = a.d_c + a.d_r;
  const int blo = r.bk0 + chunk * blocks_per_wg;
  if (blo > r.bk1) return;
  const int bhi = min(r.bk1, blo + blocks_per_wg - 1);
  const int ta = max(r.p0, blo * s + 1);
  const int tb = min(r.t_last, bhi * s + s);
  const bool staged = STAGE && gates_stage_c(a);
  merge_gates<T, ONE>(a, b, r.p0, ta, tb - ta + 1, gw, staged ? xs : nullptr);
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
      if (staged && e < a.d_c) {
#pragma unroll
        for (int u = 0; u < 4; ++u) load8(xs + static_cast<size_t>(min(t + u, t1) - ta) * a.d_c + e, x[u]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) token_chunk<T>(a, b, min(t + u, t1) - r.p0, e, x[u]);
      }
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

}  // namespace

}  // namespace mtla
