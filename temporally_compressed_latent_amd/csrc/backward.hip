// Training backward of the stride-masked parallel pass ("Multi-head Temporal
// Latent Attention", Key claims: paper Sec. 4.2 Fig. 2(c) and Sec. 4.3 Eq. 17,
// parallel training under the stride-aware causal mask; Method (1)-(3)).
//
// Forward, per sequence (tokens and keys 1-based in the formulas):
//   w_t = sigmoid(W_hyp . (c_t + pe_t)),  x_t = [c_t ; k^R_t]
//   P_j = sum over the tokens k <= j of j's block of w_k x_k
//   K^C_jh = W_UK[h] P^c_j,  V_jh = W_UV[h] P^c_j,  rope key P^R_j
//   z_ijh = tau (q^C_ih . K^C_jh + q^R_ih . P^R_j) over the keys query i sees
//   (j = i, or s | j and j < i), o_ih = sum_j softmax_j(z_ijh) V_jh.
// Backward (reverse mode, last step first):
//   p_ij = exp(z_ij - lse_i),  dp_ij = dO_i . V_j,  D_i = sum_j p_ij dp_ij,
//   ds_ij = tau p_ij (dp_ij - D_i);
//   dq_i = sum_j ds_ij [K^C_j ; P^R_j];   dK^C_j = sum_i ds_ij q^C_i,
//   dK^R_jh = sum_i ds_ij q^R_i,  dV_j = sum_i p_ij dO_i;
//   dP^c_j = sum_h W_UK[h]^T dK^C_jh + W_UV[h]^T dV_jh,  dP^R_j = sum_h dK^R_jh;
//   dW_UK[h] = sum_j dK^C_jh (P^c_j)^T, dW_UV[h] = sum_j dV_jh (P^c_j)^T;
//   G_k = sum of dP_j over j = k .. end of k's block (a reverse in-block sum);
//   dx_k = w_k G_k,  dw_k = G_k . x_k,  du_k = dw_k w_k (1 - w_k);
//   dc_k = dx^c_k + du_k W_hyp,  dk^R_k = dx^R_k,  dW_hyp = sum_k du_k (c_k + pe_k).
//
// The kernels here compute in fp32 from either storage type.  The attention
// kernels give one workgroup (one wave) to a query (dQ) or to a key (dK, dV):
// lanes take 64 keys (queries) at a time for the scores, then the same lanes
// take feature columns to accumulate the 64 weighted rows, exchanging the
// weights through LDS, so every sum runs in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

constexpr int kMaxQW = 256 + 1024;  // d_h + d_r bound (d_h <= 256, d_c + d_r <= 1024)

template <typename T>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  return Store<T>::load(static_cast<const T*>(p), i);
}
template <typename T>
__device__ __forceinline__ void st(void* p, size_t i, float v) {
  Store<T>::store(static_cast<T*>(p), i, v);
}

// Gates and cumulative in-block partial merges of every token: one wave per
// (sequence, block of s tokens); lane l holds columns l, l + 64, ... of the
// running fp32 sum.  The gate is the merge kernels' own arithmetic.
template <typename T>
__global__ __launch_bounds__(256) void bwd_partials_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = (blockIdx.x * 256 + threadIdx.x) >> 6;
  const int nblk = (a.N + a.s - 1) / a.s;
  if (wv >= a.B * nblk) return;
  const int b = wv / nblk, blk = wv % nblk;
  const int W = a.d_c + a.d_r;
  const int t0 = blk * a.s, t1 = min(t0 + a.s, a.N);
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  for (int t = t0; t < t1; ++t) {
    const size_t row = static_cast<size_t>(b) * a.N + t;
    const float w = gate_of_token<T>(static_cast<const T*>(a.c) + row * a.d_c, a.pe + static_cast<size_t>(t) * a.d_c,
                                     a.w_hyp + static_cast<size_t>(t % a.s) * a.wh_stride, a.d_c, lane);
    if (lane == 0) a.gate[row] = w;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = lane + 64 * j;
      if (e >= W) break;
      const float x = e < a.d_c ? ld<T>(a.c, row * a.d_c + e) : ld<T>(a.k_r, row * a.d_r + (e - a.d_c));
      acc[j] = fmaf(w, x, acc[j]);
      st<T>(a.P, row * W + e, acc[j]);
    }
  }
}

// The same for d_c = 64 GE and d_r <= 64, with every load of a round of TB
// tokens in flight together: lane l holds elements l + 64 j of c_t, pe_t and
// the W_hyp row (the gate's inputs, which are also the merge's c columns) and
// element l of k^R_t; the gate is gate_from_lane_values (the same bits as
// gate_of_token), the running sums the same fmaf chain in token order.
template <typename T, int GE>
__global__ __launch_bounds__(256) void bwd_partials_lanes_kernel(BwdArgs a) {
  constexpr int TB = 4;
  const int lane = threadIdx.x & 63;
  const int wv = (blockIdx.x * 256 + threadIdx.x) >> 6;
  const int nblk = (a.N + a.s - 1) / a.s;
  if (wv >= a.B * nblk) return;
  const int b = wv / nblk, blk = wv % nblk;
  const int W = a.d_c + a.d_r;
  const int t0 = blk * a.s, t1 = min(t0 + a.s, a.N);
  const int r_l = min(lane, a.d_r > 0 ? a.d_r - 1 : 0);
  float acc[GE + 1];
#pragma unroll
  for (int j = 0; j <= GE; ++j) acc[j] = 0.f;
  for (int tb = t0; tb < t1; tb += TB) {
    float x[TB][GE], pv[TB][GE], wh[TB][GE], xr[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = min(tb + u, t1 - 1);  // past the block: re-read its last token (not used)
      const size_t row = static_cast<size_t>(b) * a.N + t;
      const float* whr = a.w_hyp + static_cast<size_t>(t % a.s) * a.wh_stride;
#pragma unroll
      for (int j = 0; j < GE; ++j) {
        x[u][j] = ld<T>(a.c, row * a.d_c + lane + 64 * j);
        pv[u][j] = a.pe[static_cast<size_t>(t) * a.d_c + lane + 64 * j];
        wh[u][j] = whr[lane + 64 * j];
      }
      xr[u] = a.d_r > 0 ? ld<T>(a.k_r, row * a.d_r + r_l) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = tb + u;
      if (t >= t1) break;
      const size_t row = static_cast<size_t>(b) * a.N + t;
      const float w = gate_from_lane_values<GE>(x[u], pv[u], wh[u]);
      if (lane == 0) a.gate[row] = w;
#pragma unroll
      for (int j = 0; j < GE; ++j) {
        acc[j] = fmaf(w, x[u][j], acc[j]);
        st<T>(a.P, row * W + lane + 64 * j, acc[j]);
      }
      acc[GE] = fmaf(w, xr[u], acc[GE]);
      if (lane < a.d_r) st<T>(a.P, row * W + a.d_c + lane, acc[GE]);
    }
  }
}

// Key row (0-based token) of the kk-th key query i (0-based) sees: the
// completed slots' last tokens s*m - 1 (m = 1..(i)/s, i.e. completed_slots of
// the 1-based query), then the query's own token.
__device__ __forceinline__ int key_row(int kk, int ncomp, int i, int s) { return kk < ncomp ? s * (kk + 1) - 1 : i; }

// Score and dO . V of query i against key row j for head h.
template <typename T>
__device__ __forceinline__ void score_and_dp(const BwdArgs& a, int b, int h, int j, const float* sq, const float* sdo,
                                             float& z, float& dp) {
  const int W = a.d_c + a.d_r, KV2 = 2 * a.H * a.d_h;
  const size_t rj = static_cast<size_t>(b) * a.N + j;
  float acc = 0.f, accv = 0.f;
  for (int e = 0; e < a.d_h; ++e) {
    acc = fmaf(sq[e], ld<T>(a.KV, rj * KV2 + h * a.d_h + e), acc);
    accv = fmaf(sdo[e], ld<T>(a.KV, rj * KV2 + a.H * a.d_h + h * a.d_h + e), accv);
  }
  for (int r = 0; r < a.d_r; ++r) acc = fmaf(sq[a.d_h + r], ld<T>(a.P, rj * W + a.d_c + r), acc);
  z = a.scale * acc;
  dp = accv;
}

// dQ of one (sequence, head, query): pass 1 gives lse and D with an online
// softmax over the query's keys, pass 2 the weighted sum of the key rows.
template <typename T>
__global__ __launch_bounds__(64) void bwd_dq_kernel(BwdArgs a) {
  __shared__ float sq[kMaxQW];
  __shared__ float sdo[256];
  __shared__ float sdq[kMaxQW];
  __shared__ float sds[64];
  __shared__ int srow[64];
  const int lane = threadIdx.x;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int QW = a.d_h + a.d_r, W = a.d_c + a.d_r;
  const size_t qi = (static_cast<size_t>(b) * a.N + i) * a.H + h;
  for (int e = lane; e < QW; e += 64) {
    sq[e] = e < a.d_h ? ld<T>(a.q_c, qi * a.d_h + e) : ld<T>(a.q_r, qi * a.d_r + (e - a.d_h));
    sdq[e] = 0.f;
  }
  for (int e = lane; e < a.d_h; e += 64) sdo[e] = ld<T>(a.d_o, qi * a.d_h + e);
  __syncthreads();
  const int ncomp = i / a.s;  // completed slots seen by the 1-based query i + 1
  const int nk = ncomp + 1;
  float m = -INFINITY, l = 0.f, dsum = 0.f;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int kk = k0 + lane;
    float z = -INFINITY, dp = 0.f;
    if (kk < nk) score_and_dp<T>(a, b, h, key_row(kk, ncomp, i, a.s), sq, sdo, z, dp);
    const float mn = fmaxf(m, wave_max(z));
    const float e = kk < nk ? expf(z - mn) : 0.f;
    const float f = expf(m - mn);
    l = l * f + wave_sum(e);
    dsum = dsum * f + wave_sum(e * dp);
    m = mn;
  }
  const float lse = m + logf(l), D = dsum / l;
  const size_t si = (static_cast<size_t>(b) * a.H + h) * a.N + i;
  if (lane == 0) {
    a.lse[si] = lse;
    a.D[si] = D;
  }
  const int KV2 = 2 * a.H * a.d_h;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int kk = k0 + lane;
    float ds = 0.f;
    int j = i;
    if (kk < nk) {
      float z, dp;
      j = key_row(kk, ncomp, i, a.s);
      score_and_dp<T>(a, b, h, j, sq, sdo, z, dp);
      ds = a.scale * expf(z - lse) * (dp - D);
    }
    sds[lane] = ds;
    srow[lane] = j;
    __syncthreads();
    const int cnt = min(64, nk - k0);
    for (int e = lane; e < QW; e += 64) {
      float acc = sdq[e];
      for (int k = 0; k < cnt; ++k) {
        const size_t rj = static_cast<size_t>(b) * a.N + srow[k];
        const float kv = e < a.d_h ? ld<T>(a.KV, rj * KV2 + h * a.d_h + e) : ld<T>(a.P, rj * W + a.d_c + (e - a.d_h));
        acc = fmaf(sds[k], kv, acc);
      }
      sdq[e] = acc;
    }
    __syncthreads();
  }
  for (int e = lane; e < QW; e += 64) {
    if (e < a.d_h)
      st<T>(a.g_q_c, qi * a.d_h + e, sdq[e]);
    else
      st<T>(a.g_q_r, qi * a.d_r + (e - a.d_h), sdq[e]);
  }
}

// dK^C, dK^R and dV of one (sequence, head, key token j): the queries that
// see key j are j itself and, when s | j + 1 (a block's last token, i.e. a
// completed slot), every later query.
template <typename T>
__global__ __launch_bounds__(64) void bwd_dkv_kernel(BwdArgs a) {
  __shared__ float sk[kMaxQW];
  __shared__ float sv[256];
  __shared__ float sdk[kMaxQW];
  __shared__ float sdv[256];
  __shared__ float sp[64];
  __shared__ float sds[64];
  const int lane = threadIdx.x;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int QW = a.d_h + a.d_r, W = a.d_c + a.d_r, KV2 = 2 * a.H * a.d_h;
  const size_t rj = static_cast<size_t>(b) * a.N + j;
  for (int e = lane; e < QW; e += 64) {
    sk[e] = e < a.d_h ? ld<T>(a.KV, rj * KV2 + h * a.d_h + e) : ld<T>(a.P, rj * W + a.d_c + (e - a.d_h));
    sdk[e] = 0.f;
  }
  for (int e = lane; e < a.d_h; e += 64) {
    sv[e] = ld<T>(a.KV, rj * KV2 + a.H * a.d_h + h * a.d_h + e);
    sdv[e] = 0.f;
  }
  __syncthreads();
  const int nq = (j + 1) % a.s == 0 ? a.N - j : 1;  // queries j .. j + nq - 1
  for (int q0 = 0; q0 < nq; q0 += 64) {
    const int i = j + q0 + lane;
    float p = 0.f, ds = 0.f;
    if (q0 + lane < nq) {
      const size_t qi = (static_cast<size_t>(b) * a.N + i) * a.H + h;
      float acc = 0.f, dp = 0.f;
      for (int e = 0; e < a.d_h; ++e) {
        acc = fmaf(ld<T>(a.q_c, qi * a.d_h + e), sk[e], acc);
        dp = fmaf(ld<T>(a.d_o, qi * a.d_h + e), sv[e], dp);
      }
      for (int r = 0; r < a.d_r; ++r) acc = fmaf(ld<T>(a.q_r, qi * a.d_r + r), sk[a.d_h + r], acc);
      const size_t si = (static_cast<size_t>(b) * a.H + h) * a.N + i;
      p = expf(a.scale * acc - a.lse[si]);
      ds = a.scale * p * (dp - a.D[si]);
    }
    sp[lane] = p;
    sds[lane] = ds;
    __syncthreads();
    const int cnt = min(64, nq - q0);
    for (int e = lane; e < QW; e += 64) {
      float acc = sdk[e];
      for (int k = 0; k < cnt; ++k) {
        const size_t qi = (static_cast<size_t>(b) * a.N + j + q0 + k) * a.H + h;
        const float qv = e < a.d_h ? ld<T>(a.q_c, qi * a.d_h + e) : ld<T>(a.q_r, qi * a.d_r + (e - a.d_h));
        acc = fmaf(sds[k], qv, acc);
      }
      sdk[e] = acc;
    }
    for (int e = lane; e < a.d_h; e += 64) {
      float acc = sdv[e];
      for (int k = 0; k < cnt; ++k) {
        const size_t qi = (static_cast<size_t>(b) * a.N + j + q0 + k) * a.H + h;
        acc = fmaf(sp[k], ld<T>(a.d_o, qi * a.d_h + e), acc);
      }
      sdv[e] = acc;
    }
    __syncthreads();
  }
  const int ldk = KV2 + a.H * a.d_r;
  for (int e = lane; e < QW; e += 64) {
    if (e < a.d_h)
      st<T>(a.dKV, rj * ldk + h * a.d_h + e, sdk[e]);
    else
      st<T>(a.dKV, rj * ldk + KV2 + h * a.d_r + (e - a.d_h), sdk[e]);
  }
  for (int e = lane; e < a.d_h; e += 64) st<T>(a.dKV, rj * ldk + a.H * a.d_h + h * a.d_h + e, sdv[e]);
}

// Reverse in-block sum of dP and the gate backward: one wave per (sequence,
// block of s tokens), its tokens last to first; lane l holds columns l,
// l + 64, ... (JW of them) of the running sum G.  Tokens go in rounds of TB
// whose loads are all issued before the round's sequential part (the
// running sum, one wave reduction per token, the stores).  Writes dc, dk^R
// and du of every token.  TB = s for s = 3 (one round, no re-read token).
template <typename T, int JW, int TB>
__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = (blockIdx.x * 256 + threadIdx.x) >> 6;
  const int nblk = (a.N + a.s - 1) / a.s;
  if (wv >= a.B * nblk) return;
  const int b = wv / nblk, blk = wv % nblk;
  const int W = a.d_c + a.d_r, KV2 = 2 * a.H * a.d_h, ldk = KV2 + a.H * a.d_r;
  const int t0 = blk * a.s, t1 = min(t0 + a.s, a.N);
  float G[JW];
#pragma unroll
  for (int j = 0; j < JW; ++j) G[j] = 0.f;
  for (int tt = t1 - 1; tt >= t0; tt -= TB) {
    float x[TB][JW], dP[TB][JW], w[TB];
    // Every load of the round is issued unconditionally (indices clamped into
    // the row, values selected afterwards), so that they are in flight
    // together rather than one round trip each behind a branch.  The rope
    // gradient of column r (lane r < d_r) is summed over the heads in head
    // order (the first 8 heads' loads together, further heads after).
    float rp[TB], xr[TB];
    const int r_l = min(lane, a.d_r > 0 ? a.d_r - 1 : 0);
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      // tokens before the block's first re-read that token (not used)
      const size_t row = static_cast<size_t>(b) * a.N + max(tt - u, t0);
      w[u] = a.gate[row];
#pragma unroll
      for (int j = 0; j < JW; ++j) {
        const int ec = min(lane + 64 * j, a.d_c - 1);
        dP[u][j] = a.dPc[row * a.d_c + ec];
        x[u][j] = ld<T>(a.c, row * a.d_c + ec);
      }
      rp[u] = 0.f;
      xr[u] = 0.f;
    }
    if (a.d_r > 0) {
      float v[TB][8];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const size_t row = static_cast<size_t>(b) * a.N + max(tt - u, t0);
        xr[u] = ld<T>(a.k_r, row * a.d_r + r_l);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[u][k] = ld<T>(a.dKV, row * ldk + KV2 + min(k, a.H - 1) * a.d_r + r_l);
      }
#pragma unroll
      for (int u = 0; u < TB; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < a.H) rp[u] += v[u][k];
    }
    if (a.H > 8) {
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const size_t row = static_cast<size_t>(b) * a.N + max(tt - u, t0);
        for (int hh = 8; hh < a.H; ++hh) rp[u] += ld<T>(a.dKV, row * ldk + KV2 + hh * a.d_r + r_l);
      }
    }
    // columns e >= d_c: the rope values of lane e - d_c
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int e = lane + 64 * j;
      if (64 * j + 63 < a.d_c) continue;  // (uniform) no rope column in this j
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int src = e - a.d_c;
        const float pr = a.d_c % 64 == 0 ? rp[u] : __shfl(rp[u], max(src, 0), 64);
        const float px = a.d_c % 64 == 0 ? xr[u] : __shfl(xr[u], max(src, 0), 64);
        if (e >= a.d_c) {
          dP[u][j] = e < W ? pr : 0.f;
          x[u][j] = e < W ? px : 0.f;
        }
      }
    }
    // the W_hyp values the stores below use (row (t - 1) mod s per token when
    // there is one row per place), loaded with the round's other loads
    float whv[TB][JW];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const float* whr = a.w_hyp + static_cast<size_t>(max(tt - u, t0) % a.s) * a.wh_stride;
#pragma unroll
      for (int j = 0; j < JW; ++j) whv[u][j] = whr[min(lane + 64 * j, a.d_c - 1)];
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = tt - u;
      if (t < t0) break;
      const size_t row = static_cast<size_t>(b) * a.N + t;
      float dwl = 0.f;
#pragma unroll
      for (int j = 0; j < JW; ++j) {
        G[j] += dP[u][j];
        dwl = fmaf(G[j], x[u][j], dwl);
      }
      const float du = wave_sum(dwl) * w[u] * (1.f - w[u]);
      if (lane == 0) a.du[row] = du;
#pragma unroll
      for (int j = 0; j < JW; ++j) {
        const int e = lane + 64 * j;
        if (e < a.d_c)
          st<T>(a.g_c, row * a.d_c + e, fmaf(du, whv[u][j], w[u] * G[j]));
        else if (e < W)
          st<T>(a.g_k_r, row * a.d_r + (e - a.d_c), w[u] * G[j]);
      }
    }
  }
}

// Partial sums of dW_hyp = sum_r du_r (c_r + pe_t(r)) over one chunk of rows:
// 64 columns x 4 row groups per workgroup, the groups added in a fixed order.
// With one W_hyp row per place in the block (wh_rows = s), blockIdx.z is the
// place and takes the tokens t with t mod s == blockIdx.z.
template <typename T>
__global__ __launch_bounds__(256) void dwhyp_kernel(BwdArgs a, int rows_per_split) {
  __shared__ float red[4][64];
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cl;
  const int R = a.B * a.N;
  const int r0 = blockIdx.y * rows_per_split, r1 = min(R, r0 + rows_per_split);
  const int place = blockIdx.z;
  float acc = 0.f;
  // eight rows' loads in flight at a time (row indices clamped, the rows
  // past r1 or of another place skipped), added in row order
  if (col < a.d_c)
    for (int rb = r0 + rg; rb < r1; rb += 32) {
      float dv[8], cv[8], pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = min(rb + 4 * k, r1 - 1), t = r % a.N;
        dv[k] = a.du[r];
        cv[k] = ld<T>(a.c, static_cast<size_t>(r) * a.d_c + col);
        pv[k] = a.pe[static_cast<size_t>(t) * a.d_c + col];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = rb + 4 * k;
        if (r < r1 && (a.wh_rows == 1 || (r % a.N) % a.s == place)) acc = fmaf(dv[k], cv[k] + pv[k], acc);
      }
    }
  red[rg][cl] = acc;
  __syncthreads();
  if (rg == 0 && col < a.d_c)
    a.wh_part[(static_cast<size_t>(blockIdx.y) * a.wh_rows + place) * a.d_c + col] =
        (red[0][cl] + red[1][cl]) + (red[2][cl] + red[3][cl]);
}

template <typename T>
__global__ __launch_bounds__(256) void transpose_w_kernel(int KV2h, int d_c, const T* w_uk, const T* w_uv, T* wt) {
  const int idx = blockIdx.x * 256 + threadIdx.x;  // over the output [d_c, 2 KV2h]
  const int K2 = 2 * KV2h;
  if (idx >= d_c * K2) return;
  const int n = idx / K2, k = idx % K2;
  wt[idx] = k < KV2h ? w_uk[static_cast<size_t>(k) * d_c + n] : w_uv[static_cast<size_t>(k - KV2h) * d_c + n];
}

// Split-K product over rows: part[split][m][n] = sum over the split's rows r
// of A[r, m] Bm[r, n].  64 x 64 output tile, 16 rows per LDS stage, each
// thread a 4 x 4 block.
template <typename T>
__global__ __launch_bounds__(256) void wgrad_kernel(int R, int M, int N, const T* A, int lda, const T* Bm, int ldb,
                                                    float* part, int rows_per_split) {
  __shared__ float sa[16][64 + 4];
  __shared__ float sb[16][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64, split = blockIdx.z;
  const int r0 = split * rows_per_split, r1 = min(R, r0 + rows_per_split);
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int r = r0; r < r1; r += 16) {
    // 16 rows x 64 columns of each operand: 4 elements per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, rr = idx >> 6, cc = idx & 63;
      const int row = r + rr;
      sa[rr][cc] = (row < r1 && m0 + cc < M) ? Store<T>::load(A, static_cast<size_t>(row) * lda + m0 + cc) : 0.f;
      sb[rr][cc] = (row < r1 && n0 + cc < N) ? Store<T>::load(Bm, static_cast<size_t>(row) * ldb + n0 + cc) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = sa[rr][ty * 4 + i];
        bv[i] = sb[rr][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) part[(static_cast<size_t>(split) * M + m) * N + n] = acc[i][j];
    }
  }
}

// out rows m < m0_rows go to out0[m], the rest to out1[m - m0_rows].
__global__ __launch_bounds__(256) void sum_split_rows_kernel(const float* part, int splits, int M, int N, float* out0,
                                                             int m0_rows, float* out1) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t n = static_cast<size_t>(M) * N;
  if (idx >= n) return;
  // eight parts' loads in flight at a time, added in part order
  float acc = 0.f;
  for (int p0 = 0; p0 < splits; p0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = part[min(p0 + k, splits - 1) * n + idx];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (p0 + k < splits) acc += v[k];
  }
  const int m = static_cast<int>(idx / N);
  if (m < m0_rows)
    out0[idx] = acc;
  else
    out1[idx - static_cast<size_t>(m0_rows) * N] = acc;
}

// out[i] = sum over p of part[p n + i]: 64 columns x 4 groups of parts per
// workgroup, the groups added in a fixed order.
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* part, int parts, int n, float* out) {
  __shared__ float red[4][64];
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cl;
  float acc = 0.f;
  // eight parts' loads in flight at a time, added in part order
  if (col < n)
    for (int p0 = rg; p0 < parts; p0 += 32) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = part[static_cast<size_t>(min(p0 + 4 * k, parts - 1)) * n + col];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (p0 + 4 * k < parts) acc += v[k];
    }
  red[rg][cl] = acc;
  __syncthreads();
  if (rg == 0 && col < n) out[col] = (red[0][cl] + red[1][cl]) + (red[2][cl] + red[3][cl]);
}

// ---------------------------------------------------------------------------
// MFMA pieces (bf16 storage, 32x32x16 bf16 MFMA with fp32 accumulation).
//
// Accumulator layout of a 32x32 product C (f32x16 per lane): lane
// (grp = lane / 32, c32 = lane % 32) holds column c32, rows 8 (i / 4) +
// 4 grp + i % 4 for i = 0..15.  A product that contracts over those 32 rows
// takes them 16 at a time (chunk c) as the B operand, with contraction index
// kappa = 8 grp + r standing for row 16 c + 4 grp + r (r < 4) or
// 16 c + 8 + 4 grp + (r - 4) (r >= 4); its A operand is read from a
// row-major LDS tile with that same row order by transposing LDS reads.  The
// same transposing read gives the B operand of a product whose two operands
// both contract over the rows of LDS tiles.
// ---------------------------------------------------------------------------
constexpr int BTS = 64;  // rows of one LDS tile: slots (dQ) or queries (dK, dV)

// Chunk c (0 or 1) of one 32-row accumulator x: its rows 16 c .. 16 c + 15.
__device__ __forceinline__ bf16x8 acc_chunk_bf16(const f32x16& x, int c) {
  const int jb = 2 * c;
  u16x8 pk;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pk[r] = f32_to_bf16_bits(x[4 * jb + r]);
    pk[4 + r] = f32_to_bf16_bits(x[4 * (jb + 1) + r]);
  }
  return __builtin_bit_cast(bf16x8, pk);
}

// Operand with rows (A) or columns (B) = tile columns 32 ft .. 32 ft + 31,
// contraction over the tile's rows 16 c .. 16 c + 15 in acc_chunk_bf16's order.
__device__ __forceinline__ bf16x8 lds_tr_operand(const uint16_t* tile, int pitch, int c, int ft, int lane) {
  const int q16 = lane >> 4, k16 = lane & 15;
  const int sb0 = 16 * c + 4 * (q16 >> 1);
  const int col0 = 32 * ft + 16 * (q16 & 1);
  const uint16_t* base = tile + (sb0 + (k16 >> 2)) * pitch + col0 + 4 * (k16 & 3);
  const s16x4 lo4 = lds_read_tr16(base);
  const s16x4 hi4 = lds_read_tr16(base + 8 * pitch);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float dot8_bf16(const uint4 x, const uint4 y) {
  const u16x8 a = __builtin_bit_cast(u16x8, x), b = __builtin_bit_cast(u16x8, y);
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) acc = fmaf(bf16_bits_to_f32(a[r]), bf16_bits_to_f32(b[r]), acc);
  return acc;
}

__device__ __forceinline__ uint4 scale8_bf16(const uint4 x, float f) {
  const u16x8 a = __builtin_bit_cast(u16x8, x);
  u16x8 o;
#pragma unroll
  for (int r = 0; r < 8; ++r) o[r] = f32_to_bf16_bits(bf16_bits_to_f32(a[r]) * f);
  return __builtin_bit_cast(uint4, o);
}

__device__ __forceinline__ uint2 pack4_bf16(float x0, float x1, float x2, float x3) {
  return uint2{static_cast<uint32_t>(f32_to_bf16_bits(x0)) | (static_cast<uint32_t>(f32_to_bf16_bits(x1)) << 16),
               static_cast<uint32_t>(f32_to_bf16_bits(x2)) | (static_cast<uint32_t>(f32_to_bf16_bits(x3)) << 16)};
}

__device__ __forceinline__ void unpack4_bf16(const uint2 v, float (&x)[4]) {
  x[0] = __uint_as_float(v.x << 16);
  x[1] = __uint_as_float(v.x & 0xffff0000u);
  x[2] = __uint_as_float(v.y << 16);
  x[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Workgroup -> (pair, tile), XCD-aware.  Workgroup L runs on XCD L % 8; with
// B*H a multiple of 8 an XCD takes the (sequence, head) pairs x, x + 8, ...
// one after another, so its concurrent workgroups share a few pairs' rows in
// its L2.  `high_first` deals a pair's tiles from the last one down.
__device__ __forceinline__ void pair_and_tile(int L, int npair, int ntile, bool high_first, int& pair, int& tile) {
  int k;
  if (npair % 8 == 0) {
    k = L >> 3;
    pair = (L & 7) + 8 * (k / ntile);
    k %= ntile;
  } else {
    pair = L % npair;
    k = L / npair;
  }
  tile = high_first ? ntile - 1 - k : k;
}

// Split-K product over rows on MFMA (bf16): part[split][m][n] = sum over the
// split's rows r of A[r, m] Bm[r, n], a 128 x 128 tile per workgroup (four
// waves of 64 x 64, 32x32x16 MFMA).  Both operands contract over the token
// rows, which run along the rows of their LDS tiles, so both are read by the
// transposing LDS read in one and the same row order.  Rows past the split's
// end read as zero through bounded buffer resources.
constexpr int WGT = 64;  // token rows per LDS stage

__global__ __launch_bounds__(256) void wgrad_mfma_kernel(int R, int M, int N, const uint16_t* A, int lda,
                                                         const uint16_t* Bm, int ldb, float* part,
                                                         int rows_per_split) {
  constexpr int TP = 128 + 8;
  __shared__ __align__(16) uint16_t sA[2][WGT * TP];
  __shared__ __align__(16) uint16_t sB[2][WGT * TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int grp = lane >> 5, c32 = lane & 31;
  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 128, split = blockIdx.z;
  const int r0 = split * rows_per_split, nrows = max(0, min(R, r0 + rows_per_split) - r0);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + static_cast<size_t>(r0) * lda + m0), static_cast<short>(0),
      nrows > 0 ? ((nrows - 1) * lda + 128) * 2 : 0, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Bm + static_cast<size_t>(r0) * ldb + n0), static_cast<short>(0),
      nrows > 0 ? ((nrows - 1) * ldb + 128) * 2 : 0, kBufferRsrcWord3);
  constexpr int CPT = WGT * 128 / 8 / 256;  // 16-byte chunks per thread and operand
  int off_a[CPT], off_b[CPT], lds_o[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i, row = c / 16, cc = c % 16;
    off_a[i] = (row * lda + cc * 8) * 2;
    off_b[i] = (row * ldb + cc * 8) * 2;
    lds_o[i] = row * TP + cc * 8;
  }
  uint4 ra[CPT], rb[CPT];
  auto load = [&](int k0) {
    const int sa = k0 * lda * 2, sb = k0 * ldb * 2;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_a, off_a[i], sa, 0);
      ra[i] = uint4{v[0], v[1], v[2], v[3]};
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs_b, off_b[i], sb, 0);
      rb[i] = uint4{u[0], u[1], u[2], u[3]};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      *reinterpret_cast<uint4*>(sA[buf] + lds_o[i]) = ra[i];
      *reinterpret_cast<uint4*>(sB[buf] + lds_o[i]) = rb[i];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  int buf = 0;
  if (nrows > 0) {
    load(0);
    store(0);
    if (WGT < nrows) load(WGT);
  }
  __syncthreads();
  for (int k0 = 0; k0 < nrows; k0 += WGT, buf ^= 1) {
    if (k0 + WGT < nrows) {
      store(buf ^ 1);
      if (k0 + 2 * WGT < nrows) load(k0 + 2 * WGT);
    }
#pragma unroll
    for (int c = 0; c < WGT / 16; ++c) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = lds_tr_operand(sA[buf], TP, c, 2 * wm + i, lane);
        bv[i] = lds_tr_operand(sB[buf], TP, c, 2 * wn + i, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // acc[i][j][e]: row m0 + 64 wm + 32 i + 8 (e / 4) + 4 grp + e % 4, column n0 + 64 wn + 32 j + c32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (e / 4) + 4 * grp + (e % 4);
        const int n = n0 + 64 * wn + 32 * j + c32;
        part[(static_cast<size_t>(split) * M + m) * N + n] = acc[i][j][e];
      }
}

// dQ of 128 queries of one (sequence, head): 4 waves of 32 queries, two
// passes over 64-slot tiles (K^C | P^R and V in LDS, the next tile in flight).
//   Pass 1: S^T = K Q^T and dP^T = V dO^T give, with an online maximum, each
//           query's normaliser lse (log2 domain, the diagonal key included)
//           and D_i = sum_j p_ij dp_ij from the same fp32 probabilities, so
//           that every row of dS sums to zero as it should.
//   Pass 2: dS^T = tau P^T (dP^T - D), dQ^T += [K^C | P^R]^T dS^T.
// Between them each query's diagonal key (j = i) gives p_ii and ds_ii (kept
// for the dK/dV kernel), the whole dK/dV rows of tokens that are not a
// completed slot's key, and dQ's diagonal term ds_ii [K^C_i ; P^R_i].
template <int DH, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_mfma_kernel(BwdArgs a) {
  constexpr int DQK = DH + DR, KK = DQK / 16, KD = DH / 16, FT = DQK / 32;
  constexpr int KP = DQK + 8, VP = DH + 8;
  __shared__ __align__(16) uint16_t sKb[2][BTS * KP];
  __shared__ __align__(16) uint16_t sVb[2][BTS * VP];

  int pair, qt;
  pair_and_tile(blockIdx.x, a.B * a.H, a.nqt, true, pair, qt);
  const int h = pair % a.H, b = pair / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 5, c32 = lane & 31;
  const int N = a.N, H = a.H, s = a.s, W = a.d_c + DR, KV2 = 2 * H * DH, ldk = KV2 + H * DR;
  const int q0 = qt * 128, qw0 = q0 + wave * 32;
  const float qk = a.scale * kLog2e;
  const int qi = qw0 + c32;
  const bool qok = qi < N;

  const uint16_t* qc = static_cast<const uint16_t*>(a.q_c);
  const uint16_t* qr = static_cast<const uint16_t*>(a.q_r);
  const uint16_t* dO = static_cast<const uint16_t*>(a.d_o);
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* vv = static_cast<const uint16_t*>(a.v) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* Pb = static_cast<const uint16_t*>(a.P) + static_cast<size_t>(b) * N * W;
  const size_t qrow = (static_cast<size_t>(b) * N + (qok ? qi : 0)) * H + h;

  // prologue: operands of this lane's query and its diagonal key
  bf16x8 qreg[KK], dreg[KD];
  float zp = 0.f, dpp = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int d0 = 16 * kk + 8 * grp;
    uint4 qv = uint4{0u, 0u, 0u, 0u}, kv = uint4{0u, 0u, 0u, 0u};
    if (qok) {
      if (d0 < DH) {
        qv = *reinterpret_cast<const uint4*>(qc + qrow * DH + d0);
        kv = *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(qi) * DH + d0);
      } else {
        qv = *reinterpret_cast<const uint4*>(qr + qrow * DR + (d0 - DH));
        kv = *reinterpret_cast<const uint4*>(Pb + static_cast<size_t>(qi) * W + a.d_c + (d0 - DH));
      }
    }
    qreg[kk] = __builtin_bit_cast(bf16x8, qv);
    zp += dot8_bf16(qv, kv);
  }
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    const int d0 = 16 * kk + 8 * grp;
    uint4 dv = uint4{0u, 0u, 0u, 0u}, vr = uint4{0u, 0u, 0u, 0u};
    if (qok) {
      dv = *reinterpret_cast<const uint4*>(dO + qrow * DH + d0);
      vr = *reinterpret_cast<const uint4*>(vv + static_cast<size_t>(qi) * DH + d0);
    }
    dreg[kk] = __builtin_bit_cast(bf16x8, dv);
    dpp += dot8_bf16(dv, vr);
  }
  zp += __shfl_xor(zp, 32, 64);
  dpp += __shfl_xor(dpp, 32, 64);

  // completed slots seen by the workgroup's / this wave's last query, and by
  // every query of this wave
  const int nk = (min(q0 + 128, N) - 1) / s;
  const int nk_w = qw0 < N ? (min(qw0 + 32, N) - 1) / s : 0;
  const int full_w = qw0 / s;
  // completed slot j (0-based) is visible to this lane's query qi iff
  // s (j + 1) <= qi, i.e. j < vis
  const int vis = qi / s;

  // slot m's keys are token row s m + s - 1; loads past the last completed
  // slot's row read as zero through bounded buffer resources
  constexpr int KN = BTS * DH / 8 / 256, RN = BTS * DR / 8 / 256;
  static_assert(KN * 256 == BTS * DH / 8 && RN * 256 == BTS * DR / 8, "chunks per thread");
  const int rows_end = s * nk;
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kc), static_cast<short>(0), rows_end * DH * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vv), static_cast<short>(0), rows_end * DH * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Pb + a.d_c), static_cast<short>(0), rows_end > 0 ? (rows_end - 1) * W * 2 + DR * 2 : 0,
      kBufferRsrcWord3);
  int off_k[KN], off_r[RN], lds_k[KN], lds_r[RN], lds_v[KN];
#pragma unroll
  for (int i = 0; i < KN; ++i) {
    const int c = tid + 256 * i, row = c / (DH / 8), cc = c % (DH / 8);
    off_k[i] = ((s * row + s - 1) * DH + cc * 8) * 2;
    lds_k[i] = row * KP + cc * 8;
    lds_v[i] = row * VP + cc * 8;
  }
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = tid + 256 * i, row = c / (DR / 8), cc = c % (DR / 8);
    off_r[i] = ((s * row + s - 1) * W + cc * 8) * 2;
    lds_r[i] = row * KP + DH + cc * 8;
  }
  uint4 pk[KN], pr[RN], pv[KN];
  auto load_tile = [&](int j0) {
    const int so_kv = s * j0 * DH * 2, so_r = s * j0 * W * 2;
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_k, off_k[i], so_kv, 0);
      pk[i] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int i = 0; i < RN; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_r, off_r[i], so_r, 0);
      pr[i] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_v, off_k[i], so_kv, 0);
      pv[i] = uint4{v[0], v[1], v[2], v[3]};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KN; ++i) *reinterpret_cast<uint4*>(sKb[buf] + lds_k[i]) = pk[i];
#pragma unroll
    for (int i = 0; i < RN; ++i) *reinterpret_cast<uint4*>(sKb[buf] + lds_r[i]) = pr[i];
#pragma unroll
    for (int i = 0; i < KN; ++i) *reinterpret_cast<uint4*>(sVb[buf] + lds_v[i]) = pv[i];
  };
  // S^T and dP^T of one 32-slot half (rt) of the tile in LDS
  auto scores = [&](const uint16_t* sK, const uint16_t* sV, int rt, f32x16& sc, f32x16& dp) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sK + (32 * rt + c32) * KP + 16 * kk + 8 * grp);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[kk], sc, 0, 0, 0);
    }
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(sV + (32 * rt + c32) * VP + 16 * kk + 8 * grp);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dreg[kk], dp, 0, 0, 0);
    }
  };
  // one sweep over the slot tiles; body(sK, sV, j0) runs on the tiles this
  // wave's queries see
  auto sweep = [&](auto body) {
    int buf = 0;
    if (nk > 0) {
      load_tile(0);
      store_tile(0);
      if (BTS < nk) load_tile(BTS);
    }
    __syncthreads();
    for (int j0 = 0; j0 < nk; j0 += BTS, buf ^= 1) {
      if (j0 + BTS < nk) {
        store_tile(buf ^ 1);
        if (j0 + 2 * BTS < nk) load_tile(j0 + 2 * BTS);
      }
      if (j0 < nk_w) body(sKb[buf], sVb[buf], j0);
      __syncthreads();
    }
  };

  // pass 1: online normaliser and D, starting from the diagonal key
  float m = zp * qk;                  // running maximum (log2 units), the same in both lane halves
  float ls = grp == 0 ? 1.f : 0.f;    // this lane's share of sum exp2(z - m)
  float dsum = grp == 0 ? dpp : 0.f;  // and of sum exp2(z - m) dp
  sweep([&](const uint16_t* sK, const uint16_t* sV, int j0) {
    const bool boundary = j0 + BTS > full_w;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 sc, dp;
      scores(sK, sV, rt, sc, dp);
      if (boundary) {
        // slot j0 + 32 rt + 8 (i / 4) + 4 grp + i % 4 is hidden iff >= vis
        const int rel = vis - j0 - 32 * rt - 4 * grp;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i / 4) + (i % 4) >= rel) sc[i] = -INFINITY;
      }
      // the maximum of the raw scores, scaled once (tau log2 e > 0: the
      // scaled scores have the same maximum); each score is scaled inside
      // its exponent's fma
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m, mx * qk);
      const float f = fast_exp2(m - mn);
      ls *= f;
      dsum *= f;
      m = mn;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(fmaf(sc[i], qk, -m));
        ls += e;
        dsum = fmaf(e, dp[i], dsum);
      }
    }
  });
  const float L = ls + __shfl_xor(ls, 32, 64);
  const float lse2 = qok ? m + log2f(L) : INFINITY;
  const float Dq = qok ? (dsum + __shfl_xor(dsum, 32, 64)) / L : 0.f;
  // pass 2's exponent offset: tau p = exp2(z tau log2 e - lse2 + log2 tau)
  const float lts = log2f(a.scale) - lse2;
  const float pii = qok ? fast_exp2(fmaf(zp, qk, -lse2)) : 0.f;
  const float dsii = a.scale * pii * (dpp - Dq);
  const size_t si = (static_cast<size_t>(b) * H + h) * N + (qok ? qi : 0);
  if (qok && grp == 0) {
    a.lse[si] = lse2;
    a.D[si] = Dq;
    a.pd[si] = pii;
    a.dsd[si] = dsii;
  }
  if (qok && (qi + 1) % s != 0) {
    // not a completed slot's key: the diagonal is its only query
    uint16_t* row = static_cast<uint16_t*>(a.dKV) + (static_cast<size_t>(b) * N + qi) * ldk;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int d0 = 16 * kk + 8 * grp;
      uint16_t* dst = d0 < DH ? row + h * DH + d0 : row + KV2 + h * DR + (d0 - DH);
      *reinterpret_cast<uint4*>(dst) = scale8_bf16(__builtin_bit_cast(uint4, qreg[kk]), dsii);
    }
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int d0 = 16 * kk + 8 * grp;
      *reinterpret_cast<uint4*>(row + H * DH + h * DH + d0) = scale8_bf16(__builtin_bit_cast(uint4, dreg[kk]), pii);
    }
  }
  // dQ^T (rows: features, column: this lane's query) starts at ds_ii K_i
  f32x16 dq[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f0 = 32 * ft + 8 * j + 4 * grp;
      uint2 kv = uint2{0u, 0u};
      if (qok)
        kv = f0 < DH ? *reinterpret_cast<const uint2*>(kc + static_cast<size_t>(qi) * DH + f0)
                     : *reinterpret_cast<const uint2*>(Pb + static_cast<size_t>(qi) * W + a.d_c + (f0 - DH));
      float k4[4];
      unpack4_bf16(kv, k4);
#pragma unroll
      for (int r = 0; r < 4; ++r) dq[ft][4 * j + r] = dsii * k4[r];
    }
  }

  // pass 2: dS^T and dQ^T
  sweep([&](const uint16_t* sK, const uint16_t* sV, int j0) {
    const bool boundary = j0 + BTS > full_w;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 sc, dp;
      scores(sK, sV, rt, sc, dp);
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = fast_exp2(fmaf(sc[i], qk, lts));  // tau p
      if (boundary) {
        const int rel = vis - j0 - 32 * rt - 4 * grp;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i / 4) + (i % 4) >= rel) sc[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] *= dp[i] - Dq;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 db = acc_chunk_bf16(sc, c);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
          dq[ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand(sK, KP, 2 * rt + c, ft, lane), db, dq[ft],
                                                           0, 0, 0);
      }
    }
  });

  if (qok) {
    uint16_t* gqc = static_cast<uint16_t*>(a.g_q_c) + qrow * DH;
    uint16_t* gqr = static_cast<uint16_t*>(a.g_q_r) + qrow * DR;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f0 = 32 * ft + 8 * j + 4 * grp;
        const uint2 v = pack4_bf16(dq[ft][4 * j], dq[ft][4 * j + 1], dq[ft][4 * j + 2], dq[ft][4 * j + 3]);
        *reinterpret_cast<uint2*>(f0 < DH ? gqc + f0 : gqr + (f0 - DH)) = v;
      }
  }
}

// dK^C, dK^R and dV of 128 completed slots of one (sequence, head): 4 waves
// of 32 slots, the slot keys and values held in registers as B operands.  The
// loop runs over 64-query tiles (q^C | q^R, dO, lse and D in LDS, the next
// tile in flight) from the first query that sees the workgroup's first slot,
// each tile as two 32-query halves:
//   S = Q K^T, dP = dO V^T, P = exp2(S tau log2 e - lse) where visible,
//   dS = tau P (dP - D),  dV^T += dO^T P,  dK^T += Q^T dS.
// The epilogue adds each slot token's own diagonal query (p_jj dO_j and
// ds_jj q_j) before storing the rows.
template <int DH, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkv_mfma_kernel(BwdArgs a, int nslots, int nst) {
  constexpr int DQK = DH + DR, KK = DQK / 16, KD = DH / 16, FT = DQK / 32, DT = DH / 32;
  constexpr int QP = DQK + 8, OP = DH + 8;
  __shared__ __align__(16) uint16_t sQb[2][BTS * QP];
  __shared__ __align__(16) uint16_t sOb[2][BTS * OP];
  __shared__ __align__(16) float sLb[2][BTS];
  __shared__ __align__(16) float sDb[2][BTS];

  int pair, st;
  pair_and_tile(blockIdx.x, a.B * a.H, nst, false, pair, st);
  const int h = pair % a.H, b = pair / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 5, c32 = lane & 31;
  const int N = a.N, H = a.H, s = a.s, W = a.d_c + DR, KV2 = 2 * H * DH, ldk = KV2 + H * DR;
  const float qk = a.scale * kLog2e;
  const int ms0 = st * 128, msw = ms0 + 32 * wave;
  const int m = msw + c32;
  const bool mok = m < nslots;
  const int jt = s * (m + 1) - 1;  // the slot's key token
  const int qm = jt + 1;           // the first query that sees the slot

  const uint16_t* qc = static_cast<const uint16_t*>(a.q_c);
  const uint16_t* qr = static_cast<const uint16_t*>(a.q_r);
  const uint16_t* dO = static_cast<const uint16_t*>(a.d_o);
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* vv = static_cast<const uint16_t*>(a.v) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* Pb = static_cast<const uint16_t*>(a.P) + static_cast<size_t>(b) * N * W;
  const float* lse2 = a.lse + (static_cast<size_t>(b) * H + h) * N;
  const float* Dv = a.D + (static_cast<size_t>(b) * H + h) * N;

  bf16x8 kreg[KK], vreg[KD];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int d0 = 16 * kk + 8 * grp;
    uint4 kv = uint4{0u, 0u, 0u, 0u};
    if (mok)
      kv = d0 < DH ? *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(jt) * DH + d0)
                   : *reinterpret_cast<const uint4*>(Pb + static_cast<size_t>(jt) * W + a.d_c + (d0 - DH));
    kreg[kk] = __builtin_bit_cast(bf16x8, kv);
  }
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    const int d0 = 16 * kk + 8 * grp;
    uint4 vr = uint4{0u, 0u, 0u, 0u};
    if (mok) vr = *reinterpret_cast<const uint4*>(vv + static_cast<size_t>(jt) * DH + d0);
    vreg[kk] = __builtin_bit_cast(bf16x8, vr);
  }
  f32x16 dvt[DT], dkt[FT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dvt[t][i] = 0.f;
#pragma unroll
  for (int t = 0; t < FT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkt[t][i] = 0.f;

  // query tiles: queries of this (sequence, head) are rows q of q_c / q_r / dO
  // at element (b N + q) H + h; rows past N read as zero
  constexpr int CN = BTS * DH / 8 / 256, CR = BTS * DR / 8 / 256;
  static_assert(CN * 256 == BTS * DH / 8 && CR * 256 == BTS * DR / 8, "chunks per thread");
  const size_t rowbase = static_cast<size_t>(b) * N * H + h;
  const __amdgpu_buffer_rsrc_t rs_qc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(qc + rowbase * DH), static_cast<short>(0), ((N - 1) * H * DH + DH) * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(qr + rowbase * DR), static_cast<short>(0), ((N - 1) * H * DR + DR) * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_do = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(dO + rowbase * DH), static_cast<short>(0), ((N - 1) * H * DH + DH) * 2, kBufferRsrcWord3);
  int off_c[CN], off_rr[CR], lq_c[CN], lq_r[CR], lo_c[CN];
#pragma unroll
  for (int i = 0; i < CN; ++i) {
    const int c = tid + 256 * i, row = c / (DH / 8), cc = c % (DH / 8);
    off_c[i] = (row * H * DH + cc * 8) * 2;
    lq_c[i] = row * QP + cc * 8;
    lo_c[i] = row * OP + cc * 8;
  }
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    const int c = tid + 256 * i, row = c / (DR / 8), cc = c % (DR / 8);
    off_rr[i] = (row * H * DR + cc * 8) * 2;
    lq_r[i] = row * QP + DH + cc * 8;
  }
  uint4 tq[CN], tr[CR], td[CN];
  float tl = 0.f;
  auto load_tile = [&](int q0) {
    const int so_c = q0 * H * DH * 2, so_r = q0 * H * DR * 2;
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_qc, off_c[i], so_c, 0);
      tq[i] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_qr, off_rr[i], so_r, 0);
      tr[i] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs_do, off_c[i], so_c, 0);
      td[i] = uint4{v[0], v[1], v[2], v[3]};
    }
    // threads 0..63 take lse (+inf past N: probability 0), 64..127 take D
    if (tid < 2 * BTS) {
      const int q = q0 + (tid & (BTS - 1));
      tl = tid < BTS ? (q < N ? lse2[q] : INFINITY) : (q < N ? Dv[q] : 0.f);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CN; ++i) *reinterpret_cast<uint4*>(sQb[buf] + lq_c[i]) = tq[i];
#pragma unroll
    for (int i = 0; i < CR; ++i) *reinterpret_cast<uint4*>(sQb[buf] + lq_r[i]) = tr[i];
#pragma unroll
    for (int i = 0; i < CN; ++i) *reinterpret_cast<uint4*>(sOb[buf] + lo_c[i]) = td[i];
    if (tid < BTS)
      sLb[buf][tid] = tl;
    else if (tid < 2 * BTS)
      sDb[buf][tid - BTS] = tl;
  };

  // the first query that sees slot m is token s (m + 1) (0-based)
  const int qbeg = (s * (ms0 + 1)) / BTS * BTS;
  const bool wave_on = msw < nslots;
  const int qfirst_w = s * (msw + 1);  // first query that sees this wave's first slot
  const int qfull_w = s * (msw + 32);  // from here on every query sees all 32 slots
  int buf = 0;
  if (qbeg < N) {
    load_tile(qbeg);
    store_tile(0);
    if (qbeg + BTS < N) load_tile(qbeg + BTS);
  }
  __syncthreads();
  for (int q0 = qbeg; q0 < N; q0 += BTS, buf ^= 1) {
    if (q0 + BTS < N) {
      store_tile(buf ^ 1);
      if (q0 + 2 * BTS < N) load_tile(q0 + 2 * BTS);
    }
    const uint16_t* sQ = sQb[buf];
    const uint16_t* sO = sOb[buf];
    if (wave_on && q0 + BTS > qfirst_w) {
      const bool boundary = q0 < qfull_w;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        // S and dP of the tile's 32-query half rt (rows) against this wave's slots (columns)
        f32x16 sc, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + (32 * rt + c32) * QP + 16 * kk + 8 * grp);
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[kk], sc, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const bf16x8 ao = *reinterpret_cast<const bf16x8*>(sO + (32 * rt + c32) * OP + 16 * kk + 8 * grp);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vreg[kk], dp, 0, 0, 0);
        }
        // query q0 + 32 rt + 8 i4 + 4 grp + r is hidden from slot m iff it is
        // below qm = s (m + 1): one per-lane bound against compile-time offsets
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = 32 * rt + 8 * i4 + 4 * grp;
          const float4 L4 = *reinterpret_cast<const float4*>(&sLb[buf][r0]);
          const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * i4 + r] = fast_exp2(fmaf(sc[4 * i4 + r], qk, -Lr[r]));
        }
        if (boundary) {
          // completed slot m is visible to query q iff s (m + 1) <= q
          const int relq = qm - q0 - 32 * rt - 4 * grp;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (8 * (i / 4) + (i % 4) < relq) sc[i] = 0.f;
        }
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = 32 * rt + 8 * i4 + 4 * grp;
          const float4 D4 = *reinterpret_cast<const float4*>(&sDb[buf][r0]);
          const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) dp[4 * i4 + r] = a.scale * sc[4 * i4 + r] * (dp[4 * i4 + r] - Dr[r]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pb = acc_chunk_bf16(sc, c);
          const bf16x8 db = acc_chunk_bf16(dp, c);
#pragma unroll
          for (int t = 0; t < DT; ++t)
            dvt[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand(sO, OP, 2 * rt + c, t, lane), pb, dvt[t],
                                                             0, 0, 0);
#pragma unroll
          for (int t = 0; t < FT; ++t)
            dkt[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand(sQ, QP, 2 * rt + c, t, lane), db, dkt[t],
                                                             0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (!mok) return;
  // the slot token's own (diagonal) query, then the rows
  const size_t si = (static_cast<size_t>(b) * H + h) * N + jt;
  const float pjj = a.pd[si], dsjj = a.dsd[si];
  const size_t qrow = (static_cast<size_t>(b) * N + jt) * H + h;
  uint16_t* row = static_cast<uint16_t*>(a.dKV) + (static_cast<size_t>(b) * N + jt) * ldk;
  // the query and dO values first (all loads in flight together: the stores
  // below could alias them as far as the compiler knows)
  uint2 qv[FT][4], dv[DT][4];
#pragma unroll
  for (int t = 0; t < FT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f0 = 32 * t + 8 * j + 4 * grp;
      qv[t][j] = f0 < DH ? *reinterpret_cast<const uint2*>(qc + qrow * DH + f0)
                         : *reinterpret_cast<const uint2*>(qr + qrow * DR + (f0 - DH));
    }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) dv[t][j] = *reinterpret_cast<const uint2*>(dO + qrow * DH + 32 * t + 8 * j + 4 * grp);
#pragma unroll
  for (int t = 0; t < FT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f0 = 32 * t + 8 * j + 4 * grp;
      float q4[4];
      unpack4_bf16(qv[t][j], q4);
      const uint2 v = pack4_bf16(fmaf(dsjj, q4[0], dkt[t][4 * j]), fmaf(dsjj, q4[1], dkt[t][4 * j + 1]),
                                 fmaf(dsjj, q4[2], dkt[t][4 * j + 2]), fmaf(dsjj, q4[3], dkt[t][4 * j + 3]));
      *reinterpret_cast<uint2*>(f0 < DH ? row + h * DH + f0 : row + KV2 + h * DR + (f0 - DH)) = v;
    }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f0 = 32 * t + 8 * j + 4 * grp;
      float d4[4];
      unpack4_bf16(dv[t][j], d4);
      const uint2 v = pack4_bf16(fmaf(pjj, d4[0], dvt[t][4 * j]), fmaf(pjj, d4[1], dvt[t][4 * j + 1]),
                                 fmaf(pjj, d4[2], dvt[t][4 * j + 2]), fmaf(pjj, d4[3], dvt[t][4 * j + 3]));
      *reinterpret_cast<uint2*>(row + H * DH + h * DH + f0) = v;
    }
}

}  // namespace

hipError_t launch_bwd_partials(const BwdArgs& a, int dtype, hipStream_t st) {
  const int waves = a.B * ((a.N + a.s - 1) / a.s);
  const dim3 grid((waves + 3) / 4);
  const bool lanes = (a.d_c == 256 || a.d_c == 512) && a.d_r <= 64;
  if (dtype == 0) {
    if (lanes && a.d_c == 256) bwd_partials_lanes_kernel<float, 4><<<grid, 256, 0, st>>>(a);
    else if (lanes) bwd_partials_lanes_kernel<float, 8><<<grid, 256, 0, st>>>(a);
    else bwd_partials_kernel<float><<<grid, 256, 0, st>>>(a);
  } else {
    if (lanes && a.d_c == 256) bwd_partials_lanes_kernel<uint16_t, 4><<<grid, 256, 0, st>>>(a);
    else if (lanes) bwd_partials_lanes_kernel<uint16_t, 8><<<grid, 256, 0, st>>>(a);
    else bwd_partials_kernel<uint16_t><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_attention(const BwdArgs& a, int dtype, hipStream_t st) {
  const dim3 grid(a.N, a.H, a.B);
  if (dtype == 0) {
    bwd_dq_kernel<float><<<grid, 64, 0, st>>>(a);
    bwd_dkv_kernel<float><<<grid, 64, 0, st>>>(a);
  } else {
    bwd_dq_kernel<uint16_t><<<grid, 64, 0, st>>>(a);
    bwd_dkv_kernel<uint16_t><<<grid, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T, int TB>
static void scan_launch_tb(const BwdArgs& a, dim3 grid, hipStream_t st) {
  const int W = a.d_c + a.d_r;
  if (W <= 5 * 64)
    bwd_scan_kernel<T, 5, TB><<<grid, 256, 0, st>>>(a);
  else if (W <= 9 * 64)
    bwd_scan_kernel<T, 9, TB><<<grid, 256, 0, st>>>(a);
  else
    bwd_scan_kernel<T, 16, TB><<<grid, 256, 0, st>>>(a);
}

template <typename T>
static void scan_launch(const BwdArgs& a, dim3 grid, hipStream_t st) {
  if (a.s == 3)
    scan_launch_tb<T, 3>(a, grid, st);
  else
    scan_launch_tb<T, 4>(a, grid, st);
}

hipError_t launch_bwd_scan(const BwdArgs& a, int dtype, hipStream_t st) {
  const int waves = a.B * ((a.N + a.s - 1) / a.s);
  const dim3 grid((waves + 3) / 4);
  if (dtype == 0)
    scan_launch<float>(a, grid, st);
  else
    scan_launch<uint16_t>(a, grid, st);
  return hipGetLastError();
}

hipError_t launch_bwd_dwhyp(const BwdArgs& a, float* out, int dtype, hipStream_t st) {
  const int R = a.B * a.N;
  const int rows_per_split = (R + a.wh_parts - 1) / a.wh_parts;
  const dim3 grid((a.d_c + 63) / 64, a.wh_parts, a.wh_rows);
  if (dtype == 0)
    dwhyp_kernel<float><<<grid, 256, 0, st>>>(a, rows_per_split);
  else
    dwhyp_kernel<uint16_t><<<grid, 256, 0, st>>>(a, rows_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_parts(a.wh_part, a.wh_parts, a.wh_rows * a.d_c, out, st);
}

hipError_t launch_bwd_transpose_w(int KV2h, int d_c, const void* w_uk, const void* w_uv, void* wt, int dtype,
                                  hipStream_t st) {
  const int n = 2 * KV2h * d_c;
  const dim3 grid((n + 255) / 256);
  if (dtype == 0)
    transpose_w_kernel<float><<<grid, 256, 0, st>>>(KV2h, d_c, static_cast<const float*>(w_uk),
                                                    static_cast<const float*>(w_uv), static_cast<float*>(wt));
  else
    transpose_w_kernel<uint16_t><<<grid, 256, 0, st>>>(KV2h, d_c, static_cast<const uint16_t*>(w_uk),
                                                       static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(wt));
  return hipGetLastError();
}

static bool wgrad_mfma(int M, int N, int dtype) { return dtype != 0 && M % 128 == 0 && N % 128 == 0; }

int bwd_wgrad_tiles(int M, int N, int dtype) {
  return wgrad_mfma(M, N, dtype) ? (M / 128) * (N / 128) : ((M + 63) / 64) * ((N + 63) / 64);
}

hipError_t launch_bwd_wgrad(int R, int M, int N, const void* A, int lda, const void* Bm, int ldb, float* part,
                            int splits, float* out0, int m0_rows, float* out1, int dtype, hipStream_t st) {
  const int rows_per_split = (R + splits - 1) / splits;
  const dim3 grid((N + 63) / 64, (M + 63) / 64, splits);
  if (wgrad_mfma(M, N, dtype))
    wgrad_mfma_kernel<<<dim3(N / 128, M / 128, splits), 256, 0, st>>>(
        R, M, N, static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(Bm), ldb, part, rows_per_split);
  else if (dtype == 0)
    wgrad_kernel<float><<<grid, 256, 0, st>>>(R, M, N, static_cast<const float*>(A), lda,
                                              static_cast<const float*>(Bm), ldb, part, rows_per_split);
  else
    wgrad_kernel<uint16_t><<<grid, 256, 0, st>>>(R, M, N, static_cast<const uint16_t*>(A), lda,
                                                 static_cast<const uint16_t*>(Bm), ldb, part, rows_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = static_cast<size_t>(M) * N;
  sum_split_rows_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, st>>>(part, splits, M, N, out0,
                                                                                      m0_rows, out1);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* part, int parts, int n, float* out, hipStream_t st) {
  sum_parts_kernel<<<dim3((n + 63) / 64), 256, 0, st>>>(part, parts, n, out);
  return hipGetLastError();
}

bool bwd_mfma_supported(int d_h, int d_r) { return d_h == 64 && d_r == 32; }

hipError_t launch_bwd_attention_mfma(const BwdArgs& a0, hipStream_t st) {
  if (!bwd_mfma_supported(a0.d_h, a0.d_r)) return hipErrorNotSupported;
  BwdArgs a = a0;
  const int npair = a.B * a.H;
  a.nqt = (a.N + 127) / 128;
  bwd_dq_mfma_kernel<64, 32><<<a.nqt * npair, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nslots = a.N / a.s;
  if (nslots == 0) return hipSuccess;
  const int nst = (nslots + 127) / 128;
  bwd_dkv_mfma_kernel<64, 32><<<nst * npair, 256, 0, st>>>(a, nslots, nst);
  return hipGetLastError();
}

}  // namespace mtla
