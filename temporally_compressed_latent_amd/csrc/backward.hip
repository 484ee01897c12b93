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
                                     a.w_hyp, a.d_c, lane);
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
// block), blocks dealt out to wh_parts waves in turn; each wave keeps its own
// fp32 partial sum of dW_hyp.
template <typename T>
__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = (blockIdx.x * 256 + threadIdx.x) >> 6;
  if (wv >= a.wh_parts) return;
  const int nblk = (a.N + a.s - 1) / a.s;
  const int W = a.d_c + a.d_r, KV2 = 2 * a.H * a.d_h, ldk = KV2 + a.H * a.d_r;
  float whp[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) whp[j] = 0.f;
  for (int blkid = wv; blkid < a.B * nblk; blkid += a.wh_parts) {
    const int b = blkid / nblk, blk = blkid % nblk;
    const int t0 = blk * a.s, t1 = min(t0 + a.s, a.N);
    float G[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) G[j] = 0.f;
    for (int t = t1 - 1; t >= t0; --t) {
      const size_t row = static_cast<size_t>(b) * a.N + t;
      const float w = a.gate[row];
      float x[16], dwl = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = lane + 64 * j;
        x[j] = 0.f;
        if (e >= W) continue;
        float dP;
        if (e < a.d_c) {
          dP = a.dPc[row * a.d_c + e];
          x[j] = ld<T>(a.c, row * a.d_c + e);
        } else {
          const int r = e - a.d_c;
          dP = 0.f;
          for (int hh = 0; hh < a.H; ++hh) dP += ld<T>(a.dKV, row * ldk + KV2 + hh * a.d_r + r);
          x[j] = ld<T>(a.k_r, row * a.d_r + r);
        }
        G[j] += dP;
        dwl = fmaf(G[j], x[j], dwl);
      }
      const float du = wave_sum(dwl) * w * (1.f - w);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = lane + 64 * j;
        if (e >= W) continue;
        if (e < a.d_c) {
          st<T>(a.g_c, row * a.d_c + e, fmaf(du, a.w_hyp[e], w * G[j]));
          whp[j] = fmaf(du, x[j] + a.pe[static_cast<size_t>(t) * a.d_c + e], whp[j]);
        } else {
          st<T>(a.g_k_r, row * a.d_r + (e - a.d_c), w * G[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = lane + 64 * j;
    if (e < a.d_c) a.wh_part[static_cast<size_t>(wv) * a.d_c + e] = whp[j];
  }
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
  float acc = 0.f;
  for (int p = 0; p < splits; ++p) acc += part[p * n + idx];
  const int m = static_cast<int>(idx / N);
  if (m < m0_rows)
    out0[idx] = acc;
  else
    out1[idx - static_cast<size_t>(m0_rows) * N] = acc;
}

__global__ __launch_bounds__(256) void sum_parts_kernel(const float* part, int parts, int n, float* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int p = 0; p < parts; ++p) acc += part[static_cast<size_t>(p) * n + i];
  out[i] = acc;
}

}  // namespace

hipError_t launch_bwd_partials(const BwdArgs& a, int dtype, hipStream_t st) {
  const int waves = a.B * ((a.N + a.s - 1) / a.s);
  const dim3 grid((waves + 3) / 4);
  if (dtype == 0)
    bwd_partials_kernel<float><<<grid, 256, 0, st>>>(a);
  else
    bwd_partials_kernel<uint16_t><<<grid, 256, 0, st>>>(a);
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

hipError_t launch_bwd_scan(const BwdArgs& a, int dtype, hipStream_t st) {
  const dim3 grid((a.wh_parts + 3) / 4);
  if (dtype == 0)
    bwd_scan_kernel<float><<<grid, 256, 0, st>>>(a);
  else
    bwd_scan_kernel<uint16_t><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
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

hipError_t launch_bwd_wgrad(int R, int M, int N, const void* A, int lda, const void* Bm, int ldb, float* part,
                            int splits, float* out0, int m0_rows, float* out1, int dtype, hipStream_t st) {
  const int rows_per_split = (R + splits - 1) / splits;
  const dim3 grid((N + 63) / 64, (M + 63) / 64, splits);
  if (dtype == 0)
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
  sum_parts_kernel<<<dim3((n + 255) / 256), 256, 0, st>>>(part, parts, n, out);
  return hipGetLastError();
}

}  // namespace mtla
