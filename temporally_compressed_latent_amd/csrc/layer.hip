// The decoder layer around the MTLA core ("Multi-head Temporal Latent
// Attention", Method; "Multi-Head Latent Attention and Sparse Indexers",
// "Latent attention changes the representation"):
//   c_t  = W_DKV h_t                      the latent that is merged and cached
//   q_t  = W_Q h_t, per head [q^C ; q^R]  the queries
//   k^R_t = W_R h_t                       the one rope key all heads share
//   q^R and k^R rotated by RoPE at position t-1 (interleaved pairs, base 10000)
//   y_t  = W_O [o_{t,1}; ...; o_{t,H}]    the output projection
//
// Both projections are one NT GEMM, C[m, n] = sum_k A[m, k] Wt[n, k], with A
// the rows (h, or the heads' outputs) and Wt the weight rows; the input
// projection reads its weight rows from the three matrices in turn
// ([W_DKV ; W_Q ; W_R]) and scatters its columns to c, q^C, q^R and k^R,
// rotating the rope pairs on the way.  64x64 output tiles, 4 waves, K step 32,
// double-buffered LDS; 16x16x32 bf16 MFMA for bf16 storage, fp32 FMA for fp32
// storage.  The C tile is staged in LDS, so a rope pair (2k, 2k+1) - two
// adjacent columns of one tile - is read by the thread that writes it.
#include "common.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

constexpr int LBM = 64, LBN = 64, LBK = 32;
constexpr int LP = LBK + 8;  // operand LDS pitch (elements)
constexpr int LCP = LBN + 4; // C tile pitch (floats)

template <typename T>
struct LayerSmem {
  T a[2][LBM * LP];
  T w[2][LBN * LP];
};

// Weight row n of the virtual [N, K] matrix [w0 ; w1 ; w2].
template <typename T>
__device__ __forceinline__ const T* weight_row(const LayerGemmArgs& g, int n) {
  if (n < g.n0) return static_cast<const T*>(g.w0) + static_cast<size_t>(n) * g.K;
  n -= g.n0;
  if (n < g.n1) return static_cast<const T*>(g.w1) + static_cast<size_t>(n) * g.K;
  n -= g.n1;
  return static_cast<const T*>(g.w2) + static_cast<size_t>(n) * g.K;
}

template <typename T>
__device__ __forceinline__ void store_val(void* p, size_t i, float v) {
  Store<T>::store(static_cast<T*>(p), i, v);
}

// Epilogue for one output element (row m, column n) of the input projection.
// x is C[m, n]; xp its rope partner C[m, n ^ 1] (used on rope columns only).
template <typename T>
__device__ __forceinline__ void project_store(const LayerGemmArgs& g, int m, int n, float x, float xp) {
  const int QW = g.d_h + g.d_r;
  const int HQ = g.H * QW;
  auto rotate = [&](int e) {  // e: index in the rope vector of width d_r
    const int b = m / g.T, t = m % g.T;
    const int pos = (g.pos0 ? g.pos0[b] : g.p0_all) + t - 1;  // 0-based position of the token
    const int k = e >> 1;
    const double ang = static_cast<double>(pos) * pow(10000.0, -2.0 * k / g.d_r);
    const float cs = static_cast<float>(cos(ang)), sn = static_cast<float>(sin(ang));
    // pair (x_even, x_odd) -> (x_even cos - x_odd sin, x_even sin + x_odd cos)
    return (e & 1) == 0 ? x * cs - xp * sn : xp * sn + x * cs;
  };
  if (n < g.d_c) {
    store_val<T>(g.c, static_cast<size_t>(m) * g.d_c + n, x);
  } else if (n < g.d_c + HQ) {
    const int hh = (n - g.d_c) / QW, e = (n - g.d_c) % QW;
    if (e < g.d_h)
      store_val<T>(g.q_c, (static_cast<size_t>(m) * g.H + hh) * g.d_h + e, x);
    else
      store_val<T>(g.q_r, (static_cast<size_t>(m) * g.H + hh) * g.d_r + (e - g.d_h), rotate(e - g.d_h));
  } else {
    const int e = n - g.d_c - HQ;
    store_val<T>(g.k_r, static_cast<size_t>(m) * g.d_r + e, rotate(e));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void layer_gemm_kernel(LayerGemmArgs g) {
  __shared__ __align__(16) unsigned char smem_raw[sizeof(LayerSmem<T>) > LBM * LCP * 4 ? sizeof(LayerSmem<T>)
                                                                                         : LBM * LCP * 4];
  LayerSmem<T>& sm = *reinterpret_cast<LayerSmem<T>*>(smem_raw);
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * LBM, n0 = blockIdx.x * LBN;
  const int M = g.M, N = g.N, K = g.K;
  constexpr int EPC = 16 / sizeof(T);               // elements per 16-byte chunk
  constexpr int CPR = LBK / EPC;                    // chunks per tile row
  constexpr int CPT = (LBM * CPR + 255) / 256;      // chunks per thread (A and W each)
  // chunk c of a tile: row c / CPR, columns (c % CPR) * EPC
  const T* arow[CPT];
  const T* wrow[CPT];
  int kofs[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i, r = c / CPR;
    kofs[i] = (c % CPR) * EPC;
    arow[i] = static_cast<const T*>(g.A) + static_cast<size_t>(min(m0 + r, M - 1)) * K;
    wrow[i] = weight_row<T>(g, min(n0 + r, N - 1));
  }
  uint4 ra[CPT], rw[CPT];
  // chunks past K read as zero (K is a multiple of EPC)
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int k = k0 + kofs[i];
      ra[i] = k < K ? *reinterpret_cast<const uint4*>(arow[i] + k) : uint4{0u, 0u, 0u, 0u};
      rw[i] = k < K ? *reinterpret_cast<const uint4*>(wrow[i] + k) : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i, r = c / CPR;
      *reinterpret_cast<uint4*>(&sm.a[buf][r * LP + kofs[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&sm.w[buf][r * LP + kofs[i]]) = rw[i];
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;   // bf16: wave's 32x32 sub-tile
  const int ty = tid >> 4, tx = tid & 15;    // fp32: thread's 4x4 block
  f32x4 acc[2][2];
  float accv[4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accv[i][j] = 0.f;

  const int nk = (K + LBK - 1) / LBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * LBK);
    if constexpr (sizeof(T) == 2) {
      bf16x8 af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&sm.a[buf][(wm * 32 + i * 16 + c16) * LP + 8 * g16]);
        wf[i] = *reinterpret_cast<const bf16x8*>(&sm.w[buf][(wn * 32 + i * 16 + c16) * LP + 8 * g16]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
    } else {
#pragma unroll 4
      for (int k = 0; k < LBK; ++k) {
        float av[4], wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[i] = reinterpret_cast<const float*>(sm.a[buf])[(ty * 4 + i) * LP + k];
          wv[i] = reinterpret_cast<const float*>(sm.w[buf])[(tx * 4 + i) * LP + k];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) accv[i][j] = fmaf(av[i], wv[j], accv[i][j]);
      }
    }
    __syncthreads();
    if (kt + 1 < nk) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // stage the C tile (fp32) in LDS, reusing the operand buffers
  float* sC = reinterpret_cast<float*>(smem_raw);
  if constexpr (sizeof(T) == 2) {
    // acc[i][j][q]: row wm*32 + i*16 + 4*g16 + q, column wn*32 + j*16 + c16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sC[(wm * 32 + i * 16 + 4 * g16 + q) * LCP + wn * 32 + j * 16 + c16] = acc[i][j][q];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sC[(ty * 4 + i) * LCP + tx * 4 + j] = accv[i][j];
  }
  __syncthreads();
  for (int idx = tid; idx < LBM * LBN; idx += 256) {
    const int r = idx / LBN, cc = idx % LBN;
    const int m = m0 + r, n = n0 + cc;
    if (m >= M || n >= N) continue;
    const float x = sC[r * LCP + cc];
    if (g.mode == 0)
      store_val<T>(g.out, static_cast<size_t>(m) * N + n, x);
    else
      project_store<T>(g, m, n, x, sC[r * LCP + (cc ^ 1)]);
  }
}

}  // namespace

hipError_t launch_layer_gemm(const LayerGemmArgs& g, int dtype, hipStream_t st) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  dim3 grid((g.N + LBN - 1) / LBN, (g.M + LBM - 1) / LBM);
  if (dtype == 0)
    layer_gemm_kernel<float><<<grid, 256, 0, st>>>(g);
  else
    layer_gemm_kernel<uint16_t><<<grid, 256, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace mtla
