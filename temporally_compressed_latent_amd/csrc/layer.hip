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
// storage.  The C tile is staged in LDS and stored by column pairs, so a rope
// pair (2k, 2k+1) - two adjacent columns of one tile - is rotated by the one
// thread that stores both.  Few rows (decode) take a skinny variant that
// splits K over the waves instead, many rows in bf16 a 128 x 128 MFMA
// variant.
#include "common.hpp"
#include "gemm_tile.hpp"
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

// Quotient and remainder by a positive divisor, by shifts when it is a power
// of two (these run ahead of the first loads of the small-M product).
__device__ __forceinline__ int div_rows(int x, int d) { return (d & (d - 1)) == 0 ? x >> __builtin_ctz(d) : x / d; }
__device__ __forceinline__ int mod_rows(int x, int d) { return (d & (d - 1)) == 0 ? x & (d - 1) : x % d; }

// Weight row n of the virtual [N, K] matrix [w0 ; w1 ; w2].  For the input
// projection (mode 1) the rows of w1 = W_Q are taken grouped by kind: first
// the q^C rows of every head, then the q^R rows of every head, so that a
// column tile of the product holds one kind of output (c, q^C, q^R or k^R)
// and only the q^R and k^R tiles rotate.
template <typename T>
__device__ __forceinline__ const T* weight_row(const LayerGemmArgs& g, int n) {
  if (n < g.n0) return static_cast<const T*>(g.w0) + static_cast<size_t>(n) * g.K;
  n -= g.n0;
  if (n < g.n1) {
    if (g.mode != 0) {
      const int QW = g.d_h + g.d_r, HC = g.H * g.d_h;
      n = n < HC ? div_rows(n, g.d_h) * QW + mod_rows(n, g.d_h)
                 : div_rows(n - HC, g.d_r) * QW + g.d_h + mod_rows(n - HC, g.d_r);
    }
    return static_cast<const T*>(g.w1) + static_cast<size_t>(n) * g.K;
  }
  n -= g.n1;
  return static_cast<const T*>(g.w2) + static_cast<size_t>(n) * g.K;
}

template <typename T>
__device__ __forceinline__ void store_val(void* p, size_t i, float v) {
  Store<T>::store(static_cast<T*>(p), i, v);
}

// Where the even output column n of a GEMM goes: plain output (mode 0), or, for
// the input projection, c, q^C, q^R or k^R; a rope pair carries its frequency
// 10000^(-2k/d_r), k the pair's index in the rope vector.
struct PairDest {
  int kind;      // 0 plain, 1 c, 2 q^C, 3 q^R, 4 k^R
  int head, e;   // head and element index inside its section
  double theta;  // rope frequency (kinds 3 and 4)
};

__device__ __forceinline__ PairDest pair_dest(const LayerGemmArgs& g, int n) {
  PairDest p{0, 0, n, 0.0};
  if (g.mode == 0) return p;
  // columns in weight_row's order: c, then q^C of every head, then q^R of
  // every head, then k^R
  const int QW = g.d_h + g.d_r, HQ = g.H * QW, HC = g.H * g.d_h;
  if (n < g.d_c) {
    p.kind = 1;
  } else if (n < g.d_c + HC) {
    p.kind = 2;
    p.head = (n - g.d_c) / g.d_h;
    p.e = (n - g.d_c) % g.d_h;
  } else if (n < g.d_c + HQ) {
    p.kind = 3;
    p.head = (n - g.d_c - HC) / g.d_r;
    p.e = (n - g.d_c - HC) % g.d_r;
  } else {
    p.kind = 4;
    p.e = n - g.d_c - HQ;
  }
  if (p.kind >= 3) p.theta = pow(10000.0, -static_cast<double>(p.e) / g.d_r);  // e = 2k
  return p;
}

// The same destination as an array, a row stride and an offset: output pair
// (m, n) goes to elements m * stride + off, +1 of dst.  Resolved once per
// column pair, so that a store loop over rows has no per-row branch on the
// kind of output.
struct PairStore {
  void* dst;
  int stride, off;
  bool rope, f32, single;  // rotate (q^R, k^R); fp32 output; last column of an odd N
  double theta;
};
__device__ __forceinline__ PairStore pair_store(const LayerGemmArgs& g, int n) {
  const PairDest p = pair_dest(g, n);
  switch (p.kind) {
    case 0: return PairStore{g.out, g.N, n, false, g.out_f32 != 0, n + 1 >= g.N, 0.0};
    case 1: return PairStore{g.c, g.d_c, n, false, false, false, 0.0};
    case 2: return PairStore{g.q_c, g.H * g.d_h, p.head * g.d_h + p.e, false, false, false, 0.0};
    case 3: return PairStore{g.q_r, g.H * g.d_r, p.head * g.d_r + p.e, true, false, false, p.theta};
    default: return PairStore{g.k_r, g.d_r, p.e, true, false, false, p.theta};
  }
}

// Eight consecutive output columns n .. n+7 (n a multiple of 8) with one
// destination (when the launcher sets vec8): four pairs, one 16-byte store
// of bf16 (two of fp32) per row.
struct ChunkStore {
  void* dst;
  int stride, off;
  bool rope, f32;
  double theta[4];
};
__device__ __forceinline__ ChunkStore chunk_store(const LayerGemmArgs& g, int n) {
  const PairStore p0 = pair_store(g, n);
  ChunkStore c{p0.dst, p0.stride, p0.off, p0.rope, p0.f32, {0.0, 0.0, 0.0, 0.0}};
  if (p0.rope)
#pragma unroll
    for (int p = 0; p < 4; ++p) c.theta[p] = pair_store(g, n + 2 * p).theta;
  return c;
}

// Rotate the pair (x0, x1) by the angle pos * theta: the angle is formed and
// reduced to [-pi, pi] in double, so that large positions keep their
// accuracy, and its sine and cosine are taken in float.
__device__ __forceinline__ void rope_rotate(int pos, double theta, float& x0, float& x1) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double ang = static_cast<double>(pos) * theta;
  const double rev = rint(ang * (1.0 / kTwoPi));
  const float r = static_cast<float>(fma(-rev, kTwoPi, ang));
  float sn, cs;
  sincosf(r, &sn, &cs);
  const float y0 = x0 * cs - x1 * sn;
  const float y1 = x0 * sn + x1 * cs;
  x0 = y0;
  x1 = y1;
}

// The same rotation with the angle reduced, in double, to revolutions in
// [-1/2, 1/2] and the hardware sine and cosine of 2 pi r: for bf16 outputs,
// whose rounding (2^-9) is far above the hardware functions' error.
__device__ __forceinline__ void rope_rotate_rev(int pos, double theta, float& x0, float& x1) {
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  const double rev = static_cast<double>(pos) * theta * kInvTwoPi;
  const float r = static_cast<float>(rev - rint(rev));
  const float sn = __builtin_amdgcn_sinf(r), cs = __builtin_amdgcn_cosf(r);
  const float y0 = x0 * cs - x1 * sn;
  const float y1 = x0 * sn + x1 * cs;
  x0 = y0;
  x1 = y1;
}

// 0-based position of the token in GEMM row m (sequence m / T, token m % T).
__device__ __forceinline__ int row_position(const LayerGemmArgs& g, int m) {
  const int b = div_rows(m, g.T), t = mod_rows(m, g.T);
  return (g.pos0 ? g.pos0[b] : g.p0_all) + t - 1;
}

// Two consecutive elements at an even index i of a 16-byte aligned array, in
// one store.
__device__ __forceinline__ void store2(float* p, size_t i, float x0, float x1) {
  *reinterpret_cast<float2*>(p + i) = float2{x0, x1};
}
__device__ __forceinline__ void store2(uint16_t* p, size_t i, float x0, float x1) {
  *reinterpret_cast<uint32_t*>(p + i) =
      static_cast<uint32_t>(f32_to_bf16_bits(x0)) | (static_cast<uint32_t>(f32_to_bf16_bits(x1)) << 16);
}

// Store the output pair C[m, n], C[m, n + 1] (n even) at its destination; pos
// is row m's token position (used by rope pairs only).  Every destination
// index is even (d_c, d_r, d_h and a plain output's N are even) and every
// destination 16-byte aligned, so a pair is one store.
template <typename T, bool kRev = false>
__device__ __forceinline__ void store_pair(const LayerGemmArgs& g, const PairDest& p, int m, int n, int pos,
                                           float x0, float x1) {
  size_t i;
  switch (p.kind) {
    case 0:
      i = static_cast<size_t>(m) * g.N + n;
      if (n + 1 >= g.N) {  // (an odd N's last column)
        if (g.out_f32)
          static_cast<float*>(g.out)[i] = x0;
        else
          store_val<T>(g.out, i, x0);
      } else if (g.out_f32) {
        store2(static_cast<float*>(g.out), i, x0, x1);
      } else {
        store2(static_cast<T*>(g.out), i, x0, x1);
      }
      return;
    case 1:
      i = static_cast<size_t>(m) * g.d_c + n;
      store2(static_cast<T*>(g.c), i, x0, x1);
      return;
    case 2:
      i = (static_cast<size_t>(m) * g.H + p.head) * g.d_h + p.e;
      store2(static_cast<T*>(g.q_c), i, x0, x1);
      return;
    default: {
      if constexpr (kRev)
        rope_rotate_rev(pos, p.theta, x0, x1);
      else
        rope_rotate(pos, p.theta, x0, x1);
      void* dst = p.kind == 3 ? g.q_r : g.k_r;
      i = p.kind == 3 ? (static_cast<size_t>(m) * g.H + p.head) * g.d_r + p.e
                      : static_cast<size_t>(m) * g.d_r + p.e;
      store2(static_cast<T*>(dst), i, x0, x1);
      return;
    }
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
    arow[i] = static_cast<const T*>(g.A) + static_cast<size_t>(min(m0 + r, M - 1)) * (g.lda ? g.lda : K);
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
  // each thread stores one column pair of the tile on every 8th row
  const int pc = tid & (LBN / 2 - 1), n = n0 + 2 * pc;
  if (n >= N) return;
  const PairDest pd = pair_dest(g, n);
  for (int r = tid / (LBN / 2); r < LBM; r += 256 / (LBN / 2)) {
    const int m = m0 + r;
    if (m >= M) break;
    store_pair<T>(g, pd, m, n, pd.kind >= 3 ? row_position(g, m) : 0, sC[r * LCP + 2 * pc],
                  sC[r * LCP + 2 * pc + 1]);
  }
}

// The same product for many rows in bf16: 128 x 128 output tiles, four waves
// of 64 x 64 (2 x 2 tiles of 32x32x16 MFMA), K step 32 or 64 through
// double-buffered LDS with the next step's operands prefetched into
// registers.  Workgroup L runs on XCD L % 8; the column tiles of one
// 128-row stripe of A are dealt to one XCD, so the stripe is fetched into
// that XCD's L2 once for all of them.  The C tile is staged in LDS in two
// 64-row halves and stored by column pairs, as in the smaller kernel.
constexpr int MBM = 128, MBN = 128;
constexpr int MCP = MBN + 4;  // C half-tile pitch (floats)

// MBK: the K step (32 for short K: half the LDS, three workgroups per CU
// instead of two, which hides more load latency when there are few steps;
// 64 for long K).
// MBK = 0: 256-row tiles on gemm_tile (K a multiple of 32); otherwise
// 128-row tiles, K steps of MBK through two register sets and two LDS
// buffers (any K that is a multiple of 8).
template <int MBK>
constexpr int layer_tile_rows() { return MBK == 0 ? 256 : MBM; }

template <int MBK>
__global__ __launch_bounds__(256) void layer_gemm_mfma_kernel(LayerGemmArgs g, int nrt, int nct) {
  constexpr int MP = MBK + 8;  // operand pitch (elements)
  constexpr int TMR = layer_tile_rows<MBK>(), NI = TMR / 64;
  __shared__ __align__(16) uint16_t smem[MBK == 0 ? TileShape<256>::SmemElems : 2 * (MBM + MBN) * MP];
  __shared__ int sPos[TMR];
  static_assert(64 * MCP * 4 <= sizeof(smem), "C quarter tile fits in the operand buffers");
  const int L = blockIdx.x;
  const int xcd = L & 7, k8 = L >> 3;
  const int rt = 8 * (k8 / nct) + xcd, ct = k8 % nct;
  if (rt >= nrt) return;
  const int m0 = rt * TMR, n0 = ct * MBN;
  const int M = g.M, N = g.N, K = g.K, lda = g.lda ? g.lda : K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, grp = lane >> 5, c32 = lane & 31;
  f32x16 acc[NI][2];
  if constexpr (MBK == 0) {
    const uint16_t* arow[NI];
    const uint16_t* wrow[2];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = 16 * (4 * k + wave) + (lane >> 2);
      arow[k] = static_cast<const uint16_t*>(g.A) + static_cast<size_t>(min(m0 + r, M - 1)) * lda;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) wrow[k] = weight_row<uint16_t>(g, min(n0 + 16 * (4 * k + wave) + (lane >> 2), N - 1));
    gemm_tile<256, false>(arow, wrow, K, smem, acc);
  } else {
  // per stage and operand 128 rows x 64 k = 1024 chunks of 8: 4 per thread
  constexpr int CPT = MBM * (MBK > 0 ? MBK : 8) / 8 / 256;
  const uint16_t* arow[CPT];
  const uint16_t* wrow[CPT];
  int kofs[CPT], lofs[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i, r = c / (MBK / 8);
    kofs[i] = (c % (MBK / 8)) * 8;
    lofs[i] = r * MP + kofs[i];
    arow[i] = static_cast<const uint16_t*>(g.A) + static_cast<size_t>(min(m0 + r, M - 1)) * lda;
    wrow[i] = weight_row<uint16_t>(g, min(n0 + r, N - 1));
  }
  // Two K steps are in flight: each step's chunks land in one of two register
  // sets and go to LDS one step later.  Chunks past K read as zero (K is a
  // multiple of 8): the address is kept inside the row and the value masked
  // when it is stored, so no load sits under a branch or waits early.
  struct Regs {
    uint4 a[CPT], w[CPT];
  };
  auto gload = [&](Regs& R, int k0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int kk = min(k0 + kofs[i], K - 8);
      R.a[i] = *reinterpret_cast<const uint4*>(arow[i] + kk);
      R.w[i] = *reinterpret_cast<const uint4*>(wrow[i] + kk);
    }
    // keep the loads where they are issued (the scheduler would sink them
    // towards their LDS stores, which then wait for a full round trip)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lstore = [&](const Regs& R, int k0, int buf) {
    uint16_t* sA = smem + buf * (MBM + MBN) * MP;
    uint16_t* sW = sA + MBM * MP;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      // (a mask, not a select of the vectors, which the compiler would
      // route through scratch memory)
      const uint32_t keep = k0 + kofs[i] < K ? 0xffffffffu : 0u;
      const uint4 va = R.a[i], vw = R.w[i];
      *reinterpret_cast<uint4*>(sA + lofs[i]) = uint4{va.x & keep, va.y & keep, va.z & keep, va.w & keep};
      *reinterpret_cast<uint4*>(sW + lofs[i]) = uint4{vw.x & keep, vw.y & keep, vw.z & keep, vw.w & keep};
    }
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto compute = [&](int buf) {
    const uint16_t* sA = smem + buf * (MBM + MBN) * MP;
    const uint16_t* sW = sA + MBM * MP;
#pragma unroll
    for (int kc = 0; kc < MBK / 16; ++kc) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (64 * wm + 32 * i + c32) * MP + 16 * kc + 8 * grp);
        b[i] = *reinterpret_cast<const bf16x8*>(sW + (64 * wn + 32 * i + c32) * MP + 16 * kc + 8 * grp);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  // step kt is computed from LDS buffer kt & 1; meanwhile step kt + 1 sits in
  // registers (stored after the compute) and step kt + 2 is being loaded.
  // Loads and stores are unconditional, steps past the end re-reading the
  // last one, so that the waits before the stores count only the older set
  // and the loads are not sunk next to their stores.
  const int nk = (K + MBK - 1) / MBK;
  Regs R0, R1;
  gload(R0, 0);
  gload(R1, min(1, nk - 1) * MBK);
  lstore(R0, 0, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    gload(R0, min(kt + 2, nk - 1) * MBK);
    compute(0);
    lstore(R1, (kt + 1) * MBK, 1);
    __syncthreads();
    gload(R1, min(kt + 3, nk - 1) * MBK);
    compute(1);
    lstore(R0, min(kt + 2, nk - 1) * MBK, 0);
    __syncthreads();
  }
  if (kt < nk) {  // odd step count: the last step is in buffer 0
    compute(0);
    __syncthreads();
  }
  }

  // epilogue, one 64-row quarter at a time: acc[i][j][e] is row
  // (TMR/2) wm + 32 i + 8 (e / 4) + 4 grp + e % 4, column 64 wn + 32 j + c32.
  // The rows' token positions (rope pairs) are computed once per row.
  float* sC = reinterpret_cast<float*>(smem);
  const int pc = tid & 63, n = n0 + 2 * pc;
  const PairStore ps = pair_store(g, min(n, N - 2));
  if (g.mode != 0)
    for (int r = tid; r < TMR; r += 256) sPos[r] = row_position(g, min(m0 + r, M - 1));
  if (g.vec8) {
    // thread (row r, chunk q): 8 columns n0 + 8 q .. +7 of rows r, r + 16,
    // ... of each quarter, one 16-byte (bf16) or two (fp32) stores per row
    const int q = tid & 15, n8 = n0 + 8 * q;
    const ChunkStore cs = chunk_store(g, min(n8, N - 8));
#pragma unroll
    for (int hh = 0; hh < TMR / 64; ++hh) {
      if (wm == hh / (NI / 2)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              sC[(32 * i + 8 * (e / 4) + 4 * grp + (e % 4)) * MCP + 64 * wn + 32 * j + c32] =
                  acc[2 * (hh % (NI / 2)) + i][j][e];
      }
      __syncthreads();
      if (n8 < N) {
        for (int r = tid >> 4; r < 64; r += 16) {
          const int m = m0 + 64 * hh + r;
          if (m >= M) break;
          const float4 lo = *reinterpret_cast<const float4*>(sC + r * MCP + 8 * q);
          const float4 hi = *reinterpret_cast<const float4*>(sC + r * MCP + 8 * q + 4);
          float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          if (cs.rope) {
            const int pos = sPos[64 * hh + r];
#pragma unroll
            for (int p = 0; p < 4; ++p) rope_rotate_rev(pos, cs.theta[p], x[2 * p], x[2 * p + 1]);
          }
          const size_t i = static_cast<size_t>(m) * cs.stride + cs.off;
          if (cs.f32) {
            float* d = static_cast<float*>(cs.dst) + i;
            *reinterpret_cast<float4*>(d) = float4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<float4*>(d + 4) = float4{x[4], x[5], x[6], x[7]};
          } else {
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
              w[p] = static_cast<uint32_t>(f32_to_bf16_bits(x[2 * p])) |
                     (static_cast<uint32_t>(f32_to_bf16_bits(x[2 * p + 1])) << 16);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(cs.dst) + i) = uint4{w[0], w[1], w[2], w[3]};
          }
        }
      }
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int hh = 0; hh < TMR / 64; ++hh) {
    // quarter hh: rows 32 i of wave row hh / (NI / 2), i = 2 (hh % (NI / 2)) + 0, 1
    if (wm == hh / (NI / 2)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sC[(32 * i + 8 * (e / 4) + 4 * grp + (e % 4)) * MCP + 64 * wn + 32 * j + c32] =
                acc[2 * (hh % (NI / 2)) + i][j][e];
    }
    __syncthreads();
    if (n < N) {
      for (int r = tid >> 6; r < 64; r += 4) {
        const int m = m0 + 64 * hh + r;
        if (m >= M) break;
        float x0 = sC[r * MCP + 2 * pc], x1 = sC[r * MCP + 2 * pc + 1];
        if (ps.rope) rope_rotate_rev(sPos[64 * hh + r], ps.theta, x0, x1);
        const size_t i = static_cast<size_t>(m) * ps.stride + ps.off;
        if (ps.f32) {
          float* d = static_cast<float*>(ps.dst);
          if (ps.single) d[i] = x0; else store2(d, i, x0, x1);
        } else {
          uint16_t* d = static_cast<uint16_t*>(ps.dst);
          if (ps.single) d[i] = f32_to_bf16_bits(x0); else store2(d, i, x0, x1);
        }
      }
    }
    __syncthreads();
  }
}

// The same product for few rows (M <= 64, one token per sequence in decode),
// in bf16: every lane loads its MFMA operand fragments straight from memory
// (A row c16 and weight row c16, 8 consecutive k at 8 * g16), the
// workgroup's four waves split K between them (wave w takes the 32-wide
// k-steps w, w + 4, ...) with sixteen k-steps' loads in flight per round, and
// the four partial tiles are summed through LDS.  One workgroup per 16 output
// columns and 16 * NB rows (blockIdx.y: the block of rows).
constexpr int SKN = 16;

// The leading scalar arguments (A, the first weight matrix, M, N, K, that
// matrix's row count and A's row stride) repeat fields of g ahead of it so
// that the build can preload them into scalar registers: the first operand
// loads then issue without a round trip to the kernel-argument segment.
template <int NB>
__global__ __launch_bounds__(256) void layer_gemm_skinny_kernel(const uint16_t* __restrict__ A0,
                                                                const uint16_t* __restrict__ W0, int M, int N,
                                                                int K, int n0_rows, int lda0, LayerGemmArgs g) {
  __shared__ float sP[4][16 * NB * (SKN + 1)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * SKN;
  const int m0 = 16 * NB * blockIdx.y;  // first row of this workgroup's block of rows
  // epilogue item of this thread: column pair pc on rows er[0], er[1]; their
  // token positions are loaded first, so that they arrive with the operands
  constexpr int ER = (16 * NB + 31) / 32;
  const int pc = tid & (SKN / 2 - 1), n = n0 + 2 * pc;
  int er[ER], epos[ER];
#pragma unroll
  for (int j = 0; j < ER; ++j) {
    er[j] = tid / (SKN / 2) + 32 * j;
    epos[j] = g.mode != 0 ? row_position(g, min(m0 + er[j], M - 1)) : 0;
  }
  // (a tile wholly inside the first weight matrix takes its rows from the
  // preloaded pointer)
  const int nw = min(n0 + c16, N - 1);
  const uint16_t* wr = (n0 + SKN <= n0_rows ? W0 + static_cast<size_t>(nw) * K : weight_row<uint16_t>(g, nw)) + 8 * g16;
  const uint16_t* ar[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    ar[i] = A0 + static_cast<size_t>(min(m0 + 16 * i + c16, M - 1)) * (lda0 ? lda0 : K) + 8 * g16;
  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  bf16x8 wf[4], af[4][NB];
  auto load_round = [&](int kb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kb + 128 * s;
      const bool in = k + 8 * g16 < K;  // K is a multiple of 8: a fragment is wholly in or out
      wf[s] = in ? *reinterpret_cast<const bf16x8*>(wr + k) : zero;
#pragma unroll
      for (int i = 0; i < NB; ++i) af[s][i] = in ? *reinterpret_cast<const bf16x8*>(ar[i] + k) : zero;
    }
  };
  auto mma_round = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][i], wf[s], acc[i], 0, 0, 0);
  };
  // wave w takes the 32-wide k-steps w, w + 4, ...: sixteen per round
  int kb = 32 * wave;
  load_round(kb);
  __builtin_amdgcn_sched_barrier(0);
  const PairDest pd = pair_dest(g, min(n, N - 2));  // the rope frequency is computed under the loads
  __builtin_amdgcn_sched_barrier(0);
  mma_round();
  for (kb += 512; kb < K; kb += 512) {
    load_round(kb);
    mma_round();
  }
  // acc[i][q]: row 16 i + 4 g16 + q, column c16
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) sP[wave][(16 * i + 4 * g16 + q) * (SKN + 1) + c16] = acc[i][q];
  __syncthreads();
  if (n >= N) return;
#pragma unroll
  for (int j = 0; j < ER; ++j) {
    const int r = er[j];
    if (m0 + r >= M || r >= 16 * NB) break;
    float x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x0 += sP[w][r * (SKN + 1) + 2 * pc];
      x1 += sP[w][r * (SKN + 1) + 2 * pc + 1];
    }
    store_pair<uint16_t>(g, pd, m0 + r, n, epos[j], x0, x1);
  }
}

}  // namespace

namespace {
// Every 8-column chunk of an output row lies in one destination at a 16-byte
// boundary: N and the section widths multiples of 8, the arrays 16-byte
// aligned.
bool chunk_stores_ok(const LayerGemmArgs& g) {
  auto al = [](const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (g.N % 8 != 0) return false;
  if (g.mode == 0) return al(g.out);
  return g.d_c % 8 == 0 && g.d_h % 8 == 0 && g.d_r % 8 == 0 && al(g.c) && al(g.q_c) && al(g.q_r) && al(g.k_r);
}
}  // namespace

hipError_t launch_layer_gemm(const LayerGemmArgs& g, int dtype, hipStream_t st) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (dtype != 0 && g.M <= 64) {
    // one 16-row block per workgroup: the operand loads are spread over
    // (M / 16) times more compute units (each load of 16 rows x 64 bytes
    // takes a compute unit's memory pipeline about 32 cycles)
    const dim3 sgrid((g.N + SKN - 1) / SKN, (g.M + 15) / 16);
    const uint16_t* A0 = static_cast<const uint16_t*>(g.A);
    const uint16_t* W0 = static_cast<const uint16_t*>(g.w0);
    layer_gemm_skinny_kernel<1><<<sgrid, 256, 0, st>>>(A0, W0, g.M, g.N, g.K, g.n0, g.lda, g);
    return hipGetLastError();
  }
  if (dtype != 0) {
    const int nrt = (g.M + MBM - 1) / MBM, nct = (g.N + MBN - 1) / MBN;
    LayerGemmArgs gv = g;
    gv.vec8 = chunk_stores_ok(g) ? 1 : 0;
    if (g.K % 32 == 0) {
      const int nrt2 = (g.M + 255) / 256;
      layer_gemm_mfma_kernel<0><<<dim3(8 * ((nrt2 + 7) / 8) * nct), 256, 0, st>>>(gv, nrt2, nct);
    } else if (g.K <= 1024)
      layer_gemm_mfma_kernel<32><<<dim3(8 * ((nrt + 7) / 8) * nct), 256, 0, st>>>(gv, nrt, nct);
    else
      layer_gemm_mfma_kernel<64><<<dim3(8 * ((nrt + 7) / 8) * nct), 256, 0, st>>>(gv, nrt, nct);
    return hipGetLastError();
  }
  dim3 grid((g.N + LBN - 1) / LBN, (g.M + LBM - 1) / LBM);
  layer_gemm_kernel<float><<<grid, 256, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace mtla
