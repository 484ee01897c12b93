// Parallel prefill under the stride-aware causal mask ("Multi-head Temporal
// Latent Attention", Key claims: paper Sec. 4.2 Fig. 2(c) and Sec. 4.3
// Eq. 17; Method (2)-(3)).
//
// Query i attends key j iff j == i, or s | j and j/s < ceil(i/s).  The keys
// j = s*b are the completed slots 1..floor((i-1)/s); the key j = i is the
// query's own cumulative partial merge P_i.  So the attention is dense over
// the compacted completed slots (a staircase in slot space) plus one
// per-query "diagonal" key, which seeds the online softmax.
//
//   K/V GEMM  : K^C = P^c W_UK^T and V = P^c W_UV^T for all N rows (MFMA GEMM,
//               output [B, H, N, d_h])
//   attention : per (query tile, head, sequence): diagonal init, then slot
//               tiles 0 .. floor((i_max-1)/s); only boundary tiles are masked,
//               tiles past the last visible slot are never visited.
#include "common.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

// ---------------------------------------------------------------------------
// Up-projection GEMM: C[m, col] = sum_k A[m, k] * Bw[col, k]
//   A  = P^c: rows m = (b, n) of the partial merges, row stride W, K = d_c
//   Bw = [W_UK ; W_UV] viewed as [2*H*d_h, d_c]
// 128x128 output tile per workgroup, 4 waves in a 2x2 grid of 64x64, K step
// 32, double-buffered LDS.  Output column col -> (K or V, head, e).
// ---------------------------------------------------------------------------
constexpr int GBM = 128, GBN = 128, GBK = 32;
constexpr int GP = GBK + 8;  // LDS pitch (elements)

__global__ __launch_bounds__(256) void prefill_kv_kernel(int M, int N, int H, int d_h, int d_c,
                                                        int W, const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ w_uk,
                                                        const uint16_t* __restrict__ w_uv,
                                                        uint16_t* __restrict__ kout,
                                                        uint16_t* __restrict__ vout) {
  __shared__ __align__(16) uint16_t sA[2][GBM * GP];
  __shared__ __align__(16) uint16_t sB[2][GBN * GP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int col0 = blockIdx.x * GBN;
  const int row0 = blockIdx.y * GBM;
  const int HD = H * d_h;

  // Each thread copies 2 chunks of A and 2 of B per K step (16 B each).
  uint4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = tid + 256 * j;
      const int r = id >> 2, ch = id & 3;
      const int m = row0 + r;
      ra[j] = m < M ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(m) * W + k0 + ch * 8)
                    : uint4{0u, 0u, 0u, 0u};
      const int col = col0 + r;
      const uint16_t* bsrc = col < HD ? w_uk + static_cast<size_t>(col) * d_c
                                      : w_uv + static_cast<size_t>(col - HD) * d_c;
      rb[j] = *reinterpret_cast<const uint4*>(bsrc + k0 + ch * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = tid + 256 * j;
      const int r = id >> 2, ch = id & 3;
      *reinterpret_cast<uint4*>(&sA[buf][r * GP + ch * 8]) = ra[j];
      *reinterpret_cast<uint4*>(&sB[buf][r * GP + ch * 8]) = rb[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = d_c / GBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GBK);
    bf16x8 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][(wm * 64 + i * 16 + c16) * GP + 8 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[buf][(wn * 64 + j * 16 + c16) * GP + 8 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j][q]: row wm*64 + i*16 + 4g + q, column wn*64 + j*16 + c16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = col0 + wn * 64 + j * 16 + c16;
    const bool isk = col < HD;
    const int cc = isk ? col : col - HD;
    const int hh = cc / d_h, e = cc % d_h;
    uint16_t* dst = isk ? kout : vout;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = row0 + wm * 64 + i * 16 + 4 * g + q;
        if (m < M) {
          const int bb = m / N, nn = m % N;
          dst[((static_cast<size_t>(bb) * H + hh) * N + nn) * d_h + e] = f32_to_bf16_bits(acc[i][j][q]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stride-masked attention, explicit per-head form, bf16 in / fp32 accumulate.
// Workgroup: 128 queries of one (sequence, head); wave w owns queries
// 32w..32w+31 as two 16-query MFMA column tiles.  Scores are computed
// transposed, S^T[slot, query] = K . Q^T, so that each lane holds a query
// column: the row max is in-lane plus two shuffles, and the probabilities
// are already in the B-operand layout of O^T += V^T . P^T (no LDS trip).
// The MFMA contraction index kappa = 8g + r maps to slot
//   r < 4 : 32*ks2 + 4g + r          (score tile 2*ks2)
//   r >= 4: 32*ks2 + 16 + 4g + r - 4 (score tile 2*ks2 + 1)
// and the V^T operand is read from a transposed LDS tile with that mapping.
// ---------------------------------------------------------------------------
template <int DH, int DR>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int DQK = DH + DR;
  constexpr int KSQ = DQK / 32;
  constexpr int DT = DH / 16;
  constexpr int TS = 64;
  constexpr int QT = 128;
  constexpr int KP = DQK + 8;  // sK pitch
  constexpr int VTP = TS + 4;  // sVT pitch
  static_assert(DH % 32 == 0 && DR % 32 == 0, "shape");
  constexpr int KCH = DQK / 8;  // 16-byte chunks per key row
  constexpr int VCH = DH / 8;   // 16-byte chunks per value row

  __shared__ __align__(16) uint16_t sK[TS * KP];
  __shared__ __align__(16) uint16_t sVT[DH * VTP];

  const int nqt = gridDim.x;
  const int qt = nqt - 1 - static_cast<int>(blockIdx.x);  // heavy tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int N = a.N, H = a.H, s = a.s;
  const int W = a.d_c + DR;
  const int q0 = qt * QT;
  const float qk_scale = a.scale * kLog2e;

  const uint16_t* qc = static_cast<const uint16_t*>(a.q_c);
  const uint16_t* qr = static_cast<const uint16_t*>(a.q_r);
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* vv = static_cast<const uint16_t*>(a.v) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* Pb = static_cast<const uint16_t*>(a.partials) + static_cast<size_t>(b) * N * W;

  // Query operands (registers for the whole kernel) and the diagonal state.
  bf16x8 qreg[2][KSQ];
  float m[2], lp[2];
  f32x4 acc[DT][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int qi = q0 + 32 * wave + 16 * t + c16;  // 0-based query token
    const bool qok = qi < N;
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
      const int d0 = ks * 32 + 8 * g;
      uint4 qv = uint4{0u, 0u, 0u, 0u}, kv = uint4{0u, 0u, 0u, 0u};
      if (qok) {
        if (d0 < DH) {
          qv = *reinterpret_cast<const uint4*>(qc + (static_cast<size_t>(b) * N + qi) * H * DH +
                                               static_cast<size_t>(h) * DH + d0);
          kv = *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(qi) * DH + d0);
        } else {
          qv = *reinterpret_cast<const uint4*>(qr + (static_cast<size_t>(b) * N + qi) * H * DR +
                                               static_cast<size_t>(h) * DR + (d0 - DH));
          kv = *reinterpret_cast<const uint4*>(Pb + static_cast<size_t>(qi) * W + a.d_c + (d0 - DH));
        }
      }
      qreg[t][ks] = __builtin_bit_cast(bf16x8, qv);
      const u16x8 qs = __builtin_bit_cast(u16x8, qv), kk = __builtin_bit_cast(u16x8, kv);
#pragma unroll
      for (int r = 0; r < 8; ++r) dpart = fmaf(bf16_bits_to_f32(qs[r]), bf16_bits_to_f32(kk[r]), dpart);
    }
    dpart += __shfl_xor(dpart, 16, 64);
    dpart += __shfl_xor(dpart, 32, 64);
    m[t] = dpart * qk_scale;
    lp[t] = g == 0 ? 1.f : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint2 v2 = uint2{0u, 0u};
      if (qok) v2 = *reinterpret_cast<const uint2*>(vv + static_cast<size_t>(qi) * DH + dt * 16 + 4 * g);
      acc[dt][t][0] = bf16_bits_to_f32(static_cast<uint16_t>(v2.x & 0xffffu));
      acc[dt][t][1] = bf16_bits_to_f32(static_cast<uint16_t>(v2.x >> 16));
      acc[dt][t][2] = bf16_bits_to_f32(static_cast<uint16_t>(v2.y & 0xffffu));
      acc[dt][t][3] = bf16_bits_to_f32(static_cast<uint16_t>(v2.y >> 16));
    }
  }

  const int qlast = min(q0 + QT, N) - 1;
  const int nk = qlast / s;     // completed slots seen by the tile's last query
  const int full = q0 / s;      // slots < full are seen by every query of the tile
  for (int j0 = 0; j0 < nk; j0 += TS) {
    // K tile [slot][K^C | P^R] and transposed V tile [d][slot]
    for (int id = tid; id < TS * KCH; id += 256) {
      const int row = id / KCH, ch = id % KCH;
      const int slot = j0 + row;
      uint4 v = uint4{0u, 0u, 0u, 0u};
      if (slot < nk) {
        const int tk = s * slot + s - 1;  // token holding the completed slot
        v = ch < DH / 8
                ? *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(tk) * DH + ch * 8)
                : *reinterpret_cast<const uint4*>(Pb + static_cast<size_t>(tk) * W + a.d_c + (ch - DH / 8) * 8);
      }
      *reinterpret_cast<uint4*>(sK + row * KP + ch * 8) = v;
    }
    for (int id = tid; id < TS * VCH; id += 256) {
      const int row = id / VCH, ch = id % VCH;
      const int slot = j0 + row;
      uint4 v = uint4{0u, 0u, 0u, 0u};
      if (slot < nk) v = *reinterpret_cast<const uint4*>(vv + static_cast<size_t>(s * slot + s - 1) * DH + ch * 8);
      const u16x8 e = __builtin_bit_cast(u16x8, v);
#pragma unroll
      for (int r = 0; r < 8; ++r) sVT[(ch * 8 + r) * VTP + row] = e[r];
    }
    __syncthreads();

    // S^T = K Q^T: sc[mt][t][i] = score(slot j0 + 16mt + 4g + i, query col t)
    f32x4 sc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sK + (mt * 16 + c16) * KP + ks * 32 + 8 * g);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          sc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qreg[t][ks], sc[mt][t], 0, 0, 0);
      }
    }
    const bool boundary = j0 + TS > full;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int qi = q0 + 32 * wave + 16 * t + c16;
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[mt][t][i] * qk_scale;
          if (boundary) {
            const int slot = j0 + mt * 16 + 4 * g + i;
            // completed slot (0-based) visible to query qi (0-based): s*(slot+1) <= qi
            if (s * (slot + 1) > qi) v = -INFINITY;
          }
          sc[mt][t][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m[t], mx);
      const float alpha = fast_exp2(m[t] - mn);
      m[t] = mn;
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(sc[mt][t][i] - mn);
          sc[mt][t][i] = p;
          ls += p;
        }
      }
      lp[t] = lp[t] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt][t] *= alpha;
    }

    // O^T += V^T P^T over the tile's 64 slots (two 32-slot k steps)
#pragma unroll
    for (int ks2 = 0; ks2 < TS / 32; ++ks2) {
      bf16x8 pb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u16x8 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[i] = f32_to_bf16_bits(sc[2 * ks2][t][i]);
          pk[4 + i] = f32_to_bf16_bits(sc[2 * ks2 + 1][t][i]);
        }
        pb[t] = __builtin_bit_cast(bf16x8, pk);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* src = sVT + (dt * 16 + c16) * VTP + ks2 * 32 + 4 * g;
        const uint2 lo4 = *reinterpret_cast<const uint2*>(src);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(src + 16);
        const bf16x8 av = __builtin_bit_cast(bf16x8, uint4{lo4.x, lo4.y, hi4.x, hi4.y});
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[t], acc[dt][t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float l = lp[t];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.f / l;
    const int qi = q0 + 32 * wave + 16 * t + c16;
    if (qi < N) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint16_t* dst = out + ((static_cast<size_t>(b) * N + qi) * H + h) * DH + dt * 16 + 4 * g;
        const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][0] * inv)) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][1] * inv)) << 16);
        const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][2] * inv)) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(dst) = uint2{w0, w1};
      }
    }
  }
}

}  // namespace

bool prefill_mfma_supported(int H, int d_h, int d_c, int d_r) {
  const bool shape = (d_h == 64 && d_r == 32) || (d_h == 128 && d_r == 64);
  return shape && d_c % GBK == 0 && (2 * H * d_h) % GBN == 0;
}

hipError_t launch_prefill_kv(int B, int N, int H, int d_h, int d_c, int d_r,
                            const void* partials, const void* w_uk, const void* w_uv,
                            void* k_out, void* v_out, hipStream_t st) {
  const int M = B * N;
  dim3 grid((2 * H * d_h) / GBN, (M + GBM - 1) / GBM);
  prefill_kv_kernel<<<grid, 256, 0, st>>>(M, N, H, d_h, d_c, d_c + d_r,
                                         static_cast<const uint16_t*>(partials),
                                         static_cast<const uint16_t*>(w_uk),
                                         static_cast<const uint16_t*>(w_uv),
                                         static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t st) {
  dim3 grid((a.N + 127) / 128, a.H, a.B);
  if (a.d_h == 64 && a.d_r == 32)
    prefill_attn_kernel<64, 32><<<grid, 256, 0, st>>>(a);
  else if (a.d_h == 128 && a.d_r == 64)
    prefill_attn_kernel<128, 64><<<grid, 256, 0, st>>>(a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace mtla
