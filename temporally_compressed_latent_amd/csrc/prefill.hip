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
  // Tile order: workgroups are dealt to the 8 XCDs round-robin by linear id
  // (id L runs on XCD L % 8).  Tiles are numbered row-major (the column tiles
  // of a row tile consecutive) and XCD x takes the x-th eighth of them, so
  // the column tiles that share an A row tile run on one XCD and read it from
  // one L2.  (When the tile count is not a multiple of 8, linear order.)
  const int ncol = gridDim.x, ntiles = gridDim.x * gridDim.y;
  const int L = blockIdx.x + gridDim.x * blockIdx.y;
  const int t = ntiles % 8 == 0 ? (L % 8) * (ntiles / 8) + L / 8 : L;
  const int col0 = (t % ncol) * GBN;
  const int row0 = (t / ncol) * GBM;
  const int HD = H * d_h;

  // Each thread copies 2 chunks of A and 2 of B per K step (16 B each).  A
  // goes through a buffer resource over its M rows (rows past M read as
  // zero); the B tile lies wholly in W_UK or in W_UV (HD is a multiple of
  // GBN), so its base is uniform.
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A), static_cast<short>(0), M * W * 2, kBufferRsrcWord3);
  const uint16_t* bmat = col0 < HD ? w_uk + static_cast<size_t>(col0) * d_c
                                   : w_uv + static_cast<size_t>(col0 - HD) * d_c;
  // Two K steps are in flight: each step's chunks land in one of two named
  // register sets (not arrays, so they are never placed in scratch) and go
  // to LDS one step later.
  const int r0 = tid >> 2, r1 = (tid + 256) >> 2, ch = tid & 3;  // chunk (r, ch), two per thread
  struct Regs {
    uint4 a0, a1, b0, b1;
  };
  auto gload = [&](Regs& R, int k0) {
    const int so = (row0 * W + k0) * 2;
    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rs_a, (r0 * W + ch * 8) * 2, so, 0);
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rs_a, (r1 * W + ch * 8) * 2, so, 0);
    R.a0 = uint4{v0[0], v0[1], v0[2], v0[3]};
    R.a1 = uint4{v1[0], v1[1], v1[2], v1[3]};
    R.b0 = *reinterpret_cast<const uint4*>(bmat + static_cast<size_t>(r0) * d_c + k0 + ch * 8);
    R.b1 = *reinterpret_cast<const uint4*>(bmat + static_cast<size_t>(r1) * d_c + k0 + ch * 8);
    // keep the loads where they are issued (the scheduler would sink them
    // towards their LDS stores, which then wait for a full round trip)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lstore = [&](const Regs& R, int buf) {
    *reinterpret_cast<uint4*>(&sA[buf][r0 * GP + ch * 8]) = R.a0;
    *reinterpret_cast<uint4*>(&sA[buf][r1 * GP + ch * 8]) = R.a1;
    *reinterpret_cast<uint4*>(&sB[buf][r0 * GP + ch * 8]) = R.b0;
    *reinterpret_cast<uint4*>(&sB[buf][r1 * GP + ch * 8]) = R.b1;
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
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
  };

  // step kt is computed from LDS buffer kt & 1; while it is, step kt + 1 sits
  // in registers (stored after the compute) and step kt + 2 is being loaded
  const int nk = d_c / GBK;
  Regs R0, R1;
  gload(R0, 0);
  gload(R1, min(1, nk - 1) * GBK);
  lstore(R0, 0);
  __syncthreads();
  // (the loads are issued unconditionally, steps past the end re-reading the
  // last one, so that the waits before the LDS stores count only the older set)
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    gload(R0, min(kt + 2, nk - 1) * GBK);
    compute(0);
    lstore(R1, 1);
    __syncthreads();
    gload(R1, min(kt + 3, nk - 1) * GBK);
    compute(1);
    lstore(R0, 0);  // unconditional, or the loads would be sunk next to it
    __syncthreads();
  }
  if (kt < nk) {  // odd step count: the last step is in buffer 0
    compute(0);
    __syncthreads();
  }

  // Epilogue: stage the 128x128 tile as bf16 in LDS (reusing the operand
  // buffers), then write each (token, head) row of d_h values with 16-byte
  // stores.  acc[i][j][q] is row wm*64 + i*16 + 4g + q, column wn*64 + j*16 + c16.
  constexpr int CP = GBN + 8;
  static_assert(GBM * CP <= 2 * 2 * GBM * GP, "C tile must fit in the operand buffers");
  uint16_t* sC = &sA[0][0];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sC[(wm * 64 + i * 16 + 4 * g + q) * CP + wn * 64 + j * 16 + c16] = f32_to_bf16_bits(acc[i][j][q]);
  __syncthreads();
  const bool isk = col0 < HD;
  uint16_t* dst = isk ? kout : vout;
  const int cbase = isk ? col0 : col0 - HD;
  for (int id = tid; id < GBM * (GBN / 8); id += 256) {
    const int r = id / (GBN / 8), cc = id % (GBN / 8);
    const int m = row0 + r;
    if (m < M) {
      const int col = cbase + cc * 8;
      const int hh = col / d_h, e = col % d_h;
      const int bb = m / N, nn = m % N;
      *reinterpret_cast<uint4*>(dst + ((static_cast<size_t>(bb) * H + hh) * N + nn) * d_h + e) =
          *reinterpret_cast<const uint4*>(sC + r * CP + cc * 8);
    }
  }
}

// ---------------------------------------------------------------------------
// Stride-masked attention, explicit per-head form, bf16 in / fp32 accumulate,
// on v_mfma_f32_32x32x16_bf16.
//
// Workgroup: 256 queries of one (sequence, head); wave w owns queries
// 64w..64w+63 as two 32-query MFMA column tiles.  Scores are computed
// transposed, S^T[slot, query] = K . Q^T (A = key rows from LDS, B = the
// wave's queries, held in registers for the whole kernel), so each lane holds
// one query column: the row max is in-lane plus one shuffle, and the
// probabilities are already laid out as the B operand of O^T += V^T . P^T.
// For a 16-slot chunk c of the tile the MFMA contraction index
// kappa = 8*grp + r (grp = lane / 32) maps to slot
//   r < 4 : 16c + 4*grp + r,      r >= 4 : 16c + 8 + 4*grp + (r - 4),
// which is exactly where the score tile left those probabilities; the V^T
// operand is read with that mapping by transposing LDS loads of the
// row-major value tile.
//
// The keys are the completed slots (token s*b - 1, 0-based, of slot b - 1),
// loaded 64 at a time; the next tile is fetched into registers while the
// current one is used.  Tiles past a wave's last visible slot are skipped by
// that wave, and only tiles that cross its staircase are masked.
//
// Vector-ALU budget (a wave64 VALU instruction takes 4 cycles, exp 16, and a
// 32x32x16 MFMA 32): the queries are pre-scaled by tau*log2(e), the score
// accumulators start at -m so the MFMA returns s - m directly, and the
// running max m is only moved (with the rescale of O and l) when some score
// of the wave exceeds it by more than 2^kLazyLog2; otherwise probabilities
// are taken against the stale max, which is exact after the final division
// by l and stays far from fp32 overflow.
// ---------------------------------------------------------------------------
template <int DH, int DR, int NQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NQ == 1 && DH == 64 ? 3 : 1)))
void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int DQK = DH + DR;
  constexpr int KK = DQK / 16;       // k-chunks of the score MFMA
  constexpr int DT = DH / 32;        // 32-row tiles of O^T
  constexpr int TS = 64;             // slots per tile
  constexpr int QW = 32 * NQ;        // queries per wave (NQ column tiles of 32)
  constexpr int QT = 4 * QW;         // queries per workgroup
  constexpr int KP = DQK + 8;        // key tile pitch (elements)
  constexpr int VP = DH + 8;         // value tile pitch
  static_assert(DH % 32 == 0 && DR % 16 == 0, "shape");
  constexpr float kLazyLog2 = 8.f;

  // two K/V tile buffers: the next tile is stored while this one is used
  __shared__ __align__(16) uint16_t sKb[2][TS * KP];
  __shared__ __align__(16) uint16_t sVb[2][TS * VP];

  // One-dimensional grid of B*H*nqt workgroups.  Workgroups are dealt to the
  // 8 XCDs round-robin by linear id (id L runs on XCD L % 8).  When B*H is a
  // multiple of 8, XCD x takes the (sequence, head) pairs x, x+8, ... one
  // after another, each pair's query tiles heaviest first: the workgroups an
  // XCD runs at once then share the K/V rows of two or three pairs, which stay
  // in its L2 (dealt by head instead, an XCD's working set was 16 sequences'
  // rows, several times its L2).  Otherwise every pair takes its heaviest
  // query tile before any lighter one.
  const int nqt = a.nqt;
  const int npair = a.B * a.H;
  const int L = blockIdx.x;
  int pair, qt;
  if (npair % 8 == 0) {
    const int k = L >> 3;
    pair = (L & 7) + 8 * (k / nqt);
    qt = nqt - 1 - k % nqt;
  } else {
    pair = L % npair;
    qt = nqt - 1 - L / npair;
  }
  const int h = pair % a.H, b = pair / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 5, c32 = lane & 31;
  const int N = a.N, H = a.H, s = a.s;
  const int W = a.d_c + DR;
  const int q0 = qt * QT;
  const int qw0 = q0 + wave * QW;
  const float qk_scale = a.scale * kLog2e;

  const uint16_t* qc = static_cast<const uint16_t*>(a.q_c);
  const uint16_t* qr = static_cast<const uint16_t*>(a.q_r);
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* vv = static_cast<const uint16_t*>(a.v) + (static_cast<size_t>(b) * H + h) * N * DH;
  const uint16_t* Pb = static_cast<const uint16_t*>(a.partials) + static_cast<size_t>(b) * N * W;
  // completed slot j (0-based) has its keys at row sm*j + sa of the slot
  // arrays; the queries are tokens t0+1 .. t0+N
  const int t0 = a.t0, sm = a.slot_mul, sa = a.slot_add;
  const uint16_t* ksl =
      static_cast<const uint16_t*>(a.kslot) + (static_cast<size_t>(b) * H + h) * a.slot_rows * DH;
  const uint16_t* vsl =
      static_cast<const uint16_t*>(a.vslot) + (static_cast<size_t>(b) * H + h) * a.slot_rows * DH;
  const uint16_t* Rb = static_cast<const uint16_t*>(a.rslot) + static_cast<size_t>(b) * a.rslot_rows * W;

  // Queries (B operands, registers) and the diagonal key j = i as the initial
  // online-softmax state: m = score(i, i), l = 1, O = V_i.
  bf16x8 qreg[NQ][KK];
  float m[NQ], lp[NQ];
  f32x16 acc[DT][NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int qi = qw0 + 32 * t + c32;  // 0-based query token
    const bool qok = qi < N;
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int d0 = 16 * kk + 8 * grp;
      uint4 qv = uint4{0u, 0u, 0u, 0u}, kv = uint4{0u, 0u, 0u, 0u};
      if (qok) {
        if (d0 < DH) {
          qv = *reinterpret_cast<const uint4*>(qc + ((static_cast<size_t>(b) * N + qi) * H + h) * DH + d0);
          kv = *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(qi) * DH + d0);
        } else {
          qv = *reinterpret_cast<const uint4*>(qr + ((static_cast<size_t>(b) * N + qi) * H + h) * DR + (d0 - DH));
          kv = *reinterpret_cast<const uint4*>(Pb + static_cast<size_t>(qi) * W + a.d_c + (d0 - DH));
        }
      }
      const u16x8 qs = __builtin_bit_cast(u16x8, qv), ks = __builtin_bit_cast(u16x8, kv);
      u16x8 qsc;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float qf = bf16_bits_to_f32(qs[r]);
        dpart = fmaf(qf, bf16_bits_to_f32(ks[r]), dpart);
        qsc[r] = f32_to_bf16_bits(qf * qk_scale);
      }
      qreg[t][kk] = __builtin_bit_cast(bf16x8, qsc);
    }
    dpart += __shfl_xor(dpart, 32, 64);
    m[t] = dpart * qk_scale;
    lp[t] = grp == 0 ? 1.f : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 v2 = uint2{0u, 0u};
        if (qok)
          v2 = *reinterpret_cast<const uint2*>(vv + static_cast<size_t>(qi) * DH + 32 * dt + 8 * j + 4 * grp);
        acc[dt][t][4 * j + 0] = __uint_as_float(v2.x << 16);
        acc[dt][t][4 * j + 1] = __uint_as_float(v2.x & 0xffff0000u);
        acc[dt][t][4 * j + 2] = __uint_as_float(v2.y << 16);
        acc[dt][t][4 * j + 3] = __uint_as_float(v2.y & 0xffff0000u);
      }
    }
  }

  // completed slots (0-based) visible to this lane's queries: slot j is seen
  // by query token t0 + qi + 1 iff s (j + 1) <= t0 + qi, i.e. j < vis[t]
  int vis[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) vis[t] = (t0 + qw0 + 32 * t + c32) / s;
  // completed slots seen by the workgroup's / this wave's last query, and the
  // slots every query of this wave sees
  const int nk = (t0 + min(q0 + QT, N) - 1) / s;
  const int nk_w = qw0 < N ? (t0 + min(qw0 + QW, N) - 1) / s : 0;
  const int full_w = (t0 + qw0) / s;

  // Tile loads through buffer resources bounded at the last completed slot's
  // key row (rows_end rows): slot rows past nk read as zero and touch no
  // memory.  Each load instruction uses one resource, so the chunks are split
  // by kind: per thread KN chunks of K^C, RN of the rope key and KN of V (16
  // bytes each); their offsets within a tile are loop invariant and the tile
  // offset is a scalar.
  constexpr int KN = TS * DH / 8 / 256, RN = TS * DR / 8 / 256;
  static_assert(KN * 256 == TS * DH / 8 && RN * 256 == TS * DR / 8, "chunks per thread");
  const int rows_end = nk > 0 ? sm * (nk - 1) + sa + 1 : 0;
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ksl), static_cast<short>(0), rows_end * DH * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vsl), static_cast<short>(0), rows_end * DH * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Rb + a.d_c), static_cast<short>(0),
      rows_end > 0 ? (rows_end - 1) * W * 2 + DR * 2 : 0, kBufferRsrcWord3);
  int off_k[KN], off_r[RN], lds_k[KN], lds_r[RN], lds_v[KN];
#pragma unroll
  for (int i = 0; i < KN; ++i) {
    const int c = tid + 256 * i, row = c / (DH / 8), cc = c % (DH / 8);
    off_k[i] = ((sm * row + sa) * DH + cc * 8) * 2;
    lds_k[i] = row * KP + cc * 8;
    lds_v[i] = row * VP + cc * 8;
  }
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = tid + 256 * i, row = c / (DR / 8), cc = c % (DR / 8);
    off_r[i] = ((sm * row + sa) * W + cc * 8) * 2;
    lds_r[i] = row * KP + DH + cc * 8;
  }
  uint4 pk[KN], pr[RN], pv[KN];
  auto load_tile = [&](int j0) {
    const int so_kv = sm * j0 * DH * 2, so_r = sm * j0 * W * 2;
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

  // Tile j0 sits in buffer `buf` at the top of each iteration and the loads
  // of tile j0+TS are in flight; the iteration stores tile j0+TS into the
  // other buffer, issues the loads of j0+2TS, uses tile j0, and ends with the
  // tile loop's only barrier.
  int buf = 0;
  if (nk > 0) {
    load_tile(0);
    store_tile(0);
    if (TS < nk) load_tile(TS);
  }
  __syncthreads();
  for (int j0 = 0; j0 < nk; j0 += TS, buf ^= 1) {
    if (j0 + TS < nk) {
      store_tile(buf ^ 1);
      if (j0 + 2 * TS < nk) load_tile(j0 + 2 * TS);
    }
    const uint16_t* sK = sKb[buf];
    const uint16_t* sV = sVb[buf];

    if (j0 < nk_w) {
      // S^T = K Q^T - m: sc[rt][t][i] = score(slot j0 + 32rt + 8(i/4) + 4grp + i%4,
      // query t) - m[t], in log2 units
      f32x16 sc[2][NQ];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int t = 0; t < NQ; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[rt][t][i] = -m[t];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sK + (32 * rt + c32) * KP + 16 * kk + 8 * grp);
#pragma unroll
          for (int t = 0; t < NQ; ++t)
            sc[rt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[t][kk], sc[rt][t], 0, 0, 0);
        }
      }
      const bool boundary = j0 + TS > full_w;
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        if (boundary) {
          // slot j0 + 32 rt + 8 (i / 4) + 4 grp + i % 4 is hidden iff it is
          // >= vis[t]: one per-lane bound against compile-time offsets
          const int rel = vis[t] - j0 - 4 * grp;
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * rt + 8 * (i / 4) + (i % 4) >= rel) sc[rt][t][i] = -INFINITY;
          }
        }
        // this lane's maximum over its 32 scores (four independent chains;
        // the file is built without NaN semantics, so these become
        // three-input maxima on the raw MFMA results); the other half of
        // the query's slots sits in lane ^ 32, which only the rare rescale
        // below needs
        float m4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) m4[u] = fmaxf(sc[0][t][u], sc[1][t][u]);
#pragma unroll
        for (int i = 4; i < 16; ++i) m4[i % 4] = fmaxf(m4[i % 4], fmaxf(sc[0][t][i], sc[1][t][i]));
        float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        if (__any(mx > kLazyLog2)) {
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float d = fmaxf(mx, 0.f);
          const float alpha = fast_exp2(-d);
          m[t] += d;
          lp[t] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[dt][t] *= alpha;
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[rt][t][i] -= d;
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[rt][t][i] = fast_exp2(sc[rt][t][i]);
        }
      }

      // O^T += V^T P^T over the tile's four 16-slot chunks
      const int q16 = lane >> 4, k16 = lane & 15;
      float lsum[NQ][2];
#pragma unroll
      for (int t = 0; t < NQ; ++t) lsum[t][0] = lsum[t][1] = 0.f;
#pragma unroll
      for (int c = 0; c < TS / 16; ++c) {
        const int rt = c / 2, jb = 2 * (c % 2);
        bf16x8 pb[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          u16x8 pk;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pk[r] = f32_to_bf16_bits(sc[rt][t][4 * jb + r]);
            pk[4 + r] = f32_to_bf16_bits(sc[rt][t][4 * (jb + 1) + r]);
          }
          pb[t] = __builtin_bit_cast(bf16x8, pk);
          // the row sum takes the bf16 probabilities the product uses: one
          // v_dot2 against (1, 1) per pair
          const uint4 pw = __builtin_bit_cast(uint4, pk);
          const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
          lsum[t][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.x), one2, lsum[t][0], false);
          lsum[t][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.y), one2, lsum[t][1], false);
          lsum[t][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.z), one2, lsum[t][0], false);
          lsum[t][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.w), one2, lsum[t][1], false);
        }
        const int sb0 = 16 * c + 4 * (q16 >> 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int col0 = 32 * dt + 16 * (q16 & 1);
          const uint16_t* base = sV + (sb0 + (k16 >> 2)) * VP + col0 + 4 * (k16 & 3);
          const s16x4 lo4 = lds_read_tr16(base);
          const s16x4 hi4 = lds_read_tr16(base + 8 * VP);
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NQ; ++t)
            acc[dt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[t], acc[dt][t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < NQ; ++t) lp[t] += lsum[t][0] + lsum[t][1];
    }
    __syncthreads();
  }

  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const float l = lp[t] + __shfl_xor(lp[t], 32, 64);
    const float inv = 1.f / l;
    const int qi = qw0 + 32 * t + c32;
    if (qi < N) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint16_t* dst = out + ((static_cast<size_t>(b) * N + qi) * H + h) * DH + 32 * dt + 8 * j + 4 * grp;
          const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][4 * j + 0] * inv)) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][4 * j + 1] * inv)) << 16);
          const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][4 * j + 2] * inv)) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(acc[dt][t][4 * j + 3] * inv)) << 16);
          *reinterpret_cast<uint2*>(dst) = uint2{w0, w1};
        }
      }
    }
  }
}

// 32-query column tiles per wave of the d_h = 64 attention kernel.
#ifndef MTLA_PREFILL_QUERY_TILES
#define MTLA_PREFILL_QUERY_TILES 1
#endif
constexpr int kPrefillQueryTiles = MTLA_PREFILL_QUERY_TILES;

}  // namespace

bool prefill_mfma_supported(int H, int d_h, int d_c, int d_r) {
  const bool shape = (d_h == 64 && d_r == 32) || (d_h == 128 && d_r == 64);
  // the GEMM's 128-column tiles must not straddle the K^C / V halves
  return shape && d_c % GBK == 0 && (H * d_h) % GBN == 0;
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

hipError_t launch_prefill_attn(const PrefillAttnArgs& a0, hipStream_t st) {
  PrefillAttnArgs a = a0;
  if (!a.kslot) {  // slot keys from the token-indexed arrays: slot j is token s*j + s - 1
    a.kslot = a.kc;
    a.vslot = a.v;
    a.rslot = a.partials;
    a.slot_rows = a.rslot_rows = a.N;
    a.slot_mul = a.s;
    a.slot_add = a.s - 1;
  }
  if (a.d_h == 64 && a.d_r == 32) {
    constexpr int nq = kPrefillQueryTiles;
    PrefillAttnArgs b = a;
    b.nqt = (a.N + 128 * nq - 1) / (128 * nq);
    prefill_attn_kernel<64, 32, nq><<<b.nqt * a.B * a.H, 256, 0, st>>>(b);
  } else if (a.d_h == 128 && a.d_r == 64) {
    PrefillAttnArgs b = a;
    b.nqt = (a.N + 127) / 128;
    prefill_attn_kernel<128, 64, 1><<<b.nqt * a.B * a.H, 256, 0, st>>>(b);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace mtla
