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
//   K/V GEMM  : K^C = P^c W_UK^T and V = P^c W_UV^T of the completed slots'
//               key rows only (MFMA GEMM, output [B, H, slots, d_h]; fp16 for
//               the attention below; over every token, bf16, for the training
//               backward)
//   attention : per (query tile, head, sequence): the diagonal key's K^C_i
//               and V_i formed from P_i in the kernel, then slot tiles
//               0 .. floor((i_max-1)/s); only boundary tiles are masked, tiles
//               past the last visible slot are never visited.
#include "common.hpp"
#include "gemm_tile.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

// ---------------------------------------------------------------------------
// Up-projection GEMM: C[m, col] = sum_k A[m, k] * Bw[col, k]
//   A  = P^c: the rows of partial merges or of cache slots that are keys
//        (a row selection per sequence), row stride W, K = d_c
//   Bw = [W_UK ; W_UV] viewed as [2*H*d_h, d_c]
// 256x128 output tiles (gemm_tile, transposed product), staged through LDS
// as fp16 or bf16 and written as 16-byte row chunks.  Output column col
// -> (K or V, head, e).
// ---------------------------------------------------------------------------
constexpr int GBM = 256, GBN = 128, GBK = 32;

template <bool F16OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kv_kernel(int B, int N, int a_seq_rows, int a_mul, int a_add,
                                                        int H, int d_h, int d_c, int W,
                                                        const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ w_uk,
                                                        const uint16_t* __restrict__ w_uv,
                                                        uint16_t* __restrict__ kout,
                                                        uint16_t* __restrict__ vout) {
  __shared__ __align__(16) uint16_t smem[TileShape<GBM>::SmemElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 5, c32 = lane & 31;
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
  const int M = B * N;

  // Output row m (sequence m / N, row j = m % N) reads input row
  // a_seq_rows*(m / N) + a_mul*j + a_add; rows past M read row M - 1 (their
  // products are not stored).  The 128 weight rows of a column tile lie
  // wholly in W_UK or in W_UV (HD is a multiple of GBN).
  const uint16_t* bmat = col0 < HD ? w_uk + static_cast<size_t>(col0) * d_c
                                   : w_uv + static_cast<size_t>(col0 - HD) * d_c;
  constexpr int NI = GBM / 64;
  const uint16_t* arow[NI];
  const uint16_t* wrow[2];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int m = min(row0 + 16 * (4 * k + wave) + (lane >> 2), M - 1);
    arow[k] = A + static_cast<size_t>((m / N) * a_seq_rows + (m % N) * a_mul + a_add) * W;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) wrow[k] = bmat + static_cast<size_t>(16 * (4 * k + wave) + (lane >> 2)) * d_c;
  f32x16 acc[NI][2];
  gemm_tile<GBM, true>(arow, wrow, d_c, smem, acc);

  // Epilogue: stage the 256x128 tile as fp16 (F16OUT) or bf16 in LDS, then
  // write each (token, head) row of d_h values with 16-byte stores.
  // acc[i][j][e] is row (GBM / 2) wm + 32 i + c32, column 64 wn + 32 j + 8 (e / 4)
  // + 4 grp + e % 4: one 8-byte LDS store per four values.
  constexpr int CP = GBN + 8;
  static_assert(GBM * CP <= TileShape<GBM>::SmemElems, "C tile must fit in the operand stages");
  uint16_t* sC = smem;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x16& c = acc[i][j];
        uint32_t w0, w1;
        if constexpr (F16OUT) {
          w0 = f32_to_f16_bits(c[4 * e4]) | (uint32_t(f32_to_f16_bits(c[4 * e4 + 1])) << 16);
          w1 = f32_to_f16_bits(c[4 * e4 + 2]) | (uint32_t(f32_to_f16_bits(c[4 * e4 + 3])) << 16);
        } else {
          w0 = f32_to_bf16_bits(c[4 * e4]) | (uint32_t(f32_to_bf16_bits(c[4 * e4 + 1])) << 16);
          w1 = f32_to_bf16_bits(c[4 * e4 + 2]) | (uint32_t(f32_to_bf16_bits(c[4 * e4 + 3])) << 16);
        }
        *reinterpret_cast<uint2*>(&sC[((GBM / 2) * wm + 32 * i + c32) * CP + 64 * wn + 32 * j + 8 * e4 + 4 * grp]) =
            uint2{w0, w1};
      }
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
// Stride-masked attention, explicit per-head form, fp16 operands / fp32
// accumulate, on v_mfma_f32_32x32x16_f16.  The slot keys and values K^C, V
// are the K/V GEMM's fp16 output, the scaled queries, the rope keys and the
// probabilities are converted to fp16 here (the diagonal key is formed and
// used in fp32): every operand then carries 11
// significant bits (bf16: 8), so the attention adds 8x less rounding than
// with bf16 operands, at the same MFMA rate.  The queries and rope keys are
// bf16 storage and convert exactly.
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
  // bound on the running max's magnitude (log2 units), inside fp16's range
  constexpr float kMaxRef = 60000.f;

  // two K/V tile buffers (the next tile is stored while this one is used),
  // in one array: before the first tile it holds the diagonal's weights
  __shared__ __align__(16) uint16_t smem[2 * TS * KP + 2 * TS * VP];
  auto kbuf = [&](int buf) { return smem + buf * (TS * KP); };
  auto vbuf = [&](int buf) { return smem + 2 * TS * KP + buf * (TS * VP); };

  // One-dimensional grid of B*H*nqt workgroups.  Workgroups are dealt to the
  // 8 XCDs round-robin by linear id (id L runs on XCD L % 8).  When B*H is a
  // multiple of 8, XCD x takes the x-th eighth of the (sequence, head) pairs
  // (pair = sequence*H + head), one pair after another, each pair's query
  // tiles heaviest first: the workgroups an XCD runs at once then share the
  // K/V rows of two or three pairs and the partial merges and rope keys of
  // one sequence, which stay in its L2.  Otherwise every pair takes its
  // heaviest query tile before any lighter one.
  const int nqt = a.nqt;
  const int npair = a.B * a.H;
  const int L = blockIdx.x;
  int pair, qt;
  if (npair % 8 == 0) {
    const int k = L >> 3;
    pair = (L & 7) * (npair / 8) + k / nqt;
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
  const uint16_t* Pb = static_cast<const uint16_t*>(a.partials) + static_cast<size_t>(b) * N * W;
  // completed slot j (0-based) has K^C, V at row j of the slot arrays and its
  // rope key at row rm*j + ra of the rope array; the queries are tokens
  // t0+1 .. t0+N
  const int t0 = a.t0, rm = a.rslot_mul, ra = a.rslot_add;
  const uint16_t* ksl =
      static_cast<const uint16_t*>(a.kslot) + (static_cast<size_t>(b) * H + h) * a.slot_rows * DH;
  const uint16_t* vsl =
      static_cast<const uint16_t*>(a.vslot) + (static_cast<size_t>(b) * H + h) * a.slot_rows * DH;
  const uint16_t* Rb = static_cast<const uint16_t*>(a.rslot) + static_cast<size_t>(b) * a.rslot_rows * W;

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
  // rows: slot rows past nk read as zero and touch no memory.  Each load instruction uses one resource, so the chunks are split
  // by kind: per thread KN chunks of K^C, RN of the rope key and KN of V (16
  // bytes each); their offsets within a tile are loop invariant and the tile
  // offset is a scalar.
  constexpr int KN = TS * DH / 8 / 256, RN = TS * DR / 8 / 256;
  static_assert(KN * 256 == TS * DH / 8 && RN * 256 == TS * DR / 8, "chunks per thread");
  const int rope_end = nk > 0 ? rm * (nk - 1) + ra + 1 : 0;
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ksl), static_cast<short>(0), nk * DH * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vsl), static_cast<short>(0), nk * DH * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Rb + a.d_c), static_cast<short>(0),
      rope_end > 0 ? (rope_end - 1) * W * 2 + DR * 2 : 0, kBufferRsrcWord3);
  int off_k[KN], off_r[RN], lds_k[KN], lds_r[RN], lds_v[KN];
#pragma unroll
  for (int i = 0; i < KN; ++i) {
    const int c = tid + 256 * i, row = c / (DH / 8), cc = c % (DH / 8);
    off_k[i] = (row * DH + cc * 8) * 2;
    lds_k[i] = row * KP + cc * 8;
    lds_v[i] = row * VP + cc * 8;
  }
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = tid + 256 * i, row = c / (DR / 8), cc = c % (DR / 8);
    off_r[i] = ((rm * row + ra) * W + cc * 8) * 2;
    lds_r[i] = row * KP + DH + cc * 8;
  }
  uint4 pk[KN], pr[RN], pv[KN];
  auto load_tile = [&](int j0) {
    const int so_kv = j0 * DH * 2, so_r = rm * j0 * W * 2;
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
    for (int i = 0; i < KN; ++i) *reinterpret_cast<uint4*>(kbuf(buf) + lds_k[i]) = pk[i];
#pragma unroll
    for (int i = 0; i < RN; ++i) {
      // the rope key: bf16 storage to fp16 (exact in fp16's normal range)
      const uint32_t w4[4] = {pr[i].x, pr[i].y, pr[i].z, pr[i].w};
      uint32_t h4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f16x2 h = {static_cast<_Float16>(__uint_as_float(w4[k] << 16)),
                         static_cast<_Float16>(__uint_as_float(w4[k] & 0xffff0000u))};
        h4[k] = __builtin_bit_cast(uint32_t, h);
      }
      *reinterpret_cast<uint4*>(kbuf(buf) + lds_r[i]) = uint4{h4[0], h4[1], h4[2], h4[3]};
    }
#pragma unroll
    for (int i = 0; i < KN; ++i) *reinterpret_cast<uint4*>(vbuf(buf) + lds_v[i]) = pv[i];
  };

  if (nk > 0) load_tile(0);

  // The diagonal key j = i.  Its K^C_i = W_UK[h] P^c_i and V_i = W_UV[h] P^c_i
  // are formed here, for the wave's queries, as D^T[e, query] = W[e, :] .
  // P^c[query, :] on 32x32x16 bf16 MFMAs (exact products, fp32 sums).  The
  // weights go through LDS, shared by the four waves, in rounds of RC
  // columns of both blocks: each round's loads are issued at once straight
  // into LDS (no registers), with the 16-byte pieces of a row permuted by
  // piece ^ (row % 16) so that the MFMA operand reads are free of bank
  // conflicts.  The partial merges are the B operands, read straight from
  // memory (rows past N read as zero).  A product's layout (lane = query,
  // rows 8(i/4) + 4 grp + i%4 of each 32-row tile) is that of the O^T
  // accumulators, so V_i is the initial O^T as it comes out.  The first key
  // tile's loads are already in flight.
  constexpr int RC = 128;               // weight columns per round
  constexpr int RP = RC / 8;            // 16-byte pieces per row and round
  constexpr int WROWS = 2 * DH;         // the W_UK[h] rows, then W_UV[h]'s
  constexpr int WLD = WROWS * RP / 256; // loads per thread and round
  static_assert(WROWS * RC <= 2 * TS * KP + 2 * TS * VP, "a round of weights fits in the tile buffers");
  static_assert(WLD % 2 == 0 && DH % 4 == 0, "each load lies wholly in one weight block");
  const int wbytes = a.H * DH * a.d_c * 2;
  const i32x4_t rs_wk = make_rsrc_words(a.w_uk, wbytes), rs_wv = make_rsrc_words(a.w_uv, wbytes);
  const uint32_t lds_w = lds_addr(smem);
  const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Pb), static_cast<short>(0), N * W * 2, kBufferRsrcWord3);
  int poff[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) poff[t] = ((qw0 + 32 * t + c32) * W + 8 * grp) * 2;
  f32x16 kd[DT][NQ];
  f32x16 acc[DT][NQ];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int t = 0; t < NQ; ++t) kd[dt][t] = acc[dt][t] = f32x16{};
  for (int c0 = 0; c0 < a.d_c; c0 += RC) {
    // load k of this wave writes LDS pieces 64 (4k + wave) .. + 63: rows
    // 4 (4k + wave) .. + 3 of the round, in W_UK[h] for k < WLD/2
#pragma unroll
    for (int k = 0; k < WLD; ++k) {
      const int q = (4 * k + wave) * 64 + lane;
      const int r = q / RP, pc = (q % RP) ^ (r % RP);
      const int voff = ((h * DH + r % DH) * a.d_c + 8 * pc) * 2;
      const uint32_t dst = lds_w + __builtin_amdgcn_readfirstlane((4 * k + wave) * 1024);
      buffer_load_lds16_cached(2 * k < WLD ? rs_wk : rs_wv, dst, voff, c0 * 2);
    }
    // the B operands of the round's (up to) RC/16 chunks (loaded for all RC/16:
    // past d_c they read the next row or zero, and are not used)
    const int kcn = min(RC, a.d_c - c0) / 16;
    bf16x8 pf[NQ][RC / 16];
#pragma unroll
    for (int kc = 0; kc < RC / 16; ++kc)
#pragma unroll
      for (int t = 0; t < NQ; ++t)
        pf[t][kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_p, poff[t], (c0 + 16 * kc) * 2, 0));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < RC / 16; ++kc) {
      if (kc < kcn) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rk = 32 * dt + c32, rv = DH + 32 * dt + c32;  // rk % 16 == rv % 16 == c32 % 16
          const int pc = (2 * kc + grp) ^ (c32 % RP);
          const bf16x8 wk = *reinterpret_cast<const bf16x8*>(smem + rk * RC + 8 * pc);
          const bf16x8 wv = *reinterpret_cast<const bf16x8*>(smem + rv * RC + 8 * pc);
#pragma unroll
          for (int t = 0; t < NQ; ++t) {
            kd[dt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wk, pf[t][kc], kd[dt][t], 0, 0, 0);
            acc[dt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, pf[t][kc], acc[dt][t], 0, 0, 0);
          }
        }
      }
    }
    // every wave is done with this round's weights before they are replaced
    // (or, after the last round, overwritten by the first key tile)
    __syncthreads();
  }

  // Queries (B operands, registers) and the diagonal key as the initial
  // online-softmax state: m = score(i, i), l = 1, O = V_i.
  f16x8 qreg[NQ][KK];
  // The running max m enters the score product as a 7th k-chunk: the query
  // side holds -m (element 0 of lane group 0) and the key side a constant 1,
  // so the MFMA returns s - m with no per-score subtraction or accumulator
  // initialisation.  m is therefore kept fp16-representable, and the
  // diagonal's weight is taken against that same value.
  f16x8 qm[NQ];
  f16x8 kone;
#pragma unroll
  for (int r = 0; r < 8; ++r) kone[r] = static_cast<_Float16>(grp == 0 && r == 0 ? 1.f : 0.f);
  float m[NQ], lp[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int qi = qw0 + 32 * t + c32;  // 0-based query token
    const bool qok = qi < N;
    const uint16_t* qrow = qc + ((static_cast<size_t>(b) * N + qi) * H + h) * DH;
    // q^C . K^C_i over this lane's rows of kd (the other half is in lane ^ 32)
    float dpart = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 q2 = qok ? *reinterpret_cast<const uint2*>(qrow + 32 * dt + 8 * j + 4 * grp) : uint2{0u, 0u};
        dpart = fmaf(__uint_as_float(q2.x << 16), kd[dt][t][4 * j + 0], dpart);
        dpart = fmaf(__uint_as_float(q2.x & 0xffff0000u), kd[dt][t][4 * j + 1], dpart);
        dpart = fmaf(__uint_as_float(q2.y << 16), kd[dt][t][4 * j + 2], dpart);
        dpart = fmaf(__uint_as_float(q2.y & 0xffff0000u), kd[dt][t][4 * j + 3], dpart);
      }
    // the query operands, and q^R . P^R_i over this lane's half of the rope
    // columns
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int d0 = 16 * kk + 8 * grp;
      uint4 qv = uint4{0u, 0u, 0u, 0u}, kv = uint4{0u, 0u, 0u, 0u};
      if (qok) {
        if (d0 < DH) {
          qv = *reinterpret_cast<const uint4*>(qrow + d0);
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
        if (d0 >= DH) dpart = fmaf(qf, bf16_bits_to_f32(ks[r]), dpart);
        qsc[r] = f32_to_f16_bits(qf * qk_scale);
      }
      qreg[t][kk] = __builtin_bit_cast(f16x8, qsc);
    }
    dpart += __shfl_xor(dpart, 32, 64);
    const float sii = dpart * qk_scale;
    m[t] = f16_round(fminf(fmaxf(sii, -kMaxRef), kMaxRef));
    const float pii = fast_exp2(sii - m[t]);
    lp[t] = grp == 0 ? pii : 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) qm[t][r] = static_cast<_Float16>(grp == 0 && r == 0 ? -m[t] : 0.f);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt][t] *= pii;
  }

  // Tile j0 sits in buffer `buf` at the top of each iteration and the loads
  // of tile j0+TS are in flight; the iteration stores tile j0+TS into the
  // other buffer, issues the loads of j0+2TS, uses tile j0, and ends with the
  // tile loop's only barrier.
  int buf = 0;
  if (nk > 0) {
    store_tile(0);
    if (TS < nk) load_tile(TS);
  }
  __syncthreads();
  for (int j0 = 0; j0 < nk; j0 += TS, buf ^= 1) {
    if (j0 + TS < nk) {
      store_tile(buf ^ 1);
      if (j0 + 2 * TS < nk) load_tile(j0 + 2 * TS);
    }
    const uint16_t* sK = kbuf(buf);
    const uint16_t* sV = vbuf(buf);

    if (j0 < nk_w) {
      // S^T = K Q^T - m: sc[rt][t][i] = score(slot j0 + 32rt + 8(i/4) + 4grp + i%4,
      // query t) - m[t], in log2 units (the last k-chunk is 1 x -m)
      f32x16 sc[2][NQ];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int t = 0; t < NQ; ++t) sc[rt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kone, qm[t], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const f16x8 ak = *reinterpret_cast<const f16x8*>(sK + (32 * rt + c32) * KP + 16 * kk + 8 * grp);
#pragma unroll
          for (int t = 0; t < NQ; ++t)
            sc[rt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qreg[t][kk], sc[rt][t], 0, 0, 0);
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
          // the new reference, fp16-representable, and the exact shift to it
          const float mnew = f16_round(fminf(m[t] + fmaxf(mx, 0.f), kMaxRef));
          const float d = mnew - m[t];
          const float alpha = fast_exp2(-d);
          m[t] = mnew;
#pragma unroll
          for (int r = 0; r < 8; ++r) qm[t][r] = static_cast<_Float16>(grp == 0 && r == 0 ? -mnew : 0.f);
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
        f16x8 pb[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          f16x8 pk;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pk[r] = static_cast<_Float16>(sc[rt][t][4 * jb + r]);
            pk[4 + r] = static_cast<_Float16>(sc[rt][t][4 * (jb + 1) + r]);
          }
          pb[t] = pk;
          // the row sum takes the fp16 probabilities the product uses: one
          // v_dot2 against (1, 1) per pair
          const f16x2 one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
          lsum[t][0] = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk, pk, 0, 1), one2, lsum[t][0], false);
          lsum[t][1] = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk, pk, 2, 3), one2, lsum[t][1], false);
          lsum[t][0] = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk, pk, 4, 5), one2, lsum[t][0], false);
          lsum[t][1] = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk, pk, 6, 7), one2, lsum[t][1], false);
        }
        const int sb0 = 16 * c + 4 * (q16 >> 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int col0 = 32 * dt + 16 * (q16 & 1);
          const uint16_t* base = sV + (sb0 + (k16 >> 2)) * VP + col0 + 4 * (k16 & 3);
          const s16x4 lo4 = lds_read_tr16(base);
          const s16x4 hi4 = lds_read_tr16(base + 8 * VP);
          const f16x8 av = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NQ; ++t)
            acc[dt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[t], acc[dt][t], 0, 0, 0);
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
          const bf16x2 p0 = {static_cast<__bf16>(acc[dt][t][4 * j + 0] * inv),
                             static_cast<__bf16>(acc[dt][t][4 * j + 1] * inv)};
          const bf16x2 p1 = {static_cast<__bf16>(acc[dt][t][4 * j + 2] * inv),
                             static_cast<__bf16>(acc[dt][t][4 * j + 3] * inv)};
          *reinterpret_cast<uint2*>(dst) = uint2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
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

hipError_t launch_prefill_kv(int B, int n_rows, int a_seq_rows, int a_mul, int a_add, int H, int d_h, int d_c,
                            int d_r, const void* a, const void* w_uk, const void* w_uv, void* k_out, void* v_out,
                            bool out_fp16, hipStream_t st) {
  const int M = B * n_rows;
  if (M == 0) return hipSuccess;
  dim3 grid((2 * H * d_h) / GBN, (M + GBM - 1) / GBM);
  auto args = [&](auto kern) {
    kern<<<grid, 256, 0, st>>>(B, n_rows, a_seq_rows, a_mul, a_add, H, d_h, d_c, d_c + d_r,
                               static_cast<const uint16_t*>(a),
                               static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
                               static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  };
  if (out_fp16)
    args(prefill_kv_kernel<true>);
  else
    args(prefill_kv_kernel<false>);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t st) {
  if (a.B == 0 || a.N == 0) return hipSuccess;
  if (a.d_c % 32 != 0) return hipErrorInvalidValue;
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
