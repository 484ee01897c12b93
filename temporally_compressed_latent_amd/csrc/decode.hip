// Absorbed-form attention over the slot cache ("Multi-head Temporal Latent
// Attention", Method: W_UK folded into the query, W_UV applied after the
// weighted latent sum; "Multi-Head Latent Attention and Sparse Indexers",
// "Latent attention changes the representation").
//
//   absorb     : q~[r, h] = W_UK[h]^T q_c[r, h]  (plus the rope query, copied)
//   attention  : split-K over cache slots; per split an online-softmax partial
//                (running max m, sum l, latent accumulator acc[d_c]); the
//                splits are merged in a fixed order into o_lat = acc / l
//   up-project : out[r, h] = W_UV[h] o_lat[r, h]
//
// Every head reads the same slot rows, so the MFMA decode kernel puts all
// heads of a sequence in one workgroup (heads are the MFMA M dimension) and
// reads each cache row from HBM once.
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "merge_body.hpp"

namespace mtla {

namespace {

constexpr int kAbsorbMaxDh = 256;  // rows of the staged W_UK tile (d_h bound)

// ---------------------------------------------------------------------------
// absorb: one workgroup per (head, block of RB rows).
//   q~[r, k] = sum_e q_c[r, e] W_UK[h, e, k]
// Thread t owns the 8 latent columns of chunk kc = t % KC (KC = d_c / 8) for
// the rows e = eg, eg + EG, ... (EG = 256 / KC groups); each W_UK row chunk
// is one 16-byte load, reused for all RB query rows.  The EG partial sums are
// added in group order through LDS.
// ---------------------------------------------------------------------------
template <typename T, int RB>
__global__ __launch_bounds__(256) void absorb_kernel(int R, int H, int d_h, int d_c, int d_r,
                                                     const T* __restrict__ q_c,
                                                     const T* __restrict__ q_r,
                                                     const T* __restrict__ w_uk,
                                                     float* __restrict__ qbuf) {
  extern __shared__ float smem[];
  float* sq = smem;               // [RB][d_h]
  float* red = smem + RB * d_h;   // [EG][RB][d_c]
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * RB;
  const int W = d_c + d_r;
  const int KC = d_c / 8, EG = 256 / KC;
  const int t = threadIdx.x, kc = t % KC, eg = t / KC;
  for (int idx = t; idx < RB * d_h; idx += 256) {
    const int rr = idx / d_h, e = idx % d_h;
    const int r = r0 + rr;
    sq[idx] = r < R ? Store<T>::load(q_c, (static_cast<size_t>(r) * H + h) * d_h + e) : 0.f;
  }
  __syncthreads();
  if (eg < EG) {
    float acc[RB][8];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[rr][j] = 0.f;
    // rows e = eg, eg + EG, ... in batches of 8 loads issued together (the
    // index is clamped, and rows past d_h get a zero query)
    for (int e0 = eg; e0 < d_h; e0 += 8 * EG) {
      float w[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = min(e0 + u * EG, d_h - 1);
        load8(w_uk + (static_cast<size_t>(h) * d_h + e) * d_c + kc * 8, w[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * EG;
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          const float q = e < d_h ? sq[rr * d_h + e] : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[rr][j] = fmaf(q, w[u][j], acc[rr][j]);
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[(eg * RB + rr) * d_c + kc * 8 + j] = acc[rr][j];
  }
  __syncthreads();
  for (int idx = t; idx < RB * d_c; idx += 256) {
    const int rr = idx / d_c, k = idx % d_c;
    float v = 0.f;
    for (int g2 = 0; g2 < EG; ++g2) v += red[(g2 * RB + rr) * d_c + k];
    if (r0 + rr < R) qbuf[(static_cast<size_t>(r0 + rr) * H + h) * W + k] = v;
  }
  for (int idx = t; idx < RB * d_r; idx += 256) {
    const int rr = idx / d_r, e = idx % d_r;
    const int r = r0 + rr;
    if (r < R)
      qbuf[(static_cast<size_t>(r) * H + h) * W + d_c + e] =
          Store<T>::load(q_r, (static_cast<size_t>(r) * H + h) * d_r + e);
  }
}

// ---------------------------------------------------------------------------
// Key set of query row r.
//   decode : slots 1..ceil(pos/s) of sequence r (no extra row)
//   prefill: completed slots 1..floor((i-1)/s) of sequence b, then the query's
//            own cumulative partial merge P_i (the "diagonal" key)
// ---------------------------------------------------------------------------
struct KeySet {
  int b;
  int n;             // cache rows
  const void* diag;  // extra row or nullptr
  bool ok;
};

template <typename T>
__device__ __forceinline__ KeySet key_set(const AttendArgs& a, int r) {
  KeySet k;
  const int W = a.d_c + a.d_r;
  if (a.N == 0) {
    k.b = r;
    const int pos = a.pos[r];
    k.ok = pos >= 1;
    k.n = k.ok ? slot_of(pos, a.s) : 0;
    k.ok = k.ok && k.n <= a.max_slots;
    if (!k.ok) k.n = 0;
    k.diag = nullptr;
  } else {
    k.b = r / a.N;
    const int i = a.t0 + r % a.N + 1;
    k.n = completed_slots(i, a.s);
    k.diag = static_cast<const T*>(a.diag) + static_cast<size_t>(r) * W;
    k.ok = true;
  }
  return k;
}

// ---------------------------------------------------------------------------
// Portable attention: one wave per (split, head, query row).  Lanes own
// columns e = lane + 64 k; each key row costs one wave reduction.
// ---------------------------------------------------------------------------
template <typename T, int MAXE>
__global__ __launch_bounds__(64) void attend_portable_kernel(AttendArgs a) {
  const int split = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x;
  const int W = a.d_c + a.d_r;
  const KeySet ks = key_set<T>(a, r);
  float qv[MAXE];
#pragma unroll
  for (int k = 0; k < MAXE; ++k) {
    const int e = lane + 64 * k;
    qv[k] = e < W ? a.qbuf[(static_cast<size_t>(r) * a.H + h) * W + e] : 0.f;
  }
  const int lo = static_cast<int>((static_cast<long long>(split) * ks.n) / a.splits);
  const int hi = static_cast<int>((static_cast<long long>(split + 1) * ks.n) / a.splits);
  float m = -INFINITY, l = 0.f;
  float acc[MAXE];
#pragma unroll
  for (int k = 0; k < MAXE; ++k) acc[k] = 0.f;

  auto visit = [&](const T* row) {
    float x[MAXE];
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < MAXE; ++k) {
      const int e = lane + 64 * k;
      x[k] = e < W ? Store<T>::load(row, e) : 0.f;
      d = fmaf(qv[k], x[k], d);
    }
    const float z = wave_sum(d) * a.scale;
    const float mn = fmaxf(m, z);
    const float alpha = expf(m - mn);
    const float p = expf(z - mn);
    l = l * alpha + p;
#pragma unroll
    for (int k = 0; k < MAXE; ++k) acc[k] = acc[k] * alpha + p * x[k];
    m = mn;
  };

  const T* cache = static_cast<const T*>(a.cache) + static_cast<size_t>(ks.b) * a.max_slots * W;
  for (int j = lo; j < hi; ++j) visit(cache + static_cast<size_t>(j) * W);
  if (ks.diag && split == 0) visit(static_cast<const T*>(ks.diag));

  const size_t pi = (static_cast<size_t>(r) * a.splits + split) * a.H + h;
  if (lane == 0) {
    a.part.m[pi] = m;
    a.part.l[pi] = l;
  }
#pragma unroll
  for (int k = 0; k < MAXE; ++k) {
    const int e = lane + 64 * k;
    if (e < a.d_c) a.part.acc[pi * a.d_c + e] = acc[k];
  }
}

// ---------------------------------------------------------------------------
// Split merge (portable path): one workgroup per (head, row); the splits'
// (m, l, acc) are merged in split order into o_lat[r, h, :] (fp32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_merge_kernel(int H, int d_c, int splits, Partials p,
                                                          float* __restrict__ o_lat) {
  const int h = blockIdx.x, r = blockIdx.y;
  const size_t base = static_cast<size_t>(r) * splits * H + h;  // + k * H
  float M = -INFINITY;
  for (int k = 0; k < splits; ++k) M = fmaxf(M, p.m[base + static_cast<size_t>(k) * H]);
  float L = 0.f;
  for (int k = 0; k < splits; ++k)
    L = fmaf(p.l[base + static_cast<size_t>(k) * H], expf(p.m[base + static_cast<size_t>(k) * H] - M), L);
  for (int e = threadIdx.x; e < d_c; e += blockDim.x) {
    float v = 0.f;
    for (int k = 0; k < splits; ++k) {
      const size_t pk = base + static_cast<size_t>(k) * H;
      v = fmaf(p.acc[pk * d_c + e], expf(p.m[pk] - M), v);
    }
    o_lat[(static_cast<size_t>(r) * H + h) * d_c + e] = v / L;
  }
}

// ---------------------------------------------------------------------------
// Up-projection: out[r, h, e] = sum_k W_UV[h, e, k] o_lat[r, h, k].
// One workgroup per (head, block of RB rows).  TPO consecutive threads share
// output row e and split its d_c / 8 chunks; each chunk is one 16-byte load of
// W_UV, reused for all RB rows, and the TPO partial dots are added with
// butterfly shuffles.
// ---------------------------------------------------------------------------
template <typename T, int RB>
__global__ __launch_bounds__(256) void up_project_kernel(int R, int H, int d_h, int d_c, int tpo,
                                                         const float* __restrict__ o_lat,
                                                         const T* __restrict__ w_uv,
                                                         T* __restrict__ out) {
  extern __shared__ float olat[];  // [RB][d_c]
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * RB;
  const int t = threadIdx.x;
  for (int idx = t; idx < RB * d_c; idx += 256) {
    const int rr = idx / d_c, k = idx % d_c;
    const int r = r0 + rr;
    olat[idx] = r < R ? o_lat[(static_cast<size_t>(r) * H + h) * d_c + k] : 0.f;
  }
  __syncthreads();
  const int e = t / tpo, p = t % tpo;
  const int KC = d_c / 8;
  float acc[RB];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) acc[rr] = 0.f;
  if (e < d_h) {
    // chunks c = p, p + tpo, ... in batches of 8 loads issued together (the
    // index is clamped; chunks past KC are skipped)
    for (int c0 = p; c0 < KC; c0 += 8 * tpo) {
      float w[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        load8(w_uv + (static_cast<size_t>(h) * d_h + e) * d_c + min(c0 + u * tpo, KC - 1) * 8, w[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * tpo;
        if (c < KC) {
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) {
            const float* o = olat + rr * d_c + c * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[rr] = fmaf(w[u][j], o[j], acc[rr]);
          }
        }
      }
    }
  }
  for (int off = tpo / 2; off >= 1; off >>= 1) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) acc[rr] += __shfl_xor(acc[rr], off, 64);
  }
  if (p == 0 && e < d_h) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
      if (r0 + rr < R) Store<T>::store(out, (static_cast<size_t>(r0 + rr) * H + h) * d_h + e, acc[rr]);
  }
}

// ---------------------------------------------------------------------------
// MFMA latent attention core (bf16 cache), shared by the split-K decode
// kernel and the fused one-token step kernel.  A workgroup of NW waves takes
// all heads of one sequence (padded to HT*16 MFMA rows) over a slot range.
//
// Per TS-slot tile:
//   1. the tile (TS rows x W bf16) is copied HBM -> registers -> LDS, and the
//      next tile's loads are issued before this tile is used;
//   2. scores S[head, slot] = Q~ . row via v_mfma_f32_16x16x32_bf16; the first
//      TS/16 waves own 16 slots each, A = scaled queries (LDS, a bf16 high
//      and low part, two products per k-step, so the fp32 query keeps 16
//      significant bits), B = rows (LDS);
//   3. the tile max per head is shared through LDS, p = exp2(S - m) goes to
//      LDS as bf16, and every wave rescales its running (m, acc);
//   4. acc[head, col] += P . rows, wave w owning latent columns
//      w*DC/NW .. (w+1)*DC/NW-1.  The B operand (8 slots of one column) comes
//      from two ds_read_b64_tr_b16 transposing loads of the row-major tile.
// Scores are carried in the log2 domain (queries pre-scaled by tau*log2 e).
// ---------------------------------------------------------------------------
template <int HT, int DC, int DR, int NW, int TS>
struct MfmaAttn {
  static constexpr int W = DC + DR;
  static constexpr int KS = W / 32;
  static constexpr int HP = HT * 16;
  static constexpr int PITCH = W + 8;  // LDS row pitch (elements)
  static constexpr int PP = TS + 8;    // probability tile pitch
  static constexpr int QKW = TS / 16;  // waves that score
  static constexpr int CPW = DC / NW;  // PV latent columns per wave
  static constexpr int CT = CPW / 16;
  static constexpr int CPR = W / 8;    // 16-byte chunks per row
  static constexpr int NT = NW * 64;
  static constexpr int CHUNKS = TS * CPR;
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;
  static_assert(W % 32 == 0 && TS % 32 == 0 && QKW <= NW, "tile shape");
  static_assert(DC % NW == 0 && CPW % 16 == 0, "column split");

  struct __align__(16) Smem {
    uint16_t q[HP * PITCH];   // scaled queries, bf16 high part
    uint16_t ql[HP * PITCH];  // and low part (q = q + ql to 16 bits)
    uint16_t k[TS * PITCH];
    uint16_t p[HP * PP];
    float red[NW][HP];
  };

  struct State {
    float m[HT][4];
    float l[HT][4];
    f32x4 acc[HT][CT];
  };

  __device__ __forceinline__ static void init(State& st) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st.m[ht][i] = -INFINITY;
        st.l[ht][i] = 0.f;
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) st.acc[ht][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Buffer resource over the memory rows [0, hm) of a sequence (hm * W bf16
  // from `rows`): a load past them returns zero and touches no memory.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* rows, int hm) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(rows), static_cast<short>(0),
                                             hm * W * 2, kBufferRsrcWord3);
  }

  // Issue the loads of the tile of slots j0 .. j0+TS-1 into registers: chunk
  // id = tid + NT*k of the tile is 16 bytes at byte j0*W*2 + id*16 of the
  // rows (the tile's rows are contiguous), so every load shares one offset
  // register.  All of a thread's loads are in flight together; rows at or
  // past hm read as zero.
  __device__ __forceinline__ static void load_tile(uint4* pre, __amdgpu_buffer_rsrc_t rs, int j0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, j0 * (W * 2) + k * (NT * 16), 0);
      pre[k] = uint4{v[0], v[1], v[2], v[3]};
    }
  }

  // Issue the loads of the first PD tiles of slots [lo, ..).
  template <int PD>
  __device__ __forceinline__ static void prefetch(uint4* pre, __amdgpu_buffer_rsrc_t rs, int lo) {
#pragma unroll
    for (int d = 0; d < PD; ++d) load_tile(pre + d * CPT, rs, lo + d * TS);
  }

  // Slots [lo, hi) of one sequence.  Rows below hm come from memory through
  // the buffer resource rs (rows_rsrc(rows, hm)), via the PD register tiles
  // `pre` (PD * CPT vectors) that prefetch<PD> filled; the next PD-th tile's
  // loads are issued as soon as a tile has been stored to LDS.  With kPatch
  // the row hm (== hi - 1) is taken from `patch` (LDS).
  template <bool kPatch, int PD>
  __device__ __forceinline__ static void run(State& st, Smem& sm, __amdgpu_buffer_rsrc_t rs, int lo, int hi,
                                             int hm, const uint16_t* patch, uint4* pre) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    // The registers are only ever stored (never selected against another
    // source), so they stay registers: the patch row is skipped here and
    // copied into its place by CPR threads, at disjoint addresses.
    auto store_tile = [&](int j0, const uint4* p) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int id = tid + NT * k;
        if (CHUNKS % NT == 0 || id < CHUNKS) {
          const int row = id / CPR, ch = id % CPR;
          if (!kPatch || j0 + row != hm) *reinterpret_cast<uint4*>(sm.k + row * PITCH + ch * 8) = p[k];
        }
      }
      if constexpr (kPatch) {
        if (tid < CPR && hm >= j0 && hm < j0 + TS)
          *reinterpret_cast<uint4*>(sm.k + (hm - j0) * PITCH + tid * 8) =
              *reinterpret_cast<const uint4*>(patch + tid * 8);
      }
    };

    auto tile = [&](int j0, uint4* p) {
      store_tile(j0, p);
      __syncthreads();
      if (j0 + PD * TS < hm) load_tile(p, rs, j0 + PD * TS);

      f32x4 sc[HT];
      if (wave < QKW) {
        // scores: wave owns slots 16*wave .. 16*wave+15 of the tile
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 bk =
              *reinterpret_cast<const bf16x8*>(sm.k + (16 * wave + c16) * PITCH + ks * 32 + 8 * g);
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            const int qo = (ht * 16 + c16) * PITCH + ks * 32 + 8 * g;
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sm.q + qo);
            const bf16x8 aql = *reinterpret_cast<const bf16x8*>(sm.ql + qo);
            sc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, sc[ht], 0, 0, 0);
            sc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aql, bk, sc[ht], 0, 0, 0);
          }
        }
        // sc[ht][i] = score of head ht*16 + 4g + i against slot j0 + 16*wave + c16
        const bool valid = j0 + 16 * wave + c16 < hi;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = valid ? sc[ht][i] : -INFINITY;
            sc[ht][i] = v;
            v = row16_max(v);
            if (c16 == 0) sm.red[wave][ht * 16 + 4 * g + i] = v;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int head = ht * 16 + 4 * g + i;
          float mt = sm.red[0][head];
#pragma unroll
          for (int w = 1; w < QKW; ++w) mt = fmaxf(mt, sm.red[w][head]);
          const float mn = fmaxf(st.m[ht][i], mt);
          const float alpha = fast_exp2(st.m[ht][i] - mn);
          st.m[ht][i] = mn;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st.acc[ht][ct][i] *= alpha;
          if (wave < QKW) {
            const float pv = fast_exp2(sc[ht][i] - mn);
            st.l[ht][i] = st.l[ht][i] * alpha + pv;
            sm.p[head * PP + 16 * wave + c16] = f32_to_bf16_bits(pv);
          }
        }
      }
      __syncthreads();

      // acc[head, col] += sum_slot P[head, slot] * row[slot, col]
#pragma unroll
      for (int ks2 = 0; ks2 < TS / 32; ++ks2) {
        bf16x8 ap[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          ap[ht] = *reinterpret_cast<const bf16x8*>(sm.p + (ht * 16 + c16) * PP + ks2 * 32 + 8 * g);
        // Lane (g, c16) needs rows ks2*32 + 8g + 0..7 of column col0 + c16.  A
        // transposing read covers 4 rows: lane k of a 16-lane group points at
        // row base + k/4, columns col0 + 4*(k%4) .. +3; lane i then receives as
        // element r the (i%4)-th value of lane 4r + i/4, i.e. row base + r of
        // column col0 + i.
        const uint16_t* rbase = sm.k + (ks2 * 32 + 8 * g + (c16 >> 2)) * PITCH + 4 * (c16 & 3);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int col0 = wave * CPW + ct * 16;
          const s16x4 lo4 = lds_read_tr16(rbase + col0);
          const s16x4 hi4 = lds_read_tr16(rbase + 4 * PITCH + col0);
          const s16x8 v8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 bb = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            st.acc[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[ht], bb, st.acc[ht][ct], 0, 0, 0);
        }
      }
      __syncthreads();
    };

    for (int j0 = lo; j0 < hi; j0 += PD * TS) {
      tile(j0, pre);
      if constexpr (PD == 2) {
        if (j0 + TS < hi) tile(j0 + TS, pre + CPT);
      }
    }
  }

  // Softmax denominators: sum over the 16 slot lanes and the scoring waves,
  // in a fixed order.  Leaves L of head h in sm.red[0][h].
  __device__ __forceinline__ static void finish(State& st, Smem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    if (wave < QKW) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = st.l[ht][i];
          v = row16_sum(v);
          if (c16 == 0) sm.red[wave][ht * 16 + 4 * g + i] = v;
        }
      }
    }
    __syncthreads();
    if (tid < HP) {
      float L = 0.f;
      for (int w = 0; w < QKW; ++w) L += sm.red[w][tid];
      sm.red[0][tid] = L;  // row 0 was read above by this thread only
    }
    __syncthreads();
  }
};

// ---------------------------------------------------------------------------
// Split-K latent attention for long caches: one workgroup of 4 waves per
// (split, sequence), 64-slot tiles.  With a single split the workgroup
// normalises and writes o_lat itself; otherwise it stores its (m, l, acc)
// partial and split_merge_kernel, launched next on the stream, merges the
// splits in split order.  (Merging inside this kernel, by the last workgroup
// to finish, would need device-scope release/acquire fences per workgroup,
// which on this multi-XCD part write back and invalidate L2.)
// ---------------------------------------------------------------------------
template <int HT, int DC, int DR>
__global__ __launch_bounds__(256) void decode_mfma_kernel(AttendArgs a) {
  using A = MfmaAttn<HT, DC, DR, 4, 64>;
  constexpr int W = A::W, HP = A::HP, PITCH = A::PITCH, CPW = A::CPW, CT = A::CT;
  __shared__ typename A::Smem sm;
  const int split = blockIdx.x, b = blockIdx.y;
  const int nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int H = a.H;

  int n = 0;
  {
    const int pos = a.pos[b];
    if (pos >= 1) {
      n = slot_of(pos, a.s);
      if (n > a.max_slots) n = 0;
    }
  }
  const int lo = static_cast<int>((static_cast<long long>(split) * n) / nsplit);
  const int hi = static_cast<int>((static_cast<long long>(split + 1) * n) / nsplit);

  const float qscale = a.scale * kLog2e;
  for (int idx = tid; idx < HP * W; idx += 256) {
    const int hh = idx / W, e = idx % W;
    const float v = hh < H ? a.qbuf[(static_cast<size_t>(b) * H + hh) * W + e] * qscale : 0.f;
    split_bf16(v, sm.q[hh * PITCH + e], sm.ql[hh * PITCH + e]);
  }
  typename A::State st;
  A::init(st);
  const uint16_t* rows =
      static_cast<const uint16_t*>(a.cache) + static_cast<size_t>(b) * a.max_slots * W;
  const auto rs = A::rows_rsrc(rows, hi);
  uint4 pre[A::CPT];
  A::template prefetch<1>(pre, rs, lo);
  A::template run<false, 1>(st, sm, rs, lo, hi, hi, nullptr, pre);
  A::finish(st, sm);

  if (nsplit == 1) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        if (head < H) {
          const float inv = 1.f / sm.red[0][head];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            a.o_lat[(static_cast<size_t>(b) * H + head) * DC + wave * CPW + ct * 16 + c16] =
                st.acc[ht][ct][i] * inv;
        }
      }
    }
    return;
  }
  const size_t pbase = (static_cast<size_t>(b) * nsplit + split) * H;
  if (wave == 0 && c16 == 0) {
    // the running max is in log2 units; partials use natural-log units
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        if (head < H) {
          a.part.m[pbase + head] = st.m[ht][i] * kLn2;
          a.part.l[pbase + head] = sm.red[0][head];
        }
      }
    }
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = ht * 16 + 4 * g + i;
      if (head < H) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          a.part.acc[(pbase + head) * DC + wave * CPW + ct * 16 + c16] = st.acc[ht][ct][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K latent attention for long caches of the 576-wide row (d_c = 512,
// d_R = 64).  One workgroup of 8 waves per (split, sequence), all heads
// (HT*16 MFMA rows), 64-slot tiles; split k of S takes tiles k, k+S, ...
//
// The cache streams HBM -> LDS through non-temporal buffer loads that write
// LDS directly (no staging registers), double buffered: the loads of the
// split's tile after next go out as soon as every wave is done with the
// current one, so one tile (74 KB) is always in flight.  The loads are waited for by count (the compiler does not track
// them, see buffer_load_lds16); barriers inside the tile loop wait only for
// LDS operations.
//
// LDS tile layout: 16-byte chunk c of row r sits at chunk slot
// r * 72 + (c ^ ((r >> 1) & 7)).  The XOR (within 8-chunk groups, so a row
// stays within its 72 slots) spreads the 16 rows an MFMA operand read touches
// over all LDS banks; load instruction i of wave w fills slots
// (9w + i) * 64 + lane, so each lane fetches the chunk that belongs there.
//
// Per tile: eight score items (head tile, 16-slot group), one per wave, with
// the wave's scaled query rows held in registers; the tile max per head is
// shared through LDS, probabilities go to LDS as bf16, then each wave
// accumulates its 64 latent columns for all heads.  Scores are in log2 units
// (queries pre-scaled by tau * log2 e).
// ---------------------------------------------------------------------------
template <int HT>
__global__ __launch_bounds__(512) void decode_stream_kernel(AttendArgs a) {
  constexpr int DC = 512, DR = 64, W = DC + DR, NW = 8;
  constexpr int TS = 64;
  constexpr int CPR = W / 8;                // chunks per row
  constexpr int TCH = TS * CPR;             // chunks per tile
  constexpr int LPW = TCH / (64 * NW);      // load instructions per wave per tile
  static_assert(LPW * 64 * NW == TCH && CPR % 8 == 0 && LPW == 9, "tile shape");
  constexpr int HP = HT * 16, PP = TS + 8;
  constexpr int KS = W / 32;                // score k-steps
  constexpr int NSG = TS / 16;              // 16-slot groups per tile
  constexpr int ITEMS = HT * NSG;           // score items per tile
  static_assert(ITEMS <= NW, "one score item per wave");
  constexpr int CPW = DC / NW, CT = CPW / 16;
  __shared__ __align__(16) uint16_t sp[HP * PP];
  __shared__ float red[NSG][HP];
  // the two tile buffers are separate objects, each named statically (the
  // tile loop is unrolled by two)
  __shared__ __align__(16) uint16_t kb0[TCH * 8];
  __shared__ __align__(16) uint16_t kb1[TCH * 8];

  const int split = blockIdx.x, b = blockIdx.y;
  const int nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int H = a.H;

  int n = 0;
  {
    const int pos = a.pos[b];
    if (pos >= 1) {
      n = slot_of(pos, a.s);
      if (n > a.max_slots) n = 0;
    }
  }
  // split k takes the sequence's 64-slot tiles k, k + nsplit, k + 2 nsplit,
  // ... (interleaved: the workgroups of a sequence read neighbouring rows at
  // about the same time)
  const int lo = split * TS, hi = n, step = nsplit * TS;

  // rows of this sequence up to hi; past them the loads read zero
  const uint16_t* rows = static_cast<const uint16_t*>(a.cache) + static_cast<size_t>(b) * a.max_slots * W;
  const i32x4_t rs = make_rsrc_words(rows, hi * W * 2);
  auto swz = [](int r) { return (r >> 1) & 7; };
  int voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int slot = (wave * LPW + i) * 64 + lane;
    const int r = slot / CPR, c = (slot % CPR) ^ swz(r);
    voff[i] = (r * W + c * 8) * 2;
  }
  auto issue_tile = [&](int j0, uint16_t* dst) {
    const uint32_t base = lds_addr(dst + wave * LPW * 64 * 8);
    const int so = __builtin_amdgcn_readfirstlane(j0 * (W * 2));
#pragma unroll
    for (int i = 0; i < LPW; ++i) buffer_load_lds16(rs, base + i * 64 * 16, voff[i], so);
  };

  if (lo < hi) issue_tile(lo, kb0);
  if (lo + step < hi) issue_tile(lo + step, kb1);

  // this wave's score item and its query rows (A operand, bf16, scaled)
  const int item_ht = wave % HT, item_sg = wave / HT;
  const bool scorer = wave < ITEMS;
  const float qscale = a.scale * kLog2e;
  bf16x8 qa[KS];
  {
    const int head = item_ht * 16 + c16;
    const float* qrow = a.qbuf + (static_cast<size_t>(b) * H + (head < H ? head : 0)) * W;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float v[8];
      load8(qrow + ks * 32 + 8 * g, v);
      u16x8 u;
#pragma unroll
      for (int r = 0; r < 8; ++r) u[r] = head < H ? f32_to_bf16_bits(v[r] * qscale) : uint16_t(0);
      qa[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  float m[HT][4], l[4];
  f32x4 acc[HT][CT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m[ht][i] = -INFINITY;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ht][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = 0.f;

  // one tile: `kt` holds slots j0 .. j0+TS-1; afterwards it receives the
  // split's tile after next, j0 + 2 step .. (loads issued once every wave is
  // done with it)
  auto tile = [&](int j0, uint16_t* kt) {
    // at most one later tile (j0+step) of this wave's loads may still be in flight
    if (j0 + step < hi)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // this tile visible to every wave

    // scores of item (item_ht, item_sg): sc[i] = head item_ht*16 + 4g + i
    // against slot j0 + 16*item_sg + c16
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (scorer) {
      const int r = 16 * item_sg + c16;
      const uint16_t* krow = kt + r * CPR * 8;
      const int sr = swz(r);
      f32x4 s2 = f32x4{0.f, 0.f, 0.f, 0.f};  // two accumulation chains
#pragma unroll
      for (int ks = 0; ks < KS; ks += 2) {
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(krow + ((4 * ks + g) ^ sr) * 8);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(krow + ((4 * (ks + 1) + g) ^ sr) * 8);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b0, sc, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks + 1], b1, s2, 0, 0, 0);
      }
      const bool valid = j0 + 16 * item_sg + c16 < hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = valid ? sc[i] + s2[i] : -INFINITY;
        sc[i] = v;
        const float mx = row16_max(v);
        if (c16 == 0) red[item_sg][item_ht * 16 + 4 * g + i] = mx;
      }
    }
    lds_barrier();
    // new running max per head (the same values in every wave), rescale
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        float mt = red[0][head];
#pragma unroll
        for (int sg = 1; sg < NSG; ++sg) mt = fmaxf(mt, red[sg][head]);
        const float mn = fmaxf(m[ht][i], mt);
        const float alpha = fast_exp2(m[ht][i] - mn);
        m[ht][i] = mn;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ht][ct][i] *= alpha;
        if (scorer && ht == item_ht) {
          const float pv = fast_exp2(sc[i] - mn);
          l[i] = l[i] * alpha + pv;
          sp[head * PP + 16 * item_sg + c16] = f32_to_bf16_bits(pv);
        }
      }
    }
    lds_barrier();
    // acc[head, col] += sum_slot P[head, slot] row[slot, col]; the B operand
    // (8 slots of one column) comes from two transposing reads
#pragma unroll
    for (int ks2 = 0; ks2 < TS / 32; ++ks2) {
      bf16x8 ap[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        ap[ht] = *reinterpret_cast<const bf16x8*>(sp + (ht * 16 + c16) * PP + ks2 * 32 + 8 * g);
      const int r0 = ks2 * 32 + 8 * g + (c16 >> 2), r1 = r0 + 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = wave * CPW + ct * 16 + 4 * (c16 & 3);
        const int ch = col >> 3, wi = col & 7;
        const s16x4 lo4 = lds_read_tr16(kt + (r0 * CPR + (ch ^ swz(r0))) * 8 + wi);
        const s16x4 hi4 = lds_read_tr16(kt + (r1 * CPR + (ch ^ swz(r1))) * 8 + wi);
        const bf16x8 bb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[ht], bb, acc[ht][ct], 0, 0, 0);
      }
    }
    lds_barrier();  // every wave is done with kt (and with sp, red)
    if (j0 + 2 * step < hi) issue_tile(j0 + 2 * step, kt);
  };
  for (int j0 = lo; j0 < hi; j0 += 2 * step) {
    tile(j0, kb0);
    if (j0 + step < hi) tile(j0 + step, kb1);
  }

  // softmax denominators: sum over the slot lanes, then over the slot groups
  // in order
  if (scorer) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = row16_sum(l[i]);
      if (c16 == 0) red[item_sg][item_ht * 16 + 4 * g + i] = v;
    }
  }
  __syncthreads();
  float L[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = ht * 16 + 4 * g + i;
      float v = 0.f;
#pragma unroll
      for (int sg = 0; sg < NSG; ++sg) v += red[sg][head];
      L[ht][i] = v;
    }
  }

  if (nsplit == 1) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        if (head < H) {
          const float inv = 1.f / L[ht][i];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            a.o_lat[(static_cast<size_t>(b) * H + head) * DC + wave * CPW + ct * 16 + c16] = acc[ht][ct][i] * inv;
        }
      }
    }
    return;
  }
  const size_t pbase = (static_cast<size_t>(b) * nsplit + split) * H;
  if (wave == 0 && c16 == 0) {
    // the running max is in log2 units; partials use natural-log units
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        if (head < H) {
          a.part.m[pbase + head] = m[ht][i] * kLn2;
          a.part.l[pbase + head] = L[ht][i];
        }
      }
    }
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = ht * 16 + 4 * g + i;
      if (head < H) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          a.part.acc[(pbase + head) * DC + wave * CPW + ct * 16 + c16] = acc[ht][ct][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused decode step for short caches.  One workgroup of 16 waves per
// (sequence, group of HG heads) does everything for one token:
//   merge            : gate w_t and slot ceil(t/s) <- reset ? w x : acc + w x,
//                      computed by every group of the sequence; group 0 writes
//                      the cache row and the fp32 state, the others only use
//                      the row (kept in LDS) as the tile's last key;
//   absorb           : q~[h] = W_UK[h]^T q_c[h] for the group's heads, scaled,
//                      bf16, into LDS;
//   attention        : the MFMA core over slots 1..ceil(t/s), two tiles of
//                      cache rows in flight in registers;
//   up-projection    : out[h] = W_UV[h] o_lat[h], o_lat kept in LDS.
// Splitting the heads spreads the per-step weight traffic (W_UK and W_UV, the
// largest reads at short caches) over more compute units; every group reads
// the sequence's cache rows, and all groups of a sequence run on one XCD so
// those rows are fetched into one L2.  The open slot's fp32 state is double
// buffered by token parity: step t reads [b, (t-1) % 2] and writes
// [b, t % 2], so no group reads what another is writing.
// ---------------------------------------------------------------------------
// W_UK / W_UV load shapes of the step kernel (nth threads) for a group of hg
// heads of width d_h: absorb row groups eg_n and W_UK rows per thread nl;
// up-projection threads per output tpo and W_UV chunks per thread nv.
struct StepShape {
  int eg_n, nl, tpo, nv;
};
__host__ __device__ constexpr StepShape step_shape(int nth, int hg, int d_h, int d_c) {
  const int KC = d_c / 8;
  const int eg_n = nth / (KC * hg);
  const int nout = hg * d_h;
  int tpo = 1;
  while (tpo < 64 && 2 * tpo * nout <= nth) tpo *= 2;
  return StepShape{eg_n, eg_n > 0 ? (d_h + eg_n - 1) / eg_n : 1 << 30, tpo,
                   nout <= nth ? (KC + tpo - 1) / tpo : 1 << 30};
}

// Instances: (d_c, d_R, tile slots, heads per group, largest d_h, threads,
// cache tiles in flight, merge the token first).
template <int DC, int DR, int TS, int HG, int DH, int NTH, int PD, bool MERGE>
__global__ __launch_bounds__(NTH) void decode_step_kernel(const int32_t* __restrict__ kpos, int G, int nB, int,
                                                          int, const uint16_t*, const uint16_t*, const uint16_t*,
                                                          StepArgs a) {
  using A = MfmaAttn<1, DC, DR, NTH / 64, TS>;
  constexpr int W = A::W, HP = A::HP, PITCH = A::PITCH, CPW = A::CPW, CT = A::CT, NT = A::NT;
  constexpr int KC = DC / 8;
  constexpr int GE = DC / 64;
  constexpr StepShape SMAX = step_shape(NTH, HG, DH, DC);
  constexpr int MAXK = SMAX.nl, MAXV = SMAX.nv;  // in-flight W_UK / W_UV vectors per thread
  static_assert(NT == NTH, "thread count");
  static_assert(MAXK <= 16 && MAXV <= 16, "load shape");
  __shared__ typename A::Smem sm;
  __shared__ __align__(16) uint16_t s_new[W];
  // Workgroups are dealt to the 8 XCDs round-robin by linear id: id L runs on
  // XCD L % 8.  Sequence b goes to XCD b % 8 with all of its head groups.
  const int L = blockIdx.x, xcd = L & 7, k8 = L >> 3;
  const int grp = k8 % G, b = 8 * (k8 / G) + xcd;
  if (b >= nB) return;
  const int H = a.H, d_h = a.d_h, h0 = grp * HG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const StepShape sh = step_shape(NTH, HG, d_h, DC);

  const int pos = kpos[b];
  // Every load below is issued unconditionally (indices clamped into the
  // tensors, unused values dropped at their use), so the compiler can count
  // the loads in flight and wait only for the ones each phase needs.
  // Loads that do not depend on the position go out first: W_UK rows and the
  // matching query elements (absorb), and the merge's token values and W_hyp.
  const int kc = tid % KC, hl = (tid / KC) % HG, eg = tid / (KC * HG);
  const int nl = eg < sh.eg_n ? (d_h - eg + sh.eg_n - 1) / sh.eg_n : 0;
  uint4 wk[MAXK];
  uint16_t qb[MAXK];
#pragma unroll
  for (int i = 0; i < MAXK; ++i) {
    const int e = min(eg + i * sh.eg_n, d_h - 1);
    wk[i] = *reinterpret_cast<const uint4*>(a.w_uk + (static_cast<size_t>(h0 + hl) * d_h + e) * DC + kc * 8);
    qb[i] = a.q_c[(static_cast<size_t>(b) * H + h0 + hl) * d_h + e];
  }
  // W_UV rows of the up-projection, in flight until the end: tpo threads per
  // output (hl, e), chunks c = p, p + tpo, ...
  const int nout = HG * d_h;
  const int o = tid / sh.tpo, p = tid % sh.tpo;
  const int nv = o < nout ? (KC - p + sh.tpo - 1) / sh.tpo : 0;
  const uint16_t* wrow = a.w_uv + (static_cast<size_t>(h0) * d_h + (o < nout ? o : 0)) * DC;
  uint4 wv[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) wv[i] = *reinterpret_cast<const uint4*>(wrow + min(p + i * sh.tpo, KC - 1) * 8);
  const int te = min(tid, W - 1);  // merge column of this thread (tid < W)
  uint16_t gxb[GE], mxb = 0;
  float gw[GE];
  if constexpr (MERGE) {
#pragma unroll
    for (int j = 0; j < GE; ++j) {
      gxb[j] = a.c[static_cast<size_t>(b) * DC + lane + 64 * j];
      gw[j] = a.w_hyp[lane + 64 * j];
    }
    mxb = te < DC ? a.c[static_cast<size_t>(b) * DC + te] : a.k_r[static_cast<size_t>(b) * DR + te - DC];
  }

  const int n = pos >= 1 ? slot_of(pos, a.s) : 0;
  const bool ok = pos >= 1 && n <= a.max_slots && (!MERGE || pos <= a.pe_rows);
  uint16_t* out = a.out + (static_cast<size_t>(b) * H + h0) * d_h;
  if (!ok) {
    for (int idx = tid; idx < HG * d_h; idx += NT) out[idx] = 0x7fc0u;  // NaN
    return;
  }
  // Position-dependent loads: pe row, the open slot's state, then the first
  // PD tiles of cache rows.  Memory rows are the completed slots 0..n-2 when
  // merging (row n-1 is the new one, taken from LDS; group 0 writes it to
  // memory meanwhile), else 0..n-1.
  float gp[GE], macc = 0.f;
  const bool cont = (pos - 1) % a.s != 0;  // the token continues an open block
  if constexpr (MERGE) {
#pragma unroll
    for (int j = 0; j < GE; ++j) gp[j] = a.pe[static_cast<size_t>(pos - 1) * DC + lane + 64 * j];
    macc = a.open_acc[(static_cast<size_t>(b) * 2 + (pos - 1) % 2) * W + te];
  }
  const uint16_t* rows = a.cache + static_cast<size_t>(b) * a.max_slots * W;
  const int hm = MERGE ? n - 1 : n;
  // rope query element of this group's heads (thread tid < HP * DR takes
  // element tid % DR of local head tid / DR)
  static_assert(HP * DR <= NT, "one rope query element per thread");
  const int tq = min(tid, HP * DR - 1);
  const uint16_t qrb = a.q_r[(static_cast<size_t>(b) * H + h0 + min(tq / DR, HG - 1)) * DR + tq % DR];
  const auto rs = A::rows_rsrc(rows, hm);
  uint4 pre[PD * A::CPT];
  A::template prefetch<PD>(pre, rs, 0);

  // absorb: partial sums of q~[hl, kc*8 .. +8] over this thread's rows
  float* red = reinterpret_cast<float*>(sm.k);  // [HG][eg_n][DC], scratch in the tile buffer
  if (nl > 0) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
    for (int i = 0; i < MAXK; ++i) {
      if (i < nl) {
        const float q = bf16_bits_to_f32(qb[i]);
        const uint32_t w4[4] = {wk[i].x, wk[i].y, wk[i].z, wk[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = fmaf(q, __uint_as_float(w4[j] << 16), acc[2 * j]);
          acc[2 * j + 1] = fmaf(q, __uint_as_float(w4[j] & 0xffff0000u), acc[2 * j + 1]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[(hl * sh.eg_n + eg) * DC + kc * 8 + j] = acc[j];
  }
  // every wave computes the gate (same values, same order: the same bits)
  float gate = 0.f;
  if constexpr (MERGE) {
    float gx[GE];
#pragma unroll
    for (int j = 0; j < GE; ++j) gx[j] = bf16_bits_to_f32(gxb[j]);
    gate = gate_from_lane_values<GE>(gx, gp, gw);
  }
  __syncthreads();
  if constexpr (MERGE) {
    if (tid < W) {
      const float v = fmaf(gate, bf16_bits_to_f32(mxb), cont ? macc : 0.f);
      const uint16_t u = f32_to_bf16_bits(v);
      if (grp == 0) {
        a.open_acc[(static_cast<size_t>(b) * 2 + pos % 2) * W + tid] = v;
        a.cache[(static_cast<size_t>(b) * a.max_slots + n - 1) * W + tid] = u;
      }
      s_new[tid] = u;
    }
  } else if (tid < W) {
    s_new[tid] = 0;  // row n of the last tile (past the slots) reads as zero
  }
  const float qscale = a.scale * kLog2e;
  for (int idx = tid; idx < HP * DC; idx += NT) {
    const int h = idx / DC, k = idx % DC;
    float v = 0.f;
    if (h < HG)
      for (int r = 0; r < sh.eg_n; ++r) v += red[(h * sh.eg_n + r) * DC + k];
    split_bf16(v * qscale, sm.q[h * PITCH + k], sm.ql[h * PITCH + k]);
  }
  if (tid < HP * DR) {
    const int h = tid / DR, e = tid % DR;
    split_bf16(h < HG ? bf16_bits_to_f32(qrb) * qscale : 0.f, sm.q[h * PITCH + DC + e],
               sm.ql[h * PITCH + DC + e]);
  }
  __syncthreads();

  typename A::State st;
  A::init(st);
  A::template run<true, PD>(st, sm, rs, 0, n, hm, s_new, pre);
  A::finish(st, sm);

  // o_lat (fp32, normalised) into the tile buffer, then the up-projection
  float* olat = reinterpret_cast<float*>(sm.k);  // [HP][DC]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 4 * g + i;
    const float inv = 1.f / sm.red[0][head];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) olat[head * DC + wave * CPW + ct * 16 + c16] = st.acc[0][ct][i] * inv;
  }
  __syncthreads();
  float acc = 0.f;
  if (nv > 0) {
    const float* orow = olat + (o / d_h) * DC;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      if (i < nv) {
        const int c = p + i * sh.tpo;
        const uint32_t w4[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(__uint_as_float(w4[j] << 16), orow[c * 8 + 2 * j], acc);
          acc = fmaf(__uint_as_float(w4[j] & 0xffff0000u), orow[c * 8 + 2 * j + 1], acc);
        }
      }
    }
  }
  for (int off = sh.tpo / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (p == 0 && o < nout) out[o] = f32_to_bf16_bits(acc);
}

// ---------------------------------------------------------------------------
// Fused decode step for 256-wide latents (rows of d_c + d_R = 288): one
// workgroup of 8 waves per (sequence, group of HG heads).
//   absorb        : q~[h] = W_UK[h]^T q_c[h]; each thread takes 8 latent
//                   columns and pairs of W_UK rows, v_dot2 on bf16 pairs;
//   merge         : as in the kernel above (group 0 writes the cache row and
//                   the fp32 state, every group keeps the row in LDS);
//   attention     : wave-private flash decoding.  Wave w takes slot chunks
//                   w, w + 8, ... of 16 slots and keeps its own running max,
//                   sum and o_lat accumulator, with no barrier:
//                     S^T[slot, head] = rows . q~^T  (16x16x32 MFMA; the
//                       chunk's rows are loaded as whole lines into a
//                       wave-private LDS buffer and read back in the A
//                       layout, q~ from LDS),
//                     O^T[col, head] += V^T P^T      (16x16x16 MFMA; P^T
//                       stays in the score registers, V^T is read transposed
//                       from the same buffer);
//                   q~ and P enter both products as a bf16 high and low
//                   part (16 significant bits): head h takes MFMA column h
//                   for the high parts and column HG + h for the low parts;
//                   a quad-permute add folds the two score columns, and the
//                   two O^T columns are added when the waves are combined;
//                   the 8 waves' partial results are merged once, in wave
//                   order;
//   up-projection : out[h] = W_UV[h] o_lat[h] on MFMA, one 16-row tile of
//                   W_UV per wave (row-major, or in tile order when the
//                   caller packed it); o_lat goes in as bf16 hi + lo parts
//                   (o_lat = hi + lo to 16 bits), two products per k-step.
// Heads occupy the MFMA's 16-wide N dimension (2 HG columns with the low
// parts); the columns past 2 HG read q~ from a zero row.
// ---------------------------------------------------------------------------
// The leading scalar arguments (positions, head groups, batch, heads, d_h and
// the W_UK, query and token pointers) come ahead of the argument struct so
// that the build can preload them into scalar registers: the position load,
// which everything waits for, and the first loads of W_UK, the queries and the
// token then issue at once instead of after a round trip to the
// kernel-argument segment.
// Timeline instance only: lane 0 of the calling wave writes the real-time
// counter (100 MHz), read once `dep` is available, to reading k of workgroup
// wg.
__device__ __forceinline__ void timeline_stamp(unsigned long long* tl, int wg, int k, float dep) {
  asm volatile("" ::"v"(dep) : "memory");
  const unsigned long long t = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) tl[static_cast<size_t>(wg) * kStepTimelineSlots + k] = t;
}

// TL: the timeline instance (the same work, plus the counter readings listed
// with kStepTimelineSlots).
template <int DC, int DR, int HG, int DH, bool MERGE, bool PP = false, bool TL = false>
__global__ __launch_bounds__(512) void decode_step_wave_kernel(const int32_t* __restrict__ kpos, int G, int nB, int H,
                                                              int d_h, const uint16_t* __restrict__ w_uk,
                                                              const uint16_t* __restrict__ q_c,
                                                              const uint16_t* __restrict__ c_tok, StepArgs a) {
  constexpr int NT = 512, NWV = 8;
  constexpr int W = DC + DR;
  constexpr int KSW = W / 32;                            // score k-steps
  constexpr int KSU = DC / 32;                           // up-projection k-steps
  constexpr int CTW = DC / 16;                           // PV column tiles
  constexpr int KC = DC / 8;                             // 8-column chunks of a latent row
  constexpr int GE = DC / 64;
  constexpr int EGN = NT / (KC * HG);                    // absorb row groups
  constexpr int NP = (DH + 2 * EGN - 1) / (2 * EGN);     // W_UK row pairs per thread
  constexpr int MT = (DH + 15) / 16;                     // up-projection tiles per head
  constexpr int RP = W + 8;                              // row buffer pitch (elements)
  constexpr int QP = W + 8;                              // q~ pitch (elements)
  static_assert(W % 32 == 0 && NT % (KC * HG) == 0 && EGN >= 1, "shape");
  static_assert(HG * DC <= NT && HG * DR <= NT && HG <= 16, "one q~ element per thread");
  static_assert(HG * MT <= NWV, "one up-projection tile per wave");
  // the low-part column of head h is h + HG, its partner within a quad of
  // lanes: quad_perm (1,0,3,2) for one head, (2,3,0,1) for two
  static_assert(HG == 1 || HG == 2, "high/low column pairs within a lane quad");
  constexpr int kPartner = HG == 1 ? 0xB1 : 0x4E;

  struct Absorb {
    float red[HG][EGN][DC];
  };
  struct Rows {
    uint16_t r[NWV][16][RP];
  };
  struct Combine {
    float o[NWV][2 * HG][DC];  // per wave, O^T's high-part and low-part columns
    float m[NWV][HG];
    float l[NWV][HG];
    uint16_t ob[2][HG][DC];  // o_lat: bf16 hi, bf16 lo
    uint16_t zero[DC];
  };
  // The absorb's partial sums are dead once q~ is formed, so the combine
  // buffer overlaps them; it does not overlap the row buffers, so a wave can
  // store its partial result as soon as its own attention is done.
  union Phases {
    Absorb ab;
    Combine cb;
  };
  __shared__ __align__(16) Phases u;
  __shared__ __align__(16) Rows rw;
  // q~ rows, scaled, bf16: high parts in rows 0..HG-1, low parts in rows
  // HG..2HG-1, row 2HG is zero
  __shared__ __align__(16) uint16_t sq[2 * HG + 1][QP];
  __shared__ __align__(16) uint16_t s_new[W];

  // Workgroups are dealt to the 8 XCDs round-robin by linear id: id L runs on
  // XCD L % 8.  Sequence b goes to XCD b % 8 with all of its head groups.
  // (shifts when the group count is a power of two: the division would sit
  // ahead of the first loads)
  const int L = blockIdx.x, xcd = L & 7, k8 = L >> 3;
  int grp, kq;
  if ((G & (G - 1)) == 0) {
    grp = k8 & (G - 1);
    kq = k8 >> __builtin_ctz(G);
  } else {
    grp = k8 % G;
    kq = k8 / G;
  }
  const int b = 8 * kq + xcd;
  if (b >= nB) return;
  const int h0 = grp * HG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  if constexpr (TL) {
    if (wave == 0) timeline_stamp(a.timeline, L, 0, 0.f);
  }

  const int pos = kpos[b];
  // (the position load goes out before anything else: the scheduler would
  // otherwise place it after the loads below)
  __builtin_amdgcn_sched_barrier(0);
  // Loads that do not depend on the position go out first, unconditionally
  // (indices clamped into the tensors, unused values dropped at their use).
  // absorb: thread (kc, hl, eg) takes columns kc*8 .. +7 of head hl and the
  // row pairs e = 2 (eg + j EGN) + {0, 1}
  const int kc = tid % KC, hl = (tid / KC) % HG, eg = tid / (KC * HG);
  const auto r_uk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w_uk + static_cast<size_t>(h0) * d_h * DC), static_cast<short>(0), HG * d_h * DC * 2,
      kBufferRsrcWord3);
  const auto r_q = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(q_c + (static_cast<size_t>(b) * H + h0) * d_h), static_cast<short>(0), HG * d_h * 2,
      kBufferRsrcWord3);
  uint4 wk0[NP], wk1[NP];
  uint32_t qp[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e0 = 2 * (eg + j * EGN);
    const int r0 = min(e0, d_h - 1), r1 = min(e0 + 1, d_h - 1);
    auto v0 = __builtin_amdgcn_raw_buffer_load_b128(r_uk, ((hl * d_h + r0) * DC + kc * 8) * 2, 0, 0);
    auto v1 = __builtin_amdgcn_raw_buffer_load_b128(r_uk, ((hl * d_h + r1) * DC + kc * 8) * 2, 0, 0);
    wk0[j] = uint4{v0[0], v0[1], v0[2], v0[3]};
    wk1[j] = uint4{v1[0], v1[1], v1[2], v1[3]};
    // rows past d_h read as zero (the resource ends at the group's last row)
    const uint32_t q0 = __builtin_amdgcn_raw_buffer_load_b16(r_q, (hl * d_h + e0) * 2, 0, 0);
    const uint32_t q1 = __builtin_amdgcn_raw_buffer_load_b16(r_q, (hl * d_h + e0 + 1) * 2, 0, 0);
    qp[j] = (e0 < d_h ? q0 : 0u) | ((e0 + 1 < d_h ? q1 : 0u) << 16);
  }
  // up-projection: wave w takes rows mt*16 .. +15 of head hu (waves past
  // HG * ceil(d_h / 16) load a clamped tile and store nothing); lane (g, c16)
  // holds row mt*16 + c16, columns 32 ks + 8g .. +7: the MFMA A layout
  const int mt_n = (d_h + 15) / 16;
  const int hu = min(wave / mt_n, HG - 1), mt = wave % mt_n;
  const bool up_wave = wave < HG * mt_n;
  // W_UV row-major: load ks reads 16 rows x 64 bytes (rows past d_h clamped,
  // their products not stored); in tile order: the same values as one
  // contiguous kilobyte per load (rows past d_h zero)
  const bool tiles = a.w_uv_tiles != nullptr;
  const auto r_uv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(tiles ? a.w_uv_tiles + static_cast<size_t>(h0) * mt_n * 16 * DC
                                  : a.w_uv + static_cast<size_t>(h0) * d_h * DC),
      static_cast<short>(0), (tiles ? mt_n * 16 : d_h) * HG * DC * 2, kBufferRsrcWord3);
  const int vu = tiles ? (hu * mt_n + mt) * KSU * 1024 + 16 * lane : ((hu * d_h + min(mt * 16 + c16, d_h - 1)) * DC + 8 * g) * 2;
  const int vstep = tiles ? 1024 : 64;
  uint4 wv[KSU];  // loaded after the cache rows (see below)
  const int te = min(tid, W - 1);  // merge column of this thread (tid < W)
  uint16_t gxb[GE], mxb = 0;
  float gw[GE];
  if constexpr (MERGE) {
#pragma unroll
    for (int j = 0; j < GE; ++j) {
      gxb[j] = c_tok[static_cast<size_t>(b) * DC + lane + 64 * j];
      if constexpr (!PP) gw[j] = a.w_hyp[lane + 64 * j];  // (PP: the row is known with the position)
    }
    mxb = te < DC ? c_tok[static_cast<size_t>(b) * DC + te] : a.k_r[static_cast<size_t>(b) * DR + te - DC];
  }

  // slot and place in the block of the position (shifts when s is a power of
  // two: this sits between the position load and the cache-row loads)
  const int sblk = a.s;
  int n, place;
  if ((sblk & (sblk - 1)) == 0) {
    n = (pos + sblk - 1) >> __builtin_ctz(sblk);
    place = (pos - 1) & (sblk - 1);
  } else {
    n = slot_of(pos, sblk);
    place = (pos - 1) % sblk;
  }
  if (pos < 1) n = 0;
  if constexpr (TL) {
    if (wave == 0) timeline_stamp(a.timeline, L, 1, static_cast<float>(n));
  }
  const bool ok = pos >= 1 && n <= a.max_slots && (!MERGE || pos <= a.pe_rows);
  uint16_t* out = a.out + (static_cast<size_t>(b) * H + h0) * d_h;
  if (!ok) {
    for (int idx = tid; idx < HG * d_h; idx += NT) out[idx] = 0x7fc0u;  // NaN
    return;
  }
  // Position-dependent loads: pe row, the open slot's state, the rope query
  // and the first two chunks of cache rows.  Memory rows are the completed
  // slots 0..n-2 when merging (row n-1 is the new one, taken from LDS), else
  // 0..n-1.
  float gp[GE], macc = 0.f;
  const bool cont = place != 0;  // the token continues an open block
  if constexpr (MERGE && PP) {
    // one W_hyp row per place in the block
#pragma unroll
    for (int j = 0; j < GE; ++j) gw[j] = a.w_hyp[static_cast<size_t>(place) * a.wh_stride + lane + 64 * j];
  }
  if constexpr (MERGE) {
#pragma unroll
    for (int j = 0; j < GE; ++j) gp[j] = a.pe[static_cast<size_t>(pos - 1) * DC + lane + 64 * j];
    macc = a.open_acc[(static_cast<size_t>(b) * 2 + (pos - 1) % 2) * W + te];
  }
  const int tq = min(tid, HG * DR - 1);
  const uint16_t qrb = a.q_r[(static_cast<size_t>(b) * H + h0 + tq / DR) * DR + tq % DR];
  const uint16_t* rows = a.cache + static_cast<size_t>(b) * a.max_slots * W;
  const int hm = MERGE ? n - 1 : n;
  // rows [0, hm) of the sequence; a load past them reads zero
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(rows), static_cast<short>(0), hm * W * 2,
                                                    kBufferRsrcWord3);
  // chunk ci = slots 16 ci .. +15, 16 W elements contiguous in memory; load
  // ks takes its bytes 1024 ks + 16 lane .. +15 (whole 128-byte lines: a load
  // of 16 rows x 64 bytes, the MFMA operand layout, costs the memory pipeline
  // twice the cycles); the rows reach the MFMA layout through the wave's row
  // buffer
  uint4 ra[KSW], rb[KSW];
  auto load_chunk = [&](int ci, uint4 (&r)[KSW]) {
    if (16 * ci >= hm) return;  // no memory rows (a load past them would still take issue slots)
    const int so = __builtin_amdgcn_readfirstlane(ci * 16 * W * 2);
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + ks * 1024, so, 0);
      r[ks] = uint4{v[0], v[1], v[2], v[3]};
    }
  };
  load_chunk(wave, ra);
  load_chunk(wave + NWV, rb);
  // W_UV is needed last: its loads go out behind the W_UK and cache-row loads
  // in the compute unit's memory pipeline (ahead of them they delay the
  // absorb and the attention), and before the absorb, so that they have
  // arrived when the waves are combined
#pragma unroll
  for (int ks = 0; ks < KSU; ++ks) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_uv, vu + ks * vstep, 0, 0);
    wv[ks] = uint4{v[0], v[1], v[2], v[3]};
  }

  // absorb: partial sums over this thread's rows, W_UK row pairs against
  // (q_c[e0], q_c[e0 + 1]) pairs
  {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const uint32_t x0[4] = {wk0[j].x, wk0[j].y, wk0[j].z, wk0[j].w};
      const uint32_t x1[4] = {wk1[j].x, wk1[j].y, wk1[j].z, wk1[j].w};
      const bf16x2 qv = __builtin_bit_cast(bf16x2, qp[j]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // (row e0, row e0 + 1) of column 2d, then of column 2d + 1
        const uint32_t lo = __builtin_amdgcn_perm(x1[d], x0[d], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(x1[d], x0[d], 0x07060302u);
        acc[2 * d] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lo), qv, acc[2 * d], false);
        acc[2 * d + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), qv, acc[2 * d + 1], false);
      }
    }
    float* dst = &u.ab.red[hl][eg][kc * 8];
    *reinterpret_cast<float4*>(dst) = float4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<float4*>(dst + 4) = float4{acc[4], acc[5], acc[6], acc[7]};
    if constexpr (TL) {
      if (wave == 0) timeline_stamp(a.timeline, L, 2, acc[7]);
    }
  }
  // every wave computes the gate (same values, same order: the same bits)
  float gate = 0.f;
  if constexpr (MERGE) {
    float gx[GE];
#pragma unroll
    for (int j = 0; j < GE; ++j) gx[j] = bf16_bits_to_f32(gxb[j]);
    gate = gate_from_lane_values<GE>(gx, gp, gw);
  }
  __syncthreads();
  if constexpr (MERGE) {
    if (tid < W) {
      const float v = fmaf(gate, bf16_bits_to_f32(mxb), cont ? macc : 0.f);
      const uint16_t w16 = f32_to_bf16_bits(v);
      if (grp == 0) {
        a.open_acc[(static_cast<size_t>(b) * 2 + pos % 2) * W + tid] = v;
        a.cache[(static_cast<size_t>(b) * a.max_slots + n - 1) * W + tid] = w16;
      }
      s_new[tid] = w16;
    }
  }
  const float qscale = a.scale * kLog2e;
  if (tid < HG * DC) {
    const int h = tid / DC, k = tid % DC;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < EGN; ++r) v += u.ab.red[h][r][k];
    split_bf16(v * qscale, sq[h][k], sq[HG + h][k]);
  }
  if (tid < HG * DR)
    split_bf16(bf16_bits_to_f32(qrb) * qscale, sq[tid / DR][DC + tid % DR], sq[HG + tid / DR][DC + tid % DR]);
  for (int e = tid; e < W; e += NT) sq[2 * HG][e] = 0;
  __syncthreads();
  if constexpr (TL) {
    if (wave == 0) timeline_stamp(a.timeline, L, 3, 0.f);
  }

  // attention
  bf16x8 qk[KSW];
  {
    const uint16_t* qrow = sq[c16 < 2 * HG ? c16 : 2 * HG];
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) qk[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + 8 * g);
  }
  constexpr float kLazyLog2 = 8.f;
  float m = -INFINITY, l = 0.f;
  f32x4 acc[CTW];
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row buffer: the chunk's 16 rows at a pitch of W + 8 elements (rows 16
  // bytes apart in the banks, so that the MFMA-layout reads of 16 rows at one
  // column spread over them).  Piece p = 64 ks + lane of a chunk load is
  // row p / (W/8), 16-byte column p % (W/8).
  uint16_t* wb = &rw.r[wave][0][0];
  int woff[KSW];
#pragma unroll
  for (int j = 0; j < KSW; ++j) {
    const int p = 64 * j + lane;
    woff[j] = (p / (W / 8)) * RP + 8 * (p % (W / 8));
  }
  const uint16_t* arow = wb + c16 * RP + 8 * g;
  const uint16_t* vb = wb + (4 * g + (c16 >> 2)) * RP + 4 * (c16 & 3);
  auto do_chunk = [&](int ci, uint4 (&r)[KSW]) {
    const int base = 16 * ci;
    if (base >= n) return;
    if (MERGE && base >= hm) {  // only the new row: nothing was loaded
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) r[ks] = uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < KSW; ++j) *reinterpret_cast<uint4*>(wb + woff[j]) = r[j];
    // the new row (slot hm, merging) comes from LDS (its loaded row read as
    // zero)
    if (MERGE && hm >= base && hm < base + 16 && lane < W / 8)
      *reinterpret_cast<uint4*>(wb + (hm - base) * RP + 8 * lane) = *reinterpret_cast<const uint4*>(s_new + 8 * lane);
    // rows in the MFMA A layout: lane (g, c16) takes row c16, elements
    // 32 ks + 8g .. +7
    bf16x8 arr[KSW];
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) arr[ks] = *reinterpret_cast<const bf16x8*>(arow + 32 * ks);
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const bf16x8 ar = arr[ks];
      if (ks % 2 == 0)
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, qk[ks], sa, 0, 0, 0);
      else
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, qk[ks], sb, 0, 0, 0);
    }
    // sa[i] + sb[i]: the high (column h) or low (column HG + h) part of the
    // score of slot base + 4g + i against head h; added to its partner's, it
    // is the whole score (log2 units), the same bits in both columns
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float part = sa[i] + sb[i];
      const float whole = part + dpp_mov<kPartner>(part);
      sc[i] = base + 4 * g + i < n ? whole : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    // The running max moves only when a score passes it by 2^kLazyLog2; it
    // then becomes the head's exact maximum so far.  Any reference point
    // gives the same softmax after the final division by the sum, and the
    // terms stay below 2^kLazyLog2.
    if (__any(mx > m + kLazyLog2)) {
      const float mn = fmaxf(m, cross_row_max(mx));
      if (ci != wave) {  // nothing accumulated before this wave's first chunk
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) acc[ct] *= alpha;
      }
      m = mn;
    }
    // P^T: column h takes the probabilities' bf16 high parts, column HG + h
    // their low parts
    s16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = fast_exp2(sc[i] - m);
      l += pv;
      uint16_t ph, pl;
      split_bf16(pv, ph, pl);
      pb[i] = static_cast<short>(c16 < HG ? ph : pl);
    }
    // V^T from the wave's row buffer: lane (g, k) of a 16-lane group points
    // at row 4g + k/4, columns 16 ct + 4 (k%4) .. +3, and receives rows
    // 4g .. 4g+3 of column 16 ct + k
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const s16x4 va = lds_read_tr16(vb + ct * 16);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[ct], 0, 0, 0);
    }
  };
  // The first two chunks were loaded ahead; later ones (caches of more than
  // 2 x 8 x 16 slots) one at a time, so that no load is left in flight past
  // the loop (later code reusing its registers would wait on it).
  const int nch = (n + 15) / 16;
  do_chunk(wave, ra);
  do_chunk(wave + NWV, rb);
  for (int ci = wave + 2 * NWV; ci < nch; ci += NWV) {
    load_chunk(ci, ra);
    do_chunk(ci, ra);
  }
  // this wave's sum for head c16: the four lane groups, in a fixed order
  const float lw = cross_row_sum(l);
  if constexpr (TL) timeline_stamp(a.timeline, L, 4 + wave, lw);
  // the wave's O^T columns (head h's high part at column h, low part at
  // HG + h) and its running max and sum (the same in both columns)
  if (c16 < 2 * HG) {
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) *reinterpret_cast<f32x4*>(&u.cb.o[wave][c16][ct * 16 + 4 * g]) = acc[ct];
    if (g == 0 && c16 < HG) {
      u.cb.m[wave][c16] = m;
      u.cb.l[wave][c16] = lw;
    }
  }
  __syncthreads();
  // o_lat[h, col]: the waves' partial results (high + low column) rescaled to
  // a common max and summed in wave order, normalised, split into bf16 hi + lo
  if (tid < HG * DC) {
    const int h = tid / DC, col = tid % DC;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, u.cb.m[w][h]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float f = fast_exp2(u.cb.m[w][h] - M);
      Ls += f * u.cb.l[w][h];
      O += f * (u.cb.o[w][h][col] + u.cb.o[w][HG + h][col]);
    }
    const float v = O / Ls;
    const uint16_t hi = f32_to_bf16_bits(v);
    u.cb.ob[0][h][col] = hi;
    u.cb.ob[1][h][col] = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
  }
  for (int e = tid; e < DC; e += NT) u.cb.zero[e] = 0;
  __syncthreads();
  if constexpr (TL) {
    if (wave == 0) timeline_stamp(a.timeline, L, 12, 0.f);
  }

  // up-projection: C[e, n] = sum_k W_UV[hu][mt*16 + e][k] B[k, n], with
  // column 0 of B = o_lat hi (first product) or lo (second), the other
  // columns zero
  if (up_wave) {
    const uint16_t* bh = c16 == 0 ? &u.cb.ob[0][hu][8 * g] : &u.cb.zero[8 * g];
    const uint16_t* bl = c16 == 0 ? &u.cb.ob[1][hu][8 * g] : &u.cb.zero[8 * g];
    // four independent accumulation chains (hi / lo x even / odd k-steps)
    f32x4 co[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) co[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSU; ++ks) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, wv[ks]);
      co[ks % 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, *reinterpret_cast<const bf16x8*>(bh + ks * 32),
                                                           co[ks % 2], 0, 0, 0);
      co[2 + ks % 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, *reinterpret_cast<const bf16x8*>(bl + ks * 32),
                                                               co[2 + ks % 2], 0, 0, 0);
    }
    // lane (g, 0) holds rows 4g .. 4g+3 of column 0
    if (c16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = mt * 16 + 4 * g + i;
        if (e < d_h) out[hu * d_h + e] = f32_to_bf16_bits((co[0][i] + co[1][i]) + (co[2][i] + co[3][i]));
      }
    }
    if constexpr (TL) {
      if (wave == 0) timeline_stamp(a.timeline, L, 13, co[0][0]);
    }
  }
}

// ---------------------------------------------------------------------------
// The same two products on MFMA (bf16 storage), for long caches where they
// run as their own launches.  A workgroup computes a 32 x 32 tile of the
// output (32 rows r, 32 columns) with 32x32x16 MFMA; its four waves split the
// contraction and add their partial tiles through LDS in wave order.
// Accumulator layout: lane (grp, c32) holds column c32, rows
// 8 (i / 4) + 4 grp + i % 4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void reduce4_store(float (*part)[32 * 33], const f32x16& acc, int wave, int grp,
                                              int c32) {
#pragma unroll
  for (int i = 0; i < 16; ++i) part[wave][(8 * (i / 4) + 4 * grp + (i % 4)) * 33 + c32] = acc[i];
}

// q~[r, h, n] = sum_e q_c[r, h, e] W_UK[h, e, n] for n in the 32-column tile
// n0, head h and the 32 rows from r0 (one workgroup of 256 threads).  W_UK is
// row-major in e, so its tile (d_h rows x 32 columns) is staged in LDS and
// read by transposing reads, which take the contraction rows in the order
// 16 c + 4 grp + r (r < 4), 16 c + 8 + 4 grp + (r - 4); the query fragments
// are loaded in that same order.  Wave w takes the 16-row chunks c = w, w + 4,
// ...  The n0 == 0 tile also copies the rope part of the query beside it.
// Every load of the tile is issued before any is waited for.  The weight
// tile is the launch's dynamic LDS (absorb_lds_bytes(d_h)), so that a
// workgroup takes only what its d_h needs.
constexpr int kAbsorbPitch = 32 + 8;  // LDS pitch of the weight tile (elements)
inline size_t absorb_lds_bytes(int d_h) { return static_cast<size_t>(d_h) * kAbsorbPitch * sizeof(uint16_t); }
__device__ __forceinline__ void absorb_tile(int n0, int h, int r0, int R, int H, int d_h, int d_c, int d_r,
                                            const uint16_t* __restrict__ q_c,
                                            const uint16_t* __restrict__ q_r,
                                            const uint16_t* __restrict__ w_uk, float* __restrict__ qbuf) {
  constexpr int WP = kAbsorbPitch;
  extern __shared__ __align__(16) uint16_t sW[];
  __shared__ float part[4][32 * 33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 5, c32 = lane & 31;
  const int W = d_c + d_r;
  // this wave's query fragments for chunks c = wave + 4 u (u < d_h / 64 <= 4)
  const int r = min(r0 + c32, R - 1);
  const uint16_t* qrow = q_c + (static_cast<size_t>(r) * H + h) * d_h;
  constexpr int UA = kAbsorbMaxDh / 64;
  const int nu = d_h / 64;
  uint4 qa[UA];
#pragma unroll
  for (int u = 0; u < UA; ++u) {
    const int c = wave + 4 * min(u, nu - 1);
    const uint2 lo = *reinterpret_cast<const uint2*>(qrow + 16 * c + 4 * grp);
    const uint2 hi = *reinterpret_cast<const uint2*>(qrow + 16 * c + 8 + 4 * grp);
    qa[u] = uint4{lo.x, lo.y, hi.x, hi.y};
  }
  // weight tile: d_h rows x 4 chunks of 8 columns, thread tid takes chunks
  // tid, tid + 256, ... (all loads first, then the LDS stores)
  constexpr int WC = kAbsorbMaxDh * 4 / 256;
  uint4 wv[WC];
#pragma unroll
  for (int k = 0; k < WC; ++k) {
    const int c = min(tid + 256 * k, d_h * 4 - 1);
    const int e = c >> 2, cc = c & 3;
    wv[k] = *reinterpret_cast<const uint4*>(w_uk + (static_cast<size_t>(h) * d_h + e) * d_c + n0 + cc * 8);
  }
  // rope part of the query (tile n0 == 0): thread tid takes 8-element chunk
  // tid of the 32 rows x d_r / 8 chunks (one pass for d_r <= 64; wider rope
  // parts are copied by a loop at the end)
  const int rch = d_r / 8;
  const bool rope = n0 == 0 && 32 * rch <= 256 && tid < 32 * rch;
  const int rr_r = rope ? tid / rch : 0, re_r = rope ? (tid % rch) * 8 : 0;
  const bool rope_row = rope && r0 + rr_r < R;
  uint4 rv = uint4{0u, 0u, 0u, 0u};
  if (rope_row)
    rv = *reinterpret_cast<const uint4*>(q_r + (static_cast<size_t>(r0 + rr_r) * H + h) * d_r + re_r);
#pragma unroll
  for (int k = 0; k < WC; ++k) {
    const int c = tid + 256 * k;
    if (c < d_h * 4) *reinterpret_cast<uint4*>(sW + (c >> 2) * WP + (c & 3) * 8) = wv[k];
  }
  __syncthreads();
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int q16 = lane >> 4, k16 = lane & 15;
#pragma unroll
  for (int u = 0; u < UA; ++u) {
    if (u >= nu) break;
    const int c = wave + 4 * u;
    const uint16_t* base = sW + (16 * c + 4 * (q16 >> 1) + (k16 >> 2)) * WP + 16 * (q16 & 1) + 4 * (k16 & 3);
    const s16x4 b0 = lds_read_tr16(base);
    const s16x4 b1 = lds_read_tr16(base + 8 * WP);
    const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[u]), b, acc, 0, 0, 0);
  }
  reduce4_store(part, acc, wave, grp, c32);
  if (rope_row) {
    float* dst = qbuf + (static_cast<size_t>(r0 + rr_r) * H + h) * W + d_c + re_r;
    const uint32_t w4[4] = {rv.x, rv.y, rv.z, rv.w};
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(static_cast<uint16_t>(w4[j] & 0xffffu));
      v[2 * j + 1] = bf16_bits_to_f32(static_cast<uint16_t>(w4[j] >> 16));
    }
    store8(dst, v);
  }
  if (n0 == 0 && 32 * rch > 256) {
    for (int idx = tid; idx < 32 * d_r; idx += 256) {
      const int rr = idx / d_r, e = idx % d_r;
      if (r0 + rr < R)
        qbuf[(static_cast<size_t>(r0 + rr) * H + h) * W + d_c + e] =
            bf16_bits_to_f32(q_r[(static_cast<size_t>(r0 + rr) * H + h) * d_r + e]);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 32 * 32; idx += 256) {
    const int rr = idx >> 5, col = idx & 31;
    if (r0 + rr >= R) continue;
    const float v = (part[0][rr * 33 + col] + part[1][rr * 33 + col]) + (part[2][rr * 33 + col] + part[3][rr * 33 + col]);
    qbuf[(static_cast<size_t>(r0 + rr) * H + h) * W + n0 + col] = v;
  }
}

__global__ __launch_bounds__(256) void absorb_mfma_kernel(int R, int H, int d_h, int d_c, int d_r,
                                                          const uint16_t* __restrict__ q_c,
                                                          const uint16_t* __restrict__ q_r,
                                                          const uint16_t* __restrict__ w_uk,
                                                          float* __restrict__ qbuf) {
  absorb_tile(blockIdx.x * 32, blockIdx.y, blockIdx.z * 32, R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf);
}

// The first step of the staged decode step, in one launch: workgroups 0..B-1
// merge token pos[b] of sequence b into its slot (merge_blocks, one block per
// workgroup, the state written in place), the others are absorb tiles
// (n-tile fastest, then head, then row block).  The two parts touch disjoint
// memory: the merge writes the cache and open_acc, the absorb reads the
// queries and W_UK and writes q~.
__global__ __launch_bounds__(256, 5) void merge_absorb_kernel(MergeArgs m, int H, int d_h, int d_r,
                                                           const uint16_t* __restrict__ q_c,
                                                           const uint16_t* __restrict__ q_r,
                                                           const uint16_t* __restrict__ w_uk,
                                                           float* __restrict__ qbuf) {
  const int L = blockIdx.x;
  if (L < m.B) {
    merge_blocks<uint16_t, true>(m, L, 0, 1, 1);
    return;
  }
  const int t = L - m.B, nx = m.d_c / 32;
  absorb_tile((t % nx) * 32, (t / nx) % H, (t / (nx * H)) * 32, m.B, H, d_h, m.d_c, d_r, q_c, q_r, w_uk, qbuf);
}

// out[r, h, e] = sum_k W_UV[h, e, k] o_lat[r, h, k] for e in the 32-row tile
// e0 of W_UV, head h and the 32 rows from r0 (one workgroup of 256 threads).
// Both operands are contiguous in k, so every lane loads its fragments
// directly; the fp32 o_lat enters as a pair of bf16 operands whose sum carries
// it to ~16 significant bits.  Wave w takes the 16-wide k-steps w, w + 4, ...
// The latent rows come from `orow_of(r)`: a pointer to o_lat[r, h, 8 grp],
// in global memory or in LDS.
// The W_UV fragments of one round of k-steps (see up_project_rows), loaded
// ahead of the latent rows where those are still being formed.
constexpr int kUpRound = 8;
struct UpW {
  uint4 bw[kUpRound];
};
__device__ __forceinline__ const uint16_t* up_w_row(const uint16_t* w_uv, int e0, int h, int d_h, int d_c) {
  const int lane = threadIdx.x & 63;
  return w_uv + (static_cast<size_t>(h) * d_h + e0 + (lane & 31)) * d_c + 8 * (lane >> 5);
}
__device__ __forceinline__ void up_w_round(UpW& w, const uint16_t* wrow, int kb, int d_c) {
#pragma unroll
  for (int u = 0; u < kUpRound; ++u) w.bw[u] = *reinterpret_cast<const uint4*>(wrow + min(kb + 64 * u, d_c - 16));
}

// The first round's W fragments may come preloaded (`first`, for
// kb = 16 * wave).
template <typename RowOf>
__device__ __forceinline__ void up_project_rows(int e0, int h, int r0, int R, int H, int d_h, int d_c,
                                                RowOf orow_of, const uint16_t* __restrict__ w_uv,
                                                uint16_t* __restrict__ out, float (*part)[32 * 33],
                                                const UpW* first = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 5, c32 = lane & 31;
  const float* orow = orow_of(c32, grp);
  const uint16_t* wrow = up_w_row(w_uv, e0, h, d_h, d_c);
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // rounds of UP k-steps with all their loads in flight; steps past d_c load
  // a valid address and contribute zero
  constexpr int UP = kUpRound;
  for (int kb = 16 * wave; kb < d_c; kb += 64 * UP) {
    float4 x0[UP], x1[UP];
    UpW w;
    if (first && kb == 16 * wave)
      w = *first;
    else
      up_w_round(w, wrow, kb, d_c);
    const uint4* bw = w.bw;
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int k = min(kb + 64 * u, d_c - 16);
      x0[u] = *reinterpret_cast<const float4*>(orow + k);
      x1[u] = *reinterpret_cast<const float4*>(orow + k + 4);
    }
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const float keep = kb + 64 * u < d_c ? 1.f : 0.f;
      const float xs[8] = {x0[u].x, x0[u].y, x0[u].z, x0[u].w, x1[u].x, x1[u].y, x1[u].z, x1[u].w};
      u16x8 ah, al;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = xs[j] * keep;
        ah[j] = f32_to_bf16_bits(x);
        al[j] = f32_to_bf16_bits(x - bf16_bits_to_f32(ah[j]));
      }
      const bf16x8 b = __builtin_bit_cast(bf16x8, bw[u]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah), b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al), b, acc, 0, 0, 0);
    }
  }
  reduce4_store(part, acc, wave, grp, c32);
  __syncthreads();
  for (int idx = tid; idx < 32 * 32; idx += 256) {
    const int rr = idx >> 5, col = idx & 31;
    if (r0 + rr >= R) continue;
    const float v = (part[0][rr * 33 + col] + part[1][rr * 33 + col]) + (part[2][rr * 33 + col] + part[3][rr * 33 + col]);
    out[(static_cast<size_t>(r0 + rr) * H + h) * d_h + e0 + col] = f32_to_bf16_bits(v);
  }
}

__global__ __launch_bounds__(256) void up_project_mfma_kernel(int R, int H, int d_h, int d_c,
                                                              const float* __restrict__ o_lat,
                                                              const uint16_t* __restrict__ w_uv,
                                                              uint16_t* __restrict__ out) {
  __shared__ float part[4][32 * 33];
  const int h = blockIdx.y, r0 = blockIdx.z * 32;
  auto orow_of = [&](int c32, int grp) {
    return o_lat + (static_cast<size_t>(min(r0 + c32, R - 1)) * H + h) * d_c + 8 * grp;
  };
  up_project_rows(blockIdx.x * 32, h, r0, R, H, d_h, d_c, orow_of, w_uv, out, part);
}

// The split merge and the up-projection in one launch.  A workgroup forms the
// latent rows o_lat[r, h] of its 32 rows in LDS from the `splits` partials of
// the split-K attention, with split_merge_kernel's arithmetic (M = max_k m_k,
// L = sum_k l_k e^(m_k - M), o = (sum_k acc_k e^(m_k - M)) / L, both sums in
// split order, so the same bits), then runs up_project_rows on them.  The
// d_h / 32 workgroups of one (head, row block) form the same rows: the grid
// puts them 8 apart, so that they run on one XCD and the partials are
// fetched into one L2.  The W_UV fragments of the first k-round and the
// partials of the first rows are loaded before the merge weights are
// waited for.  S: the split count (rows are formed 16 / S at a time, all
// their partials in flight).  Dynamic LDS: 32 rows x (d_c + 4) floats.
constexpr int kCombineMaxSplits = 8;
template <int S>
__global__ __launch_bounds__(256) void combine_up_project_kernel(int R, int H, int d_h, int d_c, Partials p,
                                                                 const uint16_t* __restrict__ w_uv,
                                                                 uint16_t* __restrict__ out) {
  constexpr int SMAX = S, splits = S;
  extern __shared__ __align__(16) float so[];
  __shared__ float part[4][32 * 33];
  __shared__ float rw[32][SMAX];
  __shared__ float rl[32];
  constexpr int RI = 16 / SMAX;  // rows formed per iteration by a thread
  const int nx = d_h / 32, nrb = (R + 31) / 32;
  const int L = blockIdx.x;
  const int P = (L / (8 * nx)) * 8 + L % 8, x = (L / 8) % nx;
  if (P >= H * nrb) return;
  const int h = P % H, r0 = (P / H) * 32;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int OP = d_c + 4;  // LDS pitch of a latent row (floats)
  UpW w0;
  up_w_round(w0, up_w_row(w_uv, x * 32, h, d_h, d_c), 16 * wave, d_c);
  // thread tid forms columns 4 ch .. +3 and d_c/2 + 4 ch .. +3 (ch = tid % CR)
  // of rows tid / CR + RP j: a wave's loads of a split's row then read whole
  // 128-byte lines
  const int CR = d_c / 8, RP = 256 / CR;
  const int ch = tid % CR;
  auto load_rows = [&](int rr0, float4 (&a)[RI][SMAX][2]) {
#pragma unroll
    for (int q = 0; q < RI; ++q) {
      const int rr = min(rr0 + q * RP, 31);
      const size_t base = static_cast<size_t>(min(r0 + rr, R - 1)) * splits * H + h;
#pragma unroll
      for (int k = 0; k < S; ++k) {
        const float* src = p.acc + (base + static_cast<size_t>(k) * H) * d_c + 4 * ch;
        a[q][k][0] = *reinterpret_cast<const float4*>(src);
        a[q][k][1] = *reinterpret_cast<const float4*>(src + d_c / 2);
      }
    }
  };
  float4 a[RI][SMAX][2];
  load_rows(tid / CR, a);
  // per row: the merge weights e^(m_k - M) and the denominator L
  if (tid < 32) {
    const size_t base = static_cast<size_t>(min(r0 + tid, R - 1)) * splits * H + h;  // + k * H
    float mk[SMAX], lk[SMAX];
#pragma unroll
    for (int k = 0; k < S; ++k) {
      mk[k] = p.m[base + static_cast<size_t>(k) * H];
      lk[k] = p.l[base + static_cast<size_t>(k) * H];
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < S; ++k) M = fmaxf(M, mk[k]);
    float Ls = 0.f;
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const float w = expf(mk[k] - M);
      rw[tid][k] = w;
      Ls = fmaf(lk[k], w, Ls);
    }
    rl[tid] = Ls;
  }
  __syncthreads();
  for (int rr0 = tid / CR; rr0 < 32; rr0 += RI * RP) {
    if (rr0 != tid / CR) load_rows(rr0, a);
#pragma unroll
    for (int q = 0; q < RI; ++q) {
      const int rr = rr0 + q * RP;
      if (rr >= 32) break;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < S; ++k) {
        const float w = rw[rr][k];
        const float av[8] = {a[q][k][0].x, a[q][k][0].y, a[q][k][0].z, a[q][k][0].w,
                             a[q][k][1].x, a[q][k][1].y, a[q][k][1].z, a[q][k][1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = fmaf(av[j], w, v[j]);
      }
      const float Ls = rl[rr];
      float* dst = so + rr * OP + 4 * ch;
      *reinterpret_cast<float4*>(dst) = float4{v[0] / Ls, v[1] / Ls, v[2] / Ls, v[3] / Ls};
      *reinterpret_cast<float4*>(dst + d_c / 2) = float4{v[4] / Ls, v[5] / Ls, v[6] / Ls, v[7] / Ls};
    }
  }
  __syncthreads();
  auto orow_of = [&](int c32, int grp) -> const float* { return so + c32 * OP + 8 * grp; };
  up_project_rows(x * 32, h, r0, R, H, d_h, d_c, orow_of, w_uv, out, part, &w0);
}

// Rows per workgroup of absorb / up-projection: one row while there are few
// (row, head) pairs, so the launch fills the chip; four when there are many,
// so each W_UK / W_UV chunk loaded serves four rows.
int rows_per_wg(int R, int H) { return static_cast<long long>(R) * H > 1024 ? 4 : 1; }

template <typename T, int RB>
hipError_t absorb_rb(int R, int H, int d_h, int d_c, int d_r, const void* q_c, const void* q_r,
                     const void* w_uk, float* qbuf, hipStream_t st) {
  dim3 grid(H, (R + RB - 1) / RB);
  const size_t smem = (static_cast<size_t>(RB) * d_h + static_cast<size_t>(256 / (d_c / 8)) * RB * d_c) *
                      sizeof(float);
  absorb_kernel<T, RB><<<grid, 256, smem, st>>>(R, H, d_h, d_c, d_r, static_cast<const T*>(q_c),
                                                static_cast<const T*>(q_r),
                                                static_cast<const T*>(w_uk), qbuf);
  return hipGetLastError();
}

bool absorb_mfma_ok(int d_h, int d_c) { return d_h % 64 == 0 && d_h <= kAbsorbMaxDh && d_c % 32 == 0; }

template <typename T>
hipError_t absorb_t(int R, int H, int d_h, int d_c, int d_r, const void* q_c, const void* q_r,
                    const void* w_uk, float* qbuf, hipStream_t st) {
  if (std::is_same<T, uint16_t>::value && absorb_mfma_ok(d_h, d_c)) {
    absorb_mfma_kernel<<<dim3(d_c / 32, H, (R + 31) / 32), 256, absorb_lds_bytes(d_h), st>>>(
        R, H, d_h, d_c, d_r, static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
        static_cast<const uint16_t*>(w_uk), qbuf);
    return hipGetLastError();
  }
  switch (rows_per_wg(R, H)) {
    case 4: return absorb_rb<T, 4>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st);
    default: return absorb_rb<T, 1>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st);
  }
}

template <typename T>
hipError_t attend_t(const AttendArgs& a, hipStream_t st) {
  const int W = a.d_c + a.d_r;
  dim3 grid(a.splits, a.H, a.R);
  if (W <= 64 * 4)
    attend_portable_kernel<T, 4><<<grid, 64, 0, st>>>(a);
  else if (W <= 64 * 8)
    attend_portable_kernel<T, 8><<<grid, 64, 0, st>>>(a);
  else
    attend_portable_kernel<T, 16><<<grid, 64, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  split_merge_kernel<<<dim3(a.H, a.R), 256, 0, st>>>(a.H, a.d_c, a.splits, a.part, a.o_lat);
  return hipGetLastError();
}

template <typename T, int RB>
hipError_t up_project_rb(int R, int H, int d_h, int d_c, const float* o_lat, const void* w_uv,
                         void* out, hipStream_t st) {
  int tpo = 1;
  while (tpo < 64 && 2 * tpo * d_h <= 256) tpo *= 2;
  dim3 grid(H, (R + RB - 1) / RB);
  up_project_kernel<T, RB><<<grid, 256, static_cast<size_t>(RB) * d_c * sizeof(float), st>>>(
      R, H, d_h, d_c, tpo, o_lat, static_cast<const T*>(w_uv), static_cast<T*>(out));
  return hipGetLastError();
}

template <typename T>
hipError_t up_project_t(int R, int H, int d_h, int d_c, const float* o_lat, const void* w_uv,
                        void* out, hipStream_t st) {
  if (std::is_same<T, uint16_t>::value && d_h % 32 == 0 && d_c % 64 == 0) {
    up_project_mfma_kernel<<<dim3(d_h / 32, H, (R + 31) / 32), 256, 0, st>>>(
        R, H, d_h, d_c, o_lat, static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out));
    return hipGetLastError();
  }
  switch (rows_per_wg(R, H)) {
    case 4: return up_project_rb<T, 4>(R, H, d_h, d_c, o_lat, w_uv, out, st);
    default: return up_project_rb<T, 1>(R, H, d_h, d_c, o_lat, w_uv, out, st);
  }
}

}  // namespace

hipError_t launch_absorb(int R, int H, int d_h, int d_c, int d_r, const void* q_c,
                         const void* q_r, const void* w_uk, float* qbuf, int dtype,
                         hipStream_t st) {
  return dtype == 0 ? absorb_t<float>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st)
                    : absorb_t<uint16_t>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st);
}

bool merge_absorb_supported(int d_h, int d_c, int dtype) { return dtype == 1 && absorb_mfma_ok(d_h, d_c); }

hipError_t launch_merge_absorb(const MergeArgs& m, int H, int d_h, int d_r, const void* q_c,
                               const void* q_r, const void* w_uk, float* qbuf, hipStream_t st) {
  if (m.T != 1 || !absorb_mfma_ok(d_h, m.d_c)) return hipErrorInvalidValue;
  const long long tiles = static_cast<long long>(m.d_c / 32) * H * ((m.B + 31) / 32);
  merge_absorb_kernel<<<static_cast<unsigned>(m.B + tiles), 256, absorb_lds_bytes(d_h), st>>>(
      m, H, d_h, d_r, static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
      static_cast<const uint16_t*>(w_uk), qbuf);
  return hipGetLastError();
}

hipError_t launch_attend_portable(const AttendArgs& a, int dtype, hipStream_t st) {
  return dtype == 0 ? attend_t<float>(a, st) : attend_t<uint16_t>(a, st);
}

hipError_t launch_up_project(int R, int H, int d_h, int d_c, const float* o_lat, const void* w_uv,
                             void* out, int dtype, hipStream_t st) {
  return dtype == 0 ? up_project_t<float>(R, H, d_h, d_c, o_lat, w_uv, out, st)
                    : up_project_t<uint16_t>(R, H, d_h, d_c, o_lat, w_uv, out, st);
}

namespace {
// One thread per 16-byte piece of the tile order (see kernels.hpp).
__global__ __launch_bounds__(256) void pack_w_uv_tiles_kernel(int H, int d_h, int d_c, size_t pieces,
                                                              const uint16_t* __restrict__ w_uv,
                                                              uint16_t* __restrict__ tiles) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int nks = d_c / 32, nt = (d_h + 15) / 16;
  const int q = static_cast<int>(i % 64);
  const size_t blk = i / 64;
  const int ks = static_cast<int>(blk % nks);
  const int t = static_cast<int>((blk / nks) % nt);
  const int h = static_cast<int>(blk / (static_cast<size_t>(nks) * nt));
  const int row = 16 * t + q % 16, col = 32 * ks + 8 * (q / 16);
  uint4 v = uint4{0u, 0u, 0u, 0u};
  if (row < d_h) v = *reinterpret_cast<const uint4*>(w_uv + (static_cast<size_t>(h) * d_h + row) * d_c + col);
  *reinterpret_cast<uint4*>(tiles + 8 * i) = v;
}
}  // namespace

size_t w_uv_tiles_elems(int H, int d_h, int d_c) {
  return static_cast<size_t>(H) * ((d_h + 15) / 16) * 16 * d_c;
}

hipError_t launch_pack_w_uv_tiles(int H, int d_h, int d_c, const uint16_t* w_uv, uint16_t* tiles, hipStream_t st) {
  const size_t pieces = w_uv_tiles_elems(H, d_h, d_c) / 8;
  if (pieces == 0) return hipSuccess;
  pack_w_uv_tiles_kernel<<<static_cast<unsigned>((pieces + 255) / 256), 256, 0, st>>>(H, d_h, d_c, pieces, w_uv,
                                                                                     tiles);
  return hipGetLastError();
}

namespace {
template <int DC, int DR, int TS, int HG, int DH, int NTH, int PD>
void step_launch(const StepArgs& a, unsigned grid, hipStream_t st) {
  if (a.merge)
    decode_step_kernel<DC, DR, TS, HG, DH, NTH, PD, true><<<grid, NTH, 0, st>>>(a.pos, a.groups, a.B, a.H, a.d_h, a.w_uk, a.q_c, a.c, a);
  else
    decode_step_kernel<DC, DR, TS, HG, DH, NTH, PD, false><<<grid, NTH, 0, st>>>(a.pos, a.groups, a.B, a.H, a.d_h, a.w_uk, a.q_c, a.c, a);
}
template <int DC, int DR, int HG, int DH>
void step_wave_launch(const StepArgs& a, unsigned grid, hipStream_t st) {
  if (a.timeline)  // (callers take this path only to merge with one W_hyp row)
    decode_step_wave_kernel<DC, DR, HG, DH, true, false, true><<<grid, 512, 0, st>>>(a.pos, a.groups, a.B, a.H, a.d_h, a.w_uk, a.q_c, a.c, a);
  else if (a.merge && a.wh_stride != 0)
    decode_step_wave_kernel<DC, DR, HG, DH, true, true><<<grid, 512, 0, st>>>(a.pos, a.groups, a.B, a.H, a.d_h, a.w_uk, a.q_c, a.c, a);
  else if (a.merge)
    decode_step_wave_kernel<DC, DR, HG, DH, true><<<grid, 512, 0, st>>>(a.pos, a.groups, a.B, a.H, a.d_h, a.w_uk, a.q_c, a.c, a);
  else
    decode_step_wave_kernel<DC, DR, HG, DH, false><<<grid, 512, 0, st>>>(a.pos, a.groups, a.B, a.H, a.d_h, a.w_uk, a.q_c, a.c, a);
}

// Heads per group the step kernel is instantiated for, per latent shape.
bool step_hg_instantiated(int d_c, int d_r, int hg, int d_h) {
  if (d_c == 256 && d_r == 32) return (hg == 1 || hg == 2) && d_h <= 64;
  if (d_c == 512 && d_r == 64) return hg == 1 && d_h <= 128;
  return false;
}
}  // namespace

bool decode_step_supported(int H, int d_h, int d_c, int d_r) {
  return d_h >= 1 && step_hg_instantiated(d_c, d_r, 1, d_h) && H >= 1;
}

int decode_step_groups(int B, int H, int d_h, int d_c, int requested) {
  // Most head groups that still fit the launch in one round of workgroups
  // (B * groups <= 256: one 512-thread workgroup fills a compute unit's
  // registers), among the instantiated group sizes; the fewest groups when
  // even that does not fit.  A requested count is taken when it is valid.
  const int d_r = d_c == 256 ? 32 : 64;
  auto ok = [&](int g) { return g >= 1 && H % g == 0 && step_hg_instantiated(d_c, d_r, H / g, d_h); };
  if (ok(requested)) return requested;
  int fewest = 0, best = 0;
  for (int g = 1; g <= H; ++g) {
    if (!ok(g)) continue;
    if (fewest == 0) fewest = g;
    if (static_cast<long long>(B) * g <= 256) best = g;
  }
  return best ? best : fewest;
}

hipError_t launch_decode_step(const StepArgs& a0, hipStream_t st) {
  StepArgs a = a0;
  a.groups = decode_step_groups(a.B, a.H, a.d_h, a.d_c, a0.groups);
  if (a.groups < 1) return hipErrorNotSupported;
  const int hg = a.H / a.groups;
  const unsigned grid = 8u * static_cast<unsigned>(a.groups) * static_cast<unsigned>((a.B + 7) / 8);
  if (a.d_c == 256 && a.d_r == 32 && hg == 1) {
    step_wave_launch<256, 32, 1, 64>(a, grid, st);
  } else if (a.d_c == 256 && a.d_r == 32 && hg == 2) {
    step_wave_launch<256, 32, 2, 64>(a, grid, st);
  } else if (a.d_c == 512 && a.d_r == 64 && hg == 1 && !(a.merge && a.wh_stride != 0)) {
    step_launch<512, 64, 64, 1, 128, 1024, 1>(a, grid, st);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

bool decode_mfma_supported(int H, int d_c, int d_r) {
  if (d_c == 256 && d_r == 32) return H <= 32;
  if (d_c == 512 && d_r == 64) return H <= 32;
  return false;
}

hipError_t launch_decode_mfma(const AttendArgs& a, hipStream_t st, bool merge_splits) {
  dim3 grid(a.splits, a.R);
  if (a.d_c == 256 && a.d_r == 32) {
    if (a.H <= 16)
      decode_mfma_kernel<1, 256, 32><<<grid, 256, 0, st>>>(a);
    else
      decode_mfma_kernel<2, 256, 32><<<grid, 256, 0, st>>>(a);
  } else if (a.d_c == 512 && a.d_r == 64) {
    if (a.H <= 16)
      decode_stream_kernel<1><<<grid, 512, 0, st>>>(a);
    else
      decode_stream_kernel<2><<<grid, 512, 0, st>>>(a);
  } else {
    return hipErrorNotSupported;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1 || !merge_splits) return e;
  split_merge_kernel<<<dim3(a.H, a.R), 256, 0, st>>>(a.H, a.d_c, a.splits, a.part, a.o_lat);
  return hipGetLastError();
}

bool combine_up_project_supported(int d_h, int d_c, int splits, int dtype) {
  return dtype == 1 && d_h % 32 == 0 && d_c % 64 == 0 && d_c <= 1024 && splits >= 2 &&
         splits <= kCombineMaxSplits;
}

hipError_t launch_combine_up_project(int R, int H, int d_h, int d_c, int splits, const Partials& p,
                                     const void* w_uv, void* out, hipStream_t st) {
  if (!combine_up_project_supported(d_h, d_c, splits, 1)) return hipErrorInvalidValue;
  const long long pairs = static_cast<long long>(H) * ((R + 31) / 32);
  const long long grid = (pairs + 7) / 8 * 8 * (d_h / 32);
  const size_t smem = static_cast<size_t>(32) * (d_c + 4) * sizeof(float);
  const dim3 g(static_cast<unsigned>(grid));
  const uint16_t* w = static_cast<const uint16_t*>(w_uv);
  uint16_t* o = static_cast<uint16_t*>(out);
  switch (splits) {
    case 2: combine_up_project_kernel<2><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
    case 3: combine_up_project_kernel<3><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
    case 4: combine_up_project_kernel<4><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
    case 5: combine_up_project_kernel<5><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
    case 6: combine_up_project_kernel<6><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
    case 7: combine_up_project_kernel<7><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
    default: combine_up_project_kernel<8><<<g, 256, smem, st>>>(R, H, d_h, d_c, p, w, o); break;
  }
  return hipGetLastError();
}

}  // namespace mtla
