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
#include "common.hpp"
#include "kernels.hpp"

namespace mtla {

namespace {

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
    for (int e = eg; e < d_h; e += EG) {
      float w[8];
      load8(w_uk + (static_cast<size_t>(h) * d_h + e) * d_c + kc * 8, w);
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const float q = sq[rr * d_h + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rr][j] = fmaf(q, w[j], acc[rr][j]);
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
    const int i = r % a.N + 1;
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
    L += p.l[base + static_cast<size_t>(k) * H] * expf(p.m[base + static_cast<size_t>(k) * H] - M);
  for (int e = threadIdx.x; e < d_c; e += blockDim.x) {
    float v = 0.f;
    for (int k = 0; k < splits; ++k) {
      const size_t pk = base + static_cast<size_t>(k) * H;
      v += p.acc[pk * d_c + e] * expf(p.m[pk] - M);
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
    for (int c = p; c < KC; c += tpo) {
      float w[8];
      load8(w_uv + (static_cast<size_t>(h) * d_h + e) * d_c + c * 8, w);
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const float* o = olat + rr * d_c + c * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rr] = fmaf(w[j], o[j], acc[rr]);
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
// MFMA latent attention for decode (bf16 cache).  One workgroup (4 waves) per
// (split, sequence), all heads padded to HT*16 MFMA rows.
//
// Per 64-slot tile:
//   1. the tile (64 rows x W bf16) is copied HBM -> registers -> LDS, and the
//      next tile's loads are issued before this tile is used;
//   2. scores S[head, slot] = Q~ . row via v_mfma_f32_16x16x32_bf16; wave w
//      owns slots 16w..16w+15, A = scaled queries (LDS), B = slot rows (LDS);
//   3. the tile max per head is shared through LDS, p = exp2(S - m) goes to
//      LDS as bf16, and the running (m, l, acc) are rescaled;
//   4. acc[head, col] += P . rows, wave w owning latent columns
//      w*DC/4 .. (w+1)*DC/4-1.  The B operand (8 slots of one column) comes
//      from two ds_read_b64_tr_b16 transposing loads of the row-major tile.
// Scores are carried in the log2 domain (queries pre-scaled by tau*log2 e).
//
// With a single split the workgroup normalises and writes o_lat itself;
// otherwise it stores its (m, l, acc) partial and split_merge_kernel, launched
// next on the stream, merges the splits in split order.  (A last-arriving-
// workgroup merge inside this kernel would need device-scope release/acquire
// fences per workgroup, which on this multi-XCD part write back and invalidate
// L2 and cost far more than the extra launch.)
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

template <int HT, int DC, int DR>
__global__ __launch_bounds__(256) void decode_mfma_kernel(AttendArgs a) {
  constexpr int W = DC + DR;
  constexpr int KS = W / 32;
  constexpr int HP = HT * 16;
  constexpr int TS = 64;
  constexpr int PITCH = W + 8;
  constexpr int PP = TS + 8;
  constexpr int CPW = DC / 4;
  constexpr int CT = CPW / 16;
  constexpr int CPR = W / 8;  // 16-byte chunks per row
  static_assert(W % 32 == 0 && DC % 64 == 0, "tile shape");
  static_assert((TS * CPR) % 256 == 0, "tile copy");
  constexpr int CPT = TS * CPR / 256;  // chunks per thread

  __shared__ __align__(16) uint16_t sQ[HP * PITCH];
  __shared__ __align__(16) uint16_t sK[TS * PITCH];
  __shared__ __align__(16) uint16_t sP[HP * PP];
  __shared__ float sRed[4][HP];

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
    sQ[hh * PITCH + e] = f32_to_bf16_bits(v);
  }

  float m_run[HT][4], l_part[HT][4];
  f32x4 acc[HT][CT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[ht][i] = -INFINITY;
      l_part[ht][i] = 0.f;
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ht][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* cache_b =
      static_cast<const uint16_t*>(a.cache) + static_cast<size_t>(b) * a.max_slots * W;
  uint4 pre[CPT];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int id = tid + 256 * k;
      const int row = id / CPR, ch = id % CPR;
      const int slot = j0 + row;
      if (slot < hi)
        pre[k] = *reinterpret_cast<const uint4*>(cache_b + static_cast<size_t>(slot) * W + ch * 8);
      else
        pre[k] = uint4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int id = tid + 256 * k;
      const int row = id / CPR, ch = id % CPR;
      *reinterpret_cast<uint4*>(sK + row * PITCH + ch * 8) = pre[k];
    }
  };

  if (lo < hi) load_tile(lo);
  for (int j0 = lo; j0 < hi; j0 += TS) {
    store_tile();
    __syncthreads();
    if (j0 + TS < hi) load_tile(j0 + TS);

    // scores: wave owns slots 16*wave .. 16*wave+15 of the tile
    f32x4 sc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bk =
          *reinterpret_cast<const bf16x8*>(sK + (16 * wave + c16) * PITCH + ks * 32 + 8 * g);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const bf16x8 aq =
            *reinterpret_cast<const bf16x8*>(sQ + (ht * 16 + c16) * PITCH + ks * 32 + 8 * g);
        sc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, sc[ht], 0, 0, 0);
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
        v = fmaxf(v, __shfl_xor(v, 1, 64));
        v = fmaxf(v, __shfl_xor(v, 2, 64));
        v = fmaxf(v, __shfl_xor(v, 4, 64));
        v = fmaxf(v, __shfl_xor(v, 8, 64));
        if (c16 == 0) sRed[wave][ht * 16 + 4 * g + i] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        const float mt =
            fmaxf(fmaxf(sRed[0][head], sRed[1][head]), fmaxf(sRed[2][head], sRed[3][head]));
        const float mn = fmaxf(m_run[ht][i], mt);
        const float alpha = fast_exp2(m_run[ht][i] - mn);
        m_run[ht][i] = mn;
        const float pv = fast_exp2(sc[ht][i] - mn);
        l_part[ht][i] = l_part[ht][i] * alpha + pv;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ht][ct][i] *= alpha;
        sP[head * PP + 16 * wave + c16] = f32_to_bf16_bits(pv);
      }
    }
    __syncthreads();

    // acc[head, col] += sum_slot P[head, slot] * row[slot, col]
#pragma unroll
    for (int ks2 = 0; ks2 < TS / 32; ++ks2) {
      bf16x8 ap[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        ap[ht] = *reinterpret_cast<const bf16x8*>(sP + (ht * 16 + c16) * PP + ks2 * 32 + 8 * g);
      // Lane (g, c16) needs rows ks2*32 + 8g + 0..7 of column col0 + c16.  A
      // transposing read covers 4 rows: lane k of a 16-lane group points at
      // row base + k/4, columns col0 + 4*(k%4) .. +3; lane i then receives as
      // element r the (i%4)-th value of lane 4r + i/4, i.e. row base + r of
      // column col0 + i.
      const uint16_t* rbase = sK + (ks2 * 32 + 8 * g + (c16 >> 2)) * PITCH + 4 * (c16 & 3);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col0 = wave * CPW + ct * 16;
        const s16x4 lo4 = lds_read_tr16(rbase + col0);
        const s16x4 hi4 = lds_read_tr16(rbase + 4 * PITCH + col0);
        const s16x8 v8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 bb = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[ht], bb, acc[ht][ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // l: sum over the 16 slot lanes and the 4 waves
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = l_part[ht][i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      if (c16 == 0) sRed[wave][ht * 16 + 4 * g + i] = v;
    }
  }
  __syncthreads();

  if (nsplit == 1) {
    // single split: normalise in registers and write o_lat directly
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        if (head < H) {
          const float L = (sRed[0][head] + sRed[1][head]) + (sRed[2][head] + sRed[3][head]);
          const float inv = 1.f / L;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            a.o_lat[(static_cast<size_t>(b) * H + head) * DC + wave * CPW + ct * 16 + c16] =
                acc[ht][ct][i] * inv;
        }
      }
    }
    return;
  }

  const size_t pbase = (static_cast<size_t>(b) * nsplit + split) * H;
  if (wave == 0 && c16 == 0) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = ht * 16 + 4 * g + i;
        if (head < H) {
          // the running max is in log2 units; partials use natural-log units
          a.part.m[pbase + head] = m_run[ht][i] * kLn2;
          a.part.l[pbase + head] =
              (sRed[0][head] + sRed[1][head]) + (sRed[2][head] + sRed[3][head]);
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

template <typename T>
hipError_t absorb_t(int R, int H, int d_h, int d_c, int d_r, const void* q_c, const void* q_r,
                    const void* w_uk, float* qbuf, hipStream_t st) {
  return rows_per_wg(R, H) == 4 ? absorb_rb<T, 4>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st)
                                : absorb_rb<T, 1>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st);
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
  return rows_per_wg(R, H) == 4 ? up_project_rb<T, 4>(R, H, d_h, d_c, o_lat, w_uv, out, st)
                                : up_project_rb<T, 1>(R, H, d_h, d_c, o_lat, w_uv, out, st);
}

}  // namespace

hipError_t launch_absorb(int R, int H, int d_h, int d_c, int d_r, const void* q_c,
                         const void* q_r, const void* w_uk, float* qbuf, int dtype,
                         hipStream_t st) {
  return dtype == 0 ? absorb_t<float>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st)
                    : absorb_t<uint16_t>(R, H, d_h, d_c, d_r, q_c, q_r, w_uk, qbuf, st);
}

hipError_t launch_attend_portable(const AttendArgs& a, int dtype, hipStream_t st) {
  return dtype == 0 ? attend_t<float>(a, st) : attend_t<uint16_t>(a, st);
}

hipError_t launch_up_project(int R, int H, int d_h, int d_c, const float* o_lat, const void* w_uv,
                             void* out, int dtype, hipStream_t st) {
  return dtype == 0 ? up_project_t<float>(R, H, d_h, d_c, o_lat, w_uv, out, st)
                    : up_project_t<uint16_t>(R, H, d_h, d_c, o_lat, w_uv, out, st);
}

bool decode_mfma_supported(int H, int d_c, int d_r) {
  if (d_c == 256 && d_r == 32) return H <= 32;
  if (d_c == 512 && d_r == 64) return H <= 32;
  return false;
}

hipError_t launch_decode_mfma(const AttendArgs& a, hipStream_t st) {
  dim3 grid(a.splits, a.R);
  if (a.d_c == 256 && a.d_r == 32) {
    if (a.H <= 16)
      decode_mfma_kernel<1, 256, 32><<<grid, 256, 0, st>>>(a);
    else
      decode_mfma_kernel<2, 256, 32><<<grid, 256, 0, st>>>(a);
  } else if (a.d_c == 512 && a.d_r == 64) {
    if (a.H <= 16)
      decode_mfma_kernel<1, 512, 64><<<grid, 256, 0, st>>>(a);
    else
      decode_mfma_kernel<2, 512, 64><<<grid, 256, 0, st>>>(a);
  } else {
    return hipErrorNotSupported;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  split_merge_kernel<<<dim3(a.H, a.R), 256, 0, st>>>(a.H, a.d_c, a.splits, a.part, a.o_lat);
  return hipGetLastError();
}

}  // namespace mtla
