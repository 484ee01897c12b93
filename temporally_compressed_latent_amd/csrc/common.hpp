// Device helpers shared by the MTLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Storage types: fp32 is stored as float, bf16 as its 16-bit pattern.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// fp16 (IEEE binary16, round to nearest even) bit patterns.  A bf16 value in
// fp16's normal range (2^-14 .. 65504 in magnitude) converts exactly: bf16
// has 8 significant bits, fp16 11.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
// v rounded to the nearest fp16 value (returned as fp32)
__device__ __forceinline__ float f16_round(float v) { return static_cast<float>(static_cast<_Float16>(v)); }

// An fp32 value as the sum of two bf16 values: hi = round(v), lo =
// round(v - hi).  hi + lo carries v to 16 significant bits, so an MFMA that
// takes both parts as operands keeps an fp32 operand's accuracy to within
// 2^-16 relative.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Store<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16_bits(v);
  }
};

// Eight consecutive stored elements (16-byte aligned for bf16, 32 for fp32)
// as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// ---------------------------------------------------------------------------
// Slot arithmetic and the stride-aware mask (integers, exact).
//   Token t (1-based) lives in slot ceil(t/s) (1-based).  Query i attends key
//   j iff j == i, or s | j and j/s < ceil(i/s).  In slot terms: query i sees
//   the completed slots b = 1..floor((i-1)/s) plus its own partial slot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int slot_of(int t, int s) { return (t + s - 1) / s; }
__device__ __forceinline__ int completed_slots(int i, int s) { return (i - 1) / s; }
__device__ __forceinline__ bool stride_visible(int i, int j, int s) {
  return (j == i) || ((j % s) == 0 && (j / s) < slot_of(i, s));
}

// ---------------------------------------------------------------------------
// Wave64 reductions.
// ---------------------------------------------------------------------------
// Reductions over the 16 lanes of each DPP row (lanes 16r .. 16r+15); every
// lane of the row receives the result.  Four DPP moves, no LDS traffic:
// swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), then
// row_half_mirror (lane i <- 7 - i within 8) and row_mirror (lane i <- 15 - i)
// bring in the other quad and the other half.  The pairs combined at each
// step are the same for every lane, so all lanes hold bit-identical sums.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// Across the four 16-lane rows of a wave, for each lane position: the max
// (sum) of the value at lanes c, c+16, c+32, c+48, returned to all four.
// v_permlane16_swap exchanges rows 1 <-> 0 and 3 <-> 2 between its two
// operands, v_permlane32_swap the halves; with both operands holding the
// same value, afterwards each holds a row's own value or its partner's, and
// combining the two gives every lane the same pair.  Sums are
// (r0 + r1) + (r2 + r3).  Written as VALU asm (two read-write operands in
// distinct registers): the builtins' two results were folded into one by
// the compiler when both inputs are the same value.  s_nop 1 covers the
// VALU-write to permlane-read hazard.
__device__ __forceinline__ void permlane16_swap_regs(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap_regs(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float cross_row_max(float v) {
  float a = v, b = v;
  permlane16_swap_regs(a, b);
  v = fmaxf(a, b);
  a = v;
  b = v;
  permlane32_swap_regs(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float cross_row_sum(float v) {
  float a = v, b = v;
  permlane16_swap_regs(a, b);
  v = a + b;
  a = v;
  b = v;
  permlane32_swap_regs(a, b);
  return a + b;
}

// Sum over the 64 lanes of a wave, returned to every lane: the four 16-lane
// row sums (DPP), then (row0 + row1) + (row2 + row3) from lanes 0, 16, 32, 48.
// The order is fixed, so every kernel that uses it gets the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a0 + a1) + (a2 + a3);
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// Workgroup barrier that waits only for this wave's LDS operations, not for
// vector-memory loads still in flight (__syncthreads' fence waits for those
// too, which would drain a ring of tiles being loaded straight into LDS).
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte load from a raw buffer straight into LDS: lane i's 16 bytes, at
// byte voff (+ soff) of the buffer `rsrc`, go to LDS byte lds_base + 16 * i
// (lds_base wave-uniform).  Offsets past the buffer's num_records read zero.
// The load is non-temporal (nt): the data streams through once and is not
// kept in the caches, which lets HBM reads run measurably faster for a
// stream of cache rows read once per call.
// Issued in inline asm so that the compiler does not insert its own waits for
// it before every later LDS read (it cannot tell the LDS range apart): the
// caller waits for these loads itself, by count, with wait_vmcnt() before the
// barrier that publishes the data.  The asm has no output register; its
// operands are read when it issues.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buffer_load_lds16(i32x4_t rsrc, uint32_t lds_base, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// The same load with the default cache policy, for data that other
// workgroups read again (weights).
__device__ __forceinline__ void buffer_load_lds16_cached(i32x4_t rsrc, uint32_t lds_base, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// Raw buffer resource words for a wave-uniform base address and size.
__device__ __forceinline__ i32x4_t make_rsrc_words(const void* base, int nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(nbytes);
  r.w = 0x00020000;
  return r;
}
// LDS byte address of a pointer into shared memory, made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p))));
}

// Word 3 of a raw buffer resource on gfx9-family parts (CDNA): 32-bit data
// format, no swizzle, offsets checked against num_records.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Gates of NTOK tokens, computed by one wave ("Multi-head Temporal Latent
// Attention", Key claims, paper Sec. 4.1 Eq. 13):
//   w_t = sigmoid(W_hyp . (c_t + pe_t)).
// For each token, lane l accumulates columns l, l+64, ... in order and the
// lanes are then added with a butterfly; the NTOK tokens are independent
// instruction streams, so their loads are in flight together.  Every kernel
// that gates a token uses this arithmetic, so a token gets bit-identical
// gates whichever entry point merges it.  Tokens with c_rows[k] == nullptr
// are skipped (their gate is 0).
// wh_rows[k] is the W_hyp row token k takes (the same row for every token
// unless W_hyp has one row per place in the block).
template <int NTOK, typename T>
__device__ __forceinline__ void gates_of_tokens(const T* const (&c_rows)[NTOK],
                                                const float* const (&pe_rows)[NTOK],
                                                const float* const (&wh_rows)[NTOK], int d_c, int lane,
                                                float (&w)[NTOK]) {
  float acc[NTOK];
#pragma unroll
  for (int k = 0; k < NTOK; ++k) acc[k] = 0.f;
  for (int e = lane; e < d_c; e += 64) {
#pragma unroll
    for (int k = 0; k < NTOK; ++k)
      if (c_rows[k]) acc[k] = fmaf(Store<T>::load(c_rows[k], e) + pe_rows[k][e], wh_rows[k][e], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < NTOK; ++k) {
    const float z = wave_sum(acc[k]);
    w[k] = c_rows[k] ? 1.f / (1.f + expf(-z)) : 0.f;
  }
}

// The same gate from values a lane has already loaded: x[j], pe[j] and wh[j]
// are element lane + 64 j of c_t, pe_t and W_hyp (GE = d_c / 64).  Same
// operation order as gates_of_tokens, so the result is bit-identical.
template <int GE>
__device__ __forceinline__ float gate_from_lane_values(const float (&x)[GE], const float (&pe)[GE],
                                                       const float (&wh)[GE]) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < GE; ++j) acc = fmaf(x[j] + pe[j], wh[j], acc);
  const float z = wave_sum(acc);
  return 1.f / (1.f + expf(-z));
}

template <typename T>
__device__ __forceinline__ float gate_of_token(const T* c_row, const float* pe_row,
                                               const float* w_hyp, int d_c, int lane) {
  const T* const rows[1] = {c_row};
  const float* const pes[1] = {pe_row};
  const float* const whs[1] = {w_hyp};
  float w[1];
  gates_of_tokens<1, T>(rows, pes, whs, d_c, lane, w);
  return w[0];
}

// Eight consecutive fp32 values stored to the storage type (16-byte aligned
// for bf16, 32 for fp32), rounded to nearest even.
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 u;
  u.x = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  u.z = static_cast<uint32_t>(f32_to_bf16_bits(v[4])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[5])) << 16);
  u.w = static_cast<uint32_t>(f32_to_bf16_bits(v[6])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[7])) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<float4*>(p + 4) = float4{v[4], v[5], v[6], v[7]};
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane k supplies the address of 4 consecutive 16-bit values; lane i receives
// as element r the (i % 4)-th value of lane 4r + i/4.  With lane k pointing at
// row base + k/4, columns col0 + 4*(k%4) of a row-major tile, lane i gets
// rows base..base+3 of column col0 + i: a K-contiguous MFMA operand read from
// a tile whose contiguous dimension is the MFMA's M or N.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

}  // namespace mtla
