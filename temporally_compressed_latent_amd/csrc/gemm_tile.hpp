// One TM x 128 tile of C = A W^T (bf16 operands, fp32 sums, TM = 128 or
// 256) for the GEMMs around the attention (K/V up-projection, layer
// projections).
//
// The K loop streams 32-column stages of the A and W row panels through a
// ring of LDS stages.  Every stage is filled by direct-to-LDS loads (no
// registers hold data in flight), issued up to three stages ahead.  What
// bounds these GEMMs is the operand traffic from L2 into each CU (16 bytes
// per 1024 flops with 128x128 tiles, about the per-CU load rate at full MFMA
// speed), so the 256-row tile, which moves 12, is the one used where M is
// large.  LDS rows are 64 bytes, unpadded (a direct load writes 64
// consecutive 16-byte pieces); the four pieces of row r sit in slot
// piece ^ ((r / 4) % 4), so the MFMA operand reads of 16 consecutive rows hit
// 16 different bank groups.
//
// Four waves in a 2x2 grid of (TM/2)x64; each multiplies 32x32x16 bf16
// tiles: acc[i][j] is rows (TM/2) wm + 32 i .., columns 64 wn + 32 j .. of C
// (SWAP: the same tile of C^T, i.e. acc[i][j][e] is C row (TM/2) wm + 32 i +
// c32 (lane c32), column 64 wn + 32 j + 8 (e / 4) + 4 grp + e % 4).
#pragma once
#include "common.hpp"

namespace mtla {

// TM = 128 or 256 rows of A per tile (128 of W).  Each stage holds TM + 128
// rows of 32 columns; NS stages (NS - 1 issued ahead).
template <int TM>
struct TileShape {
  static constexpr int K = 32;                                  // columns per stage
  static constexpr int NS = TM == 128 ? 4 : 3;                   // ring depth
  static constexpr int StageElems = (TM + 128) * K;              // A rows, then W rows
  static constexpr int SmemElems = NS * StageElems;              // 64 KB / 72 KB
  static constexpr int ALoads = TM / 64, WLoads = 2;             // direct loads per thread and stage
  static constexpr int I = TM / 64;                              // 32-row MFMA tiles per wave
};
constexpr int kTileSmemElems = TileShape<128>::SmemElems;

// 16 bytes per lane from a global address straight into LDS, at byte
// lds_base + 16 * lane (lds_base wave-uniform).  Issued in inline asm so that
// the compiler does not wait for it before every later LDS read; the caller
// waits by count (s_waitcnt vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void global_load_lds16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds_base), "v"(gptr) : "memory", "m0");
}

// Wait until at most n of this thread's vector memory operations are
// outstanding (n: 0, 4, 6, 8 or 12).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// arow[k] (k < TM / 64), wrow[k] (k < 2): the A and W rows 16 (4k + wave) +
// lane / 4 of the tile (rows past the matrix clamped to a real row: their
// products are never stored).  K: a multiple of 32.  smem:
// TileShape<TM>::SmemElems elements.  acc[i][j] (i < TM / 64, j < 2): rows
// (TM / 2) wm + 32 i, columns 64 wn + 32 j of the tile (SWAP: of C^T, see
// above).
template <int TM, bool SWAP>
__device__ __forceinline__ void gemm_tile(const uint16_t* const (&arow)[TM / 64], const uint16_t* const (&wrow)[2],
                                          int K, uint16_t* smem, f32x16 (&acc)[TM / 64][2]) {
  using S = TileShape<TM>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, grp = lane >> 5, c32 = lane & 31;
  // this thread's piece of each load: row r = 16 (4k + wave) + lane / 4 and
  // LDS slot lane % 4, which holds the row's piece (lane % 4) ^ ((r / 4) % 4)
  const uint16_t* src[S::ALoads + S::WLoads];
#pragma unroll
  for (int k = 0; k < S::ALoads + S::WLoads; ++k) {
    const int kr = k < S::ALoads ? k : k - S::ALoads;
    const int r = 16 * (4 * kr + wave) + (lane >> 2);
    const int piece = (lane & 3) ^ ((r >> 2) & 3);
    src[k] = (k < S::ALoads ? arow[kr] : wrow[kr]) + 8 * piece;
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (kt % S::NS) * (S::StageElems * 2);
#pragma unroll
    for (int k = 0; k < S::ALoads; ++k) global_load_lds16(src[k] + kt * S::K, st + (4 * k + wave) * 1024);
#pragma unroll
    for (int k = 0; k < S::WLoads; ++k)
      global_load_lds16(src[S::ALoads + k] + kt * S::K, st + TM * S::K * 2 + (4 * k + wave) * 1024);
  };
#pragma unroll
  for (int i = 0; i < S::I; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int nk = K / S::K;
#pragma unroll
  for (int p = 0; p < S::NS - 1; ++p)
    if (p < nk) issue(p);
  const int sw = (c32 >> 2) & 3;  // (row / 4) % 4 of every operand row this lane reads
  constexpr int per = S::ALoads + S::WLoads;
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads of stage kt are done when at most the later
    // stages' are outstanding
    wait_vm(per * min(nk - 1 - kt, S::NS - 2));
    // every thread's stage kt is in LDS, and every wave is done with stage
    // kt - 1, whose slot the next issue refills
    __syncthreads();
    if (kt + S::NS - 1 < nk) issue(kt + S::NS - 1);
    const uint16_t* sA = smem + (kt % S::NS) * S::StageElems;
    const uint16_t* sW = sA + TM * S::K;
#pragma unroll
    for (int kc = 0; kc < S::K / 16; ++kc) {
      const int slot = (2 * kc + grp) ^ sw;
      bf16x8 a[S::I], b[2];
#pragma unroll
      for (int i = 0; i < S::I; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sA + ((TM / 2) * wm + 32 * i + c32) * S::K + 8 * slot);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(sW + (64 * wn + 32 * j + c32) * S::K + 8 * slot);
#pragma unroll
      for (int i = 0; i < S::I; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // the operand stages are free for the caller's epilogue
  __syncthreads();
}

}  // namespace mtla
