// One 128x128 tile of C = A W^T (bf16 operands, fp32 sums) for the GEMMs
// around the attention (K/V up-projection, layer projections).
//
// The K loop streams 32-column stages of the A and W row panels through a
// ring of four 16 KB LDS stages.  Every stage is filled by direct-to-LDS
// loads (no registers hold data in flight), issued three stages ahead, so a
// workgroup keeps 48 KB of loads outstanding while it multiplies: with short
// K (256..1024) the loop is otherwise a chain of memory round trips.  LDS
// rows are 64 bytes, unpadded (a direct load writes 64 consecutive 16-byte
// pieces); the four pieces of row r sit in slot piece ^ ((r / 4) % 4), so the
// MFMA operand reads of 16 consecutive rows hit 16 different bank groups.
//
// Four waves in a 2x2 grid of 64x64; each multiplies 32x32x16 bf16 tiles:
// acc[i][j] is rows 64 wm + 32 i .., columns 64 wn + 32 j .. of C (SWAP:
// the same tile of C^T, i.e. acc[i][j][e] is C row 64 wm + 32 i + c32 (lane
// c32), column 64 wn + 32 j + 8 (e / 4) + 4 grp + e % 4).
#pragma once
#include "common.hpp"

namespace mtla {

constexpr int kTileRows = 128, kTileK = 32, kTileStages = 4;
constexpr int kTileStageElems = 2 * kTileRows * kTileK;  // A then W, 16 KB
constexpr int kTileSmemElems = kTileStages * kTileStageElems;

// 16 bytes per lane from a global address straight into LDS, at byte
// lds_base + 16 * lane (lds_base wave-uniform).  Issued in inline asm so that
// the compiler does not wait for it before every later LDS read; the caller
// waits by count (s_waitcnt vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void global_load_lds16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds_base), "v"(gptr) : "memory", "m0");
}

// arow[k], wrow[k] (k = 0, 1): the A and W rows 16 (4k + wave) + lane / 4 of
// the tile (rows past the matrix clamped to a real row: their products are
// never stored).  K: a multiple of 32.  smem: kTileSmemElems elements.
template <bool SWAP>
__device__ __forceinline__ void gemm_tile_128(const uint16_t* const (&arow)[2], const uint16_t* const (&wrow)[2],
                                              int K, uint16_t* smem, f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, grp = lane >> 5, c32 = lane & 31;
  // this thread's piece of each load: row r = 16 (4k + wave) + lane / 4 and
  // LDS slot lane % 4, which holds the row's piece (lane % 4) ^ ((r / 4) % 4)
  const uint16_t* src[4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = 16 * (4 * k + wave) + (lane >> 2);
    const int piece = (lane & 3) ^ ((r >> 2) & 3);
    src[k] = arow[k] + 8 * piece;
    src[2 + k] = wrow[k] + 8 * piece;
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (kt % kTileStages) * (kTileStageElems * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      global_load_lds16(src[k] + kt * kTileK, st + (4 * k + wave) * 1024);
      global_load_lds16(src[2 + k] + kt * kTileK, st + kTileRows * kTileK * 2 + (4 * k + wave) * 1024);
    }
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int nk = K / kTileK;
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  const int sw = (c32 >> 2) & 3;  // (row / 4) % 4 of every operand row this lane reads
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads of stage kt are done when at most the later stages'
    // (four loads each) are outstanding
    const int ahead = min(nk - 1 - kt, 2);
    if (ahead == 2)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (ahead == 1)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // every thread's stage kt is in LDS, and every wave is done with stage
    // kt - 1, whose slot the next issue refills
    __syncthreads();
    if (kt + 3 < nk) issue(kt + 3);
    const uint16_t* sA = smem + (kt % kTileStages) * kTileStageElems;
    const uint16_t* sW = sA + kTileRows * kTileK;
#pragma unroll
    for (int kc = 0; kc < kTileK / 16; ++kc) {
      const int slot = (2 * kc + grp) ^ sw;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (64 * wm + 32 * i + c32) * kTileK + 8 * slot);
        b[i] = *reinterpret_cast<const bf16x8*>(sW + (64 * wn + 32 * i + c32) * kTileK + 8 * slot);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
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
