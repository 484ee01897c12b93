// Host-side launchers of the MTLA kernels (called by the C-ABI layer only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtla {

struct MergeArgs {
  int B, T, d_c, d_r, s, max_slots, pe_rows;
  const int32_t* pos0;  // [B] or nullptr (= 1 for every sequence)
  const void* c;        // [B, T, d_c]
  const void* k_r;      // [B, T, d_r]
  const float* w_hyp;   // [d_c], or [s, d_c] (wh_stride = d_c)
  const float* pe;      // [pe_rows, d_c]
  void* cache;          // [B, max_slots, W]
  float* open_acc;      // [B, 2, W]: state after token t at [b, t % 2]
  float* gate_out;      // [B, T] or nullptr
  void* partials;       // [B, T, W] cumulative in-block merges, or nullptr
  int p0_all = 1;       // first appended token of every sequence when pos0 is nullptr
  int wh_stride = 0;    // token t takes W_hyp row (t - 1) mod s at w_hyp + row * wh_stride
};

// Gate + temporal merge.  dtype: 0 fp32, 1 bf16.
hipError_t launch_merge(const MergeArgs& a, int dtype, hipStream_t st);

// Beam reorder of the decode state (out of place): destination b takes the
// slots 1..ceil(pos[src[b]]/s), both open-slot rows and the token count of
// sequence src[b].
struct ReorderArgs {
  int B, s, max_slots;
  int row_bytes;         // bytes of one cache row, (d_c + d_r) * element size
  int open_floats;       // floats of one sequence's open-slot state (2 * W)
  const int32_t* src;    // [B]
  const int32_t* pos;    // [B] tokens held by each sequence before the reorder
  const void* cache_in;  // [B, max_slots, W]
  void* cache_out;
  const float* open_in;  // [B, 2, W]
  float* open_out;
  int32_t* pos_out;      // [B] or nullptr
};
hipError_t launch_reorder(const ReorderArgs& a, hipStream_t st);

// Layer projections: one NT GEMM C[m, n] = sum_k A[m, k] Wt[n, k], with the
// weight rows Wt = [w0 (n0 rows) ; w1 (n1 rows) ; w2 (the rest)].
//   mode 0: out [M, N] row-major (the output projection).
//   mode 1: the input projection; rows m = (b, t) of B sequences of T tokens,
//           columns [c (d_c) | per head q^C (d_h), q^R (d_r) | k^R (d_r)],
//           q^R and k^R rotated at position pos0[b] + t - 1 (p0_all when
//           pos0 is null).
struct LayerGemmArgs {
  int M, N, K;
  const void* A;
  const void* w0;
  int n0;
  const void* w1;
  int n1;
  const void* w2;
  int mode;
  void* out;
  int T, H, d_h, d_r, d_c;
  const int32_t* pos0;
  int p0_all;
  void* c;
  void* k_r;
  void* q_c;
  void* q_r;
  int lda = 0;          // row stride of A in elements (0: K)
  int out_f32 = 0;      // mode 0: out is fp32 whatever the storage type
  int vec8 = 0;         // set by the launcher: every 8-column chunk of a row has one 16-byte-aligned destination
};
hipError_t launch_layer_gemm(const LayerGemmArgs& g, int dtype, hipStream_t st);

// Training backward of the parallel pass.  Rows r = b * N + t (token t,
// 0-based, of sequence b); R = B * N; QW = d_h + d_r; KV2 = 2 * H * d_h.
struct BwdArgs {
  int B, N, H, d_h, d_c, d_r, s;
  float scale;
  const void* q_c;    // [B, N, H, d_h]
  const void* q_r;    // [B, N, H, d_r]
  const void* c;      // [R, d_c]
  const void* k_r;    // [R, d_r]
  const float* w_hyp; // [d_c], or [s, d_c] (wh_stride = d_c): token t (0-based) takes row t mod s
  const float* pe;    // [>= N, d_c], row t for token t
  const void* d_o;    // [B, N, H, d_h]
  void* P;            // [R, d_c + d_r] partial merges (written by the partials kernel)
  float* gate;        // [R]
  const void* KV;     // [R, KV2]: K^C of (h, e) at column h d_h + e, V at H d_h + h d_h + e
  float* lse;         // [B, H, N] softmax normaliser of each query (log2 domain on the MFMA path)
  float* D;           // [B, H, N] sum_j p_ij (dO_i . V_j) = dO_i . o_i
  void* dKV;          // [R, KV2 + H d_r]: dK^C, dV as KV, then dK^R of (h, r) at KV2 + h d_r + r
  const float* dPc;   // [R, d_c] fp32: gradient of P^c through the up-projection
  void* g_q_c;        // gradients written: [B, N, H, d_h], [B, N, H, d_r], [R, d_c], [R, d_r]
  void* g_q_r;
  void* g_c;
  void* g_k_r;
  float* du;          // [R] gradient of each token's gate pre-activation u = W_hyp . (c + pe)
  float* wh_part;     // [wh_parts, wh_rows, d_c] fp32 partial sums of dW_hyp over row chunks
  int wh_parts;
  int wh_stride;      // 0 (one W_hyp row) or d_c (one row per place in the block)
  int wh_rows;        // W_hyp rows: 1, or s
  // MFMA path (bf16, d_h = 64, d_r = 32): K^C and V in the forward's layout,
  // and lse in the log2 domain (scores scaled by tau log2 e)
  const void* kc;     // [B, H, N, d_h] K^C of every token
  const void* v;      // [B, H, N, d_h] V of every token
  float* pd;          // [B, H, N] p_ii, the diagonal key's probability
  float* dsd;         // [B, H, N] ds_ii
  int nqt;            // query tiles per (sequence, head), set at launch
};
bool bwd_mfma_supported(int d_h, int d_r);
hipError_t launch_bwd_attention_mfma(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_partials(const BwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_bwd_attention(const BwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_bwd_scan(const BwdArgs& a, int dtype, hipStream_t st);
// Wt[n, k] = stacked [W_UK ; W_UV] ([KV2, d_c]) transposed: [d_c, KV2].
hipError_t launch_bwd_transpose_w(int KV2h, int d_c, const void* w_uk, const void* w_uv, void* wt, int dtype,
                                  hipStream_t st);
// out[m, n] = sum over rows r of A[r, m] Bm[r, n] (m < M, n < N), rows split
// into `splits` chunks whose fp32 partial products go to part[split, M, N];
// then out = the fixed-order sum of the partials.
hipError_t launch_bwd_wgrad(int R, int M, int N, const void* A, int lda, const void* Bm, int ldb, float* part,
                            int splits, float* out0, int m0_rows, float* out1, int dtype, hipStream_t st);
// Workgroup tiles of launch_bwd_wgrad's product for (M, N): it runs on MFMA
// (128 x 128 tiles) for bf16 with M and N multiples of 128.
int bwd_wgrad_tiles(int M, int N, int dtype);
// dW_hyp = sum over rows r of du[r] (c_r + pe_t(r)), through wh_parts row-chunk partials.
hipError_t launch_bwd_dwhyp(const BwdArgs& a, float* out, int dtype, hipStream_t st);
// out[i] = sum_{p < parts} part[p * n + i], in order of p.
hipError_t launch_sum_parts(const float* part, int parts, int n, float* out, hipStream_t st);

hipError_t launch_sinusoidal_pe(int rows, int d, float* pe, hipStream_t st);
hipError_t launch_debug_mask(int n, int s, uint8_t* mask, hipStream_t st);
hipError_t launch_debug_limits(int n, int s, int32_t* hi, hipStream_t st);

// Absorbed query rows: qbuf[r, h, :] = [W_UK[h]^T q_c[r, h] ; q_r[r, h]] (fp32).
hipError_t launch_absorb(int R, int H, int d_h, int d_c, int d_r, const void* q_c,
                         const void* q_r, const void* w_uk, float* qbuf, int dtype,
                         hipStream_t st);

// One-token merge (m.T == 1, bf16) and the absorbed query rows of the same
// B = m.B sequences in one launch: the same results as launch_merge followed
// by launch_absorb.  Only where merge_absorb_supported().
bool merge_absorb_supported(int d_h, int d_c, int dtype);
hipError_t launch_merge_absorb(const MergeArgs& m, int H, int d_h, int d_r, const void* q_c,
                               const void* q_r, const void* w_uk, float* qbuf, hipStream_t st);

// Split partials: m, l [R, splits, H], acc [R, splits, H, d_c] (fp32).
struct Partials {
  float* m;
  float* l;
  float* acc;
};

struct AttendArgs {
  int R;          // query rows (decode: B; prefill: B * N)
  int N;          // prefill tokens per sequence (0 for decode)
  int H, d_c, d_r, s, max_slots, splits;
  float scale;
  const int32_t* pos;   // decode positions [B] (decode only)
  const float* qbuf;    // [R, H, W]
  const void* cache;    // [B, max_slots, W]
  const void* diag;     // prefill: partial merges [B, N, W]; decode: nullptr
  Partials part;
  float* o_lat;         // [R, H, d_c] output (fp32)
  int t0 = 0;           // prefill: tokens already in the cache (queries are t0+1 ..)
};

// Vector-ALU split attention + split merge (any shape, fp32 or bf16 storage).
hipError_t launch_attend_portable(const AttendArgs& a, int dtype, hipStream_t st);

// MFMA latent attention for decode (bf16 storage); a split-merge kernel
// follows when splits > 1 and merge_splits (otherwise the caller merges the
// partials, see launch_combine_up_project).  Returns hipErrorNotSupported when no instantiation covers
// (H, d_c, d_r).
bool decode_mfma_supported(int H, int d_c, int d_r);
hipError_t launch_decode_mfma(const AttendArgs& a, hipStream_t st, bool merge_splits = true);

// The split merge of the attention's partials and the up-projection in one
// launch: the same out as split_merge_kernel (o_lat) followed by
// launch_up_project, without writing o_lat.  Only where
// combine_up_project_supported() (bf16, 2..8 splits).
bool combine_up_project_supported(int d_h, int d_c, int splits, int dtype);
hipError_t launch_combine_up_project(int R, int H, int d_h, int d_c, int splits, const Partials& p,
                                     const void* w_uv, void* out, hipStream_t st);

// Fused one-token decode step (bf16, short caches): optional merge of the
// token, absorb, latent attention and up-projection in one kernel, one
// workgroup per sequence.
struct StepArgs {
  int B, H, d_h, d_c, d_r, s, max_slots, pe_rows, merge;
  int groups;             // head groups per sequence requested (0: launch_decode_step chooses)
  float scale;
  const int32_t* pos;     // [B]
  const uint16_t* c;      // [B, d_c]  token to merge (merge only)
  const uint16_t* k_r;    // [B, d_r]
  const float* w_hyp;     // [d_c]
  const float* pe;        // [pe_rows, d_c]
  const uint16_t* q_c;    // [B, H, d_h]
  const uint16_t* q_r;    // [B, H, d_r]
  const uint16_t* w_uk;   // [H, d_h, d_c]
  const uint16_t* w_uv;   // [H, d_h, d_c]
  uint16_t* cache;        // [B, max_slots, W]
  float* open_acc;        // [B, 2, W]: state after token t at [b, t % 2]
  uint16_t* out;          // [B, H, d_h]
  int wh_stride = 0;      // d_c: W_hyp has one row per place in the block (256-wide latents only)
  // W_UV in tile order (launch_pack_w_uv_tiles), or null: the 256-wide fused
  // step then reads it as whole lines (same values, same bits)
  const uint16_t* w_uv_tiles = nullptr;
  // Timeline instance of the 256-wide fused step (measurement only): each
  // workgroup writes kStepTimelineSlots real-time counter readings, or null.
  unsigned long long* timeline = nullptr;
};
// Readings per workgroup of the fused step's timeline instance: 0 entry,
// 1 position known, 2 absorb partial sums formed, 3 scaled q~ in LDS,
// 4 + w wave w's attention done (w < 8), 12 o_lat in LDS, 13 output stored.
constexpr int kStepTimelineSlots = 16;
bool decode_step_supported(int H, int d_h, int d_c, int d_r);
// Head groups per sequence the step kernel uses for a batch of B sequences
// (`requested` when it is a valid group count, else the launcher's choice).
int decode_step_groups(int B, int H, int d_h, int d_c, int requested);
hipError_t launch_decode_step(const StepArgs& a, hipStream_t st);
// W_UV [H, d_h, d_c] (bf16, d_c a multiple of 32) in the fused step's tile
// order: for head h, 16-row tile t and 32-column step ks, a 1 KB block whose
// 16-byte piece q holds row 16 t + q % 16, columns 32 ks + 8 (q / 16) .. +7
// (rows past d_h zero): [H, ceil(d_h / 16), d_c / 32, 64, 8] elements.
size_t w_uv_tiles_elems(int H, int d_h, int d_c);
hipError_t launch_pack_w_uv_tiles(int H, int d_h, int d_c, const uint16_t* w_uv, uint16_t* tiles, hipStream_t st);

// out[r, h, :] = W_UV[h] o_lat[r, h].
hipError_t launch_up_project(int R, int H, int d_h, int d_c, const float* o_lat, const void* w_uv,
                             void* out, int dtype, hipStream_t st);

// Prefill MFMA path (bf16): up-projection GEMM and stride-masked attention.
bool prefill_mfma_supported(int H, int d_h, int d_c, int d_r);
// K^C and V of n_rows rows of a [.., W] bf16 array per sequence: output row j
// of sequence b takes input row b*a_seq_rows + a_mul*j + a_add.  Written
// [B, H, n_rows, d_h] in fp16 (out_fp16: the forward attention's operands)
// or bf16 (the training backward's).  B*a_seq_rows*W*2 must stay below 2^31.
hipError_t launch_prefill_kv(int B, int n_rows, int a_seq_rows, int a_mul, int a_add, int H, int d_h, int d_c,
                            int d_r, const void* a, const void* w_uk, const void* w_uv, void* k_out, void* v_out,
                            bool out_fp16, hipStream_t st);

struct PrefillAttnArgs {
  int B, N, H, d_h, d_c, d_r, s;
  int nqt;               // query tiles per (sequence, head) (set at launch)
  float scale;
  const void* q_c;       // [B, N, H, d_h]
  const void* q_r;       // [B, N, H, d_r]
  const void* partials;  // [B, N, W]: P_i of each query, its diagonal key
  const void* w_uk;      // [H, d_h, d_c]: the diagonal's K^C = W_UK P^c_i ...
  const void* w_uv;      // [H, d_h, d_c]: ... and V = W_UV P^c_i, formed in the kernel
  void* out;             // [B, N, H, d_h]
  int t0;                // the queries are tokens t0+1 .. t0+N
  // completed slot j (0-based): K^C and V at row j of kslot / vslot ([B, H,
  // slot_rows, d_h] fp16); the rope key at row rslot_mul*j + rslot_add of
  // rslot ([B, rslot_rows, W], last d_r columns)
  const void* kslot;
  const void* vslot;
  int slot_rows;
  const void* rslot;
  int rslot_rows, rslot_mul, rslot_add;
};
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t st);

// Measurement kernels (calib.hip): streaming read of `bytes` (a multiple of
// 16) by `workgroups` workgroups of 256 threads, one word per wave into sink;
// MFMA chains on registers (`workgroups` x 4 waves, `iters` rounds of four
// 32x32x16 products), one float per thread into out; an empty kernel.
hipError_t launch_calib_read(const void* src, size_t bytes, int workgroups, uint32_t* sink, hipStream_t st);
hipError_t launch_calib_mfma(bool f16, int workgroups, int iters, float* out, hipStream_t st);
double calib_mfma_flops(int workgroups, int iters);
hipError_t launch_calib_empty(hipStream_t st);
// A compute unit's cost of one 16-byte-per-lane load instruction: pattern 0
// contiguous kilobytes, 1 sixteen rows of 64 bytes; one workgroup per unit,
// per-workgroup s_memtime cycles of 8 waves x 32 loads into cycles.
hipError_t launch_calib_load_pattern(int pattern, int workgroups, const void* buf, size_t bytes, uint32_t* cycles,
                                     hipStream_t st);
hipError_t launch_calib_tile_stream(const void* rows, int seqs, int rows_per_seq, int splits, bool interleave,
                                    bool nt, uint32_t* sink, hipStream_t st);

}  // namespace mtla
