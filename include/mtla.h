/*
 * mtla.h - C ABI of the MI355X (gfx950) Multi-head Temporal Latent Attention
 * hot path: hyper-network merge into a temporally compressed latent cache,
 * absorbed-form decode over that cache, and parallel prefill under the
 * stride-aware causal mask.
 *
 * Sources (cited by page title and section):
 *   "Multi-head Temporal Latent Attention" (wiki summary of the NeurIPS 2025
 *   paper): Key claims (paper Sec. 4.1 Eq. 13, Sec. 4.2 Fig. 2(c), Sec. 4.3
 *   Eq. 17, Sec. 6.1) and Method (1)-(3).
 *   "Multi-Head Latent Attention and Sparse Indexers": "Latent attention
 *   changes the representation" (absorption algebra).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Indexing: tokens t are 1-based; token t belongs to cache slot ceil(t/s)
 *   (1-based), stored at row ceil(t/s)-1.  The first token of a block
 *   ((t-1) mod s == 0) overwrites its slot, later tokens of the block add to
 *   it, so a cache never needs clearing.
 * Memory: every tensor argument is a caller-owned DEVICE pointer to a dense,
 *   row-major array (innermost dimension last, no strides).  Tensors the
 *   kernels move in 16-byte vectors (cache, open_acc, c, k_r, q_c, q_r,
 *   w_uk, w_uv, out and the workspace) must start 16-byte aligned; the
 *   others need only their element alignment (pos, pos0, w_hyp, pe,
 *   gate_out, q_lat, o_lat: 4 bytes).  The library never allocates, frees or synchronises;
 *   `stream` is a hipStream_t (NULL = the default stream) and every call only
 *   enqueues work on it.
 * dtypes: `dims->dtype` is the storage type of c, k_r, q_c, q_r, w_uk, w_uv,
 *   the cache and the outputs (fp32 or bf16, round-to-nearest-even).  w_hyp,
 *   pe and open_acc are always fp32.  Accumulation is always fp32.
 * Open-slot state: open_acc is [B, 2, d_c + d_r] fp32.  The unrounded fp32
 *   value of the open slot after token t is kept at open_acc[b, t % 2]; a call
 *   that continues a block at token t reads open_acc[b, (t-1) % 2].  (Keeping
 *   the state by token parity lets the several workgroups that decode one
 *   sequence in mtla_decode_step read the old state while one of them writes
 *   the new one.)  Only the half for the last token a call appends is
 *   written; the other half is left as it was.
 * Errors: all argument checks run before anything is enqueued; on a failed
 *   check the call returns a negative mtla_status, enqueues nothing, and
 *   mtla_last_error() describes the failure.  A kernel launch failure returns
 *   MTLA_ERR_HIP.  batch == 0 or a zero token count is a no-op returning
 *   MTLA_OK.  Positions read from device memory cannot be checked on the
 *   host: a sequence whose position is out of range (t < 1, ceil(t/s) >
 *   max_slots, or t > pe_rows) is skipped by the merge (nothing written), and
 *   its decode output is NaN.
 * Threads: calls are stateless and may be made from several host threads;
 *   calls that write the same cache concurrently race.
 */
#ifndef MTLA_H
#define MTLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTLA_OK = 0,
  MTLA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or shape   */
  MTLA_ERR_UNSUPPORTED = -2, /* valid but outside the supported dimensions   */
  MTLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  MTLA_ERR_HIP = -4          /* the HIP runtime reported a launch failure    */
} mtla_status;

typedef enum { MTLA_FP32 = 0, MTLA_BF16 = 1 } mtla_dtype;

/* Force the portable (vector-ALU) kernels even where the MFMA kernels apply. */
#define MTLA_FLAG_PORTABLE 1
/* Per-position gate: W_hyp has s rows ([stride_s, d_c] fp32, and so has
 * grad_w_hyp) and token t takes row (t-1) mod s, its place in its block:
 *   w_t = sigmoid(W_hyp[(t-1) mod s] . (c_t + pe_t)).
 * The reading of "Multi-head Temporal Latent Attention", Method (1), in which
 * the hyper-network's linear layer outputs the merge weights W_t in R^s. */
#define MTLA_FLAG_GATE_PER_POSITION 2

/* Supported dimensions: d_c and d_r multiples of 8, d_c + d_r <= 1024,
 * d_h <= 256, s <= 256 (MTLA_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int32_t batch;       /* B: sequences                                          */
  int32_t heads;       /* H: attention heads                                    */
  int32_t d_h;         /* per-head content width of queries/values              */
  int32_t d_c;         /* latent width (cached)                                 */
  int32_t d_r;         /* decoupled-RoPE key width (cached beside the latent)   */
  int32_t stride_s;    /* s: tokens merged into one cache slot                  */
  int32_t max_slots;   /* cache rows per sequence                               */
  int32_t dtype;       /* mtla_dtype of stored tensors                          */
  float softmax_scale; /* tau applied to scores; 1/sqrt(d_h + d_r) is usual     */
  int32_t flags;       /* 0, or MTLA_FLAG_PORTABLE | MTLA_FLAG_GATE_PER_POSITION */
  /* Launch choices; 0 (the usual value) lets the library choose.
   * decode_splits: 1..64 slot splits of the decode's latent attention
   *   (clamped to the kernel's limit for max_slots); it must be the same when
   *   the decode workspace is sized and when decode runs.  Values outside
   *   0..64 are MTLA_ERR_INVALID_ARG.
   * step_groups: head groups per sequence of the one-kernel decode step; used
   *   when it divides heads and the step kernel has an instance for
   *   heads / step_groups heads per group, otherwise the library chooses.
   *   Negative values are MTLA_ERR_INVALID_ARG.  Neither changes a result
   *   beyond the order of fp32 sums. */
  int32_t decode_splits;
  int32_t step_groups;
} mtla_dims;

/* Row width of the cache: W = d_c + d_r elements. */

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t mtla_version(void);

/* Static text for a status code. */
const char* mtla_status_string(int32_t status);

/* Text of the last failure of a call made from this host thread ("" if none). */
const char* mtla_last_error(void);

/*
 * Sinusoidal positional-embedding table for the merge gate.
 *   pe[p, 2k] = sin(p * 10000^(-2k/d)), pe[p, 2k+1] = cos(same), p = 0..rows-1
 * (row p is used for token t = p+1).  Computed in double, stored fp32.
 * Page: "Multi-head Temporal Latent Attention", Key claims (paper Sec. 4.1):
 * the hyper-network is conditioned on the latent plus a positional embedding.
 *   pe: device [rows, d] fp32, written.  rows >= 1, d >= 1.
 */
int32_t mtla_sinusoidal_pe(int32_t rows, int32_t d, float* pe, void* stream);

/*
 * Merge / append (gate + temporal merge) for n_tokens consecutive tokens of
 * every sequence.  Page: "Multi-head Temporal Latent Attention", Key claims
 * (paper Sec. 4.1 Eq. 13) and Method (1):
 *   w_t = sigmoid(W_hyp . (c_t + pe_t))              (one scalar per token)
 *   slot ceil(t/s) <- (t opens a block ? 0 : open slot) + w_t [c_t ; k^R_t]
 * Sequence b appends tokens t = pos0[b] .. pos0[b] + n_tokens - 1.
 *   pos0     device [B] int32, 1-based position of the first appended token.
 *   c        device [B, n_tokens, d_c]   storage dtype.
 *   k_r      device [B, n_tokens, d_r]   storage dtype, RoPE already applied.
 *   w_hyp    device [d_c] fp32 ([s, d_c] with MTLA_FLAG_GATE_PER_POSITION).
 *   pe       device [pe_rows, d_c] fp32; row t-1 is used for token t.
 *   cache    device [B, max_slots, d_c + d_r] storage dtype, in/out: every
 *            slot touched by the appended tokens is written (rounded once from
 *            the fp32 sum); other rows are untouched.
 *   open_acc device [B, 2, d_c + d_r] fp32, in/out: open-slot state (see
 *            the conventions above): [b, (pos0[b]-1) % 2] is read only when
 *            pos0[b] continues a block; [b, t_last % 2] is written, t_last =
 *            pos0[b] + n_tokens - 1.
 *   gate_out device [B, n_tokens] fp32 or NULL: the gates w_t.
 */
int32_t mtla_merge_append(const mtla_dims* dims, const int32_t* pos0, int32_t n_tokens,
                          const void* c, const void* k_r, const float* w_hyp,
                          const float* pe, int32_t pe_rows, void* cache, float* open_acc,
                          float* gate_out, void* stream);

/* Bytes of workspace mtla_decode needs for these dims (written to *bytes). */
int32_t mtla_decode_workspace_bytes(const mtla_dims* dims, size_t* bytes);

/*
 * Absorbed-form decode of one query per sequence over slots 1..ceil(pos/s).
 * Pages: "Multi-head Temporal Latent Attention", Method (W_UK absorbed into
 * the query, W_UV applied after the weighted latent sum; per-token cost
 * O(N/s), Key claims Sec. 6.1); "Multi-Head Latent Attention and Sparse
 * Indexers", "Latent attention changes the representation".
 *   q~_h  = W_UK[h]^T q^C_h                                   (d_h -> d_c)
 *   z_h,j = tau (q~_h . S^c_j + q^R_h . S^R_j),  j = 1..ceil(pos/s)
 *   o_h   = W_UV[h] sum_j softmax_j(z_h)_j S^c_j
 *   pos   device [B] int32: the current token t of each sequence (its slot
 *         must already hold token t, i.e. merge first).
 *   q_c   device [B, H, d_h];  q_r device [B, H, d_r] (rotated).
 *   w_uk, w_uv device [H, d_h, d_c].
 *   cache device [B, max_slots, d_c + d_r], read only.
 *   out   device [B, H, d_h], written.
 *   workspace device, >= mtla_decode_workspace_bytes(); contents undefined
 *         after the call.
 * The result is bit-reproducible: split partials are combined in a fixed
 * order.
 */
int32_t mtla_decode(const mtla_dims* dims, const int32_t* pos, const void* q_c,
                    const void* q_r, const void* w_uk, const void* w_uv, const void* cache,
                    void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Host-only query of how mtla_decode / mtla_decode_step will run for these
 * dims: *splits = slot splits of the latent attention, *fused = 1 when one
 * kernel (one workgroup per sequence) does the whole step.
 */
int32_t mtla_decode_plan(const mtla_dims* dims, int32_t* splits, int32_t* fused);

/*
 * One decode step: merge token pos[b] (mtla_merge_append with n_tokens = 1)
 * and decode it (mtla_decode), in one call.  Same arguments as those two
 * calls: c [B, d_c], k_r [B, d_r] are the token's latent and rotated rope
 * key; everything else as above (workspace: mtla_decode_workspace_bytes()).
 * Page: "Multi-head Temporal Latent Attention", Method (1): during inference
 * each step updates the open slot (or opens a new one) and attends
 * ceil(t/s) slots.  For a short cache (one split) with bf16 storage this is
 * a single kernel with one workgroup per (sequence, group of heads) (with
 * MTLA_FLAG_GATE_PER_POSITION and d_c other than 256 the merge runs first,
 * as its own kernel); the open-slot state is read at [b, (pos[b]-1) % 2] and
 * written at [b, pos[b] % 2].
 */
int32_t mtla_decode_step(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                         const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                         const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                         float* open_acc, void* out, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * mtla_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The same work and the same results (bit
 * for bit) as mtla_decode_step; the workspace is a static device array of
 * MTLA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  No call allocates or frees memory.
 *   Arguments: those of mtla_decode_step without workspace and ws_bytes.
 *   Limit: dims whose mtla_decode_workspace_bytes() exceeds
 *     MTLA_NOALLOC_SCRATCH_BYTES are rejected with MTLA_ERR_WORKSPACE
 *     before anything is enqueued (the LLM-scale step, B=64, H=32, d_c=512,
 *     d_r=64, needs about 26 MB).
 *   Sharing: every call on one GPU uses that GPU's one array, and the array
 *     keeps the last call's contents (no call needs it to start at zero:
 *     each call writes everything it reads).  Calls that overlap on one GPU
 *     (concurrent streams, or host threads) race on it; serialise them.
 *   The stream must belong to the current device; the array's device address
 *     is resolved once per device, on the first call made with it current.
 */
#define MTLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t mtla_decode_step_noalloc(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                                 const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                                 const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                                 float* open_acc, void* out, void* stream);

/*
 * W_UV in the order in which the fused decode step's up-projection reads
 * it, for callers that run many decode steps with the same weights (the
 * up-projection of "Multi-head Temporal Latent Attention", Method (3),
 * unchanged: the same values in another order).  For head h, 16-row tile t
 * (rows 16t .. 16t+15 of W_UV[h]) and 32-column step ks, one 1,024-byte
 * block whose 16-byte piece q (0..63) holds row 16t + q % 16, columns
 * 32 ks + 8 (q / 16) .. +7; rows past d_h are zero.  Loaded in this order,
 * every load instruction of the up-projection reads whole 128-byte lines.
 *   mtla_w_uv_tiles_bytes: *bytes = H * ceil(d_h/16) * 16 * d_c * 2.
 *   mtla_pack_w_uv_tiles: w_uv device [H, d_h, d_c] bf16, 16-byte aligned;
 *     w_uv_tiles device, >= mtla_w_uv_tiles_bytes bytes, 16-byte aligned,
 *     written (enqueued on stream).
 * bf16 only, d_c a multiple of 32 (MTLA_ERR_UNSUPPORTED otherwise).
 */
int32_t mtla_w_uv_tiles_bytes(const mtla_dims* dims, size_t* bytes);
int32_t mtla_pack_w_uv_tiles(const mtla_dims* dims, const void* w_uv, void* w_uv_tiles, void* stream);

/*
 * mtla_decode_step with W_UV also given in tile order (mtla_pack_w_uv_tiles
 * of the same w_uv): the same outputs, cache rows and open-slot state, bit
 * for bit.  The fused step kernel of 256-wide latents reads w_uv_tiles; the
 * other paths read w_uv.  Arguments and errors as for mtla_decode_step, and
 * the checks of mtla_pack_w_uv_tiles on w_uv_tiles.
 */
int32_t mtla_decode_step_tiles(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                               const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                               const void* q_r, const void* w_uk, const void* w_uv, const void* w_uv_tiles,
                               void* cache, float* open_acc, void* out, void* workspace, size_t ws_bytes,
                               void* stream);

/*
 * Staged form of mtla_decode, for callers that fuse the two projections into
 * their own GEMMs (mtla_decode runs exactly these three stages).
 *
 * mtla_absorb_query: q_lat[r, h] = [W_UK[h]^T q^C[r, h] ; q^R[r, h]], fp32.
 * Pages: "Multi-head Temporal Latent Attention", Method (W_UK absorbed into
 * the query); "Multi-Head Latent Attention and Sparse Indexers", "Latent
 * attention changes the representation" (q^T (U_K c) = (U_K^T q)^T c).
 *   q_c device [n_rows, H, d_h], q_r device [n_rows, H, d_r] (storage dtype);
 *   w_uk device [H, d_h, d_c]; q_lat device [n_rows, H, d_c + d_r] fp32, written.
 */
int32_t mtla_absorb_query(const mtla_dims* dims, int32_t n_rows, const void* q_c, const void* q_r,
                          const void* w_uk, float* q_lat, void* stream);

/* Bytes of workspace mtla_decode_attention needs. */
int32_t mtla_decode_attention_workspace_bytes(const mtla_dims* dims, size_t* bytes);

/*
 * Latent-space attention of one absorbed query per sequence over slots
 * 1..ceil(pos/s):  o_lat[b, h] = sum_j softmax_j(tau q_lat[b, h] . S_j) S^c_j.
 * Page: "Multi-head Temporal Latent Attention", Method and Key claims
 * (Sec. 6.1: a query at step t reads ceil(t/s) slots).
 * With bf16 storage and a supported shape it runs an MFMA split-K kernel over
 * the slots (one split, hence one kernel, for caches up to ~512 slots; more
 * splits, merged in a fixed order by a second kernel, for longer ones).
 *   pos   device [B] int32; q_lat device [B, H, d_c + d_r] fp32;
 *   cache device [B, max_slots, d_c + d_r]; o_lat device [B, H, d_c] fp32,
 *   written.
 *   workspace device, >= mtla_decode_attention_workspace_bytes(); scratch.
 */
int32_t mtla_decode_attention(const mtla_dims* dims, const int32_t* pos, const float* q_lat,
                              const void* cache, float* o_lat, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * mtla_up_project: out[r, h] = W_UV[h] o_lat[r, h] (rounded to storage).
 * Page: "Multi-Head Latent Attention and Sparse Indexers", "Latent attention
 * changes the representation" (sum_j a_j U_V c_j = U_V sum_j a_j c_j).
 *   o_lat device [n_rows, H, d_c] fp32; w_uv device [H, d_h, d_c];
 *   out device [n_rows, H, d_h], written.
 */
int32_t mtla_up_project(const mtla_dims* dims, int32_t n_rows, const float* o_lat,
                        const void* w_uv, void* out, void* stream);

/* Bytes of workspace mtla_prefill needs for n_tokens tokens. */
int32_t mtla_prefill_workspace_bytes(const mtla_dims* dims, int32_t n_tokens, size_t* bytes);

/*
 * Parallel prefill of tokens 1..n_tokens of every sequence under the
 * stride-aware causal mask.  Page: "Multi-head Temporal Latent Attention",
 * Key claims (paper Sec. 4.2 Fig. 2(c); Sec. 4.3 Eq. 17) and Method (2)-(3):
 *   P_j = sum_{k = s*floor((j-1)/s)+1}^{j} w_k x_k   (cumulative in-block merges)
 *   query i attends key j iff j == i, or s | j and j/s < ceil(i/s);
 *   K^C_j,h = W_UK[h] P^c_j,  V_j,h = W_UV[h] P^c_j,  rope key P^R_j;
 *   o_i,h = sum_j softmax_j(tau (q^C_i,h . K^C_j,h + q^R_i,h . P^R_j)) V_j,h.
 * Its output equals token-by-token decoding (merge then decode per token).
 *   q_c device [B, N, H, d_h]; q_r device [B, N, H, d_r].
 *   c   device [B, N, d_c];    k_r device [B, N, d_r].
 *   w_hyp, pe, pe_rows: as for mtla_merge_append (pe_rows >= N).
 *   w_uk, w_uv device [H, d_h, d_c].
 *   cache device [B, max_slots, d_c + d_r], written: slots 1..ceil(N/s).
 *   open_acc device [B, 2, d_c + d_r] fp32: [b, N % 2] is written with the
 *         fp32 value of slot ceil(N/s), so that decoding can continue at
 *         token N+1.
 *   out device [B, N, H, d_h], written.
 *   N <= s * max_slots.
 */
int32_t mtla_prefill(const mtla_dims* dims, int32_t n_tokens, const void* q_c, const void* q_r,
                     const void* c, const void* k_r, const float* w_hyp, const float* pe,
                     int32_t pe_rows, const void* w_uk, const void* w_uv, void* cache,
                     float* open_acc, void* out, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * Staged form of mtla_prefill (tokens 1..n_tokens, bf16 storage, a shape with
 * the MFMA path: d_h 64 with d_r 32 or d_h 128 with d_r 64, d_c a multiple
 * of 32, heads * d_h a multiple of 128; otherwise MTLA_ERR_UNSUPPORTED), for
 * callers that want the intermediate tensors or time the stages apart.
 * mtla_prefill runs exactly these three calls.  Page: "Multi-head Temporal
 * Latent Attention", Key claims (paper Sec. 4.2 Fig. 2(c), Sec. 4.3 Eq. 17)
 * and Method (2)-(3).
 * mtla_prefill_partials: gates and cumulative in-block partial merges
 *     P_j = sum_{k = s*floor((j-1)/s)+1}^{j} w_k x_k   (j = 1..n_tokens)
 *   partials device [B, n_tokens, d_c + d_r] storage dtype, written (each
 *   value rounded once from its fp32 sum); cache and open_acc written as
 *   mtla_prefill leaves them; the other arguments as for mtla_prefill.
 * mtla_prefill_keys: K^C_b,h = W_UK[h] P^c_{s*b} and V_b,h = W_UV[h] P^c_{s*b}
 *   of the completed slots b = 1 .. n_keys that some query of the call
 *   attends, n_keys = floor((n_tokens - 1) / s) (0 for n_tokens = 0):
 *   k_c, v device [B, H, n_keys, d_h] fp16 (IEEE binary16, rounded to
 *   nearest even from fp32 accumulation), written; partials read only.
 *   Nothing is launched when n_keys is 0 (k_c and v may then be NULL).
 * mtla_prefill_attention: the stride-masked attention of queries
 *   1..n_tokens (query i attends the partial merges j = i and j = s*b for
 *   b < ceil(i/s)): q_c, q_r, w_uk, w_uv as for mtla_prefill; partials and
 *   the slot keys k_c, v from the two calls above (read only); out
 *   [B, n_tokens, H, d_h], written.  Each query's own key j = i (K^C_i =
 *   W_UK[h] P^c_i, V_i = W_UV[h] P^c_i) is formed inside this call, in
 *   fp32, from partials and the weights.
 * The fp16 keys and values bound their magnitudes by 65504.
 */
int32_t mtla_prefill_partials(const mtla_dims* dims, int32_t n_tokens, const void* c, const void* k_r,
                              const float* w_hyp, const float* pe, int32_t pe_rows, void* cache, float* open_acc,
                              void* partials, void* stream);
int32_t mtla_prefill_keys(const mtla_dims* dims, int32_t n_tokens, const void* partials, const void* w_uk,
                          const void* w_uv, void* k_c, void* v, void* stream);
int32_t mtla_prefill_attention(const mtla_dims* dims, int32_t n_tokens, const void* q_c, const void* q_r,
                               const void* partials, const void* w_uk, const void* w_uv, const void* k_c,
                               const void* v, void* out, void* stream);

/* Bytes of workspace mtla_prefill_at needs for n_tokens tokens after t0. */
int32_t mtla_prefill_at_workspace_bytes(const mtla_dims* dims, int32_t t0, int32_t n_tokens,
                                        size_t* bytes);

/*
 * Chunked prefill: tokens t0+1 .. t0+n_tokens of every sequence, after t0
 * tokens already merged into `cache` and `open_acc` (by mtla_prefill,
 * mtla_prefill_at or token-by-token merges; t0 need not end a block).  Page:
 * "Multi-head Temporal Latent Attention", Key claims (paper Sec. 4.2
 * Fig. 2(c), Sec. 4.3 Eq. 17) and Method (2)-(3): the same mask and keys as
 * mtla_prefill with queries i = t0+1 .. t0+n_tokens; the block open at t0
 * continues from its fp32 state, and completed slots written before the
 * call are keys like the new ones.  The result equals token-by-token
 * decoding of the same tokens.
 *   t0 >= 0, uniform over the batch (0: the same as mtla_prefill).
 *   q_c, q_r, c, k_r, out: the new tokens only, as for mtla_prefill with
 *         N = n_tokens.
 *   pe_rows >= t0 + n_tokens; t0 + n_tokens <= s * max_slots.
 *   cache device [B, max_slots, d_c + d_r]: slots 1..ceil(t0/s) read (the
 *         last one, if open, is rewritten), slots ..ceil((t0+n_tokens)/s)
 *         written.
 *   open_acc device [B, 2, d_c + d_r] fp32: [b, t0 % 2] read when t0 is not
 *         at a block boundary; [b, (t0 + n_tokens) % 2] written.
 *   workspace device, >= mtla_prefill_at_workspace_bytes(); scratch.  On
 *         the MFMA path it holds K^C and V of the completed slots the new
 *         queries attend (floor((t0 + n_tokens - 1) / s) per sequence).
 */
int32_t mtla_prefill_at(const mtla_dims* dims, int32_t t0, int32_t n_tokens, const void* q_c,
                        const void* q_r, const void* c, const void* k_r, const float* w_hyp,
                        const float* pe, int32_t pe_rows, const void* w_uk, const void* w_uv,
                        void* cache, float* open_acc, void* out, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * Beam-search reorder of the decode state, out of place.  Page: the MTLA
 * repository summary, "Highlighted Details" (models are evaluated with
 * Fairseq-style parallel beam search: after a step every kept hypothesis b
 * continues hypothesis src[b]; a parent may be kept several times or
 * dropped).  Destination b receives
 *   cache_out[b, 0 .. ceil(pos[src[b]]/s) - 1] = cache_in[src[b], same rows]
 *   open_out[b] = open_in[src[b]]            (both parity rows)
 *   pos_out[b] = pos[src[b]]                 (when pos_out is not NULL)
 * Rows of cache_out past the copied slots are untouched.  A destination
 * whose src is outside [0, B) is left untouched.
 *   src     device [B] int32, parent index per destination.
 *   pos     device [B] int32, tokens each sequence holds before the reorder.
 *   cache_in, cache_out  device [B, max_slots, d_c + d_r] storage dtype.
 *   open_in, open_out    device [B, 2, d_c + d_r] fp32.
 *   pos_out device [B] int32 or NULL.
 * The outputs must not alias the inputs (checked for equal pointers only).
 */
int32_t mtla_reorder_state(const mtla_dims* dims, const int32_t* src, const int32_t* pos,
                           const void* cache_in, const float* open_in, void* cache_out,
                           float* open_out, int32_t* pos_out, void* stream);

/*
 * The decoder layer around the MTLA core.  Page: "Multi-head Temporal Latent
 * Attention", Method (the latent c_t = W_DKV h_t is what is merged and
 * cached; decoupled RoPE keys as in MLA), and "Multi-Head Latent Attention and
 * Sparse Indexers", "Latent attention changes the representation" (queries
 * and the output projection W_O over the heads).  Per token t of sequence b:
 *   c_t = W_DKV h_t;  [q^C_t,h ; q^R_t,h] = (W_Q h_t) split per head;
 *   k^R_t = W_R h_t;  q^R and k^R rotated by RoPE at position t-1:
 *     interleaved pairs (2k, 2k+1) turned by (t-1) * 10000^(-2k/d_r);
 *   y_t = W_O [o_t,1 ; ... ; o_t,H].
 * Weights (storage dtype, row-major): w_dkv [d_c, d_model];
 * w_q [H * (d_h + d_r), d_model] (per head the d_h query rows, then the d_r
 * rope rows); w_r [d_r, d_model]; w_o [d_model, H * d_h].
 * d_model and H * d_h must be multiples of 8, d_h even.
 *
 * mtla_project_inputs: the input projections of n_tokens consecutive tokens
 * of every sequence; row t of sequence b is token pos0[b] + t.
 *   pos0 device [B] int32 (1-based position of each sequence's first row);
 *   h device [B, n_tokens, d_model]; outputs c [B, n_tokens, d_c],
 *   k_r [B, n_tokens, d_r], q_c [B, n_tokens, H, d_h],
 *   q_r [B, n_tokens, H, d_r], written (the layouts mtla_merge_append,
 *   mtla_decode_step and mtla_prefill take).
 */
int32_t mtla_project_inputs(const mtla_dims* dims, int32_t d_model, int32_t n_tokens, const int32_t* pos0,
                            const void* h, const void* w_dkv, const void* w_q, const void* w_r, void* c,
                            void* k_r, void* q_c, void* q_r, void* stream);

/*
 * mtla_output_project: y[r] = W_O o[r] for n_rows rows.
 *   o device [n_rows, H, d_h]; w_o device [d_model, H * d_h];
 *   y device [n_rows, d_model], written.
 */
int32_t mtla_output_project(const mtla_dims* dims, int32_t d_model, int32_t n_rows, const void* o,
                            const void* w_o, void* y, void* stream);

/* Bytes of workspace mtla_layer_decode_step needs. */
int32_t mtla_layer_decode_workspace_bytes(const mtla_dims* dims, int32_t d_model, size_t* bytes);

/*
 * One decode step of the whole layer from h: input projections of token
 * pos[b] of every sequence, mtla_decode_step (merge + attention), output
 * projection.  All checks run before anything is enqueued.
 *   pos device [B] int32 as for mtla_decode_step; h device [B, d_model];
 *   y device [B, d_model], written; cache, open_acc as for mtla_decode_step;
 *   workspace device, >= mtla_layer_decode_workspace_bytes(); scratch.
 */
int32_t mtla_layer_decode_step(const mtla_dims* dims, int32_t d_model, const int32_t* pos, const void* h,
                               const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                               const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                               const void* w_uv, void* cache, float* open_acc, void* y, void* workspace,
                               size_t ws_bytes, void* stream);

/*
 * mtla_layer_decode_step with W_UV also given in tile order
 * (mtla_pack_w_uv_tiles of the same w_uv): the same y, cache rows and
 * open-slot state, bit for bit; the decode step inside is
 * mtla_decode_step_tiles.  Arguments and errors as for
 * mtla_layer_decode_step, and the checks of mtla_pack_w_uv_tiles on
 * w_uv_tiles.
 */
int32_t mtla_layer_decode_step_tiles(const mtla_dims* dims, int32_t d_model, const int32_t* pos, const void* h,
                                     const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                                     const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                                     const void* w_uv, const void* w_uv_tiles, void* cache, float* open_acc,
                                     void* y, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace mtla_layer_prefill needs. */
int32_t mtla_layer_prefill_workspace_bytes(const mtla_dims* dims, int32_t d_model, int32_t t0,
                                           int32_t n_tokens, size_t* bytes);

/*
 * The whole layer over tokens t0+1 .. t0+n_tokens of every sequence from h:
 * input projections, mtla_prefill_at (t0 = 0: mtla_prefill), output
 * projection.  All checks run before anything is enqueued.
 *   h device [B, n_tokens, d_model]; y device [B, n_tokens, d_model],
 *   written; the rest as for mtla_prefill_at.
 */
int32_t mtla_layer_prefill(const mtla_dims* dims, int32_t d_model, int32_t t0, int32_t n_tokens, const void* h,
                           const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                           const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                           const void* w_uv, void* cache, float* open_acc, void* y, void* workspace,
                           size_t ws_bytes, void* stream);

/* Bytes of workspace mtla_prefill_backward needs for n_tokens tokens. */
int32_t mtla_prefill_backward_workspace_bytes(const mtla_dims* dims, int32_t n_tokens, size_t* bytes);

/*
 * Training backward of the parallel pass that mtla_prefill computes (tokens
 * 1..n_tokens of every sequence, no cache involved).  Page: "Multi-head
 * Temporal Latent Attention", Key claims (paper Sec. 4.2 Fig. 2(c), Sec. 4.3
 * Eq. 17: training in parallel under the stride-aware mask) and Method
 * (1)-(3).  With L = sum(grad_out * o), it writes the gradients of L:
 *   p_ij = softmax_j(z_ij), dp_ij = dO_i . V_j, D_i = sum_j p_ij dp_ij,
 *   ds_ij = tau p_ij (dp_ij - D_i);
 *   grad_q_c_i = sum_j ds_ij K^C_j, grad_q_r_i = sum_j ds_ij P^R_j;
 *   dK^C_j = sum_i ds_ij q^C_i, dV_j = sum_i p_ij dO_i, dP^R_j = sum_h,i ds_ij q^R_i;
 *   dP^c_j = sum_h W_UK[h]^T dK^C_j + W_UV[h]^T dV_j;
 *   grad_w_uk[h] = sum_j dK^C_j (P^c_j)^T, grad_w_uv[h] = sum_j dV_j (P^c_j)^T;
 *   G_k = sum of dP_j over j = k .. the end of k's block (reverse in-block sum);
 *   du_k = (G_k . x_k) w_k (1 - w_k);
 *   grad_c_k = w_k G^c_k + du_k W_hyp,  grad_k_r_k = w_k G^R_k,
 *   grad_w_hyp = sum_k du_k (c_k + pe_k)  (with MTLA_FLAG_GATE_PER_POSITION,
 *   W_hyp and grad_w_hyp row r over the tokens k with (k-1) mod s = r).
 * The forward pieces it needs (gates, partial merges, K^C and V, softmax
 * normalisers) are recomputed from the inputs.
 *   q_c, q_r, c, k_r, w_hyp, pe, pe_rows, w_uk, w_uv: as for mtla_prefill.
 *   grad_out  device [B, N, H, d_h] (storage dtype): dL/do.
 *   grad_q_c  device [B, N, H, d_h], grad_q_r [B, N, H, d_r],
 *   grad_c    device [B, N, d_c],    grad_k_r [B, N, d_r] (storage dtype),
 *             written.
 *   grad_w_hyp device [d_c] ([s, d_c] per position) fp32; grad_w_uk, grad_w_uv device [H, d_h, d_c]
 *             fp32: written (not accumulated), summed over the B sequences.
 *   workspace device, >= mtla_prefill_backward_workspace_bytes(), 16-byte
 *             aligned; scratch.
 * Requires heads * d_h a multiple of 4, batch and heads <= 65535.  With
 * batch or n_tokens 0 only the weight gradients are written (as zeros).
 * All checks run before anything is enqueued.
 */
int32_t mtla_prefill_backward(const mtla_dims* dims, int32_t n_tokens, const void* q_c, const void* q_r,
                              const void* c, const void* k_r, const float* w_hyp, const float* pe,
                              int32_t pe_rows, const void* w_uk, const void* w_uv, const void* grad_out,
                              void* grad_q_c, void* grad_q_r, void* grad_c, void* grad_k_r, float* grad_w_hyp,
                              float* grad_w_uk, float* grad_w_uv, void* workspace, size_t ws_bytes, void* stream);

/*
 * Test hooks: the integer predicates the kernels use, exported for bit-exact
 * comparison.  Page: "Multi-head Temporal Latent Attention", Key claims (paper
 * Sec. 4.2 Fig. 2(c)).
 *   mask device [n, n] uint8: mask[i-1, j-1] = 1 iff query i attends key j.
 *   hi   device [n] int32: hi[i-1] = completed slots query i attends,
 *        floor((i-1)/s).
 */
int32_t mtla_debug_stride_mask(int32_t n, int32_t s, uint8_t* mask, void* stream);
int32_t mtla_debug_slot_limits(int32_t n, int32_t s, int32_t* hi, void* stream);

/*
 * Measurement hooks.  They compute no part of the method: they measure the
 * rates this GPU achieves, against which the kernels' roofline fractions are
 * reported beside the published peaks.
 *   mtla_calib_stream_read: reads `bytes` bytes at src (device, 16-byte
 *     aligned; bytes a positive multiple of 16) with `workgroups` workgroups
 *     of 256 threads, eight 16-byte loads in flight per thread; writes one
 *     word per wave to sink (device, workgroups * 4 uint32).
 *   mtla_calib_mfma: `workgroups` workgroups of four waves; each wave runs
 *     four independent chains of `iters` 32x32x16 MFMAs on register operands
 *     (fp16 operands when f16 != 0, else bf16; fp32 accumulation) and writes
 *     one float per thread to out (device, workgroups * 256 floats).
 *     *flops (host, may be NULL) receives the multiply-add flops performed.
 *   mtla_calib_empty: launches one kernel that does nothing (the launch
 *     floor, for instance as a graph node).
 *   mtla_calib_tile_stream: the long-cache decode attention's load schedule
 *     with no arithmetic: `seqs` sequences of `rows_per_seq` rows of 1,152
 *     bytes, contiguous from rows (device, 16-byte aligned); `splits`
 *     workgroups of 512 threads per sequence stream 64-row tiles into LDS,
 *     two tile buffers.  flags bit 0: split k takes tiles k, k+splits, ...
 *     (else a contiguous range); bit 1: non-temporal loads.  sink (device,
 *     seqs * splits * 8 uint32) is written only on a pattern no real data
 *     here produces.  rows_per_seq * 1152 must fit in 31 bits; splits 1..64.
 *   mtla_calib_load_pattern: a compute unit's issue cost of 16-byte-per-lane
 *     load instructions from L2-resident data.  `workgroups` workgroups of 8
 *     waves (one per compute unit when workgroups <= 256); every wave issues
 *     32 loads, all in flight before any is used, twice over the same
 *     addresses, and cycles[w] (device, workgroups + 64 uint32, the extra
 *     words written only on a pattern no data here produces) receives
 *     workgroup w's s_memtime cycles for the second pass.  pattern 0: each
 *     load reads 1,024 contiguous bytes; 1: 16 rows of 64 bytes at a 576-byte
 *     pitch.  buf device, 16-byte aligned, bytes 128 KiB..2 GiB (read only
 *     inside [buf, buf + bytes)).
 */
int32_t mtla_calib_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);
int32_t mtla_calib_mfma(int32_t f16, int32_t workgroups, int32_t iters, float* out, double* flops, void* stream);
int32_t mtla_calib_empty(void* stream);
int32_t mtla_calib_load_pattern(int32_t pattern, int32_t workgroups, const void* buf, size_t bytes,
                                uint32_t* cycles, void* stream);
int32_t mtla_calib_tile_stream(const void* rows, int32_t seqs, int32_t rows_per_seq, int32_t splits, int32_t flags,
                               uint32_t* sink, void* stream);

/*
 * mtla_calib_step_timeline: where the time of one fused decode step goes.
 * It runs mtla_decode_step_tiles (same arguments, checks, work and
 * results) through an instance of the one-kernel step that also records,
 * per workgroup, 16 readings of the GPU's constant 100 MHz real-time
 * counter into timeline (device, uint64, 8-byte aligned), row L of 16 for
 * workgroup L: [0] entry, [1] the position known, [2] the absorb's partial
 * sums formed (W_UK and the query arrived), [3] the scaled absorbed query
 * in LDS, [4 + w] wave w's attention over its slot chunks done (w < 8),
 * [12] o_lat in LDS, [13] the output stored; [14], [15] unused.  A reading
 * is taken once the value it names is available in the wave that takes it.
 * Workgroup L serves sequence 8 (k / G) + L % 8 and head group
 * (L / 8) % G, k = L / 8, where G is the head-group count the launch uses;
 * rows of workgroups past the batch are not written.  timeline_entries must
 * be at least 16 * 8 * G * ceil(batch / 8) (the launch's workgroups).
 * Supported only where the step runs as one kernel on bf16 with d_c = 256,
 * d_r = 32 and one W_hyp row (else MTLA_ERR_UNSUPPORTED).  The readings add
 * a few scalar reads and stores to the step, so it runs slightly longer
 * than mtla_decode_step_tiles.
 */
int32_t mtla_calib_step_timeline(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                                 const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                                 const void* q_r, const void* w_uk, const void* w_uv, const void* w_uv_tiles,
                                 void* cache, float* open_acc, void* out, void* workspace, size_t ws_bytes,
                                 uint64_t* timeline, size_t timeline_entries, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MTLA_H */
