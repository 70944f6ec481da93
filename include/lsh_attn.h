/*
 * lsh_attn.h - C ABI of the gfx950 (MI355X) shared-QK angular-LSH attention
 * forward pass (Reformer).
 *
 * The method (Reformer explainer, akshathtiwari.co.in/blog/reformer, and the
 * Reformer abstract, "Reformer: The Efficient Transformer"):
 *   1. hash   - each token's shared query/key x is put in the angular sector
 *               it falls in after a random rotation: bucket = argmax of
 *               [x R_r ; -x R_r], one rotation R_r per hash round;
 *   2. sort   - tokens are sorted by (round, bucket, position);
 *   3. chunk attention - the sorted sequence is cut into equal chunks; each
 *               chunk attends to itself and the previous chunk;
 *   4. unsort - per-round results are put back in token order;
 *   5. combine - rounds are merged with weights softmax_r(lse_r), the union
 *               of the rounds' buckets.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees, synchronises or prints.  It is stateless.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; device faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative status and enqueues nothing.
 *   - Layouts are contiguous, row-major.  B = batch, H = heads, L = sequence
 *     length, D = head dim (64), n_b = buckets, n_h = hash rounds,
 *     C = chunk length (64).  "BH" = B*H independent problems.
 *   - qk, v, out, rot, o_sorted use the element type `dt` (fp32 or bf16);
 *     lse arrays are fp32; index arrays are int32.
 *   - Limits: D == 64, C == 64, L % C == 0, n_b == 1 or even in [2, 4096],
 *     1 <= n_h <= 16, B*H*n_h*L <= 2^31 - 1.
 *   - Empty problems: with B, H or L equal to 0 (and the other arguments
 *     valid) a call returns LSH_OK without reading any pointer or enqueuing
 *     any kernel, and the workspace-size queries report 0 bytes.
 *   - Outputs must not overlap inputs (LSH_ERR_ALIAS).
 */
#ifndef LSH_ATTN_H
#define LSH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LSH_F32 = 0, LSH_BF16 = 1 } lsh_dtype;

enum {
  LSH_OK = 0,
  LSH_ERR_NULL = -1,        /* a required pointer is NULL */
  LSH_ERR_SHAPE = -2,       /* B, H or L < 0, D or n_h <= 0, L % C != 0, or an index overflows int32 */
  LSH_ERR_BUCKETS = -3,     /* n_b < 1, odd n_b > 1, or n_b > 4096 */
  LSH_ERR_UNSUPPORTED = -4, /* D != 64, C != 64, n_h > 16, unknown dtype or attend bits */
  LSH_ERR_WORKSPACE = -5,   /* workspace pointer NULL or smaller than required */
  LSH_ERR_ALIAS = -6,       /* an output overlaps an input */
  LSH_ERR_HIP = -7,         /* a kernel launch or event record failed */
  LSH_ERR_TOO_LARGE = -8    /* reformer_lsh_attn_fwd_noalloc: one (batch, head) problem does not
                               fit its fixed scratch */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* lsh_status_string(int status);

/* Step 1, hashing (explainer page: angular LSH after a random rotation, several
 * independent rounds).
 *   qk      [B, H, L, D]      shared query/key vectors, element type dt.
 *   rot     [n_h, D, n_b/2]   rotations, element type dt, shared by all (b, h);
 *                             may be NULL when n_b == 1.
 *   buckets [B, H, n_h, L]    out: bucket of token i in round r, in [0, n_b):
 *                             the index of the largest entry of
 *                             [x R_r ; -x R_r], lowest index on exact ties.
 *   ws      workspace of at least lsh_hash_workspace_bytes(...) bytes.
 * The decision is exact for finite inputs: fp32 MFMA scores are certified
 * against a rigorous rounding bound; a token whose top two scores are closer
 * than that bound is re-scored in float64 against a bound of its own, and the
 * columns still inside it (and a winner's sign within it of zero) are decided
 * by exact summation of the float64 products. */
int lsh_hash_workspace_bytes(int B, int H, int L, int D, int n_b, int n_h, lsh_dtype dt,
                             size_t* bytes);
int lsh_hash(const void* qk, const void* rot, int32_t* buckets, int B, int H, int L, int D,
             int n_b, int n_h, lsh_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* How many token-rounds the last hashing on this workspace could not certify in
 * fp32 and re-decided in the fixup pass: the near-ties of the argmax, counted
 * by the GPU (same decision rule as lsh_hash above).
 *   ws      the workspace of the last lsh_hash or reformer_lsh_attn_fwd /
 *           _fwd_ex / _fwd_train call (the hashing part sits at the start of
 *           both layouts), called with the same B, H, L, n_b, n_h and dt;
 *           ws_bytes its size.
 *   count   out (host memory): the count; 0 when n_b == 1 or the problem is
 *           empty.
 * Waits for the work queued on stream, then copies one int from the device.
 * Errors: LSH_ERR_NULL (count NULL), the shape / bucket / dtype errors of
 * lsh_hash, LSH_ERR_WORKSPACE (ws NULL or smaller than the hashing part),
 * LSH_ERR_HIP (the copy failed). */
int lsh_hash_uncertified(const void* ws, size_t ws_bytes, int B, int H, int L, int n_b, int n_h,
                         lsh_dtype dt, int* count, void* stream);

/* Step 2, sort by (round, bucket, position) (explainer page: sort by bucket).
 *   buckets    [B, H, n_h, L]  input, values in [0, n_b) (not checked on device).
 *   sorted_idx [B, H, n_h*L]   out: slot g = r*L + k holds the original position
 *                              of the k-th token of round r's stable order.
 *   undo_idx   [B, H, n_h, L]  out: the slot g of position i in round r.
 *   ws         workspace of at least lsh_sort_workspace_bytes(...) bytes. */
int lsh_sort_workspace_bytes(int B, int H, int L, int n_b, int n_h, size_t* bytes);
int lsh_sort(const int32_t* buckets, int32_t* sorted_idx, int32_t* undo_idx, int B, int H, int L,
             int n_b, int n_h, void* ws, size_t ws_bytes, void* stream);

/* Step 3, chunked attention (explainer page: equal chunks of the sorted order).
 * Slots g in [0, n_h*L) are cut into chunks of C; chunk c attends to chunks
 * (c-1) mod (n_h*L/C) and c (2C keys).  For query i = sorted_idx[g] and key j:
 * logit = (x_i . x_j / max(|x_j|, 1e-12)) / sqrt(D); j == i gets -1e5 (so a token
 * sees itself only when nothing else is left); causal != 0 drops j > i.
 *   qk, v      [B, H, L, D]       element type dt.
 *   sorted_idx [B, H, n_h*L]      from lsh_sort.
 *   o_sorted   [B, H, n_h*L, D]   out: softmax-weighted sum of V per slot (dt).
 *   lse_sorted [B, H, n_h*L]      out: log-sum-exp of the slot's logits (fp32). */
int lsh_chunk_attn(const void* qk, const void* v, const int32_t* sorted_idx, void* o_sorted,
                   float* lse_sorted, int B, int H, int L, int D, int n_h, int C, int causal,
                   lsh_dtype dt, void* stream);

/* Step 3 with a different attended set (explainer page: each token "attends to
 * its bucket-mates" after the sort, and the rounds "union the buckets"; read
 * literally, these name two variants of the window above).  `attend` is 0 (the
 * window as in lsh_chunk_attn, identical results) or an OR of:
 *   LSH_ATTEND_SAME_BUCKET - a key slot counts only if it holds the query's
 *       (round, bucket): the window is cut down to bucket-mates of the same
 *       round.  The self logit and the causal rule are as above.
 *   LSH_ATTEND_DEDUP - every distinct key token counts once over the union of
 *       the query's windows in all rounds: each kept logit of the pair (i, j),
 *       the self pair included, is lowered by ln N_ij, with N_ij the number of
 *       (occurrence of i, occurrence of j) pairs over all rounds' windows that
 *       the other masks keep.  After the combine step, out_i is then the
 *       softmax over the set union of i's keys, each key once.
 *   buckets  [B, H, n_h, L]  from lsh_hash; read with LSH_ATTEND_SAME_BUCKET
 *                            (may be NULL otherwise).
 *   undo_idx [B, H, n_h, L]  from lsh_sort; read with LSH_ATTEND_DEDUP (may be
 *                            NULL otherwise).
 *   ws       workspace of at least lsh_chunk_attn_ex_workspace_bytes(...) bytes
 *            (0 without LSH_ATTEND_DEDUP, when ws may be NULL): a token-major
 *            copy of every round's bucket and chunk, B*H*L*n_h int32.
 * Other arguments as in lsh_chunk_attn.  Bucket values must be in [0, 4096)
 * and undo_idx must be lsh_sort's inverse of sorted_idx (neither is checked on
 * the device; other values give meaningless results but no out-of-bounds
 * access).  With a variant bit set every chunk takes the exact softmax path,
 * so expect the call to be slower than lsh_chunk_attn. */
#define LSH_ATTEND_SAME_BUCKET 1
#define LSH_ATTEND_DEDUP 2
int lsh_chunk_attn_ex_workspace_bytes(int B, int H, int L, int n_h, int attend, size_t* bytes);
int lsh_chunk_attn_ex(const void* qk, const void* v, const int32_t* sorted_idx,
                      const int32_t* buckets, const int32_t* undo_idx, void* o_sorted,
                      float* lse_sorted, int B, int H, int L, int D, int n_h, int C, int causal,
                      int attend, lsh_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* Steps 4-5, unsort and combine (explainer page: union of the rounds).
 * LSE_i = logsumexp_r lse_r(i), out_i = sum_r exp(lse_r(i) - LSE_i) o_r(i), with
 * o_r(i) = o_sorted[undo_idx[r][i]].
 *   out     [B, H, L, D]   out, element type dt.
 *   lse_out [B, H, L]      optional out (NULL to skip), fp32. */
int lsh_unsort_combine(const void* o_sorted, const float* lse_sorted, const int32_t* undo_idx,
                       void* out, float* lse_out, int B, int H, int L, int D, int n_h,
                       lsh_dtype dt, void* stream);

/* The whole forward pass, steps 1-5, with all intermediates in the workspace.
 * Arguments as above.  `stage_events` is optional: NULL, or an array of
 * LSH_FWD_N_EVENTS hipEvent_t (as void*) that are recorded on `stream` before
 * the first and after every kernel launch, in the order of the
 * LSH_FWD_KERNEL_* list, for per-kernel timing.  A NULL entry is skipped, so
 * a caller can time one kernel (entries k and k+1) without the cost of the
 * other records (each adds a few microseconds between kernels).  The same holds
 * for every stage_events array below. */
#define LSH_FWD_KERNEL_PREP 0      /* rotation transpose + norms */
#define LSH_FWD_KERNEL_HASH 1      /* MFMA projection + certified argmax */
#define LSH_FWD_KERNEL_FIXUP 2     /* float64/exact re-decision of uncertified tokens */
#define LSH_FWD_KERNEL_HIST 3      /* per-tile bucket histograms */
#define LSH_FWD_KERNEL_SCATTER 4   /* histogram scan + stable in-tile ranking + scatter */
#define LSH_FWD_KERNEL_ATTN 5      /* chunked attention */
#define LSH_FWD_KERNEL_COMBINE 6   /* unsort + combine */
#define LSH_FWD_N_KERNELS 7
#define LSH_FWD_N_EVENTS (LSH_FWD_N_KERNELS + 1)

int lsh_fwd_workspace_bytes(int B, int H, int L, int D, int n_b, int n_h, int C, lsh_dtype dt,
                            size_t* bytes);
int reformer_lsh_attn_fwd(const void* qk, const void* v, const void* rot, int n_buckets,
                          int n_hashes, int chunk_len, int causal, int B, int H, int L, int D,
                          lsh_dtype dt, void* out, float* lse_out, void* ws, size_t ws_bytes,
                          void* stream, void* const* stage_events);

/* The whole forward pass with an attended-set variant (`attend` as in
 * lsh_chunk_attn_ex; 0 gives reformer_lsh_attn_fwd).  lsh_fwd_workspace_bytes
 * covers both calls; other arguments as in reformer_lsh_attn_fwd.  The
 * LSH_ATTEND_DEDUP variant adds one kernel before the attention, timed with it
 * (the LSH_FWD_KERNEL_ATTN stage). */
int reformer_lsh_attn_fwd_ex(const void* qk, const void* v, const void* rot, int n_buckets,
                             int n_hashes, int chunk_len, int causal, int attend, int B, int H,
                             int L, int D, lsh_dtype dt, void* out, float* lse_out, void* ws,
                             size_t ws_bytes, void* stream, void* const* stage_events);

/* The whole forward pass (as reformer_lsh_attn_fwd, attend = 0, no stage
 * events) without a workspace argument and without allocating: for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops with a fixed memory plan, harnesses that forbid hipMalloc).
 *   The intermediates live in a fixed scratch array of
 *   LSH_NOALLOC_SCRATCH_BYTES (256 MiB) per device, part of the library's code
 *   object: every device the library runs on holds it from the library's load
 *   until the process ends.  Problems are processed in groups of (batch, head)
 *   problems whose workspace (lsh_fwd_workspace_bytes) fits the scratch, one
 *   group after another on `stream`; results are bit-identical to
 *   reformer_lsh_attn_fwd.  A problem fits when lsh_fwd_workspace_bytes for
 *   B = H = 1 is at most the scratch size: in bf16 up to n_h * L = 2^20
 *   token-rounds (L = 65536 with 16 rounds: 164.5 MiB), in fp32 up to 2^19
 *   (L = 65536 with 8 rounds: 141.8 MiB).
 *   Returns LSH_ERR_TOO_LARGE, before anything is enqueued, when one problem's
 *   workspace exceeds the scratch; other errors as in reformer_lsh_attn_fwd.
 *   The first call on a device looks up that device's scratch address (with
 *   the device current) and keeps it; a failure there returns LSH_ERR_HIP.
 *   All calls on one device share its scratch, which keeps the last call's
 *   contents (every kernel writes what it later reads; nothing needs clearing).
 *   Calls that overlap in time on one device - on different streams, or from
 *   different host threads - race on the scratch: order them on one stream or
 *   synchronise between them. */
#define LSH_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int reformer_lsh_attn_fwd_noalloc(const void* qk, const void* v, const void* rot, int n_buckets,
                                  int n_hashes, int chunk_len, int causal, int B, int H, int L,
                                  int D, lsh_dtype dt, void* out, float* lse_out, void* stream);

/* Backward of the forward pass with respect to qk and v (Reformer explainer:
 * the method's pipeline, differentiated; hashing and sorting are piecewise
 * constant, so the forward's permutation is reused and no gradient flows
 * through them).  The loss is sum_i dout_i . out_i + dlse_i LSE_i.
 *   qk, v       [B, H, L, D]     the forward's inputs (dt).
 *   sorted_idx  [B, H, n_h*L]    from lsh_sort (the forward's permutation).
 *   undo_idx    [B, H, n_h, L]   from lsh_sort.
 *   lse_sorted  [B, H, n_h*L]    from lsh_chunk_attn (per-round log-sum-exp).
 *   out         [B, H, L, D]     the forward's output (dt).
 *   dout        [B, H, L, D]     gradient of the loss w.r.t. out (dt).
 *   dlse        [B, H, L]        gradient w.r.t. the forward's lse output
 *                                (fp32), or NULL for none.
 *   dqk, dv     [B, H, L, D]     out: gradients w.r.t. qk and v (dt).
 *   ws          workspace of at least lsh_attn_bwd_workspace_bytes(...) bytes.
 *   stage_events  NULL, or LSH_BWD_N_EVENTS hipEvent_t recorded before the
 *               first and after every kernel (LSH_BWD_KERNEL_* order).
 * Per slot the combined weight of every key occurrence is recomputed from qk
 * and lse_sorted; the self key (logit -1e5) passes no gradient to qk.  A
 * round in which only the self key is left (lse near -1e5) is recognised as
 * such; the method assumes |qk_i| / 8 stays far below 1e5.  The call is
 * deterministic (no atomics): repeated calls give identical bits. */
#define LSH_BWD_KERNEL_PREP 0    /* combine weights per slot, key scales */
#define LSH_BWD_KERNEL_ATTN 1    /* chunk attention backward, per slot */
#define LSH_BWD_KERNEL_REDUCE 2  /* sum of each token's rounds */
#define LSH_BWD_N_KERNELS 3
#define LSH_BWD_N_EVENTS (LSH_BWD_N_KERNELS + 1)
int lsh_attn_bwd_workspace_bytes(int B, int H, int L, int D, int n_h, int C, lsh_dtype dt,
                                 size_t* bytes);
int lsh_attn_bwd(const void* qk, const void* v, const int32_t* sorted_idx, const int32_t* undo_idx,
                 const float* lse_sorted, const void* out, const void* dout, const float* dlse,
                 void* dqk, void* dv, int B, int H, int L, int D, int n_h, int C, int causal,
                 lsh_dtype dt, void* ws, size_t ws_bytes, void* stream, void* const* stage_events);

/* The fused forward for training: as reformer_lsh_attn_fwd, and it also writes
 * the state lsh_attn_bwd reuses to caller buffers (not the workspace):
 *   sorted_idx [B, H, n_h*L], undo_idx [B, H, n_h, L] (int32) and
 *   lse_sorted [B, H, n_h*L] (fp32); none may be NULL, none may overlap. */
int reformer_lsh_attn_fwd_train(const void* qk, const void* v, const void* rot, int n_buckets,
                                int n_hashes, int chunk_len, int causal, int B, int H, int L,
                                int D, lsh_dtype dt, void* out, float* lse_out,
                                int32_t* sorted_idx, int32_t* undo_idx, float* lse_sorted,
                                void* ws, size_t ws_bytes, void* stream,
                                void* const* stage_events);

/* Building blocks of the reversible block below, exposed for staged use.
 * lsh_layer_norm: y = (x - mean) / sqrt(var + 1e-5) * gamma + beta over each
 * row of `dim` features (bf16 in and out, fp32 arithmetic; dim % 8 == 0,
 * dim <= 1024).
 * lsh_linear: c = epilogue(a . w^T), w [N, K] row-major (a Linear layer's
 * [out, in]), bf16 in and out, fp32 accumulation; N % 128 == 0, K % 64 == 0.
 * Layouts: LSH_LAYOUT_ROWS is [M, K] / [M, N] row-major; LSH_LAYOUT_HEADS is
 * the attention's [B, H, L, 64] with M = B L and K (for a) or N (for c) =
 * 64 heads (not both).  Epilogue: 0, BIAS|GELU (+ bias[n], then GELU, the erf
 * form), RESID (+ resid[m][n], rows layout; c must use rows), BIAS|RESID. */
#define LSH_LAYOUT_ROWS 0
#define LSH_LAYOUT_HEADS 1
#define LSH_EPI_BIAS 1
#define LSH_EPI_GELU 2
#define LSH_EPI_RESID 4
int lsh_layer_norm(const void* x, const void* gamma, const void* beta, void* y, int rows, int dim,
                   lsh_dtype dt, void* stream);
int lsh_linear(const void* a, int a_layout, const void* w, const void* bias, const void* resid,
               void* c, int c_layout, int M, int N, int K, int L, int heads, int epilogue,
               lsh_dtype dt, void* stream);

/* One reversible Reformer block around the LSH attention (Reformer abstract:
 * reversible residual layers; Reformer explainer: reversible layers and a
 * chunked feed-forward, with LSH attention, fit about 64K tokens on one
 * accelerator):
 *   y1 = x1 + F(x2),  F(x) = W_o . LSHAttn(LN1(x) W_qk^T, LN1(x) W_v^T)
 *   y2 = x2 + G(y1),  G(y) = W2 . GELU(W1 . LN2(y) + b1) + b2
 * with LayerNorm LN(x) = (x - mean) / sqrt(var + 1e-5) * g + b over the
 * features, the attention of reformer_lsh_attn_fwd on each of `heads` heads
 * (head h takes features 64h .. 64h+63; the rotations rot are shared by all
 * heads), GELU the erf form, and G taken over chunks of chunk_rows rows (0 =
 * all rows at once): the hidden activation needs chunk_rows * 4 dim elements.
 *   x1, x2, y1, y2  [B, L, dim] bf16, dim = 64 heads (heads even, <= 16).
 *   params          LSH_BLOCK_N_PARAMS device pointers, bf16, in the order
 *                   below; weights [out, in] row-major (a Linear layer's
 *                   layout).
 *   ws              workspace of at least reformer_block_workspace_bytes.
 *   stage_events    NULL, or LSH_BLOCK_N_EVENTS events recorded between the
 *                   LSH_BLOCK_STAGE_* stages.
 * Only bf16 is supported (LSH_ERR_UNSUPPORTED otherwise).  The inverse of the
 * block (x2 = y2 - G(y1), x1 = y1 - F(x2)) needs no extra kernel: it is two
 * sublayer evaluations with the residual subtracted, which callers recompute
 * in a reversible backward pass. */
#define LSH_BLOCK_LN1_G 0  /* [dim] */
#define LSH_BLOCK_LN1_B 1  /* [dim] */
#define LSH_BLOCK_W_QK 2   /* [dim, dim] shared query/key projection */
#define LSH_BLOCK_W_V 3    /* [dim, dim] */
#define LSH_BLOCK_W_O 4    /* [dim, dim] */
#define LSH_BLOCK_LN2_G 5  /* [dim] */
#define LSH_BLOCK_LN2_B 6  /* [dim] */
#define LSH_BLOCK_W1 7     /* [4 dim, dim] */
#define LSH_BLOCK_B1 8     /* [4 dim] */
#define LSH_BLOCK_W2 9     /* [dim, 4 dim] */
#define LSH_BLOCK_B2 10    /* [dim] */
#define LSH_BLOCK_N_PARAMS 11
#define LSH_BLOCK_STAGE_LN1 0
#define LSH_BLOCK_STAGE_QKV 1   /* shared-QK and V projections (head-major output) */
#define LSH_BLOCK_STAGE_ATTN 2  /* the LSH attention forward pass */
#define LSH_BLOCK_STAGE_OUT 3   /* output projection + residual (head-major input) */
#define LSH_BLOCK_STAGE_LN2 4
#define LSH_BLOCK_STAGE_FFN 5   /* both feed-forward GEMMs over all row chunks */
#define LSH_BLOCK_N_STAGES 6
#define LSH_BLOCK_N_EVENTS (LSH_BLOCK_N_STAGES + 1)
int reformer_block_workspace_bytes(int B, int L, int heads, int n_buckets, int n_hashes,
                                   int chunk_len, int chunk_rows, lsh_dtype dt, size_t* bytes);
int reformer_block_fwd(const void* x1, const void* x2, const void* rot, const void* const* params,
                       int B, int L, int heads, int n_buckets, int n_hashes, int chunk_len,
                       int causal, int chunk_rows, lsh_dtype dt, void* y1, void* y2, void* ws,
                       size_t ws_bytes, void* stream, void* const* stage_events);

/* Timing helpers for callers that have no HIP runtime binding of their own:
 * create/destroy a hipEvent_t (returned as void*), and the elapsed time in
 * milliseconds between two recorded events (synchronises on `end`).  The
 * events are for timing only (created with hipEventDisableSystemFence): their
 * completion does not make device writes visible to the host, so synchronise
 * the stream or the device before reading results on the host. */
int lsh_event_create(void** event);
int lsh_event_destroy(void* event);
int lsh_event_record(void* event, void* stream);
int lsh_event_elapsed_ms(void* start, void* end, float* ms);

/* Measured shader clock, for reporting beside roofline fractions (which use
 * the published peaks).  Every CU runs a dependent-FMA spin of about spin_us
 * microseconds (2048 blocks of 256 threads); each block counts shader-clock
 * cycles (s_memtime) against the constant-rate real-time counter
 * (s_memrealtime, whose rate is hipDeviceAttributeWallClockRate).
 *   ticks    device memory, LSH_CLOCK_TICKS_BYTES, caller-owned scratch
 *            (overwritten: per block the two counter deltas);
 *   spin_us  1 .. 100000;
 *   mhz      out (host): mean over the blocks of cycles / real time, in MHz;
 *   stream   HIP stream (NULL: the null stream); the call synchronises it.
 * Errors: LSH_ERR_NULL (ticks or mhz NULL), LSH_ERR_SHAPE (spin_us out of
 * range), LSH_ERR_HIP (attribute query, launch or copy failed). */
#define LSH_CLOCK_TICKS_BYTES (2 * 2048 * 8)
int lsh_measure_clock(void* ticks, int spin_us, double* mhz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LSH_ATTN_H */
