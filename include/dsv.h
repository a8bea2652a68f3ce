/*
 * dsv.h -- C ABI of the DSV dynamic block-sparse attention library (libdsv.so) for
 * AMD MI355X (gfx950).
 *
 * The method: DSV, as described by the explainer pages titled "DSV: Exploiting
 * Dynamic Sparsity to Accelerate Large-Scale Video DiT Training"
 * (gist.science/de/paper/2502.07590 -- cited [de] -- and
 * gist.science/es/paper/2502.07590 -- cited [es]; section numbers refer to the
 * pages' technical summaries).  A cheap per-head low-rank predictor estimates
 * Q K^T, the critical KV blocks of every query block are chosen by top-k, and
 * exact softmax attention runs over those blocks only, forward and backward.
 *
 * The four compute calls, in pipeline order:
 *   dsv_predict          predicted attention mass per (query block, KV block)
 *   dsv_predict_representative  (alternative) the mass of one representative row per query block
 *   dsv_predict_select_representative  (alternative) that predictor fused with top-k: indices only
 *   dsv_select_topk      the k most important KV blocks of each query block
 *   dsv_select_mass      (alternative) the fewest blocks carrying a fraction tau of the score
 *   dsv_sparse_attn_fwd  softmax attention restricted to the selected blocks
 *   dsv_sparse_attn_bwd  its gradients with respect to Q, K and V
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every tensor argument is a DEVICE pointer into memory the caller
 *   allocated (hipMalloc or equivalent) on the current HIP device.  The library
 *   never allocates, frees or retains a pointer after the call returns.  Tensor
 *   pointers must be 16-byte aligned; workspace pointers 256-byte aligned.
 * Layout.  All tensors are dense, row-major (C order), no strides:
 *     q, k, v, o, dout, dq, dk, dv   [B, H, N, d]   element type = problem.dtype
 *     wq, wk                          [H, d, r]      element type = problem.dtype
 *     lse                             [B, H, N]      float32
 *     block_scores                    [B, H, N/Bq, N/Bk]  float32
 *     block_idx                       [B, H, N/Bq, k]     int32
 *   bf16 tensors hold IEEE bfloat16 bit patterns (uint16 storage).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Calls only enqueue work on it and return; nothing is synchronised.
 * Errors.  Arguments are validated on the host before any launch; on failure the
 *   call returns a non-zero dsv_status, enqueues nothing, and dsv_last_error()
 *   describes the problem (thread-local string, valid until the next call on the
 *   same thread).  A failed launch returns DSV_ERR_HIP.  Non-finite inputs are
 *   not checked: they propagate into the outputs.
 * State.  The library has no global mutable state (only the optional per-thread
 *   timing record below, and the device arrays of dsv_pack_kv_noalloc and of the
 *   debug check below); calls are thread-safe and may run concurrently on
 *   different streams with different buffers.  All calls are
 *   deterministic (bitwise repeatable for the same inputs and problem), and a
 *   head's results do not depend on the other heads of the call or on the
 *   device's compute-unit count: predicting heads one call at a time or all at
 *   once gives the same bits.
 * Block lists.  Every call that takes block_idx uses, per query block, its first
 *   block_counts[qb] entries (clamped to [0, k]) or all k when block_counts is
 *   NULL.  Results are defined only when those entries are distinct indices in
 *   [0, N/Bk) (the selection calls always emit such lists; entries past a count,
 *   such as dsv_select_mass's -1 padding, are never read).  For any other list
 *   every access still stays inside the tensors -- an out-of-range entry is
 *   clamped into range by the forward and the dQ kernel and skipped by the
 *   dK/dV kernel's transposed lists, and a repeated entry is used twice by the
 *   forward and dQ but once by dK/dV -- but the outputs are unspecified, and the
 *   backward is then not the forward's gradient.  (dsv_pack_kv states its own,
 *   defined treatment of out-of-range entries.)
 * Debug check.  With the environment variable DSV_DEBUG_VALIDATE=1 (read at each
 *   call), dsv_sparse_attn_fwd and dsv_sparse_attn_bwd first check the lists on
 *   the device and return DSV_ERR_INVALID_ARGUMENT, having launched nothing else,
 *   if a query block's used entries are out of range or repeated.  The check
 *   BLOCKS (it waits for the stream) and keeps its count in a device word of the
 *   library, so checked calls must not overlap in time on one GPU.  It is meant
 *   for debugging, not for timed runs.
 */
#ifndef DSV_H_
#define DSV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSV_OK = 0,
  DSV_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, inconsistent sizes   */
  DSV_ERR_UNSUPPORTED = 2,        /* valid problem outside the compiled instances  */
  DSV_ERR_WORKSPACE_TOO_SMALL = 3,
  DSV_ERR_HIP = 4                 /* a HIP runtime or launch error                 */
} dsv_status;

typedef enum { DSV_F32 = 0, DSV_BF16 = 1 } dsv_dtype;

/*
 * The problem.  Sizes follow the pages' statement: per attention head
 * ([es] §2.A: the predictor approximates Q K^T of each head independently),
 * queries grouped into blocks of consecutive tokens that share one selection
 * ([de] §2.B; [es] §2.B, query grouping), keys grouped into KV blocks that are
 * the unit of selection, and k blocks kept per query block ([de] §2.B top-k).
 *
 *   batch, heads        B, H >= 1
 *   seq_len             N >= 1 tokens (a flattened T x H x W video latent)
 *   head_dim            d
 *   q_block, kv_block   Bq, Bk; N % Bq == 0, N % Bk == 0, Bq % Bk == 0
 *   topk                k, 1 <= k <= N / Bk
 *   rank                r, the predictor rank
 *   dtype               DSV_F32 or DSV_BF16 (storage and MFMA operand type)
 *   sm_scale            softmax scale of the attention; <= 0 means 1/sqrt(d)
 *   pred_scale          scale of the predicted logits;   <= 0 means 1/sqrt(d)
 *
 * Compiled instances (others return DSV_ERR_UNSUPPORTED):
 *   bf16: d in {64, 128}, r in {16, 32}, Bq in {64, 128}, Bk = 64, N/Bk <= 4096;
 *         dsv_predict additionally needs N % 256 == 0
 *   f32 : d <= 128, r <= 64, any Bq/Bk satisfying the divisibility rules,
 *         N/Bk <= 4096 (a plain VALU path meant for small problems)
 */
typedef struct {
  int32_t batch;
  int32_t heads;
  int32_t seq_len;
  int32_t head_dim;
  int32_t q_block;
  int32_t kv_block;
  int32_t topk;
  int32_t rank;
  int32_t dtype;      /* dsv_dtype */
  float sm_scale;
  float pred_scale;
} dsv_problem;

/* Workspace bytes dsv_predict needs for this problem (0 if the problem is invalid).
   The size depends on the current device's compute-unit count: query it on the
   device the call will run on. */
size_t dsv_predict_workspace_size(const dsv_problem* p);

/*
 * dsv_predict -- low-rank sparsity predictor ([es] §2.A; [de] §2.A;
 * [de] §2.B, the fused matmul and top-k; [de] §2.B query grouping).
 *
 *   Q~   = round(pred_scale log2(e) Q Wq[h]),  K_lr = round(K Wk[h])
 *                                  (round = once, to dtype, RNE; fp32 keeps them exact)
 *   l_ij = ln(2) <Q~_i, K_lr_j>    (= pred_scale <Q Wq[h], K_lr_j> up to the rounding;
 *                                   all j: no causal mask)
 *   P_ij = exp(l_ij) / sum_j' exp(l_ij')                  (row softmax over all N keys)
 *   block_scores[b,h,qb,kb] = sum_{i in qb} sum_{j in kb} P_ij
 * i.e. the predicted attention mass of query block qb on KV block kb, summed
 * over the block's rows (each score row sums to Bq).  The N x N matrix is never
 * written to memory.
 *
 *   q, k          [B, H, N, d]   inputs
 *   wq, wk        [H, d, r]      predictor weights
 *   workspace     >= dsv_predict_workspace_size(p) bytes, caller-owned scratch.
 *                 On return its first bytes hold Q~ then K_lr, each
 *                 [B, H, N, r] in dtype (a by-product callers may inspect).
 *   block_scores  [B, H, N/Bq, N/Bk] float32 output.
 */
dsv_status dsv_predict(const dsv_problem* p, const void* q, const void* k, const void* wq,
                       const void* wk, void* workspace, size_t workspace_bytes,
                       float* block_scores, void* stream);

/*
 * dsv_predict_representative -- the representative-row variant of the predictor ([de] §2.B,
 * query grouping: the critical pairs of a group of neighbouring queries are estimated for one
 * representative of the group).  Same inputs, projections and workspace as dsv_predict; the
 * score of (qb, kb) is the predicted softmax mass that the single query row
 * qb * Bq + rep_row puts on KV block kb (each score row sums to 1):
 *   score[qb, kb] = sum_{j in kb} exp(l_ij - LSE_i),   i = qb * Bq + rep_row.
 * The ranking of a row's blocks equals the ranking of their in-block log-sum-exp of logits,
 * so top-k on these scores needs no statistics of other rows.  Feed the scores to
 * dsv_select_topk or dsv_select_mass.  Costs 1/Bq of dsv_predict's logit sweep.
 *
 *   rep_row       0 <= rep_row < Bq
 *   block_scores  [B, H, N/Bq, N/Bk] float32 output
 * The bf16 instance needs the same sizes as dsv_predict.
 */
dsv_status dsv_predict_representative(const dsv_problem* p, const void* q, const void* k, const void* wq,
                                      const void* wk, int32_t rep_row, void* workspace, size_t workspace_bytes,
                                      float* block_scores, void* stream);

/*
 * dsv_predict_select_representative -- the fused predictor and top-k selection of the pages
 * ([de] §2.B: one kernel does the low-rank matmul and the top-k, without an O(S^2) intermediate;
 * query grouping: the critical pairs of a group of neighbouring queries are estimated for one
 * representative).  block_idx[b,h,qb] = the k KV blocks with the largest predicted softmax mass
 * of the single query row i = qb * Bq + rep_row (the scores of dsv_predict_representative), ties
 * toward the smaller block index, written ascending -- equal to dsv_predict_representative
 * followed by dsv_select_topk up to floating-point rounding of near-equal masses.  The bf16
 * instance ranks each row's blocks by their unnormalised mass (the same order as the score,
 * since the row's normaliser is common; by their in-block log-sum-exp of logits where the masses
 * leave fp32's range) inside the predictor's sweep and writes no score matrix; the fp32 instance
 * computes the scores into the workspace and selects from them.
 *
 *   q, k, wq, wk  as dsv_predict;  rep_row  0 <= rep_row < Bq;  k = problem.topk
 *   workspace     >= dsv_predict_workspace_size(p) bytes; on return it holds Q~ and K_lr as for
 *                 dsv_predict (the rest is scratch)
 *   block_idx     [B, H, N/Bq, k] int32 output
 * The bf16 instance needs the same sizes as dsv_predict.
 */
dsv_status dsv_predict_select_representative(const dsv_problem* p, const void* q, const void* k, const void* wq,
                                             const void* wk, int32_t rep_row, void* workspace, size_t workspace_bytes,
                                             int32_t* block_idx, void* stream);

/*
 * dsv_select_topk -- critical-KV selection ([de] §2.B, top-k selection;
 * [es] §2.B).  For every (b, h, qb) the k KV blocks with the largest
 * block_scores, ties broken toward the smaller block index, written ascending
 * (distinct indices).  Scores are compared as IEEE floats; a NaN sorts above +inf.
 *
 *   block_scores  [B, H, N/Bq, N/Bk] float32 input
 *   block_idx     [B, H, N/Bq, k] int32 output
 */
dsv_status dsv_select_topk(const dsv_problem* p, const float* block_scores, int32_t* block_idx,
                           void* stream);

/*
 * dsv_select_mass -- mass-threshold selection: keep the critical KV blocks that carry most of
 * the predicted score ([de] §2.A and [es] §2.A: ~90% of the attention score lies in few KV
 * pairs).  For every (b, h, qb): the smallest set of KV blocks, taken by descending
 * block_scores with ties toward the smaller block index, whose scores sum to at least
 * tau * (the row's total score); at most k = problem.topk blocks, never empty.
 *
 *   block_scores  [B, H, N/Bq, N/Bk] float32 input (dsv_predict's output)
 *   tau           target fraction, 0 < tau <= 1
 *   block_idx     [B, H, N/Bq, k] int32 output: the chosen blocks ascending, then -1 padding
 *   block_counts  [B, H, N/Bq] int32 output: number of chosen blocks (1 .. k)
 * Pass block_idx and block_counts on to the attention calls.  The count is an integer
 * decided by a float32 sum; where the cumulative score at the cut lies within rounding of
 * the target, it may differ by one from a sum formed in another order or precision.
 */
dsv_status dsv_select_mass(const dsv_problem* p, const float* block_scores, float tau, int32_t* block_idx,
                           int32_t* block_counts, void* stream);

/*
 * dsv_head_density -- per-block activation of sparse attention: the pages switch a block of
 * the model from full to sparse attention once its attention is sparse enough ([de] §2.A,
 * stage 2).  The measure is each head's selected density,
 *   S[b,h] = sum over query blocks of the list length (block_counts clamped to [0, k], or k
 *            when block_counts is NULL),   density[b,h] = S / (N/Bq * N/Bk)  (float32 of the
 *            exact quotient),
 * and the head is flagged dense (dense[b,h] = 1, else 0) when S > floor(dense_above * N/Bq *
 * N/Bk), the product taken in double precision on the host.  A caller runs flagged heads (or
 * a layer with any flagged head) with every block selected, i.e. dense attention through the
 * same kernels.
 *   block_counts  [B, H, N/Bq] int32 (dsv_select_mass's counts) or NULL
 *   dense_above   finite, >= 0 (e.g. 0.5);  density [B, H] float32 output;
 *   dense         [B, H] int32 output, or NULL
 * Uses problem.batch, heads, seq_len, q_block, kv_block and topk (= the lists' width k).
 */
dsv_status dsv_head_density(const dsv_problem* p, const int32_t* block_counts, float dense_above, float* density,
                            int32_t* dense, void* stream);

/*
 * dsv_block_recall -- sparsity profiler: the true attention mass a selection captures ([de]
 * §2.A: the critical KV carry most of the attention score).  For query row i with selected
 * keys J_i, the captured mass is sum_{j in J_i} softmax(s_i)_j over ALL keys
 * = exp(LSE_J(i) - LSE_all(i)); recall[b, h, qb] is its mean over the rows of query block qb.
 *
 *   lse_selected  [B, H, N] float32: dsv_sparse_attn_fwd's lse for the selection
 *   lse_all       [B, H, N] float32: dsv_sparse_attn_fwd's lse with every block selected
 *                 (k = N/Bk, block_idx[qb] = 0 .. N/Bk - 1), same q, k and scale
 *   recall        [B, H, N/Bq] float32 output, in [0, 1]
 * Only problem.batch, heads, seq_len and q_block are used.
 */
dsv_status dsv_block_recall(const dsv_problem* p, const float* lse_selected, const float* lse_all, float* recall,
                            void* stream);

/* Workspace bytes dsv_pack_kv needs (0 if the problem is invalid). */
size_t dsv_pack_kv_workspace_size(const dsv_problem* p);

/*
 * dsv_pack_kv -- the one-GPU share of sequence-sharded context parallelism ([de] §2.C,
 * [es] §2.C: shard long sequences over GPUs and move only the KV that the sparsity needs).
 * For the receiver's query blocks [qb_begin, qb_end): per (b, h) the union of the KV blocks
 * their lists select (block_counts as in dsv_sparse_attn_fwd; out-of-range entries ignored),
 * ascending, and its K and V rows copied contiguously:
 *   packed_blocks [B, H, N/Bk] int32  the union ascending, then -1 padding
 *   packed_counts [B, H] int32        its size U
 *   k_packed, v_packed [B, H, N, d]   rows [u*Bk, (u+1)*Bk) hold block packed_blocks[u] of
 *                                     k, v for u < U (later rows are not written)
 *   packed_idx [B, H, qb_end - qb_begin, k] int32  the shard's lists rewritten to positions in
 *                                     the union (-1 past a row's count or for an ignored entry)
 * The receiver's forward is dsv_sparse_attn_fwd on (its Q rows, k_packed, v_packed,
 * packed_idx), which equals the forward over the original k, v for those rows.  Bk must be 64.
 */
dsv_status dsv_pack_kv(const dsv_problem* p, const void* k, const void* v, const int32_t* block_idx,
                       const int32_t* block_counts, int32_t qb_begin, int32_t qb_end, void* k_packed,
                       void* v_packed, int32_t* packed_blocks, int32_t* packed_counts, int32_t* packed_idx,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsv_pack_kv_noalloc -- dsv_pack_kv without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, outputs and results as dsv_pack_kv, minus `workspace`.  The
 * union flags and positions live instead in a device array inside the library: one copy per
 * GPU, allocated with the code object and held until the process ends, sized for
 * B * H * N/Bk <= 262144 (2 MiB in all).  The call allocates and frees nothing; it clears
 * what must start at zero with a kernel of its own on `stream`.
 * Limits and races: a larger problem returns DSV_ERR_UNSUPPORTED (use dsv_pack_kv).  Every
 * call on one GPU shares that GPU's array, so calls that may overlap in time on one GPU
 * (different streams, or different host threads) race and must be serialised by the caller;
 * calls queued on one stream are ordered and safe.
 */
dsv_status dsv_pack_kv_noalloc(const dsv_problem* p, const void* k, const void* v, const int32_t* block_idx,
                               const int32_t* block_counts, int32_t qb_begin, int32_t qb_end, void* k_packed,
                               void* v_packed, int32_t* packed_blocks, int32_t* packed_counts, int32_t* packed_idx,
                               void* stream);

/* Workspace bytes dsv_sparse_attn_fwd needs when o_lo is requested (DSV_BF16: an fp16 copy
   of V plus a few bytes per head); 0 for DSV_F32 or an invalid problem.  A forward without
   o_lo needs no workspace (`workspace` may then be NULL). */
size_t dsv_sparse_attn_fwd_workspace_size(const dsv_problem* p);

/*
 * dsv_sparse_attn_fwd -- exact softmax attention over the selected KV blocks
 * only (the custom sparse attention kernels of [es] §3 and [de] §3, used for
 * sparse training, [de] §2.A stage 2).  For each query row i of block qb, with
 * J = the keys of the blocks in block_idx[b,h,qb]:
 *   s_ij = sm_scale <q_i, k_j>,  O_i = sum_{j in J} softmax_J(s_i)_j v_j,
 *   lse_i = log sum_{j in J} exp(s_ij)   (natural log)
 * The list entries used must be distinct indices in [0, N/Bk) (see "Block lists"
 * above); their order does not matter (dsv_select_topk emits them ascending).
 *
 *   q, k, v     [B, H, N, d] inputs;  block_idx [B, H, N/Bq, k]
 *   block_counts  optional [B, H, N/Bq] int32, or NULL: query block qb uses the first
 *               block_counts[qb] entries of its block_idx row (clamped to [0, k]; the
 *               rest are never read).  NULL means all k.  A query block with an empty
 *               list gets O = 0 and lse = -inf.
 *   o           [B, H, N, d] output (dtype);  lse [B, H, N] float32 output
 *   o_lo        optional [B, H, N, d] bf16 output, or NULL.  DSV_BF16 only (must
 *               be NULL for DSV_F32).  When given (the training forward), the
 *               forward first copies V to fp16 with a power-of-two per-head
 *               scale (exact for bf16 values) into the workspace, computes P V
 *               with P rounded to fp16 (2^-11 relative, against bf16's 2^-8),
 *               and writes the rounding residual bf16(O - o) here, so that
 *               o + o_lo carries O to ~16 bits.  Passing it on to
 *               dsv_sparse_attn_bwd makes the backward's row term
 *               D = rowsum(dO o O) accurate instead of limited by bf16
 *               rounding, which otherwise dominates dQ's error.  Pass it for
 *               training; an inference forward leaves it NULL.
 *   workspace   >= dsv_sparse_attn_fwd_workspace_size(p) bytes when o_lo is
 *               given (256-byte aligned); ignored otherwise
 */
dsv_status dsv_sparse_attn_fwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, const int32_t* block_counts, void* o, float* lse,
                               void* o_lo, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dsv_sparse_attn_bwd needs (0 if the problem is invalid). */
size_t dsv_sparse_attn_bwd_workspace_size(const dsv_problem* p);

/*
 * dsv_sparse_attn_bwd -- gradients of the sparse attention (the method trains
 * with it: [de] §2.A stage 2; [es] §2.A phase 2).  With P the sparse softmax of
 * the forward and dO = dout:
 *   dV_J += P^T dO,  dP = dO V_J^T,  dS = P o (dP - D),  D_i = sum_c dO_ic O_ic,
 *   dQ = sm_scale dS K_J,  dK_J += sm_scale dS^T Q.
 * o and lse must be the forward's outputs for the same q, k, v, block_idx.
 * No gradient flows to the predictor or to block_idx.
 *
 *   q, k, v, o, dout  [B, H, N, d];  lse [B, H, N];  block_idx [B, H, N/Bq, k]
 *   block_counts      the forward's block_counts, or NULL (all k)
 *   o_lo              the forward's o_lo output, or NULL (then D uses o alone).
 *                     DSV_BF16 only; must be NULL for DSV_F32.
 *   dq, dk, dv        [B, H, N, d] outputs (dtype), fully overwritten
 *   workspace         >= dsv_sparse_attn_bwd_workspace_size(p) bytes (256-byte aligned).
 *                     DSV_BF16: the row statistics, the transposed block lists, and fp16
 *                     copies of Q, K and dO (3 x B*H*N*d*2 bytes): every product of the
 *                     bf16 backward runs in fp16 on copies scaled per head by powers of two
 *                     (exact for bf16 values), with dS scaled before its fp16 rounding, and
 *                     every scale undone exactly.  Requires sm_scale in [2^-40, 2^40].
 */
dsv_status dsv_sparse_attn_bwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                               const void* o, const void* o_lo, const void* dout, const float* lse,
                               const int32_t* block_idx, const int32_t* block_counts, void* dq, void* dk,
                               void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Static English name of a status code. */
const char* dsv_status_string(dsv_status s);

/* Detail of the last failure on this thread ("" if none). */
const char* dsv_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t dsv_version(void);

/*
 * Kernel timing (diagnostics).  dsv_timing_begin() makes every kernel launch the
 * library issues from the calling thread be bracketed by two HIP events on the
 * launch's stream (a few microseconds of host overhead per launch; the GPU work
 * is unchanged).  dsv_timing_end() waits for those events, aggregates the
 * elapsed times by kernel name into `out` (at most `capacity` entries, in order
 * of first launch), frees the events, stops timing, and returns the number of
 * distinct names.  The only per-thread state of the library is this record.
 */
typedef struct {
  char name[64];
  int32_t launches;
  double total_ms;
  float min_ms;
  float max_ms;
} dsv_kernel_stat;

dsv_status dsv_timing_begin(void);
int32_t dsv_timing_end(dsv_kernel_stat* out, int32_t capacity);

/*
 * Peak-rate probes (measurement).  The rates this device sustains for the operations the hot
 * path's kernels are bound by, so that a kernel's rate can be stated as a fraction of a measured
 * peak beside the vendor's: the attention products run on the matrix cores (MFMA 32x32x16, bf16
 * and fp16 operands), the predictor on the transcendental unit (one v_exp_f32 per predicted
 * logit), selection and the copies on HBM.  Each probe kernel does only that operation, over
 * enough waves to fill every SIMD:
 *   DSV_PEAK_MFMA_BF16, DSV_PEAK_MFMA_F16   rate in flop/s (2*32*32*16 per instruction)
 *   DSV_PEAK_EXP_F32                        rate in exponentials/s
 *   DSV_PEAK_HBM_COPY                       rate in bytes/s, read + written, over 1 GiB of workspace
 *   DSV_PEAK_HBM_READ                       rate in bytes/s, loads only, over 1 GiB of workspace
 *
 *   kind        one of dsv_peak_kind
 *   repeats     launches to time, 1..100; the fastest is reported
 *   workspace   >= dsv_peak_probe_workspace_size(kind) bytes, 256-byte aligned, caller-owned
 *               device scratch (its contents are overwritten)
 *   rate        host pointer, receives the rate
 * Unlike every other call this one BLOCKS: it records HIP events around each launch on `stream`
 * and waits for them.  Errors: DSV_ERR_INVALID_ARGUMENT (unknown kind, repeats out of range, null
 * pointers), DSV_ERR_WORKSPACE_TOO_SMALL, DSV_ERR_HIP.
 */
typedef enum {
  DSV_PEAK_MFMA_BF16 = 0,
  DSV_PEAK_MFMA_F16 = 1,
  DSV_PEAK_EXP_F32 = 2,
  DSV_PEAK_HBM_COPY = 3,
  DSV_PEAK_HBM_READ = 4
} dsv_peak_kind;

/* Workspace bytes of a probe (0 for an unknown kind). */
size_t dsv_peak_probe_workspace_size(int32_t kind);
dsv_status dsv_peak_probe(int32_t kind, int32_t repeats, void* workspace, size_t workspace_bytes, double* rate,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSV_H_ */
