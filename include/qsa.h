/*
 * qsa.h -- C ABI of libqsa, the gfx950 (MI355X) forward pass of one Qwen
 * Sparse Attention (QSA) layer: the compressed lightweight indexer followed by
 * sparse core attention.
 *
 * Sources (cited by page title and section):
 *   [concept]  "QSA (Qwen Sparse Attention)" research-hub concept page,
 *              "Key math / How it works": (A) compressed lightweight indexer,
 *              (B) sparse core attention, and "Config" (K = 2048, r = 4).
 *   [gallery]  "Qwen Sparse Attention" architecture-gallery page: the
 *              selection unit/budget table, "How block selection works"
 *              (its pseudocode) and the QSA-vs-DSA table.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is DEVICE memory owned by the caller, dense and
 *     row-major in the layout stated.  The library never allocates, frees
 *     or synchronises; it only enqueues kernels on the caller's stream.
 *     Scratch memory comes from a caller-supplied workspace whose size
 *     qsa_workspace_size() returns.
 *   - Positions are absolute, 0-based token indices; K/V/raw-key row t of a
 *     sequence holds the token at position t.  Blocks are r = block_size
 *     consecutive positions: block b covers r*b .. r*b + r - 1.
 *   - dtype QSA_BF16: tensors marked "(dtype)" hold bf16; QSA_F32: fp32.
 *     Arithmetic always accumulates in fp32 (compression: fp64).
 *   - Host validation runs before anything is enqueued.  A non-QSA_OK
 *     return means nothing was launched; qsa_last_error() (thread-local)
 *     then describes the problem.  QSA_ERR_DEVICE reports a failed launch.
 *   - Device-resident position arrays are read by the kernels only.  They
 *     must satisfy the stated preconditions; kernels clamp every index so a
 *     violation gives wrong values, never an out-of-bounds access.
 *   - Calls are re-entrant and enqueue-only; concurrent calls on different
 *     streams must use different workspaces.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment    */
  QSA_ERR_UNSUPPORTED = 2,      /* a setting the library does not implement */
  QSA_ERR_WORKSPACE = 3,        /* workspace missing or too small          */
  QSA_ERR_DEVICE = 4            /* HIP reported an error at launch         */
} qsa_status;

typedef enum { QSA_F32 = 0, QSA_BF16 = 1 } qsa_dtype;

typedef enum {
  QSA_OP_INDEX_BUILD = 0,
  QSA_OP_SELECT = 1,
  QSA_OP_PREFILL = 2,
  QSA_OP_DECODE = 3,
  QSA_OP_DECODE_STEP = 4,
  QSA_OP_BACKWARD = 5,
  QSA_OP_DISTILL = 6
} qsa_op;

/* Layer configuration.  Supported values are listed per field; anything
 * else returns QSA_ERR_UNSUPPORTED (or INVALID_ARGUMENT when meaningless). */
typedef struct {
  int32_t block_size;    /* r: tokens per micro-block: 4 in the pages'
                            configuration ([concept] Config; [gallery]
                            selection-unit table); r = 1 selects single
                            tokens, the token-level end of the [gallery]
                            QSA-vs-DSA table.  Supported: a power of two
                            from 1 to 128 (qsa_decode_step: 4 only; the
                            backward, the distillation and the offload:
                            r >= 4).                                        */
  int32_t token_budget;  /* K: selected tokens; k_B = ceil(K / r) blocks are
                            kept ([concept] (A) top-k_B; Config K = 2048).
                            Supported: k_B * r <= 2048, and k_B <= 512 when
                            r >= 4 (so r = 1 keeps up to 2048 tokens).      */
  int32_t idx_heads;     /* indexer query heads sharing one key head: 4
                            ([concept] (A) MQA head layout).                */
  int32_t idx_dim;       /* indexer head dim: 128 ([concept] (A)).          */
  int32_t rope_dims;     /* rotated dims [0, rope_dims) of each compressed
                            key, rotate-half pairs (j, j + rope_dims/2):
                            64 of 128 ([concept] (A) partial RoPE).  Any
                            multiple of 4 up to idx_dim.                    */
  int32_t q_heads;       /* main attention query heads (Hq).                */
  int32_t kv_heads;      /* main attention KV heads (Hkv), Hq % Hkv == 0;
                            head h reads KV head floor(h * Hkv / Hq).       */
  int32_t head_dim;      /* main attention head dim: 64 or 128.             */
  int32_t dtype;         /* qsa_dtype of every tensor marked (dtype).       */
  float rms_eps;         /* RMSNorm epsilon of the pooled key (the pages
                            give none; 1e-6 is the customary value).        */
  float softmax_scale;   /* attention logit scale; <= 0 means
                            1/sqrt(head_dim) ([concept] (B) "scaled").      */
  double rope_base;      /* RoPE base: theta_j = base^(-2j/rope_dims).      */
} qsa_config;

/* qsa_index_build -- block compression of the indexer keys.
 * [concept] (A) block compression and partial RoPE; [gallery] "How block
 * selection works": the keys of each complete block are averaged, the
 * pooled key is normalised, then rotated at the block's first position.
 *
 * For every sequence s, builds each block b with
 *     floor(len_before[s] / r) <= b < floor(len_after[s] / r)
 * as  k_cmp[s][b] = RoPE_{r*b}( RMSNorm( mean_{t<r} k_idx[s][r*b+t] ) * gain ),
 * computed in fp64 and rounded to nearest-even into the storage dtype.
 *
 *   k_idx      (dtype) [batch][cap_tokens][idx_dim] raw indexer keys.
 *   len_before int32 [batch] device: tokens already covered by built blocks.
 *   len_after  int32 [batch] device: tokens present after this call
 *              (precondition: len_before <= len_after <= cap_tokens).
 *   max_new_blocks  host upper bound of floor(len_after/r) -
 *              floor(len_before/r) over sequences; sizes the grid only
 *              (every block in range is built whatever the bound).
 *   rms_gain   float [idx_dim] device, or NULL for a gain of 1.
 *   k_cmp      (dtype) [batch][cap_tokens / r][idx_dim]; only the rows of
 *              the built blocks are written.
 * A decode step calls it with len_after = len_before + 1; it builds a block
 * only when that token completes one.                                     */
qsa_status qsa_index_build(const qsa_config* cfg, int32_t batch, const void* k_idx,
                           int64_t cap_tokens, const int32_t* len_before,
                           const int32_t* len_after, int32_t max_new_blocks,
                           const float* rms_gain, void* k_cmp, hipStream_t stream);

/* qsa_select_topk -- block importance and top-k_B block selection.
 * [concept] (A) block-importance equation I_ib = sum_h ReLU(<q_i^h, k_b>)
 * with block-causal masking, and top-k_B selection; [gallery] pseudocode
 * ("scores", "selected_blocks") and budget table (up to 512 blocks).
 *
 * Query j of sequence s sits at position p = q_pos0[s] + j.  Its candidate
 * blocks are the complete blocks before its own block, b < c = floor(p/r).
 * It keeps count = min(k_B, c) blocks of largest I; equal scores go to the
 * lower block id.  The selection is written in ascending block order.
 *
 *   q_idx      (dtype) [batch][n_q][idx_heads][idx_dim], used as given.
 *   q_pos0     int32 [batch] device.
 *   max_pos_end host bound: q_pos0[s] + n_q <= max_pos_end <= cap_tokens.
 *   k_cmp      (dtype) [batch][cap_tokens / r][idx_dim]; blocks < c built.
 *   sel_blocks int32 [batch][n_q][k_B]: ascending ids, then -1 padding.
 *   sel_count  int32 [batch][n_q].
 *   sel_scores float [batch][n_q][k_B] or NULL: I of each selected block
 *              (same order as sel_blocks; 0 in padding).  With bf16 data
 *              and n_q >= 16 the scores are kept as 16-bit keys (the top
 *              half of the fp32 bits, truncated: relative error below
 *              2^-7); blocks whose keys tie at the selection threshold are
 *              rescored in fp32 to decide the selection, and report that
 *              fp32 value.  The selection itself follows the fp32 scores.
 *   workspace  >= qsa_workspace_size(QSA_OP_SELECT, batch, n_q, max_pos_end).
 */
qsa_status qsa_select_topk(const qsa_config* cfg, int32_t batch, int32_t n_q,
                           const void* q_idx, const int32_t* q_pos0, int32_t max_pos_end,
                           const void* k_cmp, int64_t cap_tokens, int32_t* sel_blocks,
                           int32_t* sel_count, float* sel_scores, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* qsa_sparse_attn_prefill -- sparse core attention for a chunk of queries.
 * [concept] (B): full scaled-dot-product attention restricted to the
 * selected blocks' tokens; [concept] (A) and [gallery] pseudocode/table:
 * each selected block is expanded to its r tokens and the visible tokens of
 * the query's own (incomplete) block are always added.
 *
 * The token set of the query at p is S = { r*b + t : b in selection, t < r }
 * plus the tail r*floor(p/r) .. p; every main head attends over S.
 *
 *   q          (dtype) [batch][n_q][q_heads][head_dim].
 *   k_cache, v_cache (dtype) [batch][cap_tokens][kv_heads][head_dim];
 *              rows 0 .. p written for every query.
 *   q_pos0, max_pos_end  as in qsa_select_topk.
 *   sel_blocks, sel_count  as written by qsa_select_topk (any ascending or
 *              unordered list of distinct complete blocks b < floor(p/r)).
 *   out        (dtype) [batch][n_q][q_heads][head_dim].
 *   lse        float [batch][n_q][q_heads] natural-log normaliser, or NULL.
 *   workspace  >= qsa_workspace_size(QSA_OP_PREFILL, ...).  For bf16 with 16
 *              query heads, (kv_heads, head_dim) in {(2,128), (2,64),
 *              (1,128)} and block_size >= 2: 8 bytes per query row (a sort
 *              key and a walk start),
 *              12 when batch*n_q >= 1024 and batch <= 1024 (plus a slot of the
 *              row order); else 0 bytes.  Rows whose selections cluster in
 *              one region of the cache are run together, each starting its
 *              walk in that region, so that their K/V reads hit the same L2.
 *              A row's bits depend on its own inputs only, not on the call.
 */
qsa_status qsa_sparse_attn_prefill(const qsa_config* cfg, int32_t batch, int32_t n_q,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   int64_t cap_tokens, const int32_t* q_pos0,
                                   int32_t max_pos_end, const int32_t* sel_blocks,
                                   const int32_t* sel_count, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* qsa_sparse_attn_decode -- sparse core attention for one new token per
 * sequence (the decode loop), split over the token set for parallelism and
 * combined with a log-sum-exp merge.  Same token set as the prefill call.
 * [concept] (B); the concept page's "Why it matters" reports decode-phase
 * kernel speed-ups at 1M context.
 *
 *   q          (dtype) [batch][q_heads][head_dim].
 *   q_pos      int32 [batch] device: position of the new token, whose K/V
 *              rows are already written.  max_pos_end > every q_pos[s].
 *   sel_blocks int32 [batch][k_B]; sel_count int32 [batch].
 *   out        (dtype) [batch][q_heads][head_dim]; lse float [batch][q_heads]
 *              or NULL.
 *   workspace  >= qsa_workspace_size(QSA_OP_DECODE, batch, 1, max_pos_end).
 */
qsa_status qsa_sparse_attn_decode(const qsa_config* cfg, int32_t batch, const void* q,
                                  const void* k_cache, const void* v_cache, int64_t cap_tokens,
                                  const int32_t* q_pos, int32_t max_pos_end,
                                  const int32_t* sel_blocks, const int32_t* sel_count,
                                  void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* qsa_decode_step -- one whole decode step in a single launch:
 * qsa_index_build of the block the new token may complete (len_before =
 * q_pos, len_after = q_pos + 1), qsa_select_topk for the new token (n_q = 1)
 * and qsa_sparse_attn_decode, with results bit-identical to those three
 * calls.  [concept] (A) and (B), and the decode-phase report under "Why it
 * matters"; [gallery] "How block selection works".  The stages hand their
 * data to each other inside the launch (score -> selection -> attention ->
 * split merge) instead of across kernel boundaries.
 *
 *   q_idx      (dtype) [batch][idx_heads][idx_dim] indexer query of the new
 *              token of each sequence.
 *   q          (dtype) [batch][q_heads][head_dim] its main query.
 *   k_idx, k_cmp, rms_gain   as in qsa_index_build; k_idx row q_pos[s] holds
 *              the new token's raw indexer key.  Only the completed block's
 *              row of k_cmp is written (it is not a candidate of this step).
 *   k_cache, v_cache, cap_tokens, q_pos, max_pos_end   as in
 *              qsa_sparse_attn_decode (the new token's K/V rows written).
 *   sel_blocks, sel_count, sel_scores   as in qsa_select_topk with n_q = 1.
 *   out, lse   as in qsa_sparse_attn_decode.
 *   workspace  >= qsa_workspace_size(QSA_OP_DECODE_STEP, batch, 1,
 *              max_pos_end) bytes.  Its first 3,325,952 bytes are a control
 *              area that must be ZERO-FILLED BEFORE THE FIRST CALL; between
 *              calls it holds the calls' own state, which the caller leaves
 *              alone (zero-filling it again between calls is always
 *              allowed).  As int32 words: per-row generation words at 0
 *              (row s: calls made since the last fill), the error word at
 *              2048, per-row split flags at 4096 + 32 s, per-row scoring
 *              flags at 36864 + 264 s, and two buffers of 256 per-row
 *              score-bin counts at 307200 + 512 s.  The error word is 1 if a
 *              wait ever gave up (never expected; the outputs of that call
 *              are then invalid, and the area must be zero-filled again).
 * Supported: dtype bf16, block_size 4, idx_heads 4, q_heads 16 with
 * (kv_heads, head_dim) in {(2,128), (2,64), (1,128)}, batch <= 1024 and
 * floor((max_pos_end-1)/r)
 * <= 264192 (contexts up to 1,056,768 tokens); anything else returns
 * QSA_ERR_UNSUPPORTED and the three separate calls apply.                  */
qsa_status qsa_decode_step(const qsa_config* cfg, int32_t batch, const void* q_idx,
                           const void* q, const void* k_idx, void* k_cmp,
                           const float* rms_gain, const void* k_cache, const void* v_cache,
                           int64_t cap_tokens, const int32_t* q_pos, int32_t max_pos_end,
                           int32_t* sel_blocks, int32_t* sel_count, float* sel_scores,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* qsa_decode_step_noalloc -- qsa_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and results
 * as qsa_decode_step, without the workspace: the step workspace is a 32 MiB
 * array in the library's own device memory, one per GPU, held until the
 * process ends.  The call allocates nothing.  The first call on a device
 * also enqueues a clear of the array's control area on its stream; later
 * calls keep their state there, as qsa_decode_step's calls do.
 *   Limits: sizes whose qsa_workspace_size(QSA_OP_DECODE_STEP, batch, 1,
 *   max_pos_end) exceeds 32 MiB return QSA_ERR_UNSUPPORTED (batch 8 at
 *   256K context needs about 11 MB).
 *   Concurrency: every call on a GPU uses that GPU's one array, so calls
 *   that overlap on one GPU (other streams, other threads) race and give
 *   wrong results; order them on one stream.  If a call's wait ever gives
 *   up (word 2048 of the control area, as in qsa_decode_step), the array is
 *   not readable from the host: that call's outputs are invalid and later
 *   calls may be too.                                                      */
qsa_status qsa_decode_step_noalloc(const qsa_config* cfg, int32_t batch, const void* q_idx,
                                   const void* q, const void* k_idx, void* k_cmp,
                                   const float* rms_gain, const void* k_cache,
                                   const void* v_cache, int64_t cap_tokens, const int32_t* q_pos,
                                   int32_t max_pos_end, int32_t* sel_blocks, int32_t* sel_count,
                                   float* sel_scores, void* out, float* lse, hipStream_t stream);

/* Workspace bytes needed by op (a qsa_op) for these sizes.  n_q is 1 for
 * QSA_OP_DECODE and QSA_OP_DECODE_STEP; QSA_OP_INDEX_BUILD needs none.  The
 * select workspace holds the materialised score rows, per-segment score
 * histograms and the candidate hand-over area of long rows; it carries no
 * state between calls (the decode-step workspace does: see above).
 * Alignment: tensors read with 16-byte vector loads (q_idx, k_cmp
 * in select, q, k_cache, v_cache, workspaces) must be 16-byte aligned, the
 * others 4- or 8-byte aligned as the validation messages state.           */
qsa_status qsa_workspace_size(const qsa_config* cfg, int32_t op, int32_t batch, int32_t n_q,
                              int32_t max_pos_end, size_t* bytes);

const char* qsa_status_string(qsa_status status);
const char* qsa_last_error(void);  /* thread-local text of the last failure */
/* qsa_sparse_attn_backward -- gradients of qsa_sparse_attn_prefill.
 * The pages define the forward only ([concept] (B) over the token sets of
 * (A)); this is its exact derivative with every query's token set held
 * fixed: the selection is piecewise constant, so no gradient reaches the
 * indexer through it.  Per query, head h (KV head g) and token j of S:
 *   P_j = exp(scale <q_h, K_j> - lse_h),  dP_j = <dO_h, V_j>,
 *   D_h = sum_j P_j dP_j,  dS_j = P_j (dP_j - D_h),
 *   dq_h = scale sum_j dS_j K_j,  dK_j += scale dS_j q_h,  dV_j += P_j dO_h.
 *
 *   q, k_cache, v_cache, q_pos0, max_pos_end, sel_blocks, sel_count
 *              as given to the forward call.
 *   out        (dtype) [batch][n_q][q_heads][head_dim]: the forward output.
 *              bf16 layers with 16 query heads read it for a reference
 *              D~ = <dO, out> that keeps the dq weights small; D itself is
 *              always recomputed from the token set, so the result is exact
 *              (up to rounding) for any out, most accurate for the forward's.
 *              Other layouts validate it only.
 *   lse        float [batch][n_q][q_heads]: the forward's log-sum-exp.
 *   dout       (dtype) [batch][n_q][q_heads][head_dim]: dL/dout.
 *   dq         (dtype) [batch][n_q][q_heads][head_dim]: written.
 *   dk, dv     float [batch][cap_tokens][kv_heads][head_dim]: the gradients
 *              of this call are ADDED (zero them first, or accumulate the
 *              chunks of a sequence); rows no query attends are untouched.
 *   workspace  >= qsa_workspace_size(QSA_OP_BACKWARD, batch, n_q,
 *              max_pos_end): transposed query lists and per-head sums; for
 *              bf16 layers with 16 query heads also q/dO transposed and
 *              8 bytes per (query, token of its set, head) of softmax
 *              values -- about 4.3 GB for 16,384 queries at k_B = 512 --
 *              and 12 bytes per query of row order (queries whose
 *              selections cluster in one region of the cache run together,
 *              as in the forward).  Nothing is kept in it between calls.
 * Supported: kv_heads <= 2 (any dtype, head_dim, block size the forward
 * takes); sel_blocks ascending without repeats, as qsa_select_topk writes
 * them.  dq is deterministic; dk/dv sum each token's queries in an order
 * that can change from run to run (the last bits can differ).             */
qsa_status qsa_sparse_attn_backward(const qsa_config* cfg, int32_t batch, int32_t n_q,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    int64_t cap_tokens, const int32_t* q_pos0,
                                    int32_t max_pos_end, const int32_t* sel_blocks,
                                    const int32_t* sel_count, const void* out, const float* lse,
                                    const void* dout, void* dq, float* dk, float* dv,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* qsa_index_build_backward -- gradient back through qsa_index_build.
 * For the blocks qsa_index_build builds with the same (len_before,
 * len_after), adds dL/dk_idx given dL/dk_cmp: the rotation transposed
 * (RoPE at minus the block's angle), the RMSNorm Jacobian
 *     dx = (g dy) / rms - x sum(g dy x) / (idx_dim rms^3),
 *     rms = sqrt(mean(x^2) + eps),  x = the block mean,
 * then dx / r to each of the block's r rows; the storage rounding of k_cmp
 * is passed straight through.  fp64 arithmetic, as the forward.
 *
 *   k_idx, len_before, len_after, max_new_blocks, rms_gain
 *              as given to qsa_index_build (batch <= 65535).
 *   dk_cmp     float [batch][cap_tokens / r][idx_dim]: dL/dk_cmp.
 *   dk_idx     float [batch][cap_tokens][idx_dim]: ADDED into at the rows of
 *              the blocks in range.                                        */
qsa_status qsa_index_build_backward(const qsa_config* cfg, int32_t batch, const void* k_idx,
                                    int64_t cap_tokens, const int32_t* len_before,
                                    const int32_t* len_after, int32_t max_new_blocks,
                                    const float* rms_gain, const float* dk_cmp, float* dk_idx,
                                    hipStream_t stream);

/* qsa_indexer_distill -- stage-1 indexer distillation loss and gradients.
 * [concept] "Native trainability", stage 1: only the indexer trains, its
 * scores pulled by a KL divergence toward the dense model's attention after
 * a max over each block, while the model still attends densely.  The pages
 * leave the details open; taken here: for the query at p (c = floor(p/r) candidate
 * blocks), the teacher is the dense causal attention over tokens 0..p
 * averaged over the q_heads heads (head h reads KV head h*Hkv/Hq, the
 * forward's scale); t_b is its max over block b's r tokens, renormalised over
 * b < c; the student is softmax_b(I_b) over the same blocks, I as in
 * qsa_select_topk; the loss of the query is KL(t || softmax(I)), 0 when
 * c = 0.  The teacher sends no gradient; ReLU'(0) = 0.  With
 * dI_b = softmax(I)_b - t_b:
 *     dq_idx^h = sum_b dI_b [<q_idx^h, k_b> > 0] k_b,
 *     dk_cmp_b += sum over the call's queries of dI_b sum_h [..] q_idx^h.
 *
 *   q, k_cache, cap_tokens, q_pos0, max_pos_end
 *              as for qsa_sparse_attn_prefill (the teacher's query rows and
 *              keys; values are not needed).
 *   q_idx, k_cmp  as for qsa_select_topk (blocks below floor(p/r) built).
 *   loss       float [batch][n_q]: each query's KL, written.
 *   dq_idx     float [batch][n_q][idx_heads][idx_dim]: written.
 *   dk_cmp     float [batch][cap_tokens / r][idx_dim]: ADDED into.
 *   workspace  >= qsa_workspace_size(QSA_OP_DISTILL, batch, n_q,
 *              max_pos_end): per-head teacher sums, the teacher's maximum
 *              per (query, 4-token unit), and per (query, candidate block)
 *              I_b / dI_b and the ReLU mask; with bf16 and 4 indexer heads
 *              also q_idx and k_cmp regrouped for the MFMA operands
 *              (about 5 GB for 16,384 queries over 135K tokens).  Nothing is
 *              kept between calls.
 * Supported: q_heads <= 16, kv_heads <= 2, head_dim a multiple of 8 up to
 * 128, idx_heads <= 8, every dtype and block size of the forward.       */
qsa_status qsa_indexer_distill(const qsa_config* cfg, int32_t batch, int32_t n_q, const void* q,
                               const void* k_cache, int64_t cap_tokens, const int32_t* q_pos0,
                               int32_t max_pos_end, const void* q_idx, const void* k_cmp,
                               float* loss, float* dq_idx, float* dk_cmp, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* qsa_offload_stage -- decode with the KV history in host memory.
 * The "QSA" knowledge-card page (Timeline; All Facts) reports a serving
 * port that keeps the full history in host memory, only hot data and a
 * staging area in GPU memory, fetching on demand what each layer's own
 * selection picks.  Taken here: for each sequence's decode query at
 * q_pos[s], with the selection of qsa_select_topk (made on the compressed
 * index, which stays in GPU memory), gathers the query's token set -- the
 * selected blocks in ascending order, then the tail -- into stage_k /
 * stage_v, 4-token unit by unit: from the hot cache when the unit's slot
 * (unit id mod hot_units) holds it, else from host memory; then writes the
 * missed units into their slots (one per slot when several miss to it).
 * Only complete units (all four rows at or before q_pos[s]) are cached or
 * read from the cache; the unit holding q_pos[s] always comes from host
 * memory, since its later rows are written by later steps.  It also writes
 * the selection in staging coordinates, so that
 *     qsa_sparse_attn_decode(cfg, batch, q, stage_k, stage_v, stage_tokens,
 *                            stage_pos, stage_tokens, stage_sel, stage_cnt, ...)
 * attends over exactly the query's token set (in another order: equal up to
 * the rounding of the softmax sums).
 *
 *   q_pos, sel_blocks, sel_count  as for qsa_sparse_attn_decode.
 *   k_host, v_host  bf16 [batch][cap_tokens][kv_heads][head_dim] in pinned,
 *              device-mapped host memory (hipHostMalloc); read only.  Row t
 *              must hold its final value from the step at position t on and
 *              never change after (the hot cache keeps copies).
 *   hot_k, hot_v    bf16 [batch][hot_units][4][kv_heads][head_dim] GPU memory.
 *   hot_tag    int32 [batch][hot_units]: the unit each slot holds, -1 for
 *              none; the caller fills it with -1 once; every call keeps it
 *              consistent with hot_k / hot_v.
 *   stage_k, stage_v  bf16 [batch][stage_tokens][kv_heads][head_dim] GPU
 *              memory, stage_tokens >= (k_B + 1) * block_size.
 *   stage_sel int32 [batch][k_B], stage_cnt int32 [batch],
 *   stage_pos int32 [batch]: written (blocks 0 .. count-1, -1 padding; the
 *              query's position in the staging buffer).
 *   stats      int32 [batch][2]: units read from the hot cache, from host.
 * Supported: block_size >= 4 (units of 4 tokens).  Calls on one stream are
 * ordered; concurrent calls must not share a hot cache.                   */
qsa_status qsa_offload_stage(const qsa_config* cfg, int32_t batch, const int32_t* q_pos,
                             const int32_t* sel_blocks, const int32_t* sel_count,
                             const void* k_host, const void* v_host, int64_t cap_tokens,
                             void* hot_k, void* hot_v, int32_t* hot_tag, int32_t hot_units,
                             void* stage_k, void* stage_v, int64_t stage_tokens,
                             int32_t* stage_sel, int32_t* stage_cnt, int32_t* stage_pos,
                             int32_t* stats, hipStream_t stream);

/* qsa_abi_version -- 2: the prefill attention and the backward take a
 * workspace for their row order (version 1 took none for the prefill).    */
int32_t qsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QSA_H */
