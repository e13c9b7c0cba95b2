/*
 * mp.h -- C ABI of libmp, one GPU's share of a Megatron-style tensor
 * (intra-layer) model-parallel transformer layer, for AMD MI355X (gfx950).
 *
 * Pages this library follows (title, then the section on that page):
 *   MLM-review  "[NLP Paper Review] Megatron-LM: Training Multi-Billion
 *               Parameter Language Models Using Model Parallelism"
 *   PAR-survey  "From GPU Engineering to Scientific Discovery: Parallelism
 *               Techniques for Large Language Models"
 *   MLM-notes   "GTC-2020 Megatron-LM: Training Multi-Billion Parameter
 *               Language Models Using Model Parallelism"
 *   MOE-core    "Scalable Training of Mixture-of-Experts Models with
 *               Megatron Core" (technical summary, sections 1 and 2.1-2.6)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Status: every call returns MP_OK (0) or a negative MP_ERR_* code and never
 *   throws.  mp_last_error() returns a thread-local message for the last
 *   failing call on the calling thread.
 * - Asynchrony: calls validate their host-visible arguments, enqueue kernels
 *   on the caller's stream `s` (0 = the legacy default stream) and return
 *   without synchronising.  A validation failure enqueues nothing.
 * - Ownership: the caller owns every buffer (inputs, outputs, workspaces and
 *   host arrays of device pointers).  Device buffers must stay alive until the
 *   stream has executed the enqueued work; host arrays are read before the
 *   call returns.  The library allocates no device memory and keeps no
 *   pointer after a call returns.
 * - Layout: row-major.  Tokens are flattened t = b*L + l, activations are
 *   [T, features]; weights are stored [out, in] (K-contiguous).  The fused
 *   QKV weight of a rank holds the Q rows of its heads, then the K rows, then
 *   the V rows, d consecutive rows per head; rank i of N owns heads
 *   [i*h, (i+1)*h) of the full model.
 * - Dtypes: MP_BF16 (bfloat16 storage, fp32 accumulation, round-to-nearest-
 *   even on output) or MP_F32.  Weight and bias gradients are always fp32.
 * - Alignment: every device pointer must be 16-byte aligned (MP_ERR_ALIGN);
 *   the contiguous dimension of every bf16 matrix must be a multiple of 8
 *   and of every fp32 matrix a multiple of 4 (MP_ERR_SHAPE), so rows stay
 *   16-byte aligned.
 * - Device-data preconditions (labels and token ids in [0, V), expert ids
 *   in [0, E)) are documented, not checked on the fast path.  With the
 *   environment variable MP_DEBUG_CHECKS set (to anything but "0"), every
 *   call that reads labels, token ids or expert ids first copies them to the
 *   host (synchronising its stream) and fails with MP_ERR_DATA if one is
 *   negative -- the one bound a single shard can check, since it is not told
 *   V or E.  mp_check_indices checks a full range on the device.
 * - Only gfx950 is supported; mp_device_supported() says so per device.
 */
#ifndef MP_H
#define MP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ types */

/* The two range sentinels make every int a valid mp_dtype value, so a bad
 * value from a caller is rejected with MP_ERR_DTYPE rather than being
 * undefined behaviour once it is read as the enum type. */
typedef enum {
  MP_F32 = 0,
  MP_BF16 = 1,
  MP_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  MP_DTYPE_RANGE_MAX_ = 2147483647
} mp_dtype;

/* Activation of the column-parallel linear.  GeLU is not defined on the
 * pages; MP_ACT_GELU_ERF is the exact z*Phi(z) (via erf), MP_ACT_GELU_TANH the
 * tanh approximation. */
typedef enum {
  MP_ACT_NONE = 0,
  MP_ACT_GELU_ERF = 1,
  MP_ACT_GELU_TANH = 2,
  MP_ACT_RANGE_MIN_ = -2147483647 - 1,
  MP_ACT_RANGE_MAX_ = 2147483647
} mp_act;

#define MP_OK              0
#define MP_ERR_NULL       -1  /* a required pointer is NULL                     */
#define MP_ERR_SHAPE      -2  /* non-positive / inconsistent / indivisible dims */
#define MP_ERR_DTYPE      -3  /* dtype not supported by this call               */
#define MP_ERR_UNSUPPORTED -4 /* e.g. head dim not in {64,128}, not gfx950      */
#define MP_ERR_ALIGN      -5  /* a device pointer is not 16-byte aligned        */
#define MP_ERR_WORKSPACE  -6  /* workspace NULL or smaller than required        */
#define MP_ERR_HIP        -7  /* a HIP runtime call or kernel launch failed     */
#define MP_ERR_ARG        -8  /* an argument value is out of range (e.g. p)     */
#define MP_ERR_DATA       -9  /* device data violates a precondition (debug)    */

#define MP_MAX_SHARDS 16      /* largest N accepted by the reduce/combine calls */

/* ------------------------------------------------------------ utilities */

/* Library version, major*10000 + minor*100 + patch. */
int mp_version(void);

/* Data check of an index array (labels or token ids against [0, V), expert
 * ids against [0, E)), for callers that validate inputs before the hot path:
 * *bad_count (device memory, 8-byte aligned) receives the number of
 * idx[0..n) outside [lo, hi), enqueued on s (no synchronisation; read it
 * after the stream reaches this point).  The count is exact (integer
 * atomics).  Errors: MP_ERR_SHAPE (n < 0 or lo > hi), MP_ERR_NULL,
 * MP_ERR_ALIGN. */
int mp_check_indices(const int32_t* idx, int64_t n, int64_t lo, int64_t hi, uint64_t* bad_count,
                     hipStream_t s);

/* MP_OK if device `device` is a gfx950 part, MP_ERR_UNSUPPORTED otherwise,
 * MP_ERR_HIP if the device cannot be queried. */
int mp_device_supported(int device);

/* Message describing the last failing call on this thread ("" if none). */
const char* mp_last_error(void);

/* ------------------------------------------- column- and row-parallel MLP */

/* Column-parallel linear with fused bias + activation (MLM-notes, "Model
 * Parallel Transformers", MLP paragraph; PAR-survey, "How": column parallelism
 * splits the output dimension; MLM-review, "approach": GEMM fusion).
 *   Y_i = act(X * A_i^T + a_i)
 * X [T,K] (in_dtype), A_i [Fi,K] (in_dtype; the rank's rows of A), a_i [Fi]
 * (in_dtype) or NULL, Y_i [T,Fi] (out_dtype), Z_save [T,Fi] (out_dtype) or
 * NULL: receives the pre-activation X*A_i^T + a_i for the backward.
 * in_dtype MP_BF16 runs on bf16 MFMA; MP_F32 on an fp32 path (out must then
 * be MP_F32).  act = MP_ACT_NONE with out_dtype = MP_F32 is the vocab-parallel
 * logits GEMM Z_i = H * E_i^T (MLM-notes, output paragraph). */
int mp_column_linear_gelu(mp_dtype in_dtype, mp_dtype out_dtype, int64_t T, int64_t K,
                          int64_t Fi, const void* X, const void* A_i, const void* a_i,
                          int act, void* Y_i, void* Z_save, hipStream_t s);

/* Workspace bytes mp_column_linear_gelu_bwd needs for these sizes. */
size_t mp_column_linear_gelu_bwd_workspace(mp_dtype dtype, int64_t T, int64_t K, int64_t Fi);

/* Backward of mp_column_linear_gelu (dtype = in_dtype = out_dtype of the
 * forward).  dZ = dY_i * act'(Z_save);  dX_partial = dZ * A_i  [T,K] (dtype),
 * this rank's share of the input gradient (summing the shares with
 * mp_shard_reduce is the backward all-reduce, MLM-notes "Model Parallel
 * Transformers", communication paragraph);  dA_i = dZ^T * X  [Fi,K] fp32;
 * da_i = column sums of dZ [Fi] fp32 or NULL.  Z_save may be NULL only when
 * act = MP_ACT_NONE. */
int mp_column_linear_gelu_bwd(mp_dtype dtype, int64_t T, int64_t K, int64_t Fi,
                              const void* X, const void* A_i, const void* Z_save,
                              const void* dY_i, int act, void* dX_partial, float* dA_i,
                              float* da_i, void* ws, size_t ws_bytes, hipStream_t s);

/* Row-parallel linear, partial sum (MLM-notes, "Model Parallel Transformers";
 * PAR-survey, "How": row parallelism splits the input dimension).
 *   P_i = Y_i * B_i^T           (no bias: it is added once, after the sum)
 * Y_i [T,Fi], B_i [K,Fi] (the rank's columns of B, contiguous), P_i [T,K]. */
int mp_row_linear_partial(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K, const void* Y_i,
                          const void* B_i, void* P_i, hipStream_t s);

/* Workspace bytes mp_row_linear_partial_bwd needs. */
size_t mp_row_linear_partial_bwd_workspace(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K);

/* Backward of mp_row_linear_partial: dY_i = dOut * B_i [T,Fi] (dtype) and
 * dB_i = dOut^T * Y_i [K,Fi] fp32, with dOut [T,K] the replicated upstream
 * gradient of the reduced output. */
int mp_row_linear_partial_bwd(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K,
                              const void* Y_i, const void* B_i, const void* dOut, void* dY_i,
                              float* dB_i, void* ws, size_t ws_bytes, hipStream_t s);

/* mp_row_linear_partial_bwd without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results (bit for
 * bit) and errors as mp_row_linear_partial_bwd, minus ws/ws_bytes: the
 * split-K partials of the weight gradient go to a static scratch array of
 * mp_row_linear_partial_bwd_static_max_bytes() bytes (64 MiB) that the
 * library holds on every GPU it runs on until the process ends.  A shape
 * whose partials need more (mp_row_linear_partial_bwd_workspace > that)
 * fails with MP_ERR_WORKSPACE before anything is enqueued.  The call
 * allocates nothing; the first call on a device looks up the array's
 * address there.  Every call on one GPU shares the array: calls that
 * overlap in time on one GPU (different streams, or threads) race on it
 * and must be serialised by the caller.  Nothing in it needs clearing: each
 * call writes every partial it reads. */
size_t mp_row_linear_partial_bwd_static_max_bytes(void);
int mp_row_linear_partial_bwd_static(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K,
                                     const void* Y_i, const void* B_i, const void* dOut,
                                     void* dY_i, float* dB_i, hipStream_t s);

/* mp_row_linear_partial_bwd for the second GEMM of the MLP block, whose input
 * Y_i = act(Z_save) came from mp_column_linear_gelu (MLM-notes, "Model
 * Parallel Transformers": the GeLU sits between the column- and the
 * row-parallel GEMM of one rank).  The input gradient leaves the GEMM already
 * passed through the activation gradient:
 *   dZ_i = (dOut * B_i) .* act'(Z_save)   [T,Fi] (dtype, one rounding)
 * so mp_column_linear_gelu_bwd then runs with act = MP_ACT_NONE on dZ_i.
 * dB_i, workspace (mp_row_linear_partial_bwd_workspace) and errors as
 * mp_row_linear_partial_bwd; act must be a GeLU and Z_save [T,Fi] non-NULL. */
int mp_row_linear_partial_bwd_dact(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K,
                                   const void* Y_i, const void* B_i, const void* dOut,
                                   const void* Z_save, int act, void* dZ_i, float* dB_i,
                                   void* ws, size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------ reduce and dropout */

/* Local N-way shard reduce standing in for the all-reduce after each
 * partitioned block (MLM-notes, "Model Parallel Transformers": one all-reduce
 * completes the layer), with the replicated bias, the synchronised dropout
 * (MLM-review, "key terms") and the residual fused:
 *   out = residual + Drop(sum_{j=0..N-1} partials[j] + bias)
 * partials: host array of N device pointers, each [rows,cols] in dtype,
 * summed in fp32 in order j = 0..N-1.  bias [cols] or NULL, residual
 * [rows,cols] or NULL, out [rows,cols] (may alias residual), mask_out: the
 * keep flags as bits (format as in mp_shared_seed_dropout) or NULL; for the
 * backward, see mp_dropout_mask_bwd.  Dropout as mp_shared_seed_dropout with
 * element (r,c) at flat index index_base + r*cols + c.  1 <= N <= MP_MAX_SHARDS;
 * 0 <= p < 1 (p = 0: no dropout). */
int mp_shard_reduce(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                    const void* const* partials, const void* bias, const void* residual,
                    float p, uint64_t seed, uint64_t offset, uint64_t index_base, void* out,
                    uint8_t* mask_out, hipStream_t s);

/* Shared-seed dropout (MLM-review, "key terms" and "approach": every device
 * applies the same mask).  Element j (flat index index_base + i of x[i]) is
 * kept iff word (j mod 4) of Philox4x32-10(counter = (j div 4 as 64 bits,
 * offset as 64 bits), key = seed) is >= floor(p * 2^32) computed from the
 * float32 p; kept values are scaled by 1/(1-p), the rest set to 0.  The mask
 * depends on (seed, offset, j) only, never on the rank, so every shard draws
 * it identically; applied to an upstream gradient with the same arguments it
 * is the backward.  x, y [n] in dtype (y may alias x).  mask_out: NULL, or
 * ceil(n/8) bytes receiving the keep flags as bits, bit (i & 7) of byte i >> 3
 * for x[i] (1 = kept), so a backward can apply the mask without drawing it
 * again (mp_dropout_mask_bwd). */
int mp_shared_seed_dropout(mp_dtype dtype, int64_t n, const void* x, void* y,
                           uint8_t* mask_out, float p, uint64_t seed, uint64_t offset,
                           uint64_t index_base, hipStream_t s);

/* Backward of a dropout whose forward saved its keep flags as bits (mask_out
 * of mp_shared_seed_dropout, mp_shard_reduce or mp_shard_reduce_layernorm;
 * MLM-review, "key terms": the mask is the one all ranks drew from the shared
 * seed, and its backward reuses it):
 *   dx = dy .* keep / (1 - p)        [rows,cols] dtype (dx may alias dy)
 *   dbias = column sums of dx        [cols] fp32 or NULL: the gradient of the
 *                                    bias added before the dropout.
 * keep_bits: ceil(rows*cols/8) bytes, element (r,c) at bit index r*cols + c.
 * ws: mp_dropout_mask_bwd_workspace bytes when dbias is non-NULL.  The column
 * sums are of dx as stored, in a fixed order (deterministic). */
size_t mp_dropout_mask_bwd_workspace(int64_t rows, int64_t cols);
int mp_dropout_mask_bwd(mp_dtype dtype, int64_t rows, int64_t cols, const void* dy,
                        const uint8_t* keep_bits, float p, void* dx, float* dbias, void* ws,
                        size_t ws_bytes, hipStream_t s);

/* All-gather stand-in for the sequence-parallel layer (PAR-survey,
 * "Achievement" item 4 and the sequence-parallelism bullet of "How": with
 * TP+SP the operations outside the tensor-parallel GEMMs -- LayerNorm,
 * dropout, the residual -- are spread over the ranks along the sequence).
 * Reading (the page names no collective): each per-block all-reduce splits
 * into a reduce-scatter, after which those operations work on the rank's
 * token slice, and an all-gather that restores the full sequence before the
 * next column-parallel GEMM.  out [N*rows, cols] receives slice j
 * (a host array of N device pointers, each [rows, cols] dtype) in rows
 * [j*rows, (j+1)*rows); slices[j] may be those very rows of out.  The
 * reduce-scatter side needs no call of its own: it is mp_shard_reduce,
 * mp_shard_reduce_layernorm or their backward on the rank's rows of each
 * partial, with index_base = first row * cols so the dropout mask is the one
 * the whole sequence would draw.  1 <= N <= MP_MAX_SHARDS. */
int mp_all_gather_rows(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                       const void* const* slices, void* out, hipStream_t s);

/* Column sums of dy [rows,cols] (dtype) into db [cols] fp32: the gradient of
 * a bias added to every row (deterministic, fixed summation order). */
size_t mp_bias_grad_workspace(int64_t rows, int64_t cols);
int mp_bias_grad(mp_dtype dtype, int64_t rows, int64_t cols, const void* dy, float* db,
                 void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------- attention */

/* Head-partitioned causal self-attention with the fused QKV GEMM over the
 * rank's heads (MLM-notes, "Model Parallel Transformers", attention
 * paragraph: heads are independent and assigned to GPUs; MLM-review,
 * "approach": the Q, K, V products are split across GPUs).
 *   qkv = X * Wqkv_i^T + bqkv_i;  per (batch, head):
 *   ctx = softmax(Q K^T / sqrt(d), keys m <= l if causal) * V
 * bf16 only; d in {64, 128}.  X [T=B*L, K], Wqkv_i [3*h*d, K], bqkv_i [3*h*d]
 * or NULL, ctx_i [T, h*d] (head-major columns), qkv [T, 3*h*d] (written; also
 * read by the backward), lse [B, h, L] fp32: natural-log softmax normaliser
 * per query.  The out-projection is mp_row_linear_partial on ctx_i. */
int mp_head_attention(mp_dtype dtype, int B, int L, int K, int h, int d, int causal,
                      const void* X, const void* Wqkv_i, const void* bqkv_i, void* ctx_i,
                      void* qkv, float* lse, hipStream_t s);

/* Workspace bytes of mp_head_attention_bwd (0 for an unsupported shape):
 * dQKV, the per-query rowsum(dO * O), and one region shared by the weight
 * products' scratch and, when B * h * ceil(L/128) < 512 and L <= 4096, the
 * bf16 dS^T of every (batch, head) pair in 64 x 64 tiles
 * (B * h * ceil(L/64)^2 * 8 KiB), which the dQ kernel reads back instead of
 * recomputing S and dP. */
size_t mp_head_attention_bwd_workspace(mp_dtype dtype, int B, int L, int K, int h, int d);

/* Backward of mp_head_attention (P recomputed from lse).  Inputs as saved by
 * the forward plus dctx_i [T, h*d]; outputs dX_partial [T,K] (this rank's
 * share of the input gradient), dWqkv_i [3*h*d, K] fp32, dbqkv_i [3*h*d] fp32
 * or NULL.  On return the first T*3*h*d bf16 of ws hold dQKV [T, 3*h*d], the
 * gradient of qkv in its column order (the attention core's dQ, dK, dV). */
int mp_head_attention_bwd(mp_dtype dtype, int B, int L, int K, int h, int d, int causal,
                          const void* X, const void* Wqkv_i, const void* qkv,
                          const void* ctx_i, const float* lse, const void* dctx_i,
                          void* dX_partial, float* dWqkv_i, float* dbqkv_i, void* ws,
                          size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------- vocab-parallel path */

/* Vocab-parallel embedding lookup (MLM-notes, "Model Parallel Transformers",
 * embedding paragraph: split the embedding, replicate the ids, look up, then
 * all-reduce).  The split is along V: out_partial[t] = E_i[ids[t] - v_start]
 * if v_start <= ids[t] < v_start + Vi, else zeros.  ids [T] int32,
 * E_i [Vi,K], out_partial [T,K].  Summing the N partials with
 * mp_shard_reduce reproduces the full lookup exactly. */
int mp_vocab_parallel_embedding(mp_dtype dtype, int64_t T, int64_t Vi, int64_t v_start,
                                int64_t K, const int32_t* ids, const void* E_i,
                                void* out_partial, hipStream_t s);

/* Backward of mp_vocab_parallel_embedding with respect to the rank's shard
 * (MLM-notes, "Model Parallel Transformers", embedding paragraph; with the
 * output layer's tied weight, the embedding's and the logits GEMM's
 * gradients of E_i add up):
 *   dE_i[v] (+)= sum of dOut[t] over tokens t with ids[t] = v_start + v,
 *                in ascending t (deterministic; rows no token picked get 0,
 *                or keep their value when accumulate != 0).
 * ids [T] int32, dOut [T, K] dtype (the gradient of the reduced embedding,
 * replicated on every rank), dE_i [Vi, K] fp32, K % 8 == 0. */
int mp_vocab_parallel_embedding_bwd(mp_dtype dtype, int64_t T, int64_t Vi, int64_t v_start,
                                    int64_t K, const int32_t* ids, const void* dOut, float* dE_i,
                                    int accumulate, hipStream_t s);

/* Per-shard cross-entropy statistics (MLM-notes, "Model Parallel
 * Transformers", output paragraph: each GPU computes its exponentials, then
 * the row sums are combined).  One pass over the rank's fp32 logits
 * Z_i [T,Vi]: triples[t] = (m, s, tgt) with m = max_v Z_i[t,v],
 * s = sum_v exp(Z_i[t,v] - m), tgt = Z_i[t, labels[t] - v_start] if the label
 * is owned by this shard else 0.  labels [T] int32 (global ids),
 * triples [T,3] fp32. */
int mp_vocab_parallel_xent(int64_t T, int64_t Vi, int64_t v_start, const float* Z_i,
                           const int32_t* labels, float* triples, hipStream_t s);

/* The logits GEMM and the per-shard statistics in one pass (a11 + a12 fused;
 * MLM-notes, output paragraph: each shard reduces its own logits so only
 * (max, sum, target) triples cross GPUs, never the [T, V_i] logits).  The
 * fp32 logits Z_i = H * E_i^T live only in the GEMM's accumulators: its
 * epilogue folds every row over each wave's columns into (max, exp-sum,
 * target logit) partials in the workspace, and a second pass folds those in a
 * fixed order into triples [T, 3] fp32 exactly as mp_vocab_parallel_xent
 * defines them (up to summation order), so the 4*T*V_i-byte logits round
 * trip disappears.  H [T, K] bf16, E_i [V_i, K] bf16 (K % 8 == 0), labels
 * [T] int32 (global ids), v_start as in mp_vocab_parallel_xent.  bf16 only.
 * ws: mp_vocab_parallel_logits_xent_workspace bytes.  (The backward still
 * needs the logits: recompute them, or use the unfused calls.) */
size_t mp_vocab_parallel_logits_xent_workspace(int64_t T, int64_t K, int64_t Vi);
int mp_vocab_parallel_logits_xent(mp_dtype dtype, int64_t T, int64_t K, int64_t Vi, int64_t v_start,
                                  const void* H, const void* E_i, const int32_t* labels,
                                  float* triples, void* ws, size_t ws_bytes, hipStream_t s);

/* Combine N shards' triples into the loss: M = max_j m_j,
 * S = sum_j s_j exp(m_j - M), loss[t] = ln S + M - sum_j tgt_j.  triples: host
 * array of N device pointers to [T,3] fp32; loss [T] fp32; stats [T,2] fp32
 * receives (M, S) for the backward (or NULL); mean_loss [1] fp32 receives the
 * mean over T (or NULL). */
int mp_vocab_xent_combine(int N, int64_t T, const float* const* triples, float* loss,
                          float* stats, float* mean_loss, hipStream_t s);

/* Backward of the loss sum scaled by g (g = 1/T for the mean) on one shard:
 * dZ_i[t,v] = g * (exp(Z_i[t,v] - M_t) / S_t - [v_start + v == labels[t]]).
 * stats [T,2] from mp_vocab_xent_combine; dZ_i [T,Vi] in out_dtype (fp32 may
 * alias Z_i). */
int mp_vocab_parallel_xent_bwd(int64_t T, int64_t Vi, int64_t v_start, const float* Z_i,
                               const int32_t* labels, const float* stats, float g,
                               mp_dtype out_dtype, void* dZ_i, hipStream_t s);

/* ---------------------------------------------------------------- MoE shard */

/* Worst-case workspace bytes of mp_grouped_expert_gemm (a bound computed from
 * the sizes alone, so no host synchronisation is ever needed). */
size_t mp_grouped_expert_gemm_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk,
                                        int E_loc);

/* One expert-parallel shard of a MoE layer (MOE-core, technical summary: 2.4
 * grouped GEMM and sync-free kernels, 2.2 permutation; 1: small per-expert
 * GEMMs and dynamic shapes).  Local experts are e_start .. e_start+E_loc-1.
 *  1. permutation: list the local picks (t,k) with topk_ids[t,k] local,
 *     ordered by expert, then token, then slot (a token that picks one
 *     expert in two slots gets two rows); perm_picks[r] = t*topk + k;
 *     expert_offsets[e] = first row of local expert e (exclusive scan of the
 *     per-expert counts; expert_offsets[E_loc] = R).  Shapes stay on the
 *     device: nothing is copied back to the host.
 *  2. grouped gate/up GEMM with fused SwiGLU: for the rows of expert e,
 *     act = silu(x W_g,e^T) * (x W_u,e^T) with W_gu[e] = [W_g,e ; W_u,e]
 *     ([2*Fe, Hd], gate rows first).
 *  3. grouped down GEMM: y = act * W_d,e^T, W_d [E_loc, Hd, Fe].
 *  4. unpermute: out[t] = sum over local picks k (ascending) of
 *     topk_w[t,k] * y(t,k), fp32 sum, zeros for tokens without local picks.
 * X [T,Hd] bf16, topk_ids [T,topk] int32, topk_w [T,topk] fp32,
 * out [T,Hd] bf16, perm_picks [T*topk] int32 or NULL (entries >= R untouched;
 * with distinct ids per token R <= T*min(topk,E_loc)), expert_offsets
 * [E_loc+1] int32 or NULL; ws >= mp_grouped_expert_gemm_workspace().  T = 0
 * (no tokens) returns MP_OK without touching any buffer (all may be NULL);
 * so do the other MoE forward calls below. */
int mp_grouped_expert_gemm(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                           int e_start, const void* X, const int32_t* topk_ids,
                           const float* topk_w, const void* W_gu, const void* W_d, void* out,
                           int32_t* perm_picks, int32_t* expert_offsets, void* ws,
                           size_t ws_bytes, hipStream_t s);

/* Memory-efficient permutation form of mp_grouped_expert_gemm (MOE-core,
 * technical summary 2.2: the routing weight is applied before the expert's
 * activation leaves it, so the backward needs no saved expert output).  Steps
 * 1 and 3 as above; in step 2 the activation row of pick (t,k) is
 * topk_w[t,k] * silu(x W_g,e^T) * (x W_u,e^T), scaled in fp32 before its bf16
 * rounding; step 4 sums the down-projection rows per token without weights.
 * Equal to mp_grouped_expert_gemm in exact arithmetic (the down projection is
 * linear); arguments, layouts, workspace and errors are the same. */
int mp_grouped_expert_gemm_weighted_act(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                                        int e_start, const void* X, const int32_t* topk_ids,
                                        const float* topk_w, const void* W_gu, const void* W_d,
                                        void* out, int32_t* perm_picks, int32_t* expert_offsets,
                                        void* ws, size_t ws_bytes, hipStream_t s);

/* Training forward of mp_grouped_expert_gemm (same arguments, layouts and
 * errors; no perm_picks / expert_offsets: they stay in ws).  It also writes
 * gu_save [T*topk, 2*Fe] bf16: row r of the permuted order holds that pick's
 * gate pre-activation x W_g,e^T in columns [0, Fe) and its up pre-activation
 * x W_u,e^T in [Fe, 2*Fe) (rows >= R untouched).  ws then holds the
 * permutation, the expert schedule, the activation and the expert outputs
 * that mp_grouped_expert_gemm_bwd reads: keep it, and gu_save, unchanged
 * until that call. */
int mp_grouped_expert_gemm_fwd_train(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                                     int e_start, const void* X, const int32_t* topk_ids,
                                     const float* topk_w, const void* W_gu, const void* W_d,
                                     void* out, void* gu_save, void* ws, size_t ws_bytes,
                                     hipStream_t s);

/* Worst-case workspace bytes of mp_grouped_expert_gemm_bwd (sizes alone). */
size_t mp_grouped_expert_gemm_bwd_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk,
                                            int E_loc);

/* Backward of the MoE shard (MOE-core, technical summary 2.4: the expert
 * GEMMs of the backward are grouped like the forward's, with the shapes on
 * the device).  Given dOut [T,Hd] bf16, the gradient of the shard's output,
 * and the state left by mp_grouped_expert_gemm_fwd_train with the same
 * sizes (gu_save; fwd_ws of fwd_ws_bytes), for every local pick (t,k) of
 * expert e (row r of the permutation):
 *   dy_r = topk_w[t,k] * dOut[t];  dtopk_w[t,k] = dOut[t] . y_r (fp32);
 *   d act_r = dy_r W_d,e;  dW_d[e] = sum_r dy_r^T act_r;
 *   d gate = d act * up * s (1 + gate (1 - s)), s = sigmoid(gate);
 *   d up = d act * silu(gate);
 *   dW_gu[e] = sum_r [d gate_r ; d up_r]^T x_t;
 *   dX[t] = sum over t's local picks (k ascending, fp32) of
 *           d gate_r W_g,e + d up_r W_u,e.
 * dX [T,Hd] bf16 (zeros for tokens without a local pick); dW_gu
 * [E_loc,2*Fe,Hd] and dW_d [E_loc,Hd,Fe] fp32, overwritten (zeros for an
 * expert without rows); dtopk_w [T,topk] fp32 (zero for picks on other
 * shards).  Weight gradients sum their rows in a fixed order
 * (deterministic).  ws >= mp_grouped_expert_gemm_bwd_workspace().  Same
 * shape limits and errors as the forward.  T = 0: only dW_gu and dW_d are
 * written (zeros); every other buffer may be NULL. */
int mp_grouped_expert_gemm_bwd(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                               const void* X, const float* topk_w, const void* W_gu,
                               const void* W_d, const void* dOut, const void* gu_save,
                               const void* fwd_ws, size_t fwd_ws_bytes, void* dX, float* dW_gu,
                               float* dW_d, float* dtopk_w, void* ws, size_t ws_bytes,
                               hipStream_t s);

/* Training forward of mp_grouped_expert_gemm_weighted_act (the memory-
 * efficient form): arguments, outputs, gu_save (unweighted gate and up
 * pre-activations) and the kept workspace as mp_grouped_expert_gemm_fwd_train;
 * the activation kept in ws is the weighted one. */
int mp_grouped_expert_gemm_weighted_act_fwd_train(int64_t T, int64_t Hd, int64_t Fe, int topk,
                                                  int E_loc, int e_start, const void* X,
                                                  const int32_t* topk_ids, const float* topk_w,
                                                  const void* W_gu, const void* W_d, void* out,
                                                  void* gu_save, void* ws, size_t ws_bytes,
                                                  hipStream_t s);

/* Backward of the memory-efficient form (MOE-core, technical summary 2.2: the
 * routing weight sits before the expert's output, so the backward reads no
 * saved expert output).  With act = silu(gate) * up and act_w = topk_w[t,k] *
 * act as the forward stored it, for every local pick (t,k) of expert e:
 *   dy_r = dOut[t];  d act_w = dy_r W_d,e;  dW_d[e] = sum_r dy_r^T act_w,r;
 *   dtopk_w[t,k] = d act_w . act (fp32, fixed order);
 *   d act = topk_w[t,k] * d act_w, then d gate, d up, dW_gu and dX as in
 *   mp_grouped_expert_gemm_bwd.
 * Needs the state of mp_grouped_expert_gemm_weighted_act_fwd_train; arguments,
 * outputs, workspace (mp_grouped_expert_gemm_bwd_workspace()) and errors as
 * mp_grouped_expert_gemm_bwd. */
int mp_grouped_expert_gemm_weighted_act_bwd(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                                            const void* X, const float* topk_w, const void* W_gu,
                                            const void* W_d, const void* dOut, const void* gu_save,
                                            const void* fwd_ws, size_t fwd_ws_bytes, void* dX,
                                            float* dW_gu, float* dW_d, float* dtopk_w, void* ws,
                                            size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------------ MXFP8 */

/* MXFP8 block quantisation (MOE-core, technical summary 2.5: expert GEMMs and
 * their activations in a low-precision format, MXFP8 among the recipes; the
 * format itself is read as OCP Microscaling).  Each row of x [rows, K] bf16
 * (row stride ld elements, ld >= K, ld % 8 == 0; K % 32 == 0) is split into
 * 32-value blocks along K; a block with largest magnitude X gets the E8M0
 * exponent se = floor(log2 X) - 8, clamped to [-127, 127] (-127 when
 * X < 2^-126), stored as se + 127; each value becomes the E4M3 code of
 * x / 2^se (nearest, ties to the even code, saturating at 448, sign kept).
 * q [rows, K] uint8 (8-byte aligned); scales [rows, 4*ceil(K/128)] uint8,
 * block b of a row at byte b, the bytes past the last block set to 127.
 * Inputs must be finite. */
int mp_mxfp8_quantize(int64_t rows, int64_t K, const void* x, int64_t ld, uint8_t* q,
                      uint8_t* scales, hipStream_t s);

size_t mp_grouped_expert_gemm_mxfp8_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk,
                                              int E_loc);

/* The MoE shard of mp_grouped_expert_gemm with both expert GEMMs in MXFP8
 * (selective precision, MOE-core 2.5: the routing, the unpermute's fp32 sum
 * and the output stay high precision).  The token rows are quantised along Hd
 * inside the call (mp_mxfp8_quantize's rules); the weights arrive quantised:
 * W_gu_q [E_loc, 2*Fe, Hd] with W_gu_s [E_loc, 2*Fe, 4*ceil(Hd/128)], W_d_q
 * [E_loc, Hd, Fe] with W_d_s [E_loc, Hd, 4*ceil(Fe/128)] (scale arrays 4-byte
 * aligned).  Each expert's gate/up products accumulate in fp32 on gfx950's
 * block-scaled MFMA; the SwiGLU activation is rounded to bf16 and quantised
 * along Fe (the gate/up GEMM's epilogue writes only its codes and scales),
 * then projected down the same way; the unpermute is the weighted fp32
 * sum of mp_grouped_expert_gemm.  Hd % 32 == 0, Fe % 32 == 0; other arguments,
 * outputs and errors as mp_grouped_expert_gemm, with the workspace from
 * mp_grouped_expert_gemm_mxfp8_workspace(). */
int mp_grouped_expert_gemm_mxfp8(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                                 int e_start, const void* X, const int32_t* topk_ids,
                                 const float* topk_w, const uint8_t* W_gu_q,
                                 const uint8_t* W_gu_s, const uint8_t* W_d_q,
                                 const uint8_t* W_d_s, void* out, int32_t* perm_picks,
                                 int32_t* expert_offsets, void* ws, size_t ws_bytes,
                                 hipStream_t s);

/* --------------------------------------------------------------- LayerNorm */

/* LayerNorm over the last dim (MLM-review, "approach": LayerNorm placement
 * matters for deep BERT-like models); a replicated op, not partitioned.
 * y = (x - mean) * rstd * gamma + beta, biased variance, fp32 statistics.
 * x, y [T,K] dtype; gamma, beta [K] dtype; mean, rstd [T] fp32 (or NULL). */
int mp_layernorm(mp_dtype dtype, int64_t T, int64_t K, const void* x, const void* gamma,
                 const void* beta, float eps, void* y, float* mean, float* rstd,
                 hipStream_t s);

size_t mp_layernorm_bwd_workspace(int64_t T, int64_t K);

/* Backward of mp_layernorm: dx = dres + LN'(dy) (dres [T,K] or NULL is an
 * extra gradient added to dx, e.g. a residual branch; it may alias dx),
 * dgamma, dbeta [K] fp32 (each may be NULL). */
int mp_layernorm_bwd(mp_dtype dtype, int64_t T, int64_t K, const void* x, const void* gamma,
                     const float* mean, const float* rstd, const void* dy, const void* dres,
                     void* dx, float* dgamma, float* dbeta, void* ws, size_t ws_bytes,
                     hipStream_t s);

/* ------------------------------------------- reduce fused with LayerNorm */

/* The all-reduce stand-in followed by the LayerNorm it feeds (MLM-notes,
 * "Model Parallel Transformers": the all-reduce after the attention block
 * precedes the next block's LayerNorm), in one pass per row:
 *   out = residual + Drop(sum_{j=0..N-1} partials[j] + bias)   (as mp_shard_reduce)
 *   y   = (out - mean) * rstd * gamma + beta                    (as mp_layernorm of out)
 * Same arguments and rules as mp_shard_reduce plus gamma, beta [cols] dtype,
 * eps > 0, y [rows,cols] dtype, mean, rstd [rows] fp32 (or NULL).  out and
 * mask_out equal mp_shard_reduce's bit for bit; the LN statistics are those of
 * the stored out (rounded to dtype), summed in a fixed order, so y matches
 * mp_layernorm(out) to rounding.  cols <= 16*64*(16/size); with mask_out,
 * cols % 8 == 0. */
int mp_shard_reduce_layernorm(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                              const void* const* partials, const void* bias,
                              const void* residual, float p, uint64_t seed, uint64_t offset,
                              uint64_t index_base, void* out, uint8_t* mask_out,
                              const void* gamma, const void* beta, float eps, void* y,
                              float* mean, float* rstd, hipStream_t s);

/* Workspace bytes of the dgamma/dbeta (and dbias) partials of
 * mp_shard_reduce_layernorm_bwd and mp_shard_reduce_layernorm_bwd_dropout. */
size_t mp_shard_reduce_layernorm_bwd_workspace(int64_t rows, int64_t cols);

/* The backward all-reduce of the input-gradient partials fused with the
 * LayerNorm backward it feeds (MLM-notes, "Model Parallel Transformers": one
 * all-reduce in each block's backward):
 *   dy = sum_{j=0..N-1} partials[j]   (rounded to dtype, never stored)
 *   dx, dgamma, dbeta as mp_layernorm_bwd(x, gamma, mean, rstd, dy, dres).
 * partials as in mp_shard_reduce; x [rows,cols] is the LayerNorm input, mean,
 * rstd its saved statistics; dres [rows,cols] or NULL (may alias dx); dgamma,
 * dbeta [cols] fp32 or NULL (then ws may be NULL).  The parameter gradients
 * are summed in a fixed order (deterministic). */
int mp_shard_reduce_layernorm_bwd(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                                  const void* const* partials, const void* x,
                                  const void* gamma, const float* mean, const float* rstd,
                                  const void* dres, void* dx, float* dgamma, float* dbeta,
                                  void* ws, size_t ws_bytes, hipStream_t s);

/* mp_shard_reduce_layernorm_bwd followed, in the same pass, by the start of
 * the backward of the branch that feeds this residual join (MLM-notes,
 * "Model Parallel Transformers": each block ends in bias, dropout and the
 * residual add), with the keep bits that branch's forward dropout saved:
 *   ddrop = Drop(dx)       as mp_dropout_mask_bwd(dx, keep_bits, p) on dx as
 *                          stored, [rows,cols] dtype;
 *   dbias = column sums of ddrop  [cols] fp32 or NULL (the branch's bias
 *                          gradient).
 * dx, dgamma, dbeta, workspace and errors as mp_shard_reduce_layernorm_bwd;
 * keep_bits and ddrop must be non-NULL, ddrop 16-byte aligned; ws is needed
 * when any of dgamma, dbeta, dbias is non-NULL.  0 <= p < 1. */
int mp_shard_reduce_layernorm_bwd_dropout(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                                          const void* const* partials, const void* x,
                                          const void* gamma, const float* mean, const float* rstd,
                                          const void* dres, void* dx, float* dgamma, float* dbeta,
                                          float p, const uint8_t* keep_bits, void* ddrop,
                                          float* dbias, void* ws, size_t ws_bytes, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* MP_H */
