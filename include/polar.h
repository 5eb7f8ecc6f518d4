/*
 * libpolar — Polar Attention forward for AMD Instinct MI355X (gfx950).  C ABI, version 7
 * (POLAR_ABI_VERSION below; polar_abi_version() reports the loaded library's).
 *
 * The operation is the attention mixing step of the ATMA hybrid decoder as described in
 * "ATMA: Length-Invariant Language Modeling via Polar Attention and Gated-Delta
 * Compression Memory" (gist.science technical summary), section 2.1 "Polar Attention:
 * A Three-Channel Decomposition", and its kernels in section 2.2 "Hardware-Software
 * Codesign" (a fused Polar Attention kernel computing participation ratios online in
 * O(block) memory, and a GQA-grouped decode kernel reading paged KV cache blocks).
 *
 * For query row i of head h (KV head g = h / (Hq/Hkv)), seeing n keys j (n = i+1 in causal
 * prefill, n = seq_len in decode):
 *   tau    = max(1, ln n / ln train_len)          if POLAR_FLAG_LENGTH_TEMP, else 1
 *   l_j    = beta_h * tau * <q_i, k_j>             (q, k are unit vectors: caller's job)
 *   p_j    = softmax_j(l_j);   lse = log sum_j exp(l_j)
 *   n_eff  = 1 / sum_j p_j^2                        (participation ratio)
 *   u      = sum_j p_j v_j;    dir = u / |u|        (direction / content channel)
 *   floor  = b_h + (beta_h * tau / sqrt(d)) * sqrt(2 ln n)   if POLAR_FLAG_NULL_FLOOR,
 *            else b_h
 *   gate   = sigmoid(max_j l_j - floor)             (signal-detection confidence)
 *   count  = gate * tanh(ln n_eff) * w_h            (magnitude / count channel)
 * The pages give out = content + count + memory; the memory stream is a separate
 * operation, so dir and count are returned separately and the caller adds them.
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers; the params/outputs structs are HOST structs.
 *  - The caller allocates and owns every buffer.  The library allocates nothing and keeps
 *    no pointer after a call returns.  Inputs are never written; outputs are fully
 *    overwritten; inputs and outputs must not alias.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL = default stream).
 *  - All validation happens before any launch.  On an error nothing is launched and
 *    nothing is written; polar_last_error() gives a thread-local description.
 *  - Launch failures return POLAR_ERR_HIP.  Faults inside kernels surface at the caller's
 *    next synchronisation.  Nothing throws, aborts or exits across this interface.
 *  - beta_h must be positive and finite; other values give unspecified (but memory-safe)
 *    results.
 */
#ifndef POLAR_H
#define POLAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: polar_variant gained the key-rotation workspace.
 * 3: polar_decode_workspace_bytes lost its page_size argument (the only page size is 64 and
 *    the workspace never depended on it).
 * 4: polar_delta_sequence (the memory stream over T tokens) added; nothing else changed.
 * 5: polar_attn_fwd_mixed (the three streams summed into one output) added.
 * 6: the training forward and the backward of the window and RoPE variants added
 *    (polar_attn_fwd_train_variant, polar_attn_bwd_variant and their workspace sizes).
 * 7: polar_cotangents gained attn, the gradient of the plain softmax read-out, and
 *    polar_attn_fwd_train_variant writes that read-out (var.attn). */
#define POLAR_ABI_VERSION 7

#if defined(__GNUC__)
#define POLAR_API __attribute__((visibility("default")))
#else
#define POLAR_API
#endif

typedef enum {
  POLAR_OK = 0,
  POLAR_ERR_NULL_POINTER = 1,       /* a required pointer is NULL                         */
  POLAR_ERR_BAD_SHAPE = 2,          /* negative size, Hq % Hkv != 0, bad stride, ...      */
  POLAR_ERR_UNSUPPORTED = 3,        /* head_dim != 64, page_size != 64, unknown dtype ... */
  POLAR_ERR_MISALIGNED = 4,         /* a tensor pointer is not 16-byte aligned            */
  POLAR_ERR_WORKSPACE_TOO_SMALL = 5,
  POLAR_ERR_HIP = 6                 /* the HIP runtime refused a launch                   */
} polar_status;

typedef enum {
  POLAR_DTYPE_F32 = 0,              /* q, k, v in float32; MFMA f32                        */
  POLAR_DTYPE_BF16 = 1              /* q, k, v in bfloat16; MFMA bf16, fp32 accumulation   */
} polar_dtype;

enum {
  POLAR_FLAG_LENGTH_TEMP = 1u,      /* apply tau(n)                                       */
  POLAR_FLAG_NULL_FLOOR = 2u        /* add the sqrt(2 ln n) extreme-value term to b_h      */
};

typedef struct {
  int32_t n_q_heads;                /* Hq >= 1                                            */
  int32_t n_kv_heads;               /* Hkv >= 1, Hq % Hkv == 0                             */
  int32_t head_dim;                 /* d; must be 64 (only size)                         */
  int32_t train_len;                /* T_train; must be >= 2 when LENGTH_TEMP is set       */
  uint32_t flags;                   /* POLAR_FLAG_* bits                                   */
  const float *beta;                /* device [Hq] logit scale beta_h; NULL -> sqrt(d)     */
  const float *null_bias;           /* device [Hq] null scalar b_h; NULL -> 0              */
  const float *count_vec;           /* device [Hq*d] count vectors w_h; required iff
                                       outputs.count != NULL                             */
} polar_params;

/* Output tensors, float32, device.  dir and n_eff are required; count, gate and lse may
 * be NULL (not computed).  Prefill layouts: dir, count [B,T,Hq,d]; n_eff, gate, lse
 * [B,T,Hq].  Decode layouts: dir, count [B,Hq,d]; n_eff, gate, lse [B,Hq].  dir and count
 * must be 16-byte aligned. */
typedef struct {
  float *dir;
  float *count;
  float *n_eff;
  float *gate;
  float *lse;
} polar_outputs;

/*
 * Causal Polar Attention prefill (the fused kernel of section 2.2: one pass over K/V tiles
 * with streaming max, sum and sum-of-squares accumulators; the T x T scores are never
 * stored).
 *   q  [B,T,Hq,d], k and v [B,T,Hkv,d], row-major contiguous, dtype `dt`, 16-byte aligned.
 *   Row i of head h attends keys 0..i of KV head h / (Hq/Hkv).
 *   B == 0 or T == 0 is a valid empty call (nothing is launched).
 */
POLAR_API polar_status polar_attn_fwd(const polar_params *p, polar_dtype dt, int32_t B, int32_t T,
                            const void *q, const void *k, const void *v,
                            const polar_outputs *out, void *stream);

/*
 * The layer's output as the sum of its three streams (section 2.1 of the technical
 * summary: content plus count plus memory), for callers that want only the sum:
 *   mixed[b,t,h,:] = dir + count + memory[b,t,h,:]
 * with dir and count exactly as polar_attn_fwd defines them for row t of head h, and
 * memory the memory stream's output for the same token and head (polar_delta_sequence
 * run with H = Hq heads).  Written once, in place of dir and count.
 *   memory   optional device float32 [B,T,Hq,d], 16-byte aligned; NULL = no memory
 *            stream.  May alias mixed (each element is read before it is written).
 *   mixed    device float32 [B,T,Hq,d], 16-byte aligned.
 *   out      the scalar outputs as for polar_attn_fwd (n_eff required, gate and lse
 *            optional); out->dir and out->count must be NULL.
 *   params.count_vec NULL = no count stream.
 * Errors as for polar_attn_fwd, plus POLAR_ERR_UNSUPPORTED when out->dir or out->count is
 * set.
 */
POLAR_API polar_status polar_attn_fwd_mixed(const polar_params *p, polar_dtype dt, int32_t B,
                                            int32_t T, const void *q, const void *k,
                                            const void *v, const float *memory, float *mixed,
                                            const polar_outputs *out, void *stream);

/*
 * Variant modes of the prefill (the comparison arms and position schemes the pages
 * evaluate alongside Polar Attention: a plain softmax read-out, RoPE, sliding-window
 * attention).
 *   window      W >= 1: row i attends keys max(0, i-W+1)..i and n = min(i+1, W) is the key
 *               count that drives tau and the floor; 0 = all earlier keys.
 *   rope_theta  > 0: q and k are rotated on load by rotary position embeddings (RoFormer
 *               form: the pair of dimensions (2t, 2t+1) of the vector at position p turns
 *               by the angle p * rope_theta^(-2t/d)); positions are the row indices 0..T-1.
 *               0 = no rotation.
 *   attn        optional device float32 [B,T,Hq,d], 16-byte aligned: the plain softmax
 *               attention output u = sum_j p_j v_j.  NULL = not written.
 *   workspace   optional device buffer, 16-byte aligned, of workspace_bytes >=
 *               polar_variant_workspace_bytes(): with rope_theta > 0 the keys are rotated
 *               once into it, before the attention kernel, instead of in every workgroup
 *               that stages them.  The results are bit-identical either way.  NULL (or
 *               rope_theta == 0) = not used; a buffer that is too small is an error.  The
 *               caller owns it; its contents are scratch.
 */
typedef struct {
  int32_t window;
  float rope_theta;
  float *attn;
  void *workspace;
  size_t workspace_bytes;
} polar_variant;

/*
 * Bytes of the key-rotation workspace of polar_attn_fwd_variant: B*T*Hkv*d elements of
 * dtype `dt` (0 on invalid arguments).
 */
POLAR_API size_t polar_variant_workspace_bytes(const polar_params *p, polar_dtype dt, int32_t B,
                                     int32_t T);

/*
 * polar_attn_fwd with the variant modes above.  Same arguments, outputs and conventions
 * as polar_attn_fwd; var == NULL, or all fields zero, gives polar_attn_fwd's results.
 */
POLAR_API polar_status polar_attn_fwd_variant(const polar_params *p, const polar_variant *var,
                                    polar_dtype dt, int32_t B, int32_t T, const void *q,
                                    const void *k, const void *v, const polar_outputs *out,
                                    void *stream);

/*
 * Workspace bytes polar_attn_decode_paged needs for this batch size and length bound
 * (0 on invalid arguments: p NULL, B < 1, max_seq_len < 1, bad head counts).  The value
 * depends only on the arguments; it holds the split-KV partials (M, max, S, Q, u[d]) of
 * every (sequence, query head, key split).
 */
POLAR_API size_t polar_decode_workspace_bytes(const polar_params *p, int32_t B,
                                              int32_t max_seq_len);

/*
 * One-token GQA-grouped decode over a paged KV cache (section 2.2: the decode kernel reads
 * paged KV blocks directly; the Hq/Hkv query heads sharing a KV head are served by a
 * single read of each K/V byte).
 *   q                [B,Hq,d] dtype `dt`: the newest token of each sequence; its own key
 *                    and value are already in the cache, so it sees seq_lens[b] keys
 *                    (the same result as causal prefill row seq_lens[b]-1).
 *   k_cache, v_cache [num_pages,Hkv,page_size,d] dtype `dt`: page-major pools, one
 *                    contiguous page_size x d block per (page, KV head).
 *   page_table       device int32 [B,page_table_stride]: logical page p of sequence b is
 *                    physical page page_table[b*stride + p].  Ids outside [0,num_pages)
 *                    are skipped (their keys are masked out) so a bad table cannot read
 *                    outside the pools.
 *   seq_lens         device int32 [B], each in [1, max_seq_len]; values outside are
 *                    clamped to that range.
 *   max_seq_len      host upper bound of seq_lens; sizes the split-KV grid;
 *                    page_table_stride >= ceil(max_seq_len / page_size).
 *   workspace        device scratch of >= polar_decode_workspace_bytes(...) bytes,
 *                    16-byte aligned; its contents on entry are ignored.
 *   page_size must be 64 in this version.
 */
POLAR_API polar_status polar_attn_decode_paged(const polar_params *p, polar_dtype dt, int32_t B,
                                     const void *q, const void *k_cache, const void *v_cache,
                                     int32_t num_pages, int32_t page_size,
                                     const int32_t *page_table, int32_t page_table_stride,
                                     const int32_t *seq_lens, int32_t max_seq_len,
                                     void *workspace, size_t workspace_bytes,
                                     const polar_outputs *out, void *stream);

/*
 * polar_attn_decode_paged for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and conventions as polar_attn_decode_paged, without the workspace: the split
 * partials live in a static device array of the library, POLAR_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, held from the library's first use on that GPU until the process ends.
 * Nothing on this call path allocates (no hipMalloc, hipFree or allocating library call).
 *   - The scratch is looked up on the current device (hipGetDevice) on its first call
 *     there; `stream` must belong to the current device.
 *   - A decode needing more than POLAR_NOALLOC_SCRATCH_BYTES of partials
 *     (polar_decode_workspace_bytes) returns POLAR_ERR_WORKSPACE_TOO_SMALL and launches
 *     nothing.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 *     different streams or threads without ordering between them) race and give
 *     unspecified results.  Calls ordered on one stream are safe; the scratch keeps the
 *     last call's partials, which the next call overwrites before it reads them.
 */
#define POLAR_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
POLAR_API polar_status polar_attn_decode_paged_noalloc(const polar_params *p, polar_dtype dt,
                                                       int32_t B, const void *q,
                                                       const void *k_cache, const void *v_cache,
                                                       int32_t num_pages, int32_t page_size,
                                                       const int32_t *page_table,
                                                       int32_t page_table_stride,
                                                       const int32_t *seq_lens,
                                                       int32_t max_seq_len,
                                                       const polar_outputs *out, void *stream);

/* ---------------------------------------------------------------------------------
 * Training: forward with residuals, and the backward pass of the causal prefill.
 *
 * The backward differentiates the prefill definitions above with respect to q, k, v and
 * the per-head parameters beta, null_bias and count_vec, for caller-given upstream
 * gradients of the five outputs.  max_j l_j (through the gate) is differentiated as the
 * subgradient that sends its whole gradient to the lowest key position attaining the
 * maximum (the forward records that key).  The pages train at 2K context; the backward
 * is what makes the fused kernel of section 2.2 usable for training.
 * --------------------------------------------------------------------------------- */

/* Per-row residuals of the forward pass that the backward reads, device, [B,T,Hq]. */
typedef struct {
  float *u_norm;                    /* |u|, the norm of the softmax-weighted value sum     */
  int32_t *arg_max;                 /* lowest key position j attaining max_j l_j           */
} polar_saved;

/* Upstream gradients of the outputs, float32, device, in the polar_outputs layouts
 * ([B,T,Hq,d] for dir and count, [B,T,Hq] for the rest).  NULL means zero.  dir and
 * count must be 16-byte aligned; count != NULL needs params.count_vec.
 *   attn  [B,T,Hq,d], 16-byte aligned: gradient of the plain softmax read-out
 *         u = sum_j p_j v_j (the polar_variant.attn output; u = dir * u_norm), for the
 *         softmax arm the pages compare against.  Its term adds p_j (v_j - u) . attn to
 *         the gradient of logit j and p_j attn to dv_j. */
typedef struct {
  const float *dir;
  const float *count;
  const float *n_eff;
  const float *gate;
  const float *lse;
  const float *attn;
} polar_cotangents;

/* Gradients written by polar_attn_bwd, float32, device.  dq [B,T,Hq,d], dk and dv
 * [B,T,Hkv,d] are required and 16-byte aligned; d_beta [Hq], d_null_bias [Hq] and
 * d_count_vec [Hq*d] may be NULL (not computed).  All are fully overwritten. */
typedef struct {
  float *dq;
  float *dk;
  float *dv;
  float *d_beta;
  float *d_null_bias;
  float *d_count_vec;
} polar_grads;

/*
 * polar_attn_fwd plus the residuals of the backward pass.  Same arguments, outputs and
 * results as polar_attn_fwd; additionally out->gate and out->lse are required, and
 * saved->u_norm and saved->arg_max are written.
 */
POLAR_API polar_status polar_attn_fwd_train(const polar_params *p, polar_dtype dt, int32_t B,
                                  int32_t T, const void *q, const void *k, const void *v,
                                  const polar_outputs *out, const polar_saved *saved,
                                  void *stream);

/* Workspace bytes polar_attn_bwd needs (0 on invalid arguments); depends only on the
 * arguments. */
POLAR_API size_t polar_bwd_workspace_bytes(const polar_params *p, int32_t B, int32_t T);

/*
 * Backward pass of the causal prefill.  bf16 inputs only in this version
 * (POLAR_ERR_UNSUPPORTED for float32).
 *   p, dt, B, T, q, k, v  exactly as passed to polar_attn_fwd_train.
 *   fwd                   its outputs: dir, n_eff, gate and lse are read (count unused).
 *   saved                 its residuals.
 *   cot                   upstream gradients (fields may be NULL).
 *   grads                 outputs (see polar_grads).
 *   workspace             device scratch of >= polar_bwd_workspace_bytes bytes, 256-byte
 *                         aligned; contents on entry are ignored.
 * Results are deterministic: no atomics; every reduction has a fixed order.
 * B == 0 or T == 0 writes zeros to the requested parameter gradients and nothing else.
 */
POLAR_API polar_status polar_attn_bwd(const polar_params *p, polar_dtype dt, int32_t B,
                            int32_t T, const void *q, const void *k, const void *v,
                            const polar_outputs *fwd, const polar_saved *saved,
                            const polar_cotangents *cot, const polar_grads *grads,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training forward and backward of the variant modes (the sliding-window and RoPE arms
 * trained beside NoPE Polar Attention in the technical summary's section 3.1, "Ablation
 * Insights").  var->window and
 * var->rope_theta as for polar_attn_fwd_variant.  var == NULL, or window and rope_theta
 * both 0 (and no attn), gives polar_attn_fwd_train and polar_attn_bwd.
 *
 * The plain softmax read-out: polar_attn_fwd_train_variant writes it to var->attn when
 * that is non-NULL (as polar_attn_fwd_variant does), and its gradient enters the backward
 * as cot->attn.  The backward takes no var->attn (POLAR_ERR_UNSUPPORTED).
 *
 * With RoPE both calls rotate q and k into their workspace first (rounded to the input
 * type, as polar_attn_fwd_variant rotates them), run the causal kernels on the rotated
 * vectors, and the backward turns dq and dk back by the transposed rotation, so its
 * gradients are with respect to the unrotated q and k (the rounding of the rotated
 * vectors is passed through unchanged).
 *
 * polar_train_variant_workspace_bytes: bytes polar_attn_fwd_train_variant needs in
 *   var->workspace (16-byte aligned, contents scratch): B*T*(Hq+Hkv)*d elements of dt
 *   with RoPE, 0 without (then var->workspace may be NULL).  0 also on invalid arguments.
 * polar_attn_fwd_train_variant: as polar_attn_fwd_train (outputs, residuals, errors),
 *   with the variant's window and rotation; its outputs are those of
 *   polar_attn_fwd_variant for the same arguments.
 * polar_bwd_variant_workspace_bytes: bytes of polar_attn_bwd_variant's workspace
 *   (polar_bwd_workspace_bytes plus, with RoPE, room for the rotated q and k); 0 on
 *   invalid arguments.  var->workspace is not used by the backward.
 * polar_attn_bwd_variant: as polar_attn_bwd, for the outputs and residuals of
 *   polar_attn_fwd_train_variant with the same var; bf16 inputs only.
 */
POLAR_API size_t polar_train_variant_workspace_bytes(const polar_params *p,
                                                     const polar_variant *var, polar_dtype dt,
                                                     int32_t B, int32_t T);
POLAR_API polar_status polar_attn_fwd_train_variant(const polar_params *p,
                                                    const polar_variant *var, polar_dtype dt,
                                                    int32_t B, int32_t T, const void *q,
                                                    const void *k, const void *v,
                                                    const polar_outputs *out,
                                                    const polar_saved *saved, void *stream);
POLAR_API size_t polar_bwd_variant_workspace_bytes(const polar_params *p,
                                                   const polar_variant *var, int32_t B,
                                                   int32_t T);
POLAR_API polar_status polar_attn_bwd_variant(const polar_params *p, const polar_variant *var,
                                              polar_dtype dt, int32_t B, int32_t T,
                                              const void *q, const void *k, const void *v,
                                              const polar_outputs *fwd,
                                              const polar_saved *saved,
                                              const polar_cotangents *cot,
                                              const polar_grads *grads, void *workspace,
                                              size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Paged KV cache: append and chunked prefill (the step before decode in section 2.2: new
 * keys and values are written into cache pages, then the new tokens attend the paged
 * prefix).  Pools, page table and page_size are as for polar_attn_decode_paged.
 *   start_pos   device int32 [B]: position of the chunk's first token in its sequence
 *               (the number of tokens already cached).  Both calls clamp each value to
 *               [0, max_seq_len - C] the same way (a device value cannot be checked before
 *               the launch), so a chunk appended and then attended with the same
 *               arguments always lands at, and reads from, the same positions.
 *   max_seq_len host bound, >= C: start_pos[b] + C <= max_seq_len;
 *               page_table_stride >= ceil(max_seq_len / page_size).
 * --------------------------------------------------------------------------------- */

/*
 * Writes k_new, v_new [B,C,Hkv,d] (dtype `dt`, 16-byte aligned) into the pools: token t of
 * sequence b goes to position pos = s + t with s = start_pos[b] clamped to
 * [0, max_seq_len - C], page page_table[b, pos / page_size], slot pos % page_size.  Tokens
 * whose page id lies outside [0, num_pages) are dropped.  The pools are the only memory
 * written.  Only n_kv_heads and head_dim of `p` are used.
 */
POLAR_API polar_status polar_kv_append(const polar_params *p, polar_dtype dt, int32_t B, int32_t C,
                             const void *k_new, const void *v_new, void *k_cache,
                             void *v_cache, int32_t num_pages, int32_t page_size,
                             const int32_t *page_table, int32_t page_table_stride,
                             const int32_t *start_pos, int32_t max_seq_len, void *stream);

/*
 * Chunked causal prefill over the paged cache: q [B,C,Hq,d] are the queries of C new
 * tokens per sequence; row t (position pos = s + t, s = start_pos[b] clamped to
 * [0, max_seq_len - C]) attends keys 0..pos of its
 * sequence, read from the pools through the page table (append the chunk's own keys and
 * values first).  n = pos + 1 drives tau and the floor, so the rows equal causal prefill
 * rows s..s+C-1 of the whole sequence.  Keys on pages with ids
 * outside [0, num_pages) are masked out.  Outputs as for polar_attn_fwd with T = C.
 */
POLAR_API polar_status polar_attn_prefill_paged(const polar_params *p, polar_dtype dt, int32_t B,
                                      int32_t C, const void *q, const void *k_cache,
                                      const void *v_cache, int32_t num_pages, int32_t page_size,
                                      const int32_t *page_table, int32_t page_table_stride,
                                      const int32_t *start_pos, int32_t max_seq_len,
                                      const polar_outputs *out, void *stream);

/* ---------------------------------------------------------------------------------
 * Recurrent memory stream: the in-place gated-delta step (section 2.1's third channel, a
 * gated-delta memory derived from gated DeltaNet with L2-normalised keys and queries; its
 * step kernel of section 2.2 updates the recurrent state in place, without gathering
 * states into a batch and scattering them back).  The pages print no update rule; this is
 * the gated delta rule, one token per sequence:
 *   k <- k/|k|, q <- q/|q|            (when POLAR_DELTA_NORMALIZE_QK; |x| = sqrt(x.x + 1e-12))
 *   S' = alpha S (I - beta k k^T) + beta v k^T,   o = S' q
 * with S the [d_v, d_k] state of one (sequence, head).
 * --------------------------------------------------------------------------------- */
enum { POLAR_DELTA_NORMALIZE_QK = 1u };

typedef struct {
  int32_t n_heads;                  /* H >= 1                                              */
  int32_t key_dim;                  /* d_k; must be 64 (only size)                       */
  int32_t value_dim;                /* d_v; must be 64 (only size)                       */
  uint32_t flags;                   /* POLAR_DELTA_* bits                                  */
} polar_delta_params;

/*
 * One step for B sequences.
 *   state_pool  device float32 [num_slots, H, d_v, d_k], row-major; sequence b's state is
 *               slot slots[b] and is updated in place.  Slots outside [0, num_slots) are
 *               skipped (their outputs are zero, no state is touched).  Two sequences
 *               naming the same slot race (unspecified result).
 *   slots       device int32 [B].
 *   q, k        [B,H,d_k] and v [B,H,d_v], dtype `dt`, 16-byte aligned.
 *   alpha, beta device float32 [B,H]: gate and write strength (normally in [0, 1]).
 *   out         device float32 [B,H,d_v], 16-byte aligned: o = S' q.
 */
POLAR_API polar_status polar_delta_step(const polar_delta_params *p, polar_dtype dt, int32_t B,
                              float *state_pool, int32_t num_slots, const int32_t *slots,
                              const void *q, const void *k, const void *v, const float *alpha,
                              const float *beta, float *out, void *stream);

/*
 * The memory stream over a sequence: for t = 0..T-1 in order, the step above on token t of
 * each of the B sequences, o_t = S_t q_t for every token (the recurrent channel of section
 * 2.1 run over a prompt or a training sequence, its state updated in place as in section
 * 2.2).  The result equals T chained polar_delta_step calls up to fp32 rounding order.
 *   state_pool  as for the step: slot slots[b] holds sequence b's state on entry and its
 *               state after token T-1 on return.  Slots outside [0, num_slots) are
 *               skipped (outputs zero, no state touched); two sequences naming the same
 *               slot race.
 *   q, k        [B,T,H,d_k] and v [B,T,H,d_v], dtype `dt`, row-major, 16-byte aligned.
 *   alpha, beta device float32 [B,T,H].
 *   out         device float32 [B,T,H,d_v], 16-byte aligned: o_t.
 * T = 0 or B = 0 is a no-op.  Errors: POLAR_ERR_NULL_POINTER, POLAR_ERR_BAD_SHAPE (T < 0,
 * B*T*H beyond 2^56), POLAR_ERR_MISALIGNED, POLAR_ERR_UNSUPPORTED as for the step.
 */
POLAR_API polar_status polar_delta_sequence(const polar_delta_params *p, polar_dtype dt,
                                            int32_t B, int32_t T, float *state_pool,
                                            int32_t num_slots, const int32_t *slots,
                                            const void *q, const void *k, const void *v,
                                            const float *alpha, const float *beta, float *out,
                                            void *stream);

/* Static description of a status code. */
POLAR_API const char *polar_status_str(polar_status s);
/* Thread-local detail of the last non-OK return on this thread ("" if none). */
POLAR_API const char *polar_last_error(void);
/* POLAR_ABI_VERSION of the loaded library. */
POLAR_API int32_t polar_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* POLAR_H */
