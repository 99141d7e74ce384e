/*
 * qwen3_attn.h -- C ABI of the MI355X (gfx950) Qwen3 self-attention block.
 *
 * The block (cited by page title and section):
 *   - q/k/v projections without bias, weights stored [out, in]
 *     ("Hand-Writing a Vision-Language Model, Part 1", section "Attention:
 *     Grouped-Query Attention"; "Learning 10", section "Part 2 - tensor by
 *     tensor");
 *   - per-head RMSNorm of q and of k over d_head with learned gains
 *     q_norm / k_norm, eps inside the square root ("Qwen 3 From Scratch",
 *     section "The idea"; "Qwen3 Architecture Layer-by-Layer", section
 *     "Primitives - Qwen3RMSNorm");
 *   - RoPE on q and k, pairing dimension i with i + d_head/2, angle
 *     p * rope_theta^(-2i/d_head) ("Assembling a large model from scratch",
 *     section "The complete code": rope_cos_sin / rotate_half);
 *   - causal grouped-query attention, query head h reading KV head
 *     h / (n_q / n_kv), scores scaled by 1/sqrt(d_head), softmax in fp32
 *     (same sections; mask tril(diagonal = S - T));
 *   - heads merged in head order and projected by o_proj [d, n_q*d_head].
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *     of the descriptor's dtype (fp32 or bf16) unless stated otherwise;
 *     positions are int32 in [0, 2^24) (16,777,216: every such position is
 *     exact in fp32, and the RoPE angle is formed from it exactly).
 *     Accumulation is always fp32.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call is
 *     asynchronous on that stream and never synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued: on any
 *     non-OK status nothing has been launched.  Device-side preconditions
 *     (positions in range) are documented, not checked.  Kernel faults
 *     surface at the caller's next synchronisation of the stream.
 *   - The forward calls allocate nothing; scratch memory is the caller's
 *     workspace.  Two calls in flight at once need two workspaces.
 *   - A handle's weights never change after create.  Its one mutable part is
 *     the optional stage timing (qwen3_attn_enable_stage_timing): while it is
 *     on, each forward call records events into the handle, so calls on one
 *     handle must then not overlap (from several host threads or streams).
 */
#ifndef QWEN3_ATTN_H
#define QWEN3_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qwen3_attn qwen3_attn_t; /* opaque handle */

typedef enum {
  QWEN3_ATTN_F32 = 0,  /* fp32 storage, fp32 arithmetic */
  QWEN3_ATTN_BF16 = 1  /* bf16 storage, fp32 accumulation */
} qwen3_attn_dtype;

typedef enum {
  QWEN3_ATTN_OK = 0,
  QWEN3_ATTN_EINVAL = 1,       /* null pointer, non-positive size, bad combination */
  QWEN3_ATTN_EUNSUPPORTED = 2, /* valid, but outside what the kernels implement */
  QWEN3_ATTN_ENOMEM = 3,       /* device allocation in create failed */
  QWEN3_ATTN_EWORKSPACE = 4,   /* workspace missing or smaller than required */
  QWEN3_ATTN_EHIP = 5          /* a HIP runtime call or kernel launch failed */
} qwen3_attn_status;

/* Block configuration.  Supported: d_head == 128; n_q % n_kv == 0;
 * d_model % 128 == 0; eps >= 0; rope_theta > 1; sliding_window >= 0.
 * The decode calls also need n_q / n_kv in {1, 2, 3, 4, 5, 6, 8, 16}
 * (they return EUNSUPPORTED for any other group size; the prefill calls take
 * every n_q / n_kv). */
typedef struct {
  int32_t d_model;   /* hidden size d */
  int32_t n_q;       /* query heads */
  int32_t n_kv;      /* key/value heads */
  int32_t d_head;    /* head dim (128) */
  float eps;         /* RMSNorm epsilon of q_norm / k_norm (1e-6 for Qwen3) */
  double rope_theta; /* RoPE base (1e6 for Qwen3) */
  int32_t dtype;     /* a qwen3_attn_dtype */
  /* 0: full causal attention.  W > 0: a sliding-window layer -- the token at
   * cache slot i sees only slots i-W+1 .. i, the W most recent keys with its
   * own ("Qwen3 Architecture Layer-by-Layer", sections "Layer 1 -
   * Qwen3Model" and "Layer 3 - Qwen3Attention": the per-layer
   * sliding_window and the sliding-window causal mask).  The caches keep
   * every key.  Keys older than every window of a call are not read, apart
   * from the rest of the key tile holding a window's first key (64 keys in
   * prefill, 16 in decode). */
  int32_t sliding_window;
} qwen3_attn_desc;

/* Device pointers, row-major [out, in] as stored in the checkpoints:
 *   wq [n_q*d_head, d_model], wk / wv [n_kv*d_head, d_model],
 *   wo [d_model, n_q*d_head], q_norm / k_norm [d_head]. */
typedef struct {
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* q_norm;
  const void* k_norm;
} qwen3_attn_weights;

/* Create a handle.  Validates `desc` on the host first (EINVAL /
 * EUNSUPPORTED before any HIP call), then allocates handle-owned device
 * memory and copies the weights into it on `stream` (q/k/v merged into one
 * [(n_q+2*n_kv)*d_head, d_model] matrix).  The caller may free its weight
 * buffers once `stream` has completed.  The weights are immutable
 * afterwards (only the stage-timing state below changes).  On error *out is
 * set to NULL. */
qwen3_attn_status qwen3_attn_create(const qwen3_attn_desc* desc,
                                    const qwen3_attn_weights* weights,
                                    void* stream, qwen3_attn_t** out);

/* As qwen3_attn_create, for a handle that computes the attention half of a
 * decoder layer: every forward call returns
 *     out = hidden + block(RMSNorm(hidden) * input_norm)
 * -- the pre-attention RMSNorm over d_model (eps inside the square root,
 * eps from the descriptor) and the residual add around the block
 * ("Assembling a large model from scratch", section "The complete code": the
 * decoder layer's input_layernorm, attention and residual; "Qwen3
 * Architecture Layer-by-Layer", section "Primitives - Qwen3RMSNorm").
 *   input_norm [d_model] device array of the descriptor's dtype (copied into
 *              the q/k/v weights: the gain is folded into their columns).
 * The residual and the normalised input are both read from `hidden`; out
 * must not overlap hidden.  EINVAL if input_norm is NULL, else as
 * qwen3_attn_create. */
qwen3_attn_status qwen3_attn_create_with_input_norm(const qwen3_attn_desc* desc,
                                                    const qwen3_attn_weights* weights,
                                                    const void* input_norm, void* stream,
                                                    qwen3_attn_t** out);

/* Bytes of workspace a forward call needs (0 if the arguments are invalid).
 * Pure host computation, no HIP call.
 *   is_decode = 0: prefill of B_or_N sequences of T tokens (cache_cap unused);
 *   is_decode = 1: decode of B_or_N sequences (T must be 1), caches of
 *                  cache_cap slots -- contiguous, or paged with cache_cap =
 *                  max_blocks * block_size: the size serves either (a
 *                  contiguous cache may need less). */
size_t qwen3_attn_workspace_size(const qwen3_attn_desc* desc, int32_t is_decode,
                                 int32_t B_or_N, int32_t T, int64_t cache_cap);

/* Prefill: B sequences of T new tokens each, over EMPTY caches
 * ("Assembling a large model from scratch", section "The complete code": the
 * Attention forward with an empty KVCache, so S = T keys and the mask
 * tril(diagonal = S - T) is the plain causal one; the block's steps in the
 * order of "Qwen3 Architecture Layer-by-Layer", section "Layer 3 -
 * Qwen3Attention": projections, q_norm / k_norm, RoPE, attention, o_proj).
 *   hidden    [B, T, d_model]
 *   positions [B, T] int32, drives RoPE only (the mask is by token index:
 *             token t sees cache slots 0..t)
 *   k_cache, v_cache [B, n_kv, cache_cap, d_head]: token t's post-norm,
 *             post-RoPE key and its value are written to slot t; slots
 *             >= T are not touched.  Requires T <= cache_cap.
 *   out       [B, T, d_model]
 * Workspace layout after the call (informative, for tests): the rotated
 * queries [B*T, n_q*d_head], stored multiplied by log2(e)/sqrt(d_head)
 * (the factor the attention kernels need in front of their exp2), then the
 * merged attention output [B*T, n_q*d_head], both of the dtype, each padded
 * to 256 bytes, then (few query tiles only) fp32 partial results of the
 * attention's key-range split. */
qwen3_attn_status qwen3_attn_forward_prefill(qwen3_attn_t* h, const void* hidden,
                                             const int32_t* positions,
                                             void* k_cache, void* v_cache,
                                             int64_t cache_cap, void* out,
                                             int32_t B, int32_t T,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/* Chunked prefill: B sequences each append T new tokens to caches that
 * already hold past_len[b] tokens ("Assembling a large model from scratch",
 * section "The complete code": the KVCache concatenates the new keys and
 * values after the cached ones, and the mask is tril(diagonal = S - T) with
 * S = past_len[b] + T keys).
 *   hidden    [B, T, d_model]
 *   positions [B, T] int32, drives RoPE only (typically past_len[b] + t)
 *   past_len  [B] int32 DEVICE array: cached tokens of sequence b before this
 *             chunk.  Precondition (not checked, device data):
 *             0 <= past_len[b] and past_len[b] + T <= cache_cap.
 *   k_cache, v_cache [B, n_kv, cache_cap, d_head]: slots 0..past_len[b]-1
 *             are read; chunk token t's post-norm, post-RoPE key and its
 *             value are written to slot past_len[b] + t, and it attends to
 *             slots 0..past_len[b] + t.  Other slots are not touched.
 *   out       [B, T, d_model]
 * Same workspace size and layout as qwen3_attn_forward_prefill with the
 * same B and T; qwen3_attn_forward_prefill is this call with every
 * past_len[b] = 0.  EINVAL if past_len is NULL or for the argument errors of
 * qwen3_attn_forward_prefill. */
qwen3_attn_status qwen3_attn_forward_prefill_chunk(qwen3_attn_t* h, const void* hidden,
                                                   const int32_t* positions,
                                                   const int32_t* past_len,
                                                   void* k_cache, void* v_cache,
                                                   int64_t cache_cap, void* out,
                                                   int32_t B, int32_t T,
                                                   void* workspace, size_t workspace_bytes,
                                                   void* stream);

/* Paged KV cache.  The pages name a preallocated pool of paged memory, read
 * directly by the attention kernels, as what real serving systems use in
 * place of a cache grown with torch.cat ("Assembling a large model from
 * scratch": the self-test's fifth answer, the notes after "The complete
 * code", and "Inference view").  They fix no layout; the one here:
 *   k_pool, v_pool [num_blocks, n_kv, block_size, d_head], dtype of the block;
 *   block_table    [B or N, max_blocks] int32 DEVICE array: the keys/values of
 *                  token position p of sequence b live in physical block
 *                  block_table[b * max_blocks + p / block_size], row
 *                  p % block_size.
 * block_size must be a power of two >= 64 (EINVAL otherwise); max_blocks > 0.
 * Device preconditions (not checked): every table entry a sequence uses
 * indexes a block of the pools, and no two sequences write the same block.
 *
 * Chunked prefill over a paged cache: as qwen3_attn_forward_prefill_chunk
 * with slot p of sequence b at the block the table gives.  past_len may be
 * NULL (empty caches).  Precondition: past_len[b] + T <= max_blocks *
 * block_size.  Workspace: qwen3_attn_workspace_size(desc, 0, B, T, 0). */
qwen3_attn_status qwen3_attn_forward_prefill_paged(qwen3_attn_t* h, const void* hidden,
                                                   const int32_t* positions,
                                                   const int32_t* past_len,
                                                   const int32_t* block_table,
                                                   int32_t max_blocks,
                                                   void* k_pool, void* v_pool,
                                                   int32_t block_size, void* out,
                                                   int32_t B, int32_t T,
                                                   void* workspace, size_t workspace_bytes,
                                                   void* stream);

/* Variable-length batch: the tokens of B requests of different lengths packed
 * into one token list, each request attending only to its own keys ("Assembling
 * a large model from scratch", section "Inference view": the tokens of many
 * requests form one batch with attention computed per request; the summary
 * list after the section's opening: flattened tokens plus batching metadata).
 *   hidden     [total_tokens, d_model], the requests one after another
 *   positions  [total_tokens] int32, drives RoPE only
 *   cu_seqlens [B + 1] int32 DEVICE array: request b owns token rows
 *              cu_seqlens[b] .. cu_seqlens[b+1]-1.  Preconditions (not
 *              checked, device data): cu_seqlens[0] = 0, non-decreasing,
 *              cu_seqlens[B] = total_tokens, every length <= max_seqlen
 *              (empty requests are allowed).
 *   past_len   [B] int32 DEVICE array or NULL: tokens request b already
 *              holds in its cache; its token t is written to slot
 *              past_len[b] + t and sees slots 0 .. past_len[b] + t (as
 *              qwen3_attn_forward_prefill_chunk).
 *   block_table NULL: k_cache, v_cache are [B, n_kv, cache_cap, d_head]
 *              (max_blocks and block_size unused); else they are pools
 *              [num_blocks, n_kv, block_size, d_head] addressed through the
 *              table [B, max_blocks] as qwen3_attn_forward_prefill_paged
 *              (cache_cap unused).  Precondition: past_len[b] + length of b
 *              <= the cache's slots per request.
 *   out        [total_tokens, d_model]
 *   max_seqlen the longest request (1 <= max_seqlen <= total_tokens); the
 *              kernels are sized for it, so a far larger value only wastes
 *              launches.
 * With every length equal to T this is qwen3_attn_forward_prefill_chunk
 * (or _paged) bit for bit.  EINVAL if cu_seqlens is NULL, if
 * B * max_seqlen < total_tokens, or for the argument errors of those calls.
 * Workspace: qwen3_attn_workspace_size_varlen(desc, B, total_tokens,
 * max_seqlen); layout as qwen3_attn_forward_prefill with total_tokens rows. */
qwen3_attn_status qwen3_attn_forward_prefill_varlen(
    qwen3_attn_t* h, const void* hidden, const int32_t* positions, const int32_t* cu_seqlens,
    const int32_t* past_len, const int32_t* block_table, int32_t max_blocks, void* k_cache,
    void* v_cache, int64_t cache_cap, int32_t block_size, void* out, int32_t B,
    int32_t total_tokens, int32_t max_seqlen, void* workspace, size_t workspace_bytes,
    void* stream);

/* Workspace bytes of qwen3_attn_forward_prefill_varlen (0 if invalid).  Pure
 * host computation. */
size_t qwen3_attn_workspace_size_varlen(const qwen3_attn_desc* desc, int32_t B,
                                        int32_t total_tokens, int32_t max_seqlen);

/* Decode over a paged cache: as qwen3_attn_forward_decode (positions[s] =
 * L_s cached tokens; the new token is written at position L_s and attends to
 * positions 0..L_s), with the rows found through the block table.
 * Precondition: L_s < max_blocks * block_size.  Workspace:
 * qwen3_attn_workspace_size(desc, 1, N, 1, max_blocks * block_size). */
qwen3_attn_status qwen3_attn_forward_decode_paged(qwen3_attn_t* h, const void* hidden,
                                                  const int32_t* positions,
                                                  const int32_t* block_table,
                                                  int32_t max_blocks,
                                                  void* k_pool, void* v_pool,
                                                  int32_t block_size, void* out, int32_t N,
                                                  void* workspace, size_t workspace_bytes,
                                                  void* stream);

/* Decode: one new token for each of N sequences ("Assembling a large model
 * from scratch", section "The complete code": KVCache.update appends the new
 * key and value after the L cached ones, and the mask tril(diagonal = S - T)
 * with T = 1, S = L + 1 lets the new token see every key, its own included;
 * the generate loop calls this once per new token).
 *   hidden    [N, d_model]
 *   positions [N] int32 device array, positions[s] = L_s = the number of
 *             tokens already cached for sequence s (0 allowed).  Precondition
 *             (not checked, device data): 0 <= L_s < cache_cap.
 *   k_cache, v_cache [N, n_kv, cache_cap, d_head]: slots 0..L_s-1 hold the
 *             sequence's cached keys/values; the new token's key/value are
 *             written to slot L_s and it attends to slots 0..L_s.
 *   out       [N, d_model]
 * Re-running the same call is idempotent (same slot, same values). */
qwen3_attn_status qwen3_attn_forward_decode(qwen3_attn_t* h, const void* hidden,
                                            const int32_t* positions,
                                            void* k_cache, void* v_cache,
                                            int64_t cache_cap, void* out, int32_t N,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* Scratch bytes available to qwen3_attn_forward_decode_noalloc (64 MiB). */
#define QWEN3_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory at all -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation:
 * qwen3_attn_forward_decode with the same arguments, validation, kernels and
 * results, minus the workspace.  Its scratch memory is a static device array
 * of QWEN3_ATTN_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * held until the process ends; the call allocates and frees nothing.
 *   - A call that needs more than QWEN3_ATTN_NOALLOC_SCRATCH_BYTES of scratch
 *     (at most qwen3_attn_workspace_size(desc, 1, N, 1, cache_cap)) returns
 *     EWORKSPACE and launches nothing (the 0.6B shape fits 64 sequences with
 *     caches of 32832 slots).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on a
 *     GPU (several streams or host threads) race and give wrong results.
 *     Serialise them, or use qwen3_attn_forward_decode with a workspace each.
 *   - The first call on each device looks the array's device address up
 *     (EHIP if that fails). */
qwen3_attn_status qwen3_attn_forward_decode_noalloc(qwen3_attn_t* h, const void* hidden,
                                                    const int32_t* positions,
                                                    void* k_cache, void* v_cache,
                                                    int64_t cache_cap, void* out, int32_t N,
                                                    void* stream);

/* Free the handle's device memory (synchronises the device first so no
 * enqueued work still reads it).  NULL is a no-op. */
void qwen3_attn_destroy(qwen3_attn_t* h);

/* Measurement aid.  With capacity > 0, each later forward call on this handle
 * records a HIP event on its stream before each of its three kernels
 * (q/k/v projection, attention, o_proj) and one after the last, for up to
 * `capacity` calls; capacity 0 turns it off.  This is the handle's only
 * mutable state: while timing is on, forward calls on the handle must not
 * overlap (not thread-safe).  The handle's results are unaffected. */
qwen3_attn_status qwen3_attn_enable_stage_timing(qwen3_attn_t* h, int32_t capacity);

/* Waits for the last recorded call, then returns in ms[0..2] the summed
 * kernel durations (ms) over the calls recorded since the previous read, and
 * their number in *n_calls; then starts a new recording window.  `ms` is a
 * host array of at least 3 floats. */
qwen3_attn_status qwen3_attn_stage_times(qwen3_attn_t* h, float* ms, int32_t* n_calls);

/* Static description of a status code. */
const char* qwen3_attn_status_string(qwen3_attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* QWEN3_ATTN_H */
