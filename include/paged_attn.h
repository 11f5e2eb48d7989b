/*
 * paged_attn.h -- C ABI of libpagedattn.so, paged KV-cache attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow the attention layer of the Nano-vLLM engine as
 * described on "Nano-vLLM System Architecture Analysis", section 2 "Core
 * Components":
 *   - "Paged KV Cache": the KV cache is split into fixed 256-token blocks
 *     drawn from a free pool; blocks may be shared between sequences.
 *   - "Attention with Paged Cache": computed K/V entries are stored into the
 *     paged cache via slot_mapping; prefill with a prefix cache gathers cached
 *     K/V and concatenates the newly computed ones; decode gathers all cached
 *     K/V before attention.
 * and section 3 "Lifecycle of a Request" (prepare_inputs builds block tables
 * and slot mappings per step). Attention itself is softmax(q k^T * scale) v
 * (Baidu article on Nano-vLLM, "TorchScript Optimization"), with grouped-query
 * heads ("Differences from Normal nanoGPT Inference", item 6).
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout. All tensors are dense and row-major, in device memory.
 *   pools    k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim]
 *            The token at logical position p of sequence i lives in block
 *            block_tables[i][p / block_size], row p % block_size; its flat
 *            slot is block_id * block_size + row.
 *   block_tables : int32 [num_seqs, max_blocks_per_seq]; entries past
 *            ceil(context_lens[i] / block_size) are never read (-1 by habit).
 *   q / out  : decode [num_seqs, num_q_heads, head_dim];
 *              prefill [total_q, num_q_heads, head_dim].
 *   GQA      : query head g reads KV head g / (num_q_heads / num_kv_heads).
 * Types. pa_dtype names the element type of q, k, v, the pools and out
 *   (all the same). Accumulation is fp32; bf16 outputs are rounded to
 *   nearest-even. Metadata is int32.
 * Supported shapes. block_size == 256; head_dim in {64, 128};
 *   num_q_heads % num_kv_heads == 0; num_blocks * block_size < 2^31.
 * Streams. `stream` is a hipStream_t (NULL = the legacy default stream).
 *   PA_OK means the work was enqueued on `stream`; it runs asynchronously.
 * Ownership. The caller allocates and frees every buffer, including the
 *   workspace. The library keeps no pointer after a call returns and
 *   allocates no device memory.
 * Errors. Each call validates its host-side arguments before touching the
 *   device and returns a pa_status; nothing aborts or throws across the ABI.
 *   Device-side metadata (block ids, slots, lengths) is the caller's
 *   contract: out-of-range ids, duplicate slots or lengths beyond the table
 *   are undefined behaviour, not detected errors.
 * Threading. Calls are re-entrant. Calls that run concurrently (different
 *   streams) must not share a workspace.
 * Workspaces. The split-context calls keep partial results and 64-bit piece
 *   counters in a caller workspace. Each counter word carries the tag of the
 *   call that counts on it (a fresh epoch per call), and a call's first
 *   arrival on a word raises it to that tag, so words left by any earlier
 *   call -- completed, or abandoned part-way -- need no clearing between
 *   calls. Zero-fill a workspace once before its first use: memory that was
 *   never cleared may hold words above the call's tag, which the kernels
 *   cannot reuse; such an item's output rows are then written as NaN (never
 *   left stale, never merged from missing pieces) and the workspace's error
 *   word is set, which pa_workspace_status reports as PA_ERR_WORKSPACE.
 *   Decode and prefill lay out their scratch differently: one workspace
 *   serves any number of calls of ONE of the two entry points, whatever
 *   their sizes, never both.
 */
#ifndef PAGED_ATTN_H_
#define PAGED_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, non-positive or inconsistent size */
  PA_ERR_UNSUPPORTED = -2, /* valid but not built: dtype, head_dim, block_size */
  PA_ERR_WORKSPACE = -3,   /* workspace missing, too small, or found uncleared */
  PA_ERR_HIP = -4,         /* the HIP runtime reported a launch error */
  PA_ERR_NO_BLOCKS = -5    /* block manager: too few free blocks (preempt, retry) */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

typedef void* pa_stream_t; /* a hipStream_t */

/* Library version string, e.g. "pagedattn 0.1.0 gfx950". Never NULL. */
const char* pa_version(void);

/* Human-readable name of a status code. Never NULL. */
const char* pa_status_string(pa_status status);

/*
 * pa_kv_store -- scatter new K/V rows into the pools through slot_mapping.
 *
 * Defined by "Nano-vLLM System Architecture Analysis", section 2, "Attention
 * with Paged Cache" (computed K/V entries are stored into the paged cache via
 * slot_mapping) and section 3 (prepare_inputs builds the slot mappings).
 *
 * k, v         : [num_tokens, num_kv_heads, head_dim] in `dtype`, read only.
 * slot_mapping : int32 [num_tokens]. Token t is copied, bit for bit, to flat
 *                slot slot_mapping[t] of both pools; a negative entry means
 *                the token is not stored.
 * k_cache, v_cache : the pools, written only at the named slots.
 * num_tokens == 0 is a valid no-op. Duplicate non-negative slots, or slots
 * >= num_blocks * block_size, are undefined behaviour.
 * Supported dtypes: PA_F32, PA_BF16.
 */
pa_status pa_kv_store(void* k_cache, void* v_cache, const void* k, const void* v,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                      pa_stream_t stream);

/*
 * pa_rope_kv_store -- rotary position embedding of the new tokens' q and k,
 * with the rotated k and the plain v stored into the pools (one pass).
 *
 * The pages name RoPE among the features of the model Nano-vLLM serves
 * ("Nano-vLLM System Architecture Analysis", section "Differences from Normal
 * nanoGPT Inference", item 6) and store computed K/V via slot_mapping
 * (section 2, "Attention with Paged Cache"); they give no formula. The
 * rotation implemented: elements i and i + head_dim/2 of a head row form pair
 * i (i < head_dim/2); at position p the pair (a, b) becomes
 * (a cos t - b sin t, b cos t + a sin t) with t = p * rope_theta^(-2i/head_dim).
 * Every query head and KV head of a token turns the same way; v is not
 * rotated.
 *
 * q            : [num_tokens, num_q_heads, head_dim], read only.
 * q_out        : [num_tokens, num_q_heads, head_dim], the rotated q; may be q
 *                itself (in place). Must not overlap k, v or the pools.
 * k, v         : [num_tokens, num_kv_heads, head_dim], read only.
 * positions    : int32 [num_tokens], each token's position in its sequence.
 * slot_mapping : int32 [num_tokens] as in pa_kv_store: the rotated k row and
 *                the v row of token t go to flat slot slot_mapping[t]; a
 *                negative entry stores nothing (q is rotated regardless).
 * rope_theta   : the base of the angles, finite and > 0.
 * The angles are formed in double precision and reduced modulo 2 pi before
 * the single-precision rotation, so large positions keep full accuracy.
 * num_tokens == 0 is a valid no-op. Same dtypes, head dims and error codes as
 * pa_kv_store; num_q_heads must be a positive multiple of num_kv_heads.
 */
pa_status pa_rope_kv_store(void* q_out, void* k_cache, void* v_cache, const void* q, const void* k,
                           const void* v, const int32_t* positions, const int32_t* slot_mapping,
                           int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks, float rope_theta,
                           pa_dtype dtype, pa_stream_t stream);

/*
 * pa_qknorm_rope_kv_store -- pa_rope_kv_store with QK-Norm first: every q and
 * k head row x (head_dim elements) becomes x / sqrt(mean(x^2) + eps) * w,
 * with w = q_norm_weight for q heads and k_norm_weight for k heads ([head_dim]
 * each, in `dtype`, 16-byte aligned, shared by all heads), and is then rotated
 * as in pa_rope_kv_store; v is stored as given. The pages list QK-Norm among
 * the served model's features next to RoPE ("Nano-vLLM System Architecture
 * Analysis", "Differences from Normal nanoGPT Inference", item 6) without a
 * formula; the normalisation above is the reading taken. Arithmetic is fp32,
 * with one rounding to `dtype` at the end. eps must be finite and >= 0; null
 * weights are PA_ERR_INVALID_ARG. Other arguments and errors as in
 * pa_rope_kv_store.
 */
pa_status pa_qknorm_rope_kv_store(void* q_out, void* k_cache, void* v_cache, const void* q, const void* k,
                                  const void* v, const void* q_norm_weight, const void* k_norm_weight, float eps,
                                  const int32_t* positions, const int32_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float rope_theta, pa_dtype dtype, pa_stream_t stream);

/*
 * pa_paged_attn_decode -- one query token per sequence attending over its
 * whole paged context.
 *
 * Defined by "Nano-vLLM System Architecture Analysis", section 2, "Attention
 * with Paged Cache" (decode attends over all cached K/V of the sequence's
 * blocks) and section 3 (decode produces one token per sequence per step).
 * The K/V are streamed from the blocks in place; no gathered copy is made.
 *
 * out          : [num_seqs, num_q_heads, head_dim] in `dtype`, written.
 * q            : [num_seqs, num_q_heads, head_dim] in `dtype`.
 * context_lens : int32 [num_seqs], each in [1, max_context_len]; the count
 *                includes the token stored in the same step. (A length
 *                outside that range is a caller error: it is clamped to what
 *                the block table holds and a non-positive one leaves that
 *                sequence's output unwritten.)
 * max_context_len : host-side upper bound of context_lens; must not exceed
 *                max_blocks_per_seq * block_size.
 * scale        : multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 * workspace    : device scratch of at least pa_decode_workspace_bytes(...)
 *                bytes for the split-context partial results, 16-byte
 *                aligned, zero-filled once before its first use and then
 *                reused without clearing (see Workspaces above).
 *                workspace may be NULL when max_context_len <= 64
 *                (pa_decode_workspace_bytes returns 0 then).
 * Supported dtypes: PA_F32, PA_BF16.
 */
pa_status pa_paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               pa_dtype dtype, void* workspace, size_t workspace_bytes,
                               pa_stream_t stream);

/*
 * pa_paged_attn_decode_noalloc -- pa_paged_attn_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Same arguments, rules, results
 * (bit for bit) and errors as pa_paged_attn_decode, without the workspace:
 * the split-context scratch is a fixed array inside the library, one per GPU,
 * of pa_decode_noalloc_scratch_bytes() bytes (about 8.9 MB), held until the
 * process ends. It covers up to 65536 (sequence, query head) pairs; larger
 * calls return PA_ERR_WORKSPACE before touching the device. The call
 * allocates nothing: its first call on a GPU looks up that GPU's copy of the
 * array (a symbol-address query), later calls reuse the address. `stream`
 * must belong to the current device. Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (other streams, other
 * threads) race on it: issue them one after another. Nothing needs clearing
 * between calls (the piece counters carry a fresh tag per call).
 */
pa_status pa_paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_context_len, float scale, pa_dtype dtype, pa_stream_t stream);

/* Bytes of the per-GPU scratch array pa_paged_attn_decode_noalloc uses. */
size_t pa_decode_noalloc_scratch_bytes(void);

/*
 * pa_paged_attn_decode_ex -- pa_paged_attn_decode with an explicit number of
 * workgroups, 0 to 2048 (0 = the library's choice, the same as
 * pa_paged_attn_decode; more than 2048 is PA_ERR_INVALID_ARG). The decode
 * work -- every 64 tokens of every (sequence, query-head group) -- is cut
 * into num_workgroups equal contiguous shares, so a long context may be split
 * over several workgroups and merged afterwards. Results for one
 * num_workgroups value are bit-identical from run to run; different values
 * agree to rounding.
 */
pa_status pa_paged_attn_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                  pa_dtype dtype, int32_t num_workgroups, void* workspace,
                                  size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_paged_attn_decode_store -- the decode step in one launch: the store of
 * the step's new K/V rows (pa_kv_store) fused with pa_paged_attn_decode.
 *
 * The pages store each step's computed K/V via slot_mapping and then attend
 * over all cached K/V ("Nano-vLLM System Architecture Analysis", section 2,
 * "Attention with Paged Cache"). Here sequence t's new token is k_new[t],
 * v_new[t] ([num_seqs, num_kv_heads, head_dim], one new token per sequence,
 * in sequence order): it is written to flat slot slot_mapping[t] of the pools
 * (nothing when negative) and, within the same launch, read in flight as
 * position context_lens[t] - 1 of the sequence's context. The result equals
 * pa_kv_store followed by pa_paged_attn_decode whenever slot_mapping[t] is the
 * slot of position context_lens[t] - 1 of sequence t (the engine's layout); no
 * other sequence may read that slot in the same call. Other arguments, rules
 * and errors as for pa_paged_attn_decode (library-chosen grid).
 */
pa_status pa_paged_attn_decode_store(void* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                     const void* v_new, const int32_t* slot_mapping, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                     pa_dtype dtype, void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Number of workgroups pa_paged_attn_decode launches for these sizes on the
 * current device: one per compute unit, capped by the number of work units,
 * by 8 per (sequence, query-head group) item (small batches) and by 2048.
 * 0 for sizes the library does not support. Queries the HIP runtime (falls
 * back to 256 compute units when no device is visible).
 */
int32_t pa_decode_num_workgroups(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, pa_dtype dtype);

/*
 * Workspace bytes that decode needs for these sizes with any number of
 * workgroups: a 256-byte header, two partial-result slots per workgroup of
 * the largest grid and one 8-byte counter per (sequence, query head), so it
 * does not grow with the context length (0 when max_context_len <= 64,
 * where nothing is ever split). max_q_len is ignored (decode has one query
 * token per sequence).
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_q_len, int32_t max_context_len);

/*
 * pa_paged_attn_prefill -- causal attention of new tokens over each
 * sequence's cached blocks followed by the new tokens themselves.
 *
 * Defined by "Nano-vLLM System Architecture Analysis", section 2, "Attention
 * with Paged Cache" (prefill with a prefix cache gathers the cached K/V and
 * concatenates the newly computed ones) and "Scheduler" (chunked prefill
 * splits a long prompt over steps, so a chunk follows cached tokens). It also
 * serves speculative verification, where the target model checks a few
 * proposed tokens in one parallel mini-prefill ("What Is an Inference Engine,
 * Anyway?", Technical details).
 *
 * q            : [total_q, num_q_heads, head_dim]; k, v : [total_q,
 *                num_kv_heads, head_dim]: the new tokens' projections.
 * cu_seqlens   : int32 [num_seqs + 1], cu_seqlens[0] = 0, non-decreasing,
 *                cu_seqlens[num_seqs] = total_q. Sequence i owns rows
 *                cu_seqlens[i] .. cu_seqlens[i+1]-1 (n_i <= max_q_len).
 * context_lens : int32 [num_seqs] = cached + new tokens; the first
 *                c_i = context_lens[i] - n_i positions come from the pools
 *                through block_tables, the last n_i from k/v (the pools are
 *                not read at those positions, whether or not they were stored).
 * Causality    : new token j of sequence i (position c_i + j) attends to
 *                positions 0 .. c_i + j.
 * out          : [total_q, num_q_heads, head_dim], written.
 * workspace    : as for decode, sized by pa_prefill_workspace_bytes; used
 *                when short query chunks are split along the context.
 * Accuracy     : fp32 scores, softmax and accumulation; the weights are
 *                rounded to bf16 for the matrix cores (row sums taken from
 *                the same rounded weights). Where a row's context is split
 *                over workgroups, each piece's normalised output is kept as
 *                bf16 (its log-sum-exp as fp32) until the pieces are
 *                combined, in piece order, so results do not vary from run
 *                to run.
 * Supported dtypes: PA_BF16 (PA_F32 returns PA_ERR_UNSUPPORTED).
 */
pa_status pa_paged_attn_prefill(void* out, const void* q, const void* k, const void* v,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_q,
                                int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                pa_stream_t stream);

/*
 * pa_paged_attn_prefill_ex -- pa_paged_attn_prefill with an explicit number
 * of workgroups: 0 is the library's choice (the same as
 * pa_paged_attn_prefill); a positive value is used up to the largest grid of
 * the row tile the call gets (256 workgroups for 256-row tiles, taken when
 * max_q_len * num_q_heads / num_kv_heads > 128; 512 for 128-row tiles; 1024
 * for 32-row tiles), larger values are lowered to it; negative values return
 * PA_ERR_INVALID_ARG. The key tiles of all (sequence, KV head, query tile)
 * items are cut into num_workgroups equal contiguous shares, so an item may
 * be split over several workgroups and merged afterwards. Results for one
 * num_workgroups value are bit-identical from run to run; different values
 * agree to rounding.
 */
pa_status pa_paged_attn_prefill_ex(void* out, const void* q, const void* k, const void* v,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_q,
                                   int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                   pa_dtype dtype, int32_t num_workgroups, void* workspace,
                                   size_t workspace_bytes, pa_stream_t stream);

/* Workspace bytes prefill needs for these sizes (an upper bound; may be 0). */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_q_len, int32_t max_context_len);

/*
 * pa_workspace_status -- waits for the work queued on `stream`, then reads
 * and clears the workspace's error word. PA_OK: no call since the last check
 * met a counter it could not reuse. PA_ERR_WORKSPACE: some call did (the
 * workspace was not zero-filled before its first use; the affected items'
 * output rows hold NaN); zero-fill it and repeat those calls.
 * PA_ERR_INVALID_ARG for a NULL workspace or one under 256 bytes; PA_ERR_HIP
 * when the copy or the wait fails. Synchronises `stream`: a diagnostic, not
 * for the hot path. Works for decode, fp8 decode, decode-graph and prefill
 * workspaces alike.
 */
pa_status pa_workspace_status(void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * fp8 KV cache. The pages mention quantised KV-cache transfers ("Why
 * Understand Inference Engine Architecture?", Tensor Parallelism
 * Optimization, item 3) but fix no format. Reading taken: codes are OCP FP8
 * E4M3 (bias 7, subnormals, S.1111.111 = NaN, largest finite 448), one code
 * per element, pools uint8 [num_blocks, 256, num_kv_heads, head_dim] with one
 * fp32 scale per pool (k_scale, v_scale > 0, finite). Element x is stored as
 * the code nearest to clamp(fp32(x) * fp32(1/s), -448, 448), ties to even
 * (1/s formed in fp32 by the library); code c reads back as value(c) * s.
 * Supported: head_dim 128, bf16 k/v/q/out.
 */

/* pa_kv_store with quantisation: bf16 k, v [num_tokens, num_kv_heads, 128]
 * become fp8 codes at the slots slot_mapping names (negative: not stored).
 * The codes are a deterministic function of the inputs (bit-exact). */
pa_status pa_kv_store_fp8(void* k_cache, void* v_cache, const void* k, const void* v,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, float k_scale,
                          float v_scale, pa_stream_t stream);

/* Workspace bytes of pa_paged_attn_decode_fp8: the same as
 * pa_decode_workspace_bytes for these sizes, under the same rules
 * (zero-filled once before the first call; one workspace per stream of
 * calls). 0 when none is needed or the sizes are unsupported (head_dim other
 * than 128). */
size_t pa_decode_fp8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                     int32_t max_context_len);

/* pa_paged_attn_decode over fp8 pools: q and out bf16 [num_seqs,
 * num_q_heads, 128]; attention over the dequantised K/V (score =
 * scale * q.(code_k * k_scale), output = sum p (code_v * v_scale) / sum p),
 * fp32 accumulation, bf16 output rounded to nearest-even. One launch on
 * `stream`, the work split and in-kernel merge of pa_paged_attn_decode
 * (results bit-identical from run to run). Same argument rules as
 * pa_paged_attn_decode. */
pa_status pa_paged_attn_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_context_len, float scale, float k_scale, float v_scale,
                                   void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Decode-step graphs -- the store of the step's new K/V and paged decode, as
 * pa_paged_attn_decode_store runs them (one kernel), captured once as HIP
 * graphs for batch buckets 1, 2, 4, ... up to max_batch (<= 512; the last
 * bucket is max_batch itself) and replayed with one launch per step. As for
 * pa_paged_attn_decode_store, slot_mapping[t] must be the slot of position
 * context_lens[t] - 1 of sequence t (or -1); the result then equals
 * pa_kv_store followed by pa_paged_attn_decode.
 *
 * Defined by "Nano-vLLM System Architecture Analysis", section 2 "CUDA
 * Graphs" (decode steps captured as graphs, eager mode beyond 512 sequences)
 * and "Differences from Normal nanoGPT Inference", item 4 (graphs captured
 * for batch sizes 1, 2, 4, 8, ... 512; a step runs the closest one that
 * holds it).
 *
 * The graphs read and write the static buffers named at creation (device
 * pointers, rows for max_batch sequences, layouts as for pa_kv_store and
 * pa_paged_attn_decode). Before each launch the caller writes the first
 * num_seqs rows of q, k_new, v_new, slot_mapping, block_tables and
 * context_lens. The launch then makes rows num_seqs .. bucket-1 inert
 * (slot -1: nothing stored; context 0: no output written) and writes the
 * replay's piece-counter tag into the workspace header, with a small kernel
 * on `stream`, and replays the bucket's graph on `stream`: out rows
 * 0 .. num_seqs-1 receive the step's attention. Contexts may be up to
 * max_blocks_per_seq * block_size tokens (the graphs are captured for that
 * bound). The workspace (required; zero-filled before the first launch,
 * sized by pa_decode_workspace_bytes(max_batch, num_q_heads, head_dim, 0,
 * max_blocks_per_seq * block_size)) belongs to the graph set alone; launches
 * on one graph set must not overlap. num_seqs > max_batch returns
 * PA_ERR_INVALID_ARG (run eagerly instead); num_seqs == 0 is a no-op.
 */
typedef struct pa_decode_graphs pa_decode_graphs;

typedef struct {
  void* out;                   /* [max_batch, num_q_heads, head_dim] */
  const void* q;               /* [max_batch, num_q_heads, head_dim] */
  const void* k_new;           /* [max_batch, num_kv_heads, head_dim] */
  const void* v_new;           /* [max_batch, num_kv_heads, head_dim] */
  int32_t* slot_mapping;       /* [max_batch] */
  const int32_t* block_tables; /* [max_batch, max_blocks_per_seq] */
  int32_t* context_lens;       /* [max_batch] */
  void* k_cache;               /* [num_blocks, block_size, num_kv_heads, head_dim] */
  void* v_cache;
  void* workspace;
  size_t workspace_bytes;
} pa_decode_graph_buffers;

/* Captures the bucket graphs (nothing runs). *out receives the handle. The
 * capture uses a stream of the library's own; `bufs` is copied. */
pa_status pa_decode_graphs_create(const pa_decode_graph_buffers* bufs, int32_t max_batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, float scale, pa_dtype dtype,
                                  pa_decode_graphs** out);

/* One decode step over the first num_seqs rows (see above). */
pa_status pa_decode_graphs_launch(pa_decode_graphs* graphs, int32_t num_seqs, pa_stream_t stream);

/* The bucket a step of num_seqs sequences runs in; 0 when none holds it. */
int32_t pa_decode_graphs_bucket(const pa_decode_graphs* graphs, int32_t num_seqs);

/* Releases the graphs. NULL is a no-op. */
void pa_decode_graphs_destroy(pa_decode_graphs* graphs);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H_ */
