/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-head Latent Attention hot path.
 *
 * What the library computes (page titles and page parts):
 *   - "MLA low-rank attention" tech note [what the KV cache stores]: per token
 *     only the latent c^KV (d_c values) and one RoPE key k^R shared by all heads
 *     (d_h^R values) are cached; [(2) Key] k^R = RoPE(W^KR h) comes from h, not
 *     from c^KV; [(4) attention and output] o_{t,i} = sum_{j<=t}
 *     softmax_j(q_{t,i} . k_{j,i} / sqrt(d_h^C + d_h^R)) v^C_{j,i}.
 *   - "From LLaMA to DeepSeek [01] - MLA (part 1)" [section 6, matrix
 *     absorption]: decode transforms the query once and dots it with the cached
 *     latent rows, and applies W^UV once at the end; [section 7] prefill expands
 *     K and V instead.
 *   - atyun.com MLA explainer [KV cache]: each decode step appends the new
 *     token's entry to the cache and reuses the rest; [RoPE] consecutive pairs
 *     of dimensions are rotated by position-dependent angles.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *     never allocates or frees memory, never synchronises, and only enqueues
 *     work on the stream it is given (a hipStream_t; NULL = the null stream).
 *   - Tensors are dense row-major.  Element type is bf16 or fp32 as given by
 *     mla_dims.dtype, except int32 index arrays.  Weights are stored out x in
 *     per head: W^UK and W^UV are [n_heads, d_nope, d_latent], head i's block
 *     mapping a latent row to that head's d_nope-long key/value.
 *   - One cached row is [c^KV (d_latent) ; RoPE(k^R, position) (d_rope)],
 *     d_latent + d_rope elements; rows live in pages of page_size rows.  Token
 *     at position p of sequence b is in slot p % page_size of physical page
 *     page_table[b * max_pages + p / page_size].
 *   - RoPE: pair k = (x_2k, x_2k+1) is rotated by angle p * base^(-2k/d_rope)
 *     with [[cos, -sin], [sin, cos]], computed in fp64.
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     on a non-OK status nothing was launched and no memory was touched.
 *     Values that live in device memory (lengths, positions, page ids) are the
 *     caller's precondition: page ids outside [0, num_pages) are skipped by the
 *     kernels (nothing is read from or written to such a page), other
 *     violations give unspecified results but stay inside the given buffers.
 *     A failing kernel launch returns MLA_ERR_HIP.  mla_last_error() returns a
 *     thread-local description of the last non-OK status.
 *   - Alignment: the pool, every floating-point tensor and the workspace must
 *     be 16-byte aligned; int32 arrays (page_table, start_pos, seq_lens) 4-byte
 *     aligned.
 *   - Thread safety: the library keeps no state besides a per-device property
 *     cache; calls are re-entrant.  Calls that share a workspace race unless
 *     they are ordered on one stream.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, bad dims   */
  MLA_ERR_UNSUPPORTED = 2, /* dims outside every implemented kernel family           */
  MLA_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_size() result   */
  MLA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed             */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* Sizes of one MLA layer (symbols of the tech note's symbol table).
 * Two kernel families exist:
 *   - the MFMA family for the DeepSeek-V2 sizes: n_heads 128, d_nope 128,
 *     d_rope 64, d_latent 512, page_size 64, dtype MLA_BF16;
 *   - a generic fp32-arithmetic family for small layers: d_latent <= 1024,
 *     d_nope <= 256, 2 <= d_rope <= 256 (even), n_heads <= 1024,
 *     page_size <= 4096, either dtype.                                          */
typedef struct {
  int32_t n_heads;   /* n_h                                                     */
  int32_t d_nope;    /* d_h^C: per-head content dimension                       */
  int32_t d_rope;    /* d_h^R: RoPE dimension, even, shared key                 */
  int32_t d_latent;  /* d_c: KV latent rank                                     */
  int32_t page_size; /* cached rows per page                                    */
  int32_t dtype;     /* mla_dtype of every floating-point tensor                */
  float sm_scale;    /* softmax scale; 0 selects 1/sqrt(d_nope + d_rope)        */
  float reserved;    /* must be 0                                               */
  double rope_base;  /* RoPE base, > 0 (10000 for the V2 layer)                 */
} mla_dims;

/* A paged latent cache. */
typedef struct {
  void* pool;                 /* [num_pages, page_size, d_latent + d_rope]         */
  int32_t num_pages;          /* pages in the pool (>= 1)                          */
  int32_t max_pages;          /* columns of page_table (>= 1)                      */
  const int32_t* page_table;  /* [batch, max_pages] physical page ids; device mem  */
} mla_paged_cache;

/* Append n_new tokens to each of `batch` sequences.
 * Token k of sequence b has position p = start_pos[b] + k and is written to its
 * slot as [c_kv[b, k, :] verbatim ; RoPE(k_rope[b, k, :], p) rounded to dtype
 * (round to nearest even from the fp64 rotation)].  Lengths are not tracked:
 * the caller passes start_pos (device int32 [batch]) and later seq_lens.
 * c_kv:   [batch, n_new, d_latent]     k_rope: [batch, n_new, d_rope] (pre-RoPE)
 * The cache's page_table is read as [batch, max_pages].                        */
mla_status mla_cache_append(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                            const int32_t* start_pos, int32_t n_new, const void* c_kv,
                            const void* k_rope, void* stream);

/* Bytes of device workspace mla_decode needs for `batch` sequences when it runs
 * with n_workgroups split-KV workgroups (0 = one per compute unit of the
 * current device; enough for any page-table width).                            */
size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t n_workgroups);

/* Weight-absorbed decode: one query per sequence over its paged latent cache.
 * seq_lens: device int32 [batch], the number of cached tokens each query
 *   attends (positions 0 .. seq_lens[b]-1); the query sits at position
 *   seq_lens[b]-1.  A sequence with seq_lens[b] == 0 produces zeros.
 * q_nope: [batch, n_heads, d_nope]   q_rope: [batch, n_heads, d_rope] (pre-RoPE)
 * w_uk, w_uv: [n_heads, d_nope, d_latent]
 * out: [batch, n_heads, d_nope] = per head W^UV_i (sum_j p_ij c_j), before W^O.
 * Steps: q_lat_i = W^UK_i^T q^C_i and RoPE of q^R; split-KV attention over the
 * 576-wide rows with an online softmax; log-sum-exp combine of the splits;
 * output projection through W^UV.
 * n_workgroups: number of split-KV workgroups (0 = one per compute unit, but
 *   no more than batch x max_pages, one per page the table can address); it
 *   changes how the work is split, not the result beyond rounding.
 * workspace: device memory of at least mla_decode_workspace_size(dims, batch,
 *   n_workgroups) bytes; its contents on entry do not matter.
 * timing_events: NULL, or two hipEvent_t that are recorded on `stream`
 *   immediately before and after the attention kernel (profiling only).
 * Range (V2 sizes): the splits hand their normalised latent sums to the
 *   combine in fp16, so every cached c^KV element must have magnitude below
 *   65504 (the largest fp16 value); a larger latent gives non-finite outputs,
 *   never a fault.  bf16 c^KV of the magnitudes a projection produces are far
 *   inside this range.  The generic family has no such limit.                  */
mla_status mla_decode(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                      const int32_t* seq_lens, const void* q_nope, const void* q_rope,
                      const void* w_uk, const void* w_uv, void* out, void* workspace,
                      size_t workspace_bytes, int32_t n_workgroups, void* const* timing_events,
                      void* stream);

/* One decode step: append the newest token of every sequence, then decode.
 * Equivalent to mla_cache_append with start_pos[b] = seq_lens[b] - 1 and
 * n_new = 1 (sequences with seq_lens[b] == 0 append nothing) followed by
 * mla_decode with the same seq_lens, so each query attends its own token
 * ("atyun.com MLA explainer" [KV cache]: a step writes the new token's entry
 * and reuses the cached rest).  For the V2 sizes the append runs inside the
 * first decode kernel, beside the query absorption, instead of as a launch
 * of its own.
 * c_kv_new: [batch, d_latent]   k_rope_new: [batch, d_rope] (pre-RoPE)
 * Every other argument, the workspace size and the errors are as for
 * mla_decode.                                                                */
mla_status mla_decode_step(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                           const int32_t* seq_lens, const void* c_kv_new, const void* k_rope_new,
                           const void* q_nope, const void* q_rope, const void* w_uk,
                           const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                           int32_t n_workgroups, void* const* timing_events, void* stream);
/* mla_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing; its kernels use a
 * static device array inside the library (80 MiB, one copy on every GPU the
 * library runs on, held until the process ends) as their workspace.
 * Limit: the workspace mla_decode_workspace_size(dims, batch, n_workgroups)
 * reports must fit in 80 MiB (batch up to about 170 with 256 workgroups);
 * larger calls return MLA_ERR_WORKSPACE before anything is enqueued.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array has to
 * start at zero (each call writes the parts it reads).  V2 sizes only
 * (MLA_ERR_UNSUPPORTED otherwise).  Every other argument, the results and
 * the errors are as for mla_decode_step.                                    */
mla_status mla_decode_step_noalloc(const mla_dims* dims, const mla_paged_cache* cache,
                                   int32_t batch, const int32_t* seq_lens, const void* c_kv_new,
                                   const void* k_rope_new, const void* q_nope, const void* q_rope,
                                   const void* w_uk, const void* w_uv, void* out,
                                   int32_t n_workgroups, void* const* timing_events, void* stream);

/* Bytes of device workspace mla_decode_hidden needs (0 for unsupported sizes). */
size_t mla_decode_hidden_workspace_size(const mla_dims* dims, int32_t batch, int32_t n_workgroups,
                                        int32_t d_model, int32_t d_q);

/* One decode step that starts from each sequence's newest hidden state h_t:
 * the projections in front of the attention ("MLA low-rank attention" tech
 * note [three-branch computation]: (1) Query c^Q = W^DQ h, q^C = W^UQ c^Q,
 * q^R = W^QR c^Q; (2) Key c^KV = W^DKV h, k^R = W^KR h, the latter from h and
 * shared by all heads), then exactly mla_decode_step with c_kv_new = c^KV,
 * k_rope_new = k^R, q_nope = q^C and q_rope = q^R.  The projections
 * accumulate in fp32 and round their outputs to bf16 (round to nearest
 * even), the storage dtype the step's inputs have.
 * d_model: d (K of the first projections); d_q: d_c' (K of W^UQ and W^QR);
 *   in [1, 2^20], and multiples of 64 for the V2 sizes.
 * h:     [batch, d_model] (the token at position seq_lens[b] - 1)
 * w_dkv: [d_latent, d_model]   w_kr: [d_rope, d_model]   w_dq: [d_q, d_model]
 * w_uq:  [n_heads * d_nope, d_q]   w_qr: [n_heads * d_rope, d_q]
 *   (out x in; head i owns rows i*d_nope .. and i*d_rope .. of W^UQ / W^QR)
 * w_uk, w_uv, out, seq_lens, n_workgroups: as for mla_decode_step.
 * workspace: at least mla_decode_hidden_workspace_size(...) bytes.
 * timing_events: NULL, or two hipEvent_t recorded immediately before the
 *   first projection and after the last one (profiling only).
 * Both kernel families implement it: the MFMA family streams the weights
 * through LDS; the generic family (small layers, either dtype) runs plain
 * fp32-accumulating projections and stores the projected tensors in the
 * layer's dtype.  Errors as for mla_decode_step; the generic family also
 * needs batch <= 65535.                                                     */
mla_status mla_decode_hidden(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                             const int32_t* seq_lens, int32_t d_model, int32_t d_q, const void* h,
                             const void* w_dkv, const void* w_kr, const void* w_dq,
                             const void* w_uq, const void* w_qr, const void* w_uk,
                             const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                             int32_t n_workgroups, void* const* timing_events, void* stream);

/* The whole attention layer of one decode step, from each sequence's newest
 * hidden state h_t to the layer output u_t: exactly mla_decode_hidden, then
 * u = W^O [o_1; ...; o_{n_heads}] ("MLA low-rank attention" tech note [(4)
 * attention and output]: the heads' outputs concatenated head-major and
 * mapped back to d_model), accumulated in fp32 and rounded to bf16 (round to
 * nearest even).
 * w_o: [d_model, n_heads * d_nope] (out x in; column i*d_nope + r takes head
 *   i's element r).   u: [batch, d_model].
 * workspace: at least mla_decode_hidden_workspace_size(...) bytes (the same
 *   layout, which holds the heads' outputs o between the two steps).
 * timing_events: NULL, or two hipEvent_t recorded immediately before and
 *   after the W^O projection (profiling only).
 * Every other argument and error as for mla_decode_hidden (both kernel
 * families).                                                                */
mla_status mla_decode_layer(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                            const int32_t* seq_lens, int32_t d_model, int32_t d_q, const void* h,
                            const void* w_dkv, const void* w_kr, const void* w_dq,
                            const void* w_uq, const void* w_qr, const void* w_uk,
                            const void* w_uv, const void* w_o, void* u, void* workspace,
                            size_t workspace_bytes, int32_t n_workgroups,
                            void* const* timing_events, void* stream);

/* Pre-merge the fixed query up-projection with the key absorption ("From
 * LLaMA to DeepSeek [01]" [section 6]: both matrices are fixed, so their
 * product can be formed once in advance): W^UQK_i = W^UK_i^T W^UQ_i, so that
 * the absorbed content query is q_lat_i = W^UQK_i c^Q.  A one-time weight
 * preparation for mla_decode_hidden_merged, not part of a step.
 * w_uq: [n_heads * d_nope, d_q]   w_uk: [n_heads, d_nope, d_latent]
 * w_uqk (output, caller-allocated): [n_heads, d_latent, d_q], fp32 sums
 *   rounded to bf16 (round to nearest even).
 * d_q: a positive multiple of 64.  V2 sizes only (MLA_ERR_UNSUPPORTED
 * otherwise).                                                              */
mla_status mla_merge_query_weights(const mla_dims* dims, int32_t d_q, const void* w_uq,
                                  const void* w_uk, void* w_uqk, void* stream);

/* mla_decode_hidden with the pre-merged query weight: c^Q = W^DQ h as there,
 * then q_lat_i = W^UQK_i c^Q and q^R = W^QR c^Q in one projection stage, and
 * the decode step with q_lat in place of W^UK_i^T q^C_i.  The same result as
 * mla_decode_hidden up to rounding (q^C is never formed).  It reads
 * n_heads * d_latent * d_q weights for the query instead of n_heads * d_nope
 * * (d_q + d_latent): 4x the bytes of W^UQ plus W^UK at the V2 sizes, so at
 * decode batch sizes, which are bound by reading weights, it is slower.
 * w_uqk: from mla_merge_query_weights.  No w_uq, w_uk.  Every other argument,
 * the workspace size (mla_decode_hidden_workspace_size) and the errors as for
 * mla_decode_hidden.                                                        */
mla_status mla_decode_hidden_merged(const mla_dims* dims, const mla_paged_cache* cache,
                                    int32_t batch, const int32_t* seq_lens, int32_t d_model,
                                    int32_t d_q, const void* h, const void* w_dkv, const void* w_kr,
                                    const void* w_dq, const void* w_uqk, const void* w_qr,
                                    const void* w_uv, void* out, void* workspace,
                                    size_t workspace_bytes, int32_t n_workgroups,
                                    void* const* timing_events, void* stream);

/* Merge W^UV into W^O per head ("From LLaMA to DeepSeek [01]" [section 6]:
 * the value side is absorbed like the key side, and fixed matrices can be
 * multiplied in advance): W^OV = [W^O_1 W^UV_1, ..., W^O_nh W^UV_nh], where
 * W^O_i holds the d_nope columns of W^O that take head i.  A one-time weight
 * preparation for mla_decode_layer_merged.
 * w_o: [d_model, n_heads * d_nope]   w_uv: [n_heads, d_nope, d_latent]
 * w_ov (output, caller-allocated): [d_model, n_heads * d_latent], fp32 sums
 *   rounded to bf16 (round to nearest even).
 * d_model: a positive multiple of 64.  V2 sizes only.                       */
mla_status mla_merge_output_weights(const mla_dims* dims, int32_t d_model, const void* w_o,
                                   const void* w_uv, void* w_ov, void* stream);

/* mla_decode_layer with W^UV merged into W^O: the projections and the decode
 * as mla_decode_hidden, except that the decode ends at the normalised latent
 * outputs o_lat_i (rounded to bf16), then u = W^OV [o_lat_1; ...; o_lat_nh].
 * The same u as mla_decode_layer up to rounding.  W^OV holds n_heads *
 * d_latent * d_model weights against (n_heads * d_nope) * (d_latent +
 * d_model) for W^UV plus W^O: 3.6x the bytes at the V2 sizes, so at decode
 * batch sizes, which are bound by reading weights, it is slower.
 * w_ov: from mla_merge_output_weights; no w_uv, w_o.  Every other argument,
 * the workspace size (mla_decode_hidden_workspace_size) and the errors as for
 * mla_decode_layer (timing_events bracket the W^OV projection).              */
mla_status mla_decode_layer_merged(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                                   const int32_t* seq_lens, int32_t d_model, int32_t d_q,
                                   const void* h, const void* w_dkv, const void* w_kr,
                                   const void* w_dq, const void* w_uq, const void* w_qr,
                                   const void* w_uk, const void* w_ov, void* u, void* workspace,
                                   size_t workspace_bytes, int32_t n_workgroups,
                                   void* const* timing_events, void* stream);

/* Bytes of device workspace mla_prefill needs. */
size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t seq_len);

/* Un-absorbed causal prefill of `batch` prompts of seq_len tokens at positions
 * 0 .. seq_len-1.  Writes the latent cache for every prompt token (as
 * mla_cache_append with start_pos 0), expands K^C = W^UK c and V^C = W^UV c per
 * head, and runs causal attention with q = [q^C ; RoPE(q^R, t)] and
 * k = [K^C ; cached RoPE(k^R, j)], scale as in mla_dims.
 * q_nope: [batch, seq_len, n_heads, d_nope]  q_rope: [batch, seq_len, n_heads, d_rope]
 * c_kv:   [batch, seq_len, d_latent]         k_rope: [batch, seq_len, d_rope]
 * out:    [batch, seq_len, n_heads, d_nope]
 * The page table needs at least ceil(seq_len / page_size) columns
 * (MLA_ERR_INVALID_ARG otherwise).
 * timing_events: NULL, or two hipEvent_t recorded immediately before the K/V
 *   expansion and after the causal attention kernel (profiling only).       */
mla_status mla_prefill(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                       int32_t seq_len, const void* q_nope, const void* q_rope,
                       const void* c_kv, const void* k_rope, const void* w_uk,
                       const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                       void* const* timing_events, void* stream);

/* How mla_prefill_chunk computes a chunk.  EXPAND: expand K^C and V^C for
 * every position and run the causal attention (the prompt form).  ABSORB:
 * treat chunk row t as a decode query at position start_pos[b] + t over the
 * cache (the decode form: each row absorbed, scored against the latent rows),
 * for chunks of at most 256 tokens, V2 sizes only.  AUTO: the cheaper of the
 * two for the chunk length and max_context, from costs measured on MI355X
 * (a short chunk after a long prefix is cheaper absorbed: expanding the
 * prefix costs as much as attending it many times).                         */
typedef enum { MLA_CHUNK_AUTO = 0, MLA_CHUNK_EXPAND = 1, MLA_CHUNK_ABSORB = 2 } mla_chunk_mode;

/* Bytes of device workspace mla_prefill_chunk needs in the given mode: the
 * form the call will run (AUTO: the form AUTO picks for chunk_len and
 * max_context), so a short chunk after a long prefix run absorbed needs no
 * room for expanded keys.  The absorbed form is sized for the current
 * device's compute units.  0 for invalid sizes or modes (ABSORB outside the
 * V2 sizes or above 256 tokens).                                            */
size_t mla_prefill_chunk_workspace_size(const mla_dims* dims, int32_t batch, int32_t chunk_len,
                                        int32_t max_context, int32_t mode);

/* Chunked prefill over an existing latent cache: every sequence b continues
 * with chunk_len prompt tokens at positions start_pos[b] .. start_pos[b] +
 * chunk_len - 1, its earlier positions already cached (by an earlier chunk,
 * mla_prefill or decode steps).  The cache layout is the latent one in both
 * phases and a prompt is processed by expanding it ("MLA low-rank attention"
 * tech note [what the KV cache stores], the hybrid mode; "From LLaMA to
 * DeepSeek [01]" [section 7]: prompts are compute-bound and not absorbed).
 * Steps: append the chunk's rows (as mla_cache_append with start_pos), expand
 * K^C = W^UK c and V^C = W^UV c per head for every position 0 .. start_pos[b]
 * + chunk_len - 1 from the latent rows in the cache, and run causal attention:
 * chunk row t attends positions 0 .. start_pos[b] + t with q = [q^C ;
 * RoPE(q^R, start_pos[b] + t)] and k = [K^C ; cached RoPE(k^R, j)].
 * start_pos: device int32 [batch]; the caller guarantees 0 <= start_pos[b]
 *   and start_pos[b] + chunk_len <= max_context (the kernels clamp start_pos[b]
 *   into that range, so a violation gives wrong results, not a fault).
 * max_context: host int, bound on start_pos[b] + chunk_len; sizes the
 *   workspace (keys are expanded into it for max_context positions per
 *   sequence); the page table needs ceil(max_context / page_size) columns.
 * q_nope, q_rope, c_kv, k_rope, out: as for mla_prefill with seq_len =
 *   chunk_len (the chunk's tokens only).
 * mode: an mla_chunk_mode (MLA_CHUNK_ABSORB with more than 256 tokens:
 *   MLA_ERR_INVALID_ARG; outside the V2 sizes: MLA_ERR_UNSUPPORTED; AUTO
 *   uses EXPAND there).
 * mla_prefill(..., seq_len, ...) is this call with start_pos[b] = 0,
 * max_context = seq_len and MLA_CHUNK_EXPAND.  timing_events as for
 * mla_prefill (ABSORB: around the split-KV attention kernel).               */
mla_status mla_prefill_chunk(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                             const int32_t* start_pos, int32_t chunk_len, int32_t max_context,
                             int32_t mode, const void* q_nope, const void* q_rope, const void* c_kv,
                             const void* k_rope, const void* w_uk, const void* w_uv, void* out,
                             void* workspace, size_t workspace_bytes, void* const* timing_events,
                             void* stream);

/* Static name of a status code. */
const char* mla_status_string(mla_status status);

/* Thread-local description of the last non-OK status ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
