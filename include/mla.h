/*
 * mla.h -- C ABI of the MI355X (gfx950) library for Multi-head Latent
 * Attention with decoupled RoPE in its weight-absorbed form.
 *
 * What is computed (per head i, query at position m, cached token t):
 *
 *   q~_i      = W_UK,i^T q^C_i                       (query absorption)
 *   s_t       = scale * ( q~_i . c_t + R_m q^R_i . R_t k^R_t )
 *   alpha     = softmax_t(s)            over the visible tokens
 *   obar_i    = sum_t alpha_t c_t                    (latent output)
 *   o_i       = W_UV,i obar_i                        (output absorption)
 *
 * Sources: "AI decoupled RoPE MLA" (operatorworld.com) -- recap section for
 * the two absorbed forms (q~ = W^UK^T q, Attn = W^UV sum alpha c), and the
 * decoupled-RoPE section for the score as the sum of a content term and a
 * rotated position term with a d_r-wide position key; "Latent Attention Meets
 * RoPE" (sahipadhai.cc), "Two small, telling details": the position key is
 * one vector per token shared by every head, and the cache holds only the
 * latent and that key; "Multi-Head Latent Attention" (talalahmed.dev), "Why
 * this matters on a GPU": decode still runs the softmax and the weighted sum.
 *
 * Conventions for every call
 * --------------------------
 * - Every pointer to tensor data is DEVICE memory unless its name ends in
 *   _host.  Tensors are dense and row-major in the shapes given.  The caller
 *   owns every buffer; the library allocates nothing and keeps no pointer
 *   after a call returns.
 * - dtype: the cache, q_rope, q_nope, kv_latent, k_rope and the weights
 *   share dims->dtype (MLA_F32 or MLA_BF16).  q_lat has dims->work_dtype.
 *   The latent output out_latent (obar, the input of mla_out_proj), the
 *   layer output of mla_out_proj and lse are always float32, so the path's
 *   roundings stop at the softmax weights (and, for a decode split over the
 *   cache at d_latent 512 with bf16 work_dtype, at its split partials, kept
 *   in the workspace as float16 scaled by a power of two per 128 columns:
 *   2^-11 relative to each group's largest value; float32 everywhere else);
 *   indices are int32.  Accumulation is float32 in every kernel.
 * - Work is enqueued on `stream` (a hipStream_t, NULL = default stream) and
 *   is asynchronous: no call synchronises.  Keep buffers alive until the
 *   stream has passed the work.
 * - Errors: arguments the host can see are checked before anything is
 *   launched; a failed check returns a status code and launches nothing.
 *   mla_last_error() then returns a thread-local description.  Device data
 *   (positions, page ids, lengths) is not validated on the host: an
 *   out-of-range page id or sequence index makes the kernels skip (for
 *   writes) or clamp (for reads) that access, so memory stays safe but the
 *   affected outputs are unspecified.
 * - Debug mode: with MLA_DEBUG_VALIDATE=1 in the environment, every call that
 *   reads or writes the paged cache first checks on the device the
 *   block-table entries (every page of every sequence it will read) and the
 *   cache rows (kv_seq, kv_pos) it will write, and that the device lengths
 *   (seq_lens, or cu_q and q_start_pos) equal their host copies.  It waits for
 *   that check (synchronising `stream`, so not under graph capture) and on a
 *   bad entry returns MLA_ERR_INVALID_ARG, naming the entry, having launched
 *   nothing else.  The check allocates nothing.
 * - Page size must be 64 tokens.  Supported (n_heads, d_latent, d_rope)
 *   for MLA_BF16 attention: (16, 256, 32) and (128, 512, 64); MLA_F32
 *   accepts any n_heads <= 1024, d_latent <= 1024, d_rope <= 128.
 * - Outputs never alias inputs, except that mla_rope_apply and mla_absorb_q
 *   (or mla_rope_absorb_q, both at once) write disjoint column ranges of the
 *   same q_lat buffer.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, negative size, odd d_rope, ... */
  MLA_ERR_UNSUPPORTED = 2, /* a shape / dtype combination with no kernel  */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than needed    */
  MLA_ERR_HIP = 4          /* a HIP runtime call or launch failed         */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef struct {
  int32_t n_heads;     /* H: query heads                                  */
  int32_t d_head;      /* d_h: content query / key width per head        */
  int32_t d_v;         /* value width per head                           */
  int32_t d_latent;    /* d_c: width of the cached latent c_t            */
  int32_t d_rope;      /* d_r: width of the decoupled RoPE channel, even */
  int32_t page_size;   /* tokens per cache page (must be 64)             */
  int32_t dtype;       /* mla_dtype of cache, inputs and weights          */
  int32_t work_dtype;  /* the attention's working precision, and the
                        * mla_dtype of q_lat.  MLA_BF16 (with dtype
                        * MLA_BF16): q_lat, and the softmax weights fed to
                        * the weighted sum, are bf16 -- the fast path.
                        * MLA_F32 with dtype MLA_BF16, the float32 working
                        * precision: q_lat is float32, the score takes q~
                        * as a two-term bf16 split (hi = bf16(x), lo =
                        * bf16(x - hi)) and the weighted sum takes the
                        * softmax weights the same way, so neither is
                        * rounded to bf16 once (twice the MFMA work).
                        * Supported for d_latent + d_rope <= 288.  With
                        * dtype MLA_F32 it must be MLA_F32.               */
  float softmax_scale; /* scale on the content part of the score          */
  float position_scale; /* scale on the position part of the score.  Equal
                        * to softmax_scale: one scale on the summed score.
                        * The two-scale score of "AI decoupled RoPE MLA"
                        * (decoupled-RoPE section: content over sqrt(d),
                        * position over sqrt(d_r)) sets them apart.  The
                        * calls that write the rotated query (mla_rope_apply,
                        * mla_q_project, mla_q_project_folded) multiply it
                        * by position_scale / softmax_scale before its one
                        * rounding, so the attention calls score
                        * softmax_scale * (q~ . c_t) + position_scale *
                        * (R_m q^R . R_t k^R_t) with no extra work.  Finite
                        * and positive.                                    */
  double rope_base;    /* theta_j = rope_base^(-2j/d_r)                  */
} mla_dims;

/* A paged latent cache.  Row (page, slot) holds [ c_t | R_t k^R_t ]: the
 * latent (d_latent) followed by the position key already rotated to its own
 * position t (d_rope).  Sequence b's position p is in physical page
 * block_table[b * max_pages_per_seq + p / page_size], row p % page_size. */
typedef struct {
  void* data;                 /* [num_pages, page_size, d_latent + d_rope]  */
  int64_t num_pages;
  const int32_t* block_table; /* [num_seqs, max_pages_per_seq], -1 = none   */
  int32_t num_seqs;
  int32_t max_pages_per_seq;
} mla_paged_cache;

/* mla_rope_apply -- the decoupled RoPE channel ("AI decoupled RoPE MLA",
 * decoupled-RoPE section: RoPE is applied to the d_r-wide q^R and k^R only;
 * "Detailed Illustration of the Problem", Step 1: rotation by R_{Theta,p}).
 *
 * Query part: for n < n_q and every head h,
 *   q_lat[n, h, d_latent : d_latent + d_rope] = R_{q_pos[n]} q_rope[n, h, :]
 *   q_rope [n_q, H, d_rope], q_pos [n_q], q_lat [n_q, H, d_latent + d_rope].
 * Cache part: for m < n_kv, the row of (kv_seq[m], kv_pos[m]) becomes
 *   [ kv_latent[m, :] | R_{kv_pos[m]} k_rope[m, :] ]
 *   kv_latent [n_kv, d_latent], k_rope [n_kv, d_rope].
 * Angles p * theta_j and their sine / cosine are formed in float64.  Either
 * part may be empty (n = 0; its pointers may then be NULL).  Rows whose
 * sequence, position or page id is out of range are skipped. */
mla_status mla_rope_apply(const mla_dims* dims, const mla_paged_cache* cache,
                          const void* q_rope, const int32_t* q_pos, int64_t n_q, void* q_lat,
                          const void* kv_latent, const void* k_rope, const int32_t* kv_seq,
                          const int32_t* kv_pos, int64_t n_kv, void* stream);

/* mla_absorb_q -- query absorption ("AI decoupled RoPE MLA", recap section:
 * q~_m = W^UK^T q_m, merged ahead of time and independent of the cache).
 *   q_lat[n, h, 0 : d_latent] = W_UK[h]^T q_nope[n, h, :]
 *   q_nope [n_q, H, d_head]; w_uk [H, d_head, d_latent] (stored [out, in],
 *   so k^C = W_UK[h] c); q_lat [n_q, H, d_latent + d_rope]. */
mla_status mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk, int64_t n_q,
                        void* q_lat, void* stream);

/* mla_rope_absorb_q -- mla_rope_apply and mla_absorb_q in one launch: both
 * sides of the query ("AI decoupled RoPE MLA", recap section: q~ = W^UK^T q
 * ahead of the cache; the position part rotated by its own R_m, the
 * decoupled-RoPE section), and the new tokens' cache rows.  Arguments as in
 * the two calls (q_lat gets q~ in [0, d_latent) and R_m q^R in
 * [d_latent, d_latent + d_rope)); the results are bit-identical to calling
 * mla_rope_apply then mla_absorb_q.  With MLA_F32 dims, or n_q = 0, it
 * enqueues the two launches instead.  Every check of both calls runs before
 * anything is launched. */
mla_status mla_rope_absorb_q(const mla_dims* dims, const mla_paged_cache* cache, const void* q_nope,
                             const void* w_uk, const void* q_rope, const int32_t* q_pos, int64_t n_q, void* q_lat,
                             const void* kv_latent, const void* k_rope, const int32_t* kv_seq,
                             const int32_t* kv_pos, int64_t n_kv, void* stream);

/* Bytes of workspace mla_decode needs for this batch (0 when no sequence is
 * split).  seq_lens_host [batch] must hold the same lengths later passed to
 * mla_decode. */
size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host);

/* mla_decode -- absorbed decode attention over the latent cache, split over
 * the cache ("Multi-Head Latent Attention", "Why this matters on a GPU":
 * decode reads the whole cache and still runs softmax and the weighted sum;
 * "AI decoupled RoPE MLA", decoupled-RoPE score equation).
 *   query b sits at position seq_lens[b] - 1 and sees cached positions
 *   0 .. seq_lens[b] - 1;  q_lat [batch, H, d_latent + d_rope] (from
 *   mla_rope_apply + mla_absorb_q);  out_latent [batch, H, d_latent]
 *   (float32) gets obar = sum_t alpha_t c_t;  lse [batch, H] (float32, may be NULL) gets
 *   log sum_t exp(s_t).  A sequence of length 0 yields obar = 0, lse = -inf.
 * seq_lens is the device copy, seq_lens_host the same values on the host
 * (used to plan the split).  workspace: device memory of at least
 * mla_decode_workspace_size() bytes (may be NULL when that is 0).
 * The result is bitwise reproducible and independent of which physical
 * pages hold which positions.  Environment MLA_DECODE_SPLIT_PAGES=k forces
 * splits of k pages (tests); it must be set identically for the size query. */
mla_status mla_decode(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                      const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch,
                      void* out_latent, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Bytes of workspace mla_decode_proj needs for this batch: on bf16 caches a
 * partial slot (and its lse) for every work item of the split plan, split or
 * not; on float32 caches the float32 obar [batch, H, d_latent].  0 when batch
 * is 0, when no sequence has a token (bf16), or when the arguments are
 * rejected.  seq_lens_host as for mla_decode_workspace_size. */
size_t mla_decode_proj_workspace_size(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host);

/* mla_decode_proj -- mla_decode followed by mla_out_proj in one call, the
 * layer's decode output ("AI decoupled RoPE MLA", recap section: the output
 * is W^UV applied to sum_t alpha_t c_t; "Multi-Head Latent Attention", "Why
 * this matters on a GPU").  The split merge and the output absorption run as
 * one launch: obar goes from the merged partials to the projection through
 * on-chip memory and is not written.
 *   q_lat, seq_lens, seq_lens_host, batch, cache as for mla_decode;  w_uv
 *   [H, d_v, d_latent] in the cache dtype;  out [batch, H, d_v] float32 gets
 *   W_UV[h] obar[b, h, :];  lse [batch, H] (float32, may be NULL) as for
 *   mla_decode.  d_v must be 128 (MLA_ERR_UNSUPPORTED otherwise).  A sequence
 *   of length 0 yields out = 0, lse = -inf.
 * workspace: device memory of at least mla_decode_proj_workspace_size()
 * bytes (may be NULL when that is 0); its contents on entry do not matter.
 * On bf16 caches every work item leaves a partial, so a sequence of one item
 * also takes the merge; for a sequence of several items the merge and the
 * projection are mla_decode's and mla_out_proj's arithmetic in the same
 * order, so out and lse equal those two calls' bit for bit; for a sequence of
 * one item obar carries its partial's rounding (float16 scaled per 128
 * columns at d_latent = 512, float32 otherwise).  Bitwise reproducible and
 * independent of which physical pages hold which positions, as mla_decode.
 * Errors: those of mla_decode and mla_out_proj; nothing is launched on a
 * failed check. */
mla_status mla_decode_proj(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                           const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch,
                           const void* w_uv, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* mla_decode_split_kv, mla_merge_out_proj -- mla_decode_proj's two launches
 * as two calls, for callers that enqueue them apart or time each step alone.
 * The first is the split-KV attention over the cache ("Multi-Head Latent
 * Attention", "Why this matters on a GPU"; "AI decoupled RoPE MLA",
 * decoupled-RoPE score equation): every work item of the split plan leaves
 * its normalised partial obar_s and lse_s in the workspace.  The second
 * merges each sequence's partials in split order (lse = log sum_s e^{lse_s},
 * obar = sum_s e^{lse_s - lse} obar_s) and applies the output absorption
 * ("AI decoupled RoPE MLA", recap section: W^UV on the output side).
 *   mla_decode_split_kv: dims, cache, q_lat, seq_lens, seq_lens_host, batch
 *   as for mla_decode_proj; it writes only the workspace.
 *   mla_merge_out_proj: the same dims, seq_lens, seq_lens_host and batch;
 *   w_uv, out, lse as for mla_decode_proj; it reads the workspace the first
 *   call filled.
 * workspace: at least mla_decode_proj_workspace_size() bytes, the same buffer
 * in both calls; its contents between them are private to the library (the
 * partials' format is not part of the interface).  Enqueued in that order on
 * one stream with nothing writing the workspace between them, the pair gives
 * mla_decode_proj's out and lse bit for bit.  bf16 caches only
 * (MLA_ERR_UNSUPPORTED otherwise).  Errors as mla_decode_proj; nothing is
 * launched on a failed check.  mla_merge_out_proj with lengths other than
 * those the workspace was filled with leaves out unspecified (it reads no
 * memory outside the workspace's work items). */
mla_status mla_decode_split_kv(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                               const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch,
                               void* workspace, size_t workspace_bytes, void* stream);
mla_status mla_merge_out_proj(const mla_dims* dims, const int32_t* seq_lens, const int32_t* seq_lens_host,
                              int32_t batch, const void* w_uv, void* out, float* lse, const void* workspace,
                              size_t workspace_bytes, void* stream);

/* mla_decode_noalloc -- mla_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The same computation, arguments, results and errors as
 * mla_decode, with no workspace: the split partials go to a fixed scratch
 * array of 96 MiB that the library holds on each device it runs on until the
 * process ends.  A batch whose partials need more than that
 * (mla_decode_workspace_size) returns MLA_ERR_WORKSPACE and launches nothing.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents (nothing in it needs clearing): calls that overlap on one
 * device (two streams, two threads) race and must be ordered by the caller.
 * Allocates nothing (no hipMalloc or hipFree, no allocating library call). */
mla_status mla_decode_noalloc(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                              const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch,
                              void* out_latent, float* lse, void* stream);

/* mla_prefill -- causal chunked prefill in the same absorbed form.
 *   Sequence b contributes queries cu_q[b] .. cu_q[b+1]-1; its j-th query
 *   sits at position q_start_pos[b] + j and sees cached positions t <= that
 *   position (the chunk's own rows must already be in the cache, written by
 *   mla_rope_apply).  q_lat [cu_q[batch], H, d_latent + d_rope];
 *   out_latent [cu_q[batch], H, d_latent] (float32); lse [cu_q[batch], H] or
 *   NULL.
 * cu_q_host / q_start_pos_host are host copies of cu_q / q_start_pos. */
mla_status mla_prefill(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                       const int32_t* cu_q, const int32_t* q_start_pos, const int32_t* cu_q_host,
                       const int32_t* q_start_pos_host, int32_t batch, void* out_latent, float* lse,
                       void* stream);

/* Bytes of workspace mla_prefill_mha needs: the up-projected keys and values
 * of every position 0 .. T_b - 1 (T_b = q_start_pos[b] + n_q(b)) of every
 * sequence, each sequence's range padded to a multiple of 128 positions:
 * 2 * n_heads * sum_b ceil(T_b / 128) * 128 * 128 float16 values (0 when
 * the arguments are rejected; mla_last_error() says why).  The padded total
 * may not exceed 2^24 - 128 positions. */
size_t mla_prefill_mha_workspace_size(const mla_dims* dims, int32_t batch, const int32_t* cu_q_host,
                                      const int32_t* q_start_pos_host);

/* mla_prefill_mha -- the same causal chunked prefill in the materialised
 * form ("Multi-Head Latent Attention" (talalahmed.dev), the MLA dataflow:
 * each head's key is [W_UK c_t ; R_t k^R_t] and its value W_UV c_t; the
 * "ropeabsorb" README: this and the absorbed form are the same result).  It
 * up-projects every visible position's latent once per head into the
 * workspace, then runs standard causal attention per head (score width
 * d_head + d_rope, value width d_v), which costs 2 n_h (d_h + d_r + d_v) flop
 * per visible (query, key) pair instead of 2 n_h (2 d_c + d_r) -- the cheaper
 * form for long chunks -- and writes the layer output directly.
 *   Queries and positions as in mla_prefill.  q_nope [cu_q[batch], H, d_head]
 *   (the un-absorbed content query); q_lat [cu_q[batch], H, d_latent + d_rope]
 *   of which only the rotated tail [d_latent, d_latent + d_rope) is read
 *   (mla_rope_apply writes it); w_uk [H, d_head, d_latent]; w_uv
 *   [H, d_v, d_latent]; out [cu_q[batch], H, d_v] float32 gets
 *   o = sum_t alpha_t W_UV c_t; lse [cu_q[batch], H] float32 or NULL.
 * workspace: device memory of at least mla_prefill_mha_workspace_size()
 * bytes (otherwise MLA_ERR_WORKSPACE).  The up-projected keys and values,
 * the content query and the softmax weights are rounded to float16; the
 * rotated part stays bf16.  A key, value or content-query element whose
 * float16 rounding would overflow (|x| >= 65520) is stored as NaN instead, so
 * the outputs of that head that it reaches (every query that sees the key,
 * and possibly other queries of the chunk) come out NaN: an input outside
 * float16 range is flagged, never turned into finite wrong values.
 * bf16 inputs and work_dtype only, d_head = d_v = 128,
 * (n_heads, d_latent, d_rope) = (128, 512, 64) or (16, 256, 32); other
 * shapes return MLA_ERR_UNSUPPORTED. */
mla_status mla_prefill_mha(const mla_dims* dims, const mla_paged_cache* cache, const void* q_nope, const void* q_lat,
                           const void* w_uk, const void* w_uv, const int32_t* cu_q, const int32_t* q_start_pos,
                           const int32_t* cu_q_host, const int32_t* q_start_pos_host, int32_t batch, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Per-head position keys ------------------------------------------------
 * The simplified MLA-style cache of "Multi-Head Latent Attention"
 * (talalahmed.dev), "A concrete size comparison": each token keeps the latent
 * and one RoPE key per head, d_latent + n_heads * d_rope numbers (256 + 16 x 32
 * = 768 for that page's example), where the decoupled design keeps one key
 * shared by every head.  Supported for that example's shape only: bf16,
 * n_heads 16, d_latent 256, d_rope 32 (else MLA_ERR_UNSUPPORTED).
 *
 * Cache rows are [ c_t | R_t k^R_{t,0} | ... | R_t k^R_{t,H-1} ], each key
 * rotated to its own position; paging as in mla_paged_cache, with rows of
 * d_latent + n_heads * d_rope elements.  The query side is unchanged: q_lat
 * rows are [ q~_i | R_m q^R_i ] as written by mla_absorb_q and mla_rope_apply
 * (which also applies position_scale). */

/* mla_cache_write_per_head -- write n_kv token rows.
 *   kv_latent [n_kv, d_latent] bf16; k_rope [n_kv, n_heads, d_rope] bf16
 *   (un-rotated); kv_seq / kv_pos [n_kv] int32 device arrays.  Rows whose
 *   (sequence, position) has no page in the block table are skipped.  Angles
 *   and rotation in float64, rounded once. */
mla_status mla_cache_write_per_head(const mla_dims* dims, const mla_paged_cache* cache, const void* kv_latent,
                                    const void* k_rope, const int32_t* kv_seq, const int32_t* kv_pos, int64_t n_kv,
                                    void* stream);

/* mla_decode_per_head -- decode over a per-head-key cache: head i scores
 * softmax_scale * (q~_i . c_t + R_m q^R_i . R_t k^R_{t,i}) over keys
 * 0 .. T_b - 1 and returns obar_i = sum_t alpha_{i,t} c_t and lse, with the
 * arguments, output layout, workspace (mla_decode_workspace_size with the same
 * dims and lengths) and errors of mla_decode.  work_dtype may be MLA_BF16 or
 * MLA_F32 (float32 q_lat; q~ and the softmax weights enter as two-term bf16
 * splits). */
mla_status mla_decode_per_head(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                               const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch, void* out_latent,
                               float* lse, void* workspace, size_t ws_bytes, void* stream);

/* mla_decode_per_head_proj -- mla_decode_per_head followed by mla_out_proj,
 * with the split merge and the output absorption in one launch, as
 * mla_decode_proj is for the shared-key cache: out [batch, H, d_v] float32,
 * lse [batch, H] or NULL; workspace of mla_decode_proj_workspace_size() bytes
 * with the same dims and lengths.  Partials are float32 on this layout, so
 * out and lse equal the two separate calls' bit for bit.  d_v must be 128. */
mla_status mla_decode_per_head_proj(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                                    const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch,
                                    const void* w_uv, void* out, float* lse, void* workspace, size_t ws_bytes,
                                    void* stream);

/* mla_out_proj -- output absorption ("AI decoupled RoPE MLA", recap section:
 * Attn_m = W^UV sum_t alpha_mt c_t).
 *   out[n, h, :] = W_UV[h] out_latent[n, h, :]
 *   out_latent [n, H, d_latent] float32 (with bf16 weights it enters as a
 *   two-term bf16 split); w_uv [H, d_v, d_latent]; out [n, H, d_v] float32
 *   (the float32 accumulator is kept, not rounded to dtype). */
mla_status mla_out_proj(const mla_dims* dims, const void* out_latent, const void* w_uv, int64_t n,
                        void* out, void* stream);

/* ---- The front of the layer: projections from the hidden state h ---------
 * "AI decoupled RoPE MLA" (operatorworld.com), recap: the latent is the
 * down-projection c_t = W^DKV h_t; decoupled-RoPE section: the position
 * channel k^R_t = W^KR h_t is shared by the heads and is the only part
 * rotated.  "Detailed Illustration of the Problem" (notion.site), Step 1: the
 * query goes through a compressed latent c^Q = W^DQ h and is projected up
 * from it; Step 4: with no rotation between them, W^UK folds into the query
 * weight, W^{Q'} = (W^UQ)^T W^UK.  Here both query channels come from the
 * query latent: q^C_i = W_UQ,i c^Q, q^R_i = W_QR,i c^Q.
 * Weights are stored [out, in]: W_DKV [d_latent, d_model], W_KR [d_rope,
 * d_model], W_DQ [d_qlat, d_model], W_UQ [H, d_head, d_qlat], W_QR [H, d_rope,
 * d_qlat], the folded W_fold [H, d_latent, d_qlat] = W_UK,i^T W_UQ,i.
 * bf16 only (dims->dtype and work_dtype), d_model and d_qlat multiples of 32,
 * h and the weights 16-byte aligned; otherwise MLA_ERR_UNSUPPORTED or
 * MLA_ERR_INVALID_ARG and nothing is launched.  Accumulation is float32 over
 * K splits summed in a fixed order (bitwise repeatable); RoPE angles are
 * float64, as in mla_rope_apply.  The workspace holds float32 partial sums
 * and the bf16 query latent; it is the caller's, and calls on one stream may
 * share it. */

/* Bytes of workspace the front calls need for n tokens (d_qlat = 0 for
 * mla_kv_project alone); 0 when the arguments are rejected. */
size_t mla_front_workspace_size(const mla_dims* dims, int64_t n, int32_t d_model, int32_t d_qlat);

/* mla_kv_project -- the cache side of the front, fused with the cache write:
 *   c = W_DKV h[j],  k^R = W_KR h[j],  cache row of (kv_seq[j], kv_pos[j]) =
 *   [c | R_{kv_pos[j]} k^R] (bf16), for j < n.
 *   h [n, d_model]; kv_seq, kv_pos int32 [n] device.  Rows whose sequence,
 *   position or page id is negative or out of range are skipped (as in
 *   mla_rope_apply). */
mla_status mla_kv_project(const mla_dims* dims, const mla_paged_cache* cache, const void* h, int64_t n,
                          int32_t d_model, const void* w_dkv, const void* w_kr, const int32_t* kv_seq,
                          const int32_t* kv_pos, void* workspace, size_t workspace_bytes, void* stream);

/* mla_q_project -- the query side through the query latent:
 *   c^Q = W_DQ h[j] (rounded to bf16), q_nope[j, i, :] = W_UQ,i c^Q,
 *   q_lat[j, i, d_latent:] = R_{q_pos[j]} W_QR,i c^Q.
 *   h [n, d_model]; q_pos int32 [n] device; q_nope [n, H, d_head];
 *   q_lat [n, H, d_latent + d_rope] (only the tail is written; mla_absorb_q
 *   writes the head from q_nope). */
mla_status mla_q_project(const mla_dims* dims, const void* h, int64_t n, int32_t d_model, int32_t d_qlat,
                         const void* w_dq, const void* w_uq, const void* w_qr, const int32_t* q_pos, void* q_nope,
                         void* q_lat, void* workspace, size_t workspace_bytes, void* stream);

/* mla_q_project_folded -- the same query with W_UK folded in ahead of time:
 *   q_lat[j, i, :d_latent] = W_fold,i c^Q (the absorbed query q~),
 *   q_lat[j, i, d_latent:] = R_{q_pos[j]} W_QR,i c^Q.  No mla_absorb_q follows. */
mla_status mla_q_project_folded(const mla_dims* dims, const void* h, int64_t n, int32_t d_model, int32_t d_qlat,
                                const void* w_dq, const void* w_fold, const void* w_qr, const int32_t* q_pos,
                                void* q_lat, void* workspace, size_t workspace_bytes, void* stream);

/* mla_fold_q_weights -- W_fold,i = W_UK,i^T W_UQ,i ([H, d_latent, d_qlat],
 * float32 sums rounded once to bf16), once per weight set. */
mla_status mla_fold_q_weights(const mla_dims* dims, int32_t d_qlat, const void* w_uq, const void* w_uk, void* w_fold,
                              void* stream);

/* Static text for a status code. */
const char* mla_status_string(mla_status status);

/* Thread-local description of the last failed call on this thread ("" if
 * none).  Valid until the next call on the same thread. */
const char* mla_last_error(void);

/* Split plan mla_decode would use: pages per split and the number of work
 * items (sequence, split) it launches.  For tests and benchmarks. */
mla_status mla_decode_plan(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host,
                           int32_t* split_pages, int64_t* n_items);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
