/*
 * mla.h -- C ABI of libmla: Multi-head Latent Attention (MLA) decoding over a
 * paged, compressed latent KV cache on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are the web pages this method is described on):
 *  - "Transformer升级之路：21、MLA好在哪里？（下）", section 双重投影 (the two-column
 *    table): at decode time MLA is an MQA whose key and value are the cached
 *    latent c itself; W_UK moves to the query side (q_lat = W_UK^T q_nope) and
 *    W_UV to the output side (o = W_UV o_lat), per head.  Section 总而言之: a
 *    shared low-dimensional RoPE key is concatenated to the key.
 *  - "DeepSeek-V3 解读：Multi-head Latent Attention", section 为什么需要解耦 RoPE:
 *    the per-head query part q_R and one shared key k_R carry the rotary
 *    position; only the latent c_KV and the rotated k_R are cached.  Section
 *    RoPE（旋转式位置编码）: consecutive pairs of dimensions are rotated by a
 *    position-dependent angle.
 *  - Tencent Cloud MLA article listing, FlashMLA snippet: decoding runs over a
 *    paged cache addressed by a block table with per-sequence cache lengths and
 *    returns (o, lse); splits of the key range are merged by log-sum-exp.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller (allocate them
 *    however you like); the library never frees them, never keeps them after
 *    the call returns, and never allocates device memory itself.
 *  - Tensors are dense, row-major, with the shapes given below.  Element types
 *    follow mla_dims.act_dtype ("act") and mla_dims.cache_dtype.  Every tensor
 *    and workspace pointer should be 16-byte aligned (any device allocator's
 *    default); mla_decode rejects unaligned q_abs / cache_pool / o_latent /
 *    workspace with MLA_ERR_INVALID_ARG where its tuned kernel applies, the
 *    other calls fall back to their generic kernels.
 *  - Each call validates its arguments on the host first.  On any invalid
 *    argument it returns an error status and launches nothing (outputs are left
 *    untouched).  Otherwise it enqueues its kernels asynchronously on `stream`
 *    (a hipStream_t; NULL = the default stream) and returns MLA_OK, or
 *    MLA_ERR_LAUNCH if the runtime rejected a launch.  Faults inside a kernel
 *    surface at the caller's next synchronisation.  No call synchronises.
 *  - Integer index arrays (positions, sequence ids, block tables, lengths) are
 *    int32 device arrays; the host cannot read them without synchronising, so
 *    their contents are checked by the kernels: a block-table entry < 0 or
 *    >= n_pool_blocks (the pool size every call that reads or writes the pool
 *    takes) is padding and is never dereferenced, and a token whose position
 *    falls outside its sequence's table is skipped.  What padding means for
 *    each call is stated with it.
 *  - No call keeps mutable global state; concurrent calls on different streams
 *    are safe as long as their output/workspace buffers do not overlap.
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
  MLA_ERR_INVALID_ARG = 1,   /* NULL pointer, non-positive size, bad dims      */
  MLA_ERR_UNSUPPORTED = 2,   /* valid but unsupported dtype / dims combination */
  MLA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required     */
  MLA_ERR_LAUNCH = 4         /* the HIP runtime rejected a kernel launch       */
} mla_status;

typedef enum {
  MLA_F32 = 0,               /* IEEE binary32                                  */
  MLA_BF16 = 1,              /* bfloat16                                       */
  MLA_FP8_E4M3 = 2           /* OCP E4M3FN (cache only)                        */
} mla_dtype;

typedef void* mla_stream_t;  /* a hipStream_t */

/*
 * Problem dimensions, shared by every call.
 *   n_heads       query heads H
 *   d_c           latent width (also the value width of the absorbed form)
 *   d_rope        decoupled RoPE width d_R (even)
 *   d_nope        per-head NoPE query/key width (contracted with W_UK)
 *   d_v           per-head output width (rows of W_UV)
 *   block_size    tokens per cache block (the paging unit)
 *   softmax_scale scale applied to q.k before the softmax (1/sqrt(d_nope + d_rope))
 *   rope_base     RoPE base: pair i of a vector at position p turns by
 *                 p * rope_base^(-2i/d_rope) radians.  The angle is formed in
 *                 float64, its cos/sin are rounded to float32, and the rotated
 *                 pair (x cos - y sin, x sin + y cos) is formed in float64 and
 *                 rounded to the storage type.
 *   act_dtype     dtype of q_nope, q_rope, c_kv, k_rope, W_UK, W_UV, q_abs,
 *                 o_latent and out: MLA_F32 or MLA_BF16
 *   cache_dtype   MLA_F32 (needs act F32), MLA_BF16 (needs act BF16) or
 *                 MLA_FP8_E4M3 (needs act BF16)
 *
 * Cache pool layout: n_pool_blocks blocks of block_bytes each (see
 * mla_cache_block_bytes), block b starting at byte b * block_bytes.
 *   F32 / BF16 cache: a block is [block_size][d_c + d_rope] elements; row t of
 *     block holds [c_KV | RoPE(k_R)] of one token.
 *   FP8 cache: a block is [block_size][d_c] E4M3FN codes, then [block_size]
 *     float32 scales, then [block_size][d_rope] bf16 rotated k_R.  A token's
 *     latent is code * scale, scale = amax(|c_KV|)/448 (1 when amax is 0).
 */
typedef struct {
  int32_t n_heads, d_c, d_rope, d_nope, d_v, block_size;
  float softmax_scale;
  float rope_base;
  int32_t act_dtype;
  int32_t cache_dtype;
} mla_dims;

/* Bytes of one cache block for these dims (0 if the dims are invalid). */
size_t mla_cache_block_bytes(const mla_dims* dims);

/* Human-readable text for a status code (static storage, never NULL). */
const char* mla_status_string(mla_status status);

/*
 * mla_absorb_q -- absorb W_UK into the query and rotate the RoPE part
 * ("Transformer升级之路：21、MLA好在哪里？（下）", 双重投影, decoding column:
 * q = x W_q W_k^T; "DeepSeek-V3 解读", 为什么需要解耦 RoPE: RoPE on q_R).
 *   q_abs[t, s, 0:d_c]          = sum_n q_nope[t, s, n] * w_uk[s, n, :]
 *   q_abs[t, s, d_c:d_c+d_rope] = RoPE(q_rope[t, s, :], pos[t])
 * Shapes: q_nope [n_tok, H, d_nope], q_rope [n_tok, H, d_rope] (unrotated),
 * pos [n_tok] int32 (>= 0), w_uk [H, d_nope, d_c], q_abs [n_tok, H, d_c + d_rope]
 * (output, act dtype; accumulation in float32).  n_tok may be 0 (no launch).
 * With d_rope = 0 there is no RoPE part: q_rope and pos may be null and are
 * not read; with d_rope > 0 a null q_rope or pos is MLA_ERR_INVALID_ARG.
 */
mla_status mla_absorb_q(const mla_dims* dims, int32_t n_tok, const void* q_nope,
                        const void* q_rope, const int32_t* pos, const void* w_uk,
                        void* q_abs, mla_stream_t stream);

/*
 * mla_append_cache -- write new tokens into the paged latent cache
 * ("DeepSeek-V3 解读", 为什么需要解耦 RoPE: the cached variables are the latent
 * and the rotated shared key; FlashMLA snippet: block_table addressing).
 * Token n (sequence seq_id[n], position pos[n]) is stored in physical block
 * block_table[seq_id[n] * max_blocks + pos[n] / block_size], row
 * pos[n] % block_size, as [c_kv[n] | RoPE(k_rope[n], pos[n])] at the cache
 * dtype (FP8: per-token scale, RNE-saturated E4M3FN codes, bf16 rotated k_R).
 * Shapes: c_kv [n_tok, d_c], k_rope [n_tok, d_rope] (act dtype, unrotated),
 * seq_id/pos [n_tok] int32, block_table [n_seq, max_blocks] int32,
 * cache_pool: n_pool_blocks blocks.  A token whose sequence id is outside
 * [0, n_seq), whose position is negative or beyond the table, or whose block
 * entry is < 0 or >= n_pool_blocks is skipped.  Nothing else in the pool is
 * written.  Two tokens with the same (sequence, position) in one call race.
 */
mla_status mla_append_cache(const mla_dims* dims, int32_t n_tok, const void* c_kv,
                            const void* k_rope, const int32_t* seq_id, const int32_t* pos,
                            const int32_t* block_table, int32_t n_seq, int32_t max_blocks,
                            void* cache_pool, int64_t n_pool_blocks, mla_stream_t stream);

/*
 * Workspace bytes mla_decode/mla_combine need for this problem (host only, no
 * launch).  `max_blocks` is the block-table row length and bounds every
 * sequence length; `num_splits` as for mla_decode (0 = automatic).
 */
size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t n_seq, int32_t q_per_seq,
                                  int32_t max_blocks, int32_t num_splits);

/*
 * mla_project_down -- the down-projections of the hidden state fused with the
 * cache append ("DeepSeek-V3 解读", MLA：高层次的思路: the latent c^KV = W^DKV h,
 * and the queries are compressed to a latent the same way; 为什么需要解耦
 * RoPE: the shared RoPE key comes from h).  With W_down = [W_DQ; W_DKV; W_KR]
 * stored [d_cq + d_c + d_rope, d_model] (row-major, contraction-contiguous):
 *   [c_q[n] | c_kv[n] | k_rope[n]] = W_down h[n]   (fp32 accumulation, each rounded once to bf16)
 * c_q [n_tok, d_cq] is written (the query latent, for mla_absorb_from_latent;
 * d_cq = 0 means no query latent, c_q may be null); [c_kv | k_rope] is then
 * appended exactly as mla_append_cache does (same arguments and skipping
 * rules), so the call equals projecting and appending.  h [n_tok, d_model]
 * bf16.  workspace: at least mla_project_down_workspace_bytes, 16-byte
 * aligned (split-K partials and the projected rows).  Supported: bf16
 * activations, d_model a multiple of 16, d_cq + d_c + d_rope a multiple of 8
 * (else MLA_ERR_UNSUPPORTED).  n_tok may be 0 (no launch).
 */
size_t mla_project_down_workspace_bytes(const mla_dims* dims, int32_t n_tok, int32_t d_model,
                                        int32_t d_cq);
mla_status mla_project_down(const mla_dims* dims, int32_t n_tok, int32_t d_model, int32_t d_cq,
                            const void* h, const void* w_down, const int32_t* seq_id,
                            const int32_t* pos, const int32_t* block_table, int32_t n_seq,
                            int32_t max_blocks, void* cache_pool, int64_t n_pool_blocks, void* c_q,
                            void* workspace, size_t workspace_bytes, mla_stream_t stream);

/*
 * mla_absorb_from_latent -- the query up-projections fused with the
 * absorption ("DeepSeek-V3 解读", 为什么需要解耦 RoPE: the per-head query and
 * its RoPE part are restored from the query latent; W^UK can be absorbed into
 * the query side).  w_uq [H, d_nope + d_rope, d_cq] holds per head the W_UQ
 * rows, then the W_QR rows:
 *   [q_nope[t,s] | q_rope[t,s]] = w_uq[s] c_q[t]     (fp32 accumulation, rounded once to bf16)
 * then q_abs as mla_absorb_q with those q_nope, q_rope, pos and w_uk.  The two
 * factors are chained, not composed into one d_c x d_cq matrix per head
 * (which would triple the weight bytes at DeepSeek-V3 shape).  c_q [n_tok,
 * d_cq] bf16; q_abs [n_tok, H, d_c + d_rope].  workspace: at least
 * mla_absorb_from_latent_workspace_bytes, 16-byte aligned.  Supported: bf16,
 * d_cq a multiple of 16, H (d_nope + d_rope) a multiple of 8.  n_tok may be 0.
 */
size_t mla_absorb_from_latent_workspace_bytes(const mla_dims* dims, int32_t n_tok, int32_t d_cq);
mla_status mla_absorb_from_latent(const mla_dims* dims, int32_t n_tok, int32_t d_cq,
                                  const void* c_q, const void* w_uq, const int32_t* pos,
                                  const void* w_uk, void* q_abs, void* workspace,
                                  size_t workspace_bytes, mla_stream_t stream);

/*
 * mla_absorb_append -- mla_absorb_q and mla_append_cache in one launch (they
 * are independent; the short appends fill the CUs the absorb leaves idle).
 * Arguments as the two calls (n_q query tokens at q_pos, n_kv new tokens at
 * seq_id / pos); the results are identical to calling them in turn, which is
 * what happens where the tuned absorb does not apply.  Every argument is
 * checked before any launch.
 */
mla_status mla_absorb_append(const mla_dims* dims, int32_t n_q, const void* q_nope,
                             const void* q_rope, const int32_t* q_pos, const void* w_uk,
                             void* q_abs, int32_t n_kv, const void* c_kv, const void* k_rope,
                             const int32_t* seq_id, const int32_t* pos,
                             const int32_t* block_table, int32_t n_seq, int32_t max_blocks,
                             void* cache_pool, int64_t n_pool_blocks, mla_stream_t stream);

/*
 * mla_decode -- latent attention, the absorbed form ("Transformer升级之路：21、
 * MLA好在哪里？（下）", 双重投影, decoding column: every head attends with key
 * [c | k_R] and value c, shared by all heads).
 * For sequence b with L = cache_seqlens[b] cached tokens (the q_per_seq new
 * tokens included, already appended), query row j sits at position
 * p = L - q_per_seq + j and sees tokens 0..p:
 *   z_t  = softmax_scale * <q_abs[b, j, s, :], [c_t | kR_t]>
 *   lse  = ln sum_t exp(z_t)
 *   o_lat[b, j, s, :] = sum_t exp(z_t - lse) * c_t
 * Shapes: q_abs [n_seq, q_per_seq, H, d_c + d_rope] (act), cache_seqlens
 * [n_seq] int32 with q_per_seq <= L <= max_blocks * block_size,
 * block_table [n_seq, max_blocks], cache_pool: n_pool_blocks (> 0) blocks.
 * The tokens of a block-table entry < 0 or >= n_pool_blocks are left out of
 * the softmax (never read); a query row that sees no token gets o_lat = 0
 * and lse = -inf.  Outputs o_latent [n_seq, q_per_seq, H, d_c] (act) and
 * lse [n_seq, q_per_seq, H] (float32).  MLA_ERR_UNSUPPORTED when
 * max_blocks * block_size > 2^30, n_seq * q_per_seq * H >= 2^31 or
 * n_seq * ceil(max_blocks * block_size / 32) >= 2^31 (32-token key tiles).
 * The key range may be split over work-groups ("num_splits": 0 = automatic,
 * > 0 = that many work units); the partial results then go to `workspace`
 * (at least mla_decode_workspace_bytes) and mla_combine must follow with the
 * same arguments.  Whether mla_combine has work is reported by
 * mla_decode_needs_combine; calling it when it has none is a cheap no-op.
 */
mla_status mla_decode(const mla_dims* dims, int32_t n_seq, int32_t q_per_seq,
                      const void* q_abs, const void* cache_pool, int64_t n_pool_blocks,
                      const int32_t* block_table, int32_t max_blocks,
                      const int32_t* cache_seqlens, int32_t num_splits, void* workspace,
                      size_t workspace_bytes, void* o_latent, float* lse, mla_stream_t stream);

/*
 * mla_decode_noalloc -- mla_decode followed by mla_combine, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, results and errors as
 * mla_decode, without the workspace: the split partials go to a static
 * device array inside the library, MLA_DECODE_NOALLOC_MAX_BYTES long, one per
 * GPU the library runs on, held until the process ends.  A problem whose
 * workspace (mla_decode_workspace_bytes with the same arguments) exceeds that
 * size returns MLA_ERR_WORKSPACE before any launch.  Nothing is allocated
 * and nothing needs clearing (every partial is written before it is read).
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * partials: two calls that overlap in time on one GPU (different streams
 * without ordering, or threads) race.  The first call on a device looks up
 * the array's device address (hipGetSymbolAddress) with that device current.
 */
#define MLA_DECODE_NOALLOC_MAX_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_dims* dims, int32_t n_seq, int32_t q_per_seq,
                              const void* q_abs, const void* cache_pool, int64_t n_pool_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* cache_seqlens, int32_t num_splits, void* o_latent,
                              float* lse, mla_stream_t stream);

/* 1 if mla_decode with these arguments leaves partials for mla_combine, else 0. */
int32_t mla_decode_needs_combine(const mla_dims* dims, int32_t n_seq, int32_t q_per_seq,
                                 int32_t max_blocks, int32_t num_splits);

/*
 * mla_check_block_table -- host-side check of a block table before a decode or
 * a paged prefill (FlashMLA snippet: the block table maps a sequence's
 * token t to block block_table[b][t / block_size] of the pool).  The kernels
 * read an entry outside [0, n_pool_blocks) as padding (its tokens masked);
 * this check finds such entries instead, for callers that want them reported.
 * block_table [n_seq][max_blocks] and cache_seqlens [n_seq] are HOST int32
 * arrays, read only.  For every sequence b, the entries
 * 0 .. ceil(L_b / block_size) - 1 that its L_b = cache_seqlens[b] tokens use
 * must lie in [0, n_pool_blocks); entries past them are not read.  A length
 * outside [0, max_blocks * block_size] is an error too.  Returns MLA_OK, or
 * MLA_ERR_INVALID_ARG with *first_bad (if not NULL) set to the flat index
 * b * max_blocks + i of the first bad entry, or to -(b + 1) for a bad length
 * of sequence b, or to INT64_MIN for bad sizes or pointers.  Launches nothing.
 */
mla_status mla_check_block_table(const int32_t* block_table, int32_t n_seq, int32_t max_blocks,
                                 const int32_t* cache_seqlens, int32_t block_size,
                                 int64_t n_pool_blocks, int64_t* first_bad);

/*
 * mla_combine -- merge split partials by log-sum-exp (FlashMLA snippet: the
 * (o, lse) pair per split): lse = ln sum_k exp(lse_k),
 * o_lat = sum_k exp(lse_k - lse) o_k; a split that saw no token has
 * lse_k = -inf and weight 0.  Arguments as passed to mla_decode.
 */
mla_status mla_combine(const mla_dims* dims, int32_t n_seq, int32_t q_per_seq,
                       const int32_t* cache_seqlens, int32_t max_blocks, int32_t num_splits,
                       const void* workspace, size_t workspace_bytes, void* o_latent, float* lse,
                       mla_stream_t stream);

/*
 * mla_up_proj -- move W_UV back onto the output ("Transformer升级之路：21、
 * MLA好在哪里？（下）", 双重投影, decoding column: o = [o^(1) W_v^(1), ...]).
 *   out[t, s, v] = sum_c w_uv[s, v, c] * o_latent[t, s, c]
 * Shapes: o_latent [n_tok, H, d_c], w_uv [H, d_v, d_c], out [n_tok, H, d_v]
 * (act dtype; accumulation in float32).  n_tok may be 0 (no launch).
 */
mla_status mla_up_proj(const mla_dims* dims, int32_t n_tok, const void* o_latent,
                       const void* w_uv, void* out, mla_stream_t stream);

/*
 * mla_up_proj_gated -- the up-projection with an output gate (gated MLA: MLA
 * with an elementwise output gate on each head's attention output, named in
 * the reader comments of "Transformer升级之路：21、MLA好在哪里？（下）").
 *   out[t, s, v] = sigmoid(gate[t, s, v]) * sum_c w_uv[s, v, c] * o_latent[t, s, c]
 * gate [n_tok, H, d_v] holds the gate logits (act dtype; computed upstream
 * from the hidden state).  The product is formed in float32 (sigmoid(g) =
 * 1 / (1 + e^-g)) and rounded once to the act dtype.  Other arguments and the
 * error behaviour as mla_up_proj; a null gate with n_tok > 0 is
 * MLA_ERR_INVALID_ARG.
 */
mla_status mla_up_proj_gated(const mla_dims* dims, int32_t n_tok, const void* o_latent,
                             const void* w_uv, const void* gate, void* out, mla_stream_t stream);

/*
 * mla_combine_up_proj -- mla_combine followed by mla_up_proj (or
 * mla_up_proj_gated with a gate) on the rows of mla_decode, in one call:
 * the split partials are merged by log-sum-exp as in mla_combine and the
 * merged latent rows go through W_UV as in mla_up_proj ("Transformer升级之路：
 * 21、MLA好在哪里？（下）", 双重投影, decoding column), without the merged rows
 * making a round trip through memory.  Arguments: those of mla_combine for
 * the decode that left the workspace, then w_uv [H, d_v, d_c], gate
 * [n_seq * q_per_seq, H, d_v] or null, out [n_seq * q_per_seq, H, d_v].
 * o_latent is read for the rows mla_decode finished itself (a sequence that
 * lies inside one work unit, or has no token); with write_latent != 0 the
 * merged rows are written back to it as mla_combine writes them.  With
 * write_latent == 0 the caller gives up those rows: the one-kernel path leaves
 * them as mla_decode left them, and the two-launch path (taken where the
 * one-kernel path does not apply: no split, an unaligned buffer, or a shape
 * it does not support) writes the merged values; either way every other
 * output is the same.  lse is written for the merged rows as
 * mla_combine writes it.  The results are bit-identical to the two calls.
 * Errors as mla_combine and mla_up_proj, checked before any launch.
 */
mla_status mla_combine_up_proj(const mla_dims* dims, int32_t n_seq, int32_t q_per_seq,
                               const int32_t* cache_seqlens, int32_t max_blocks,
                               int32_t num_splits, const void* workspace,
                               size_t workspace_bytes, void* o_latent, int32_t write_latent,
                               const void* w_uv, const void* gate, void* out, float* lse,
                               mla_stream_t stream);

/*
 * mla_prefill -- causal attention over whole prompts in the MHA form
 * ("Transformer升级之路：21、MLA好在哪里？（下）", 双重投影, training/prefill
 * column: each head gets its own key k = [c W_k^(s) | k_R] and value
 * v = c W_v^(s); 总而言之: the shared RoPE key is concatenated; "DeepSeek-V3
 * 解读", 为什么需要解耦 RoPE: q_R and k_R are rotated).  Per head s and token i
 * of a sequence (position i, seeing tokens 0..i of the same sequence):
 *   key_t   = [W_UK[s] c_t | RoPE(k_rope_t, t)],  value_t = W_UV[s] c_t
 *   query_i = [q_nope[i,s] | RoPE(q_rope[i,s], i)]
 *   z_t = softmax_scale <query_i, key_t>,  out[i,s] = sum_t softmax(z)_t value_t,
 *   lse[i,s] = ln sum_t exp(z_t).
 * RoPE follows the rule of mla_dims.rope_base (the rotated pair formed in
 * float64 and rounded to float32; the rotated key is then stored in bf16, as a
 * bf16 cache holds it).  The decompression multiplies the bf16 latent by the
 * bf16 weights with float32 sums; the attention's operands -- the query, the
 * decompressed key and value, the rotated keys and the softmax weights -- are
 * fp16 (each bf16 input converts exactly, each computed operand is rounded to
 * nearest even) with float32 sums.  Decompressed keys and values must stay
 * inside fp16's range (|x| < 65504).  The parity tests compare with the form
 * above computed exactly.
 * Sequences are packed: cu_seqlens [n_seq + 1] (device int32, trusted: 0 =
 * cu[0] <= cu[1] <= ... <= cu[n_seq] = total_tokens, every length <= max_seqlen,
 * a host value); q_nope [T, H, d_nope], q_rope [T, H, d_rope] (unrotated),
 * c_kv [T, d_c], k_rope [T, d_rope] (unrotated), w_uk [H, d_nope, d_c],
 * w_uv [H, d_v, d_c], all bf16; out [T, H, d_v] (bf16) and lse [T, H] (float32)
 * are written.  gate: null, or [T, H, d_v] bf16 output-gate logits (gated
 * MLA, as mla_up_proj_gated): out = sigmoid(gate) * o in float32 before the
 * rounding; lse is not gated.  workspace: at least mla_prefill_workspace_bytes (the
 * decompressed keys and values and the rotated parts live there), 16-byte
 * aligned.  Supported: bf16, d_c 512, d_nope 128, d_rope 64, d_v 128 (else
 * MLA_ERR_UNSUPPORTED).  T = 0 launches nothing.
 */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t total_tokens);
mla_status mla_prefill(const mla_dims* dims, int32_t n_seq, const int32_t* cu_seqlens,
                       int32_t total_tokens, int32_t max_seqlen, const void* q_nope,
                       const void* q_rope, const void* c_kv, const void* k_rope,
                       const void* w_uk, const void* w_uv, const void* gate, void* workspace,
                       size_t workspace_bytes, void* out, float* lse, mla_stream_t stream);

/*
 * mla_prefill_paged -- chunked prefill: the MHA form of mla_prefill, with the
 * keys and values decompressed from the paged latent cache, so a chunk of new
 * tokens attends to the prompt's cached prefix as well as to itself
 * (positions and visibility as in mla_decode: "Transformer升级之路：21、
 * MLA好在哪里？（下）", 双重投影, training/prefill column, for the form; the
 * FlashMLA snippet of the Tencent Cloud article for the paged cache).
 * Sequence b has Lq_b = cu_q[b+1] - cu_q[b] query tokens (its newest ones,
 * already appended with mla_append_cache) and Lk_b = cu_k[b+1] - cu_k[b]
 * cached tokens, Lq_b <= Lk_b.  Query j sits at position Lk_b - Lq_b + j and
 * sees cached tokens 0..Lk_b - Lq_b + j:
 *   key_t   = [W_UK[s] c_t | k_R'_t],  value_t = W_UV[s] c_t   (c_t, k_R'_t: cache row of token t)
 *   query_j = [q_nope[j,s] | RoPE(q_rope[j,s], Lk_b - Lq_b + j)]
 * cu_q, cu_k [n_seq + 1]: device int32, trusted (0 = cu[0] <= ... <=
 * cu[n_seq] = total_q / total_k, Lq_b <= Lk_b, every Lq_b <= max_q, a host
 * value).  cache_pool (n_pool_blocks > 0 blocks) and block_table [n_seq,
 * max_blocks] as mla_decode; the blocks covering tokens 0..Lk_b - 1 should
 * be valid: an entry there that is < 0 or >= n_pool_blocks is never read and
 * its tokens enter as a zero latent and key.  q_nope
 * [total_q, H, d_nope], q_rope [total_q, H, d_rope] (unrotated), w_uk, w_uv,
 * gate (null or [total_q, H, d_v]), out [total_q, H, d_v] and lse [total_q, H]
 * as mla_prefill.  workspace: at least mla_prefill_paged_workspace_bytes,
 * 16-byte aligned.  Supported: the dims of mla_prefill with a bf16 or fp8
 * cache (else MLA_ERR_UNSUPPORTED); an fp8 latent enters the decompression as
 * its codes (exact) and the token's scale multiplies the float32 sums
 * (W (code * scale) = scale * (W code)), before k_C and v are rounded to
 * bf16.  total_q = 0 launches nothing.
 */
size_t mla_prefill_paged_workspace_bytes(const mla_dims* dims, int32_t total_q, int32_t total_k);
mla_status mla_prefill_paged(const mla_dims* dims, int32_t n_seq, const int32_t* cu_q,
                             int32_t total_q, int32_t max_q, const int32_t* cu_k, int32_t total_k,
                             const void* q_nope, const void* q_rope, const void* cache_pool,
                             int64_t n_pool_blocks, const int32_t* block_table, int32_t max_blocks,
                             const void* w_uk, const void* w_uv, const void* gate, void* workspace,
                             size_t workspace_bytes, void* out, float* lse, mla_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
