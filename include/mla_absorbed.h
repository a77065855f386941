/*
 * mla_absorbed.h -- C ABI of the MI355X (gfx950) absorbed Multi-Head Latent
 * Attention decode library (libmla_absorbed.so).
 *
 * One decode step of one attention layer is four calls, all enqueued in order
 * on the caller's HIP stream:
 *
 *   mla_absorb_q      q_lat = q_nope . W_UK[h]              (per head)
 *   mla_decode_paged  split-K attention of [q_lat; q_rope] over the paged
 *                     latent cache, one normalised partial + lse per split
 *   mla_combine_lse   log-sum-exp merge of the splits -> o_lat, lse
 *   mla_up_v          out = o_lat . W_UV[h]                  (per head)
 *
 * mla_combine_up_v does the last two in one launch without writing o_lat;
 * mla_append_kv writes the new tokens' records into the cache beforehand;
 * mla_prefill_kv / mla_prefill_attention attend a whole prompt in the MLA form.
 *
 * What the method is, and where the pages say it:
 *  - Only one low-rank latent c_KV per token is cached, next to one decoupled
 *    RoPE key that every head shares (TPLA abstract, taxoreview pages for
 *    dblp:408/6122 and dblp:256/5536-3; TransMLA review page on pith.science,
 *    core_discovery).
 *  - The RoPE-free key up-projection W_UK is folded into the query ("absorb"),
 *    so attention runs in the latent space and the cache is never expanded
 *    (TransMLA abstracts on the taxoreview pages; TransMLA review page,
 *    key_machinery; the Eq. (26) interaction matrix in
 *    referee_report.major_comments[0]).
 *  - With the absorb, all heads read the same cache record: the MQA form of
 *    MLA (GQLA abstract, "GQA-to-MLA" Daily Papers listing).
 *  - The value up-projection W_UV is applied after attention (early TransMLA
 *    abstract on that listing).
 *  - Decode is bound by memory traffic (TPLA and CLOVER abstracts; the OI/CF
 *    abstract on the Daily Papers listing), and the softmax is computed online
 *    (BLASST abstract on that listing) so that splits of the token axis can be
 *    merged exactly by their log-sum-exp.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers, owned by the caller; the library
 *    never allocates, frees or synchronises, and keeps no per-call state.
 *    Every call only enqueues work on `stream` (0 = the null stream).
 *  - Tensors are dense row-major in the shapes given, bf16 as raw IEEE
 *    bfloat16, fp8 as OCP E4M3 (e4m3fn: bias 7, max 448, no infinities).
 *  - The shape structure is read on the host during the call only.
 *  - Errors detectable on the host (null pointers, bad sizes, misalignment,
 *    shapes without a kernel) return a status before anything is enqueued;
 *    a failed launch returns MLA_ERR_HIP.  Device-side faults surface at the
 *    caller's next synchronisation.  mla_last_error() gives a message for the
 *    calling thread's most recent failure.  Calls are thread-safe.
 *  - Queries: the q_len = S_q tokens of a step are the LAST S_q positions of
 *    each sequence; seq_lens[b] counts cached tokens including them.  Query s
 *    sees positions t <= seq_lens[b] - S_q + s (causal among themselves).  A
 *    query row that sees no position (seq_lens[b] == 0 for an idle batch slot)
 *    yields out = 0 and lse = -inf.
 *  - lse is the natural-log log-sum-exp of the scaled scores.
 */
#ifndef MLA_ABSORBED_H
#define MLA_ABSORBED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad stride or alignment  */
  MLA_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for              */
  MLA_ERR_HIP = 3          /* a HIP runtime call (device query or launch) failed         */
} mla_status_t;

typedef enum { MLA_BF16 = 0, MLA_FP8_E4M3 = 1, MLA_FP32 = 2, MLA_FP16 = 3 } mla_dtype_t;

/* Tokens per decode tile; the split plan below is counted in tiles. */
#define MLA_TILE_TOKENS 32

typedef struct {
  int32_t batch;              /* B >= 1                                          */
  int32_t num_heads;          /* H >= 1                                          */
  int32_t q_len;              /* S_q, 1..8                                       */
  int32_t d_nope;             /* query/key RoPE-free width; 128                  */
  int32_t d_rope;             /* decoupled RoPE width; 64                        */
  int32_t d_latent;           /* latent rank d_c; 512 or 256                     */
  int32_t d_v;                /* value width; 128                                */
  int32_t block_size;         /* tokens per cache page: 32 * 2^k (64)          */
  int32_t max_blocks_per_seq; /* row stride (entries) of block_table, >= 1       */
  float softmax_scale;        /* multiplies q.k, finite and > 0; usually 1/sqrt(d_nope + d_rope) */
  mla_dtype_t cache_dtype;    /* MLA_BF16 or MLA_FP8_E4M3                        */
  mla_dtype_t out_dtype;      /* MLA_BF16 or MLA_FP32 (dtype of `out`)           */
  mla_dtype_t partial_dtype;  /* MLA_FP32 or MLA_FP16 (dtype of `o_part`)        */
} mla_shape_t;

/*
 * mla_absorb_q -- fold W_UK into the query.
 *   q_lat[b,s,h,:] = q_nope[b,s,h,:] . W_UK[h]        (fp32 accumulation, bf16 RNE result)
 *   q_nope  bf16 [B, S_q, H, d_nope]
 *   w_uk    bf16 [H, d_nope, d_latent]     (k_nope of head h = W_UK[h] . c)
 *   q_lat   bf16 [B, S_q, H, d_latent]     (written)
 * Pointers 16-byte aligned.
 */
mla_status_t mla_absorb_q(const mla_shape_t* shape, const void* q_nope, const void* w_uk, void* q_lat,
                          hipStream_t stream);

/*
 * mla_decode_num_parts -- host query: how many partial slots mla_decode_paged
 * should use on the current device (o_part / lse_part are sized by it).  The
 * value is max(B, the number of decode work-groups that fill the device's
 * compute units once).  Any value >= B may be passed to the decode and
 * combine calls instead; it only changes how the token axis is split.
 */
mla_status_t mla_decode_num_parts(const mla_shape_t* shape, int32_t* num_parts);

/*
 * mla_decode_paged -- split-K attention over the paged latent cache.
 *
 * Cache: page p, slot j (0 <= j < block_size) holds one token's record.
 *   latent  of that token at  (const char*)c_kv   + p*block_stride + j*token_stride
 *   RoPE key of that token at (const char*)k_rope + p*block_stride + j*token_stride
 *   element type: bf16 (MLA_BF16) or e4m3 (MLA_FP8_E4M3), d_latent resp. d_rope values.
 * The two parts must share the record: 0 < k_rope - c_kv, the latent ends at
 * or before the RoPE key, and the RoPE key ends within token_stride.  The
 * native layout is the interleaved record [c_KV | k_rope] of 576 values
 * (k_rope = c_kv + d_latent elements, token_stride = 576 * elem,
 * block_stride = block_size * token_stride).  c_kv, k_rope, token_stride and
 * block_stride must be multiples of 16 bytes.
 * kv_scale (fp8 only, else NULL): fp32 [pages][block_size], the dequantisation
 *   scale of each token, applied to its whole record.
 * block_table int32 [B, max_blocks_per_seq]: logical block i of sequence b is
 *   page block_table[b][i]; only entries i < ceil(seq_lens[b] / block_size) are read.
 * seq_lens int32 [B]: tokens in each sequence (0 = idle slot, else >= S_q).
 *   Cache slots at positions >= seq_lens[b] are never used in a way that can
 *   change results (they may hold NaN).
 * q_lat bf16 [B, S_q, H, d_latent] (from mla_absorb_q), q_rope bf16 [B, S_q, H, d_rope].
 *
 * Split plan (so that callers and tests can reproduce it; R = S_q * H rows,
 * row r = s*H + h):
 *   n_b = ceil(L_b / MLA_TILE_TOKENS) tiles in sequence b (0 if idle)
 *   W   = the smallest W >= 1 with sum_b ceil(n_b / W) <= num_parts
 *   p_b = ceil(n_b / W) parts of sequence b, in slots s_b .. s_b + p_b - 1,
 *         s_b = sum_{b' < b} p_{b'} (sequence order)
 *   part j of sequence b (slot s_b + j) is the partial over positions
 *   [j*W, min((j+1)*W, n_b)) * MLA_TILE_TOKENS, clipped to L_b and to what
 *   each query may see.  A part never spans two sequences.
 * o_part   [num_parts, R, d_latent] in shape->partial_dtype: sum_t p_t c_t,
 *          normalised within the split (a convex combination of latent rows).
 *          MLA_FP16 (round to nearest even) halves the bytes written here and
 *          read back by mla_combine_lse; it needs |latent value| < 65504 (the
 *          scaled value for an e4m3 cache), else the row becomes +-inf/NaN.
 * lse_part fp32 [num_parts, R]: the split's log-sum-exp (-inf if it sees nothing)
 * Slots that no (sequence, part) pair maps to are left untouched.
 */
mla_status_t mla_decode_paged(const mla_shape_t* shape, const void* q_lat, const void* q_rope,
                              const void* c_kv, const void* k_rope, int64_t token_stride,
                              int64_t block_stride, const float* kv_scale, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t num_parts, void* o_part,
                              float* lse_part, hipStream_t stream);

/*
 * mla_combine_lse -- merge the splits written by mla_decode_paged (same
 * shape, including partial_dtype, num_parts and seq_lens):
 *   lse[b,r]   = log sum_k exp(lse_part[k,r])
 *   o_lat[b,r] = sum_k exp(lse_part[k,r] - lse[b,r]) o_part[k,r]
 * over sequence b's slots; splits with lse = -inf weigh nothing; a row with
 * no visible position gets o_lat = 0 and lse = -inf.
 *   o_lat fp32 [B, S_q, H, d_latent], lse fp32 [B, S_q, H] (written)
 */
mla_status_t mla_combine_lse(const mla_shape_t* shape, int32_t num_parts, const void* o_part,
                             const float* lse_part, const int32_t* seq_lens, float* o_lat, float* lse,
                             hipStream_t stream);

/*
 * mla_up_v -- value up-projection of the latent output.
 *   out[b,s,h,:] = o_lat[b,s,h,:] . W_UV[h]           (fp32 accumulation)
 *   o_lat fp32 [B, S_q, H, d_latent]
 *   w_uv  bf16 [H, d_latent, d_v]
 *   out   [B, S_q, H, d_v] in shape->out_dtype (bf16 RNE or fp32) (written)
 * For a latent-split shard (d_latent = 256 of a wider latent) the fp32 out
 * together with the lse from mla_combine_lse is that shard's result for an
 * external merge.
 */
mla_status_t mla_up_v(const mla_shape_t* shape, const float* o_lat, const void* w_uv, void* out,
                      hipStream_t stream);

/*
 * mla_combine_up_v -- mla_combine_lse and mla_up_v in one launch: the
 * log-sum-exp merge of the splits (online softmax state merged exactly, BLASST
 * abstract on the "GQA-to-MLA" Daily Papers listing) followed by the value
 * up-projection applied after attention (early TransMLA abstract on that
 * listing), with the merged latent row kept on chip:
 *   lse[b,s,h]   = log sum_k exp(lse_part[k,r])                  (as mla_combine_lse)
 *   out[b,s,h,:] = (sum_k exp(lse_part[k,r] - lse[b,s,h]) o_part[k,r]) . W_UV[h]
 * with r = s*H + h over sequence b's slots, fp32 merge and accumulation.
 * Arguments as for the two calls (same shape, num_parts and seq_lens as the
 * decode that wrote o_part / lse_part):
 *   w_uv bf16 [H, d_latent, d_v]; out [B, S_q, H, d_v] in shape->out_dtype,
 *   lse fp32 [B, S_q, H] (both written); o_part, w_uv, out 16-byte aligned.
 * A row with no visible position gets out = 0 and lse = -inf.
 * Kernels exist for d_latent 512 or 256 with d_v 64 or 128 (else
 * MLA_ERR_UNSUPPORTED: use the two calls).  The merge weighs the splits in
 * batches of a different size than mla_combine_lse, so the two paths agree
 * to rounding, not bit for bit; each is deterministic.
 */
mla_status_t mla_combine_up_v(const mla_shape_t* shape, int32_t num_parts, const void* o_part,
                              const float* lse_part, const int32_t* seq_lens, const void* w_uv, void* out,
                              float* lse, hipStream_t stream);

/*
 * mla_append_kv -- write the records of the S_q new tokens of every sequence
 * into the paged cache (the step before mla_decode_paged).
 *   y        = x[b,s,:] . W                     (fp32 accumulation)
 *   c_KV     = y[0 : d_latent]                  (the latent: x . W_DKV)
 *   k_rope   = RoPE_pos(y[d_latent : d_latent + d_rope])
 *   record   -> page block_table[b][pos / block_size], slot pos % block_size,
 *               pos = seq_lens[b] - S_q + s (the new tokens are the last S_q
 *               positions, the queries' convention); an idle slot (0) is skipped.
 * The latent is the down-projection W_DKV of Eq. (11) on the TransMLA review
 * page (referee_report.minor_comments); only it and one RoPE key shared by all
 * heads are cached (core_discovery on that page; TPLA abstract).
 *   x      bf16 [B, S_q, d_model]; d_model a multiple of 256 up to 65536
 *   w_dkv  bf16 [d_model, d_latent + d_rope]: [W_DKV | W_KR], latent columns first
 *   rope_base  RoPE base (> 1, e.g. 10000): pair (2i, 2i+1) of the d_rope
 *          values turns by pos * rope_base^(-2i/d_rope), counter-clockwise
 *   cache  as for mla_decode_paged (same c_kv, k_rope, strides, block_table,
 *          seq_lens); bf16 records are rounded to nearest even; for an e4m3
 *          cache the record is stored as e4m3 (nearest even) of v / scale with
 *          scale = max|v| / 448 over the record (1 if all zero) written to
 *          kv_scale[page][slot].
 *   workspace  device scratch of at least mla_append_kv_workspace_bytes, 16-byte
 *          aligned, owned by the caller; its contents are not needed afterwards.
 * Two kernels are enqueued (the product, then the records).  Only the new
 * tokens' slots (and their scales) are written.  x, w_dkv, c_kv, k_rope 16-byte
 * aligned.
 */
mla_status_t mla_append_kv_workspace_bytes(const mla_shape_t* shape, int32_t d_model, size_t* bytes);
mla_status_t mla_append_kv(const mla_shape_t* shape, int32_t d_model, const void* x, const void* w_dkv,
                           float rope_base, void* c_kv, void* k_rope, int64_t token_stride,
                           int64_t block_stride, float* kv_scale, const int32_t* block_table,
                           const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Size of the library's fixed scratch array used by mla_append_kv_noalloc. */
#define MLA_APPEND_NOALLOC_MAX_BYTES (8u << 20)

/*
 * mla_append_kv_noalloc -- mla_append_kv without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * checks and results as mla_append_kv; the split-K partial products go to a
 * device array inside the library of MLA_APPEND_NOALLOC_MAX_BYTES (8 MiB),
 * one per GPU, held from library load until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 *   Limit: mla_append_kv_workspace_bytes(shape, d_model), i.e.
 *   B * S_q * (d_model / 256) * (d_latent + d_rope) * 4 bytes, must not exceed
 *   MLA_APPEND_NOALLOC_MAX_BYTES, else MLA_ERR_UNSUPPORTED is returned before
 *   anything is enqueued (e.g. B * S_q up to 227 rows at d_model 4096, d_latent 512).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams, or threads without ordering) race on it and give
 *   undefined records.  Nothing in the array needs to start at zero: each call
 *   writes every partial product before reading it, so a later call never
 *   sees an earlier call's contents.
 * The first call on a device resolves the array's address on that device
 * (a host-side runtime lookup, no device work); a failure there returns
 * MLA_ERR_HIP.
 */
mla_status_t mla_append_kv_noalloc(const mla_shape_t* shape, int32_t d_model, const void* x, const void* w_dkv,
                                   float rope_base, void* c_kv, void* k_rope, int64_t token_stride,
                                   int64_t block_stride, float* kv_scale, const int32_t* block_table,
                                   const int32_t* seq_lens, hipStream_t stream);

/*
 * Prefill in the MLA form.  A prompt is compute-bound, so it is attended with
 * keys and values reconstructed per head from the latent (the form the
 * prefill-decode separation of the TPLA abstract keeps for prefill), not in
 * the absorbed form the decode uses.  The prompts of the batch are padded to
 * prompt_len = P positions; sequence b uses its first seq_lens[b] (<= P).
 *
 * mla_prefill_kv -- per-head keys and values of every position t < seq_lens[b]:
 *   k_nope[b,h,t,:] = W_UK[h] . c[b,t]        (d_nope values)
 *   v[b,h,t,:]      = c[b,t] . W_UV[h]        (d_v values)
 *   fp32 accumulation, bf16 RNE results, written in the tile-native layout
 *   the attention reads: for sequence b, head h and tile j = t / 32
 *   (T = ceil(P / 32) tiles per sequence), 4096 bf16 at element
 *   ((b H + h) T + j) 4096, holding 16 granule rows g (elements 8g..8g+7)
 *   of 32 slots each, position t in slot (t % 32) ^ (4 (g & 1)).  Positions
 *   from seq_lens[b] to the end of their tile are written as zeros; later
 *   tiles are not written.  Each of k_nope and v holds
 *   mla_prefill_kv_elems(shape, P) bf16 values.
 *   ckr    bf16 [B, P, d_latent + d_rope]: the prompt's records [c_KV | k_rope]
 *   w_uk   bf16 [H, d_nope, d_latent], w_uv bf16 [H, d_latent, d_v]
 *   seq_lens int32 [B] (device), clamped to [0, P]
 *   workspace of at least mla_prefill_workspace_bytes (W_UV transposed).
 * mla_prefill_attention -- causal attention of each position s < seq_lens[b]
 * over positions t <= s, per head:
 *   z = scale (q_nope . k_nope + q_rope . k_rope),  out = softmax(z) . v
 *   q_nope bf16 [B, P, H, d_nope], q_rope bf16 [B, P, H, d_rope] (already rotated),
 *   k_rope = ckr[..., d_latent:] (shared by all heads), k_nope and v from
 *   mla_prefill_kv with the same seq_lens;
 *   out bf16 [B, P, H, d_v] and lse fp32 [B, P, H] for positions < seq_lens[b];
 *   the other positions are left untouched.
 * Kernels exist for d_nope = d_v = 128, d_rope = 64, d_latent 512 or 256,
 * and 1 <= P <= 2^20 with B P <= 2^24; shape->cache_dtype and
 * shape->out_dtype must be MLA_BF16 (MLA_ERR_UNSUPPORTED otherwise).  All
 * tensors 16-byte aligned.
 */
mla_status_t mla_prefill_workspace_bytes(const mla_shape_t* shape, size_t* bytes);
mla_status_t mla_prefill_kv_elems(const mla_shape_t* shape, int32_t prompt_len, int64_t* elems);
mla_status_t mla_prefill_kv(const mla_shape_t* shape, int32_t prompt_len, const void* ckr, const void* w_uk,
                            const void* w_uv, const int32_t* seq_lens, void* k_nope, void* v, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
mla_status_t mla_prefill_attention(const mla_shape_t* shape, int32_t prompt_len, const void* q_nope,
                                   const void* q_rope, const void* k_nope, const void* ckr, const void* v,
                                   const int32_t* seq_lens, void* out, float* lse, hipStream_t stream);

/*
 * TPLA latent split, run on one device.  TPLA splits the cached latent, and
 * each head's input dimension with it, over n devices; each shard attends on
 * its slice with the whole RoPE key, and an all-reduce adds the shards'
 * outputs.  An orthogonal Hadamard change of basis of the latent, applied
 * first, evens out the shards; full MLA is unchanged by it (TPLA abstract on
 * the taxoreview pages for dblp:408/6122 and dblp:256/5536-3).  Shard i
 * (of n) holds latent channels [i d_latent/n, (i+1) d_latent/n).  Its decode
 * is the ordinary one at d_latent / n: mla_absorb_q with its W_UK slice,
 * mla_decode_paged over the records viewed from latent channel i d_latent/n
 * (c_kv advanced by that many elements, k_rope and the strides unchanged),
 * and mla_combine_up_v with its W_UV slice into fp32; mla_tpla_reduce then
 * adds the n results.  With H = R / sqrt(d_latent), R the Sylvester-ordered
 * Hadamard matrix of order d_latent:
 *
 * mla_tpla_split_weights -- per-shard weight slices, in the changed basis if
 *   `hadamard` is non-zero (W_UK' = W_UK H, W_UV' = H^T W_UV), else as given:
 *   w_uk_shards[i][h] = W_UK'[h][:, S_i]   bf16 [n, H, d_nope, d_latent / n]
 *   w_uv_shards[i][h] = W_UV'[h][S_i, :]   bf16 [n, H, d_latent / n, d_v]
 *   fp32 transform, bf16 RNE results; n_shards 1, 2 or 4.
 * mla_tpla_rotate_cache -- in place, c' = c H for the d_latent latent values
 *   of every slot of pages 0 .. num_pages - 1 (slot j of page p at
 *   c_kv + p block_stride + j token_stride bytes); bf16 caches only.  This is
 *   the cache the same model would hold with W_DKV H as its down-projection.
 * mla_tpla_reduce -- out = sum over i < n of parts[i]:
 *   parts fp32 [n, B, S_q, H, d_v], out [B, S_q, H, d_v] in shape->out_dtype.
 * All tensors are device pointers, 16-byte aligned.
 */
mla_status_t mla_tpla_split_weights(const mla_shape_t* shape, int32_t n_shards, int32_t hadamard, const void* w_uk,
                                    const void* w_uv, void* w_uk_shards, void* w_uv_shards, hipStream_t stream);
mla_status_t mla_tpla_rotate_cache(const mla_shape_t* shape, void* c_kv, int64_t token_stride, int64_t block_stride,
                                   int32_t num_pages, hipStream_t stream);
mla_status_t mla_tpla_reduce(const mla_shape_t* shape, int32_t n_shards, const float* parts, void* out,
                             hipStream_t stream);

/*
 * GQLA's GQA decoding path.  GQLA weights expose two equivalent decoding
 * paths: MLA's absorbed MQA path over the latent (the calls above) and a GQA
 * path over a cache expanded per head group, which GQLA runs with two query
 * tokens per step (GQLA abstract on the "GQA-to-MLA" Daily Papers listing).
 * Heads h of a model with G groups belong to group h / (H / G).  The per-group
 * cache holds, for each stream s = b G + g, records
 *   [K_nope (d_nope) | V (d_v) | k_rope (d_rope)]   (the RoPE key is the token's
 *   one shared key), paged like the latent cache with its own block-table row.
 * The path is the latent decode run with a view shape: batch B G, num_heads
 * H / G, d_latent = d_nope + d_v (256 or 512), the same d_rope, q_len,
 * softmax_scale and block_size:
 *   1. mla_gqa_queries  -- q_cat[s, t, j] = [q_nope[b, t, g H/G + j] | 0]
 *      bf16 [B G, S_q, H/G, d_nope + d_v], and q_rope_g likewise
 *      bf16 [B G, S_q, H/G, d_rope];
 *   2. mla_decode_paged (view shape) with q_lat = q_cat, q_rope = q_rope_g,
 *      c_kv = the records, k_rope = c_kv + (d_nope + d_v) elements, the
 *      per-stream block table and seq_lens (each sequence's length repeated
 *      for its G streams); the scores are exactly q_nope . K_nope + q_rope . k_rope;
 *   3. mla_combine_lse (view shape) -> o_lat fp32 [B G, S_q, H/G, d_nope + d_v]
 *      and lse fp32 [B G, S_q, H/G]: the last d_v columns of o_lat are sum_t p_t V_t;
 *   4. mla_gqa_output -- out[b, t, h, :] = o_lat[s, t, j, d_nope:] in
 *      shape->out_dtype, lse[b, t, h] = lse_g[s, t, j] (fp32 [B, S_q, H]).
 * `shape` here is the model's (batch B, num_heads H, q_len, d_nope, d_rope,
 * d_v); `groups` must divide H and B G <= 1024.  All tensors are device
 * pointers; q_nope, q_rope, q_cat, q_rope_g, o_lat and out 16-byte aligned.
 */
mla_status_t mla_gqa_queries(const mla_shape_t* shape, int32_t groups, const void* q_nope, const void* q_rope,
                             void* q_cat, void* q_rope_g, hipStream_t stream);
mla_status_t mla_gqa_output(const mla_shape_t* shape, int32_t groups, const float* o_lat, const float* lse_g,
                            void* out, float* lse, hipStream_t stream);

/*
 * Calibration probes.  Not part of the decode: they measure the device's
 * achievable rates, the reference points that roofline fractions are also
 * reported against (nominal peaks: HBM 8 TB/s, bf16 MFMA 2.5 PFLOP/s).  Each
 * enqueues one kernel on `stream` and returns; the caller times it (HIP
 * events around the call).
 *
 * mla_probe_hbm_read -- streams `bytes` (a positive multiple of 16) of the
 *   device buffer `buf` (16-byte aligned) through registers: eight
 *   work-groups per CU, each streaming one contiguous chunk with sixteen
 *   non-temporal 16-byte loads in flight per lane.  Rate = bytes / time.  `sink` (device, 4 bytes) is written only in the unlikely
 *   case that the data XOR to a fixed value; it keeps the loads.
 * mla_probe_mfma -- `iters` (> 0) rounds of four independent
 *   v_mfma_f32_32x32x16_bf16 chains in two work-groups of four waves per CU;
 *   *flops receives the launch's flop count (host value, set before the
 *   launch).  `sink` (device, one float) receives work-group 0's sum.
 * mla_probe_tile_copy -- the copies of the bf16 decode for more than 64 query
 *   rows alone: the same split plan, grid, copy instructions and three-image
 *   LDS ring as mla_decode_paged, one barrier per tile, no products, over the
 *   cache described exactly as for mla_decode_paged (bf16 cache only,
 *   q_len * num_heads > 64, else MLA_ERR_UNSUPPORTED).  Rate = the launch's
 *   cache bytes / time.  `sink` as for mla_probe_hbm_read.
 */
mla_status_t mla_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
mla_status_t mla_probe_mfma(int32_t iters, float* sink, int64_t* flops, hipStream_t stream);
mla_status_t mla_probe_tile_copy(const mla_shape_t* shape, const void* c_kv, const void* k_rope, int64_t token_stride,
                                 int64_t block_stride, const int32_t* block_table, const int32_t* seq_lens,
                                 int32_t num_parts, uint32_t* sink, hipStream_t stream);

/* Static description of a status code. */
/*
 * Input validation.
 *
 * mla_validate_decode_inputs -- counts, on the device, the violations of the
 *   conditions mla_decode_paged (and the merges after it) assume of the
 *   per-sequence inputs it reads from device memory and cannot check on the
 *   host: for every sequence b, seq_lens[b] is 0 (an idle slot) or lies in
 *   [S_q, max_blocks_per_seq * block_size]; and each of its first
 *   ceil(seq_lens[b] / block_size) entries block_table[b][i] is a page id in
 *   [0, num_pages) (the paged record cache of mla_decode_paged: pages of
 *   block_size records, a row of physical page ids per sequence).  Entries
 *   past those are not read; a sequence whose length fails counts once and
 *   its entries are not examined.
 *   violations (device, one int32, 4-byte aligned) receives the count, 0 when
 *   every condition holds.  The call is enqueued on `stream` like the others
 *   and the caller reads the count after synchronizing.  One work-group: a
 *   check for debug runs and tests, not for the decode's hot path.
 *   Errors (MLA_ERR_INVALID_ARG): NULL pointers, num_pages <= 0, a misaligned
 *   violations pointer, or a shape the decode would reject.
 */
mla_status_t mla_validate_decode_inputs(const mla_shape_t* shape, const int32_t* block_table, const int32_t* seq_lens,
                                        int64_t num_pages, int32_t* violations, hipStream_t stream);

const char* mla_status_string(mla_status_t status);

/* Message for the calling thread's most recent non-OK status ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORBED_H */
