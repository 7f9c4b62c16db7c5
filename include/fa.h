/*
 * fa.h - C ABI of the MI355X (gfx950) exact tiled attention library (libfa.so).
 *
 * What the library computes
 * -------------------------
 * Exact attention forward, O = softmax(S) V with S = scale * Q K^T plus the
 * optional score transforms below, evaluated tile by tile so the Nq x Nk score
 * matrix never reaches device memory: tiles of Q, K and V are staged on chip,
 * a running row maximum and running row sum (online softmax) renormalise the
 * partial output after each key tile, and the per-row log-sum-exp is emitted
 * ("IO感知技术革命: FlashAttention如何重塑大模型训练的经济学", the sections on
 * block-wise tiling and on the online softmax; "FlashAttention及变种改进",
 * section 二.1 for the standard attention it reproduces).
 *
 * Score transforms and masks, applied in this order (the flash-attn v2.0-v2.7
 * update article, v2.1 to v2.6 entries):
 *   1. s = scale * q.k
 *   2. softcap > 0:        s = softcap * tanh(s / softcap)                 (v2.6)
 *   3. alibi_slopes != 0:  s = s - slope[h] * |i + (Nk - Nq) - j|          (v2.4)
 *   4. mask (bottom-right aligned, off = Nk - Nq; v2.1 and v2.3):
 *        causal:            keep j <= i + off
 *        window_left  >= 0: keep j >= i + off - window_left
 *        window_right >= 0: keep j <= i + off + window_right
 *      (-1 leaves that side unbounded; causal acts as window_right = 0.)
 * LSE[i] = ln(sum over kept keys of exp(s_ij)). A row with no kept key gets
 * O = 0 and LSE = -inf.
 *
 * Memory layout (all row-major, contiguous, head_dim innermost):
 *   q                [batch, seqlen_q, heads, head_dim]      in_dtype
 *   k, v             [batch, seqlen_k, heads, head_dim]      in_dtype (fa_fwd)
 *   k_cache, v_cache [num_pages, page_size, heads, head_dim] in_dtype (fa_fwd_splitkv)
 *   block_table      [batch, max_pages_per_seq] int32; entry p of sequence b is the
 *                    physical page holding logical keys [p*page_size, (p+1)*page_size)
 *   o                [batch, seqlen_q, heads, head_dim]      o_dtype (FA_FP32 or FA_BF16)
 *   lse              [batch, heads, seqlen_q] float32, natural log; may be NULL
 *   o_part           [num_splits, batch, heads, seqlen_q, head_dim] float32
 *   lse_part         [num_splits, batch, heads, seqlen_q] float32
 *   alibi_slopes     [heads] float32, or NULL for no bias
 *
 * Ownership and execution: every pointer is a device pointer owned by the
 * caller. The library allocates no device memory and keeps no mutable global
 * state, except the static row-term buffer that fa_bwd_noalloc uses on each
 * GPU (see there); calls are enqueued on `stream` (a hipStream_t passed as
 * void*; NULL is the null stream) and return without synchronising, so results
 * are ready once the stream has reached the call. Calls on different streams
 * may run concurrently as long as they do not write the same buffers (and, for
 * fa_bwd_noalloc, do not overlap on one GPU).
 *
 * Errors: all arguments are validated on the host before any HIP call; on a
 * validation error nothing is launched and nothing is written. FA_ERR_HIP
 * means a launch was rejected by the runtime (hipGetLastError after launch).
 * Block-table contents are not checked: ids outside [0, num_pages) are
 * undefined behaviour (the table is maintained by the caller).
 *
 * Supported: in_dtype FA_BF16 or FA_FP32 (bf16 runs on bf16 MFMA with fp32
 * accumulation, fp32 on fp32 MFMA); head_dim 64 or 128; any positive sizes
 * with batch*heads*seqlen and every tensor's element count below 2^31 per
 * dimension product as stated in fa_status_string(FA_ERR_SHAPE).
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype { FA_FP32 = 0, FA_BF16 = 1 };

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* a size <= 0, too large, or inconsistent */
  FA_ERR_UNSUPPORTED = 3, /* head_dim or dtype not instantiated */
  FA_ERR_MASK = 4,        /* window < -1, or causal with window_right > 0 */
  FA_ERR_HIP = 5,         /* the HIP runtime rejected a launch */
  FA_ERR_VALUE = 6,       /* softmax_scale not finite and > 0, softcap < 0 or not finite */
  FA_ERR_SCRATCH = 7      /* fa_bwd_noalloc: the problem exceeds its static buffer */
};

/*
 * fa_fwd - exact attention forward over contiguous K/V.
 *
 * Follows the tiled IO-aware forward of the pages (see the header comment):
 * one workgroup per (query tile, head, batch) streams the key tiles its rows
 * can see, skipping tiles that the causal/window mask removes entirely (the
 * v2.3 entry: only the in-window part is computed).
 *
 * Writes o (all batch*seqlen_q*heads rows) and, if lse != NULL, lse.
 * Returns FA_OK or an fa_status error code.
 */
int fa_fwd(const void* q, const void* k, const void* v, int in_dtype,
           void* o, int o_dtype, float* lse,
           int batch, int heads, int seqlen_q, int seqlen_k, int head_dim,
           float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_fwd_splitkv - split-KV forward over a paged KV cache (the update article's
 * v2.2 entry for the split along the key sequence, v2.5 for the paged cache
 * addressed through block_table).
 *
 * The logical keys [0, seqlen_k) of each sequence are cut into num_splits
 * contiguous chunks of C keys, C = ceil(seqlen_k / num_splits) rounded up to a
 * multiple of page_size (so a chunk never cuts a page); trailing chunks may be
 * empty. For every split s the call writes the attention of the queries over
 * the keys of chunk s alone, with every mask and bias evaluated at the keys'
 * absolute positions: o_part[s] is that chunk's normalised output and
 * lse_part[s] its log-sum-exp (-inf, with o_part = 0, when no key of the chunk
 * is kept). fa_splitkv_combine merges the splits into the full result.
 *
 * Requires max_pages_per_seq * page_size >= seqlen_k. Only the first
 * ceil(seqlen_k / page_size) entries of each block_table row are read.
 */
int fa_fwd_splitkv(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                   const int* block_table, int max_pages_per_seq, int page_size,
                   float* o_part, float* lse_part, int num_splits,
                   int batch, int heads, int seqlen_q, int seqlen_k, int head_dim,
                   float softmax_scale, int causal, int window_left, int window_right,
                   const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_fwd_split - split-KV forward over contiguous K/V (the update article's
 * v2.2 entry: splitting the key sequence when the query tiles alone leave the
 * GPU idle, as with a short query set over a long key range).
 *
 * Same inputs as fa_fwd; bf16 only (FA_ERR_UNSUPPORTED for fp32). The keys
 * [0, seqlen_k) are cut into num_splits chunks of C keys, C =
 * ceil(seqlen_k / num_splits) rounded up to a multiple of 64 (the key tile;
 * fa_split_chunk_len(seqlen_k, num_splits, 64) returns it); trailing chunks may
 * be empty. Writes, per split s, o_part[s] [batch, heads, seqlen_q, head_dim]
 * (normalised) and lse_part[s] [batch, heads, seqlen_q] exactly as
 * fa_fwd_splitkv does; fa_splitkv_combine merges them. The caller owns the
 * partial buffers (num_splits * batch * heads * seqlen_q * (head_dim + 1)
 * floats); the library allocates nothing.
 */
int fa_fwd_split(const void* q, const void* k, const void* v, int in_dtype,
                 float* o_part, float* lse_part, int num_splits,
                 int batch, int heads, int seqlen_q, int seqlen_k, int head_dim,
                 float softmax_scale, int causal, int window_left, int window_right,
                 const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_fwd_splitkv_seqlens - fa_fwd_splitkv over a cache whose sequences hold
 * different numbers of keys (variable sequence lengths, named as a feature in
 * the closing section of "FlashAttention深度解析：从算法创新到产业变革的全面影响";
 * the paged cache and its block_table are the update article's v2.5 entry).
 *
 * cache_seqlens: device int32 [batch]; sequence b holds keys [0, cache_seqlens[b])
 * and is treated exactly as fa_fwd_splitkv treats a batch of one sequence with
 * seqlen_k = cache_seqlens[b]: its causal/window/ALiBi geometry is aligned to
 * its own last key (off = cache_seqlens[b] - seqlen_q), and its split chunks are
 * C_b = ceil(cache_seqlens[b] / num_splits) rounded up to a multiple of
 * page_size (a sequence with 0 keys gets o_part = 0 and lse_part = -inf in every
 * split). Rows of the cache past a sequence's length are never read.
 *
 * max_seqlen_k bounds the lengths and sizes the table: max_pages_per_seq *
 * page_size >= max_seqlen_k. The lengths live in device memory and are not
 * checked on the host; each is clamped to [0, max_seqlen_k] on the device.
 * Other arguments and layouts as fa_fwd_splitkv. NULL cache_seqlens is
 * FA_ERR_NULL.
 */
int fa_fwd_splitkv_seqlens(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                           const int* block_table, int max_pages_per_seq, int page_size,
                           const int* cache_seqlens, float* o_part, float* lse_part,
                           int num_splits, int batch, int heads, int seqlen_q, int max_seqlen_k,
                           int head_dim, float softmax_scale, int causal, int window_left,
                           int window_right, const float* alibi_slopes, float softcap,
                           void* stream);

/*
 * fa_fwd_splitkv_append - append each sequence's new keys to its paged cache,
 * then run the split pass over the cached keys followed by the new ones. (The key-value cache of "解密FlashAttention：如何让大语言模型推理
 * 速度翻倍": processed keys are kept and reused, and each step only adds its own
 * new tokens; page addressing as the update article's v2.5 entry.)
 *
 *   k_new, v_new   [batch, seqlen_q, heads, head_dim] in_dtype: one new key and
 *                  value per query row of this step
 *   cache_seqlens  device int32 [batch]: keys already cached per sequence, n_b
 *
 * Row i of k_new[b] / v_new[b] is written into logical key n_b + i of sequence
 * b (page block_table[b, t / page_size], row t % page_size). The partials are
 * those of fa_fwd_splitkv_seqlens with lengths n_b + seqlen_q: the queries
 * line up with the new keys (bottom-right rule), so under causal the last
 * query sees every key. In one launch (one query row, fp32, or page sizes
 * that are not a multiple of 16) the new keys are read from k_new / v_new,
 * never from the cache rows being written; with several bf16 rows and pages of
 * a multiple of 16 keys the append is a launch of its own and the pass that
 * follows it on the stream reads every key from the cache. Either way, when
 * the call has completed the cache holds the new keys.
 * cache_seqlens is not updated (the caller owns it and adds seqlen_q).
 *
 * Requires max_seqlen_k >= seqlen_q and max_pages_per_seq * page_size >=
 * max_seqlen_k; n_b is clamped on the device to [0, max_seqlen_k - seqlen_q],
 * so every write stays inside the mapped pages. Two sequences whose tables
 * share a page row written here race (the table is the caller's). Other
 * arguments as fa_fwd_splitkv; NULL cache_seqlens, k_new or v_new is
 * FA_ERR_NULL.
 */
int fa_fwd_splitkv_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, int in_dtype, const int* block_table,
                          int max_pages_per_seq, int page_size, const int* cache_seqlens,
                          float* o_part, float* lse_part, int num_splits, int batch, int heads,
                          int seqlen_q, int max_seqlen_k, int head_dim, float softmax_scale,
                          int causal, int window_left, int window_right,
                          const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_fwd_varlen - exact attention forward over a packed batch of sequences of
 * different lengths (variable sequence lengths: closing section of
 * "FlashAttention深度解析：从算法创新到产业变革的全面影响"). Each sequence is its
 * own attention problem, computed as fa_fwd computes one batch entry, with its
 * mask and ALiBi distances aligned to its own bottom-right corner
 * (off_b = nk_b - nq_b, the update article's v2.1 rule per sequence).
 *
 *   q, o           [total_q, heads, head_dim]   rows of sequence b: [cu_seqlens_q[b], cu_seqlens_q[b+1])
 *   k, v           [total_k, heads, head_dim]   rows of sequence b: [cu_seqlens_k[b], cu_seqlens_k[b+1])
 *   lse            [heads, total_q] float32, or NULL
 *   cu_seqlens_q/k device int32 [batch + 1], non-decreasing, starting at 0
 *
 * max_seqlen_q (>= 1) and max_seqlen_k (>= 0) bound the sequence lengths and
 * size the launch. The offsets live in device memory and are not checked on
 * the host; on the device they are clamped into [0, total] and each length to
 * its maximum, so every access stays inside the tensors, but rows of a
 * sequence beyond max_seqlen_q, and rows that no sequence owns, are not
 * written. A sequence with no key gets O = 0 and LSE = -inf. total_q = 0
 * returns FA_OK with nothing launched; q/o (k/v) may be NULL when total_q
 * (total_k) is 0. Dtypes, head_dim, masks and scores as fa_fwd.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, int in_dtype,
                  void* o, int o_dtype, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int batch, int heads, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int head_dim,
                  float softmax_scale, int causal, int window_left, int window_right,
                  const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_fwd_fp8 - fa_fwd for FP8 inputs (FlashAttention-3's FP8 forward: the
 * section on H100 and FP8 of "IO感知技术革命: FlashAttention如何重塑大模型训练的
 * 经济学"; FP8 forward support on the roadmap of "FlashAttention深度解析：从算法
 * 创新到产业变革的全面影响").
 *
 *   q, k, v   [batch, seqlen, heads, head_dim] E4M3 codes (OCP "E4M3FN": bias 7,
 *             no infinities, largest 448), one byte per element
 *   q_descale, k_descale, v_descale  per-tensor factors: element x stands for
 *             descale * e4m3(x); finite and > 0 (FA_ERR_VALUE otherwise)
 * Computes exactly what fa_fwd computes for the dequantised Q, K, V (same
 * masks, ALiBi, softcap, LSE and empty-row rules; o and lse as in fa_fwd).
 * Both products run on FP8 matrix instructions with fp32 accumulation. The
 * probabilities are scaled so that a row's largest is 2^8 and rounded to E4M3
 * (nearest even) for the output product, so O can differ from the exact
 * result by up to 2^-4 * sum_j P_ij |v_j| (plus fp32 rounding); O and LSE are
 * normalised by the unrounded row sum. head_dim 64 or 128 (FA_ERR_UNSUPPORTED
 * otherwise).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_descale, float k_descale,
               float v_descale, void* o, int o_dtype, float* lse, int batch, int heads,
               int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
               int window_left, int window_right, const float* alibi_slopes, float softcap,
               void* stream);

/*
 * fa_fwd_split_fp8 - fa_fwd_split for FP8 inputs: the FP8 forward of
 * fa_fwd_fp8 with its key range cut into splits (the update article's v2.2
 * split-KV entry applied to the FP8 forward on the deep-analysis page's
 * roadmap), for short query sets over long key ranges.
 *
 * Inputs, descales, score rules and the probability rounding as fa_fwd_fp8
 * (head_dim 64 or 128). The keys [0, seqlen_k) are cut into num_splits chunks
 * of C keys, C = ceil(seqlen_k / num_splits) rounded up to a multiple of 128
 * (the FP8 key tile; fa_split_chunk_len(seqlen_k, num_splits, 128) returns it);
 * trailing chunks may be empty. Writes, per split s, o_part[s] [batch, heads,
 * seqlen_q, head_dim] fp32 (normalised, v_descale applied) and lse_part[s]
 * [batch, heads, seqlen_q] as fa_fwd_split does; fa_splitkv_combine merges them.
 * Within a split the probabilities are rounded to E4M3 relative to the split's
 * own largest, so each partial carries fa_fwd_fp8's error bound over its own
 * keys. Errors as fa_fwd_fp8 and fa_fwd_split (num_splits in [1, 65536]).
 */
int fa_fwd_split_fp8(const void* q, const void* k, const void* v, float q_descale,
                     float k_descale, float v_descale, float* o_part, float* lse_part,
                     int num_splits, int batch, int heads, int seqlen_q, int seqlen_k,
                     int head_dim, float softmax_scale, int causal, int window_left,
                     int window_right, const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_fwd_splitkv_fp8 - fa_fwd_splitkv for one query row over a paged cache of
 * E4M3 codes (the FP8 forward support of the roadmap in "FlashAttention深度
 * 解析：从算法创新到产业变革的全面影响", applied to the stored keys and values
 * of the decode step; paging and splits as the update article's v2.2 and v2.5
 * entries). Half the bytes of a bf16 cache per key.
 *
 *   q                  [batch, 1, heads, head_dim] bf16
 *   k_cache, v_cache   [num_pages, page_size, heads, head_dim] E4M3 codes (as
 *                      fa_fwd_fp8), one byte per element
 *   k_descale, v_descale  per-tensor factors: code x stands for
 *                      descale * e4m3(x); finite and > 0 (FA_ERR_VALUE otherwise)
 *   cache_seqlens      device int32 [batch] keys per sequence, or NULL for
 *                      seqlen_k keys everywhere (as fa_fwd_splitkv_seqlens)
 * The partials are fa_fwd_splitkv's for the dequantised cache, computed in fp32
 * (the codes widen exactly; no rounding of the probabilities). seqlen_q must be
 * 1 and head_dim 64 or 128 (FA_ERR_UNSUPPORTED otherwise). Other arguments,
 * outputs and errors as fa_fwd_splitkv; merge with fa_splitkv_combine.
 */
int fa_fwd_splitkv_fp8(const void* q, const void* k_cache, const void* v_cache,
                       float k_descale, float v_descale, const int* block_table,
                       int max_pages_per_seq, int page_size, const int* cache_seqlens,
                       float* o_part, float* lse_part, int num_splits, int batch, int heads,
                       int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
                       int window_left, int window_right, const float* alibi_slopes,
                       float softcap, void* stream);

/*
 * fa_fwd_paged_fp8 - the FP8 forward of fa_fwd_split_fp8 over a paged cache:
 * E4M3 queries (any number of rows, e.g. a chunk of a prompt) against keys and
 * values stored as E4M3 codes in pages (the FP8 forward support on the
 * roadmap of "FlashAttention深度解析：从算法创新到产业变革的全面影响", with the
 * update article's v2.2 split and v2.5 paged-cache entries).
 *
 *   q                  [batch, seqlen_q, heads, head_dim] E4M3 codes
 *   k_cache, v_cache   [num_pages, page_size, heads, head_dim] E4M3 codes
 *   q_descale, k_descale, v_descale  per-tensor factors as fa_fwd_fp8
 *   block_table        device int32 [batch, max_pages_per_seq], as fa_fwd_splitkv
 *   cache_seqlens      device int32 [batch] keys per sequence (clamped to
 *                      seqlen_k), or NULL for seqlen_k keys everywhere
 * Any page_size (pages of a multiple of 32 keys are copied in slabs of the
 * 128-key tile; others row by row); head_dim 64 or 128. Splits as
 * fa_fwd_splitkv (chunks of whole pages, cut from each sequence's own key
 * count); scores, masks, biases and the rounding of the probabilities as
 * fa_fwd_split_fp8. Writes o_part [num_splits, batch, heads, seqlen_q, head_dim]
 * fp32 (normalised, v_descale applied) and lse_part [num_splits, batch, heads,
 * seqlen_q]; merge with fa_splitkv_combine. With equal key counts and split
 * chunks of a multiple of 128 keys the partials are fa_fwd_split_fp8's over
 * the gathered keys. Errors as fa_fwd_splitkv and fa_fwd_fp8.
 */
int fa_fwd_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float q_descale,
                     float k_descale, float v_descale, const int* block_table,
                     int max_pages_per_seq, int page_size, const int* cache_seqlens,
                     float* o_part, float* lse_part, int num_splits, int batch, int heads,
                     int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
                     int window_left, int window_right, const float* alibi_slopes, float softcap,
                     void* stream);

/*
 * fa_bwd - backward pass of fa_fwd: dQ, dK, dV from dO, with the attention
 * probabilities recomputed from the forward's LSE (no Nq x Nk matrix is
 * stored; "IO感知技术革命: FlashAttention如何重塑大模型训练的经济学", tiling and
 * O(N) memory, whose training figures rest on this pass). Every mask and
 * score transform of fa_fwd is differentiated through: with S the scaled,
 * capped, ALiBi-shifted and masked scores and P = exp(S - LSE),
 *   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO * O)_i,  dS = P * (dP - D),
 *   dZ = dS * (1 - tanh^2(scale q.k / softcap)) with a cap (dZ = dS without),
 *   dQ = scale dZ K,  dK = scale dZ^T Q.
 * Deterministic: no atomics; each gradient element is written by one
 * workgroup in a fixed order, so repeated calls give identical bits (the
 * update article's v2.4 entry lists a deterministic backward).
 *
 *   q, dout        [batch, seqlen_q, heads, head_dim] in_dtype (FA_BF16 only)
 *   k, v           [batch, seqlen_k, heads, head_dim] in_dtype
 *   o              [batch, seqlen_q, heads, head_dim] o_dtype: fa_fwd's output
 *   lse            [batch, heads, seqlen_q] float32: fa_fwd's log-sum-exp
 *   dq / dk, dv    shaped as q / k, v, in grad_dtype (FA_FP32 or FA_BF16)
 *   workspace      fa_bwd_workspace_bytes(batch, heads, seqlen_q) bytes of device
 *                  memory owned by the caller (2 floats per query row, rows
 *                  rounded up to a multiple of 32 per (batch, head)); overwritten
 * P and dZ are rounded to bf16 as matrix-core operands (accumulation in
 * fp32). Masks, scale, ALiBi and softcap must be those of the forward call.
 * Two launches run in order on `stream`: the per-row terms, then dK/dV and dQ
 * together. Errors as fa_fwd; fp32 inputs are FA_ERR_UNSUPPORTED.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv,
           int grad_dtype, float* workspace, int batch, int heads, int seqlen_q, int seqlen_k,
           int head_dim, float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, float softcap, void* stream);

/* Bytes of the workspace fa_bwd needs (-1 for a size <= 0). */
long long fa_bwd_workspace_bytes(int batch, int heads, int seqlen_q);

/* Size of fa_bwd_noalloc's static row-term buffer on each GPU. */
#define FA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

/*
 * fa_bwd_noalloc - fa_bwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving or training loops, and harnesses that
 * forbid hipMalloc. Same arguments, gradients, rounding, determinism and errors
 * as fa_bwd, without the workspace argument: the per-row terms live in a static
 * device buffer of FA_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on
 * every GPU it runs on until the process ends. The call allocates nothing.
 *
 * Limit: fa_bwd_workspace_bytes(batch, heads, seqlen_q) must not exceed
 * FA_NOALLOC_SCRATCH_BYTES (batch * heads * ceil(seqlen_q / 32) <= 65536), else
 * FA_ERR_SCRATCH with nothing launched.
 *
 * Sharing: every call on one GPU uses that GPU's one buffer, which keeps the
 * last call's contents (each call writes every row term it reads before
 * reading it, so no clearing is needed). Calls that overlap in time on one GPU
 * (on different streams, or from different host threads without ordering)
 * race on the buffer and may produce wrong gradients: order them, e.g. on one
 * stream. The first call on a device looks up the buffer's address there (a
 * HIP runtime query, after argument validation).
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv,
                   int grad_dtype, int batch, int heads, int seqlen_q, int seqlen_k,
                   int head_dim, float softmax_scale, int causal, int window_left,
                   int window_right, const float* alibi_slopes, float softcap, void* stream);

/*
 * fa_bwd_varlen - backward of fa_fwd_varlen: dQ, dK, dV of a packed batch of
 * sequences of different lengths (variable sequence lengths: closing section
 * of "FlashAttention深度解析：从算法创新到产业变革的全面影响"), each sequence
 * differentiated on its own as fa_bwd differentiates one batch entry, with its
 * mask and ALiBi distances aligned to its own bottom-right corner.
 *
 *   q, dout, o, dq [total_q, heads, head_dim]   rows of sequence b: [cu_seqlens_q[b], cu_seqlens_q[b+1])
 *   k, v, dk, dv   [total_k, heads, head_dim]   rows of sequence b: [cu_seqlens_k[b], cu_seqlens_k[b+1])
 *   lse            [heads, total_q] float32: fa_fwd_varlen's log-sum-exp
 *   cu_seqlens_q/k device int32 [batch + 1], non-decreasing, starting at 0
 *   workspace      fa_bwd_workspace_bytes(batch, heads, max_seqlen_q) bytes of
 *                  caller-owned device memory; overwritten
 *
 * The offsets are clamped on the device as in fa_fwd_varlen, so every access
 * stays inside the tensors; rows that no sequence owns, and rows of a
 * sequence beyond max_seqlen_q (max_seqlen_k), are not written. A key seen by
 * no query gets dK = dV = 0; a query with no key gets dQ = 0. With
 * total_q = total_k = 0 nothing is launched; q, dout, o, lse, dq (k, v, dk,
 * dv) may be NULL when total_q (total_k) is 0. Dtypes, rounding, determinism
 * and errors as fa_bwd; sizes as fa_fwd_varlen.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv,
                  int grad_dtype, float* workspace, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int batch, int heads, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int head_dim, float softmax_scale,
                  int causal, int window_left, int window_right, const float* alibi_slopes,
                  float softcap, void* stream);

/*
 * fa_splitkv_combine - the separate reduce step that merges split partials
 * (the update article's v2.2 entry): for every (b, h, i),
 *   L = ln(sum_s exp(lse_part[s])),  O = sum_s exp(lse_part[s] - L) * o_part[s].
 * Rows where every split is empty get O = 0 and L = -inf.
 *
 * Writes o [batch, seqlen_q, heads, head_dim] in o_dtype and, if lse != NULL,
 * lse [batch, heads, seqlen_q]. Any float alignment is accepted; with at most
 * head_dim / 4 splits, o_part on a 16-byte boundary and o on a 16-byte (fp32)
 * or 8-byte (bf16) boundary, rows are merged in 16-byte pieces (the faster form;
 * results differ from the other form only in rounding).
 */
int fa_splitkv_combine(const float* o_part, const float* lse_part, int num_splits,
                       int batch, int heads, int seqlen_q, int head_dim,
                       void* o, int o_dtype, float* lse, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_status_string(int status);

/* Split chunk length C used by fa_fwd_splitkv (page_size = the cache's page size),
 * fa_fwd_split (page_size = 64) or fa_fwd_split_fp8 (page_size = 128) for these
 * sizes, or -1 on bad sizes. */
int fa_split_chunk_len(int seqlen_k, int num_splits, int page_size);

/*
 * A split count for the split passes (fa_fwd_splitkv and its _seqlens, _append
 * and _fp8 forms, with page_size = the cache's page size and fp8_cache set for
 * an E4M3 cache; fa_fwd_split with page_size = 64): the smallest count whose
 * launch has at least two workgroups per compute unit (the split pass of the
 * update article's v2.2 entry, which exists to occupy a GPU that the batch and
 * heads alone leave idle; for a single query row the workgroups are counted
 * with the decode's wide head groups at head_dim 128), at most one split per
 * page (per 64 keys) and at most 64.
 * num_cus <= 0 asks the current HIP device for its compute-unit count. Returns
 * -1 on bad sizes (any size <= 0, head_dim not 64 or 128) or when no device
 * answers.
 */
int fa_num_splits(int batch, int heads, int seqlen_q, int seqlen_k, int head_dim, int page_size,
                  int fp8_cache, int num_cus);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
