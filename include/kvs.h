/*
 * kvs.h - C ABI of libkvs: the KV-sparsity prefill-and-compress path on MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM" (blog post).
 *   [PAG] Ultralytics glossary, "PagedAttention".
 *
 * The path, per layer and batch of prompts:
 *   kvs_prefill_attn_lse  causal attention that also returns each row's log-sum-exp
 *   kvs_window_score      the observation-window score S per KV head, rebuilt from that LSE
 *   kvs_topk_select       the kept token indices per KV head
 *   kvs_compact_paged     copy of the kept K/V rows into 16-token blocks through block tables
 *   kvs_paged_decode      attention of one new token per sequence over the paged cache
 * with chunked-prefill variants (*_chunk) and a gather of cached blocks for prefix reuse,
 * 8-bit (E4M3) variants of the cache calls (*_fp8), decode-time scoring and eviction,
 * a host block allocator (free list, reference counts, copy-on-write) and the device
 * block copy that copy-on-write needs.
 *
 * Conventions shared by every call
 *   - Return value: KVS_OK (0) or a negative KVS_E_* code; kvs_last_error() gives a
 *     message for the calling thread.  Scalar arguments are checked on the host before
 *     anything is launched; a failed check launches nothing.
 *   - Pointers named *_dev / the tensors below are DEVICE pointers, owned by the caller
 *     (the library never allocates device memory and never frees a caller's buffer).
 *     Device integer arrays (cu_seqlens, keep_offsets, keep_idx, block tables, ctx_lens,
 *     slot offsets, copy pairs) are trusted: the host does not read them back.  Kernels
 *     skip any pool access whose block id lies outside [0, num_blocks).
 *   - bf16 tensors are passed as void* (IEEE bfloat16, 2 bytes); fp32 as float*; indices
 *     and tables as int32_t*.
 *   - Every device call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the host with the device.
 *   - Shapes: head_dim d in {64, 128}; hq % hkv == 0 and G = hq / hkv <= 16; query head h
 *     reads KV head h / G.  The block size is fixed at KVS_BLOCK_SIZE = 16 tokens.
 *   - Token-major ragged batches: prompt s owns tokens [cu_seqlens[s], cu_seqlens[s+1]) of
 *     Q [total][hq][d] and K, V [total][hkv][d]; indices inside a prompt are 0-based.
 *   - Thread safety: device calls may be made from any thread; an allocator object must
 *     not be used by two threads at once.
 */
#ifndef KVS_H_
#define KVS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVS_BLOCK_SIZE 16

enum {
  KVS_OK = 0,
  KVS_E_INVAL = -1,    /* bad shape or argument; nothing launched            */
  KVS_E_NOBLOCKS = -2, /* allocator: no free block                           */
  KVS_E_STATE = -3,    /* allocator: reference count misuse                  */
  KVS_E_HIP = -4       /* a HIP launch or runtime call failed                */
};

/* Message of the last failure on the calling thread ("" if none). */
const char* kvs_last_error(void);
/* Library version string. */
const char* kvs_version(void);

/*
 * kvs_prefill_attn_lse - causal attention over every prompt, with the row statistics
 * FlashAttention computes but does not return.
 *   [KVS] Key techniques, 2. "Attention modification": FlashAttention2 (first Fig. 7)
 *   walks Q in chunks over KV blocks, carrying O, P and the row maximum and dividing by
 *   l at the end; rowmax and l are computed but not returned, and the modification
 *   (second Fig. 7) outputs them at negligible cost.
 * Computes, for every prompt s, query head h and row j < n_s, with s_ji = scale*<q_j,k_i>
 * for i <= j:  m_j = max_i s_ji,  l_j = sum_i exp(s_ji - m_j),
 *              O_j = sum_i exp(s_ji - m_j) v_i / l_j,  lse_j = m_j + ln(l_j).
 * In:  q [total][hq][d], k, v [total][hkv][d] bf16; cu_seqlens [num_seqs+1] int32 (device).
 *      max_seqlen >= every n_s; total_tokens = cu_seqlens[num_seqs]; scale > 0 (1/sqrt(d)).
 * Out: o [total][hq][d] bf16 (round to nearest even); lse [hq][total_tokens] fp32 natural
 *      log; rowmax_opt, ell_opt [hq][total_tokens] fp32 (m_j and l_j; NULL to skip).  With
 *      lse NULL as well the call is the unmodified attention (first Fig. 7): nothing but o
 *      is written, which measures what returning the statistics costs.
 * Errors: KVS_E_INVAL on a bad shape or when max_seqlen * hkv * d * 2 exceeds 2^31 - 1 (one
 *         prompt's K or V rows are addressed with 32-bit byte offsets), KVS_E_HIP if the
 *         launch fails.
 */
int kvs_prefill_attn_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                         int num_seqs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
                         float scale, void* o, float* lse, float* rowmax_opt, float* ell_opt,
                         void* stream);

/*
 * kvs_window_score - the observation-window score, rebuilt from the saved LSE.
 *   [KVS] Key techniques, 2. "Attention modification": the last alpha prompt tokens are
 *   the window; a token's score is the sum of its softmax values over the window rows,
 *   p = exp(qk - rowmax)/l from the saved statistics, summed row-wise; the loop order is
 *   swapped to k.q so the sum stays in registers, and the causal mask plus the window
 *   bound limit the work to the window rows (second Fig. 7).
 * Computes, with a = min(alpha, n_s) and G = hq / hkv:
 *   S[g][i] = sum_{h: h/G = g} sum_{j = max(i, n_s - a)}^{n_s - 1} exp(scale*<q_hj, k_gi> - lse[h][j])
 * In:  q, k as in prefill (only the last a rows of q are read); lse [hq][total_tokens].
 * Out: scores [hkv][total_tokens] fp32 (indexed by the prompt's global token position).
 * Errors: KVS_E_INVAL if alpha < 1 or on a bad shape; KVS_E_HIP on launch failure.
 */
int kvs_window_score(const void* q, const void* k, const float* lse, const int32_t* cu_seqlens,
                     int num_seqs, int total_tokens, int max_seqlen, int alpha, int hq, int hkv,
                     int d, float scale, float* scores, void* stream);

/*
 * Chunked prefill and prefix reuse.  [PAG] "Sharing blocks between sequences": sharing
 * extends across requests by hashing full blocks (how vLLM caches prompts); [KVS]
 * Conclusion lists chunked prefill and prefix caching as not yet supported there.  A chunk
 * is the last m_s query rows of prompt s, whose keys K/V hold all n_s >= m_s prompt tokens
 * (a reused prefix first gathered back from the cache): query row r sits at prompt position
 * n_s - m_s + r and sees keys 0 .. n_s - m_s + r, so its O and LSE are those of the whole
 * prompt's prefill and nothing is carried between chunks.
 */

/*
 * kvs_prefill_attn_lse_chunk - kvs_prefill_attn_lse for chunks.
 * In:  q [total_q][hq][d] (rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1), k, v
 *      [total_k][hkv][d] (rows cu_seqlens_k[s] ..), bf16; both cu arrays [num_seqs+1] int32
 *      (device); max_q >= every m_s, max_k >= every n_s, and n_s >= m_s (trusted).
 * Out: o [total_q][hq][d]; lse, rowmax_opt, ell_opt [hq][total_q], as kvs_prefill_attn_lse.
 * Errors: as kvs_prefill_attn_lse (the size limit applies to max_k); KVS_E_INVAL also if
 *         cu_seqlens_k is NULL or max_k < max_q.
 */
int kvs_prefill_attn_lse_chunk(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int num_seqs, int total_q, int max_q, int max_k, int hq,
                               int hkv, int d, float scale, void* o, float* lse, float* rowmax_opt, float* ell_opt,
                               void* stream);

/*
 * kvs_window_score_chunk - kvs_window_score when q and lse hold only a prompt's last m_s rows
 * (the chunk of kvs_prefill_attn_lse_chunk).  The window, a = min(alpha, n_s) rows, must lie
 * inside the chunk (a <= m_s); window rows before the chunk would not be counted.
 * In:  q [total_q][hq][d], lse [hq][total_q]; k [total_k][hkv][d]; cu arrays as above.
 * Out: scores [hkv][total_k] fp32, indexed by the key's position in k.
 * Errors: as kvs_window_score; KVS_E_INVAL also if cu_seqlens_k is NULL.
 */
int kvs_window_score_chunk(const void* q, const void* k, const float* lse, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int num_seqs, int total_q, int total_k, int max_k, int alpha,
                           int hq, int hkv, int d, float scale, float* scores, void* stream);

/*
 * kvs_gather_paged - tokens 0 .. counts[s]-1 of sequence s read back through its block table
 * (layouts of kvs_compact_paged) into contiguous rows: k_dst[dst_start[s] + t][g][:] =
 * K of slot t, and likewise v_dst.  counts, dst_start [num_seqs] int32 (device); max_count
 * >= every count.  Used to put a reused prefix in front of a chunk's own K/V.
 * Errors: KVS_E_INVAL on a NULL tensor or bad shape; KVS_E_HIP on launch failure.
 */
int kvs_gather_paged(const void* k_pool, const void* v_pool, int num_blocks, const int32_t* block_tables,
                     int max_blocks, int num_seqs, int hkv, int d, const int32_t* counts, const int32_t* dst_start,
                     int max_count, void* k_dst, void* v_dst, void* stream);

/*
 * kvs_topk_select - the tokens each KV head keeps, per prompt.
 *   [KVS] Key techniques, 2. "Attention modification": in every layer and head the k_l
 *   highest-scoring tokens are kept and the rest dropped for the whole generation;
 *   [KVS] System model: pairs with a high score and greater proximity are kept.
 * Rule: with a = min(alpha, n_s): if k_budget >= n_s keep all n_s tokens; otherwise keep
 * the window {n_s-a .. n_s-1} plus the k_budget - a highest S among tokens i < n_s - a,
 * equal scores going to the lower index.  Indices are written in ascending order.
 * In:  scores [hkv][total_tokens] fp32, every value >= +0 and not NaN (as the window score
 *      produces); keep_offsets [num_seqs+1] int32 (device), keep_offsets[s] =
 *      sum_{s'<s} min(k_budget, n_s').
 * Out: keep_idx int32: prompt s, head g, rank t at keep_idx[hkv*keep_offsets[s] +
 *      g*k_eff_s + t], k_eff_s = min(k_budget, n_s); values are prompt-local indices.
 * Errors: KVS_E_INVAL if k_budget < alpha or alpha < 1; KVS_E_HIP on launch failure.
 */
int kvs_topk_select(const float* scores, const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                    int max_seqlen, int hkv, int alpha, int k_budget, const int32_t* keep_offsets,
                    int32_t* keep_idx, void* stream);

/*
 * kvs_compact_paged - write kept K/V rows into 16-token blocks through block tables.
 *   [PAG] "How paging works": the cache lives in fixed 16-token blocks anywhere in GPU
 *   memory; a per-request block table records their order, and token p goes to block
 *   table[p / 16], slot p % 16.  [KVS] Key techniques 1: the first layers keep a full
 *   cache (keep_idx == NULL writes every token).
 * For prompt s, head g, rank t < k_eff_s and p = dst_slot_offset[s] + t (0 if NULL):
 *   k_pool[table_s[p/16]][g][p%16][:] = k_src[cu_seqlens[s] + keep(g, t)][g][:]
 *   v_pool[table_s[p/16]][g][:][p%16] = v_src[cu_seqlens[s] + keep(g, t)][g][:]
 * keep(g, t) = keep_idx as laid out by kvs_topk_select, or t when keep_idx is NULL (then
 * k_eff_s = n_s and keep_offsets is ignored).  Slots outside [off, off + k_eff) are not
 * written, so a partially filled first block keeps its earlier slots.
 * Pool layouts: k_pool [num_blocks][hkv][16][d], v_pool [num_blocks][hkv][d][16] bf16.
 * block_tables [num_seqs][max_blocks] int32; max_keep >= every k_eff_s.
 * Errors: KVS_E_INVAL on a bad shape; KVS_E_HIP on launch failure.  Source and pools must
 * not overlap.
 */
int kvs_compact_paged(const void* k_src, const void* v_src, const int32_t* cu_seqlens,
                      int num_seqs, int hkv, int d, const int32_t* keep_idx,
                      const int32_t* keep_offsets, int max_keep, void* k_pool, void* v_pool,
                      int num_blocks, const int32_t* block_tables, int max_blocks,
                      const int32_t* dst_slot_offset, void* stream);

/*
 * kvs_topk_compact - kvs_topk_select followed by kvs_compact_paged of the kept rows, in one
 * launch (same results, bit for bit).
 *   [KVS] Key techniques, 2: the k_l highest-scoring tokens of every head are kept, the rest
 *   dropped; [PAG] "How paging works": the kept rows go to 16-token blocks through the
 *   sequence's block table.
 * Arguments as in the two calls: scores, cu_seqlens, max_seqlen, alpha, k_budget,
 * keep_offsets and keep_idx (written, the kvs_topk_select layout) as in kvs_topk_select;
 * k_src, v_src [total_tokens][hkv][d] bf16, pools, block tables and dst_slot_offset (NULL: 0)
 * as in kvs_compact_paged with max_keep = min(k_budget, max_seqlen).  One workgroup per
 * (prompt, KV head, block) repeats the selection and writes its block; when that would be
 * more than 256 workgroups (one per CU), or max_seqlen exceeds 16384, the two kernels run one
 * after the other instead (a small batch gains a launch and the compaction's metadata round
 * trips; a wide one would run the repeated selections one after another).
 * Errors: as the two calls; source and pools must not overlap.
 */
int kvs_topk_compact(const float* scores, const void* k_src, const void* v_src, const int32_t* cu_seqlens,
                     int num_seqs, int total_tokens, int max_seqlen, int hkv, int d, int alpha, int k_budget,
                     const int32_t* keep_offsets, int32_t* keep_idx, void* k_pool, void* v_pool, int num_blocks,
                     const int32_t* block_tables, int max_blocks, const int32_t* dst_slot_offset, void* stream);

/*
 * kvs_paged_decode - attention of one new token per sequence over its paged cache.
 *   [PAG] "How paging works": the attention kernel follows the request's block table to
 *   read keys and values block by block.  [KVS] Key techniques, 2: PagedAttention does
 *   the decode side of the same computation over the compressed cache.
 * For sequence b with L = ctx_lens[b] >= 1 (the new token included) and query head h:
 *   o[b][h] = sum_{t<L} softmax_t(scale*<q_bh, K_t>) V_t,  K_t/V_t read through table_b.
 * If new_k and new_v are not NULL, they are first stored at slot L-1 (block
 * table_b[(L-1)/16] must already be allocated) and the token attends to itself.
 * In:  q [batch][hq][d] bf16; new_k, new_v [batch][hkv][d] bf16 or NULL; pools and tables
 *      as in kvs_compact_paged; max_ctx >= every L.
 * Out: o [batch][hq][d] bf16; lse_opt [batch][hq] fp32 (natural log) or NULL.
 * Workspace: a device buffer of at least kvs_paged_decode_workspace_size(batch, hq, hkv, d,
 * max_ctx) bytes (may be NULL when that size is 0).  The context is split so that about
 * 2048 workgroups run; each split stores a (max, sum, output) partial there and a second
 * kernel merges them.  Two calls that share a workspace must not run concurrently.
 * Errors: KVS_E_INVAL on a bad shape or a short workspace; KVS_E_HIP on launch failure.
 */
size_t kvs_paged_decode_workspace_size(int batch, int hq, int hkv, int d, int max_ctx);
int kvs_paged_decode(const void* q, void* k_pool, void* v_pool, int num_blocks,
                     const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                     int batch, int max_ctx, int hq, int hkv, int d, float scale,
                     const void* new_k, const void* new_v, void* o, float* lse_opt,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-time scores and eviction in a compressed layer.
 *   [KVS] Key techniques 1 (step preparation): the layers after the third use a
 *   sliding-window strategy that replaces the KV entries with the lowest scores under a
 *   fixed budget; Key techniques 2, last paragraph: PagedAttention shares FlashAttention's
 *   goal of computing the score S.
 * Slot state, per sequence b, KV head g and slot t, row stride slot_stride (>= the
 * cache's capacity; slot t lives at block table_b[t/16], slot t%16):
 *   slot_scores [B][hkv][slot_stride] fp32  accumulated score, >= 0;
 *   slot_pos    [B][hkv][slot_stride] int32 prompt-local position of the token, -1 if empty.
 * A decode step of a full cache: kvs_decode_select_slot picks each head's slot for the new
 * token, then kvs_paged_decode_scored writes it there, attends and adds every live slot's
 * probability (summed over the group's query heads) to its score.
 */

/*
 * kvs_slot_init - slot state after compaction.  Slot t < k_eff_s of head g gets the kept
 * token keep(g, t) (layout of kvs_topk_select; t itself when keep_idx is NULL) with score
 * S[g][cu_seqlens[s] + keep(g, t)]; slots from k_eff_s to slot_stride-1 get score 0 and
 * position -1.  scores: [hkv][total_tokens] fp32 (kvs_window_score's output).
 * Errors: KVS_E_INVAL on a NULL tensor or bad shape; KVS_E_HIP on launch failure.
 */
int kvs_slot_init(const float* scores, const int32_t* keep_idx, const int32_t* keep_offsets,
                  const int32_t* cu_seqlens, int num_seqs, int total_tokens, int hkv, int slot_stride,
                  float* slot_scores, int32_t* slot_pos, void* stream);

/*
 * kvs_decode_select_slot - where each KV head writes the new token of sequence b, whose
 * cache holds n_filled[b] tokens before the step, at position new_pos[b].
 *   n_filled[b] < cap: slot n_filled[b] (append, every head);
 *   otherwise: the slot with the lowest score among tokens at positions
 *   < new_pos[b] - alpha (the alpha most recent tokens stay), ties to the lower position.
 * The chosen slot's score becomes 0 and its position new_pos[b] (slot_scores, slot_pos are
 * read and written).  Out: dst_slot [B][hkv] int32.
 * Errors: KVS_E_INVAL unless 0 <= alpha < cap <= slot_stride; KVS_E_HIP on launch failure.
 */
int kvs_decode_select_slot(float* slot_scores, int32_t* slot_pos, int slot_stride, const int32_t* n_filled,
                           int batch, int hkv, int cap, const int32_t* new_pos, int alpha, int32_t* dst_slot,
                           void* stream);

/*
 * kvs_paged_decode_scored - kvs_paged_decode whose new token goes to slot dst_slots[b][g]
 * of head g (NULL: slot L-1 for every head), and which adds, for every live slot t < L,
 * sum_{h in group(g)} exp(scale*<q_bh, K_t> - lse_bh) to slot_scores[b][g][t] after the
 * attention.  ctx_lens[b] = L counts the live slots after the write.  slot_stride >=
 * max_ctx.  Workspace: kvs_paged_decode_scored_workspace_size(...) bytes (never 0): the
 * split partials and the step's logits.  Calls sharing a workspace must not overlap.
 * Errors: as kvs_paged_decode; KVS_E_INVAL also for a NULL slot_scores or dst_slots given
 * without new_k/new_v.
 */
size_t kvs_paged_decode_scored_workspace_size(int batch, int hq, int hkv, int d, int max_ctx);
int kvs_paged_decode_scored(const void* q, void* k_pool, void* v_pool, int num_blocks, const int32_t* block_tables,
                            int max_blocks, const int32_t* ctx_lens, int batch, int max_ctx, int hq, int hkv, int d,
                            float scale, const void* new_k, const void* new_v, const int32_t* dst_slots,
                            float* slot_scores, int slot_stride, void* o, float* lse_opt, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * kvs_paged_decode_scored_select - kvs_paged_decode_scored followed by what
 *   kvs_decode_select_slot would do for the next step, in the same launches: the workgroup
 *   that adds a (sequence, KV head)'s probabilities to its slot scores then picks the slot of
 *   the next token, with n_filled = ctx_lens[b] (the live slots after this step) and position
 *   next_pos[b], under cap and alpha, and marks it (score 0, position next_pos[b]).  One
 *   decode step with eviction is then two launches instead of three; the first step's slot
 *   comes from kvs_decode_select_slot.  [KVS] Key techniques 1 (step preparation: the lowest
 *   score is replaced) and 2, last paragraph.
 * In: as kvs_paged_decode_scored, plus slot_pos [B][Hkv][slot_stride] int32 (read and
 *   written), cap, alpha, next_pos [B] int32.  Out: next_dst_slots [B][Hkv] int32.
 * Errors: as kvs_paged_decode_scored; KVS_E_INVAL also for a NULL slot_pos, next_pos or
 *   next_dst_slots, or unless 0 <= alpha < cap <= slot_stride and max_ctx <= cap.
 */
int kvs_paged_decode_scored_select(const void* q, void* k_pool, void* v_pool, int num_blocks,
                                   const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens, int batch,
                                   int max_ctx, int hq, int hkv, int d, float scale, const void* new_k,
                                   const void* new_v, const int32_t* dst_slots, float* slot_scores, int32_t* slot_pos,
                                   int slot_stride, int cap, int alpha, const int32_t* next_pos,
                                   int32_t* next_dst_slots, void* o, float* lse_opt, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * kvs_copy_blocks - device side of copy-on-write: whole-block copies in both pools.
 *   [PAG] "Sharing blocks between sequences": a sequence that must write a block still
 *   used by others copies it first.
 * src_dst_pairs [n_pairs][2] int32 (device): block src is copied to block dst (K and V,
 * every head).  Pairs must not chain (no dst is another pair's src).
 * Errors: KVS_E_INVAL on a bad shape; KVS_E_HIP on launch failure.
 */
int kvs_copy_blocks(void* k_pool, void* v_pool, int num_blocks, int hkv, int d,
                    const int32_t* src_dst_pairs, int n_pairs, void* stream);

/*
 * 8-bit cache.  [PAG] "Related techniques": an FP8 cache keeps the cached keys and values at
 * 8 bits, about half the memory of a 16-bit cache.  Format: OCP E4M3 (largest finite value
 * 448), one fp32 scale per cached row (token, KV head):
 *   scale = amax / 448,  code_c = E4M3(x_c * (448 / amax))  (round to nearest even,
 *   saturating), with amax = max_c |x_c| and each quotient and product rounded once in fp32;
 *   a row with amax < 2^-112 is stored as scale 0 and codes 0.  The value of a slot is
 *   code * scale.
 * Pools: k_pool [num_blocks][hkv][16][d] and v_pool [num_blocks][hkv][d][16] bytes (the same
 * element order as the 16-bit pools), k_scale and v_scale [num_blocks][hkv][16] fp32.
 */

/*
 * kvs_compact_paged_fp8 - kvs_compact_paged into an 8-bit cache: each written row is
 * quantized as above and its scale stored at the same (block, head, slot).  Arguments,
 * layout of the sources and tables, and errors as kvs_compact_paged.
 */
int kvs_compact_paged_fp8(const void* k_src, const void* v_src, const int32_t* cu_seqlens, int num_seqs, int hkv,
                          int d, const int32_t* keep_idx, const int32_t* keep_offsets, int max_keep, void* k_pool,
                          void* v_pool, float* k_scale, float* v_scale, int num_blocks, const int32_t* block_tables,
                          int max_blocks, const int32_t* dst_slot_offset, void* stream);

/*
 * kvs_paged_decode_fp8 - kvs_paged_decode over an 8-bit cache: K_t and V_t are the slots'
 * values code * scale, and new_k/new_v (bf16) are quantized into slot L-1 first.  The
 * query and the output stay bf16.  Workspace: kvs_paged_decode_workspace_size(...) bytes,
 * as for kvs_paged_decode.  Errors as kvs_paged_decode; KVS_E_INVAL also for a NULL scale
 * array.
 */
int kvs_paged_decode_fp8(const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale, int num_blocks,
                         const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens, int batch, int max_ctx,
                         int hq, int hkv, int d, float scale, const void* new_k, const void* new_v, void* o,
                         float* lse_opt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_paged_decode_scored_fp8 - kvs_paged_decode_scored over an 8-bit cache: the new token
 * is quantized into its chosen slot, the logits and scores use the slots' values code *
 * scale.  Workspace: kvs_paged_decode_scored_workspace_size(...) bytes.  Errors as
 * kvs_paged_decode_scored; KVS_E_INVAL also for a NULL scale array.
 */
int kvs_paged_decode_scored_fp8(const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                int num_blocks, const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                                int batch, int max_ctx, int hq, int hkv, int d, float scale, const void* new_k,
                                const void* new_v, const int32_t* dst_slots, float* slot_scores, int slot_stride,
                                void* o, float* lse_opt, void* workspace, size_t workspace_bytes, void* stream);
/* kvs_paged_decode_scored_select on the 8-bit cache (as kvs_paged_decode_scored_fp8). */
int kvs_paged_decode_scored_select_fp8(const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                       int num_blocks, const int32_t* block_tables, int max_blocks,
                                       const int32_t* ctx_lens, int batch, int max_ctx, int hq, int hkv, int d,
                                       float scale, const void* new_k, const void* new_v, const int32_t* dst_slots,
                                       float* slot_scores, int32_t* slot_pos, int slot_stride, int cap, int alpha,
                                       const int32_t* next_pos, int32_t* next_dst_slots, void* o, float* lse_opt,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_paged_decode_noalloc - kvs_paged_decode for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, meaning, layouts and results as kvs_paged_decode, without the workspace:
 * the split partials go to a scratch array of 16 MiB that the library holds on every device
 * it runs on until the process ends (its address is looked up on the first call on a device).
 * The call uses the scratch of the device current on the calling thread; the stream (NULL for
 * the default one) must belong to that device.  Nothing needs to start at zero there: every
 * call writes each partial it reads.  All calls on one device share that array, so calls that
 * overlap on one device (concurrent streams or threads) race; calls in one stream do not.
 * Nothing is allocated: no hipMalloc, no hipFree, no allocating library routine.
 * Errors: as kvs_paged_decode; KVS_E_INVAL also when kvs_paged_decode_workspace_size for the
 * shape exceeds 16 MiB (use kvs_paged_decode with a workspace), or when the stream belongs to
 * another device; KVS_E_HIP if the scratch address cannot be obtained.
 */
int kvs_paged_decode_noalloc(const void* q, void* k_pool, void* v_pool, int num_blocks,
                             const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                             int batch, int max_ctx, int hq, int hkv, int d, float scale,
                             const void* new_k_opt, const void* new_v_opt, void* o, float* lse_opt,
                             void* stream);

/*
 * kvs_copy_blocks_fp8 - kvs_copy_blocks for an 8-bit cache: code blocks and scale rows.
 */
int kvs_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int num_blocks, int hkv, int d,
                        const int32_t* src_dst_pairs, int n_pairs, void* stream);

/*
 * kvs_probe_stream_read - measurement helper: read `bytes` of device memory once, 16 bytes
 *   per lane with four loads in flight, and fold the words per workgroup.  It gives the
 *   read rate a plain streaming kernel reaches, the practical ceiling the memory-bound
 *   steps (compaction, paged decode) are compared with beside the published HBM peak.
 * In:  buf device, 16-byte aligned; bytes a positive multiple of 16; grid workgroups of 256
 *      threads (1 .. 2^20).  sink: device array of grid words, written only where a
 *      workgroup's folded word equals key (the caller picks a key that does not occur).
 * Errors: KVS_E_INVAL on a NULL pointer, misalignment or a bad size; KVS_E_HIP on launch failure.
 */
int kvs_probe_stream_read(const void* buf, size_t bytes, int grid, uint32_t key, uint32_t* sink, void* stream);

/*
 * kvs_probe_timestamp - measurement helper: one lane stores the GPU's real-time counter (a
 *   fixed 100 MHz clock on MI355X, independent of the shader clock) when the kernel runs.
 *   Two stamps placed as the first and last launches of a captured graph give the GPU time
 *   of the work between them from the moment the graph starts running.
 * In/out: out device pointer to one uint64, 8-byte aligned (written, counter ticks).
 * Errors: KVS_E_INVAL on a NULL or misaligned pointer; KVS_E_HIP on launch failure.
 */
int kvs_probe_timestamp(uint64_t* out, void* stream);

/*
 * Host block allocator.  [PAG] "How paging works": a request gets a new block only when
 * its last block is full, from any free block (the worked example pops from the front of
 * the free list).  [PAG] "Sharing blocks between sequences": a reference count per block;
 * copy-on-write.  [PAG] "Related techniques": a finished sequence's blocks return to the
 * free pool at once.
 * The free list is FIFO: allocation pops the front, a block whose count reaches 0 is
 * appended at the back.  The object is owned by the caller (create / destroy).
 */
typedef struct kvs_alloc kvs_alloc;
/* initial_free_order: host array of n_initial distinct ids in [0, num_blocks) forming the
 * free list (NULL: 0..num_blocks-1, n_initial ignored).  Blocks not listed start in use
 * with count 1. */
int kvs_alloc_create(int num_blocks, const int32_t* initial_free_order, int n_initial,
                     kvs_alloc** out);
void kvs_alloc_destroy(kvs_alloc* a);
/* Pop the front of the free list; its count becomes 1.  KVS_E_NOBLOCKS if empty. */
int kvs_alloc_block(kvs_alloc* a, int32_t* out_block);
/* Share a live block.  KVS_E_STATE if the block is free. */
int kvs_alloc_incref(kvs_alloc* a, int32_t block);
/* Drop one reference; at 0 the block is appended to the free list.  KVS_E_STATE if free. */
int kvs_alloc_decref(kvs_alloc* a, int32_t block);
/* Count of a block (0 = free), or KVS_E_INVAL for an id out of range. */
int kvs_alloc_refcount(const kvs_alloc* a, int32_t block);
int kvs_alloc_num_free(const kvs_alloc* a);
/* Copy up to cap ids of the free list, front first; returns the number written. */
int kvs_alloc_free_list(const kvs_alloc* a, int32_t* out, int cap);
/* Copy-on-write: count > 1 -> a fresh block is allocated, the old one loses a reference,
 * *out_block = new id and *copied = 1 (the caller copies the data if a live slot survives);
 * count == 1 -> *out_block = block, *copied = 0.  KVS_E_NOBLOCKS / KVS_E_STATE as above. */
int kvs_alloc_cow(kvs_alloc* a, int32_t block, int32_t* out_block, int* copied);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H_ */
