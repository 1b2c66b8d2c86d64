/*
 * kvc.h -- C ABI of libkvc: one decode step of attention over a per-head,
 * budget-limited KV cache on AMD Instinct MI355X (gfx950), and the eviction
 * that keeps that cache at budget.
 *
 * Sources, cited by page and section:
 *  [GUIDE] "Rethinking KV Cache Compression: from memory savings back to real
 *          serving end-to-end gains" -- section 2 (cost structure of the four
 *          baselines: 64 sink/heavy + 448 recent = cache 512) and section 16
 *          (the KV capacity formula; the four methods step by step; prefill,
 *          decode and TP accounting; limits -- H2O needs the attention
 *          probabilities that a fused attention kernel does not expose).
 *  [BLOG]  "KV Cache eviction in practice: when to drop the scorer and evict
 *          at random" -- sections "scorers are overrated", "six steps to land
 *          it" and "reference implementation" (per-head uniform eviction with
 *          the prompt pinned, equal per-head counts, no union across heads).
 *  [EMP]   "Practical Online KV Cache Compaction for LLM Agents: An Empirical
 *          Study" -- section 4.2 (mark evicted tokens, then compact the
 *          survivors, with a logical-to-physical index map).
 *
 * Conventions shared by every call
 *  - All pointers in kvc_cache and all array arguments are DEVICE pointers
 *    unless stated otherwise; the kvc_cache / kvc_policy structs themselves
 *    are read on the host during the call and not retained.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    keeps a pointer after a call returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Arguments are validated on the host first; a call that
 *    returns an error has enqueued nothing.  Faults surface at the caller's
 *    next synchronisation.
 *  - A "unit" is one (sequence b, kv head h); units are independent.
 *  - Query head i reads kv head floor(i / G), G = q_heads / kv_heads.
 *  - Attention scale: the caller passes it (1/sqrt(head_dim) is the usual).
 *  - Inputs must be finite; NaN/Inf are outside the contract.
 *  - Device-side contract violations (a unit whose n_slots is negative, above
 *    the capacity, or equal to the capacity when a token must be appended)
 *    are clamped so that no access leaves the buffers, and reported by OR-ing
 *    KVC_FLAG_* bits into *flags when kvc_cache.flags is not NULL.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_INVALID_ARG = 1, /* null pointer, bad count, inconsistent policy */
    KVC_ERR_UNSUPPORTED = 2, /* head_dim / dtype / group size not built */
    KVC_ERR_SHAPE = 3,       /* q_heads % kv_heads != 0, paged geometry, ... */
    KVC_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
    KVC_ERR_HIP = 5          /* a HIP runtime call failed */
} kvc_status;

typedef enum kvc_dtype {
    KVC_BF16 = 0,     /* K, V, q, k_new, v_new stored as bfloat16 */
    KVC_F32 = 1,      /* ... as float32 */
    /* K, V stored as 8-bit floats E5M2 (OCP 8-bit floating point: sign, 5
     * exponent bits with bias 15, 2 mantissa bits; no scale), the fp8
     * KV-cache dtype of the serving command in [BLOG] "reference
     * implementation"; q, k_new, v_new are bfloat16.  A new token is stored
     * as the nearest E5M2 value (ties to even, magnitudes beyond 57344
     * saturate) and attended as stored.  [BLOG] advises measuring the cache
     * dtype apart from eviction: a KVC_BF16 cache of the same shape is that
     * reference. */
    KVC_FP8_E5M2 = 2
} kvc_dtype;

/* bits OR-ed into *kvc_cache.flags by kernels */
#define KVC_FLAG_FULL 1      /* n_slots == capacity at an append: token not stored */
#define KVC_FLAG_BAD_COUNT 2 /* n_slots outside [0, capacity]: clamped */
#define KVC_FLAG_BAD_BLOCK 4 /* block_table entry outside the pool: block 0 used */

/*
 * The cache.  Per unit, slots 0 .. n_slots-1 are filled; slot order is free
 * (attention is permutation invariant because keys already carry their
 * position encoding [BLOG "reference implementation", note on sort()]), and
 * pos[] maps each slot to the token's original position [EMP 4.2].
 * Limits: capacity <= 65,536 slots, q_heads / kv_heads <= 16 and
 * batch * kv_heads <= 16,777,216 units (KVC_ERR_UNSUPPORTED beyond).
 *
 * Contiguous layout (block_size == 0):
 *   k, v       [batch, kv_heads, capacity, head_dim] of dtype
 * Paged layout (block_size > 0, e.g. 16):
 *   k, v       pool [num_blocks, kv_heads, block_size, head_dim]
 *   block_table[batch, max_blocks]: slot j of sequence b, head h lives in
 *              block block_table[b*max_blocks + j/block_size], row
 *              j % block_size; capacity must equal max_blocks*block_size.
 * Both layouts:
 *   pos        [batch, kv_heads, capacity] int32 original token positions
 *   n_slots    [batch, kv_heads] int32 filled slots per unit
 *   flags      optional int32 word (see KVC_FLAG_*), may be NULL
 */
typedef struct kvc_cache {
    int32_t batch;
    int32_t q_heads;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t capacity;
    int32_t dtype; /* kvc_dtype */
    int32_t block_size;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t reserved;
    void *k;
    void *v;
    const int32_t *block_table;
    int32_t *pos;
    int32_t *n_slots;
    int32_t *flags;
} kvc_cache;

typedef enum kvc_policy_kind {
    KVC_POLICY_FULL = 0,      /* keep everything (no eviction) */
    KVC_POLICY_STREAMING = 1, /* n_sink first + n_recent most recent */
    KVC_POLICY_H2O = 2,       /* n_heavy by accumulated attention + n_recent */
    KVC_POLICY_RANDOM = 3     /* prompt pinned + n_keep uniform per head */
} kvc_policy_kind;

typedef struct kvc_policy {
    int32_t kind; /* kvc_policy_kind */
    int32_t n_sink;
    int32_t n_heavy;
    int32_t n_recent;
    int32_t prompt_len;
    int32_t n_keep;
    uint64_t seed;
    /* KVC_POLICY_H2O only.  0: scores accumulate the group-summed
     * probabilities (plain H2O).  0 < decay < 1: they are a decayed attention
     * activity, s <- decay * s + (1 - decay) * sum_i p_i, a new slot starting
     * from 0 [EMP 3.1: accumulation with a decay coefficient on earlier
     * attention; EMP 4.1: the incremental update, decay e.g. 0.99].  The
     * kept set is chosen from these scores exactly as for plain H2O. */
    float decay;
} kvc_policy;

/* ------------------------------------------------------------------------
 * Host-only helpers
 * ---------------------------------------------------------------------- */

/* KV bytes per token = 2 (K and V) x layers x kv_heads x head_dim x
 * dtype_bytes [GUIDE 16, capacity formula; BLOG "six steps", memory
 * accounting].  `layers` counts attention layers only (linear-attention
 * layers of hybrid models hold no KV [BLOG "what are you compressing"]).
 * Returns 0 if any argument is not positive. */
size_t kvc_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                           int32_t dtype_bytes);

/* Kept generated tokens of a one-shot random eviction over n_candidates
 * tokens after the prompt: max(1, trunc(n_candidates * keep_ratio)), clamped
 * to n_candidates; 0 when n_candidates <= 0 [BLOG "reference
 * implementation"]. */
int64_t kvc_n_keep(int64_t n_candidates, double keep_ratio);

/* Static, never-freed description of a status code (a kvc_status value;
 * any other int gives "unknown status"). */
const char *kvc_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *kvc_last_error(void);

/* Workspace (device bytes) that kvc_decode_attn / kvc_decode_step /
 * kvc_h2o_accumulate need for `c` when no unit attends more than
 * max_len_hint entries (n_slots + 1).  0 means no workspace is needed. */
size_t kvc_workspace_bytes(const kvc_cache *c, int32_t max_len_hint);

/* ------------------------------------------------------------------------
 * Device calls
 * ---------------------------------------------------------------------- */

/*
 * Decode attention for one new token per sequence [GUIDE 16, "prefill,
 * decode, TP": a decode step reads all kept history].
 *
 * For every unit (b, h) with n = n_slots[b,h] and every query head i of the
 * group of h:  out[b,i,:] = sum_j p_j v_j  with p = softmax(scale * q K^T)
 * over the n cached slots AND the new token (k_new[b,h], v_new[b,h]).
 * The new token is then stored at slot n with pos = new_pos[b], and
 * n_slots[b,h] becomes n + 1 (capacity must exceed n; see KVC_FLAG_FULL).
 *
 * If h2o_scores ([batch, kv_heads, capacity] fp32) is not NULL, the group's
 * summed probabilities are added to it: scores[b,h,j] += sum_i p_ij for every
 * cached slot, and the new slot is set to its own probability sum -- the
 * accumulated-attention statistic of H2O [GUIDE 2 and 16, "the 4 methods":
 * accumulate attention scores and update the kept set; GUIDE 16 "limits":
 * a fused kernel must expose these probabilities].
 *
 *   new_pos  [batch] int32 position of the new token
 *   q        [batch, q_heads, head_dim]  dtype
 *   k_new,v_new [batch, kv_heads, head_dim] dtype
 *   out      [batch, q_heads, head_dim] fp32
 *            q, k_new, v_new and out must be 16-byte aligned (they are read
 *            and written in 16-byte pieces); KVC_ERR_INVALID_ARG otherwise.
 *   score_decay  0 for the sums above; 0 < score_decay < 1 updates each score
 *            as s <- score_decay * s + (1 - score_decay) * sum_i p_i instead
 *            (decayed attention activity, see kvc_policy.decay); other values
 *            are rejected.  Ignored when h2o_scores is NULL.
 *   max_len_hint  upper bound on n_slots + 1 over the batch (<= capacity+1);
 *            sizes the split of long units over workgroups.  A unit longer
 *            than the hint is still computed exactly (less parallel).
 *   workspace     kvc_workspace_bytes(c, max_len_hint) device bytes (may be
 *            NULL when that is 0).
 */
kvc_status kvc_decode_attn(const kvc_cache *c, const int32_t *new_pos,
                           const void *q, const void *k_new, const void *v_new,
                           float *out, float *h2o_scores, float scale,
                           float score_decay, int32_t max_len_hint,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Unfused H2O score pass: adds the group-summed softmax probabilities of
 * m_rows query rows per sequence to h2o_scores, over each unit's current
 * n_slots slots (no append).  Row r of sequence b sees the slots whose pos is
 * <= q_pos[b*m_rows + r] when q_pos is not NULL (causal prompt scoring), all
 * slots otherwise.  This is the "extra traversal" that maintaining H2O scores
 * costs when attention does not expose its probabilities [GUIDE 16 "limits"],
 * and the prefill scoring of H2O [GUIDE 16 "prefill, decode, TP"]: with the
 * prompt's queries as the rows and q_pos their positions, the scores are the
 * attention the prompt's own causal attention gave each cached token.
 *   q_rows [batch, m_rows, q_heads, head_dim] dtype;  q_pos NULL or
 *   [batch, m_rows] int32.
 *   workspace  kvc_h2o_accumulate_workspace_bytes(c, m_rows) device bytes
 *            (bf16, head_dim 128: one fp32 log-sum-exp per query row and head;
 *            0 bytes and NULL allowed otherwise).
 * bf16 caches with head_dim 128 run on the matrix cores (two exact passes:
 * the rows' softmax statistics, then every slot's probability sum in fp64,
 * a fixed summation order) when one sequence's query rows
 * (m_rows * q_heads * 256 bytes) and one unit's K rows (capacity * 256 bytes)
 * are each under 2 GiB; other shapes use a VALU pass.
 */
size_t kvc_h2o_accumulate_workspace_bytes(const kvc_cache *c, int32_t m_rows);
kvc_status kvc_h2o_accumulate(const kvc_cache *c, const void *q_rows,
                              int32_t m_rows, const int32_t *q_pos,
                              float *h2o_scores, float scale, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Selection ("mark" of mark-then-compact [EMP 4.2]).  Reads each unit's
 * n_slots and pos (and scores), writes the kept slot indices in ascending
 * slot order to keep_slots[b,h, 0 .. n_out[b,h]-1] ([batch, kv_heads,
 * capacity] int32) and the count to n_out ([batch, kv_heads] int32).  The
 * cache is not modified.  L = 1 + the largest position in the unit (its
 * newest token).
 *
 * StreamingLLM [GUIDE 2, 16 "the 4 methods"]: keep pos < n_sink and
 * pos >= L - n_recent.
 */
kvc_status kvc_evict_streaming(const kvc_cache *c, int32_t n_sink,
                               int32_t n_recent, int32_t *keep_slots,
                               int32_t *n_out, void *stream);

/* H2O [GUIDE 2, 16 "the 4 methods"]: keep pos >= L - n_recent, and among the
 * other slots the n_heavy with the largest h2o_scores, ties to the lower
 * position. */
kvc_status kvc_evict_h2o(const kvc_cache *c, const float *h2o_scores,
                         int32_t n_heavy, int32_t n_recent,
                         int32_t *keep_slots, int32_t *n_out, void *stream);

/* Per-head uniform random eviction with the prompt pinned [BLOG "scorers are
 * overrated", "six steps", "reference implementation"]: slots with
 * pos < prompt_len are kept; among the others each unit keeps the n_keep
 * whose key is smallest (ties to the lower position), the key of a token
 * being word 0 of Philox4x32-10 (Salmon et al., SC'11) with counter
 * (pos, step, kv head, sequence) and key (seed low 32 bits, seed high 32
 * bits).  Every unit draws its own set; nothing is merged across heads.  With
 * at most n_keep candidates everything is kept. */
kvc_status kvc_evict_random(const kvc_cache *c, int32_t prompt_len,
                            int32_t n_keep, uint64_t seed, uint32_t step,
                            int32_t *keep_slots, int32_t *n_out, void *stream);

/*
 * Compaction ("compact" of mark-then-compact [EMP 4.2]).
 * In place (ordered_dst == NULL): with n_out kept of n slots, the kept slots
 * at index >= n_out move, in ascending order, into the evicted slots below
 * n_out, in ascending order; K row, V row, pos and (if h2o_scores is not
 * NULL) score move together; n_slots becomes n_out.  Sources and
 * destinations are disjoint.
 * Ordered (ordered_dst != NULL): the kept entries are gathered into
 * ordered_dst in ascending position, slot i holding the i-th kept position --
 * the regular [kv_heads, prompt_len + n_keep, head_dim] layout of the
 * blog's hook [BLOG "reference implementation"]; ordered_dst's n_slots is
 * set, its scores are not written, the source cache is not modified.
 * ordered_dst must have the same batch/heads/head_dim/dtype and a capacity
 * of at least every n_out; at most 8192 kept entries per unit.
 */
kvc_status kvc_compact(const kvc_cache *c, const int32_t *keep_slots,
                       const int32_t *n_out, float *h2o_scores,
                       const kvc_cache *ordered_dst, void *stream);

/*
 * One whole decode step: kvc_decode_attn, then the policy's selection, then
 * in-place compaction, with the same results as those three calls in that
 * order (kept sets identical, the new token placed where the compaction
 * would put it, identical outputs and scores).  For KVC_POLICY_H2O,
 * h2o_scores is required; `step` keys the random draws.
 */
kvc_status kvc_decode_step(const kvc_cache *c, const kvc_policy *policy,
                           uint32_t step, const int32_t *new_pos,
                           const void *q, const void *k_new, const void *v_new,
                           float *out, float *h2o_scores, float scale,
                           int32_t max_len_hint, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * kvc_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as kvc_decode_step without the workspace: its
 * scratch is one static device array of KVC_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends.  The call
 * allocates nothing.  A cache and length hint whose workspace
 * (kvc_workspace_bytes) exceeds the array are rejected with
 * KVC_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares its array: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 */
#define KVC_NOALLOC_SCRATCH_BYTES (128u << 20)
kvc_status kvc_decode_step_noalloc(const kvc_cache *c, const kvc_policy *policy,
                                   uint32_t step, const int32_t *new_pos, const void *q,
                                   const void *k_new, const void *v_new, float *out,
                                   float *h2o_scores, float scale, int32_t max_len_hint,
                                   void *stream);

/*
 * Measurement helper, not part of a decode step: reads `bytes` bytes of
 * device memory at `src` once, with fully coalesced 16-byte loads spread over
 * the whole GPU, and writes `sink` (one uint32_t of device memory) only if the
 * data hold a pattern that the caller's buffer does not.  Its duration gives
 * the read-only streaming rate this GPU reaches in practice, the figure a
 * decode step's achieved HBM rate is compared with next to the nominal peak.
 * `src` must be 16-byte aligned and `bytes` a positive multiple of 16;
 * nothing is enqueued otherwise (KVC_ERR_INVALID_ARG).
 */
kvc_status kvc_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* ============================================================================
 * KIVI-style quantized KV cache: keep every token, fewer bits per element
 * [GUIDE] section 2 (KIVI with group 32 and a 128-token residual), section 16
 * "KV capacity formula" (quantisation keeps all tokens at 4 bits instead of
 * 16, with a full-precision residual of recent tokens), "the four methods"
 * (K quantised along channels, V along tokens, groups of 32; a decode step
 * dequantises or runs a quantised kernel) and "limits" (scale granularity;
 * a full residual converts its old tokens, periodic work).
 *
 * Per unit (sequence b, kv head h) the cache holds n_quant[u] tokens
 * (a multiple of 32) as 4-bit codes, oldest first, then n_res[u] <= 128
 * newest tokens as given (bf16), oldest first.  Grids: every group of 32
 * consecutive quantised tokens has, per channel d, one grid for K (those 32
 * tokens' K[., d]), and per token, one grid for V per 32 consecutive channels.
 * A grid over values x: lo = min x, scale = (max x - lo) / 15,
 * code = round-half-to-even((x - lo) / scale) clamped to [0, 15] (0 when
 * scale is 0), every operation in binary32; the element's value is
 * code * scale + lo.
 *
 * A decode step attends each of the G query heads over the dequantised
 * tokens, the residual and the new token, and writes out[b, i, :] (fp32);
 * then, if the residual holds 128 tokens, its 32 oldest become the next
 * quantised group and leave it; then the new token joins the residual.  So
 * the residual keeps 97..128 tokens once a sequence is longer than 128, and
 * the conversion runs every 32 steps.
 *
 * Layout (head_dim 128, 4-bit codes, 64 bytes per token and tensor; u = b *
 * kv_heads + h, T = max_quant):
 *   k_codes [u][T][64] uint8.  Dim d of a token: dword 4*((d%32)/8) + d/32 of
 *           its row (bytes 16*((d%32)/8) + 4*(d/32) ..), nibble slot k of
 *           that dword (bits 4k..4k+3) with e = d % 8 = 2k (k < 4) or
 *           2(k-4)+1 (k >= 4).
 *   k_scale, k_lo [u][T/32][128] float: the grid of channel d of group g.
 *   v_codes [u][T/16][1024] uint8: tiles of 16 consecutive tokens.  The 16
 *           bytes at 16*(16r + c) of a tile (r < 4, c < 16) hold dims c + 16m
 *           (m < 8) of the tile's tokens r, r+4, r+8, r+12 as four little-
 *           endian words: word 0 even m of tokens r (bits 0..15) and r+4
 *           (bits 16..31), word 1 odd m of the same two, words 2 and 3 the
 *           same for tokens r+8 and r+12; in a half, dim c + 16m at bits
 *           4*(m/2).
 *   v_scale, v_lo [u][T][4] float: the grid of channels 32c..32c+31 of a token.
 *   k_res, v_res [u][128][128] bf16: residual rows 0 .. n_res-1, oldest first;
 *           a k_res row in dim order, a v_res row with dim d at element
 *           8*(d%16) + d/16 (the dims of a V code lane's 16 bytes).
 *   n_quant, n_res [u] int32.
 * These layouts put one lane's matrix-core operands of a 16-token tile in
 * one 16-byte load and widen two codes with two ALU instructions.  The workspace holds the partials of
 * a unit's shares of the quantised tokens when max_quant_hint gives it more
 * than one; with one share per unit a step is a single launch.
 * ========================================================================== */
typedef struct kvc_kivi_cache {
    int32_t batch, q_heads, kv_heads, head_dim;  /* head_dim 128; q_heads / kv_heads <= 8;
                                                    batch * kv_heads <= 16,777,216 */
    int32_t max_quant;                           /* T: quantised tokens per unit, a multiple of 32 */
    int32_t bits;                                /* 4 */
    uint8_t *k_codes, *v_codes;
    float *k_scale, *k_lo, *v_scale, *v_lo;
    void *k_res, *v_res;                         /* bf16 */
    int32_t *n_quant, *n_res;
    int32_t *flags;                              /* nullable; KVC_FLAG_* as for kvc_cache */
} kvc_kivi_cache;

/* Device bytes of the workspace of kvc_kivi_decode when every unit holds at
 * most max_quant_hint quantised tokens (<= 0: max_quant). */
size_t kvc_kivi_workspace_bytes(const kvc_kivi_cache *c, int32_t max_quant_hint);

/*
 * Prefill: sequence b's prompt of lengths[b] tokens (device int32, clipped
 * to [0, max_len]) from k, v [batch][kv_heads][max_len][128] bf16 (device).
 * The oldest tokens become whole quantised groups, as few as keep the
 * residual within 128 (32 * ceil(max(L - 128, 0) / 32) tokens), the rest
 * the residual; n_quant and n_res are set.  The grids of max_len tokens must
 * fit: 32 * ceil(max(max_len - 128, 0) / 32) <= max_quant (KVC_ERR_SHAPE).
 */
kvc_status kvc_kivi_prefill(const kvc_kivi_cache *c, const void *k, const void *v,
                            int32_t max_len, const int32_t *lengths, void *stream);

/*
 * One decode step as described above.  q [batch][q_heads][128], k_new and
 * v_new [batch][kv_heads][128] bf16; out [batch][q_heads][128] fp32.
 * max_quant_hint bounds n_quant of every unit (<= 0: max_quant) and sizes the
 * split of the quantised tokens over workgroups; a unit above it is still
 * exact, only slower.  A conversion that would exceed max_quant is skipped,
 * the new token is not stored, and KVC_FLAG_FULL is raised.
 */
kvc_status kvc_kivi_decode(const kvc_kivi_cache *c, const void *q, const void *k_new,
                           const void *v_new, float *out, float scale,
                           int32_t max_quant_hint, void *workspace, size_t workspace_bytes,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
