/*
 * Streaming attention forward for AMD Instinct MI355X (gfx950): C ABI.
 *
 * The entry points compute softmax(scale * Q K^T + causal mask) V tile by
 * tile with an online softmax (running max m, running sum l, rescaled output
 * O), so the score and probability matrices never reach memory:
 *
 *   attn_prefill         fused forward over a query block (GQA, causal or not)
 *   attn_prefill_splitkv the same with the key range cut into splits, each
 *                        yielding a partial result (merged by attn_combine_lse)
 *   attn_decode_splitkv  one query token per sequence, the KV range cut into
 *                        splits that each yield a partial result
 *   attn_combine_lse     merge of the split partials by log-sum-exp
 *   attn_decode          the split-KV decode and the merge in one launch
 *   attn_decode_paged    T_q >= 1 new tokens per sequence over a paged KV cache
 *                        with per-sequence lengths (optionally split)
 *
 * The method is the one of "ADR-0060: AHBM GQA Fused Attention kernel
 * (Llama3-70B)": per-tile online softmax (its section 3), log-sum-exp merge of
 * partials (section 4), GQA M-fold (section 5.2), causal tile classes (section
 * 5.4), and the kernel I/O contract (section 0.5: post-RoPE Q, read-only K/V
 * caches, a query block that carries its global position, softmax_scale).
 * "AttentionRegion Transformation" (sections 5-8) states the same streaming
 * structure: Q tile resident, K/V tiles streamed, S and P never materialised.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller (for example a
 *    torch tensor's data_ptr()).  The library allocates nothing, keeps no
 *    state between calls and is reentrant.
 *  - Tensors are dense and contiguous, row-major, in the shapes given below
 *    (last index fastest).  Every tensor pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t; NULL means the default stream.  All work is
 *    enqueued asynchronously on it; buffers must stay alive until the stream
 *    has passed the kernels.
 *  - Return value: ATTN_OK, or an error code.  On any error nothing has been
 *    enqueued and no output has been written.  Argument errors are detected on
 *    the host before any HIP call.  A failed kernel launch returns
 *    ATTN_ERR_LAUNCH.
 *  - Query head h reads KV head h / G with G = Hq / Hkv: the G query heads of
 *    one KV head are consecutive (ADR-0060 section 0, "CUBE Group").
 *  - Exponentials and logarithms are natural in every output; LSE = m + ln l.
 *  - Element types: attn_prefill takes bf16 or fp32; every other entry point
 *    that reads Q, K and V takes bf16 only (the split-KV, decode and paged
 *    kernels exist for the bf16 serving path) and returns
 *    ATTN_ERR_UNSUPPORTED for fp32.
 *  - Accumulation is fp32.  With bf16 inputs the probabilities are rounded to
 *    bf16 (round to nearest even) before the P V product, and O is rounded to
 *    bf16 on output.  LSE and split partials are always fp32.
 */
#ifndef STREAMING_ATTENTION_ATTN_H
#define STREAMING_ATTENTION_ATTN_H

#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
  ATTN_DTYPE_F32 = 0,
  ATTN_DTYPE_BF16 = 1
} attn_dtype_t;

/* Status codes. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                       */
  ATTN_ERR_SHAPE = 2,       /* a size, the scale or the causal/size relation is invalid */
  ATTN_ERR_UNSUPPORTED = 3, /* valid request the library does not implement     */
  ATTN_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned          */
  ATTN_ERR_LAUNCH = 5,      /* the HIP kernel launch failed                     */
  ATTN_ERR_WORKSPACE = 6    /* larger than attn_decode_noalloc's fixed workspace */
};

/*
 * attn_prefill -- fused streaming attention forward over a block of queries.
 *
 * Defined by ADR-0060 section 3 (per-tile sequence: score GEMM scaled by
 * softmax_scale, boundary mask, running max/sum update, rescale of O, P V GEMM,
 * O / l once at the end), section 5.2 (the G query heads of a KV head are
 * stacked into the GEMM M dimension so one K/V tile serves all of them) and
 * section 5.4 (KV tiles wholly after the query block are skipped, tiles wholly
 * before it take no mask, straddling tiles take the triangular mask).
 *
 *   q    [B, Hq,  Sq,  d]  dtype      post-RoPE queries
 *   k    [B, Hkv, Skv, d]  dtype      keys
 *   v    [B, Hkv, Skv, d]  dtype      values
 *   o    [B, Hq,  Sq,  d]  dtype      output (written)
 *   lse  [B, Hq,  Sq]      float32    natural-log sum of exp of the visible
 *                                     scaled scores (written); may be NULL
 *   d        64 or 128
 *   dtype    ATTN_DTYPE_BF16 or ATTN_DTYPE_F32
 *   causal   nonzero: query row t sits at global position q_start + t with
 *            q_start = Skv - Sq (the query block is the last Sq positions, as
 *            the query-block metadata {q_start, T_q} of ADR-0060 section 0.5.3
 *            places it) and sees keys j <= q_start + t.  Requires Sq <= Skv.
 *   scale    multiplies Q K^T before mask and softmax; finite and > 0.
 *
 * Sizes: B, Sq, Skv >= 0; Hq, Hkv >= 1 with Hq % Hkv == 0.  B == 0 or Sq == 0
 * is an empty call (returns ATTN_OK, enqueues nothing).  Skv == 0 (non-causal)
 * gives O = 0 and LSE = -inf.  k and v may be NULL when Skv == 0.  The Q rows
 * of one KV head (G * Sq * d elements) and the K or V rows of one (batch, KV
 * head) (Skv * d elements) must each span less than 2 GiB.
 * Errors: ATTN_ERR_NULL (q, o, or k/v with Skv > 0), ATTN_ERR_SHAPE,
 * ATTN_ERR_UNSUPPORTED (d not 64/128, unknown dtype, a slice of 2 GiB or
 * more), ATTN_ERR_ALIGN.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Skv, int32_t d,
                 attn_dtype_t dtype, int32_t causal, float scale, hipStream_t stream);

/*
 * attn_prefill_splitkv -- attn_prefill with the key range cut into splits, for
 * query blocks too small to occupy the GPU (a short chunk of queries after a
 * long prefix).  Every split yields a normalised partial result per query row;
 * attn_combine_lse merges them.
 *
 * Defined by ADR-0060 section 5.5 (ring prefill: each step folds one K/V block
 * into the running state of every query block; on one device the blocks
 * become splits) and section 4 (each split's (m_i, l_i, O_i), merged by
 * log-sum-exp), with the causal rules of attn_prefill.
 *
 *   q, k, v, B, Hq, Hkv, Sq, Skv, d, causal, scale   as for attn_prefill
 *   dtype      ATTN_DTYPE_BF16 only
 *   num_splits 1 .. 256
 *   part_o     [B, Hq, Sq, num_splits, d] float32 (written)
 *   part_lse   [B, Hq, Sq, num_splits]    float32 (written)
 *
 * Split plan (part of the contract): with T = ceil(Skv / 64) key tiles of 64
 * and c = ceil(T / num_splits), split s covers keys [64 s c, min(64 (s + 1) c,
 * Skv)).  part_lse[b,h,t,s] is the natural-log sum of exp of row t's visible
 * scaled scores over that range and part_o[b,h,t,s,:] its attention output
 * over that range alone; a row that sees no key of the range (or an empty
 * range) gets (-inf, 0).  Every entry is written.
 *
 * The final result: attn_combine_lse(part_o, part_lse, NULL, B * Hq * Sq, 1,
 * num_splits, d, o, lse, ATTN_DTYPE_BF16, stream) with o [B, Hq, Sq, d] and
 * lse [B, Hq, Sq] -- the partial tensors are laid out as [rows, splits, ...]
 * for exactly that call.
 * Errors: as attn_prefill, plus ATTN_ERR_SHAPE (num_splits out of range) and
 * ATTN_ERR_UNSUPPORTED (dtype other than bf16).
 */
int attn_prefill_splitkv(const void* q, const void* k, const void* v, float* part_o, float* part_lse,
                         int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Skv, int32_t d,
                         int32_t num_splits, attn_dtype_t dtype, int32_t causal, float scale, hipStream_t stream);

/*
 * attn_decode_splitkv -- one query token per sequence against a KV cache,
 * the valid key range of each sequence cut into contiguous splits, each split
 * producing a normalised partial result.
 *
 * Defined by ADR-0060 section 5.2 (decode: T_q = 1, attends to all past keys,
 * only the ragged last tile is masked; the G query heads of a KV head are
 * stacked into M), section 5.3 and section 4 (each split sweeps its own KV
 * range and yields (m_i, l_i, O_i)), and section 2.1 (contiguous key blocks per
 * split).  The cache is read only; the caller has already appended the new
 * token's K/V row (ADR-0060 section 0.5.1, precondition P3).
 *
 *   q          [B, Hq, 1, d]        bf16
 *   k_cache    [B, Hkv, S_cap, d]   bf16
 *   v_cache    [B, Hkv, S_cap, d]   bf16
 *   kv_len     [B] int32 device, or NULL (every sequence has S_cap keys).
 *              Values are clamped to [0, S_cap]; cache slots at or beyond
 *              kv_len[b] are never read.
 *   num_splits [B] int32 device, or NULL (max_splits for every sequence).
 *              Values are clamped to [1, max_splits].
 *   max_splits 1 .. 256
 *   part_o     [B, Hq, max_splits, d] float32 (written)
 *   part_lse   [B, Hq, max_splits]    float32 (written)
 *
 * Split plan (part of the contract): with len = kv_len[b], n = num_splits[b],
 * chunk = 64 * ceil(ceil(len / n) / 64), split s < n covers keys
 * [s * chunk, min((s + 1) * chunk, len)).  part_lse[b,h,s] is the natural-log
 * sum of exp of the scaled scores over that range and part_o[b,h,s,:] the
 * attention output over that range alone, i.e. the pages' (m_i, l_i, O_i)
 * carried as (m_i + ln l_i, O_i / l_i).  An empty range gives (-inf, 0).
 * Entries s >= n are not written.
 *
 * Sizes: B, S_cap >= 0; Hq, Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= 16; d 64 or
 * 128; scale finite and > 0.  B == 0 is an empty call.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED (dtype other than
 * bf16, d not 64/128, more than 16 query heads per KV head), ATTN_ERR_ALIGN.
 */
int attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_len, const int32_t* num_splits,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d,
                        int32_t max_splits, attn_dtype_t dtype, float scale,
                        float* part_o, float* part_lse, hipStream_t stream);

/*
 * attn_decode -- split-KV decode and the log-sum-exp merge in one launch.
 *
 * Same computation, arguments and split plan as attn_decode_splitkv followed
 * by attn_combine_lse, fused: every split workgroup of a (sequence, KV head)
 * writes its partial and counts itself in; the last one to arrive merges that
 * group's partials and writes the final output.  Nothing waits on anything
 * (ADR-0060 section 4.3: a node merges as its children arrive, and the root
 * normalises once).  This saves the second launch and its ramp.
 *
 *   (q ... part_lse)  exactly as for attn_decode_splitkv; part_o / part_lse
 *                     are the workspace the splits publish into (and hold the
 *                     partials afterwards)
 *   counters   [B * Hkv] int32 device workspace.  Must be all zero on entry;
 *              every entry is zero again when the launch has completed.
 *              Launches that share a counters buffer must not overlap.
 *   o          [B, Hq, 1, d] bf16 (written)
 *   lse        [B, Hq] float32 (written); may be NULL
 *
 * A sequence with kv_len = 0 gets O = 0 and LSE = -inf.
 * Errors: as attn_decode_splitkv, plus ATTN_ERR_NULL for counters or o.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* kv_len, const int32_t* num_splits,
                int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d,
                int32_t max_splits, attn_dtype_t dtype, float scale,
                float* part_o, float* part_lse, int32_t* counters,
                void* o, float* lse, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode_splitkv followed by attn_combine_lse, with
 * the split partials kept in a fixed workspace inside the library instead of
 * caller buffers.  For callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It calls no allocating routine.
 *
 *   (q ... scale)   exactly as for attn_decode_splitkv (same split plan)
 *   o          [B, Hq, 1, d] bf16 (written)
 *   lse        [B, Hq] float32 (written); may be NULL
 *
 * Workspace: a device array of the library, (128 + 1) * 4 bytes per partial for
 * ATTN_NOALLOC_MAX_PARTIALS partials (32.25 MiB), one copy per GPU, held
 * until the process ends.  Requires B * Hq * max_splits <=
 * ATTN_NOALLOC_MAX_PARTIALS, else ATTN_ERR_WORKSPACE.  Every call on one GPU
 * uses the same array and leaves the last call's partials in it: calls that
 * overlap in time on one GPU (on different streams) race; calls ordered on
 * one stream do not.
 * Errors: as attn_decode_splitkv, plus ATTN_ERR_NULL for o and
 * ATTN_ERR_WORKSPACE.
 */
#define ATTN_NOALLOC_MAX_PARTIALS 65536
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_len, const int32_t* num_splits,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d,
                        int32_t max_splits, attn_dtype_t dtype, float scale,
                        void* o, float* lse, hipStream_t stream);

/*
 * attn_decode_paged -- multi-token decode over a paged KV cache: every
 * sequence b has T_q new query tokens, which are the last T_q of its kv_len[b]
 * positions and attend causally (bottom-right) to its keys.  T_q = 1 is the
 * ordinary decode.
 *
 * Defined by ADR-0060 section 0.5.3 (the query block carries its start and
 * length, q_block_meta {q_start, T_q}; here q_start = kv_len[b] - T_q), section
 * 2.2 (the kernel derives the valid length and read range from a counter; here
 * kv_len[b]) and section 2.1 (a sequence's keys may sit in a non-contiguous
 * placement that plain arithmetic maps back to global positions; here a block
 * table), with the per-tile sequence of section 3 and the split merge of
 * section 4.
 *
 *   q           [B, Hq, T_q, d]              bf16
 *   k_pages     [num_pages, Hkv, 64, d]      bf16, page pool (a page holds 64
 *   v_pages     [num_pages, Hkv, 64, d]      bf16   consecutive positions of one
 *                                                   sequence for every KV head)
 *   block_table [B, max_pages] int32 device: logical page p of sequence b
 *               (positions 64 p .. 64 p + 63) is pool page block_table[b, p].
 *               Entries are clamped into [0, num_pages); only the first
 *               ceil(kv_len[b] / 64) entries of a row are read.
 *   kv_len      [B] int32 device; clamped to [0, 64 * max_pages].  Pool rows at
 *               or past kv_len[b] in the sequence's last page are never used.
 *   num_splits  1 .. 256.  1: o [B, Hq, T_q, d] bf16 and lse [B, Hq, T_q] fp32
 *               (may be NULL) are written; part_o / part_lse may be NULL.
 *               > 1: part_o [B, Hq, T_q, num_splits, d] and part_lse
 *               [B, Hq, T_q, num_splits] fp32 are written; o / lse are not
 *               touched and may be NULL.
 *   num_splits_seq  [B] int32 device, or NULL (num_splits for every sequence):
 *               sequence b uses n_b = num_splits_seq[b] splits, clamped to
 *               [1, num_splits]; ignored when num_splits is 1.  Split s < n_b
 *               covers keys [64 s c, min(64 (s + 1) c, kv_len[b])) with
 *               c = ceil(ceil(kv_len[b] / 64) / n_b); entries s >= n_b are not
 *               written.  Merge with attn_combine_lse(part_o, part_lse,
 *               num_splits_seq, B, Hq * T_q, num_splits, d, o, lse,
 *               ATTN_DTYPE_BF16, stream): its rows are (b, head, token).
 *
 * A query token before the sequence's first key (kv_len[b] < T_q) and an
 * empty split give O = 0 and LSE = -inf.
 * Sizes: B, T_q >= 0 (0 is an empty call); Hq, Hkv >= 1, Hq % Hkv == 0;
 * num_pages, max_pages >= 1 with 64 * max_pages < 2^31; d 64 or 128.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED (dtype other than
 * bf16, d not 64/128), ATTN_ERR_ALIGN (q, the pools and the written outputs
 * must be 16-byte aligned).
 */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* kv_len, const int32_t* num_splits_seq, int32_t B, int32_t Hq, int32_t Hkv,
                      int32_t T_q, int32_t num_pages, int32_t max_pages, int32_t d, int32_t num_splits,
                      attn_dtype_t dtype, float scale, float* part_o, float* part_lse, void* o, float* lse,
                      hipStream_t stream);

/*
 * attn_combine_lse -- merge split partials into the final decode output.
 *
 * Defined by ADR-0060 section 4: the merge of two partials takes
 * m = max(m_a, m_b), weights exp(m_a - m) and exp(m_b - m), adds l and O with
 * those weights, and normalises once at the end.  With partials carried as
 * (lse_s, O_s): M = max_s lse_s, w_s = exp(lse_s - M),
 * O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s.
 *
 *   part_o     [B, Hq, max_splits, d] float32
 *   part_lse   [B, Hq, max_splits]    float32
 *   num_splits [B] int32 device, or NULL (max_splits); clamped to
 *              [1, max_splits]; only the first num_splits[b] entries are read.
 *   o          [B, Hq, 1, d] out_dtype (written)
 *   lse        [B, Hq] float32 (written); may be NULL
 *   out_dtype  ATTN_DTYPE_BF16 or ATTN_DTYPE_F32
 *
 * A sequence whose partials are all empty gets O = 0 and LSE = -inf.
 * Sizes: B >= 0, Hq >= 1, max_splits 1 .. 256, d 64 or 128.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGN.
 */
int attn_combine_lse(const float* part_o, const float* part_lse, const int32_t* num_splits,
                     int32_t B, int32_t Hq, int32_t max_splits, int32_t d,
                     void* o, float* lse, attn_dtype_t out_dtype, hipStream_t stream);

/* Short English text for a status code (static storage). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* STREAMING_ATTENTION_ATTN_H */
