/*
 * oscar.h -- C ABI of the OSCAR INT2-history decode library for AMD Instinct MI355X (gfx950).
 *
 * OSCAR keeps each sequence's KV cache in three segments: a BF16 attention sink of 64 tokens, a
 * history stored as rotated INT2 codes, and a BF16 window of the 256 most recent tokens.  A
 * history key (value) x is stored as the 2-bit group codes of x' = clip(x R_k) (x R_v), where
 * R = U * Hadamard * bit-reversal is fixed per layer and KV head.  Decode attention runs over the
 * BF16 segments and the INT2 segment separately and merges the two with an online softmax.
 *
 * Sources (web pages on OSCAR), cited by key:
 *   [W1] "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化" (66bd.net article 13430),
 *        section "OSCAR 的设计" -- the rotation R = U * Hadamard * bit-reversal per layer and
 *        head, calibrated clipping, the three-segment pool (64 | INT2 | 256), demotion of the
 *        oldest recent token by a fused rotate / clip / quantise / pack step, 4 two-bit codes per
 *        byte, INT2 decode with scale / zero-point dequantisation and float accumulation, a
 *        separate BF16 sink / recent pass, an online-softmax merge, paged-KV compatibility.
 *   [W3] the repost of [W1] on m.kljzs.com (article 2026060659440) -- keeps the evaluation part:
 *        the 100k-context system figures (Fig. 5: prefix-cache-hit decode, batch throughput) and
 *        the prefix-cache hit-rate frontier (Fig. 6), and the closing comparison with TurboQuant.
 *   [P]  "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization",
 *        ModelScope paper page of arXiv 2605.17757, "摘要" and "Abstract" -- an INT2 attention
 *        kernel that stays compatible with paged KV caches and fused decode pipelines.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All buffers are caller-owned device memory (allocated by the caller, e.g. through PyTorch).
 *    The library never allocates, frees or synchronises; it keeps no state between calls and is
 *    safe to call from several host threads on different streams.  (One exception, for callers
 *    that cannot allocate: oscar_decode_step_noalloc takes its workspace from a device array the
 *    library owns, one per GPU, and concurrent calls on one GPU race on it.)
 *  - Every compute call is asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *  - All argument checks that can be made on the host run before any HIP call; on failure the
 *    call returns a negative status and touches no device memory.  A kernel launch failure
 *    returns OSCAR_ERR_HIP.  oscar_last_error() gives a message for the calling thread.
 *  - Values that live in device memory (page ids, lengths, history positions) are trusted; a
 *    host copy can be checked with oscar_check_page_table().
 *  - bf16 = IEEE binary32 truncated to its upper 16 bits (round-to-nearest-even when produced);
 *    fp16 = IEEE binary16.  Multi-byte values are little endian.
 *
 * Pool layout (per layer)
 * -----------------------
 *  INT2 pool: num_pages pages; a page holds 64 consecutive history tokens of one sequence for
 *  every KV head: pool bytes [page][kv_head][block], block = oscar_page_block_bytes().  A block
 *  (d = 128 channels, g = group_size, G = d / g groups) is:
 *      offset 0      key codes    2048 bytes = 512 words of 16 codes (4 bytes each)
 *      offset 2048   value codes  2048 bytes = 512 words of 16 codes
 *      offset 4096   meta         [64 tokens][key: G x (fp16 scale, fp16 zero),
 *                                             value: G x (fp16 scale, fp16 zero)]
 *  Key word (t, w) holds channels 16w .. 16w+15 of token t (w < 8); inside it, element 4b+i of
 *  the 16 sits in bits [2i, 2i+1] of byte b.  Value word (c, u) holds channel c of the 16 tokens
 *  16 s + 4 u + j (s, j = 0..3: four consecutive tokens of every 16-token tile), the code of token
 *  16 s + 4 u + j at position 8 (j / 2) + 2 s + (j % 2) (bits [2 pos, 2 pos + 1] of the word); this
 *  order makes the word, spread to nibbles, the matrix cores' FP4 operand in the token order the
 *  score tiles produce.  Words are tiled for 16-byte loads by a 64-lane wave: each region is
 *  two rows of 64 chunks of 16 bytes (4 words), and
 *      key word (t = 16 st + n, w = 4 hf + q)  ->  word index 4 (64 (st / 2) + 16 q + n) + 2 (st % 2) + hf
 *      value word (c = 16 nt + n, u)           ->  word index 4 (64 (nt / 4) + 16 u + n) + nt % 4
 *  so chunk (row j, lane l) is exactly the code words lane l of a wave needs as matrix-core
 *  operands for key sub-tiles 2j, 2j+1 and value channel tiles 4j .. 4j+3.
 *  (4,608 bytes per block at g = 128, i.e. 72 bytes per token and KV head; 5,120 at g = 64.)
 *  Codes are of the rotated, clipped vector in rotated-channel order; the value of element j of
 *  token t in group m = j / g is  scale[t][m] * code[t][j] + zero[t][m]  (rotated space).
 *  History index h of a sequence (h = position - 64) lives in page page_table[b][h / 64],
 *  slot h % 64.  Prefix sharing is expressed by page-table aliasing only; the caller must not
 *  demote into a page that other sequences alias (copy-on-write is the caller's job; a sequence
 *  whose next history index lies in a shared page needs a private copy of that page first, and
 *  oscar_check_page_table() rejects a table that breaks this rule).
 *
 *  BF16 sink:   [max_seqs][num_kv_heads][64][d]  bf16, token at position p < 64 in row p.
 *  BF16 recent: [max_seqs][num_kv_heads][256][d] bf16 ring, token at position p >= 64 in row
 *               p % 256.  A sequence of length L caches positions 0 .. min(L,64)-1 in the sink,
 *               history indices 0 .. L-321 in the pool (when L > 320) and positions
 *               max(64, L-256) .. L-1 in the recent ring.
 *
 * Rotation inputs: U_k, U_v fp32 [num_kv_heads][d][d] row-major (U[h][i][j] is row i, column j);
 * x' = x U H P / sqrt(d) for a row vector x, with H the Sylvester Hadamard matrix and P the
 * bit-reversal permutation of the 7-bit channel index.  clip_k, clip_v fp32 [num_kv_heads]
 * (finite, > 0, <= 65504).
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_ABI_VERSION 8u

typedef int32_t oscar_status;

#define OSCAR_OK              0
#define OSCAR_ERR_NULL       -1   /* a required pointer is NULL */
#define OSCAR_ERR_SHAPE      -2   /* unsupported or inconsistent sizes */
#define OSCAR_ERR_ALIGN      -3   /* a pointer or stride is not suitably aligned */
#define OSCAR_ERR_RANGE      -4   /* a value is out of range (page id, length, count) */
#define OSCAR_ERR_WORKSPACE  -5   /* workspace missing or smaller than required */
#define OSCAR_ERR_HIP        -6   /* the HIP runtime reported an error */

/* Geometry of one layer's cache.  The GPU kernels support exactly: head_dim 128, group_size 128
 * or 64, page_tokens 64, sink_tokens 64, recent_tokens 256 ([W1] OSCAR 的设计 fixes the 64 / 256
 * segment sizes), num_q_heads a multiple of num_kv_heads with a quotient (GQA group) of 1, 2, 4 or 8. */
typedef struct oscar_layout {
  int32_t head_dim;           /* d */
  int32_t group_size;         /* g: channels per (scale, zero) group */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv */
  int32_t page_tokens;        /* history tokens per page */
  int32_t sink_tokens;        /* BF16 sink tokens */
  int32_t recent_tokens;      /* BF16 recent-window tokens */
  int32_t num_pages;          /* physical pages in the INT2 pool */
  int32_t max_seqs;           /* sequence slots in the BF16 sink / recent arrays */
  int32_t max_pages_per_seq;  /* row stride of the page table */
  int32_t levels_kind;        /* what levels_k / levels_v hold: 0 = (lo, step) of an equally
                                 spaced codebook; 1 = (l0, l1) of a codebook symmetric about 1.5
                                 (see oscar_demote) */
} oscar_layout;

/* Library ABI version (OSCAR_ABI_VERSION of the build). */
uint32_t oscar_abi_version(void);

/* Static description of a status code.  Never NULL. */
const char* oscar_status_string(oscar_status status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* oscar_last_error(void);

/* OSCAR_OK if the layout is supported by the kernels, else OSCAR_ERR_NULL / OSCAR_ERR_SHAPE. */
oscar_status oscar_layout_check(const oscar_layout* layout);

/* Size queries; each returns 0 for an unsupported layout. */
size_t oscar_page_block_bytes(const oscar_layout* layout);   /* one (page, KV head) block */
size_t oscar_page_bytes(const oscar_layout* layout);         /* one page, all KV heads */
size_t oscar_pool_bytes(const oscar_layout* layout);         /* num_pages pages */
size_t oscar_sink_bytes(const oscar_layout* layout);         /* keys or values: one array */
size_t oscar_recent_bytes(const oscar_layout* layout);       /* keys or values: one array */

/* Device workspace oscar_decode_attn needs for `batch` sequences of at most `max_seq_len`
 * tokens (0 for invalid arguments). */
size_t oscar_decode_workspace_bytes(const oscar_layout* layout, int32_t batch,
                                    int32_t max_seq_len);

/* Work plan of oscar_decode_attn for `batch` sequences of at most `max_seq_len` tokens: returns
 * the number of INT2 work items (splits) per (sequence, KV head) and stores the history pages
 * each covers in *pages_per_split (when not NULL); -1 for invalid arguments.  Host only. */
int32_t oscar_decode_splits(const oscar_layout* layout, int32_t batch, int32_t max_seq_len,
                            int32_t* pages_per_split);

/* Host-side check of a host copy of a page table and sequence lengths: every page that a
 * sequence of length seq_lens[b] + extra_tokens uses must be in [0, num_pages), fit in
 * max_pages_per_seq, and no two sequences may share a page beyond the pages they share from
 * position 0 (shared pages must be a common prefix of both rows).  With extra_tokens > 0 (that
 * many decode steps will follow), every page those steps demote into -- history indices
 * [seq_lens[b] - 320, seq_lens[b] + extra_tokens - 320) -- must be used by that sequence alone:
 * a page shared with another sequence must be replaced by a private copy (copy-on-write) before
 * the first write.  Touches no device memory. */
oscar_status oscar_check_page_table(const oscar_layout* layout, const int32_t* host_page_table,
                                    const int32_t* host_seq_lens, int32_t batch,
                                    int32_t extra_tokens);

/* Device workspace oscar_decode_attn_prefix / oscar_decode_step_prefix need for `batch`
 * sequences of at most `max_seq_len` tokens over a shared prefix of `prefix_pages` history pages
 * (0 for invalid arguments).  With prefix_pages 0 it is oscar_decode_workspace_bytes. */
size_t oscar_decode_workspace_bytes_prefix(const oscar_layout* layout, int32_t batch,
                                           int32_t max_seq_len, int32_t prefix_pages);

/* Host-side check of the shared-prefix description oscar_decode_attn_prefix takes, against a host
 * copy of the page table: prefix_ids[0 .. prefix_pages) in [0, num_pages), prefix_pages at most
 * max_pages_per_seq, and for every sequence b, shared_pages[b] in [0, prefix_pages] with
 * page_table[b][j] == prefix_ids[j] for every j < shared_pages[b].  All pointers are host memory
 * (page_table and shared_pages may be NULL when batch is 0).  Touches no device memory.
 * Returns OSCAR_OK, or NULL / SHAPE / RANGE. */
oscar_status oscar_check_shared_prefix(const oscar_layout* layout, const int32_t* host_page_table,
                                       int32_t batch, const int32_t* host_prefix_ids,
                                       const int32_t* host_shared_pages, int32_t prefix_pages);

/* Demotion into the INT2 history ([W1] OSCAR 的设计: the oldest recent tokens are rotated,
 * clipped, quantised and packed into the history; four 2-bit codes per byte).
 *
 * For every sequence b < batch, token i < n_tokens and KV head h, the key vector
 *   k = k_src[b * stride_b + i * stride_t + h * stride_h + (0..d-1)]  (bf16 elements)
 * (and likewise the value vector from v_src) is encoded and written to history index
 * hist_start[b] + i of sequence b:
 *   1. x' = x U H P / sqrt(d) computed in fp64, then rounded to fp32;
 *   2. x'' = min(max(x', -clip), clip)  (fp32);
 *   3. per group m of g rotated channels: mn = min, mx = max, r = (mx - mn) / 3;
 *      scale = fp16(r * step), zero = fp16(mn + r * lo) (fp32 arithmetic, each product and sum
 *      rounded on its own, round-to-nearest-even); (lo, step) = (0, 1), i.e. scale = fp16(r) and
 *      zero = fp16(mn), unless levels_k / levels_v give them;
 *   4. code_j = min(max(rint((x''_j - zero) / scale), 0), 3) in fp32 with ties to even, or 0 for
 *      every j of a group whose fp16 scale is 0;
 *   5. codes and meta are stored in the block layout described above.
 * levels_k / levels_v: NULL for the plain grid (lo, step) = (0, 1), or device fp32 [num_kv_heads][2] =
 * (lo, step) per KV head, 4-byte aligned: an equally spaced codebook whose four levels sit at
 * lo + step * c in units of (mx - mn) / 3 above the group minimum -- the Lloyd-Max codebook that
 * OSCAR's newer code pairs with its rotation ([W3], closing comparison with TurboQuant), held to
 * equal spacing so that decoding stays scale * code + zero and the attention kernels are
 * unchanged.  lo and step must be finite, step > 0 (the library does not read device memory to
 * check); fitted values lie near lo = 0.5, step = 2/3.
 * With layout->levels_kind 1, levels_k / levels_v (then required) hold (l0, l1) per KV head of a
 * Lloyd-Max codebook symmetric about 1.5: steps 3 and 4 become scale = fp16(r), zero = fp16(mn)
 * and code_j = the number of the midpoints (l0 + l1) / 2, 1.5, 3 - (l0 + l1) / 2 (in fp64)
 * strictly below t = (x''_j - zero) / scale (fp32; t = 0 for a zero scale), i.e. the nearest of
 * the levels (l0, l1, 3 - l1, 3 - l0), a value on a midpoint taking the lower code; such a history
 * decodes to scale * level + zero (oscar_decode_attn_codebook).  Requires l0 <= l1 <= 1.5.
 * pool: oscar_pool_bytes(layout) bytes, 16-byte aligned.  page_table: int32
 * [batch][max_pages_per_seq].  U_k / U_v / clip_k / clip_v as described above.  hist_start:
 * int32 [batch].  Strides are in bf16 elements, >= 0; k_src / v_src 2-byte aligned.  The call
 * must not run concurrently with a decode over the same pages (stream order suffices).
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE (negative batch or n_tokens) / HIP. */
oscar_status oscar_demote(const oscar_layout* layout, void* pool, const int32_t* page_table,
                          const float* u_k, const float* u_v, const float* clip_k,
                          const float* clip_v, const float* levels_k, const float* levels_v,
                          const void* k_src, const void* v_src,
                          int64_t stride_b, int64_t stride_t, int64_t stride_h,
                          const int32_t* hist_start, int32_t batch, int32_t n_tokens,
                          void* stream);

/* One decode-step write ([W1] OSCAR 的设计: a new token first enters the recent window; the
 * oldest recent token is then demoted into the history).
 *
 * For each b < batch with P = seq_lens[b] (the length before this token, i.e. its position) and
 * s = seq_slot[b]: if P < 64 the new key / value (k_new / v_new, bf16 [batch][Hkv][d]) go to
 * sink row P of slot s.  Otherwise they go to recent ring row P % 256 of slot s, and when
 * P >= 320 the token held in that row (position P - 256) is first demoted (as oscar_demote) to
 * history index P - 320.  The caller advances seq_lens afterwards.  sink / recent arrays as in
 * the layout above; seq_slot, seq_lens int32 [batch] device arrays; levels_k / levels_v as for
 * oscar_demote.
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / HIP. */
oscar_status oscar_append(const oscar_layout* layout, void* pool, const int32_t* page_table,
                          void* sink_k, void* sink_v, void* recent_k, void* recent_v,
                          const float* u_k, const float* u_v, const float* clip_k,
                          const float* clip_v, const float* levels_k, const float* levels_v,
                          const void* k_new, const void* v_new, const int32_t* seq_slot,
                          const int32_t* seq_lens, int32_t batch, void* stream);

/* Decode attention over the three-segment cache ([W1] OSCAR 的设计: INT2 unpack and
 * scale / zero-point dequantisation with float accumulation, a BF16 sink / recent pass, an
 * online-softmax merge; [P] Abstract: an INT2 attention kernel over a paged KV cache).
 *
 * For each sequence b and query head i (KV head i / (Hq / Hkv)), with L = seq_lens[b]:
 *   out[b][i] = sum_t softmax_t(sm_scale * q[b][i] . k_t) v_t   over the L cached tokens, where
 * history keys / values are k_t = (scale * code + zero) R^T (dequantised in rotated space and
 * mapped back).  The kernels work in the rotated frame: q' = q R_k scores the history directly,
 * the history's value accumulator is mapped back by R_v^T once per head after the split-KV merge.
 * q: bf16 [batch][Hq][d].  out: fp32 [batch][Hq][d].  lse: optional fp32 [batch][Hq] natural-log
 * sum of exp(sm_scale * scores) (NULL to skip).  sm_scale <= 0 selects 1/sqrt(d).
 * seq_lens[b] must be in [1, max_seq_len]; max_seq_len is a host-side bound used for work
 * planning, at most 64 * 256 * 1024 + 320 tokens (RANGE beyond).  workspace: at least
 * oscar_decode_workspace_bytes(layout, batch, max_seq_len) bytes, 256-byte aligned; its contents
 * on entry do not matter.  A layout with levels_kind 1 needs the codebook levels: use
 * oscar_decode_attn_codebook (SHAPE here).
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE / HIP. */
oscar_status oscar_decode_attn(const oscar_layout* layout, const void* pool,
                               const int32_t* page_table, const void* sink_k, const void* sink_v,
                               const void* recent_k, const void* recent_v,
                               const int32_t* seq_slot, const int32_t* seq_lens, const void* q,
                               const float* u_k, const float* u_v, float sm_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               int32_t batch, int32_t max_seq_len, void* stream);

/* Stages of oscar_decode_attn, selectable with a bit mask, for callers that schedule them
 * separately -- for example the BF16 pass on a second stream next to the INT2 pass, or a
 * profiler bracketing one stage with events.  The stages communicate through the workspace:
 * OSCAR_STAGE_QUERY (rotate the queries) must complete before OSCAR_STAGE_INT2; OSCAR_STAGE_INT2
 * and OSCAR_STAGE_BF16 may run in either order or concurrently; OSCAR_STAGE_MERGE needs both.
 * Every call of a sequence of stages must pass the same arguments, workspace and max_seq_len.
 * oscar_decode_attn(...) is oscar_decode_attn_stages(..., OSCAR_STAGE_ALL, ...). */
#define OSCAR_STAGE_QUERY 1u
#define OSCAR_STAGE_INT2  2u
#define OSCAR_STAGE_BF16  4u
#define OSCAR_STAGE_MERGE 8u
#define OSCAR_STAGE_ALL   15u

oscar_status oscar_decode_attn_stages(const oscar_layout* layout, const void* pool,
                                      const int32_t* page_table, const void* sink_k,
                                      const void* sink_v, const void* recent_k,
                                      const void* recent_v, const int32_t* seq_slot,
                                      const int32_t* seq_lens, const void* q, const float* u_k,
                                      const float* u_v, float sm_scale, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, int32_t batch,
                                      int32_t max_seq_len, uint32_t stages, void* stream);

/* oscar_decode_attn_stages over a history encoded with symmetric Lloyd-Max codebooks
 * (layout->levels_kind 1; see oscar_demote): history keys / values are (scale * level_code +
 * zero) R^T with levels (l0, l1, 3 - l1, 3 - l0) from levels_k / levels_v (device fp32
 * [num_kv_heads][2], 4-byte aligned, required) -- the Lloyd-Max codebook of [W3]'s closing
 * comparison with TurboQuant, restricted to levels symmetric about 1.5 so that a level is
 * a + b code + d (code >> 1), two matrix-core contractions of the stored bits.  Supported for up
 * to four query heads per KV head and group_size 128 (SHAPE otherwise).  With levels_kind 0 the
 * levels are ignored and the call is oscar_decode_attn_stages.
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE / HIP. */
oscar_status oscar_decode_attn_codebook(const oscar_layout* layout, const void* pool,
                                        const int32_t* page_table, const void* sink_k,
                                        const void* sink_v, const void* recent_k,
                                        const void* recent_v, const int32_t* seq_slot,
                                        const int32_t* seq_lens, const void* q, const float* u_k,
                                        const float* u_v, const float* levels_k,
                                        const float* levels_v, float sm_scale, float* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        int32_t batch, int32_t max_seq_len, uint32_t stages,
                                        void* stream);

/* oscar_decode_attn_stages for a batch whose sequences share a prefix through the page table
 * ([W1] OSCAR 的设计 and [W3] Fig. 5 / Fig. 6: the paged INT2 pool works with a radix prefix
 * cache, whose hits alias one physical copy of a prefix's pages in many sequences' rows).  The
 * result is that of oscar_decode_attn_stages on the same arguments; only the work differs: the
 * INT2 pass reads each whole chunk of 12 shared pages of a KV head once for a group of 16
 * sequences (a cascade block stages the chunk in LDS and runs every sequence of the group against
 * it), and the split-KV items take each sequence's remaining pages.
 *   prefix_ids    device int32 [prefix_pages]: physical page ids of the shared prefix, in order.
 *   shared_pages  device int32 [batch]: how many leading pages of sequence b's page-table row are
 *                 prefix_ids[0 ..) (0 .. prefix_pages; a short sequence, or one whose prefix
 *                 diverges, shares fewer).  Both arrays 4-byte aligned and trusted like the page
 *                 table; oscar_check_shared_prefix checks host copies.
 *   prefix_pages  0 .. min(num_pages, max_pages_per_seq); 0 (with NULL arrays) is
 *                 oscar_decode_attn_stages.  Pages of the prefix past max_seq_len's history and a
 *                 trailing part of fewer than 12 pages are taken by the split items as usual.
 * workspace: oscar_decode_workspace_bytes_prefix(layout, batch, max_seq_len, prefix_pages) bytes.
 * The cascade runs on layouts with up to four query heads per KV head, group_size 128 and
 * levels_kind 0; other layouts take the split items alone (the same result).  A layout with
 * levels_kind 1 is refused (SHAPE).  The cascade blocks run in the segment launch (stage
 * OSCAR_STAGE_INT2), beside the split items.
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE / HIP. */
oscar_status oscar_decode_attn_prefix(const oscar_layout* layout, const void* pool,
                                      const int32_t* page_table, const void* sink_k,
                                      const void* sink_v, const void* recent_k,
                                      const void* recent_v, const int32_t* seq_slot,
                                      const int32_t* seq_lens, const void* q, const float* u_k,
                                      const float* u_v, const int32_t* prefix_ids,
                                      const int32_t* shared_pages, int32_t prefix_pages,
                                      float sm_scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                                      uint32_t stages, void* stream);

/* One whole decode step of a layer ([W1] OSCAR 的设计: a new token enters the recent window, the
 * token it displaces is demoted into the INT2 history, then attention runs over the three
 * segments): the same result as
 *   oscar_append(..., seq_slot, seq_pos, ...)  followed by
 *   oscar_decode_attn(..., seq_lens = seq_pos + 1, ...)
 * (oscar_decode_attn_codebook with the same levels for a layout with levels_kind 1).
 * With at most four query heads per KV head, one group per vector and levels_kind 0, two
 * launches: the segment launch also rotates the query (in each INT2 block) and appends the token
 * (one BF16 block per (sequence, KV head) demotes the displaced token and signals the one wave
 * that reads its page through a flag word per (sequence, KV head) in the workspace); otherwise
 * three, the append and the query rotation sharing the first.  Both give the same bytes.
 * seq_pos[b] = position of the new token = tokens cached before the step; seq_pos[b] + 1 must be
 * in [1, max_seq_len].  Arguments are those of the two calls, with the same requirements; the
 * workspace must be zero-filled before its first use (every call leaves the flag words zero).
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE / HIP; nothing is launched
 * unless every argument check passes. */
oscar_status oscar_decode_step(const oscar_layout* layout, void* pool, const int32_t* page_table,
                               void* sink_k, void* sink_v, void* recent_k, void* recent_v,
                               const float* u_k, const float* u_v, const float* clip_k,
                               const float* clip_v, const float* levels_k,
                               const float* levels_v, const void* k_new, const void* v_new,
                               const int32_t* seq_slot, const int32_t* seq_pos, const void* q,
                               float sm_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                               void* stream);

/* How many launches oscar_decode_step makes for this layout and shape: 2 when the segment launch
 * appends and rotates the query itself (at most four query heads per KV head, one group per
 * vector, levels_kind 0), else 3; 0 for an invalid layout or shape.  (oscar_decode_step_prefix
 * always makes 3.) */
int32_t oscar_decode_step_launches(const oscar_layout* layout, int32_t batch, int32_t max_seq_len);

/* The launches of oscar_decode_step that `stages` selects (a mask as in oscar_decode_attn_stages):
 * OSCAR_STAGE_QUERY the preparation launch (append + query rotation; nothing when the segment
 * launch does both), OSCAR_STAGE_INT2 | OSCAR_STAGE_BF16 the segment launch (when it appends, the
 * two go together: RANGE otherwise), OSCAR_STAGE_MERGE the merge.  Selected in that order, over
 * calls, they make one step; one launch alone, repeated (to time it), appends again each time.
 * Arguments and results otherwise as oscar_decode_step. */
oscar_status oscar_decode_step_stages(const oscar_layout* layout, void* pool,
                                      const int32_t* page_table, void* sink_k, void* sink_v,
                                      void* recent_k, void* recent_v, const float* u_k,
                                      const float* u_v, const float* clip_k, const float* clip_v,
                                      const float* levels_k, const float* levels_v,
                                      const void* k_new, const void* v_new,
                                      const int32_t* seq_slot, const int32_t* seq_pos,
                                      const void* q, float sm_scale, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, int32_t batch,
                                      int32_t max_seq_len, uint32_t stages, void* stream);

/* oscar_decode_step over a shared prefix: oscar_append followed by oscar_decode_attn_prefix
 * (seq_lens = seq_pos + 1), in three launches (the append and the query rotation share the first).
 * The new tokens' demotions must not land in a shared page (oscar_check_page_table with
 * extra_tokens); a layout with levels_kind 1 is refused (SHAPE).  Arguments
 * are those of oscar_decode_step and oscar_decode_attn_prefix, with the same requirements;
 * workspace: oscar_decode_workspace_bytes_prefix bytes.
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE / HIP. */
oscar_status oscar_decode_step_prefix(const oscar_layout* layout, void* pool,
                                      const int32_t* page_table, void* sink_k, void* sink_v,
                                      void* recent_k, void* recent_v, const float* u_k,
                                      const float* u_v, const float* clip_k, const float* clip_v,
                                      const void* k_new, const void* v_new,
                                      const int32_t* seq_slot, const int32_t* seq_pos,
                                      const void* q, const int32_t* prefix_ids,
                                      const int32_t* shared_pages, int32_t prefix_pages,
                                      float sm_scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                                      void* stream);

/* oscar_decode_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  The same step, with the
 * same arguments minus the workspace: the library takes its workspace from a device array it owns,
 * 16 MiB on each GPU it runs on (held until the process ends, its address looked up on the first
 * call on each device).  Calls whose plan needs more than 16 MiB of workspace (as reported by
 * oscar_decode_workspace_bytes) are rejected with OSCAR_ERR_WORKSPACE before anything is
 * launched.  The call allocates and frees nothing.  Every call on one GPU uses that GPU's one
 * array, zero when the library is loaded; each call writes every byte it reads before reading it,
 * apart from the step's flag words, which it leaves zero: calls that overlap on one GPU -- on
 * different streams without ordering between them, or from several host threads -- race on it
 * and give wrong results.
 * Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE / HIP. */
oscar_status oscar_decode_step_noalloc(const oscar_layout* layout, void* pool,
                                       const int32_t* page_table, void* sink_k, void* sink_v,
                                       void* recent_k, void* recent_v, const float* u_k,
                                       const float* u_v, const float* clip_k, const float* clip_v,
                                       const float* levels_k, const float* levels_v,
                                       const void* k_new, const void* v_new,
                                       const int32_t* seq_slot, const int32_t* seq_pos,
                                       const void* q, float sm_scale, float* out, float* lse,
                                       int32_t batch, int32_t max_seq_len, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Paged BF16 baseline.  The pages report the INT2 history's system gains against a history kept
 * in BF16 ([W1] and its repost, evaluation part: about 8x less KV memory, up to 3x faster
 * batch-1 decoding at 100k context with a full prefix-cache hit, up to 7x throughput at large
 * batch under one memory budget; [P] Abstract: batch-1 decoding up to 3x faster than BF16).  These
 * entry points keep every cached token of a sequence, from position 0, in BF16 pages on the same
 * kind of page table, and compute the same attention without rotation or quantisation.
 *
 * BF16 pool: num_pages pages; pool bytes [page][kv_head][block], block =
 * oscar_bf16_page_block_bytes() = 32,768 bytes for 64 tokens of one KV head, stored as 32 rows
 * of 64 chunks of 16 bytes (8 bf16 elements) in matrix-core operand order:
 *     key   (slot t, channel c): row 16 (t / 32) + 4 ((t / 16) % 2) + c / 32,
 *                                chunk 16 ((c % 32) / 8) + t % 16, element c % 8
 *     value (slot t, channel c): row 16 (t / 32) + 8 + c / 16,
 *                                chunk 16 ((t % 32) / 8) + c % 16, element t % 8
 * (byte offset = 1024 row + 16 chunk + 2 element), so that each row is exactly what one load
 * instruction of a 64-lane wave fetches for its key or value operands.
 * Token at position t of sequence b lives in page page_table[b][t / 64], slot t % 64.  Slots past
 * a sequence's length may hold any bits; the kernels never let them reach a result.
 * Of the layout, these calls use head_dim (128), num_q_heads, num_kv_heads, page_tokens (64),
 * num_pages and max_pages_per_seq; the other fields must still pass oscar_layout_check().
 * --------------------------------------------------------------------------------------------- */

/* Size queries (0 for an unsupported layout). */
size_t oscar_bf16_page_block_bytes(const oscar_layout* layout);   /* one (page, KV head) block */
size_t oscar_bf16_page_bytes(const oscar_layout* layout);         /* one page, all KV heads */
size_t oscar_bf16_pool_bytes(const oscar_layout* layout);         /* num_pages pages */
/* Device workspace oscar_bf16_decode_attn needs (0 for invalid arguments). */
size_t oscar_bf16_decode_workspace_bytes(const oscar_layout* layout, int32_t batch,
                                         int32_t max_seq_len);

/* Writes keys and values into the BF16 pool: for every sequence b < batch, token i < n_tokens
 * and KV head h, k_src[b * stride_b + i * stride_t + h * stride_h + (0..127)] (bf16 elements;
 * likewise v_src) goes to position start_pos[b] + i of sequence b (key row and value column of
 * its slot).  A decode step appends its token with n_tokens = 1 and start_pos = the token's
 * position.  pool: oscar_bf16_pool_bytes(layout) bytes, 16-byte aligned; page_table int32
 * [batch][max_pages_per_seq]; start_pos int32 [batch] (device).  Strides >= 0, in elements.
 * Returns OSCAR_OK, or NULL / ALIGN / RANGE (negative batch, n_tokens or stride) / SHAPE / HIP. */
oscar_status oscar_bf16_store(const oscar_layout* layout, void* pool, const int32_t* page_table,
                              const void* k_src, const void* v_src, int64_t stride_b,
                              int64_t stride_t, int64_t stride_h, const int32_t* start_pos,
                              int32_t batch, int32_t n_tokens, void* stream);

/* Decode attention over the BF16 pool: for each sequence b and query head i (KV head
 * i / (Hq / Hkv)), with L = seq_lens[b] in [1, max_seq_len],
 *   out[b][i] = sum_{t < L} softmax_t(sm_scale * q[b][i] . k_t) v_t.
 * Split-KV over pages (scores and value sums on the bf16 matrix cores with fp32 accumulation;
 * the softmax weights enter the value products as a bf16 hi + lo pair), then a log-sum-exp merge
 * of the splits.  q: bf16 [batch][Hq][128], 16-byte aligned.  out: fp32 [batch][Hq][128].  lse:
 * optional fp32 [batch][Hq] (natural log of sum exp(sm_scale * scores)).  sm_scale <= 0 selects
 * 1/sqrt(128).  max_seq_len: host bound for work planning, at most 64 * 256 * 1024 tokens and
 * 64 * max_pages_per_seq (RANGE beyond).  workspace: at least
 * oscar_bf16_decode_workspace_bytes(layout, batch, max_seq_len) bytes, 256-byte aligned.
 * Two launches on `stream`.  Returns OSCAR_OK, or NULL / SHAPE / ALIGN / RANGE / WORKSPACE /
 * HIP. */
oscar_status oscar_bf16_decode_attn(const oscar_layout* layout, const void* pool,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    const void* q, float sm_scale, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, int32_t batch,
                                    int32_t max_seq_len, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Memory probes.  Not part of the method: plain reads with no arithmetic, for the practical HBM
 * ceilings that the attention kernel's bandwidth is read against (each is timed by the caller,
 * e.g. with events on `stream`).  The sink receives a word only in the case no data produces
 * (it keeps the loads from being optimised away); its contents are unspecified.
 * --------------------------------------------------------------------------------------------- */

/* Streaming read of `bytes` (a multiple of 16) from `buf` (16-byte aligned) with 16-byte
 * non-temporal loads, `blocks` workgroups of 256 threads in a grid-stride loop.  sink: device
 * uint32 array of at least `blocks` words.  Returns OSCAR_OK, or NULL / ALIGN / RANGE / SHAPE /
 * HIP. */
oscar_status oscar_probe_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                              int32_t blocks, void* stream);

/* Reads the INT2 pool's (page, KV head) blocks of the pages page_table_row[0 .. n_pages) (device
 * int32, entries in [0, num_pages)), every KV head, in the decode kernel's order: workgroups of
 * four waves on `pages_per_split` (1..256) consecutive logical pages of one KV head, wave w taking
 * the w-th contiguous quarter of them, its page ids read once before any page, pairs of pages
 * loaded into `sets` (1..4) register sets used in turn -- the next sets' loads in flight while one
 * is consumed -- and `work` (0..2^20) dependency-free fp32 multiply-adds per lane on each pair as
 * it is consumed (a stand-in for the attention arithmetic that sits on each wave's path between
 * one pair's arrival and the next pair's issue).  sink: device uint32 array of at least
 * 4 * ceil(n_pages / pages_per_split) * num_kv_heads words.  Returns OSCAR_OK, or NULL / SHAPE /
 * ALIGN / RANGE / HIP. */
oscar_status oscar_probe_gather(const oscar_layout* layout, const void* pool,
                                const int32_t* page_table_row, int32_t n_pages,
                                int32_t pages_per_split, int32_t sets, int32_t work,
                                uint32_t* sink, size_t sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
