/*
 * oscar.h — C ABI of the MI355X (gfx950) implementation of OSCAR's
 * three-segment 2-bit KV cache: the eviction path (rotate, clip, quantize,
 * pack) and decode attention over the segmented pool.
 *
 * Source of the method: the news article on OSCAR "Beyond TurboQuant:
 * Together AI brings 2-bit KV Cache to real serving" (sanyangsrq.com),
 *   [A] section "OSCAR aims the rotation at attention": the rotation is
 *       R = U . Hadamard . bit-reversal, with R and the clip thresholds fixed
 *       offline per layer and head and reused unchanged at inference;
 *   [B] section "From offline calibration to online inference": the token
 *       pool is BF16 sink (64 tokens) | INT2 history | BF16 recent
 *       (256 tokens); new tokens enter the recent window; the oldest recent
 *       token is rotated, clipped, quantized and packed into the history,
 *       four 2-bit values per byte; decode runs an INT2 kernel (unpack,
 *       scale/zero-point dequantization, float accumulation) and a BF16
 *       kernel over sink and recent, and merges the two with an online
 *       softmax; the layout works with a paged KV cache;
 *   [C] section "Not better vector compression but protecting attention":
 *       2-bit integers have only four levels.
 * Readings where the article is silent (group-wise fp16 scale and zero,
 * per-channel symmetric clipping, row-vector rotation x . R, page size,
 * allocation order) are fixed below and in the design notes.
 *
 * Conventions for every function:
 *   - return 0 on success or a negative OSCAR_E* code; oscar_last_error()
 *     then describes the failure (thread-local, valid until the next call
 *     on the same thread);
 *   - every argument is validated on the host before anything is enqueued;
 *     a failing call changes no host or device state;
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory owned by the caller; the library
 *     never calls hipMalloc and never frees caller memory (its only device
 *     memory of its own is the static workspace of oscar_decode_step_static);
 *   - `stream` is a hipStream_t (NULL = the default stream); device work is
 *     enqueued asynchronously on it unless stated otherwise;
 *   - bf16 and fp16 values are passed as their uint16_t bit patterns;
 *   - a pool is not thread-safe: use it from one thread and one stream at a
 *     time.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_SINK_TOKENS   64   /* [B] BF16 attention sink                       */
#define OSCAR_RECENT_TOKENS 256  /* [B] BF16 recent window                         */
#define OSCAR_PAGE_TOKENS   64   /* history tokens per page of the paged pool     */
#define OSCAR_MAX_BATCH_PER_LAUNCH 256

#define OSCAR_OK       0
#define OSCAR_EHIP    (-5)   /* a HIP runtime call failed                          */
#define OSCAR_ENOMEM  (-12)  /* the pool has too few free pages                    */
#define OSCAR_EINVAL  (-22)  /* invalid argument or shape                          */
#define OSCAR_ERANGE  (-34)  /* a sequence would exceed max_pages_per_seq pages    */

/* Pool flag: keep only the host bookkeeping (lengths, page tables, free
 * list); never touch device memory.  For capacity planning and for testing
 * the host logic without a GPU.  Decode and export then fail with EINVAL. */
#define OSCAR_POOL_HOST_ONLY 1u

/* Pool flag: decode results are bitwise reproducible from call to call and
 * independent of where pages sit in the pool.  By default the waves of a
 * decode block hand history pages out among themselves as they finish them,
 * which balances their progress but lets the summation order and the fp16
 * rounding of the softmax weights vary between calls; with this flag each
 * wave takes a fixed set of pages.  Either mode computes the same attention
 * within the kernel's rounding (relative differences of order 1e-4). */
#define OSCAR_POOL_DETERMINISTIC 2u

/* Pool flag: keep the history in BF16 instead of INT2: the oldest recent
 * token is copied into its page as it is (no rotation, clipping or
 * quantization), everything else (sink, recent window, pages, allocator,
 * merge) as in the INT2 pool.  The baseline the 2-bit history is measured
 * against ([N-results]: ~3x faster decode than BF16 at 100K context,
 * batch 1).  Decode and append work as for INT2 pools (a step runs the
 * append in its own launch); prefill attention and the code exports are
 * INT2 only (EINVAL); oscar_export_history_bf16 exports the history. */
#define OSCAR_POOL_BF16_HISTORY 4u

/* Pool flag: the Lloyd-Max codebook variant ([A]; the news article's
 * section "Why this matters for long-context agents": the OSCAR code pairs
 * the attention-aware rotation with a Lloyd-Max codebook).  A history group
 * keeps its fp16 scale s and zero point z; its four levels are
 * z + (L_k / 64) s for a per-(kv head, K|V) codebook L_0 <= .. <= L_3 of
 * bytes set by oscar_pool_set_codebook (fitted offline by
 * oscar_lloyd_max_codebook) instead of z + k s, and a channel takes the
 * nearest level: u = (y - z) / s (fp32) against the midpoints
 * t_k = (L_k + L_{k+1}) / 128, a value on a midpoint taking the lower level;
 * s = 0 gives code 0.  Layout, allocator, exports, decode, step and prefill
 * attention are the INT2 pool's (the kernels read levels instead of codes).
 * Excludes OSCAR_POOL_BF16_HISTORY. */
#define OSCAR_POOL_LLOYD_MAX 8u

typedef struct oscar_pool oscar_pool;  /* opaque, host side */

typedef struct oscar_pool_config {
    int32_t  max_seqs;          /* sequence ids are 0 .. max_seqs-1                  */
    int32_t  num_q_heads;       /* Hq                                                */
    int32_t  num_kv_heads;      /* Hkv, Hq % Hkv == 0, Hq / Hkv <= 16                */
    int32_t  head_dim;          /* d: 64 or 128                                      */
    int32_t  group_size;        /* G: 64 or 128 channels per scale/zero, G <= d      */
    int32_t  num_pages;         /* history pages in the pool (>= 0)                  */
    int32_t  max_pages_per_seq; /* page-table width                                  */
    uint32_t flags;             /* OR of OSCAR_POOL_* flags                          */
    uint64_t page_shuffle_seed; /* seeds the free-list order                         */
} oscar_pool_config;

/* Bytes of device memory a pool with this configuration needs (its layout:
 * rotation and clip tables, page table, sink and recent windows for every
 * sequence slot, and num_pages history pages).  Host only. */
int oscar_pool_bytes(const oscar_pool_config *cfg, size_t *device_bytes);

/* Both sizes a pool needs, in one call: *device_bytes as oscar_pool_bytes,
 * *workspace_bytes as oscar_decode_workspace_bytes for a batch of
 * min(max_seqs, OSCAR_MAX_BATCH_PER_LAUNCH) sequences (a workspace of that
 * size serves every decode call, which is cut into launches of at most that
 * many).  Host only; allocates nothing.  Errors: EINVAL. */
int oscar_pool_required_bytes(const oscar_pool_config *cfg, size_t *device_bytes,
                              size_t *workspace_bytes);

/* Bytes of device workspace oscar_decode_attn needs for batches of up to
 * max_batch sequences.  Host only. */
int oscar_decode_workspace_bytes(const oscar_pool_config *cfg, int32_t max_batch,
                                 size_t *bytes);

/* Create a pool in caller-owned device memory `device_buf` (at least
 * oscar_pool_bytes bytes, 256-byte aligned).
 *   R_K, R_V:      host fp32 [Hkv][d][d], row-major; a token x (row vector)
 *                  is stored rotated as x . R ([A]);
 *   clip_K, clip_V host fp32 [Hkv][d]; rotated channel j of head h is clipped
 *                  to [-clip[h][j], clip[h][j]] before quantization ([A], [B]).
 *                  Every threshold must be finite, > 0 and small enough that
 *                  fp16(2 c / 3) is finite (the largest possible scale).
 * The tables are copied into the pool (the call waits for the copy); the
 * host arrays may be freed on return.  The free list is a Fisher-Yates
 * shuffle of the page ids driven by SplitMix64(page_shuffle_seed); pages are
 * handed out from its front.  With OSCAR_POOL_HOST_ONLY, device_buf, the
 * tables and the stream are ignored (they may be NULL).
 * Errors: EINVAL (shapes, null pointers, bad thresholds, buffer too small),
 * EHIP. */
int oscar_pool_create(const oscar_pool_config *cfg, void *device_buf, size_t bytes,
                      const float *R_K, const float *R_V,
                      const float *clip_K, const float *clip_V,
                      void *stream, oscar_pool **out);

/* Destroy the host side of a pool (the device buffer stays the caller's). */
int oscar_pool_destroy(oscar_pool *pool);

/* Fill an empty sequence with a prompt of L tokens ([B]): positions
 * 0..min(L,64)-1 go to the sink, the last min(L-64, 256) positions to the
 * recent window, and the n_hist = max(0, L-320) positions in between are
 * encoded into ceil(n_hist/64) history pages taken from the free list in
 * history order.  k, v: device bf16 [L][Hkv][d].  Inputs may be released
 * once the stream has passed this call.
 * Errors: EINVAL (bad seq, sequence not empty, L < 0, null), ENOMEM, ERANGE. */
int oscar_prefill(oscar_pool *pool, int32_t seq, const uint16_t *k,
                  const uint16_t *v, int32_t L, void *stream);

/* Append one token to each listed sequence ([B]).  For a sequence of length
 * L before the call the token at position L goes to the sink (L < 64) or to
 * recent slot (L-64) mod 256 (L >= 64).  When the recent window is full
 * (L >= 320), the oldest recent token (position 64 + n_hist, n_hist = L-320,
 * held in that same slot) is first rotated, clipped, quantized and packed
 * into history index n_hist (page n_hist/64, slot n_hist%64); a new page is
 * taken from the free list when n_hist % 64 == 0, and also when slot
 * n_hist%64 lies in a page that another sequence also holds (after
 * oscar_fork_seq): then the page is first copied into the new one, which
 * replaces it in this sequence's table (copy on write).  Sequences are
 * served in the order of seq_ids, each seeing the references the earlier
 * ones dropped.
 *   seq_ids: host int32 [n], distinct;  k_new, v_new: device bf16 [n][Hkv][d].
 * Errors: EINVAL (n < 0, bad or repeated id, null), ENOMEM, ERANGE. */
int oscar_append_evict(oscar_pool *pool, const int32_t *seq_ids, int32_t n,
                       const uint16_t *k_new, const uint16_t *v_new, void *stream);

/* Decode attention for one new query per listed sequence ([B]).  For query
 * head h (kv head h / (Hq/Hkv)) the result is softmax attention with scale
 * `softmax_scale` over every token of the sequence: sink and recent tokens
 * as stored (bf16), history tokens as decoded, i.e. dequantized with their
 * group scale and zero point and mapped back by R_V^T / R_K^T.  Internally
 * the history is attended in the rotated basis (q . R_K, then acc . R_V^T),
 * split over pages, and merged with the window by an online softmax (by a
 * merge kernel when some pair of a launch is split over several blocks, else
 * inside each pair's block).
 *   seq_ids: host int32 [n] (every sequence non-empty);
 *   q:       device bf16 [n][Hq][d];   out: device fp32 [n][Hq][d];
 *   workspace: device, >= oscar_decode_workspace_bytes(cfg, n) bytes.
 * Errors: EINVAL (bad id, empty sequence, workspace too small, null,
 * host-only pool), EHIP. */
int oscar_decode_attn(oscar_pool *pool, const int32_t *seq_ids, int32_t n,
                      const uint16_t *q, float *out, float softmax_scale,
                      void *workspace, size_t workspace_bytes, void *stream);

/* One decode step in one call: the append of oscar_append_evict(seq_ids,
 * k_new, v_new) followed by the attention of oscar_decode_attn(seq_ids, q,
 * out), the serving loop's per-token pair ([N-pipeline]: the newest token
 * enters the recent window, the oldest recent token moves into the INT2
 * history, then the query attends over all three segments).  The pool ends
 * in the same state bit for bit as after the two calls (same pages taken,
 * in seq_ids order), and out holds the same attention within the kernels'
 * rounding.  The append runs inside the decode launch: the block of each
 * (sequence, kv head) that holds its window also writes the new token and
 * packs the evicted one, ahead of reading them.
 *   seq_ids: host int32 [n], distinct;  k_new, v_new: device bf16 [n][Hkv][d];
 *   q: device bf16 [n][Hq][d];  out: device fp32 [n][Hq][d];
 *   workspace: device, >= oscar_decode_workspace_bytes(cfg, n) bytes.
 * Errors: every error of the two calls, reported before anything changes
 * (EINVAL, ENOMEM, ERANGE), and EHIP. */
int oscar_decode_step(oscar_pool *pool, const int32_t *seq_ids, int32_t n,
                      const uint16_t *k_new, const uint16_t *v_new,
                      const uint16_t *q, float *out, float softmax_scale,
                      void *workspace, size_t workspace_bytes, void *stream);

/* oscar_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, with the decode partials in the library's
 * static workspace instead of a caller workspace.  That workspace is one
 * 32 MiB device array per GPU the library runs on, held until the process
 * ends; its address is looked up when a pool is created on the device (or
 * at the first such call on another device).  The call allocates nothing.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams at once) race and give undefined results; calls on
 * one stream are ordered.
 *   Arguments as oscar_decode_step, without workspace.
 * Errors: those of oscar_decode_step; EINVAL when the step's workspace
 * (what oscar_decode_workspace_bytes would require for its plan) exceeds
 * 32 MiB, before anything changes; EHIP. */
int oscar_decode_step_static(oscar_pool *pool, const int32_t *seq_ids, int32_t n,
                             const uint16_t *k_new, const uint16_t *v_new,
                             const uint16_t *q, float *out, float softmax_scale,
                             void *stream);

/* Wait for `stream` and report whether every decode step so far ran as
 * specified.  Inside a decode launch some waves wait, bounded, for other
 * waves of their block (the window waits for the appended token's slot, the
 * pair's last page for the evicted token's codes, the de-rotation table for
 * the append to finish with the rotation table).  A wait that reaches its
 * bound gives up rather than hang, which leaves that step's attention, and
 * possibly the evicted token's codes, undefined; it sets a sticky flag in
 * the pool's device status word.  The bound is 2^22 polls (seconds), or the
 * value of the environment variable OSCAR_WAIT_SPIN_LIMIT when the pool was
 * created (0 gives up at once: a test hook).  oscar_export_history,
 * oscar_export_window and oscar_profile_end check the flag too.
 * Errors: EINVAL (NULL), EHIP (a wait gave up, or a HIP call failed).
 * Host-only pools always pass. */
int oscar_pool_check(oscar_pool *pool, void *stream);

/* Bytes of device workspace oscar_prefill_attn needs for n_q queries.
 * Host only.  Errors: EINVAL. */
int oscar_prefill_workspace_bytes(const oscar_pool_config *cfg, int32_t n_q, size_t *bytes);

/* Prefill attention over the three-segment pool ([B]: the step before
 * decode; the prompt, or one chunk of it, attends over everything before
 * it).  The sequence holds L tokens; the n_q queries are those of its last
 * n_q positions, query i at position p = L - n_q + i, and each attends with
 * softmax (scale `softmax_scale`) to positions 0..p of the pool as it
 * stands: sink and recent tokens as stored (bf16), history tokens as
 * decoded (dequantized with their group scale and zero point and mapped
 * back by R^T), exactly the tokens decode attention would see at length
 * p + 1.  A chunked prefill appends a chunk (oscar_prefill for an empty
 * sequence, oscar_append_evict otherwise) and then calls this with the
 * chunk's queries.
 *   q:   device bf16 [n_q][Hq][d];   out: device fp32 [n_q][Hq][d];
 *   workspace: device, >= oscar_prefill_workspace_bytes(cfg, n_q) bytes.
 * The (query, head) rows of each kv head are cut in tiles of 128 rows
 * (every INT2 pool shape, affine or Lloyd-Max levels: query preparation,
 * history and finish launches on the matrix cores); each row is masked
 * past its own query's position.
 * Errors: EINVAL (bad seq, n_q outside [1, min(L, 65535)], NULL, workspace
 * too small, host-only pool), EHIP. */
int oscar_prefill_attn(oscar_pool *pool, int32_t seq, int32_t n_q, const uint16_t *q,
                       float *out, float softmax_scale, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Drop a sequence's references to its pages and set its length to 0; the
 * pages no other sequence holds go to the back of the free list, in
 * page-table order.  Host only.  Errors: EINVAL. */
int oscar_release_seq(oscar_pool *pool, int32_t seq);

/* Prefix sharing, read from OSCAR's serving integration (the paged pool
 * works with a radix prefix cache; news article on OSCAR, section "From
 * offline calibration to online inference").  Give the empty sequence dst
 * the whole state of sequence src: the same length, a copy of its sink and
 * recent window, and its history pages, shared (each page counts the
 * sequences that hold it).  Both sequences then decode and grow on their
 * own: only a history's last page is ever written again, and oscar_append_evict
 * / oscar_decode_step copy it first while it is shared.  A fork of an empty
 * src leaves dst empty.  The copy is enqueued on `stream` after src's
 * earlier work there; no page is taken.
 * Errors: EINVAL (bad id, src == dst, dst not empty), EHIP. */
int oscar_fork_seq(oscar_pool *pool, int32_t src, int32_t dst, void *stream);

/* Lloyd-Max pools: set the codebook, levels_k and levels_v host uint8
 * [Hkv][4] (each row non-decreasing), while every sequence is empty; the
 * pool refuses prefill and appends until it is set.  Synchronous on
 * `stream`.  Errors: EINVAL (not such a pool, order, a non-empty sequence,
 * null), EHIP. */
int oscar_pool_set_codebook(oscar_pool *pool, const uint8_t *levels_k, const uint8_t *levels_v,
                            void *stream);

/* Current length of a sequence (host mirror).  Errors: EINVAL. */
int oscar_seq_length(const oscar_pool *pool, int32_t seq, int32_t *L);

/* Copy a sequence's page-table row (host mirror) into pages[capacity];
 * *n_pages receives its length.  Errors: EINVAL (capacity too small). */
int oscar_page_table(const oscar_pool *pool, int32_t seq, int32_t *pages,
                     int32_t capacity, int32_t *n_pages);

/* Number of pages currently on the free list.  Errors: EINVAL. */
int oscar_free_pages(const oscar_pool *pool, int32_t *n_free);

/* Copy history entries [first, first+count) of a sequence to host memory in
 * a canonical layout independent of the physical pages:
 *   codes:  uint8 [count][Hkv][2 (K,V)][d/4], four consecutive channels per
 *           byte, first channel in the low bits;
 *   params: uint16 [count][Hkv][2 (K,V)][d/G][2 (scale, zero)] fp16 bits.
 * Synchronous: waits for `stream`.  Errors: EINVAL (range, host-only), EHIP
 * (also when a bounded wait of a decode step gave up, see oscar_pool_check). */
int oscar_export_history(oscar_pool *pool, int32_t seq, int32_t first, int32_t count,
                         uint8_t *codes, uint16_t *params, void *stream);

/* A sequence's whole state in the canonical layout, without a host copy of
 * the pages: its page-table row (host mirror) into page_table_host
 * [max_pages_per_seq] (entries past the row set to -1), and, enqueued on
 * `stream`, its n_hist = max(0, L - 320) history entries into
 *   codes_dev:  device uint8 [n_hist][Hkv][2 (K,V)][d/4], four consecutive
 *               channels per byte, the first in the low bits;
 *   params_dev: device uint16 [n_hist][Hkv][2 (K,V)][d/G][2 (scale, zero)],
 *               fp16 bits
 * ([B]: the paged history, independent of where its pages sit).  Both
 * buffers caller-owned, 4-byte aligned (may be NULL when n_hist = 0).
 * Errors: EINVAL (bad seq, host-only pool, NULL or misaligned buffers), EHIP. */
int oscar_export_state(oscar_pool *pool, int32_t seq, int32_t *page_table_host,
                       void *codes_dev, void *params_dev, void *stream);

/* BF16-history pools: history entries [first, first+count) of a sequence
 * to host memory, k and v bf16 [count][Hkv][d].  Synchronous.
 * Errors: EINVAL (range, not a device BF16-history pool), EHIP. */
int oscar_export_history_bf16(oscar_pool *pool, int32_t seq, int32_t first, int32_t count,
                              uint16_t *k, uint16_t *v, void *stream);

/* Copy a sequence's BF16 windows to host memory: sink_k/sink_v
 * [64][Hkv][d] (slot = position) and recent_k/recent_v [256][Hkv][d]
 * (slot = (position - 64) mod 256); slots not holding a token are copied as
 * they are.  Synchronous.  Errors: EINVAL, EHIP (as oscar_export_history). */
int oscar_export_window(oscar_pool *pool, int32_t seq, uint16_t *sink_k,
                        uint16_t *sink_v, uint16_t *recent_k, uint16_t *recent_v,
                        void *stream);

/* Offline: R = U . H . Pi ([A]) for one head, host fp32 U[d][d] -> R[d][d].
 * H is the Sylvester-ordered Hadamard matrix scaled by 1/sqrt(d), Pi the
 * bit-reversal permutation (Pi[i][j] = 1 iff j = bitrev(i)).  U . H_unscaled
 * is formed with a fast Walsh-Hadamard transform in fp64 (exact when U lies
 * on a fixed-point grid), divided by sqrt(d) in fp64 and rounded to fp32.
 * d must be a power of two <= 1024.  Errors: EINVAL. */
int oscar_build_rotation(int32_t d, const float *U, float *R);

/* Offline: per-channel clip thresholds for one head:
 * clip[j] = percentile(|(x R)[j]|, pct) over n host bf16 tokens x[n][d],
 * with (x R) evaluated exactly as the eviction does (fp32 FMA chain) and
 * the percentile interpolated linearly between order statistics in fp64:
 * h = (n-1) pct/100, k = floor(h), a[k] + (h-k)(a[k+1]-a[k]).
 * Errors: EINVAL. */
int oscar_calibrate_clip(int32_t d, int64_t n, const uint16_t *x, const float *R,
                         double pct, float *clip);

/* Offline: the Lloyd-Max codebook of one head ([A]) from n host bf16
 * calibration tokens x[n][d], its rotation R[d][d] and clip thresholds
 * clip[d], group size G: the normalised values u = (y - z) / s of every
 * channel of a group with s != 0 (rotation, clip, fp16 s and z exactly as
 * the eviction computes them), taken on the grid of 2^-20; Lloyd's
 * algorithm for `iters` iterations from the levels 0, 1, 2, 3 (cells split
 * at the midpoints, a value on a midpoint in the lower cell; each level
 * moves to its cell's mean, exact integer sums, fp64 division; an empty
 * cell keeps its level); levels[k] = rint(64 level_k) clamped to 0..255.
 * Errors: EINVAL. */
int oscar_lloyd_max_codebook(int32_t d, int32_t G, int64_t n, const uint16_t *x, const float *R,
                             const float *clip, int32_t iters, uint8_t *levels);

/* Offline calibration statistics ([A]; the news article's section "OSCAR
 * aims the rotation at attention": the K rotation follows the query
 * covariance Q^T Q, the V rotation the score-weighted value covariance
 * V^T S^T S V, per layer and head, from a few calibration samples).
 * Inputs are one calibration sequence of n tokens of one layer:
 *   q: device bf16 [n][Hq][d] (2-byte aligned);  k: device bf16 [n][Hkv][d]
 *   (16-byte aligned);  v: device bf16 [n][Hkv][d] (4-byte aligned);
 *   d = 64 or 128; Hq a multiple of Hkv; query head h uses kv head h/(Hq/Hkv).
 * S is the causal attention of the sequence: row t is the softmax of
 * softmax_scale q_t . k_j over j <= t.
 *
 * oscar_calib_attention: out = S V per query head, device fp32 [n][Hq][d]
 * (the attention output; V^T S^T S V = out^T out).
 * oscar_calib_covariance: for each kv head h, ADDS to cov_k[h] the sum over
 * its query heads of Q^T Q and to cov_v[h] the sum of (S V)^T (S V); cov_k,
 * cov_v: device fp32 [Hkv][d][d] (the caller zeroes them before the first
 * sequence; several sequences accumulate).  Products and sums in fp32 (the
 * Gram matrices on matrix cores).  workspace: device, >=
 * oscar_calib_workspace_bytes(n, Hq, d) bytes (it receives S V).
 * n = 0 does nothing.  Errors: EINVAL (shape, alignment, null, workspace too
 * small, scale not finite), EHIP. */
int oscar_calib_workspace_bytes(int32_t n, int32_t num_q_heads, int32_t head_dim, size_t *bytes);
int oscar_calib_attention(int32_t n, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          const uint16_t *q, const uint16_t *k, const uint16_t *v, float softmax_scale,
                          float *out, void *stream);
int oscar_calib_covariance(int32_t n, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v, float softmax_scale,
                           float *cov_k, float *cov_v, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Offline: the rotation of one head from its covariance ([A]): U is the
 * eigenbasis of the symmetric host fp32 cov[d][d] (symmetrised as
 * (C + C^T)/2 in fp64; cyclic Jacobi in fp64): column c is the eigenvector
 * of the c-th largest eigenvalue, signed so that its first entry of largest
 * magnitude is positive, rounded to fp32 and then to the nearest multiple
 * of 2^-40.  R = U . H . Pi as oscar_build_rotation.  Outputs (host): R
 * [d][d] fp32; U [d][d] fp32 and eigenvalues [d] fp64 (descending), each
 * optional (NULL).  d a power of two <= 1024.  Errors: EINVAL (d, null,
 * non-finite entry). */
int oscar_calib_rotation(int32_t d, const float *cov, float *U, float *R, double *eigenvalues);

/* Kernel timing with HIP events recorded on the launch stream around the
 * kernels selected by `kernels` (OSCAR_PROFILE_* bits) in the pool's decode
 * and append calls.  oscar_profile_begin creates event pairs for up to
 * max_calls timed launches of each selected kernel: launches 0, every,
 * 2 every, ... of each kernel are timed (every >= 1), later ones and the
 * rest go untimed.  oscar_profile_end waits for the events, writes the
 * number of timed launches and their summed durations (milliseconds), and
 * releases the events.  The events carry no system-scope fence (timing
 * only).  Each timed launch still starts a few microseconds after the
 * kernel before it, and the interval counts that gap, so time only the
 * kernels of interest, or a sample of their launches.  oscar_profile_end
 * waits for the device and checks the pool status (oscar_pool_check).
 * Errors: EINVAL, EHIP. */
typedef struct oscar_profile {
    int32_t n_decode_main;   float ms_decode_main;   /* query prep, INT2 history, BF16 window */
    int32_t n_decode_merge;  float ms_decode_merge;  /* merge of the partials (launches with a
                                                         split pair; none otherwise)         */
    int32_t n_append;        float ms_append;        /* append / eviction                     */
} oscar_profile;

#define OSCAR_PROFILE_DECODE_MAIN  1u  /* main decode kernel               */
#define OSCAR_PROFILE_DECODE_MERGE 2u  /* merge kernel                     */
#define OSCAR_PROFILE_APPEND       4u  /* append / eviction kernel         */

int oscar_profile_begin(oscar_pool *pool, int32_t max_calls, uint32_t kernels, int32_t every);
int oscar_profile_end(oscar_pool *pool, oscar_profile *out);

const char *oscar_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OSCAR_H */
