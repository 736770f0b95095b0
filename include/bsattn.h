/*
 * bsattn.h — block-sparse FlashAttention forward for AMD MI355X (gfx950).
 *
 * Plain C ABI.  Every tensor argument is a caller-owned, contiguous, row-major
 * DEVICE buffer; bfloat16 tensors are passed as their uint16 bit patterns.
 * The library never allocates device memory (its one static array, the
 * scratch of bsattn_decode_gqa_noalloc, is part of the loaded code object)
 * and never synchronises the host: each call only enqueues kernels on `stream` (a hipStream_t; NULL =
 * the default stream) — kernel launches only, no memset or copy, so calls can
 * be captured into a HIP graph and replayed.  Outputs are valid once the stream reaches the end of
 * the call.  Equal inputs give bitwise equal outputs (no atomics on any
 * value path).
 *
 * Host state: the only state kept between calls is per device and
 * write-once in effect — the device's compute-unit count (read on first use,
 * for the default decode split count and the forward's launch shape), the
 * largest dynamic-LDS size each kernel has been granted, and the address of
 * the static scratch array of bsattn_decode_gqa_noalloc.  All are atomics,
 * so the library is safe to call from several host threads (that scratch
 * array itself is shared: see bsattn_decode_gqa_noalloc).
 *
 * Errors: all argument checks run on the host BEFORE any launch.  On an
 * error nothing is enqueued and no output is touched.  A launch failure
 * reported by the HIP runtime returns BSATTN_ERR_HIP.  Data content is never
 * an error: a nonzero mask byte means "selected", a block index outside the
 * valid range selects nothing; non-finite scores give unspecified masks.
 * Only the keys and values of selected blocks (and, in decode, of rows
 * before each sequence's end) are read: anything, NaN included, may sit in
 * the rest.  What is read must be finite; a NaN or infinity there gives
 * unspecified outputs.
 *
 * The block size is fixed at 64 tokens (BSATTN_BLOCK) for both the query and
 * the key/value dimension, as in the TileLang block-sparse Flash-Attention
 * guide (§4.1: block_M = block_N = 64, equal to the mask's downsampling
 * block).
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSATTN_BLOCK 64

typedef struct ihipStream_t* bsattn_stream_t; /* same type as hipStream_t */

typedef enum bsattn_status {
  BSATTN_OK = 0,
  BSATTN_ERR_NULL = 1,        /* a required pointer is NULL                         */
  BSATTN_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree          */
  BSATTN_ERR_UNSUPPORTED = 3, /* valid but not built (head dim, group size)        */
  BSATTN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required        */
  BSATTN_ERR_HIP = 5          /* the HIP runtime reported an error at launch time  */
} bsattn_status;

/* Static text for a status code (never NULL). */
const char* bsattn_status_string(bsattn_status s);

/* Library version as "major.minor.patch". */
const char* bsattn_version(void);

/* ------------------------------------------------------------------------ */
/* Block masks                                                               */
/* ------------------------------------------------------------------------ */

/*
 * Top-k block mask (TileLang block-sparse Flash-Attention guide, §3.1).
 *   scores : float32 [B, H, nb, nb], block importance scores; row i holds the
 *            scores of key blocks 0..nb-1 for query block i.
 *   mask   : uint8   [B, H, nb, nb], written with 0/1.
 * Per row, the `topk` highest scores over the WHOLE row are selected (ties go
 * to the lower column index).  Then, if dense_last_two_rows, rows nb-2 and
 * nb-1 are set all ones (before the causal cut, as in the guide's builder);
 * then every column j > i is cleared (tril); then, if force_diagonal, the
 * diagonal block is set (the causal diagonal block is always kept in the
 * XAttention guide, "algorithm flow", phase 3).
 * Errors: NULL pointers; B, H, nb <= 0, topk < 0 or topk > nb, or more than
 * 2^31 - 1 rows B*H*nb (SHAPE).
 */
bsattn_status bsattn_build_mask_topk(const float* scores, int B, int H, int nb, int topk,
                                     int dense_last_two_rows, int force_diagonal, uint8_t* mask,
                                     bsattn_stream_t stream);

/*
 * Threshold block mask (same guide, §3.2): a block is selected when its score
 * is strictly greater than `threshold`; then the same dense-last-two-rows,
 * tril and diagonal steps as bsattn_build_mask_topk.
 * Errors: NULL pointers; B, H, nb <= 0 or more than 2^31 - 1 rows B*H*nb
 * (SHAPE).
 */
bsattn_status bsattn_build_mask_threshold(const float* scores, int B, int H, int nb,
                                          float threshold, int dense_last_two_rows,
                                          int force_diagonal, uint8_t* mask,
                                          bsattn_stream_t stream);

/*
 * Compaction of a block mask into per-row active-block lists: the list form
 * of the causal loop bound and the block-skip branch of the same guide, §4.4.
 *   mask : uint8 [B, H, nb, nb], nonzero = selected.
 *   idx  : int32 [B, H, nb, nb]; row (b,h,i) lists ascending every j with
 *          mask != 0 (and j <= i when is_causal), then -1 padding.
 *   cnt  : int32 [B, H, nb], the list lengths.
 * Errors: NULL pointers; B, H, nb <= 0, or more rows B*H*nb than one launch
 * covers (four rows per work-group, at most 2^31 - 1 work-groups) (SHAPE).
 */
bsattn_status bsattn_mask_to_indices(const uint8_t* mask, int B, int H, int nb, int is_causal,
                                     int32_t* idx, int32_t* cnt, bsattn_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Prefill                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * Block-sparse attention forward (same guide, §4: the block-sparse
 * Flash-Attention kernel; §5: its reference check).
 *   q, k, v, out : bfloat16 [B, H, S, D] (K/V heads = query heads).
 *   block_mask   : uint8 [B, H, nb, nb] with nb = ceil(S / 64); nonzero =
 *                  query block i attends to key block j.
 * For query row r the visible keys are the tokens t < S of the selected key
 * blocks, with t <= r when is_causal; out[r] = softmax(q_r . k_t / sqrt(D)) V
 * over those keys (fp32 accumulation, probabilities rounded to bfloat16
 * before the P.V product, output rounded to nearest even).  A row that sees
 * no key is written as zeros.  Each query block's mask row is compacted on
 * the device into its ascending active-block list before the block loop.
 * With is_causal, a query block whose list holds more than 128 key blocks
 * is split in two: a second work-group takes the second half of its list,
 * both halves leave fp32 rows and their (row max, row sum) in the workspace,
 * and a merge launch writes the row as the log-sum-exp weighted mean of the
 * halves (the combination of the split-KV decode, same guide, §6.2), so no
 * row runs far longer than the rest.  A split row agrees with the unsplit
 * pass within the output tolerance, not bit for bit: each half rounds its
 * probabilities to bfloat16 against its own running exponent offset.
 * workspace: device memory of bsattn_fwd_workspace_bytes bytes, 16-byte
 * aligned, used by causal calls only (may be NULL when that size is 0);
 * calls that overlap in time need workspaces of their own.
 * Errors: NULL pointers; B, H, S <= 0 (SHAPE); D not 64 or 128, or
 * ceil(S/64) above bsattn_fwd_max_key_blocks(D) (UNSUPPORTED); workspace
 * NULL, misaligned or below bsattn_fwd_workspace_bytes (WORKSPACE).
 */
/* Workspace of bsattn_fwd (and of the fused bsattn_fwd_topk and
 * bsattn_fwd_threshold): nonzero when S spans more than 128 key blocks
 * (B * H * (nb - 128) query blocks can split, each needing two fp32
 * [64, D] halves, 2 x 64 (row max, row sum) pairs and a flag, every part
 * 256-byte aligned); 0 when no row can split, when the split would need more
 * than 2 GiB (such calls then run unsplit), or for arguments out of range. */
size_t bsattn_fwd_workspace_bytes(int B, int H, int S, int D);

/* The most key blocks (ceil(Sk/64)) a forward call takes at head dim D: each
 * work item holds its ascending active-block list in on-chip memory beside
 * its K/V tiles, 2 bytes per block.  0 for a head dim the forward does not
 * take.  Every forward form (bsattn_fwd, _indices, _chunk, _topk,
 * _threshold) returns UNSUPPORTED above it. */
int bsattn_fwd_max_key_blocks(int D);

bsattn_status bsattn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint8_t* block_mask, int B, int H, int S, int D, int is_causal,
                         uint16_t* out, void* workspace, size_t workspace_bytes,
                         bsattn_stream_t stream);

/*
 * The same forward pass driven by precomputed lists (the output of
 * bsattn_mask_to_indices with the same is_causal): idx int32 [B, H, nb, nb]
 * and cnt int32 [B, H, nb].  List entries outside [0, nb) are skipped, and
 * with is_causal entries above the diagonal are skipped.  For callers that
 * reuse one mask across many calls.  Errors as bsattn_fwd.
 */
bsattn_status bsattn_fwd_indices(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* idx, const int32_t* cnt, int B, int H, int S,
                                 int D, int is_causal, uint16_t* out, bsattn_stream_t stream);

/*
 * The whole prefill hot path in one launch: each work item selects its
 * query block's row from the fp32 block scores [B, H, nb, nb] exactly as
 * bsattn_build_mask_topk / bsattn_build_mask_threshold do (guide §3.1 / §3.2:
 * top-k with ties to the lower column, or score > threshold; optional dense
 * last two rows; tril; forced diagonal), writes that row to mask_out when
 * mask_out is not NULL (uint8 0/1 [B, H, nb, nb], byte-identical to the
 * builders' output), compacts it, and runs the forward pass of bsattn_fwd on
 * it.  Long causal rows split as in bsattn_fwd (both work-groups of a split
 * row select the same row; only the first writes it to mask_out), so the
 * output is bit-identical to bsattn_fwd on that mask and workspace layout.
 * q/k/v/out, is_causal, workspace and workspace_bytes as bsattn_fwd (the
 * size is bsattn_fwd_workspace_bytes; NULL when it is 0 or is_causal is 0).
 * With nb > 256 (S > 16384) a row's keys no longer fit the registers the
 * one-launch form holds them in: the call then runs as two launches, the
 * builder writing mask_out and bsattn_fwd reading it, with the same mask
 * bytes and output; mask_out is required there (NULL: UNSUPPORTED).
 * Errors: as bsattn_fwd and the builders (topk < 0 or topk > nb: SHAPE);
 * all are reported before anything is launched.
 */
bsattn_status bsattn_fwd_topk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* block_scores, int B, int H, int S, int D, int topk,
                              int dense_last_two_rows, int force_diagonal, int is_causal,
                              uint8_t* mask_out, uint16_t* out, void* workspace,
                              size_t workspace_bytes, bsattn_stream_t stream);
bsattn_status bsattn_fwd_threshold(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const float* block_scores, int B, int H, int S, int D,
                                   float threshold, int dense_last_two_rows, int force_diagonal,
                                   int is_causal, uint8_t* mask_out, uint16_t* out,
                                   void* workspace, size_t workspace_bytes,
                                   bsattn_stream_t stream);

/*
 * Forward pass for a chunk of queries at the end of a longer context
 * (chunked or incremental prefill): q and out bfloat16 [B, H, Sq, D], k and
 * v bfloat16 [B, H, Sk, D] with Sq <= Sk, block_mask uint8
 * [B, H, ceil(Sq/64), ceil(Sk/64)] (nonzero = selected).  Query row r is
 * position r + (Sk - Sq) of the context: with is_causal it sees key t only
 * when t <= r + Sk - Sq (the TileLang FlashAttention guide's BHSD example,
 * past_len = seq_kv - seq_q; the block-sparse guide's §8 Triton reference,
 * PAST_LEN).  Keys at or past Sk are masked; rows with no visible key output
 * 0.  Sq = Sk is bsattn_fwd.  Needs no workspace.
 * Errors: NULL pointers; B, H, Sq <= 0 or Sk < Sq (SHAPE); D not 64 or 128,
 * or ceil(Sk/64) above bsattn_fwd_max_key_blocks(D) (UNSUPPORTED).
 */
bsattn_status bsattn_fwd_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint8_t* block_mask, int B, int H, int Sq, int Sk, int D,
                               int is_causal, uint16_t* out, bsattn_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Sparse GQA decode                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Split count for bsattn_decode_gqa (same guide, §6.3: the smallest split
 * count whose wave efficiency n_waves / ceil(n_waves) reaches 85% of the best,
 * n_waves = m_blocks * splits / num_cus, searched up to min(128, num_cus,
 * max_selected_blocks); one split when the m-blocks already fill 80% of the
 * machine or there are at most 4 blocks).  One (batch, KV head) pair is one
 * m-block.  Returns a value >= 1, or 0 when an argument is out of range.
 * The guide sizes a KV head as blocks * 64 * (dim + dim_v) * 2 bytes for its
 * branch that splits m-blocks larger than the L2; that branch needs two
 * m-blocks per compute unit per (batch, KV head), which decode never has, so
 * the value head dim does not enter and D stands for both.
 */
int bsattn_decode_num_splits(int B, int Hq, int Hkv, int max_selected_blocks, int D,
                             int num_cus);

/* Workspace for bsattn_decode_gqa and its mask and paged forms: what the
 * split stage hands the merge stage (same guide, §6.1: one partial output
 * and one log-sum-exp per split) — fp32 partial outputs [B, Hq, splits, Dv]
 * and their base-2 log-sum-exp [B, Hq, splits], each part 256-byte aligned;
 * Dv is the value head dim.  0 when num_splits is 1 (the split kernel then
 * writes out directly) or an argument is out of range (including more than
 * 2^31 - 1 partials, B * Hq * num_splits, which the decode refuses). */
size_t bsattn_decode_workspace_bytes(int B, int Hq, int Dv, int num_splits);

/*
 * Split-KV sparse GQA decode over packed variable-length KV (same guide,
 * §6, §6.1, §6.2), one query token per sequence.
 *   q            : bfloat16 [B, Hq, D]
 *   k            : bfloat16 [total_k, Hkv, D], sequence b occupies rows
 *                  cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *   v            : bfloat16 [total_k, Hkv, Dv] (Dv, the value head dim, may
 *                  differ from D: the guide's dim_v, §9.2)
 *   cu_seqlens_k : int32 [B + 1], nondecreasing, cu[0] = 0, cu[B] <= total_k
 *   block_indices: int32 [B, Hkv, max_selected_blocks]; entry i selects
 *                  tokens [64 i, min(64 i + 64, len_b)) of the sequence; -1
 *                  (or any i < 0 or i >= ceil(len_b / 64)) selects nothing.
 *                  Order does not matter; duplicates are not allowed.
 *   out          : bfloat16 [B, Hq, Dv]
 * Query head hq reads KV head hq / (Hq / Hkv) (consecutive query heads share
 * a KV head; up to 64 per KV head, the guide's §6.1 block_H).
 * out = softmax(q . k_t / sqrt(D)) V over the selected tokens;
 * zeros when nothing is selected.  The slot list of each (batch, KV head) is
 * cut into num_splits contiguous ranges (the first (slots mod splits) ranges
 * one slot longer); each range yields a partial output and a log-sum-exp,
 * and a second kernel merges them with weights 2^(lse - max lse).
 * num_splits <= 0 uses bsattn_decode_num_splits with the device's CU count.
 * A sequence whose cu_seqlens_k range is decreasing or ends beyond total_k
 * is treated as empty.
 * Errors: NULL pointers; B, Hq, Hkv, max_selected_blocks, total_k <= 0,
 * Hq % Hkv != 0, num_splits > max_selected_blocks, B * Hq * num_splits
 * above 2^31 - 1 (SHAPE); D or Dv not 64 or
 * 128, or Hq / Hkv > 64 (UNSUPPORTED); workspace smaller than
 * bsattn_decode_workspace_bytes for the split count used (WORKSPACE).
 */
bsattn_status bsattn_decode_gqa(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* cu_seqlens_k, const int32_t* block_indices, int B,
                                int Hq, int Hkv, int D, int Dv, int max_selected_blocks,
                                int total_k, int num_splits, uint16_t* out, void* workspace,
                                size_t workspace_bytes, bsattn_stream_t stream);

/*
 * bsattn_decode_gqa without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of bsattn_decode_gqa (same kernels; equal inputs and split count give
 * bitwise-equal outputs).  The split stage's partials go to a static device
 * array inside the library, bsattn_decode_noalloc_scratch_bytes() = 8 MiB,
 * one copy per GPU, held until the process ends; its address is looked up
 * once per device on the first call there.  A call whose split count needs
 * more (bsattn_decode_workspace_bytes above 8 MiB) returns
 * BSATTN_ERR_WORKSPACE and enqueues nothing.  Nothing in the scratch needs
 * clearing: every split writes its partial and log-sum-exp before the merge
 * reads them.  All calls on one GPU share the array, so calls that may
 * overlap in time on one GPU (several streams, several host threads) race
 * and must be serialised by the caller.  The call itself allocates nothing.
 */
bsattn_status bsattn_decode_gqa_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* cu_seqlens_k, const int32_t* block_indices,
                                        int B, int Hq, int Hkv, int D, int Dv,
                                        int max_selected_blocks, int total_k, int num_splits,
                                        uint16_t* out, bsattn_stream_t stream);

/* Size of the static scratch array of bsattn_decode_gqa_noalloc (8 MiB). */
size_t bsattn_decode_noalloc_scratch_bytes(void);

/*
 * Mask-form sparse GQA decode (same guide, §6: the variant of the varlen
 * decode that marks selected blocks in a boolean mask instead of listing
 * their indices).
 *   block_mask : uint8 [B, Hkv, num_blocks]; block j of sequence b is
 *                selected for KV head kvh when block_mask[b, kvh, j] != 0 and
 *                j < ceil(len_b / 64) (columns past the sequence end are
 *                ignored).
 * Everything else (q, k, v, cu_seqlens_k, out, the split count, workspace,
 * GQA head mapping, the merge) is as in bsattn_decode_gqa, with num_blocks
 * in the place of max_selected_blocks, except that the split count divides
 * the row's selected blocks, taken in column order, into even shares (split
 * s takes ranks [s*n/num_splits, (s+1)*n/num_splits) up to rounding, n the
 * row's selected count), so the work is even wherever the selected columns sit.
 * Errors as bsattn_decode_gqa (num_blocks <= 0 or num_splits > num_blocks:
 * SHAPE).
 */
bsattn_status bsattn_decode_gqa_mask(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* cu_seqlens_k, const uint8_t* block_mask, int B,
                                     int Hq, int Hkv, int D, int Dv, int num_blocks, int total_k,
                                     int num_splits, uint16_t* out, void* workspace,
                                     size_t workspace_bytes, bsattn_stream_t stream);

/*
 * Paged-KV sparse GQA decode (same guide, §7: the index-form decode over a
 * page-organised KV cache, as kept by paged-attention serving engines).
 *   k_cache          : bfloat16 [num_pages, page_size, Hkv, D]; page_size a
 *                      multiple of 64
 *   v_cache          : bfloat16 [num_pages, page_size, Hkv, Dv]
 *   cache_seqlens    : int32 [B], sequence lengths (negative: empty)
 *   block_table      : int32 [B, max_blocks_per_seq]; logical page p of
 *                      sequence b is physical page block_table[b, p]
 *   block_indices    : int32 [B, Hkv, max_selected_blocks], logical 64-token
 *                      block indices as in bsattn_decode_gqa
 * Logical block i of sequence b is rows (i % r) * 64 .. +63 of physical page
 * block_table[b, i / r], r = page_size / 64.  An index selects nothing when
 * it is < 0 or >= ceil(len_b / 64), when i / r >= max_blocks_per_seq, or when
 * its table entry is outside [0, num_pages).  q, out, split count, workspace,
 * GQA head mapping and merge as in bsattn_decode_gqa.
 * Errors: NULL pointers; num_pages, page_size, max_blocks_per_seq <= 0 or
 * page_size % 64 != 0, and the shape errors of bsattn_decode_gqa (SHAPE);
 * D / group size as bsattn_decode_gqa (UNSUPPORTED); workspace (WORKSPACE).
 */
bsattn_status bsattn_decode_gqa_paged(const uint16_t* q, const uint16_t* k_cache,
                                      const uint16_t* v_cache, const int32_t* cache_seqlens,
                                      const int32_t* block_table, const int32_t* block_indices,
                                      int B, int Hq, int Hkv, int D, int Dv, int num_pages,
                                      int page_size,
                                      int max_blocks_per_seq, int max_selected_blocks,
                                      int num_splits, uint16_t* out, void* workspace,
                                      size_t workspace_bytes, bsattn_stream_t stream);

/* The split count bsattn_decode_gqa would use for num_splits <= 0 on the
 * current device (queries the CU count once per device). Returns 0 on error. */
int bsattn_decode_default_splits(int B, int Hq, int Hkv, int max_selected_blocks, int D);

/* ------------------------------------------------------------------------ */
/* XAttention block-importance estimator (upstream of the block mask)        */
/* ------------------------------------------------------------------------ */

/*
 * Block sums of the stride-reshaped attention estimate (XAttention guide,
 * "algorithm flow" phases 1-2; stride-reshape section, inverse mode; the
 * softmax + block-sum kernel description).
 *   q : bfloat16 [B, H, Sq, D];  k : bfloat16 [B, H, Sk, D];  Sq <= Sk, the
 *       queries being the last Sq of Sk positions
 *   block_sums : float32 [B, H, nbq, nbk], nbq = ceil(Sq / 64), nbk = ceil(Sk / 64)
 * With s = stride, reshaped key row t' is key rows t's .. t's+s-1 and
 * reshaped query row r' is query rows r's+s-1 down to r's, each concatenated;
 * the logit of (r', t') is their dot product / (sqrt(D) * s * norm); with
 * is_causal, t' is visible to r' when t' <= r' + (Sk - Sq) / s.  Each
 * reshaped row is softmax-normalised over its visible t', and
 * block_sums[b, h, i, j] is the sum of those weights over the reshaped rows
 * of query block i and the reshaped columns of key block j (64 / s each).
 * A row of block_sums therefore adds up to the number of reshaped rows of
 * its query block.
 * workspace: at least bsattn_xattn_workspace_bytes(B, H, Sq, Sk, stride).
 * Errors: NULL pointers; B, H, Sq <= 0, B * H > 65535, Sk < Sq, Sq or Sk not
 * a multiple of stride, (Sk - Sq) % 64 != 0, norm not finite and > 0 (SHAPE);
 * D not 64 or 128, stride not 4, 8 or 16, nbk > 1024 (UNSUPPORTED);
 * workspace missing or smaller than bsattn_xattn_workspace_bytes (WORKSPACE).
 */
/* 0 for sizes the estimator refuses (shape or key-block count). */
size_t bsattn_xattn_workspace_bytes(int B, int H, int Sq, int Sk, int stride);

bsattn_status bsattn_xattn_block_sums(const uint16_t* q, const uint16_t* k, int B, int H, int Sq,
                                      int Sk, int D, int stride, float norm, int is_causal,
                                      float* block_sums, void* workspace, size_t workspace_bytes,
                                      bsattn_stream_t stream);

/*
 * Block selection by cumulative weight (XAttention guide, block-selection
 * section).  block_sums float32 [B, H, nbq, nbk] -> mask uint8 0/1
 * [B, H, nbq, nbk]; query block i sits at key block d = i + nbk - nbq.  Per
 * row: total = the row's sum; required = threshold * total; column 0 (when
 * keep_sink) and column d (when keep_diagonal) are kept and their weights set
 * to 0; the columns are ranked by weight (ties: lower column first), and a
 * column is kept when the weight ranked above it is below required, i.e. the
 * shortest ranked prefix reaching required.  With is_causal, columns after d
 * are then cleared.  Sums and the comparison are float64: the total in
 * ascending column order, the ranked sum in rank order.
 * Errors: NULL pointers; B, H, nbq <= 0, nbk < nbq (SHAPE); nbk > 1024
 * (UNSUPPORTED).
 */
bsattn_status bsattn_build_mask_cumulative(const float* block_sums, int B, int H, int nbq, int nbk,
                                           float threshold, int keep_sink, int keep_diagonal,
                                           int is_causal, uint8_t* mask, bsattn_stream_t stream);

/*
 * The whole estimator (XAttention guide, "algorithm flow" phases 1-3):
 * bsattn_xattn_block_sums, then bsattn_build_mask_cumulative on its output.
 * block_sums may be NULL (the workspace then holds them).  The mask is the
 * block_mask input of bsattn_fwd (Sq = Sk) or bsattn_fwd_chunk.
 * Errors: those of the two calls.
 */
bsattn_status bsattn_xattn_estimate(const uint16_t* q, const uint16_t* k, int B, int H, int Sq,
                                    int Sk, int D, int stride, float norm, float threshold,
                                    int keep_sink, int keep_diagonal, int is_causal,
                                    float* block_sums, uint8_t* mask, void* workspace,
                                    size_t workspace_bytes, bsattn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
