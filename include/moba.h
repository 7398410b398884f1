/*
 * moba.h -- C ABI of the MoBA (Mixture of Block Attention) forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (cited by page title and section; see the design notes for
 * the readings taken where the pages are silent):
 *   "MoBA: Mixture of Block Attention for Long-Context LLMs" (summary page on
 *   paper-graph-ui.vercel.app), section 3.4:
 *     - "Context Partitioning": every sequence is split into blocks of
 *       block_size rows; blocks restart at each sequence boundary and the last
 *       block of a sequence may be short;
 *     - "Affinity Scoring": block representative = mean of the block's keys,
 *       gate score = <q, representative> (no scaling);
 *     - "Top-k Gating": each query head keeps its topk best blocks; the block
 *       holding the query is always kept and counts toward topk;
 *     - "Causality Enforcement": later blocks are never chosen (score -inf);
 *       inside the query's own block a causal mask applies;
 *     - "The Core MoBA Attention Equation": softmax attention over the union
 *       of the chosen blocks;
 *     - "Implementation: Mapping the Algorithm to Efficient GPU Kernels",
 *       steps 1-4: pooled keys, gate, regrouping of queries by block,
 *       per-block attention, log-sum-exp combination of the partial outputs.
 *   The paperhub.cn review page, authors' rebuttal W1: selection is per query
 *   head (no sharing inside a GQA group).
 *
 * Tensor layout ("THD", packed variable-length batch, all device memory):
 *   q   [T][Hq][d], k and v [T][Hkv][d], out [T][Hq][d], rows contiguous, no
 *       padding (moba_fwd_strided also takes other row and head strides);
 *       element type given by moba_dtype_t; every tensor 16-byte aligned;
 *   lse [Hq][T] float32, natural-log log-sum-exp of the scaled logits;
 *   cu_seqlens [S+1] int32 on the device: cu[0] = 0, non-decreasing,
 *       cu[S] = T; sequence s owns rows [cu[s], cu[s+1]); empty sequences are
 *       allowed.
 *   Query head h reads kv head h / (Hq / Hkv).
 *
 * Ownership: the caller owns every pointer; the library never frees caller
 * memory. Entry points that take a workspace use only that memory; moba_fwd
 * and moba_dense_causal_fwd (with a NULL workspace) allocate stream-ordered
 * scratch with hipMallocAsync/hipFreeAsync on the given stream.
 *
 * Execution: all GPU work is enqueued on `stream`; no entry point synchronises
 * the host. Results are valid once the caller synchronises the stream. The
 * library keeps no state between calls apart from a per-thread error message,
 * so it may be used from several threads and streams at once (calls that
 * share a workspace must be ordered by the caller).
 *
 * Errors: arguments are checked on the host before anything is launched; on
 * an error nothing is launched, outputs are untouched, and moba_last_error()
 * describes the problem. A failed launch returns MOBA_ERROR_HIP. Faults inside
 * kernels surface at the caller's next synchronisation.
 *
 * Device-side input check: what lives only in device memory is checked by the
 * first kernel, which builds the block table: cu_seqlens must start at 0,
 * never decrease and end at total_tokens, and no sequence may be longer than
 * the shape's max_seqlen hint allows (the hint sizes the workspace plan, the
 * gate's index width and the dispatch and decode launches; understating it is
 * a contract violation). When the check fails, the table marks every block
 * invalid, no kernel reads rows through it, and the outputs of the call (out
 * and lse; dq, dk and dv; the decode outputs) are set to NaN, so a bad call
 * never returns stale or partial numbers. Such a call still returns
 * MOBA_SUCCESS, since nothing was synchronised; moba_workspace_status()
 * reports the failure afterwards, and with the environment variable
 * MOBA_CHECK=1 the whole-pass entry points (moba_fwd, moba_fwd_ex,
 * moba_fwd_gated, moba_fwd_strided, moba_bwd, moba_decode_prepare, moba_dense_causal_fwd)
 * synchronise the stream once right after the check and return
 * MOBA_ERROR_INVALID_VALUE without launching anything further.
 *
 * Limits of the GPU path: head_dim == 128; block_size a positive multiple of
 * 64; T < 2^31 and T*Hq*topk < 2^32; topk <= 33 unless topk is at least the
 * number of blocks of the longest sequence (then every earlier block is
 * chosen and the result is dense causal attention). Other shapes return
 * MOBA_ERROR_UNSUPPORTED.
 */
#ifndef MOBA_H
#define MOBA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moba_status {
  MOBA_SUCCESS = 0,
  MOBA_ERROR_INVALID_VALUE = 1,      /* bad pointer, size or layout */
  MOBA_ERROR_UNSUPPORTED = 2,        /* valid but outside the GPU path's limits */
  MOBA_ERROR_WORKSPACE_TOO_SMALL = 3,
  MOBA_ERROR_HIP = 4                 /* a HIP runtime call or launch failed */
} moba_status_t;

typedef enum moba_dtype {
  MOBA_DTYPE_FP32 = 0,
  MOBA_DTYPE_BF16 = 1
} moba_dtype_t;

/* Shape of one call. */
typedef struct moba_shape {
  int64_t total_tokens;   /* T, rows of q/k/v/out */
  int32_t num_seqs;       /* S, cu_seqlens holds S+1 entries */
  int32_t max_seqlen;     /* host-known upper bound on any sequence length, 0 = unknown (T);
                           * a sequence longer than this bound allows (in blocks) fails the
                           * device-side input check */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv, divides Hq */
  int32_t head_dim;       /* d, 128 on the GPU path */
  int32_t dtype;          /* element type of q, k, v and out: a moba_dtype_t value (an
                           * integer field, so that any value a caller passes can be
                           * checked) */
} moba_shape_t;

/* Workspace plan: byte offsets of every intermediate inside one workspace.
 * Work on the query heads is done in passes of kv_heads_per_pass kv heads
 * (and their Hq/Hkv query heads each); per-pass buffers are reused. */
/* Gate variants (moba_fwd_gated). Every gate keeps the query's own block and
 * never selects a later block; all three share the attention and merge. */
typedef enum {
  /* top-k by the mean-pooled keys (section 3.4, "Affinity Scoring" and
   * "Top-k Gating"): moba_gate */
  MOBA_GATE_MEAN = 0,
  /* fixed: the n_sink initial blocks and the topk - n_sink most recent ones
   * (section 3.4, "Context Partitioning": sliding window, attention sink):
   * moba_gate_window */
  MOBA_GATE_WINDOW = 1,
  /* the mean gate's topk - extra_max - extra_min - 1 earlier blocks plus the
   * extra_max best by max-pooled and the extra_min best by min-pooled keys
   * (review page, authors' rebuttals on mean pooling and on QUEST), as a
   * union: moba_gate_pooled */
  MOBA_GATE_POOLED = 2
} moba_gate_kind_t;

typedef struct moba_gate {
  int32_t kind;       /* a moba_gate_kind_t value (an integer field, so that any value a
                       * caller passes can be checked) */
  int32_t n_sink;     /* WINDOW: initial blocks always kept, 0 <= n_sink < topk */
  int32_t extra_max;  /* POOLED: extra blocks by max-pooled keys, 0..16 */
  int32_t extra_min;  /* POOLED: extra blocks by min-pooled keys, 0..16;
                       * extra_max + extra_min < topk */
} moba_gate_t;

typedef struct moba_layout {
  int64_t num_blocks_bound;   /* NBb = ceil(T/block_size) + S >= number of blocks */
  int64_t padded_tokens;      /* T rounded up to 64 (informational) */
  int32_t kv_heads_per_pass;  /* P */
  int32_t q_heads_per_pass;   /* Hp = P * Hq / Hkv */
  int32_t max_blocks_per_seq; /* ceil(max_seqlen / block_size) */
  int32_t reserved;
  /* int32 blk_first[S+1] (first global block of each sequence), int32 copy
   * of cu_seqlens[S+1], int32 status (0, or the failed device-side input
   * check: 1 = malformed cu_seqlens, 2 = a sequence with more than
   * max_blocks_per_seq blocks), then (16-byte aligned) int32
   * blk_info[NBb][4] = {sequence, first row, rows, local block index}
   * (sequence = -1 for indices past the last block, and for every index
   * when status != 0). Written by moba_seqtable. table_offset is 0 in every
   * plan. */
  size_t table_offset;
  /* float32 kbar[NBb][Hkv][d]: mean-pooled keys of every block, followed by
   * bf16 kbar_split[NBb][Hkv][2][d]: hi = bf16(kbar), lo = bf16(kbar - hi);
   * then the same pair for the max-pooled keys (kmax, kmax_split) and for the
   * min-pooled keys (kmin, kmin_split). */
  size_t kbar_offset;
  /* element type, vt[P][NBb][d][block_size]: for each kv head of the pass
   * and each block, the block's value rows transposed (zero past its rows);
   * then (256-byte aligned) float32 knorm[P][NBb]: the largest Euclidean norm
   * of the key rows of each block. */
  size_t vt_offset;
  /* int32 idx[T][Hp][topk]: chosen local block ids of the pass's query heads,
   * ascending, unused entries -1; the query's own block c is always at
   * position min(topk, c + 1) - 1 (the mean and window gates fill every
   * position before it; the pooled gate may leave some -1 there). */
  size_t idx_offset;
  /* dispatch tables over bins b = p*NBb + global_block (p < P), uint32:
   * count[P*NBb], offset[P*NBb+1], tile_offset[P*NBb+1] (tiles of the
   * attention kernel's query rows: 256 for bf16, 128 for float32),
   * cursor[P*NBb], a flag (1: the gate already filled count, so
   * moba_dispatch does not recount); then, 16-byte aligned, int32x4 tile records
   * [max_tiles] = {first item, rows, bin, first token of the bin's block},
   * where max_tiles = ceil(T*Hp*(topk-1)/R) + P*NBb, with R the query rows
   * of a tile above, bounds the tile count. */
  size_t bins_offset;
  /* uint32 items[T*Hp*(topk-1)]: per bin, the slots (t*Hp + hl)*topk + s that
   * chose the bin's block as an earlier block (order inside a bin unspecified). */
  size_t items_offset;
  /* part_o[T*Hp*topk][d] (element type of the inputs) and float32
   * part_lse[T*Hp*topk]: attention of slot (t, hl, s) over block idx[t][hl][s]
   * alone (normalised), and its lse. */
  size_t part_o_offset;
  size_t part_lse_offset;
  size_t total_bytes;
} moba_layout_t;

/* Name of a status code. */
const char *moba_status_string(moba_status_t status);

/* Message describing the last non-success status returned on this thread. */
const char *moba_last_error(void);

/* Result of the device-side input check (see "Device-side input check"
 * above) of the last call that built a block table in `workspace` (any
 * forward, backward, decode or dense-baseline workspace: the table sits at
 * its start); num_seqs is that call's S. Synchronises `stream`, then returns
 * MOBA_SUCCESS, or MOBA_ERROR_INVALID_VALUE with moba_last_error() naming the
 * failed check. */
moba_status_t moba_workspace_status(int32_t num_seqs, const void *workspace, hipStream_t stream);

/* Host only. Checks the shape and fills *layout for a pass size of
 * kv_heads_per_pass kv heads (0 = all of them, values are clamped to
 * [1, Hkv]; the pass may be lowered further to fit the dispatch stage's LDS
 * histogram, see layout->kv_heads_per_pass). */
moba_status_t moba_plan(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                        int32_t kv_heads_per_pass, moba_layout_t *layout);

/* Bytes of workspace moba_fwd_ex needs for the given pass size (0 = all kv
 * heads in one pass); 0 if the arguments are invalid. */
size_t moba_fwd_workspace_size(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                               int32_t kv_heads_per_pass);

/* ---- Stages of the forward pass (section 3.4 "Implementation", steps 1-4).
 * Each works on a workspace laid out by moba_plan with the same shape,
 * block_size and topk. moba_seqtable must run first on that workspace.
 * kv_head_begin selects the pass: kv heads [kv_head_begin, kv_head_begin+P)
 * (clipped to Hkv) and their query heads. */

/* Block table from the device cu_seqlens ("Context Partitioning"), with the
 * device-side input check against the layout's max_blocks_per_seq. */
moba_status_t moba_seqtable(const int32_t *cu_seqlens, const moba_shape_t *shape,
                            int32_t block_size, const moba_layout_t *layout, void *workspace,
                            hipStream_t stream);

/* kbar = mean of each block's key rows, over the rows the block has
 * ("Affinity Scoring"; step 1). Reads k, writes the kbar region. */
moba_status_t moba_meanpool(const void *k, const moba_shape_t *shape, int32_t block_size,
                            const moba_layout_t *layout, void *workspace, hipStream_t stream);

/* Gate ("Affinity Scoring", "Top-k Gating", "Causality Enforcement"; step 1):
 * for every row t and query head of the pass, scores <q, kbar_j> for the
 * earlier blocks j of its sequence, keeps the topk-1 best (ties to the lower
 * index), adds its own block and writes the idx region. Needs moba_meanpool. */
moba_status_t moba_gate(const void *q, const moba_shape_t *shape, int32_t block_size,
                        int32_t topk, const moba_layout_t *layout, void *workspace,
                        int32_t kv_head_begin, hipStream_t stream);

/* kmax / kmin = elementwise max / min of each block's key rows (the block
 * representations of the pooled gate). Reads k, writes their parts of the
 * kbar region. */
moba_status_t moba_minmaxpool(const void *k, const moba_shape_t *shape, int32_t block_size,
                              const moba_layout_t *layout, void *workspace, hipStream_t stream);

/* Fixed gate (MOBA_GATE_WINDOW): writes the idx region with, for every row
 * and query head of the pass, the n_sink initial blocks and the
 * topk - n_sink most recent blocks up to its own (all blocks so far when
 * there are at most topk). Reads only the block table; 0 <= n_sink < topk. */
moba_status_t moba_gate_window(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                               int32_t n_sink, const moba_layout_t *layout, void *workspace,
                               int32_t kv_head_begin, hipStream_t stream);

/* Pooled-key gate (MOBA_GATE_POOLED): the union of the mean gate's
 * topk - extra_max - extra_min - 1 earlier blocks, the extra_max best by
 * <q, kmax_j> and the extra_min best by <q, kmin_j> (same tie rule), plus the
 * own block, in the idx layout above; slots left empty are -1 and their
 * part_lse entries are set to -inf so that the merge skips them. Uses the
 * part_o region as scratch; needs moba_meanpool and moba_minmaxpool. */
moba_status_t moba_gate_pooled(const void *q, const moba_shape_t *shape, int32_t block_size,
                               int32_t topk, int32_t extra_max, int32_t extra_min,
                               const moba_layout_t *layout, void *workspace,
                               int32_t kv_head_begin, hipStream_t stream);

/* Regroup queries by chosen block (step 2): histogram, prefix sum and scatter
 * of the earlier-block entries of idx into the bins and items regions. The
 * query's own block is not dispatched (the diagonal attention covers it).
 * moba_gate may already have filled the histogram (for bf16 with groups of a
 * multiple of 4 query heads, top-k <= 17 and at most 289 blocks per
 * sequence); every gate stage records in the bins region whether it did, so
 * moba_dispatch must follow a gate stage on the same workspace and pass. */
moba_status_t moba_dispatch(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                            const moba_layout_t *layout, void *workspace, int32_t kv_head_begin,
                            hipStream_t stream);

/* Block attention (step 3): transposes the pass's values into vt, then
 * computes, for every (row, query head) slot, softmax attention over its own
 * block with a causal mask and over each dispatched earlier block without
 * one, writing part_o / part_lse. softmax_scale 0 means 1/sqrt(d). */
moba_status_t moba_attn_fwd(const void *q, const void *k, const void *v,
                            const moba_shape_t *shape, int32_t block_size, int32_t topk,
                            float softmax_scale, const moba_layout_t *layout, void *workspace,
                            int32_t kv_head_begin, hipStream_t stream);

/* The two halves of moba_attn_fwd, for callers that time or overlap them:
 * _diag transposes the pass's values into vt and runs the own-block (causal)
 * attention; _hist runs the earlier-block attention over the dispatched bins
 * and needs vt from _diag (or moba_attn_prep) of the same pass. */
moba_status_t moba_attn_fwd_diag(const void *q, const void *k, const void *v,
                                 const moba_shape_t *shape, int32_t block_size, int32_t topk,
                                 float softmax_scale, const moba_layout_t *layout,
                                 void *workspace, int32_t kv_head_begin, hipStream_t stream);
moba_status_t moba_attn_fwd_hist(const void *q, const void *k, const moba_shape_t *shape,
                                 int32_t block_size, int32_t topk, float softmax_scale,
                                 const moba_layout_t *layout, void *workspace,
                                 int32_t kv_head_begin, hipStream_t stream);

/* Log-sum-exp combination (step 4): out[t][h] = sum_s exp(lse_s - L) o_s with
 * L = log sum_s exp(lse_s), over the slots before and at the own block's
 * position in ascending block order (slots whose lse is -inf hold no block
 * and are skipped); lse[h][t] = L (lse may be NULL). Writes the pass's heads
 * of out and lse. */
moba_status_t moba_merge(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                         const moba_layout_t *layout, void *workspace, int32_t kv_head_begin,
                         void *out, float *lse, hipStream_t stream);

/* Steps 3 and 4 with the own block last, as moba_fwd runs them: _prep
 * transposes the pass's values into vt and takes the largest key norm of
 * every block; moba_attn_fwd_hist (after _prep) writes the earlier-block
 * partial results; _own_merge then runs the own-block (causal) attention and
 * combines it with those partial results into out and lse (lse may be NULL),
 * with the same bits as moba_attn_fwd_diag followed by moba_merge. For bf16
 * it is one kernel and the own block's partial result is never stored; for
 * float32 it runs those two stages. Like moba_merge it writes NaN to the
 * pass's rows of out and lse when moba_seqtable rejected cu_seqlens. */
moba_status_t moba_attn_prep(const void *k, const void *v, const moba_shape_t *shape,
                             int32_t block_size, int32_t topk, const moba_layout_t *layout,
                             void *workspace, int32_t kv_head_begin, hipStream_t stream);
moba_status_t moba_attn_fwd_own_merge(const void *q, const void *k, const moba_shape_t *shape,
                                      int32_t block_size, int32_t topk, float softmax_scale,
                                      const moba_layout_t *layout, void *workspace,
                                      int32_t kv_head_begin, void *out, float *lse,
                                      hipStream_t stream);

/* ---- Whole forward pass. */

/* All stages, in passes sized to fit workspace_bytes (at least
 * moba_fwd_workspace_size(shape, block_size, topk, 1)). */
moba_status_t moba_fwd_ex(const void *q, const void *k, const void *v,
                          const int32_t *cu_seqlens, const moba_shape_t *shape,
                          int32_t block_size, int32_t topk, float softmax_scale, void *out,
                          float *lse, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* The same with a gate variant (gate must be non-NULL; MOBA_GATE_MEAN is
 * moba_fwd_ex). topk is the number of slots per (row, head). */
moba_status_t moba_fwd_gated(const void *q, const void *k, const void *v,
                             const int32_t *cu_seqlens, const moba_shape_t *shape,
                             int32_t block_size, int32_t topk, const moba_gate_t *gate,
                             float softmax_scale, void *out, float *lse, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Strided q, k, v and out for the whole forward pass: element strides of a
 * [T][H][d] tensor between rows t and t + 1 (token) and between heads h and
 * h + 1 of one row (head); the d elements of one head stay contiguous. The
 * contiguous layout is token = H * d, head = d; q, k and v taken as views of
 * one fused projection output, or a head-major [H][T][d] tensor (token = d,
 * head = T * d), need no copy. Every stride must be a positive multiple of 16
 * bytes (8 bf16 or 4 float32 elements) and every pointer 16-byte aligned; out's
 * (row, head) vectors must not overlap; block_size rows of k must span less
 * than 2 GiB (k_token * element size * block_size < 2^31). Violations return
 * MOBA_ERROR_INVALID_VALUE (MOBA_ERROR_UNSUPPORTED for the 2 GiB bound)
 * before any work is queued. The stage entry points take contiguous tensors. */
typedef struct moba_strides {
  int64_t q_token, q_head;
  int64_t k_token, k_head;
  int64_t v_token, v_head;
  int64_t out_token, out_head;
} moba_strides_t;

/* moba_fwd_gated over strided tensors: strides NULL means contiguous, gate
 * NULL means MOBA_GATE_MEAN. Results equal moba_fwd_gated's on the same
 * values bit for bit (the layout changes only where rows are read and
 * written). The workspace and lse are as for moba_fwd_ex. */
moba_status_t moba_fwd_strided(const void *q, const void *k, const void *v,
                               const int32_t *cu_seqlens, const moba_shape_t *shape,
                               const moba_strides_t *strides, int32_t block_size, int32_t topk,
                               const moba_gate_t *gate, float softmax_scale, void *out, float *lse,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Same as moba_fwd_ex with softmax_scale = 1/sqrt(d) and stream-ordered scratch of at most
 * MOBA_WORKSPACE_LIMIT_GIB GiB (environment, default 48) per call. */
moba_status_t moba_fwd(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                       const moba_shape_t *shape, int32_t block_size, int32_t topk, void *out,
                       float *lse, hipStream_t stream);

/* ---- Forward pass without allocation, for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same as moba_fwd_ex, on a workspace the library owns: a static
 * device array of MOBA_NOALLOC_WORKSPACE_BYTES that each GPU the library runs
 * on holds until the process ends (its device address is looked up on the
 * first call on each device). Calls no hipMalloc, hipFree or other
 * allocating routine. Shapes whose workspace with one kv head per pass
 * exceeds the array return MOBA_ERROR_UNSUPPORTED (moba_fwd_workspace_size
 * with kv_heads_per_pass = 1 gives that size); otherwise the largest pass
 * that fits is used. Every call on a GPU shares that GPU's array (the kernels
 * clear what must start at zero), so calls that overlap on one GPU -- on
 * different streams or from different threads -- race and must be ordered by
 * the caller. */
#define MOBA_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)
moba_status_t moba_fwd_noalloc(const void *q, const void *k, const void *v,
                               const int32_t *cu_seqlens, const moba_shape_t *shape,
                               int32_t block_size, int32_t topk, float softmax_scale, void *out,
                               float *lse, hipStream_t stream);

/* ---- Decode: one new query per sequence over its KV cache (section 3.4's
 * gate and block attention applied to a single query; the review page's
 * GSM-Infinite table reports MoBA used for both prefill and decode).
 * The cache is k_cache, v_cache [T][Hkv][d] packed by cu_seqlens[S+1] (the
 * shape describes it: total_tokens = T, num_seqs = S); sequence s's cache
 * already holds the new token as its last row L_s - 1, the query's position.
 * q is [S][Hq][d]; out [S][Hq][d] (element type of q) and lse [Hq][S]
 * (float32, may be NULL). The query's own block is the cache's last block,
 * attended up to the last row; its k-1 earlier blocks are chosen as in
 * moba_gate. A sequence with an empty cache gets out = 0 and lse = -inf.
 * The workspace holds the block table and pooled keys of the cache, which
 * moba_decode_prepare computes (once per cache; a caller that keeps them
 * up to date may skip it), plus per-call scratch. */
size_t moba_decode_workspace_size(const moba_shape_t *cache_shape, int32_t block_size,
                                  int32_t topk);
moba_status_t moba_decode_prepare(const void *k_cache, const int32_t *cu_seqlens,
                                  const moba_shape_t *cache_shape, int32_t block_size,
                                  int32_t topk, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);
moba_status_t moba_decode(const void *q, const void *k_cache, const void *v_cache,
                          const moba_shape_t *cache_shape, int32_t block_size, int32_t topk,
                          float softmax_scale, void *out, float *lse, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ---- Backward pass (section 3.4: MoBA is trained end to end; gradients
 * flow through the attention over the chosen blocks, and the block choice,
 * a discrete top-k, passes none to the gate or the pooled keys).
 * With P the softmax of the scaled logits over the query's chosen union (own
 * block causal), D = <dO, O> per (row, head) and dS = P (dO V^T - D):
 *   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dO,
 * each kv head summing over the query heads that read it.
 * Inputs: q, k, v as for the forward pass; out [T][Hq][d] and lse [Hq][T]
 * (natural log) as the forward pass with the same gate, block_size, topk
 * and softmax_scale wrote them; dout [T][Hq][d]. Outputs dq [T][Hq][d],
 * dk and dv [T][Hkv][d], all overwritten (element type of q). The gate is
 * recomputed from q and k (it is deterministic), so out and lse must come
 * from these very inputs; the probabilities are recomputed from lse.
 * gate may be NULL (MOBA_GATE_MEAN). bf16 only: fp32 returns
 * MOBA_ERROR_UNSUPPORTED. Same limits as the forward pass otherwise. */

/* Host only. Workspace plan of the backward pass for a pass size (0 = all kv
 * heads; see moba_plan): the forward plan's regions, except that the vt
 * region is unused, part_o_offset is the fp32 partial dq of each
 * (row, head, slot) ([T][Hp][topk][d]) and part_lse_offset is D ([Hq][T]
 * float32), followed by the dk/dv stage's own areas: 256 bytes it zeroes and
 * reads, two per-bin prefix arrays, and fp32 partials for bins it splits into
 * segments of MOBA_DKDV_SEGMENT_ROWS rows (environment variable, a multiple
 * of 32; default 262144; read by the plan and by the stage, which must agree).
 * */
moba_status_t moba_bwd_plan(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                            int32_t kv_heads_per_pass, moba_layout_t *layout);
/* Bytes of workspace moba_bwd needs for the given pass size; 0 if invalid. */
size_t moba_bwd_workspace_size(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                               int32_t kv_heads_per_pass);
/* Whole backward pass, in passes sized to fit workspace_bytes (at least
 * moba_bwd_workspace_size(shape, block_size, topk, 1)). */
moba_status_t moba_bwd(const void *q, const void *k, const void *v, const void *out,
                       const float *lse, const void *dout, const int32_t *cu_seqlens,
                       const moba_shape_t *shape, int32_t block_size, int32_t topk,
                       const moba_gate_t *gate, float softmax_scale, void *dq, void *dk,
                       void *dv, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Stages of moba_bwd, on a workspace laid out by moba_bwd_plan (moba_seqtable,
 * moba_meanpool / moba_minmaxpool, the gate stages and moba_dispatch accept
 * that plan too and run first, as in the forward pass). Per pass
 * kv_head_begin: gate, dispatch, moba_attn_bwd_dq, moba_attn_bwd_dq_sum,
 * moba_attn_bwd_dkdv; moba_bwd_delta once before. */

/* D[h][t] = <dout[t][h], out[t][h]> (float32) into the part_lse region. */
moba_status_t moba_bwd_delta(const void *out, const void *dout, const moba_shape_t *shape,
                             int32_t block_size, int32_t topk, const moba_layout_t *layout,
                             void *workspace, hipStream_t stream);
/* Partial dq of every (row, head, slot) of the pass: which = 1 the own block
 * (causal), 2 the earlier blocks of the bins, 3 both. Needs the gate,
 * dispatch and moba_bwd_delta. */
moba_status_t moba_attn_bwd_dq(const void *q, const void *k, const void *v, const void *dout,
                               const float *lse, const moba_shape_t *shape, int32_t block_size,
                               int32_t topk, float softmax_scale, const moba_layout_t *layout,
                               void *workspace, int32_t kv_head_begin, int32_t which,
                               hipStream_t stream);
/* dq of the pass's query heads = sum of their slots' partials (own block
 * first, then the earlier blocks in slot order). */
moba_status_t moba_attn_bwd_dq_sum(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                                   const moba_layout_t *layout, void *workspace,
                                   int32_t kv_head_begin, void *dq, hipStream_t stream);
/* dk, dv of the pass's kv heads (own-block rows of their query heads, then
 * the rows of the bins). Needs the gate, dispatch and moba_bwd_delta. */
moba_status_t moba_attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout,
                                 const float *lse, const moba_shape_t *shape, int32_t block_size,
                                 int32_t topk, float softmax_scale, const moba_layout_t *layout,
                                 void *workspace, int32_t kv_head_begin, void *dk, void *dv,
                                 hipStream_t stream);

/* ---- Dense causal attention on the same layout ("Standard Attention
 * Baseline" with a causal mask, per sequence): the full-attention reference
 * the pages compare MoBA against. workspace may be NULL (then scratch is
 * allocated stream-ordered); otherwise it must hold
 * moba_dense_causal_workspace_size(shape) bytes. */
size_t moba_dense_causal_workspace_size(const moba_shape_t *shape);
moba_status_t moba_dense_causal_fwd(const void *q, const void *k, const void *v,
                                    const int32_t *cu_seqlens, const moba_shape_t *shape,
                                    float softmax_scale, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H */
