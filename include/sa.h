/*
 * sa.h -- C ABI of the MI355X (gfx950) sparse flash-attention forward library (libsa_hip.so).
 *
 * Three sibling forward paths and their host-side helpers:
 *   - skip-softmax attention: KV tiles whose scores are negligible under a threshold lambda are
 *     skipped inside the FlashAttention loop (Model-Optimizer "Skip-Softmax Sparse Attention for
 *     Diffusion Models" README: introduction and "Threshold Modes");
 *   - N:M sparse softmax: in every M consecutive keys keep the top-N scores, the rest become -inf
 *     before the softmax, with dense attention-sink and recent-token windows (Model-Optimizer
 *     "Attention Sparsity for HuggingFace Models": "N:M Sparse Softmax");
 *   - proxy-compensated block-sparse attention driven by packed UInt32 exact-block bitmaps, with
 *     omitted KV blocks represented by a mean-K / summed-V summary and the denominator corrected
 *     by the token mass of each summary (FlashInfer block-sparse proxy description quoted in the
 *     TensorRT-LLM "add VisualGen SOL sparse attention" PR: "Description", "Bitmask format");
 *   - the calibrated threshold lowering a*exp(b*s)/seq_k ("Threshold Modes").
 *
 * Conventions shared by every entry point:
 *   - Ownership: every buffer is allocated by the caller; device buffers are device pointers
 *     (e.g. from torch), host scalars are passed by value.  The library allocates nothing and keeps
 *     no state between calls; calls are reentrant.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Every kernel is enqueued
 *     asynchronously on it; nothing synchronises the host.
 *   - Errors: all argument checks run on the host before any HIP call.  On an error status nothing
 *     has been enqueued or written.  SA_ERR_HIP reports a failed launch (hipGetLastError).
 *   - Dtypes: Q, K, V, O and the proxy summaries are bf16 (uint16 bit patterns), fp32 accumulate.
 *   - Layout: Q/O are [batch, seqlen_q, heads_q, head_dim], K/V are [batch, seqlen_k, heads_kv,
 *     head_dim], each addressed through three element strides (batch, sequence, head) with a unit
 *     head_dim stride.  Every (batch, seq, head) row must start 16-byte aligned: base pointers
 *     16-byte aligned and strides multiples of 8 elements.
 *   - GQA: query head h reads KV head h / (heads_q / heads_kv).
 *   - Causal masking is top-left: query i sees keys k <= i (requires seqlen_q == seqlen_k).
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,       /* non-positive size, heads_q % heads_kv != 0, causal with Sq != Sk */
  SA_ERR_UNSUPPORTED = 3, /* head_dim / tile / (n, m) / causal-proxy combination not implemented */
  SA_ERR_ALIGN = 4,       /* non-16-byte-aligned pointer or stride */
  SA_ERR_VALUE = 5,       /* bad scalar: lambda, softmax_scale, calibration inputs, sink/recent */
  SA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  SA_ERR_SCRATCH = 7      /* needs more scratch than the fixed device buffer holds (noalloc) */
} sa_status;

/* Human-readable name of a status code (static string). */
const char* sa_status_str(sa_status status);

/* Decision granularity of skip-softmax (sa_skip_softmax_fwd_ex). */
typedef enum {
  SA_SKIP_GRAN_TILE = 0,  /* the whole block_q x block_k tile is kept or skipped */
  SA_SKIP_GRAN_WAVE = 1   /* each block of 32 query rows (one wavefront) decides on its own */
} sa_skip_granularity;

/* Shape and layout of one attention call. */
typedef struct {
  int32_t batch, heads_q, heads_kv;
  int32_t seqlen_q, seqlen_k;
  int32_t head_dim;        /* 64 or 128 */
  int32_t causal;          /* 0 or 1 */
  int32_t block_q;         /* query tile (skip, N:M) or query block (proxy) rows: 64 or 128 */
  int32_t block_k;         /* key tile (skip, N:M) or semantic KV block (proxy): 64 or 128 */
  float softmax_scale;     /* > 0 and finite, usually 1/sqrt(head_dim) */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];  /* batch, seq, head (elements) */
} sa_attn_desc;

/*
 * Skip-softmax forward (Model-Optimizer skip-softmax README: introduction, "Threshold Modes").
 *
 * FlashAttention over key tiles of block_k keys, in ascending order, per query tile of block_q rows.
 * With t = softmax_scale*log2(e)*q.k and M_j[r] the row maxima of visited tile j, tile j is skipped
 * -- no exponentials, no V load, no P.V -- when every valid row r of the query tile satisfies
 *     M_j[r] < fl32(m[r] + L),   L = (float)log2((double)lambda),
 * where m[r] is the fp32 running max over the tiles kept so far.  A skipped tile leaves the running
 * max, sum and accumulator untouched.  lambda == 0 never skips (dense attention); any finite
 * lambda >= 0 is accepted.
 *
 *   lambda            finite, >= 0.
 *   tile_state        optional, uint8 [B, Hq, nQT, nKT] (nQT = ceil(Sq/block_q), nKT =
 *                     ceil(Sk/block_k)): 0 kept, 1 skipped, 2 not visited (causal).
 *   head_counters     optional, uint32 [B, Hq, 2] = {visited tiles, skipped tiles}, ADDED to
 *                     (the caller zeroes them to start a count).
 *   lse               optional, fp32 [B, Hq, Sq], natural-log log-sum-exp of the scaled logits
 *                     over the kept keys.
 *   dbg_tile_rowmax   optional debug export, fp32 [B, Hq, nQT, nKT, block_q]: the M_j[r] the
 *                     decision used (log2 domain); -inf for unvisited tiles and empty rows.
 * Supported: head_dim 64/128, block_q 64/128, block_k 64/128 (the Model-Optimizer HuggingFace
 * attention-sparsity page, "Custom Configuration", uses br = bc = 128).
 */
sa_status sa_skip_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                              const void* v, void* o, float lambda, uint8_t* tile_state,
                              uint32_t* head_counters, float* lse, float* dbg_tile_rowmax,
                              void* stream);

/*
 * Skip-softmax forward with a choice of decision granularity (the same rule; the HuggingFace
 * attention-sparsity page, "Custom Configuration", sets the br x bc block the decisions are made
 * on).  granularity SA_SKIP_GRAN_TILE is sa_skip_softmax_fwd.  SA_SKIP_GRAN_WAVE decides every
 * block of R = 32 query rows on its own -- its own running max, its own skips -- exactly as
 * sa_skip_softmax_fwd with 32-row query tiles would; block_q then only sets how many such blocks
 * share one pass over K/V, and a V tile is loaded when any of them keeps it.
 *
 *   granularity       SA_SKIP_GRAN_TILE or SA_SKIP_GRAN_WAVE (SA_ERR_VALUE otherwise).
 *   tile_state        optional, uint8 [B, Hq, nR, nKT] with nR = ceil(Sq/R), R = block_q (tile) or
 *                     32 (wave): 0 kept, 1 skipped, 2 not visited (no unmasked key of the block).
 *   head_counters     optional, uint32 [B, Hq, 2]: {visited, skipped} (R-row block, key tile)
 *                     pairs, added to.
 *   lse               optional, fp32 [B, Hq, Sq].
 *   dbg_tile_rowmax   optional, fp32 [B, Hq, nR, nKT, R].
 * Other arguments and the supported sizes as sa_skip_softmax_fwd.
 */
sa_status sa_skip_softmax_fwd_ex(const sa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float lambda, int32_t granularity,
                                 uint8_t* tile_state, uint32_t* head_counters, float* lse,
                                 float* dbg_tile_rowmax, void* stream);

/*
 * N:M sparse softmax forward (Model-Optimizer HuggingFace attention sparsity: "N:M Sparse
 * Softmax").  For every query row and every group of m consecutive keys (groups aligned to key 0,
 * the last one clipped to Sk), keys ranked below the top n by raw score q.k (ties to the lower
 * key index) are set to -inf before the softmax, except keys k < dense_sink_tokens and keys with
 * 0 <= row - k < dense_recent_tokens, which stay dense.  Masked (causal) keys rank last.
 *
 *   (n, m)            m == 4 with n in 1..4, or m == 8 with n in 1..8 (n == m is dense).
 *   dense_sink_tokens, dense_recent_tokens   >= 0.
 *   lse               optional, fp32 [B, Hq, Sq].
 *   dbg_keep_bits     optional debug export, uint32 [B, Hq, Sq, ceil(Sk/32)]: bit k&31 of word
 *                     k>>5 set when key k is kept (LSB first); padding bits 0.
 *   dbg_scores        optional debug export, fp32 [B, Hq, Sq, Sk]: the raw q.k the ranking used
 *                     (-inf where causally masked).
 * Supported: head_dim 64/128, block_q 64/128, block_k 64/128 (the result does not depend on
 * block_k, which the rule does not use).
 */
sa_status sa_nm_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                            const void* v, void* o, int32_t n, int32_t m,
                            int32_t dense_sink_tokens, int32_t dense_recent_tokens, float* lse,
                            uint32_t* dbg_keep_bits, float* dbg_scores, void* stream);

/*
 * Skip-softmax and N:M sparse softmax in one forward (Model-Optimizer HuggingFace attention
 * sparsity: the skip_softmax_calib_sparse24 configuration, calibrated skip-softmax together with
 * 2:4 sparse softmax).  Reading: the N:M rule of sa_nm_softmax_fwd first fixes which keys of each
 * query row may enter the softmax; the skip-softmax loop of sa_skip_softmax_fwd then runs over the
 * tiles of those masked logits.  Top-n keeps every group maximum, so a tile's masked row maxima
 * equal its unmasked ones and the skip decisions are exactly those of sa_skip_softmax_fwd at the
 * same lambda; kept tiles contribute only their N:M-kept keys.
 *
 *   lambda, tile_state, head_counters, lse, dbg_tile_rowmax   as sa_skip_softmax_fwd.
 *   (n, m), dense_sink_tokens, dense_recent_tokens, dbg_keep_bits, dbg_scores
 *                     as sa_nm_softmax_fwd; dbg_keep_bits are the N:M bits of every visited
 *                     tile, whether the tile was then kept or skipped.
 * Supported: head_dim 64/128, block_q 64/128, block_k 64/128 (decision tiles as sa_skip_softmax_fwd).
 */
sa_status sa_skip_nm_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float lambda, int32_t n, int32_t m,
                                 int32_t dense_sink_tokens, int32_t dense_recent_tokens,
                                 uint8_t* tile_state, uint32_t* head_counters, float* lse,
                                 float* dbg_tile_rowmax, uint32_t* dbg_keep_bits,
                                 float* dbg_scores, void* stream);

/*
 * Decode-phase skip-softmax forward: one query token per (batch, query head) against a KV cache
 * (Model-Optimizer skip-softmax rule as in sa_skip_softmax_fwd, used in the decode phase with its
 * own threshold: the HuggingFace attention-sparsity configuration gives phase-specific thresholds,
 * decode 1e-4).  The query tile is the single query row, so with t = softmax_scale*log2(e)*q.k the
 * key tile j of head h is skipped when
 *     M_j < fl32(m + L),   L = (float)log2((double)lambda),
 * m the fp32 running max of the tiles kept so far -- sa_skip_softmax_fwd with seqlen_q = 1 and a
 * one-row query tile, evaluated independently per query head.
 *
 * The key axis is split over workgroups.  For lambda <= 1 this is exact: a skipped tile could not
 * have raised the running max, so each split starts from the max of all earlier tile maxima.  For
 * lambda > 1 the decisions depend on the order of the kept tiles and the call runs one split
 * (num_splits > 1 is then SA_ERR_UNSUPPORTED).
 *
 *   desc              seqlen_q == 1 and causal == 0 (SA_ERR_UNSUPPORTED otherwise); seqlen_k is the
 *                     cache capacity; block_k 64 or 128 is the decision tile; block_q is ignored.
 *                     heads_q/heads_kv <= 16 (head_dim 128) or <= 8 (head_dim 64).
 *   q, o              [B, 1, Hq, D] (strides as in the descriptor); k, v [B, Sk, Hkv, D].
 *   seqlens_k         optional device int32 [B]: keys of each sequence, clamped to [0, Sk]; NULL
 *                     means Sk for all.  Tiles past a sequence's end are not visited (state 2); a
 *                     sequence of 0 keys gets O = 0 and lse = -inf.
 *   num_splits        0 picks a split count; otherwise the number of key-axis splits.
 *   workspace         device memory of at least sa_skip_softmax_decode_workspace bytes for the
 *                     same desc, lambda and num_splits, 256-byte aligned; contents are scratch.
 *   tile_state        optional uint8 [B, Hq, nKT]: 0 kept, 1 skipped, 2 not visited.
 *   head_counters     optional uint32 [B, Hq, 2] {visited, skipped}, added to.
 *   lse               optional fp32 [B, Hq].
 *   dbg_tile_rowmax   optional fp32 [B, Hq, nKT]: the M_j used (log2 domain), -inf when not
 *                     visited.
 * Kernels on the stream: when the call runs one split (num_splits 1, or num_splits 0 with
 * lambda > 1) and the head group's scores over the whole cache fit in 128 KiB, one kernel with one
 * workgroup per (batch, KV head) keeps them in LDS (the workspace is then not touched, though a
 * buffer of the queried size is still required); otherwise three: scores and tile maxima,
 * decisions and P.V over kept tiles, merge of the splits.
 */
sa_status sa_skip_softmax_decode_workspace(const sa_attn_desc* desc, float lambda,
                                           int32_t num_splits, size_t* workspace_bytes,
                                           int32_t* num_splits_used);
sa_status sa_skip_softmax_decode_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                                     const void* v, void* o, float lambda,
                                     const int32_t* seqlens_k, int32_t num_splits,
                                     void* workspace, size_t workspace_bytes,
                                     uint8_t* tile_state, uint32_t* head_counters, float* lse,
                                     float* dbg_tile_rowmax, void* stream);

/*
 * Decode-phase skip-softmax forward that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation).  Same arguments, kernels and results as sa_skip_softmax_decode_fwd without the
 * workspace pair: the workspace lives in a fixed device array inside the library, one copy per GPU,
 * SA_DECODE_SCRATCH_BYTES long and held until the process ends.
 *
 *   - A call whose sa_skip_softmax_decode_workspace size exceeds SA_DECODE_SCRATCH_BYTES returns
 *     SA_ERR_SCRATCH (nothing enqueued).
 *   - The first call on a device looks up that device's copy of the array (hipGetSymbolAddress,
 *     with the device current); make one call before capturing a graph around later ones.
 *   - Every call on a GPU shares that GPU's array, and it keeps the last call's contents: calls
 *     that overlap on one GPU (on different streams, or from different threads) race and must be
 *     serialised by the caller.  Nothing in the array needs clearing between calls (every region
 *     is written before it is read).
 */
#define SA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
sa_status sa_skip_softmax_decode_fwd_noalloc(const sa_attn_desc* desc, const void* q,
                                             const void* k, const void* v, void* o, float lambda,
                                             const int32_t* seqlens_k, int32_t num_splits,
                                             uint8_t* tile_state, uint32_t* head_counters,
                                             float* lse, float* dbg_tile_rowmax, void* stream);

/*
 * Route preparation, the "plan" step of the block-sparse path (FlashInfer proxy description,
 * "Bitmask format").  nKB = ceil(Sk/block_k), nQB = ceil(Sq/block_q), W = ceil(nKB/32).
 *
 *   bitmask     uint32 [B, Hkv, nQB, W] packed exact-block bitmaps, one per (batch, KV head,
 *               query block); block j is exact when bit j&31 of word j>>5 is set (LSB first);
 *               bits j >= nKB are padding and are ignored.
 *   n_exact     int32 [B, Hkv, nQB]: number of exact blocks.
 *   exact_idx   int32 [B, Hkv, nQB, nKB]: exact block indices in ascending order, -1 after them.
 *   proxy_keep  uint32 [B, Hkv, nQB, W]: complement of the exact bits over j < nKB (the blocks a
 *               proxy summary stands for), padding bits 0.
 * Only the shape fields of desc are used (strides and scale are ignored).
 */
sa_status sa_bitmask_route_prep(const sa_attn_desc* desc, const uint32_t* bitmask,
                                int32_t* n_exact, int32_t* exact_idx, uint32_t* proxy_keep,
                                void* stream);

/*
 * Route preparation from canonical BSR, the other "plan" input (FlashInfer proxy description,
 * "Bitmask format": BSR block_indptr / block_indices and bitmaps are prepared into the same route
 * stream, with bitwise-identical results).  Rows r = (b, kv head, q block), row-major, nQB, nKB as
 * for sa_bitmask_route_prep.
 *
 *   block_indptr   int32 [B*Hkv*nQB + 1]: row r owns entries block_indptr[r] .. block_indptr[r+1]-1.
 *   block_indices  int32 [nnz]: exact KV block indices (may be NULL when nnz == 0).  A canonical
 *                  row is strictly ascending within [0, nKB).
 *   nnz            length of block_indices; no entry at or past it is read.
 *   n_exact, exact_idx, proxy_keep   exactly as sa_bitmask_route_prep produces them for the bitmap
 *                  holding the same blocks.
 *   bad_rows       optional uint32 [1], caller-zeroed: incremented once per row that is not
 *                  canonical (pointer outside [0, nnz] or reversed, entry outside [0, nKB),
 *                  entries not strictly ascending).
 * Non-canonical rows are still prepared as sets: duplicates collapse, order is ignored, entries
 * outside [0, nKB) are dropped, and a pointer range is clamped to [0, nnz] (empty when reversed).
 * Requires nKB <= 65536 (SA_ERR_UNSUPPORTED otherwise).  Only the shape fields of desc are used.
 */
sa_status sa_bsr_route_prep(const sa_attn_desc* desc, const int32_t* block_indptr,
                            const int32_t* block_indices, int64_t nnz, int32_t* n_exact,
                            int32_t* exact_idx, uint32_t* proxy_keep, uint32_t* bad_rows,
                            void* stream);

/*
 * Proxy-compensated block-sparse forward, the "run" step (FlashInfer proxy description,
 * "Description").  For a query in block qb: exact blocks from (n_exact, exact_idx) contribute
 * their tokens exactly; when use_proxy != 0, every block j with bit j set in proxy_keep contributes
 * one summary key k_mean[j] with value v_sum[j] and token mass c_j = min(block_k, Sk - j*block_k):
 *   O = [sum_t e^{s_t} v_t + sum_j e^{s^_j} v_sum_j] / [sum_t e^{s_t} + sum_j c_j e^{s^_j}],
 *   s = softmax_scale * q.k.   A row with nothing to attend to gets O = 0 and lse = -inf.
 *
 *   k_mean, v_sum   bf16 [B, Hkv, nKB, head_dim], contiguous (caller-provided summaries).
 *   n_exact, exact_idx, proxy_keep   as produced by sa_bitmask_route_prep.  The kernel reads
 *                   n_exact clamped to [0, nKB] and the first n_exact entries of the row's
 *                   exact_idx; an entry outside [0, nKB) (such as the -1 fill after the real
 *                   entries, read when n_exact exceeds them) contributes nothing and reads no K/V.
 *                   Entries are otherwise trusted: a repeated block is attended once per entry.
 *   lse             optional, fp32 [B, Hq, Sq].
 * Non-causal only (causal -> SA_ERR_UNSUPPORTED).  Supported: head_dim 128 (and 64),
 * block_q 128 or 64, block_k 64 or 128.
 */
sa_status sa_proxy_block_sparse_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const void* k_mean, const void* v_sum,
                                    const int32_t* n_exact, const int32_t* exact_idx,
                                    const uint32_t* proxy_keep, int32_t use_proxy, void* o,
                                    float* lse, void* stream);

/*
 * Calibrated threshold lowering, host only ("Threshold Modes"): scale_factor = a*exp(b*s) in
 * double; lambda = scale_factor / seq_k; outputs are optional.  *lambda_out is the float lambda to
 * pass to sa_skip_softmax_fwd and *log2_lambda_out = (float)log2((double)*lambda_out), the value
 * the kernel then uses.  Requires a > 0, finite b, 0 <= target_sparsity < 1, seq_k >= 1.
 */
sa_status sa_threshold_from_calib(double a, double b, double target_sparsity, int64_t seq_k,
                                  double* scale_factor_out, float* lambda_out,
                                  float* log2_lambda_out);

/*
 * Calibration sweep (Model-Optimizer diffusion README, "Calibrated threshold"; HuggingFace
 * attention-sparsity page, calibration.threshold_trials): runs sa_skip_softmax_fwd once per trial
 * threshold on the same inputs and returns each trial's tile sparsity, skipped / visited tiles
 * summed over all (batch, query head) counters.
 *
 *   o               bf16 output, overwritten by every trial (a work buffer for the caller).
 *   trial_lambdas   host float [n_trials], each >= 0 and finite (SA_ERR_VALUE otherwise).
 *   head_counters   device uint32 [B, Hq, 2] work buffer; the call zeroes it before each trial.
 *   sparsities_out  host double [n_trials].
 * Unlike the other entry points this one blocks: after each trial it copies the counters to the
 * host and synchronizes the stream.  Shape rules as sa_skip_softmax_fwd.
 */
sa_status sa_skip_softmax_calibrate(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, void* o, const float* trial_lambdas,
                                    int32_t n_trials, uint32_t* head_counters,
                                    double* sparsities_out, void* stream);

/*
 * Log-space fit of the calibrated threshold model, host only (Model-Optimizer diffusion README:
 * scale_factor = a*exp(b*target_sparsity) calibrated once, log-space fitting recommended;
 * "Known Issues": targets below the smallest sparsity reached extrapolate).  Each trial i ran at
 * threshold lambda_i with measured tile sparsity s_i, i.e. scale factor lambda_i * seq_k.  Ordinary
 * least squares of ln(lambda_i * seq_k) on s_i over the usable trials (lambda_i > 0 finite and
 * 0 < s_i < 1) gives b (slope) and ln a (intercept).  min/max_sparsity_out (optional) receive the
 * range of usable sparsities: targets outside it are extrapolations.  SA_ERR_VALUE when fewer than
 * two usable trials remain or their sparsities are all equal.
 */
sa_status sa_fit_threshold_calib(const double* trial_lambdas, const double* sparsities,
                                 int32_t n_trials, int64_t seq_k, double* a_out, double* b_out,
                                 double* min_sparsity_out, double* max_sparsity_out);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
