/*
 * rf.h -- C ABI of the MI355X (gfx950) RainFusion2.0 block-sparse attention
 * hot path.
 *
 * Sources, cited by page title and section:
 *   [RF2] "RainFusion2.0: Temporal-Spatial Awareness and Hardware-Efficient
 *         Block-wise Sparse Attention" (arXiv 2512.24086): Abstract key
 *         insights (1) block-wise mean values as representative tokens for
 *         sparse mask prediction, (2) spatiotemporal-aware token
 *         permutation, (3) first-frame sink; TL;DR (3D window permutation,
 *         blockwise representative tokens); Figure 2 and 3 captions.
 *   [RF1] "RainFusion: Adaptive Video Generation Acceleration via
 *         Multi-Dimensional Visual Redundancy" (arXiv 2505.21036): Abstract;
 *         review page, Assumptions (softmax attention, Eq. (1)), "What
 *         carries the argument" and "Core claim" (head patterns, ARM),
 *         free parameters (bandwidth, stride tau, threshold alpha).
 *
 * One attention call of a diffusion transformer runs, on the caller's HIP
 * stream:
 *   rf_permute(Q), rf_permute(K), rf_permute(V, RF_TILES_T)   3D windows
 *   rf_block_means(Qp, Kp)                                     Qbar, Kbar
 *     (or rf_permute_means(Q), rf_permute_means(K): both in one pass)
 *   rf_predict_mask(Qbar, Kbar)                                kept tiles
 *   rf_sparse_attn(Qp, Kp, Vt, kept)                           Op
 *   rf_unpermute(Op)                                           O
 * With the v1 head patterns in place of the predicted mask:
 *   rf_arm_recall(local, temporal), rf_arm_recall(global, spatial),
 *   rf_arm_classify -> head patterns; rf_pattern_mask -> kept rows;
 *   rf_sparse_attn_rows(Qp, Kp, Vt, rows) -> Op.
 *
 * Conventions
 *   Token tensors are contiguous [B][H][tokens][d] (RF_ROWS).  Raster token
 *   n = (t*H + h)*W + w of a T x H x W latent grid; n_text text tokens follow
 *   the N = T*H*W video tokens.  The permuted sequence has Np padded video
 *   slots (window order, pad slots zero) followed by the text tokens:
 *   Lp = Np + n_text slots.  Blocks ("tiles") are bs = wt*wh*ww consecutive
 *   slots: nb video blocks, then ceil(n_text/bs) text tiles.  Permuted
 *   tensors hold whole tiles: Lt = n_tiles*bs rows, the rows after Lp (the
 *   rest of a partial last text tile) being pad.
 *   Window order: blocks row-major over (frame, row, column) block
 *   coordinates of the grid padded up to whole windows; tokens row-major
 *   inside a block.  With permute = 0 the slots are the raster tokens and
 *   the last block is padded.
 *   All pointers passed to the GPU calls are device pointers that must be
 *   16-byte aligned; calls only enqueue work on `stream` (never synchronise,
 *   never allocate), and return before any launch when an argument is bad.
 *   A plan is bound to the device that was current at rf_plan_create; call
 *   the GPU functions with that device current.  Plans are immutable after
 *   creation and may be shared by threads.
 *   Errors: every function returns an rf_status; rf_last_error() gives a
 *   thread-local message for the last failure.  Nothing aborts or prints.
 */
#ifndef RF_H
#define RF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RF_OK = 0,
  RF_ERR_INVALID_ARG = 1,      /* null/misaligned pointer, bad size or value */
  RF_ERR_UNSUPPORTED = 2,      /* valid but not implemented (d, bs, dtype) */
  RF_ERR_HIP = 3,              /* HIP runtime error (no device, launch, copy) */
  RF_ERR_BUFFER_TOO_SMALL = 4  /* host table buffer smaller than required */
} rf_status;

typedef enum { RF_F32 = 0, RF_BF16 = 1 } rf_dtype;

/* Head patterns of RainFusion v1 [RF1 review, "What carries the argument"],
 * as tile masks.  Band half-width `band` (tiles) and checkerboard stride
 * `tau` are parameters; bandwidth b maps to band = floor(b*nb + 1/2), and
 * b = 1/4 keeps 1 - (3/4)^2 = 7/16 of the video tile pairs.
 *   RF_SPATIAL   video tile i keeps video tile j when |i - j| <= band
 *                (tiles in frame-major order, the block index);
 *   RF_TEMPORAL  |r(i) - r(j)| <= band, r = position of the tile when the
 *                tiles are sorted by (h, w, t) of their first valid token;
 *   RF_TEXTURAL  j = i (mod tau).
 * Text tiles are appended to every video row; text query rows keep every
 * tile. */
typedef enum { RF_SPATIAL = 0, RF_TEMPORAL = 1, RF_TEXTURAL = 2 } rf_pattern;

/* Order of a permuted tensor in memory. */
typedef enum {
  RF_ROWS = 0,    /* [B][H][Lt][d]: one row of d values per slot */
  RF_TILES_T = 1  /* [B][H][n_tiles][d][bs]: each tile transposed, the bs
                     slots of one feature contiguous (pad slots zero).  The
                     V operand of rf_sparse_attn uses this order. */
} rf_order;

/* Latent grid, window and switches of one attention call. */
typedef struct {
  int32_t T, H, W;      /* latent frames, rows, columns (T = 1 for images) */
  int32_t wt, wh, ww;   /* window; bs = wt*wh*ww must be 64 or 128 */
  int32_t n_text;       /* text tokens after the video tokens (>= 0) */
  int32_t permute;      /* 1 = 3D window order [RF2 insight (2)], 0 = raster */
  int32_t sink;         /* 1 = key blocks holding a frame-0 token are always
                           kept [RF2 insight (3)] */
} rf_layout;

typedef struct {
  int64_t N;            /* video tokens T*H*W */
  int64_t Np;           /* padded video slots, nb*bs */
  int64_t L;            /* N + n_text: rows of an unpermuted tensor */
  int64_t Lp;           /* Np + n_text: slots holding video pad or tokens */
  int64_t Lt;           /* n_tiles*bs: rows of a permuted RF_ROWS tensor */
  int32_t bs;           /* slots per block */
  int32_t nb;           /* video blocks */
  int32_t n_text_tiles; /* ceil(n_text / bs) */
  int32_t n_tiles;      /* nb + n_text_tiles: query and key tiles */
  int32_t n_sink;       /* sink blocks (0 when the sink is off) */
} rf_sizes;

/* Keep counts of the mask rule for one sparsity s (percent):
 * k = floor((nb*(100 - s) + 50) / 100), k_eff = max(k, n_sink, 1).
 * A video query tile keeps k_eff video blocks plus every text tile; a text
 * query tile keeps all n_tiles tiles. */
typedef struct {
  int32_t k;
  int32_t k_eff;
  int32_t row_len_video;  /* k_eff + n_text_tiles */
  int32_t row_len_text;   /* n_tiles */
  int64_t nnz_per_head;   /* nb*row_len_video + n_text_tiles*row_len_text */
} rf_keep;

/* ---- host-only helpers (no device needed) ------------------------------ */

/* Sizes of a layout.  RF_ERR_INVALID_ARG for non-positive grid or window
 * extents, negative n_text, switches other than 0/1, or sizes beyond 2^31
 * slots; RF_ERR_UNSUPPORTED when bs is not 64 or 128. */
rf_status rf_layout_sizes(const rf_layout* lay, rf_sizes* out);

/* The plan's index tables, into caller-owned host buffers of the given
 * element capacities:
 *   slot_src[Lt]   raster token of each slot, -1 for pad;
 *   tok_slot[L]    slot of each raster token;
 *   tile_count[n_tiles]  valid slots per tile;
 *   is_sink[nb]    1 for sink blocks.
 * RF_ERR_BUFFER_TOO_SMALL if a capacity is short. */
rf_status rf_layout_tables(const rf_layout* lay, int32_t* slot_src,
                           int64_t cap_slot_src, int32_t* tok_slot,
                           int64_t cap_tok_slot, int32_t* tile_count,
                           int64_t cap_tile_count, uint8_t* is_sink,
                           int64_t cap_is_sink);

/* Keep counts for sparsity_pct in [0, 99] [RF2 Abstract: 80% sparsity;
 * Figure 2: 60% for image editing], from a layout.  RF_ERR_INVALID_ARG for
 * a null output or a sparsity outside [0, 99]. */
rf_status rf_layout_keep(const rf_layout* lay, int32_t sparsity_pct,
                         rf_keep* out);

/* Band half-width, in video tiles, of the v1 band patterns for a bandwidth
 * fraction b in [0, 1] [RF1 review, free parameters: bandwidth 1/4 giving a
 * 9/16 cut]: *band = floor(b*nb + 1/2), so that the band |i - j| <= band
 * keeps 1 - (1 - b)^2 of the video tile pairs (7/16 at b = 1/4).
 * RF_ERR_INVALID_ARG for b outside [0, 1] or a null output. */
rf_status rf_band_tiles(const rf_layout* lay, double bandwidth, int32_t* band);

/* r(i) of RF_TEMPORAL for every video tile, into a host buffer of at least
 * nb elements (a permutation of 0..nb-1). */
rf_status rf_tile_rank(const rf_layout* lay, int32_t* rank, int64_t cap);

/* Row width that holds every row of the pattern masks for (band, tau):
 * max(min(2*band + 1, nb), ceil(nb/tau)) + n_text_tiles, or n_tiles when
 * there is text.  band >= 0, tau >= 1. */
rf_status rf_pattern_row_width(const rf_layout* lay, int32_t band, int32_t tau,
                               int32_t* width);

/* Number of ARM samples: ceil(H*W / stride) for the local sample (every
 * stride-th raster token of frame 0, local != 0) or ceil(N / stride) for
 * the global one (every stride-th video token).  stride >= 1. */
rf_status rf_arm_sample_count(const rf_layout* lay, int32_t local,
                              int32_t stride, int32_t* n);

const char* rf_status_str(rf_status s);
const char* rf_last_error(void);

/* ---- plan -------------------------------------------------------------- */

typedef struct rf_plan rf_plan;   /* opaque: layout, sizes, device tables */

/* Build the index tables of `lay` on the host and copy them to the current
 * device (the only allocation and the only synchronising call of the
 * library).  *out receives the plan, owned by the caller; RF_ERR_HIP when no
 * device is usable. */
rf_status rf_plan_create(const rf_layout* lay, rf_plan** out);
void rf_plan_destroy(rf_plan* plan);
rf_status rf_plan_sizes(const rf_plan* plan, rf_sizes* out);
/* The same sizes one by one (each output pointer may be null): video tokens
 * N, padded slots Np, video blocks nb, block size bs, sink blocks n_sink and
 * text tiles n_text_tiles. */
rf_status rf_plan_info(const rf_plan* plan, int64_t* N, int64_t* Np, int32_t* nb,
                       int32_t* bs, int32_t* n_sink, int32_t* n_text_tiles);

/* Keep counts of the plan's layout for sparsity_pct in [0, 99] (the rule of
 * rf_layout_keep [RF2 Abstract insights (1), (3)]): *k_eff = video blocks
 * kept per video query row, *nnz_per_head = int32 entries of one head's
 * kept list, the size of the kept_idx buffer per (b, h) that
 * rf_predict_mask writes and rf_sparse_attn reads.  Either output may be
 * null.  RF_ERR_INVALID_ARG for a null plan or a sparsity outside [0, 99].
 * Host only: reads no device memory. */
rf_status rf_keep_count(const rf_plan* plan, int32_t sparsity_pct, int32_t* k_eff,
                        int64_t* nnz_per_head);

/* ---- hot path (asynchronous on `stream`) ------------------------------- */

/* 3D window permutation [RF2 Abstract insight (2); TL;DR; Figure 3].
 * x: [B][H][L][d] raster tokens (then text).  xp: permuted tensor in
 * `order` (RF_ROWS: [B][H][Lt][d]; RF_TILES_T: [B][H][n_tiles][d][bs]).
 * Pad slots are written as zeros.  dtype RF_BF16 or RF_F32; d in {64, 128}.
 * x and xp must not overlap. */
rf_status rf_permute(const rf_plan* plan, const void* x, void* xp, int32_t B,
                     int32_t H, int32_t d, rf_dtype dtype, rf_order order,
                     hipStream_t stream);

/* rf_permute (RF_ROWS) fused with rf_block_means on the same tensor: the
 * permuted rows of x go to xp and the mean of each video block's valid
 * slots [RF2 Abstract insight (1)] to xbar, fp32 [B][H][nb][d], in one
 * pass over x.  xp may be null: then only the means are written (for a Q
 * that rf_sparse_attn_raster reads in raster order).  Same arguments and
 * errors as rf_permute. */
rf_status rf_permute_means(const rf_plan* plan, const void* x, void* xp,
                           float* xbar, int32_t B, int32_t H, int32_t d,
                           rf_dtype dtype, hipStream_t stream);

/* Inverse permutation: xp [B][H][Lt][d] (RF_ROWS) -> x [B][H][L][d]; pad
 * slots are dropped, text rows copied back. */
rf_status rf_unpermute(const rf_plan* plan, const void* xp, void* x,
                       int32_t B, int32_t H, int32_t d, rf_dtype dtype,
                       hipStream_t stream);

/* Representative tokens [RF2 Abstract insight (1)]: the mean of each video
 * block's valid slots, accumulated in fp32.  qp, kp: [B][H][Lt][d]
 * (RF_ROWS; pad slots are ignored whatever they hold).  qbar, kbar:
 * fp32 [B][H][nb][d].  Text tiles are not pooled. */
rf_status rf_block_means(const rf_plan* plan, const void* qp, const void* kp,
                         float* qbar, float* kbar, int32_t B, int32_t H,
                         int32_t d, rf_dtype dtype, hipStream_t stream);

/* Online mask prediction [RF2 Abstract insights (1), (3)].  For each video
 * query block i the logits l_ij = qbar_i . kbar_j / sqrt(d) (fp32) rank the
 * non-sink video key blocks; the row keeps the sink blocks plus the
 * k_eff - n_sink best blocks (ties to the lower index), then every text
 * tile.  Text query tiles keep all tiles.
 * kept_idx: int32 [B][H][nnz_per_head], rows in tile order, each row
 * ascending (row r of a head starts at r*row_len_video for r < nb and at
 * nb*row_len_video + (r - nb)*row_len_text after that).
 * mask_or_null: optional uint8 [B][H][n_tiles][n_tiles] dense copy of the
 * kept sets (1 where row i keeps tile j, else 0), for inspection.
 * logits_or_null: optional fp32 [B][H][nb][nb] copy of l.  Both optional
 * outputs are written only when non-null and cost extra writes of their
 * full size. */
rf_status rf_predict_mask(const rf_plan* plan, const float* qbar,
                          const float* kbar, int32_t B, int32_t H, int32_t d,
                          int32_t sparsity_pct, int32_t* kept_idx,
                          uint8_t* mask_or_null, float* logits_or_null,
                          hipStream_t stream);

/* Block-sparse attention forward [RF2 Abstract: skipping computations for
 * insignificant tokens; RF1 review, Eq. (1)].  For each valid query slot of
 * tile i: o = sum_j softmax_j(scale * q . k_j) v_j over the valid slots of
 * the tiles listed in row i of kept_idx; pad query rows are written as 0.
 * qp, kp, op: [B][H][Lt][d] RF_ROWS; vt: [B][H][n_tiles][d][bs] RF_TILES_T.
 * Precondition: the pad slots of kp (its rows at pad slots) and of vt (its
 * columns at pad slots) hold zeros, as rf_permute writes them.  The
 * 128-slot kernels rely on it: a pad key then scores exactly 0 and adds
 * nothing to o, so they leave pad keys unmasked when every query's tile
 * maximum is positive and take the pads' weights out of the row sum; with
 * other pad values the result is unspecified (finite pad values give a
 * finite result).  Pad query rows of qp are not read.
 * kept_idx as produced by rf_predict_mask for the same sparsity_pct; every
 * entry must lie in [0, n_tiles).  RF_BF16: bf16 operands, fp32
 * accumulation and softmax, bf16 output; RF_F32: fp32 throughout.
 * lse_or_null: optional fp32 [B][H][Lt] (4-byte aligned) receiving each
 * query's log-sum-exp over its kept keys, ln sum_j exp(scale * q . k_j),
 * the natural-log softmax normaliser that merges this output with other
 * partial attentions; -inf at pad query slots and for a query with no
 * valid kept key.  With RF_BF16 the sum is taken over the fp32 weights
 * (the PV product uses them rounded to bf16), within about 1e-4 of the
 * exact value.  d in {64, 128}. */
rf_status rf_sparse_attn(const rf_plan* plan, const void* qp, const void* kp,
                         const void* vt, const int32_t* kept_idx,
                         int32_t sparsity_pct, void* op, float* lse_or_null,
                         int32_t B, int32_t H, int32_t d, float scale,
                         rf_dtype dtype, hipStream_t stream);

/* rf_sparse_attn with raster-order query and output: q [B][H][L][d] is the
 * unpermuted query tensor (the slot of each query is found through the
 * plan's tables, pad slots are never read), and o [B][H][L][d] receives the
 * attention output of every token at its raster row, which is what
 * rf_unpermute would make of rf_sparse_attn's output, bit for bit;
 * lse_or_null, if given, is fp32 [B][H][L] in raster order.  kp and vt as
 * for rf_sparse_attn (permuted, with the zero-pad precondition), kept_idx
 * and sparsity_pct as for rf_sparse_attn.  Removes the permuted-Q write and
 * the rf_unpermute pass from the path: rf_permute_means(Q, xp = null) gives
 * the query means.  q and o must not overlap. */
rf_status rf_sparse_attn_raster(const rf_plan* plan, const void* q, const void* kp,
                                const void* vt, const int32_t* kept_idx,
                                int32_t sparsity_pct, void* o, float* lse_or_null,
                                int32_t B, int32_t H, int32_t d, float scale,
                                rf_dtype dtype, hipStream_t stream);

/* Attention-recall diagnostic [RF1 review, "What carries the argument":
 * the masked recall R', attention mass that survives a mask over the mass
 * with no mask].  For each sampled query tile t = sample_tiles[s] and each
 * valid query slot of it: recall = the sum of exp(scale * q . k_j) over the
 * valid slots j of the tiles listed in row t of kept_idx, divided by the
 * same sum over every valid slot of the sequence (the dense softmax
 * denominator).  fp32 arithmetic with a running maximum (bf16 or fp32
 * operands); cost is dense attention logits for the sampled tiles only.
 * qp, kp: [B][H][Lt][d] RF_ROWS; kept_idx as for rf_sparse_attn (entries
 * out of range are ignored); sample_tiles: device int32 [n_sample], an id
 * outside [0, n_tiles) yields NaN for the whole sample; recall: fp32
 * [B][H][n_sample][bs], NaN at pad query slots.  n_sample >= 1,
 * n_tiles <= 262144, d in {64, 128}. */
rf_status rf_attention_recall(const rf_plan* plan, const void* qp,
                              const void* kp, const int32_t* kept_idx,
                              int32_t sparsity_pct,
                              const int32_t* sample_tiles, int32_t n_sample,
                              int32_t B, int32_t H, int32_t d, float scale,
                              rf_dtype dtype, float* recall,
                              hipStream_t stream);

/* ---- padded kept rows and the v1 head patterns ------------------------- */

/* Kept rows in the padded layout: int32 [B][H][n_tiles][row_width], row t
 * of a head holding the kept tile ids of query tile t in ascending order
 * followed by -1 up to row_width (the length of a row is the position of
 * its first negative entry; an empty row gives output 0).  Entries outside
 * [0, n_tiles) before the first -1 are skipped.  1 <= row_width <= n_tiles.
 * Otherwise identical to rf_sparse_attn / rf_attention_recall (including
 * the zero-pad precondition on kp and vt). */
rf_status rf_sparse_attn_rows(const rf_plan* plan, const void* qp,
                              const void* kp, const void* vt,
                              const int32_t* kept_rows, int32_t row_width,
                              void* op, float* lse_or_null, int32_t B,
                              int32_t H, int32_t d, float scale, rf_dtype dtype,
                              hipStream_t stream);
rf_status rf_attention_recall_rows(const rf_plan* plan, const void* qp,
                                   const void* kp, const int32_t* kept_rows,
                                   int32_t row_width,
                                   const int32_t* sample_tiles,
                                   int32_t n_sample, int32_t B, int32_t H,
                                   int32_t d, float scale, rf_dtype dtype,
                                   float* recall, hipStream_t stream);

/* Head-pattern mask [RF1 review, "What carries the argument": striped
 * bands for spatial and temporal heads, checkerboard for textural heads]:
 * writes the padded kept rows (layout above) of every (b, h) from its
 * pattern head_pattern[b*H + h] (device int32, an rf_pattern; any other
 * value gives empty video rows).  row_width must lie in
 * [rf_pattern_row_width(band, tau), n_tiles]; kept_rows holds
 * B*H*n_tiles*row_width int32. */
rf_status rf_pattern_mask(const rf_plan* plan, const int32_t* head_pattern,
                          int32_t B, int32_t H, int32_t band, int32_t tau,
                          int32_t* kept_rows, int32_t row_width,
                          hipStream_t stream);

/* ARM recall [RF1 review, "What carries the argument": R' = S(Q', K', M') /
 * S(Q', K', M_init) on sampled queries and keys; "Core claim": first-frame
 * tokens for the local pattern, equally spaced tokens for the global one].
 * The sample is every stride-th raster token of frame 0 (local != 0) or of
 * the video; sampled tokens are both the queries and the keys.  For sampled
 * query a: recall[b][h][a] = sum of exp(scale * q_a . k_b) over the sampled
 * keys b whose tile the query's tile keeps under `pattern` (band, tau),
 * divided by the same sum over all sampled keys.  fp32 arithmetic (bf16 or
 * fp32 operands).  qp, kp: [B][H][Lt][d] RF_ROWS; recall: fp32
 * [B][H][n], n from rf_arm_sample_count.  d in {64, 128}. */
rf_status rf_arm_recall(const rf_plan* plan, const void* qp, const void* kp,
                        int32_t local, int32_t stride, int32_t pattern,
                        int32_t band, int32_t tau, int32_t B, int32_t H,
                        int32_t d, float scale, rf_dtype dtype, float* recall,
                        hipStream_t stream);

/* ARM decision [RF1 review, "Core claim": temporal first, then spatial,
 * otherwise textural]: per head bh < BH, bR = mean of local_recall[bh][:]
 * (n_local values, recall of the temporal mask on the local sample) and
 * eR = mean of global_recall[bh][:] (the spatial mask on the global
 * sample), fp32; head_pattern[bh] = RF_TEMPORAL if bR >= alpha, else
 * RF_SPATIAL if eR >= alpha, else RF_TEXTURAL.  mean_or_null: optional fp32
 * [BH][2] = (bR, eR).  All buffers on the device. */
rf_status rf_arm_classify(const float* local_recall, int32_t n_local,
                          const float* global_recall, int32_t n_global,
                          int32_t BH, float alpha, int32_t* head_pattern,
                          float* mean_or_null, hipStream_t stream);

/* ---- FP8 variant -------------------------------------------------------- */

/* e4m3 operands for the FP8 attention [RF2 TL;DR: integration with
 * quantization named as future work].  OCP e4m3 codes (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; largest finite 448), rounded to
 * nearest, ties to even, from x * 2^-e with one power-of-two scale 2^e per
 * group, e the smallest integer with amax <= 448 * 2^e (e = 0 for an
 * all-zero group).  Groups:
 *   order RF_ROWS:    xp [B][H][Lt][d] -> x8 [B][H][Lt][d] uint8, one scale
 *                     per (b, h, tile): scale fp32 [B][H][n_tiles] = 2^e;
 *   order RF_TILES_T: xp [B][H][n_tiles][d][bs] -> x8 in the same order, one
 *                     scale per (b, h, feature) over all slots: scale fp32
 *                     [B][H][d] (used as scratch while the call runs).
 * xp is bf16 (RF_BF16 only) with finite values; x8 16-byte aligned. */
rf_status rf_quantize_fp8(const rf_plan* plan, const void* xp, rf_order order,
                          void* x8, float* scale, int32_t B, int32_t H,
                          int32_t d, rf_dtype dtype, hipStream_t stream);

/* rf_permute (or rf_permute_means) fused with rf_quantize_fp8: the raster
 * bf16 tensor x [B][H][L][d] goes straight to permuted e4m3 codes x8 and
 * scales, bit for bit those of rf_permute followed by rf_quantize_fp8 with
 * the same order; for RF_ROWS, xbar_or_null (fp32 [B][H][nb][d], or null)
 * receives the block means of the bf16 values, bit for bit those of
 * rf_permute_means.  RF_TILES_T takes no xbar.  One pass over x for
 * RF_ROWS; for RF_TILES_T a read of x for the feature maxima, then one
 * pass. */
rf_status rf_permute_fp8(const rf_plan* plan, const void* x, rf_order order,
                         void* x8, float* scale, float* xbar_or_null,
                         int32_t B, int32_t H, int32_t d, rf_dtype dtype,
                         hipStream_t stream);

/* Block-sparse attention on e4m3 operands: q8, k8 [B][H][Lt][d] (RF_ROWS)
 * with per-tile scales q_scale, k_scale [B][H][n_tiles]; v8
 * [B][H][n_tiles][d][bs] (RF_TILES_T) with per-feature scales v_scale
 * [B][H][d] (16-byte aligned), all from rf_quantize_fp8.  The pad slots of
 * k8 and v8 must hold zero codes, as rf_quantize_fp8 and rf_permute_fp8
 * write them (the precondition of rf_sparse_attn).  For each valid
 * query slot: o = sum_j w_j (v8_j * v_scale) / sum_j w_j over the valid
 * slots of the kept tiles, w_j = the e4m3 rounding of 16 exp(x_j - m) for
 * the logit x_j = scale * (q8 . k8_j) * q_scale * k_scale and a running
 * reference m at most 4 ln 2 below the row maximum (weights down to 2^-10
 * of the largest stay normal e4m3 numbers), accumulated in fp32; op bf16
 * [B][H][Lt][d], pad query rows 0.  kept_idx and sparsity_pct as for
 * rf_sparse_attn; lse_or_null as for rf_sparse_attn: m - ln 16 +
 * ln sum_j w_j, the log-sum-exp of the logits with the e4m3 weights.
 * d = 128 and bs = 128 only (RF_ERR_UNSUPPORTED otherwise). */
rf_status rf_sparse_attn_fp8(const rf_plan* plan, const void* q8,
                             const float* q_scale, const void* k8,
                             const float* k_scale, const void* v8,
                             const float* v_scale, const int32_t* kept_idx,
                             int32_t sparsity_pct, void* op, float* lse_or_null,
                             int32_t B, int32_t H, int32_t d, float scale,
                             hipStream_t stream);

/* rf_sparse_attn_fp8 writing its output in raster order, so that no
 * rf_unpermute pass follows it: o bf16 [B][H][L][d] (L = N + n_text, text
 * rows after the video rows) and lse_or_null fp32 [B][H][L], each row the
 * value rf_sparse_attn_fp8 gives the slot holding that token, bit for bit;
 * pad slots have no output row.  q8, k8, v8, the scales and kept_idx as
 * for rf_sparse_attn_fp8 (the quantized Q stays in RF_ROWS slot order).
 * Every row of o is written; the caller owns o, which must not be one of
 * the operand buffers (RF_ERR_INVALID_ARG). */
rf_status rf_sparse_attn_fp8_raster(const rf_plan* plan, const void* q8,
                                    const float* q_scale, const void* k8,
                                    const float* k_scale, const void* v8,
                                    const float* v_scale, const int32_t* kept_idx,
                                    int32_t sparsity_pct, void* o, float* lse_or_null,
                                    int32_t B, int32_t H, int32_t d, float scale,
                                    hipStream_t stream);

/* rf_sparse_attn_fp8 on padded kept rows (the layout of
 * rf_sparse_attn_rows). */
rf_status rf_sparse_attn_fp8_rows(const rf_plan* plan, const void* q8,
                                  const float* q_scale, const void* k8,
                                  const float* k_scale, const void* v8,
                                  const float* v_scale,
                                  const int32_t* kept_rows, int32_t row_width,
                                  void* op, float* lse_or_null, int32_t B,
                                  int32_t H, int32_t d, float scale,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RF_H */
