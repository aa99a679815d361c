/*
 * bsp.h - C ABI of the dynamic block-sparse causal prefill attention library
 * (libbsp.so, HIP kernels for gfx950 / MI355X).
 *
 * The method is the three-stage pipeline of the FlashPrefill summary page
 * (paperlayer.ai, "FlashPrefill: Instantaneous Pattern Discovery and
 * Thresholding for Ultra-Fast Long-Context Prefilling"): instantaneous
 * pattern discovery over pooled blocks, max-based dynamic thresholding with
 * block selection, then block-sparse attention (Appendix B "Detailed
 * Implementation").  One call per stage:
 *
 *   bsp_score     pool Q and K into B-token blocks, score query blocks against
 *                 causally valid key blocks, normalise each row;
 *   bsp_mask      keep blocks whose score reaches gamma times the row maximum,
 *                 OR the sink and local-window blocks, AND causal, and compress
 *                 each row into an ascending list of key-block indices;
 *   bsp_attn_fwd  online-softmax attention over the kept key blocks only.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing, keeps no global state and never synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and completes asynchronously.
 *   - All checks run on the host before any launch.  On any error status
 *     nothing is launched and no output is touched.  BSP_ERR_HIP means a
 *     launch was rejected (hipGetLastError after the launch); faults inside
 *     a kernel surface at the caller's next synchronisation.
 *   - Layouts are row-major and contiguous: Q [hq][seq][d], K and V
 *     [hkv][seq][d].  q head h reads kv head h / (hq / hkv) (GQA).
 *   - Base pointers are expected to be 16-byte aligned, as hipMalloc and
 *     torch allocations are: the kernels move data in 16-byte vectors
 *     wherever the row strides keep them aligned.
 *   - nb = ceil(seq / block).  A last block shorter than `block` holds the
 *     seq % block tail tokens; it pools over those tokens only.
 *   - seq == 0 is valid and does nothing (after the descriptor checks; the
 *     tensor pointers are then not checked and may be NULL).
 *   - Calls on different streams with disjoint outputs may run concurrently;
 *     the library is thread-safe.
 */
#ifndef BSP_H
#define BSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSP_ABI_VERSION 8

typedef enum bsp_status {
  BSP_OK = 0,
  BSP_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  BSP_ERR_BAD_SHAPE = 2,    /* sizes out of range or inconsistent */
  BSP_ERR_BAD_DTYPE = 3,    /* unknown dtype, or fp8 scales missing / given for non-fp8 */
  BSP_ERR_BAD_VALUE = 4,    /* gamma, sm_scale or window sizes out of range */
  BSP_ERR_UNSUPPORTED = 5,  /* valid request this build does not serve (non-causal) */
  BSP_ERR_HIP = 6           /* the HIP runtime rejected a launch */
} bsp_status;

typedef enum bsp_dtype {
  BSP_DTYPE_F32 = 0,      /* IEEE binary32 */
  BSP_DTYPE_BF16 = 1,     /* bfloat16 */
  BSP_DTYPE_FP8_E4M3 = 2, /* OCP e4m3fn (bias 7, max 448, no inf) times a per-head fp32 scale */
  /* Q and K as BSP_DTYPE_FP8_E4M3; V in bfloat16 times v_scale[g].  With V
   * from bsp_widen_e4m3 (exact) the attention result is bit-identical to
   * BSP_DTYPE_FP8_E4M3 on the codes, and the launch is faster: V tiles then
   * reach LDS by direct loads instead of being widened in every workgroup.
   * Entry points that read only Q and K treat it as BSP_DTYPE_FP8_E4M3. */
  BSP_DTYPE_FP8_E4M3_V_BF16 = 3
} bsp_dtype;

/* Limits checked by every entry point. */
#define BSP_MAX_HEADS 1024
#define BSP_MAX_SEQ (1 << 21)

/* Problem description, read on the host during the call only. */
typedef struct bsp_desc {
  int32_t hq;           /* query heads, 1..BSP_MAX_HEADS */
  int32_t hkv;          /* key/value heads, divides hq */
  int32_t seq;          /* tokens, 0..BSP_MAX_SEQ */
  int32_t d;            /* head dimension: 64 or 128 */
  int32_t block;        /* B, tokens per block: 64 or 128 (the page uses 128, Appendix A) */
  float gamma;          /* threshold factor in [0, 1] (the page's alpha, section 3 / Appendix A) */
  float sm_scale;       /* softmax scale c; <= 0 selects 1/sqrt(d); must be finite */
  int32_t causal;       /* must be 1 (prefill attention is causal) */
  int32_t sink_blocks;  /* leading key blocks always kept (>= 0); Appendix A keeps a sink */
  int32_t local_blocks; /* key blocks ending at the diagonal always kept (>= 0); 1 = diagonal */
  int32_t dtype;        /* bsp_dtype of Q, K and V */
  const float *q_scale; /* fp8 only, device [hq]:  Q = code * q_scale[h] */
  const float *k_scale; /* fp8 only, device [hkv]: K = code * k_scale[g] */
  const float *v_scale; /* fp8 only, device [hkv]: V = code (or its bf16 widening) * v_scale[g] */
} bsp_desc;

/*
 * bsp_score - stage 1, pattern discovery (FlashPrefill summary page, section 3
 * "Instantaneous Pattern Discovery" and "Block Approximation"; Appendix B).
 *
 *   q_pool[h][I][:]  = mean of Q[h][t][:] over the tokens t of block I
 *   k_pool[g][J][:]  = mean of K[g][t][:] over the tokens t of block J
 *                      (fp8: means of the dequantised values)
 *   S[h][I][J]       = c * q_pool[h][I] . k_pool[g(h)][J]          for J <= I
 *   score[h][I][J]   = exp(S - max_J' S) / sum_J'<=I exp(S - max_J' S)  for J <= I
 *   score[h][I][J]   = 0                                             for J > I
 *
 * q, k:    device, storage dtype, [hq][seq][d] and [hkv][seq][d]
 * q_pool:  device float [hq][nb][d]     (written)
 * k_pool:  device float [hkv][nb][d]    (written)
 * score:   device float [hq][nb][nb]    (written, every entry)
 * Needs desc->q_scale and desc->k_scale for fp8 (v_scale is not read).
 */
bsp_status bsp_score(const bsp_desc *desc, const void *q, const void *k, float *q_pool,
                     float *k_pool, float *score, void *stream);

/*
 * bsp_score_arith - stage 1 with the per-query block approximation (section
 * 3 "Instantaneous Pattern Discovery": pooled key blocks stand in for their
 * tokens and a block's significance is the average over its queries; "Block
 * Approximation for Kernel Optimization": a single fused pass on the
 * (L/B) x (L/B) grid, no L x (L/B) intermediate).  Kbar as in bsp_score;
 * for J <= I
 *   score[h][I][J] = mean over the valid tokens i of block I of
 *                    exp(c * q_i . Kbar[g][J]) / sum_{J' <= I} exp(c * q_i . Kbar[g][J'])
 * and 0 for J > I; every row sums to 1.  q_i is dequantised (times
 * q_scale[h]) for fp8.  The result feeds bsp_mask like bsp_score's.
 * Arithmetic: fp32-accurate scores (fp32 MFMA for fp32 inputs; otherwise bf16
 * MFMA on exact queries against an exact three-way bf16 split of Kbar).
 *
 * q, k:    device, storage dtype, [hq][seq][d] and [hkv][seq][d]
 * k_pool:  device float [hkv][nb][d]    (written)
 * score:   device float [hq][nb][nb]    (written, every entry)
 * Needs desc->q_scale and desc->k_scale for fp8 (v_scale is not read).
 */
bsp_status bsp_score_arith(const bsp_desc *desc, const void *q, const void *k, float *k_pool,
                           float *score, void *stream);

/*
 * bsp_mask - stage 2, max-based dynamic thresholding and block selection
 * (section 3 "Max-based Dynamic Thresholding"; Appendix A structural
 * retention; Appendix B "Dynamic Thresholding and Block Selection").
 *
 * Without user_mask, for J <= I:
 *   keep[h][I][J] = score[h][I][J] >= gamma * max_J'<=I score[h][I][J']
 *                   OR J < sink_blocks OR I - J < local_blocks
 * With user_mask (device uint8 [hq][nb][nb], nonzero = keep), the threshold
 * and the forced blocks are replaced by it: keep = user_mask != 0 AND J <= I.
 * keep is 0 for J > I.  No sort and no cumulative sum is used.
 *
 * score:     device float [hq][nb][nb] as written by bsp_score; may be NULL
 *            iff user_mask is given (then it is not read)
 * user_mask: device uint8 [hq][nb][nb] or NULL
 * mask:      device uint8 [hq][nb][nb] or NULL; written with keep (0/1)
 * kv_idx:    device int32 [hq][nb][nb]; row (h, I) receives the kept J in
 *            ascending order in its first kv_cnt[h][I] entries (the diagonal,
 *            when kept, last); entries past the count are not written
 * kv_cnt:    device int32 [hq][nb]
 * Reads desc->gamma, sink_blocks, local_blocks, hq, seq, block (not dtype).
 */
bsp_status bsp_mask(const bsp_desc *desc, const float *score, const uint8_t *user_mask,
                    uint8_t *mask, int32_t *kv_idx, int32_t *kv_cnt, void *stream);

/*
 * bsp_score_mask - stages 1 and 2 (threshold path) in one pass: exactly
 * bsp_score followed by bsp_mask without a caller mask, every output bit for
 * bit the same (FlashPrefill summary page, section 3 "Max-based Dynamic
 * Thresholding": the threshold is gamma times the row's peak score, which
 * the score pass already holds when it normalises a row: the peak of P is
 * 1 / (the row's sum of exp), so the mask is decided as P is written and P
 * is never read back; Appendix B: the three stages in order).
 *
 * q, k, q_pool, k_pool, score: as for bsp_score (all written)
 * mask, kv_idx, kv_cnt:        as for bsp_mask (mask may be NULL)
 * Reads desc->gamma, sink_blocks and local_blocks like bsp_mask.
 */
bsp_status bsp_score_mask(const bsp_desc *desc, const void *q, const void *k, float *q_pool,
                          float *k_pool, float *score, uint8_t *mask, int32_t *kv_idx,
                          int32_t *kv_cnt, void *stream);

/*
 * bsp_score_rescue - rescue branch of the scores (thelatestinai page,
 * RBS-Attention abstract: a block centroid can hide one highly relevant key;
 * a rescue branch built on the maximum key-block radius flags such blocks).
 * The page gives no formula; this library computes
 *   k_radius[g][J] = max over the valid keys k of block J of ||k - Kbar[g][J]||
 *   R[h][I][J]     = c * (Qbar[h][I] . Kbar[g][J] + ||Qbar[h][I]|| * k_radius[g][J])
 * (an upper bound on c * Qbar . k for every key k of the block, by
 * Cauchy-Schwarz) and, like bsp_score, its softmax over J <= I:
 *   rescue[h][I][J] = exp(R - max_J' R) / sum_{J' <= I} exp(R - max_J' R), 0 for J > I.
 *
 * k:        device, storage dtype, [hkv][seq][d] (re-read for the radii)
 * q_pool, k_pool: device float, as written by bsp_score on the same inputs
 * k_radius: device float [hkv][nb]      (written)
 * rescue:   device float [hq][nb][nb]   (written, every entry)
 * Needs desc->k_scale for fp8 (q_scale and v_scale are not read).
 */
bsp_status bsp_score_rescue(const bsp_desc *desc, const void *k, const float *q_pool,
                            const float *k_pool, float *k_radius, float *rescue, void *stream);

/*
 * bsp_mask_dual - the two branches thresholded independently and their masks
 * combined (RBS-Attention abstract).  For J <= I:
 *   keep = score[h][I][J]  >= desc->gamma  * max_J'<=I score[h][I][J']
 *       OR rescue[h][I][J] >= gamma_rescue * max_J'<=I rescue[h][I][J']
 *       OR J < sink_blocks OR I - J < local_blocks
 * and 0 for J > I.  Outputs and their layout as for bsp_mask.
 *
 * score:   device float [hq][nb][nb] from bsp_score (or bsp_score_arith)
 * rescue:  device float [hq][nb][nb] from bsp_score_rescue
 * gamma_rescue: 0 <= gamma_rescue <= 1
 */
bsp_status bsp_mask_dual(const bsp_desc *desc, const float *score, const float *rescue,
                         float gamma_rescue, uint8_t *mask, int32_t *kv_idx, int32_t *kv_cnt,
                         void *stream);

/*
 * bsp_attn_fwd - stage 3, block-sparse attention (Appendix B "Block Sparse
 * Attention": iterate only over the selected blocks, causal masking where
 * required, online softmax, final normalisation).
 *
 * For every query token i of block I of head h, over the tokens j of the key
 * blocks listed in kv_idx[h][I][0 .. kv_cnt[h][I]) with j <= i:
 *   o[h][i][:] = sum_j softmax_j(c * q_i . k_j) * v_j[:]
 *   lse[h][i]  = ln sum_j exp(c * q_i . k_j)      (natural log)
 * An empty set gives o = 0 and lse = -inf.  Block indices must be distinct;
 * entries outside [0, I] are skipped and kv_cnt is clamped to [0, nb], so a
 * malformed list never reads out of bounds.  The order of a row does not
 * change the result beyond rounding.
 *
 * q, k, v:  device, storage dtype (v in bfloat16 for BSP_DTYPE_FP8_E4M3_V_BF16);
 *           the fp8 dtypes need all three desc scales
 * kv_idx, kv_cnt: device, as produced by bsp_mask; both NULL = dense causal
 *           (every J <= I); one NULL and not the other is an error
 * o:        device [hq][seq][d]; float for BSP_DTYPE_F32, bfloat16 otherwise
 * lse:      device float [hq][seq], or NULL
 * Arithmetic: f32 inputs use fp32 FMA; bf16 and fp8 use MFMA with fp32
 * accumulation and an fp32 softmax.
 */
bsp_status bsp_attn_fwd(const bsp_desc *desc, const void *q, const void *k, const void *v,
                        const int32_t *kv_idx, const int32_t *kv_cnt, void *o, float *lse,
                        void *stream);

/*
 * bsp_calibrate_gamma - host helper that picks the threshold factor for a
 * target share of kept blocks (Appendix A "Hyperparameter Configurations":
 * the single threshold hyperparameter is calibrated on computational density,
 * about 70% at 4K, with block size and structural retention held fixed).
 *
 * density(gamma) = sum of kv_cnt / (hq * nb * (nb + 1) / 2) for the masks
 * bsp_mask builds from `score` with desc's sink_blocks and local_blocks.  It
 * never increases with gamma (the kept sets nest), so bisection on [0, 1]
 * (midpoints in float) finds the largest gamma, to within tol, whose density
 * is at least target; if gamma = 1 already keeps target, the result is 1.
 *
 * score:     device float [hq][nb][nb] from bsp_score
 * target:    0 < target <= 1
 * tol:       0 < tol < 1; bisection stops when the bracket is this narrow
 * mask, kv_idx, kv_cnt: device work buffers as for bsp_mask (mask may be
 *            NULL); on return they hold bsp_mask's result at *gamma_out
 * cnt_host:  host int32 [hq * nb], staging for the counts
 * gamma_out, density_out: host; the chosen gamma and its density
 * Blocks the calling thread: every step launches the mask kernel on stream,
 * copies the counts to cnt_host and waits for the stream.  desc->gamma is not
 * read.  Allocates nothing.  seq == 0 gives gamma 1 and density 1.
 */
bsp_status bsp_calibrate_gamma(const bsp_desc *desc, const float *score, float target, float tol,
                               uint8_t *mask, int32_t *kv_idx, int32_t *kv_cnt, int32_t *cnt_host,
                               float *gamma_out, float *density_out, void *stream);

/*
 * Packed variable-length batch over a paged K/V cache (FlashPrefill V2
 * abstract on the thelatestinai page: paged KV cache and continuous batching
 * for serving).  Sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1] of
 * q, o and lse ([heads][desc->seq][d], desc->seq = total tokens) and query
 * blocks cu_blocks[s] .. cu_blocks[s+1] (ceil(len_s / block) of them).  Its
 * key block J lives in cache page page_table[s][J]; the caches are laid out
 * [pages][hkv][block][d] in the storage dtype (one page = one key block).
 * The device arrays are the caller's contract (the host never reads them):
 * cu_seqlens[0] = 0, nondecreasing, cu_seqlens[nseq] = desc->seq;
 * cu_blocks[0] = 0, cu_blocks[nseq] = total_blocks; every page index valid.
 */
typedef struct {
  const int32_t *cu_seqlens;  /* device [nseq + 1] */
  const int32_t *cu_blocks;   /* device [nseq + 1] */
  const int32_t *page_table;  /* device [nseq][max_pages] */
  int32_t nseq;               /* >= 1 */
  int32_t total_blocks;       /* query blocks in the batch, >= 0 */
  int32_t max_pages;          /* row length of page_table, >= 1 */
  int32_t idx_stride;         /* row stride of kv_idx, >= 1 (>= a sequence's block count) */
  const int32_t *block_order; /* device [total_blocks], optional: a permutation of the batch's
                                 query blocks in launch order (heaviest first balances the
                                 tail); NULL = descending batch index */
} bsp_varlen;

/*
 * bsp_attn_fwd_varlen - bsp_attn_fwd for a packed batch over a paged cache.
 * Per sequence, exactly bsp_attn_fwd on its own tokens: query block I of
 * sequence s and head h reads its kept key blocks (indices local to s, in
 * [0, I]) from kv_idx[(h * total_blocks + cu_blocks[s] + I) * idx_stride ..]
 * with count kv_cnt[h * total_blocks + cu_blocks[s] + I]; both NULL = dense
 * causal.  A sequence's last page may be partly filled: rows past the
 * sequence end are never read.
 *
 * q:        device [hq][desc->seq][d], storage dtype (bf16 or fp8)
 * k_cache, v_cache: device [pages][hkv][block][d], storage dtype (v_cache
 *           in bfloat16 for BSP_DTYPE_FP8_E4M3_V_BF16)
 * o, lse:   as for bsp_attn_fwd, over the packed tokens
 * fp32 inputs return BSP_ERR_UNSUPPORTED.
 */
bsp_status bsp_attn_fwd_varlen(const bsp_desc *desc, const bsp_varlen *vl, const void *q,
                               const void *k_cache, const void *v_cache, const int32_t *kv_idx,
                               const int32_t *kv_cnt, void *o, float *lse, void *stream);

/*
 * bsp_score_varlen - bsp_score for a packed batch over a paged K cache
 * (FlashPrefill V2 abstract: paged KV cache and continuous batching; the
 * stage itself as for bsp_score).  Per sequence s, exactly bsp_score on its
 * own tokens; the block means of all sequences are laid out in batch block
 * order and each sequence's score matrix occupies rows
 * cu_blocks[s] .. cu_blocks[s+1] of a [hq][total_blocks][idx_stride] array:
 *   q_pool[h][gb][:] = mean of Q[h][t][:] over the tokens t of batch block gb
 *   k_pool[g][gb][:] = mean of the valid rows of cache page page_table[s][I]
 *   score[h][gb][J]  = the row softmax of c * q_pool[h][gb] . k_pool[g][cb + J]
 *                      over J <= I, 0 for I < J < nb_s
 * with gb = cb + I, cb = cu_blocks[s], nb_s = cu_blocks[s+1] - cb.  Entries
 * J >= nb_s of a row are not written.  The scores are fp32 dot products.
 *
 * q:        device [hq][desc->seq][d], storage dtype (desc->seq = tokens in the batch)
 * k_cache:  device [pages][hkv][block][d], storage dtype
 * q_pool:   device float [hq][total_blocks][d]   (written)
 * k_pool:   device float [hkv][total_blocks][d]  (written)
 * score:    device float [hq][total_blocks][idx_stride] (written as above)
 * vl:       as for bsp_attn_fwd_varlen (block_order is not read);
 *           idx_stride >= the largest nb_s
 * Needs desc->q_scale and desc->k_scale for fp8 (v_scale is not read).
 */
bsp_status bsp_score_varlen(const bsp_desc *desc, const bsp_varlen *vl, const void *q,
                            const void *k_cache, float *q_pool, float *k_pool, float *score,
                            void *stream);

/*
 * bsp_mask_varlen - bsp_mask for a packed batch: per sequence, exactly
 * bsp_mask on its rows (the threshold against its own row maximum, sink and
 * local window counted from its own first block), with rows gb =
 * cu_blocks[s] + I of stride idx_stride.  The lists it writes are what
 * bsp_attn_fwd_varlen reads: block indices local to the sequence.
 *
 * score:     device float [hq][total_blocks][idx_stride] from bsp_score_varlen;
 *            may be NULL iff user_mask is given
 * user_mask: device uint8 [hq][total_blocks][idx_stride] or NULL (replaces the
 *            threshold and the forced blocks, ANDed with causal)
 * mask:      device uint8 [hq][total_blocks][idx_stride] or NULL; entries
 *            J < nb_s of each row are written
 * kv_idx:    device int32 [hq][total_blocks][idx_stride]; first kv_cnt entries
 * kv_cnt:    device int32 [hq][total_blocks]
 * vl:        cu_seqlens, cu_blocks, nseq, total_blocks, idx_stride are read
 */
bsp_status bsp_mask_varlen(const bsp_desc *desc, const bsp_varlen *vl, const float *score,
                           const uint8_t *user_mask, uint8_t *mask, int32_t *kv_idx,
                           int32_t *kv_cnt, void *stream);

/* Static description of a status code (host, never NULL). */
/*
 * bsp_widen_e4m3 - dst[i] = the bfloat16 value of OCP e4m3fn code src[i],
 * for 0 <= i < n (FP8 inference of the FlashPrefill V2 abstract on the
 * thelatestinai page: e4m3 operands; the P V product runs on bf16 matrix
 * cores, so V is widened once here rather than inside every attention
 * workgroup).  Exact: every e4m3 value is a bf16 value.  Scales are not
 * applied (V = dst * v_scale[g] as for the codes).
 *
 * src:    device, n bytes, 16-byte aligned
 * dst:    device, n bfloat16 (2n bytes), 16-byte aligned; must not overlap src
 * n:      >= 0; 0 is a no-op
 * Errors: BSP_ERR_BAD_SHAPE for n < 0, BSP_ERR_NULL_POINTER, BSP_ERR_BAD_VALUE
 * for a misaligned or overlapping pair.  Allocates nothing.
 */
bsp_status bsp_widen_e4m3(const void *src, void *dst, int64_t n, void *stream);

const char *bsp_status_string(int32_t status);

/* BSP_ABI_VERSION of the loaded library. */
int32_t bsp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSP_H */
