/*
 * btq.h -- C ABI of libbtq, the hybrid int4/BF16 codec for tensor-parallel
 * partial sums on AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the page "Revolutionizing LLM Inference: The Power of
 * Efficient Low-Bit Communication" (aiexpert.world), a summary of the paper
 * "Towards Efficient Low-Bit Communication for Tensor Parallel LLM Inference".
 * Its section "The Hybrid Quantization Algorithm" gives three steps:
 *   Calibration  -- per-feature parameters from moving averages of the
 *                   minimum and maximum observed on each device;
 *   Selection    -- rank features by quantization range and keep a number
 *                   of them in BF16;
 *   Inference    -- the selected features stay BF16 and the others are sent
 *                   as 4-bit integers; after communication everything is
 *                   converted back and summed across devices.
 * Section "Combating Quantization Errors with Tensor Parallelism" places the
 * quantization on each device's partial sum, before the sum.
 *
 * Four calls follow those steps: btq_calib_update, btq_select_outliers,
 * btq_compress_pack (the sender) and btq_decompress_reduce (the receiver).
 * Here all P shards' partial sums sit in one GPU's HBM, so the exchange
 * between devices is the identity: the buffers written by btq_compress_pack
 * are the ones read by btq_decompress_reduce. The other calls widen the path:
 * a bf16-output receiver, other readings of the selection step and a packed
 * row pitch.
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or from PyTorch) to
 *    caller-owned, contiguous, row-major memory with the last index fastest.
 *    The library never allocates, frees or keeps them.
 *  - bf16 values are raw 16-bit patterns (uint16_t).
 *  - A pointer must be aligned to its element type (BTQ_ERR_ALIGN
 *    otherwise). Fast kernels run when x, packed, outliers and y are 16-byte
 *    aligned, the per-feature arrays 16-byte aligned, and H and H-k are
 *    multiples of 8 (the receivers: up to 8 shards per launch, see
 *    btq_decompress_reduce); every other layout runs on a general kernel
 *    that is correct but much slower.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call checks its arguments on the host, enqueues its kernels on
 *    `stream` and returns. It does not synchronize, print, throw or abort.
 *    The library holds no mutable global state, so calls on different
 *    streams may run concurrently as long as their buffers do not overlap.
 *  - Return value: BTQ_OK (0) or a negative btq_status. On an argument or
 *    shape error nothing is enqueued and no HIP call is made. A fault while
 *    the kernels run surfaces at the caller's next synchronization.
 *  - Sizes: 1 <= P <= 65535, 1 <= H <= 2^30, 0 <= k <= H, T >= 0, and
 *    P*T*H < 2^62. T == 0 is an empty batch: compress and decompress do
 *    nothing, and calibration rejects it (its min/max would be undefined).
 *  - Floating point: every fp32 step is one IEEE round-to-nearest-even
 *    operation. Divisions are correctly rounded. Nothing is flushed to zero.
 *    Inputs must be finite; NaN and Inf give unspecified (but in-bounds)
 *    results.
 *
 * Layouts
 *  x            bf16 [P,T,H]     partial sums, one [T,H] block per shard
 *  run_min/max  fp32 [P,H]
 *  scale        fp32 [P,H]       4-bit step of feature h on shard p
 *  rscale       fp32 [P,H]       1/scale
 *  zero_point   u8   [P,H]       0..15
 *  outlier_idx  i32  [k]         BF16 features, ascending h
 *  fmap         i32  [H]         fmap[h] = j (int4 slot j of h), or -1-i when
 *                                h = outlier_idx[i]
 *  cmap         i32  [H-k]       cmap[j] = h of int4 slot j, ascending
 *  packed       u8   [P,T,Bq]    Bq = btq_packed_row_bytes(H,k) = ceil((H-k)/2);
 *                                slot 2b in the low nibble of byte b, slot
 *                                2b+1 in the high nibble; an odd H-k leaves
 *                                the last high nibble 0
 *  outliers     bf16 [P,T,k]     outliers[p,t,i] = x[p,t,outlier_idx[i]]
 *  y            fp32 [T,H]       (bf16 [T,H] for the bf16-output receiver)
 */
#ifndef BTQ_H
#define BTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BTQ_OK = 0,
  BTQ_ERR_ARG = -1,        /* null pointer, or momentum outside [0,1) / NaN    */
  BTQ_ERR_SHAPE = -2,      /* P, T, H, k or the pitch out of range              */
  BTQ_ERR_ALIGN = -3,      /* pointer not aligned to its element type           */
  BTQ_ERR_WORKSPACE = -4,  /* workspace smaller than the *_workspace_bytes size */
  BTQ_ERR_HIP = -5,        /* a HIP call failed (hipGetLastError, cleared)      */
  BTQ_ERR_SCRATCH = -6     /* sizes beyond btq_calib_update_noalloc's scratch    */
} btq_status;

/*
 * Calibration -- "The Hybrid Quantization Algorithm", Calibration bullet.
 *
 * For every shard p and feature h, takes the batch minimum and maximum over
 * the T tokens of x[p,:,h]. Then it updates the running extremes:
 *   first_batch != 0 : run = batch value
 *   otherwise        : run = fl(fl(a*run) + fl(c*batch)),  a = momentum,
 *                      c = fl(1 - a), all fp32 (moving average; the page
 *                      gives no formula -- the momentum weights the old value)
 *   x        bf16 [P,T,H]   in, T >= 1
 *   momentum in [0,1): the weight of the running value (BTQ_ERR_ARG
 *            otherwise, NaN included)
 *   run_min  fp32 [P,H]     in/out (ignored on input when first_batch != 0)
 *   run_max  fp32 [P,H]     in/out
 *   workspace  device scratch of at least btq_calib_workspace_bytes(P,T,H)
 *              bytes (may be NULL if that size is 0); its contents are
 *              overwritten and need no initial value.
 * Batch extremes are exact, and -0 and +0 count as equal. The result does
 * not depend on how the kernels split the token axis.
 */
int btq_calib_update(const uint16_t *x, int64_t P, int64_t T, int64_t H,
                     float momentum, int first_batch,
                     float *run_min, float *run_max,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for btq_calib_update (0 for invalid sizes). */
size_t btq_calib_workspace_bytes(int64_t P, int64_t T, int64_t H);

/*
 * btq_calib_update without a workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, checks and results are those of btq_calib_update, bit for bit
 * (the result does not depend on how the token axis is split). The partial
 * extremes live in a static device array of BTQ_NOALLOC_SCRATCH_BYTES on
 * each GPU, held until the process ends; the call uses as many token chunks
 * as that array holds, so 2*P*H*4 bytes must fit it (P*H <= 2^20), else it
 * returns BTQ_ERR_SCRATCH and enqueues nothing. It calls no hipMalloc or
 * hipFree; its first call on a device looks up the array's address there.
 * Every call on one GPU uses that GPU's one array: calls that may overlap
 * on one GPU (different streams, or host threads) race and must be ordered
 * by the caller. Nothing in the array needs an initial value.
 */
#define BTQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int btq_calib_update_noalloc(const uint16_t *x, int64_t P, int64_t T, int64_t H,
                             float momentum, int first_batch,
                             float *run_min, float *run_max, void *stream);

/*
 * Selection -- "The Hybrid Quantization Algorithm", Calibration bullet
 * (per-feature parameters) and Selection bullet (rank by range, keep k).
 *
 * Per (p,h):  lo = min(run_min,0), hi = max(run_max,0), width = hi - lo,
 *             scale = width/15 (1 if below 2^-126), rscale = 1/scale,
 *             zero_point = clamp(rint_half_even(-lo/scale), 0, 15).
 * Per h:      score = width[0,h] + width[1,h] + ... (fp32, p ascending).
 * The k features with the highest score are kept in BF16 (ties: lower h
 * first). They are shared by all shards, because the receiver must know
 * every sender's layout.
 *   run_min, run_max  fp32 [P,H]  in
 *   scale, rscale     fp32 [P,H]  out
 *   zero_point        u8   [P,H]  out, values 0..15
 *   outlier_idx       i32  [k]    out, the BF16 features in ascending h
 *   fmap              i32  [H]    out
 *   cmap              i32  [H-k]  out
 *   workspace  at least btq_select_workspace_bytes(P,H,k) bytes of scratch.
 * Pointers for zero-length outputs (k == 0, or k == H for cmap) may be NULL.
 */
int btq_select_outliers(const float *run_min, const float *run_max,
                        int64_t P, int64_t H, int64_t k,
                        float *scale, float *rscale, uint8_t *zero_point,
                        int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes for the ranked selections: P*H floats (0 for invalid sizes). */
size_t btq_select_workspace_bytes(int64_t P, int64_t H, int64_t k);

/*
 * Sender side of inference -- "The Hybrid Quantization Algorithm", Inference
 * bullet; quantization before the sum per "Combating Quantization Errors
 * with Tensor Parallelism".
 *
 * For each token row (p,t), the int4 slots j = 0..H-k-1 take feature
 * h = cmap[j]:  q = clamp(rint_half_even(fl(x*rscale[p,h])) + zero_point[p,h],
 * 0, 15), packed two per byte into a row of Bq = btq_packed_row_bytes(H,k)
 * bytes (rows follow each other with no gap). The BF16 features are copied
 * bit for bit: outliers[p,t,i] = x[p,t,outlier_idx[i]].
 *   x            bf16 [P,T,H]    in
 *   rscale       fp32 [P,H], zero_point u8 [P,H]   in (from a selection call)
 *   outlier_idx  i32 [k], cmap i32 [H-k]           in (from a selection call)
 *   packed       u8   [P,T,Bq]   out
 *   outliers     bf16 [P,T,k]    out
 * The maps are trusted: outlier_idx and cmap must partition 0..H-1, each in
 * ascending order, as the selection calls write them.
 */
int btq_compress_pack(const uint16_t *x, int64_t P, int64_t T, int64_t H, int64_t k,
                      const float *rscale, const uint8_t *zero_point,
                      const int32_t *outlier_idx, const int32_t *cmap,
                      uint8_t *packed, uint16_t *outliers, void *stream);

/*
 * Receiver side of inference -- "The Hybrid Quantization Algorithm",
 * Inference bullet (convert back, sum across devices).
 *
 * y[t,h] = sum over p = 0..P-1 of term_p, in fp32, where
 *   fmap[h] = j >= 0:  term_p = (q_p - zero_point[p,h]) * scale[p,h], q_p
 *                      the code of slot j in packed row (p,t)
 *   fmap[h] = -1-i:    term_p = the bf16 value outliers[p,t,i]
 * Features kept in BF16 are summed in p order from +0, so they equal a
 * sequential fp32 sum bit for bit. int4 features are evaluated as
 * fma(q_p, scale, acc) from the constant -sum_p zero_point*scale, which
 * stays within 1e-3*|y| + 1e-2*max_p scale[p,h] of the sequential sum.
 * (The 512 features of a block that holds a scale of 2^104 or more are
 * computed as the sequential sum itself.)
 *   packed [P,T,Bq], outliers [P,T,k]   in, as written by btq_compress_pack
 *   scale fp32 [P,H], zero_point u8 [P,H], fmap i32 [H]   in
 *   y      fp32 [T,H]   out
 * Fast kernel: H a multiple of 8, Bq a multiple of 4 and at least 8,
 * 16-byte aligned scale, fmap and y, and the message and outlier block of
 * every 8 shards under 2^31 bytes. More than 8 shards, or a message past
 * 2^31 bytes, run it once per group of shards (8, or fewer so that each
 * group's message fits), in shard order; each later group starts from the y
 * the earlier ones wrote (y is read as well as written), so BF16 features
 * keep their sequential sum. Anything else takes a general kernel (correct,
 * much slower, and exactly the sequential sum).
 */
int btq_decompress_reduce(const uint8_t *packed, const uint16_t *outliers,
                          int64_t P, int64_t T, int64_t H, int64_t k,
                          const float *scale, const uint8_t *zero_point, const int32_t *fmap,
                          float *y, void *stream);

/* Code bytes per packed row: ceil((H-k)/2); -1 if H < 1 or k is outside [0,H]. */
int64_t btq_packed_row_bytes(int64_t H, int64_t k);

/* ------------------------------------------------------------------------
 * Widened path.
 * ------------------------------------------------------------------------ */

/*
 * Receiver with bf16 output -- "The Hybrid Quantization Algorithm",
 * Inference bullet (after communication the tensors convert back to BF16).
 *
 * The same sum as btq_decompress_reduce, rounded once from fp32 to bf16
 * (round to nearest even): y[t,h] = bf16(fp32 sum), bit for bit the rounding
 * of what btq_decompress_reduce writes. y is bf16 [T,H] (uint16 bits), 2-byte
 * aligned (16-byte aligned for the fast kernel). More than 8 shards take the
 * general kernel here (there is no fp32 buffer to carry a group's sum): the
 * result is then the rounding of the sequential sum, bit for bit.
 */
int btq_decompress_reduce_bf16(const uint8_t *packed, const uint16_t *outliers,
                               int64_t P, int64_t T, int64_t H, int64_t k,
                               const float *scale, const uint8_t *zero_point,
                               const int32_t *fmap, uint16_t *y, void *stream);

/* How a feature's P per-shard ranges become its rank score. */
typedef enum {
  BTQ_SCORE_SUM = 0,   /* width[0,h] + width[1,h] + ... (fp32, p ascending)    */
  BTQ_SCORE_MAX = 1    /* max over p of width[p,h] (exact)                     */
} btq_score_rule;

/*
 * btq_select_outliers with a choice of rank score -- "The Hybrid
 * Quantization Algorithm", Selection bullet: features are ranked by their
 * quantization ranges, which are per device, and the page does not say how
 * one feature's ranges on the P devices combine. BTQ_SCORE_SUM is the
 * reading btq_select_outliers uses; BTQ_SCORE_MAX ranks a feature by its
 * widest shard. Only the score (and so the set and maps) changes; every
 * other output and argument is as in btq_select_outliers. Any other
 * score_rule returns BTQ_ERR_ARG.
 */
int btq_select_outliers_rule(const float *run_min, const float *run_max,
                             int64_t P, int64_t H, int64_t k, int score_rule,
                             float *scale, float *rscale, uint8_t *zero_point,
                             int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Selection with the BF16 set given by the caller -- the comparison in
 * "Key Observations and Future Directions" (features picked at random
 * instead of by range), and any other selection rule computed elsewhere.
 *
 * Same parameters and maps as btq_select_outliers, with the ranking
 * replaced by the given set:
 *   features      i32 [k]  in, HOST memory: k distinct features in
 *                          ascending order, each in [0, H). Anything else
 *                          returns BTQ_ERR_ARG and enqueues nothing.
 *   outlier_idx   i32 [k]  out (device): a copy of features, made by a
 *                          host-to-device copy on `stream`. Keep `features`
 *                          unchanged until the stream has passed this call.
 * Every other argument is as in btq_select_outliers. No workspace is needed.
 */
int btq_select_features(const float *run_min, const float *run_max,
                        int64_t P, int64_t H, int64_t k, const int32_t *features,
                        float *scale, float *rscale, uint8_t *zero_point,
                        int32_t *outlier_idx, int32_t *fmap, int32_t *cmap, void *stream);

/*
 * Per-shard BF16 sets -- a second reading of "The Hybrid Quantization
 * Algorithm", Selection bullet: the ranges that rank features are per
 * device, so every shard keeps its own k widest features (ranked by its own
 * range, ties to the lower h) in BF16. The message keeps its size (k BF16
 * values and H-k codes per row), but each shard lays it out by its own map,
 * so the receiver reads every shard's map.
 *
 * btq_select_outliers_per_shard: parameters as in btq_select_outliers, plus
 *   outlier_idx  i32 [P,k]      out, shard p's BF16 features, ascending h
 *   fmap         i32 [P,H]      out, shard p's map (slot j, or -1-i)
 *   cmap         i32 [P,H-k]    out, shard p's int4 features, ascending h
 *   workspace    at least btq_select_workspace_bytes(P,H,k) bytes.
 * btq_compress_pack_per_shard: btq_compress_pack with outlier_idx [P,k] and
 *   cmap [P,H-k]; row (p,t) is coded with shard p's maps. Same layouts.
 * btq_decompress_reduce_per_shard: btq_decompress_reduce with fmap [P,H]:
 *   term_p follows shard p's map. Features BF16 on every shard are summed in
 *   shard order from +0, exactly; the others are within the receiver's
 *   tolerance of the sequential sum. Past 8 shards (or a message past 2^31
 *   bytes) the fast kernel runs once per group of up to 6 shards, each
 *   later group adding to y as in btq_decompress_reduce.
 */
int btq_select_outliers_per_shard(const float *run_min, const float *run_max,
                                  int64_t P, int64_t H, int64_t k,
                                  float *scale, float *rscale, uint8_t *zero_point,
                                  int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                                  void *workspace, size_t workspace_bytes, void *stream);
int btq_compress_pack_per_shard(const uint16_t *x, int64_t P, int64_t T, int64_t H, int64_t k,
                                const float *rscale, const uint8_t *zero_point,
                                const int32_t *outlier_idx, const int32_t *cmap,
                                uint8_t *packed, uint16_t *outliers, void *stream);
int btq_decompress_reduce_per_shard(const uint8_t *packed, const uint16_t *outliers,
                                    int64_t P, int64_t T, int64_t H, int64_t k,
                                    const float *scale, const uint8_t *zero_point,
                                    const int32_t *fmap, float *y, void *stream);

/* Set layout of the *_ex calls: one set for all shards, or one per shard. */
typedef enum { BTQ_SETS_SHARED = 0, BTQ_SETS_PER_SHARD = 1 } btq_sets;
/* Output type of btq_decompress_reduce_ex. */
typedef enum { BTQ_Y_F32 = 0, BTQ_Y_BF16 = 1 } btq_ytype;

/*
 * The sender and receiver with every option: the set layout, the output
 * type, and a packed row pitch. Row (p,t) of the message starts at byte
 * (p*T+t)*packed_pitch; its first Bq bytes hold the codes and the sender
 * writes the rest of the row as zeros, which the receiver never reads.
 * packed_pitch = Bq is the layout of btq_compress_pack; btq_packed_pitch(H,k)
 * (Bq rounded up to 128) starts every row on a cache line, so the kernels
 * write and read whole lines (the message grows by less than 128 bytes a
 * row). packed_pitch < Bq returns BTQ_ERR_SHAPE. The fast kernels need a
 * pitch that is a multiple of 4.
 * For sets == BTQ_SETS_PER_SHARD outlier_idx, cmap and fmap carry one set
 * per shard as in the *_per_shard calls. y_type BTQ_Y_BF16 makes y bf16
 * [T,H] (uint16 bits). Any other sets or y_type returns BTQ_ERR_ARG.
 */
int btq_compress_pack_ex(const uint16_t *x, int64_t P, int64_t T, int64_t H, int64_t k,
                         const float *rscale, const uint8_t *zero_point,
                         const int32_t *outlier_idx, const int32_t *cmap, int sets,
                         uint8_t *packed, int64_t packed_pitch, uint16_t *outliers,
                         void *stream);
int btq_decompress_reduce_ex(const uint8_t *packed, int64_t packed_pitch,
                             const uint16_t *outliers, int64_t P, int64_t T, int64_t H, int64_t k,
                             const float *scale, const uint8_t *zero_point, const int32_t *fmap,
                             int sets, void *y, int y_type, void *stream);

/* Recommended packed row pitch for the *_ex calls: the code bytes rounded up
 * to a multiple of 128; -1 for invalid sizes. */
int64_t btq_packed_pitch(int64_t H, int64_t k);

/* Static text for a btq_status value (never NULL). */
const char *btq_status_str(int status);

/* Library version, "major.minor.patch". */
const char *btq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BTQ_H */
