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
 * One call per step. Here all P shards' partial sums sit in one GPU's HBM,
 * so the exchange between devices is the identity: the buffers written by
 * btq_compress_pack are the ones read by btq_decompress_reduce.
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or from PyTorch) to
 *    caller-owned, contiguous, row-major memory with the last index fastest.
 *    The library never allocates, frees or keeps them.
 *  - bf16 values are raw 16-bit patterns (uint16_t).
 *  - A pointer must be aligned to its element type. Faster paths are taken
 *    when x/packed/outliers/y are 16-byte aligned and H, H-k are multiples
 *    of 8; every other layout runs on a slower general path.
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
  BTQ_ERR_ARG = -1,        /* null pointer, or momentum outside [0,1] / NaN    */
  BTQ_ERR_SHAPE = -2,      /* P, T, H or k out of range                         */
  BTQ_ERR_ALIGN = -3,      /* pointer not aligned to its element type           */
  BTQ_ERR_WORKSPACE = -4,  /* workspace smaller than the *_workspace_bytes size */
  BTQ_ERR_HIP = -5         /* a kernel launch failed (hipGetLastError, cleared)  */
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
 *   x        bf16 [P,T,H]   in
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

size_t btq_calib_workspace_bytes(int64_t P, int64_t T, int64_t H);

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
 *   fmap              i32  [H]    out, fmap[h] = j (the int4 slot of h), or
 *                                 -1-i when h = outlier_idx[i]
 *   cmap              i32  [H-k]  out, cmap[j] = h of int4 slot j (ascending)
 *   enc_table   fp32 [P, H-k, 2]  out: (rscale, zero_point) of slot j's
 *                                 feature cmap[j], per shard: the sender's
 *                                 parameters in message order
 *   dec_table   fp32 [2P+1, H-k]  out: rows 0..P-1 scale, rows P..2P-1
 *                                 zero_point, row 2P the per-slot constant
 *                                 -sum_p zero_point*scale (fp32 steps in
 *                                 shard order): the receiver's parameters in
 *                                 message order
 *   workspace  at least btq_select_workspace_bytes(P,H) bytes of scratch.
 * The two tables only reorder the per-feature parameters (and add one
 * derived sum), so the hot kernels read them with contiguous vector loads.
 * Pointers for zero-length outputs (k == 0, or k == H for cmap and the
 * tables) may be NULL. The tables should be 16-byte aligned (other
 * alignments run on the general path).
 */
int btq_select_outliers(const float *run_min, const float *run_max,
                        int64_t P, int64_t H, int64_t k,
                        float *scale, float *rscale, uint8_t *zero_point,
                        int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                        float *enc_table, float *dec_table,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes for the ranked selections: P*H floats (0 for invalid sizes). */
size_t btq_select_workspace_bytes(int64_t P, int64_t H);

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
 * widest shard. Only the score (and so the set, maps and tables) changes;
 * every other output and argument is as in btq_select_outliers. Any other
 * score_rule returns BTQ_ERR_ARG.
 */
int btq_select_outliers_rule(const float *run_min, const float *run_max,
                             int64_t P, int64_t H, int64_t k, int score_rule,
                             float *scale, float *rscale, uint8_t *zero_point,
                             int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                             float *enc_table, float *dec_table,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Selection with the BF16 set given by the caller -- the comparison in
 * "Key Observations and Future Directions" (features picked at random
 * instead of by range), and any other selection rule computed elsewhere.
 *
 * Same parameters, maps and tables as btq_select_outliers, with the
 * ranking replaced by the given set:
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
                        int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                        float *enc_table, float *dec_table, void *stream);

/* Floats in enc_table (2*P*(H-k)) and dec_table ((2P+1)*(H-k)); -1 for
 * invalid sizes. */
int64_t btq_enc_table_floats(int64_t P, int64_t H, int64_t k);
int64_t btq_dec_table_floats(int64_t P, int64_t H, int64_t k);

/*
 * Sender side of inference -- "The Hybrid Quantization Algorithm", Inference
 * bullet; quantization before the sum per "Combating Quantization Errors
 * with Tensor Parallelism".
 *
 * For each token row (p,t), the int4 slots j = 0..H-k-1 take feature
 * h = cmap[j]:  q = clamp(rint_half_even(fl(x*rscale)) + zero_point, 0, 15),
 * with (rscale, zero_point) = enc_table[p,j]. Codes are packed two per byte:
 * slot 2b in the low nibble of byte b, slot 2b+1 in the high nibble. An odd
 * H-k leaves the last high nibble 0. The BF16 features are copied bit for
 * bit: outliers[p,t,i] = x[p,t,outlier_idx[i]].
 *   x          bf16 [P,T,H]                       in
 *   enc_table  fp32 [P,H-k,2]                     in (from a selection call)
 *   outlier_idx i32 [k], cmap i32 [H-k]           in (from a selection call)
 *   packed     u8   [P,T,packed_pitch]            out: row (p,t) holds its
 *              Bq = btq_packed_row_bytes(H,k) code bytes, then packed_pitch-Bq
 *              zero bytes
 *   packed_pitch  bytes per packed row, >= Bq. btq_packed_pitch(H,k) (Bq
 *              rounded up to 128) lets every row start on a cache line, so
 *              the kernels write whole lines; Bq gives the densest message.
 *   outliers   bf16 [P,T,k]                       out
 * The maps are trusted: outlier_idx and cmap must partition 0..H-1, each in
 * ascending order, as the selection calls write them.
 */
int btq_compress_pack(const uint16_t *x, int64_t P, int64_t T, int64_t H, int64_t k,
                      const float *enc_table, const int32_t *outlier_idx,
                      const int32_t *cmap, uint8_t *packed, int64_t packed_pitch,
                      uint16_t *outliers, void *stream);

/*
 * Receiver side of inference -- "The Hybrid Quantization Algorithm",
 * Inference bullet (convert back, sum across devices).
 *
 * y[t,h] = sum over p = 0..P-1 of term_p, in fp32, where
 *   int4 feature h = cmap[j]:       term_p = (q_p - zero_point) * scale
 *                                   (q_p = nibble j of packed row (p,t);
 *                                   scale, zero_point from dec_table[.,j])
 *   BF16 feature h = outlier_idx[i]: term_p = the bf16 value outliers[p,t,i]
 * BF16 features are summed in p order starting from 0, so they match a
 * sequential fp32 sum bit for bit. int4 features may be evaluated as
 * fma(q_p, scale, acc) seeded with the table's per-slot constant, which
 * stays within 1e-3*|y| + 1e-2*max_p scale of the sequential sum.
 *   packed, outliers  as written by btq_compress_pack (P shards)  in
 *   packed_pitch      bytes per packed row, >= btq_packed_row_bytes(H,k);
 *                     only the code bytes of a row are read
 *   dec_table fp32 [2P+1,H-k], outlier_idx [k], cmap [H-k]        in
 *   y    fp32 [T,H]  out
 * Kernel choice: P <= 8, H a multiple of 4 and H-k of 8, a pitch that is a
 * multiple of 4, and a message (P*T*pitch bytes, and P*T*k*2 for the BF16
 * block) under 2^31 bytes take the fast kernel. Anything else, such as more
 * than 8 shards or a larger batch (which a caller can also split by tokens),
 * takes a general kernel, which is correct but much slower.
 */
int btq_decompress_reduce(const uint8_t *packed, int64_t packed_pitch,
                          const uint16_t *outliers, int64_t P, int64_t T, int64_t H,
                          int64_t k, const float *dec_table, const int32_t *outlier_idx,
                          const int32_t *cmap, float *y, void *stream);

/*
 * Receiver with bf16 output -- "The Hybrid Quantization Algorithm",
 * Inference bullet (after communication the tensors convert back to BF16).
 *
 * The same sum as btq_decompress_reduce, rounded once from fp32 to bf16
 * (round to nearest even): y[t,h] = bf16(fp32 sum). Arguments, layouts and
 * errors as for btq_decompress_reduce, except:
 *   y    bf16 [T,H] (uint16 bits)  out, 2-byte aligned (8-byte aligned for
 *        the fast path)
 * For BF16 features the result is the bf16 rounding of the exact sequential
 * fp32 sum. For int4 features it is the bf16 rounding of the value that
 * btq_decompress_reduce writes.
 */
int btq_decompress_reduce_bf16(const uint8_t *packed, int64_t packed_pitch,
                               const uint16_t *outliers, int64_t P, int64_t T, int64_t H,
                               int64_t k, const float *dec_table, const int32_t *outlier_idx,
                               const int32_t *cmap, uint16_t *y, void *stream);

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
 *   enc_table    fp32 [P,H-k,2] out, (rscale, zero_point) of cmap[p,j] on p
 *   workspace    at least btq_select_workspace_bytes(P,H) bytes.
 * The receiver reads scale and zero_point by feature, so there is no
 * decoder table.
 *
 * btq_compress_pack_per_shard: btq_compress_pack with outlier_idx [P,k] and
 *   cmap [P,H-k] from btq_select_outliers_per_shard; row (p,t) is coded with
 *   shard p's maps. Same packed and outliers layouts.
 *
 * btq_decompress_reduce_per_shard: y[t,h] = sum over p of the dequantized
 *   value of feature h on shard p: (q - zero_point[p,h]) * scale[p,h], q
 *   being shard p's code of h at slot fmap[p,h], or the BF16 value
 *   outliers[p,t,-1-fmap[p,h]]. scale fp32 [P,H], zero_point u8 [P,H], fmap
 *   i32 [P,H] in; y fp32 [T,H] out. The maps are trusted, as in
 *   btq_decompress_reduce. Kernel choice:
 *   - T > 2, P <= 8, H a multiple of 8, a pitch that is a multiple of 4 and
 *     at least 8, a 4-byte aligned packed, 8-byte aligned zero_point, 16-byte
 *     aligned fmap, scale and y, and message, outlier blocks and maps each
 *     under 2^30 bytes: the lane-window kernel. It seeds each feature with
 *     -sum_p z*s and adds one fma per int4 term, then the BF16 values, so
 *     its output is within fp32 rounding of the sequential sum (features
 *     BF16 on every shard are summed in shard order from +0, exactly);
 *   - otherwise P <= 8 with H a multiple of 4 (same alignments, zero_point
 *     4-byte aligned): a register kernel; any P with H a multiple of 8: a
 *     shard-loop kernel; everything else a per-element kernel. These three
 *     evaluate fl(q - z) * s and add the terms in shard order from +0, so
 *     their outputs agree bit for bit.
 */
int btq_select_outliers_per_shard(const float *run_min, const float *run_max,
                                  int64_t P, int64_t H, int64_t k,
                                  float *scale, float *rscale, uint8_t *zero_point,
                                  int32_t *outlier_idx, int32_t *fmap, int32_t *cmap,
                                  float *enc_table, void *workspace, size_t workspace_bytes,
                                  void *stream);
int btq_compress_pack_per_shard(const uint16_t *x, int64_t P, int64_t T, int64_t H, int64_t k,
                                const float *enc_table, const int32_t *outlier_idx,
                                const int32_t *cmap, uint8_t *packed, int64_t packed_pitch,
                                uint16_t *outliers, void *stream);
int btq_decompress_reduce_per_shard(const uint8_t *packed, int64_t packed_pitch,
                                    const uint16_t *outliers, int64_t P, int64_t T, int64_t H,
                                    int64_t k, const float *scale, const uint8_t *zero_point,
                                    const int32_t *fmap, float *y, void *stream);

/* Code bytes per packed row: ceil((H-k)/2); -1 if H < 1 or k is outside [0,H]. */
int64_t btq_packed_row_bytes(int64_t H, int64_t k);

/* Recommended packed row pitch: the code bytes rounded up to a multiple of
 * 128; -1 for invalid sizes. */
int64_t btq_packed_pitch(int64_t H, int64_t k);

/* Static text for a btq_status value (never NULL). */
const char *btq_status_str(int status);

/* Library version, "major.minor.patch". */
const char *btq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BTQ_H */
