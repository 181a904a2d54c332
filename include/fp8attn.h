/*
 * fp8attn.h - C ABI of libfp8attn.so, an FP8 (E4M3) flash-attention forward
 * for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * What is computed (FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page,
 * the formula for out[a:b, h] and the cu_seqlens / softmax_scale parameters):
 * for every segment [a, b) of cu_seqlens and every head h,
 *
 *     out[a:b, h] = softmax(q[a:b, h] @ k[a:b, h]^T * softmax_scale) @ v[a:b, h]
 *
 * dense and non-causal, head_dim 128, BF16 in and BF16 out.  The method is the
 * one of sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for
 * SM120 GPUs" ("Modifications"): quantize Q/K/V per head to E4M3 in two passes
 * (amax, then pack), then one flash-attention forward with E4M3 operands for
 * both products, FP32 accumulation, an FP32 online softmax and the
 * probabilities packed to E4M3 in registers; the output is rounded to BF16 once.
 *
 * Three calls make one attention:
 *     fp8attn_plan      (host, once per cu_seqlens/heads; synchronous)
 *     fp8attn_quantize  (stream-ordered, no host sync)
 *     fp8attn_forward   (stream-ordered, no host sync)
 *
 * Ownership: the caller owns every large device buffer (q, k, v, out, lse and
 * the workspace).  The library keeps no pointer to any of them after a call
 * returns.  A plan owns only its host tables and a small device copy of them
 * (tens to hundreds of KB), freed by fp8attn_plan_destroy.  A plan may be used
 * from several threads and streams at once provided each concurrent use has
 * its own workspace.
 *
 * Errors: every call returns a status.  Arguments are validated before
 * anything is enqueued, so a non-OK status means no work was launched.
 * fp8attn_last_error() returns a text for the last non-OK status of the
 * calling thread.  A GPU fault inside an enqueued kernel surfaces at the
 * caller's next synchronization, as for any HIP work.
 */
#ifndef FP8ATTN_H
#define FP8ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8ATTN_HEAD_DIM 128

typedef struct fp8attn_plan_s* fp8attn_plan_t;

typedef enum {
  FP8ATTN_OK = 0,
  FP8ATTN_EINVAL = 1,        /* bad argument (NULL, size, stride, alignment, cu_seqlens) */
  FP8ATTN_EUNSUPPORTED = 2,  /* a size beyond the library's limits (32-bit offsets, static buffer) */
  FP8ATTN_ENOMEM = 3,        /* host or device allocation of plan tables failed */
  FP8ATTN_EWORKSPACE = 4,    /* workspace pointer NULL/misaligned or smaller than needed */
  FP8ATTN_EHIP = 5           /* a HIP runtime call or kernel launch failed */
} fp8attn_status;

/* Workspace regions, for fp8attn_workspace_region().  D = the plan's kernel
   width: 128, or 64 for plans of at most 64 channels (written 128 below);
   channels past the plan's head_dim hold zero codes and zero means. */
typedef enum {
  FP8ATTN_REGION_Q_CODES = 0, /* uint8 [H][rows][128]                                  */
  FP8ATTN_REGION_K_CODES = 1, /* uint8 [H][rows][128] (centred K)                       */
  FP8ATTN_REGION_V_CODES = 2, /* uint8 [H][128][rows], keys permuted in 64-key groups  */
  FP8ATTN_REGION_SCALES = 3,  /* float [3][S][H]: rows Q, K, V; S = num_segments with
                                 FP8ATTN_PLAN_SEGMENT_SCALES, else 1                   */
  FP8ATTN_REGION_MU = 4,      /* float [num_segments][H][128]: per-channel K means     */
  FP8ATTN_REGION_ROWMAP = 5,  /* plan-owned device int32 [num_segments]: first workspace
                                 row of each segment (rows are padded per segment)    */
  /* FP8ATTN_PLAN_MXFP4 plans (E2M1 codes two per byte, low nibble first; E8M0
     scale bytes, one per 32 elements).  For these plans Q_CODES and K_CODES are
     uint8 [H][rows][64], V_CODES is uint8 [H][rows/64][128][32] (one 4 KB
     block per 64-key tile: channel d, keys 2i and 2i+1 of the tile in byte i of
     the channel's 32), and SCALES is not used.                                 */
  FP8ATTN_REGION_Q_BSCALES = 6,  /* uint8 [H][rows][4]: channel blocks 0, 2, 1, 3     */
  FP8ATTN_REGION_K_BSCALES = 7,  /* uint8 [H][rows][4]: channel blocks 0, 2, 1, 3     */
  FP8ATTN_REGION_V_BSCALES = 8,  /* uint8 [H][rows/64][256]: per tile, byte
                                    4*(32*b + d%32) + d/32 for channel d, keys
                                    32b .. 32b+31 of the tile                        */
  FP8ATTN_REGION_QM_CODES = 9,   /* uint8 [H][rows/128][64]: block-mean operand codes */
  FP8ATTN_REGION_QM_SCALES = 10, /* uint8 [H][rows/128][4]: its scales (0, 2, 1, 3)   */
  /* The statistics of fp8attn_quantize, the last bytes of the workspace:
     dims_out[0] = their size in bytes.  The pointer's offset into the
     workspace is the size that fp8attn_quantize_noalloc and fp8attn_forward
     need (they do not touch the statistics).                                 */
  FP8ATTN_REGION_STATS = 11,
  /* E4M3 plans with FP8ATTN_PLAN_Q_CENTRE.                                    */
  FP8ATTN_REGION_QMEAN = 12,   /* float [H][rows/128][128]: block means qm of Q; block g
                                  holds workspace rows [128 g, 128 g + 128) (zero for
                                  the guard rows)                                     */
  FP8ATTN_REGION_QM_TERM = 13  /* uint32 [H][dims_out[1]]: the mean-term table, one
                                  entry per (block, key) of a segment: for segment s
                                  (Lr = its rows rounded up to 128, E_s = the sum of
                                  (Lr/128) * Lr over the segments before it), block b
                                  of s and key j < Lr, entry
                                  E_s + ((j / 64) * (Lr / 128) + b) * 64 + j % 64
                                  holds qm . k in the frame of the score products as two
                                  bf16 (high half: the rounding of the value; low
                                  half: the rounding of the rest)                     */
} fp8attn_region;

/*
 * fp8attn_plan - validate a segment table and build the work schedule.
 *
 *   plan_out         receives the new plan (set to NULL on error).
 *   tokens           T >= 0, total tokens of the packed batch.
 *   heads            1 <= H <= 65535 (FP8ATTN_EUNSUPPORTED above).
 *   cu_seqlens_host  host int32 array of num_segments + 1 entries: cu[0] == 0,
 *                    non-decreasing, cu[num_segments] == tokens (FlashInfer page,
 *                    parameter "cu_seqlens").  Copied; the caller keeps ownership.
 *                    Empty segments are allowed and produce no work.
 *   num_segments     >= 1.
 *   softmax_scale    finite and > 0 (1/sqrt(128) is the usual value).
 *   device           HIP device ordinal on which the plan will run; the plan's
 *                    device tables are uploaded there (one synchronous copy).
 *                    A negative value makes a host-only plan: tables are built
 *                    and can be inspected, but quantize/forward reject it.
 *
 * Workspace rows: each segment occupies round_up(L, 128) rows of the code
 * regions, segments in order, followed by 128 guard rows; every row past a
 * segment's end is written as zero codes by fp8attn_quantize.  A plan whose
 * rows times head_dim, or rows / 64 times heads, passes 2^31 - 1 is rejected
 * with FP8ATTN_EUNSUPPORTED (32-bit code offsets and grid sizes).
 */
fp8attn_status fp8attn_plan(fp8attn_plan_t* plan_out, int64_t tokens, int32_t heads,
                            const int32_t* cu_seqlens_host, int32_t num_segments,
                            float softmax_scale, int32_t device);

/* Flags of fp8attn_plan_ex. */
#define FP8ATTN_PLAN_SEGMENT_SCALES 1u
#define FP8ATTN_PLAN_MXFP4 2u
#define FP8ATTN_PLAN_Q_CENTRE 4u
#define FP8ATTN_PLAN_CAUSAL 8u
#define FP8ATTN_PLAN_HEAD_DIM_64 16u
#define FP8ATTN_PLAN_EXACT_PROBS 32u
/* head_dim d (a multiple of 8, 8 <= d <= 128) in bits 8..12 of the flags; 0
   there means 128 (or 64 with FP8ATTN_PLAN_HEAD_DIM_64). */
#define FP8ATTN_PLAN_HEAD_DIM(d) ((uint32_t)((d) / 8) << 8)

/*
 * fp8attn_plan_ex - fp8attn_plan with flags (fp8attn_plan is flags == 0).
 *
 * FP8ATTN_PLAN_SEGMENT_SCALES: one scale per (tensor, segment, head) instead
 *   of per (tensor, head): every segment is quantized by the per-head rule of
 *   fp8attn_quantize applied to its own tokens, so no segment's codes depend
 *   on another segment's values (a packed batch of unrelated sequences).  An
 *   empty segment gets the scales of an all-zero head.  The attention reads
 *   each segment's scales.
 * FP8ATTN_PLAN_MXFP4: block-scaled FP4 operands instead of E4M3 (FlashInfer
 *   "minimax_h3_sm120_varlen_attention_nvfp4" page, description of the
 *   kernel), in the OCP MX form that gfx950's scaled matrix products take:
 *   Q, K, V and the probabilities as E2M1 codes with one power-of-two (E8M0)
 *   scale per 32 elements of the contraction axis (Q, K: channels; V: keys of
 *   a segment, from its start; probabilities: keys).  A block's scale is 2^e
 *   with e the smallest integer for which amax <= 6 * 2^e (-127 for an
 *   all-zero block), its codes E2M1(x * 2^-e) rounded to nearest even.  K is
 *   centred by its segment's per-channel mean as for E4M3.  The score factor
 *   c = fl32(softmax_scale * log2(e)) is folded into Q before quantization:
 *   Q's operand is fl32(fl32(q - qm) * c), qm = 0 unless
 *   FP8ATTN_PLAN_Q_CENTRE.  A query's probabilities in key block b are
 *   2^E * E2M1(2^(x - E)) with x its scores in log2 units and
 *   E = ceil(max_b x - log2 6); out = sum phat V / sum phat, rounded to BF16.
 *   Expect several times the E4M3 error (the page reports about 4x for its
 *   NVFP4 recipe).  The LSE (if requested) is the natural-log log-sum-exp of
 *   the uncentred scores from the dequantized operands, taken as the log of
 *   the row's normalizer: ln 2 * (log2 sum_j phat_j + (Qhat + QMhat) . mu).  Work items split along
 *   the keys as for E4M3 plans (128-query items, two workgroups per CU).
 * FP8ATTN_PLAN_Q_CENTRE: Q rows are centred by the mean qm of their 128-row
 *   block (blocks of a segment from its start; the mean is a float64 sum over
 *   the block's rows in order, divided by the row count, rounded to float32)
 *   and the term qm . k is added back to the scores, so the softmax is that
 *   of the uncentred Q (the FlashInfer page's Q centring).
 *   With FP8ATTN_PLAN_MXFP4: the block-mean operand fl32(qm * c), quantized
 *   like a Q row, is multiplied with K inside the kernel and added to the
 *   scores.
 *   E4M3 plans (any head size): Q's amax, scale and codes are those of
 *   fl32(q - qm); a rounded mean would carry as much error as centring
 *   removes, so fp8attn_quantize also writes the mean term of every
 *   (block, key) pair of a segment, f * (qm . khat) with khat the K codes
 *   and f = softmax_scale * s_k * log2(e) (times 8 unless
 *   FP8ATTN_PLAN_EXACT_PROBS), as a bf16 pair (FP8ATTN_REGION_QM_TERM; qm is
 *   carried in three E4M3 parts with power-of-two scales, about 12
 *   significant bits), and the attention adds it to the scores through one
 *   small matrix product per 32-key block.  The table takes 4 bytes per
 *   (block, key) of every segment and head (1.6 GB at 30272 tokens and 56
 *   heads); plans with a segment longer than 262016 tokens (its part of a
 *   head's table would pass 2^31 bytes) or whose table would pass 1 TiB are
 *   rejected with FP8ATTN_EUNSUPPORTED.  The LSE (if requested) is that of the uncentred
 *   scores, ln 2 * (log2 l - offset) + softmax_scale * (s_q qhat + qm) . mu.
 * FP8ATTN_PLAN_CAUSAL: query i of a segment attends only to the
 *   keys j <= i of the same segment, positions counted from the segment start
 *   (the pages send causal attention to another backend; this is the plain
 *   reading for self-attention).  A work item attends to the key tiles up to
 *   its last query; the tiles from its first query on are masked per element.
 *   The LSE (if requested) is over the visible keys.  Causal plans never split
 *   work items.  With FP8ATTN_PLAN_MXFP4 a query's last probability block
 *   holds its visible keys only (its scale comes from their maximum).
 * FP8ATTN_PLAN_HEAD_DIM_64 (E4M3 plans): q, k, v and out have 64 channels
 *   per head instead of FP8ATTN_HEAD_DIM (P1 lists other head sizes among the
 *   cases it sends elsewhere): every region, stride and scale rule below
 *   holds with 64 in place of 128.  Combines with the other E4M3 flags.
 * FP8ATTN_PLAN_HEAD_DIM(d) (E4M3 plans): q, k, v and out have d channels per
 *   head, d a multiple of 8 from 8 to 128.  The kernels run at the width 64
 *   (d <= 64) or 128 with the missing channels taken as zeros: they add
 *   nothing to any score, their K mean is 0, they are left out of every
 *   amax (so the codes of the d channels are those of an unpadded
 *   quantizer), and out receives the d channels only.  The same as
 *   FP8ATTN_PLAN_HEAD_DIM_64 for d = 64.
 * FP8ATTN_PLAN_EXACT_PROBS (E4M3 plans): the probabilities are the E4M3
 *   rounding (nearest, ties to even) of the FP32 exp2 of the scores, as in the
 *   sglang PR's recipe, instead of the default log-linear code (see
 *   fp8attn_forward): about 12% slower, relative RMS error about 0.054 instead
 *   of 0.056 on the pages' normally distributed workloads.
 * Unknown flag bits,
 * FP8ATTN_PLAN_EXACT_PROBS with FP8ATTN_PLAN_MXFP4,
 * FP8ATTN_PLAN_MXFP4 with FP8ATTN_PLAN_SEGMENT_SCALES (its scales are already
 * local to 32 elements) or with a head_dim other than 128, a head_dim that is
 * not a multiple of 8 in [8, 128], or FP8ATTN_PLAN_HEAD_DIM_64 with another
 * FP8ATTN_PLAN_HEAD_DIM(d): FP8ATTN_EINVAL.
 */
fp8attn_status fp8attn_plan_ex(fp8attn_plan_t* plan_out, int64_t tokens, int32_t heads,
                               const int32_t* cu_seqlens_host, int32_t num_segments,
                               float softmax_scale, int32_t device, uint32_t flags);

/* Bytes of workspace fp8attn_quantize/fp8attn_forward need for this plan (0 on NULL). */
size_t fp8attn_workspace_bytes(fp8attn_plan_t plan);

/*
 * fp8attn_quantize - BF16 Q/K/V views -> E4M3 codes + per-head scales in the workspace.
 *
 * q, k, v       device pointers to bfloat16 data viewed as
 *               [tokens][heads][head_dim] (head_dim 128 unless the plan says
 *               otherwise): element (t, h, d) is at
 *               base[t * strides[0] + h * strides[1] + d]
 *               (strides in elements, dim stride 1).  Strides must be positive
 *               multiples of 8 and bases 16-byte aligned.  Views of one fused
 *               [T][3][H][128] buffer are fine.  Read-only.
 * workspace     device buffer of at least fp8attn_workspace_bytes(plan) bytes,
 *               256-byte aligned.  Its prior contents do not matter.
 * stream        hipStream_t to enqueue on (NULL = default stream).
 *
 * Per head h and tensor X in {K, V}: s_X[h] = fl32(amax / 448), or 1.0 when
 * amax == 0.  Q's scale is that value rounded up to make the score factor
 * softmax_scale * s_Q * s_K * log2(e) a power of two: with b = the amax/448
 * scale of Q and f = fl32(fl32(softmax_scale * s_K[h]) * log2(e)),
 * s_Q[h] = fl32(2^m / f) for the smallest m with 2^m >= fl32(f * b) (b itself
 * if fl32(f * b) is not a normal float), so Q's largest code lies in
 * (224, 448].  Codes = E4M3(fl32(y / s_X[h])) with round-to-nearest-even,
 * subnormals kept and the sign copied; y = x for Q and V; for K, y =
 * fl32(x - mu[seg][h][d]) with mu the segment's per-channel mean, summed in
 * float64 in 256-token chunks from the segment start (ascending inside a chunk,
 * then chunk sums ascending) and rounded to float32.  Centring K leaves the
 * softmax unchanged (FlashInfer page, description of the K mean).
 * The pass is two-phase (sglang PR, "Modifications", fused_prep: amax, then
 * pack): three launches (stats, finalize, pack) on `stream`.  For
 * FP8ATTN_PLAN_MXFP4 plans the codes and block scales of fp8attn_plan_ex are
 * written instead (the statistics pass then reads K only).
 */
fp8attn_status fp8attn_quantize(fp8attn_plan_t plan, const void* q, const void* k,
                                const void* v, const int64_t q_strides[2],
                                const int64_t k_strides[2], const int64_t v_strides[2],
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8attn_quantize_noalloc - fp8attn_quantize for callers that cannot
 * allocate (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation): the same launches and the same codes, scales and means
 * (bit for bit), but the statistics pass writes its per-chunk partials into a
 * static device buffer of the library (16 MiB, one per device, held until the
 * process ends) instead of the workspace's statistics region.
 *
 * Arguments as for fp8attn_quantize, except:
 * workspace_bytes  at least the offset of FP8ATTN_REGION_STATS (the code,
 *                  scale, mean and partial regions; the statistics region
 *                  need not exist and is never touched).
 * Errors as for fp8attn_quantize, plus FP8ATTN_EUNSUPPORTED (checked first,
 * also for host-only plans) when the plan's statistics exceed the static
 * buffer: 2 KB per (256-token chunk, head) at head_dim 128 (1 KB at 64) plus
 * 8 bytes per (chunk, head), e.g. about 8000 chunk-heads at head_dim 128
 * (30272 tokens x 56 heads need 6664).  It calls no allocator: the buffer's
 * device address is looked up once per device on the first call there.
 * Every call on a device shares that device's buffer and overwrites every
 * entry it reads, so nothing carries over from earlier calls; calls that
 * overlap on one device (several streams or threads at once) race on it and
 * must be serialized by the caller.
 */
fp8attn_status fp8attn_quantize_noalloc(fp8attn_plan_t plan, const void* q, const void* k,
                                        const void* v, const int64_t q_strides[2],
                                        const int64_t k_strides[2], const int64_t v_strides[2],
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8attn_forward - attention over the codes that the last fp8attn_quantize
 * into `workspace` wrote (stream order).
 *
 * out           device bfloat16 [tokens][heads][head_dim] with element (t, h, d) at
 *               out[t * out_strides[0] + h * out_strides[1] + d]; strides positive
 *               multiples of 8, base 16-byte aligned.  Every row of every
 *               non-empty segment is written.
 * lse           NULL, or device float [heads][tokens]: natural-log
 *               log-sum-exp of softmax_scale * q.k over the row's keys
 *               (uncentred keys), taken as the log of the denominator that
 *               normalizes the row: for E4M3 plans the sum of the
 *               probability weights applied to V (each within a factor
 *               [0.9203, 1.0645] of the exact exp with the default code, see
 *               below, and [1 - 2^-4, 1 + 2^-4] with
 *               FP8ATTN_PLAN_EXACT_PROBS), so partial results combine by it
 *               exactly; for FP4 plans likewise the sum of the block-scaled
 *               E2M1 weights.
 * stream        hipStream_t (NULL = default stream).
 *
 * workspace     the workspace the codes were quantized into.  Forward reads
 *               the code, scale and mean regions and writes only its
 *               partial-output region (used by split work items);
 *               workspace_bytes must reach at least the offset of
 *               FP8ATTN_REGION_STATS (the statistics are not needed).
 *
 * Probabilities (E4M3 plans): per query, the scores are taken relative to a
 * running reference that maps the row maximum to 112 (moved only when a
 * probability would pass 448), and packed to E4M3 in registers before the
 * second product.  By default each probability's E4M3 code is its base-2
 * logarithm read log-linearly: code = round(8 log2(p) + 55.54), the exponent
 * from the integer part and the 3-bit mantissa from the fraction (2^f taken as
 * 1 + f, centred); one conversion per probability instead of an exp2 and a
 * pack.  The row sum that normalizes the output adds the same E4M3 values.
 * FP8ATTN_PLAN_EXACT_PROBS rounds the FP32 exp2 instead.  On E4M3's normal
 * codes a log-linear weight is the exact 2^x times a factor in
 * [0.9203, 1.0645], so the default LSE is within [-0.083, +0.063] of the
 * exact one (about 1e-3 on rows of many keys; the error is centred); asking
 * for it costs nothing extra.  With FP8ATTN_PLAN_EXACT_PROBS the LSE costs an
 * FP32 addition per score.
 *
 * One attention launch, plus one combine launch when the plan splits work
 * items along the keys (fp8attn_plan_work_items shows the split; it happens
 * only to fill an otherwise half-empty last round of workgroups).  A split
 * item's pieces each attend to a contiguous range of key tiles and the
 * combine merges them by their log-sum-exp weights (the combination over key
 * ranges that the sglang PR "[DSA] Enable tilelang fp8_e4m3 KV cache ..."
 * describes for cross-rank reduction of partial attention).  Output rows are
 * written exactly once; repeated calls on the same workspace give
 * bit-identical results.
 */
fp8attn_status fp8attn_forward(fp8attn_plan_t plan, void* workspace, size_t workspace_bytes,
                               void* out, const int64_t out_strides[2], float* lse, void* stream);

/*
 * fp8attn_workspace_region - where a region lives (for tests and tools).
 *
 * ptr_out    receives a device pointer into `workspace` (or, for
 *            FP8ATTN_REGION_ROWMAP, into the plan's own device table).
 * dims_out   int64[3] receives the region's logical dimensions as listed in
 *            fp8attn_region (unused trailing entries set to 1).
 *
 * V code layout: for head h, channel d, 64-key group g of workspace rows
 * [64g, 64g + 64), byte p = 32*j + 16*b + 4*r + i (j, b in {0,1}; r, i in
 * 0..3) of the group holds key row 64g + 32*b + 8*r + 4*j + i.
 */
fp8attn_status fp8attn_workspace_region(fp8attn_plan_t plan, const void* workspace, int which,
                                        const void** ptr_out, int64_t dims_out[3]);

/*
 * fp8attn_plan_info - schedule facts (for tests and tools).
 *   info_out int64[14]: {tokens, heads, num_segments, workspace_rows,
 *                        work_items, stat_chunks, query_tile, key_tile,
 *                        segment_scales (0 or 1), partial_slots,
 *                        mxfp4 (0 or 1), q_centre (0 or 1), causal (0 or 1),
 *                        head_dim (128 or 64)}
 */
fp8attn_status fp8attn_plan_info(fp8attn_plan_t plan, int64_t info_out[14]);

/*
 * fp8attn_plan_work_items - copy the ordered work list to host memory.
 *   items_out int32[4 * capacity]: per item {segment, first query of the tile
 *   (segment-relative), head, split}; padding items have segment == -1.
 *   split == 0: the item attends to every key of its segment.  Otherwise
 *   bits 0-3 hold the piece index i, bits 4-7 the piece count n (2..8) and
 *   bits 8-31 the item's first partial slot; piece i attends to key tiles
 *   [nkt*i/n, nkt*(i+1)/n) of the segment's nkt = ceil(len/64) tiles.
 *   count_out receives the number of items (which may exceed capacity; only
 *   min(count, capacity) are copied).
 */
fp8attn_status fp8attn_plan_work_items(fp8attn_plan_t plan, int32_t* items_out, int64_t capacity,
                                       int64_t* count_out);

/* Free a plan (NULL is a no-op).  Work already enqueued with it must be complete. */
fp8attn_status fp8attn_plan_destroy(fp8attn_plan_t plan);

/* Text of the calling thread's last non-OK status ("" if none).  Valid until the next call. */
const char* fp8attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8ATTN_H */
