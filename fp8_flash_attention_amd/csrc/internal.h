// Internal definitions shared by the planner (api.cpp) and the HIP kernels.
// Not part of the public ABI (include/fp8attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8attn {

constexpr int kHeadDim = 128;
constexpr int kRowPad = 128;     // workspace rows of a segment are padded to this multiple
constexpr int kGuardRows = 128;  // zero rows after the last segment
constexpr int kStatChunk = 256;  // tokens per stats chunk; fixes the K-mean summation order
constexpr int kPackRows = 64;    // workspace rows per pack block (one V key group)
constexpr int kBM = 256;         // queries per E4M3 work item (one wave per 32); 128 for plans with few rounds
constexpr int kPartRows = 256;   // rows of one partial-output slot (the largest query tile)
constexpr int kBN = 64;          // keys per inner tile
constexpr int kNumXcd = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kMaxSplit = 8;     // key pieces of one split work item, at most
constexpr int kMinPieceTiles = 8;  // key tiles of one piece, at least

// Work item {x, y, z, w}: x = segment (or -1: padding), y = first query of the
// tile (segment-relative), z = head, w = key split.  w == 0: all keys of the
// segment, output written directly.  Otherwise bits 0-3 = piece index i,
// bits 4-7 = piece count n (2..kMaxSplit), bits 8-31 = first partial slot of
// the item; piece i covers key tiles [nkt*i/n, nkt*(i+1)/n) and writes partial
// slot (w >> 8) + i, which a combine pass merges.  Combine items carry the
// same x, y, z and w with bits 0-3 zero.
__host__ __device__ inline int split_pieces(int w) { return (w >> 4) & 15; }
__host__ __device__ inline int split_index(int w) { return w & 15; }
__host__ __device__ inline int split_slot0(int w) { return (int)((unsigned)w >> 8); }

struct SegInfo {
  int32_t start;   // first token of the segment
  int32_t len;     // tokens in the segment (0 allowed)
  int32_t row0;    // first workspace row (multiple of kRowPad)
  int32_t chunk0;  // first stats chunk
};

struct Chunk {
  int32_t seg;
  int32_t tok0;
  int32_t ntok;    // 1..kStatChunk
  int32_t pad;
};

// Per (chunk, head, channel) statistics of K: fixed-order float64 sum, min, max.
struct KStat {
  double sum;
  float mn;
  float mx;
};

// Block-scaled FP4 operands (plans made with FP8ATTN_PLAN_MXFP4): E2M1 codes,
// two per byte (low nibble first), one E8M0 scale byte per 32 elements.
constexpr int kMxBlock = 32;               // elements per scale
constexpr int kMxRow = kHeadDim / 2;       // code bytes of one Q or K row
constexpr int kMxQBlock = 128;             // Q rows per mean block
constexpr int kMxTile = kBN * kHeadDim / 2;   // code bytes of one K (or V^T) tile
constexpr int kMxTileScales = 256;         // scale bytes of one K (or V^T) tile
constexpr int kMxBM = 128;                 // queries per FP4 work item (4 waves)
constexpr int kMxWgPerCu = 2;              // FP4 attention workgroups resident per CU

// E4M3 plans with Q centring (FP8ATTN_PLAN_Q_CENTRE): Q rows are centred by
// the mean of their 128-row block (blocks of a segment from its start; with
// segments padded to kRowPad = 128 rows, block g holds workspace rows
// [128 g, 128 g + 128)).  The mean term qm . k of every (block, key) pair of a
// segment is precomputed in the frame of the score products and stored as a
// bf16 pair (high part, then the rounding of the rest) per entry: for head h,
// segment s (Lr = its padded rows, nb = Lr / 128 blocks), block b of s and key
// j < Lr, entry h * mt_per_head + mt_seg[s] + ((j / 64) * nb + b) * 64 + j % 64
// of a uint32 table (tile-major: the 64-key chunks of all blocks of one key
// tile are adjacent).
constexpr int kQmBlock = 128;
constexpr int kQmUnitKeys = 1024;            // keys per workgroup of the mean-term kernel
constexpr int kQmUnitBlocks = 32;            // Q blocks per workgroup of the mean-term kernel

struct WorkspaceLayout {
  int64_t rows;        // workspace rows (all segments padded + guard)
  int64_t npieces;     // partial slots of split work items
  size_t q_off, k_off, v_off, scale_off, mu_off, kstat_off, amax_off;
  // FP4 plans: Q, K scales [H][rows][4] (blocks in byte order 0, 2, 1, 3);
  // V^T scales [H][rows/64][256] (tile-major, byte (32*(key/32) + d%32)*4 + d/32);
  // block-mean codes [H][rows/128][64] and scales [H][rows/128][4] (order 0, 2, 1, 3)
  size_t qs_off, ks_off, vs_off, qm_off, qms_off;
  size_t part_o_off;   // float [npieces][kPartRows][128]: normalized partial outputs (scaled by s_v)
  size_t part_w_off;   // float [npieces][kPartRows]: log2 weight of each partial row
  size_t part_lse_off; // float [npieces][kPartRows]: natural-log LSE of each partial row
  size_t stats_off;    // start of the statistics (kstat, amax), the last regions
  // E4M3 plans with Q centring: block means float [H][rows/128][D], the mean-term
  // table uint32 [H][mt_per_head], and (statistics) the blocks' centred amax
  // partials float [rows/128][H][D/8]
  size_t qmean_off, mt_off, qamax_off;
  int64_t mt_per_head;
  size_t total;
};

// Device buffer for the statistics of fp8attn_quantize_noalloc (a static
// device array of kStaticStatsBytes, one per device); its address on the
// current device, looked up once per device.
constexpr size_t kStaticStatsBytes = size_t(16) << 20;
hipError_t static_stats_buffer(int device, uint8_t** ptr);

struct QuantizeArgs {
  const uint16_t* x[3];      // bf16 Q, K, V
  int64_t ts[3], hs[3];      // token and head strides in elements
  uint8_t* codes[3];         // Q, K: [H][rows][128]; V: [H][128][rows] permuted
  float* scales;             // [3][S][H], S = nseg with per-segment scales, else 1
  float* mu;                 // [nseg][H][128]
  KStat* kstat;              // [nchunks][H][128]
  float* amax;               // [2][nchunks][H]  (Q, V partial amax)
  const SegInfo* segs;
  const Chunk* chunks;
  const int32_t* group_seg;  // [ngroups]: segment of each 64-row pack group, -1 = guard
  int32_t heads, nseg, nchunks, ngroups;
  int32_t seg_scales;        // 1: one scale per (tensor, segment, head)
  int32_t head_dim;          // D: kernel width, 128 or 64 (E4M3 plans)
  int32_t d_real;            // channels present in q, k, v (<= D; the rest read as zeros)
  int64_t rows;
  float softmax_scale;       // fixes Q's scale (see k_finalize)
  // FP4 plans
  int32_t mx;                // 1: block-scaled FP4 operands (codes[] and the fields below)
  int32_t q_centre;          // 1: Q centred by its 128-row block mean
  uint8_t* bscale[3];        // Q, K, V^T block scales (WorkspaceLayout)
  uint8_t* qm_codes;
  uint8_t* qm_scales;
  // E4M3 plans with q_centre: Q block means and centred amax partials, the mean-term table
  float* qamax;              // [rows/128][H][D/8]
  float* qmean;              // [H][rows/128][D]
  uint32_t* mt;              // [H][mt_per_head]
  const int64_t* mt_seg;     // [nseg]: first entry of each segment's part of a head's table
  const int4* qmt_units;     // work of the mean-term kernel: {segment, block group, first key, head}; segment -1: none
  int32_t nqmt_units;
  int32_t exact_probs;       // frame of the mean term: x (1) or y = 8 x (0)
  int64_t mt_per_head;
};

struct AttentionArgs {
  const uint8_t* q_codes;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* scales;       // [3][S][H]
  const float* mu;
  const SegInfo* segs;
  const int4* items;         // work items (encoding above)
  uint16_t* out;             // bf16
  int64_t os0, os1;          // output token and head strides (elements)
  float* lse;                // nullable, [H][T]
  float* part_o;             // partial outputs of split items (see WorkspaceLayout)
  float* part_w;
  float* part_lse;
  int64_t tokens;
  int64_t rows;
  int32_t heads;
  int32_t nitems;
  int32_t nscale;            // S: scale sets (segments with per-segment scales, else 1)
  int32_t causal;            // 1: query i of a segment attends keys j <= i only
  int32_t head_dim;          // D: kernel width, 128 or 64
  int32_t d_real;            // channels written to out (<= D)
  int32_t bm;                // queries per work item: 256, or 128 (D = 128 only)
  int32_t exact_probs;       // 1: p = E4M3(exp2(x)); 0: the log-linear code of 2^x
  int32_t q_centre;          // 1: Q centred by its 128-row block mean, mean term from mt
  float softmax_scale;
  const float* qmean;        // q_centre: [H][rows/128][D]
  const uint32_t* mt;        // q_centre: [H][mt_per_head]
  const int64_t* mt_seg;     // q_centre: [nseg]
  int64_t mt_per_head;
};

struct CombineArgs {
  const int4* items;         // one per split work item
  int32_t nitems;
  const SegInfo* segs;
  const float* part_o;
  const float* part_w;
  const float* part_lse;
  uint16_t* out;             // bf16
  int64_t os0, os1;
  float* lse;                // nullable, [H][T]
  int64_t tokens;
  int32_t head_dim;          // D: kernel width, 128 or 64
  int32_t d_real;            // channels written to out (<= D)
  int32_t bm;                // queries per split item (128 or 256)
};

// FP4 attention: codes and block scales as in WorkspaceLayout.
struct MxAttentionArgs {
  const uint8_t* q_codes;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* q_scales;
  const uint8_t* k_scales;
  const uint8_t* v_scales;
  const uint8_t* qm_codes;   // used with q_centre
  const uint8_t* qm_scales;
  const float* mu;           // [nseg][H][128]: K's segment means (for the LSE)
  const SegInfo* segs;
  const int4* items;         // work items (encoding above)
  uint16_t* out;             // bf16
  int64_t os0, os1;
  float* lse;                // nullable, [H][T]
  float* part_o;             // partial outputs of split items (as for E4M3 plans)
  float* part_w;
  float* part_lse;
  int64_t tokens;
  int64_t rows;
  int32_t heads;
  int32_t nitems;
  int32_t q_centre;
  int32_t causal;            // 1: query i of a segment attends keys j <= i only
};

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream);
hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_mx(const MxAttentionArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace fp8attn
