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
#ifndef FP8ATTN_BM
#define FP8ATTN_BM 128
#endif
constexpr int kBM = FP8ATTN_BM;  // queries per attention work item (one wave per 32)
constexpr int kBN = 64;          // keys per inner tile
constexpr int kNumXcd = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs

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

struct WorkspaceLayout {
  int64_t rows;        // workspace rows (all segments padded + guard)
  size_t q_off, k_off, v_off, scale_off, mu_off, kstat_off, amax_off, total;
};

struct QuantizeArgs {
  const uint16_t* x[3];      // bf16 Q, K, V
  int64_t ts[3], hs[3];      // token and head strides in elements
  uint8_t* codes[3];         // Q, K: [H][rows][128]; V: [H][128][rows] permuted
  float* scales;             // [3][H]
  float* mu;                 // [nseg][H][128]
  KStat* kstat;              // [nchunks][H][128]
  float* amax;               // [2][nchunks][H]  (Q, V partial amax)
  const SegInfo* segs;
  const Chunk* chunks;
  const int32_t* group_seg;  // [ngroups]: segment of each 64-row pack group, -1 = guard
  int32_t heads, nseg, nchunks, ngroups;
  int64_t rows;
  float softmax_scale;       // fixes Q's scale (see k_finalize)
};

struct AttentionArgs {
  const uint8_t* q_codes;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* scales;
  const float* mu;
  const SegInfo* segs;
  const int4* items;         // {segment or -1, first query (segment-relative), head, 0}
  uint16_t* out;             // bf16
  int64_t os0, os1;          // output token and head strides (elements)
  float* lse;                // nullable, [H][T]
  int64_t tokens;
  int64_t rows;
  int32_t heads;
  int32_t nitems;
  float softmax_scale;
};

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream);
hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream);

}  // namespace fp8attn
