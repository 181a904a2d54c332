// FP8 (E4M3) flash-attention forward for gfx950.
//
// Method (sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for
// SM120 GPUs", "Modifications", kernel.py item): E4M3 operands for both
// products with FP32 accumulation, an online softmax kept in registers, the
// probabilities packed to E4M3 inside registers, and K/V tiles prefetched
// ahead so the copy overlaps the math.  The output is rounded to BF16 once
// (FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page).
//
// gfx950 mapping
//   * One workgroup = kBM/32 waves (8 for kBM = 256) of 32 queries each, all
//     on one (segment, head), one workgroup per CU, so every SIMD runs two
//     waves (up to 256 registers each).  Keys are walked in tiles of kBN = 64.
//     Eight waves share each K/V tile load: against two 4-wave workgroups per
//     CU this halves the L2-to-LDS traffic and the LDS writes, and the power
//     saved shows as a higher clock under load (about +6%, for a few percent
//     less matrix-core occupancy since a SIMD's two waves now share barriers).
//   * A single wave issues one vector instruction every ~5 clocks, two waves
//     together one every ~2.7, and the exp2 and the E4M3 conversion take ~8.5
//     clocks each; per score the vector work is about as long as the matrix
//     work.  So each wave overlaps the two within its own instruction stream:
//     iteration t runs the softmax of tile t on the vector unit while the
//     matrix core computes the scores of tile t+1 and the P V product of tile
//     t-1.  Nothing in an iteration waits for a matrix result of the same
//     iteration.  The body is laid out as nine slots of one matrix product
//     each, separated by scheduling fences; the rare paths (a reference
//     shift, the rescale it asks for) are branches laid out of line.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x64_f8f6f4 (A = 32 keys x 64 channels read from LDS,
//     B = 32 queries x 64 channels held in registers for the whole loop).  In
//     the 32x32 accumulator layout lane l holds query l%32 and 16 keys of a
//     32-key block, so a row maximum is in-lane plus one exchange between
//     lanes l and l^32 (v_permlane32_swap).
//   * The accumulators of the two 32-key blocks of a tile, converted to E4M3
//     codes in registers (below), are exactly the B operand (64 keys x 32
//     queries) of O^T += V^T P^T.  The key order this implies inside a 64-key group is
//     baked into the workspace V layout by the pack pass, so the P registers
//     never leave the lane.
//   * Row sums l come from the matrix core too: one
//     v_mfma_f32_16x16x128_f8f6f4 per tile multiplies the packed P^T by a
//     constant 0/1 selector, which adds the 64 key bytes of query j (lanes j
//     and j+32) into row 0 and those of query 16+j (lanes j+16 and j+48) into
//     row 1.  l is the sum of the E4M3 probabilities that actually weight V.
//     The LSE, when asked for, is the log of l (the denominator the output
//     is normalized by, so partial results combine exactly by it), with
//     either probability encoding.
//   * Probabilities: p = 2^x, x = c*s + nbx with c = softmax_scale * s_q *
//     s_k * log2(e) and nbx = log2(112) - c*m for a per-query reference
//     maximum m.  The quantizer makes c a power of two, so the score products
//     run on the scaled MFMA (E8M0 factor c) with the offset as the initial
//     accumulator and deliver the exponent itself.  By default they deliver
//     y = 8 x + kYBias (factor 8 c), and the E4M3 code of p is y rounded to
//     an integer, one v_cvt_pk_u8_f32 per score: the integer part of 8 x steps
//     the code's exponent, the fraction its 3-bit mantissa (2^f read as 1 + f,
//     centred by kYBias), about 0.031 relative RMS of the kernel's own error
//     against 0.026 for exact rounding, 12% faster.  With exact probabilities
//     they deliver x, and p = E4M3(exp2(x)): an exp2 and half a conversion.
//     The first tile sets m to its row maximum (mapped to 112 = 448/4).
//     Later tiles move m only when their maximum would give a p above 448,
//     the largest E4M3 value, so most tiles need no rescale: the common path
//     is a max tree (integer maxima of the float bits, which order like the
//     floats above the threshold) and one wave-wide vote; the rare path
//     shifts the scores, the offset and the accumulator initial value, and
//     the rescale of O and l by 2^shift runs at the top of the next
//     iteration, after the P V product of the older tiles and before that of
//     the tile that moved m.
//   * K and V^T tiles reach LDS by direct buffer loads (no register staging):
//     a K ring and a V ring of four 8 KB slots each.  Iteration t reads K of
//     tile t+1 for its score products, and V of tile t for the P V product of
//     the next iteration, so that product starts with its operands already in
//     registers.  Barriers come every second iteration: at even t, after
//     waiting for the loads issued at t-2, the wave passes the barrier and
//     loads K of tiles t+3, t+4 and V of tiles t+2, t+3 for the next two
//     iterations, into the slots whose last reads the barrier has just
//     retired.  16-byte chunks are XOR-swizzled against bank conflicts of the
//     operand reads; the swizzle is applied to the source addresses of the
//     lane-linear loads.
#include "internal.h"

namespace fp8attn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr float kLog2e = 1.4426950408889634f;
// Probability frames.  Exact probabilities (FP8ATTN_PLAN_EXACT_PROBS): the
// score products deliver x = log2(p) and p = E4M3(exp2(x)).  Log-linear (the
// default): they deliver y = 8 x + kYBias and the E4M3 code of p is y rounded
// to an integer (v_cvt_pk_u8_f32, round to nearest even, clamped to [0, 255]):
// an E4M3 code is 8 * (biased exponent) + mantissa, so the integer part of
// 8 x + 56 steps the exponent and the fraction the 3-bit mantissa linearly
// (2^f read as 1 + f on each octave); kYBias = 56 - 0.4588 centres that
// approximation and puts the reference at code 110 (the value 112).
constexpr float kLog2Ref = 6.807354922057604f;   // log2(112): reference maximum maps to 448 / 4
constexpr float kLog2Max = 8.807354922057604f;   // log2(448), the largest E4M3 value
constexpr float kYBias = 55.54116061995f;        // y = 8 x + kYBias
constexpr float kYRef = 110.0f;                  // y of the reference maximum: code 110 = 112
constexpr float kYMax = 126.5f;                  // above this y a code would pass 0x7E (448)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSlots = 4;                        // ring slots per operand
constexpr int kBarEvery = kSlots / 2;            // iterations per barrier
constexpr int kBufferFlags = 0x00020000;         // raw buffer descriptor word 3 (gfx9 family)
static_assert(kBN == 64, "64-key tiles");

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  // cbsz = blgp = 0 selects E4M3 for both operands; zero scales select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// a*b scaled by 2^(ea - 127) (ea an E8M0 code, the same in every lane), plus c.
__device__ __forceinline__ v16f mfma_fp8_scaled(const v8i& a, const v8i& b, const v16f& c, int ea) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, 127);
}
__device__ __forceinline__ v4f mfma16_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// Q centring: the initial accumulator of a 32-key block's score products, one
// 32x32x16 bf16 product.  A (lanes l and l+32: key l%32) = {mt_hi, mt_lo, 1, 1,
// 0 ...}, B (lanes 0-31: query l; lanes 32-63 zero) = {1, 1, nb_hi, nb_lo,
// 0 ...}, so entry (key, query) = mean term of the key + offset of the query.
constexpr uint32_t kBf16Ones = 0x3F803F80u;   // two bf16 1.0
__device__ __forceinline__ v16f mt_init(uint32_t mt, const v4i& bq) {
  const v4i av = v4i{(int)mt, (int)kBf16Ones, 0, 0};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf16, av), __builtin_bit_cast(v8bf16, bq),
                                                 v16f{}, 0, 0, 0);
}
// x as a bf16 pair (high half bf16(x), low half bf16 of the rest) and the
// float sum of the two halves, the value the pair stands for.
__device__ __forceinline__ uint32_t bf16_pair(float x, float& value) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t hi = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const float rest = x - __uint_as_float(hi << 16);
  const uint32_t v = __float_as_uint(rest);
  const uint32_t lo = (v + 0x7fffu + ((v >> 16) & 1u)) >> 16;
  value = __uint_as_float(hi << 16) + __uint_as_float(lo << 16);
  return hi | (lo << 16);
}

// sum of x over lanes l and l^32.  v_permlane32_swap on (x, x) leaves
// {x[l], x[l^32]} in its two results (in an order that depends on the lane
// half), so combining both results needs no lane select.
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 codes of four floats in one dword.  Both halves are written, so the
// first conversion's merge operand is left undefined (no register to clear).
__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
  int u;
  asm volatile("" : "=v"(u));   // an arbitrary register: no instruction to clear it
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__device__ __forceinline__ v8i lds_read32(const uint8_t* base, int off_lo, int off_hi) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + off_lo);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + off_hi);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// LDS tile geometry.  K slot: [64 keys][D B]; D = 128: row r chunk c at
// r*128 + ((c ^ ((r >> 1) & 7)) * 16); D = 64: at r*64 + ((c ^ ((r >> 2) & 3)) * 16)
// (either way the 16 lanes of a read phase hit 16 distinct bank groups).
// V^T slot: [D channels][64 B], row d chunk c at d*64 + ((c ^ ((d >> 2) & 3)) * 16).
template <int D>
__device__ __forceinline__ int k_swz(int row) { return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3); }
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int chunk) { return row * D + ((chunk ^ k_swz<D>(row)) << 4); }
__device__ __forceinline__ int v_lds_off(int d, int chunk) { return d * 64 + ((chunk ^ ((d >> 2) & 3)) << 4); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4] = 7, lgkmcnt[11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}

// Workgroup barrier that the compiler may not move memory operations across;
// this wave's LDS reads have completed when it passes.
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One direct load of 16 bytes per lane from buffer `rsrc` at byte offset
// voff + soff into LDS at lds + 16 * lane.  Issued as inline assembly so that
// the compiler does not serialize later LDS reads behind it (it cannot tell
// the slots apart); completion is tracked by the explicit vmcnt waits.
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds" : : "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff));
}
// The same with 4 bytes per lane (LDS at lds + 4 * lane).
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dword %1, %2, %3 offen lds" : : "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff));
}

// Scheduling fence: the compiler keeps every instruction on its side.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Pins the computation of v before this point (an empty instruction that
// reads it), so the softmax of a tile is not moved into the next iteration.
__device__ __forceinline__ void keep(const v8i& v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void keep(const v16f& v) { asm volatile("" ::"v"(v)); }

// iter(t + I, I + 1 mod N) for I = 0 .. N-1 (one pass over an N-slot ring).
template <int I, int N, typename F>
__device__ __forceinline__ void unroll_iters(F& iter, int t) {
  if constexpr (I < N) {
    iter(t + I, std::integral_constant<int, (I + 1) % N>{});
    unroll_iters<I + 1, N>(iter, t);
  }
}
// The remaining iterations (at most N after whole passes, the last one of the
// loop among them), phases P, P + 1, ... mod N.
template <int P, int E, int N, typename F>
__device__ __forceinline__ void tail_iters(F& iter, int& t, int nkt) {
  if constexpr (P < E) {
    if (t < nkt) iter(t++, std::integral_constant<int, P % N>{});
    tail_iters<P + 1, E, N>(iter, t, nkt);
  }
}

// BM queries per work item (256: one 8-wave workgroup per CU; 128: two 4-wave
// workgroups per CU), D channels per head.
template <bool LSE, bool CAUSAL, int D, int BM, bool EXACT, bool QC>
__global__ __launch_bounds__(2 * BM, 256 / BM) void k_attn(AttentionArgs a) {
  constexpr int kWavesWG = BM / 32;              // waves per workgroup, 32 queries each
  // frame constants in the units the score products deliver (x, or y = 8 x + kYBias)
  constexpr float kRef = EXACT ? kLog2Ref : kYRef;
  constexpr float kMax = EXACT ? kLog2Max : kYMax;
  constexpr float kUnit = EXACT ? 1.f : 0.125f;   // log2 units per unit of the frame
  static_assert(BM == 128 || BM == 256, "4 or 8 waves x 32 queries");
  constexpr int kTile = kBN * D;                 // bytes of one K (or V^T) tile
  constexpr int kVRing = kSlots * kTile;         // V ring follows the K ring in LDS
  constexpr int NH = D / 64;                     // 64-channel halves of Q and K
  constexpr int NDB = D / 32;                    // 32-channel blocks of O
  // Direct 1 KB loads per tile: every wave loads kLoadsPerTile of each K and V
  // tile, or (D = 64, 4 loads a tile) waves 0-3 load K and waves 4-7 V^T.
  constexpr int kLoads = kTile / 1024;
  constexpr bool kSplitLoads = kLoads < kWavesWG;
  constexpr int kLoadsPerTile = kSplitLoads ? 1 : kLoads / kWavesWG;
  static_assert(D == 128 || (D == 64 && kWavesWG == 8), "head_dim 128, or 64 with 256-query items");
  // Q centring: a ring of mean-term tiles after the V ring, one 512-byte slot
  // per key tile (the 64 keys of each of the item's 128-query blocks)
  constexpr int kMtSlot = 512;
  constexpr int kMtRing = QC ? kSlots * kMtSlot : 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kVRing + kMtRing];

  const int4 it = a.items[blockIdx.x];
  if (it.x < 0) return;
  const SegInfo si = a.segs[it.x];
  const int q0 = it.y;
  const int h = it.z;
  const int L = si.len;
  // Key range: every tile of the segment (causal: up to the item's last
  // query), or one piece of a split item.
  const int nkt_seg = ((CAUSAL ? min(L, q0 + BM) : L) + kBN - 1) / kBN;
  int kt0 = 0, nkt = nkt_seg, slot = -1;
  if (it.w != 0) {
    const int n = split_pieces(it.w), i = split_index(it.w);
    kt0 = nkt_seg * i / n;
    nkt = nkt_seg * (i + 1) / n - kt0;
    slot = split_slot0(it.w) + i;
  }
  const int Lk = min(L - kt0 * kBN, nkt * kBN);   // keys of the range, counted from its first tile
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int lg = lane >> 5;

  const size_t hrow = (size_t)h * a.rows + si.row0;
  const uint8_t* Qh = a.q_codes + hrow * D;
  const uint8_t* Kh = a.k_codes + hrow * D + (size_t)kt0 * kTile;
  const uint8_t* Vh = a.v_codes + (size_t)h * D * a.rows + si.row0 + (size_t)kt0 * kBN;

  // scales [3][S][H]: S = 1, or one set per segment
  const int sset = a.nscale > 1 ? it.x : 0;
  const float s_q = a.scales[(0 * a.nscale + sset) * a.heads + h];
  const float s_k = a.scales[(1 * a.nscale + sset) * a.heads + h];
  const float s_v = a.scales[(2 * a.nscale + sset) * a.heads + h];
  // Score factor c = softmax_scale * s_q * s_k * log2(e).  The quantizer picks
  // s_q so that c is a power of two up to the rounding of this product, so its
  // E8M0 code (the biased exponent rounded to nearest) scales the score
  // products exactly: x = c * (q . k) + nb comes out of the matrix core with the
  // per-query exp2 offset nb as the accumulator's initial value.
  const float c = a.softmax_scale * s_q * s_k * kLog2e;
  const int c_e8m0 = min((int)((__float_as_uint(c) + 0x400000u) >> 23) + (EXACT ? 0 : 3), 254);   // c, or 8 c

  // Q as B operands: queries q0 + 32*wave + (lane%32), channels
  // 64*half + 32*(lane/32) .. +32.  Rows past the segment end read zero codes,
  // guard rows or the next segment's rows and are never stored.
  v8i qf[NH];
#pragma unroll
  for (int half = 0; half < NH; half++)
    qf[half] = *reinterpret_cast<const v8i*>(Qh + (size_t)(q0 + 32 * wave + lq) * D + 64 * half + 32 * lg);

  // Per-lane LDS read offsets inside a slot.
  int koff[NH][2];   // [half][sub]
#pragma unroll
  for (int half = 0; half < NH; half++)
#pragma unroll
    for (int sub = 0; sub < 2; sub++) koff[half][sub] = k_lds_off<D>(lq, 4 * half + 2 * lg + sub);
  int voff[2];
#pragma unroll
  for (int sub = 0; sub < 2; sub++) voff[sub] = v_lds_off(lq, 2 * lg + sub);

  // Direct loads: a tile is 8 KB = 8 loads of 1 KB (64 lanes x 16 B, written
  // lane-linearly to LDS); wave w issues loads 2w and 2w+1 of each tile.  The
  // 16-byte slot p = 64*i + lane of load i receives the global chunk that the
  // swizzle places there.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kh, (short)0, (int)((a.rows - si.row0) * D - (int64_t)kt0 * kTile), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Vh, (short)0, (int)(a.rows * D - si.row0 - (int64_t)kt0 * kBN), kBufferFlags);
  // with split loads, waves 0..kLoads-1 load K and the others V^T
  const bool k_wave = !kSplitLoads || wave < kLoads;
  const int lw = kSplitLoads ? wave % kLoads : wave;   // this wave's load index within a tile
  int ksrc[kLoadsPerTile], vsrc[kLoadsPerTile];
#pragma unroll
  for (int u = 0; u < kLoadsPerTile; u++) {
    const int p = 64 * (kLoadsPerTile * lw + u) + lane;
    const int kr = p / (D / 16);                    // K row of 16-byte slot p, D/16 chunks a row
    ksrc[u] = kr * D + (((p % (D / 16)) ^ k_swz<D>(kr)) << 4);
    vsrc[u] = (p >> 2) * (int)a.rows + (((p & 3) ^ ((p >> 4) & 3)) << 4);   // V^T row p/4, swizzled chunk p%4
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)smem + 1024 * kLoadsPerTile * lw;   // LDS byte address of this wave's loads
  // Tile indices past the segment's last tile are clamped: such loads only
  // refill a free slot with valid data, and every iteration issues the same
  // number of loads, which the vmcnt waits rely on.
  auto load_k_tile = [&](int kt, int slot) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    if (k_wave) {
#pragma unroll
      for (int u = 0; u < kLoadsPerTile; u++) lds_dma(krs, lds0 + slot * kTile + u * 1024, ksrc[u], kt * kTile);
    }
  };
  auto load_v = [&](int kt, int slot) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    if (!kSplitLoads || !k_wave) {
#pragma unroll
      for (int u = 0; u < kLoadsPerTile; u++) lds_dma(vrs, lds0 + kVRing + slot * kTile + u * 1024, vsrc[u], kt * kBN);
    }
  };
  // Q centring: this wave's 128-query block (bw) and its row of the mean-term
  // table (the segment's padded rows lr long, from the range's first key);
  // the first wave of each block loads the block's 64 entries of every key
  // tile with the K tile, into slot bw of the tile's mean-term ring slot.  A
  // block past the segment's last one (the upper half of a 256-query item
  // whose queries end in its lower half) takes the last block's row: its
  // waves' rows are never stored.
  const int bw = wave >> 2;
  const bool mt_wave = QC && (wave & 3) == 0;
  const int lr = (L + kRowPad - 1) / kRowPad * kRowPad;
  const int nqb_seg = lr / kQmBlock;                         // the segment's blocks
  const int qblk = min(q0 / kQmBlock + bw, nqb_seg - 1);     // block of this wave within the segment
  // the table is tile-major: the chunk of key tile kt and block b is entry
  // (kt * nqb_seg + b) * 64 of the segment's part
  const uint32_t* mrow = nullptr;
  int mbytes = 0;
  if constexpr (QC) {
    const int64_t e0 = ((int64_t)kt0 * nqb_seg + qblk) * kBN;
    mrow = a.mt + (size_t)h * a.mt_per_head + a.mt_seg[it.x] + e0;
    mbytes = (int)(((int64_t)nqb_seg * lr - e0) * 4);
  }
  const __amdgpu_buffer_rsrc_t mtrs = __builtin_amdgcn_make_buffer_rsrc((void*)mrow, (short)0, mbytes, kBufferFlags);
  const uint32_t lds_mt = (uint32_t)(uintptr_t)(lds_ptr_t)smem + 2 * kVRing + 256 * bw;
  auto load_mt = [&](int kt, int slot) __attribute__((always_inline)) {
    if constexpr (QC) {
      kt = kt < nkt ? kt : nkt - 1;
      if (mt_wave) lds_dma4(mtrs, lds_mt + slot * kMtSlot, 4 * lane, kt * nqb_seg * kBN * 4);
    }
  };
  auto load_k = [&](int kt, int slot) __attribute__((always_inline)) {
    load_k_tile(kt, slot);
    load_mt(kt, slot);
  };

  // q_hat . mu per query, for the natural-log LSE of the uncentred scores:
  // every centred key differs from the uncentred one by the segment mean mu,
  // so the centred LSE is short by softmax_scale * (q_hat . mu).
  float qmu = 0.f;
  if (LSE) {
    const float* mu = a.mu + ((size_t)it.x * a.heads + h) * D;
    float dot = 0.f;
#pragma unroll
    for (int half = 0; half < NH; half++)
#pragma unroll
      for (int w = 0; w < 8; w++) {
        const float* md = mu + 64 * half + 32 * lg + 4 * w;
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 0) * md[0];
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 1) * md[1];
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 2) * md[2];
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 3) * md[3];
      }
    qmu = sum_pair32(dot);
  }
  // Q centring: the block mean's part of the same correction, qm . mu
  float qmm = 0.f;
  if (LSE && QC) {
    const float* mu = a.mu + ((size_t)it.x * a.heads + h) * D;
    const float* qmr = a.qmean + ((size_t)h * (a.rows / kQmBlock) + si.row0 / kQmBlock + qblk) * D;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < D / 2; j++) dot += qmr[(D / 2) * lg + j] * mu[(D / 2) * lg + j];
    qmm = sum_pair32(dot);
  }

  // Row-sum selector for the 16x16x128 product: E4M3 1.0 in every byte of
  // lanes 0 and 32 (row 0: lanes j and j+32 of P, query j) and lanes 17 and
  // 49 (row 1: lanes 16+j and 48+j, query 16+j), zero elsewhere.
  const bool sel_lane = lane == 0 || lane == 32 || lane == 17 || lane == 49;
  const int one = sel_lane ? 0x38383838 : 0;
  const v8i sel = v8i{one, one, one, one, one, one, one, one};

  v16f O[NDB];     // O^T: lane l holds query l%32, channels 32*db + 8*(r/4) + 4*(l/32) + r%4
  v4f lacc = {};   // row sums of the packed P: lane j < 16 holds query j (row 0) and 16+j (row 1)
  float nb = 0.f;  // exp2 argument offset: x = c*s + nb
  float pshift = 0.f;   // reference shift still to be applied to O and l (log2 of the factor)
  bool pending = false; // wave-uniform: some lane has a pshift
#pragma unroll
  for (int db = 0; db < NDB; db++) O[db] = v16f{};
  v16f NB = {};    // nb in every register: the initial accumulator of the score products
  // Q centring: nb enters through the mean-term product instead (B operand
  // {1, 1, nb_hi, nb_lo, 0 ...} in lanes 0-31, zero in lanes 32-63)
  v4i bq = v4i{lg ? 0 : (int)kBf16Ones, 0, 0, 0};
  auto set_nb = [&](float target) __attribute__((always_inline)) {
    // nb becomes the value of the bf16 pair nearest target; returns the change
    float value;
    const uint32_t pair = bf16_pair(target, value);
    bq[1] = lg ? 0 : (int)pair;
    const float d = value - nb;
    nb = value;
    return d;
  };
  auto mt_read = [&](int ks, int kb) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint32_t*>(smem + 2 * kVRing + ks * kMtSlot + 256 * bw + 4 * (32 * kb + lq));
  };
  v16f S[2];       // exp2 arguments x of the current tile [32-key block], refilled with the next tile's
  v8i P;           // packed probabilities of the previous tile, then of the current one

  // Scores of the tile whose K is in slot ks into S.
  auto qk = [&](int ks) __attribute__((always_inline)) {
    const uint8_t* kb_base = smem + ks * kTile;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      const v8i k0 = lds_read32(kb_base + kb * 32 * D, koff[0][0], koff[0][1]);
      if constexpr (NH == 2) {
        const v8i k1 = lds_read32(kb_base + kb * 32 * D, koff[1][0], koff[1][1]);
        v16f init;
        if constexpr (QC)
          init = mt_init(mt_read(ks, kb), bq);
        else
          init = NB;
        S[kb] = mfma_fp8_scaled(k1, qf[1], mfma_fp8_scaled(k0, qf[0], init, c_e8m0), c_e8m0);
      } else if constexpr (QC) {
        S[kb] = mfma_fp8_scaled(k0, qf[0], mt_init(mt_read(ks, kb), bq), c_e8m0);
      } else {
        S[kb] = mfma_fp8_scaled(k0, qf[0], NB, c_e8m0);
      }
    }
  };
  // Apply a pending reference shift to O and l (rare; wave-uniform branch):
  // they hold the products of tiles up to t-1, computed in the old frame.
  auto rescale = [&]() __attribute__((always_inline)) {
    if (__builtin_expect(pending, 0)) {
      const float alpha = __builtin_amdgcn_exp2f(pshift * kUnit);
      auto pa = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
      lacc[0] *= alpha;
      lacc[1] *= __uint_as_float(pa[1]);   // lane j < 16: alpha of query 16+j
#pragma unroll
      for (int db = 0; db < NDB; db++) O[db] *= alpha;
      pshift = 0.f;
      pending = false;
    }
  };
  // Reference update for the tile whose exp2 arguments are in S.  FIRST sets
  // the reference from the tile maximum.  Keys past the end of the range have
  // been set to -inf (mask_tail) before this runs.  Register r of block kb in
  // lane l holds key kbase + 32*kb + 8*(r/4) + 4*(l/32) + r%4.
  // The rare path: the row maxima of the pair lanes, the shift that puts them
  // on kRef (only where they pass kMax), applied to S, the offset of later
  // tiles (NB) and the rescale flagged for O and l.
  auto apply_shift = [&](float tl) __attribute__((always_inline)) {
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(tl), __float_as_uint(tl), false, false);
    const float xm = __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    const bool over = xm > kMax;
    float shift = over ? kRef - xm : 0.f;
    if constexpr (QC) {
      if (over) shift = set_nb(nb + shift);   // the change the rounded pair makes
    } else {
      nb += shift;
    }
    pshift = shift;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      S[0][i] += shift;
      S[1][i] += shift;
      if constexpr (!QC) NB[i] += shift;
    }
  };
  // FIRST: set the reference from this tile.  Otherwise vote, and unless
  // VOTE_ONLY apply a shift at once; VOTE_ONLY returns the lane maximum for
  // the caller to apply later (before anything reads S or NB).
  auto rowmax_update = [&](auto first_c, auto vote_only_c) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool VOTE_ONLY = decltype(vote_only_c)::value;
    // this lane's maximum of x: 16 three-input maxima (the pair lane holds the
    // other half of the row).  After the first tile only "is any x above kMax"
    // matters, and for that the maximum of the bit patterns as signed
    // integers serves: they order like the floats on positive values and
    // every negative float is a negative integer (kMax > 0), with no NaN
    // canonicalization in the integer maximum.  The float maximum is then
    // exact whenever it exceeds kMax, the only case the rare path uses it.
    auto mx3 = [](auto a, auto b, auto c) {
      if constexpr (FIRST)
        return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
      else
        return max(max(a, b), c);
    };
    auto val = [&](int kb, int r) {
      if constexpr (FIRST)
        return S[kb][r];
      else
        return __float_as_int(S[kb][r]);
    };
    using T = decltype(val(0, 0));
    T m8[8];
#pragma unroll
    for (int i = 0; i < 5; i++) m8[i] = mx3(val(0, 3 * i), val(0, 3 * i + 1), val(0, 3 * i + 2));
    m8[5] = mx3(val(0, 15), val(1, 0), val(1, 1));
#pragma unroll
    for (int i = 0; i < 2; i++) m8[6 + i] = mx3(val(1, 2 + 3 * i), val(1, 3 + 3 * i), val(1, 4 + 3 * i));
    const T n0 = mx3(val(1, 8), val(1, 9), val(1, 10));
    const T n1 = mx3(val(1, 11), val(1, 12), val(1, 13));
    const T n2 = mx3(val(1, 14), val(1, 15), m8[0]);
    const T n3 = mx3(m8[1], m8[2], m8[3]);
    const T n4 = mx3(m8[4], m8[5], m8[6]);
    const T n5 = mx3(m8[7], n0, n1);
    const T tb = mx3(mx3(n2, n3, n4), n5, n5);
    float tl;
    if constexpr (FIRST)
      tl = tb;
    else
      tl = __int_as_float(tb);
    if (FIRST) {
      auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(tl), __float_as_uint(tl), false, false);
      const float tm = __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      float shift = kRef - tm;
      if constexpr (QC)
        shift = set_nb(shift);   // nb was 0: the pair's value
      else
        nb = shift;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        S[0][i] += shift;
        S[1][i] += shift;
        if constexpr (!QC) NB[i] = shift;
      }
    } else {
      // move the reference only if the tile's largest p would exceed 448: one
      // vote over the wave; the row maxima and shifts only on the rare path
      pending = __builtin_amdgcn_ballot_w64(tb > __float_as_int(kMax)) != 0;
      if constexpr (!VOTE_ONLY)
        if (pending) apply_shift(tl);
    }
    return tl;
  };
  // E4M3 probabilities of keys 8*q4 + 4*(lane/32) + 0..3 of block kb (one P dword).
  auto probs4 = [&](int kb, int q4, int kbase) __attribute__((always_inline)) {
    if constexpr (EXACT) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(S[kb][4 * q4 + i]);
      return cvt4(p[0], p[1], p[2], p[3]);
    } else {
      uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(S[kb][4 * q4 + 0], 0, 0u);
      w = __builtin_amdgcn_cvt_pk_u8_f32(S[kb][4 * q4 + 1], 1, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(S[kb][4 * q4 + 2], 2, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(S[kb][4 * q4 + 3], 3, w);
      return (int)w;
    }
  };
  // Scores of this lane's keys with tile-relative offset 32*kb + 8*(r/4) + r%4
  // (register r of block kb; the lane's keys add 4*lg) above dlim to -inf:
  // min(S, +-inf) with the sign of dlim + 1/2 - offset, so no compare or
  // condition register per score.
  auto mask_after = [&](int dlim) __attribute__((always_inline)) {
    const float df = (float)dlim + 0.5f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float d = df - (float)(32 * kb + 8 * (r >> 2) + (r & 3));
        S[kb][r] = __builtin_fminf(S[kb][r], __uint_as_float((__float_as_uint(d) & 0x80000000u) | 0x7f800000u));
      }
  };
  // Causal: scores of keys after this lane's query to -inf in tile t (only
  // tiles from q0 on hold such keys).  Register r of block kb holds key
  // t*64 + 32*kb + 8*(r/4) + 4*lg + r%4.
  const int qq = q0 + 32 * wave + lq;
  auto mask_causal = [&](int t) __attribute__((always_inline)) { mask_after(qq - t * kBN - 4 * lg); };
  // Keys past the end of the range (the last tile of a segment whose length is
  // not a multiple of 64) to -inf in tile t, before the reference update.
  // Their K rows are zero codes, so unmasked they would score exactly 0: a
  // whole segment's centred keys average to zero, so some real score is >= 0
  // and such a key could not move the reference, but the keys of one piece of
  // a split item need not average to zero, and a zero score far above every
  // real one would take the reference and flush the real probabilities.
  // (Causal: keys past the segment end lie after every stored query and are
  // masked by mask_causal.)
  const bool ragged = !CAUSAL && Lk < nkt * kBN;
  auto mask_tail = [&](int t) __attribute__((always_inline)) { mask_after(Lk - 1 - t * kBN - 4 * lg); };
  // Softmax of tile 0 (reference from its maximum) into P, then the scores of
  // tile 1 (K in slot 1) into S.
  auto first_tile = [&]() __attribute__((always_inline)) {
    if (ragged && nkt == 1) mask_tail(0);
    if (CAUSAL && q0 == 0) mask_causal(0);
    rowmax_update(std::true_type{}, std::false_type{});
#pragma unroll
    for (int w = 0; w < 8; w++) P[w] = probs4(w >> 2, w & 3, 0);
    qk(1);
  };

  // Prologue: K(0), then the loads an iteration -2 would issue (K(1), K(2),
  // V(0), V(1)).  Even iteration t waits for the loads of iteration t-2, which
  // hold the K(t+1), K(t+2) and V(t), V(t+1) that iterations t and t+1 read,
  // passes the barrier, and issues K(t+3), K(t+4), V(t+2), V(t+3).  Slot
  // (t+3)%4 last held K(t-1) and V(t-1), slot t%4 K(t), slot (t+2)%4 V(t-2):
  // all read before the barrier, which waits for every LDS read of the wave.
  load_k(0, 0);
#pragma unroll
  for (int i = 1; i <= kBarEvery; i++) load_k(i, i);
#pragma unroll
  for (int i = 0; i < kBarEvery; i++) load_v(i, i);
  // K(0) has landed once only the later loads are outstanding (with split
  // loads only the K waves issued K loads, and only they need to wait)
  if constexpr (kSplitLoads) {
    // K waves wait for K(0) (those that also load mean-term tiles for their
    // MT(0), issued after it); a V wave that loads mean-term tiles waits for MT(0)
    if (k_wave && mt_wave)
      wait_vmcnt<kBarEvery * (kLoadsPerTile + 1)>();
    else if (k_wave)
      wait_vmcnt<kBarEvery * kLoadsPerTile>();
    else if (mt_wave)
      wait_vmcnt<kBarEvery * (kLoadsPerTile + 1)>();
  } else if (mt_wave) {
    wait_vmcnt<kBarEvery * (2 * kLoadsPerTile + 1)>();   // its mean-term loads follow each K load
  } else {
    wait_vmcnt<2 * kBarEvery * kLoadsPerTile>();
  }
  barrier();
  qk(0);
  // Iteration 0: reference from tile 0; nothing to add to O yet.
  wait_vmcnt<0>();
  barrier();
#pragma unroll
  for (int i = 1; i <= kBarEvery; i++) load_k(kBarEvery + i, (kBarEvery + i) % kSlots);
#pragma unroll
  for (int i = 0; i < kBarEvery; i++) load_v(kBarEvery + i, (kBarEvery + i) % kSlots);
  first_tile();
  keep(P);
  // V operands of the next product, read at the end of the iteration before it.
  v8i vf[NDB];
#pragma unroll
  for (int db = 0; db < NDB; db++) vf[db] = lds_read32(smem + kVRing + db * 2048, voff[0], voff[1]);
  // Iteration t (S holds tile t's scores, P tile t-1's probabilities, vf the
  // V(t-1) operands): at even t the barrier and the loads above; a pending
  // rescale; O += P(t-1) V(t-1), softmax of tile t with the scores of tile
  // t+1 computed into S as its blocks free up, and V(t) read into vf.  The
  // scores computed by the last iteration (of a clamped copy of the last
  // tile) are not used.
  //
  // The body is laid out as nine slots, each one matrix product plus about a
  // ninth of the vector work, with the LDS reads of later products' operands
  // issued one or more slots ahead; scheduling fences keep the compiler from
  // merging the slots.  The two score chains are interleaved (first halves of
  // both 32-key blocks, then the second halves) so neither waits on the
  // other's accumulator.
  const int tdiag = q0 / kBN;   // causal: tiles from here on hold keys after some query
  auto iter = [&](int t, auto ph_c, auto tail_c) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_c)::value;   // t % kSlots
    constexpr bool TAIL = decltype(tail_c)::value;   // may be the last tile: mask keys past the range end
    if (PH % kBarEvery == 0) {
      wait_vmcnt<0>();
      barrier();
    }
    rescale();
    if (PH % kBarEvery == 0) {
#pragma unroll
      for (int i = 1; i <= kBarEvery; i++) load_k(t + kBarEvery + i, (PH + kBarEvery + i) % kSlots);
#pragma unroll
      for (int i = 0; i < kBarEvery; i++) load_v(t + kBarEvery + i, (PH + kBarEvery + i) % kSlots);
    }
    const uint8_t* vn = smem + kVRing + PH * kTile;                  // V(t), read for the next iteration
    const uint8_t* kb = smem + ((PH + 1) % kSlots) * kTile;          // K(t+1)
    const int kbase = t * kBN;
    v8i Pn;
    if constexpr (QC && NH == 2) {
      // Q centring: as below, with the two mean-term products (the initial
      // accumulators of the score chains, nb included) ahead of the chains
      v8i kf[2][2];
      const uint32_t mtv0 = mt_read((PH + 1) % kSlots, 0);
      const uint32_t mtv1 = mt_read((PH + 1) % kSlots, 1);
      kf[0][0] = lds_read32(kb, koff[0][0], koff[0][1]);
      kf[1][0] = lds_read32(kb + 4096, koff[0][0], koff[0][1]);
      fence();
      O[0] = mfma_fp8(vf[0], P, O[0]);
      kf[0][1] = lds_read32(kb, koff[1][0], koff[1][1]);
      if (CAUSAL && t >= tdiag) mask_causal(t);
      if (TAIL && ragged && t == nkt - 1) mask_tail(t);
      const float tlv = rowmax_update(std::false_type{}, std::integral_constant<bool, !EXACT>{});
      fence();
      O[1] = mfma_fp8(vf[1], P, O[1]);
      kf[1][1] = lds_read32(kb + 4096, koff[1][0], koff[1][1]);
      if constexpr (!EXACT)
        if (__builtin_expect(pending, 0)) apply_shift(tlv);
      Pn[0] = probs4(0, 0, kbase);
      fence();
      O[2] = mfma_fp8(vf[2], P, O[2]);
      Pn[1] = probs4(0, 1, kbase);
      fence();
      O[3] = mfma_fp8(vf[3], P, O[3]);
      Pn[2] = probs4(0, 2, kbase);
      fence();
      lacc = mfma16_fp8(sel, P, lacc);
      vf[0] = lds_read32(vn + 0 * 2048, voff[0], voff[1]);
      vf[1] = lds_read32(vn + 1 * 2048, voff[0], voff[1]);
      Pn[3] = probs4(0, 3, kbase);
      fence();
      const v16f m0 = mt_init(mtv0, bq);
      Pn[4] = probs4(1, 0, kbase);
      fence();
      const v16f m1 = mt_init(mtv1, bq);
      Pn[5] = probs4(1, 1, kbase);
      fence();
      const v16f s0 = mfma_fp8_scaled(kf[0][0], qf[0], m0, c_e8m0);
      Pn[6] = probs4(1, 2, kbase);
      fence();
      const v16f s1 = mfma_fp8_scaled(kf[1][0], qf[0], m1, c_e8m0);
      vf[2] = lds_read32(vn + 2 * 2048, voff[0], voff[1]);
      vf[3] = lds_read32(vn + 3 * 2048, voff[0], voff[1]);
      Pn[7] = probs4(1, 3, kbase);
      fence();
      S[0] = mfma_fp8_scaled(kf[0][1], qf[1], s0, c_e8m0);
      fence();
      S[1] = mfma_fp8_scaled(kf[1][1], qf[1], s1, c_e8m0);
    } else if constexpr (NH == 2) {
      v8i kf[2][2];
      kf[0][0] = lds_read32(kb, koff[0][0], koff[0][1]);
      kf[1][0] = lds_read32(kb + 4096, koff[0][0], koff[0][1]);
      fence();
      O[0] = mfma_fp8(vf[0], P, O[0]);
      kf[0][1] = lds_read32(kb, koff[1][0], koff[1][1]);
      if (CAUSAL && t >= tdiag) mask_causal(t);   // wave-uniform branch, diagonal tiles only
      if (TAIL && ragged && t == nkt - 1) mask_tail(t);   // wave-uniform branch, last tile only
      // log-linear codes: the vote's outcome is looked at one product later,
      // so the branch does not wait on the maximum tree
      const float tlv = rowmax_update(std::false_type{}, std::integral_constant<bool, !EXACT>{});
      fence();
      O[1] = mfma_fp8(vf[1], P, O[1]);
      kf[1][1] = lds_read32(kb + 4096, koff[1][0], koff[1][1]);
      if constexpr (!EXACT)
        if (__builtin_expect(pending, 0)) apply_shift(tlv);
      Pn[0] = probs4(0, 0, kbase);
      fence();
      O[2] = mfma_fp8(vf[2], P, O[2]);
      Pn[1] = probs4(0, 1, kbase);
      fence();
      O[3] = mfma_fp8(vf[3], P, O[3]);
      Pn[2] = probs4(0, 2, kbase);
      fence();
      lacc = mfma16_fp8(sel, P, lacc);
      vf[0] = lds_read32(vn + 0 * 2048, voff[0], voff[1]);
      vf[1] = lds_read32(vn + 1 * 2048, voff[0], voff[1]);
      Pn[3] = probs4(0, 3, kbase);
      fence();
      const v16f s0 = mfma_fp8_scaled(kf[0][0], qf[0], NB, c_e8m0);
      Pn[4] = probs4(1, 0, kbase);
      fence();
      const v16f s1 = mfma_fp8_scaled(kf[1][0], qf[0], NB, c_e8m0);
      vf[2] = lds_read32(vn + 2 * 2048, voff[0], voff[1]);
      vf[3] = lds_read32(vn + 3 * 2048, voff[0], voff[1]);
      Pn[5] = probs4(1, 1, kbase);
      fence();
      S[0] = mfma_fp8_scaled(kf[0][1], qf[1], s0, c_e8m0);
      Pn[6] = probs4(1, 2, kbase);
      fence();
      Pn[7] = probs4(1, 3, kbase);
      S[1] = mfma_fp8_scaled(kf[1][1], qf[1], s1, c_e8m0);
    } else if constexpr (QC) {
      // head_dim 64 with Q centring: the two mean-term products ahead of the
      // two score products
      v8i kf[2];
      const uint32_t mtv0 = mt_read((PH + 1) % kSlots, 0);
      const uint32_t mtv1 = mt_read((PH + 1) % kSlots, 1);
      kf[0] = lds_read32(kb, koff[0][0], koff[0][1]);
      kf[1] = lds_read32(kb + 32 * D, koff[0][0], koff[0][1]);
      fence();
      O[0] = mfma_fp8(vf[0], P, O[0]);
      if (CAUSAL && t >= tdiag) mask_causal(t);
      if (TAIL && ragged && t == nkt - 1) mask_tail(t);
      rowmax_update(std::false_type{}, std::false_type{});
      Pn[0] = probs4(0, 0, kbase);
      fence();
      O[1] = mfma_fp8(vf[1], P, O[1]);
      Pn[1] = probs4(0, 1, kbase);
      Pn[2] = probs4(0, 2, kbase);
      fence();
      lacc = mfma16_fp8(sel, P, lacc);
      vf[0] = lds_read32(vn + 0 * 2048, voff[0], voff[1]);
      vf[1] = lds_read32(vn + 1 * 2048, voff[0], voff[1]);
      Pn[3] = probs4(0, 3, kbase);
      fence();
      const v16f m0 = mt_init(mtv0, bq);
      Pn[4] = probs4(1, 0, kbase);
      fence();
      const v16f m1 = mt_init(mtv1, bq);
      Pn[5] = probs4(1, 1, kbase);
      fence();
      const v16f s0 = mfma_fp8_scaled(kf[0], qf[0], m0, c_e8m0);
      Pn[6] = probs4(1, 2, kbase);
      fence();
      const v16f s1 = mfma_fp8_scaled(kf[1], qf[0], m1, c_e8m0);
      Pn[7] = probs4(1, 3, kbase);
      S[0] = s0;
      S[1] = s1;
    } else {
      // head_dim 64: two score products and two P V products a tile; the
      // vector work is the same as for 128 channels, so it sets the pace
      v8i kf[2];
      kf[0] = lds_read32(kb, koff[0][0], koff[0][1]);
      kf[1] = lds_read32(kb + 32 * D, koff[0][0], koff[0][1]);
      fence();
      O[0] = mfma_fp8(vf[0], P, O[0]);
      if (CAUSAL && t >= tdiag) mask_causal(t);
      if (TAIL && ragged && t == nkt - 1) mask_tail(t);
      rowmax_update(std::false_type{}, std::false_type{});
      Pn[0] = probs4(0, 0, kbase);
      fence();
      O[1] = mfma_fp8(vf[1], P, O[1]);
      Pn[1] = probs4(0, 1, kbase);
      Pn[2] = probs4(0, 2, kbase);
      fence();
      lacc = mfma16_fp8(sel, P, lacc);
      vf[0] = lds_read32(vn + 0 * 2048, voff[0], voff[1]);
      vf[1] = lds_read32(vn + 1 * 2048, voff[0], voff[1]);
      Pn[3] = probs4(0, 3, kbase);
      Pn[4] = probs4(1, 0, kbase);
      fence();
      const v16f s0 = mfma_fp8_scaled(kf[0], qf[0], NB, c_e8m0);
      Pn[5] = probs4(1, 1, kbase);
      fence();
      const v16f s1 = mfma_fp8_scaled(kf[1], qf[0], NB, c_e8m0);
      Pn[6] = probs4(1, 2, kbase);
      Pn[7] = probs4(1, 3, kbase);
      S[0] = s0;
      S[1] = s1;
    }
    P = Pn;
    keep(P);
    keep(S[0]);   // the next tile's score products stay in this iteration
    keep(S[1]);
  };
  // Unrolled by the ring depth so that every slot address is static; the
  // last tile's iteration is always one of the tail's, where the masking of a
  // ragged end lives.
  auto iter_body = [&](int t, auto ph_c) __attribute__((always_inline)) { iter(t, ph_c, std::false_type{}); };
  auto iter_tail = [&](int t, auto ph_c) __attribute__((always_inline)) { iter(t, ph_c, std::true_type{}); };
  int t = 1;
  for (; t + kSlots < nkt; t += kSlots) unroll_iters<0, kSlots>(iter_body, t);
  tail_iters<1, kSlots + 1, kSlots>(iter_tail, t, nkt);
  // O += P(nkt-1) V(nkt-1) once every load has landed; the row sum counts
  // only keys before the segment end.  Selector byte b of lane 0 or 17 (32 or
  // 49) weights key 32*(b/16) + 8*((b/4)%4) + b%4 (+4) of the tile.
  wait_vmcnt<0>();
  barrier();
  rescale();
  {
    const int klim = Lk - (nkt - 1) * kBN - 4 * lg;
    v8i msel;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      int word = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int b = 4 * w + i;
        const int key = 32 * (b >> 4) + 8 * ((b >> 2) & 3) + (b & 3);
        word |= (key < klim ? 0x38 : 0) << (8 * i);
      }
      msel[w] = sel_lane ? word : 0;
    }
#pragma unroll
    for (int db = 0; db < NDB; db++) O[db] = mfma_fp8(vf[db], P, O[db]);
    lacc = mfma16_fp8(msel, P, lacc);
    // with every lane active: a matrix instruction moved into the stores'
    // lane-divergent branches would read inactive lanes' operands as zero
#pragma unroll
    for (int db = 0; db < NDB; db++) keep(O[db]);
  }

  // epilogue: lane l holds O^T for query l%32, channels
  // 32*db + 8*(r/4) + 4*(l/32) + r%4 in register r of block db.
  const int qrow = q0 + 32 * wave + lq;
  // the frame offset in log2 units: p = 2^(c s + nbx) for every key
  const float nbx = EXACT ? nb : (nb - kYBias) * 0.125f;
  // row sum of the E4M3 probabilities (the weights actually applied to V)
  const float l0 = __shfl(lacc[0], lq & 15);
  const float l1 = __shfl(lacc[1], lq & 15);
  const float lt = lq < 16 ? l0 : l1;
  if (slot >= 0) {
    // one piece of a split item: the normalized partial output (in output
    // units) and the log2 of its weight sum in a frame shared by all pieces
    // (p = 2^(c s) for every key), for the combine pass.  The reference is the
    // maximum of the piece's first tile, so some probability is >= 112 and
    // lt > 0; a zero sum would still give weight 0 (w = -inf) and O = 0.
    if (qrow < L) {
      const int prow = slot * kPartRows + 32 * wave + lq;
      const float inv = lt > 0.f ? s_v / lt : 0.f;
      float* orow = a.part_o + (size_t)prow * D;
#pragma unroll
      for (int db = 0; db < NDB; db++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
          *reinterpret_cast<float4*>(orow + 32 * db + 8 * q4 + 4 * lg) =
              make_float4(O[db][4 * q4 + 0] * inv, O[db][4 * q4 + 1] * inv, O[db][4 * q4 + 2] * inv,
                          O[db][4 * q4 + 3] * inv);
      if (lg == 0) a.part_w[prow] = lt > 0.f ? __log2f(lt) - nbx : -__builtin_huge_valf();
    }
  } else if (qrow < L) {
    const float inv = s_v / lt;
    uint16_t* orow = a.out + (int64_t)(si.start + qrow) * a.os0 + (int64_t)h * a.os1;
#pragma unroll
    for (int db = 0; db < NDB; db++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int d = 32 * db + 8 * q4 + 4 * lg;
        if (d < a.d_real) {   // channels past head_dim are padding
          const uint32_t b0 = f32_to_bf16_rne(O[db][4 * q4 + 0] * inv);
          const uint32_t b1 = f32_to_bf16_rne(O[db][4 * q4 + 1] * inv);
          const uint32_t b2 = f32_to_bf16_rne(O[db][4 * q4 + 2] * inv);
          const uint32_t b3 = f32_to_bf16_rne(O[db][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        }
      }
  }
  if (LSE) {
    // the log of the denominator l (keys past the end of the range were
    // masked, so they added nothing), back in the frame of the uncentred scores
    if (lg == 0 && qrow < L) {
      const float lse2 = __log2f(lt) - nbx;
      const float v = QC ? lse2 * kLn2 + a.softmax_scale * (s_q * qmu + qmm) : lse2 * kLn2 + a.softmax_scale * s_q * qmu;
      if (slot >= 0)
        a.part_lse[slot * kPartRows + 32 * wave + lq] = v;
      else
        a.lse[(int64_t)h * a.tokens + si.start + qrow] = v;
    }
  }
}

// Merge of the pieces of one split work item: for every query row of the
// item, out = sum_i W_i O_i / sum_i W_i with O_i the piece's normalized output
// and log2 W_i its weight (log-sum-exp combination over disjoint key ranges),
// rounded to BF16 once; the LSE is the log-sum-exp of the pieces' LSEs.
// 64 threads per 32 query rows (blockIdx.y picks the 32-row block of the
// item, so even a few split items spread over many compute units): thread t
// takes row t/2, channels (D/2)*(t%2) .. +D/2.  The pieces are added in index
// order, so the result is deterministic.
constexpr int kCombineRows = 32;
template <int D>
__global__ __launch_bounds__(2 * kCombineRows) void k_combine(CombineArgs a) {
  constexpr int HD = D / 2;   // channels per thread
  const int4 it = a.items[blockIdx.x];
  const SegInfo si = a.segs[it.x];
  const int n = split_pieces(it.w);
  const int slot0 = split_slot0(it.w);
  const int r = kCombineRows * blockIdx.y + (threadIdx.x >> 1);
  const int half = threadIdx.x & 1;
  const int qrow = it.y + r;
  if (qrow >= si.len) return;
  float w[kMaxSplit];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kMaxSplit; i++)
    if (i < n) {
      w[i] = a.part_w[(slot0 + i) * kPartRows + r];
      m = __builtin_fmaxf(m, w[i]);
    }
  // a piece of zero weight has w = -inf and contributes nothing; if every
  // piece had zero weight the row would be written as zeros
  if (m == -__builtin_huge_valf()) m = 0.f;
  float acc[HD];
#pragma unroll
  for (int j = 0; j < HD; j++) acc[j] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxSplit; i++)
    if (i < n) {
      const float alpha = __builtin_amdgcn_exp2f(w[i] - m);
      den += alpha;
      const float4* src = reinterpret_cast<const float4*>(a.part_o + ((size_t)(slot0 + i) * kPartRows + r) * D + HD * half);
#pragma unroll
      for (int j = 0; j < HD / 4; j++) {
        const float4 v = src[j];
        acc[4 * j + 0] += alpha * v.x;
        acc[4 * j + 1] += alpha * v.y;
        acc[4 * j + 2] += alpha * v.z;
        acc[4 * j + 3] += alpha * v.w;
      }
    }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* orow = a.out + (int64_t)(si.start + qrow) * a.os0 + (int64_t)it.z * a.os1 + HD * half;
#pragma unroll
  for (int j = 0; j < HD / 8; j++) {
    if (HD * half + 8 * j >= a.d_real) break;   // channels past head_dim are padding
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; e++) b[e] = f32_to_bf16_rne(acc[8 * j + e] * inv);
    *reinterpret_cast<uint4*>(orow + 8 * j) =
        make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
  }
  if (a.lse != nullptr && half == 0) {
    float lm = -__builtin_huge_valf();
    float lv[kMaxSplit];
#pragma unroll
    for (int i = 0; i < kMaxSplit; i++)
      if (i < n) {
        lv[i] = a.part_lse[(slot0 + i) * kPartRows + r];
        lm = __builtin_fmaxf(lm, lv[i]);
      }
    float se = 0.f;
    if (lm != -__builtin_huge_valf()) {
#pragma unroll
      for (int i = 0; i < kMaxSplit; i++)
        if (i < n) se += __expf(lv[i] - lm);
    }
    a.lse[(int64_t)it.z * a.tokens + si.start + qrow] = lm + __logf(se);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.nitems == 0) return hipSuccess;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(k_combine<64>, dim3(a.nitems, a.bm / kCombineRows), dim3(2 * kCombineRows), 0, stream, a);
  else
    hipLaunchKernelGGL(k_combine<kHeadDim>, dim3(a.nitems, a.bm / kCombineRows), dim3(2 * kCombineRows), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BM, bool EXACT, bool QC>
void launch_attention_d(const AttentionArgs& a, hipStream_t stream) {
  const dim3 g(a.nitems), b(2 * BM);
  if (a.causal) {
    // causal plans always use 256-query items (the planner picks 128 only
    // for small non-causal work), so no 128-query causal kernel is built
    if constexpr (BM == 256) {
      if (a.lse != nullptr)
        hipLaunchKernelGGL((k_attn<true, true, D, BM, EXACT, QC>), g, b, 0, stream, a);
      else
        hipLaunchKernelGGL((k_attn<false, true, D, BM, EXACT, QC>), g, b, 0, stream, a);
    }
  } else if (a.lse != nullptr) {
    hipLaunchKernelGGL((k_attn<true, false, D, BM, EXACT, QC>), g, b, 0, stream, a);
  } else {
    hipLaunchKernelGGL((k_attn<false, false, D, BM, EXACT, QC>), g, b, 0, stream, a);
  }
}

template <bool EXACT>
void launch_attention_e(const AttentionArgs& a, hipStream_t stream) {
  if (a.head_dim == 64 && a.q_centre)
    launch_attention_d<64, 256, EXACT, true>(a, stream);       // 64 channels: 256-query items only
  else if (a.head_dim == 64)
    launch_attention_d<64, 256, EXACT, false>(a, stream);
  else if (a.q_centre && a.bm == 128)
    launch_attention_d<kHeadDim, 128, EXACT, true>(a, stream);
  else if (a.q_centre)
    launch_attention_d<kHeadDim, 256, EXACT, true>(a, stream);
  else if (a.bm == 128)
    launch_attention_d<kHeadDim, 128, EXACT, false>(a, stream);
  else
    launch_attention_d<kHeadDim, 256, EXACT, false>(a, stream);
}

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream) {
  if (a.nitems == 0) return hipSuccess;
  if (a.causal && a.bm != 256) return hipErrorInvalidValue;   // see launch_attention_d
  if (a.exact_probs)
    launch_attention_e<true>(a, stream);
  else
    launch_attention_e<false>(a, stream);
  return hipGetLastError();
}

}  // namespace fp8attn
