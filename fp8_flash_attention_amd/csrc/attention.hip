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
//   * One workgroup = 4 waves = kBM queries of one (segment, head); each wave
//     owns kBM/4 queries as kQB blocks of 32 (kBM = 128: one block per wave).
//     Three workgroups share a CU, so every SIMD runs three waves and
//     interleaves one wave's softmax (VALU) with another's matrix products
//     (MFMA).  Keys are walked in tiles of kBN = 64.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x64_f8f6f4 (A = 32 keys x 64 channels read from LDS,
//     B = 32 queries x 64 channels held in registers for the whole loop).
//     With kQB = 2 each A fragment read from LDS would feed the MFMAs of both
//     query blocks; at kQB = 1 the LDS reads (~160 B/clk per CU) still stay
//     below the MFMA time and the smaller register file buys the third wave.
//   * In the 32x32 accumulator layout lane l holds query l%32 and 16 keys of
//     a 32-key block, so the row max is in-lane plus one exchange between
//     lanes l and l^32 (v_permlane32_swap).
//   * The accumulators of two 32-key blocks, converted to E4M3 with
//     v_cvt_pk_fp8_f32, are exactly the B operand (64 keys x 32 queries) of
//     O^T += V^T P^T.  The key order this implies inside a 64-key group is
//     baked into the workspace V layout by the pack pass, so the P registers
//     never leave the lane.
//   * Row sums l come from the matrix core too: one
//     v_mfma_f32_16x16x128_f8f6f4 per tile multiplies the packed P^T by a
//     constant 0/1 selector, which adds the 64 key bytes of query j (lanes j
//     and j+32) into row 0 and those of query 16+j (lanes j+16 and j+48) into
//     row 1.  l is the sum of the E4M3 probabilities that actually weight V,
//     and no vector adds are spent on it.  When the caller asks for the LSE,
//     an FP32 sum of the unrounded probabilities is kept as well.
//   * Probabilities: p = exp2(c*s - (c*m - log2 112)) with
//     c = softmax_scale * s_q * s_k * log2(e) and m a per-query reference
//     maximum.  m is only moved (and O, l rescaled) when a 32-key block holds
//     a score above m + 2/c, i.e. when some p could exceed 448, the largest
//     E4M3 value; otherwise 112 * 4 bounds p.  The test is wave-uniform, so
//     the rescale runs only on the rare blocks where a maximum grows by more
//     than a factor 4.  If that happens in the second key block of a tile,
//     the first block's probabilities (already packed against the old m) are
//     re-encoded scaled by the same factor.  The final O = acc * s_v / l.
//   * K/V tiles go through three LDS stages: while tile j is consumed, tile
//     j+2 is fetched into registers in two halves (its K part during the first
//     key block, its V part during the second) and written to its stage after
//     each half, so at most two 16-byte chunks per lane are in flight and one
//     barrier per tile suffices.  The loop is unrolled over the stages so
//     every LDS address is a per-lane base plus an immediate.  16-byte chunks
//     are XOR-swizzled against bank conflicts of the operand reads.
#include <type_traits>

#include "internal.h"

namespace fp8attn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2Ref = 6.807354922057604f;   // log2(112): reference maximum maps to 448 / 4
constexpr float kLog2Max = 8.807354922057604f;   // log2(448), the largest E4M3 value
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kQB = kBM / (4 * 32);              // 32-query blocks per wave
constexpr int kQW = 32 * kQB;                    // queries per wave
static_assert(kQB == 1 || kQB == 2, "4 waves x 32 or 64 queries");
constexpr int kKTile = kBN * kHeadDim;           // bytes of one K (or V) tile
constexpr int kStage = 2 * kKTile;               // K tile + V tile
constexpr int kStages = 3;
constexpr int kBufferFlags = 0x00020000;         // raw buffer descriptor word 3 (gfx9 family)

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  // cbsz = blgp = 0 selects E4M3 for both operands; zero scales select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// max / sum of x over lanes l and l^32.  v_permlane32_swap on (x, x) leaves
// {x[l], x[l^32]} in its two results (in an order that depends on the lane
// half), so combining both results needs no lane select.
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max of the 16 values of one accumulator block as a v_max3 tree
__device__ __forceinline__ float max16(const v16f& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
  const float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
  const float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 codes of four floats in one dword.  Both halves are written, so the
// first conversion's merge operand is left undefined (no register to clear).
__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_nondeterministic_value(0), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__device__ __forceinline__ v8i lds_read32(const uint8_t* base, int off_lo, int off_hi) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + off_lo);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + off_hi);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// LDS tile geometry inside a stage: K tile [64 keys][128 B] at 0, V^T tile
// [128 channels][64 B] at kKTile.  Chunk swizzles: K row r, chunk c at
// r*128 + ((c ^ ((r >> 1) & 7)) * 16); V^T row d, chunk c at
// kKTile + d*64 + ((c ^ ((d >> 2) & 3)) * 16).
__device__ __forceinline__ int k_lds_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
__device__ __forceinline__ int v_lds_off(int d, int chunk) { return kKTile + d * 64 + ((chunk ^ ((d >> 2) & 3)) << 4); }

__device__ __forceinline__ v4f mfma16_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <bool EXACT_SUM>
__global__ __launch_bounds__(256, kQB == 1 ? 3 : 2) void k_attn(AttentionArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];

  const int4 it = a.items[blockIdx.x];
  if (it.x < 0) return;
  const SegInfo si = a.segs[it.x];
  const int q0 = it.y;
  const int h = it.z;
  const int L = si.len;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int lg = lane >> 5;

  const size_t hrow = (size_t)h * a.rows + si.row0;
  const uint8_t* Qh = a.q_codes + hrow * kHeadDim;
  const uint8_t* Kh = a.k_codes + hrow * kHeadDim;
  const uint8_t* Vh = a.v_codes + (size_t)h * kHeadDim * a.rows + si.row0;

  const float s_q = a.scales[h];
  const float s_k = a.scales[a.heads + h];
  const float s_v = a.scales[2 * a.heads + h];
  const float c = a.softmax_scale * s_q * s_k * kLog2e;

  // Q as B operands: block qb holds queries q0 + 64*wave + 32*qb + (lane%32),
  // channels 64*half + 32*(lane/32) .. +32.  Rows past the segment end read
  // zero codes, guard rows or the next segment's rows and are never stored.
  v8i qf[kQB][2];
#pragma unroll
  for (int qb = 0; qb < kQB; qb++)
#pragma unroll
    for (int half = 0; half < 2; half++)
      qf[qb][half] = *reinterpret_cast<const v8i*>(
          Qh + (size_t)(q0 + kQW * wave + 32 * qb + lq) * kHeadDim + 64 * half + 32 * lg);

  // Per-lane LDS read offsets (the rest of every address is an immediate).
  int koff[2][2];   // [half][sub]
#pragma unroll
  for (int half = 0; half < 2; half++)
#pragma unroll
    for (int sub = 0; sub < 2; sub++) koff[half][sub] = k_lds_off(lq, 4 * half + 2 * lg + sub);
  int voff[2];
#pragma unroll
  for (int sub = 0; sub < 2; sub++) voff[sub] = v_lds_off(lq, 2 * lg + sub);

  // Copy geometry: thread t moves 16-byte chunks t and t+256 of the K tile
  // (64 rows x 8 chunks) and of the V^T tile (128 rows x 4 chunks).  Loads go
  // through buffer descriptors of this head's K and V^T regions: the lane
  // offset is a 32-bit register, the tile offset a scalar, so no vector
  // address arithmetic runs per tile.
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kh, (short)0, (int)((a.rows - si.row0) * kHeadDim), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Vh, (short)0, (int)(a.rows * kHeadDim - si.row0), kBufferFlags);
  int ksrc[2], vsrc[2];   // per-lane byte offsets inside a tile
  int kdst[2], vdst[2];   // per-lane LDS offsets inside a stage
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int ci = tid + 256 * u;
    ksrc[u] = (ci >> 3) * kHeadDim + (ci & 7) * 16;
    kdst[u] = k_lds_off(ci >> 3, ci & 7);
    vsrc[u] = (ci >> 2) * (int)a.rows + (ci & 3) * 16;
    vdst[u] = v_lds_off(ci >> 2, ci & 3);
  }
  const int nkt = (L + kBN - 1) / kBN;
  u32x4 stg0, stg1;   // two staged 16-byte chunks (separate variables keep them in registers)
  // clamped tile index: always a valid tile of this segment
  auto fetch_k = [&](int kt) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    stg0 = __builtin_amdgcn_raw_buffer_load_b128(krs, ksrc[0], kt * kBN * kHeadDim, 0);
    stg1 = __builtin_amdgcn_raw_buffer_load_b128(krs, ksrc[1], kt * kBN * kHeadDim, 0);
  };
  auto fetch_v = [&](int kt) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    stg0 = __builtin_amdgcn_raw_buffer_load_b128(vrs, vsrc[0], kt * kBN, 0);
    stg1 = __builtin_amdgcn_raw_buffer_load_b128(vrs, vsrc[1], kt * kBN, 0);
  };
  auto put_k = [&](uint8_t* stage) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(stage + kdst[0]) = stg0;
    *reinterpret_cast<u32x4*>(stage + kdst[1]) = stg1;
  };
  auto put_v = [&](uint8_t* stage) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(stage + vdst[0]) = stg0;
    *reinterpret_cast<u32x4*>(stage + vdst[1]) = stg1;
  };

  // q_hat . mu per query, for the natural-log LSE of the uncentred scores:
  // every centred key differs from the uncentred one by the segment mean mu,
  // so the centred LSE is short by softmax_scale * (q_hat . mu).
  float qmu[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) qmu[qb] = 0.f;
  if (EXACT_SUM) {
    const float* mu = a.mu + ((size_t)it.x * a.heads + h) * kHeadDim;
#pragma unroll
    for (int qb = 0; qb < kQB; qb++) {
      float dot = 0.f;
#pragma unroll
      for (int half = 0; half < 2; half++)
#pragma unroll
        for (int w = 0; w < 8; w++) {
          const float* md = mu + 64 * half + 32 * lg + 4 * w;
          dot += __builtin_amdgcn_cvt_f32_fp8(qf[qb][half][w], 0) * md[0];
          dot += __builtin_amdgcn_cvt_f32_fp8(qf[qb][half][w], 1) * md[1];
          dot += __builtin_amdgcn_cvt_f32_fp8(qf[qb][half][w], 2) * md[2];
          dot += __builtin_amdgcn_cvt_f32_fp8(qf[qb][half][w], 3) * md[3];
        }
      qmu[qb] = sum_pair32(dot);
    }
  }

  // Row-sum selector for the 16x16x128 product: E4M3 1.0 in every byte of
  // lanes 0 and 32 (row 0: lanes j and j+32 of P, query j) and lanes 17 and
  // 49 (row 1: lanes 16+j and 48+j, query 16+j), zero elsewhere.
  const int one = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x38383838 : 0;
  const v8i sel = v8i{one, one, one, one, one, one, one, one};
  v4f lacc[kQB];   // row sums of the packed P: lane j < 16 holds query j (row 0) and 16+j (row 1)

  v16f O[kQB][4];
  float nb[kQB];   // exp2 argument offset: x = c*s + nb, i.e. nb = log2(112) - c*m
  float l[kQB];    // partial row sums (this lane's keys)
  v8i P[kQB];      // packed probabilities; kept across tiles so packing needs no cleared register
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
#pragma unroll
    for (int db = 0; db < 4; db++) O[qb][db] = v16f{};
    l[qb] = 0.f;
    lacc[qb] = v4f{};
    P[qb] = v8i{};
  }

  // 32x32 score block S^T = K Q^T for key block kb of the tile in `sb`.
  auto scores = [&](const uint8_t* sb, int kb, int qb) __attribute__((always_inline)) {
    const v8i k0 = lds_read32(sb + kb * 32 * 128, koff[0][0], koff[0][1]);
    const v8i k1 = lds_read32(sb + kb * 32 * 128, koff[1][0], koff[1][1]);
    return mfma_fp8(k1, qf[qb][1], mfma_fp8(k0, qf[qb][0], v16f{}));
  };
  // keys at or past the segment end -> -inf.  Register r of lane l holds key
  // kbase + 32*kb + 8*(r/4) + 4*(l/32) + r%4.
  auto mask = [&](v16f& S, int kbase, int kb) __attribute__((always_inline)) {
    const int lim = L - kbase - 32 * kb - 4 * lg;
#pragma unroll
    for (int r = 0; r < 16; r++)
      if (8 * (r >> 2) + (r & 3) >= lim) S[r] = -__builtin_inff();
  };

  // One 64-key tile from LDS stage `sb`.  Main-loop tiles (MASKED false)
  // fetch tile kt+2 into stage `nxt` along the way; the last tile (MASKED
  // true) fetches nothing and masks keys at or past the segment end.
  //
  // Per 32x32 block: x = c*s + nb are the exp2 arguments; p = 2^x <= 448 as
  // long as max x <= log2(448).  Otherwise (rare) the reference moves so that
  // the block maximum maps to 112: x, nb shift by log2(112) - max x, and O, l
  // (and the tile's already packed first block) scale by 2^shift.  The max is
  // taken over x, FMA results, which need no NaN canonicalization.
  auto tile = [&](const uint8_t* sb, int kt, uint8_t* nxt, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr bool PREFETCH = !MASKED;
    const int kbase = kt * kBN;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (PREFETCH) {
        if (kb == 0) fetch_k(kt + 2);
        else {
          put_k(nxt);
          fetch_v(kt + 2);
        }
      }
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) {
        v16f S = scores(sb, kb, qb);
        if (MASKED) mask(S, kbase, kb);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; r++) x[r] = __builtin_fmaf(S[r], c, nb[qb]);
        // v_max3 tree: 5 + 2 + 1 instructions
        const float m0 = fmaxf(fmaxf(x[0], x[1]), x[2]), m1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
        const float m2 = fmaxf(fmaxf(x[6], x[7]), x[8]), m3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
        const float m4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
        const float tb = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), x[15]));
        auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(tb), __float_as_uint(tb), false, false);
        const float t0 = __uint_as_float(pr[0]), t1 = __uint_as_float(pr[1]);
        if (__ballot(t0 > kLog2Max || t1 > kLog2Max)) {
          const float tm = fmaxf(t0, t1);
          const float shift = tm > kLog2Max ? kLog2Ref - tm : 0.f;
          const float alpha = __builtin_amdgcn_exp2f(shift);
          if (kb == 1) {
            // the first key block's probabilities were packed against the old
            // reference: re-encode them scaled by alpha
#pragma unroll
            for (int w = 0; w < 4; w++) {
              const int v = P[qb][w];
              P[qb][w] = cvt4(__builtin_amdgcn_cvt_f32_fp8(v, 0) * alpha, __builtin_amdgcn_cvt_f32_fp8(v, 1) * alpha,
                              __builtin_amdgcn_cvt_f32_fp8(v, 2) * alpha, __builtin_amdgcn_cvt_f32_fp8(v, 3) * alpha);
            }
          }
          if (EXACT_SUM) l[qb] *= alpha;
          {
            auto pa = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
            lacc[qb][0] *= alpha;
            lacc[qb][1] *= __uint_as_float(pa[1]);   // lane j < 16: alpha of query 16+j
          }
#pragma unroll
          for (int db = 0; db < 4; db++) O[qb][db] *= alpha;
          nb[qb] += shift;
#pragma unroll
          for (int r = 0; r < 16; r++) x[r] += shift;
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(x[4 * q4 + i]);
          if (EXACT_SUM) l[qb] += (p[0] + p[1]) + (p[2] + p[3]);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], P[qb][4 * kb + q4], false);
          P[qb][4 * kb + q4] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        }
      }
    }

#pragma unroll
    for (int db = 0; db < 4; db++) {
      const v8i vf = lds_read32(sb + db * 32 * 64, voff[0], voff[1]);
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) O[qb][db] = mfma_fp8(vf, P[qb], O[qb][db]);
    }
#pragma unroll
    for (int qb = 0; qb < kQB; qb++) lacc[qb] = mfma16_fp8(sel, P[qb], lacc[qb]);
    if (PREFETCH) put_v(nxt);
  };

  // Pipeline: tile j lives in stage j % 3 and tile j+1 is already in its
  // stage; tile j+2 is fetched while tile j is consumed.  Every tile but the
  // last runs unmasked with static stage addresses; the last one runs masked.
  uint8_t* const stage0 = smem;
  fetch_k(0);
  put_k(stage0);
  fetch_v(0);
  put_v(stage0);
  fetch_k(1);
  put_k(stage0 + kStage);
  fetch_v(1);
  put_v(stage0 + kStage);
  // Initial reference: the maximum score of the first key block of tile 0
  // (masked when the segment is shorter than the block), mapped to 112.
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    v16f S = scores(stage0, 0, qb);
    if (L < 32) mask(S, 0, 0);
    float t = S[0];
#pragma unroll
    for (int r = 1; r < 16; r++) t = fmaxf(t, S[r]);
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    t = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    nb[qb] = kLog2Ref - c * t;
  }
  auto step = [&](auto stage_c, int kt) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_c)::value;
    __syncthreads();              // tile kt is in stage ST; stage (ST+2)%3 is free
    tile(stage0 + ST * kStage, kt, stage0 + ((ST + 2) % kStages) * kStage, std::false_type{});
  };
  const int last = nkt - 1;
  int kt = 0;
  for (; kt + kStages <= last; kt += kStages) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
    step(std::integral_constant<int, 2>{}, kt + 2);
  }
  if (kt < last) {
    step(std::integral_constant<int, 0>{}, kt);
    if (++kt < last) {
      step(std::integral_constant<int, 1>{}, kt);
      ++kt;
    }
  }
  __syncthreads();
  tile(stage0 + (last % kStages) * kStage, last, nullptr, std::true_type{});

  // epilogue: lane l holds O^T for query (l%32) of each block, channels
  // 32*db + 8*(r/4) + 4*(l/32) + r%4 in register r of block db.
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    const int qrow = q0 + kQW * wave + 32 * qb + lq;
    // row sum of the E4M3 probabilities (the weights actually applied to V)
    const float l0 = __shfl(lacc[qb][0], lq & 15);
    const float l1 = __shfl(lacc[qb][1], lq & 15);
    const float lt = lq < 16 ? l0 : l1;
    if (qrow < L) {
      const float inv = s_v / lt;
      uint16_t* orow = a.out + (int64_t)(si.start + qrow) * a.os0 + (int64_t)h * a.os1;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int d = 32 * db + 8 * q4 + 4 * lg;
          const uint32_t b0 = f32_to_bf16_rne(O[qb][db][4 * q4 + 0] * inv);
          const uint32_t b1 = f32_to_bf16_rne(O[qb][db][4 * q4 + 1] * inv);
          const uint32_t b2 = f32_to_bf16_rne(O[qb][db][4 * q4 + 2] * inv);
          const uint32_t b3 = f32_to_bf16_rne(O[qb][db][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        }
    }
    if (EXACT_SUM) {
      const float le = sum_pair32(l[qb]);
      if (lg == 0 && qrow < L) {
      const float lse2 = __log2f(le) - nb[qb];
      a.lse[(int64_t)h * a.tokens + si.start + qrow] = lse2 * kLn2 + a.softmax_scale * s_q * qmu[qb];
      }
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream) {
  if (a.nitems == 0) return hipSuccess;
  if (a.lse != nullptr)
    hipLaunchKernelGGL(k_attn<true>, dim3(a.nitems), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_attn<false>, dim3(a.nitems), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp8attn
