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
//   * One workgroup = 4 waves = 256 queries of one (segment, head); each wave
//     owns 64 queries as two blocks of 32.  Two workgroups share a CU, so
//     every SIMD runs two waves and interleaves one wave's softmax (VALU)
//     with the other's matrix products (MFMA).  Keys are walked in tiles of 64.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x64_f8f6f4 (A = 32 keys x 64 channels read from LDS,
//     B = 32 queries x 64 channels held in registers for the whole loop).
//     Each A fragment read from LDS feeds the MFMAs of both query blocks,
//     which halves the LDS read traffic per MFMA (LDS bandwidth, ~160 B/clk
//     per CU, would otherwise bound the loop).
//   * In the 32x32 accumulator layout lane l holds query l%32 and 16 keys of
//     a 32-key block, so the row max and row sum are in-lane plus one
//     exchange between lanes l and l^32 (v_permlane32_swap).
//   * The accumulators of two 32-key blocks, converted to E4M3 with
//     v_cvt_pk_fp8_f32, are exactly the B operand (64 keys x 32 queries) of
//     O^T += V^T P^T.  The key order this implies inside a 64-key group is
//     baked into the workspace V layout by the pack pass, so the P registers
//     never leave the lane.
//   * Probabilities: p = exp2(c*s - (c*m - log2 112)) with
//     c = softmax_scale * s_q * s_k * log2(e) and m a per-query reference
//     maximum.  m is only moved (and O, l rescaled) when a 32-key block holds
//     a score above m + 2/c, i.e. when some p could exceed 448, the largest
//     E4M3 value; otherwise 112 * 4 bounds p.  The test is wave-uniform, so
//     the rescale runs only on the rare blocks where a maximum grows by more
//     than a factor 4.  If that happens in the second key block of a tile,
//     the first block's probabilities (already packed against the old m) are
//     first added into O with an MFMA whose other half of P is zero.  The row
//     sum l accumulates the FP32 p; the final O = acc * s_v / l.
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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2Ref = 6.807354922057604f;   // log2(112): reference maximum maps to 448 / 4
constexpr float kSlack = 2.0f;                   // log2 headroom between 112 and 448
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kQB = kBM / (4 * 32);              // 32-query blocks per wave
constexpr int kQW = 32 * kQB;                    // queries per wave
static_assert(kQB == 1 || kQB == 2, "4 waves x 32 or 64 queries");
constexpr int kKTile = kBN * kHeadDim;           // bytes of one K (or V) tile
constexpr int kStage = 2 * kKTile;               // K tile + V tile
constexpr int kStages = 3;

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  // cbsz = blgp = 0 selects E4M3 for both operands; zero scales select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Value from lane l^32 of x.
__device__ __forceinline__ float swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const int lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
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
  const float thr = kSlack / c;   // raw-score headroom before p could pass 448

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
  // (64 rows x 8 chunks) and of the V^T tile (128 rows x 4 chunks).
  uint32_t ksrc[2], vsrc[2];   // per-lane byte offsets from the tile base
  int kdst[2], vdst[2];        // per-lane LDS offsets inside a stage
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int ci = tid + 256 * u;
    ksrc[u] = (uint32_t)((ci >> 3) * kHeadDim + (ci & 7) * 16);
    kdst[u] = k_lds_off(ci >> 3, ci & 7);
    vsrc[u] = (uint32_t)((ci >> 2) * a.rows + (ci & 3) * 16);
    vdst[u] = v_lds_off(ci >> 2, ci & 3);
  }
  const int nkt = (L + kBN - 1) / kBN;
  uint4 stg0, stg1;   // two staged 16-byte chunks (separate variables keep them in registers)
  // clamped tile index: always a valid tile of this segment
  auto fetch_k = [&](int kt) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    const uint8_t* base = Kh + (size_t)kt * kBN * kHeadDim;
    stg0 = *reinterpret_cast<const uint4*>(base + ksrc[0]);
    stg1 = *reinterpret_cast<const uint4*>(base + ksrc[1]);
  };
  auto fetch_v = [&](int kt) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    const uint8_t* base = Vh + (size_t)kt * kBN;
    stg0 = *reinterpret_cast<const uint4*>(base + vsrc[0]);
    stg1 = *reinterpret_cast<const uint4*>(base + vsrc[1]);
  };
  auto put_k = [&](uint8_t* stage) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(stage + kdst[0]) = stg0;
    *reinterpret_cast<uint4*>(stage + kdst[1]) = stg1;
  };
  auto put_v = [&](uint8_t* stage) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(stage + vdst[0]) = stg0;
    *reinterpret_cast<uint4*>(stage + vdst[1]) = stg1;
  };

  // q_hat . mu per query, for the natural-log LSE of the uncentred scores:
  // every centred key differs from the uncentred one by the segment mean mu,
  // so the centred LSE is short by softmax_scale * (q_hat . mu).
  float qmu[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) qmu[qb] = 0.f;
  if (a.lse != nullptr) {
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
      qmu[qb] = dot + swap32(dot);
    }
  }

  v16f O[kQB][4];
  float m[kQB], l[kQB];   // reference max (raw score units); partial row sums (this lane's keys)
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
#pragma unroll
    for (int db = 0; db < 4; db++) O[qb][db] = v16f{};
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
  }

  // One 64-key tile from LDS stage `sb`.  Main-loop tiles (MASKED false)
  // fetch tile kt+2 into stage `nxt` along the way; the last tile (MASKED
  // true) fetches nothing and sets keys at or past the segment end to -inf.
  auto tile = [&](const uint8_t* sb, int kt, uint8_t* nxt, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr bool PREFETCH = !MASKED;
    const int kbase = kt * kBN;
    v8i P[kQB];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      const v8i k0 = lds_read32(sb + kb * 32 * 128, koff[0][0], koff[0][1]);
      const v8i k1 = lds_read32(sb + kb * 32 * 128, koff[1][0], koff[1][1]);
      if (PREFETCH) {
        if (kb == 0) fetch_k(kt + 2);
        else {
          put_k(nxt);
          fetch_v(kt + 2);
        }
      }
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) {
        v16f S = mfma_fp8(k0, qf[qb][0], v16f{});
        S = mfma_fp8(k1, qf[qb][1], S);
        if (MASKED) {
          // key of register r: kbase + 32*kb + 8*(r/4) + 4*(lane/32) + r%4
          const int lim = L - kbase - 32 * kb - 4 * lg;
#pragma unroll
          for (int r = 0; r < 16; r++)
            if (8 * (r >> 2) + (r & 3) >= lim) S[r] = -__builtin_inff();
        }
        float t = fmaxf(S[0], S[1]);
#pragma unroll
        for (int r = 2; r < 16; r++) t = fmaxf(t, S[r]);
        t = fmaxf(t, swap32(t));
        if (__ballot(t > m[qb] + thr)) {
          const float mn = fmaxf(m[qb], t);
          const float alpha = __builtin_amdgcn_exp2f(c * (m[qb] - mn));
          if (kb == 1) {
            // the first key block's probabilities were packed against the old
            // reference: re-encode them scaled by alpha
#pragma unroll
            for (int w = 0; w < 4; w++) {
              const int x = P[qb][w];
              P[qb][w] = cvt4(__builtin_amdgcn_cvt_f32_fp8(x, 0) * alpha, __builtin_amdgcn_cvt_f32_fp8(x, 1) * alpha,
                              __builtin_amdgcn_cvt_f32_fp8(x, 2) * alpha, __builtin_amdgcn_cvt_f32_fp8(x, 3) * alpha);
            }
          }
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; db++) O[qb][db] *= alpha;
          m[qb] = mn;
        }
        const float nb = kLog2Ref - c * m[qb];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * q4 + i], c, nb));
          l[qb] += (p[0] + p[1]) + (p[2] + p[3]);
          P[qb][4 * kb + q4] = cvt4(p[0], p[1], p[2], p[3]);
        }
      }
    }

#pragma unroll
    for (int db = 0; db < 4; db++) {
      const v8i vf = lds_read32(sb + db * 32 * 64, voff[0], voff[1]);
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) O[qb][db] = mfma_fp8(vf, P[qb], O[qb][db]);
    }
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
    const float lt = l[qb] + swap32(l[qb]);
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
    if (a.lse != nullptr && lg == 0 && qrow < L) {
      const float lse2 = c * m[qb] + __log2f(lt) - kLog2Ref;
      a.lse[(int64_t)h * a.tokens + si.start + qrow] = lse2 * kLn2 + a.softmax_scale * s_q * qmu[qb];
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream) {
  if (a.nitems == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn, dim3(a.nitems), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp8attn
