// FP8 (E4M3) flash-attention forward for gfx950.
//
// Method (sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for
// SM120 GPUs", "Modifications", kernel.py item): E4M3 operands for both
// products with FP32 accumulation, an online softmax kept in registers, the
// probabilities packed to E4M3 inside registers, and K/V tiles prefetched one
// stage ahead so the copy overlaps the math.  The output is rounded to BF16
// once (FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page).
//
// gfx950 mapping
//   * One workgroup = 4 waves = 128 queries of one (segment, head); each wave
//     owns 32 queries.  Keys are walked in tiles of 64.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x64_f8f6f4 (A = 32 keys x 64 channels from LDS, B = the
//     wave's 32 queries x 64 channels held in registers for the whole loop).
//     In the 32x32 accumulator layout lane l holds query l%32 and 16 keys, so
//     the row max and row sum are in-lane, plus one exchange between lanes l
//     and l^32 (v_permlane32_swap).
//   * The accumulator registers of two 32-key blocks, converted to E4M3 with
//     v_cvt_pk_fp8_f32, are exactly the B operand (64 keys x 32 queries) of
//     O^T += V^T P^T.  The key order this implies inside a 64-key group is
//     baked into the workspace V layout by the pack pass, so the P registers
//     never leave the lane.
//   * Probabilities are scaled so that the running row maximum maps to 448,
//     the largest E4M3 value: p = exp2(c*s - (c*m - log2 448)) with
//     c = softmax_scale * s_q * s_k * log2(e).  The row sum l accumulates the
//     FP32 p; the final O = acc * s_v / l.
//   * Rescaling of the accumulators is skipped when no row maximum of the
//     wave grew (a wave-uniform branch).
//   * LDS tiles are double-buffered; the next tile is fetched into registers
//     while the current one is consumed and stored after it, so one barrier
//     per tile suffices.  16-byte chunks are XOR-swizzled against bank
//     conflicts of the operand reads.
#include "internal.h"

namespace fp8attn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448)
constexpr float kLn2 = 0.6931471805599453f;

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

// LDS tile geometry: K tile [64 keys][128 B], V^T tile [128 channels][64 B].
__device__ __forceinline__ int k_lds_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
__device__ __forceinline__ int v_lds_off(int d, int chunk) { return d * 64 + ((chunk ^ ((d >> 2) & 3)) << 4); }

__global__ __launch_bounds__(256, 2) void k_attn(AttentionArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][kBN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][kHeadDim * kBN];

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

  // The wave's 32 queries as the B operand: lane l holds query l%32, channels
  // 64*half + 32*(l/32) .. +32.  Query rows past the segment end read zero codes.
  const int qrow = q0 + wave * 32 + lq;
  v8i qf[2];
#pragma unroll
  for (int half = 0; half < 2; half++)
    qf[half] = *reinterpret_cast<const v8i*>(Qh + (size_t)qrow * kHeadDim + 64 * half + 32 * lg);

  // Tile staging: each thread moves two 16-byte chunks of K and two of V^T.
  uint4 kreg[2], vreg[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int ci = tid + 256 * u;
      const int kr = ci >> 3, kc = ci & 7;
      kreg[u] = *reinterpret_cast<const uint4*>(Kh + (size_t)(kt * kBN + kr) * kHeadDim + kc * 16);
      const int vd = ci >> 2, vc = ci & 3;
      vreg[u] = *reinterpret_cast<const uint4*>(Vh + (size_t)vd * a.rows + kt * kBN + vc * 16);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int ci = tid + 256 * u;
      *reinterpret_cast<uint4*>(&sK[buf][k_lds_off(ci >> 3, ci & 7)]) = kreg[u];
      *reinterpret_cast<uint4*>(&sV[buf][v_lds_off(ci >> 2, ci & 3)]) = vreg[u];
    }
  };

  v16f O[4];
#pragma unroll
  for (int i = 0; i < 4; i++) O[i] = v16f{};
  float m = -__builtin_inff();   // running max of raw scores of this lane's query
  float l = 0.f;                  // partial row sum (this lane's keys)

  const int nkt = (L + kBN - 1) / kBN;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; kt++) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);

    // S^T for two 32-key blocks
    v16f S[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      S[kb] = v16f{};
      const int row = 32 * kb + lq;
#pragma unroll
      for (int half = 0; half < 2; half++) {
        const int ch = 4 * half + 2 * lg;
        const uint4 lo = *reinterpret_cast<const uint4*>(&sK[buf][k_lds_off(row, ch)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&sK[buf][k_lds_off(row, ch + 1)]);
        const v8i av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        S[kb] = mfma_fp8(av, qf[half], S[kb]);
      }
    }

    // mask keys past the segment end (only the last tile can have any)
    const int kbase = kt * kBN;
    if (kbase + kBN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = kbase + 32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (key >= L) S[kb][r] = -__builtin_inff();
        }
    }

    float mx = S[0][0];
#pragma unroll
    for (int r = 1; r < 16; r++) mx = fmaxf(mx, S[0][r]);
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, S[1][r]);
    mx = fmaxf(mx, swap32(mx));
    const float mnew = fmaxf(m, mx);
    if (__ballot(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(c * (m - mnew));
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 4; i++) O[i] *= alpha;
      m = mnew;
    }
    const float bias = c * m - kLog2_448;

    v8i P;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][4 * q + i], c, -bias));
          l += p[i];
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        P[4 * kb + q] = w;
      }
    }

#pragma unroll
    for (int db = 0; db < 4; db++) {
      const int d = 32 * db + lq;
      const uint4 lo = *reinterpret_cast<const uint4*>(&sV[buf][v_lds_off(d, 2 * lg)]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&sV[buf][v_lds_off(d, 2 * lg + 1)]);
      const v8i av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      O[db] = mfma_fp8(av, P, O[db]);
    }

    if (kt + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue
  l += swap32(l);
  if (qrow >= L) return;
  const float inv = s_v / l;
  uint16_t* orow = a.out + (int64_t)(si.start + qrow) * a.os0 + (int64_t)h * a.os1;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int d = 32 * db + 8 * q + 4 * lg;
      const uint32_t b0 = f32_to_bf16_rne(O[db][4 * q + 0] * inv);
      const uint32_t b1 = f32_to_bf16_rne(O[db][4 * q + 1] * inv);
      const uint32_t b2 = f32_to_bf16_rne(O[db][4 * q + 2] * inv);
      const uint32_t b3 = f32_to_bf16_rne(O[db][4 * q + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }

  if (a.lse != nullptr) {
    // natural-log LSE of the uncentred scores: the centred LSE plus
    // softmax_scale * (q_hat . mu), since every centred key differs from the
    // uncentred one by the segment mean mu.
    const float* mu = a.mu + ((size_t)it.x * a.heads + h) * kHeadDim;
    float dot = 0.f;
#pragma unroll
    for (int half = 0; half < 2; half++)
#pragma unroll
      for (int w = 0; w < 8; w++) {
        const float* md = mu + 64 * half + 32 * lg + 4 * w;
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 0) * md[0];
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 1) * md[1];
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 2) * md[2];
        dot += __builtin_amdgcn_cvt_f32_fp8(qf[half][w], 3) * md[3];
      }
    dot += swap32(dot);
    if (lg == 0) {
      const float lse2 = c * m + __log2f(l) - kLog2_448;
      a.lse[(int64_t)h * a.tokens + si.start + qrow] = lse2 * kLn2 + a.softmax_scale * s_q * dot;
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
