// Block-scaled FP4 (MXFP4) flash-attention forward for gfx950: the variant of
// the FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page (description
// under the output formula) on gfx950's scaled matrix products.
//
// Method: both products take E2M1 operands with one power-of-two (E8M0) scale
// per 32 elements of the contraction axis; the softmax stays in FP32; the
// probabilities are converted to E2M1 in registers with one scale per 32 keys;
// K is centred by its segment's per-channel mean and Q by its 128-row block's
// mean, whose term qm . k is added back to the scores; the output is rounded to
// BF16 once.
//
// gfx950 mapping (shared with the E4M3 kernel where it carries over)
//   * One workgroup = 4 waves of 32 queries (128 queries of one segment and
//     head), two per CU; key tiles of 64.  Each SIMD then runs one wave of
//     each workgroup, so a wave waiting at its workgroup's barrier leaves the
//     SIMD to a wave that is not (8.7% faster than one 8-wave workgroup per
//     CU, whose two waves per SIMD share every barrier; the halved tile bytes
//     of FP4 keep the doubled L2-to-LDS traffic cheap).  Scores are computed transposed,
//     S^T = K Q^T, on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands
//     E2M1 (cbsz = blgp = 4; 32 clocks a product, half the E4M3 time).  Q and
//     the block-mean operand stay in registers; K comes from LDS.
//   * The K rows of a tile are read into the A operand in an order that gives
//     lane l (query l%32, half h = l/32) keys 32h .. 32h+31 of the tile in its
//     32 score registers: A row m of 32-key block kb holds key
//     32*((m/4)%2) + 16*kb + 4*(m/8) + m%4.  A lane's 32 probabilities are then
//     one scale block of the P V product's B operand: its E8M0 scale is the
//     lane's own, taken from the lane's maximum with no exchange, and V^T needs
//     no key permutation.
//   * Score offsets: the accumulators start at a per-query whole number nb, so
//     x = c (q . k) + nb and p = exp2(x) need no other vector work, and every
//     rescale of O and l is an exact power of two.  The probability codes
//     E2M1(p / 2^e), e = ceil(max - log2 6), then depend on the scores alone
//     (the reference cancels).  Unlike E4M3 the codes never saturate, so the
//     reference moves only when a tile's maximum would bring p near the top of
//     the float range (above 2^kRefMax).
//   * The block-mean term: two more score products per 32-key block with the
//     block-mean operand (the same for all 32 queries of a wave) as B, chained
//     in front of the Q products, so it lands in the accumulator with no vector
//     work.  Without Q centring the kernel is instantiated without them.
//   * Row sums: v_mfma_scale_f32_16x16x128_f8f6f4 of the packed P with a 0/1
//     selector, P's per-lane scale as the B scale.
//   * K and V^T tiles (4 KB of codes + 256 B of scales each) reach LDS by direct
//     buffer loads into four-slot rings (34 KB a workgroup); barriers every
//     second iteration; the
//     last tile's scores past the segment end are masked to -inf before its
//     maximum, so padding never moves a probability scale.
#include "internal.h"

namespace fp8attn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLog2Six = 2.584962500721156f;   // log2(6), the largest E2M1 value
constexpr float kRefMax = 24.f;                  // move the reference once a score passes this
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSlot = kMxTile + kMxTileScales;  // bytes of one ring slot (codes, then scales)
constexpr int kSlots = 4;
constexpr int kBarEvery = kSlots / 2;
constexpr int kWaves = kMxBM / 32;            // 4 waves of 32 queries
constexpr int kVRing = kSlots * kSlot;
constexpr int kBufferFlags = 0x00020000;
static_assert(kMxBM == 128 && kBN == 64, "4 waves x 32 queries, 64-key tiles");

__device__ __forceinline__ v8i widen(const v4i& a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1); }

// a (E2M1, scale byte SA of sa) x b (E2M1, scale byte SB of sb) + c
template <int SA, int SB>
__device__ __forceinline__ v16f mfma4(const v4i& a, const v4i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a), widen(b), c, 4, 4, SA, sa, SB, sb);
}
__device__ __forceinline__ v4f mfma16_4(const v4i& a, const v4i& b, const v4f& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(a), widen(b), c, 4, 4, 0, 127, 0, sb);
}

// sum of x over lanes l and l^32 (v_permlane32_swap of (x, x) hands each
// lane the other half's value in one of the two results)
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// value of an E2M1 code (OCP MX: sign, 2 exponent bits with bias 1, 1
// mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), built as float bits
__device__ __forceinline__ float e2m1_value(uint32_t n) {
  const uint32_t e = (n >> 1) & 3u, m = n & 1u;
  const uint32_t mag = e != 0u ? ((e + 126u) << 23) | (m << 22) : (m != 0u ? 126u << 23 : 0u);
  return __uint_as_float(mag | ((n & 8u) << 28));
}

// sum over this lane's 64 channels of an E2M1 B operand (f[kk]: channels
// 64*kk + 32*(lane/32) .. +32, two per byte, low nibble first; scale byte kk
// of sc) times mu (mu[c] for those channels, c = 64*kk + j, already offset by
// 32*(lane/32))
__device__ __forceinline__ float dot_mu(const v4i f[2], int sc, const float* mu) {
  float s = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; kk++) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++)
#pragma unroll
      for (int j = 0; j < 8; j++) t += e2m1_value(((uint32_t)f[kk][w] >> (4 * j)) & 15u) * mu[64 * kk + 8 * w + j];
    s += __builtin_ldexpf(t, ((sc >> (8 * kk)) & 255) - 127);
  }
  return s;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// E2M1 codes of p[0..7] / scale, two per byte, low nibble first.
__device__ __forceinline__ int cvt8(const float* p, float scale) {
  int u;
  asm volatile("" : "=v"(u));   // every byte is written: no register to clear
  u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, p[0], p[1], scale, 0);
  u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, p[2], p[3], scale, 1);
  u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, p[4], p[5], scale, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, p[6], p[7], scale, 3);
}

__device__ __forceinline__ v4i lds_read16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// LDS slot geometry.  K: [64 keys][64 B], 16-byte chunk c of key r at
// r*64 + 16*(c ^ sk(r)), sk(r) = bit 2 of r | bit 5 of r << 1 (the 16 lanes of
// a read phase then hit 16 distinct bank groups).  V^T: [128 channels][32 B],
// chunk c of channel d at d*32 + 16*(c ^ bit 3 of d).  Scales follow the codes.
__device__ __forceinline__ int k_swz(int r) { return ((r >> 2) & 1) | (((r >> 5) & 1) << 1); }
__device__ __forceinline__ int k_lds_off(int r, int c) { return r * 64 + ((c ^ k_swz(r)) << 4); }
__device__ __forceinline__ int v_lds_off(int d, int c) { return d * 32 + ((c ^ ((d >> 3) & 1)) << 4); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds" : : "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff));
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dword %1, %2, %3 offen lds" : : "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff));
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ void keep(const v4i& v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void keep(const v16f& v) { asm volatile("" ::"v"(v)); }

template <int I, int N, typename F>
__device__ __forceinline__ void unroll_iters(F& iter, int t) {
  if constexpr (I < N) {
    iter(t + I, std::integral_constant<int, (I + 1) % N>{});
    unroll_iters<I + 1, N>(iter, t);
  }
}
template <int P, int N, typename F>
__device__ __forceinline__ void tail_iters(F& iter, int& t, int nlast) {
  if constexpr (P < N) {
    if (t < nlast) iter(t++, std::integral_constant<int, P>{});
    tail_iters<P + 1, N>(iter, t, nlast);
  }
}

template <bool QC, bool LSE, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves, 2) void k_attn_mx(MxAttentionArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kVRing];

  const int4 it = a.items[blockIdx.x];
  if (it.x < 0) return;
  const SegInfo si = a.segs[it.x];
  const int q0 = it.y;
  const int h = it.z;
  const int L = si.len;
  // key tiles of the item (causal: up to its last query), or of one piece of
  // a split item: tiles [kt0, kt0 + nkt), whose keys past the range end (Lk
  // keys from the range start) are masked in the last tile
  const int nkt_seg = ((CAUSAL ? min(L, q0 + kMxBM) : L) + kBN - 1) / kBN;
  int kt0 = 0, nkt = nkt_seg, slot = -1;
  if (it.w != 0) {
    const int n = split_pieces(it.w), i = split_index(it.w);
    kt0 = nkt_seg * i / n;
    nkt = nkt_seg * (i + 1) / n - kt0;
    slot = split_slot0(it.w) + i;
  }
  const int Lk = min(L - kt0 * kBN, nkt * kBN);
  const int tdiag = q0 / kBN;   // causal: tiles from here on hold keys after some query of the item
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int lg = lane >> 5;

  const int64_t hrow = (int64_t)h * a.rows + si.row0;          // first workspace row of the segment
  const int64_t htile = (int64_t)h * (a.rows / kBN) + si.row0 / kBN;
  const int qi = q0 + 32 * wave + lq;                           // this lane's query (segment-relative)

  // Q (B operand): query q0 + 32*wave + lq, channels 64*kk + 32*lg .. +32, and
  // the two scale bytes of those blocks (bytes kk = 0, 1).
  const int64_t qrow_ws = hrow + q0 + 32 * wave + lq;
  v4i qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; kk++) qf[kk] = *reinterpret_cast<const v4i*>(a.q_codes + qrow_ws * kMxRow + 32 * kk + 16 * lg);
  const int qsc = *reinterpret_cast<const uint16_t*>(a.q_scales + qrow_ws * 4 + 2 * lg);
  v4i mf[2];
  int msc = 0;
  if (QC) {
    const int64_t blk = (int64_t)h * (a.rows / kMxQBlock) + (si.row0 + q0) / kMxQBlock;
#pragma unroll
    for (int kk = 0; kk < 2; kk++) mf[kk] = *reinterpret_cast<const v4i*>(a.qm_codes + blk * kMxRow + 32 * kk + 16 * lg);
    msc = *reinterpret_cast<const uint16_t*>(a.qm_scales + blk * 4 + 2 * lg);
  }

  // Per-lane LDS read offsets: K row of A row lq in block kb, chunks 2*kk + lg.
  int koff[2][2], kso[2];
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
    const int key = 32 * ((lq >> 2) & 1) + 16 * kb + 4 * (lq >> 3) + (lq & 3);
#pragma unroll
    for (int kk = 0; kk < 2; kk++) koff[kb][kk] = k_lds_off(key, 2 * kk + lg);
    kso[kb] = kMxTile + key * 4 + 2 * lg;   // this lane's two K scale bytes
  }
  int voff[4];
#pragma unroll
  for (int db = 0; db < 4; db++) voff[db] = v_lds_off(32 * db + lq, lg);
  const int vso = kMxTile + (32 * lg + lq) * 4;   // V^T scale bytes of channels lq + 32*db

  // Direct loads: every wave loads 1 KB of each K tile's codes and 1 KB of
  // each V^T tile's (the 16-byte LDS chunk p = 64*wave + lane receives the
  // global chunk the swizzle places there); wave 0 also loads the K tile's 256
  // scale bytes, wave 1 the V^T tile's.  Tile indices past the last tile are
  // clamped (a free slot refilled with valid data).
  const int p = 64 * wave + lane;
  int srck, srcv;
  {
    const int r = p >> 2;
    srck = r * kMxRow + (((p & 3) ^ k_swz(r)) << 4);
    const int d = p >> 1;
    srcv = d * (kBN / 2) + (((p & 1) ^ ((d >> 3) & 1)) << 4);
  }
  const uint8_t* kcb = a.k_codes + (hrow + kt0 * kBN) * kMxRow;
  const uint8_t* vcb = a.v_codes + (htile + kt0) * kMxTile;
  const uint8_t* ksb = a.k_scales + (hrow + kt0 * kBN) * 4;
  const uint8_t* vsb = a.v_scales + (htile + kt0) * kMxTileScales;
  const __amdgpu_buffer_rsrc_t kcrs = __builtin_amdgcn_make_buffer_rsrc((void*)kcb, (short)0, nkt * kMxTile, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vcrs = __builtin_amdgcn_make_buffer_rsrc((void*)vcb, (short)0, nkt * kMxTile, kBufferFlags);
  const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)ksb, (short)0, nkt * kMxTileScales, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vsrs = __builtin_amdgcn_make_buffer_rsrc((void*)vsb, (short)0, nkt * kMxTileScales, kBufferFlags);
  const uint32_t lds_k = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  const uint32_t lds_v = lds_k + kVRing;
  auto load_k = [&](int kt, int slot) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    lds_dma16(kcrs, lds_k + slot * kSlot + 1024 * wave, srck, kt * kMxTile);
    if (wave == 0) lds_dma4(ksrs, lds_k + slot * kSlot + kMxTile, 4 * lane, kt * kMxTileScales);
  };
  auto load_v = [&](int kt, int slot) __attribute__((always_inline)) {
    kt = kt < nkt ? kt : nkt - 1;
    lds_dma16(vcrs, lds_v + slot * kSlot + 1024 * wave, srcv, kt * kMxTile);
    if (wave == 1) lds_dma4(vsrs, lds_v + slot * kSlot + kMxTile, 4 * lane, kt * kMxTileScales);
  };

  // Row-sum selector: E2M1 1.0 (code 2) in every nibble of lanes 0 and 32 (row
  // 0: query j = lanes j, j+32 of P) and 17 and 49 (row 1: query 16+j).
  const bool sel_lane = lane == 0 || lane == 32 || lane == 17 || lane == 49;
  const int one = sel_lane ? 0x22222222 : 0;
  const v4i sel = v4i{one, one, one, one};

  v16f O[4];       // O^T: lane l holds query l%32, channels 32*db + 8*(r/4) + 4*(l/32) + r%4
  v4f lacc = {};   // row sums: lane j < 16 holds query j (row 0) and 16+j (row 1)
  float nb = 0.f;  // whole-number offset of the exp2 arguments
  float pshift = 0.f;
  bool pending = false;
#pragma unroll
  for (int db = 0; db < 4; db++) O[db] = v16f{};
  v16f NB = {};    // nb in every register: the score products' initial accumulator
  v16f S[2];       // exp2 arguments of the current tile, lane keys 32*lg + 16*kb + r
  v4i P;           // E2M1 probabilities of the previous tile, then of the current one
  int pe = 127;    // E8M0 scale byte of this lane's probabilities

  auto scores = [&](const v4i kf[2][2], const int ks[2], v16f& s0, v16f& s1) __attribute__((always_inline)) {
    if (QC) {
      s0 = mfma4<0, 0>(kf[0][0], mf[0], NB, ks[0], msc);
      s1 = mfma4<0, 0>(kf[1][0], mf[0], NB, ks[1], msc);
      s0 = mfma4<1, 1>(kf[0][1], mf[1], s0, ks[0], msc);
      s1 = mfma4<1, 1>(kf[1][1], mf[1], s1, ks[1], msc);
      s0 = mfma4<0, 0>(kf[0][0], qf[0], s0, ks[0], qsc);
      s1 = mfma4<0, 0>(kf[1][0], qf[0], s1, ks[1], qsc);
    } else {
      s0 = mfma4<0, 0>(kf[0][0], qf[0], NB, ks[0], qsc);
      s1 = mfma4<0, 0>(kf[1][0], qf[0], NB, ks[1], qsc);
    }
    s0 = mfma4<1, 1>(kf[0][1], qf[1], s0, ks[0], qsc);
    s1 = mfma4<1, 1>(kf[1][1], qf[1], s1, ks[1], qsc);
  };
  auto read_k = [&](const uint8_t* kb_base, v4i kf[2][2], int ks[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int kk = 0; kk < 2; kk++) kf[kb][kk] = lds_read16(kb_base + koff[kb][kk]);
      ks[kb] = *reinterpret_cast<const uint16_t*>(kb_base + kso[kb]);
    }
  };
  auto rescale = [&]() __attribute__((always_inline)) {
    if (pending) {
      const float alpha = __builtin_amdgcn_exp2f(pshift);   // a power of two: exact
      auto pa = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
      lacc[0] *= alpha;
      lacc[1] *= __uint_as_float(pa[1]);   // lane j < 16: alpha of query 16+j
#pragma unroll
      for (int db = 0; db < 4; db++) O[db] *= alpha;
      pshift = 0.f;
      pending = false;
    }
  };
  // Lane maximum, reference update and this lane's probability scale.
  // FIRST sets the reference: nb = -rint(row maximum).  Later tiles move it
  // only when a score would pass kRefMax (a wave-wide vote; rare).
  auto rowmax_update = [&](auto first_c) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_c)::value;
    float m8[8];
#pragma unroll
    for (int i = 0; i < 5; i++) m8[i] = __builtin_fmaxf(__builtin_fmaxf(S[0][3 * i], S[0][3 * i + 1]), S[0][3 * i + 2]);
    m8[5] = __builtin_fmaxf(__builtin_fmaxf(S[0][15], S[1][0]), S[1][1]);
#pragma unroll
    for (int i = 0; i < 2; i++)
      m8[6 + i] = __builtin_fmaxf(__builtin_fmaxf(S[1][2 + 3 * i], S[1][3 + 3 * i]), S[1][4 + 3 * i]);
    const float n0 = __builtin_fmaxf(__builtin_fmaxf(S[1][8], S[1][9]), S[1][10]);
    const float n1 = __builtin_fmaxf(__builtin_fmaxf(S[1][11], S[1][12]), S[1][13]);
    const float n2 = __builtin_fmaxf(__builtin_fmaxf(S[1][14], S[1][15]), m8[0]);
    const float n3 = __builtin_fmaxf(__builtin_fmaxf(m8[1], m8[2]), m8[3]);
    const float n4 = __builtin_fmaxf(__builtin_fmaxf(m8[4], m8[5]), m8[6]);
    const float n5 = __builtin_fmaxf(__builtin_fmaxf(m8[7], n0), n1);
    float tl = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(n2, n3), n4), n5);
    if (FIRST) {
      auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(tl), __float_as_uint(tl), false, false);
      const float tm = __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      const float shift = __builtin_rintf(-tm);
      nb = shift;
      tl += shift;
#pragma unroll
      for (int i = 0; i < 16; i++) { S[0][i] += shift; S[1][i] += shift; NB[i] = shift; }
    } else {
      pending = __builtin_amdgcn_ballot_w64(tl > kRefMax) != 0;
      if (pending) {
        auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(tl), __float_as_uint(tl), false, false);
        const float xm = __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
        const float shift = xm > kRefMax ? __builtin_rintf(-xm) : 0.f;
        nb += shift;
        pshift = shift;
        tl += shift;
#pragma unroll
        for (int i = 0; i < 16; i++) { S[0][i] += shift; S[1][i] += shift; NB[i] += shift; }
      }
    }
    // e = ceil(max - log2 6), at least -126 (a lane with every key masked has
    // max = -inf and all-zero codes)
    const float ef = __builtin_fmaxf(__builtin_ceilf(tl - kLog2Six), -126.f);
    return (int)ef;
  };
  // E2M1 probabilities of lane keys 8*w .. 8*w+7 (one P dword).
  auto probs8 = [&](int w, float scale) __attribute__((always_inline)) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; i++) p[i] = __builtin_amdgcn_exp2f(S[w >> 1][8 * (w & 1) + i]);
    return cvt8(p, scale);
  };
  auto scale_of = [](int e) { return __uint_as_float((uint32_t)(e + 127) << 23); };
  // scores of tile-relative keys >= klim to -inf (klim may differ per lane)
  // Without compares: min(S, +-inf) with the sign of (klim - key - 1/2).
  auto mask_tail = [&](int klim) __attribute__((always_inline)) {
    const float kf = (float)(klim - 32 * lg) - 0.5f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float d = kf - (float)(16 * kb + r);
        S[kb][r] = __builtin_fminf(S[kb][r], __uint_as_float((__float_as_uint(d) & 0x80000000u) | 0x7f800000u));
      }
  };
  // the limit of tile t: keys past the range end and, causal, keys after this
  // lane's query
  auto klim_of = [&](int t) __attribute__((always_inline)) {
    return CAUSAL ? min(Lk, qi + 1) - t * kBN : Lk - t * kBN;
  };

  // Prologue: K(0), K(1), K(2), V(0), V(1); wait for K(0): the loads issued
  // after it are 6 instructions for waves 0 and 1 (their scale loads) and 4
  // for waves 2 and 3.
  load_k(0, 0);
  load_k(1, 1);
  load_k(2, 2);
  load_v(0, 0);
  load_v(1, 1);
  if (wave == 0) wait_vmcnt<6>(); else if (wave == 1) wait_vmcnt<6>(); else wait_vmcnt<4>();
  barrier();
  {
    v4i kf[2][2];
    int ks[2];
    read_k(smem, kf, ks);
    scores(kf, ks, S[0], S[1]);
  }
  wait_vmcnt<0>();
  barrier();
#pragma unroll
  for (int i = 1; i <= kBarEvery; i++) load_k(kBarEvery + i, (kBarEvery + i) % kSlots);
#pragma unroll
  for (int i = 0; i < kBarEvery; i++) load_v(kBarEvery + i, (kBarEvery + i) % kSlots);
  if (nkt == 1 || (CAUSAL && tdiag == 0)) mask_tail(klim_of(0));
  {
    pe = rowmax_update(std::true_type{});
    const float sc = scale_of(pe);
#pragma unroll
    for (int w = 0; w < 4; w++) P[w] = probs8(w, sc);
    pe += 127;
  }
  keep(P);
  if (nkt > 1) {
    v4i kf[2][2];
    int ks[2];
    read_k(smem + 1 * kSlot, kf, ks);
    scores(kf, ks, S[0], S[1]);
  }
  v4i vf[4];
  int vsc = *reinterpret_cast<const int*>(smem + kVRing + vso);
#pragma unroll
  for (int db = 0; db < 4; db++) vf[db] = lds_read16(smem + kVRing + voff[db]);

  // Iteration t (1 <= t <= nkt - 2): S holds tile t's scores, P tile t-1's
  // probabilities, vf/vsc V(t-1).  The score products of tile t+1 are spread
  // between the P V products and the softmax of tile t (no scheduling fences:
  // the compiler interleaves them; 4% faster than fenced slots with Q
  // centring, the same without).  At even t the barrier and the loads of K(t+3),
  // K(t+4), V(t+2), V(t+3); a pending rescale;
  // O += P(t-1) V(t-1); the softmax of tile t; the scores of tile t+1; V(t)
  // read for the next iteration.
  auto iter = [&](int t, auto ph_c) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_c)::value;
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
    const uint8_t* vn = smem + kVRing + PH * kSlot;                  // V(t)
    const uint8_t* kbp = smem + ((PH + 1) % kSlots) * kSlot;         // K(t+1)
    v4i kf[2][2], Pn;
    int ks[2];
    read_k(kbp, kf, ks);
    O[0] = mfma4<0, 0>(vf[0], P, O[0], vsc, pe);
    if (CAUSAL && t >= tdiag) mask_tail(klim_of(t));   // wave-uniform branch, diagonal tiles only
    const int e = rowmax_update(std::false_type{});
    const float sc = scale_of(e);
    v16f s0, s1;
    O[1] = mfma4<1, 0>(vf[1], P, O[1], vsc, pe);
    if (QC) {
      s0 = mfma4<0, 0>(kf[0][0], mf[0], NB, ks[0], msc);
      s1 = mfma4<0, 0>(kf[1][0], mf[0], NB, ks[1], msc);
    } else {
      s0 = mfma4<0, 0>(kf[0][0], qf[0], NB, ks[0], qsc);
    }
    Pn[0] = probs8(0, sc);
    O[2] = mfma4<2, 0>(vf[2], P, O[2], vsc, pe);
    if (QC) {
      s0 = mfma4<1, 1>(kf[0][1], mf[1], s0, ks[0], msc);
      s1 = mfma4<1, 1>(kf[1][1], mf[1], s1, ks[1], msc);
    } else {
      s1 = mfma4<0, 0>(kf[1][0], qf[0], NB, ks[1], qsc);
    }
    Pn[1] = probs8(1, sc);
    O[3] = mfma4<3, 0>(vf[3], P, O[3], vsc, pe);
    lacc = mfma16_4(sel, P, lacc, pe);
    if (QC) {
      s0 = mfma4<0, 0>(kf[0][0], qf[0], s0, ks[0], qsc);
      s1 = mfma4<0, 0>(kf[1][0], qf[0], s1, ks[1], qsc);
    } else {
      s0 = mfma4<1, 1>(kf[0][1], qf[1], s0, ks[0], qsc);
    }
    vsc = *reinterpret_cast<const int*>(vn + vso);
#pragma unroll
    for (int db = 0; db < 4; db++) vf[db] = lds_read16(vn + voff[db]);
    Pn[2] = probs8(2, sc);
    if (QC) {
      s0 = mfma4<1, 1>(kf[0][1], qf[1], s0, ks[0], qsc);
      s1 = mfma4<1, 1>(kf[1][1], qf[1], s1, ks[1], qsc);
    } else {
      s1 = mfma4<1, 1>(kf[1][1], qf[1], s1, ks[1], qsc);
    }
    Pn[3] = probs8(3, sc);
    P = Pn;
    pe = e + 127;
    S[0] = s0;
    S[1] = s1;
    keep(P);
    keep(S[0]);
    keep(S[1]);
  };
  int t = 1;
  const int nlast = nkt - 1;   // the last tile's softmax runs after the loop
  for (; t + kSlots - 1 < nlast; t += kSlots) unroll_iters<0, kSlots>(iter, t);
  tail_iters<1, kSlots>(iter, t, nlast);

  // Last tile (t = nkt - 1 >= 1): every load has landed; mask its padding,
  // O += P(t-1) V(t-1), its softmax, then O += P(t) V(t).
  wait_vmcnt<0>();
  barrier();
  rescale();
  if (nkt > 1) {
    const int tl = nkt - 1;
#pragma unroll
    for (int db = 0; db < 4; db++) O[db] = mfma4<0, 0>(vf[db], P, O[db], __builtin_amdgcn_ubfe(vsc, 8 * db, 8), pe);
    lacc = mfma16_4(sel, P, lacc, pe);
    mask_tail(klim_of(tl));
    const int e = rowmax_update(std::false_type{});
    rescale();
    const float sc = scale_of(e);
#pragma unroll
    for (int w = 0; w < 4; w++) P[w] = probs8(w, sc);
    pe = e + 127;
    const uint8_t* vn = smem + kVRing + (tl % kSlots) * kSlot;
    vsc = *reinterpret_cast<const int*>(vn + vso);
#pragma unroll
    for (int db = 0; db < 4; db++) vf[db] = lds_read16(vn + voff[db]);
  }
#pragma unroll
  for (int db = 0; db < 4; db++) O[db] = mfma4<0, 0>(vf[db], P, O[db], __builtin_amdgcn_ubfe(vsc, 8 * db, 8), pe);
  lacc = mfma16_4(sel, P, lacc, pe);
  // The products must run with every lane active: a matrix instruction inside
  // the store's lane-divergent branch would read the operands of inactive
  // lanes (other queries' keys and channels) as zero.
#pragma unroll
  for (int db = 0; db < 4; db++) keep(O[db]);

  // epilogue: out = O / l, rounded to BF16 once; O^T: lane l holds query
  // l%32, channels 32*db + 8*(r/4) + 4*(l/32) + r%4 in register r of block db
  const int qrow = qi;
  const float l0 = __shfl(lacc[0], lq & 15);
  const float l1 = __shfl(lacc[1], lq & 15);
  const float lt = lq < 16 ? l0 : l1;
  if (slot >= 0) {
    // one piece of a split item: the normalized partial output and the log2
    // of its weight sum with the frame offset taken out (the probabilities
    // scale by exactly 2^nb), for the combine pass.  The piece's first tile
    // sets nb so that its largest probability is near 1, so lt > 0; a zero
    // sum would still give weight 0 (w = -inf) and O = 0.
    if (qrow < L) {
      const int prow = slot * kPartRows + 32 * wave + lq;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* orow = a.part_o + (size_t)prow * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
          *reinterpret_cast<float4*>(orow + 32 * db + 8 * q4 + 4 * lg) =
              make_float4(O[db][4 * q4 + 0] * inv, O[db][4 * q4 + 1] * inv, O[db][4 * q4 + 2] * inv,
                          O[db][4 * q4 + 3] * inv);
      if (lg == 0) a.part_w[prow] = lt > 0.f ? __log2f(lt) - nb : -__builtin_huge_valf();
    }
  } else if (qrow < L) {
    const float inv = 1.f / lt;
    uint16_t* orow = a.out + (int64_t)(si.start + qrow) * a.os0 + (int64_t)h * a.os1;
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int d = 32 * db + 8 * q4 + 4 * lg;
        const uint32_t b0 = f32_to_bf16_rne(O[db][4 * q4 + 0] * inv);
        const uint32_t b1 = f32_to_bf16_rne(O[db][4 * q4 + 1] * inv);
        const uint32_t b2 = f32_to_bf16_rne(O[db][4 * q4 + 2] * inv);
        const uint32_t b3 = f32_to_bf16_rne(O[db][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
  }
  if (LSE) {
    // natural-log LSE of the uncentred scores: the log of the row's
    // normalizer l (the sum of the block-scaled E2M1 weights applied to V;
    // masked keys added 0), the frame offset nb taken out, plus
    // (Qhat + QMhat) . mu, the part of every score that centring K by its
    // segment mean mu took out (both operands carry the score factor, so the
    // term is in log2 units).  Each lane holds half of its query's channels.
    const float* mu = a.mu + ((size_t)it.x * a.heads + h) * kHeadDim + 32 * lg;
    float qmu = dot_mu(qf, qsc, mu);
    if (QC) qmu += dot_mu(mf, msc, mu);
    const float qm_all = sum_pair32(qmu);
    if (lg == 0 && qrow < L) {
      const float v = (__log2f(lt) - nb + qm_all) * kLn2;
      if (slot >= 0)
        a.part_lse[slot * kPartRows + 32 * wave + lq] = v;
      else
        a.lse[(int64_t)h * a.tokens + si.start + qrow] = v;
    }
  }
}

}  // namespace

template <bool QC>
void launch_mx_q(const MxAttentionArgs& a, hipStream_t stream) {
  const dim3 g(a.nitems), b(64 * kWaves);
  if (a.causal) {
    if (a.lse != nullptr)
      hipLaunchKernelGGL((k_attn_mx<QC, true, true>), g, b, 0, stream, a);
    else
      hipLaunchKernelGGL((k_attn_mx<QC, false, true>), g, b, 0, stream, a);
  } else if (a.lse != nullptr) {
    hipLaunchKernelGGL((k_attn_mx<QC, true, false>), g, b, 0, stream, a);
  } else {
    hipLaunchKernelGGL((k_attn_mx<QC, false, false>), g, b, 0, stream, a);
  }
}

hipError_t launch_attention_mx(const MxAttentionArgs& a, hipStream_t stream) {
  if (a.nitems == 0) return hipSuccess;
  if (a.q_centre)
    launch_mx_q<true>(a, stream);
  else
    launch_mx_q<false>(a, stream);
  return hipGetLastError();
}

}  // namespace fp8attn
