// Per-head E4M3 quantization of BF16 Q/K/V views into the attention workspace.
//
// Two passes over the inputs, as in the fused_prep item of sglang PR
// "[diffusion] attention: add fp8_fa_sm120 FP8 backend for SM120 GPUs"
// ("Modifications"): a statistics pass (amax of Q and V; float64 sum, min and
// max of K per channel) and a pack pass that writes the codes.  A tiny
// finalize launch in between turns the statistics into per-head scales and
// per-(segment, head, channel) K means.  K is centred by its segment's
// per-channel mean (FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page,
// description of the K operand: the mean leaves the softmax unchanged).
//
// All three kernels are bound by HBM bandwidth: the stats pass reads 2 B per
// element, the pack pass reads 2 B and writes 1 B per element.
#include "internal.h"

#include <mutex>

namespace fp8attn {

// Statistics of fp8attn_quantize_noalloc: per (chunk, head, channel) K sums,
// minima and maxima and the per (chunk, head) amax partials of Q and V, held
// in this static device array instead of the caller's workspace.  Every device
// the library runs on holds its own copy until the process ends; each call on
// a device overwrites every entry it reads, so nothing needs clearing, and
// calls that overlap on one device race on it.
static __device__ __align__(256) uint8_t scratch[kStaticStatsBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_stats_buffer(int device, uint8_t** ptr) {
  // The array's name is a host-side stand-in; the device address is looked up
  // once per device, with that device current (the caller makes it current).
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = static_cast<uint8_t*>(p);
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

namespace {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Unpack 8 bf16 values held in a 16-byte vector.
__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// 8 BF16 channels at p, or zeros when the thread's channels lie past the
// plan's head_dim (p then points at channel 0 of the same row, so the load
// stays in bounds and is not a branch).
__device__ __forceinline__ uint4 load8(const uint16_t* p, bool live) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return live ? v : make_uint4(0u, 0u, 0u, 0u);
}

// E4M3 codes of 4 floats packed little-endian into one dword.  v_cvt_pk_fp8_f32
// on gfx950 converts to OCP E4M3 with round-to-nearest-even and keeps
// subnormals; the quantizer's inputs lie within a few ulps of +-448 at most,
// inside the range where it rounds (inputs of 464 and above would become NaN).
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// ---------------------------------------------------------------------------
// Pass 1: statistics.  D channels per head row; grid = (nchunks, ceil(H/HPB), 3),
// block = HPB * TPH threads (at most 256; the heads are spread evenly over the
// groups, so no group runs half empty).  Thread t handles head HPB*blockIdx.y + t/TPH and channels
// 8*(t%TPH) .. +8 over the chunk's tokens in ascending order (TPH = D/8
// threads per head row, HPB = 256/TPH heads per block).
// ---------------------------------------------------------------------------
// Fixed-order float64 sum, minimum and maximum of 8 channels over tokens
// [tok0 + j0, tok0 + j1), in ascending token order, written to out[0..7].
__device__ __forceinline__ void stat_rows(const uint16_t* base, int64_t ts, int tok0, int j0, int j1, bool live,
                                          KStat* out) {
  double sum[8];
  float mn[8], mx[8];
#pragma unroll
  for (int i = 0; i < 8; i++) { sum[i] = 0.0; mn[i] = __builtin_inff(); mx[i] = -__builtin_inff(); }
#pragma unroll 32
  for (int j = j0; j < j1; j++) {   // unrolled: 32 loads in flight, sums still in token order
    const uint4 v = load8(base + (int64_t)(tok0 + j) * ts, live);
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      sum[i] = sum[i] + (double)f[i];
      mn[i] = fminf(mn[i], f[i]);
      mx[i] = fmaxf(mx[i], f[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = KStat{sum[i], mn[i], mx[i]};
}

template <int D, bool QC>
__global__ __launch_bounds__(256) void k_stats(QuantizeArgs a) {
  constexpr int TPH = D / 8;
  const int HPB = blockDim.x / TPH;
  const int c = blockIdx.x;
  const int tensor = a.mx ? 1 : blockIdx.z;   // FP4 plans need only K's statistics
  const int t = threadIdx.x;
  const int h = blockIdx.y * HPB + t / TPH;
  const int c0 = (t % TPH) * 8;
  const bool active = h < a.heads;
  const Chunk ch = a.chunks[c];
  const bool live = c0 < a.d_real;   // channels past head_dim read as zeros
  const uint16_t* base = a.x[tensor] + (int64_t)h * a.hs[tensor] + (live ? c0 : 0);
  const int64_t ts = a.ts[tensor];

  if (tensor == 1) {
    if (!active) return;
    stat_rows(base, ts, ch.tok0, 0, ch.ntok, live, a.kstat + ((int64_t)c * a.heads + h) * D + c0);
    return;
  }
  if (QC && tensor == 0) {
    // Q centring (a kernel of its own, so the other's registers are unchanged):
    // the same statistics per 128-row Q block (a chunk starts on a
    // block boundary of its segment and covers one or two blocks), turned
    // into the block mean qm = fl32(sum64 / n) and this thread's part of the
    // block's centred amax, max |fl32(max - qm)|, |fl32(min - qm)| over its 8
    // channels (exact: rounding is monotone).
    if (!active) return;
    const SegInfo si = a.segs[ch.seg];
    const int64_t g0 = (si.row0 + (ch.tok0 - si.start)) / kQmBlock;
    const int64_t nqb = a.rows / kQmBlock;
    for (int half = 0; half < 2; half++) {
      const int j0 = half * kQmBlock, j1 = min(ch.ntok, j0 + kQmBlock);
      if (j0 >= j1) break;
      KStat st[8];
      stat_rows(base, ts, ch.tok0, j0, j1, live, st);
      float qm[8];
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        qm[i] = (float)(st[i].sum / (double)(j1 - j0));
        m = fmaxf(m, fmaxf(fabsf(st[i].mx - qm[i]), fabsf(st[i].mn - qm[i])));
      }
      float4* dst = reinterpret_cast<float4*>(a.qmean + ((int64_t)h * nqb + g0 + half) * D + c0);
      dst[0] = make_float4(qm[0], qm[1], qm[2], qm[3]);
      dst[1] = make_float4(qm[4], qm[5], qm[6], qm[7]);
      a.qamax[((g0 + half) * a.heads + h) * TPH + (t % TPH)] = m;
    }
    return;
  }

  float m = 0.f;
  if (active) {
#pragma unroll 32
    for (int j = 0; j < ch.ntok; j++) {   // unrolled: 32 loads in flight, sums still in token order
      const uint4 v = load8(base + (int64_t)(ch.tok0 + j) * ts, live);
      float f[8];
      unpack8(v, f);
#pragma unroll
      for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(f[i]));
    }
  }
  // reduce over the TPH lanes that share a head (consecutive lanes of one wave)
#pragma unroll
  for (int off = TPH / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, TPH));
  if (active && (t % TPH) == 0) {
    const int slot = tensor == 0 ? 0 : 1;
    a.amax[((int64_t)slot * a.nchunks + c) * a.heads + h] = m;
  }
}

// ---------------------------------------------------------------------------
// Pass 1b: finalize.  grid = H, block = D (thread = channel d).
// mu[s][h][d] = fl32(sum64 / L) with chunk sums added in ascending order from
// +0.0; K amax = max over segments and channels of |fl32(max - mu)| and
// |fl32(min - mu)|, which equals max |fl32(x - mu)| over the tokens because
// rounding is monotone; s = fl32(amax / 448), or 1 for amax == 0, for K and
// V; Q's scale is rounded up from that (q_scale_of).  With per-segment
// scales the same is done for every segment over its own chunks only.
// ---------------------------------------------------------------------------
template <int D>
__device__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if constexpr (D == 64) return v;   // one wave
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x % 64) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(red[0], red[1]);
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

// Q's scale: amax/448 rounded up to the nearest value that makes the score
// factor c = softmax_scale * s_q * s_k * log2(e) a power of two, so that the
// attention kernel applies c exactly as an E8M0 factor of its score products.
// The largest Q code stays in (224, 448] (E4M3 keeps its relative precision
// over that range).  fl32(2^m / f) can fall an ulp below amax/448; the
// largest code then rounds to 448 all the same.  If f * amax/448 is not a
// normal float the plain amax/448 scale is kept.
__device__ __forceinline__ float q_scale_of(float qa, float s_k, float softmax_scale) {
  const float base = scale_of(qa);
  const float f = softmax_scale * s_k * 1.4426950408889634f;   // c / s_q
  const float t = f * base;
  if (!(t >= 0x1p-126f && t < 0x1p126f)) return base;
  int e;
  const float fr = frexpf(t, &e);            // t = fr * 2^e, fr in [0.5, 1)
  const int m = fr == 0.5f ? e - 1 : e;      // smallest 2^m >= t
  return ldexpf(1.0f, m) / f;
}

template <int D>
__global__ __launch_bounds__(D) void k_finalize(QuantizeArgs a) {
  __shared__ float red[2];
  const int h = blockIdx.x;
  const int d = threadIdx.x;
  float qa = 0.f, va = 0.f;
  if (a.mx) {
    // FP4 plans: the K means only (the block scales are set by the pack pass)
    for (int s = 0; s < a.nseg; s++) {
      const SegInfo si = a.segs[s];
      const int nch = (si.len + kStatChunk - 1) / kStatChunk;
      float mu = 0.f;
      if (si.len > 0) {
        double sum = 0.0;
#pragma unroll 8
        for (int c = si.chunk0; c < si.chunk0 + nch; c++) sum = sum + a.kstat[((int64_t)c * a.heads + h) * D + d].sum;
        mu = (float)(sum / (double)si.len);
      }
      a.mu[((int64_t)s * a.heads + h) * D + d] = mu;
    }
    return;
  }
  const int64_t nqb = a.rows / kQmBlock;   // Q blocks of the workspace (Q centring)
  if (!a.seg_scales) {
    for (int c = d; c < a.nchunks; c += D) {
      if (!a.q_centre) qa = fmaxf(qa, a.amax[(int64_t)c * a.heads + h]);
      va = fmaxf(va, a.amax[((int64_t)a.nchunks + c) * a.heads + h]);
    }
  }
  if (a.q_centre) a.qmean[((int64_t)h * nqb + nqb - 1) * D + d] = 0.f;   // the guard rows' block
  float ka = 0.f;
  for (int s = 0; s < a.nseg; s++) {
    const SegInfo si = a.segs[s];
    const int nch = (si.len + kStatChunk - 1) / kStatChunk;
    float mu = 0.f, kas = 0.f;
    if (si.len > 0) {
      double sum = 0.0;
      float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll 8
      for (int c = si.chunk0; c < si.chunk0 + nch; c++) {   // loads issued ahead, sums in chunk order
        const KStat st = a.kstat[((int64_t)c * a.heads + h) * D + d];
        sum = sum + st.sum;
        mn = fminf(mn, st.mn);
        mx = fmaxf(mx, st.mx);
      }
      mu = (float)(sum / (double)si.len);
      kas = fmaxf(fabsf(mx - mu), fabsf(mn - mu));
    }
    a.mu[((int64_t)s * a.heads + h) * D + d] = mu;
    // Q centring: Q's amax over the segment is the maximum of its blocks'
    // centred amax partials (D/8 per block and head, from the statistics pass)
    float qcs = 0.f;
    if (a.q_centre) {
      constexpr int TPH = D / 8;
      const int64_t g0 = si.row0 / kQmBlock;
      const int n = (si.len + kQmBlock - 1) / kQmBlock * TPH;
      for (int e = d; e < n; e += D) qcs = fmaxf(qcs, a.qamax[((g0 + e / TPH) * a.heads + h) * TPH + e % TPH]);
      if (!a.seg_scales) qa = fmaxf(qa, qcs);
    }
    if (a.seg_scales) {
      // this segment's own amax of Q, K and V (its chunks' partials), so its
      // scales do not depend on the other segments
      float qs = a.q_centre ? qcs : 0.f, vs = 0.f;
      for (int c = si.chunk0 + d; c < si.chunk0 + nch; c += D) {
        if (!a.q_centre) qs = fmaxf(qs, a.amax[(int64_t)c * a.heads + h]);
        vs = fmaxf(vs, a.amax[((int64_t)a.nchunks + c) * a.heads + h]);
      }
      qs = block_max<D>(qs, red);
      vs = block_max<D>(vs, red);
      const float ks = block_max<D>(kas, red);
      if (d == 0) {
        const int64_t o = (int64_t)s * a.heads + h;      // scales [3][nseg][H]
        const int64_t n = (int64_t)a.nseg * a.heads;
        a.scales[o] = q_scale_of(qs, scale_of(ks), a.softmax_scale);
        a.scales[n + o] = scale_of(ks);
        a.scales[2 * n + o] = scale_of(vs);
      }
    } else {
      ka = fmaxf(ka, kas);
    }
  }
  if (!a.seg_scales) {
    qa = block_max<D>(qa, red);
    va = block_max<D>(va, red);
    ka = block_max<D>(ka, red);
    if (d == 0) {
      a.scales[h] = q_scale_of(qa, scale_of(ka), a.softmax_scale);
      a.scales[a.heads + h] = scale_of(ka);
      a.scales[2 * a.heads + h] = scale_of(va);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 2: pack.  grid = (ngroups * H, 1, 3), block = 256.  One block writes one
// 64-row group of one head of one tensor; rows past the segment's end (and the
// guard rows) are written as zero codes, so every workspace byte the attention
// kernel can read is defined and finite.  Blocks run head-fastest (the blocks
// in flight together read whole token rows of the [T][H][128] input) and in
// reverse (V, K, Q; last groups first), starting on rows the statistics pass
// read last, which the last-level cache may still hold: 0.685 -> 0.647 ms for
// the whole quantize at S=30272, H=56 (with 16 statistics loads in flight,
// 0.635 ms).
//
// Q, K codes: row-major [H][rows][128].  V codes: transposed [H][128][rows]
// with the keys of each 64-row group permuted so that the attention kernel's
// probability registers line up with the V operand: byte p = 32j + 16b + 4r + i
// of a group holds key 32b + 8r + 4j + i.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_pack(QuantizeArgs a) {
  constexpr int TPH = D / 8;        // threads per row, 8 channels each
  constexpr int RPP = 256 / TPH;    // rows per pass
  __shared__ uint8_t tile[kPackRows][D + 16];
  const int bx = gridDim.x - 1 - blockIdx.x;
  const int g = bx / a.heads;
  const int h = bx % a.heads;
  const int tensor = 2 - blockIdx.z;
  const int t = threadIdx.x;
  const int seg = a.group_seg[g];
  const int64_t R = (int64_t)g * kPackRows;  // first workspace row of the group
  SegInfo si{0, 0, 0, 0};
  if (seg >= 0) si = a.segs[seg];
  const int nset = a.seg_scales ? a.nseg : 1;       // scales [3][nset][H]
  const int sset = a.seg_scales && seg >= 0 ? seg : 0;
  const float s = a.scales[((int64_t)tensor * nset + sset) * a.heads + h];
  const int c0 = (t % TPH) * 8;
  const bool live = c0 < a.d_real;   // channels past head_dim read as zeros (codes 0)
  const uint16_t* base = a.x[tensor] + (int64_t)h * a.hs[tensor] + (live ? c0 : 0);
  const int64_t ts = a.ts[tensor];
  float mu[8];
  if (tensor == 1 && seg >= 0) {
    const float* m = a.mu + ((int64_t)seg * a.heads + h) * D + c0;
#pragma unroll
    for (int i = 0; i < 8; i++) mu[i] = m[i];
  } else if (tensor == 0 && a.q_centre && seg >= 0) {
    // Q centring: the mean of the group's 128-row block
    const float* m = a.qmean + ((int64_t)h * (a.rows / kQmBlock) + R / kQmBlock) * D + c0;
#pragma unroll
    for (int i = 0; i < 8; i++) mu[i] = m[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) mu[i] = 0.f;
  }

#pragma unroll
  for (int pass = 0; pass < kPackRows / RPP; pass++) {
    const int i = pass * RPP + t / TPH;              // row within the group
    const int rel = (int)(R - (seg >= 0 ? si.row0 : 0)) + i;  // segment-relative row
    uint2 code = make_uint2(0u, 0u);
    if (seg >= 0 && rel < si.len) {
      const uint4 v = load8(base + (int64_t)(si.start + rel) * ts, live);
      float f[8];
      unpack8(v, f);
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; j++) y[j] = (f[j] - mu[j]) / s;   // K: fl32(x - mu); Q: fl32(x - qm) or x; V: x
      code.x = cvt4(y[0], y[1], y[2], y[3]);
      code.y = cvt4(y[4], y[5], y[6], y[7]);
    }
    if (tensor < 2) {
      uint8_t* dst = a.codes[tensor] + ((int64_t)h * a.rows + R + i) * D + c0;
      *reinterpret_cast<uint2*>(dst) = code;
    } else {
      *reinterpret_cast<uint2*>(&tile[i][c0]) = code;
    }
  }
  if (tensor < 2) return;
  __syncthreads();
  // transposed, permuted write: thread t -> channel d = t/2, bytes p in [32*(t%2), +32)
  if (t >= 2 * D) return;
  const int d = t / 2;
  const int j = t % 2;
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; q++) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int pp = 4 * q + i;               // byte within this lane's 32: 16b + 4r + i
      const int b = pp / 16, r = (pp % 16) / 4;
      const int key = 32 * b + 8 * r + 4 * j + i;
      acc |= (uint32_t)tile[key][d] << (8 * i);
    }
    w[q] = acc;
  }
  uint8_t* dst = a.codes[2] + ((int64_t)h * D + d) * a.rows + R + 32 * j;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
}

// ---------------------------------------------------------------------------
// Pass 3 (E4M3 plans with Q centring): the mean-term table.
//
// FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page, description of
// the Q operand: Q rows are centred by their 128-row block mean and the term
// qm . k is added back to the scores.  With E4M3 operands the error of a
// rounded mean would be as large as the centring saves, so the term is kept
// near-exact: for every (block, key) pair of a segment, t = f * (qm . khat)
// with khat the E4M3 codes of the centred K row and f = softmax_scale * s_k *
// log2(e) (times 8 in the log-linear frame), the frame the attention's score
// products deliver, stored as a bf16 pair (hi = bf16(t), lo = bf16(t - hi)).
//
// The dot products run on the scaled FP8 matrix core: A = qm (32 blocks x 64
// channels), split into three E4M3 parts with power-of-two scales 2^e,
// 2^(e-4), 2^(e-8) per block and 64 channels (each part takes the rounding error of the
// previous one, so the parts carry about 12 significant bits of every mean),
// B = khat^T (64 channels x 32 keys), all six products of the 128 channels
// chained into one FP32 accumulator.  grid = units, block = 256: unit
// {s, bg, k0, h} covers blocks 32 bg .. +32 of segment s and keys k0 .. +1024
// of head h (s = -1: an empty unit);
// each wave splits the means once and then takes 32 keys a step.
// ---------------------------------------------------------------------------
typedef int v8i_q __attribute__((ext_vector_type(8)));
typedef float v16f_q __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
__global__ __launch_bounds__(256) void k_qmterm(QuantizeArgs a) {
  constexpr int NH = D / 64;   // 64-channel halves
  const int4 u = a.qmt_units[blockIdx.x];
  if (u.x < 0) return;   // padding of the work list
  const int h = u.w;
  const SegInfo si = a.segs[u.x];
  const int lr = (si.len + kRowPad - 1) / kRowPad * kRowPad;   // the segment's padded rows
  const int nblk = lr / kQmBlock;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lq = lane & 31, lg = lane >> 5;
  const int blk = kQmUnitBlocks * u.y + lq;   // this lane's A row (zero past the segment's blocks)
  const bool blk_live = blk < nblk;
  const int64_t nqb = a.rows / kQmBlock;
  const float* qm = a.qmean + ((int64_t)h * nqb + si.row0 / kQmBlock + (blk_live ? blk : 0)) * D;

  // A operands, once per wave: the block means of this lane's row over
  // channels 64 half + 32 lg .. +32, in three E4M3 parts
  v8i_q ap[NH][3];
  int sp[NH][3];
#pragma unroll
  for (int half = 0; half < NH; half++) {
    const int ch0 = 64 * half + 32 * lg;
    float r[32];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float4 x = blk_live ? *reinterpret_cast<const float4*>(qm + ch0 + 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
      r[4 * j + 0] = x.x;
      r[4 * j + 1] = x.y;
      r[4 * j + 2] = x.z;
      r[4 * j + 3] = x.w;
    }
#pragma unroll
    for (int j = 0; j < 32; j++) m = fmaxf(m, fabsf(r[j]));
    // one scale per row and 64-channel half: lanes l and l + 32 hold the same
    // row, and a per-32-element scale of an FP8 operand is not guaranteed to
    // cover exactly the 32 bytes one lane holds
    m = fmaxf(m, __shfl_xor(m, 32));
    // smallest e with m <= 448 * 2^e, kept where every part's scale is a normal E8M0 value
    int e = 0;
    if (m > 0.f) {
      int ex;
      const float fr = frexpf(m / 448.0f, &ex);
      e = fr == 0.5f ? ex - 1 : ex;
      e = max(-119, min(e, 126));
    }
#pragma unroll
    for (int part = 0; part < 3; part++) {
      const int ep = e - 4 * part;
      const float inv = __uint_as_float((uint32_t)(127 - ep) << 23);   // 2^-ep
      const float sc = __uint_as_float((uint32_t)(127 + ep) << 23);    // 2^ep
#pragma unroll
      for (int w = 0; w < 8; w++) {
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * w + 0] * inv, r[4 * w + 1] * inv, 0, false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * w + 2] * inv, r[4 * w + 3] * inv, c, true);
        ap[half][part][w] = c;
        r[4 * w + 0] -= __builtin_amdgcn_cvt_f32_fp8(c, 0) * sc;   // exact: what the next part takes
        r[4 * w + 1] -= __builtin_amdgcn_cvt_f32_fp8(c, 1) * sc;
        r[4 * w + 2] -= __builtin_amdgcn_cvt_f32_fp8(c, 2) * sc;
        r[4 * w + 3] -= __builtin_amdgcn_cvt_f32_fp8(c, 3) * sc;
      }
      sp[half][part] = ep + 127;
    }
  }
  const int nset = a.seg_scales ? a.nseg : 1;
  const int sset = a.seg_scales ? u.x : 0;
  const float s_k = a.scales[((int64_t)1 * nset + sset) * a.heads + h];
  const float f = a.softmax_scale * s_k * 1.4426950408889634f * (a.exact_probs ? 1.0f : 8.0f);
  uint32_t* seg_tab = a.mt + (int64_t)h * a.mt_per_head + a.mt_seg[u.x];
  const int kend = min(u.z + kQmUnitKeys, lr);
  // 32 keys per wave and step: B = khat^T, lane l key key0 + l%32, channels
  // 64 half + 32 lg .. +32; the next step's K bytes are loaded ahead
  int key0 = u.z + 32 * wave;
  if (key0 >= kend) return;   // wave-uniform
  auto load_b = [&](int k0, uint4 (&b)[2 * NH]) __attribute__((always_inline)) {
    const uint8_t* krow = a.codes[1] + ((int64_t)h * a.rows + si.row0 + k0 + lq) * D + 32 * lg;
#pragma unroll
    for (int half = 0; half < NH; half++) {
      b[2 * half] = *reinterpret_cast<const uint4*>(krow + 64 * half);
      b[2 * half + 1] = *reinterpret_cast<const uint4*>(krow + 64 * half + 16);
    }
  };
  uint4 bn[2 * NH];
  load_b(key0, bn);
  for (; key0 < kend; key0 += 128) {
    uint4 b[2 * NH];
#pragma unroll
    for (int j = 0; j < 2 * NH; j++) b[j] = bn[j];
    if (key0 + 128 < kend) load_b(key0 + 128, bn);
    v16f_q acc = {};
#pragma unroll
    for (int half = 0; half < NH; half++) {
      const uint4 b0 = b[2 * half], b1 = b[2 * half + 1];
      const v8i_q bk = v8i_q{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
      for (int part = 0; part < 3; part++)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ap[half][part], bk, acc, 0, 0, 0, sp[half][part], 0,
                                                             127);
    }
    // lane l holds key key0 + l%32 and blocks 8*(r/4) + 4*lg + r%4 of the unit;
    // tile-major table: entry ((key / 64) * nblk + b) * 64 + key % 64 of the segment
    uint32_t* dst = seg_tab + (int64_t)(key0 / kBN) * nblk * kBN + key0 % kBN + lq;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int b = kQmUnitBlocks * u.y + 8 * (i >> 2) + 4 * lg + (i & 3);
      if (b < nblk) {
        const float t = f * acc[i];
        const uint32_t hi = bf16_rne_bits(t);
        const uint32_t lo = bf16_rne_bits(t - __uint_as_float(hi << 16));
        dst[b * kBN] = hi | (lo << 16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Block-scaled FP4 pack (plans made with FP8ATTN_PLAN_MXFP4).
//
// FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page, description of
// the operands: E2M1 codes with one scale per block of elements along the
// contraction axis, K centred by its segment's per-channel mean, Q centred by
// the mean of its 128-row block (the mean term is added back in the attention
// kernel).  On gfx950's scaled matrix products the scale is an E8M0 power of
// two per 32 elements: 2^e with e the smallest integer for which
// amax <= 6 * 2^e, and codes E2M1(x * 2^-e) (round to nearest even).  The
// score factor c = softmax_scale * log2(e) is folded into Q (and into the
// block mean) before quantization, so scores come out in log2 units.
// ---------------------------------------------------------------------------

// Smallest e with amax <= 6 * 2^e, clamped to [-127, 126]: amax = f * 2^E with
// f in [1, 2) needs e = E - 2 when f <= 1.5 and E - 1 above; zero and
// subnormal amax (below 2^-126) clamp to -127.
__device__ __forceinline__ int mx_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ef = (int)((u >> 23) & 255u);
  if (ef == 0) return -127;
  const int e = ef - 129 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^-e as a float (e in [-127, 126]: 127 - e in [1, 254], a normal float).
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// E2M1 codes of 8 values (already divided by the block scale; the products
// by a power of two are exact), two per byte, low nibble first.
__device__ __forceinline__ uint32_t cvt8_fp4(const float y[8]) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], 1.0f, 3);
}

// Byte position of channel block j (0..3) in a row's 4 scale bytes: blocks
// 0, 2, 1, 3, so that lanes reading channels 32*(lane/32) + 64*k find their
// scales for k = 0, 1 in one 16-bit word.
__device__ __forceinline__ int mx_scale_pos(int j) { return ((j & 1) << 1) | (j >> 1); }

// One row of 128 channels, 16 threads x 8 channels (threads 4j..4j+3 of the 16
// hold block j): codes and the block exponents of y.
__device__ __forceinline__ void mx_row(const float y[8], uint8_t* code_row, uint8_t* scale_row, int tq, bool live) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(y[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  const int e = mx_exp(m);
  const float inv = mx_inv_scale(e);
  float z[8];
#pragma unroll
  for (int i = 0; i < 8; i++) z[i] = y[i] * inv;
  const uint32_t code = live ? cvt8_fp4(z) : 0u;
  *reinterpret_cast<uint32_t*>(code_row + 4 * tq) = code;
  if ((tq & 3) == 0) scale_row[mx_scale_pos(tq >> 2)] = live ? (uint8_t)(e + 127) : 0;
}

// grid = (ngroups * H, 1, 3), block = 256, heads fastest and in reverse
// order as for the E4M3 pack (0.619 -> 0.531 ms for the whole FP4 quantize
// at S=30272, H=56; 0.829 -> 0.647 ms with Q centring).  tensor 0 (Q): even
// groups take a 128-row mean block (two groups), odd groups return; tensor 1
// (K) and 2 (V): one 64-row group.  Rows past a segment's end and guard rows get zero codes
// and zero scale bytes.
__global__ __launch_bounds__(256) void k_pack_mx(QuantizeArgs a) {
  __shared__ float tile[kPackRows][kHeadDim + 1];
  __shared__ float qm_s[kHeadDim];
  const int bx = gridDim.x - 1 - blockIdx.x;
  const int g = bx / a.heads;
  const int h = bx % a.heads;
  const int tensor = 2 - blockIdx.z;
  const int t = threadIdx.x;
  if (tensor == 0 && (g & 1)) return;
  const int seg = a.group_seg[g];
  const int64_t R = (int64_t)g * kPackRows;
  SegInfo si{0, 0, 0, 0};
  if (seg >= 0) si = a.segs[seg];
  const int rel0 = seg >= 0 ? (int)(R - si.row0) : 0;   // segment-relative first row
  const int nreal = seg >= 0 ? max(0, min(tensor == 0 ? kMxQBlock : kPackRows, si.len - rel0)) : 0;
  const int tq = t % 16;
  const int c0 = tq * 8;
  const uint16_t* base = a.x[tensor] + (int64_t)h * a.hs[tensor] + c0;
  const int64_t ts = a.ts[tensor];
  const float cf = a.softmax_scale * 1.4426950408889634f;   // score factor c

  if (tensor == 0) {
    // block mean: thread d sums the block's rows in order (float64)
    if (t < kHeadDim) {
      float qm = 0.f;
      if (a.q_centre && nreal > 0) {
        const uint16_t* col = a.x[0] + (int64_t)h * a.hs[0] + t + (int64_t)(si.start + rel0) * ts;
        double sum = 0.0;
#pragma unroll 8
        for (int i = 0; i < nreal; i++) sum = sum + (double)bf16_to_f32(col[(int64_t)i * ts]);
        qm = (float)(sum / (double)nreal);
      }
      qm_s[t] = qm;
      // the block-mean operand fl32(qm * c), quantized like a Q row: lanes of
      // one wave hold channels 64*(t/64) .. +64, two blocks of 32
      const float y = qm * cf;
      float m = fabsf(y);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 32));
      const int e = mx_exp(m);
      const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y * mx_inv_scale(e), 0.f, 1.0f, 0) & 15u;
      const uint32_t hi = __shfl_down(c, 1, 64);
      const int64_t blk = (int64_t)h * (a.rows / kMxQBlock) + R / kMxQBlock;
      if ((t & 1) == 0) a.qm_codes[blk * kMxRow + t / 2] = (uint8_t)(c | (hi << 4));
      if ((t & 31) == 0) a.qm_scales[blk * 4 + mx_scale_pos(t >> 5)] = nreal > 0 ? (uint8_t)(e + 127) : 0;
    }
    __syncthreads();
    float qm[8];
#pragma unroll
    for (int i = 0; i < 8; i++) qm[i] = qm_s[c0 + i];
#pragma unroll
    for (int pass = 0; pass < kMxQBlock / 16; pass++) {
      const int i = pass * 16 + t / 16;
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const bool live = i < nreal;
      if (live) {
        const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)(si.start + rel0 + i) * ts);
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int j = 0; j < 8; j++) y[j] = (f[j] - qm[j]) * cf;   // fl32(fl32(q - qm) * c)
      }
      const int64_t row = (int64_t)h * a.rows + R + i;
      mx_row(y, a.codes[0] + row * kMxRow, a.bscale[0] + row * 4, tq, live);
    }
    return;
  }

  if (tensor == 1) {
    float mu[8];
#pragma unroll
    for (int i = 0; i < 8; i++) mu[i] = seg >= 0 ? a.mu[((int64_t)seg * a.heads + h) * kHeadDim + c0 + i] : 0.f;
#pragma unroll
    for (int pass = 0; pass < kPackRows / 16; pass++) {
      const int i = pass * 16 + t / 16;
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const bool live = i < nreal;
      if (live) {
        const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)(si.start + rel0 + i) * ts);
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int j = 0; j < 8; j++) y[j] = f[j] - mu[j];            // fl32(k - mu)
      }
      const int64_t row = (int64_t)h * a.rows + R + i;
      mx_row(y, a.codes[1] + row * kMxRow, a.bscale[1] + row * 4, tq, live);
    }
    return;
  }

  // V: the group's 64 keys x 128 channels through LDS, then per (channel,
  // 32-key block) scales and transposed codes: thread t -> channel d = t/2,
  // keys 32*(t%2) .. +32 (padding keys are zeros, which leave amax unchanged).
#pragma unroll
  for (int pass = 0; pass < kPackRows / 16; pass++) {
    const int i = pass * 16 + t / 16;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (i < nreal) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)(si.start + rel0 + i) * ts);
      unpack8(v, f);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) tile[i][c0 + j] = f[j];
  }
  __syncthreads();
  const int d = t / 2;
  const int kh = t % 2;
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 32; j++) m = fmaxf(m, fabsf(tile[32 * kh + j][d]));
  const bool live = 32 * kh < nreal;
  const int e = mx_exp(m);
  const float inv = mx_inv_scale(e);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    float z[8];
#pragma unroll
    for (int j = 0; j < 8; j++) z[j] = tile[32 * kh + 8 * q + j][d] * inv;
    w[q] = live ? cvt8_fp4(z) : 0u;
  }
  const int64_t tile_idx = (int64_t)h * (a.rows / kBN) + g;    // a 64-row group is one key tile
  uint8_t* dst = a.codes[2] + tile_idx * kMxTile + d * (kBN / 2) + 16 * kh;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  a.bscale[2][tile_idx * kMxTileScales + (32 * kh + d % 32) * 4 + d / 32] = live ? (uint8_t)(e + 127) : 0;
}

}  // namespace

template <int D>
hipError_t launch_quantize_d(const QuantizeArgs& a, hipStream_t stream) {
  constexpr int TPH = D / 8;
  const int ngrp = (a.heads + 256 / TPH - 1) / (256 / TPH);   // head groups of at most 256 / TPH heads
  const int HPB = (a.heads + ngrp - 1) / ngrp;                // heads per stats block, spread evenly
  if (a.nchunks > 0) {
    if (a.q_centre && !a.mx)
      hipLaunchKernelGGL((k_stats<D, true>), dim3(a.nchunks, (a.heads + HPB - 1) / HPB, 3), dim3(HPB * TPH), 0, stream, a);
    else
      hipLaunchKernelGGL((k_stats<D, false>), dim3(a.nchunks, (a.heads + HPB - 1) / HPB, a.mx ? 1 : 3), dim3(HPB * TPH), 0,
                         stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_finalize<D>, dim3(a.heads), dim3(D), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.mx)
    hipLaunchKernelGGL(k_pack_mx, dim3(a.ngroups * a.heads, 1, 3), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_pack<D>, dim3(a.ngroups * a.heads, 1, 3), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.mx && a.q_centre && a.nqmt_units > 0) {
    hipLaunchKernelGGL(k_qmterm<D>, dim3(a.nqmt_units), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return launch_quantize_d<64>(a, stream);
  return launch_quantize_d<kHeadDim>(a, stream);
}

}  // namespace fp8attn
