// C ABI of libfp8attn.so (declared in include/fp8attn.h): argument validation,
// the segment planner / scheduler, workspace layout and launches.
//
// The planner follows the varlen contract of the FlashInfer
// "minimax_h3_sm120_varlen_attention_nvfp4" page: any token count and any
// segment lengths, including empty segments and segments shorter than one
// tile, from a host copy of cu_seqlens (parameters "cu_seqlens" and
// "cu_seqlens_host"; the plan is built once per segment table and head count).
// As in the plan rework of sglang PR "[diffusion] attention: add fp8_fa_sm120
// FP8 backend for SM120 GPUs" (review thread), a plan holds only small host
// and device tables and never retains input or output buffers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/fp8attn.h"
#include "internal.h"

using namespace fp8attn;

struct fp8attn_plan_s {
  int64_t tokens = 0;
  int32_t heads = 0;
  int32_t nseg = 0;
  int32_t seg_scales = 0;         // FP8ATTN_PLAN_SEGMENT_SCALES
  int32_t nscale = 1;             // scale sets: nseg with segment scales, else 1
  int32_t mx = 0;                 // FP8ATTN_PLAN_MXFP4
  int32_t q_centre = 0;           // FP8ATTN_PLAN_Q_CENTRE
  int32_t causal = 0;             // FP8ATTN_PLAN_CAUSAL
  int32_t head_dim = kHeadDim;    // channels of q, k, v and out (FP8ATTN_PLAN_HEAD_DIM_64, FP8ATTN_PLAN_HEAD_DIM)
  int32_t dk = kHeadDim;          // kernel width: 64 for head_dim <= 64, else 128 (missing channels are zeros)
  int32_t exact_probs = 0;        // FP8ATTN_PLAN_EXACT_PROBS
  int32_t bm = kBM;               // queries per work item (kMxBM for FP4 plans; see choose_query_tile)
  int32_t wg_per_cu = 1;          // attention workgroups resident per CU
  float scale = 0.f;
  int device = -1;
  std::vector<int32_t> cu;
  std::vector<SegInfo> segs;
  std::vector<Chunk> chunks;
  std::vector<int32_t> group_seg;
  std::vector<int4> items;        // in launch order (XCD-remapped)
  std::vector<int4> combine;      // one per split work item
  std::vector<int64_t> mt_seg;    // E4M3 Q centring: first mean-term entry of each segment (per head)
  std::vector<int4> qmt_units;    // E4M3 Q centring: work units of the mean-term kernel
  int64_t mt_per_head = 0;
  int64_t real_items = 0;
  int64_t npieces = 0;
  WorkspaceLayout ws{};
  // device copies, one allocation
  void* dev = nullptr;
  SegInfo* d_segs = nullptr;
  Chunk* d_chunks = nullptr;
  int32_t* d_group_seg = nullptr;
  int4* d_items = nullptr;
  int4* d_combine = nullptr;
  int32_t* d_rowmap = nullptr;
  int64_t* d_mt_seg = nullptr;
  int4* d_qmt_units = nullptr;
};

namespace {

#ifndef FP8ATTN_CAUSAL_ROUNDS
#define FP8ATTN_CAUSAL_ROUNDS 4
#endif
constexpr int kCausalRounds = FP8ATTN_CAUSAL_ROUNDS;   // see build_items

thread_local std::string g_last_error;

fp8attn_status fail(fp8attn_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// FP4 plans: codes of half the size, block scales, block-mean operand.
WorkspaceLayout make_layout_mx(int64_t rows, int heads, int nseg, int nchunks, int64_t npieces) {
  WorkspaceLayout w{};
  w.rows = rows;
  w.npieces = npieces;
  const size_t codes = (size_t)heads * rows * kMxRow;
  const size_t scales = (size_t)heads * rows * 4;
  const size_t qblocks = (size_t)heads * (rows / kMxQBlock);
  size_t off = 0;
  w.q_off = off; off = align_up(off + codes, 256);
  w.k_off = off; off = align_up(off + codes, 256);
  w.v_off = off; off = align_up(off + codes, 256);
  w.qs_off = off; off = align_up(off + scales, 256);
  w.ks_off = off; off = align_up(off + scales, 256);
  w.vs_off = off; off = align_up(off + scales, 256);   // rows/64 tiles x 256 bytes
  w.qm_off = off; off = align_up(off + qblocks * kMxRow, 256);
  w.qms_off = off; off = align_up(off + qblocks * 4, 256);
  w.mu_off = off; off = align_up(off + sizeof(float) * (size_t)nseg * heads * kHeadDim, 256);
  w.part_o_off = off; off = align_up(off + sizeof(float) * (size_t)npieces * kPartRows * kHeadDim, 256);
  w.part_w_off = off; off = align_up(off + sizeof(float) * (size_t)npieces * kPartRows, 256);
  w.part_lse_off = off; off = align_up(off + sizeof(float) * (size_t)npieces * kPartRows, 256);
  w.stats_off = off;
  w.kstat_off = off; off = align_up(off + sizeof(KStat) * (size_t)nchunks * heads * kHeadDim, 256);
  w.total = off;
  return w;
}

WorkspaceLayout make_layout(int64_t rows, int heads, int nseg, int nscale, int nchunks, int64_t npieces, int D,
                            int64_t mt_per_head) {
  WorkspaceLayout w{};
  w.rows = rows;
  w.npieces = npieces;
  w.mt_per_head = mt_per_head;
  const size_t codes = (size_t)heads * rows * D;
  const size_t qblocks = (size_t)(rows / kQmBlock);
  size_t off = 0;
  w.q_off = off; off = align_up(off + codes, 256);
  w.k_off = off; off = align_up(off + codes, 256);
  w.v_off = off; off = align_up(off + codes, 256);
  w.scale_off = off; off = align_up(off + sizeof(float) * 3 * (size_t)nscale * heads, 256);
  w.mu_off = off; off = align_up(off + sizeof(float) * (size_t)nseg * heads * D, 256);
  if (mt_per_head > 0) {   // Q centring: block means and the mean-term table
    w.qmean_off = off; off = align_up(off + sizeof(float) * (size_t)heads * qblocks * D, 256);
    w.mt_off = off; off = align_up(off + sizeof(uint32_t) * (size_t)heads * (size_t)mt_per_head, 256);
  }
  w.part_o_off = off; off = align_up(off + sizeof(float) * (size_t)npieces * kPartRows * D, 256);
  w.part_w_off = off; off = align_up(off + sizeof(float) * (size_t)npieces * kPartRows, 256);
  w.part_lse_off = off; off = align_up(off + sizeof(float) * (size_t)npieces * kPartRows, 256);
  // the statistics of fp8attn_quantize come last: fp8attn_quantize_noalloc and
  // fp8attn_forward do not need them
  w.stats_off = off;
  w.kstat_off = off; off = align_up(off + sizeof(KStat) * (size_t)nchunks * heads * D, 256);
  w.amax_off = off; off = align_up(off + sizeof(float) * 2 * (size_t)nchunks * heads, 256);
  if (mt_per_head > 0) {
    w.qamax_off = off; off = align_up(off + sizeof(float) * qblocks * heads * (D / 8), 256);
  }
  w.total = off;
  return w;
}

// Work list: head-major; inside a head, longer segments first, then query
// tiles in order.  The list is split into kNumXcd contiguous parts of equal
// count and interleaved so that workgroup w, which the hardware sends to XCD
// w % 8, takes item w / 8 of part w % 8: each XCD walks its own contiguous run,
// so the concurrent workgroups of an XCD mostly read the same head's K/V
// through that XCD's L2.
//
// Each part is ordered longest item first (stable, so head order is kept).
// An XCD runs p->wg_per_cu workgroups on each of its cus = CUs / kNumXcd
// compute units (one 256-query E4M3 workgroup, or two 128-query FP4 ones).  When the part's item count leaves R <= cus / 2 items for a last
// round, those run nearly alone; they are split along the keys into n pieces
// (n <= kMaxSplit, n * R <= cus, at least kMinPieceTiles key tiles a piece),
// which go last.  A piece writes an unnormalized-frame partial (output, log2 weight,
// LSE) and one combine pass merges the pieces of each split item, the
// log-sum-exp combination over key ranges that the pages use to merge partial
// attention (sglang PR "[DSA] Enable tilelang fp8_e4m3 KV cache ...", note that
// the FP8 path must return the LSE for cross-rank reduction).
void build_items(fp8attn_plan_s* p, int cus, bool allow_split) {
  const int bm = p->bm;
  const int slots = p->wg_per_cu * cus;
  std::vector<int> order(p->nseg);
  for (int s = 0; s < p->nseg; s++) order[s] = s;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return p->segs[x].len > p->segs[y].len; });
  // key tiles an item attends to (causal: up to its last query)
  auto tiles = [&](const int4& it) {
    const int L = p->segs[it.x].len;
    return ((p->causal ? std::min(L, it.y + bm) : L) + kBN - 1) / kBN;
  };
  std::vector<int4> list;
  for (int h = 0; h < p->heads; h++)
    for (int s : order) {
      const int L = p->segs[s].len;
      const int n = (L + bm - 1) / bm;
      // causal items get shorter with q0: longest (last query tile) first
      for (int i = 0; i < n; i++) list.push_back(int4{s, bm * (p->causal ? n - 1 - i : i), h, 0});
    }
  if (p->causal) {
    // Causal items differ in length.  The head-major list is cut into kNumXcd
    // contiguous parts of equal work (key tiles); each part runs in windows of
    // consecutive heads holding at least kCausalRounds rounds of its longest
    // item, longest item first inside a window.  A window keeps an XCD's
    // concurrent workgroups on a few heads, which walk the same K/V tiles
    // together through its L2; the longest-first order inside it bounds the
    // idle tail when items are long against the work per compute unit.
    int64_t total = 0;
    int maxt = 1;
    for (const int4& it : list) {
      total += tiles(it);
      maxt = std::max(maxt, tiles(it));
    }
    std::vector<std::vector<int4>> parts(kNumXcd);
    int64_t acc = 0;
    for (const int4& it : list) {
      const int x = (int)std::min<int64_t>(kNumXcd - 1, acc * kNumXcd / std::max<int64_t>(1, total));
      parts[x].push_back(it);
      acc += tiles(it);
    }
    const int64_t window = (int64_t)kCausalRounds * p->wg_per_cu * cus * maxt;
    for (auto& part : parts) {
      size_t b = 0;
      while (b < part.size()) {
        int64_t w = 0;
        size_t e = b;
        // whole heads: extend to the end of the head at which the window is full
        while (e < part.size() && (w < window || part[e].z == part[e - 1].z)) w += tiles(part[e++]);
        std::stable_sort(part.begin() + b, part.begin() + e,
                         [&](const int4& u, const int4& v) { return tiles(u) > tiles(v); });
        b = e;
      }
    }
    p->combine.clear();
    p->npieces = 0;
    size_t longest = 0;
    p->real_items = 0;
    for (const auto& part : parts) {
      longest = std::max(longest, part.size());
      p->real_items += (int64_t)part.size();
    }
    p->items.assign(longest * kNumXcd, int4{-1, 0, 0, 0});
    for (int x = 0; x < kNumXcd; x++)
      for (size_t j = 0; j < parts[x].size(); j++) p->items[j * kNumXcd + x] = parts[x][j];
    return;
  }
  const size_t per = (list.size() + kNumXcd - 1) / kNumXcd;
  std::vector<std::vector<int4>> parts(kNumXcd);
  int64_t slot = 0;
  p->combine.clear();
  for (int x = 0; x < kNumXcd; x++) {
    std::vector<int4>& part = parts[x];
    const size_t b = std::min(list.size(), x * per), e = std::min(list.size(), (x + 1) * per);
    part.assign(list.begin() + b, list.begin() + e);
    std::stable_sort(part.begin(), part.end(), [&](const int4& u, const int4& v) { return tiles(u) > tiles(v); });
    const size_t R = part.size() % (size_t)slots;
    if (!allow_split || R == 0 || 2 * R > (size_t)cus) continue;
    std::vector<int4> tail(part.end() - R, part.end()), pieces;
    part.resize(part.size() - R);
    for (const int4& it : tail) {
      const int n = std::min({kMaxSplit, cus / (int)R, tiles(it) / kMinPieceTiles});
      if (n < 2) {
        part.push_back(it);
        continue;
      }
      const int w = (int)(slot << 8) | (n << 4);
      p->combine.push_back(int4{it.x, it.y, it.z, w});
      for (int i = 0; i < n; i++) pieces.push_back(int4{it.x, it.y, it.z, w | i});
      slot += n;
    }
    part.insert(part.end(), pieces.begin(), pieces.end());
  }
  p->npieces = slot;
  size_t longest = 0;
  p->real_items = 0;
  for (const auto& part : parts) {
    longest = std::max(longest, part.size());
    p->real_items += (int64_t)part.size();
  }
  p->items.assign(longest * kNumXcd, int4{-1, 0, 0, 0});
  for (int x = 0; x < kNumXcd; x++)
    for (size_t j = 0; j < parts[x].size(); j++) p->items[j * kNumXcd + x] = parts[x][j];
}

// Query tile of a non-causal 128-channel E4M3 plan.  256-query items (one
// 8-wave workgroup per CU) halve the L2-to-LDS traffic per flop and run faster
// when every CU has a lot of work: S=30272 with 56 heads is 3% slower with
// 128-query items, and the 7-head shard of it (1539 key-tile iterations of
// 256-query items per CU) 1.5% slower.  With little work per CU, 128-query
// items (two 4-wave workgroups per CU, so a SIMD runs the other workgroup's
// wave while one waits at its barrier) finish sooner: S=4096 with 56 heads
// (224 iterations per CU) is 4% faster.  Same-box A/B, 7 x 10 launches each.
constexpr int64_t kSmallWorkPerCu = 768;   // key-tile iterations of 256-query items per CU

void choose_query_tile(fp8attn_plan_s* p, int cus) {
  if (p->mx || p->causal || p->dk != kHeadDim) return;
  int64_t work = 0;
  for (const SegInfo& s : p->segs) work += (int64_t)((s.len + kBM - 1) / kBM) * ((s.len + kBN - 1) / kBN);
  work *= p->heads;
  if (work < kSmallWorkPerCu * cus) {
    p->bm = 128;
    p->wg_per_cu = 2;
  }
}

bool strides_ok(const int64_t s[2]) {
  return s != nullptr && s[0] > 0 && s[1] > 0 && s[0] % 8 == 0 && s[1] % 8 == 0;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

extern "C" {

fp8attn_status fp8attn_plan(fp8attn_plan_t* plan_out, int64_t tokens, int32_t heads,
                            const int32_t* cu, int32_t num_segments, float softmax_scale,
                            int32_t device) {
  return fp8attn_plan_ex(plan_out, tokens, heads, cu, num_segments, softmax_scale, device, 0u);
}

fp8attn_status fp8attn_plan_ex(fp8attn_plan_t* plan_out, int64_t tokens, int32_t heads,
                               const int32_t* cu, int32_t num_segments, float softmax_scale,
                               int32_t device, uint32_t flags) {
  if (plan_out == nullptr) return fail(FP8ATTN_EINVAL, "plan_out is NULL");
  *plan_out = nullptr;
  if ((flags & ~(FP8ATTN_PLAN_SEGMENT_SCALES | FP8ATTN_PLAN_MXFP4 | FP8ATTN_PLAN_Q_CENTRE | FP8ATTN_PLAN_CAUSAL |
                 FP8ATTN_PLAN_HEAD_DIM_64 | FP8ATTN_PLAN_EXACT_PROBS | FP8ATTN_PLAN_HEAD_DIM(248))) != 0)
    return fail(FP8ATTN_EINVAL, "unknown plan flags");
  int32_t head_dim = (int32_t)((flags >> 8) & 31u) * 8;
  if (flags & FP8ATTN_PLAN_HEAD_DIM_64) {
    if (head_dim != 0 && head_dim != 64)
      return fail(FP8ATTN_EINVAL, "FP8ATTN_PLAN_HEAD_DIM_64 with another FP8ATTN_PLAN_HEAD_DIM");
    head_dim = 64;
  }
  if (head_dim == 0) head_dim = kHeadDim;
  if (head_dim > kHeadDim) return fail(FP8ATTN_EINVAL, "head_dim must be a multiple of 8 from 8 to 128");
  if (head_dim != kHeadDim && (flags & FP8ATTN_PLAN_MXFP4))
    return fail(FP8ATTN_EINVAL, "FP8ATTN_PLAN_MXFP4 plans take head_dim 128 only");
  if ((flags & FP8ATTN_PLAN_EXACT_PROBS) && (flags & FP8ATTN_PLAN_MXFP4))
    return fail(FP8ATTN_EINVAL, "FP8ATTN_PLAN_EXACT_PROBS applies to E4M3 plans only");
  if ((flags & FP8ATTN_PLAN_MXFP4) && (flags & FP8ATTN_PLAN_SEGMENT_SCALES))
    return fail(FP8ATTN_EINVAL, "FP8ATTN_PLAN_MXFP4 does not take FP8ATTN_PLAN_SEGMENT_SCALES");
  if (cu == nullptr) return fail(FP8ATTN_EINVAL, "cu_seqlens_host is NULL");
  if (num_segments < 1) return fail(FP8ATTN_EINVAL, "num_segments must be >= 1");
  if (heads < 1) return fail(FP8ATTN_EINVAL, "heads must be >= 1");
  if (heads > 65535) return fail(FP8ATTN_EUNSUPPORTED, "heads must be <= 65535 (grid dimension)");
  if (tokens < 0) return fail(FP8ATTN_EINVAL, "tokens must be >= 0");
  if (tokens > (int64_t)INT32_MAX / 2) return fail(FP8ATTN_EUNSUPPORTED, "tokens too large (int32 indexing)");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(FP8ATTN_EINVAL, "softmax_scale must be finite and > 0");
  if (cu[0] != 0) return fail(FP8ATTN_EINVAL, "cu_seqlens[0] must be 0");
  for (int s = 0; s < num_segments; s++)
    if (cu[s + 1] < cu[s]) return fail(FP8ATTN_EINVAL, "cu_seqlens must be non-decreasing");
  if ((int64_t)cu[num_segments] != tokens)
    return fail(FP8ATTN_EINVAL, "cu_seqlens[num_segments] must equal tokens");

  fp8attn_plan_s* p = new (std::nothrow) fp8attn_plan_s();
  if (p == nullptr) return fail(FP8ATTN_ENOMEM, "host allocation failed");
  p->tokens = tokens;
  p->heads = heads;
  p->nseg = num_segments;
  p->scale = softmax_scale;
  p->device = device;
  p->seg_scales = (flags & FP8ATTN_PLAN_SEGMENT_SCALES) ? 1 : 0;
  p->nscale = p->seg_scales ? num_segments : 1;
  p->mx = (flags & FP8ATTN_PLAN_MXFP4) ? 1 : 0;
  p->q_centre = (flags & FP8ATTN_PLAN_Q_CENTRE) ? 1 : 0;
  p->causal = (flags & FP8ATTN_PLAN_CAUSAL) ? 1 : 0;
  p->head_dim = head_dim;
  p->dk = head_dim <= 64 ? 64 : kHeadDim;
  p->exact_probs = (flags & FP8ATTN_PLAN_EXACT_PROBS) ? 1 : 0;
  if (p->mx) {
    p->bm = kMxBM;
    p->wg_per_cu = kMxWgPerCu;
  }
  p->cu.assign(cu, cu + num_segments + 1);
  int64_t row = 0;
  int32_t chunk = 0;
  for (int s = 0; s < num_segments; s++) {
    const int32_t L = cu[s + 1] - cu[s];
    p->segs.push_back(SegInfo{cu[s], L, (int32_t)row, chunk});
    for (int32_t t = 0; t < L; t += kStatChunk)
      p->chunks.push_back(Chunk{s, cu[s] + t, std::min(kStatChunk, L - t), 0});
    chunk += (L + kStatChunk - 1) / kStatChunk;
    const int64_t padded = (int64_t)(L + kRowPad - 1) / kRowPad * kRowPad;
    for (int64_t g = 0; g < padded / kPackRows; g++) p->group_seg.push_back(s);
    row += padded;
  }
  for (int g = 0; g < kGuardRows / kPackRows; g++) p->group_seg.push_back(-1);
  row += kGuardRows;
  if (p->q_centre && !p->mx) {
    // mean-term table: per head, per segment, (padded rows / 128) blocks x padded rows
    p->mt_seg.resize(num_segments);
    // mean-term work units: one key chunk of one segment and head is walked by
    // all its block groups; those units go to one XCD (workgroups reach the
    // XCDs in turn, so list position p runs on XCD p % 8), where the chunk's
    // K codes are read from HBM once and then hit that XCD's L2.  Chunks are
    // dealt to the least-loaded of eight streams, the streams interleaved
    // and padded with empty units (segment -1) to one length.
    constexpr int kXcds = 8;
    std::vector<std::vector<int4>> stream(kXcds);
    int64_t e = 0;
    for (int s = 0; s < num_segments; s++) {
      const int64_t lr = (int64_t)(p->segs[s].len + kRowPad - 1) / kRowPad * kRowPad;
      // the attention addresses one segment's part of a head's table through
      // 32-bit buffer offsets: (lr / 128) * lr entries of 4 bytes must fit
      if ((lr / kQmBlock) * lr * 4 > (int64_t)INT32_MAX) {
        delete p;
        return fail(FP8ATTN_EUNSUPPORTED, "Q centring on E4M3 plans takes segments of at most 262016 tokens "
                                          "(32-bit offsets into the mean-term table)");
      }
      p->mt_seg[s] = e;
      e += (lr / kQmBlock) * lr;
    }
    p->mt_per_head = e;
    if ((double)e * 4.0 * heads > (double)((int64_t)1 << 40)) {
      delete p;
      return fail(FP8ATTN_EUNSUPPORTED, "Q-centring mean-term table above 1 TiB");
    }
    for (int h = 0; h < heads; h++)
      for (int s = 0; s < num_segments; s++) {
        const int64_t lr = (int64_t)(p->segs[s].len + kRowPad - 1) / kRowPad * kRowPad;
        const int64_t nbg = (lr / kQmBlock + kQmUnitBlocks - 1) / kQmUnitBlocks;
        for (int64_t k0 = 0; k0 < lr; k0 += kQmUnitKeys) {
          int best = 0;
          for (int x = 1; x < kXcds; x++)
            if (stream[x].size() < stream[best].size()) best = x;
          for (int64_t bg = 0; bg < nbg; bg++) stream[best].push_back(int4{s, (int)bg, (int)k0, h});
        }
      }
    size_t len = 0;
    for (const auto& v : stream) len = std::max(len, v.size());
    if ((double)len * kXcds > (double)INT32_MAX) {
      delete p;
      return fail(FP8ATTN_EUNSUPPORTED, "Q-centring mean-term work list above 2^31 units");
    }
    p->qmt_units.reserve(len * kXcds);
    for (size_t i = 0; i < len; i++)
      for (int x = 0; x < kXcds; x++) p->qmt_units.push_back(i < stream[x].size() ? stream[x][i] : int4{-1, 0, 0, 0});
  }
  // the attention kernel addresses one head's code rows through 32-bit buffer
  // offsets: rows * 128 bytes must fit
  if (row * p->dk > (int64_t)INT32_MAX || (row / kPackRows) * heads > (int64_t)INT32_MAX) {
    delete p;
    return fail(FP8ATTN_EUNSUPPORTED, "too many padded rows for 32-bit code offsets (about 16.7M tokens at most "
                                      "at head_dim 128) or too many 64-row groups times heads for one grid");
  }
  int cus = 256;   // MI355X; the device's own count when the plan has one
  if (device >= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && n > 0) cus = n;
  }
  choose_query_tile(p, cus);
  build_items(p, std::max(1, cus / kNumXcd), !p->causal);
  if (p->npieces >= (int64_t)1 << 23) {
    delete p;
    return fail(FP8ATTN_EUNSUPPORTED, "too many split work items");
  }
  p->ws = p->mx ? make_layout_mx(row, heads, num_segments, (int)p->chunks.size(), p->npieces)
                : make_layout(row, heads, num_segments, p->nscale, (int)p->chunks.size(), p->npieces, p->dk,
                              p->mt_per_head);

  if (device >= 0) {
    DeviceGuard g(device);
    if (!g.ok) {
      delete p;
      return fail(FP8ATTN_EHIP, "cannot select device");
    }
    const size_t b_segs = align_up(sizeof(SegInfo) * p->segs.size(), 256);
    const size_t b_chunks = align_up(sizeof(Chunk) * std::max<size_t>(1, p->chunks.size()), 256);
    const size_t b_groups = align_up(sizeof(int32_t) * p->group_seg.size(), 256);
    const size_t b_items = align_up(sizeof(int4) * std::max<size_t>(1, p->items.size()), 256);
    const size_t b_rowmap = align_up(sizeof(int32_t) * p->segs.size(), 256);
    const size_t b_combine = align_up(sizeof(int4) * std::max<size_t>(1, p->combine.size()), 256);
    const size_t b_mtseg = align_up(sizeof(int64_t) * std::max<size_t>(1, p->mt_seg.size()), 256);
    const size_t b_units = align_up(sizeof(int4) * std::max<size_t>(1, p->qmt_units.size()), 256);
    const size_t total = b_segs + b_chunks + b_groups + b_items + b_rowmap + b_combine + b_mtseg + b_units;
    std::vector<uint8_t> host(total, 0);
    size_t off = 0;
    std::memcpy(host.data() + off, p->segs.data(), sizeof(SegInfo) * p->segs.size());
    off += b_segs;
    if (!p->chunks.empty()) std::memcpy(host.data() + off, p->chunks.data(), sizeof(Chunk) * p->chunks.size());
    off += b_chunks;
    std::memcpy(host.data() + off, p->group_seg.data(), sizeof(int32_t) * p->group_seg.size());
    off += b_groups;
    if (!p->items.empty()) std::memcpy(host.data() + off, p->items.data(), sizeof(int4) * p->items.size());
    off += b_items;
    for (size_t s = 0; s < p->segs.size(); s++) {
      const int32_t r = p->segs[s].row0;
      std::memcpy(host.data() + off + 4 * s, &r, 4);
    }
    off += b_rowmap;
    if (!p->combine.empty()) std::memcpy(host.data() + off, p->combine.data(), sizeof(int4) * p->combine.size());
    off += b_combine;
    if (!p->mt_seg.empty()) std::memcpy(host.data() + off, p->mt_seg.data(), sizeof(int64_t) * p->mt_seg.size());
    off += b_mtseg;
    if (!p->qmt_units.empty()) std::memcpy(host.data() + off, p->qmt_units.data(), sizeof(int4) * p->qmt_units.size());
    hipError_t e = hipMalloc(&p->dev, total);
    if (e != hipSuccess) {
      delete p;
      return fail(FP8ATTN_ENOMEM, std::string("hipMalloc of plan tables failed: ") + hipGetErrorString(e));
    }
    e = hipMemcpy(p->dev, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(p->dev);
      delete p;
      return fail(FP8ATTN_EHIP, std::string("upload of plan tables failed: ") + hipGetErrorString(e));
    }
    uint8_t* d = static_cast<uint8_t*>(p->dev);
    p->d_segs = reinterpret_cast<SegInfo*>(d);
    p->d_chunks = reinterpret_cast<Chunk*>(d + b_segs);
    p->d_group_seg = reinterpret_cast<int32_t*>(d + b_segs + b_chunks);
    p->d_items = reinterpret_cast<int4*>(d + b_segs + b_chunks + b_groups);
    p->d_rowmap = reinterpret_cast<int32_t*>(d + b_segs + b_chunks + b_groups + b_items);
    p->d_combine = reinterpret_cast<int4*>(d + b_segs + b_chunks + b_groups + b_items + b_rowmap);
    p->d_mt_seg = reinterpret_cast<int64_t*>(d + b_segs + b_chunks + b_groups + b_items + b_rowmap + b_combine);
    p->d_qmt_units =
        reinterpret_cast<int4*>(d + b_segs + b_chunks + b_groups + b_items + b_rowmap + b_combine + b_mtseg);
  }
  *plan_out = p;
  return FP8ATTN_OK;
}

size_t fp8attn_workspace_bytes(fp8attn_plan_t p) { return p == nullptr ? 0 : p->ws.total; }

}  // extern "C"

namespace {

// Statistics bytes of a plan as laid out in the static buffer of
// fp8attn_quantize_noalloc: K statistics, then the Q/V amax partials.
size_t static_stats_bytes(const fp8attn_plan_s* p) {
  const size_t nch = p->chunks.size();
  const size_t kst = align_up(sizeof(KStat) * nch * (size_t)p->heads * (size_t)p->dk, 256);
  const size_t amx = p->mx ? 0 : align_up(sizeof(float) * 2 * nch * (size_t)p->heads, 256);
  const size_t qst = p->mt_per_head > 0
                         ? align_up(sizeof(float) * (size_t)(p->ws.rows / kQmBlock) * (size_t)p->heads * (size_t)(p->dk / 8), 256)
                         : 0;
  return kst + amx + qst;
}

// fp8attn_quantize and fp8attn_quantize_noalloc: the statistics go to the
// workspace's statistics region, or (noalloc) to the library's static buffer.
fp8attn_status quantize_impl(fp8attn_plan_t p, const void* q, const void* k, const void* v,
                             const int64_t q_strides[2], const int64_t k_strides[2],
                             const int64_t v_strides[2], void* workspace, size_t workspace_bytes,
                             void* stream, bool noalloc) {
  if (p == nullptr) return fail(FP8ATTN_EINVAL, "plan is NULL");
  if (noalloc && static_stats_bytes(p) > kStaticStatsBytes)
    return fail(FP8ATTN_EUNSUPPORTED,
                "plan needs " + std::to_string(static_stats_bytes(p)) + " bytes of statistics, more than the " +
                    std::to_string(kStaticStatsBytes) +
                    "-byte static buffer of fp8attn_quantize_noalloc (use fp8attn_quantize)");
  if (p->device < 0) return fail(FP8ATTN_EINVAL, "host-only plan cannot run");
  if (workspace == nullptr || ((uintptr_t)workspace & 255) != 0)
    return fail(FP8ATTN_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < (noalloc ? p->ws.stats_off : p->ws.total))
    return fail(FP8ATTN_EWORKSPACE, "workspace too small");
  if (p->tokens > 0) {
    if (q == nullptr || k == nullptr || v == nullptr) return fail(FP8ATTN_EINVAL, "q, k, v must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v))
      return fail(FP8ATTN_EINVAL, "q, k, v must be 16-byte aligned");
    if (!strides_ok(q_strides) || !strides_ok(k_strides) || !strides_ok(v_strides))
      return fail(FP8ATTN_EINVAL, "strides must be positive multiples of 8 elements");
  }
  DeviceGuard g(p->device);
  if (!g.ok) return fail(FP8ATTN_EHIP, "cannot select device");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* stats = ws + p->ws.kstat_off;                      // kstat, then amax (E4M3 plans), then qamax
  size_t amax_rel = p->mx ? 0 : p->ws.amax_off - p->ws.kstat_off;
  size_t qamax_rel = p->mt_per_head > 0 ? p->ws.qamax_off - p->ws.kstat_off : 0;
  if (noalloc) {
    const hipError_t e = static_stats_buffer(p->device, &stats);
    if (e != hipSuccess)
      return fail(FP8ATTN_EHIP, std::string("static statistics buffer: ") + hipGetErrorString(e));
    if (!p->mx) amax_rel = align_up(sizeof(KStat) * p->chunks.size() * (size_t)p->heads * (size_t)p->dk, 256);
    if (p->mt_per_head > 0)
      qamax_rel = amax_rel + align_up(sizeof(float) * 2 * p->chunks.size() * (size_t)p->heads, 256);
  }
  QuantizeArgs a{};
  a.x[0] = static_cast<const uint16_t*>(q);
  a.x[1] = static_cast<const uint16_t*>(k);
  a.x[2] = static_cast<const uint16_t*>(v);
  for (int i = 0; i < 3; i++) {
    const int64_t* st = i == 0 ? q_strides : (i == 1 ? k_strides : v_strides);
    a.ts[i] = p->tokens > 0 ? st[0] : 0;
    a.hs[i] = p->tokens > 0 ? st[1] : 0;
  }
  a.codes[0] = ws + p->ws.q_off;
  a.codes[1] = ws + p->ws.k_off;
  a.codes[2] = ws + p->ws.v_off;
  a.scales = reinterpret_cast<float*>(ws + p->ws.scale_off);
  a.mu = reinterpret_cast<float*>(ws + p->ws.mu_off);
  a.kstat = reinterpret_cast<KStat*>(stats);
  a.amax = reinterpret_cast<float*>(stats + amax_rel);
  a.segs = p->d_segs;
  a.chunks = p->d_chunks;
  a.group_seg = p->d_group_seg;
  a.heads = p->heads;
  a.nseg = p->nseg;
  a.nchunks = (int32_t)p->chunks.size();
  a.ngroups = (int32_t)p->group_seg.size();
  a.seg_scales = p->seg_scales;
  a.rows = p->ws.rows;
  a.softmax_scale = p->scale;
  a.mx = p->mx;
  a.q_centre = p->q_centre;
  a.head_dim = p->dk;
  a.d_real = p->head_dim;
  a.exact_probs = p->exact_probs;
  if (p->mt_per_head > 0) {
    a.qamax = reinterpret_cast<float*>(stats + qamax_rel);
    a.qmean = reinterpret_cast<float*>(ws + p->ws.qmean_off);
    a.mt = reinterpret_cast<uint32_t*>(ws + p->ws.mt_off);
    a.mt_seg = p->d_mt_seg;
    a.qmt_units = p->d_qmt_units;
    a.nqmt_units = (int32_t)p->qmt_units.size();
    a.mt_per_head = p->mt_per_head;
  }
  if (p->mx) {
    a.bscale[0] = ws + p->ws.qs_off;
    a.bscale[1] = ws + p->ws.ks_off;
    a.bscale[2] = ws + p->ws.vs_off;
    a.qm_codes = ws + p->ws.qm_off;
    a.qm_scales = ws + p->ws.qms_off;
    a.scales = nullptr;
    a.amax = nullptr;
  }
  hipError_t e = launch_quantize(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8ATTN_EHIP, std::string("quantize launch failed: ") + hipGetErrorString(e));
  return FP8ATTN_OK;
}

}  // namespace

extern "C" {

fp8attn_status fp8attn_quantize(fp8attn_plan_t p, const void* q, const void* k, const void* v,
                                const int64_t q_strides[2], const int64_t k_strides[2],
                                const int64_t v_strides[2], void* workspace, size_t workspace_bytes,
                                void* stream) {
  return quantize_impl(p, q, k, v, q_strides, k_strides, v_strides, workspace, workspace_bytes, stream, false);
}

fp8attn_status fp8attn_quantize_noalloc(fp8attn_plan_t p, const void* q, const void* k, const void* v,
                                        const int64_t q_strides[2], const int64_t k_strides[2],
                                        const int64_t v_strides[2], void* workspace, size_t workspace_bytes,
                                        void* stream) {
  return quantize_impl(p, q, k, v, q_strides, k_strides, v_strides, workspace, workspace_bytes, stream, true);
}

fp8attn_status fp8attn_forward(fp8attn_plan_t p, void* workspace, size_t workspace_bytes,
                               void* out, const int64_t out_strides[2], float* lse, void* stream) {
  if (p == nullptr) return fail(FP8ATTN_EINVAL, "plan is NULL");
  if (p->device < 0) return fail(FP8ATTN_EINVAL, "host-only plan cannot run");
  if (workspace == nullptr || ((uintptr_t)workspace & 255) != 0)
    return fail(FP8ATTN_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < p->ws.stats_off) return fail(FP8ATTN_EWORKSPACE, "workspace too small");
  if (p->tokens > 0) {
    if (out == nullptr) return fail(FP8ATTN_EINVAL, "out must be non-NULL");
    if (!aligned16(out)) return fail(FP8ATTN_EINVAL, "out must be 16-byte aligned");
    if (!strides_ok(out_strides)) return fail(FP8ATTN_EINVAL, "out strides must be positive multiples of 8");
    if (lse != nullptr && ((uintptr_t)lse & 3) != 0) return fail(FP8ATTN_EINVAL, "lse must be 4-byte aligned");
  }
  DeviceGuard g(p->device);
  if (!g.ok) return fail(FP8ATTN_EHIP, "cannot select device");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws + p->ws.part_o_off);
  float* part_w = reinterpret_cast<float*>(ws + p->ws.part_w_off);
  float* part_lse = reinterpret_cast<float*>(ws + p->ws.part_lse_off);
  const int64_t os0 = p->tokens > 0 ? out_strides[0] : 0;
  const int64_t os1 = p->tokens > 0 ? out_strides[1] : 0;
  const int32_t nitems = p->real_items > 0 ? (int32_t)p->items.size() : 0;
  hipError_t e;
  if (p->mx) {
    MxAttentionArgs m{};
    m.q_codes = ws + p->ws.q_off;
    m.k_codes = ws + p->ws.k_off;
    m.v_codes = ws + p->ws.v_off;
    m.q_scales = ws + p->ws.qs_off;
    m.k_scales = ws + p->ws.ks_off;
    m.v_scales = ws + p->ws.vs_off;
    m.qm_codes = ws + p->ws.qm_off;
    m.qm_scales = ws + p->ws.qms_off;
    m.mu = reinterpret_cast<const float*>(ws + p->ws.mu_off);
    m.segs = p->d_segs;
    m.items = p->d_items;
    m.out = static_cast<uint16_t*>(out);
    m.os0 = os0;
    m.os1 = os1;
    m.lse = lse;
    m.part_o = part_o;
    m.part_w = part_w;
    m.part_lse = part_lse;
    m.tokens = p->tokens;
    m.rows = p->ws.rows;
    m.heads = p->heads;
    m.nitems = nitems;
    m.q_centre = p->q_centre;
    m.causal = p->causal;
    e = launch_attention_mx(m, static_cast<hipStream_t>(stream));
  } else {
    AttentionArgs a{};
    a.q_codes = ws + p->ws.q_off;
    a.k_codes = ws + p->ws.k_off;
    a.v_codes = ws + p->ws.v_off;
    a.scales = reinterpret_cast<const float*>(ws + p->ws.scale_off);
    a.mu = reinterpret_cast<const float*>(ws + p->ws.mu_off);
    a.segs = p->d_segs;
    a.items = p->d_items;
    a.out = static_cast<uint16_t*>(out);
    a.os0 = os0;
    a.os1 = os1;
    a.lse = lse;
    a.part_o = part_o;
    a.part_w = part_w;
    a.part_lse = part_lse;
    a.tokens = p->tokens;
    a.rows = p->ws.rows;
    a.heads = p->heads;
    a.nitems = nitems;
    a.nscale = p->nscale;
    a.causal = p->causal;
    a.head_dim = p->dk;
    a.d_real = p->head_dim;
    a.bm = p->bm;
    a.exact_probs = p->exact_probs;
    a.softmax_scale = p->scale;
    if (p->mt_per_head > 0) {
      a.q_centre = 1;
      a.qmean = reinterpret_cast<const float*>(ws + p->ws.qmean_off);
      a.mt = reinterpret_cast<const uint32_t*>(ws + p->ws.mt_off);
      a.mt_seg = p->d_mt_seg;
      a.mt_per_head = p->mt_per_head;
    }
    e = launch_attention(a, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(FP8ATTN_EHIP, std::string("attention launch failed: ") + hipGetErrorString(e));
  if (!p->combine.empty()) {
    CombineArgs c{};
    c.items = p->d_combine;
    c.nitems = (int32_t)p->combine.size();
    c.segs = p->d_segs;
    c.part_o = part_o;
    c.part_w = part_w;
    c.part_lse = part_lse;
    c.out = static_cast<uint16_t*>(out);
    c.os0 = os0;
    c.os1 = os1;
    c.lse = lse;
    c.tokens = p->tokens;
    c.head_dim = p->dk;
    c.d_real = p->head_dim;
    c.bm = p->bm;
    e = launch_combine(c, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FP8ATTN_EHIP, std::string("combine launch failed: ") + hipGetErrorString(e));
  }
  return FP8ATTN_OK;
}

fp8attn_status fp8attn_workspace_region(fp8attn_plan_t p, const void* workspace, int which,
                                        const void** ptr_out, int64_t dims_out[3]) {
  if (p == nullptr || ptr_out == nullptr || dims_out == nullptr) return fail(FP8ATTN_EINVAL, "NULL argument");
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int64_t H = p->heads, R = p->ws.rows, D = p->dk;
  if (which == FP8ATTN_REGION_ROWMAP) {
    if (p->device < 0) return fail(FP8ATTN_EINVAL, "host-only plan has no device tables");
    *ptr_out = p->d_rowmap;
    dims_out[0] = p->nseg; dims_out[1] = 1; dims_out[2] = 1;
    return FP8ATTN_OK;
  }
  if (ws == nullptr) return fail(FP8ATTN_EWORKSPACE, "workspace is NULL");
  if (which == FP8ATTN_REGION_STATS) {
    *ptr_out = ws + p->ws.stats_off;
    dims_out[0] = (int64_t)(p->ws.total - p->ws.stats_off); dims_out[1] = 1; dims_out[2] = 1;
    return FP8ATTN_OK;
  }
  if (p->mx) {
    switch (which) {
      case FP8ATTN_REGION_Q_CODES: *ptr_out = ws + p->ws.q_off; dims_out[0] = H; dims_out[1] = R; dims_out[2] = kMxRow; break;
      case FP8ATTN_REGION_K_CODES: *ptr_out = ws + p->ws.k_off; dims_out[0] = H; dims_out[1] = R; dims_out[2] = kMxRow; break;
      case FP8ATTN_REGION_V_CODES: *ptr_out = ws + p->ws.v_off; dims_out[0] = H; dims_out[1] = R / kBN; dims_out[2] = kMxTile; break;
      case FP8ATTN_REGION_Q_BSCALES: *ptr_out = ws + p->ws.qs_off; dims_out[0] = H; dims_out[1] = R; dims_out[2] = 4; break;
      case FP8ATTN_REGION_K_BSCALES: *ptr_out = ws + p->ws.ks_off; dims_out[0] = H; dims_out[1] = R; dims_out[2] = 4; break;
      case FP8ATTN_REGION_V_BSCALES: *ptr_out = ws + p->ws.vs_off; dims_out[0] = H; dims_out[1] = R / kBN; dims_out[2] = kMxTileScales; break;
      case FP8ATTN_REGION_QM_CODES: *ptr_out = ws + p->ws.qm_off; dims_out[0] = H; dims_out[1] = R / kMxQBlock; dims_out[2] = kMxRow; break;
      case FP8ATTN_REGION_QM_SCALES: *ptr_out = ws + p->ws.qms_off; dims_out[0] = H; dims_out[1] = R / kMxQBlock; dims_out[2] = 4; break;
      case FP8ATTN_REGION_MU: *ptr_out = ws + p->ws.mu_off; dims_out[0] = p->nseg; dims_out[1] = H; dims_out[2] = D; break;
      default: return fail(FP8ATTN_EINVAL, "region not available for FP8ATTN_PLAN_MXFP4 plans");
    }
    return FP8ATTN_OK;
  }
  switch (which) {
    case FP8ATTN_REGION_Q_CODES: *ptr_out = ws + p->ws.q_off; dims_out[0] = H; dims_out[1] = R; dims_out[2] = D; break;
    case FP8ATTN_REGION_K_CODES: *ptr_out = ws + p->ws.k_off; dims_out[0] = H; dims_out[1] = R; dims_out[2] = D; break;
    case FP8ATTN_REGION_V_CODES: *ptr_out = ws + p->ws.v_off; dims_out[0] = H; dims_out[1] = D; dims_out[2] = R; break;
    case FP8ATTN_REGION_SCALES: *ptr_out = ws + p->ws.scale_off; dims_out[0] = 3; dims_out[1] = p->nscale; dims_out[2] = H; break;
    case FP8ATTN_REGION_MU: *ptr_out = ws + p->ws.mu_off; dims_out[0] = p->nseg; dims_out[1] = H; dims_out[2] = D; break;
    case FP8ATTN_REGION_QMEAN:
      if (p->mt_per_head == 0) return fail(FP8ATTN_EINVAL, "region needs an E4M3 plan with FP8ATTN_PLAN_Q_CENTRE");
      *ptr_out = ws + p->ws.qmean_off; dims_out[0] = H; dims_out[1] = R / kQmBlock; dims_out[2] = D; break;
    case FP8ATTN_REGION_QM_TERM:
      if (p->mt_per_head == 0) return fail(FP8ATTN_EINVAL, "region needs an E4M3 plan with FP8ATTN_PLAN_Q_CENTRE");
      *ptr_out = ws + p->ws.mt_off; dims_out[0] = H; dims_out[1] = p->mt_per_head; dims_out[2] = 4; break;
    default: return fail(FP8ATTN_EINVAL, "unknown region");
  }
  return FP8ATTN_OK;
}

fp8attn_status fp8attn_plan_info(fp8attn_plan_t p, int64_t info[14]) {
  if (p == nullptr || info == nullptr) return fail(FP8ATTN_EINVAL, "NULL argument");
  info[0] = p->tokens;
  info[1] = p->heads;
  info[2] = p->nseg;
  info[3] = p->ws.rows;
  info[4] = p->real_items;
  info[5] = (int64_t)p->chunks.size();
  info[6] = p->bm;
  info[7] = kBN;
  info[8] = p->seg_scales;
  info[9] = p->npieces;
  info[10] = p->mx;
  info[11] = p->q_centre;
  info[12] = p->causal;
  info[13] = p->head_dim;
  return FP8ATTN_OK;
}

fp8attn_status fp8attn_plan_work_items(fp8attn_plan_t p, int32_t* items_out, int64_t capacity,
                                       int64_t* count_out) {
  if (p == nullptr || count_out == nullptr) return fail(FP8ATTN_EINVAL, "NULL argument");
  if (capacity < 0 || (capacity > 0 && items_out == nullptr)) return fail(FP8ATTN_EINVAL, "bad capacity");
  const int64_t n = (int64_t)p->items.size();
  *count_out = n;
  const int64_t m = std::min(n, capacity);
  for (int64_t i = 0; i < m; i++) {
    items_out[4 * i + 0] = p->items[i].x;
    items_out[4 * i + 1] = p->items[i].y;
    items_out[4 * i + 2] = p->items[i].z;
    items_out[4 * i + 3] = p->items[i].w;
  }
  return FP8ATTN_OK;
}

fp8attn_status fp8attn_plan_destroy(fp8attn_plan_t p) {
  if (p == nullptr) return FP8ATTN_OK;
  if (p->dev != nullptr) {
    DeviceGuard g(p->device);
    (void)hipFree(p->dev);
  }
  delete p;
  return FP8ATTN_OK;
}

const char* fp8attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
