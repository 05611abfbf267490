// C ABI of the attention-KL library: argument validation, grid set-up and
// launches.  Every check runs on the host before anything is enqueued, so a
// rejected call writes nothing.
#include "../../include/streamkl.h"

#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "launch.hpp"

namespace {

// Backward workspace: the per-(b,h) factors sigma, the fp16 operand scales
// of q1, q2, k1, k2 ([BH][4] fp32), for bf16 inputs the chunk maxima the
// scales come from ([BH][4][kAbsChunks] fp32), then, when the query-resident
// pass is split over key chunks, its partial dQ ([splits][2][BH * NQ][D] fp32).
struct BwdLayout {
  size_t xs, part, dqp, total;
  bool split;  // the split dQ partials are part of the layout
};
inline size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// The bf16 query-resident pass runs one workgroup per CU (its LDS use); with
// fewer query tiles than CUs its key range is split into chunks so that the
// grid still covers the GPU.  fp32 inputs never split.
constexpr int64_t kDqSplitTarget = 256;  // workgroups to aim for (the CU count)
constexpr int64_t kDqSplitMax = 64;
struct DqSplit {
  int splits, kchunk;
};
DqSplit dq_split(const streamkl_problem *p) {
  DqSplit r{1, 0};
  if (p->dtype == STREAMKL_FP32 || p->NQ == 0 || p->NK == 0) return r;
  const int64_t wgs = p->B * p->H * ((p->NQ + skl::kBwdBR - 1) / skl::kBwdBR);
  if (wgs >= kDqSplitTarget) return r;
  const int64_t ktiles = (p->NK + skl::kBwdTile - 1) / skl::kBwdTile;
  int64_t sp = (kDqSplitTarget + wgs - 1) / wgs;
  if (sp > kDqSplitMax) sp = kDqSplitMax;
  if (sp > ktiles) sp = ktiles;
  if (sp <= 1) return r;
  const int64_t per = (ktiles + sp - 1) / sp;  // tiles per chunk
  r.splits = (int)((ktiles + per - 1) / per);  // no empty trailing chunk
  r.kchunk = (int)(per * skl::kBwdTile);
  return r.splits > 1 ? r : DqSplit{1, 0};
}
// The fused single-visit backward takes bf16 and fp8 problems of at most
// kFusedMaxRows queries per unit (decode and short query ranges): one
// workgroup per (unit, key chunk) with chunks of whole 32-key blocks, aiming
// at 2048 workgroups of one query block (512 of four), and a dQ partial per
// chunk when there are several ([splits][2][BH * NQ][D] fp32, at the front of
// the workspace).
bool use_fused(const streamkl_problem *p) {
  return (p->dtype == STREAMKL_BF16 || p->dtype == STREAMKL_FP8_E4M3) && p->NQ > 0 && p->NQ <= skl::kFusedMaxRows &&
         p->NK > 0;
}
DqSplit fused_split(const streamkl_problem *p) {
  const int64_t units = p->B * p->H;
  const int64_t blocks = (p->NK + 31) / 32;
  const int64_t target = skl::fused_query_blocks(p->NQ) == 1 ? 2048 : 512;
  int64_t sp = (target + units - 1) / std::max<int64_t>(units, 1);
  sp = std::max<int64_t>(1, std::min<int64_t>(sp, std::min<int64_t>(kDqSplitMax, blocks)));
  const int64_t per = (blocks + sp - 1) / sp;
  return DqSplit{(int)((blocks + per - 1) / per), (int)(per * 32)};
}
size_t fused_workspace(const streamkl_problem *p) {
  const DqSplit f = fused_split(p);
  const size_t part = f.splits > 1 ? (size_t)f.splits * 2 * (size_t)(p->B * p->H) * (size_t)p->NQ * (size_t)p->D * 4 : 0;
  return round_up(part > 16 ? part : 16, 256);
}

// Layout of a problem's backward workspace, with the split dQ partials when
// `with_split` and the query-resident pass splits its keys.
BwdLayout bwd_layout(const streamkl_problem *p, bool with_split = true) {
  BwdLayout l{};
  const size_t bh = (size_t)(p->B * p->H);
  l.xs = round_up(bh * sizeof(float) > 16 ? bh * sizeof(float) : 16, 256);
  l.part = l.xs + round_up(bh * 4 * sizeof(float) > 16 ? bh * 4 * sizeof(float) : 16, 256);
  l.dqp = l.part;
  if (p->dtype == STREAMKL_BF16) l.dqp += round_up(bh * 4 * skl::kAbsChunks * sizeof(float), 256);
  const DqSplit ds = dq_split(p);
  l.split = with_split && ds.splits > 1;
  const size_t dqp = l.split ? (size_t)ds.splits * 2 * bh * (size_t)p->NQ * (size_t)p->D * 4 : 0;
  l.total = l.dqp + round_up(dqp, 256);
  return l;
}

constexpr int kVersion = 200;  // 0.2.0
static_assert(STREAMKL_NOALLOC_SCRATCH_BYTES == skl::kSplitkScratchBytes, "scratch size in the header");

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// A dispatch's grid is at most 2^32 - 1 work-items.  The forward's largest
// grids are its query tiles x key chunks and the split-K merge (one thread
// per row); the backward's, its passes (resident tiles of 128 rows) and the
// prepare step's chunk maxima (4 tensors x up to kAbsChunks per unit).
constexpr __int128 kGridLimit = ((__int128)1 << 32) - 1;
bool fwd_grids_fit(const streamkl_problem *p, int64_t splits) {
  const __int128 bh = (__int128)p->B * p->H;
  // 64 work-items per 32 queries of a query tile.  The 4-wave shape's grid
  // (ceil(NQ / 128) x 256 work-items per head) is no larger than the main
  // shape's (256 queries, or 384 for fp8), so the main count bounds both.
  const int64_t bq = skl::fwd_block_queries(p->dtype, (int)p->D, p->NQ, false);
  const __int128 fwd = bh * ((p->NQ + bq - 1) / bq) * splits * (bq <= 32 ? 64 : 2 * bq);
  const __int128 merge = bh * ((p->NQ + 255) / 256 * 256);
  return fwd <= kGridLimit && merge <= kGridLimit;
}
bool bwd_grids_fit(const streamkl_problem *p) {
  const __int128 bh = (__int128)p->B * p->H;
  const int64_t nmax = p->NQ > p->NK ? p->NQ : p->NK;
  const __int128 bwd = bh * ((nmax + skl::kBwdBR - 1) / skl::kBwdBR) * 512 * dq_split(p).splits;
  const __int128 prep = bh * 4 * skl::kAbsChunks * 256;
  return bwd <= kGridLimit && prep <= kGridLimit;
}

// Shape / dtype checks common to every entry point.
streamkl_status check_problem(const streamkl_problem *p) {
  if (!p) return STREAMKL_ERR_NULL;
  if (p->dtype != STREAMKL_BF16 && p->dtype != STREAMKL_FP32 && p->dtype != STREAMKL_FP8_E4M3)
    return STREAMKL_ERR_DTYPE;
  if (p->B < 0 || p->H < 0 || p->NQ < 0 || p->NK < 0) return STREAMKL_ERR_SHAPE;
  if (p->D != 64 && p->D != 128) return STREAMKL_ERR_SHAPE;
  // A row with no visible key has no distribution to compare.
  if (p->B > 0 && p->H > 0 && p->NQ > 0 && p->NK == 0) return STREAMKL_ERR_SHAPE;
  if (p->causal && p->NQ > p->NK) return STREAMKL_ERR_SHAPE;
  // In-head byte offsets are 32-bit (buffer resources, per-head bases);
  // whole tensors use 64-bit bases.  The largest per-head object is an fp32
  // gradient tensor (bounded with rows rounded up to 64).
  const int64_t lim = (int64_t)1 << 31;
  const int64_t nmax = (p->NQ > p->NK ? p->NQ : p->NK);
  if (nmax >= lim || (nmax + 63) / 64 * 64 * p->D * 4 >= lim) return STREAMKL_ERR_SHAPE;
  if ((__int128)p->B * p->H >= lim) return STREAMKL_ERR_SHAPE;
  if (!(p->scale == p->scale)) return STREAMKL_ERR_SHAPE;  // NaN scale
  return STREAMKL_OK;
}

// check_problem plus the grid limit of the forward (`splits` key chunks) or
// of the backward.
streamkl_status check_fwd_problem(const streamkl_problem *p, int64_t splits) {
  const streamkl_status st = check_problem(p);
  if (st != STREAMKL_OK) return st;
  return fwd_grids_fit(p, splits) ? STREAMKL_OK : STREAMKL_ERR_SHAPE;
}
streamkl_status check_bwd_problem(const streamkl_problem *p) {
  const streamkl_status st = check_problem(p);
  if (st != STREAMKL_OK) return st;
  return bwd_grids_fit(p) ? STREAMKL_OK : STREAMKL_ERR_SHAPE;
}

bool empty_rows(const streamkl_problem *p) { return p->B == 0 || p->H == 0 || p->NQ == 0; }

streamkl_status check_inputs(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                             const void *k2) {
  if (!q1 || !k1 || !q2 || !k2) return STREAMKL_ERR_NULL;
  if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2)) return STREAMKL_ERR_ALIGN;
  (void)p;
  return STREAMKL_OK;
}

streamkl_status check_rowvecs(float *a, float *b, float *c) {
  if (!a || !b || !c) return STREAMKL_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return STREAMKL_ERR_ALIGN;
  return STREAMKL_OK;
}

int fwd_splits_max(const streamkl_problem *p) {
  return (int)((p->NK + skl::kFwdBK - 1) / skl::kFwdBK);
}

skl::FwdParams make_fwd(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                        const void *k2, float *kl, float *lse1, float *lse2) {
  skl::FwdParams f{};
  f.q1 = q1;
  f.k1 = k1;
  f.q2 = q2;
  f.k2 = k2;
  f.kl = kl;
  f.lse1 = lse1;
  f.lse2 = lse2;
  f.ws = nullptr;
  f.qmap = skl::RowMap::dense(p->NQ);
  f.kmap = skl::RowMap::dense(p->NK);
  f.BH = p->B * p->H;
  f.NQ = p->NQ;
  f.NK = p->NK;
  f.scale = p->scale;
  f.causal = p->causal ? 1 : 0;
  f.small = skl::fwd_small_shape(p->dtype, (int)p->D, p->NQ, p->causal != 0) ? 1 : 0;
  const int bq = skl::fwd_block_queries(p->dtype, (int)p->D, p->NQ, f.small != 0);
  f.nqt = (int)((p->NQ + bq - 1) / bq);
  f.splits = 1;
  f.chunk = (int)p->NK;
  return f;
}

}  // namespace

extern "C" {

const char *streamkl_status_string(int status) {
  switch (status) {
    case STREAMKL_OK: return "ok";
    case STREAMKL_ERR_NULL: return "required pointer is NULL";
    case STREAMKL_ERR_SHAPE: return "invalid problem shape";
    case STREAMKL_ERR_DTYPE: return "unsupported dtype";
    case STREAMKL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case STREAMKL_ERR_WORKSPACE: return "workspace missing or too small";
    case STREAMKL_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int streamkl_version(void) { return kVersion; }

streamkl_status streamkl_probe_mfma_bf16(int64_t iters, int64_t workgroups, float *sink, void *stream) {
  if (iters < 1 || iters > (int64_t{1} << 24) || workgroups < 1 || workgroups > (int64_t{1} << 20))
    return STREAMKL_ERR_SHAPE;
  if (!sink) return STREAMKL_ERR_NULL;
  if (!aligned16(sink)) return STREAMKL_ERR_ALIGN;
  return skl::launch_mfma_rate((int)iters, (int)workgroups, sink, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? STREAMKL_OK
             : STREAMKL_ERR_HIP;
}

streamkl_status streamkl_fwd(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                             const void *k2, float *kl, float *lse1, float *lse2, void *stream) {
  streamkl_status st = check_fwd_problem(p, 1);
  if (st != STREAMKL_OK) return st;
  if (empty_rows(p)) return STREAMKL_OK;
  if ((st = check_inputs(p, q1, k1, q2, k2)) != STREAMKL_OK) return st;
  if ((st = check_rowvecs(kl, lse1, lse2)) != STREAMKL_OK) return st;
  skl::FwdParams f = make_fwd(p, q1, k1, q2, k2, kl, lse1, lse2);
  if (skl::launch_fwd(p->dtype, (int)p->D, f, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return STREAMKL_ERR_HIP;
  return STREAMKL_OK;
}

size_t streamkl_fwd_splitk_workspace_size(const streamkl_problem *p, int num_splits) {
  if (check_problem(p) != STREAMKL_OK) return 0;
  if (num_splits < 1 || (p->NK > 0 && num_splits > fwd_splits_max(p)) || !fwd_grids_fit(p, num_splits)) return 0;
  return (size_t)5 * (size_t)num_splits * (size_t)(p->B * p->H * p->NQ) * sizeof(float);
}

}  // extern "C"

namespace {

// The split-K forward of streamkl_fwd_splitk and streamkl_fwd_splitk_noalloc.
// Host validation first; then `get_ws(need, &ws)` supplies a workspace of at
// least `need` bytes for num_splits > 1 (or the status that rejects the call).
template <class GetWs>
streamkl_status splitk_forward(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                               const void *k2, float *kl, float *lse1, float *lse2, int num_splits, void *stream,
                               GetWs get_ws) {
  streamkl_status st = check_problem(p);
  if (st != STREAMKL_OK) return st;
  if (num_splits < 1) return STREAMKL_ERR_SHAPE;
  if (empty_rows(p)) return STREAMKL_OK;
  if (num_splits > fwd_splits_max(p) || !fwd_grids_fit(p, num_splits)) return STREAMKL_ERR_SHAPE;
  if ((st = check_inputs(p, q1, k1, q2, k2)) != STREAMKL_OK) return st;
  if ((st = check_rowvecs(kl, lse1, lse2)) != STREAMKL_OK) return st;
  skl::FwdParams f = make_fwd(p, q1, k1, q2, k2, kl, lse1, lse2);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (num_splits == 1) {
    return skl::launch_fwd(p->dtype, (int)p->D, f, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
  }
  const size_t need = streamkl_fwd_splitk_workspace_size(p, num_splits);
  void *workspace = nullptr;
  if ((st = get_ws(need, &workspace)) != STREAMKL_OK) return st;
  if (!aligned16(workspace)) return STREAMKL_ERR_ALIGN;
  // Whole 128-key tiles per chunk; trailing chunks past NK are empty.
  const int64_t tiles = (p->NK + skl::kFwdChunkTile - 1) / skl::kFwdChunkTile;
  const int64_t tiles_per = (tiles + num_splits - 1) / num_splits;
  f.splits = num_splits;
  f.chunk = (int)(tiles_per * skl::kFwdChunkTile);
  f.ws = reinterpret_cast<float *>(workspace);
  // Split launches keep the 8-wave shape.
  f.small = 0;
  const int bq = skl::fwd_block_queries(p->dtype, (int)p->D, p->NQ, false);
  f.nqt = (int)((p->NQ + bq - 1) / bq);
  if (skl::launch_fwd(p->dtype, (int)p->D, f, s) != hipSuccess) return STREAMKL_ERR_HIP;
  if (skl::launch_splitk_merge(f, s) != hipSuccess) return STREAMKL_ERR_HIP;
  return STREAMKL_OK;
}

}  // namespace

extern "C" {

streamkl_status streamkl_fwd_splitk(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                                    const void *k2, float *kl, float *lse1, float *lse2, int num_splits,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  return splitk_forward(p, q1, k1, q2, k2, kl, lse1, lse2, num_splits, stream, [&](size_t need, void **ws) {
    if (!workspace || workspace_bytes < need) return STREAMKL_ERR_WORKSPACE;
    *ws = workspace;
    return STREAMKL_OK;
  });
}

streamkl_status streamkl_fwd_splitk_noalloc(const streamkl_problem *p, const void *q1, const void *k1,
                                            const void *q2, const void *k2, float *kl, float *lse1, float *lse2,
                                            int num_splits, void *stream) {
  return splitk_forward(p, q1, k1, q2, k2, kl, lse1, lse2, num_splits, stream, [&](size_t need, void **ws) {
    if (need > skl::kSplitkScratchBytes) return STREAMKL_ERR_WORKSPACE;
    float *scratch = nullptr;
    if (skl::splitk_scratch(reinterpret_cast<hipStream_t>(stream), &scratch) != hipSuccess)
      return STREAMKL_ERR_HIP;
    *ws = scratch;
    return STREAMKL_OK;
  });
}

size_t streamkl_bwd_workspace_size(const streamkl_problem *p) {
  if (check_bwd_problem(p) != STREAMKL_OK) return 0;
  const size_t split = bwd_layout(p).total;
  return use_fused(p) ? std::max(split, fused_workspace(p)) : split;
}

size_t streamkl_bwd_workspace_size_min(const streamkl_problem *p) {
  if (check_bwd_problem(p) != STREAMKL_OK) return 0;
  return bwd_layout(p, false).total;
}

}  // extern "C"

namespace {

// Validation shared by the backward entry points.  `outs` lists the gradient
// pointers of the call (pairs already checked); `need_ws` the workspace rule.
streamkl_status check_bwd(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                          const void *k2, const float *kl, const float *lse1, const float *lse2,
                          const float *g, float *const *outs, int nouts, const void *workspace,
                          size_t workspace_bytes, size_t need) {
  streamkl_status st = check_inputs(p, q1, k1, q2, k2);
  if (st != STREAMKL_OK) return st;
  for (int i = 0; i < nouts; ++i)
    if (outs[i] && !aligned16(outs[i])) return STREAMKL_ERR_ALIGN;
  if (p->NQ == 0) return STREAMKL_OK;
  if (!kl || !lse1 || !lse2 || !g) return STREAMKL_ERR_NULL;
  if (!aligned16(kl) || !aligned16(lse1) || !aligned16(lse2) || !aligned16(g)) return STREAMKL_ERR_ALIGN;
  if (!workspace || workspace_bytes < need) return STREAMKL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return STREAMKL_ERR_ALIGN;
  return STREAMKL_OK;
}

// Backward parameters over a workspace of `workspace_bytes`: sigma and the
// operand scales at the front; the query-resident pass splits its keys only
// when the workspace also holds the split partials (else it runs unsplit:
// the same results up to the fp32 summation order of dQ).
skl::BwdParams make_bwd(const streamkl_problem *p, const void *q1, const void *k1, const void *q2, const void *k2,
                        const float *kl, const float *lse1, const float *lse2, const float *g, float *dq1,
                        float *dk1, float *dq2, float *dk2, const void *workspace, size_t workspace_bytes) {
  skl::BwdParams b{};
  b.q1 = q1;
  b.k1 = k1;
  b.q2 = q2;
  b.k2 = k2;
  b.kl = kl;
  b.lse1 = lse1;
  b.lse2 = lse2;
  b.g = g;
  const BwdLayout l = bwd_layout(p, workspace_bytes >= bwd_layout(p, true).total);
  const char *w = reinterpret_cast<const char *>(workspace);
  b.sigma = reinterpret_cast<const float *>(w);
  b.xscale = reinterpret_cast<const float *>(w + l.xs);
  b.splits = 1;
  if (l.split) {
    const DqSplit ds = dq_split(p);
    b.splits = ds.splits;
    b.kchunk = ds.kchunk;
    b.dqp = const_cast<float *>(reinterpret_cast<const float *>(w + l.dqp));
  }
  b.dq1 = dq1;
  b.dk1 = dk1;
  b.dq2 = dq2;
  b.dk2 = dk2;
  b.qmap = skl::RowMap::dense(p->NQ);
  b.kmap = skl::RowMap::dense(p->NK);
  b.BH = p->B * p->H;
  b.NQ = p->NQ;
  b.NK = p->NK;
  b.scale = p->scale;
  b.causal = p->causal ? 1 : 0;
  return b;
}

// dK pass; with no query rows every key gradient is zero.
streamkl_status run_dk(const streamkl_problem *p, skl::BwdParams b, hipStream_t s) {
  if (p->NQ == 0) {
    const int64_t n = b.BH * p->NK * p->D;
    if (b.dk1 && skl::launch_zero(b.dk1, n, s) != hipSuccess) return STREAMKL_ERR_HIP;
    if (b.dk2 && skl::launch_zero(b.dk2, n, s) != hipSuccess) return STREAMKL_ERR_HIP;
    return STREAMKL_OK;
  }
  b.want1 = b.dk1 != nullptr;
  b.want2 = b.dk2 != nullptr;
  return skl::launch_bwd_dk(p->dtype, (int)p->D, b, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
}

streamkl_status run_dq(const streamkl_problem *p, skl::BwdParams b, hipStream_t s) {
  if (p->NQ == 0) return STREAMKL_OK;
  b.want1 = b.dq1 != nullptr;
  b.want2 = b.dq2 != nullptr;
  if (skl::launch_bwd_dq(p->dtype, (int)p->D, b, s) != hipSuccess) return STREAMKL_ERR_HIP;
  if (b.splits > 1 && skl::launch_dq_reduce((int)p->D, b, s) != hipSuccess) return STREAMKL_ERR_HIP;
  return STREAMKL_OK;
}

// The prepare step of `b`'s units into the front of `workspace`: sigma and,
// for bf16 inputs, the operand scales from the chunk maxima.
streamkl_status run_prepare(const streamkl_problem *p, const skl::BwdParams &b, void *workspace, hipStream_t s) {
  if (p->NQ == 0) return STREAMKL_OK;
  const BwdLayout l = bwd_layout(p, false);
  char *w = reinterpret_cast<char *>(workspace);
  skl::PrepParams pp{};
  pp.q1 = b.q1;
  pp.q2 = b.q2;
  pp.k1 = b.k1;
  pp.k2 = b.k2;
  pp.g = b.g;
  pp.qmap = b.qmap;
  pp.kmap = b.kmap;
  pp.BH = b.BH;
  pp.NQ = p->NQ;
  pp.NK = p->NK;
  pp.D = (int)p->D;
  pp.sigma = reinterpret_cast<float *>(w);
  pp.xscale = reinterpret_cast<float *>(w + l.xs);
  pp.part = p->dtype == STREAMKL_BF16 ? reinterpret_cast<float *>(w + l.part) : nullptr;
  return skl::launch_bwd_prepare(p->dtype, pp, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
}

}  // namespace

extern "C" {

streamkl_status streamkl_bwd(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                             const void *k2, const float *kl, const float *lse1, const float *lse2,
                             const float *g, float *dq1, float *dk1, float *dq2, float *dk2, void *workspace,
                             size_t workspace_bytes, void *stream) {
  streamkl_status st = check_bwd_problem(p);
  if (st != STREAMKL_OK) return st;
  if ((dq1 == nullptr) != (dk1 == nullptr) || (dq2 == nullptr) != (dk2 == nullptr)) return STREAMKL_ERR_NULL;
  if (p->B * p->H == 0 || (p->NQ == 0 && p->NK == 0)) return STREAMKL_OK;
  if (!dq1 && !dq2) return STREAMKL_OK;
  float *outs[4] = {dq1, dk1, dq2, dk2};
  st = check_bwd(p, q1, k1, q2, k2, kl, lse1, lse2, g, outs, 4, workspace, workspace_bytes,
                 streamkl_bwd_workspace_size_min(p));
  if (st != STREAMKL_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  skl::BwdParams b = make_bwd(p, q1, k1, q2, k2, kl, lse1, lse2, g, dq1, dk1, dq2, dk2, workspace, workspace_bytes);
  if (use_fused(p) && workspace_bytes >= fused_workspace(p)) {
    // Few queries: one fused single-visit pass, then the chunk partials of dQ.
    const DqSplit f = fused_split(p);
    b.splits = f.splits;
    b.kchunk = f.kchunk;
    b.dqp = f.splits > 1 ? reinterpret_cast<float *>(workspace) : nullptr;
    b.want1 = dq1 != nullptr;
    b.want2 = dq2 != nullptr;
    if (skl::launch_bwd_fused(p->dtype, (int)p->D, b, s) != hipSuccess) return STREAMKL_ERR_HIP;
    if (f.splits > 1 && skl::launch_dq_reduce((int)p->D, b, s) != hipSuccess) return STREAMKL_ERR_HIP;
    return STREAMKL_OK;
  }
  if ((st = run_prepare(p, b, workspace, s)) != STREAMKL_OK) return st;
  if ((st = run_dk(p, b, s)) != STREAMKL_OK) return st;
  return run_dq(p, b, s);
}

streamkl_status streamkl_bwd_prepare(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                                     const void *k2, const float *g, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  streamkl_status st = check_bwd_problem(p);
  if (st != STREAMKL_OK) return st;
  if (p->B * p->H == 0 || p->NQ == 0) return STREAMKL_OK;
  if ((st = check_inputs(p, q1, k1, q2, k2)) != STREAMKL_OK) return st;
  if (!g) return STREAMKL_ERR_NULL;
  if (!aligned16(g)) return STREAMKL_ERR_ALIGN;
  if (!workspace || workspace_bytes < streamkl_bwd_workspace_size_min(p)) return STREAMKL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return STREAMKL_ERR_ALIGN;
  const skl::BwdParams b = make_bwd(p, q1, k1, q2, k2, nullptr, nullptr, nullptr, g, nullptr, nullptr, nullptr,
                                    nullptr, workspace, workspace_bytes);
  return run_prepare(p, b, workspace, reinterpret_cast<hipStream_t>(stream));
}

streamkl_status streamkl_bwd_dk(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                                const void *k2, const float *kl, const float *lse1, const float *lse2,
                                const float *g, float *dk1, float *dk2, const void *workspace,
                                size_t workspace_bytes, void *stream) {
  streamkl_status st = check_bwd_problem(p);
  if (st != STREAMKL_OK) return st;
  if (p->B * p->H == 0 || p->NK == 0 || (!dk1 && !dk2)) return STREAMKL_OK;
  float *outs[2] = {dk1, dk2};
  st = check_bwd(p, q1, k1, q2, k2, kl, lse1, lse2, g, outs, 2, workspace, workspace_bytes,
                 streamkl_bwd_workspace_size_min(p));
  if (st != STREAMKL_OK) return st;
  skl::BwdParams b =
      make_bwd(p, q1, k1, q2, k2, kl, lse1, lse2, g, nullptr, dk1, nullptr, dk2, workspace, workspace_bytes);
  return run_dk(p, b, reinterpret_cast<hipStream_t>(stream));
}

streamkl_status streamkl_bwd_dq(const streamkl_problem *p, const void *q1, const void *k1, const void *q2,
                                const void *k2, const float *kl, const float *lse1, const float *lse2,
                                const float *g, float *dq1, float *dq2, const void *workspace,
                                size_t workspace_bytes, void *stream) {
  streamkl_status st = check_bwd_problem(p);
  if (st != STREAMKL_OK) return st;
  if (p->B * p->H == 0 || p->NQ == 0 || (!dq1 && !dq2)) return STREAMKL_OK;
  float *outs[2] = {dq1, dq2};
  st = check_bwd(p, q1, k1, q2, k2, kl, lse1, lse2, g, outs, 2, workspace, workspace_bytes,
                 streamkl_bwd_workspace_size_min(p));
  if (st != STREAMKL_OK) return st;
  skl::BwdParams b =
      make_bwd(p, q1, k1, q2, k2, kl, lse1, lse2, g, dq1, nullptr, dq2, nullptr, workspace, workspace_bytes);
  return run_dq(p, b, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Packed variable-length batches.  Each run of consecutive sequences with the
// same (query, key) lengths is one launchable problem whose units are
// (sequence, head) pairs addressed through row maps (b * L + h * T rows from
// the run's first row); runs are launched one after another on the stream.

namespace {

struct Run {
  int64_t b0, b1, nq, nk;
};

int64_t seq_len(const int32_t *cu, int64_t b) { return (int64_t)cu[b + 1] - (int64_t)cu[b]; }

// The problem a run stands for (B = its sequence count).
streamkl_problem run_problem(const streamkl_varlen_problem *v, const Run &r) {
  streamkl_problem p{};
  p.B = r.b1 - r.b0;
  p.H = v->H;
  p.NQ = r.nq;
  p.NK = r.nk;
  p.D = v->D;
  p.scale = v->scale;
  p.causal = v->causal;
  p.dtype = v->dtype;
  return p;
}

// Calls f(run) for the maximal runs of equal-length sequences, in order;
// stops at the first status other than OK.
template <class F>
streamkl_status for_each_run(const streamkl_varlen_problem *v, F f) {
  const int32_t *cq = v->cu_seqlens_q, *ck = v->cu_seqlens_k;
  int64_t b = 0;
  while (b < v->B) {
    const int64_t nq = seq_len(cq, b), nk = seq_len(ck, b);
    int64_t e = b + 1;
    while (e < v->B && seq_len(cq, e) == nq && seq_len(ck, e) == nk) ++e;
    const streamkl_status st = f(Run{b, e, nq, nk});
    if (st != STREAMKL_OK) return st;
    b = e;
  }
  return STREAMKL_OK;
}

streamkl_status check_varlen(const streamkl_varlen_problem *v, bool backward) {
  if (!v) return STREAMKL_ERR_NULL;
  if (v->dtype != STREAMKL_BF16 && v->dtype != STREAMKL_FP32 && v->dtype != STREAMKL_FP8_E4M3)
    return STREAMKL_ERR_DTYPE;
  if (v->B < 0 || v->H < 0) return STREAMKL_ERR_SHAPE;
  if (v->D != 64 && v->D != 128) return STREAMKL_ERR_SHAPE;
  if (!v->cu_seqlens_q || !v->cu_seqlens_k) return STREAMKL_ERR_NULL;
  const int32_t *cq = v->cu_seqlens_q, *ck = v->cu_seqlens_k;
  if (cq[0] != 0 || ck[0] != 0) return STREAMKL_ERR_SHAPE;
  for (int64_t b = 0; b < v->B; ++b)
    if (seq_len(cq, b) < 0 || seq_len(ck, b) < 0) return STREAMKL_ERR_SHAPE;
  if (v->H >= ((int64_t)1 << 31)) return STREAMKL_ERR_SHAPE;
  // Every run must be a valid problem on its own (lengths, causal shape,
  // per-sequence 32-bit offsets).
  return for_each_run(v, [&](const Run &r) {
    const streamkl_problem p = run_problem(v, r);
    return backward ? check_bwd_problem(&p) : check_fwd_problem(&p, 1);
  });
}

int64_t total_rows(const int32_t *cu, int64_t B) { return (int64_t)cu[B]; }

const void *adv_rows(const void *ptr, int64_t rows, int64_t D, int64_t es) {
  return ptr ? reinterpret_cast<const char *>(ptr) + rows * D * es : nullptr;
}
float *adv_rowsf(float *ptr, int64_t rows, int64_t D) { return ptr ? ptr + rows * D : nullptr; }

// Runs launched together: each run becomes one segment of a segmented launch
// (its workgroups follow the previous run's in one grid), so that short
// sequences share the GPU instead of each leaving most of it idle.  Segments
// go heaviest workgroups first (longest streamed range), and a launch holds at
// most kMaxSegs segments and kSegMaxWorkgroups workgroups of 512 work-items.
constexpr int64_t kSegMaxWorkgroups = (((int64_t)1 << 32) - 1) / 512;

struct SegItem {
  skl::Seg seg;     // start unused: assigned per launch
  int64_t count;    // workgroups of the segment
  int64_t weight;   // order key, larger first
};

template <class F>
streamkl_status launch_segments(std::vector<SegItem> items, F launch) {
  std::stable_sort(items.begin(), items.end(),
                   [](const SegItem &a, const SegItem &b) { return a.weight > b.weight; });
  skl::SegTable t{};
  int64_t end = 0;
  auto flush = [&]() -> streamkl_status {
    if (t.n == 0) return STREAMKL_OK;
    t.end = (uint32_t)end;
    const streamkl_status st = launch(t);
    t = skl::SegTable{};
    end = 0;
    return st;
  };
  for (const SegItem &it : items) {
    if (it.count == 0) continue;
    if (t.n == skl::kMaxSegs || end + it.count > kSegMaxWorkgroups) {
      const streamkl_status st = flush();
      if (st != STREAMKL_OK) return st;
    }
    t.seg[t.n] = it.seg;
    t.seg[t.n].start = (uint32_t)end;
    ++t.n;
    end += it.count;
  }
  return flush();
}

skl::Seg run_seg(const streamkl_varlen_problem *v, const Run &r) {
  skl::Seg g{};
  g.units = (r.b1 - r.b0) * v->H;
  g.nq = r.nq;
  g.nk = r.nk;
  g.oq = v->cu_seqlens_q[r.b0];
  g.ok = v->cu_seqlens_k[r.b0];
  g.u0 = r.b0 * v->H;
  return g;
}

// Backward workspace of a packed batch: sigma, the operand scales and (bf16
// inputs) the chunk maxima for every (sequence, head) of the runs that the
// segmented passes take, laid out like a problem's over all B * H units.  A
// run whose query-gradient pass splits its keys runs on its own afterwards,
// with the layout of its own problem at the front of the workspace.
struct VarlenLayout {
  size_t xs, part, total;
};

// The query-gradient pass splits keys only to fill the GPU: with at least
// kDqSplitTarget query tiles over the whole batch every run joins the
// segmented passes; otherwise a run whose own problem would split its keys
// runs on its own.
bool batch_fills_gpu(const streamkl_varlen_problem *v) {
  int64_t tiles = 0;
  for_each_run(v, [&](const Run &r) {
    tiles += (r.b1 - r.b0) * v->H * ((r.nq + skl::kBwdBR - 1) / skl::kBwdBR);
    return STREAMKL_OK;
  });
  return tiles >= kDqSplitTarget;
}

bool run_segmented_bwd(const streamkl_varlen_problem *v, const Run &r, bool fills) {
  if (r.nq == 0) return false;
  if (fills) return true;
  const streamkl_problem p = run_problem(v, r);
  return dq_split(&p).splits == 1;
}

VarlenLayout varlen_layout(const streamkl_varlen_problem *v) {
  VarlenLayout l{};
  const size_t units = (size_t)(v->B * v->H);
  l.xs = round_up(units * sizeof(float) > 16 ? units * sizeof(float) : 16, 256);
  l.part = l.xs + round_up(units * 4 * sizeof(float) > 16 ? units * 4 * sizeof(float) : 16, 256);
  size_t total = l.part;
  if (v->dtype == STREAMKL_BF16) total += round_up(units * 4 * skl::kAbsChunks * sizeof(float), 256);
  const bool fills = batch_fills_gpu(v);
  for_each_run(v, [&](const Run &r) {
    if (r.nq > 0 && !run_segmented_bwd(v, r, fills)) {
      const streamkl_problem p = run_problem(v, r);
      total = std::max(total, bwd_layout(&p).total);
    }
    return STREAMKL_OK;
  });
  l.total = total;
  return l;
}

}  // namespace

extern "C" {

streamkl_status streamkl_fwd_varlen(const streamkl_varlen_problem *v, const void *q1, const void *k1,
                                    const void *q2, const void *k2, float *kl, float *lse1, float *lse2,
                                    void *stream) {
  streamkl_status st = check_varlen(v, false);
  if (st != STREAMKL_OK) return st;
  const int64_t TQ = total_rows(v->cu_seqlens_q, v->B), TK = total_rows(v->cu_seqlens_k, v->B);
  if (v->B == 0 || v->H == 0 || TQ == 0) return STREAMKL_OK;
  if (!q1 || !k1 || !q2 || !k2) return STREAMKL_ERR_NULL;
  if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2)) return STREAMKL_ERR_ALIGN;
  if ((st = check_rowvecs(kl, lse1, lse2)) != STREAMKL_OK) return st;
  const int64_t es = v->dtype == STREAMKL_BF16 ? 2 : v->dtype == STREAMKL_FP8_E4M3 ? 1 : 4;
  const int D = (int)v->D;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Runs of the main kernel shape: segmented launches, all in one shape (the
  // 4-wave one at D = 64, and for causal batches whose main-shape sequences
  // are all at most kFwdSmallVarlenRows long).  Decode-shaped runs (few
  // queries per sequence) launch on their own.
  int64_t longest = 0;
  (void)for_each_run(v, [&](const Run &r) {
    if (r.nq > 0 && skl::fwd_segment_shape(v->dtype, r.nq)) longest = std::max(longest, r.nq);
    return STREAMKL_OK;
  });
  const bool small =
      (v->dtype == STREAMKL_BF16 || v->dtype == STREAMKL_FP8_E4M3) &&
      (D == 64 || (v->causal && longest <= skl::kFwdSmallVarlenRows));
  std::vector<SegItem> items;
  st = for_each_run(v, [&](const Run &r) {
    if (r.nq == 0) return STREAMKL_OK;
    if (skl::fwd_segment_shape(v->dtype, r.nq)) {
      SegItem it{run_seg(v, r), 0, r.nk};
      const int bq = skl::fwd_block_queries(v->dtype, D, r.nq, small);
      it.seg.tiles = (int32_t)((r.nq + bq - 1) / bq);
      it.count = it.seg.units * it.seg.tiles;
      items.push_back(it);
      return STREAMKL_OK;
    }
    const streamkl_problem p = run_problem(v, r);
    const int64_t oq = v->cu_seqlens_q[r.b0], ok = v->cu_seqlens_k[r.b0];
    skl::FwdParams f = make_fwd(&p, adv_rows(q1, oq, v->D, es), adv_rows(k1, ok, v->D, es),
                                adv_rows(q2, oq, v->D, es), adv_rows(k2, ok, v->D, es), kl + oq, lse1 + oq,
                                lse2 + oq);
    f.qmap = skl::RowMap{r.nq, TQ, (int)v->H, 0};
    f.kmap = skl::RowMap{r.nk, TK, (int)v->H, 0};
    return skl::launch_fwd(v->dtype, D, f, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
  });
  if (st != STREAMKL_OK || items.empty()) return st;
  const streamkl_problem p0 = run_problem(v, Run{0, 1, 0, 0});
  skl::FwdParams f = make_fwd(&p0, q1, k1, q2, k2, kl, lse1, lse2);
  f.qmap = skl::RowMap{0, TQ, (int)v->H, 0};
  f.kmap = skl::RowMap{0, TK, (int)v->H, 0};
  f.small = small ? 1 : 0;
  return launch_segments(items, [&](const skl::SegTable &t) {
    return skl::launch_fwd_segs(v->dtype, D, f, t, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
  });
}

size_t streamkl_bwd_varlen_workspace_size(const streamkl_varlen_problem *v) {
  if (check_varlen(v, true) != STREAMKL_OK) return 0;
  return varlen_layout(v).total;
}

streamkl_status streamkl_bwd_varlen(const streamkl_varlen_problem *v, const void *q1, const void *k1,
                                    const void *q2, const void *k2, const float *kl, const float *lse1,
                                    const float *lse2, const float *g, float *dq1, float *dk1, float *dq2,
                                    float *dk2, void *workspace, size_t workspace_bytes, void *stream) {
  streamkl_status st = check_varlen(v, true);
  if (st != STREAMKL_OK) return st;
  if ((dq1 == nullptr) != (dk1 == nullptr) || (dq2 == nullptr) != (dk2 == nullptr)) return STREAMKL_ERR_NULL;
  const int64_t TQ = total_rows(v->cu_seqlens_q, v->B), TK = total_rows(v->cu_seqlens_k, v->B);
  if (v->B == 0 || v->H == 0 || (TQ == 0 && TK == 0)) return STREAMKL_OK;
  if (!dq1 && !dq2) return STREAMKL_OK;
  if (!q1 || !k1 || !q2 || !k2) return STREAMKL_ERR_NULL;
  if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2)) return STREAMKL_ERR_ALIGN;
  for (float *o : {dq1, dk1, dq2, dk2})
    if (o && !aligned16(o)) return STREAMKL_ERR_ALIGN;
  if (TQ > 0) {
    if (!kl || !lse1 || !lse2 || !g) return STREAMKL_ERR_NULL;
    if (!aligned16(kl) || !aligned16(lse1) || !aligned16(lse2) || !aligned16(g)) return STREAMKL_ERR_ALIGN;
    if (!workspace || workspace_bytes < streamkl_bwd_varlen_workspace_size(v)) return STREAMKL_ERR_WORKSPACE;
    if (!aligned16(workspace)) return STREAMKL_ERR_ALIGN;
  }
  const int64_t D = v->D, H = v->H;
  const bool bf16 = v->dtype == STREAMKL_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const VarlenLayout l = varlen_layout(v);
  char *w = reinterpret_cast<char *>(workspace);

  // Query-less runs: their key gradients are zero.  Segmented runs: the
  // prepare step (chunk maxima, then sigma and the operand scales, each
  // unit's at its place in the batch), then one pass of each kind over all.
  std::vector<SegItem> abs_items, sig_items, dk_items, dq_items;
  const bool fills = batch_fills_gpu(v);
  st = for_each_run(v, [&](const Run &r) {
    const int64_t ok = v->cu_seqlens_k[r.b0];
    if (r.nq == 0) {
      const int64_t n = (r.b1 - r.b0) * r.nk * D;
      for (int64_t h = 0; h < H && n > 0; ++h)
        for (float *dk : {dk1, dk2})
          if (dk && skl::launch_zero(dk + (h * TK + ok) * D, n, s) != hipSuccess) return STREAMKL_ERR_HIP;
      return STREAMKL_OK;
    }
    if (!run_segmented_bwd(v, r, fills)) return STREAMKL_OK;
    SegItem it{run_seg(v, r), 0, 0};
    it.seg.chunks = skl::abs_chunks(r.nq, r.nk);
    const int64_t br = skl::kBwdBR;
    SegItem ab = it, us = it;
    ab.count = it.seg.units * 4 * it.seg.chunks;  // chunk maxima: (unit, tensor, chunk)
    us.count = it.seg.units;                      // sigma and scales: one workgroup per unit
    abs_items.push_back(ab);
    sig_items.push_back(us);
    SegItem a = it, b = it;
    a.count = it.seg.units * ((r.nk + br - 1) / br);  // dK pass: key tiles, streaming the queries
    a.weight = r.nq;
    b.count = it.seg.units * ((r.nq + br - 1) / br);  // dQ pass: query tiles, streaming the keys
    b.weight = r.nk;
    dk_items.push_back(a);
    dq_items.push_back(b);
    return STREAMKL_OK;
  });
  if (st != STREAMKL_OK) return st;
  if (!dk_items.empty()) {
    skl::PrepParams pp{};
    pp.q1 = q1;
    pp.q2 = q2;
    pp.k1 = k1;
    pp.k2 = k2;
    pp.g = g;
    pp.qmap = skl::RowMap{0, TQ, (int)H, 0};
    pp.kmap = skl::RowMap{0, TK, (int)H, 0};
    pp.D = (int)D;
    pp.sigma = reinterpret_cast<float *>(w);
    pp.xscale = reinterpret_cast<float *>(w + l.xs);
    pp.part = bf16 ? reinterpret_cast<float *>(w + l.part) : nullptr;
    if (bf16) {
      st = launch_segments(abs_items, [&](const skl::SegTable &t) {
        return skl::launch_absmax_segs(pp, t, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
      });
      if (st != STREAMKL_OK) return st;
    }
    st = launch_segments(sig_items, [&](const skl::SegTable &t) {
      return skl::launch_grad_scale_segs(v->dtype, pp, t, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
    });
    if (st != STREAMKL_OK) return st;
    skl::BwdParams b{};
    b.q1 = q1;
    b.k1 = k1;
    b.q2 = q2;
    b.k2 = k2;
    b.kl = kl;
    b.lse1 = lse1;
    b.lse2 = lse2;
    b.g = g;
    b.sigma = pp.sigma;
    b.xscale = pp.xscale;
    b.splits = 1;
    b.qmap = pp.qmap;
    b.kmap = pp.kmap;
    b.scale = v->scale;
    b.causal = v->causal ? 1 : 0;
    b.dk1 = dk1;
    b.dk2 = dk2;
    b.want1 = dk1 != nullptr;
    b.want2 = dk2 != nullptr;
    st = launch_segments(dk_items, [&](const skl::SegTable &t) {
      return skl::launch_bwd_dk_segs(v->dtype, (int)D, b, t, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
    });
    if (st != STREAMKL_OK) return st;
    b.dk1 = b.dk2 = nullptr;
    b.dq1 = dq1;
    b.dq2 = dq2;
    b.want1 = dq1 != nullptr;
    b.want2 = dq2 != nullptr;
    st = launch_segments(dq_items, [&](const skl::SegTable &t) {
      return skl::launch_bwd_dq_segs(v->dtype, (int)D, b, t, s) == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP;
    });
    if (st != STREAMKL_OK) return st;
  }

  // Runs whose query-gradient pass splits its keys, one after another with
  // their own layout at the front of the workspace (stream order keeps them
  // after the segmented passes that read it).
  const int64_t es = bf16 ? 2 : v->dtype == STREAMKL_FP8_E4M3 ? 1 : 4;
  return for_each_run(v, [&](const Run &r) {
    if (r.nq == 0 || run_segmented_bwd(v, r, fills)) return STREAMKL_OK;
    const int64_t oq = v->cu_seqlens_q[r.b0], ok = v->cu_seqlens_k[r.b0];
    const streamkl_problem p = run_problem(v, r);
    skl::BwdParams b = make_bwd(&p, adv_rows(q1, oq, D, es), adv_rows(k1, ok, D, es), adv_rows(q2, oq, D, es),
                                adv_rows(k2, ok, D, es), kl + oq, lse1 + oq, lse2 + oq, g + oq,
                                adv_rowsf(dq1, oq, D), adv_rowsf(dk1, ok, D), adv_rowsf(dq2, oq, D),
                                adv_rowsf(dk2, ok, D), workspace, workspace_bytes);
    b.qmap = skl::RowMap{r.nq, TQ, (int)H, 0};
    b.kmap = skl::RowMap{r.nk, TK, (int)H, 0};
    streamkl_status rs = run_prepare(&p, b, workspace, s);
    if (rs == STREAMKL_OK) rs = run_dk(&p, b, s);
    if (rs == STREAMKL_OK) rs = run_dq(&p, b, s);
    return rs;
  });
}

}  // extern "C"
