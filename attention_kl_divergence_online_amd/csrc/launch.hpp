// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Host-only declarations; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

// Row addressing of one family of per-unit tensors.  A launch runs BH units
// (one sequence of one head each); unit u starts at row
// base + (u / H) * sb + (u % H) * sh of its tensors, rows of D elements (row
// vectors: one element).  [B, H, N, D] tensors are unit after unit (row0 =
// u * N: `dense`); a run of equal-length sequences packed per head
// ([H, T, D], sequence length L, u = b * H + h, first sequence at packed row
// R) has sb = L, sh = T and base = R.
struct RowMap {
  int64_t sb, sh;
  int H;  // >= 1
  int64_t base;
  __host__ __device__ int64_t row0(int64_t u) const {
    const uint32_t uu = (uint32_t)u, hh = (uint32_t)H;
    return base + (int64_t)(uu / hh) * sb + (int64_t)(uu % hh) * sh;
  }
  static RowMap dense(int64_t N) { return RowMap{N, 0, 1, 0}; }
};

// A launch over several runs of a packed batch.  The runs' workgroups follow
// one another in the grid, segment i owning workgroups [start_i, start_i+1)
// (the last up to `end`).  A segment carries the launch parameters that differ
// between runs; the rest (pointers to the whole packed tensors, the per-head
// row stride sh of the maps, H, scale, flags) come from the launch's params.
struct Seg {
  uint32_t start;  // first workgroup
  int32_t tiles;   // query tiles (forward) per unit
  int64_t units;   // sequences x heads
  int64_t nq, nk;  // rows per sequence
  int64_t oq, ok;  // packed row of the run's first sequence, queries / keys
  int64_t u0;      // first unit of the run in the batch (per-unit sigma, scales, chunk maxima)
  int32_t chunks;  // prepare step: row chunks per tensor (abs_chunks(nq, nk))
};
constexpr int kMaxSegs = 32;
struct SegTable {
  int n;         // segments; 0: a plain launch (its params as given)
  uint32_t end;  // workgroups of the launch
  Seg seg[kMaxSegs];
};
// Segment of workgroup wg (t.n >= 1): the last one starting at or before wg.
__host__ __device__ inline int seg_index(const SegTable &t, uint32_t wg) {
  int lo = 0, hi = t.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.seg[mid].start <= wg) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
__host__ __device__ inline uint32_t seg_count(const SegTable &t, int i) {
  return (i + 1 < t.n ? t.seg[i + 1].start : t.end) - t.seg[i].start;
}

struct FwdParams {
  const void *q1, *k1, *q2, *k2;  // unit rows of NQ|NK x D in the input dtype (qmap / kmap)
  float *kl, *lse1, *lse2;         // unit rows of NQ (qmap)
  RowMap qmap, kmap;
  float *ws;                       // split-K partial states [5][splits][BH*NQ], else null
  int64_t BH, NQ, NK;
  float scale;
  int causal;
  int nqt;     // query tiles per head
  int splits;  // key chunks (1 = unsplit)
  int chunk;   // keys per chunk (multiple of the key tile)
  int small;   // unsplit bf16 main shape in 4-wave workgroups (fwd_small_shape), else 8-wave
};

struct BwdParams {
  const void *q1, *k1, *q2, *k2;      // qmap / kmap rows
  const float *kl, *lse1, *lse2, *g;  // qmap rows
  RowMap qmap, kmap;
  const float *sigma;   // per unit power-of-two factor applied to g
  const float *xscale;  // per unit 4 powers of two: fp16 operand scales of q1, q2, k1, k2 (bf16 inputs)
  float *dq1, *dk1, *dq2, *dk2;  // like the inputs (qmap / kmap rows), fp32
  // bf16 query-resident pass over `splits` key chunks of `kchunk` keys: each
  // chunk writes a partial dQ into dqp ([split][distribution][BH * NQ][D],
  // dense), and launch_dq_reduce sums them.  splits == 1: no partials.
  float *dqp;
  int splits, kchunk;
  int64_t BH, NQ, NK;
  float scale;
  int causal;
  int want1, want2;  // write teacher / student gradients
};

// Tile sizes the host needs for grids and validation.
constexpr int kFwdBK = 64;    // keys per forward stage of the split and fp32 shapes
constexpr int kFwdChunkTile = 128;  // split-K chunks are whole multiples of this (and of every forward tile)
constexpr int kBwdBR = 128;   // resident rows per backward workgroup
constexpr int kBwdTile = 64;  // streamed rows per backward stage
constexpr int kGradExp = 8;   // |g| * sigma <= 2^kGradExp before fp16 rounding of dS
// The prepare step takes each tensor's largest magnitude over C row chunks
// per unit, C = abs_chunks(NQ, NK) <= kAbsChunks (one chunk per 2048 rows of
// the longer side).
constexpr int kAbsChunks = 16;
inline int abs_chunks(int64_t NQ, int64_t NK) {
  const int64_t n = NQ > NK ? NQ : NK;
  const int64_t c = (n + 2047) / 2048;
  return (int)(c < 1 ? 1 : c > kAbsChunks ? kAbsChunks : c);
}

// Queries per forward workgroup for an input type (dtype: 0 = bf16, 1 = fp32)
// and query count per head; `small`: the 4-wave bf16 shape for the main
// (non-decode) case.
int fwd_block_queries(int dtype, int D, int64_t NQ, bool small);
// Whether an unsplit dense bf16 forward takes the 4-wave shape: always at
// D = 64, and for causal problems of at most kFwdSmallCausalRows queries at
// D = 128.  A packed batch takes it at D = 64, and when causal with every
// main-shape sequence at most kFwdSmallVarlenRows long.
constexpr int64_t kFwdSmallCausalRows = 4096;
constexpr int64_t kFwdSmallVarlenRows = 8192;
bool fwd_small_shape(int dtype, int D, int64_t NQ, bool causal);

// dtype: 0 = bf16, 1 = fp32.  Return the launch status.
hipError_t launch_fwd(int dtype, int D, const FwdParams &p, hipStream_t s);
// Unsplit forward over the segments of t (t.n >= 1), in one launch of t.end
// workgroups.  Every segment must have fwd_segment_shape(dtype, nq) and
// tiles = ceil(nq / fwd_block_queries(dtype, D, nq, p.small)); p supplies the
// whole packed tensors, the maps' sh and H, scale, causal and small.
bool fwd_segment_shape(int dtype, int64_t NQ);
hipError_t launch_fwd_segs(int dtype, int D, const FwdParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_splitk_merge(const FwdParams &p, hipStream_t s);
// Library-owned device scratch of the allocation-free split-K forward: a
// file-scope device array of kSplitkScratchBytes per GPU.  splitk_scratch
// returns its device address on the device `s` belongs to (the current device
// for the null stream), looked up once per device and kept.
constexpr size_t kSplitkScratchBytes = (size_t)64 << 20;
hipError_t splitk_scratch(hipStream_t s, float **ptr);
// The backward's prepare step: sigma per unit from g and, for bf16 inputs, the
// fp16 operand scales of q1, q2, k1, k2 from their largest magnitudes.
struct PrepParams {
  const void *q1, *q2, *k1, *k2;  // qmap / kmap rows
  const float *g;                 // qmap rows
  RowMap qmap, kmap;
  int64_t BH, NQ, NK;
  int D;
  float *sigma;   // [BH]
  float *xscale;  // [BH][4]
  float *part;    // [BH][4][kAbsChunks] chunk maxima (bf16 inputs)
};
hipError_t launch_bwd_prepare(int dtype, const PrepParams &p, hipStream_t s);
// The same over the segments of a packed batch: the chunk maxima (segment
// i holding units * 4 * chunks workgroups), then sigma and the scales (units
// workgroups); p supplies the whole packed tensors and the maps' sh and H.
hipError_t launch_absmax_segs(const PrepParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_grad_scale_segs(int dtype, const PrepParams &p, const SegTable &t, hipStream_t s);
// Backward passes; p.sigma and p.xscale must hold the prepare step's results.
hipError_t launch_bwd_dk(int dtype, int D, const BwdParams &p, hipStream_t s);
hipError_t launch_bwd_dq(int dtype, int D, const BwdParams &p, hipStream_t s);
// Either pass over the segments of t (t.n >= 1) in one launch of t.end
// workgroups, segment i holding units * ceil(resident rows / kBwdBR) of them
// (resident rows: nk for the dK pass, nq for the dQ pass; p.splits == 1).
// p supplies the whole packed tensors, the maps' sh and H, and sigma and the
// operand scales of the whole batch (each run's from its first unit u0).
hipError_t launch_bwd_dk_segs(int dtype, int D, const BwdParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_bwd_dq_segs(int dtype, int D, const BwdParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_zero(float *dst, int64_t n, hipStream_t s);
// Fused single-visit backward (bf16, at most kFusedMaxRows queries per unit):
// BH * p.splits workgroups, key chunks of p.kchunk keys (a multiple of 32);
// with p.splits > 1 dQ goes to the partials p.dqp (then launch_dq_reduce),
// else straight to dq1 / dq2; dK is written directly.  No prepare step.
// Workgroups hold fused_query_blocks(NQ) blocks of 32 queries (1 or 4).
constexpr int kFusedMaxRows = 128;
int fused_query_blocks(int64_t NQ);
hipError_t launch_bwd_fused(int dtype, int D, const BwdParams &p, hipStream_t s);
// dQ1 / dQ2 (the requested ones) = sum over the key chunks of p.dqp, in chunk order.
hipError_t launch_dq_reduce(int D, const BwdParams &p, hipStream_t s);
// Matrix-rate probe: `workgroups` workgroups of four waves, each wave `iters`
// rounds of four independent 32x32x16 bf16 products; writes one float per
// wave to sink[workgroups * 4].
hipError_t launch_mfma_rate(int iters, int workgroups, float *sink, hipStream_t s);

}  // namespace skl
