// Forward of the fused attention KL divergence: one online pass over key tiles.
//
// StreamKL (arXiv 2606.20005), gist.science "Formulacion Online": per query row
// keep running maxima m1, m2, exponential sums l1, l2 and an accumulator acc of
// the P1-weighted logit difference; emit KL = acc/l1 + LSE2 - LSE1 with
// LSE_t = m_t + log l_t.  Causal key tiles beyond the boundary are skipped
// outright.  The split-K variant ("Variante Split-K") cuts the key range into
// chunks handled by separate workgroups; a merge kernel combines their row
// states with log-sum-exp rescaling.
//
// gfx950 mapping
//  * logits are produced transposed (keys x queries) so that every lane owns
//    one query: each lane keeps its own online state over its keys of a
//    block, no cross-lane reduction happens inside the loop, and the lanes
//    sharing a query are merged once at the end;
//  * bf16 and fp8 inputs: the student's products continue the teacher's
//    chain with Q2 negated, so a block yields x1 and x1 - x2; fully visible
//    blocks are folded against the maxima a lane already holds (no block
//    maximum, no rescale), both distributions' exponentials against the mean
//    of the two, and the exact update runs only when a block's sums grow
//    past 2^24 or the two maxima lie far apart;
//  * the resident queries' Q1/Q2 fragments stay in registers for the whole
//    pass; key tiles stream through double-buffered LDS (or, for at most 16
//    queries, straight into registers);
//  * bf16 inputs: 8 waves x 32 queries over 128-key tiles (fwd2_kernel), or
//    4 waves x 32 queries over 64-key tiles at D = 64 and for short causal
//    problems (two workgroups per CU), one wave x 32 queries over 32-key
//    tiles for at most 32 queries per head, and 16x16 products for at most 16
//    (fwd16_kernel); fp8 (e4m3) inputs: the same kernel on the fp8 matrix
//    instructions, 12 waves x 32 queries (three per SIMD) in the main shape;
//    fp32 inputs: fwd_kernel with register-staged tiles and compensated sums;
//  * scores stay in raw dot-product units x = q.k; exponentials are
//    exp2((x - m) * scale * log2 e).
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace skl {

constexpr int kFwdThreads = 8 * 64;

template <typename T, int D>
struct FwdTraits {
  static constexpr int WAVES = 8;
  // 32-query blocks per wave (fp32 at D=128 keeps one so its fragments fit in registers)
  static constexpr int QB = 1;
  static constexpr int NT = WAVES * 64;
  static constexpr int BQ = WAVES * QB * 32;
  // Keys per LDS stage (fp32 at D=128 keeps 64 to fit two stages in LDS).
  static constexpr int BK = kFwdBK;
  static constexpr int NB = BK / 32;  // 32-key blocks per stage
  static constexpr int KSTEPS = D / 16;
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  static constexpr int LDS_ROW = ROW_BYTES + 16;
  static constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per row
  static constexpr int LOADS = BK * CPR / NT;
  static constexpr int STAGE_BYTES = 2 * BK * LDS_ROW;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(LOADS * NT == BK * CPR, "staging split");
};

// v + cv carries a running sum; replace it by a * (v + cv) + s.  The product
// and the sum are split into result + exact rounding error (fma residual and
// Knuth's two-sum), so the error of the running sum stays at a few ulp however
// many blocks are folded in.  Used for fp32 inputs, whose 1e-5 relative bound
// on KL leaves no room for the ~sqrt(#blocks) ulp drift of plain accumulation.
__device__ __forceinline__ void fold_compensated(float &v, float &cv, float a, float s) {
#pragma clang fp contract(off)
  const float x = v * a;
  const float ex = __builtin_fmaf(v, a, -x);
  const float t = x + s;
  const float bv = t - x;
  const float es = (x - (t - bv)) + (s - bv);
  cv = __builtin_fmaf(cv, a, ex + es);
  v = t;
}

// Running online state of one query as held by one lane (its share of the keys).
struct RowState {
  float m1, l1, m2, l2, acc;
  float c1, c2, cacc;  // compensation terms (fp32 inputs only)
};

// Fold one 32-key block of raw scores into a lane's running state.
// Element r of x1/x2 is key kbase + acc_row(r, h); keys >= klim are masked.
template <bool MASK, bool COMP>
__device__ __forceinline__ void online_update(const f32x16 &x1, const f32x16 &x2, RowState &st, float c,
                                              int kbase, int h, int klim) {
  float mx1 = st.m1, mx2 = st.m2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const bool v = !MASK || (kbase + acc_row(r, h) < klim);
    if (v) {
      mx1 = fmaxf(mx1, x1[r]);
      mx2 = fmaxf(mx2, x2[r]);
    }
  }
  const float a1 = fast_exp2((st.m1 - mx1) * c);
  const float a2 = fast_exp2((st.m2 - mx2) * c);
  st.m1 = mx1;
  st.m2 = mx2;
  const float b1 = mx1 * c, b2 = mx2 * c;
  float s1 = 0.f, s2 = 0.f, sa = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float p1 = fast_exp2(__builtin_fmaf(x1[r], c, -b1));
    float p2 = fast_exp2(__builtin_fmaf(x2[r], c, -b2));
    float d = x1[r] - x2[r];
    if (MASK) {
      const bool v = kbase + acc_row(r, h) < klim;
      p1 = v ? p1 : 0.f;
      p2 = v ? p2 : 0.f;
      d = v ? d : 0.f;
    }
    s1 += p1;
    s2 += p2;
    sa = __builtin_fmaf(p1, d, sa);
  }
  if (COMP) {
    fold_compensated(st.l1, st.c1, a1, s1);
    fold_compensated(st.l2, st.c2, a2, s2);
    fold_compensated(st.acc, st.cacc, a1, sa);
  } else {
    st.l1 = __builtin_fmaf(st.l1, a1, s1);
    st.l2 = __builtin_fmaf(st.l2, a2, s2);
    st.acc = __builtin_fmaf(st.acc, a1, sa);
  }
}

// KL, LSE1, LSE2 of a row from its merged state (raw-score units for m).
__device__ __forceinline__ void finish_row(float m1, float l1, float m2, float l2, float acc, float scale,
                                           float *kl, float *lse1, float *lse2) {
  const float ln1 = logf(l1), ln2 = logf(l2);
  *lse1 = __builtin_fmaf(scale, m1, ln1);
  *lse2 = __builtin_fmaf(scale, m2, ln2);
  *kl = scale * (acc / l1 - (m1 - m2)) - (ln1 - ln2);
}

// Head and query tile of workgroup w in an unsplit forward launch of n
// workgroups.  Each XCD runs a contiguous run of logical ids on its own heads.
// By default the run is head-major, the longest (last) query tiles of a head
// first, so that the workgroups running at once stream one head's keys and
// share them through one L2.  Causal query tiles differ in length, and with
// few tiles per head (up to kLongestFirstTiles) that order leaves the XCD's
// CUs unevenly loaded at the end; then, when the heads divide evenly over the
// XCDs, the run holds whole heads and goes longest tile first across all of
// them (list scheduling).  Measured on the forward: 20% faster at 16 query
// tiles per head, 7% at 64, and 3% slower at 256, where the L2 sharing counts
// for more than the balance.
__device__ __forceinline__ void unsplit_tile(const FwdParams &p, uint32_t w, uint32_t n, int64_t &bh, int &qt) {
  // With fewer heads than XCDs, contiguous runs would give some XCDs only the
  // long causal tiles of a head: the tiles are dealt round the XCDs in launch
  // order instead (measured 32% faster at 4 heads of 64K).  From 8 heads up
  // the runs stay, which keeps each XCD's key stream to one or two heads
  // (dealing measured 6% slower at 12 heads of 32K).
  const uint32_t L = p.causal && p.BH < kXcds ? w : xcd_remap(w, n);
  const uint32_t nqt = (uint32_t)p.nqt;
  if (p.causal && p.nqt <= kLongestFirstTiles && p.BH % kXcds == 0) {
    const uint32_t hx = (uint32_t)(p.BH / kXcds), per = hx * nqt;
    const uint32_t i = L % per;
    bh = (int64_t)(L / per) * hx + i % hx;
    qt = (int)(nqt - 1 - i / hx);
  } else {
    bh = L / nqt;
    qt = (int)(nqt - 1 - L % nqt);
  }
}

// Workgroup wg of a segmented launch (t.n > 0, unsplit): its segment's
// parameters replace the run-dependent ones in p, and wg, nwg become the
// workgroup's index and count within the segment.  A plain launch (t.n == 0)
// keeps its parameters.
__device__ __forceinline__ void select_segment(FwdParams &p, const SegTable &t, uint32_t &wg, uint32_t &nwg) {
  if (t.n == 0) return;
  const int lo = seg_index(t, wg);
  nwg = seg_count(t, lo);
  wg -= t.seg[lo].start;
  p.BH = t.seg[lo].units;
  p.NQ = t.seg[lo].nq;
  p.NK = t.seg[lo].nk;
  p.nqt = t.seg[lo].tiles;
  p.qmap.sb = t.seg[lo].nq;
  p.qmap.base = t.seg[lo].oq;
  p.kmap.sb = t.seg[lo].nk;
  p.kmap.base = t.seg[lo].ok;
}

template <typename T, int D, bool SPLIT>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_kernel(FwdParams p, const SegTable t) {
  using Tr = FwdTraits<T, D>;
  using CT = chunk_t<T>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;

  // Workgroup -> (head, query tile, key chunk).
  uint32_t wg = blockIdx.x, nwg = gridDim.x;
  select_segment(p, t, wg, nwg);
  int qt, sp;
  int64_t bh;
  if (SPLIT) {
    // Workgroups that share a key chunk are adjacent logical ids on one XCD.
    const uint32_t L = xcd_remap(wg, nwg);
    qt = (int)(L % (uint32_t)p.nqt);
    const uint32_t rest = L / (uint32_t)p.nqt;
    sp = (int)(rest % (uint32_t)p.splits);
    bh = rest / (uint32_t)p.splits;
  } else {
    unsplit_tile(p, wg, nwg, bh, qt);
    sp = 0;
  }

  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int64_t rq = p.qmap.row0(bh), rk = p.kmap.row0(bh);
  const T *Q1 = reinterpret_cast<const T *>(p.q1) + rq * D;
  const T *Q2 = reinterpret_cast<const T *>(p.q2) + rq * D;
  const char *K1 = reinterpret_cast<const char *>(reinterpret_cast<const T *>(p.k1) + rk * D);
  const char *K2 = reinterpret_cast<const char *>(reinterpret_cast<const T *>(p.k2) + rk * D);

  const int q0 = qt * Tr::BQ;
  const int qend = min(q0 + Tr::BQ, NQ);
  const int qw0 = q0 + wave * Tr::QB * 32;
  const int qw_last = min(qw0 + Tr::QB * 32 - 1, qend - 1);
  const bool wave_live = qw0 <= qw_last;

  const int kwg_end = p.causal ? min(NK, qend - 1 + off + 1) : NK;
  const int k_lo = SPLIT ? sp * p.chunk : 0;
  const int k_hi = SPLIT ? min(k_lo + p.chunk, kwg_end) : kwg_end;
  const int ntiles = k_hi > k_lo ? (k_hi - k_lo + Tr::BK - 1) / Tr::BK : 0;

  // Keys below vis_all are visible to every query of this wave; none at or above vis_any is.
  const int vis_all = min(k_hi, p.causal ? qw0 + off + 1 : NK);
  const int vis_any = min(k_hi, p.causal ? qw_last + off + 1 : NK);

  // Resident query fragments: lane owns query qw0 + qb*32 + c32, elements [16s + 8h, +8).
  CT qf1[Tr::QB][Tr::KSTEPS], qf2[Tr::QB][Tr::KSTEPS];
  int klim[Tr::QB];
#pragma unroll
  for (int qb = 0; qb < Tr::QB; ++qb) {
    const int row = qw0 + qb * 32 + c32;
    const bool ok = row < qend;
    klim[qb] = min(k_hi, p.causal ? row + off + 1 : NK);
#pragma unroll
    for (int s = 0; s < Tr::KSTEPS; ++s) {
      qf1[qb][s] = ok ? load_chunk<T>(Q1 + (int64_t)row * D + 16 * s + 8 * h) : CT{};
      qf2[qb][s] = ok ? load_chunk<T>(Q2 + (int64_t)row * D + 16 * s + 8 * h) : CT{};
    }
  }

  const float c = p.scale * kLog2e;
  constexpr bool COMP = sizeof(T) == 4;
  RowState st[Tr::QB];
#pragma unroll
  for (int qb = 0; qb < Tr::QB; ++qb) st[qb] = RowState{kNegBig, 0.f, kNegBig, 0.f, 0.f, 0.f, 0.f, 0.f};

  // Global -> register staging of the next key tile (16-byte chunks, coalesced rows).
  u32x4 stg1[Tr::LOADS], stg2[Tr::LOADS];
  auto gload = [&](int t) {
    const int kb0 = k_lo + t * Tr::BK;
#pragma unroll
    for (int i = 0; i < Tr::LOADS; ++i) {
      const int cidx = tid + Tr::NT * i;
      const int row = cidx / Tr::CPR, col = cidx % Tr::CPR;
      const int key = kb0 + row;
      if (key < NK) {
        stg1[i] = *reinterpret_cast<const u32x4 *>(K1 + (int64_t)key * Tr::ROW_BYTES + col * 16);
        stg2[i] = *reinterpret_cast<const u32x4 *>(K2 + (int64_t)key * Tr::ROW_BYTES + col * 16);
      } else {
        stg1[i] = u32x4{0u, 0u, 0u, 0u};
        stg2[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto sstore = [&](int buf) {
    char *base = smem + buf * Tr::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Tr::LOADS; ++i) {
      const int cidx = tid + Tr::NT * i;
      const int row = cidx / Tr::CPR, col = cidx % Tr::CPR;
      *reinterpret_cast<u32x4 *>(base + row * Tr::LDS_ROW + col * 16) = stg1[i];
      *reinterpret_cast<u32x4 *>(base + Tr::BK * Tr::LDS_ROW + row * Tr::LDS_ROW + col * 16) = stg2[i];
    }
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  // Scores of one 32-key block of the stage at `base` for every query block of the wave.
  auto block_scores = [&](const char *base, int kb, f32x16 *s1, f32x16 *s2) {
#pragma unroll
    for (int qb = 0; qb < Tr::QB; ++qb) {
      s1[qb] = f32x16{};
      s2[qb] = f32x16{};
    }
    const char *r1 = base + (kb * 32 + c32) * Tr::LDS_ROW + 8 * h * (int)sizeof(T);
    const char *r2 = r1 + Tr::BK * Tr::LDS_ROW;
#pragma unroll
    for (int s = 0; s < Tr::KSTEPS; ++s) {
      const CT a1 = *reinterpret_cast<const CT *>(r1 + 16 * s * (int)sizeof(T));
      const CT a2 = *reinterpret_cast<const CT *>(r2 + 16 * s * (int)sizeof(T));
#pragma unroll
      for (int qb = 0; qb < Tr::QB; ++qb) {
        s1[qb] = mma16(a1, qf1[qb][s], s1[qb]);
        s2[qb] = mma16(a2, qf2[qb][s], s2[qb]);
      }
    }
  };

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    const char *base = smem + (t & 1) * Tr::STAGE_BYTES;
    if (wave_live) {
#pragma unroll
      for (int kb = 0; kb < Tr::NB; ++kb) {
        const int kbase = k_lo + t * Tr::BK + kb * 32;
        if (kbase >= vis_any) continue;
        f32x16 s1[Tr::QB], s2[Tr::QB];
        block_scores(base, kb, s1, s2);
        if (kbase + 32 <= vis_all) {
#pragma unroll
          for (int qb = 0; qb < Tr::QB; ++qb)
            online_update<false, COMP>(s1[qb], s2[qb], st[qb], c, kbase, h, 0);
        } else {
#pragma unroll
          for (int qb = 0; qb < Tr::QB; ++qb)
            online_update<true, COMP>(s1[qb], s2[qb], st[qb], c, kbase, h, klim[qb]);
        }
      }
    }
    if (t + 1 < ntiles) sstore((t + 1) & 1);
    __syncthreads();
  }


  // Merge the two lane halves that hold disjoint keys of the same query.
#pragma unroll
  for (int qb = 0; qb < Tr::QB; ++qb) {
    const float m1 = st[qb].m1, m2 = st[qb].m2;
    const float l1 = COMP ? st[qb].l1 + st[qb].c1 : st[qb].l1;
    const float l2 = COMP ? st[qb].l2 + st[qb].c2 : st[qb].l2;
    const float acc = COMP ? st[qb].acc + st[qb].cacc : st[qb].acc;
    const float om1 = __shfl_xor(m1, 32), ol1 = __shfl_xor(l1, 32);
    const float om2 = __shfl_xor(m2, 32), ol2 = __shfl_xor(l2, 32);
    const float oacc = __shfl_xor(acc, 32);
    const float M1 = fmaxf(m1, om1), M2 = fmaxf(m2, om2);
    const float wa = fast_exp2((m1 - M1) * c), wb = fast_exp2((om1 - M1) * c);
    const float va = fast_exp2((m2 - M2) * c), vb = fast_exp2((om2 - M2) * c);
    const float L1 = __builtin_fmaf(l1, wa, ol1 * wb);
    const float A = __builtin_fmaf(acc, wa, oacc * wb);
    const float L2 = __builtin_fmaf(l2, va, ol2 * vb);
    const int row = qw0 + qb * 32 + c32;
    if (h == 0 && row < qend) {
      if (SPLIT) {
        // Partial states are indexed densely by (unit, row).
        const int64_t rows = p.BH * (int64_t)NQ;
        float *w = p.ws + (int64_t)sp * rows + bh * (int64_t)NQ + row;
        const int64_t fstride = (int64_t)p.splits * rows;
        w[0] = M1;
        w[fstride] = L1;
        w[2 * fstride] = M2;
        w[3 * fstride] = L2;
        w[4 * fstride] = A;
      } else {
        const int64_t idx = rq + row;
        finish_row(M1, L1, M2, L2, A, p.scale, p.kl + idx, p.lse1 + idx, p.lse2 + idx);
      }
    }
  }
}

// One thread per row: merge the per-chunk states in chunk order (deterministic).
__global__ __launch_bounds__(256) void splitk_merge_kernel(FwdParams p) {
  const int64_t rows = p.BH * p.NQ;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows) return;
  const float c = p.scale * kLog2e;
  const int64_t fstride = (int64_t)p.splits * rows;
  const float *w = p.ws + idx;
  float M1 = kNegBig, M2 = kNegBig;
  for (int s = 0; s < p.splits; ++s) {
    const float *ws = w + (int64_t)s * rows;
    if (ws[fstride] > 0.f) {
      M1 = fmaxf(M1, ws[0]);
      M2 = fmaxf(M2, ws[2 * fstride]);
    }
  }
  float L1 = 0.f, L2 = 0.f, A = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float *ws = w + (int64_t)s * rows;
    const float l1 = ws[fstride];
    if (l1 > 0.f) {
      const float w1 = fast_exp2((ws[0] - M1) * c);
      const float w2 = fast_exp2((ws[2 * fstride] - M2) * c);
      L1 = __builtin_fmaf(w1, l1, L1);
      A = __builtin_fmaf(w1, ws[4 * fstride], A);
      L2 = __builtin_fmaf(w2, ws[3 * fstride], L2);
    }
  }
  const int64_t u = idx / p.NQ, o = p.qmap.row0(u) + (idx - u * p.NQ);
  finish_row(M1, L1, M2, L2, A, p.scale, p.kl + o, p.lse1 + o, p.lse2 + o);
}

// ---- bf16 inputs: direct LDS staging, pipelined key blocks ----
//
// Each wave owns 32 queries; key tiles of K1 and K2 reach LDS through buffer
// loads (no staging registers, rows past NK read as zero) into double buffers
// with XOR-swizzled 16-byte chunks, one barrier per tile.  A wave walks its
// 32-key blocks as a pipeline: the logits of block b + 1 are computed while
// the online update of block b runs, in one instruction stream whenever both
// blocks are fully visible (no mask code).
//
// Two shapes: 8 waves (two per SIMD) over 64-key tiles for query tiles of
// 256, and, for at most 32 queries per head (decode), one wave over 32-key
// tiles.  The small shape's 32 KB of LDS lets about five workgroups share a
// CU, so every resident wave has live queries and several tiles of keys are
// in flight per CU; the large shape at 32 queries would leave seven of eight
// waves idle and one tile in flight.
//
// fp8 (e4m3) inputs take the same shapes with v_mfma_f32_32x32x64_f8f6f4:
// rows of D bytes, and per 64-element k-step a lane supplies 32 bytes of its
// row (elements 64 s + 32 h ..).  The instruction pairs byte j of lane (h, c)
// of A with byte j of lane (h, c') of B, so any such split of the row that
// both operands share gives the full dot product.
template <int D, int WAVES_ = 8, int BK_ = kFwdBK, bool F8_ = false>
struct Fwd2Traits {
  static constexpr bool F8 = F8_;
  static constexpr int WAVES = WAVES_;
  static constexpr int NT = 64 * WAVES;
  static constexpr int BQ = 32 * WAVES;  // 32 queries per wave
  static constexpr int BK = BK_;         // keys per tile
  static constexpr int BPT = BK / 32;    // 32-key blocks per tile
  static constexpr int KSTEPS = F8 ? D / 64 : D / 16;
  static constexpr int RB = F8 ? D : D * 2;  // row bytes
  static constexpr int CPROW = RB / 16;
  static constexpr int ROW_T = BK * RB;  // one tensor's key tile
  static constexpr int LDS_BYTES = 2 * 2 * ROW_T;
  static constexpr int CHUNKS = ROW_T / 16;            // 16-byte loads per tensor per tile
  static constexpr int LOADS = (CHUNKS + NT - 1) / NT;  // per tensor per thread (the last may be partial)
  static_assert((BK == 128 || BK == 64 || BK == 32) && NT % 64 == 0, "tiles");
};

// Bound on a lane's per-block sum in the forward's lazy update (2^24).
constexpr float kLazySumMax = 16777216.f;
constexpr float kLazyLog2Max = 24.f;
// Largest distance (log2 units) between a row's two held maxima for which
// the lazy update takes both distributions' terms against their mean: terms
// within 2^30 of their maximum are then scaled by at most 2^80, so they stay
// normal floats, and sums at most 2^24 by at most 2^104.
constexpr float kSharedSpan = 160.f;

// Queries per head at or below which bf16 inputs take the one-wave shapes:
// 16x16 products up to 16 queries, 32x32 products up to 32; fp8 inputs take
// the one-wave 32x32 shape up to 32 queries.
constexpr int kDecodeRows = 32;
constexpr int kDecode16Rows = 16;
inline bool fwd_decode_shape(int dtype, int64_t NQ) { return (dtype == 0 || dtype == 2) && NQ <= kDecodeRows; }
// Input types the matrix-core forward takes: bf16 (0) and fp8 e4m3 (2).
inline bool fwd_mfma_dtype(int dtype) { return dtype == 0 || dtype == 2; }
// Waves of the main fp8 shape.  Half-size query fragments leave the fp8
// kernel at 160 registers, so three waves share a SIMD (384 queries per
// workgroup): 3% faster than eight waves at causal 64K.  Four per SIMD
// would need 128 registers and spills.
constexpr int kF8Waves = 12;
inline bool fwd_decode16_shape(int dtype, int64_t NQ) { return dtype == 0 && NQ <= kDecode16Rows; }

template <int D, bool SPLIT, int WAVES, int BK, bool F8>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void fwd2_kernel(FwdParams p, const SegTable t) {
  using Tr = Fwd2Traits<D, WAVES, BK, F8>;
  using Frag = typename std::conditional<F8, i32x8, bf16x8>::type;  // one k-step of a lane's row
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;

  uint32_t wg = blockIdx.x, nwg = gridDim.x;
  select_segment(p, t, wg, nwg);
  int qt, sp;
  int64_t bh;
  if (SPLIT) {
    // Workgroups that share a key chunk are adjacent logical ids on one XCD.
    const uint32_t L = xcd_remap(wg, nwg);
    qt = (int)(L % (uint32_t)p.nqt);
    const uint32_t rest = L / (uint32_t)p.nqt;
    sp = (int)(rest % (uint32_t)p.splits);
    bh = rest / (uint32_t)p.splits;
  } else {
    unsplit_tile(p, wg, nwg, bh, qt);
    sp = 0;
  }

  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int64_t rq = p.qmap.row0(bh), rk = p.kmap.row0(bh);
  const char *Q1 = reinterpret_cast<const char *>(p.q1) + rq * Tr::RB;
  const char *Q2 = reinterpret_cast<const char *>(p.q2) + rq * Tr::RB;
  const BufRange rk1{reinterpret_cast<const char *>(p.k1) + rk * Tr::RB, NK * Tr::RB};
  const BufRange rk2{reinterpret_cast<const char *>(p.k2) + rk * Tr::RB, NK * Tr::RB};

  const int q0 = qt * Tr::BQ;
  const int qend = min(q0 + Tr::BQ, NQ);
  const int qw0 = q0 + wave * 32;
  const int qw_last = min(qw0 + 31, qend - 1);
  const bool wave_live = qw0 <= qw_last;

  const int kwg_end = p.causal ? min(NK, qend - 1 + off + 1) : NK;
  const int k_lo = SPLIT ? sp * p.chunk : 0;
  const int k_hi = SPLIT ? min(k_lo + p.chunk, kwg_end) : kwg_end;
  const int ntiles = k_hi > k_lo ? (k_hi - k_lo + Tr::BK - 1) / Tr::BK : 0;

  // This wave's 32-key blocks from k_lo: [0, nfull) are visible to all its
  // queries, [nfull, nlive) to some, the rest to none.
  const int vis_all = min(k_hi, p.causal ? qw0 + off + 1 : NK);
  const int vis_any = min(k_hi, p.causal ? qw_last + off + 1 : NK);
  const int nfull = wave_live ? max(0, vis_all - k_lo) / 32 : 0;
  const int nlive = wave_live ? (max(0, vis_any - k_lo) + 31) / 32 : 0;

  // Resident query fragments: lane owns query qw0 + c32; k-step s is bytes
  // [FB (2 s + h), + FB) of the row, FB = 16 (bf16) or 32 (fp8).  The
  // student's are negated (sign bits flipped): its chain, seeded with the
  // teacher's logits, yields x1 - x2.
  const int row = qw0 + c32;
  const bool row_ok = row < qend;
  const int klim = min(k_hi, p.causal ? row + off + 1 : NK);
  constexpr int FB = (int)sizeof(Frag);
  Frag qf1[Tr::KSTEPS], qf2[Tr::KSTEPS];
#pragma unroll
  for (int s = 0; s < Tr::KSTEPS; ++s) {
    qf1[s] = row_ok ? *reinterpret_cast<const Frag *>(Q1 + (int64_t)row * Tr::RB + FB * (2 * s + h)) : Frag{};
    qf2[s] = row_ok ? *reinterpret_cast<const Frag *>(Q2 + (int64_t)row * Tr::RB + FB * (2 * s + h)) : Frag{};
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qf2[s][i] ^= (int)0x80808080u;
    } else {
      qf2[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf2[s]) ^ 0x80008000u);
    }
  }

  const float c = p.scale * kLog2e;
  RowState st{kNegBig, 0.f, kNegBig, 0.f, 0.f, 0.f, 0.f, 0.f};

  // Key tile t into buffer t & 1: tensor-major, key r at r * RB, logical
  // chunk c in slot c ^ swz_row(r) (the swizzle repeats every 16 rows, so a
  // 32-key block reads the same slots in either tile shape).
  uint32_t voff[Tr::LOADS];
#pragma unroll
  for (int i = 0; i < Tr::LOADS; ++i) {
    const int C = i * Tr::NT + tid;
    const int r = C / Tr::CPROW;
    voff[i] = r * Tr::RB + ((C % Tr::CPROW) ^ swz_bytes<Tr::RB>(r)) * 16;
  }
  auto load_tile = [&](int t) {
    const uint32_t soff = (uint32_t)(k_lo + t * Tr::BK) * Tr::RB;
    char *buf = smem + (t & 1) * 2 * Tr::ROW_T;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int i = 0; i < Tr::LOADS; ++i)
        if (Tr::CHUNKS % Tr::NT == 0 || i * Tr::NT + wave * 64 < Tr::CHUNKS)  // whole waves only
          buffer_load_lds16(tn ? rk2 : rk1, buf + tn * Tr::ROW_T + (i * Tr::NT + wave * 64) * 16, voff[i], soff);
  };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Logits of block b (key block b % BPT of tile b / BPT): the teacher's x1
  // in s1 and x1 - x2 in s2 (the student's chain continues the teacher's).
  auto scores = [&](int b, f32x16 &s1, f32x16 &s2) {
    const int kr = (b % Tr::BPT) * 32 + c32;
    const int sw = swz_bytes<Tr::RB>(kr);
    const char *r1 = smem + ((b / Tr::BPT) & 1) * 2 * Tr::ROW_T + kr * Tr::RB;
    const char *r2 = r1 + Tr::ROW_T;
    s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < Tr::KSTEPS; ++s) {
      if constexpr (F8) {
        const int c0 = 4 * s + 2 * h;  // the lane's two 16-byte chunks
        const int pa = (c0 ^ sw) * 16, pb = ((c0 + 1) ^ sw) * 16;
        s1 = mma_f8(join16(*reinterpret_cast<const u32x4 *>(r1 + pa), *reinterpret_cast<const u32x4 *>(r1 + pb)),
                    qf1[s], s1);
      } else {
        s1 = mma16(*reinterpret_cast<const bf16x8 *>(r1 + ((2 * s + h) ^ sw) * 16), qf1[s], s1);
      }
    }
    s2 = s1;
#pragma unroll
    for (int s = 0; s < Tr::KSTEPS; ++s) {
      if constexpr (F8) {
        const int c0 = 4 * s + 2 * h;
        const int pa = (c0 ^ sw) * 16, pb = ((c0 + 1) ^ sw) * 16;
        s2 = mma_f8(join16(*reinterpret_cast<const u32x4 *>(r2 + pa), *reinterpret_cast<const u32x4 *>(r2 + pb)),
                    qf2[s], s2);
      } else {
        s2 = mma16(*reinterpret_cast<const bf16x8 *>(r2 + ((2 * s + h) ^ sw) * 16), qf2[s], s2);
      }
    }
  };
  // Exact update of a block from x1 and x1 - x2.
  auto exact = [&](const f32x16 &x1, const f32x16 &d, int kbase, auto mask_tag) __attribute__((always_inline)) {
    f32x16 x2;
#pragma unroll
    for (int r = 0; r < 16; ++r) x2[r] = x1[r] - d[r];
    online_update<decltype(mask_tag)::value, false>(x1, x2, st, c, kbase, h, klim);
  };
  auto update = [&](int b, const f32x16 &s1, const f32x16 &s2) {
    const int kbase = k_lo + b * 32;
    if (b < nfull)
      exact(s1, s2, kbase, std::false_type{});
    else
      exact(s1, s2, kbase, std::true_type{});
  };
  // Fully visible block after the first: the exponentials are taken against
  // the maxima the lane holds, with no new maxima and no rescaling.  The
  // running sums stay sums of exp2((x - m) c) for the held m, which is all
  // the combine step needs; m only has to keep them finite.  Both
  // distributions' terms use one offset, the mean hs of the held maxima
  // (times c): with y = x1 c - hs, the student's exponent is y - (x1 - x2) c,
  // one fused multiply-add.  A term relative to its own held maximum is the
  // computed one times w = 2^(hs - hb), a per-row constant the block sums are
  // scaled by.  The wave takes this form only while every lane's held maxima
  // lie within kSharedSpan of each other (log2 units), so that terms within
  // 2^30 of their maximum stay normal floats.  If some lane's block sum of
  // either distribution, relative to its held maximum, exceeds 2^24 (or is
  // not a number), or the maxima are too far apart, the whole wave folds the
  // block with the exact update, which raises the maxima; otherwise every
  // term of the block is at most 2^24 and the sums grow by at most that much
  // per block.
  float hs = 0.f, w1 = 1.f, w2 = 1.f;         // shared offset and the scales to each held maximum
  // Block sum bounds in shared-offset units; -1 (every sum fails it) while
  // the lane's held maxima are more than kSharedSpan apart.
  float t1 = kLazySumMax, t2 = kLazySumMax;
  auto refresh = [&] {  // after an exact update
    const float hb1 = st.m1 * c, hb2 = st.m2 * c;
    hs = 0.5f * (hb1 + hb2);
    w1 = fast_exp2(hs - hb1);
    w2 = fast_exp2(hs - hb2);
    t1 = fast_exp2(kLazyLog2Max + (hb1 - hs));
    t2 = fast_exp2(kLazyLog2Max + (hb2 - hs));
    if (!(fabsf(hb1 - hb2) <= kSharedSpan)) t1 = -1.f;
  };
  auto lazy_update = [&](const f32x16 &x1, const f32x16 &d) {
    float y = __builtin_fmaf(x1[0], c, -hs);
    float s1 = fast_exp2(y);
    float s2 = fast_exp2(__builtin_fmaf(d[0], -c, y));
    float sa = s1 * d[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      y = __builtin_fmaf(x1[r], c, -hs);
      const float e1 = fast_exp2(y);
      const float e2 = fast_exp2(__builtin_fmaf(d[r], -c, y));
      s1 += e1;
      s2 += e2;
      sa = __builtin_fmaf(e1, d[r], sa);
    }
    // The block's sums are formed before the refold test, in the same
    // instruction stream as the next block's products (left to itself the
    // compiler would sink the accumulator chain past the branch, after them).
    float nl1 = __builtin_fmaf(s1, w1, st.l1), nl2 = __builtin_fmaf(s2, w2, st.l2);
    float nacc = __builtin_fmaf(sa, w1, st.acc);
    asm volatile("" : "+v"(nl1), "+v"(nl2), "+v"(nacc));
    if (__builtin_expect(__any(!(s1 <= t1 && s2 <= t2)), 0)) {
      exact(x1, d, 0, std::false_type{});
      refresh();
    } else {
      st.l1 = nl1;
      st.l2 = nl2;
      st.acc = nacc;
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    wait_loads();
  }
  __syncthreads();

  // Step b: logits of block b and the update of block b - 1 (held in p1, p2).
  f32x16 p1 = f32x16{}, p2 = f32x16{};
  auto generic_tile = [&](int t) {
    if (t + 1 < ntiles) load_tile(t + 1);
#pragma unroll
    for (int kb = 0; kb < Tr::BPT; ++kb) {
      const int b = Tr::BPT * t + kb;
      f32x16 n1, n2;
      if (b < nfull && b > 1) {
        scores(b, n1, n2);
        lazy_update(p1, p2);
      } else if (b == 1 && nfull > 1) {
        scores(b, n1, n2);
        exact(p1, p2, k_lo, std::false_type{});
        refresh();
      } else {
        if (b < nlive) scores(b, n1, n2);
        if (b > 0 && b - 1 < nlive) update(b - 1, p1, p2);
      }
      p1 = n1;
      p2 = n2;
    }
    wait_loads();
    lds_barrier();
  };
  // Tiles [1, t_steady) hold only fully visible blocks past the first two: the
  // steady state, without mask code, its one branch the lazy update's rarely
  // taken exact refold.  Its blocks alternate between two register sets (an
  // even number per tile), so no logits are copied from one set to the other.
  const int t_steady = Tr::BPT % 2 == 0 ? nfull / Tr::BPT : 0;
  auto steady_tile = [&](int t) {
    if (t + 1 < ntiles) load_tile(t + 1);
    f32x16 a1, a2;
#pragma unroll
    for (int kb = 0; kb < Tr::BPT; kb += 2) {
      const int b = Tr::BPT * t + kb;
      scores(b, a1, a2);
      lazy_update(p1, p2);
      scores(b + 1, p1, p2);
      lazy_update(a1, a2);
    }
    wait_loads();
    lds_barrier();
  };
  int tile = 0;
  if (ntiles > 0) generic_tile(tile++);
  for (; tile < t_steady; ++tile) steady_tile(tile);
  for (; tile < ntiles; ++tile) generic_tile(tile);
  if (Tr::BPT * ntiles - 1 < nlive && ntiles > 0) update(Tr::BPT * ntiles - 1, p1, p2);

  // Merge the two lane halves that hold disjoint keys of the same query.
  {
    const float m1 = st.m1, m2 = st.m2, l1 = st.l1, l2 = st.l2, acc = st.acc;
    const float om1 = __shfl_xor(m1, 32), ol1 = __shfl_xor(l1, 32);
    const float om2 = __shfl_xor(m2, 32), ol2 = __shfl_xor(l2, 32);
    const float oacc = __shfl_xor(acc, 32);
    const float M1 = fmaxf(m1, om1), M2 = fmaxf(m2, om2);
    const float wa = fast_exp2((m1 - M1) * c), wb = fast_exp2((om1 - M1) * c);
    const float va = fast_exp2((m2 - M2) * c), vb = fast_exp2((om2 - M2) * c);
    const float L1 = __builtin_fmaf(l1, wa, ol1 * wb);
    const float A = __builtin_fmaf(acc, wa, oacc * wb);
    const float L2 = __builtin_fmaf(l2, va, ol2 * vb);
    if (h == 0 && row_ok) {
      if (SPLIT) {
        // Partial states are indexed densely by (unit, row).
        const int64_t rows = p.BH * (int64_t)NQ;
        float *w = p.ws + (int64_t)sp * rows + bh * (int64_t)NQ + row;
        const int64_t fstride = (int64_t)p.splits * rows;
        w[0] = M1;
        w[fstride] = L1;
        w[2 * fstride] = M2;
        w[3 * fstride] = L2;
        w[4 * fstride] = A;
      } else {
        const int64_t idx = rq + row;
        finish_row(M1, L1, M2, L2, A, p.scale, p.kl + idx, p.lse1 + idx, p.lse2 + idx);
      }
    }
  }
}


// ---- bf16 inputs, at most 16 queries per head: 16x16 products ----
//
// One wave per workgroup computes the logits of 16 keys x 16 queries per
// v_mfma_f32_16x16x32_bf16 (A = key rows, B = the resident queries), so no
// product row is spent on absent queries.  Lane l owns query l % 16 and keys
// 4 (l / 16) + i of each 16-key block; the four lane groups holding one query
// merge once at the end.  Every key element is used once, by this wave, so
// the key fragments stream from memory straight into registers (no LDS, no
// barriers): the next 32-key tile loads while this one is multiplied, and
// without an LDS footprint about eight such waves share a CU, each with a
// tile in flight.  The online update folds a whole tile.
template <int D>
struct Fwd16Traits {
  static constexpr int NT = 64;
  static constexpr int BQ = 16;
  static constexpr int BK = 32;
  static constexpr int BPT = BK / 16;  // 16-key blocks per tile
  static constexpr int KSTEPS = D / 32;
  static constexpr int RB = D * 2;
  static_assert(kFwdBK % BK == 0, "tiles");
};

__device__ __forceinline__ f32x4 mma16x16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fold one tile (element i of block j is key kbase + 16 j + 4 g + i) into a
// lane's running state; keys >= klim are masked.
template <bool MASK, int NB>
__device__ __forceinline__ void online_update_tile(const f32x4 (&x1)[NB], const f32x4 (&x2)[NB], RowState &st,
                                                   float c, int kbase, int g, int klim) {
  float mx1 = st.m1, mx2 = st.m2;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!MASK || kbase + 16 * j + 4 * g + i < klim) {
        mx1 = fmaxf(mx1, x1[j][i]);
        mx2 = fmaxf(mx2, x2[j][i]);
      }
  const float a1 = fast_exp2((st.m1 - mx1) * c);
  const float a2 = fast_exp2((st.m2 - mx2) * c);
  st.m1 = mx1;
  st.m2 = mx2;
  const float b1 = mx1 * c, b2 = mx2 * c;
  float s1 = 0.f, s2 = 0.f, sa = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p1 = fast_exp2(__builtin_fmaf(x1[j][i], c, -b1));
      float p2 = fast_exp2(__builtin_fmaf(x2[j][i], c, -b2));
      float d = x1[j][i] - x2[j][i];
      if (MASK) {
        const bool v = kbase + 16 * j + 4 * g + i < klim;
        p1 = v ? p1 : 0.f;
        p2 = v ? p2 : 0.f;
        d = v ? d : 0.f;
      }
      s1 += p1;
      s2 += p2;
      sa = __builtin_fmaf(p1, d, sa);
    }
  st.l1 = __builtin_fmaf(st.l1, a1, s1);
  st.l2 = __builtin_fmaf(st.l2, a2, s2);
  st.acc = __builtin_fmaf(st.acc, a1, sa);
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(64, 1) void fwd16_kernel(FwdParams p) {
  using Tr = Fwd16Traits<D>;
  using Frags = bf16x8[Tr::BPT][Tr::KSTEPS][2];  // one tile's key fragments: block, k-step, tensor

  const int lane = threadIdx.x;
  const int g = lane >> 4, c16 = lane & 15;

  int qt, sp;
  int64_t bh;
  if (SPLIT) {
    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    qt = (int)(L % (uint32_t)p.nqt);
    const uint32_t rest = L / (uint32_t)p.nqt;
    sp = (int)(rest % (uint32_t)p.splits);
    bh = rest / (uint32_t)p.splits;
  } else {
    unsplit_tile(p, blockIdx.x, gridDim.x, bh, qt);
    sp = 0;
  }

  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int64_t rq = p.qmap.row0(bh), rk = p.kmap.row0(bh);
  const bf16 *Q1 = reinterpret_cast<const bf16 *>(p.q1) + rq * D;
  const bf16 *Q2 = reinterpret_cast<const bf16 *>(p.q2) + rq * D;
  const BufRange rk1{reinterpret_cast<const bf16 *>(p.k1) + rk * D, NK * Tr::RB};
  const BufRange rk2{reinterpret_cast<const bf16 *>(p.k2) + rk * D, NK * Tr::RB};

  const int q0 = qt * Tr::BQ;
  const int qend = min(q0 + Tr::BQ, NQ);
  const int kwg_end = p.causal ? min(NK, qend - 1 + off + 1) : NK;
  const int k_lo = SPLIT ? sp * p.chunk : 0;
  const int k_hi = SPLIT ? min(k_lo + p.chunk, kwg_end) : kwg_end;
  const int ntiles = k_hi > k_lo ? (k_hi - k_lo + Tr::BK - 1) / Tr::BK : 0;
  // Tiles [0, nfull) are visible to all the queries, [nfull, nlive) to some.
  const int vis_all = min(k_hi, p.causal ? q0 + off + 1 : NK);
  const int vis_any = min(k_hi, p.causal ? qend - 1 + off + 1 : NK);
  const int nfull = max(0, vis_all - k_lo) / Tr::BK;
  const int nlive = (max(0, vis_any - k_lo) + Tr::BK - 1) / Tr::BK;

  // Resident queries (B operand): lane owns query q0 + c16, elements [32s + 8g, +8).
  const int row = q0 + c16;
  const bool row_ok = row < qend;
  const int klim = min(k_hi, p.causal ? row + off + 1 : NK);
  bf16x8 qf1[Tr::KSTEPS], qf2[Tr::KSTEPS];
#pragma unroll
  for (int s = 0; s < Tr::KSTEPS; ++s) {
    qf1[s] = row_ok ? *reinterpret_cast<const bf16x8 *>(Q1 + (int64_t)row * D + 32 * s + 8 * g) : bf16x8{};
    qf2[s] = row_ok ? *reinterpret_cast<const bf16x8 *>(Q2 + (int64_t)row * D + 32 * s + 8 * g) : bf16x8{};
  }

  const float c = p.scale * kLog2e;
  RowState st{kNegBig, 0.f, kNegBig, 0.f, 0.f, 0.f, 0.f, 0.f};

  // Key fragments of tile t: block j, k-step s, tensor tn holds key
  // 16 j + c16 of the tile, bytes [64 s + 16 g, +16) of its row.
  auto load_tile = [&](int t, Frags &f) {
    const uint32_t soff = (uint32_t)(k_lo + t * Tr::BK) * Tr::RB;
#pragma unroll
    for (int j = 0; j < Tr::BPT; ++j)
#pragma unroll
      for (int s = 0; s < Tr::KSTEPS; ++s) {
        const uint32_t voff = (uint32_t)((16 * j + c16) * Tr::RB + 64 * s + 16 * g);
        f[j][s][0] = __builtin_bit_cast(bf16x8, buffer_load16(rk1, voff, soff));
        f[j][s][1] = __builtin_bit_cast(bf16x8, buffer_load16(rk2, voff, soff));
      }
  };
  // Logits of one tile: block j holds keys 16 j .. 16 j + 15 of the tile.
  auto scores = [&](const Frags &f, f32x4(&s1)[Tr::BPT], f32x4(&s2)[Tr::BPT]) {
#pragma unroll
    for (int j = 0; j < Tr::BPT; ++j) {
      s1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      s2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < Tr::KSTEPS; ++s) {
        s1[j] = mma16x16(f[j][s][0], qf1[s], s1[j]);
        s2[j] = mma16x16(f[j][s][1], qf2[s], s2[j]);
      }
    }
  };
  auto update = [&](int t, const f32x4(&s1)[Tr::BPT], const f32x4(&s2)[Tr::BPT]) {
    const int kbase = k_lo + t * Tr::BK;
    if (t < nfull)
      online_update_tile<false, Tr::BPT>(s1, s2, st, c, kbase, g, 0);
    else
      online_update_tile<true, Tr::BPT>(s1, s2, st, c, kbase, g, klim);
  };

  // Step t: logits of tile t (fragments in `f`) and the update of tile t - 1.
  f32x4 p1[Tr::BPT], p2[Tr::BPT];
#pragma unroll
  for (int j = 0; j < Tr::BPT; ++j) p1[j] = p2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int t, const Frags &f) {
    f32x4 n1[Tr::BPT], n2[Tr::BPT];
    if (t < nfull && t > 0) {
      scores(f, n1, n2);
      online_update_tile<false, Tr::BPT>(p1, p2, st, c, k_lo + (t - 1) * Tr::BK, g, 0);
    } else {
      if (t < nlive) scores(f, n1, n2);
      if (t > 0 && t - 1 < nlive) update(t - 1, p1, p2);
    }
#pragma unroll
    for (int j = 0; j < Tr::BPT; ++j) {
      p1[j] = n1[j];
      p2[j] = n2[j];
    }
  };
  // Two register slots, alternating: tile t + 1 loads while tile t is used.
  Frags fa, fb;
  if (ntiles > 0) load_tile(0, fa);
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) load_tile(t + 1, fb);
    step(t, fa);
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) load_tile(t + 2, fa);
    step(t + 1, fb);
  }
  if (ntiles > 0 && ntiles - 1 < nlive) update(ntiles - 1, p1, p2);

  // Merge the four lane groups that hold disjoint keys of the same query.
  float m1 = st.m1, m2 = st.m2, l1 = st.l1, l2 = st.l2, acc = st.acc;
#pragma unroll
  for (int o = 16; o <= 32; o *= 2) {
    const float om1 = __shfl_xor(m1, o), ol1 = __shfl_xor(l1, o);
    const float om2 = __shfl_xor(m2, o), ol2 = __shfl_xor(l2, o);
    const float oacc = __shfl_xor(acc, o);
    const float M1 = fmaxf(m1, om1), M2 = fmaxf(m2, om2);
    const float wa = fast_exp2((m1 - M1) * c), wb = fast_exp2((om1 - M1) * c);
    const float va = fast_exp2((m2 - M2) * c), vb = fast_exp2((om2 - M2) * c);
    l1 = __builtin_fmaf(l1, wa, ol1 * wb);
    acc = __builtin_fmaf(acc, wa, oacc * wb);
    l2 = __builtin_fmaf(l2, va, ol2 * vb);
    m1 = M1;
    m2 = M2;
  }
  if (g == 0 && row_ok) {
    if (SPLIT) {
      // Partial states are indexed densely by (unit, row).
      const int64_t rows = p.BH * (int64_t)NQ;
      float *w = p.ws + (int64_t)sp * rows + bh * (int64_t)NQ + row;
      const int64_t fstride = (int64_t)p.splits * rows;
      w[0] = m1;
      w[fstride] = l1;
      w[2 * fstride] = m2;
      w[3 * fstride] = l2;
      w[4 * fstride] = acc;
    } else {
      const int64_t idx = rq + row;
      finish_row(m1, l1, m2, l2, acc, p.scale, p.kl + idx, p.lse1 + idx, p.lse2 + idx);
    }
  }
}

template <int D, bool SPLIT>
static hipError_t launch_fwd16(const FwdParams &p, hipStream_t s) {
  using Tr = Fwd16Traits<D>;
  const int64_t nblk = p.BH * (int64_t)p.nqt * p.splits;
  hipLaunchKernelGGL((fwd16_kernel<D, SPLIT>), dim3((uint32_t)nblk), dim3(Tr::NT), 0, s, p);
  return hipGetLastError();
}

// A plain launch passes an empty segment table.
const SegTable kNoSegs{};

template <int D, bool SPLIT, int WAVES, int BK, bool F8 = false>
static hipError_t launch_fwd2_shape(const FwdParams &p, const SegTable &t, hipStream_t s) {
  using Tr = Fwd2Traits<D, WAVES, BK, F8>;
  const void *fn = reinterpret_cast<const void *>(&fwd2_kernel<D, SPLIT, WAVES, BK, F8>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nblk = t.n > 0 ? (int64_t)t.end : p.BH * (int64_t)p.nqt * p.splits;
  hipLaunchKernelGGL((fwd2_kernel<D, SPLIT, WAVES, BK, F8>), dim3((uint32_t)nblk), dim3(Tr::NT), Tr::LDS_BYTES, s,
                     p, t);
  return hipGetLastError();
}

// The grid's query tiles (p.nqt) were sized by fwd_block_queries for the same
// NQ and p.small.  At D = 128 the 8-wave shape stages 128-key tiles (half the
// barriers per key of 64-key tiles: 2-4% faster); at D = 64, where a tile
// carries half the work, 64-key tiles measure faster.  The 4-wave shape
// (128 queries, 64-key tiles, 64 KB of LDS) puts two workgroups on a CU, each
// with its own barriers, and halves the causal diagonal's idle waves; it
// measured 8.5% faster at D = 64 (causal or not) and 2-8% faster for causal
// problems of up to 4096 queries at D = 128, but 2-4% slower for longer or
// non-causal D = 128 problems.  Split-K chunks are whole 128-key tiles, a
// whole number of any of these.
template <int D, bool SPLIT, bool F8 = false>
static hipError_t launch_fwd2(const FwdParams &p, hipStream_t s) {
  static_assert(kFwdChunkTile % 128 == 0, "split chunks must hold whole 128-key tiles");
  if (!F8 && fwd_decode16_shape(0, p.NQ)) return launch_fwd16<D, SPLIT>(p, s);
  if (fwd_decode_shape(F8 ? 2 : 0, p.NQ)) return launch_fwd2_shape<D, SPLIT, 1, 32, F8>(p, kNoSegs, s);
  if (!SPLIT && p.small) return launch_fwd2_shape<D, false, 4, 64, F8>(p, kNoSegs, s);
  return launch_fwd2_shape<D, SPLIT, F8 ? kF8Waves : 8, D == 128 ? 128 : 64, F8>(p, kNoSegs, s);
}

template <typename T, int D, bool SPLIT>
static hipError_t launch_fwd_t(const FwdParams &p, const SegTable &t, hipStream_t s) {
  using Tr = FwdTraits<T, D>;
  const void *fn = reinterpret_cast<const void *>(&fwd_kernel<T, D, SPLIT>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nblk = t.n > 0 ? (int64_t)t.end : p.BH * (int64_t)p.nqt * p.splits;
  hipLaunchKernelGGL((fwd_kernel<T, D, SPLIT>), dim3((uint32_t)nblk), dim3(Tr::NT), Tr::LDS_BYTES, s, p, t);
  return hipGetLastError();
}

int fwd_block_queries(int dtype, int D, int64_t NQ, bool small) {
  if (fwd_decode16_shape(dtype, NQ)) return Fwd16Traits<128>::BQ;
  if (fwd_decode_shape(dtype, NQ)) return Fwd2Traits<128, 1, 32>::BQ;
  if (fwd_mfma_dtype(dtype) && small) return Fwd2Traits<128, 4, 64>::BQ;
  if (dtype == 2) return Fwd2Traits<128, kF8Waves>::BQ;
  if (dtype == 0) return D == 128 ? Fwd2Traits<128>::BQ : Fwd2Traits<64>::BQ;
  return D == 128 ? FwdTraits<float, 128>::BQ : FwdTraits<float, 64>::BQ;
}

bool fwd_small_shape(int dtype, int D, int64_t NQ, bool causal) {
  return fwd_mfma_dtype(dtype) && !fwd_decode_shape(dtype, NQ) && (D == 64 || (causal && NQ <= kFwdSmallCausalRows));
}

hipError_t launch_fwd(int dtype, int D, const FwdParams &p, hipStream_t s) {
  const bool split = p.splits > 1;
  if (dtype == 0) {
    if (D == 128) return split ? launch_fwd2<128, true>(p, s) : launch_fwd2<128, false>(p, s);
    return split ? launch_fwd2<64, true>(p, s) : launch_fwd2<64, false>(p, s);
  }
  if (dtype == 2) {
    if (D == 128) return split ? launch_fwd2<128, true, true>(p, s) : launch_fwd2<128, false, true>(p, s);
    return split ? launch_fwd2<64, true, true>(p, s) : launch_fwd2<64, false, true>(p, s);
  }
  if (D == 128)
    return split ? launch_fwd_t<float, 128, true>(p, kNoSegs, s) : launch_fwd_t<float, 128, false>(p, kNoSegs, s);
  return split ? launch_fwd_t<float, 64, true>(p, kNoSegs, s) : launch_fwd_t<float, 64, false>(p, kNoSegs, s);
}

bool fwd_segment_shape(int dtype, int64_t NQ) { return !fwd_decode_shape(dtype, NQ); }

hipError_t launch_fwd_segs(int dtype, int D, const FwdParams &p, const SegTable &t, hipStream_t s) {
  if (dtype == 0) {
    if (D == 128) return p.small ? launch_fwd2_shape<128, false, 4, 64>(p, t, s) : launch_fwd2_shape<128, false, 8, 128>(p, t, s);
    return p.small ? launch_fwd2_shape<64, false, 4, 64>(p, t, s) : launch_fwd2_shape<64, false, 8, 64>(p, t, s);
  }
  if (dtype == 2) {
    if (D == 128)
      return p.small ? launch_fwd2_shape<128, false, 4, 64, true>(p, t, s)
                     : launch_fwd2_shape<128, false, kF8Waves, 128, true>(p, t, s);
    return p.small ? launch_fwd2_shape<64, false, 4, 64, true>(p, t, s)
                   : launch_fwd2_shape<64, false, kF8Waves, 64, true>(p, t, s);
  }
  if (D == 128) return launch_fwd_t<float, 128, false>(p, t, s);
  return launch_fwd_t<float, 64, false>(p, t, s);
}

// Partial row states of the allocation-free split-K forward.  Each GPU the
// library runs on holds its own copy until the process ends; every call on
// that GPU shares it.  In host code `scratch` names a host-side stand-in,
// never the device array: kernels get the address splitk_scratch looked up.
static __device__ __align__(256) float scratch[kSplitkScratchBytes / sizeof(float)];

hipError_t splitk_scratch(hipStream_t s, float **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float *table[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int cur = dev;
  if (s != nullptr) {
    hipDevice_t d;
    if ((e = hipStreamGetDevice(s, &d)) != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (table[dev] == nullptr) {
    // The lookup runs with the stream's device current.
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    const hipError_t r = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    table[dev] = static_cast<float *>(addr);
  }
  *ptr = table[dev];
  return hipSuccess;
}

hipError_t launch_splitk_merge(const FwdParams &p, hipStream_t s) {
  const int64_t rows = p.BH * p.NQ;
  const int64_t nblk = (rows + 255) / 256;
  hipLaunchKernelGGL(splitk_merge_kernel, dim3((uint32_t)nblk), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace skl
