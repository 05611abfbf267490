// Backward of the fused attention KL divergence by tile-wise recomputation.
//
// StreamKL (arXiv 2606.20005), gist.science "Estrategia de Recomputacion":
// only KL and the two LSE vectors are kept from the forward; attention
// probabilities are rebuilt tile by tile as P_t = exp(s_t - LSE_t).  For
// L = sum_i g_i KL_i the logit gradients are
//     dS2 = g (P2 - P1)                      (student, "Configuracion 1")
//     dS1 = g P1 (log P1 - log P2 - KL)      (teacher, "Configuracion 2")
// with log P1 - log P2 formed from logits and the saved LSEs, never from logs
// of probabilities ("Estabilidad Numerica").  Through s = scale * q.k,
// dQ_t = scale dS_t K_t and dK_t = scale dS_t^T Q_t.
//
// The pages fuse both products into one kernel with dQ atomics and fall back
// to separate kernels under contention.  Here the separate, atomic-free form
// is the design: one pass keeps a tile of keys resident and streams queries
// (dK), the other keeps queries resident and streams keys (dQ).  bf16 and
// fp8 (e4m3) inputs run bwd4_kernel (eight waves, direct LDS staging,
// pipelined stages; fp8 logits on the fp8 matrix instructions); fp32 inputs
// run bwd_fp32_kernel (four waves, register staging of a row-major and a
// transposed fp32 copy of the streamed tile).  At most 128 queries per unit
// (bf16) take the fused single-visit bwd_fused_kernel instead.
//
// Logits come out as (streamed x resident) accumulator blocks, so a lane holds
// one resident row and 16 streamed rows; that accumulator is, element for
// element, the B operand of the gradient product dR^T += X^T dS, which needs
// no shuffle.  bf16 inputs use fp16 for the gradient product: dS in bf16
// loses too much (8-bit significand) for the 2e-3 relative bound, fp16 keeps
// 11 bits.  dS is scaled by a power of two sigma per (sequence, head) with
// max|g| * sigma in [2^7, 2^8) so it sits in fp16's normal range, and the
// streamed operand by a power of two per (sequence, head, tensor) that puts
// its largest entry in [2^14, 2^15); both factors are divided out exactly at
// the end, so no input range overflows fp16.  The prepare step computes them
// (reading g and the inputs once); beyond them the backward keeps nothing in
// device memory but its outputs.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace skl {

// fp32 inputs: four waves, each owning 32 resident rows; the streamed tile is
// staged through registers as a row-major copy (logits product) and a
// transposed copy (gradient product).
template <int D, bool KEYS_RES>
struct BwdF32Traits {
  static constexpr int WAVES = 4;
  static constexpr int BR = kBwdBR;             // resident rows per workgroup
  static constexpr int BX = D == 128 ? 32 : 64;  // streamed rows per stage
  static constexpr int XB = BX / 32;
  static constexpr int KSTEPS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int ROW_BYTES = D * 4;       // one row in HBM
  static constexpr int CPR = ROW_BYTES / 16;    // 16-byte chunks per HBM row
  static constexpr int XROW = ROW_BYTES + 16;
  static constexpr int XT_STRIDE = BX * 4 + 16;
  static constexpr int XROW_BYTES = BX * XROW;
  static constexpr int XT_BYTES = D * XT_STRIDE;
  static constexpr int NSTAT = 4;  // b1, b2, KL, sign(g) of each streamed query
  static constexpr int STAT_BYTES = KEYS_RES ? NSTAT * BX * 4 : 0;
  static constexpr int OFF_XT = 2 * XROW_BYTES;
  static constexpr int OFF_STAT = OFF_XT + 2 * XT_BYTES;
  static constexpr int STAGE_BYTES = OFF_STAT + STAT_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  // Staging work per thread: items of 4 rows x 1 chunk.
  static constexpr int ITEMS = (BX / 4) * CPR;
  static constexpr int IPT = (ITEMS + 255) / 256;
  static_assert(BR == WAVES * 32, "resident tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(XROW_BYTES % 16 == 0 && XT_BYTES % 16 == 0, "LDS alignment");
};

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f16x2 v = {(f16)a, (f16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// Eight bf16 -> eight fp16 (round to nearest even; exact inside the fp16 range).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_f16(bf16lo_to_f32(w[i]), bf16hi_to_f32(w[i]));
  return o;
}

// Exponent offset for rows with g = 0: every exp2 underflows to 0 and the
// log-ratio difference (y1 - y2) stays finite (both offsets equal).
constexpr float kNoGrad = 1.0e30f;

// Per-query constants of the recomputation.  |g| * sigma is folded into the
// exponent offsets, so exp2(x * scale * log2e - b) is already P * |g| * sigma:
//   b_t = LSE_t * log2e - log2(|g| * sigma),  kl = KL,  sg = sign(g).
__device__ __forceinline__ void query_stats(float lse1, float lse2, float kl, float g, float sigma, float &b1,
                                            float &b2, float &klo, float &sg) {
  const float ag = fabsf(g) * sigma;
  sg = g < 0.f ? -1.f : 1.f;
  klo = kl;
  if (ag > 0.f) {
    const float lg = __log2f(ag);
    b1 = __builtin_fmaf(lse1, kLog2e, -lg);
    b2 = __builtin_fmaf(lse2, kLog2e, -lg);
  } else {
    b1 = b2 = kNoGrad;
  }
}

// Head, resident tile and key chunk of workgroup w in a backward pass of n =
// BH * nrt * S workgroups (S key chunks per resident tile, the query-resident
// pass only).  Each XCD runs a contiguous run of logical ids on its own heads.
// Causal resident tiles differ in length (low keys see the most queries, high
// queries the most keys).  By default the run is head-major, heaviest resident
// tiles first, with the chunks of one tile adjacent, so that the workgroups
// running at once share one head's streamed tiles through one L2.  With few
// tiles per head (up to kLongestFirstTiles, unsplit) that order leaves the
// XCD's CUs unevenly loaded at the end; then, when the heads divide evenly
// over the XCDs, the run holds whole heads and goes heaviest tile first across
// all of them.  Measured at 32 resident tiles per head: 5-8% faster.
template <bool KEYS_RES>
__device__ __forceinline__ void resident_tile(const BwdParams &p, int nrt, int S, uint32_t w, uint32_t n,
                                              int64_t &bh, int &rt, int &sp) {
  // Causal tiles differ in work: when the heads do not divide evenly over the
  // XCDs, contiguous runs would give some XCDs only the heavy tiles of a head,
  // so the tiles are dealt round the XCDs in launch order instead (measured
  // 37% faster at 4 heads of 64K, 11% at 12 heads of 32K, and a backward in
  // one-head groups as fast as with every head's copies).
  const uint32_t L = p.causal && p.BH % kXcds != 0 ? w : xcd_remap(w, n);
  if (p.causal && S == 1 && nrt <= kLongestFirstTiles && p.BH % kXcds == 0) {
    const uint32_t hx = (uint32_t)(p.BH / kXcds), per = hx * (uint32_t)nrt;
    const uint32_t i = L % per;
    bh = (int64_t)(L / per) * hx + i % hx;
    const int j = (int)(i / hx);
    rt = KEYS_RES ? j : nrt - 1 - j;
    sp = 0;
  } else {
    const uint32_t per_bh = (uint32_t)nrt * (uint32_t)S;
    bh = L / per_bh;
    const uint32_t jj = L % per_bh;
    rt = KEYS_RES ? (int)jj : nrt - 1 - (int)(jj / (uint32_t)S);
    sp = KEYS_RES ? 0 : (int)(jj % (uint32_t)S);
  }
}

// Workgroup wg of a segmented launch (t.n > 0, no key split): its segment's
// parameters replace the run-dependent ones in p (the per-unit sigma and
// operand scales move to the run's own), and wg, nwg become the
// workgroup's index and count within the segment.  A plain launch (t.n == 0)
// keeps its parameters.
__device__ __forceinline__ void select_segment(BwdParams &p, const SegTable &t, uint32_t &wg, uint32_t &nwg) {
  if (t.n == 0) return;
  const int lo = seg_index(t, wg);
  nwg = seg_count(t, lo);
  wg -= t.seg[lo].start;
  p.BH = t.seg[lo].units;
  p.NQ = t.seg[lo].nq;
  p.NK = t.seg[lo].nk;
  p.qmap.sb = t.seg[lo].nq;
  p.qmap.base = t.seg[lo].oq;
  p.kmap.sb = t.seg[lo].nk;
  p.kmap.base = t.seg[lo].ok;
  p.sigma += t.seg[lo].u0;
  if (p.xscale) p.xscale += 4 * t.seg[lo].u0;
}

template <int D, bool KEYS_RES>
__global__ __launch_bounds__(256, 1) void bwd_fp32_kernel(BwdParams p, const SegTable t) {
  using Tr = BwdF32Traits<D, KEYS_RES>;
  using T = float;
  using CG = f32x8;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;

  uint32_t wg = blockIdx.x, nwg = gridDim.x;
  select_segment(p, t, wg, nwg);
  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int NR = KEYS_RES ? NK : NQ;  // resident row count
  const int NX = KEYS_RES ? NQ : NK;  // streamed row count
  const int nrt = (NR + Tr::BR - 1) / Tr::BR;

  int64_t bh;
  int rt, sp_unused;
  resident_tile<KEYS_RES>(p, nrt, 1, wg, nwg, bh, rt, sp_unused);

  const int64_t rq = p.qmap.row0(bh), rk = p.kmap.row0(bh);
  const int64_t rr = KEYS_RES ? rk : rq, rx = KEYS_RES ? rq : rk;  // resident / streamed row bases
  const T *R1 = reinterpret_cast<const T *>(KEYS_RES ? p.k1 : p.q1) + rr * D;
  const T *R2 = reinterpret_cast<const T *>(KEYS_RES ? p.k2 : p.q2) + rr * D;
  const char *X1 = reinterpret_cast<const char *>(reinterpret_cast<const T *>(KEYS_RES ? p.q1 : p.k1) + rx * D);
  const char *X2 = reinterpret_cast<const char *>(reinterpret_cast<const T *>(KEYS_RES ? p.q2 : p.k2) + rx * D);
  const float *KLr = p.kl + rq;
  const float *LS1 = p.lse1 + rq;
  const float *LS2 = p.lse2 + rq;
  const float *Gr = p.g + rq;
  // Prepared per-head factor; stored negated when some g of the head is negative.
  const float sigma_raw = p.sigma[bh];
  const float sigma = fabsf(sigma_raw);
  const bool any_neg = sigma_raw < 0.f;

  const int r0 = rt * Tr::BR;
  const int rlast_wg = min(r0 + Tr::BR, NR) - 1;
  const int ra = r0 + wave * 32;  // this wave's resident rows [ra, ra + 32)
  const int my_r = ra + c32;      // this lane's resident row
  const bool r_ok = my_r < NR;

  // Streamed range.
  int x_lo = 0, x_hi = NX;
  if (p.causal) {
    if (KEYS_RES) {
      x_lo = max(0, r0 - off);
      x_lo -= x_lo % Tr::BX;
    } else {
      x_hi = min(NK, rlast_wg + off + 1);
    }
  }
  const int ntiles = x_hi > x_lo ? (x_hi - x_lo + Tr::BX - 1) / Tr::BX : 0;
  // Streamed tile t starts at row x_of(t).  The key-resident pass walks the
  // queries downward from the last tile: every workgroup of a head then
  // starts on the same tile and they move through L2 together, whereas their
  // causal starting points differ.
  auto x_of = [&](int t) { return x_lo + (KEYS_RES ? ntiles - 1 - t : t) * Tr::BX; };

  // Resident fragments (B operand of the logits product): lane's row, elements [16s + 8h, +8).
  CG rf1[Tr::KSTEPS], rf2[Tr::KSTEPS];
#pragma unroll
  for (int s = 0; s < Tr::KSTEPS; ++s) {
    rf1[s] = r_ok ? load_chunk<T>(R1 + (int64_t)my_r * D + 16 * s + 8 * h) : CG{};
    rf2[s] = r_ok ? load_chunk<T>(R2 + (int64_t)my_r * D + 16 * s + 8 * h) : CG{};
  }

  const float c = p.scale * kLog2e;
  // Per-query statistics when queries are resident (see query_stats).
  float qb1 = kNoGrad, qb2 = kNoGrad, qkl = 0.f, qsg = 1.f;
  if (!KEYS_RES && r_ok) query_stats(LS1[my_r], LS2[my_r], KLr[my_r], Gr[my_r], sigma, qb1, qb2, qkl, qsg);

  // ---- staging: global -> registers -> LDS ----
  u32x4 st[2][4 * Tr::IPT];
  float sv[Tr::NSTAT];
  auto gload = [&](int t) {
    const int xb0 = x_of(t);
    const u32x4 z = {0u, 0u, 0u, 0u};
    {
#pragma unroll
      for (int k = 0; k < Tr::IPT; ++k) {
        const int item = tid + 256 * k;
        const int cc = item % Tr::CPR, a = item / Tr::CPR;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = xb0 + 4 * a + u;
          const bool ok = (item < Tr::ITEMS) && row < NX;
          const int64_t o = (int64_t)row * Tr::ROW_BYTES + cc * 16;
          st[0][4 * k + u] = ok ? *reinterpret_cast<const u32x4 *>(X1 + o) : z;
          st[1][4 * k + u] = ok ? *reinterpret_cast<const u32x4 *>(X2 + o) : z;
        }
      }
    }
    if (KEYS_RES && tid < Tr::BX) {
      const int q = xb0 + tid;
      sv[0] = sv[1] = kNoGrad;
      sv[2] = 0.f;
      sv[3] = 1.f;
      if (q < NQ) query_stats(LS1[q], LS2[q], KLr[q], Gr[q], sigma, sv[0], sv[1], sv[2], sv[3]);
    }
  };
  auto sstore = [&](int buf) {
    char *base = smem + buf * Tr::STAGE_BYTES;
    {
#pragma unroll
      for (int k = 0; k < Tr::IPT; ++k) {
        const int item = tid + 256 * k;
        if (item >= Tr::ITEMS) continue;
        const int cc = item % Tr::CPR, a = item / Tr::CPR;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          char *xr = base + t2 * Tr::XROW_BYTES;
          char *xt = base + Tr::OFF_XT + t2 * Tr::XT_BYTES;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            *reinterpret_cast<u32x4 *>(xr + (4 * a + u) * Tr::XROW + cc * 16) = st[t2][4 * k + u];
          // 4 fp32 columns d = 4cc + e of rows 4a..4a+3, 16-byte stores.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x4 col = {st[t2][4 * k][e], st[t2][4 * k + 1][e], st[t2][4 * k + 2][e],
                               st[t2][4 * k + 3][e]};
            *reinterpret_cast<u32x4 *>(xt + (4 * cc + e) * Tr::XT_STRIDE + 4 * a * 4) = col;
          }
        }
      }
    }
    if (KEYS_RES && tid < Tr::BX) {
      float *sb = reinterpret_cast<float *>(base + Tr::OFF_STAT);
#pragma unroll
      for (int f = 0; f < Tr::NSTAT; ++f) sb[f * Tr::BX + tid] = sv[f];
    }
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  // Streamed tiles in which every (query, key) pair of the workgroup is
  // visible form one contiguous run [t_a, t_b) in processing order: a ragged
  // last streamed tile (first, in the key-resident pass) and the causal
  // diagonal tiles (last in both passes) lie outside it.  The run is
  // processed without any mask test; the tiles around it test every block.
  int t_a = 0, t_b = 0;
  {
    const int rlast = r0 + Tr::BR - 1;  // all resident rows of the tile, valid or not
    auto tile_full = [&](int t) {
      const int xt = x_of(t), xl = xt + Tr::BX - 1;
      if (KEYS_RES) return xl < NQ && rlast < NK && (!p.causal || rlast <= xt + off);
      return rlast < NQ && xl < NK && (!p.causal || xl <= r0 + off);
    };
    int a = 0;
    while (a < ntiles && !tile_full(a)) ++a;
    int b = a;
    while (b < ntiles && tile_full(b)) ++b;
    t_a = a;
    t_b = b;
  }

  // Everything that accumulates lives in `body`; NEG (key-resident pass, some
  // g of the head negative) multiplies dS by sign(g) of its query row.
  auto body = [&](auto neg_tag) {
    constexpr bool NEG = decltype(neg_tag)::value;
    f32x16 acc1[Tr::NDB], acc2[Tr::NDB];
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
      acc1[db] = f32x16{};
      acc2[db] = f32x16{};
    }

    // One 32-row block of the streamed tile at `base`: logits, dS, gradient products.
    // MASK is false when every (query, key) pair of the block is visible.
    auto block = [&](const char *base, int xb, int xa, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // Logits block: lane = resident row, element r = streamed row xa + acc_row(r, h).
      f32x16 x1 = f32x16{}, x2 = f32x16{};
      {
        const char *a1p = base + (xb * 32 + c32) * Tr::XROW + 8 * h * 4;
        const char *a2p = a1p + Tr::XROW_BYTES;
#pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          const CG a1 = *reinterpret_cast<const CG *>(a1p + 16 * s * 4);
          const CG a2 = *reinterpret_cast<const CG *>(a2p + 16 * s * 4);
          x1 = mma16(a1, rf1[s], x1);
          x2 = mma16(a2, rf2[s], x2);
        }
      }
      // dS, elementwise.
      f32x16 d1, d2;
      const float *sb = reinterpret_cast<const float *>(base + Tr::OFF_STAT);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 B1, B2, KV, SG;
        if (KEYS_RES) {
          const int q = xb * 32 + 8 * j + 4 * h;
          B1 = *reinterpret_cast<const f32x4 *>(sb + 0 * Tr::BX + q);
          B2 = *reinterpret_cast<const f32x4 *>(sb + 1 * Tr::BX + q);
          KV = *reinterpret_cast<const f32x4 *>(sb + 2 * Tr::BX + q);
          if (NEG) SG = *reinterpret_cast<const f32x4 *>(sb + 3 * Tr::BX + q);
        } else {
          B1 = f32x4{qb1, qb1, qb1, qb1};
          B2 = f32x4{qb2, qb2, qb2, qb2};
          KV = f32x4{qkl, qkl, qkl, qkl};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * j + u;
          // p_t = P_t * |g| * sigma; (y1 - y2) * ln 2 = (s1 - LSE1) - (s2 - LSE2).
          const float y1 = __builtin_fmaf(x1[r], c, -B1[u]);
          const float y2 = __builtin_fmaf(x2[r], c, -B2[u]);
          const float p1 = fast_exp2(y1);
          const float p2 = fast_exp2(y2);
          const float dl = __builtin_fmaf(y1 - y2, kLn2, -KV[u]);
          float v2 = p2 - p1;
          float v1 = p1 * dl;
          if (NEG) {
            v1 *= SG[u];
            v2 *= SG[u];
          }
          if (MASK) {
            const int srow = xa + acc_row(r, h);
            const int qi = KEYS_RES ? srow : my_r;
            const int kj = KEYS_RES ? my_r : srow;
            const bool vis = qi < NQ && kj < NK && (!p.causal || kj <= qi + off);
            v1 = vis ? v1 : 0.f;
            v2 = vis ? v2 : 0.f;
          }
          d1[r] = v1;
          d2[r] = v2;
        }
      }
      // Gradient product dR^T[d, resident] += X^T[d, streamed] * dS[streamed, resident].
      // Slot u of lane half h in k-step ks is streamed row 16ks + 8(u/4) + 4h + u%4.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        CG b1, b2;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          b1[u] = d1[8 * ks + u];
          b2[u] = d2[8 * ks + u];
        }
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) {
          CG a1, a2;
          {
            const int so = xb * 32 + 16 * ks + 4 * h;
            const char *t1 = base + Tr::OFF_XT + (db * 32 + c32) * Tr::XT_STRIDE + so * 4;
            const char *t2 = t1 + Tr::XT_BYTES;
            const f32x4 l1 = *reinterpret_cast<const f32x4 *>(t1);
            const f32x4 h1 = *reinterpret_cast<const f32x4 *>(t1 + 32);
            const f32x4 l2 = *reinterpret_cast<const f32x4 *>(t2);
            const f32x4 h2 = *reinterpret_cast<const f32x4 *>(t2 + 32);
            a1 = __builtin_shufflevector(l1, h1, 0, 1, 2, 3, 4, 5, 6, 7);
            a2 = __builtin_shufflevector(l2, h2, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          acc1[db] = mma16(a1, b1, acc1[db]);
          acc2[db] = mma16(a2, b2, acc2[db]);
        }
      }
    };

    auto run_tiles = [&](int t0, int t1, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      for (int t = t0; t < t1; ++t) {
        if (t + 1 < ntiles) gload(t + 1);
        const char *base = smem + (t & 1) * Tr::STAGE_BYTES;
#pragma unroll
        for (int xb = 0; xb < Tr::XB; ++xb) {
          const int xa = x_of(t) + xb * 32;  // streamed rows [xa, xa + 32)
          if (!MASK) {
            block(base, xb, xa, std::false_type{});
            continue;
          }
          bool empty;
          if (KEYS_RES)  // resident keys j, streamed queries i
            empty = xa >= NQ || ra >= NK || (p.causal && ra > xa + 31 + off);
          else  // resident queries i, streamed keys j
            empty = ra >= NQ || xa >= NK || (p.causal && xa > ra + 31 + off);
          if (!empty) block(base, xb, xa, std::true_type{});
        }
        if (t + 1 < ntiles) sstore((t + 1) & 1);
        __syncthreads();
      }
    };
    run_tiles(0, t_a, std::true_type{});
    run_tiles(t_a, t_b, std::false_type{});
    run_tiles(t_b, ntiles, std::true_type{});

    // Epilogue: lane writes its resident row, d = db*32 + 8j + 4h + (0..3).
    if (r_ok) {
      const float f = p.scale / sigma * (KEYS_RES ? 1.f : qsg);
      float *O1 = KEYS_RES ? p.dk1 : p.dq1;
      float *O2 = KEYS_RES ? p.dk2 : p.dq2;
      const int64_t rowoff = (rr + my_r) * D;
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + 8 * j + 4 * h;
          if (p.want1) {
            const f32x4 v = {acc1[db][4 * j] * f, acc1[db][4 * j + 1] * f, acc1[db][4 * j + 2] * f,
                             acc1[db][4 * j + 3] * f};
            *reinterpret_cast<f32x4 *>(O1 + rowoff + d) = v;
          }
          if (p.want2) {
            const f32x4 v = {acc2[db][4 * j] * f, acc2[db][4 * j + 1] * f, acc2[db][4 * j + 2] * f,
                             acc2[db][4 * j + 3] * f};
            *reinterpret_cast<f32x4 *>(O2 + rowoff + d) = v;
          }
        }
      }
    }
  };
  if (KEYS_RES && any_neg)
    body(std::true_type{});
  else
    body(std::false_type{});
}

// ---- bf16 inputs: two waves per SIMD, software-pipelined stages ----
//
// Eight waves.  Waves p and p + 4 (one SIMD) form a pair that shares 32
// resident rows; per 64-row streamed stage, wave p + 4e computes the logits
// and dS of streamed block e (rows 32e..32e+31) for both distributions and
// accumulates the gradient of distribution e (teacher for e = 0, student for
// e = 1) over both blocks, for all of D.  The dS of the other distribution is
// posted to LDS for the partner.  Per wave this keeps 64 accumulator
// registers, and the exchange is one fp16 operand pair per wave and stage.
//
// A single wave per SIMD serialises matrix and vector work; two waves running
// the same phases do too.  So each wave's stream is pipelined by one stage:
// after the logits of stage t, the gradient products of stage t - 1 (whose dS
// is complete) are independent of the dS arithmetic of stage t, and the two
// are interleaved in one instruction stream.
//
// The streamed operand reaches LDS once, as its original bf16 rows, through
// global_load_lds (no staging registers, no LDS write instructions) into an
// XOR-swizzled layout; the logits product reads it 16 bytes per lane (exact
// products, as in the forward).  The gradient product needs the same tile
// transposed (contraction over the streamed rows) and in fp16.  The four
// waves that multiply a 32-row block already hold its bf16 fragments in
// registers for the logits, so they also transpose it: one product against a
// one-hot operand (times the tensor's power-of-two scale) yields, in the
// accumulator layout, exactly the lane-ordered A operand of the gradient
// product, which is rounded to fp16 and written to LDS for every wave that
// needs it.  That costs two 32x32x16 products per 32x32 block and replaces a
// transposed copy of every input in device memory.
//
// fp8 (e4m3) inputs take the same passes with D-byte rows: the logits run on
// v_mfma_f32_32x32x64_f8f6f4 (a lane supplies 32 bytes of its row per
// 64-element k-step), and the transposing product takes one such k-step
// against a one-hot e4m3 operand per 32-column block.  Every e4m3 value is an
// fp16 value, so the fp16 transposed tiles are exact without a scale.
template <int D, bool KEYS_RES, bool F8_ = false>
struct Bwd4Traits {
  static constexpr bool F8 = F8_;
  static constexpr int NT = 512;
  static constexpr int BR = kBwdBR;         // resident rows per workgroup: 4 pairs x 32
  static constexpr int BX = kBwdTile;       // streamed rows per stage
  static constexpr int KSTEPS = F8 ? D / 64 : D / 16;
  static constexpr int NDB = D / 32;        // 32-column gradient blocks
  static constexpr int RB = F8 ? D : D * 2; // row bytes
  static constexpr int CPROW = RB / 16;     // 16-byte chunks per row
  static constexpr int ROW_T = BX * RB;     // one tensor's row tile
  static constexpr int SLOT = 64 * 16;      // one lane-ordered 16-byte operand
  // One stage's transposed tiles, lane-ordered fp16 operands
  // [distribution][streamed block][32-column block][k-step][lane].
  static constexpr int TRB = 2 * 2 * NDB * 2 * SLOT;
  static constexpr int DSX_T = 8 * 2 * SLOT;  // one stage's posted dS: [wave][ks]
  static constexpr int STAT_T = 1024;       // b1, b2, KL (fp32) and sign (16 bit) of 64 queries
  static constexpr int REST = 2 * TRB + 2 * DSX_T + (KEYS_RES ? 2 * STAT_T : 0);
  // Two row-tile buffers when they fit (one barrier per stage), else one
  // (a second barrier per stage releases it for the next tile).
  static constexpr int ROWBUF = 4 * ROW_T + REST <= 160 * 1024 ? 2 : 1;
  static constexpr int OFF_TR = ROWBUF * 2 * ROW_T;  // two buffers of TRB
  static constexpr int OFF_DSX = OFF_TR + 2 * TRB;   // two buffers
  static constexpr int OFF_STAT = OFF_DSX + 2 * DSX_T;
  // With one row buffer (spare LDS), and for fp8 inputs, the one-hot
  // operands of the transposing products live in LDS rather than registers:
  // [distribution][half][lane] (bf16), [32-column block parity][lane][32 B] (fp8).
  static constexpr int ID_BYTES = (ROWBUF == 1 || F8) ? 2 * 2 * SLOT : 0;
  static constexpr int OFF_ID = OFF_STAT + (KEYS_RES ? 2 * STAT_T : 0);
  static constexpr int LDS_BYTES = OFF_ID + ID_BYTES;
  static constexpr int ROW_LOADS = 2 * ROW_T / 16 / NT;  // 16-byte loads per thread per stage
  static_assert(BR == 4 * 32 && BX == 64, "tiles");
  static_assert(ROW_LOADS * 16 * NT == 2 * ROW_T, "load split");
  static_assert(ROW_T % (16 * 64) == 0, "one tensor per wave and load instruction");
  static_assert((2 * TRB + 2 * DSX_T) % (16 * NT) == 0, "clear split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// One-hot B operand of the transposing product for 16-column half j of a
// 32-column block: x[32 rows][16 k] * I gives a 32 x 32 block whose column c
// is x's column c - 16 j for c in [16 j, 16 j + 16) and zero elsewhere, times
// v.  Lane (h, c) supplies k = 8 h + u, nonzero where 16 j + 8 h + u == c.
__device__ __forceinline__ bf16x8 onehot(int c, int h, int j, float v) {
  const int u = c - 16 * j - 8 * h;
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)(i == u ? v : 0.f);
  return r;
}

// MODE 0 computes both distributions' gradients; MODE 1 only the teacher's
// (Configuration 2), MODE 2 only the student's (Configuration 1).  With one
// distribution the pair splits D instead: each wave accumulates its half of
// D over both blocks, and the dS that is not needed is never formed.
template <int D, bool KEYS_RES, int MODE, bool F8>
__global__ __launch_bounds__(512, 1) void bwd4_kernel(BwdParams p, const SegTable t) {
  using Tr = Bwd4Traits<D, KEYS_RES, F8>;
  using Frag = typename std::conditional<F8, i32x8, bf16x8>::type;  // one k-step of a lane's row
  constexpr int FB = (int)sizeof(Frag);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int pr = wave & 3;  // pair: resident rows
  const int e_rt = wave >> 2;  // streamed block for dS; distribution whose gradient this wave accumulates
  const int h = lane >> 5, c32 = lane & 31;

  uint32_t wg = blockIdx.x, nwg = gridDim.x;
  select_segment(p, t, wg, nwg);
  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int NR = KEYS_RES ? NK : NQ;
  const int NX = KEYS_RES ? NQ : NK;
  const int nrt = (NR + Tr::BR - 1) / Tr::BR;

  const int S = KEYS_RES ? 1 : p.splits;
  int64_t bh;
  int rt, sp;
  resident_tile<KEYS_RES>(p, nrt, S, wg, nwg, bh, rt, sp);

  const int64_t rq = p.qmap.row0(bh), rk = p.kmap.row0(bh);
  const int64_t rr = KEYS_RES ? rk : rq, rx = KEYS_RES ? rq : rk;  // resident / streamed row bases
  const char *R1 = reinterpret_cast<const char *>(KEYS_RES ? p.k1 : p.q1) + rr * Tr::RB;
  const char *R2 = reinterpret_cast<const char *>(KEYS_RES ? p.k2 : p.q2) + rr * Tr::RB;
  const char *X1 = reinterpret_cast<const char *>(KEYS_RES ? p.q1 : p.k1) + rx * Tr::RB;
  const char *X2 = reinterpret_cast<const char *>(KEYS_RES ? p.q2 : p.k2) + rx * Tr::RB;
  const float *KLr = p.kl + rq;
  const float *LS1 = p.lse1 + rq;
  const float *LS2 = p.lse2 + rq;
  const float *Gr = p.g + rq;
  const float sigma_raw = p.sigma[bh];
  const float sigma = fabsf(sigma_raw);
  const bool any_neg = sigma_raw < 0.f;
  // Power-of-two scales of the streamed tensors' fp16 operands (teacher, student).
  const float xs[2] = {p.xscale[bh * 4 + (KEYS_RES ? 0 : 2)], p.xscale[bh * 4 + (KEYS_RES ? 1 : 3)]};

  const int r0 = rt * Tr::BR;
  const int rlast_wg = min(r0 + Tr::BR, NR) - 1;
  const int ra = r0 + pr * 32;
  const int my_r = ra + c32;
  const bool r_ok = my_r < NR;

  int x_lo = 0, x_hi = NX;
  if (p.causal) {
    if (KEYS_RES) {
      x_lo = max(0, r0 - off);
      x_lo -= x_lo % Tr::BX;
    } else {
      x_hi = min(NK, rlast_wg + off + 1);
    }
  }
  if (S > 1) {  // this workgroup's key chunk (chunks are whole 64-key tiles)
    x_lo = max(x_lo, sp * p.kchunk);
    x_hi = min(x_hi, (sp + 1) * p.kchunk);
  }
  const int ntiles = x_hi > x_lo ? (x_hi - x_lo + Tr::BX - 1) / Tr::BX : 0;
  // Streamed tiles start at multiples of 64 rows; the key-resident pass walks
  // them downward so that all workgroups of a head share their first tiles.
  auto x_of = [&](int t) { return x_lo + (KEYS_RES ? ntiles - 1 - t : t) * Tr::BX; };

  // Resident fragments (B operand of the logits product): lane's row, k-step
  // s in bytes [FB (2 s + h), + FB), FB = 16 (bf16) or 32 (fp8).
  Frag rf1[Tr::KSTEPS], rf2[Tr::KSTEPS];
#pragma unroll
  for (int s = 0; s < Tr::KSTEPS; ++s) {
    rf1[s] = r_ok ? *reinterpret_cast<const Frag *>(R1 + (int64_t)my_r * Tr::RB + FB * (2 * s + h)) : Frag{};
    rf2[s] = r_ok ? *reinterpret_cast<const Frag *>(R2 + (int64_t)my_r * Tr::RB + FB * (2 * s + h)) : Frag{};
  }

  const float c = p.scale * kLog2e;
  float qb1 = kNoGrad, qb2 = kNoGrad, qkl = 0.f, qsg = 1.f;
  if (!KEYS_RES && r_ok) query_stats(LS1[my_r], LS2[my_r], KLr[my_r], Gr[my_r], sigma, qb1, qb2, qkl, qsg);

  // ---- staging: global -> LDS without registers ----
  // Buffer resources over this head's streamed rows: 32-bit offsets, and rows
  // past the end of the streamed operand read as zero (they only feed masked
  // pairs, and transpose to zero columns).
  const BufRange rx1{X1, NX * Tr::RB}, rx2{X2, NX * Tr::RB};
  // Per-lane source offsets within a tile: load i of the stage moves chunk
  // C = i NT + tid of the two tensors' tiles, tensor-major (tensor C / CT),
  // row r at r * RB, logical chunk c in slot c ^ swz_bytes(r).  A wave's 64
  // chunks lie in one tensor.
  constexpr int RL = Tr::ROW_LOADS;
  constexpr int CT = Tr::ROW_T / 16;                   // chunks per tensor tile
  constexpr int VL = CT >= Tr::NT ? CT / Tr::NT : 1;  // distinct offsets (load i uses i % VL)
  static_assert(CT % Tr::NT == 0 || Tr::NT % CT == 0, "load split");
  uint32_t vrow[VL];
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    const int C = (i * Tr::NT + tid) % CT;
    const int row = C / Tr::CPROW;
    vrow[i] = row * Tr::RB + ((C % Tr::CPROW) ^ swz_bytes<Tr::RB>(row)) * 16;
  }
  auto load_rows = [&](int t, int buf) {
    const uint32_t soff = (uint32_t)x_of(t) * Tr::RB;
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      const int C0 = i * Tr::NT + wave * 64;  // the wave's first chunk
      buffer_load_lds16(C0 >= CT ? rx2 : rx1, smem + buf * 2 * Tr::ROW_T + C0 * 16, vrow[i % VL], soff);
    }
  };
  // Key-resident pass: statistics of the 64 streamed queries of a stage,
  // gathered by the first wave into stat buffer `buf`.
  float sl1 = 0.f, sl2 = 0.f, skl_ = 0.f, sg_ = 0.f;
  auto stats_load = [&](int t) {
    if (KEYS_RES && tid < Tr::BX) {
      const int q = x_of(t) + tid;
      if (q < NQ) {
        sl1 = LS1[q];
        sl2 = LS2[q];
        skl_ = KLr[q];
        sg_ = Gr[q];
      }
    }
  };
  auto stats_store = [&](int t, int buf) {
    if (KEYS_RES && tid < Tr::BX) {
      float b1 = kNoGrad, b2 = kNoGrad, kv = 0.f, sg = 1.f;
      if (x_of(t) + tid < NQ) query_stats(sl1, sl2, skl_, sg_, sigma, b1, b2, kv, sg);
      float *sb = reinterpret_cast<float *>(smem + Tr::OFF_STAT + buf * Tr::STAT_T);
      sb[tid] = b1;
      sb[Tr::BX + tid] = b2;
      sb[2 * Tr::BX + tid] = kv;
      reinterpret_cast<uint16_t *>(sb + 3 * Tr::BX)[tid] = sg < 0.f ? 0x8000u : 0u;
    }
  };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // Workgroup barrier that waits for this wave's LDS operations but leaves
  // global loads in flight (the direct LDS loads are waited for explicitly).
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // The pipeline's first step multiplies the second transposed buffer and the
  // second dS buffer by zero operands: clear them so that they hold no NaN.
  {
    constexpr int NCLR = (2 * Tr::TRB + 2 * Tr::DSX_T) / 16 / Tr::NT;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NCLR; ++i) *reinterpret_cast<u32x4 *>(smem + Tr::OFF_TR + (i * Tr::NT + tid) * 16) = z;
  }
  if (ntiles > 0) {
    load_rows(0, 0);
    stats_load(0);
    stats_store(0, 0);
    wait_loads();
  }
  __syncthreads();

  int t_a = 0, t_b = 0;
  {
    const int rlast = r0 + Tr::BR - 1;
    auto tile_full = [&](int t) {
      const int xt = x_of(t), xl = xt + Tr::BX - 1;
      if (KEYS_RES) return xl < NQ && rlast < NK && (!p.causal || rlast <= xt + off);
      return rlast < NQ && xl < NK && (!p.causal || xl <= r0 + off);
    };
    int a = 0;
    while (a < ntiles && !tile_full(a)) ++a;
    int b = a;
    while (b < ntiles && tile_full(b)) ++b;
    t_a = a;
    t_b = b;
  }

  // One-hot operands of the transposing products, per distribution, scaled by
  // the streamed tensor's power of two (exact in bf16): in registers, or in
  // the LDS table.  Every wave writes the table's lane entries it reads, all
  // with the same values, so no barrier orders the writes before the reads.
  bf16x8 id0[2], id1[2];
  if constexpr (F8) {
    // fp8: for 32-column block parity v, lane (h, c) holds e4m3 1.0 at byte c
    // when h == v (element 32 v + c of the 64-element k-step), zeros elsewhere.
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      u32x4 w[2];
#pragma unroll
      for (int dw = 0; dw < 8; ++dw)
        w[dw >> 2][dw & 3] = h == v && (c32 >> 2) == dw ? 0x38u << (8 * (c32 & 3)) : 0u;
      char *idp = smem + Tr::OFF_ID + v * 2 * Tr::SLOT + lane * 32;
      *reinterpret_cast<u32x4 *>(idp) = w[0];
      *reinterpret_cast<u32x4 *>(idp + 16) = w[1];
    }
  } else {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      id0[t2] = onehot(c32, h, 0, xs[t2]);
      id1[t2] = onehot(c32, h, 1, xs[t2]);
      if (Tr::ID_BYTES) {
        char *idp = smem + Tr::OFF_ID + t2 * 2 * Tr::SLOT + lane * 16;
        *reinterpret_cast<bf16x8 *>(idp) = id0[t2];
        *reinterpret_cast<bf16x8 *>(idp + Tr::SLOT) = id1[t2];
      }
    }
  }

  // Specialised per wave role and, in the key-resident pass, per presence of
  // negative upstream gradients in the head (branch-free stage bodies).
  auto body = [&](auto e_tag, auto neg_tag) {
    constexpr int e = decltype(e_tag)::value;
    constexpr bool NEG = decltype(neg_tag)::value;
    constexpr int NACC = MODE == 0 ? Tr::NDB : Tr::NDB / 2;  // 32-column accumulator blocks
    constexpr int TEN = MODE == 0 ? e : MODE - 1;            // distribution accumulated
    constexpr int DB0 = MODE == 0 ? 0 : e * NACC;            // first 32-column block
    f32x16 acc[NACC];
  #pragma unroll
    for (int db = 0; db < NACC; ++db) acc[db] = f32x16{};

    auto empty_blk = [&](int xa) -> bool {
      if (KEYS_RES) return xa >= NQ || ra >= NK || (p.causal && ra > xa + 31 + off);
      return ra >= NQ || xa >= NK || (p.causal && xa > ra + 31 + off);
    };
    // Logits of streamed block e of the row tile at `rowb`.
    auto logits = [&](const char *rowb, f32x16 &x1, f32x16 &x2) {
      const int row = e * 32 + c32;
      const int sw = swz_bytes<Tr::RB>(row);
      const char *a1p = rowb + row * Tr::RB;
      const char *a2p = a1p + Tr::ROW_T;
      x1 = f32x16{};
      x2 = f32x16{};
      if constexpr (F8) {
        // Two k-steps of 64: all eight operand reads, then the four products.
        i32x8 a1[Tr::KSTEPS], a2[Tr::KSTEPS];
  #pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          const int pa = ((4 * s + 2 * h) ^ sw) * 16, pb = ((4 * s + 2 * h + 1) ^ sw) * 16;
          a1[s] = join16(*reinterpret_cast<const u32x4 *>(a1p + pa), *reinterpret_cast<const u32x4 *>(a1p + pb));
          a2[s] = join16(*reinterpret_cast<const u32x4 *>(a2p + pa), *reinterpret_cast<const u32x4 *>(a2p + pb));
        }
  #pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          x1 = mma_f8(a1[s], rf1[s], x1);
          x2 = mma_f8(a2[s], rf2[s], x2);
        }
      } else {
        bf16x8 a1[Tr::KSTEPS], a2[Tr::KSTEPS];
  #pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          const int pc = ((2 * s + h) ^ sw) * 16;
          a1[s] = *reinterpret_cast<const bf16x8 *>(a1p + pc);
          a2[s] = *reinterpret_cast<const bf16x8 *>(a2p + pc);
        }
  #pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          x1 = mma16(a1[s], rf1[s], x1);
          x2 = mma16(a2[s], rf2[s], x2);
        }
        // Keep four k-steps of operand reads in flight ahead of the products.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  #pragma unroll
        for (int s = 0; s < Tr::KSTEPS - 4; ++s) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
    };
    // dS of the own block (rows xa..xa+31) as gradient-product B operands:
    // mine[ks] for this wave's distribution, other[ks] for the partner's.
    auto dsblock = [&](const f32x16 &x1, const f32x16 &x2, int xa, const float *sb, auto mask_tag, f16x8(&mine)[2],
                       f16x8(&other)[2]) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // Visibility in masked blocks: element r is streamed row xa + 4h + cr(r),
      // cr(r) = 8(r/4) + r%4, and visible exactly when lo <= cr(r) < hi.
      int lo = 0, hi = 0;
      if (MASK) {
        const int base = xa + 4 * h;
        if (KEYS_RES) {  // streamed query q, resident key my_r: q < NQ, my_r < NK, my_r <= q + off
          hi = NQ - base;
          lo = !r_ok ? 1 << 30 : (p.causal ? my_r - off - base : -(1 << 30));
        } else {  // resident query my_r, streamed key k: my_r < NQ, k < NK, k <= my_r + off
          hi = min(NK - base, p.causal ? my_r + off - base + 1 : 1 << 30);
          lo = r_ok ? -(1 << 30) : 1 << 30;
        }
      }
      f16x8 b1[2], b2[2];
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 B1, B2, KV;
        if (KEYS_RES) {
          const int q = e * 32 + 8 * j + 4 * h;
          B1 = *reinterpret_cast<const f32x4 *>(sb + q);
          B2 = *reinterpret_cast<const f32x4 *>(sb + Tr::BX + q);
          KV = *reinterpret_cast<const f32x4 *>(sb + 2 * Tr::BX + q);
        } else {
          B1 = f32x4{qb1, qb1, qb1, qb1};
          B2 = f32x4{qb2, qb2, qb2, qb2};
          KV = f32x4{qkl, qkl, qkl, qkl};
        }
  #pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * j + u;
          const float y1 = __builtin_fmaf(x1[r], c, -B1[u]);
          const float y2 = __builtin_fmaf(x2[r], c, -B2[u]);
          const float p1 = fast_exp2(y1);
          const float p2 = fast_exp2(y2);
          const float dl = __builtin_fmaf(y1 - y2, kLn2, -KV[u]);
          float v2 = p2 - p1;
          float v1 = p1 * dl;
          if (MASK) {
            const int cr = 8 * (r >> 2) + (r & 3);
            const bool vis = cr >= lo && cr < hi;
            v1 = vis ? v1 : 0.f;
            v2 = vis ? v2 : 0.f;
          }
          b1[r >> 3][r & 7] = (f16)v1;
          b2[r >> 3][r & 7] = (f16)v2;
        }
      }
      // Key-resident pass with some g < 0: dS of query q carries sign(g_q).
      // Slot pair (2m, 2m+1) of k-step ks holds queries 16ks + 4h + {0,2,8,10}[m] + (0, 1).
      if (KEYS_RES && NEG) {
        const char *sgp = reinterpret_cast<const char *>(sb + 3 * Tr::BX) + (e * 32 + 4 * h) * 2;
  #pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint2 lo2 = *reinterpret_cast<const uint2 *>(sgp + 32 * ks);
          const uint2 hi2 = *reinterpret_cast<const uint2 *>(sgp + 32 * ks + 16);
          const u32x4 m = {lo2.x, lo2.y, hi2.x, hi2.y};
          b1[ks] = __builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, b1[ks]) ^ m);
          b2[ks] = __builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, b2[ks]) ^ m);
        }
      }
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (MODE == 0) {
          mine[ks] = e ? b2[ks] : b1[ks];
          other[ks] = e ? b1[ks] : b2[ks];
        } else {
          mine[ks] = other[ks] = MODE == 1 ? b1[ks] : b2[ks];
        }
      }
    };
    // This wave's share of the transposition of streamed block e of the row
    // tile into the lane-ordered fp16 tiles of its stage.  For each
    // (distribution t, 32-column block db) it owns, two products against the
    // one-hot operands give a 32x32 accumulator whose element r in lane
    // (h, c) is row acc_row(r, h) of the block, column 32 db + c, times the
    // tensor's scale: elements 8 ks .. 8 ks + 7 are exactly that lane's A
    // operand of the gradient product's k-step ks, stored at [t][e][db][ks].
    // Every wave of a block takes part whether or not its own rows see it:
    // the other waves' products read the whole tile.
    constexpr int NTR = MODE == 0 ? 2 : 1;      // distributions transposed
    constexpr int PER = NTR * Tr::NDB;          // (t, db) pairs per block, dealt over the 4 waves
    constexpr int NC = (PER + 3) / 4;           // pairs per wave (none for pr >= PER when PER < 4)
    auto tr_pair = [&](int k, int &t, int &db) {
      t = MODE != 0 ? TEN : (Tr::NDB == 4 ? k : pr >> 1);
      db = (Tr::NDB == 4 || MODE != 0) ? pr : (pr & 1);
    };
    // The products, from the row tile at `rowb`.
    auto tr_issue = [&](const char *rowb, f32x16(&T)[NC]) {
      const int row = e * 32 + c32;
      const int sw = swz_bytes<Tr::RB>(row);
  #pragma unroll
      for (int k = 0; k < NC; ++k) {
        if (PER < 4 && pr >= PER) {
          T[k] = f32x16{};
          continue;
        }
        int t, db;
        tr_pair(k, t, db);
        const char *src = rowb + t * Tr::ROW_T + row * Tr::RB;
        if constexpr (F8) {
          // The k-step holding block db (elements 64 (db / 2) ..), against the
          // one-hot operand of db's parity.
          const int c0 = 4 * (db >> 1) + 2 * h;
          const i32x8 a = join16(*reinterpret_cast<const u32x4 *>(src + (c0 ^ sw) * 16),
                                 *reinterpret_cast<const u32x4 *>(src + ((c0 + 1) ^ sw) * 16));
          const i32x8 id = *reinterpret_cast<const i32x8 *>(smem + Tr::OFF_ID + (db & 1) * 2 * Tr::SLOT + lane * 32);
          T[k] = mma_f8(a, id, f32x16{});
          continue;
        }
        const bf16x8 lo = *reinterpret_cast<const bf16x8 *>(src + ((4 * db + h) ^ sw) * 16);
        const bf16x8 hi = *reinterpret_cast<const bf16x8 *>(src + ((4 * db + 2 + h) ^ sw) * 16);
        bf16x8 i0, i1;
        if (Tr::ID_BYTES) {
          const char *idp = smem + Tr::OFF_ID + t * 2 * Tr::SLOT + lane * 16;
          i0 = *reinterpret_cast<const bf16x8 *>(idp);
          i1 = *reinterpret_cast<const bf16x8 *>(idp + Tr::SLOT);
        } else {
          i0 = t ? id0[1] : id0[0];
          i1 = t ? id1[1] : id1[0];
        }
        T[k] = mma16(lo, i0, f32x16{});
        T[k] = mma16(hi, i1, T[k]);
      }
    };
    // fp16 rounding and the lane-ordered stores.
    auto tr_store = [&](const f32x16(&T)[NC], char *trw) {
  #pragma unroll
      for (int k = 0; k < NC; ++k) {
        if (PER < 4 && pr >= PER) break;
        int t, db;
        tr_pair(k, t, db);
        f16x8 o[2];
  #pragma unroll
        for (int r = 0; r < 16; ++r) o[r >> 3][r & 7] = (f16)T[k][r];
        char *dst = trw + ((t * 2 + e) * Tr::NDB + db) * 2 * Tr::SLOT + lane * 16;
        *reinterpret_cast<f16x8 *>(dst) = o[0];
        *reinterpret_cast<f16x8 *>(dst + Tr::SLOT) = o[1];
      }
    };
    // Gradient product of this wave's distribution over streamed block xb of
    // the transposed tiles at `trb`: dR^T[d, resident] += X^T[d, streamed] * dS.
    // The transposed operand of k-step ks is stored in the dS operands' slot
    // order (the accumulator layout), one 16-byte operand per lane.
    auto grad = [&](int xb, const char *trb, const f16x8(&bo)[2]) {
      const char *tb = trb + ((TEN * 2 + xb) * Tr::NDB + DB0) * 2 * Tr::SLOT + lane * 16;
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
  #pragma unroll
        for (int db = 0; db < NACC; ++db) {
          const f16x8 a = *reinterpret_cast<const f16x8 *>(tb + (db * 2 + ks) * Tr::SLOT);
          acc[db] = mma16(a, bo[ks], acc[db]);
        }
      }
    };

    // Both blocks of a stage, own dS from registers and the partner's from LDS,
    // block TEN first: every distribution's accumulation order is the same in
    // every mode, so results do not depend on which gradients are requested.
    auto grad2 = [&](const char *trp, const f16x8(&own)[2], const f16x8(&par)[2]) {
      if (e == TEN) {
        grad(e, trp, own);
        grad(1 - e, trp, par);
      } else {
        grad(1 - e, trp, par);
        grad(e, trp, own);
      }
    };

    // Stage t: with two row buffers the next row tile starts loading; logits
    // of stage t; with one row buffer this wave's share of the stage's
    // transposition, a barrier (row tile free) and then the next row tile
    // starts loading; dS of stage t interleaved with the gradient products of
    // stage t - 1; with two row buffers the transposition; the partner's dS
    // posted; all loads land; barrier.
    f16x8 prev[2] = {f16x8{}, f16x8{}};  // own block's dS (this wave's distribution) of stage t - 1
    auto run_tiles = [&](int t0, int t1, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      for (int t = t0; t < t1; ++t) {
        const bool more = t + 1 < ntiles;
        const int xt = x_of(t);
        const bool own_live = !MASK || !empty_blk(xt + 32 * e);
        const float *sb = reinterpret_cast<const float *>(smem + Tr::OFF_STAT + (t & 1) * Tr::STAT_T);
        if (Tr::ROWBUF == 2 && more) load_rows(t + 1, (t + 1) & 1);
        if (more) stats_load(t + 1);
        f32x16 x1, x2;
        const char *rowb = smem + (Tr::ROWBUF == 2 ? (t & 1) * 2 * Tr::ROW_T : 0);
        // With one row buffer the transposition reads the row tile with the
        // logits and stores after the barrier that frees that buffer, so that
        // the products' latency overlaps the dS arithmetic.  With two it runs
        // after the stage's gradient products (the tile stays valid all
        // stage): the logits phase, which has no vector work beside it, is
        // then shorter (1.5% faster dQ pass at causal 64K).
        f32x16 T[NC];
        if (own_live) logits(rowb, x1, x2);
        if (Tr::ROWBUF == 1) {
          tr_issue(rowb, T);
          lds_barrier();
          if (more) load_rows(t + 1, 0);
          tr_store(T, smem + Tr::OFF_TR + (t & 1) * Tr::TRB);
        }
        f16x8 mine[2] = {f16x8{}, f16x8{}}, other[2] = {f16x8{}, f16x8{}};
        if (own_live) dsblock(x1, x2, xt + 32 * e, sb, mask_tag, mine, other);
        {
          // Stage t - 1: own block from registers, partner's block from LDS.
          const char *trp = smem + Tr::OFF_TR + ((t + 1) & 1) * Tr::TRB;
          const char *dsp = smem + Tr::OFF_DSX + ((t + 1) & 1) * Tr::DSX_T + ((e ? pr : pr + 4) * 2) * Tr::SLOT +
                            lane * 16;
          f16x8 pb[2];
  #pragma unroll
          for (int ks = 0; ks < 2; ++ks) pb[ks] = *reinterpret_cast<const f16x8 *>(dsp + ks * Tr::SLOT);
          grad2(trp, prev, pb);
        }
        if (Tr::ROWBUF == 2) {
          tr_issue(rowb, T);
          tr_store(T, smem + Tr::OFF_TR + (t & 1) * Tr::TRB);
        }
        {
          char *dsw = smem + Tr::OFF_DSX + (t & 1) * Tr::DSX_T + (wave * 2) * Tr::SLOT + lane * 16;
  #pragma unroll
          for (int ks = 0; ks < 2; ++ks) *reinterpret_cast<f16x8 *>(dsw + ks * Tr::SLOT) = other[ks];
        }
        prev[0] = mine[0];
        prev[1] = mine[1];
        if (more) stats_store(t + 1, (t + 1) & 1);
        wait_loads();
        lds_barrier();
      }
    };
    run_tiles(0, t_a, std::true_type{});
    run_tiles(t_a, t_b, std::false_type{});
    run_tiles(t_b, ntiles, std::true_type{});
    if (ntiles > 0) {
      // Drain: gradient products of the last stage.
      const int t = ntiles;
      const char *trp = smem + Tr::OFF_TR + ((t + 1) & 1) * Tr::TRB;
      const char *dsp =
          smem + Tr::OFF_DSX + ((t + 1) & 1) * Tr::DSX_T + ((e ? pr : pr + 4) * 2) * Tr::SLOT + lane * 16;
      f16x8 pb[2];
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) pb[ks] = *reinterpret_cast<const f16x8 *>(dsp + ks * Tr::SLOT);
      grad2(trp, prev, pb);
    }

    // Epilogue: lane writes its resident row of the accumulated distribution,
    // d = (DB0 + db)*32 + 8j + 4h + (0..3).
    // A key chunk of a split pass writes its partial (zeros if the chunk is
    // empty) in the dense [split][distribution][unit, row] layout instead.
    if (r_ok && (TEN ? p.want2 : p.want1)) {
      const float f = p.scale / sigma / xs[TEN] * (KEYS_RES ? 1.f : qsg);
      float *O = TEN ? (KEYS_RES ? p.dk2 : p.dq2) : (KEYS_RES ? p.dk1 : p.dq1);
      int64_t rowoff = (rr + my_r) * D;
      if (S > 1) {
        O = p.dqp + ((int64_t)sp * 2 + TEN) * (p.BH * (int64_t)NQ * D);
        rowoff = (bh * (int64_t)NQ + my_r) * D;
      }
  #pragma unroll
      for (int db = 0; db < NACC; ++db) {
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = (DB0 + db) * 32 + 8 * j + 4 * h;
          const f32x4 v = {acc[db][4 * j] * f, acc[db][4 * j + 1] * f, acc[db][4 * j + 2] * f, acc[db][4 * j + 3] * f};
          *reinterpret_cast<f32x4 *>(O + rowoff + d) = v;
        }
      }
    }
  };
  using E0 = std::integral_constant<int, 0>;
  using E1 = std::integral_constant<int, 1>;
  if (KEYS_RES && any_neg) {
    if (e_rt)
      body(E1{}, std::true_type{});
    else
      body(E0{}, std::true_type{});
  } else {
    if (e_rt)
      body(E1{}, std::false_type{});
    else
      body(E0{}, std::false_type{});
  }
}

// Prepare step, first kernel: the largest |x| over a chunk of rows of one
// input tensor of one unit.  Workgroup (unit u, tensor tn, chunk c) of a
// launch with C chunks per tensor covers rows [c * per, (c + 1) * per),
// per = ceil(N / C), of q1, q2, k1, k2 (tn = 0..3; N = NQ for the queries, NK
// for the keys) and writes the maximum (0 for no rows) to part[(u * 4 + tn) *
// kAbsChunks + c].  bf16 magnitudes compare as their 15 low bits.  In a
// segmented launch (t.n > 0) each segment is a run of units with its own
// lengths, rows, chunk count and first unit.
__global__ __launch_bounds__(256) void absmax_kernel(const bf16 *q1, const bf16 *q2, const bf16 *k1, const bf16 *k2,
                                                     RowMap qmap, RowMap kmap, int64_t NQ, int64_t NK, int C,
                                                     int D, float *part, const SegTable t) {
  uint32_t wg = blockIdx.x;
  int64_t u0 = 0;
  if (t.n > 0) {
    const int i = seg_index(t, wg);
    wg -= t.seg[i].start;
    NQ = t.seg[i].nq;
    NK = t.seg[i].nk;
    qmap.sb = NQ;
    qmap.base = t.seg[i].oq;
    kmap.sb = NK;
    kmap.base = t.seg[i].ok;
    C = t.seg[i].chunks;
    u0 = t.seg[i].u0;
  }
  const int64_t u = wg / (4u * (uint32_t)C);
  const int tn = (int)((wg / (uint32_t)C) % 4u), c = (int)(wg % (uint32_t)C);
  const bool keys = tn >= 2;
  const int64_t N = keys ? NK : NQ;
  const bf16 *x = tn == 0 ? q1 : tn == 1 ? q2 : tn == 2 ? k1 : k2;
  const int64_t per = (N + C - 1) / C;
  const int64_t r0 = min<int64_t>(N, (int64_t)c * per), r1 = min<int64_t>(N, r0 + per);
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + ((keys ? kmap : qmap).row0(u) + r0) * D);
  const int64_t n16 = (r1 - r0) * D / 8;  // 16-byte chunks of the rows
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < n16; i += 256) {
    const u32x4 w = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    part[((u0 + u) * 4 + tn) * kAbsChunks + c] = __uint_as_float(m << 16);
  }
}

// Power of two that puts a largest magnitude m in [2^14, 2^15) (1 for m = 0 or
// a non-finite m): the scale of a tensor's fp16 gradient-product operand.
__device__ __forceinline__ float operand_scale(float m) {
  if (!(m > 0.f) || !(m <= 3.4e38f)) return 1.f;
  const int a = 14 - ilogbf(m);
  return ldexpf(1.f, min(max(a, -126), 126));
}

// Prepare step, second kernel, one workgroup per unit:
//  sigma[u] = 2^(kGradExp - e) with 2^(e-1) <= max_i |g[u,i]| < 2^e (1 if g is
//  all zero, and 1 everywhere when `unit` is set: fp32 inputs need no
//  scaling), stored negated when some g[u,:] is negative;
//  xscale[4 u + tn] = operand_scale(max over the C chunk maxima of tensor tn)
//  for bf16 inputs (part from absmax_kernel), 1 for fp32 and fp8 inputs (no
//  part: every e4m3 value is an fp16 value).
__global__ __launch_bounds__(256) void grad_scale_kernel(const float *g, RowMap qmap, int64_t NQ, float *sigma,
                                                         float *xscale, const float *part, int C, int unit,
                                                         const SegTable t) {
  int64_t bh = blockIdx.x;
  if (t.n > 0) {  // a segmented launch: one workgroup per unit of each segment
    const int i = seg_index(t, (uint32_t)bh);
    bh -= t.seg[i].start;
    NQ = t.seg[i].nq;
    qmap.sb = NQ;
    qmap.base = t.seg[i].oq;
    sigma += t.seg[i].u0;
    xscale += 4 * t.seg[i].u0;
    if (part) part += 4 * kAbsChunks * t.seg[i].u0;
    C = t.seg[i].chunks;
  }
  if (threadIdx.x < 4) {
    float m = 0.f;
    if (!unit && part)
      for (int c = 0; c < C; ++c) m = fmaxf(m, part[(bh * 4 + threadIdx.x) * kAbsChunks + c]);
    xscale[bh * 4 + threadIdx.x] = unit || !part ? 1.f : operand_scale(m);
  }
  if (unit) {
    // fp32 inputs: no dS scaling, but the sign flag is still needed.
    const float *gu = g + qmap.row0(bh);
    int neg = 0;
    for (int64_t i = threadIdx.x; i < NQ; i += 256) neg |= gu[i] < 0.f;
    neg = __syncthreads_or(neg);
    if (threadIdx.x == 0) sigma[bh] = neg ? -1.f : 1.f;
    return;
  }
  const float *gp = g + qmap.row0(bh);
  float m = 0.f;
  int neg = 0;
  for (int64_t i = threadIdx.x; i < NQ; i += 256) {
    m = fmaxf(m, fabsf(gp[i]));
    neg |= gp[i] < 0.f;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o));
    neg |= __shfl_xor(neg, o);
  }
  __shared__ float red[4];
  __shared__ int rneg[4];
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = m;
    rneg[threadIdx.x >> 6] = neg;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    neg = rneg[0] | rneg[1] | rneg[2] | rneg[3];
    float s = 1.f;
    if (m > 0.f && m <= 3.4e38f) {
      int k = kGradExp - (ilogbf(m) + 1);
      k = min(max(k, -126), 126);
      s = ldexpf(1.f, k);
    }
    sigma[bh] = neg ? -s : s;
  }
}

// ---- bf16 inputs, at most 128 queries per unit: fused single-visit backward ----
//
// StreamKL's backward fuses the dK and dQ products in one kernel (gist.science,
// "Fusion de Kernel"), which pays most where there are few queries: then the
// split passes re-read every key tile and the key-resident pass does a single
// short stage per workgroup.  Here all queries of a unit (at most 32 x QB) are
// resident in one workgroup, so a streamed key block's dK is complete after
// one visit and is written directly; dQ accumulates over the workgroup's key
// chunk and is written as one partial per chunk (summed in chunk order by
// dq_reduce_kernel, or written directly for a single chunk).  No atomics, no
// prepare step.
//
// 2 x QB waves: wave (qb, t) holds query block qb (32 queries) and
// accumulates the gradients of distribution t, forming only its dS (both need
// both logits).  Per 32-key block:
//  - logits: key block rows (LDS) x the block's queries (LDS), lane = query;
//  - dS_t in fp32 with |g| folded into the exponent offset, split into
//    bf16 hi + lo (exact operands; the pair carries 16 significand bits,
//    against fp16's 11, and has the fp32 exponent range, so no scaling);
//  - dQ^T[d, q] += K_t^T[d, keys] dS[keys, q]: K_t^T from the block's bf16
//    rows through a one-hot product (exact), against hi and lo;
//  - dS^T from a one-hot product of dS (hi and lo each, exact); with QB > 1
//    the waves post it to LDS and each wave then forms one (distribution,
//    32-column block) of the key block's dK over all resident queries;
//  - dK^T[d, k] = Q_t^T[d, q] dS^T[q, k], against Q_t^T formed once per
//    workgroup with sign(g_q) folded in; written for the block's valid keys.
// The problem is bound by reading K and writing fp32 dK, not by the matrix
// cores, so the redundant logits and doubled gradient products cost little.
//
// fp8 (e4m3) inputs: D-byte rows, the logits on v_mfma_f32_32x32x64_f8f6f4,
// and K_t^T, Q_t^T from one such product per 32-column block against an e4m3
// one-hot operand of the block's parity; every e4m3 value is a bf16 value,
// so those operands and everything after them are as for bf16 inputs.
template <int D, int QB, bool F8_ = false>
struct FusedTraits {
  static constexpr bool F8 = F8_;
  static constexpr int NT = 128 * QB;
  static constexpr int BK = 32;          // keys per block
  static constexpr int KSTEPS = F8 ? D / 64 : D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int RB = F8 ? D : D * 2;  // row bytes
  static constexpr int CPROW = RB / 16;  // 16-byte chunks per row
  static constexpr int TILE = 32 * RB;   // one tensor's 32 rows
  static constexpr int QTILE = QB * TILE;            // one tensor's resident queries
  static constexpr int OFF_K = 2 * QTILE;            // two buffers of two key tiles
  static constexpr int SLOT = 64 * 16;               // one lane-ordered 16-byte operand
  // QB > 1: posted dS^T, [query block][distribution][k-step][hi, lo][lane].
  static constexpr int OFF_X = OFF_K + 4 * TILE;
  static constexpr int X_BYTES = QB > 1 ? QB * 2 * 2 * 2 * SLOT : 0;
  static constexpr int LDS_BYTES = OFF_X + X_BYTES;
  static constexpr int QCHUNKS = QTILE / 16;         // 16-byte loads per tensor's query tile
  static constexpr int KCHUNKS = TILE / 16;          // 16-byte loads per key tile
  static_assert(QCHUNKS % NT == 0, "query staging split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Permuted one-hot operand that transposes a dS fragment: k-step ks of the
// dS operands holds the block's rows 16 ks + 8 (u / 4) + 4 h + u % 4 in slot
// u of lane half h; as the A operand of a product against this B operand
// they land in column 16 ks + (that row), so the 32 x 32 result (two k-steps)
// is the fragment transposed.  Lane (h, c) supplies k = 8 h + u.
__device__ __forceinline__ bf16x8 onehot_perm(int c, int h, int ks) {
  const int v = c - 16 * ks;
  bf16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const bool one = v >= 0 && v < 16 && ((v >> 2) & 1) == h && u == 4 * (v >> 3) + (v & 3);
    r[u] = (bf16)(one ? 1.f : 0.f);
  }
  return r;
}

__device__ __forceinline__ bf16x8 f32x8_to_bf16x8(const f32x16 &v, int half) {
  bf16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) r[u] = (bf16)v[8 * half + u];
  return r;
}

template <int D, int QB, bool F8>
__global__ __launch_bounds__(128 * QB) void bwd_fused_kernel(BwdParams p) {
  using Tr = FusedTraits<D, QB, F8>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qb = wave >> 1, t = wave & 1;  // query block, distribution
  const int h = lane >> 5, c32 = lane & 31;

  const int S = p.splits;
  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t u = L / (uint32_t)S;
  const int sp = (int)(L % (uint32_t)S);
  const int NQ = (int)p.NQ, NK = (int)p.NK, off = NK - NQ;
  const int64_t rq = p.qmap.row0(u), rk = p.kmap.row0(u);
  const bool want = t ? p.want2 : p.want1;

  // This workgroup's keys: whole 32-key blocks [k_lo, k_hi).
  const int k_lo = sp * p.kchunk, k_hi = min(NK, k_lo + p.kchunk);
  const int nblk = k_hi > k_lo ? (k_hi - k_lo + Tr::BK - 1) / Tr::BK : 0;

  // Resident queries: lane's query q (both lane halves) of block qb.
  const int q = qb * 32 + c32;
  const bool q_ok = q < NQ;
  float qb1 = kNoGrad, qb2 = kNoGrad, qkl = 0.f, qsg = 1.f;
  if (q_ok) query_stats(p.lse1[rq + q], p.lse2[rq + q], p.kl[rq + q], p.g[rq + q], 1.f, qb1, qb2, qkl, qsg);

  // Staging: query tiles once, key tiles double-buffered, all swizzled rows
  // (the swizzle repeats every 16 rows, so block qb's rows read like block 0's).
  const BufRange rqr[2] = {{reinterpret_cast<const char *>(p.q1) + rq * Tr::RB, NQ * Tr::RB},
                           {reinterpret_cast<const char *>(p.q2) + rq * Tr::RB, NQ * Tr::RB}};
  const BufRange rkr[2] = {{reinterpret_cast<const char *>(p.k1) + rk * Tr::RB, NK * Tr::RB},
                           {reinterpret_cast<const char *>(p.k2) + rk * Tr::RB, NK * Tr::RB}};
  auto src_off = [](int C) {
    const int row = C / Tr::CPROW;
    return (uint32_t)(row * Tr::RB + ((C % Tr::CPROW) ^ swz_bytes<Tr::RB>(row)) * 16);
  };
  auto load_queries = [&](int tn) {
#pragma unroll
    for (int i = 0; i < Tr::QCHUNKS / Tr::NT; ++i)
      buffer_load_lds16(rqr[tn], smem + tn * Tr::QTILE + (i * Tr::NT + wave * 64) * 16, src_off(i * Tr::NT + tid), 0);
  };
  auto load_keys = [&](int b) {
    char *buf = smem + Tr::OFF_K + (b & 1) * 2 * Tr::TILE;
    const uint32_t soff = (uint32_t)(k_lo + b * Tr::BK) * Tr::RB;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int i = 0; i < (Tr::KCHUNKS + Tr::NT - 1) / Tr::NT; ++i)
        if (Tr::KCHUNKS % Tr::NT == 0 || i * Tr::NT + wave * 64 < Tr::KCHUNKS)  // whole waves only
          buffer_load_lds16(rkr[tn], buf + tn * Tr::TILE + (i * Tr::NT + wave * 64) * 16, src_off(i * Tr::NT + tid),
                            soff);
  };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // Fragment (row r of a 32-row tile, 16-column chunk s, lane half h), and
  // for fp8 rows the 32-byte one of 64-element k-step s (chunks 4 s + 2 h, + 1).
  const int sw = swz_bytes<Tr::RB>(c32);
  auto frag = [&](const char *tile, int s) {
    return *reinterpret_cast<const bf16x8 *>(tile + c32 * Tr::RB + ((2 * s + h) ^ sw) * 16);
  };
  auto frag8 = [&](const char *tile, int s) {
    const char *r = tile + c32 * Tr::RB;
    return join16(*reinterpret_cast<const u32x4 *>(r + ((4 * s + 2 * h) ^ sw) * 16),
                  *reinterpret_cast<const u32x4 *>(r + ((4 * s + 2 * h + 1) ^ sw) * 16));
  };
  const char *qtile1 = smem + qb * Tr::TILE, *qtile2 = smem + Tr::QTILE + qb * Tr::TILE;

  load_queries(0);
  load_queries(1);
  if (nblk > 0) load_keys(0);
  wait_loads();
  barrier();

  // One-hot operands: columns of a 32-column block (transposing K_t and Q_t),
  // and the permuted ones transposing dS.  fp8: for block parity v, e4m3 1.0
  // at byte c of lane (h, c) when h == v (element 32 v + c of the k-step).
  const bf16x8 i0 = onehot(c32, h, 0, 1.f), i1 = onehot(c32, h, 1, 1.f);
  const bf16x8 j0 = onehot_perm(c32, h, 0), j1 = onehot_perm(c32, h, 1);
  i32x8 e8[2];
#pragma unroll
  for (int v = 0; v < 2; ++v)
#pragma unroll
    for (int dw = 0; dw < 8; ++dw)
      e8[v][dw] = h == v && (c32 >> 2) == dw ? (int32_t)(0x38u << (8 * (c32 & 3))) : 0;
  // K_t^T or Q_t^T of 32-column block db from a 32-row tile (sign bits xored
  // with `flip`), as the two bf16 k-step operands of the gradient products.
  auto transpose_block = [&](const char *tile, int db, uint32_t flip, bf16x8 &o0, bf16x8 &o1) {
    f32x16 T;
    if constexpr (F8) {
      i32x8 a = frag8(tile, db >> 1);
#pragma unroll
      for (int dw = 0; dw < 8; ++dw) a[dw] ^= (int32_t)flip;
      T = mma_f8(a, e8[db & 1], f32x16{});
    } else {
      u32x4 lo = __builtin_bit_cast(u32x4, frag(tile, 2 * db)), hi = __builtin_bit_cast(u32x4, frag(tile, 2 * db + 1));
      lo ^= flip;
      hi ^= flip;
      T = mma16(__builtin_bit_cast(bf16x8, lo), i0, f32x16{});
      T = mma16(__builtin_bit_cast(bf16x8, hi), i1, T);
    }
    o0 = f32x8_to_bf16x8(T, 0);
    o1 = f32x8_to_bf16x8(T, 1);
  };

  // The dK products this wave forms: QB == 1, every 32-column block of its
  // distribution t over its own queries; QB > 1, one (distribution tk,
  // block dbk) over all resident queries (none when 2 * NDB < 2 * QB waves).
  constexpr int NK_DB = QB == 1 ? Tr::NDB : 1;
  const int tk = QB == 1 ? t : wave % 2;
  const int dbk = QB == 1 ? 0 : wave / 2;
  const bool dk_wave = QB == 1 || dbk < Tr::NDB;
  const bool want_k = dk_wave && (tk ? p.want2 : p.want1);
  // Q_tk^T with sign(g_q) folded in, as the A operands of the dK product:
  // qT[db][kk] holds, in lane (h, d), queries 16 kk + 8 (m / 4) + 4 h + m % 4
  // (k-step kk over all resident queries) of column d of block db.
  bf16x8 qT[NK_DB][2 * QB];
  {
#pragma unroll
    for (int b2 = 0; b2 < QB; ++b2) {
      const int qq = b2 * 32 + c32;  // the query row this lane supplies as an A operand
      float gq = 0.f;
      if (qq < NQ) gq = p.g[rq + qq];
      const uint32_t flip = gq < 0.f ? (F8 ? 0x80808080u : 0x80008000u) : 0u;
      const char *qt = smem + tk * Tr::QTILE + b2 * Tr::TILE;
#pragma unroll
      for (int k = 0; k < NK_DB; ++k) {
        const int db = QB == 1 ? k : dbk;
        if (QB > 1 && !dk_wave) continue;
        transpose_block(qt, db, flip, qT[k][2 * b2], qT[k][2 * b2 + 1]);
      }
    }
  }

  const float c = p.scale * kLog2e;
  f32x16 dq[Tr::NDB];
#pragma unroll
  for (int db = 0; db < Tr::NDB; ++db) dq[db] = f32x16{};
  float *dK = tk ? p.dk2 : p.dk1;

  for (int b = 0; b < nblk; ++b) {
    if (b + 1 < nblk) load_keys(b + 1);
    const char *kt1 = smem + Tr::OFF_K + (b & 1) * 2 * Tr::TILE;
    const char *kt2 = kt1 + Tr::TILE;
    const int kb = k_lo + b * Tr::BK;
    // Logits: element r of lane (h, q) is key kb + acc_row(r, h), query q.
    f32x16 x1 = f32x16{}, x2 = f32x16{};
#pragma unroll
    for (int s = 0; s < Tr::KSTEPS; ++s) {
      if constexpr (F8) {
        x1 = mma_f8(frag8(kt1, s), frag8(qtile1, s), x1);
        x2 = mma_f8(frag8(kt2, s), frag8(qtile2, s), x2);
      } else {
        x1 = mma16(frag(kt1, s), frag(qtile1, s), x1);
        x2 = mma16(frag(kt2, s), frag(qtile2, s), x2);
      }
    }
    // dS_t (times |g|), hi + lo in bf16, as the operands of k-steps 0 and 1.
    const bool edge = kb + Tr::BK > NK || (p.causal && kb + Tr::BK - 1 > off) || !q_ok;
    bf16x8 dh[2], dl[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float y1 = __builtin_fmaf(x1[r], c, -qb1);
      const float y2 = __builtin_fmaf(x2[r], c, -qb2);
      const float p1 = fast_exp2(y1), p2 = fast_exp2(y2);
      float v = t ? p2 - p1 : p1 * __builtin_fmaf(y1 - y2, kLn2, -qkl);
      if (edge) {
        const int k = kb + acc_row(r, h);
        v = (q_ok && k < NK && (!p.causal || k <= q + off)) ? v : 0.f;
      }
      const bf16 vh = (bf16)v;
      dh[r >> 3][r & 7] = vh;
      dl[r >> 3][r & 7] = (bf16)(v - (float)vh);
    }
    if (want) {
      // dQ^T[d, q] += K_t^T[d, keys] dS[keys, q].
      const char *ktt = t ? kt2 : kt1;
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
        bf16x8 a[2];
        transpose_block(ktt, db, 0u, a[0], a[1]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dq[db] = mma16(a[ks], dh[ks], dq[db]);
          dq[db] = mma16(a[ks], dl[ks], dq[db]);
        }
      }
    }
    // dS^T: element r of lane (h, k) is query 32 qb + acc_row(r, h) of key kb + k.
    bf16x8 sh[2], sl[2];
    if (QB > 1 || want) {
      f32x16 Th = mma16(dh[0], j0, f32x16{}), Tl = mma16(dl[0], j0, f32x16{});
      Th = mma16(dh[1], j1, Th);
      Tl = mma16(dl[1], j1, Tl);
      sh[0] = f32x8_to_bf16x8(Th, 0);
      sh[1] = f32x8_to_bf16x8(Th, 1);
      sl[0] = f32x8_to_bf16x8(Tl, 0);
      sl[1] = f32x8_to_bf16x8(Tl, 1);
    }
    if (QB > 1) {
      char *xw = smem + Tr::OFF_X + ((qb * 2 + t) * 4) * Tr::SLOT + lane * 16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        *reinterpret_cast<bf16x8 *>(xw + (2 * ks) * Tr::SLOT) = sh[ks];
        *reinterpret_cast<bf16x8 *>(xw + (2 * ks + 1) * Tr::SLOT) = sl[ks];
      }
      barrier();
    }
    // dK^T[d, k] = Q_tk^T[d, q] dS_tk^T[q, k] over the resident queries,
    // written for key kb + c32.
    if (want_k) {
      const int key = kb + c32;
#pragma unroll
      for (int k = 0; k < NK_DB; ++k) {
        const int db = QB == 1 ? k : dbk;
        f32x16 a = f32x16{};
#pragma unroll
        for (int b2 = 0; b2 < QB; ++b2)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 bh, bl;
            if (QB == 1) {
              bh = sh[ks];
              bl = sl[ks];
            } else {
              const char *xr = smem + Tr::OFF_X + ((b2 * 2 + tk) * 4 + 2 * ks) * Tr::SLOT + lane * 16;
              bh = *reinterpret_cast<const bf16x8 *>(xr);
              bl = *reinterpret_cast<const bf16x8 *>(xr + Tr::SLOT);
            }
            a = mma16(qT[k][2 * b2 + ks], bh, a);
            a = mma16(qT[k][2 * b2 + ks], bl, a);
          }
        if (key < NK) {
          float *o = dK + (rk + key) * D + db * 32 + 4 * h;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 v = {a[4 * j] * p.scale, a[4 * j + 1] * p.scale, a[4 * j + 2] * p.scale,
                             a[4 * j + 3] * p.scale};
            *reinterpret_cast<f32x4 *>(o + 8 * j) = v;
          }
        }
      }
    }
    wait_loads();
    barrier();
  }

  // dQ: lane's query, d = 32 db + 8 j + 4 h + (0..3); one partial per chunk.
  if (want && q_ok) {
    const float f = p.scale * qsg;
    float *O = t ? p.dq2 : p.dq1;
    int64_t rowoff = (rq + q) * D;
    if (S > 1) {
      O = p.dqp + ((int64_t)sp * 2 + t) * (p.BH * (int64_t)NQ * D);
      rowoff = (u * (int64_t)NQ + q) * D;
    }
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = {dq[db][4 * j] * f, dq[db][4 * j + 1] * f, dq[db][4 * j + 2] * f, dq[db][4 * j + 3] * f};
        *reinterpret_cast<f32x4 *>(O + rowoff + db * 32 + 8 * j + 4 * h) = v;
      }
  }
}

template <int D, int QB, bool F8>
static hipError_t launch_fused(const BwdParams &p, hipStream_t s) {
  using Tr = FusedTraits<D, QB, F8>;
  const void *fn = reinterpret_cast<const void *>(&bwd_fused_kernel<D, QB, F8>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_fused_kernel<D, QB, F8>), dim3((uint32_t)(p.BH * p.splits)), dim3(Tr::NT), Tr::LDS_BYTES,
                     s, p);
  return hipGetLastError();
}

int fused_query_blocks(int64_t NQ) { return NQ <= 32 ? 1 : 4; }

hipError_t launch_bwd_fused(int dtype, int D, const BwdParams &p, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  if (dtype == 2) {
    if (fused_query_blocks(p.NQ) == 1)
      return D == 128 ? launch_fused<128, 1, true>(p, s) : launch_fused<64, 1, true>(p, s);
    return D == 128 ? launch_fused<128, 4, true>(p, s) : launch_fused<64, 4, true>(p, s);
  }
  if (fused_query_blocks(p.NQ) == 1) return D == 128 ? launch_fused<128, 1, false>(p, s) : launch_fused<64, 1, false>(p, s);
  return D == 128 ? launch_fused<128, 4, false>(p, s) : launch_fused<64, 4, false>(p, s);
}

__global__ __launch_bounds__(256) void zero_kernel(float *dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = 0.f;
}

// A plain launch passes an empty segment table.
const SegTable kNoSegs{};

template <int D, bool KEYS_RES>
static hipError_t launch_fp32_pass(const BwdParams &p, const SegTable &t, hipStream_t s) {
  using Tr = BwdF32Traits<D, KEYS_RES>;
  const int64_t NR = KEYS_RES ? p.NK : p.NQ;
  if (t.n == 0 && NR == 0) return hipSuccess;
  const void *fn = reinterpret_cast<const void *>(&bwd_fp32_kernel<D, KEYS_RES>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nblk = t.n > 0 ? (int64_t)t.end : p.BH * ((NR + Tr::BR - 1) / Tr::BR);
  hipLaunchKernelGGL((bwd_fp32_kernel<D, KEYS_RES>), dim3((uint32_t)nblk), dim3(256), Tr::LDS_BYTES, s, p, t);
  return hipGetLastError();
}

hipError_t launch_bwd_prepare(int dtype, const PrepParams &p, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  const int C = abs_chunks(p.NQ, p.NK);
  if (dtype == 0) {
    hipLaunchKernelGGL(absmax_kernel, dim3((uint32_t)(p.BH * 4 * C)), dim3(256), 0, s,
                       reinterpret_cast<const bf16 *>(p.q1), reinterpret_cast<const bf16 *>(p.q2),
                       reinterpret_cast<const bf16 *>(p.k1), reinterpret_cast<const bf16 *>(p.k2), p.qmap, p.kmap,
                       p.NQ, p.NK, C, p.D, p.part, kNoSegs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(grad_scale_kernel, dim3((uint32_t)p.BH), dim3(256), 0, s, p.g, p.qmap, p.NQ, p.sigma,
                     p.xscale, dtype == 0 ? p.part : nullptr, C, dtype == 1 ? 1 : 0, kNoSegs);
  return hipGetLastError();
}

hipError_t launch_absmax_segs(const PrepParams &p, const SegTable &t, hipStream_t s) {
  hipLaunchKernelGGL(absmax_kernel, dim3(t.end), dim3(256), 0, s, reinterpret_cast<const bf16 *>(p.q1),
                     reinterpret_cast<const bf16 *>(p.q2), reinterpret_cast<const bf16 *>(p.k1),
                     reinterpret_cast<const bf16 *>(p.k2), p.qmap, p.kmap, (int64_t)0, (int64_t)0, 1, p.D, p.part,
                     t);
  return hipGetLastError();
}

hipError_t launch_grad_scale_segs(int dtype, const PrepParams &p, const SegTable &t, hipStream_t s) {
  hipLaunchKernelGGL(grad_scale_kernel, dim3(t.end), dim3(256), 0, s, p.g, p.qmap, (int64_t)0, p.sigma, p.xscale,
                     dtype == 0 ? p.part : nullptr, 1, dtype == 1 ? 1 : 0, t);
  return hipGetLastError();
}

template <int D, bool KEYS_RES, int MODE, bool F8>
static hipError_t launch_pass4(const BwdParams &p, const SegTable &t, hipStream_t s) {
  using Tr = Bwd4Traits<D, KEYS_RES, F8>;
  const int64_t NR = KEYS_RES ? p.NK : p.NQ;
  if (t.n == 0 && NR == 0) return hipSuccess;
  const void *fn = reinterpret_cast<const void *>(&bwd4_kernel<D, KEYS_RES, MODE, F8>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nblk =
      t.n > 0 ? (int64_t)t.end : p.BH * ((NR + Tr::BR - 1) / Tr::BR) * (KEYS_RES ? 1 : p.splits);
  hipLaunchKernelGGL((bwd4_kernel<D, KEYS_RES, MODE, F8>), dim3((uint32_t)nblk), dim3(Tr::NT), Tr::LDS_BYTES, s,
                     p, t);
  return hipGetLastError();
}

// Both distributions, the teacher's only or the student's only (bf16 or
// fp8 inputs).
template <int D, bool KEYS_RES, bool F8 = false>
static hipError_t launch_bf16_pass(const BwdParams &p, const SegTable &t, hipStream_t s) {
  if (p.want1 && p.want2) return launch_pass4<D, KEYS_RES, 0, F8>(p, t, s);
  if (p.want1) return launch_pass4<D, KEYS_RES, 1, F8>(p, t, s);
  if (p.want2) return launch_pass4<D, KEYS_RES, 2, F8>(p, t, s);
  return hipSuccess;
}

hipError_t launch_bwd_dk_segs(int dtype, int D, const BwdParams &p, const SegTable &t, hipStream_t s) {
  if (dtype == 0) return D == 128 ? launch_bf16_pass<128, true>(p, t, s) : launch_bf16_pass<64, true>(p, t, s);
  if (dtype == 2)
    return D == 128 ? launch_bf16_pass<128, true, true>(p, t, s) : launch_bf16_pass<64, true, true>(p, t, s);
  return D == 128 ? launch_fp32_pass<128, true>(p, t, s) : launch_fp32_pass<64, true>(p, t, s);
}

hipError_t launch_bwd_dq_segs(int dtype, int D, const BwdParams &p, const SegTable &t, hipStream_t s) {
  if (dtype == 0) return D == 128 ? launch_bf16_pass<128, false>(p, t, s) : launch_bf16_pass<64, false>(p, t, s);
  if (dtype == 2)
    return D == 128 ? launch_bf16_pass<128, false, true>(p, t, s) : launch_bf16_pass<64, false, true>(p, t, s);
  return D == 128 ? launch_fp32_pass<128, false>(p, t, s) : launch_fp32_pass<64, false>(p, t, s);
}

hipError_t launch_bwd_dk(int dtype, int D, const BwdParams &p, hipStream_t s) {
  return launch_bwd_dk_segs(dtype, D, p, kNoSegs, s);
}

hipError_t launch_bwd_dq(int dtype, int D, const BwdParams &p, hipStream_t s) {
  return launch_bwd_dq_segs(dtype, D, p, kNoSegs, s);
}

// dQ_t = sum of the key chunks' partials, in chunk order (deterministic); one
// thread per 4 consecutive elements of the dense [unit, row][D] layout.
__global__ __launch_bounds__(256) void dq_reduce_kernel(BwdParams p, int D) {
  const int64_t per_t = p.BH * p.NQ * D;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= per_t) return;
  const int64_t urow = e / D, d = e - urow * D;
  const int64_t u = urow / p.NQ, row = urow - u * p.NQ;
  const int64_t o = (p.qmap.row0(u) + row) * D + d;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!(t ? p.want2 : p.want1)) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < p.splits; ++sp) acc += *reinterpret_cast<const f32x4 *>(p.dqp + (sp * 2 + t) * per_t + e);
    *reinterpret_cast<f32x4 *>((t ? p.dq2 : p.dq1) + o) = acc;
  }
}

hipError_t launch_dq_reduce(int D, const BwdParams &p, hipStream_t s) {
  const int64_t n4 = p.BH * p.NQ * D / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(dq_reduce_kernel, dim3((uint32_t)((n4 + 255) / 256)), dim3(256), 0, s, p, D);
  return hipGetLastError();
}

hipError_t launch_zero(float *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t nblk = (n + 255) / 256;
  if (nblk > 65536) nblk = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3((uint32_t)nblk), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace skl
