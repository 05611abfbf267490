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
// (dK), the other keeps queries resident and streams keys (dQ).  Both are the
// same kernel template: a wave owns 32 resident rows, whose fragments stay in
// registers, and 64-row tiles of the streamed operand pass through LDS.  With
// bf16 inputs the tile is staged once, as fp16 rows: the logits product reads
// rows of it and the gradient product reads columns of it through the
// transposing LDS loads.  fp32 inputs stage a row-major and a transposed copy.
//
// Logits come out as (streamed x resident) accumulator blocks, so a lane holds
// one resident row and 16 streamed rows; that accumulator is, element for
// element, the B operand of the gradient product dR^T += X^T dS, which needs
// no shuffle.  bf16 inputs use fp16 for the gradient product: dS in bf16
// loses too much (8-bit significand) for the 2e-3 relative bound, fp16 keeps
// 11 bits.  dS is scaled by a per-(b,h) power of two sigma with
// max|g| * sigma in [2^7, 2^8) so it sits in fp16's normal range; the factor
// is divided out exactly at the end.  Q and K themselves convert to fp16
// exactly as long as they lie within the fp16 range.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace skl {

template <typename T> struct GradOp { using type = f16; };
template <> struct GradOp<float> { using type = float; };

template <typename T, int D, bool KEYS_RES>
struct BwdTraits {
  // bf16 inputs run both products on fp16 operands converted (exactly, within
  // the fp16 range) from one fp16 row-major copy of the streamed tile; the
  // gradient product reads it through the transposing LDS loads.  fp32 inputs
  // keep an fp32 row-major copy plus an fp32 transposed copy.
  static constexpr bool F16 = sizeof(T) == 2;
  using G = typename GradOp<T>::type;
  static constexpr int WAVES = 4;
  static constexpr int BR = kBwdBR;                        // resident rows per workgroup
#ifndef SKL_BWD_BX
#define SKL_BWD_BX 64
#endif
  static constexpr int BX = (!F16 && D == 128) ? 32 : (F16 ? SKL_BWD_BX : 64);  // streamed rows per stage
  static constexpr int XB = BX / 32;
  static constexpr int KSTEPS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int ROW_BYTES = D * (int)sizeof(T);  // one row in HBM
  static constexpr int CPR = ROW_BYTES / 16;            // 16-byte chunks per HBM row
  static constexpr int ES = (int)sizeof(G);             // element size of the LDS copy
  // fp16 row stride D*2 + 48 B: the 16 rows of a logits-operand read and the
  // 4 rows x 32 B of a transposing read both fall in distinct banks.
  static constexpr int XROW = F16 ? D * 2 + 48 : ROW_BYTES + 16;
  static constexpr int XT_STRIDE = F16 ? 0 : BX * 4 + 16;
  static constexpr int XROW_BYTES = BX * XROW;
  static constexpr int XT_BYTES = F16 ? 0 : D * XT_STRIDE;
  static constexpr int NSTAT = 4;  // b1, b2, KL, sign(g) of each streamed query
  static constexpr int STAT_BYTES = KEYS_RES ? NSTAT * BX * 4 : 0;
  static constexpr int OFF_XT = 2 * XROW_BYTES;
  static constexpr int OFF_STAT = OFF_XT + 2 * XT_BYTES;
  static constexpr int STAGE_BYTES = OFF_STAT + STAT_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  // Staging work per thread: bf16 -> 16-byte chunks; fp32 -> items of 4 rows x 1 chunk.
  static constexpr int CPT = F16 ? BX * CPR / 256 : 1;
  static constexpr int ITEMS = (BX / 4) * CPR;
  static constexpr int IPT = F16 ? 1 : (ITEMS + 255) / 256;
  static_assert(BR == WAVES * 32, "resident tile");
  static_assert(!F16 || CPT * 256 == BX * CPR, "staging split");
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

// Four consecutive-row fp16 elements of one column, gathered by the
// transposing LDS load: within each 16-lane group, lane 4k + q reads 8 bytes
// at `p` and lane i receives element i%4 of the reads of lanes 4k + i/4.
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
__device__ __forceinline__ f16x4 lds_read_tr16(const char *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(f16x4, v);
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

template <typename T, int D, bool KEYS_RES>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdParams p) {
  using Tr = BwdTraits<T, D, KEYS_RES>;
  using G = typename Tr::G;
  using CG = chunk_t<G>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;

  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int NR = KEYS_RES ? NK : NQ;  // resident row count
  const int NX = KEYS_RES ? NQ : NK;  // streamed row count
  const int nrt = (NR + Tr::BR - 1) / Tr::BR;

  // Head-major order, each XCD taking a contiguous run of heads (so one
  // head's streamed tiles are shared through one L2); within a head the
  // heaviest resident tiles go first: under the causal mask low keys see the
  // most queries, high queries see the most keys.
  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = L / (uint32_t)nrt;
  const int rt = KEYS_RES ? (int)(L % (uint32_t)nrt) : nrt - 1 - (int)(L % (uint32_t)nrt);

  const T *R1 = reinterpret_cast<const T *>(KEYS_RES ? p.k1 : p.q1) + bh * (int64_t)NR * D;
  const T *R2 = reinterpret_cast<const T *>(KEYS_RES ? p.k2 : p.q2) + bh * (int64_t)NR * D;
  const char *X1 = reinterpret_cast<const char *>(reinterpret_cast<const T *>(KEYS_RES ? p.q1 : p.k1) +
                                                  bh * (int64_t)NX * D);
  const char *X2 = reinterpret_cast<const char *>(reinterpret_cast<const T *>(KEYS_RES ? p.q2 : p.k2) +
                                                  bh * (int64_t)NX * D);
  const float *KLr = p.kl + bh * (int64_t)NQ;
  const float *LS1 = p.lse1 + bh * (int64_t)NQ;
  const float *LS2 = p.lse2 + bh * (int64_t)NQ;
  const float *Gr = p.g + bh * (int64_t)NQ;
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
    if constexpr (Tr::F16) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 w1 = r_ok ? *reinterpret_cast<const u32x4 *>(R1 + (int64_t)my_r * D + 16 * s + 8 * h) : z;
      const u32x4 w2 = r_ok ? *reinterpret_cast<const u32x4 *>(R2 + (int64_t)my_r * D + 16 * s + 8 * h) : z;
      rf1[s] = __builtin_bit_cast(CG, bf16x8_to_f16x8(w1));
      rf2[s] = __builtin_bit_cast(CG, bf16x8_to_f16x8(w2));
    } else {
      rf1[s] = r_ok ? load_chunk<T>(R1 + (int64_t)my_r * D + 16 * s + 8 * h) : CG{};
      rf2[s] = r_ok ? load_chunk<T>(R2 + (int64_t)my_r * D + 16 * s + 8 * h) : CG{};
    }
  }

  const float c = p.scale * kLog2e;
  // Per-query statistics when queries are resident (see query_stats).
  float qb1 = kNoGrad, qb2 = kNoGrad, qkl = 0.f, qsg = 1.f;
  if (!KEYS_RES && r_ok) query_stats(LS1[my_r], LS2[my_r], KLr[my_r], Gr[my_r], sigma, qb1, qb2, qkl, qsg);

  // ---- staging: global -> registers -> LDS ----
  u32x4 st[2][Tr::F16 ? Tr::CPT : 4 * Tr::IPT];
  float sv[Tr::NSTAT];
  auto gload = [&](int t) {
    const int xb0 = x_of(t);
    const u32x4 z = {0u, 0u, 0u, 0u};
    if constexpr (Tr::F16) {
#pragma unroll
      for (int i = 0; i < Tr::CPT; ++i) {
        const int cidx = tid + 256 * i;
        const int row = xb0 + cidx / Tr::CPR, col = cidx % Tr::CPR;
        const int64_t o = (int64_t)row * Tr::ROW_BYTES + col * 16;
        st[0][i] = row < NX ? *reinterpret_cast<const u32x4 *>(X1 + o) : z;
        st[1][i] = row < NX ? *reinterpret_cast<const u32x4 *>(X2 + o) : z;
      }
    } else {
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
    if constexpr (Tr::F16) {
#pragma unroll
      for (int i = 0; i < Tr::CPT; ++i) {
        const int cidx = tid + 256 * i;
        const int row = cidx / Tr::CPR, col = cidx % Tr::CPR;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          *reinterpret_cast<u32x4 *>(base + t2 * Tr::XROW_BYTES + row * Tr::XROW + col * 16) =
              bf16x8_to_f16x8(st[t2][i]);
      }
    } else {
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
        const char *a1p = base + (xb * 32 + c32) * Tr::XROW + 8 * h * Tr::ES;
        const char *a2p = a1p + Tr::XROW_BYTES;
#pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          const CG a1 = *reinterpret_cast<const CG *>(a1p + 16 * s * Tr::ES);
          const CG a2 = *reinterpret_cast<const CG *>(a2p + 16 * s * Tr::ES);
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
          b1[u] = (G)d1[8 * ks + u];
          b2[u] = (G)d2[8 * ks + u];
        }
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) {
          CG a1, a2;
          if constexpr (Tr::F16) {
            // 16-lane group g: columns db*32 + 16(g&1) + (0..15), rows 16ks + 4(g>>1) + (0..3) (+8).
            const int j16 = lane & 15, grp = lane >> 4;
            const int rb = xb * 32 + 16 * ks + 4 * (grp >> 1) + (j16 >> 2);
            const int d0 = db * 32 + 16 * (grp & 1) + 4 * (j16 & 3);
            const char *t1 = base + rb * Tr::XROW + d0 * 2;
            const char *t2 = t1 + Tr::XROW_BYTES;
            const f16x4 l1 = lds_read_tr16(t1), h1 = lds_read_tr16(t1 + 8 * Tr::XROW);
            const f16x4 l2 = lds_read_tr16(t2), h2 = lds_read_tr16(t2 + 8 * Tr::XROW);
            a1 = __builtin_shufflevector(l1, h1, 0, 1, 2, 3, 4, 5, 6, 7);
            a2 = __builtin_shufflevector(l2, h2, 0, 1, 2, 3, 4, 5, 6, 7);
          } else {
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
      const int64_t rowoff = (bh * (int64_t)NR + my_r) * D;
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

// ---- bf16 inputs: two waves per SIMD ----
//
// A single wave per SIMD leaves the VALU half idle (one wave issues a VALU op
// only every few cycles; two waves fill the gaps) and exposes every LDS and
// barrier wait.  This variant runs eight waves.  Waves p and p + 4 form a pair
// that shares 32 resident rows: per 64-row streamed stage, wave p + 4e
// computes logits and dS of streamed block e (rows 32e..32e+31) and posts its
// dS operands to LDS; after a barrier each wave of the pair accumulates the
// gradient product over both streamed blocks for its half of D (columns
// 64e..64e+63 at D = 128).  Per wave that halves the gradient accumulators,
// which keeps a wave within 256 registers.
template <int D, bool KEYS_RES>
struct Bwd2Traits {
  static constexpr int NT = 512;
  static constexpr int BR = kBwdBR;        // resident rows per workgroup: 4 pairs x 32
  static constexpr int BX = 64;            // streamed rows per stage
  static constexpr int KSTEPS = D / 16;
  static constexpr int NDH = D / 64;       // 32-column gradient blocks per wave
  static constexpr int ROW_BYTES = D * 2;  // one bf16 row in HBM
  static constexpr int CPR = ROW_BYTES / 16;
  static constexpr int XROW = D * 2 + 48;  // fp16 row stride in LDS
  static constexpr int XROW_BYTES = BX * XROW;
  // Key-resident pass: per streamed query the fp32 stats b1, b2, KL and a
  // 16-bit sign mask (0x8000 where g < 0), XORed onto the fp16 dS operands.
  static constexpr int NSTAT = 3;
  static constexpr int STAT_BYTES = KEYS_RES ? NSTAT * BX * 4 + BX * 2 : 0;
  static constexpr int OFF_STAT = 2 * XROW_BYTES;
  static constexpr int STAGE_BYTES = OFF_STAT + STAT_BYTES;
  static constexpr int DSX_SLOT = 64 * 16;             // one lane-ordered 16-byte operand per lane
  static constexpr int DSX_BYTES = 4 * 2 * 4 * DSX_SLOT;  // [pair][block][tensor * 2 + ks]
  static constexpr int OFF_DSX = 2 * STAGE_BYTES;
  static constexpr int LDS_BYTES = OFF_DSX + DSX_BYTES;
  static constexpr int CPT = BX * CPR / NT;  // 16-byte staging chunks per thread per tensor
  static_assert(BR == 4 * 32, "resident tile");
  static_assert(CPT * NT == BX * CPR, "staging split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGE_BYTES % 16 == 0, "LDS alignment");
};

template <int D, bool KEYS_RES>
__global__ __launch_bounds__(512, 1) void bwd2_kernel(BwdParams p) {
  using Tr = Bwd2Traits<D, KEYS_RES>;
  using CG = f16x8;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int pr = wave & 3;   // pair: resident rows
  const int e = wave >> 2;   // streamed block for dS, half of D for the gradient
  const int h = lane >> 5, c32 = lane & 31;

  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int off = NK - NQ;
  const int NR = KEYS_RES ? NK : NQ;
  const int NX = KEYS_RES ? NQ : NK;
  const int nrt = (NR + Tr::BR - 1) / Tr::BR;

  // Same workgroup order as the one-wave kernel: head-major per XCD, heaviest
  // resident tiles of a head first.
  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = L / (uint32_t)nrt;
  const int rt = KEYS_RES ? (int)(L % (uint32_t)nrt) : nrt - 1 - (int)(L % (uint32_t)nrt);

  const bf16 *R1 = reinterpret_cast<const bf16 *>(KEYS_RES ? p.k1 : p.q1) + bh * (int64_t)NR * D;
  const bf16 *R2 = reinterpret_cast<const bf16 *>(KEYS_RES ? p.k2 : p.q2) + bh * (int64_t)NR * D;
  const char *X1 = reinterpret_cast<const char *>(reinterpret_cast<const bf16 *>(KEYS_RES ? p.q1 : p.k1) +
                                                  bh * (int64_t)NX * D);
  const char *X2 = reinterpret_cast<const char *>(reinterpret_cast<const bf16 *>(KEYS_RES ? p.q2 : p.k2) +
                                                  bh * (int64_t)NX * D);
  const float *KLr = p.kl + bh * (int64_t)NQ;
  const float *LS1 = p.lse1 + bh * (int64_t)NQ;
  const float *LS2 = p.lse2 + bh * (int64_t)NQ;
  const float *Gr = p.g + bh * (int64_t)NQ;
  const float sigma_raw = p.sigma[bh];
  const float sigma = fabsf(sigma_raw);
  const bool any_neg = sigma_raw < 0.f;

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
  const int ntiles = x_hi > x_lo ? (x_hi - x_lo + Tr::BX - 1) / Tr::BX : 0;
  auto x_of = [&](int t) { return x_lo + (KEYS_RES ? ntiles - 1 - t : t) * Tr::BX; };

  // Resident fragments (B operand of the logits product), converted to fp16.
  CG rf1[Tr::KSTEPS], rf2[Tr::KSTEPS];
#pragma unroll
  for (int s = 0; s < Tr::KSTEPS; ++s) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 w1 = r_ok ? *reinterpret_cast<const u32x4 *>(R1 + (int64_t)my_r * D + 16 * s + 8 * h) : z;
    const u32x4 w2 = r_ok ? *reinterpret_cast<const u32x4 *>(R2 + (int64_t)my_r * D + 16 * s + 8 * h) : z;
    rf1[s] = __builtin_bit_cast(CG, bf16x8_to_f16x8(w1));
    rf2[s] = __builtin_bit_cast(CG, bf16x8_to_f16x8(w2));
  }

  const float c = p.scale * kLog2e;
  float qb1 = kNoGrad, qb2 = kNoGrad, qkl = 0.f, qsg = 1.f;
  if (!KEYS_RES && r_ok) query_stats(LS1[my_r], LS2[my_r], KLr[my_r], Gr[my_r], sigma, qb1, qb2, qkl, qsg);

  // ---- staging: global -> registers -> LDS (fp16 rows) ----
  u32x4 st[2][Tr::CPT];
  float sv[Tr::NSTAT];
  uint32_t sgn = 0;
  auto gload = [&](int t) {
    const int xb0 = x_of(t);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < Tr::CPT; ++i) {
      const int cidx = tid + Tr::NT * i;
      const int row = xb0 + cidx / Tr::CPR, col = cidx % Tr::CPR;
      const int64_t o = (int64_t)row * Tr::ROW_BYTES + col * 16;
      st[0][i] = row < NX ? *reinterpret_cast<const u32x4 *>(X1 + o) : z;
      st[1][i] = row < NX ? *reinterpret_cast<const u32x4 *>(X2 + o) : z;
    }
    if (KEYS_RES && tid < Tr::BX) {
      const int q = xb0 + tid;
      sv[0] = sv[1] = kNoGrad;
      sv[2] = 0.f;
      float sg = 1.f;
      if (q < NQ) query_stats(LS1[q], LS2[q], KLr[q], Gr[q], sigma, sv[0], sv[1], sv[2], sg);
      sgn = sg < 0.f ? 0x8000u : 0u;
    }
  };
  auto sstore = [&](int buf) {
    char *base = smem + buf * Tr::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Tr::CPT; ++i) {
      const int cidx = tid + Tr::NT * i;
      const int row = cidx / Tr::CPR, col = cidx % Tr::CPR;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        *reinterpret_cast<u32x4 *>(base + t2 * Tr::XROW_BYTES + row * Tr::XROW + col * 16) =
            bf16x8_to_f16x8(st[t2][i]);
    }
    if (KEYS_RES && tid < Tr::BX) {
      float *sb = reinterpret_cast<float *>(base + Tr::OFF_STAT);
#pragma unroll
      for (int f = 0; f < Tr::NSTAT; ++f) sb[f * Tr::BX + tid] = sv[f];
      reinterpret_cast<uint16_t *>(sb + Tr::NSTAT * Tr::BX)[tid] = (uint16_t)sgn;
    }
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
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

  // dS operand slots of this wave and of its partner (lane-ordered, conflict-free).
  char *own_slot = smem + Tr::OFF_DSX + (pr * 2 + e) * 4 * Tr::DSX_SLOT + lane * 16;
  const char *par_slot = smem + Tr::OFF_DSX + (pr * 2 + (1 - e)) * 4 * Tr::DSX_SLOT + lane * 16;

  {
    f32x16 acc1[Tr::NDH], acc2[Tr::NDH];
#pragma unroll
    for (int db = 0; db < Tr::NDH; ++db) {
      acc1[db] = f32x16{};
      acc2[db] = f32x16{};
    }
    // No visible pair between this pair's resident rows and streamed rows [xa, xa + 32).
    auto empty_blk = [&](int xa) -> bool {
      if (KEYS_RES) return xa >= NQ || ra >= NK || (p.causal && ra > xa + 31 + off);
      return ra >= NQ || xa >= NK || (p.causal && xa > ra + 31 + off);
    };
    // Logits and dS of streamed block xb (rows xa..xa+31) -> gradient-product B
    // operands: bo[ks] (teacher), bo[2 + ks] (student).
    auto dsblock = [&](const char *base, int xb, int xa, auto mask_tag, CG(&bo)[4]) {
      constexpr bool MASK = decltype(mask_tag)::value;
      f32x16 x1 = f32x16{}, x2 = f32x16{};
      {
        const char *a1p = base + (xb * 32 + c32) * Tr::XROW + 16 * h;
        const char *a2p = a1p + Tr::XROW_BYTES;
#pragma unroll
        for (int s = 0; s < Tr::KSTEPS; ++s) {
          const CG a1 = *reinterpret_cast<const CG *>(a1p + 32 * s);
          const CG a2 = *reinterpret_cast<const CG *>(a2p + 32 * s);
          x1 = mma16(a1, rf1[s], x1);
          x2 = mma16(a2, rf2[s], x2);
        }
      }
      const float *sb = reinterpret_cast<const float *>(base + Tr::OFF_STAT);
      f32x16 d1, d2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 B1, B2, KV;
        if (KEYS_RES) {
          const int q = xb * 32 + 8 * j + 4 * h;
          B1 = *reinterpret_cast<const f32x4 *>(sb + 0 * Tr::BX + q);
          B2 = *reinterpret_cast<const f32x4 *>(sb + 1 * Tr::BX + q);
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
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          bo[ks][u] = (f16)d1[8 * ks + u];
          bo[2 + ks][u] = (f16)d2[8 * ks + u];
        }
      }
      // Key-resident pass with some g < 0: dS of query q carries sign(g_q).
      // Slot pair (2m, 2m+1) of k-step ks holds queries 16ks + 4h + {0,2,8,10}[m] + (0, 1).
      if (KEYS_RES && any_neg) {
        const char *sgp = reinterpret_cast<const char *>(sb + Tr::NSTAT * Tr::BX) + (xb * 32 + 4 * h) * 2;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint2 lo = *reinterpret_cast<const uint2 *>(sgp + 32 * ks);
          const uint2 hi = *reinterpret_cast<const uint2 *>(sgp + 32 * ks + 16);
          const u32x4 m = {lo.x, lo.y, hi.x, hi.y};
          bo[ks] = __builtin_bit_cast(CG, __builtin_bit_cast(u32x4, bo[ks]) ^ m);
          bo[2 + ks] = __builtin_bit_cast(CG, __builtin_bit_cast(u32x4, bo[2 + ks]) ^ m);
        }
      }
    };
    // Gradient product over streamed block xb for this wave's half of D:
    // dR^T[d, resident] += X^T[d, streamed] * dS[streamed, resident].
    auto grad = [&](const char *base, int xb, const CG(&bo)[4]) {
      const int j16 = lane & 15, grp = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < Tr::NDH; ++db) {
          const int rb = xb * 32 + 16 * ks + 4 * (grp >> 1) + (j16 >> 2);
          const int d0 = (e * Tr::NDH + db) * 32 + 16 * (grp & 1) + 4 * (j16 & 3);
          const char *t1 = base + rb * Tr::XROW + d0 * 2;
          const char *t2 = t1 + Tr::XROW_BYTES;
          const f16x4 l1 = lds_read_tr16(t1), h1 = lds_read_tr16(t1 + 8 * Tr::XROW);
          const f16x4 l2 = lds_read_tr16(t2), h2 = lds_read_tr16(t2 + 8 * Tr::XROW);
          const CG a1 = __builtin_shufflevector(l1, h1, 0, 1, 2, 3, 4, 5, 6, 7);
          const CG a2 = __builtin_shufflevector(l2, h2, 0, 1, 2, 3, 4, 5, 6, 7);
          acc1[db] = mma16(a1, bo[ks], acc1[db]);
          acc2[db] = mma16(a2, bo[2 + ks], acc2[db]);
        }
      }
    };

    auto run_tiles = [&](int t0, int t1, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      for (int t = t0; t < t1; ++t) {
        const char *base = smem + (t & 1) * Tr::STAGE_BYTES;
        const int xt = x_of(t);
        const bool own_live = !MASK || !empty_blk(xt + 32 * e);
        const bool par_live = !MASK || !empty_blk(xt + 32 * (1 - e));
        CG bo[4];
        if (own_live) {
          dsblock(base, e, xt + 32 * e, mask_tag, bo);
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<CG *>(own_slot + i * Tr::DSX_SLOT) = bo[i];
        }
        __syncthreads();
        // The next stage's global loads overlap the gradient products.
        if (t + 1 < ntiles) gload(t + 1);
        if (own_live) grad(base, e, bo);
        if (par_live) {
          CG pb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pb[i] = *reinterpret_cast<const CG *>(par_slot + i * Tr::DSX_SLOT);
          grad(base, 1 - e, pb);
        }
        if (t + 1 < ntiles) sstore((t + 1) & 1);
        __syncthreads();
      }
    };
    run_tiles(0, t_a, std::true_type{});
    run_tiles(t_a, t_b, std::false_type{});
    run_tiles(t_b, ntiles, std::true_type{});

    // Epilogue: lane writes its resident row, d = (e*NDH + db)*32 + 8j + 4h + (0..3).
    if (r_ok) {
      const float f = p.scale / sigma * (KEYS_RES ? 1.f : qsg);
      float *O1 = KEYS_RES ? p.dk1 : p.dq1;
      float *O2 = KEYS_RES ? p.dk2 : p.dq2;
      const int64_t rowoff = (bh * (int64_t)NR + my_r) * D;
#pragma unroll
      for (int db = 0; db < Tr::NDH; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = (e * Tr::NDH + db) * 32 + 8 * j + 4 * h;
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
  }
}

// sigma[b,h] = 2^(kGradExp - e) with 2^(e-1) <= max_i |g[b,h,i]| < 2^e (1 if g is all zero,
// and 1 everywhere when `unit` is set: fp32 inputs need no scaling), stored
// negated when some g[b,h,:] is negative.
__global__ __launch_bounds__(256) void grad_scale_kernel(const float *g, int64_t NQ, float *sigma, int unit) {
  const int64_t bh = blockIdx.x;
  if (unit) {
    // fp32 inputs: no dS scaling, but the sign flag is still needed.
    const float *gu = g + bh * NQ;
    int neg = 0;
    for (int64_t i = threadIdx.x; i < NQ; i += 256) neg |= gu[i] < 0.f;
    neg = __syncthreads_or(neg);
    if (threadIdx.x == 0) sigma[bh] = neg ? -1.f : 1.f;
    return;
  }
  const float *gp = g + bh * NQ;
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

__global__ __launch_bounds__(256) void zero_kernel(float *dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = 0.f;
}

template <typename T, int D, bool KEYS_RES>
static hipError_t launch_pass(const BwdParams &p, hipStream_t s) {
  using Tr = BwdTraits<T, D, KEYS_RES>;
  const int64_t NR = KEYS_RES ? p.NK : p.NQ;
  if (NR == 0) return hipSuccess;
  const void *fn = reinterpret_cast<const void *>(&bwd_kernel<T, D, KEYS_RES>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nblk = p.BH * ((NR + Tr::BR - 1) / Tr::BR);
  hipLaunchKernelGGL((bwd_kernel<T, D, KEYS_RES>), dim3((uint32_t)nblk), dim3(256), Tr::LDS_BYTES, s, p);
  return hipGetLastError();
}

hipError_t launch_grad_scale(int dtype, const float *g, int64_t BH, int64_t NQ, float *sigma, hipStream_t s) {
  hipLaunchKernelGGL(grad_scale_kernel, dim3((uint32_t)BH), dim3(256), 0, s, g, NQ, sigma, dtype == 1 ? 1 : 0);
  return hipGetLastError();
}

template <int D, bool KEYS_RES>
static hipError_t launch_pass2(const BwdParams &p, hipStream_t s) {
  using Tr = Bwd2Traits<D, KEYS_RES>;
  const int64_t NR = KEYS_RES ? p.NK : p.NQ;
  if (NR == 0) return hipSuccess;
  const void *fn = reinterpret_cast<const void *>(&bwd2_kernel<D, KEYS_RES>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Tr::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nblk = p.BH * ((NR + Tr::BR - 1) / Tr::BR);
  hipLaunchKernelGGL((bwd2_kernel<D, KEYS_RES>), dim3((uint32_t)nblk), dim3(Tr::NT), Tr::LDS_BYTES, s, p);
  return hipGetLastError();
}

#ifdef SKL_BWD_ONE_WAVE
#define SKL_BF16_PASS(D, KR) launch_pass<bf16, D, KR>(p, s)
#else
#define SKL_BF16_PASS(D, KR) launch_pass2<D, KR>(p, s)
#endif

hipError_t launch_bwd_dk(int dtype, int D, const BwdParams &p, hipStream_t s) {
  if (dtype == 0) return D == 128 ? SKL_BF16_PASS(128, true) : SKL_BF16_PASS(64, true);
  return D == 128 ? launch_pass<float, 128, true>(p, s) : launch_pass<float, 64, true>(p, s);
}

hipError_t launch_bwd_dq(int dtype, int D, const BwdParams &p, hipStream_t s) {
  if (dtype == 0) return D == 128 ? SKL_BF16_PASS(128, false) : SKL_BF16_PASS(64, false);
  return D == 128 ? launch_pass<float, 128, false>(p, s) : launch_pass<float, 64, false>(p, s);
}

hipError_t launch_zero(float *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t nblk = (n + 255) / 256;
  if (nblk > 65536) nblk = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3((uint32_t)nblk), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace skl
