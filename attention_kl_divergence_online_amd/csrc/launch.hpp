// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Host-only declarations; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

struct FwdParams {
  const void *q1, *k1, *q2, *k2;  // [BH, NQ|NK, D] in the input dtype
  float *kl, *lse1, *lse2;         // [BH, NQ]
  float *ws;                       // split-K partial states [5][splits][BH*NQ], else null
  int64_t BH, NQ, NK;
  float scale;
  int causal;
  int nqt;     // query tiles per head
  int splits;  // key chunks (1 = unsplit)
  int chunk;   // keys per chunk (multiple of the key tile)
};

struct BwdParams {
  const void *q1, *k1, *q2, *k2;
  const float *kl, *lse1, *lse2, *g;
  const float *sigma;  // per (b,h) power-of-two factor applied to g (null: 1)
  // bf16 inputs: prepared transposed fp16 copies [BH][ceil(N/64)][D][64] (null for fp32)
  const void *tq1, *tq2, *tk1, *tk2;
  float *dq1, *dk1, *dq2, *dk2;
  int64_t BH, NQ, NK;
  float scale;
  int causal;
  int want1, want2;  // write teacher / student gradients
};

// Tile sizes the host needs for grids and validation.
constexpr int kFwdBK = 64;    // keys per forward stage (split chunks are multiples)
constexpr int kBwdBR = 128;   // resident rows per backward workgroup
constexpr int kBwdTile = 64;  // streamed rows per backward stage (tile of the transposed copies)
constexpr int kGradExp = 8;   // |g| * sigma <= 2^kGradExp before fp16 rounding of dS

// Queries per forward workgroup for an input type (dtype: 0 = bf16, 1 = fp32).
int fwd_block_queries(int dtype, int D);

// dtype: 0 = bf16, 1 = fp32.  Return the launch status.
hipError_t launch_fwd(int dtype, int D, const FwdParams &p, hipStream_t s);
hipError_t launch_splitk_merge(const FwdParams &p, hipStream_t s);
// Backward pieces; `p.sigma` must point at the prepared per-(b,h) factors.
hipError_t launch_grad_scale(int dtype, const float *g, int64_t BH, int64_t NQ, float *sigma, hipStream_t s);
hipError_t launch_bwd_dk(int dtype, int D, const BwdParams &p, hipStream_t s);
hipError_t launch_bwd_dq(int dtype, int D, const BwdParams &p, hipStream_t s);
hipError_t launch_zero(float *dst, int64_t n, hipStream_t s);
// bf16 inputs: transposed fp16 copy of x [BH, N, D] into out [BH][ceil(N/64)][D][64].
hipError_t launch_bwd_transpose(int D, const void *x, int64_t BH, int64_t N, void *out, hipStream_t s);

}  // namespace skl
