// Device-side building blocks shared by the attention-KL kernels (gfx950 / CDNA4).
//
// Matrix-core convention used throughout: every contraction is issued as
// 32x32 output blocks, 16 contraction elements per step.  In a step each lane
// supplies 8 consecutive contraction elements for one row of A (lane % 32)
// and one column of B (lane % 32); lane half h = lane / 32 supplies elements
// [8h, 8h+8) of the step.  Any assignment of contraction indices to (h, slot)
// pairs is valid as long as A and B use the same one, which lets the
// accumulator of one product feed the next product without a transpose.
//
// Accumulator layout of a 32x32 block (16 fp32 per lane): element r of lane l
// holds row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max start value: finite so that (m_old - m_new) never forms inf - inf.
constexpr float kNegBig = -3.0e38f;

// Eight consecutive contraction elements of one operand row, as one lane holds them.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> { using type = bf16x8; };
template <> struct Chunk<f16> { using type = f16x8; };
template <> struct Chunk<float> { using type = f32x8; };
template <typename T> using chunk_t = typename Chunk<T>::type;

// C += A * B for one 16-deep contraction step of a 32x32 block.
__device__ __forceinline__ f32x16 mma16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// fp32 inputs: eight 32x32x2 steps; slot u of both lane halves forms step u.
__device__ __forceinline__ f32x16 mma16(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int u = 0; u < 8; ++u) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], b[u], c, 0, 0, 0);
  return c;
}

// fp8 e4m3 operands (32 per lane): C += A * B for one 64-deep contraction
// step of a 32x32 block, with byte j of lane (h, c) of A meeting byte j of
// lane (h, c') of B.  No block scales (the unscaled form).
__device__ __forceinline__ f32x16 mma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// Two 16-byte pieces as one 32-byte operand (lo first).
__device__ __forceinline__ i32x8 join16(u32x4 lo, u32x4 hi) {
  return i32x8{(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
               (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row of the 32x32 accumulator block held in element r by lane half h.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Loads 8 consecutive elements (16 B for 2-byte types, 32 B for fp32) from an
// aligned address.
template <typename T>
__device__ __forceinline__ chunk_t<T> load_chunk(const T* p) {
  return *reinterpret_cast<const chunk_t<T>*>(p);
}

// Work-group id remap so that consecutive logical ids land on the same XCD:
// the dispatcher hands workgroup w to XCD w % 8, so logical id
// (w % 8) * (n / 8) + w / 8 gives each XCD a contiguous run of logical ids.
// Only applied when n is a multiple of 8 (otherwise identity).
constexpr int kXcds = 8;
// Causal launches with at most this many query (forward) or resident
// (backward) tiles per head order their workgroups longest first across the
// heads of an XCD rather than head by head.
constexpr int kLongestFirstTiles = 64;
__device__ __forceinline__ uint32_t xcd_remap(uint32_t w, uint32_t n) {
  if ((n & 7u) != 0u) return w;
  return (w & 7u) * (n >> 3) + (w >> 3);
}

// Word 3 of a raw buffer resource (no stride, no swizzle, dword data format):
// reads past num_records return zero.
constexpr int kRawBuffer = 0x00020000;

// A byte range read through a raw buffer resource.
struct BufRange {
  const void *base;
  int bytes;
};
// 16 bytes per lane from range `r` at byte voff + soff into LDS at
// lds + 16 * lane (lds must be the same for the whole wave); bytes past the
// range read as zero.
__device__ __forceinline__ void buffer_load_lds16(BufRange r, char *lds, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(r.base), 0, r.bytes,
                                                                      kRawBuffer);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}
// 16 bytes per lane from range `r` at byte voff + soff into registers; bytes
// at or past the range end read as zero (the range check counts soff).
__device__ __forceinline__ u32x4 buffer_load16(BufRange r, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(r.base), 0, r.bytes,
                                                                      kRawBuffer);
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
}

// XOR swizzles of the 16-byte chunks within a row, chosen so that the 16 lanes
// reading one logical chunk of 16 consecutive rows hit 16 distinct slots of a
// 256-byte bank row.
template <int D> __device__ __forceinline__ int swz_row(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);  // 256- or 128-byte rows
}
// The same by row length in bytes (256, 128 or 64; 64-byte rows: four
// chunks, four rows per bank row).
template <int RB> __device__ __forceinline__ int swz_bytes(int r) {
  static_assert(RB == 256 || RB == 128 || RB == 64, "row bytes");
  return RB == 256 ? (r & 15) : RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

}  // namespace skl
