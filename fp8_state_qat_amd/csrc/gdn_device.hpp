// gdn_device.hpp -- device helpers for the gfx950 gated delta rule kernels:
// E4M3 rounding, fixed-order reductions, bf16 conversion and the MFMA
// fragment conventions shared by the chunk kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kChunk = 64;     // tokens per chunk
constexpr int kTileRows = 64;  // value rows per QDQ tile
constexpr int kThreads = 256;  // 4 waves of 64

// ---------------------------------------------------------------------------
// OCP E4M3FN rounding in the value domain.  Returns the E4M3 value nearest to
// y (ties to the even code), saturating at +-448.  Normals (|y| >= 2^-6) keep
// 3 mantissa bits: add half an E4M3 ulp minus one plus the kept LSB, then
// clear the 20 dropped bits (round to nearest even on the bit pattern).
// Below 2^-6 the grid is the multiples of 2^-9: y * 2^9 is exact, rintf
// rounds to nearest even.  NaN propagates.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_rne(float y) {
  float a = fabsf(y);
  float r;
  if (a >= 0.015625f) {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    b &= 0xFFF00000u;
    r = fminf(__uint_as_float(b), 448.0f);
  } else {
    r = rintf(a * 512.0f) * 0.001953125f;
  }
  return copysignf(r, y);
}

// QDQ scale of a tile: amax / 448 as an IEEE division, 1 when not positive.
__device__ __forceinline__ float qdq_scale(float amax) {
  float s = amax / 448.0f;
  return (s > 0.0f) ? s : 1.0f;
}

// x -> RNE_E4M3(x / s) * s, both operations IEEE fp32.
__device__ __forceinline__ float qdq_value(float x, float s) { return e4m3_rne(x / s) * s; }

// ---------------------------------------------------------------------------
// Reductions in a fixed order (the same tree on every call).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Max over the 256 threads of a block; red must hold 4 floats of LDS.  All
// threads return the same value.  Contains two barriers.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ __bf16 to_bf16(float x) {
  return __builtin_bit_cast(__bf16, float_to_bf16_bits(x));
}
__device__ __forceinline__ float from_bf16(__bf16 x) {
  return bf16_bits_to_float(__builtin_bit_cast(uint16_t, x));
}

// Element loads/stores by I/O type.
template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float x) { *p = x; }
};
template <> struct io<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf16_bits_to_float(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float x) { *p = float_to_bf16_bits(x); }
};

// ---------------------------------------------------------------------------
// MFMA conventions (16 x 16 output tiles, wave64).
//
// Accumulator tile C (16 x 16): lane l holds C[4*(l/16) + i][l % 16], i = 0..3.
// Contractions run in k-blocks of 32.  Inside a k-block, lane group
// gq = l / 16 owns the eight k indices
//     kperm(gq, j) = 4*gq + j            (j = 0..3)
//                  = 16 + 4*gq + (j - 4)  (j = 4..7)
// for both operands: the A fragment of lane l holds A[l % 16][kperm(gq, j)],
// the B fragment B[kperm(gq, j)][l % 16].  Because both operands use the same
// permutation the product is the plain sum over k.  This permutation is the
// one in which two vertically stacked accumulator tiles (rows 0..15 and
// 16..31) already sit in a lane, so an accumulator can feed the next
// contraction as its B operand straight from registers.
//
// bf16 engine: one v_mfma_f32_16x16x32_bf16 per k-block (the instruction
// pairs A and B element j of the same lane group).
// fp32 engine: eight v_mfma_f32_16x16x4_f32 per k-block; instruction j takes
// element j of every lane (lane group gq supplies k = kperm(gq, j)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma_bf16(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void mma_f32(f32x4& c, const float (&a)[8], const float (&b)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

}  // namespace gdn
