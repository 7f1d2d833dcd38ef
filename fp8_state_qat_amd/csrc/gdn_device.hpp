// gdn_device.hpp -- device helpers for the gfx950 gated delta rule kernels:
// E4M3 rounding, fixed-order reductions, bf16 conversion and the MFMA
// fragment conventions shared by the chunk kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
// Non-temporal 16-byte accesses, for state tiles that are read once and
// written once per call and fit no cache level.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(float4* p, float4 x) {
  const f32x4_nt v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_nt*>(p));
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr int kChunk = 64;     // tokens per chunk
constexpr int kTileRows = 64;  // value rows per QDQ tile
constexpr int kThreads = 256;  // 4 waves of 64

// ---------------------------------------------------------------------------
// State QDQ arithmetic, IEEE fp32 throughout:
//   s = amax / 448 (IEEE division; 1 when not positive, the zero guard)
//   y = x / s      (IEEE division, computed as below)
//   c = E4M3FN value nearest to y, ties to even (hardware conversion)
//   x <- c * s     (sign of x kept for zeros)
//
// x / s is evaluated from r = RN(1 / s) (one IEEE division per tile): q = x r
// is within about 1.5 ulp of x / s, and each step q <- q + r (x - s q), with
// the remainder x - s q exact in an fma, is Markstein's correction; after two
// steps q is the correctly rounded quotient (results in the fp32 subnormal
// range, which all map to code 0, excepted).
// ---------------------------------------------------------------------------
// Log-gate of a recurrent write on the log-retention grid 2^-k (k = 0: as
// given): the nearest multiple of 2^-k, ties to even.  Scaling by a power of
// two and rint are exact in fp32, so the result is a function of g alone.
__device__ __forceinline__ float grid_gate(float g, int k) {
  return k ? ldexpf(__builtin_rintf(ldexpf(g, k)), -k) : g;
}

__device__ __forceinline__ float qdq_scale(float amax) {
  float s = amax / 448.0f;
  return (s > 0.0f) ? s : 1.0f;
}

__device__ __forceinline__ float div_rn(float x, float s, float r) {
  float q = x * r;
  float e = fmaf(-s, q, x);
  q = fmaf(e, r, q);
  e = fmaf(-s, q, x);
  return fmaf(e, r, q);
}

// QDQ of two values with scale s and r = RN(1 / s); c0, c1 receive the E4M3
// values (the codes as floats).  gfx950's v_cvt_pk_fp8_f32 rounds to the
// nearest OCP E4M3FN value (ties to even).
__device__ __forceinline__ void qdq2c(float& x0, float& x1, float s, float r, float& c0, float& c1) {
  const float y0 = div_rn(x0, s, r), y1 = div_rn(x1, s, r);
  const int p = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  c0 = __builtin_amdgcn_cvt_f32_fp8(p, 0);
  c1 = __builtin_amdgcn_cvt_f32_fp8(p, 1);
  x0 = copysignf(c0 * s, x0);
  x1 = copysignf(c1 * s, x1);
}

__device__ __forceinline__ void qdq2(float& x0, float& x1, float s, float r) {
  float c0, c1;
  qdq2c(x0, x1, s, r, c0, c1);
}

__device__ __forceinline__ void qdq4(float4& v, float s, float r) {
  qdq2(v.x, v.y, s, r);
  qdq2(v.z, v.w, s, r);
}

__device__ __forceinline__ void qdq4(f32x4& v, float s, float r) {
  float a = v[0], b = v[1], c = v[2], d = v[3];
  qdq2(a, b, s, r);
  qdq2(c, d, s, r);
  v = f32x4{a, b, c, d};
}

__device__ __forceinline__ void qdq4c(f32x4& v, float (&cv)[4], float s, float r) {
  float a = v[0], b = v[1], c = v[2], d = v[3];
  qdq2c(a, b, s, r, cv[0], cv[1]);
  qdq2c(c, d, s, r, cv[2], cv[3]);
  v = f32x4{a, b, c, d};
}

// The same codes from the quotients formed in fp64.  For fp32 x and s the
// quotient x / s is never within 2^-49 (relative) of a rounding boundary of
// fp32 without being on it, and it is never on one (a boundary has 25
// significant bits, x * 2^k / s would need them); the fp64 product x * r with
// r within 2^-52 of 1 / s is within 2^-51 of x / s, so its rounding to fp32
// is the correctly rounded quotient: three instructions per value where the
// fp32 corrections take five.
__device__ __forceinline__ double rcp_f64(float s) {
  const double d = s;
  double r = __builtin_amdgcn_rcp(d);  // relative error below 2^-22
  r = fma(r, fma(-d, r, 1.0), r);      // ... 2^-44
  return fma(r, fma(-d, r, 1.0), r);   // ... 2^-52
}
__device__ __forceinline__ float div_rn_f64(float x, double r) { return (float)((double)x * r); }
__device__ __forceinline__ void e4m3_codes4_f64(const f32x4& x, double r, float (&c)[4]) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(div_rn_f64(x[0], r), div_rn_f64(x[1], r), 0, false);
  const int p = __builtin_amdgcn_cvt_pk_fp8_f32(div_rn_f64(x[2], r), div_rn_f64(x[3], r), lo, true);
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(p, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(p, true);
  c[0] = a[0];
  c[1] = a[1];
  c[2] = b[0];
  c[3] = b[1];
}
// QDQ of four values through the fp64 quotients (r: 1 / s in fp64): x <- the
// E4M3 value of x / s times s, with the sign of x; cv receives the codes.
__device__ __forceinline__ void qdq4c_f64(f32x4& v, float (&cv)[4], float s, double r) {
  e4m3_codes4_f64(v, r, cv);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = copysignf(cv[i] * s, v[i]);
}
// The tile scale RN(amax / 448) (1 when amax is 0) through fp64: amax / 448 =
// amax / 7 / 64 is at least 2^-27 (relative) from any rounding boundary of
// fp32, and the product with the fp64 value of 1/448 is within 2^-52 of it.
// Where the quotient is subnormal it is either exactly a tie of fp32, which
// has few significant bits, so the fp64 product rounds onto it and the
// conversion breaks it to even as the division does, or at least 2^-33
// (relative) away from one (checked against the division for every amax of
// six binades down to the smallest subnormal).
__device__ __forceinline__ float qdq_scale_f64(float amax) {
  const float s = (float)((double)amax * (1.0 / 448.0));
  return (s > 0.0f) ? s : 1.0f;
}

// ---------------------------------------------------------------------------
// Reductions in a fixed order (the same tree on every call).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Max over the 64 lanes of a wave with DPP lane moves inside each row of 16
// lanes (quad swaps, then half-row and row mirrors) and the four row results
// read back as scalars.  Every lane returns the same value.
template <int kCtrl>
__device__ __forceinline__ float dpp_max(float v) {
  const int m = __builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(m));
}
// Max over each aligned group of 8 lanes; every lane of the group receives it.
__device__ __forceinline__ float lane8_max_dpp(float v) {
  v = dpp_max<0xB1>(v);      // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E>(v);      // quad_perm [2, 3, 0, 1]
  return dpp_max<0x141>(v);  // row_half_mirror
}

// INT8 block QDQ of four values of one block with scale s and r = RN(1 / s):
// code = x / s (correctly rounded) rounded half to even (v_rndne_f32),
// clamped to [-127, 127], value = code * s.
__device__ __forceinline__ float int8_scale(float amax) {
  float s = amax / 127.0f;
  return (s > 0.0f) ? s : 1.0f;
}
__device__ __forceinline__ float qdq_int8_1(float x, float s, float r) {
  const float c = fminf(fmaxf(__builtin_rintf(div_rn(x, s, r)), -127.0f), 127.0f);
  return c * s;
}
__device__ __forceinline__ void qdq_int8_4(float4& v, float s, float r) {
  v.x = qdq_int8_1(v.x, s, r);
  v.y = qdq_int8_1(v.y, s, r);
  v.z = qdq_int8_1(v.z, s, r);
  v.w = qdq_int8_1(v.w, s, r);
}
// The same through fp64: the block scale fl32(amax * fl64(1/127)) equals
// fl32(amax / 127) (a 24-bit significand over 127 is never on an fp32
// rounding boundary and at least 2^-32 (relative) away from one; subnormal
// quotients as in qdq_scale_f64), and each quotient is the correctly rounded
// one as in qdq4c_f64.
__device__ __forceinline__ float int8_scale_f64(float amax) {
  const float s = (float)((double)amax * (1.0 / 127.0));
  return (s > 0.0f) ? s : 1.0f;
}
__device__ __forceinline__ void qdq_int8_4_f64(float4& v, float s) {
  const double r = rcp_f64(s);
  auto one = [&](float x) { return fminf(fmaxf(__builtin_rintf(div_rn_f64(x, r)), -127.0f), 127.0f) * s; };
  v.x = one(v.x);
  v.y = one(v.y);
  v.z = one(v.z);
  v.w = one(v.w);
}

// Max over each row of 16 lanes; every lane of the row receives it.
__device__ __forceinline__ float row16_max_dpp(float v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  return dpp_max<0x140>(v);  // row_mirror
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  v = dpp_max<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each
// row of 16 lanes with DPP row shifts, then the running row totals carried
// into the later rows with the row broadcasts.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  const int m = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false);
  return v + __int_as_float(m);
}
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum over each group of F consecutive lanes (F = 16 or 32, groups aligned),
// every lane of a group receiving it: quad swaps and rotations by 4 and 8
// inside each row of 16 lanes (DPP), then for F = 32 the two rows of each
// 32-lane half added, one row's sum brought to the other by
// v_permlane16_swap (in the vector ALU; the two operands of the last
// addition are the same in every lane, so each lane's sum is the same
// value).  The order of the additions is fixed.
template <int F>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(F == 16 || F == 32, "group of 16 or 32 lanes");
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x124, 0xF>(v);  // row_ror:4
  v = dpp_add<0x128, 0xF>(v);  // row_ror:8
  if constexpr (F == 32) {     // rows 2i and 2i + 1 of each half: swap and add
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// Max over the 256 threads of a block; red must hold 4 floats of LDS.  All
// threads return the same value.  Contains two barriers.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_dpp(v);
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
// Two values -> two bf16 (round to nearest even, one v_cvt_pk_bf16_f32),
// first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
// Residuals of a bf16 pair h = bf16x2(a, b): a - h.lo and b - h.hi, each one
// v_dot2_f32_bf16 of h with (-1, 0) or (0, -1) accumulated onto a or b.  The
// product is exact and the difference is exactly representable (h.lo is a
// rounded to 8 significant bits), so the result is the exact residual, the
// same bits as the unpack-and-subtract it replaces, in one instruction.  The
// two masks come from scalar registers set in asm: folded as constants, the
// (-1, 0) mask has been turned into the inline constant -1.0, whose 32-bit
// pattern is the (0, -1) mask.
__device__ __forceinline__ void bf16x2_residuals(uint32_t h, float a, float b, float& ra, float& rb) {
  uint32_t m_lo, m_hi;
  asm("s_mov_b32 %0, 0xbf80" : "=s"(m_lo));
  asm("s_mov_b32 %0, 0xbf800000" : "=s"(m_hi));
  const bf16x2 hv = __builtin_bit_cast(bf16x2, h);
  ra = __builtin_amdgcn_fdot2_f32_bf16(hv, __builtin_bit_cast(bf16x2, m_lo), a, false);
  rb = __builtin_amdgcn_fdot2_f32_bf16(hv, __builtin_bit_cast(bf16x2, m_hi), b, false);
}
// hi + lo split of two values: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  float ra, rb;
  bf16x2_residuals(hi, a, b, ra, rb);
  lo = pack_bf16x2(ra, rb);
}
// three planes of two values: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid)
__device__ __forceinline__ void split3_bf16x2(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  float ra, rb;
  bf16x2_residuals(hi, a, b, ra, rb);
  split_bf16x2(ra, rb, mid, lo);
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
