// gdn_chunk_common.hpp -- pieces shared by the sequential chunk kernels
// (scalar gate: gdn_chunk.hip; per-key-channel gate: gdn_kda.hip): direct
// global->LDS loads, LDS-only barriers, the gfx950 LDS transpose read, the
// bf16 and fp32 operand engines, the key-channel relabelling of the state
// and the kernel arguments.
#pragma once

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr float kLog2e = 1.4426950408889634f;

struct Frag8 {
  float v[8];
};

// Direct global -> LDS copy: lane l of the wave writes the 16 bytes at
// base + off (base the same in every lane, off this lane's byte offset) to
// LDS byte address lds + 16 l; lds must be the same in every lane.  Issued
// from inline assembly so that the compiler does not hold later LDS accesses
// of the wave behind it: the kernel orders these copies itself, with
// wait_vmem() before the barrier that publishes them.  M0 (the LDS base of
// the copy) is restored.
__device__ __forceinline__ void lds_load16(const void* base, uint32_t off, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  // readfirstlane returns int: widen each half through uint32_t (no sign extension)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)base >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(sb), "s"(m)
      : "memory");
}
// E4M3 codes of four state values at scale s (r = RN(1 / s)), as floats:
// the correctly rounded quotient x / s (div_rn) converted to the nearest
// OCP E4M3FN value, ties to even, by v_cvt_pk_fp8_f32, and back two at a
// time.  The conversion keeps the sign of values that round to zero (-0),
// so code * s has the sign of x without a copysign.
__device__ __forceinline__ void e4m3_codes4(const f32x4& x, float s, float r, float (&c)[4]) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(div_rn(x[0], s, r), div_rn(x[1], s, r), 0, false);
  const int p = __builtin_amdgcn_cvt_pk_fp8_f32(div_rn(x[2], s, r), div_rn(x[3], s, r), lo, true);
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(p, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(p, true);
  c[0] = a[0];
  c[1] = a[1];
  c[2] = b[0];
  c[3] = b[1];
}


// LDS byte address of a pointer into the dynamic LDS block that starts at
// smem, from the block's own address (one cast per kernel, the rest is
// uniform integer arithmetic).
__device__ __forceinline__ uint32_t lds_base_u32(const char* smem) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)smem);
}
// Wait until this wave's outstanding vector memory operations (including
// direct LDS loads) have completed.  The asm wait covers the direct loads
// (issued from asm, so the compiler does not count them); the same wait as a
// builtin tells the compiler's wait-count tracking that nothing is in flight
// after it (an asm wait is opaque to it), so that it adds no waits for loads
// that have long completed (which on gfx9 would also wait for stores).
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited
}
// Workgroup barrier that orders LDS accesses only: it does not wait for the
// wave's direct LDS loads or global memory operations in flight.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// gfx950 LDS transpose read of 16-bit data: inside each group of 16 lanes,
// lane i receives, in its slot k (k = 0..3), element i % 4 of the 8 bytes
// addressed by lane 4k + i / 4 of the same group.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) char*)p));
  return __builtin_bit_cast(uint2, r);
}
// Slot of lane l inside a k/q fragment dump: each block of 16 lanes is
// rotated by 4 per block so that the transpose reads of the state update hit
// different banks.
__device__ __forceinline__ int rot_slot(int l) { return (l & 48) | ((l + ((l >> 4) << 2)) & 15); }
__device__ __forceinline__ int rot_lane(int p) { return (p & 48) | ((p - ((p >> 4) << 2)) & 15); }

// bf16 engine: LDS operands are bf16 bit patterns, fragments 8 x bf16.
struct EngBF16 {
  using E = uint16_t;
  using Fr = bf16x8;
  static constexpr bool kSplit = true;
  static constexpr int kPlanes = 2;     // hi and lo planes of split operands
  static constexpr bool kTrRead = true; // K^T fragments by LDS transpose reads
  static __device__ __forceinline__ Fr ld(const E* p) { return *reinterpret_cast<const Fr*>(p); }
  static __device__ __forceinline__ void st(E* p, const Fr& f) { *reinterpret_cast<Fr*>(p) = f; }
  static __device__ __forceinline__ void mma(f32x4& c, const Fr& a, const Fr& b) { mma_bf16(c, a, b); }
  static __device__ __forceinline__ Fr round(const float (&x)[8]) {
    return __builtin_bit_cast(Fr, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                             pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
  }
  static __device__ __forceinline__ void split(const float (&x)[8], Fr& hi, Fr& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split_bf16x2(x[2 * j], x[2 * j + 1], h[j], l[j]);
    hi = __builtin_bit_cast(Fr, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(Fr, make_uint4(l[0], l[1], l[2], l[3]));
  }
  // three planes: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid)
  // (24 significant bits)
  static __device__ __forceinline__ void split3(const float (&x)[8], Fr& hi, Fr& mid, Fr& lo) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split3_bf16x2(x[2 * j], x[2 * j + 1], h[j], m[j], l[j]);
    hi = __builtin_bit_cast(Fr, make_uint4(h[0], h[1], h[2], h[3]));
    mid = __builtin_bit_cast(Fr, make_uint4(m[0], m[1], m[2], m[3]));
    lo = __builtin_bit_cast(Fr, make_uint4(l[0], l[1], l[2], l[3]));
  }
  // fragment from two 4-element pieces (k slots 0..3 and 4..7)
  static __device__ __forceinline__ Fr ld2(const E* a, const E* b) {
    const uint2 u = *reinterpret_cast<const uint2*>(a);
    const uint2 v = *reinterpret_cast<const uint2*>(b);
    return __builtin_bit_cast(Fr, make_uint4(u.x, u.y, v.x, v.y));
  }
  static __device__ __forceinline__ Fr pack8(const E (&x)[8]) {
    return __builtin_bit_cast(Fr, make_uint4((uint32_t)x[0] | ((uint32_t)x[1] << 16),
                                             (uint32_t)x[2] | ((uint32_t)x[3] << 16),
                                             (uint32_t)x[4] | ((uint32_t)x[5] << 16),
                                             (uint32_t)x[6] | ((uint32_t)x[7] << 16)));
  }
  static __device__ __forceinline__ float to_f(E x) { return bf16_bits_to_float(x); }
  // four values -> hi at ph, lo at pl
  static __device__ __forceinline__ void st4_split(E* ph, E* pl, const float (&x)[4]) {
    uint32_t h0, l0, h1, l1;
    split_bf16x2(x[0], x[1], h0, l0);
    split_bf16x2(x[2], x[3], h1, l1);
    *reinterpret_cast<uint2*>(ph) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(pl) = make_uint2(l0, l1);
  }
};

// fp32 engine: LDS operands are fp32, fragments 8 x fp32, products on the fp32 MFMA.
struct EngF32 {
  using E = float;
  using Fr = Frag8;
  static constexpr bool kSplit = false;
  static constexpr int kPlanes = 1;
  static constexpr bool kTrRead = false; // K^T fragments from a gathered dump
  static __device__ __forceinline__ Fr ld(const E* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    Fr f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  static __device__ __forceinline__ void st(E* p, const Fr& f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
  }
  static __device__ __forceinline__ void mma(f32x4& c, const Fr& a, const Fr& b) { mma_f32(c, a.v, b.v); }
  static __device__ __forceinline__ Fr round(const float (&x)[8]) {
    Fr f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    return f;
  }
  static __device__ __forceinline__ void split(const float (&x)[8], Fr& hi, Fr& lo) {
    hi = round(x);
    (void)lo;
  }
  static __device__ __forceinline__ void split3(const float (&x)[8], Fr& hi, Fr& mid, Fr& lo) {
    hi = round(x);
    (void)mid;
    (void)lo;
  }
  static __device__ __forceinline__ Fr ld2(const E* a, const E* b) {
    const float4 u = *reinterpret_cast<const float4*>(a);
    const float4 v = *reinterpret_cast<const float4*>(b);
    Fr f;
    f.v[0] = u.x; f.v[1] = u.y; f.v[2] = u.z; f.v[3] = u.w;
    f.v[4] = v.x; f.v[5] = v.y; f.v[6] = v.z; f.v[7] = v.w;
    return f;
  }
  static __device__ __forceinline__ Fr pack8(const E (&x)[8]) { return round(x); }
  static __device__ __forceinline__ float to_f(E x) { return x; }
  static __device__ __forceinline__ void st4_split(E* ph, E* pl, const float (&x)[4]) {
    (void)pl;
    *reinterpret_cast<float4*>(ph) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

// A fragment of bf16 values (the W codes) as the engine's operand.
template <class Eng>
__device__ __forceinline__ typename Eng::Fr ld_bf16_frag(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  if constexpr (Eng::kSplit) {
    return __builtin_bit_cast(typename Eng::Fr, u);
  } else {
    typename Eng::Fr f;
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f.v[2 * q] = __uint_as_float(w4[q] << 16);
      f.v[2 * q + 1] = __uint_as_float(w4[q] & 0xffff0000u);
    }
    return f;
  }
}

// Key-channel order of the state.  The chain waves hold S^T in accumulator
// tiles whose rows are "state rows" sr = 16 t + 4 (l/16) + i; state row sr
// carries key channel
//     dkmap(sr) = 32 (sr / 32) + 8 ((sr % 16) / 4) + 4 ((sr / 16) % 2) + sr % 4.
// With this relabelling the eight k-slots kperm(gq, 0..7) of k-block kb,
// state rows 32 kb + kperm(gq, j), are the key channels 32 kb + 8 gq + j: a K
// or Q fragment lane holds 8 consecutive channels of one row, 16 contiguous
// bytes of the input, so the fragment dumps below are filled by direct
// 16-byte global->LDS loads.  Contractions over the key axis (K S^T, S Q^T,
// Q K^T) only need both operands in the same order; the relabelling is undone
// where the state meets memory.
__host__ __device__ constexpr int dkmap(int sr) {
  return 32 * (sr / 32) + 8 * ((sr % 16) / 4) + 4 * ((sr / 16) % 2) + sr % 4;
}

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* prefix_lens;
  const int32_t* chunk_offs;  // prefix sums of ceil(P_n / 64) (prep kernel)
  const void* T;              // one T record per (chunk, head) (prep kernel or producer workgroups)
  const void* Prec;           // one P record per (chunk, head), the same way
  const void* Wrec;           // W QDQ: one W record per (chunk, head), the same way
  float* w_pre;               // optional debug record of W (producer workgroups)
  float* w_post;
  const float* init;
  void* o;
  float* fin;
  const int32_t* bound_offsets;
  float* bound_pre;
  float* bound_post;
  float* bound_scales;
  int H;
  int dv;
  unsigned flags;
  int N;               // sequences
  int fused;           // the fused instantiation runs (its waits on the ready flags included)
  unsigned* ready;     // fused launch: one ready flag per (chunk, head), cleared before the launch
  int n_prep;          // fused launch: workgroups 0 .. n_prep - 1 produce the T and P records
  int prep_c0;         // fused launch: the producers start at this chunk of every sequence (the
                       // state workgroups form the chunks before it themselves)
  int32_t* status;     // the workspace's status word (index check, failed waits)
  int grid_log2;       // log-retention grid of the recurrent suffix (0: off)
  int longest_first;   // the state workgroups outnumber the compute units: workgroups take the
                       // sequences longest first (see rank_sequence)
  const int32_t* sfx_offsets;  // optional per-token record of the recurrent suffix:
  float* sfx_pre;              // state after each suffix token before its QDQ
  float* sfx_post;             // and after it ([sfx_offsets[n] + t - P_n, H, dv, dk])
};

// XCD (accelerator complex die) that runs the calling wave: hardware
// register XCC_ID, bits 3:0.  The dispatcher hands workgroup b of a launch
// to XCD b % 8; each XCD has its own L2.
__device__ __forceinline__ unsigned xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u; }

// Ready flag of a (chunk, head) record pair: bit 0 set once the records are
// complete, bits 4:1 the producer's XCD, bit 8 set when the producer also
// wrote its L2 back to memory (device-scope release).
constexpr unsigned kReadyReleased = 1u << 8;

// Bound of a consumer's wait for one ready flag: 200 ms of the 100 MHz
// real-time clock.
constexpr uint64_t kReadyWaitTicks = 20000000;

// Consumer side of the fused launch: wait (bounded) for the ready flag at
// flag, whose first reading is v0, then make the record readable.  A record
// written on this XCD sits in the shared L2 and is read through an L1 that
// never held it in this launch; one written on another XCD needs the
// producer's device-scope release, and then this wave invalidates its caches
// (device-scope acquire).  Returns false when the wait runs out or the
// record cannot be trusted.  The caller's barriers order the other waves'
// record loads after it.
__device__ __forceinline__ bool await_ready_flag(const unsigned* flag, unsigned v0, unsigned xcd_self) {
  unsigned v = (unsigned)__builtin_amdgcn_readfirstlane((int)v0);
  if (v == 0u) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + kReadyWaitTicks;
    do {
      if (__builtin_amdgcn_s_memrealtime() > t_end) return false;
      __builtin_amdgcn_s_sleep(4);
      v = (unsigned)__builtin_amdgcn_readfirstlane(
          (int)__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    } while (v == 0u);
  }
  if (((v >> 1) & 15u) != xcd_self) {
    if (!(v & kReadyReleased)) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    wait_vmem();
  }
  return true;
}

// Longest first: when the state workgroups come in several rounds, the
// sequence that workgroup-rank r works on is the one of rank r by length
// (longest first, ties by index), so that the long chains start in the first
// round.  Every thread of the workgroup takes part; `slot` is one LDS word.
// O(N^2 / blockDim) comparisons, so the host asks for it only for modest N.
__device__ __forceinline__ int rank_sequence(const int32_t* cu, const int32_t* seq_lens, int N, int r, int* slot) {
  auto len = [&](int m) { return seq_lens ? seq_lens[m] : (cu[m + 1] - cu[m]); };
  if (threadIdx.x == 0) *slot = 0;
  __syncthreads();
  for (int m = threadIdx.x; m < N; m += blockDim.x) {
    const int lm = len(m);
    int rank = 0;
    for (int j = 0; j < N; ++j) {
      const int lj = len(j);
      rank += (lj > lm || (lj == lm && j < m)) ? 1 : 0;
    }
    if (rank == r) *slot = m;
  }
  __syncthreads();
  const int n = *slot;
  __syncthreads();  // the word is free again
  return n;
}

// True when the index check of this call failed (the status word that
// chunk_offsets_kernel wrote earlier on the stream); the caller then returns
// without touching memory.
__device__ __forceinline__ bool index_check_failed(const int32_t* status) {
  return status != nullptr && (__builtin_amdgcn_readfirstlane(*status) & kStatusBadIndex) != 0;
}

// A consumer's bounded wait ran out: record it in the status word (vector
// atomic; several workgroups may report).
__device__ __forceinline__ void report_wait_timeout(int32_t* status) {
  if (status != nullptr) __hip_atomic_fetch_or(status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The sequential kernel for a per-key-channel gate (gdn_kda.hip); the prep
// kernel has filled a.T and a.Prec.
hipError_t launch_kda_state(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream);
// the scalar-gate state part for bf16 q, k, v without W QDQ (gdn_chunk_bf16.hip)
hipError_t launch_chunk_bf16(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream);
// fp32 q, k, v with dk = 128, either gate, no W QDQ: the token recurrence
// with the chunked form's QDQ points (gdn_token.hip)
hipError_t launch_chunk_token(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream);

}  // namespace gdn
