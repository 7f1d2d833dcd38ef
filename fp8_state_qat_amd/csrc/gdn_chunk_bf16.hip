// gdn_chunk_bf16.hip -- sequential part of the chunked gated delta rule
// forward with per-boundary FP8-E4M3 state QDQ for bf16 q, k, v (the
// Model-Optimizer pages: #2497 "What does this PR do?": 64-token chunks,
// WY/UT-transformed operands, dynamic per-tile state QDQ at every boundary;
// #2519: QDQ at the handoff and after every later recurrent write).  The
// scalar-gate kernel for bf16 inputs without W QDQ; fp32 inputs and W QDQ run
// in gdn_chunk.hip.
//
// Work unit: one workgroup of 8 waves per (sequence n, head h, 64-row value
// tile vt), walking its sequence chunk by chunk with its 64 x dk slice of the
// state in registers.  The tile is one QDQ tile, so its amax needs no other
// workgroup.  T and P of every chunk come through the workspace (prep kernel,
// or producer workgroups of the same launch).
//
// Waves 0..3 ("chain" waves) do all the arithmetic: chain wave c owns value
// rows 16c .. 16c+15 of the tile (dk/16 16x16 accumulator tiles of S^T) and
// forms both the state update and the outputs of those rows.  Waves 4..7
// ("loader" waves) stream the next chunk -- k, q, v, T, P and the gates --
// into the second half of double buffers and scan its gates, while the chain
// waves compute on the first half.  One workgroup barrier per chunk hands the
// buffers over.  Per chunk of n <= 64 tokens (rows past n are zero), with
// gamma the in-chunk cumulative log-gate and s the scale of the state
// entering it (1 when it is not coded):
//
//   acc  = K S^T                 (A: k rows from LDS, B: the state from registers)
//   oacc = S Q^T                 (A: the state from registers, B: q from LDS)
//   X    = V - s exp(gamma) * acc,      U' = T X          (T, X: three planes)
//   S^T <- exp(gamma_C) S^T + K^T diag(exp(gamma_C - gamma)) U'
//   O^T  = s exp(gamma) * oacc + U'^T P^T, stored to o
//   amax over the tile: each chain wave publishes its own in LDS before the
//   chunk's barrier; after it (at the start of the next chunk) the
//   QDQ: s = amax / 448, S <- RNE_E4M3(S / s) s, the codes kept as the state
//
// U' = T X is U - W S^T with U = T V and W = T (exp(gamma) * K) regrouped, so
// W is never formed.  The state's operand fragments in registers (B of K S^T)
// are also the A operand of S Q^T, and the accumulators of T X feed U'^T P^T
// and the update as A and B operands after splitting, so neither the state
// nor U' goes through LDS.
//
// Precision: q, k, v enter the MFMAs exactly; T, X and exp(gamma_C - gamma)
// U' as three bf16 planes (24 bits: the pre-QDQ state keeps fp32 accuracy
// and its E4M3 decisions match the oracle's except at ties); P and U' of the
// output as hi + lo.  After a QDQ the state is fed as its codes (exact in
// bf16) and the products are scaled by s; otherwise as hi + lo.
#include <type_traits>

#include "gdn_prep_item.hpp"

namespace gdn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreadsWg = 64 * kWaves;

// LDS layout (bytes).  A dump is 64 tokens x dk as 4 dk/32 fragments (64
// lanes x 8 bf16, lane-major), lane l of fragment (tt, kb) holding token
// 16tt + l%16, key channels 32kb + 8(l/16) .. +7 in slot rot_slot(l).
//   K, Q  2 x dump by chunk parity
//   V     2 x [64][64 + 8] bf16 rows (16 bytes of padding per row)
//   T     2 x the T record (three planes), P  2 x the P record (two planes)
//   vec   2 x 200 floats by chunk parity: [64..127] exp(gamma),
//         [128..191] exp(gamma_C - gamma), [192] exp(gamma_C)
//   red   [0..7] the chain waves' amax by chunk parity, [12] the decay
//         multiplier (1, or NaN once a wait for a record has run out)
//   O     2 x [64][64] bf16 by chunk parity: the chunk's outputs of the tile
//         (bf16 o), 16-byte piece u of row r at piece u ^ (r % 8), stored
//         to HBM by the loader waves as whole 128-byte rows
template <int DK>
struct LdsB {
  static constexpr int NKB = DK / 32;
  static constexpr size_t F = 1024;
  static constexpr size_t DUMP = 4 * NKB * F;
  static constexpr size_t RV = 64 * 2 + 16;
  static constexpr size_t VBUF = 64 * RV;
  static constexpr size_t oK = 0;
  static constexpr size_t oQ = oK + 2 * DUMP;
  static constexpr size_t oV = oQ + 2 * DUMP;
  static constexpr size_t oT = oV + 2 * VBUF;
  static constexpr size_t oP = oT + 2 * (size_t)kTRecBytes;
  static constexpr size_t oVec = oP + 2 * (size_t)kPRecBytes;
  static constexpr size_t VEC = 200;
  static constexpr size_t oRed = oVec + 2 * VEC * sizeof(float);
  static constexpr size_t OBUF = 64 * 64 * 2;
  static constexpr size_t oO = oRed + 16 * sizeof(float);
  static constexpr size_t bytes = oO + 2 * OBUF;
  static_assert(18 * F == (size_t)kTRecBytes && 12 * F == (size_t)kPRecBytes, "record geometry");
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
  static_assert(oK + (2 * DK + 64 + 8) * sizeof(float) <= oQ, "suffix buffers do not fit");
};

}  // namespace

// Instruction-order hints for the chain waves' scheduling regions: a group
// of kCount instructions of one kind (kMfma: matrix products, kValu: other
// vector ALU), placed in the order the hints are given.
// The chain is one serial dependence per chunk, so each vector ALU stage is
// placed beside matrix products it does not depend on.
constexpr int kMfma = 0x008, kValu = 0x002;
template <int kMask, int kCount>
__device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(kMask, kCount, 0);
}
template <int kCount, int kValuPer>
__device__ __forceinline__ void sched_interleave() {
#pragma unroll
  for (int i = 0; i < kCount; ++i) {
    sched_group<kMfma, 1>();
    sched_group<kValu, kValuPer>();
  }
}

template <int DK, typename TO, bool kFused>
__global__ __launch_bounds__(kThreadsWg, 1) void chunk_bf16_kernel(ChunkArgs args) {
  using Ls = LdsB<DK>;
  using Eng = EngBF16;
  using E = uint16_t;
  using Fr = bf16x8;
  using TIO = uint16_t;
  constexpr int NT = DK / 16;   // state accumulator tiles per chain wave
  constexpr int NKB = DK / 32;  // k-blocks over dk
  extern __shared__ __align__(16) char smem[];
  if (index_check_failed(args.status)) return;
  if constexpr (kFused) {
    if ((int)blockIdx.x < args.n_prep) {
      produce_records<DK, TIO, false>(args, smem);
      return;
    }
  }
  E* const sK = reinterpret_cast<E*>(smem + Ls::oK);
  E* const sQ = reinterpret_cast<E*>(smem + Ls::oQ);
  E* const sV = reinterpret_cast<E*>(smem + Ls::oV);
  E* const sT = reinterpret_cast<E*>(smem + Ls::oT);
  E* const sP = reinterpret_cast<E*>(smem + Ls::oP);
  float* const sVec = reinterpret_cast<float*>(smem + Ls::oVec);
  float* const sRed = reinterpret_cast<float*>(smem + Ls::oRed);
  float* const psn = sRed + 12;
  char* const sO = smem + Ls::oO;
  constexpr bool kStageO = sizeof(TO) == 2;  // bf16 o goes out through LDS

  const uint32_t lds0 = lds_base_u32(smem);
  auto lds_of = [&](const void* p) { return lds0 + (uint32_t)(reinterpret_cast<const char*>(p) - smem); };
  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63;
  const int gq = lane >> 4;
  const int ln = lane & 15;
  const bool chain = w < 4;
  const int c4 = w & 3;   // value block (16 rows) of a chain wave
  const int hw = w - 4;   // loader wave index
  auto slot = [lane](const E* base, int f) { return base + (f * 64 + lane) * 8; };
  const int qs = rot_slot(lane);
  auto qslot = [qs](const E* base, int f) { return base + (f * 64 + qs) * 8; };
  auto kpos = [](int t, int d) {  // element offset of k[t][d] in a dump
    return (((t >> 4) * NKB + (d >> 5)) * 64 + rot_slot(((d & 31) >> 3) * 16 + (t & 15))) * 8 + (d & 7);
  };
  constexpr int DUMPE = (int)(Ls::DUMP / 2);          // elements of one dump
  constexpr int VBUFE = (int)(Ls::VBUF / 2);
  constexpr int TRECE = kTRecBytes / 2, PRECE = kPRecBytes / 2;
  constexpr int RSV = 64 + 8;                         // padded v row stride (elements)

  const int H = args.H, dv = args.dv;
  const int tiles = dv / kTileRows;
  int nh, vt;  // the value tiles of a head on one XCD when heads come in groups of 8
  {
    const int b = (int)blockIdx.x - (kFused ? args.n_prep : 0);
    const int G = (int)gridDim.x - (kFused ? args.n_prep : 0);
    if (!kFused && args.longest_first) {
      const int per_seq = H * tiles;
      const int n0 = rank_sequence(args.cu_seqlens, args.seq_lens, args.N, b / per_seq, reinterpret_cast<int*>(smem));
      nh = n0 * H + (b % per_seq) / tiles;
      vt = b % tiles;
    } else if (tiles > 1 && G % (8 * tiles) == 0) {
      const int slot8 = b >> 3;
      vt = slot8 % tiles;
      nh = (slot8 / tiles) * 8 + (b & 7);
    } else {
      vt = b % tiles;
      nh = b / tiles;
    }
  }
  const int h = nh % H;
  const int n = nh / H;
  const int seg0 = args.cu_seqlens[n];
  const int seg1 = args.cu_seqlens[n + 1];
  const int L = args.seq_lens ? args.seq_lens[n] : (seg1 - seg0);
  const int P = args.prefix_lens ? args.prefix_lens[n] : L;
  const unsigned flags = args.flags;

  const TIO* gq_ = reinterpret_cast<const TIO*>(args.q);
  const TIO* gk_ = reinterpret_cast<const TIO*>(args.k);
  const TIO* gv_ = reinterpret_cast<const TIO*>(args.v);
  TO* go_ = reinterpret_cast<TO*>(args.o);
  const int64_t qk_row = (int64_t)H * DK;
  const int64_t v_row = (int64_t)H * dv;
  const int vcol0 = kTileRows * vt + 16 * c4 + ln;  // chain lane's value row of S (in dv)
  const int64_t state_base = ((int64_t)nh * dv + vcol0) * DK;

  const int n_chunks = (P + kChunk - 1) / kChunk;
  const int bound0 = args.bound_offsets ? args.bound_offsets[n] : 0;
  const int chunk0 = args.chunk_offs[n];

  // ---------------- loader waves: direct global -> LDS loads ----------------
  // Rows past a chunk's valid count load its last valid row: they meet zero
  // rows and columns of T and P, or outputs that are not stored.
  auto load_dump = [&](const TIO* src, E* dst, int nv) {  // src: the chunk's row 0, the head's column 0
    constexpr int NI = 4 * NKB;
#pragma unroll
    for (int ii = 0; ii < NI / 4; ++ii) {
      const int i = hw + 4 * ii;
      const int u = i * 64 + lane;
      const int f = u >> 6, l2 = rot_lane(u & 63);
      const int r = 16 * (f / NKB) + (l2 & 15);
      const int d = 32 * (f % NKB) + 8 * (l2 >> 4);
      lds_load16(src, (uint32_t)((min(r, nv - 1) * (int)qk_row + d) * 2), lds_of(dst) + i * 1024);
    }
  };
  auto load_rows = [&](const TIO* src, E* dst, int nv) {  // the tile's 64 v rows, padded
    constexpr int PPV = 8;                    // 16-byte pieces per row
    constexpr int RPI = 64 / (PPV + 1);       // rows per instruction
    constexpr int NI = (64 + RPI - 1) / RPI;  // instructions
    const int rr = lane / (PPV + 1), pc = lane % (PPV + 1);
    const int lane_off = min(pc, PPV - 1) * 8;
#pragma unroll
    for (int ii = 0; ii < (NI + 3) / 4; ++ii) {
      const int i = hw + 4 * ii;
      const int r = i * RPI + rr;
      if (i < NI && rr < RPI && r < 64)
        lds_load16(src, (uint32_t)((min(r, nv - 1) * (int)v_row + lane_off) * 2),
                   lds_of(dst) + i * RPI * (PPV + 1) * 16);
    }
  };
  auto load_record = [&](const char* rec, E* dst, int pieces) {  // pieces of 1 KiB
#pragma unroll
    for (int ii = 0; ii < 5; ++ii) {
      const int idx = hw + 4 * ii;
      if (idx < pieces) lds_load16(rec, (uint32_t)((idx * 64 + lane) * 16), lds_of(dst) + idx * 1024);
    }
  };
  float pg = 0.f;  // loader wave 0: log-gate of token `lane` of the chunk being loaded
  auto fetch_g = [&](int cc) {
    const int nv = min(kChunk, P - cc * kChunk);
    pg = args.g[(int64_t)(seg0 + cc * kChunk + min(lane, nv - 1)) * H + h];
  };
  auto scan = [&](int cc, float* vecb) {  // loader wave 0: gates of chunk cc from pg (tokens past its end count 0)
    const int nv = min(kChunk, P - cc * kChunk);
    const float x = wave_prefix_sum((lane < nv) ? pg : 0.f);
    const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    vecb[64 + lane] = __builtin_amdgcn_exp2f(x * kLog2e);
    vecb[128 + lane] = __builtin_amdgcn_exp2f((gC - x) * kLog2e);
    if (lane == 0) vecb[192] = __builtin_amdgcn_exp2f(gC * kLog2e);
  };
  // Fused launch: T and P of chunk cc come from a producer workgroup through
  // ready flag (chunk, head).  Every loader wave waits for it (bounded spin)
  // before loading its share of them; a record written on another XCD is
  // acquired device-wide by each wave.  A wait that runs out sets the decay
  // multiplier to NaN (the state and every later output show it) and
  // kStatusWaitTimeout in the workspace's status word.
  bool poisoned = false;
  const unsigned xcd_self = kFused ? xcd_id() : 0u;
  auto await_records = [&](int cc) {
    if constexpr (kFused) {
      if (cc < args.prep_c0) return;  // formed by this workgroup
      const unsigned* flag = args.ready + ((int64_t)(chunk0 + cc) * H + h);
      if (!poisoned &&
          !await_ready_flag(flag, __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), xcd_self)) {
        poisoned = true;
        if (lane == 0) {
          *psn = __builtin_nanf("");
          report_wait_timeout(args.status);
        }
      }
    }
  };
  // bf16 o of chunk cc, staged in LDS by the chain waves before the barrier
  // that ended it: each loader wave stores 16 of its 64 rows, a row as 8
  // lanes x 16 bytes (rows past the chunk's end are not stored)
  auto store_o = [&](int cc) {
    if constexpr (kStageO) {
      const int nv = min(kChunk, P - cc * kChunk);
      const char* ob = sO + (cc & 1) * Ls::OBUF;
      const int u = lane & 7;
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int r = 8 * (hw + 4 * ii) + (lane >> 3);
        const uint4 x = *reinterpret_cast<const uint4*>(ob + r * 128 + ((u ^ (r & 7)) << 4));
        if (r < nv)
          *reinterpret_cast<uint4*>(go_ + (int64_t)(seg0 + cc * kChunk + r) * v_row + (int64_t)h * dv +
                                    kTileRows * vt + 8 * u) = x;
      }
    }
  };
  // every load of chunk cc into the buffers of parity cc & 1, and its gates;
  // then the stores of chunk oc's outputs (oc < 0: none).  The loads go out
  // first: how soon they are issued shows in the chunk's time (a delay of
  // about 500 cycles made the fused launch 8% slower), the stores' does not.
  auto load_chunk = [&](int cc, int oc) {
    const int par = cc & 1;
    const int nv = min(kChunk, P - cc * kChunk);
    const int64_t row0 = seg0 + cc * kChunk;
    if (hw == 0) fetch_g(cc);
    load_dump(gk_ + row0 * qk_row + (int64_t)h * DK, sK + par * DUMPE, nv);
    load_dump(gq_ + row0 * qk_row + (int64_t)h * DK, sQ + par * DUMPE, nv);
    load_rows(gv_ + row0 * v_row + (int64_t)h * dv + kTileRows * vt, sV + par * VBUFE, nv);
    await_records(cc);
    const int64_t item = (int64_t)(chunk0 + cc) * H + h;
    load_record(reinterpret_cast<const char*>(args.T) + item * kTRecBytes, sT + par * TRECE, kTRecBytes / 1024);
    load_record(reinterpret_cast<const char*>(args.Prec) + item * kPRecBytes, sP + par * PRECE, kPRecBytes / 1024);
    if (oc >= 0) store_o(oc);
    if (hw == 0) scan(cc, sVec + par * Ls::VEC);
    wait_vmem();  // this wave's loads are in LDS before the barrier that publishes them
  };

  // ---------------- chain waves: the state and the outputs ----------------
  f32x4 st[NT];          // st[t][i] = S[vcol0][dkmap(16t + 4gq + i)] (times s_cur when coded)
  Fr sh[NKB];            // the state as an MFMA operand: its codes after a QDQ, else its hi plane
  float s_cur = 1.0f;    // scale of the coded state
  bool st_coded = false; // st holds E4M3 codes; the state is st * s_cur

  // optional records of boundary c: the state after it (st times f) and its scale
  auto record_post = [&](const int c, const float s_new, const float f) {
    const int bidx = bound0 + c;
    if (args.bound_post) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<float4*>(args.bound_post + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                   dkmap(16 * t + 4 * gq)) = make_float4(st[t][0] * f, st[t][1] * f,
                                                                         st[t][2] * f, st[t][3] * f);
    }
    if (args.bound_scales && tid == 0) args.bound_scales[((int64_t)bidx * H + h) * tiles + vt] = s_new;
  };
  // the four chain waves' amax of boundary c (published before the barrier after chunk c)
  auto tile_scale = [&](const int c) {
    const float* rd = sRed + (c & 1) * 4;
    return qdq_scale_f64(fmaxf(fmaxf(rd[0], rd[1]), fmaxf(rd[2], rd[3])));
  };
  // E4M3 codes of k-block kb of the state (r: 1 / scale in fp64) into st and sh
  auto code_block = [&](const int kb, const double r) {
    float c0[4], c1[4];
    e4m3_codes4_f64(st[2 * kb], r, c0);
    e4m3_codes4_f64(st[2 * kb + 1], r, c1);
    st[2 * kb] = f32x4{c0[0], c0[1], c0[2], c0[3]};
    st[2 * kb + 1] = f32x4{c1[0], c1[1], c1[2], c1[3]};
    const float x[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    sh[kb] = Eng::round(x);  // E4M3 values are exact in bf16
  };

  // One chunk on a chain wave.  kCoded: the boundary before it is quantized;
  // its QDQ (from the amax published before the last barrier) opens the
  // chunk, one k-block at a time, so that the codes of a block are formed
  // while the products of the block before it run.  The stages are ordered
  // the same way throughout: each half of X is split while the products of
  // the other half run, and each half of U' while the update of the other
  // half runs.  Returns nothing; leaves the output in oacc and pacc.
  f32x4 oacc[4], pacc[4];  // S Q^T and U'^T P^T of the chunk, o = s exp(gamma) oacc + pacc
  float amax_w = 0.f;      // the wave's amax of the state after the chunk
  float sc = 1.0f;         // scale of the state entering the chunk
  auto chain_chunk = [&](auto coded_tag, const int c) {
    constexpr bool kCoded = decltype(coded_tag)::value;
    const int par = c & 1;
    const E* __restrict__ kc = sK + par * DUMPE;
    const E* __restrict__ qc = sQ + par * DUMPE;
    const E* __restrict__ vb = sV + par * VBUFE;
    const E* __restrict__ tb = sT + par * TRECE;
    const E* __restrict__ pb = sP + par * PRECE;
    const float* __restrict__ vec = sVec + par * Ls::VEC;
    const float* geg = vec + 64;    // exp(gamma)
    const float* gegc = vec + 128;  // exp(gamma_C - gamma)
    // K^T fragments of token half kb by transpose reads: lane (gq, l) of each
    // 16-lane group points at k[32kb + 16h + 4gq + l/4][dkmap(16t + 4(l%4)) .. +3]
    auto read_kt = [&](const int kb, Fr (&ka)[NT]) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = dkmap(16 * t + 4 * (ln & 3));
        const int tk = 32 * kb + 4 * gq + (ln >> 2);
        const uint2 x0 = lds_read_tr16(kc + kpos(tk, d)), x1 = lds_read_tr16(kc + kpos(tk + 16, d));
        ka[t] = __builtin_bit_cast(Fr, make_uint4(x0.x, x0.y, x1.x, x1.y));
      }
    };
    // X = V - s exp(gamma) acc for tokens 32kb .. 32kb + 31, three planes
    auto form_x = [&](const int kb, const f32x4 (&acc)[4], Fr& xh, Fr& xm, Fr& xl) {
      float x8[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tt = 2 * kb + hh;
        const float4 e4 = *reinterpret_cast<const float4*>(geg + 16 * tt + 4 * gq);
        // one transpose read: lane 4k + j of each 16-lane group points at row
        // 16tt + 4gq + k, columns 16c4 + 4j .. + 3, so lane ln receives column
        // 16c4 + ln of rows 16tt + 4gq + 0..3
        const uint2 r = lds_read_tr16(vb + (16 * tt + 4 * gq + (ln >> 2)) * RSV + 16 * c4 + 4 * (ln & 3));
        const float vv[4] = {__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                             __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
        x8[4 * hh + 0] = fmaf(-sc * e4.x, acc[tt][0], vv[0]);
        x8[4 * hh + 1] = fmaf(-sc * e4.y, acc[tt][1], vv[1]);
        x8[4 * hh + 2] = fmaf(-sc * e4.z, acc[tt][2], vv[2]);
        x8[4 * hh + 3] = fmaf(-sc * e4.w, acc[tt][3], vv[3]);
      }
      Eng::split3(x8, xh, xm, xl);
    };
    // U' of tokens 32kb .. 32kb + 31 as hi + lo, and exp(gamma_C - gamma) U' as three planes
    auto split_u = [&](const int kb, const f32x4 (&uacc)[4], Fr& uh, Fr& ul, Fr& bh, Fr& bm, Fr& bl) {
      const float u8[8] = {uacc[2 * kb][0], uacc[2 * kb][1], uacc[2 * kb][2], uacc[2 * kb][3],
                           uacc[2 * kb + 1][0], uacc[2 * kb + 1][1], uacc[2 * kb + 1][2], uacc[2 * kb + 1][3]};
      Eng::split(u8, uh, ul);
      const float4 e0 = *reinterpret_cast<const float4*>(gegc + 32 * kb + 4 * gq);
      const float4 e1 = *reinterpret_cast<const float4*>(gegc + 32 * kb + 16 + 4 * gq);
      const float d8[8] = {e0.x * u8[0], e0.y * u8[1], e0.z * u8[2], e0.w * u8[3],
                           e1.x * u8[4], e1.y * u8[5], e1.z * u8[6], e1.w * u8[7]};
      Eng::split3(d8, bh, bm, bl);
    };
    // the six partial products of T pair p (ti, kb) into uacc[ti], smallest first
    auto tx_pair = [&](const int p, f32x4 (&uacc)[4], const Fr (&tf)[6], const Fr (&tm)[6], const Fr (&tl)[6],
                       const Fr (&xh)[2], const Fr (&xm)[2], const Fr (&xl)[2]) {
      const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
      Eng::mma(uacc[ti], tf[p], xl[kb]);
      Eng::mma(uacc[ti], tl[p], xh[kb]);
      Eng::mma(uacc[ti], tm[p], xm[kb]);
      Eng::mma(uacc[ti], tf[p], xm[kb]);
      Eng::mma(uacc[ti], tm[p], xh[kb]);
      Eng::mma(uacc[ti], tf[p], xh[kb]);
    };

    // ---- stage A: the state operand, K S^T (acc) and S Q^T (oacc).  A
    // coded chunk opens with the QDQ of the boundary before it, one k-block
    // at a time: the codes of block kb + 1 are formed beside the products of
    // block kb.  Each step below is its own scheduling region.
    double rs = 1.0;
    sc = 1.0f;
    if constexpr (kCoded) {
      sc = tile_scale(c - 1);
      rs = rcp_f64(sc);
    }
    f32x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      oacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    Fr kf[2][4], qf[2][4];  // K and Q fragments of k-blocks kb (slot kb & 1): f = tt (ti)
    auto read_kq = [&](const int kb) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        kf[kb & 1][tt] = Eng::ld(qslot(kc, tt * NKB + kb));
        qf[kb & 1][tt] = Eng::ld(qslot(qc, tt * NKB + kb));
      }
    };
    Fr lo[NKB];  // uncoded state: its lo plane
    auto form_state = [&](const int kb) {
      if constexpr (kCoded) {
        code_block(kb, rs);
      } else {
        const float x[8] = {st[2 * kb][0], st[2 * kb][1], st[2 * kb][2], st[2 * kb][3],
                            st[2 * kb + 1][0], st[2 * kb + 1][1], st[2 * kb + 1][2], st[2 * kb + 1][3]};
        Eng::split(x, sh[kb], lo[kb]);
      }
    };
    read_kq(0);
    read_kq(1);
    form_state(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Fr(&kfb)[4] = kf[kb & 1];
      const Fr(&qfb)[4] = qf[kb & 1];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) Eng::mma(acc[tt], kfb[tt], sh[kb]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) Eng::mma(oacc[ti], sh[kb], qfb[ti]);
      if constexpr (!kCoded) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) Eng::mma(acc[tt], kfb[tt], lo[kb]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) Eng::mma(oacc[ti], lo[kb], qfb[ti]);
      }
      if (kb + 1 < NKB) form_state(kb + 1);
      if (kb + 2 < NKB) read_kq(kb + 2);
      if constexpr (kCoded) sched_interleave<8, 6>();
      else sched_interleave<16, 1>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kCoded) {
      s_cur = sc;
      st_coded = true;
      record_post(c - 1, sc, sc);
    }

    // ---- stage B: the first half of X; then U' = T X over the
    // lower-triangular T pairs (ti, kb) (0,0) (1,0) (2,0) (3,0) (2,1) (3,1),
    // the six partial products down to 2^-16 of the leading one: the second
    // half of X and the decay of the state (exp(gamma_C), times the scale of
    // a coded state) beside the pairs of the first, the split of U' rows
    // 0..31 beside the last two pairs
    Fr tf[6], tm[6], tl[6];
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      tf[p] = Eng::ld(slot(tb, p));
      tm[p] = Eng::ld(slot(tb, 6 + p));
      tl[p] = Eng::ld(slot(tb, 12 + p));
    }
    float aC = vec[192] * sc;
    if constexpr (kFused) aC *= *psn;  // NaN after a failed wait for a record
    Fr xh[2], xm[2], xl[2];
    form_x(0, acc, xh[0], xm[0], xl[0]);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 uacc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) uacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) tx_pair(p, uacc, tf, tm, tl, xh, xm, xl);
    form_x(1, acc, xh[1], xm[1], xl[1]);
    // the decay of the state, beside the products (the update adds to it later)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[t][i] *= aC;
    st_coded = false;
    Fr ka0[NT];
    read_kt(0, ka0);
    sched_interleave<24, 3>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 4; p < 6; ++p) tx_pair(p, uacc, tf, tm, tl, xh, xm, xl);
    Fr uh[2], ul[2], bh[2], bm[2], bl[2];
    split_u(0, uacc, uh[0], ul[0], bh[0], bm[0], bl[0]);
    Fr ka1[NT];
    read_kt(1, ka1);
    sched_interleave<12, 4>();
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage C: S^T += K^T (exp(gamma_C - gamma) U') per token half (the
    // split of the second half beside the update of the first), then
    // pacc = U'^T P^T
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      Eng::mma(st[t], ka0[t], bl[0]);
      Eng::mma(st[t], ka0[t], bm[0]);
      Eng::mma(st[t], ka0[t], bh[0]);
    }
    split_u(1, uacc, uh[1], ul[1], bh[1], bm[1], bl[1]);
    Fr phs[6], pls[6];
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      phs[p] = Eng::ld(slot(pb, p));
      pls[p] = Eng::ld(slot(pb, 6 + p));
    }
    sched_interleave<24, 2>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      Eng::mma(st[t], ka1[t], bl[1]);
      Eng::mma(st[t], ka1[t], bm[1]);
      Eng::mma(st[t], ka1[t], bh[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the products U'^T P^T beside the amax of the updated state (a tree of
    // depth 5, then a DPP wave max), which only waits for the update
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) pacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
      Eng::mma(pacc[ti], uh[kb], phs[p]);
      Eng::mma(pacc[ti], ul[kb], phs[p]);
      Eng::mma(pacc[ti], uh[kb], pls[p]);
    }
    float m16[2 * NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m16[2 * t] = fmaxf(fabsf(st[t][0]), fabsf(st[t][1]));
      m16[2 * t + 1] = fmaxf(fabsf(st[t][2]), fabsf(st[t][3]));
    }
#pragma unroll
    for (int w2 = NT; w2 >= 1; w2 /= 2)
#pragma unroll
      for (int k = 0; k < w2; ++k) m16[k] = fmaxf(m16[k], m16[k + w2]);
    amax_w = wave_max_dpp(m16[0]);
    sched_interleave<18, 3>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // o row of this lane's first output (token ln of the sequence), hoisted out
  // of the chunk loop
  TO* const o_lane = go_ + (int64_t)(seg0 + ln) * v_row + (int64_t)h * dv + kTileRows * vt + 16 * c4 + 4 * gq;
  // After a chunk's products: the amax of the tile published for the QDQ
  // after the barrier (slot of this chunk's parity: the next write to it
  // comes after the next barrier), the output stored, the records.
  auto chain_finish = [&](const int c) {
    const int par = c & 1;
    const float* geg = sVec + par * Ls::VEC + 64;
    const int nv = min(kChunk, P - c * kChunk);
    if (lane == 0) sRed[par * 4 + c4] = amax_w;
    // lane holds o[tok = 16ti + ln][16c4 + 4gq .. +3] of this tile
    float egt[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) egt[ti] = sc * geg[16 * ti + ln];
    float o16[4][4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) o16[ti][i] = fmaf(egt[ti], oacc[ti][i], pacc[ti][i]);
    if constexpr (kStageO) {
      // row 16ti + ln, columns 16c4 + 4gq .. +3: half gq % 2 of piece 2c4 + gq / 2
      char* const ob = sO + par * Ls::OBUF;
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int r = 16 * ti + ln;
        *reinterpret_cast<uint2*>(ob + r * 128 + (((2 * c4 + (gq >> 1)) ^ (r & 7)) << 4) + 8 * (gq & 1)) =
            make_uint2(pack_bf16x2(o16[ti][0], o16[ti][1]), pack_bf16x2(o16[ti][2], o16[ti][3]));
      }
    } else {
      TO* const oc = o_lane + (int64_t)(c * kChunk) * v_row;
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        if (16 * ti + ln < nv)
          *reinterpret_cast<float4*>(oc + (int64_t)(16 * ti) * v_row) =
              make_float4(o16[ti][0], o16[ti][1], o16[ti][2], o16[ti][3]);
    }
    if (args.bound_pre) {
      const int bidx = bound0 + c;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<float4*>(args.bound_pre + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                   dkmap(16 * t + 4 * gq)) = make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    }
    const bool do_qdq = (flags & GDN_QDQ_CHUNK) || ((flags & GDN_QDQ_WRITE) && c == n_chunks - 1);
    if (!do_qdq) record_post(c, 1.0f, 1.0f);
  };

  // The boundary QDQ after the last chunk (the QDQ of the others opens the next chunk).
  auto chain_qdq_last = [&](const int c) {
    const float s_new = tile_scale(c);
    const double r = rcp_f64(s_new);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) code_block(kb, r);
    s_cur = s_new;
    st_coded = true;
    record_post(c, s_new, s_new);
  };

  // ---------------- prologue ----------------
  if (hw == 0 && lane == 0) *psn = 1.0f;
  if (chain) {
    if (args.init != nullptr) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4 x = *reinterpret_cast<const float4*>(args.init + state_base + dkmap(16 * t + 4 * gq));
        st[t] = f32x4{x.x, x.y, x.z, x.w};
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  barrier_lds();  // the poison word is set before any wait can overwrite it
  if constexpr (kFused) {
    // The first chunk's records: formed here by the loader waves (the chain
    // waves only take part in the item's barriers) instead of waiting for a
    // producer's first round; the LDS block at 0 is free until chunk 0 is
    // loaded.  Both value tiles of a pair write the same bytes to its slot.
    if (args.prep_c0 > 0 && n_chunks > 0) {
      PrepArgs pa;
      pa.q = args.q; pa.k = args.k; pa.beta = args.beta; pa.g = args.g; pa.cu_seqlens = args.cu_seqlens;
      pa.seq_lens = args.seq_lens; pa.prefix_lens = args.prefix_lens; pa.offs = args.chunk_offs;
      pa.T = const_cast<void*>(args.T); pa.P = const_cast<void*>(args.Prec); pa.N = args.N; pa.H = H;
      pa.W = nullptr; pa.w_pre = nullptr; pa.w_post = nullptr; pa.status = args.status;
      prep_item<DK, TIO, false>(pa, chunk0, h, seg0, min(kChunk, P), smem, chain ? tid : tid - 256, !chain);
      wait_vmem();      // this wave's record stores are complete
      __syncthreads();  // ... in every wave
    }
  }
  if (!chain && n_chunks > 0) load_chunk(0, -1);
  barrier_lds();

  // ---------------- the chunks ----------------
  // Nothing of the prologue stays in flight into the loop (the initial state
  // loads included): the wait counts inside the loop then need not cover
  // them, and the chain waves never wait there for their own output stores.
  __builtin_amdgcn_s_waitcnt(0);
  const bool qdq_chunk = (flags & GDN_QDQ_CHUNK) != 0;
  for (int c = 0; c < n_chunks; ++c) {
    if (chain) {
      if (c > 0 && qdq_chunk)
        chain_chunk(std::true_type{}, c);
      else
        chain_chunk(std::false_type{}, c);
      chain_finish(c);
    } else {
      if (c + 1 < n_chunks) load_chunk(c + 1, c - 1);  // into the other half of every buffer
      else if (c > 0) store_o(c - 1);
    }
    barrier_lds();
  }
  if (!chain && n_chunks > 0) store_o(n_chunks - 1);
  if (chain && n_chunks > 0 && (flags & (GDN_QDQ_CHUNK | GDN_QDQ_WRITE))) chain_qdq_last(n_chunks - 1);

  if (st_coded) {  // back to the state values: code * s
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[t][i] *= s_cur;
    st_coded = false;
  }

  // ---------------- recurrent suffix, tokens P < t <= L ----------------
  // optional per-token record: the chain wave's rows of the state after each
  // suffix token, before (sfx_pre) and after (sfx_post) its QDQ
  float* const sfx_pre = args.sfx_offsets ? args.sfx_pre : nullptr;
  float* const sfx_post = args.sfx_offsets ? args.sfx_post : nullptr;
  const int64_t sfx0 = args.sfx_offsets ? args.sfx_offsets[n] : 0;
  const int64_t sfx_stride = (int64_t)H * dv * DK;
  auto store_state = [&](float* base) {  // base: record entry of one token
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2)
      *reinterpret_cast<float4*>(base + ((int64_t)h * dv + vcol0) * DK + dkmap(16 * t2 + 4 * gq)) =
          make_float4(st[t2][0], st[t2][1], st[t2][2], st[t2][3]);
  };
  if (P < L) {
    float* sq = reinterpret_cast<float*>(smem + Ls::oK);  // q_t, k_t: DK each; v_t: 64; g_t, beta_t
    float* sk = sq + DK;
    float* sv = sk + DK;
    float* sgb = sv + 64;
    for (int t = P; t < L; ++t) {
      const int64_t row = seg0 + t;
      if (!chain) {
        const int th = tid - 256;
        if (th < DK) {
          sq[th] = io<TIO>::ld(gq_ + row * qk_row + (int64_t)h * DK + th);
          sk[th] = io<TIO>::ld(gk_ + row * qk_row + (int64_t)h * DK + th);
        }
        if (th < 64) sv[th] = io<TIO>::ld(gv_ + row * v_row + (int64_t)h * dv + kTileRows * vt + th);
        if (th == 0) {
          sgb[0] = args.g[row * H + h];
          sgb[1] = args.beta[row * H + h];
        }
      }
      __syncthreads();
      if (chain) {
        const float a = expf(grid_gate(sgb[0], args.grid_log2));
        const float b = sgb[1];
        float y = 0.f;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st[t2][i] *= a;
            y += st[t2][i] * sk[dkmap(16 * t2 + 4 * gq + i)];
          }
        y += __shfl_xor(y, 16, 64);
        y += __shfl_xor(y, 32, 64);
        const float u = b * (sv[16 * c4 + ln] - y);
        float z = 0.f;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st[t2][i] += u * sk[dkmap(16 * t2 + 4 * gq + i)];
            z += st[t2][i] * sq[dkmap(16 * t2 + 4 * gq + i)];
          }
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        if (gq == 0) io<TO>::st(go_ + row * v_row + (int64_t)h * dv + vcol0, z);
        if (sfx_pre) store_state(sfx_pre + (sfx0 + t - P) * sfx_stride);
        if (flags & GDN_QDQ_WRITE) {
          float amax = 0.f;
#pragma unroll
          for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
            for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(st[t2][i]));
          amax = wave_max_dpp(amax);
          if (lane == 0) sRed[c4] = amax;
        }
      }
      __syncthreads();
      if (chain && (flags & GDN_QDQ_WRITE)) {
        const float s = qdq_scale(fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3])));
        const float r = 1.0f / s;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2) qdq4(st[t2], s, r);
      }
      if (chain && sfx_post) store_state(sfx_post + (sfx0 + t - P) * sfx_stride);
    }
  }

  // ---------------- final state, zero padding rows of o ----------------
  if (chain) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<float4*>(args.fin + state_base + dkmap(16 * t + 4 * gq)) =
          make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
  }
  for (int r = L + w; r < seg1 - seg0; r += kWaves)
    io<TO>::st(go_ + (int64_t)(seg0 + r) * v_row + (int64_t)h * dv + kTileRows * vt + lane, 0.f);
}

template <int DK, typename TO, bool kFused>
static hipError_t launch_bf16_typed(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  auto kern = chunk_bf16_kernel<DK, TO, kFused>;
  constexpr size_t item_lds = 2 * (size_t)PrepItemLds<DK, uint16_t, false>::bytes;  // a producer's two items
  constexpr size_t state_lds = LdsB<DK>::bytes;
  constexpr size_t lds = (kFused && item_lds > state_lds) ? item_lds : state_lds;
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
  static PerDeviceOnce lds_attr;
  if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows) + (kFused ? a.n_prep : 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreadsWg), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_chunk_bf16(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  const bool ob = s.o_dtype == GDN_BF16;
  if (s.dk == 128) {
    if (ob) return a.fused ? launch_bf16_typed<128, uint16_t, true>(s, a, stream)
                           : launch_bf16_typed<128, uint16_t, false>(s, a, stream);
    return a.fused ? launch_bf16_typed<128, float, true>(s, a, stream)
                   : launch_bf16_typed<128, float, false>(s, a, stream);
  }
  if (ob) return a.fused ? launch_bf16_typed<64, uint16_t, true>(s, a, stream)
                         : launch_bf16_typed<64, uint16_t, false>(s, a, stream);
  return a.fused ? launch_bf16_typed<64, float, true>(s, a, stream)
                 : launch_bf16_typed<64, float, false>(s, a, stream);
}

}  // namespace gdn
