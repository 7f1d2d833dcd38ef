// gdn_chunk.hip -- sequential part of the chunked gated delta rule forward
// with per-boundary FP8-E4M3 state QDQ (Model-Optimizer #2497 "What does this
// PR do?": 64-token chunks, WY/UT-transformed operands, dynamic per-tile state
// QDQ at every boundary; #2519: QDQ at the handoff and after every later
// recurrent write).
//
// Work unit: one workgroup of 8 waves per (sequence n, head h, 64-column value
// tile vt).  It walks its sequence chunk by chunk and keeps its slice of the
// state in registers for the whole sequence.  The 64 x dk state tile is
// exactly one QDQ tile, so the QDQ amax needs no exchange with other
// workgroups.  T and P of every chunk come through the workspace, from the
// prep kernel (gdn_prep.hip) or, in the fused launch, from producer
// workgroups of this same launch (produce_records below).
//
// Waves 0..3 ("chain" waves) carry the state: chain wave c owns value columns
// 16c..16c+15 of the tile, i.e. dk/16 16x16 accumulator tiles of S^T, and
// runs everything that depends on the state.  Waves 4..7 ("helper" waves)
// produce the outputs and stage the next chunk, so each SIMD runs one wave of
// each kind and the two overlap.  With gamma the in-chunk cumulative log-gate
// and s the scale of the state entering the chunk (1 when it is not coded),
// one chunk of n <= 64 tokens (rows past n are zero) goes through two
// phases separated by workgroup barriers:
//
//   A   chain : X = V - s exp(gamma) * (K S^T), U' = T X            (MFMA)
//       helper: s exp(gamma) * (Q S^T), from the state the chain left in LDS
//   B   chain : S^T <- exp(gamma_C) S^T + K^T diag(exp(gamma_C - gamma)) U'
//               and the tile amax; the four chain waves exchange their amax
//               through LDS among themselves (no workgroup barrier), then
//               the QDQ: s = amax / 448, S <- RNE_E4M3(S / s) s
//       helper: O += P U', stored to o; the gate scan of the next chunk and
//               the wait for the next chunk's loads
// T = (I + A)^-1 diag(beta) and P[r][s] = exp(gamma_r - gamma_s) q_r . k_s
// (s <= r) arrive as records; the next chunk's k (two chunks ahead), q, v, T
// and P arrive by direct global->LDS loads issued as soon as their buffers
// are free.
//
// U' = T X is U - W S^T with U = T V and W = T (exp(gamma) * K) regrouped, so
// W is never formed.  With W QDQ (kW) W is formed by the producers, row-
// quantized (#2497: dynamic FP8 QDQ of the WY-transformed W, one scale per
// token and head) and arrives as its E4M3 codes and row scales w_s, so
//   1a  chain : U' = T V - s w_s * (W_codes S^T)
// in place of the line above, the rest unchanged.  Then the recurrent suffix
// (tokens P_n < t <= L_n, QDQ after every write) and the final state store.
//
// LDS operands are kept in MFMA fragment order ("dumps"): fragment f of a
// buffer is 64 lanes x 8 elements, lane-major, laid out exactly as the lanes
// consume it (see the conventions in gdn_device.hpp), so every operand read
// is one lane-linear load without bank conflicts.
//
// Precision (bf16 inputs, fp32 accumulate): q, k, v enter the MFMAs exactly;
// T, P, X, U' and exp(gamma_C - gamma) U' as hi + lo bf16 pairs.  After a QDQ
// the state is code * s with the code exactly representable in bf16, so it is
// fed as the codes and the products are scaled by s; otherwise (QDQ off, a
// supplied initial state) as a hi + lo pair.  fp32 inputs use the fp32 MFMA
// throughout.
#include "gdn_prep_item.hpp"

namespace gdn {

constexpr int kChunkWaves = 8;
constexpr int kChunkThreads = 64 * kChunkWaves;
constexpr int kHelperThreads = 256;  // waves 4..7

// LDS layout of the sequential kernel (bytes).  F = one fragment dump (64
// lanes x 8 elements, lane-major).
//   K   2 x [tt][kb]  dump, double-buffered by chunk parity: lane l holds
//                  k[16tt + l%16][32kb + 8(l/16) .. +7] in slot rot_slot(l);
//                  A of K S^T, A of P, K^T by transpose reads   4 NKB fragments
//   Q   [tt][kb]   the same for q (read in phase A only); B of S Q^T
//   KT  [dt][kb]   dump: A of the state update (row = state row), 2 NT
//                  fragments (fp32 engine; the bf16 engine reads these
//                  fragments from K with transpose reads)
//   V   [64][64 + 16 bytes]  the tile's v rows, row-major, padded rows
//   T   [plane][p] 6 fragments per plane, three planes (bf16) or one (fp32):
//                  the T record, copied as is
//   P   2 x [plane][p]  the P record (two planes), double-buffered by chunk
//                  parity (one buffer with W QDQ, whose W record needs the room)
//   XU  [c][plane*2 + kb]     U' as the A operand of U'^T P^T, per chain wave
//   XS  [c][plane*NKB + kb]   the state as the A operand of S Q^T, per chain wave
//   vec 2 x: (unused), exp(gamma), exp(gamma_C - gamma) [64] each; misc[8],
//       by chunk parity (the next chunk's gates are scanned while the
//       current ones are still read)
//   red the four chain waves' amax by chunk parity [2][4], their tags [4]
//       (the chunk each wave has published), the poison multiplier
//   W   (kW only) the W record of the chunk as is: 4 NKB bf16 fragments of
//       codes (A of W S^T, both engines), then the 64 row scales
template <int DK, class Eng, bool kW = false>
struct Lds {
  using E = typename Eng::E;
  static constexpr int NKB = DK / 32, NT = DK / 16, NP = Eng::kPlanes;
  static constexpr int NPT = Eng::kSplit ? 3 : 1;     // planes of the T record
  static constexpr int PBUF = kW ? 1 : 2;             // P buffers
  static constexpr size_t F = 64 * 8 * sizeof(E);
  static constexpr size_t RV = 64 * sizeof(E) + 16;    // padded v row (bytes)
  static constexpr size_t oK = 0;                      // 2 buffers by chunk parity
  static constexpr size_t oQ = oK + 2 * 4 * NKB * F;
  static constexpr size_t oKT = oQ + 4 * NKB * F;
  static constexpr size_t oV = oKT + (Eng::kTrRead ? 0 : 2 * NT * F);
  static constexpr size_t oT = oV + 64 * RV;
  static constexpr size_t oP = oT + 6 * NPT * F;
  static constexpr size_t oXU = oP + PBUF * 6 * NP * F;
  static constexpr size_t oXS = oXU + 4 * 2 * NP * F;
  static constexpr size_t oVec = oXS + 4 * NKB * NP * F;
  static constexpr size_t oRed = oVec + 2 * (3 * 64 + 8) * sizeof(float);
  static constexpr size_t oW = oRed + 16 * sizeof(float);
  static constexpr size_t bytes = oW + (kW ? (size_t)w_rec_bytes(DK) : 0);
  static_assert(6 * NPT * F <= kTRecBytes && 6 * NP * F == kPRecBytes, "records and their LDS copies differ");
  static_assert(oW % 16 == 0, "direct loads need 16-byte aligned LDS");
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
  static_assert(oK + (2 * DK + 64 + 8) * sizeof(float) <= oQ, "suffix buffers do not fit");
};



template <int DK, class Eng, typename TIO, typename TO, bool kFused, bool kW>
__global__ __launch_bounds__(kChunkThreads, 1) void chunk_fwd_kernel(ChunkArgs args) {
  using Ls = Lds<DK, Eng, kW>;
  using E = typename Eng::E;
  using Fr = typename Eng::Fr;
  constexpr int NT = DK / 16;   // state accumulator tiles per chain wave
  constexpr int NKB = DK / 32;  // k-blocks over dk
  constexpr int NP = Eng::kPlanes;
  constexpr bool kSplit = Eng::kSplit;
  extern __shared__ __align__(16) char smem[];
  if (index_check_failed(args.status)) return;
  if constexpr (kFused) {
    if ((int)blockIdx.x < args.n_prep) {
      produce_records<DK, TIO, kW>(args, smem);
      return;
    }
  }
  E* sK = reinterpret_cast<E*>(smem + Ls::oK);
  E* sQ = reinterpret_cast<E*>(smem + Ls::oQ);
  E* sKT = reinterpret_cast<E*>(smem + Ls::oKT);
  E* sV = reinterpret_cast<E*>(smem + Ls::oV);
  E* sT = reinterpret_cast<E*>(smem + Ls::oT);
  E* sP = reinterpret_cast<E*>(smem + Ls::oP);
  E* sXU = reinterpret_cast<E*>(smem + Ls::oXU);
  E* sXS = reinterpret_cast<E*>(smem + Ls::oXS);
  float* sG2 = reinterpret_cast<float*>(smem + Ls::oVec);  // gamma * log2(e)
  float* sRed = reinterpret_cast<float*>(smem + Ls::oRed);
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem + Ls::oW);  // kW only

  const uint32_t lds0 = lds_base_u32(smem);
  auto lds_of = [&](const void* p) { return lds0 + (uint32_t)(reinterpret_cast<const char*>(p) - smem); };
  const int tid = threadIdx.x;
  const int w = tid >> 6;        // wave
  const int lane = tid & 63;
  const int gq = lane >> 4;      // lane group (k-slots / accumulator rows 4gq..4gq+3)
  const int ln = lane & 15;      // accumulator column / fragment row
  const bool chain = w < 4;
  const int c4 = uniform(w) & 3; // value block (16 columns) this wave serves
  const int hw = uniform(w) - 4;    // helper wave index (waves 4..7)
  // fragment f of an LDS dump, this lane's slot
  auto slot = [lane](E* base, int f) { return base + (f * 64 + lane) * 8; };
  const int qs = rot_slot(lane);
  auto qslot = [qs](E* base, int f) { return base + (f * 64 + qs) * 8; };  // k/q dumps
  // element offset of k[t][d] in a k/q dump
  auto kpos = [](int t, int d) {
    return (((t >> 4) * (DK / 32) + (d >> 5)) * 64 + rot_slot(((d & 31) >> 3) * 16 + (t & 15))) * 8 + (d & 7);
  };

  const int H = args.H, dv = args.dv;
  const int tiles = dv / kTileRows;
  // Block -> (n*H + h, vt).  Workgroups are dispatched to the 8 XCDs round
  // robin; when heads come in groups of 8, the value tiles of one head get
  // block ids 8 apart, i.e. the same XCD, so their q/k/T reads share an L2.
  int nh, vt;
  {
    const int b = (int)blockIdx.x - (kFused ? args.n_prep : 0);
    const int G = (int)gridDim.x - (kFused ? args.n_prep : 0);
    if (tiles > 1 && G % (8 * tiles) == 0) {
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
  const int64_t qk_row = (int64_t)H * DK;   // token stride of q, k
  const int64_t v_row = (int64_t)H * dv;    // token stride of v, o
  const int vcol0 = kTileRows * vt + 16 * c4 + ln;  // chain lane's value column (in dv)
  const int64_t state_base = ((int64_t)nh * dv + vcol0) * DK;  // row vcol0 of S

  const int n_chunks = (P + kChunk - 1) / kChunk;
  const int bound0 = args.bound_offsets ? args.bound_offsets[n] : 0;
  const int chunk0 = args.chunk_offs[n];

  // ---- chain-wave state: st[t][i] = S[vcol0][dkmap(16t + 4gq + i)]
  f32x4 st[NT];
  Fr sh[NKB];            // after a chunk QDQ: the codes as the MFMA operand (bf16 engine)
  float s_cur = 1.0f;    // scale of the coded state
  bool st_coded = false; // bf16 engine after a chunk QDQ: st holds the E4M3 codes, the state is st * s_cur
  f32x4 uacc[4];         // U'[16tt + 4gq + i][vcol0], phase A -> B

  // uncoded state -> operand fragments: hi + lo (bf16 engine) / exact fp32
  auto state_frags = [&](Fr (&hi)[NKB], Fr (&lo)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float x[8] = {st[2 * kb][0], st[2 * kb][1], st[2 * kb][2], st[2 * kb][3],
                          st[2 * kb + 1][0], st[2 * kb + 1][1], st[2 * kb + 1][2], st[2 * kb + 1][3]};
      Eng::split(x, hi[kb], lo[kb]);
    }
  };
  // the state fragments for the helper wave's S Q^T (lo only when split)
  auto write_xs = [&](E* xsb, const Fr (&hi)[NKB], const Fr (&lo)[NKB], bool two) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Eng::st(slot(xsb, c4 * NP * NKB + kb), hi[kb]);
    if constexpr (kSplit) {
      if (two) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Eng::st(slot(xsb, c4 * NP * NKB + NKB + kb), lo[kb]);
      }
    }
  };

  constexpr int EPP = 16 / (int)sizeof(E);  // elements per 16-byte piece
  constexpr int PPV = kTileRows / EPP;      // pieces per v row
  constexpr int RSV = (PPV + 1) * EPP;      // padded v row stride (elements)
  static_assert(sizeof(TIO) == sizeof(E), "LDS element type is the input type");

  // Direct global -> LDS loads of chunk cc (k and q dumps, v rows, the T
  // record, the log-gates).  One instruction writes 64
  // consecutive 16-byte LDS pieces.  Rows past the chunk's valid count load
  // its last valid row: they meet zero rows and columns of T, or outputs that
  // are not stored, so they need no zeroing.
  auto load_dump = [&](const TIO* src, E* dst, int nv, int wi) {  // src: the chunk's row 0, the head's column 0
    constexpr int UPS = (int)sizeof(E) / 2;                      // 16-byte pieces per lane slot
    constexpr int NI = 4 * NKB * UPS;                            // instructions (multiple of 4)
    static_assert(NI % 4 == 0, "dump load geometry");
#pragma unroll
    for (int ii = 0; ii < NI / 4; ++ii) {
      const int i = wi + 4 * ii;
      const int u = i * 64 + lane, sl = u / UPS, part = u % UPS;
      const int f = sl >> 6, l2 = rot_lane(sl & 63);
      const int r = 16 * (f / NKB) + (l2 & 15);
      const int d = 32 * (f % NKB) + 8 * (l2 >> 4) + part * EPP;
      lds_load16(src, (uint32_t)((min(r, nv - 1) * (int)qk_row + d) * (int)sizeof(E)),
                 lds_of(dst) + i * 1024);
    }
  };
  auto load_rows = [&](const TIO* src, int stride, E* dst, int nv, int wi) {  // padded v rows
    constexpr int RPI = 64 / (PPV + 1);           // rows per instruction
    constexpr int NI = (64 + RPI - 1) / RPI;      // instructions
    const int rr = lane / (PPV + 1), pc = lane % (PPV + 1);
    const int lane_off = min(pc, PPV - 1) * EPP;
#pragma unroll
    for (int ii = 0; ii < (NI + 3) / 4; ++ii) {
      const int i = wi + 4 * ii;
      const int r = i * RPI + rr;
      if (i < NI && rr < RPI && r < 64)
        lds_load16(src, (uint32_t)((min(r, nv - 1) * stride + lane_off) * (int)sizeof(E)),
                   lds_of(dst) + i * RPI * (PPV + 1) * EPP * (int)sizeof(E));
    }
  };
  // Loads of chunk cc, by buffer lifetime: k and P have two buffers (chunk
  // parity); P and k of the next chunk are issued at the start of phase A
  // (k into the buffer of the previous chunk, whose update has read it; with
  // one P buffer, P of the chunk itself, and k at the end of phase B); v, T
  // and q (one buffer each) in phase B, once phase A has read them.  In the loop the
  // helper waves issue all of them; helper wave 0 fetches the log-gates into
  // a register.
  auto issue_k = [&](int cc, E* kdst, int wi) {
    const int nv = min(kChunk, P - cc * kChunk);
    const int64_t row0 = seg0 + cc * kChunk;
    load_dump(gk_ + row0 * qk_row + (int64_t)h * DK, kdst, nv, wi);
  };
  auto issue_v = [&](int cc, E* vdst, E* tdst, int wi) {
    const int nv = min(kChunk, P - cc * kChunk);
    const int64_t row0 = seg0 + cc * kChunk;
    load_rows(gv_ + row0 * v_row + (int64_t)h * dv + kTileRows * vt, (int)v_row, vdst, nv, wi);
    const char* rec = reinterpret_cast<const char*>(args.T) + ((int64_t)(chunk0 + cc) * H + h) * kTRecBytes;
    constexpr int NTI = (int)(6 * Ls::NPT * Ls::F / 1024);  // 1 KiB pieces of the T record
#pragma unroll
    for (int ii = 0; ii < (NTI + 3) / 4; ++ii) {
      const int idx = wi + 4 * ii;
      if (idx < NTI) lds_load16(rec, (uint32_t)((idx * 64 + lane) * 16), lds_of(tdst) + idx * 1024);
    }
  };
  auto issue_w = [&](int cc, uint16_t* wdst, int wi) {  // the W record of chunk cc (kW)
    constexpr int NI = w_rec_bytes(DK) / 1024;
    const char* rec = reinterpret_cast<const char*>(args.Wrec) + ((int64_t)(chunk0 + cc) * H + h) * w_rec_bytes(DK);
#pragma unroll
    for (int ii = 0; ii < (NI + 3) / 4; ++ii) {
      const int idx = wi + 4 * ii;
      if (idx < NI) lds_load16(rec, (uint32_t)((idx * 64 + lane) * 16), lds_of(wdst) + idx * 1024);
    }
  };
  auto issue_q = [&](int cc, E* qdst) {
    const int nv = min(kChunk, P - cc * kChunk);
    const int64_t row0 = seg0 + cc * kChunk;
    load_dump(gq_ + row0 * qk_row + (int64_t)h * DK, qdst, nv, hw);
  };
  auto issue_p = [&](int cc, E* pdst) {  // the P record of chunk cc
    const char* rec = reinterpret_cast<const char*>(args.Prec) + ((int64_t)(chunk0 + cc) * H + h) * kPRecBytes;
#pragma unroll
    for (int ii = 0; ii < kPRecBytes / 1024 / 4; ++ii) {
      const int idx = hw * (kPRecBytes / 1024 / 4) + ii;
      lds_load16(rec, (uint32_t)((idx * 64 + lane) * 16), lds_of(pdst) + idx * 1024);
    }
  };
  float pg = 0.f;  // helper wave 0: log-gate of token `lane` of the next chunk
  auto fetch_g = [&](int cc) {
    const int nv = min(kChunk, P - cc * kChunk);
    pg = args.g[(int64_t)(seg0 + cc * kChunk + min(lane, nv - 1)) * H + h];
  };
  // Helper wave 0: gates of chunk cc from pg (tokens past its end count 0).
  auto scan = [&](int cc, float* vecb) {
    const int nv = min(kChunk, P - cc * kChunk);
    const float x = wave_prefix_sum((lane < nv) ? pg : 0.f);
    const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    vecb[64 + lane] = __builtin_amdgcn_exp2f(x * kLog2e);
    vecb[128 + lane] = __builtin_amdgcn_exp2f((gC - x) * kLog2e);
    if (lane == 0) vecb[192] = __builtin_amdgcn_exp2f(gC * kLog2e);
  };
  // fp32 engine, helper waves, phase A: the K^T dump of the current chunk
  // (fragment f = 2 dt + kb, lane l holds k[32 kb + kperm(l/16, j)][dkmap(16 dt + l%16)]).
  auto transform = [&](const E* kd, E* ktd) {
    if constexpr (!Eng::kTrRead) {
#pragma unroll
      for (int m = 0; m < NT / 2; ++m) {
        const int f = hw + 4 * m, dt = f >> 1, kb = f & 1;
        const int d = dkmap(16 * dt + ln);  // key channel of this lane's state row
        E x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = kd[kpos(32 * kb + (j < 4 ? 4 * gq + j : 16 + 4 * gq + (j - 4)), d)];
        Eng::st(slot(ktd, f), Eng::pack8(x));
      }
    }
  };

  // Fused launch: the records of chunk cc come from a producer workgroup
  // through ready flag (chunk, head).  Helper wave 1 waits for it (bounded
  // spin); the barriers that follow order every wave's record loads after
  // that.  A producer on this XCD completed the records in the shared L2;
  // one on another XCD must have released them device-wide, and then this
  // wave invalidates its caches (device-scope acquire).  A wait that runs
  // out, or a record that cannot be trusted, sets the decay multiplier
  // misc[2] to NaN, so the state and every later output show it, and sets
  // kStatusWaitTimeout in the workspace's status word.
  unsigned pend = 0u;     // helper wave 1: a ready flag read ahead (used after a wait_vmem)
  bool poisoned = false;
  auto ready_ptr = [&](int cc) { return args.ready + ((int64_t)(chunk0 + cc) * H + h); };
  auto load_ready = [&](int cc) { return __hip_atomic_load(ready_ptr(cc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto read_ready = [&](int cc) { return (unsigned)__builtin_amdgcn_readfirstlane((int)load_ready(cc)); };
  const unsigned xcd_self = kFused ? xcd_id() : 0u;
  float* const psn = sRed + 12;  // decay multiplier: 1, or NaN once a wait has run out
  auto poison = [&]() {
    poisoned = true;
    if (lane == 0) {
      *psn = __builtin_nanf("");
      report_wait_timeout(args.status);
    }
  };
  auto await_ready = [&](int cc, unsigned v0) {
    if (!poisoned && !await_ready_flag(ready_ptr(cc), v0, xcd_self)) poison();
  };


  // ---------------- prologue ----------------
  if (tid < 12) sRed[tid] = 0.0f;  // amax slots, tags (0: no chunk published yet)
  if constexpr (kFused) {
    if (hw == 1 && lane == 0) *psn = 1.0f;  // before this wave's own waits can poison it
    if (hw == 1 && n_chunks > 0) {
      await_ready(0, read_ready(0));
      if (n_chunks > 1) await_ready(1, read_ready(1));
    }
    barrier_lds();
  }
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
    Fr hi[NKB], lo[NKB];
    state_frags(hi, lo);
    write_xs(sXS, hi, lo, true);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sh[kb] = hi[kb];
  }
  if (n_chunks > 0) {
    if (chain) {
      issue_k(0, sK, c4);
      issue_v(0, sV, sT, c4);
      if constexpr (kW) issue_w(0, sW, c4);
    } else {
      issue_q(0, sQ);
      issue_p(0, sP);
      if (n_chunks > 1) issue_k(1, sK + 64 * DK, hw);
      if (hw == 0) fetch_g(0);
    }
    wait_vmem();
    if (hw == 0) scan(0, sG2);
  }
  barrier_lds();

  // The boundary QDQ of chunk c on the chain waves (rd: the four waves' amax
  // of the chunk), the state fragments for the helpers' next S Q^T, the scale
  // for the next chunk's gate vector vn, and the optional records.
  auto chain_qdq = [&](const int c, const float* __restrict__ rd, E* __restrict__ xsb,
                       float* __restrict__ vn, const bool do_qdq, const bool last) {
    float s_new = 1.0f;
    if (do_qdq) {
      const float amax = fmaxf(fmaxf(rd[0], rd[1]), fmaxf(rd[2], rd[3]));
      s_new = qdq_scale_f64(amax);
      const double r = rcp_f64(s_new);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float c0[4], c1[4];
        if constexpr (kSplit) {
          // keep the codes; the scale is folded into the next decay multiply
          e4m3_codes4_f64(st[2 * kb], r, c0);
          e4m3_codes4_f64(st[2 * kb + 1], r, c1);
          st[2 * kb] = f32x4{c0[0], c0[1], c0[2], c0[3]};
          st[2 * kb + 1] = f32x4{c1[0], c1[1], c1[2], c1[3]};
          const float x[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
          sh[kb] = Eng::round(x);  // E4M3 values are exact in bf16
        } else {
          qdq4c_f64(st[2 * kb], c0, s_new, r);
          qdq4c_f64(st[2 * kb + 1], c1, s_new, r);
        }
      }
      s_cur = s_new;
      st_coded = kSplit;
    }
    if (!last) {
      if (kSplit && do_qdq) {
        write_xs(xsb, sh, sh, false);
      } else {
        Fr hi[NKB], lo[NKB];
        state_frags(hi, lo);
        write_xs(xsb, hi, lo, true);
        if constexpr (!kSplit) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) sh[kb] = hi[kb];  // fp32 engine: the exact state
        }
      }
      if (c4 == 0 && lane == 0) vn[193] = s_new;  // the scale of the state entering the next chunk
    }
    const int bidx = bound0 + c;
    if (args.bound_post) {
      const float f = st_coded ? s_cur : 1.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<float4*>(args.bound_post + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                   dkmap(16 * t + 4 * gq)) = make_float4(st[t][0] * f, st[t][1] * f,
                                                                         st[t][2] * f, st[t][3] * f);
    }
    if (args.bound_scales && tid == 0) args.bound_scales[((int64_t)bidx * H + h) * tiles + vt] = s_new;
  };

  // One chunk.  Every LDS buffer it touches arrives as a __restrict__
  // pointer, so the compiler can tell the buffers apart and does not hold LDS
  // reads behind the direct loads in flight into other buffers.
  auto step = [&](const int c, E* __restrict__ kc, E* __restrict__ kn, E* __restrict__ qc,
                  E* __restrict__ tb, E* __restrict__ vb, E* __restrict__ pb, E* __restrict__ pn,
                  E* __restrict__ xu, E* __restrict__ xs, E* __restrict__ kt, float* __restrict__ vec,
                  float* __restrict__ vecn, float* __restrict__ red, uint16_t* __restrict__ wb) {
    float* geg = vec + 64;    // exp(gamma)
    float* gegc = vec + 128;  // exp(gamma_C - gamma)
    float* gmisc = vec + 192; // [0] exp(gamma_C), [1] scale of the state entering the chunk
    const int t0 = seg0 + c * kChunk;
    const int nv = min(kChunk, P - c * kChunk);  // valid tokens in this chunk
    // the state entering this chunk is code * s_cur (bf16 engine, after a chunk QDQ)
    const bool coded_in = kSplit && c > 0 && (flags & GDN_QDQ_CHUNK);
    const bool two = kSplit && !coded_in;  // state operand as hi + lo
    const bool last = (c == n_chunks - 1);
    const bool do_qdq = (flags & GDN_QDQ_CHUNK) || ((flags & GDN_QDQ_WRITE) && last);

    f32x4 oacc[4];  // helper waves: O^T of this chunk, phase A -> B
    // ======== phase A ========
    if (chain) {
      // K S^T: A = K rows (tokens), B = the state
      const float sc = coded_in ? s_cur : 1.0f;
      f32x4 acc[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // the operand reads of a product all issued before its first MFMA, so
      // that they overlap one another instead of each waiting for the last
      Fr kf[4 * NKB];  // K rows, or with kW the W codes
      if constexpr (kW) {
#pragma unroll
        for (int f = 0; f < 4 * NKB; ++f) kf[f] = ld_bf16_frag<Eng>(wb + (f * 64 + lane) * 8);
      } else {
#pragma unroll
        for (int f = 0; f < 4 * NKB; ++f) kf[f] = Eng::ld(qslot(kc, f));  // f = tt * NKB + kb
      }
      if (two) {  // uncoded state: hi + lo from the fp32 state
        Fr hi[NKB], lo[NKB];
        state_frags(hi, lo);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            Eng::mma(acc[tt], kf[tt * NKB + kb], hi[kb]);
            Eng::mma(acc[tt], kf[tt * NKB + kb], lo[kb]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) Eng::mma(acc[tt], kf[tt * NKB + kb], sh[kb]);
      }
      Fr tf[6], tm[6], tl[6];  // T as hi, mid, lo planes (bf16 engine)
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        tf[p] = Eng::ld(slot(tb, p));
        if constexpr (kSplit) {
          tm[p] = Eng::ld(slot(tb, 6 + p));
          tl[p] = Eng::ld(slot(tb, 12 + p));
        }
      }
      if constexpr (kW) {
        // U' = T V - s w_s[t] (W S^T)[t][v]: V enters exactly, as the B
        // operand (element j = V[32kb + kperm(gq, j)][16c4 + ln])
        Fr vf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (Eng::kTrRead) {
            const uint2 r0 = lds_read_tr16(vb + (32 * kb + 4 * gq + (ln >> 2)) * RSV + 16 * c4 + 4 * (ln & 3));
            const uint2 r1 = lds_read_tr16(vb + (32 * kb + 16 + 4 * gq + (ln >> 2)) * RSV + 16 * c4 + 4 * (ln & 3));
            vf[kb] = __builtin_bit_cast(Fr, make_uint4(r0.x, r0.y, r1.x, r1.y));
          } else {
            float v8[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int i = 0; i < 4; ++i) v8[4 * hh + i] = Eng::to_f(vb[(32 * kb + 16 * hh + 4 * gq + i) * RSV + 16 * c4 + ln]);
            vf[kb] = Eng::round(v8);
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) uacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 6; ++p) {
          const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
          if constexpr (kSplit) {
            Eng::mma(uacc[ti], tl[p], vf[kb]);
            Eng::mma(uacc[ti], tm[p], vf[kb]);
          }
          Eng::mma(uacc[ti], tf[p], vf[kb]);
        }
        const float* wsc = reinterpret_cast<const float*>(wb + 4 * NKB * 512);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const float4 w4 = *reinterpret_cast<const float4*>(wsc + 16 * tt + 4 * gq);
          uacc[tt][0] = fmaf(-sc * w4.x, acc[tt][0], uacc[tt][0]);
          uacc[tt][1] = fmaf(-sc * w4.y, acc[tt][1], uacc[tt][1]);
          uacc[tt][2] = fmaf(-sc * w4.z, acc[tt][2], uacc[tt][2]);
          uacc[tt][3] = fmaf(-sc * w4.w, acc[tt][3], uacc[tt][3]);
        }
      } else {
      // X[t][v] = V[t][v] - s exp(gamma_t) (K S^T)[t][v], t = 16tt + 4gq + i
      Fr xh[2], xm[2], xl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x8[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int tt = 2 * kb + hh;
          const float4 e4 = *reinterpret_cast<const float4*>(geg + 16 * tt + 4 * gq);
          float vv[4];
          if constexpr (Eng::kTrRead) {
            // one transpose read: lane 4k + j of each 16-lane group points at row
            // 16tt + 4gq + k, columns 16c4 + 4j .. + 3, so lane ln receives column
            // 16c4 + ln of rows 16tt + 4gq + 0..3
            const uint2 r = lds_read_tr16(vb + (16 * tt + 4 * gq + (ln >> 2)) * RSV + 16 * c4 + 4 * (ln & 3));
            vv[0] = __uint_as_float(r.x << 16);
            vv[1] = __uint_as_float(r.x & 0xffff0000u);
            vv[2] = __uint_as_float(r.y << 16);
            vv[3] = __uint_as_float(r.y & 0xffff0000u);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = Eng::to_f(vb[(16 * tt + 4 * gq + i) * RSV + 16 * c4 + ln]);
          }
          x8[4 * hh + 0] = fmaf(-sc * e4.x, acc[tt][0], vv[0]);
          x8[4 * hh + 1] = fmaf(-sc * e4.y, acc[tt][1], vv[1]);
          x8[4 * hh + 2] = fmaf(-sc * e4.z, acc[tt][2], vv[2]);
          x8[4 * hh + 3] = fmaf(-sc * e4.w, acc[tt][3], vv[3]);
        }
        Eng::split3(x8, xh[kb], xm[kb], xl[kb]);
      }
      // U' = T X over the lower-triangular T pairs (ti, kb): (0,0) (1,0) (2,0)
      // (3,0) (2,1) (3,1).  bf16: T and X as three planes each (24 bits), the
      // six partial products down to 2^-16 of the leading one, smallest first
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) uacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        if constexpr (kSplit) {
          Eng::mma(uacc[ti], tf[p], xl[kb]);
          Eng::mma(uacc[ti], tl[p], xh[kb]);
          Eng::mma(uacc[ti], tm[p], xm[kb]);
          Eng::mma(uacc[ti], tf[p], xm[kb]);
          Eng::mma(uacc[ti], tm[p], xh[kb]);
        }
        Eng::mma(uacc[ti], tf[p], xh[kb]);
      }
      }  // kW
      // U' as the A operand of U'^T P^T, for the helper wave
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float u8[8] = {uacc[2 * kb][0], uacc[2 * kb][1], uacc[2 * kb][2], uacc[2 * kb][3],
                             uacc[2 * kb + 1][0], uacc[2 * kb + 1][1], uacc[2 * kb + 1][2],
                             uacc[2 * kb + 1][3]};
        Fr uh, ul;
        Eng::split(u8, uh, ul);
        Eng::st(slot(xu, c4 * 2 * NP + kb), uh);
        if constexpr (kSplit) Eng::st(slot(xu, c4 * 2 * NP + 2 + kb), ul);
      }
    } else {
      if constexpr (Ls::PBUF == 1) {
        if (c > 0) issue_p(c, pb);  // one P buffer: every helper read the last one in the previous step
      }
      if (c + 1 < n_chunks) {
        if constexpr (Ls::PBUF == 2) issue_p(c + 1, pn);  // the other P buffer
        // k of the next chunk into the buffer of the previous one (read by its update, before the barrier)
        if (Ls::PBUF == 2 && c > 0) issue_k(c + 1, kn, hw);
        if (hw == 0) fetch_g(c + 1);
      }
      transform(kc, kt);
      // O^T[v][t] = s exp(gamma_t) (S Q^T)[v][t] + (U'^T P^T)[v][t], v in block c4;
      // the first term here (XS holds the state entering the chunk), the second in phase B
      const float sc = coded_in ? gmisc[1] : 1.0f;
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) oacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      Fr qf[4 * NKB], sa[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sa[kb] = Eng::ld(slot(xs, c4 * NP * NKB + kb));
#pragma unroll
      for (int f = 0; f < 4 * NKB; ++f) qf[f] = Eng::ld(qslot(qc, f));  // f = ti * NKB + kb
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) Eng::mma(oacc[ti], sa[kb], qf[ti * NKB + kb]);
      if (two) {  // the lo plane of an uncoded state
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const Fr sb = Eng::ld(slot(xs, c4 * NP * NKB + NKB + kb));
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) Eng::mma(oacc[ti], sb, qf[ti * NKB + kb]);
        }
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const float egt = sc * geg[16 * ti + ln];
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[ti][i] *= egt;
      }
      if constexpr (Ls::PBUF == 1) wait_vmem();  // P of this chunk is read in the second phase
    }
    barrier_lds();

    // ======== phase B ========
    if (chain) {
      // S^T <- exp(gamma_C) S^T + K^T (exp(gamma_C - gamma) * U'), the
      // decayed U' as three bf16 planes (K enters exactly)
      Fr bh[2], bm[2], bl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 e0 = *reinterpret_cast<const float4*>(gegc + 32 * kb + 4 * gq);
        const float4 e1 = *reinterpret_cast<const float4*>(gegc + 32 * kb + 16 + 4 * gq);
        const float u8[8] = {e0.x * uacc[2 * kb][0], e0.y * uacc[2 * kb][1], e0.z * uacc[2 * kb][2],
                             e0.w * uacc[2 * kb][3], e1.x * uacc[2 * kb + 1][0],
                             e1.y * uacc[2 * kb + 1][1], e1.z * uacc[2 * kb + 1][2],
                             e1.w * uacc[2 * kb + 1][3]};
        Eng::split3(u8, bh[kb], bm[kb], bl[kb]);
      }
      float aC = st_coded ? gmisc[0] * s_cur : gmisc[0];  // decay, and the scale of a coded state
      if constexpr (kFused) aC *= *psn;  // NaN after a failed wait for a ready flag
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[t][i] *= aC;
      st_coded = false;
      // all K^T fragments first, so that the transpose reads overlap
      Fr ka0[NT], ka1[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Fr a0, a1;
        if constexpr (Eng::kTrRead) {
          // lane (gq, l) of each 16-lane group points at k[32kb + 16h + 4gq + l/4][dkmap(16t + 4(l%4)) .. +3]
          const int d = dkmap(16 * t + 4 * (ln & 3));
          const int t0 = 4 * gq + (ln >> 2);
          const uint2 x0 = lds_read_tr16(kc + kpos(t0, d)), x1 = lds_read_tr16(kc + kpos(t0 + 16, d));
          const uint2 y0 = lds_read_tr16(kc + kpos(t0 + 32, d)), y1 = lds_read_tr16(kc + kpos(t0 + 48, d));
          a0 = __builtin_bit_cast(Fr, make_uint4(x0.x, x0.y, x1.x, x1.y));
          a1 = __builtin_bit_cast(Fr, make_uint4(y0.x, y0.y, y1.x, y1.y));
        } else {
          a0 = Eng::ld(slot(kt, 2 * t));
          a1 = Eng::ld(slot(kt, 2 * t + 1));
        }
        ka0[t] = a0;
        ka1[t] = a1;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const Fr a0 = ka0[t], a1 = ka1[t];
        // the first 32 tokens' planes smallest first, then the second 32's
        if constexpr (kSplit) {
          Eng::mma(st[t], a0, bl[0]);
          Eng::mma(st[t], a0, bm[0]);
        }
        Eng::mma(st[t], a0, bh[0]);
        if constexpr (kSplit) {
          Eng::mma(st[t], a1, bl[1]);
          Eng::mma(st[t], a1, bm[1]);
        }
        Eng::mma(st[t], a1, bh[1]);
      }
      if (args.bound_pre) {
        const int bidx = bound0 + c;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          *reinterpret_cast<float4*>(args.bound_pre + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                     dkmap(16 * t + 4 * gq)) = make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
      }
      if (do_qdq) {
        float amax = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(st[t][i]));
        amax = wave_max_dpp(amax);
        // publish this wave's amax (slot of this chunk's parity), then its tag
        int* tags = reinterpret_cast<int*>(red + 8);
        if (lane == 0) {
          red[(c & 1) * 4 + c4] = amax;
          __hip_atomic_store(tags + c4, c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // wait until the four chain waves have published this chunk's amax
        // (the chain waves only; the helpers go on with their own work).
        // Every chain wave gets here in every chunk; the bound only keeps a
        // broken invariant from hanging the GPU.
        for (int spin = 0; spin < (1 << 22); ++spin) {
          int tmin = __hip_atomic_load(tags + 0, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
          for (int q = 1; q < 4; ++q)
            tmin = min(tmin, __hip_atomic_load(tags + q, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
          if (uniform(tmin) > c) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      chain_qdq(c, red + (c & 1) * 4, xs, vecn, do_qdq, last);
    } else {
      if (c + 1 < n_chunks) {
        issue_v(c + 1, vb, tb, hw);  // v and T were last read in phase A
        if constexpr (kW) issue_w(c + 1, wb, hw);  // and W
      }
      if constexpr (kFused) {
        if (hw == 1 && c + 2 < n_chunks) pend = load_ready(c + 2);  // checked at the end of the phase
      }
      Fr uh[2], ul[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uh[kb] = Eng::ld(slot(xu, c4 * 2 * NP + kb));
        if constexpr (kSplit) ul[kb] = Eng::ld(slot(xu, c4 * 2 * NP + 2 + kb));
      }
      // the P fragments in registers before q is issued: a wave waits at each
      // direct load until the load unit takes it, so the reads go out first
      Fr phs[6], pls[6];
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        phs[p] = Eng::ld(slot(pb, p));
        if constexpr (kSplit) pls[p] = Eng::ld(slot(pb, 6 + p));
      }
      if (c + 1 < n_chunks) issue_q(c + 1, qc);  // q was last read in phase A
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        Eng::mma(oacc[ti], uh[kb], phs[p]);
        if constexpr (kSplit) {
          Eng::mma(oacc[ti], ul[kb], phs[p]);
          Eng::mma(oacc[ti], uh[kb], pls[p]);
        }
      }
      // lane holds o[tok = 16ti + ln][16c4 + 4gq .. +3] of this tile
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int tok = 16 * ti + ln;
        if (tok < nv) {
          TO* dst = go_ + (int64_t)(t0 + tok) * v_row + (int64_t)h * dv + kTileRows * vt + 16 * c4 + 4 * gq;
          if constexpr (sizeof(TO) == 2) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(oacc[ti][0], oacc[ti][1]),
                                                        pack_bf16x2(oacc[ti][2], oacc[ti][3]));
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(oacc[ti][0], oacc[ti][1], oacc[ti][2], oacc[ti][3]);
          }
        }
      }
      if (Ls::PBUF == 1 && c + 1 < n_chunks) issue_k(c + 1, kn, hw);  // the update reads only this chunk's k
      if (c + 1 < n_chunks && hw == 0) scan(c + 1, vecn);  // gates of the next chunk, into the other vector
      wait_vmem();  // this wave's loads for the next chunk are in LDS before the barrier
      if constexpr (kFused) {
        if (hw == 1 && c + 2 < n_chunks) await_ready(c + 2, pend);  // P and T of chunk c + 2 load in the next step
      }
    }
    barrier_lds();
  };
  for (int c = 0; c < n_chunks; ++c) {
    const bool odd = c & 1;
    E* k0 = sK;
    E* k1 = sK + 64 * DK;
    E* p0 = sP;
    E* p1 = sP + (Ls::PBUF - 1) * 6 * NP * 64 * 8;
    float* v0 = sG2;
    float* v1 = sG2 + 3 * 64 + 8;
    step(c, odd ? k1 : k0, odd ? k0 : k1, sQ, sT, sV, odd ? p1 : p0, odd ? p0 : p1, sXU, sXS,
         Eng::kTrRead ? nullptr : sKT, odd ? v1 : v0, odd ? v0 : v1, sRed, sW);
  }

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
        const int th = tid - (kChunkThreads - kHelperThreads);
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
  for (int r = L + w; r < seg1 - seg0; r += kChunkWaves)
    io<TO>::st(go_ + (int64_t)(seg0 + r) * v_row + (int64_t)h * dv + kTileRows * vt + lane, 0.f);
}

template <int DK, class Eng, typename TIO, typename TO, bool kFused, bool kW>
static hipError_t launch_typed(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  auto kern = chunk_fwd_kernel<DK, Eng, TIO, TO, kFused, kW>;
  constexpr size_t item_lds = 2 * (size_t)PrepItemLds<DK, TIO, kW>::bytes;  // a producer's two items
  constexpr size_t state_lds = Lds<DK, Eng, kW>::bytes;
  constexpr size_t lds = (kFused && item_lds > state_lds) ? item_lds : state_lds;
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
  static PerDeviceOnce lds_attr;
  if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows) + (kFused ? a.n_prep : 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kChunkThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DK, class Eng, typename TIO, typename TO>
static hipError_t launch_sched(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  if (a.Wrec != nullptr)
    return a.fused ? launch_typed<DK, Eng, TIO, TO, true, true>(s, a, stream)
                   : launch_typed<DK, Eng, TIO, TO, false, true>(s, a, stream);
  return a.fused ? launch_typed<DK, Eng, TIO, TO, true, false>(s, a, stream)
                 : launch_typed<DK, Eng, TIO, TO, false, false>(s, a, stream);
}

// Compute units of the current device (0 when it cannot be read).
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

// Fused launch or two kernels.  The state part runs one workgroup per (n, h,
// value tile) for the whole sequence; when those fill at most half of the
// compute units, the idle ones produce the T and P records in the same launch
// (producer workgroups first) instead of a prep kernel that runs before it.
// Each workgroup of the launch takes a whole compute unit (its LDS), so all
// producers and consumers are resident together.
static int producer_workgroups(const gdn_shape_t& s, const gdn_debug_t* debug) {
  const int sched = debug ? debug->schedule : GDN_SCHEDULE_AUTO;
  if (sched == GDN_SCHEDULE_SPLIT || sched == GDN_SCHEDULE_FUSED_NO_PRODUCERS) return 0;
  const int64_t tiles = s.dv / kTileRows;
  const int64_t n_state = (int64_t)s.n_seqs * s.n_heads * tiles;
  // every value tile of a (sequence, head) pair on XCD nh % 8 (block mapping of the state part)
  if (tiles > 1 && ((int64_t)s.n_seqs * s.n_heads) % 8 != 0) return 0;
  const int n_cu = device_cu_count();
  if (n_cu < 16 || n_state + 8 > n_cu) return 0;
  if (sched != GDN_SCHEDULE_FUSED && 2 * n_state > n_cu) return 0;
  return (int)((n_cu - n_state) / 8 * 8);
}

hipError_t launch_chunk_fwd(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                            const float* beta, const float* g, const int32_t* cu_seqlens,
                            const int32_t* seq_lens, const int32_t* prefix_lens,
                            const float* initial_state, void* o, float* final_state,
                            void* workspace, const gdn_debug_t* debug, hipStream_t stream) {
  ChunkArgs a;
  const PrepLayout L = prep_layout(s, workspace);
  // fp32 inputs with dk = 128: the token recurrence (no per-chunk records)
  const bool token_path = s.io_dtype == GDN_F32 && s.dk == 128;
  const int n_prep = token_path ? 0 : producer_workgroups(s, debug);
  // test hook: the fused instantiation without its producers (every wait for a ready flag runs out)
  const bool no_producers = !token_path && debug && debug->schedule == GDN_SCHEDULE_FUSED_NO_PRODUCERS;
  const bool fused = n_prep > 0 || no_producers;
  hipError_t e = launch_prep(s, q, k, beta, g, cu_seqlens, seq_lens, prefix_lens, L, !fused && !token_path,
                             debug ? debug->w_pre : nullptr, debug ? debug->w_post : nullptr, stream);
  if (e != hipSuccess) return e;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
  a.cu_seqlens = cu_seqlens; a.seq_lens = seq_lens; a.prefix_lens = prefix_lens;
  a.chunk_offs = L.offs; a.T = L.T; a.Prec = L.P; a.Wrec = L.W;
  a.w_pre = debug ? debug->w_pre : nullptr;
  a.w_post = debug ? debug->w_post : nullptr;
  a.init = initial_state; a.o = o; a.fin = final_state;
  a.bound_offsets = debug ? debug->bound_offsets : nullptr;
  a.bound_pre = debug ? debug->bound_pre : nullptr;
  a.bound_post = debug ? debug->bound_post : nullptr;
  a.bound_scales = debug ? debug->scales : nullptr;
  a.H = s.n_heads; a.dv = s.dv; a.flags = s.qdq_flags;
  a.N = s.n_seqs; a.ready = L.ready; a.n_prep = n_prep; a.fused = fused ? 1 : 0;
  // the bf16 state kernel forms the first chunk's records itself when fused
  a.prep_c0 = (fused && !s.gate_per_channel && s.io_dtype == GDN_BF16 && L.W == nullptr) ? 1 : 0;
  a.status = L.status;
  a.grid_log2 = s.gate_grid_log2;
  {
    // state workgroups in more than one round: longest sequences first
    const int64_t n_state = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows);
    a.longest_first = (!fused && s.n_seqs > 1 && s.n_seqs <= 1024 && n_state > device_cu_count()) ? 1 : 0;
  }
  a.sfx_offsets = debug ? debug->suffix_offsets : nullptr;
  a.sfx_pre = debug ? debug->suffix_pre : nullptr;
  a.sfx_post = debug ? debug->suffix_post : nullptr;
  const bool ob = s.o_dtype == GDN_BF16;
  if (debug && debug->kernel_start) {
    e = hipEventRecord((hipEvent_t)debug->kernel_start, stream);
    if (e != hipSuccess) return e;
  }
  if (token_path) {
    e = launch_chunk_token(s, a, stream);
  } else if (s.gate_per_channel) {
    e = launch_kda_state(s, a, stream);
  } else if (s.io_dtype == GDN_BF16 && a.Wrec == nullptr) {
    e = launch_chunk_bf16(s, a, stream);
  } else if (s.io_dtype == GDN_BF16) {
    if (s.dk == 128)
      e = ob ? launch_sched<128, EngBF16, uint16_t, uint16_t>(s, a, stream)
             : launch_sched<128, EngBF16, uint16_t, float>(s, a, stream);
    else
      e = ob ? launch_sched<64, EngBF16, uint16_t, uint16_t>(s, a, stream)
             : launch_sched<64, EngBF16, uint16_t, float>(s, a, stream);
  } else if (s.dk == 64) {
    e = ob ? launch_sched<64, EngF32, float, uint16_t>(s, a, stream)
           : launch_sched<64, EngF32, float, float>(s, a, stream);
  } else {
    return hipErrorNotSupported;
  }
  if (e == hipSuccess && debug && debug->kernel_end)
    e = hipEventRecord((hipEvent_t)debug->kernel_end, stream);
  if (e == hipSuccess && debug && debug->status) e = launch_copy_status(L.status, debug->status, stream);
  return e;
}

}  // namespace gdn
