// gdn_kda.hip -- sequential part of the chunked forward with a per-key-channel
// gate (Model-Optimizer #2506 "What does this PR do?": per-key-channel
// retention, the decay acting on the key side of the state), with the same
// per-boundary FP8-E4M3 state QDQ as the scalar-gate kernel (#2497 "What does
// this PR do?"; #2519: QDQ at the handoff and after every later write).
//
// With gamma_r in R^dk the in-chunk cumulative log-gate of token r and
// gamma_C its value at the chunk's last token, one chunk of n <= 64 tokens
// (rows past n are zero) does ("o" is the elementwise product)
//     X  = V - s (K o exp(gamma)) S^T
//     U' = T X                                  (T: the per-chunk record)
//     O  = s (Q o exp(gamma)) S^T + P U'        (P: the per-chunk record)
//     S <- S diag(exp(gamma_C)) + U'^T (K o exp(gamma_C - gamma))
// where s is the scale of the coded state entering the chunk (1 when it is
// not coded).  Every exponential has a non-positive argument for
// non-positive gates.
//
// Work unit: one workgroup of 4 waves per (sequence n, head h, 64-row value
// tile vt).  Wave c owns value rows 16c..16c+15 of the tile (its slice of
// S^T in dk/16 fp32 accumulator fragments) and runs every product for them.
// Per chunk:
//   build  all waves: the per-channel gate prefix (DPP row scans) and the
//          scaled operands K o exp(gamma), Q o exp(gamma) and
//          K o exp(gamma_C - gamma) as MFMA fragment dumps in LDS (hi + lo
//          bf16 planes for bf16 inputs), exp(gamma_C) per key channel
//   B      per wave: X, U', O (stored), the state update, the tile amax
//   QDQ    per wave, once the four waves' amax are in LDS
// with two workgroup barriers.  The raw k, q, g of the next chunk are loaded
// into registers while the current chunk runs; v and the T and P records
// arrive by direct global->LDS loads issued one chunk ahead.  The records
// come from kda_prep_kernel or, in the fused launch, from producer
// workgroups of this same launch (produce_kda_records).  Then the
// recurrent suffix (tokens P_n < t <= L_n, QDQ after every write) and the
// final state store.
#include <type_traits>

#include "gdn_prep_item.hpp"

namespace gdn {

constexpr int kKdaThreads = 256;

// The state row that carries key channel c (the inverse of dkmap).
__host__ __device__ constexpr int dkmap_inv(int c) {
  return 32 * (c / 32) + 16 * ((c % 8) / 4) + 4 * ((c % 32) / 8) + c % 4;
}
static_assert(dkmap(dkmap_inv(77)) == 77 && dkmap_inv(dkmap(45)) == 45, "dkmap_inv");

// Inclusive prefix sum inside each row of 16 lanes (DPP row shifts).
__device__ __forceinline__ float row_prefix_sum(float v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  return v;
}
// The value of the previous lane of the row (0 in the row's first lane).
__device__ __forceinline__ float row_shift1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
}

// LDS layout (bytes).  F = one fragment dump (64 lanes x 8 elements); D = one
// plane of a 64 x dk operand (4 x dk/32 fragments).
//   Ka  [plane][tt][kb]  K o exp(gamma): lane l holds token 16tt + l%16,
//                        channels 32kb + 8(l/16) .. +7 (A of Ka S^T)
//   Qa  [plane][tt][kb]  Q o exp(gamma), the same layout (B of S Qa^T)
//   Kc  bf16: [plane][tt][kb] K o exp(gamma_C - gamma), slots rotated by
//       rot_slot (read back transposed by ds_read_b64_tr_b16); fp32: [dt][kb]
//       the transposed fragments themselves (A of the state update)
//   V   [64][64 + 16 bytes]   the tile's v rows
//   T, P  the prep kernel's records, copied as is
//   EC  exp(gamma_C) by state row [dk];  red  the four waves' amax
//   W   (kW only) the chunk's W record as is (codes, then row scales)
template <int DK, class Eng, bool kW = false>
struct KdaLds {
  using E = typename Eng::E;
  static constexpr int NKB = DK / 32, NP = Eng::kPlanes;
  static constexpr size_t F = 64 * 8 * sizeof(E);
  static constexpr size_t D = 4 * NKB * F;
  static constexpr size_t RV = 64 * sizeof(E) + 16;
  static constexpr size_t oKa = 0;
  static constexpr size_t oQa = oKa + NP * D;
  static constexpr size_t oKc = oQa + NP * D;
  static constexpr size_t oV = oKc + NP * D;
  static constexpr size_t oT = oV + 64 * RV;
  static constexpr size_t oP = oT + 6 * NP * F;
  static constexpr size_t oEC = oP + 6 * NP * F;
  static constexpr size_t oRed = oEC + DK * sizeof(float);
  static constexpr size_t oW = oRed + 8 * sizeof(float);
  static constexpr size_t bytes = oW + (kW ? (size_t)w_rec_bytes(DK) : 0);
  static_assert(6 * NP * F == kPRecBytes && 6 * NP * F <= kTRecBytes, "records and their LDS copies differ");
  static_assert(oW % 16 == 0, "direct loads need 16-byte aligned LDS");
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
  static_assert((3 * DK + 64 + 8) * sizeof(float) <= oV, "suffix buffers do not fit");
};

// Fused launch, workgroups 0 .. n_prep - 1: the T and P records of every
// (chunk, head) for a per-key-channel gate, one item at a time, published
// through the ready flags exactly as the scalar-gate producers do (same
// item order and XCD assignment, same flag bits; see gdn_chunk.hip).
template <int DK, typename TIO, bool kW>
__device__ __forceinline__ void produce_kda_records(const ChunkArgs& args, char* smem) {
  PrepArgs a;
  a.q = args.q; a.k = args.k; a.beta = args.beta; a.g = args.g; a.cu_seqlens = args.cu_seqlens;
  a.seq_lens = args.seq_lens; a.prefix_lens = args.prefix_lens; a.offs = args.chunk_offs;
  a.T = const_cast<void*>(args.T); a.P = const_cast<void*>(args.Prec); a.N = args.N; a.H = args.H;
  a.W = const_cast<void*>(args.Wrec); a.w_pre = args.w_pre; a.w_post = args.w_post;
  a.status = args.status;
  const int tid = threadIdx.x;
  const int H = args.H, NH = args.N * args.H;
  const int p = blockIdx.x, x = p & 7, r = p >> 3, R = args.n_prep >> 3;
  const unsigned xcd = xcd_id();
  const bool home = xcd == (unsigned)x;
  const int M = NH > x ? (NH - x + 7) >> 3 : 0;
  const int64_t total = (int64_t)args.chunk_offs[args.N + 1] * M;
  // item m: chunk m / M of the class's (m % M)-th pair; an item past its
  // sequence's prefix is skipped (the same for the whole workgroup)
  struct Item {
    int j, h, t0, nv;
  };
  auto item_at = [&](int64_t m, Item& it) {
    const int c = (int)(m / M), nh = x + 8 * (int)(m % M);
    const int n = nh / H;
    const int seg0 = args.cu_seqlens[n];
    const int L = args.seq_lens ? args.seq_lens[n] : (args.cu_seqlens[n + 1] - seg0);
    const int P = args.prefix_lens ? args.prefix_lens[n] : L;
    if (c * kChunk >= P) return false;
    it.j = args.chunk_offs[n] + c;
    it.h = nh % H;
    it.t0 = seg0 + c * kChunk;
    it.nv = min(kChunk, P - c * kChunk);
    return true;
  };
  auto next_item = [&](int64_t m, Item& it) {  // the first item at or after m, or total
    while (m < total && !item_at(m, it)) m += R;
    return m;
  };
  // The inputs of the next item are loaded into registers as soon as the
  // current item's are staged in LDS, so that they land while it computes.
  KdaRaw<DK, TIO> raw;
  Item cur{}, nxt{};
  int64_t m = next_item(r, cur);
  if (m < total) kda_fetch<DK, TIO>(a, cur.h, cur.t0, cur.nv, tid, raw);
  while (m < total) {
    const int64_t mn = next_item(m + R, nxt);
    // a fresh copy of the lane index per item keeps the compiler from holding
    // the item's lane-dependent LDS addresses live across the whole loop
    int tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    kda_prep_item_from<DK, TIO, kW>(a, cur.j, cur.h, cur.nv, smem, tid_i, raw, [&] {
      if (mn < total) kda_fetch<DK, TIO>(a, nxt.h, nxt.t0, nxt.nv, tid, raw);
    });
    const int j = cur.j, h = cur.h;
    cur = nxt;
    m = mn;
    wait_vmem();      // this wave's record stores are complete
    __syncthreads();  // ... in every wave; the LDS is free again
    if (tid == 0) {
      unsigned flag = 1u | (xcd << 1);
      if (!home) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        flag |= kReadyReleased;
      }
      __hip_atomic_store(args.ready + ((int64_t)j * H + h), flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int DK, class Eng, typename TIO, typename TO, bool kFused, bool kW>
__global__ __launch_bounds__(kKdaThreads, 1) void kda_fwd_kernel(ChunkArgs args) {
  using Ls = KdaLds<DK, Eng, kW>;
  using E = typename Eng::E;
  using Fr = typename Eng::Fr;
  constexpr int NT = DK / 16;
  constexpr int NKB = DK / 32;
  constexpr bool kSplit = Eng::kSplit;
  constexpr int PLANE = 4 * NKB * 64 * 8;  // elements of one operand plane
  extern __shared__ __align__(16) char smem[];
  if (index_check_failed(args.status)) return;
  if constexpr (kFused) {
    if ((int)blockIdx.x < args.n_prep) {
      produce_kda_records<DK, TIO, kW>(args, smem);
      return;
    }
  }
  E* sKa = reinterpret_cast<E*>(smem + Ls::oKa);
  E* sQa = reinterpret_cast<E*>(smem + Ls::oQa);
  E* sKc = reinterpret_cast<E*>(smem + Ls::oKc);
  E* sV = reinterpret_cast<E*>(smem + Ls::oV);
  E* sT = reinterpret_cast<E*>(smem + Ls::oT);
  E* sP = reinterpret_cast<E*>(smem + Ls::oP);
  float* sEC = reinterpret_cast<float*>(smem + Ls::oEC);
  float* sRed = reinterpret_cast<float*>(smem + Ls::oRed);
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem + Ls::oW);  // kW only

  const uint32_t lds0 = lds_base_u32(smem);
  auto lds_of = [&](const void* p) { return lds0 + (uint32_t)(reinterpret_cast<const char*>(p) - smem); };
  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);  // wave = value block of 16 rows
  const int lane = tid & 63;
  const int gq = lane >> 4;
  const int ln = lane & 15;
  const int c4 = w;
  auto slot = [lane](E* base, int f) { return base + (f * 64 + lane) * 8; };
  // element offset of Kc[t][d] in the rotated dump (bf16 engine)
  auto kpos = [](int t, int d) {
    return (((t >> 4) * (DK / 32) + (d >> 5)) * 64 + rot_slot(((d & 31) >> 3) * 16 + (t & 15))) * 8 + (d & 7);
  };

  const int H = args.H, dv = args.dv;
  const int tiles = dv / kTileRows;
  int nh, vt;  // value tiles of one head on one XCD when heads come in groups of 8
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
  const int64_t qk_row = (int64_t)H * DK;
  const int64_t v_row = (int64_t)H * dv;
  const int vcol0 = kTileRows * vt + 16 * c4 + ln;  // this lane's value row of S
  const int64_t state_base = ((int64_t)nh * dv + vcol0) * DK;
  const int n_chunks = (P + kChunk - 1) / kChunk;
  const int bound0 = args.bound_offsets ? args.bound_offsets[n] : 0;
  const int chunk0 = args.chunk_offs[n];

  // ---- state: st[t][i] = S[vcol0][dkmap(16t + 4gq + i)]
  f32x4 st[NT];
  Fr sh[NKB];          // after a chunk QDQ: the codes as the MFMA operand (bf16 engine)
  float s_cur = 1.0f;  // scale of the coded state
  auto state_frags = [&](Fr (&hi)[NKB], Fr (&lo)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float x[8] = {st[2 * kb][0], st[2 * kb][1], st[2 * kb][2], st[2 * kb][3],
                          st[2 * kb + 1][0], st[2 * kb + 1][1], st[2 * kb + 1][2], st[2 * kb + 1][3]};
      Eng::split(x, hi[kb], lo[kb]);
    }
  };

  // ---- builder lanes: channel group cg (8 channels), tokens 4 ln .. 4 ln + 3
  constexpr int NCG = DK / 8;
  constexpr int UPS = (int)sizeof(E) / 2;  // 16-byte pieces per 8 elements
  const int cg = 4 * w + gq;
  const bool builder = cg < NCG;
  uint4 rk[4][UPS], rq[4][UPS];
  float4 rg[4][2];
  // raw k, q, g of chunk cc into registers (builder lanes), per token slot t
  auto row_of = [&](int cc, int t) {
    const int nv = min(kChunk, P - cc * kChunk);
    return seg0 + cc * kChunk + (int64_t)min(4 * ln + t, nv - 1);
  };
  auto fetch_kq = [&](int cc, int t) {
    const int64_t row = row_of(cc, t);
    const uint4* kp = reinterpret_cast<const uint4*>(gk_ + row * qk_row + (int64_t)h * DK + 8 * cg);
    const uint4* qp = reinterpret_cast<const uint4*>(gq_ + row * qk_row + (int64_t)h * DK + 8 * cg);
#pragma unroll
    for (int u = 0; u < UPS; ++u) {
      rk[t][u] = kp[u];
      rq[t][u] = qp[u];
    }
  };
  auto fetch_g = [&](int cc) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4* gp = reinterpret_cast<const float4*>(args.g + (row_of(cc, t) * H + h) * DK + 8 * cg);
      rg[t][0] = gp[0];
      rg[t][1] = gp[1];
    }
  };
  auto fetch = [&](int cc) {
    if (builder) {
#pragma unroll
      for (int t = 0; t < 4; ++t) fetch_kq(cc, t);
      fetch_g(cc);
    }
  };
  auto unpack8 = [](const uint4 (&u)[UPS], float (&x)[8]) {
    if constexpr (UPS == 1) {
      const uint32_t wd[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(wd[j]);
        x[2 * j + 1] = bf16_hi(wd[j]);
      }
    } else {
      const uint32_t wd[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(wd[j]);
    }
  };
  // The operands of chunk cc from the raw values in registers; the raw
  // values of chunk nxt (if >= 0) are loaded into the same registers as soon
  // as each is consumed, so that those loads leave the load unit one at a time
  // between the build's arithmetic instead of stalling the wave in a burst.
  auto build = [&](int cc, int nxt) {
    if (builder) {
      const int nv = min(kChunk, P - cc * kChunk);
      float cum[4][8];  // prefix of the gate over this lane's tokens, natural log
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool valid = 4 * ln + t < nv;
        const float gv[8] = {rg[t][0].x, rg[t][0].y, rg[t][0].z, rg[t][0].w,
                             rg[t][1].x, rg[t][1].y, rg[t][1].z, rg[t][1].w};
#pragma unroll
        for (int m = 0; m < 8; ++m) cum[t][m] = (t ? cum[t - 1][m] : 0.f) + (valid ? gv[m] : 0.f);
      }
      if (nxt >= 0) fetch_g(nxt);
      float ex[8], gC[8];  // sum over the earlier lanes of the row; the chunk total
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        ex[m] = row_prefix_sum(row_shift1(cum[3][m]));
        gC[m] = __shfl(ex[m] + cum[3][m], lane | 15, 64);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = 4 * ln + t;
        const bool valid = tok < nv;
        float kf[8], qf[8];
        unpack8(rk[t], kf);
        unpack8(rq[t], qf);
        if (nxt >= 0) fetch_kq(nxt, t);
        float ka[8], qa[8], kc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float gt = ex[m] + cum[t][m];
          const float e1 = __builtin_amdgcn_exp2f(gt * kLog2e);
          const float e2 = __builtin_amdgcn_exp2f((gC[m] - gt) * kLog2e);
          const float kv = valid ? kf[m] : 0.f, qv = valid ? qf[m] : 0.f;
          ka[m] = kv * e1;
          qa[m] = qv * e1;
          kc[m] = kv * e2;
        }
        const int f = (tok >> 4) * NKB + (cg >> 2);
        const int lf = (tok & 15) + 16 * (cg & 3);
        E* pa = sKa + (f * 64 + lf) * 8;
        E* pq = sQa + (f * 64 + lf) * 8;
        if constexpr (kSplit) {
          Fr hi, lo;
          if constexpr (!kW) {  // with W QDQ the W codes take the place of K o exp(gamma)
            Eng::split(ka, hi, lo);
            Eng::st(pa, hi);
            Eng::st(pa + PLANE, lo);
          }
          Eng::split(qa, hi, lo);
          Eng::st(pq, hi);
          Eng::st(pq + PLANE, lo);
          E* pc = sKc + (f * 64 + rot_slot(lf)) * 8;
          Eng::split(kc, hi, lo);
          Eng::st(pc, hi);
          Eng::st(pc + PLANE, lo);
        } else {
          if constexpr (!kW) Eng::st(pa, Eng::round(ka));
          Eng::st(pq, Eng::round(qa));
          // transposed fragment f = 2 dt + kb: lane 16 g + sr % 16 holds
          // token 32 kb + kperm(g, j) of state row sr = 16 dt + sr % 16
          const int tk = tok & 31, kbt = tok >> 5;
          const int g4 = (tk & 15) >> 2, j = (tk >> 4) * 4 + (tk & 3);
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int sr = dkmap_inv(8 * cg + m);
            sKc[((2 * (sr >> 4) + kbt) * 64 + 16 * g4 + (sr & 15)) * 8 + j] = kc[m];
          }
        }
      }
      if (ln == 15) {
#pragma unroll
        for (int m = 0; m < 8; ++m) sEC[dkmap_inv(8 * cg + m)] = __builtin_amdgcn_exp2f(gC[m] * kLog2e);
      }
    }
  };

  // ---- direct loads of v rows and the T and P records of chunk cc (all waves)
  constexpr int EPP = 16 / (int)sizeof(E);
  constexpr int PPV = kTileRows / EPP;
  constexpr int RSV = (PPV + 1) * EPP;  // padded v row stride (elements)
  static_assert(sizeof(TIO) == sizeof(E), "LDS element type is the input type");
  auto issue_vtp = [&](int cc) {
    const int nv = min(kChunk, P - cc * kChunk);
    const int64_t row0 = seg0 + cc * kChunk;
    {
      constexpr int RPI = 64 / (PPV + 1);
      constexpr int NI = (64 + RPI - 1) / RPI;
      const TIO* src = gv_ + row0 * v_row + (int64_t)h * dv + kTileRows * vt;
      const int rr = lane / (PPV + 1), pc = lane % (PPV + 1);
      const int lane_off = min(pc, PPV - 1) * EPP;
#pragma unroll
      for (int ii = 0; ii < (NI + 3) / 4; ++ii) {
        const int i = w + 4 * ii;
        const int r = i * RPI + rr;
        if (i < NI && rr < RPI && r < 64)
          lds_load16(src, (uint32_t)((min(r, nv - 1) * (int)v_row + lane_off) * (int)sizeof(E)),
                     lds_of(sV) + i * RPI * (PPV + 1) * EPP * (int)sizeof(E));
      }
    }
    // T: its first two planes (hi, mid), P: both of its planes
    const char* trec = reinterpret_cast<const char*>(args.T) + ((int64_t)(chunk0 + cc) * H + h) * kTRecBytes;
    const char* prec = reinterpret_cast<const char*>(args.Prec) + ((int64_t)(chunk0 + cc) * H + h) * kPRecBytes;
#pragma unroll
    for (int ii = 0; ii < kPRecBytes / 1024 / 4; ++ii) {
      const int idx = w * (kPRecBytes / 1024 / 4) + ii;
      lds_load16(trec, (uint32_t)((idx * 64 + lane) * 16), lds_of(sT) + idx * 1024);
      lds_load16(prec, (uint32_t)((idx * 64 + lane) * 16), lds_of(sP) + idx * 1024);
    }
    if constexpr (kW) {
      constexpr int NI = w_rec_bytes(DK) / 1024;
      const char* wrec = reinterpret_cast<const char*>(args.Wrec) + ((int64_t)(chunk0 + cc) * H + h) * w_rec_bytes(DK);
#pragma unroll
      for (int ii = 0; ii < (NI + 3) / 4; ++ii) {
        const int idx = w + 4 * ii;
        if (idx < NI) lds_load16(wrec, (uint32_t)((idx * 64 + lane) * 16), lds_of(sW) + idx * 1024);
      }
    }
  };

  // ---- B: one chunk's products for this wave's 16 value rows
  // two_tag: the state enters as hi + lo (the split engine and no QDQ at the
  // boundary before the chunk), else as one plane (its E4M3 codes, or fp32);
  // a compile-time choice, so that no branch splits the products and the
  // operand reads can run ahead of them
  auto phase_b = [&](auto two_tag, int c) {
    const int t0 = seg0 + c * kChunk;
    const int nv = min(kChunk, P - c * kChunk);
    constexpr bool two = decltype(two_tag)::value;
    constexpr bool coded_in = kSplit && !two;
    const bool last = (c == n_chunks - 1);
    const bool do_qdq = (flags & GDN_QDQ_CHUNK) || ((flags & GDN_QDQ_WRITE) && last);
    const float sc = coded_in ? s_cur : 1.0f;
    Fr s_hi[NKB], s_lo[NKB];
    if constexpr (coded_in) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s_hi[kb] = sh[kb];
    } else {
      state_frags(s_hi, s_lo);
    }
    // (K o exp(gamma)) S^T: A = Ka rows (tokens), B = the state; with W QDQ
    // W_codes S^T (A = the W codes, exact in bf16: one plane)
    f32x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kW) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const Fr a = ld_bf16_frag<Eng>(sW + ((tt * NKB + kb) * 64 + lane) * 8);
          Eng::mma(acc[tt], a, s_hi[kb]);
          if constexpr (kSplit) {
            if constexpr (two) Eng::mma(acc[tt], a, s_lo[kb]);
          }
        }
    } else {
      // the fragments of a k-block are read together, then its products run
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Fr a[4], al[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          a[tt] = Eng::ld(slot(sKa, tt * NKB + kb));
          if constexpr (kSplit) al[tt] = Eng::ld(slot(sKa + PLANE, tt * NKB + kb));
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          Eng::mma(acc[tt], a[tt], s_hi[kb]);
          if constexpr (kSplit) {
            Eng::mma(acc[tt], al[tt], s_hi[kb]);
            if constexpr (two) Eng::mma(acc[tt], a[tt], s_lo[kb]);
          }
        }
      }
    }
    f32x4 uacc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) uacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kW) {
      // U' = T V - s w_s[t] (W S^T)[t][v]: V exact as the B operand
      Fr vf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float v8[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) v8[4 * hh + i] = Eng::to_f(sV[(32 * kb + 16 * hh + 4 * gq + i) * RSV + 16 * c4 + ln]);
        vf[kb] = Eng::round(v8);
      }
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        Eng::mma(uacc[ti], Eng::ld(slot(sT, p)), vf[kb]);
        if constexpr (kSplit) Eng::mma(uacc[ti], Eng::ld(slot(sT, 6 + p)), vf[kb]);
      }
      const float* wsc = reinterpret_cast<const float*>(sW + 4 * NKB * 512);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float4 w4 = *reinterpret_cast<const float4*>(wsc + 16 * tt + 4 * gq);
        uacc[tt][0] = fmaf(-sc * w4.x, acc[tt][0], uacc[tt][0]);
        uacc[tt][1] = fmaf(-sc * w4.y, acc[tt][1], uacc[tt][1]);
        uacc[tt][2] = fmaf(-sc * w4.z, acc[tt][2], uacc[tt][2]);
        uacc[tt][3] = fmaf(-sc * w4.w, acc[tt][3], uacc[tt][3]);
      }
    } else {
    // X[t][v] = V[t][v] - s (Ka S^T)[t][v], t = 16tt + 4gq + i
    Fr xh[2], xl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x8[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tt = 2 * kb + hh;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x8[4 * hh + i] = fmaf(-sc, acc[tt][i], Eng::to_f(sV[(16 * tt + 4 * gq + i) * RSV + 16 * c4 + ln]));
      }
      Eng::split(x8, xh[kb], xl[kb]);
    }
    // U' = T X over the lower-triangular pairs (ti, kb): (0,0) (1,0) (2,0) (3,0) (2,1) (3,1)
    // (T's fragments three pairs at a time, read before their products)
#pragma unroll
    for (int p0 = 0; p0 < 6; p0 += 3) {
      Fr tf[3], tl[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        tf[j] = Eng::ld(slot(sT, p0 + j));
        if constexpr (kSplit) tl[j] = Eng::ld(slot(sT, 6 + p0 + j));
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int p = p0 + j;
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        Eng::mma(uacc[ti], tf[j], xh[kb]);
        if constexpr (kSplit) {
          Eng::mma(uacc[ti], tf[j], xl[kb]);
          Eng::mma(uacc[ti], tl[j], xh[kb]);
        }
      }
    }
    }  // kW
    // U' fragments: A of U'^T P^T and B of the state update (the same registers)
    Fr uh[2], ul[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float u8[8] = {uacc[2 * kb][0], uacc[2 * kb][1], uacc[2 * kb][2], uacc[2 * kb][3],
                           uacc[2 * kb + 1][0], uacc[2 * kb + 1][1], uacc[2 * kb + 1][2],
                           uacc[2 * kb + 1][3]};
      Eng::split(u8, uh[kb], ul[kb]);
    }
    // S^T <- diag(exp(gamma_C)) S^T + (K o exp(gamma_C - gamma))^T U'
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 e = *reinterpret_cast<const float4*>(sEC + 16 * t + 4 * gq);
      st[t][0] *= e.x;
      st[t][1] *= e.y;
      st[t][2] *= e.z;
      st[t][3] *= e.w;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (Eng::kTrRead) {
        // lane (gq, l) of each 16-lane group points at Kc[32kb + 16h + 4gq + l/4][dkmap(16t + 4(l%4)) .. +3]
        const int d = dkmap(16 * t + 4 * (ln & 3));
        const int tq = 4 * gq + (ln >> 2);
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          const E* kc = sKc + pl * PLANE;
          const uint2 x0 = lds_read_tr16(kc + kpos(tq, d)), x1 = lds_read_tr16(kc + kpos(tq + 16, d));
          const uint2 y0 = lds_read_tr16(kc + kpos(tq + 32, d)), y1 = lds_read_tr16(kc + kpos(tq + 48, d));
          const Fr a0 = __builtin_bit_cast(Fr, make_uint4(x0.x, x0.y, x1.x, x1.y));
          const Fr a1 = __builtin_bit_cast(Fr, make_uint4(y0.x, y0.y, y1.x, y1.y));
          Eng::mma(st[t], a0, uh[0]);
          Eng::mma(st[t], a1, uh[1]);
          if (pl == 0) {
            Eng::mma(st[t], a0, ul[0]);
            Eng::mma(st[t], a1, ul[1]);
          }
        }
      } else {
        Eng::mma(st[t], Eng::ld(slot(sKc, 2 * t)), uh[0]);
        Eng::mma(st[t], Eng::ld(slot(sKc, 2 * t + 1)), uh[1]);
      }
    }
    // O^T[v][t] = s (S (Q o exp(gamma))^T)[v][t] + (U'^T P^T)[v][t]
    f32x4 oacc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) oacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      Fr bq[4], bql[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        bq[ti] = Eng::ld(slot(sQa, ti * NKB + kb));
        if constexpr (kSplit) bql[ti] = Eng::ld(slot(sQa + PLANE, ti * NKB + kb));
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        Eng::mma(oacc[ti], s_hi[kb], bq[ti]);
        if constexpr (kSplit) {
          Eng::mma(oacc[ti], s_hi[kb], bql[ti]);
          if constexpr (two) Eng::mma(oacc[ti], s_lo[kb], bq[ti]);
        }
      }
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[ti][i] *= sc;
#pragma unroll
    for (int p0 = 0; p0 < 6; p0 += 3) {
      Fr ph[3], pl[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        ph[j] = Eng::ld(slot(sP, p0 + j));
        if constexpr (kSplit) pl[j] = Eng::ld(slot(sP, 6 + p0 + j));
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int p = p0 + j;
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        Eng::mma(oacc[ti], uh[kb], ph[j]);
        if constexpr (kSplit) {
          Eng::mma(oacc[ti], ul[kb], ph[j]);
          Eng::mma(oacc[ti], uh[kb], pl[j]);
        }
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
      if (lane == 0) sRed[c4] = amax;
    }
  };

  // ---- QDQ of the tile once the four amax are in LDS
  auto qdq_step = [&](int c) {
    if constexpr (kFused) {  // NaN after a failed wait for a ready flag
      const float pz = sRed[4];
      if (pz != 1.0f) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[t][i] *= pz;
      }
    }
    const bool last = (c == n_chunks - 1);
    const bool do_qdq = (flags & GDN_QDQ_CHUNK) || ((flags & GDN_QDQ_WRITE) && last);
    float s_new = 1.0f;
    if (do_qdq) {
      const float amax = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
      s_new = qdq_scale_f64(amax);
      const double r = rcp_f64(s_new);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float c0[4], c1[4];
        qdq4c_f64(st[2 * kb], c0, s_new, r);
        qdq4c_f64(st[2 * kb + 1], c1, s_new, r);
        if constexpr (kSplit) {
          const float x[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
          sh[kb] = Eng::round(x);  // E4M3 values are exact in bf16
        }
      }
      s_cur = s_new;
    }
    const int bidx = bound0 + c;
    if (args.bound_post) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<float4*>(args.bound_post + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                   dkmap(16 * t + 4 * gq)) = make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    }
    if (args.bound_scales && tid == 0) args.bound_scales[((int64_t)bidx * H + h) * tiles + vt] = s_new;
  };

  // Fused launch: T and P of chunk cc come from a producer workgroup through
  // ready flag (chunk, head); wave 0 waits for it (await_ready_flag) before
  // the barrier that precedes their loads.  A failed wait sets red[4] to NaN,
  // which the next QDQ step multiplies into the state.
  unsigned pend = 0u;
  const unsigned xcd_self = kFused ? xcd_id() : 0u;
  auto ready_ptr = [&](int cc) { return args.ready + ((int64_t)(chunk0 + cc) * H + h); };
  auto load_ready = [&](int cc) { return __hip_atomic_load(ready_ptr(cc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  bool poisoned = false;
  auto await_ready = [&](int cc, unsigned v0) {
    if (!poisoned && !await_ready_flag(ready_ptr(cc), v0, xcd_self)) {
      poisoned = true;
      if (lane == 0) {
        sRed[4] = __builtin_nanf("");
        report_wait_timeout(args.status);
      }
    }
  };

  // ---------------- prologue ----------------
  if constexpr (kFused) {
    if (w == 0) {
      if (lane == 0) sRed[4] = 1.0f;
      if (n_chunks > 0) await_ready(0, load_ready(0));
    }
    barrier_lds();
  }
  if (n_chunks > 0) {
    fetch(0);
    issue_vtp(0);
  }
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
  if (n_chunks > 0) build(0, n_chunks > 1 ? 1 : -1);
  // Chunk c: B reads the operands built for c and the v/T/P loads of c; the
  // operands of c + 1 are built once every wave is past the second barrier.
  for (int c = 0; c < n_chunks; ++c) {
    wait_vmem();  // this wave's direct loads are in LDS before the barrier
    barrier_lds();
    if constexpr (kFused) {
      if (w == 0 && c + 1 < n_chunks) pend = load_ready(c + 1);  // examined after phase B
    }
    if (kSplit && !(c > 0 && (flags & GDN_QDQ_CHUNK)))
      phase_b(std::true_type{}, c);
    else
      phase_b(std::false_type{}, c);
    if constexpr (kFused) {
      if (w == 0 && c + 1 < n_chunks) await_ready(c + 1, pend);  // T and P of chunk c + 1 load after the barrier
    }
    barrier_lds();
    if (c + 1 < n_chunks) {
      build(c + 1, c + 2 < n_chunks ? c + 2 : -1);
      issue_vtp(c + 1);
    }
    qdq_step(c);
  }

  // ---------------- recurrent suffix, tokens P < t <= L ----------------
  // optional per-token record: this wave's rows of the state after each
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
    float* sq = reinterpret_cast<float*>(smem + Ls::oKa);  // q_t, k_t, g_t: DK each; v_t: 64; beta_t
    float* sk = sq + DK;
    float* sg = sk + DK;
    float* sv = sg + DK;
    float* sb = sv + 64;
    for (int t = P; t < L; ++t) {
      const int64_t row = seg0 + t;
      __syncthreads();  // the previous token's reads are done
      if (tid < DK) {
        sq[tid] = io<TIO>::ld(gq_ + row * qk_row + (int64_t)h * DK + tid);
        sk[tid] = io<TIO>::ld(gk_ + row * qk_row + (int64_t)h * DK + tid);
        sg[tid] = args.g[(row * H + h) * DK + tid];
      }
      if (tid < 64) sv[tid] = io<TIO>::ld(gv_ + row * v_row + (int64_t)h * dv + kTileRows * vt + tid);
      if (tid == 0) sb[0] = args.beta[row * H + h];
      __syncthreads();
      const float b = sb[0];
      float y = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = dkmap(16 * t2 + 4 * gq + i);
          st[t2][i] *= expf(grid_gate(sg[d], args.grid_log2));
          y += st[t2][i] * sk[d];
        }
      y += __shfl_xor(y, 16, 64);
      y += __shfl_xor(y, 32, 64);
      const float u = b * (sv[16 * c4 + ln] - y);
      float z = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = dkmap(16 * t2 + 4 * gq + i);
          st[t2][i] += u * sk[d];
          z += st[t2][i] * sq[d];
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
        __syncthreads();
        const float s = qdq_scale(fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3])));
        const float r = 1.0f / s;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2) qdq4(st[t2], s, r);
      }
      if (sfx_post) store_state(sfx_post + (sfx0 + t - P) * sfx_stride);
    }
  }

  // ---------------- final state, zero padding rows of o ----------------
#pragma unroll
  for (int t = 0; t < NT; ++t)
    *reinterpret_cast<float4*>(args.fin + state_base + dkmap(16 * t + 4 * gq)) =
        make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
  for (int r = L + w; r < seg1 - seg0; r += kKdaThreads / 64)
    io<TO>::st(go_ + (int64_t)(seg0 + r) * v_row + (int64_t)h * dv + kTileRows * vt + lane, 0.f);
}

template <int DK, class Eng, typename TIO, typename TO, bool kFused, bool kW>
static hipError_t launch_kda_typed(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  auto kern = kda_fwd_kernel<DK, Eng, TIO, TO, kFused, kW>;
  constexpr size_t prep_lds = KdaPrepLds<DK, TIO, kW>::bytes;  // a producer's item
  constexpr size_t state_lds = KdaLds<DK, Eng, kW>::bytes;
  constexpr size_t lds = (kFused && prep_lds > state_lds) ? prep_lds : state_lds;
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
  static PerDeviceOnce lds_attr;
  if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows) + (kFused ? a.n_prep : 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kKdaThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DK, class Eng, typename TIO, typename TO>
static hipError_t launch_kda_sched(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  if (a.Wrec != nullptr)
    return a.fused ? launch_kda_typed<DK, Eng, TIO, TO, true, true>(s, a, stream)
                   : launch_kda_typed<DK, Eng, TIO, TO, false, true>(s, a, stream);
  return a.fused ? launch_kda_typed<DK, Eng, TIO, TO, true, false>(s, a, stream)
                 : launch_kda_typed<DK, Eng, TIO, TO, false, false>(s, a, stream);
}

hipError_t launch_kda_state(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  const bool ob = s.o_dtype == GDN_BF16;
  if (s.io_dtype == GDN_BF16) {
    if (s.dk == 128)
      return ob ? launch_kda_sched<128, EngBF16, uint16_t, uint16_t>(s, a, stream)
                : launch_kda_sched<128, EngBF16, uint16_t, float>(s, a, stream);
    return ob ? launch_kda_sched<64, EngBF16, uint16_t, uint16_t>(s, a, stream)
              : launch_kda_sched<64, EngBF16, uint16_t, float>(s, a, stream);
  }
  if (s.dk != 64) return hipErrorNotSupported;
  return ob ? launch_kda_sched<64, EngF32, float, uint16_t>(s, a, stream)
            : launch_kda_sched<64, EngF32, float, float>(s, a, stream);
}

}  // namespace gdn
