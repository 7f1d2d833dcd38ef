// gdn_chunk.hip -- sequential part of the chunked gated delta rule forward
// with per-boundary FP8-E4M3 state QDQ (Model-Optimizer #2497 "What does this
// PR do?": 64-token chunks, WY-transformed W, dynamic per-tile state QDQ at
// every boundary; #2519: QDQ at the handoff and after every later recurrent
// write).
//
// Work unit: one workgroup (4 waves) per (sequence n, head h, 64-column value
// tile vt).  It walks its sequence chunk by chunk and keeps its slice of the
// state in registers for the whole sequence: wave w owns value columns
// 16w..16w+15 of the tile, i.e. dk/16 16x16 accumulator tiles of S^T.  The
// 64 x dk state tile is exactly one QDQ tile, so the QDQ amax needs no
// exchange with other workgroups.  T = (I + A)^-1 diag(beta) of every chunk
// comes from the prep kernel (gdn_prep.hip) through the workspace.
//
// Per chunk of n <= 64 tokens (rows past n are zero, beta = g = 0, so they
// drop out of every product), gamma = in-chunk cumulative log-gate:
//   a1  stage q, k (row-major and transposed), v (transposed) and T -> LDS;
//       gamma (wave scan), exp(gamma), exp(gamma_C - gamma).  The next
//       chunk's inputs are already in flight to registers.
//   a3  P[r][s] = exp(gamma_r - gamma_s) q_r . k_s  (s <= r)          MFMA
//   a5  W = T (exp(gamma) * K)  (as W^T = (exp(gamma) * K)^T T^T),
//       U = T V                                                        MFMA
//   a6  U' = U - W S^T                                                 MFMA
//   a7  O^T = diag-scaled S Q^T + U'^T P^T   (o lands 4 values per lane)
//   a8  S^T <- exp(gamma_C) S^T + K^T diag(exp(gamma_C - gamma)) U'    MFMA
//   a9  QDQ: amax over the 64 x dk tile (wave + LDS tree), s = amax/448,
//       S <- RNE_E4M3(S/s) s
// then the recurrent suffix (tokens P_n < t <= L_n, QDQ after every write)
// and the final state store.
//
// The state fragment built once per k-block serves as the B operand of
// W S^T and as the A operand of S Q^T: an accumulator tile already holds, in
// every lane, the eight k-slots a fragment needs (see gdn_device.hpp).
//
// Precision (bf16 inputs, fp32 accumulate): q, k, v enter the MFMAs exactly;
// T, P and U' as hi + lo bf16 pairs; exp(gamma) * K and W as one bf16 each.
// After a QDQ the state is code * s with the code exactly representable in
// bf16, so it is fed as the codes and the products are scaled by s; otherwise
// (QDQ off, supplied initial state) as a hi + lo pair.  fp32 inputs use the
// fp32 MFMA throughout.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

struct Frag8 {
  float v[8];
};

// bf16 engine: LDS operands are bf16 bit patterns.
struct EngBF16 {
  using E = uint16_t;
  using Fr = bf16x8;
  static constexpr bool kSplit = true;
  static __device__ __forceinline__ Fr load(const E* row, int kb, int gq) {
    const uint2 a = *reinterpret_cast<const uint2*>(row + 32 * kb + 4 * gq);
    const uint2 b = *reinterpret_cast<const uint2*>(row + 32 * kb + 16 + 4 * gq);
    return __builtin_bit_cast(Fr, make_uint4(a.x, a.y, b.x, b.y));
  }
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
  // fragment with every element j multiplied by f[j] (one rounding)
  static __device__ __forceinline__ Fr scale(const Fr& x, const float (&f)[8]) {
    const uint4 u = __builtin_bit_cast(uint4, x);
    const float v[8] = {bf16_lo(u.x) * f[0], bf16_hi(u.x) * f[1], bf16_lo(u.y) * f[2], bf16_hi(u.y) * f[3],
                        bf16_lo(u.z) * f[4], bf16_hi(u.z) * f[5], bf16_lo(u.w) * f[6], bf16_hi(u.w) * f[7]};
    return round(v);
  }
  static __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
  static __device__ __forceinline__ void store4_split(E* ph, E* pl, const float (&x)[4]) {
    uint32_t h0, l0, h1, l1;
    split_bf16x2(x[0], x[1], h0, l0);
    split_bf16x2(x[2], x[3], h1, l1);
    *reinterpret_cast<uint2*>(ph) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(pl) = make_uint2(l0, l1);
  }
  // two rows, same column: one 4-byte LDS write of (row r, row r+1)
  static __device__ __forceinline__ void store_pair(E* p, E a, E b) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)a | ((uint32_t)b << 16);
  }
};

// fp32 engine: LDS operands are fp32, products use the fp32 MFMA.
struct EngF32 {
  using E = float;
  using Fr = Frag8;
  static constexpr bool kSplit = false;
  static __device__ __forceinline__ Fr load(const E* row, int kb, int gq) {
    const float4 a = *reinterpret_cast<const float4*>(row + 32 * kb + 4 * gq);
    const float4 b = *reinterpret_cast<const float4*>(row + 32 * kb + 16 + 4 * gq);
    Fr f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
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
  static __device__ __forceinline__ Fr scale(const Fr& x, const float (&f)[8]) {
    Fr r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = x.v[j] * f[j];
    return r;
  }
  static __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
  static __device__ __forceinline__ void store4_split(E* ph, E* pl, const float (&x)[4]) {
    (void)pl;
    *reinterpret_cast<float4*>(ph) = make_float4(x[0], x[1], x[2], x[3]);
  }
  static __device__ __forceinline__ void store_pair(E* p, E a, E b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};

// LDS layout of the sequential kernel (bytes).  Row strides are padded so
// that the 16 rows read by one fragment load fall in different banks; [64][dk]
// rows stay 16-byte aligned for the staging stores.
template <int DK, class Eng>
struct Smem {
  using E = typename Eng::E;
  static constexpr int LDK = DK + 16 / (int)sizeof(E);  // stride of [64][DK] buffers (E)
  static constexpr int L64 = 64 + 4;                     // stride of [*][64] buffers (E)
  static constexpr int kSplitN = Eng::kSplit ? 2 : 1;
  static constexpr size_t szK = 64 * LDK * sizeof(E);
  static constexpr size_t szKT = DK * L64 * sizeof(E);
  static constexpr size_t szM = 64 * L64 * sizeof(E);  // one 64x64 operand matrix
  static constexpr size_t oK = 0;
  static constexpr size_t oKT = oK + szK;
  static constexpr size_t oQ = oKT + szKT;
  static constexpr size_t oVT = oQ + szK;
  static constexpr size_t oT = oVT + szM;               // T hi [, T lo]
  static constexpr size_t oP = oT + kSplitN * szM;      // P hi [, P lo]
  static constexpr size_t oW = oP + kSplitN * szM;      // W [64][DK]
  static constexpr size_t oVec = oW + szK;              // gamma*log2e, e^gamma, e^(gC-gamma), beta
  static constexpr size_t oRed = oVec + 4 * 64 * sizeof(float);
  static constexpr size_t bytes = oRed + 16 * sizeof(float);
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

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
  const void* T;              // 16 KiB record per (chunk, head) (prep kernel)
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
};

constexpr float kLog2e = 1.4426950408889634f;

template <int DK, class Eng, typename TIO, typename TO>
__global__ __launch_bounds__(kThreads, 1) void chunk_fwd_kernel(ChunkArgs args) {
  using S_ = Smem<DK, Eng>;
  using E = typename Eng::E;
  using Fr = typename Eng::Fr;
  constexpr int LDK = S_::LDK;
  constexpr int L64 = S_::L64;
  constexpr int NT = DK / 16;   // state accumulator tiles per wave
  constexpr int NKB = DK / 32;  // k-blocks over dk
  extern __shared__ __align__(16) char smem[];
  E* sK = reinterpret_cast<E*>(smem + S_::oK);
  E* sKT = reinterpret_cast<E*>(smem + S_::oKT);
  E* sQ = reinterpret_cast<E*>(smem + S_::oQ);
  E* sVT = reinterpret_cast<E*>(smem + S_::oVT);
  E* sTh = reinterpret_cast<E*>(smem + S_::oT);
  E* sTl = sTh + 64 * L64;
  E* sPh = reinterpret_cast<E*>(smem + S_::oP);
  E* sPl = sPh + 64 * L64;
  E* sW = reinterpret_cast<E*>(smem + S_::oW);
  float* sG2 = reinterpret_cast<float*>(smem + S_::oVec);  // gamma * log2(e)
  float* sEg = sG2 + 64;
  float* sEgc = sEg + 64;
  float* sBeta = sEgc + 64;
  float* sRed = reinterpret_cast<float*>(smem + S_::oRed);

  const int tid = threadIdx.x;
  const int w = tid >> 6;        // wave
  const int lane = tid & 63;
  const int gq = lane >> 4;      // lane group (k-slots / accumulator rows 4gq..4gq+3)
  const int ln = lane & 15;      // accumulator column / fragment row

  const int H = args.H, dv = args.dv;
  const int tiles = dv / kTileRows;
  // Block -> (n*H + h, vt).  Workgroups are dispatched to the 8 XCDs round
  // robin; when heads come in groups of 8, the value tiles of one head get
  // block ids 8 apart, i.e. the same XCD, so their q/k reads share an L2.
  int nh, vt;
  {
    const int b = blockIdx.x, G = gridDim.x;
    if (tiles > 1 && G % (8 * tiles) == 0) {
      const int slot = b >> 3;
      vt = slot % tiles;
      nh = (slot / tiles) * 8 + (b & 7);
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
  const int vcol0 = kTileRows * vt + 16 * w + ln;  // this lane's value column (in dv)

  // ---- state: st[t][i] = S^T[16t + 4gq + i][vcol] = S[vcol][16t + 4gq + i]
  f32x4 st[NT];
  const int64_t state_base = ((int64_t)nh * dv + vcol0) * DK;  // row vcol0 of S
  if (args.init != nullptr) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 x = *reinterpret_cast<const float4*>(args.init + state_base + 16 * t + 4 * gq);
      st[t] = f32x4{x.x, x.y, x.z, x.w};
    }
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool coded = false;   // state is code * s_cur with codes on the E4M3 grid
  float s_cur = 1.0f;
  float inv_s = 1.0f;

  const int n_chunks = (P + kChunk - 1) / kChunk;
  const int bound0 = args.bound_offsets ? args.bound_offsets[n] : 0;
  const int chunk0 = args.chunk_offs[n];

  // ---- staging geometry: 16-byte segments, two adjacent rows per thread
  constexpr int EPS = 16 / (int)sizeof(TIO);   // elements per segment
  constexpr int SPR = DK / EPS;                // segments per q/k row
  constexpr int NPK = 64 * SPR / kThreads / 2; // row pairs per thread (q/k)
  constexpr int VSPR = kTileRows / EPS;        // segments per v row
  constexpr int NPV = 64 * VSPR / kThreads / 2;
  constexpr int NTS = 16384 / 16 / kThreads;   // 16-byte pieces of a T record per thread
  static_assert(NPK >= 1 && NPV >= 1 && NTS == 4, "staging geometry");
  // per-thread global offsets (elements) of chunk 0; chunk c adds c * 64 rows
  int64_t kq_off[NPK][2], v_off[NPV][2];
  int kq_row[NPK][2], v_row_i[NPV][2];
#pragma unroll
  for (int j = 0; j < NPK; ++j)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * (tid / SPR + (kThreads / SPR) * j) + e;
      kq_row[j][e] = r;
      kq_off[j][e] = (int64_t)(seg0 + r) * qk_row + (int64_t)h * DK + (tid % SPR) * EPS;
    }
#pragma unroll
  for (int j = 0; j < NPV; ++j)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * (tid / VSPR + (kThreads / VSPR) * j) + e;
      v_row_i[j][e] = r;
      v_off[j][e] = (int64_t)(seg0 + r) * v_row + (int64_t)h * dv + kTileRows * vt + (tid % VSPR) * EPS;
    }
  const uint4* Trec = reinterpret_cast<const uint4*>(args.T);
  uint4 pk[NPK][2], pq[NPK][2], pv[NPV][2], pt[NTS];
  float pg = 0.f, pb = 0.f;
  // Loads are unconditional (rows past the chunk's valid count are clamped to
  // its last valid row) so they stay in flight; the zero mask is applied when
  // the data is written to LDS.
  auto fetch = [&](int c) {
    const int nv = min(kChunk, P - c * kChunk);
    const int64_t dqk = (int64_t)c * kChunk * qk_row, dvv = (int64_t)c * kChunk * v_row;
#pragma unroll
    for (int j = 0; j < NPK; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t clamp = (int64_t)(min(kq_row[j][e], nv - 1) - kq_row[j][e]) * qk_row;
        pk[j][e] = *reinterpret_cast<const uint4*>(gk_ + kq_off[j][e] + dqk + clamp);
        pq[j][e] = *reinterpret_cast<const uint4*>(gq_ + kq_off[j][e] + dqk + clamp);
      }
#pragma unroll
    for (int j = 0; j < NPV; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t clamp = (int64_t)(min(v_row_i[j][e], nv - 1) - v_row_i[j][e]) * v_row;
        pv[j][e] = *reinterpret_cast<const uint4*>(gv_ + v_off[j][e] + dvv + clamp);
      }
    const uint4* rec = Trec + ((int64_t)(chunk0 + c) * H + h) * (16384 / 16);
#pragma unroll
    for (int j = 0; j < NTS; ++j) pt[j] = rec[tid + kThreads * j];
    if (w == 0) {
      const int64_t gi = (int64_t)(seg0 + c * kChunk + min(lane, nv - 1)) * H + h;
      pg = args.g[gi];
      pb = args.beta[gi];
    }
  };
  if (n_chunks > 0) fetch(0);

  for (int c = 0; c < n_chunks; ++c) {
    const int t0 = seg0 + c * kChunk;
    const int nv = min(kChunk, P - c * kChunk);  // valid tokens in this chunk

    // ---------------- a1: staged registers -> LDS; gates ----------------
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < NPK; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (kq_row[j][e] >= nv) { pk[j][e] = zero4; pq[j][e] = zero4; }
#pragma unroll
    for (int j = 0; j < NPV; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (v_row_i[j][e] >= nv) pv[j][e] = zero4;
    if (lane >= nv) { pg = 0.f; pb = 0.f; }
#pragma unroll
    for (int j = 0; j < NPK; ++j) {
      const int r0 = kq_row[j][0], c0 = (tid % SPR) * EPS;
      *reinterpret_cast<uint4*>(sK + r0 * LDK + c0) = pk[j][0];
      *reinterpret_cast<uint4*>(sK + (r0 + 1) * LDK + c0) = pk[j][1];
      *reinterpret_cast<uint4*>(sQ + r0 * LDK + c0) = pq[j][0];
      *reinterpret_cast<uint4*>(sQ + (r0 + 1) * LDK + c0) = pq[j][1];
      E k0[EPS], k1[EPS];
      __builtin_memcpy(k0, &pk[j][0], 16);
      __builtin_memcpy(k1, &pk[j][1], 16);
#pragma unroll
      for (int e = 0; e < EPS; ++e) Eng::store_pair(sKT + (c0 + e) * L64 + r0, k0[e], k1[e]);
    }
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      const int r0 = v_row_i[j][0], c0 = (tid % VSPR) * EPS;
      E v0[EPS], v1[EPS];
      __builtin_memcpy(v0, &pv[j][0], 16);
      __builtin_memcpy(v1, &pv[j][1], 16);
#pragma unroll
      for (int e = 0; e < EPS; ++e) Eng::store_pair(sVT + (c0 + e) * L64 + r0, v0[e], v1[e]);
    }
    // T record: bf16 = hi plane then lo plane ([64][64] each); fp32 = one plane
#pragma unroll
    for (int j = 0; j < NTS; ++j) {
      const int idx = tid + kThreads * j;            // 16-byte piece
      if constexpr (Eng::kSplit) {
        const int plane = idx >> 9, rr = (idx >> 3) & 63, cc = (idx & 7) * 8;
        E* dst = (plane ? sTl : sTh) + rr * L64 + cc;
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(pt[j].x, pt[j].y);
        reinterpret_cast<uint2*>(dst)[1] = make_uint2(pt[j].z, pt[j].w);
      } else {
        const int rr = idx >> 4, cc = (idx & 15) * 4;
        *reinterpret_cast<uint4*>(sTh + rr * L64 + cc) = pt[j];
      }
    }
    if (w == 0) {
      float x = pg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float gC = __shfl(x, 63, 64);
      sG2[lane] = x * kLog2e;
      sEg[lane] = __builtin_amdgcn_exp2f(x * kLog2e);
      sEgc[lane] = __builtin_amdgcn_exp2f((gC - x) * kLog2e);
      sBeta[lane] = pb;
      if (lane == 0) sRed[4] = __builtin_amdgcn_exp2f(gC * kLog2e);
    }
    if (c + 1 < n_chunks) fetch(c + 1);   // lands in registers while this chunk computes
    __syncthreads();

    // ---------------- a3: P = decay * Q K^T (lower incl. diagonal) ----------------
    // 10 lower tiles + 2 zero tiles read by the triangular products; 3 per wave
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int job = w + 4 * jj;
      int ri, si;
      if (job < 10) {
        ri = (job < 1) ? 0 : (job < 3) ? 1 : (job < 6) ? 2 : 3;
        si = job - (ri * (ri + 1)) / 2;
      } else {
        si = (job == 10) ? 1 : 3;
        ri = si - 1;
      }
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      if (job < 10) {
        // C[s][r] = sum_d K[s][d] Q[r][d]
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        Fr af[NKB], bf[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          af[kb] = Eng::load(sK + (16 * si + ln) * LDK, kb, gq);
          bf[kb] = Eng::load(sQ + (16 * ri + ln) * LDK, kb, gq);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Eng::mma(acc, af[kb], bf[kb]);
        const int r = 16 * ri + ln;
        const float g2r = sG2[r];
        const float4 g2s = *reinterpret_cast<const float4*>(sG2 + 16 * si + 4 * gq);
        const float gs[4] = {g2s.x, g2s.y, g2s.z, g2s.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * si + 4 * gq + i;
          x[i] = (s <= r) ? __builtin_amdgcn_exp2f(g2r - gs[i]) * acc[i] : 0.f;
        }
      }
      const int r = 16 * ri + ln;
      Eng::store4_split(sPh + r * L64 + 16 * si + 4 * gq, sPl + r * L64 + 16 * si + 4 * gq, x);
    }

    // ---------------- a5: W^T = (e^gamma K)^T T^T (-> sW row-major), U = T V ----------------
    f32x4 uacc[4];
    {
      constexpr int DPW = NT / 4;  // dk tiles of W^T per wave
      // (ti, kb) pairs of the lower-triangular T: (0,0) (1,0) (2,0) (3,0) (2,1) (3,1)
      Fr th[6], tl[6];
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        th[p] = Eng::load(sTh + (16 * ti + ln) * L64, kb, gq);
        if constexpr (Eng::kSplit) tl[p] = Eng::load(sTl + (16 * ti + ln) * L64, kb, gq);
      }
      Fr ka[DPW][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 e0 = *reinterpret_cast<const float4*>(sEg + 32 * kb + 4 * gq);
        const float4 e1 = *reinterpret_cast<const float4*>(sEg + 32 * kb + 16 + 4 * gq);
        const float ef[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
          ka[dd][kb] = Eng::scale(Eng::load(sKT + (16 * (DPW * w + dd) + ln) * L64, kb, gq), ef);
      }
      const Fr vb0 = Eng::load(sVT + (16 * w + ln) * L64, 0, gq);
      const Fr vb1 = Eng::load(sVT + (16 * w + ln) * L64, 1, gq);
      f32x4 wacc[DPW][4];
#pragma unroll
      for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) wacc[dd][ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) uacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
          Eng::mma(wacc[dd][ti], ka[dd][kb], th[p]);
          if constexpr (Eng::kSplit) Eng::mma(wacc[dd][ti], ka[dd][kb], tl[p]);
        }
        Eng::mma(uacc[ti], th[p], kb ? vb1 : vb0);
        if constexpr (Eng::kSplit) Eng::mma(uacc[ti], tl[p], kb ? vb1 : vb0);
      }
      // wacc[dd][ti][i] = W^T[16di + 4gq + i][16ti + ln] = W[16ti + ln][16di + 4gq + i]
#pragma unroll
      for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
          Eng::store4(sW + (16 * ti + ln) * LDK + 16 * (DPW * w + dd) + 4 * gq, wacc[dd][ti][0],
                      wacc[dd][ti][1], wacc[dd][ti][2], wacc[dd][ti][3]);
    }
    __syncthreads();  // sP, sW complete

    // ---------------- a6 + a7 (inter part): U' = U - W S^T ; O^T = S Q^T ----------------
    // After a QDQ (bf16 engine) the state fragment holds the codes, exact in
    // bf16, and the products are scaled by s.
    const bool use_codes = Eng::kSplit && coded;
    f32x4 wacc[4], oacc[4];   // wacc: [tok][vcol] tiles ; oacc: O^T [vcol 16w+4gq+i][tok 16ti+ln]
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      wacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      oacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      Fr aw[4], bq[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        aw[ti] = Eng::load(sW + (16 * ti + ln) * LDK, kb, gq);
        bq[ti] = Eng::load(sQ + (16 * ti + ln) * LDK, kb, gq);
      }
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = st[2 * kb][i];
        sv[4 + i] = st[2 * kb + 1][i];
      }
      Fr sh, sl;
      if (use_codes) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] *= inv_s;
        sh = Eng::round(sv);
      } else {
        Eng::split(sv, sh, sl);
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        Eng::mma(wacc[ti], aw[ti], sh);   // W S^T     : A = W rows, B = state
        Eng::mma(oacc[ti], sh, bq[ti]);   // (S Q^T)   : A = state,  B = Q rows
      }
      if constexpr (Eng::kSplit) {
        if (!use_codes) {
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            Eng::mma(wacc[ti], aw[ti], sl);
            Eng::mma(oacc[ti], sl, bq[ti]);
          }
        }
      }
    }
    const float sc = use_codes ? s_cur : 1.0f;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const float egt = sc * sEg[16 * ti + ln];   // column tok = 16ti + ln of O^T
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uacc[ti][i] = fmaf(-sc, wacc[ti][i], uacc[ti][i]);
        oacc[ti][i] *= egt;
      }
    }

    // ---------------- a7 (intra part): O^T += U'^T P^T ----------------
    {
      Fr uh[2], ul[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float uv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uv[i] = uacc[2 * kb][i];
          uv[4 + i] = uacc[2 * kb + 1][i];
        }
        Eng::split(uv, uh[kb], ul[kb]);
      }
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
        const Fr ph = Eng::load(sPh + (16 * ti + ln) * L64, kb, gq);
        Eng::mma(oacc[ti], uh[kb], ph);
        if constexpr (Eng::kSplit) {
          const Fr pl = Eng::load(sPl + (16 * ti + ln) * L64, kb, gq);
          Eng::mma(oacc[ti], ul[kb], ph);
          Eng::mma(oacc[ti], uh[kb], pl);
        }
      }
    }
    // o rows: lane holds o[tok = 16ti + ln][16w + 4gq .. +3] of this tile
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int tok = 16 * ti + ln;
      if (tok < nv) {
        TO* dst = go_ + (int64_t)(t0 + tok) * v_row + (int64_t)h * dv + kTileRows * vt + 16 * w + 4 * gq;
        if constexpr (sizeof(TO) == 2) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(oacc[ti][0], oacc[ti][1]),
                                                      pack_bf16x2(oacc[ti][2], oacc[ti][3]));
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(oacc[ti][0], oacc[ti][1], oacc[ti][2], oacc[ti][3]);
        }
      }
    }

    // ---------------- a8: S^T <- e^gC S^T + K^T diag(e^(gC - gamma)) U' ----------------
    {
      Fr bh[2], bl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 e0 = *reinterpret_cast<const float4*>(sEgc + 32 * kb + 4 * gq);
        const float4 e1 = *reinterpret_cast<const float4*>(sEgc + 32 * kb + 16 + 4 * gq);
        const float uv[8] = {e0.x * uacc[2 * kb][0], e0.y * uacc[2 * kb][1], e0.z * uacc[2 * kb][2],
                             e0.w * uacc[2 * kb][3], e1.x * uacc[2 * kb + 1][0],
                             e1.y * uacc[2 * kb + 1][1], e1.z * uacc[2 * kb + 1][2],
                             e1.w * uacc[2 * kb + 1][3]};
        Eng::split(uv, bh[kb], bl[kb]);
      }
      const float aC = sRed[4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[t][i] *= aC;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const Fr a0 = Eng::load(sKT + (16 * t + ln) * L64, 0, gq);
        const Fr a1 = Eng::load(sKT + (16 * t + ln) * L64, 1, gq);
        Eng::mma(st[t], a0, bh[0]);
        Eng::mma(st[t], a1, bh[1]);
        if constexpr (Eng::kSplit) {
          Eng::mma(st[t], a0, bl[0]);
          Eng::mma(st[t], a1, bl[1]);
        }
      }
    }

    // ---------------- a9: boundary QDQ ----------------
    const bool last = (c == n_chunks - 1);
    const bool do_qdq = (flags & GDN_QDQ_CHUNK) || ((flags & GDN_QDQ_WRITE) && last);
    const int bidx = bound0 + c;
    if (args.bound_pre) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<float4*>(args.bound_pre + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                   16 * t + 4 * gq) = make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    }
    float s_new = 1.0f;
    if (do_qdq) {
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(st[t][i]));
      amax = block_max(amax, sRed);  // also orders this chunk's LDS reads before the next chunk's writes
      s_new = qdq_scale(amax);
      const float r = 1.0f / s_new;
#pragma unroll
      for (int t = 0; t < NT; ++t) qdq4(st[t], s_new, r);
      coded = true;
      s_cur = s_new;
      inv_s = r;
    } else {
      coded = false;
      __syncthreads();
    }
    if (args.bound_post) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<float4*>(args.bound_post + ((int64_t)bidx * H * dv + (int64_t)h * dv + vcol0) * DK +
                                   16 * t + 4 * gq) = make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    }
    if (args.bound_scales && tid == 0) args.bound_scales[((int64_t)bidx * H + h) * tiles + vt] = s_new;
  }

  // ---------------- a10: recurrent suffix, tokens P < t <= L ----------------
  if (P < L) {
    float* sq = reinterpret_cast<float*>(smem + S_::oW);  // q_t, k_t: DK each; v_t: 64
    float* sk = sq + 256;
    float* sv = sq + 512;
    float* sg = sq + 640;    // g_t at sg[0], beta_t at sg[DK]
    for (int t = P; t < L; ++t) {
      const int64_t row = seg0 + t;
      if (tid < DK) {
        sq[tid] = io<TIO>::ld(gq_ + row * qk_row + (int64_t)h * DK + tid);
        sk[tid] = io<TIO>::ld(gk_ + row * qk_row + (int64_t)h * DK + tid);
      }
      if (tid < 64) sv[tid] = io<TIO>::ld(gv_ + row * v_row + (int64_t)h * dv + kTileRows * vt + tid);
      if (tid == 0) {
        sg[0] = args.g[row * H + h];
        sg[DK] = args.beta[row * H + h];
      }
      __syncthreads();
      const float a = expf(sg[0]);
      const float b = sg[DK];
      float y = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          st[t2][i] *= a;
          y += st[t2][i] * sk[16 * t2 + 4 * gq + i];
        }
      y += __shfl_xor(y, 16, 64);
      y += __shfl_xor(y, 32, 64);
      const float u = b * (sv[16 * w + ln] - y);
      float z = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          st[t2][i] += u * sk[16 * t2 + 4 * gq + i];
          z += st[t2][i] * sq[16 * t2 + 4 * gq + i];
        }
      z += __shfl_xor(z, 16, 64);
      z += __shfl_xor(z, 32, 64);
      if (gq == 0) io<TO>::st(go_ + row * v_row + (int64_t)h * dv + vcol0, z);
      if (flags & GDN_QDQ_WRITE) {
        float amax = 0.f;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(st[t2][i]));
        amax = block_max(amax, sRed);
        const float s = qdq_scale(amax);
        const float r = 1.0f / s;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2) qdq4(st[t2], s, r);
      } else {
        __syncthreads();
      }
    }
  }

  // ---------------- a11: final state, zero padding rows of o ----------------
#pragma unroll
  for (int t = 0; t < NT; ++t)
    *reinterpret_cast<float4*>(args.fin + state_base + 16 * t + 4 * gq) =
        make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
  for (int r = L + (tid >> 6); r < seg1 - seg0; r += 4)
    io<TO>::st(go_ + (int64_t)(seg0 + r) * v_row + (int64_t)h * dv + kTileRows * vt + lane, 0.f);
}

template <int DK, class Eng, typename TIO, typename TO>
static hipError_t launch_typed(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  auto kern = chunk_fwd_kernel<DK, Eng, TIO, TO>;
  constexpr size_t lds = Smem<DK, Eng>::bytes;
  static bool attr_set = false;  // the attribute is per function; setting it twice is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                            const float* beta, const float* g, const int32_t* cu_seqlens,
                            const int32_t* seq_lens, const int32_t* prefix_lens,
                            const float* initial_state, void* o, float* final_state,
                            void* workspace, const gdn_debug_t* debug, hipStream_t stream) {
  if (s.gate_per_channel) return hipErrorNotSupported;
  ChunkArgs a;
  const int32_t* offs = nullptr;
  void* T = nullptr;
  hipError_t e = launch_prep(s, k, beta, g, cu_seqlens, seq_lens, prefix_lens, workspace, &offs, &T, stream);
  if (e != hipSuccess) return e;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
  a.cu_seqlens = cu_seqlens; a.seq_lens = seq_lens; a.prefix_lens = prefix_lens;
  a.chunk_offs = offs; a.T = T;
  a.init = initial_state; a.o = o; a.fin = final_state;
  a.bound_offsets = debug ? debug->bound_offsets : nullptr;
  a.bound_pre = debug ? debug->bound_pre : nullptr;
  a.bound_post = debug ? debug->bound_post : nullptr;
  a.bound_scales = debug ? debug->scales : nullptr;
  a.H = s.n_heads; a.dv = s.dv; a.flags = s.qdq_flags;
  const bool ob = s.o_dtype == GDN_BF16;
  if (debug && debug->kernel_start) {
    e = hipEventRecord((hipEvent_t)debug->kernel_start, stream);
    if (e != hipSuccess) return e;
  }
  if (s.io_dtype == GDN_BF16) {
    if (s.dk == 128)
      e = ob ? launch_typed<128, EngBF16, uint16_t, uint16_t>(s, a, stream)
             : launch_typed<128, EngBF16, uint16_t, float>(s, a, stream);
    else
      e = ob ? launch_typed<64, EngBF16, uint16_t, uint16_t>(s, a, stream)
             : launch_typed<64, EngBF16, uint16_t, float>(s, a, stream);
  } else if (s.dk == 64) {
    e = ob ? launch_typed<64, EngF32, float, uint16_t>(s, a, stream)
           : launch_typed<64, EngF32, float, float>(s, a, stream);
  } else {
    return hipErrorNotSupported;
  }
  if (e == hipSuccess && debug && debug->kernel_end)
    e = hipEventRecord((hipEvent_t)debug->kernel_end, stream);
  return e;
}

}  // namespace gdn
