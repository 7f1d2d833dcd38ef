// gdn_chunk.hip -- fused chunked gated delta rule forward with per-boundary
// FP8-E4M3 state QDQ (Model-Optimizer #2497 "What does this PR do?": 64-token
// chunks, WY-transformed W, dynamic per-tile state QDQ at every boundary;
// #2506: exact triangular solve).
//
// Work unit: one workgroup (4 waves) per (sequence n, head h, 64-column value
// tile vt).  It walks its sequence chunk by chunk and keeps its slice of the
// state, S^T (dk x 64), in registers for the whole sequence: wave w owns value
// columns 16w..16w+15 of the tile, i.e. dk/16 accumulator tiles.  The 64 x dk
// state tile is exactly one QDQ tile, so the QDQ amax needs no exchange with
// other workgroups.
//
// Per chunk of n <= 64 tokens (rows past n are zero-filled, beta = g = 0, so
// they drop out of every product), with gamma = in-chunk cumulative log-gate:
//   a1  stage q, k (row-major and transposed), v (transposed), beta, g -> LDS
//   a2  gamma, exp(gamma), exp(gamma_C - gamma)            (wave 0, scan)
//   a3  A[r][s] = beta_r exp(gamma_r - gamma_s) k_r.k_s   (s < r)      MFMA
//       P[r][s] = exp(gamma_r - gamma_s) q_r.k_s          (s <= r)     MFMA
//   a4  X = (I + A)^-1 by blocked forward substitution in fp32 (16 x 16
//       diagonal blocks, then off-diagonal blocks level by level);
//       T = X diag(beta), T' = T diag(exp(gamma))
//   a5  W = T' K  (computed as W^T = K^T T'^T so it lands row-major in LDS),
//       U = T V                                                        MFMA
//   a6  U' = U - W S^T                                                 MFMA
//   a7  O  = diag(exp(gamma)) Q S^T + P U'                             MFMA
//   a8  S^T <- exp(gamma_C) S^T + K^T diag(exp(gamma_C - gamma)) U'    MFMA
//   a9  QDQ: amax over the 64 x dk tile (wave + LDS tree), s = amax/448,
//       S <- RNE_E4M3(S/s) s
// then the recurrent suffix (tokens P_n < t <= L_n, QDQ after every write)
// and the final state store.
//
// Precision (bf16 inputs, fp32 accumulate): q, k, v enter the MFMAs exactly.
// T, T', P and U' are fed as hi + lo bf16 pairs (their rounding would cost
// about 1.6e-3 relative each in o); W enters as one bf16.  After a QDQ the
// state is code * s with the code exactly representable in bf16, so S^T is
// fed as the codes and the product is scaled by s afterwards; otherwise
// (QDQ off, supplied initial state) S^T is fed as a hi + lo pair.  fp32 inputs
// use the fp32 MFMA throughout.
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
    const uint4 u = make_uint4(a.x, a.y, b.x, b.y);
    return __builtin_bit_cast(Fr, u);
  }
  static __device__ __forceinline__ void mma(f32x4& c, const Fr& a, const Fr& b) { mma_bf16(c, a, b); }
  static __device__ __forceinline__ Fr round(const float (&x)[8]) {
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = float_to_bf16_bits(x[j]);
    return __builtin_bit_cast(Fr, h);
  }
  static __device__ __forceinline__ void split(const float (&x)[8], Fr& hi, Fr& lo) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[j] = float_to_bf16_bits(x[j]);
      l[j] = float_to_bf16_bits(x[j] - bf16_bits_to_float(h[j]));
    }
    hi = __builtin_bit_cast(Fr, h);
    lo = __builtin_bit_cast(Fr, l);
  }
  static __device__ __forceinline__ E cvt(float x) { return float_to_bf16_bits(x); }
  static __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d) {
    uint2 u;
    u.x = (uint32_t)float_to_bf16_bits(a) | ((uint32_t)float_to_bf16_bits(b) << 16);
    u.y = (uint32_t)float_to_bf16_bits(c) | ((uint32_t)float_to_bf16_bits(d) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
  // hi and lo parts of four consecutive values
  static __device__ __forceinline__ void store4_split(E* ph, E* pl, const float (&x)[4]) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = float_to_bf16_bits(x[j]);
      l[j] = float_to_bf16_bits(x[j] - bf16_bits_to_float(h[j]));
    }
    *reinterpret_cast<uint2*>(ph) = __builtin_bit_cast(uint2, h);
    *reinterpret_cast<uint2*>(pl) = __builtin_bit_cast(uint2, l);
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
  static __device__ __forceinline__ E cvt(float x) { return x; }
  static __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
  static __device__ __forceinline__ void store4_split(E* ph, E* pl, const float (&x)[4]) {
    (void)pl;
    *reinterpret_cast<float4*>(ph) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

// LDS layout of the chunk kernel (bytes).  Row strides are padded so that
// the 16 rows read by one fragment load fall in different banks; [64][dk]
// rows stay 16-byte aligned for the staging stores.
template <int DK, class Eng>
struct Smem {
  using E = typename Eng::E;
  static constexpr int LDK = DK + 16 / (int)sizeof(E);  // stride of [64][DK] buffers (E), 16-byte rows
  static constexpr int L64 = 64 + 4;                     // stride of [*][64] buffers (E or fp32)
  static constexpr int kSplitN = Eng::kSplit ? 2 : 1;
  static constexpr size_t szK = 64 * LDK * sizeof(E);
  static constexpr size_t szKT = DK * L64 * sizeof(E);
  static constexpr size_t szVT = 64 * L64 * sizeof(E);
  static constexpr size_t szF = 64 * L64 * sizeof(float);
  static constexpr size_t szXW = (szF > szK) ? szF : szK;
  static constexpr size_t szM = 64 * L64 * sizeof(E);  // one 64x64 operand matrix
  static constexpr size_t oK = 0;
  static constexpr size_t oKT = oK + szK;
  static constexpr size_t oQ = oKT + szKT;
  static constexpr size_t oVT = oQ + szK;
  static constexpr size_t oA = oVT + szVT;
  static constexpr size_t oXW = oA + szF;               // X (fp32, solve) aliased with W (E)
  static constexpr size_t oT = oXW + szXW;              // T hi [, T lo]
  static constexpr size_t oTg = oT + kSplitN * szM;     // T' hi [, lo]
  static constexpr size_t oP = oTg + kSplitN * szM;     // P hi [, lo]
  static constexpr size_t oVec = oP + kSplitN * szM;    // gamma, e^gamma, e^(gC-gamma), beta
  static constexpr size_t oRed = oVec + 4 * 64 * sizeof(float);
  static constexpr size_t bytes = oRed + 16 * sizeof(float);
  // solve scratch (3 x 16 x 16 fp32) lives in the T area before T is written
  static constexpr size_t oR = oT;
  static_assert(3 * 256 * sizeof(float) <= kSplitN * szM, "solve scratch does not fit");
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
  float* sA = reinterpret_cast<float*>(smem + S_::oA);
  float* sX = reinterpret_cast<float*>(smem + S_::oXW);
  E* sW = reinterpret_cast<E*>(smem + S_::oXW);
  E* sTh = reinterpret_cast<E*>(smem + S_::oT);
  E* sTl = sTh + 64 * L64;
  E* sTgh = reinterpret_cast<E*>(smem + S_::oTg);
  E* sTgl = sTgh + 64 * L64;
  E* sPh = reinterpret_cast<E*>(smem + S_::oP);
  E* sPl = sPh + 64 * L64;
  float* sGam = reinterpret_cast<float*>(smem + S_::oVec);
  float* sEg = sGam + 64;
  float* sEgc = sEg + 64;
  float* sBeta = sEgc + 64;
  float* sRed = reinterpret_cast<float*>(smem + S_::oRed);
  float* sR = reinterpret_cast<float*>(smem + S_::oR);

  const int tid = threadIdx.x;
  const int w = tid >> 6;        // wave
  const int lane = tid & 63;
  const int gq = lane >> 4;      // lane group (k-slots / accumulator rows 4gq..4gq+3)
  const int ln = lane & 15;      // accumulator column / fragment row

  const int H = args.H, dv = args.dv;
  const int tiles = dv / kTileRows;
  const int vt = blockIdx.x % tiles;
  const int nh = blockIdx.x / tiles;
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

  for (int c = 0; c < n_chunks; ++c) {
    const int t0 = seg0 + c * kChunk;
    const int nv = min(kChunk, P - c * kChunk);  // valid tokens in this chunk

    // ---------------- a1: stage the chunk ----------------
    {
      constexpr int EPS = 16 / sizeof(TIO);           // elements per 16-byte segment
      constexpr int SPR = DK / EPS;                   // segments per q/k row
      constexpr int NSEG = 64 * SPR / kThreads;       // per thread
#pragma unroll
      for (int j = 0; j < NSEG; ++j) {
        const int seg = tid + kThreads * j;
        const int r = seg / SPR, c0 = (seg % SPR) * EPS;
        uint4 kraw = make_uint4(0u, 0u, 0u, 0u), qraw = make_uint4(0u, 0u, 0u, 0u);
        if (r < nv) {
          const int64_t off = (int64_t)(t0 + r) * qk_row + (int64_t)h * DK + c0;
          kraw = *reinterpret_cast<const uint4*>(gk_ + off);
          qraw = *reinterpret_cast<const uint4*>(gq_ + off);
        }
        // row-major copies (LDS element type == I/O element type here)
        *reinterpret_cast<uint4*>(sK + r * LDK + c0) = kraw;
        *reinterpret_cast<uint4*>(sQ + r * LDK + c0) = qraw;
        TIO kv[EPS];
        __builtin_memcpy(kv, &kraw, 16);
#pragma unroll
        for (int e = 0; e < EPS; ++e) sKT[(c0 + e) * L64 + r] = kv[e];
      }
      constexpr int VSPR = 64 / EPS;
      constexpr int VNSEG = 64 * VSPR / kThreads;
#pragma unroll
      for (int j = 0; j < VNSEG; ++j) {
        const int seg = tid + kThreads * j;
        const int r = seg / VSPR, c0 = (seg % VSPR) * EPS;
        uint4 vraw = make_uint4(0u, 0u, 0u, 0u);
        if (r < nv) {
          const int64_t off = (int64_t)(t0 + r) * v_row + (int64_t)h * dv + kTileRows * vt + c0;
          vraw = *reinterpret_cast<const uint4*>(gv_ + off);
        }
        TIO vv[EPS];
        __builtin_memcpy(vv, &vraw, 16);
#pragma unroll
        for (int e = 0; e < EPS; ++e) sVT[(c0 + e) * L64 + r] = vv[e];
      }
      // ---------------- a2: gates (wave 0, lane = token) ----------------
      if (w == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < nv) {
          gv = args.g[(int64_t)(t0 + lane) * H + h];
          bv = args.beta[(int64_t)(t0 + lane) * H + h];
        }
        float x = gv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        const float gC = __shfl(x, 63, 64);
        sGam[lane] = x;
        sEg[lane] = expf(x);
        sEgc[lane] = expf(gC - x);
        sBeta[lane] = bv;
        if (lane == 0) sRed[4] = expf(gC);
      }
    }
    __syncthreads();

    // ---------------- a3: A (strict lower) and P (lower incl. diagonal) ----------------
    // Job list: 10 lower tiles of A, 10 lower tiles of P, 2 zero tiles of P.
    for (int job = w; job < 22; job += 4) {
      int si, ri, kind;  // kind 0: A, 1: P, 2: P zero tile
      if (job < 20) {
        const int jj = job % 10;
        kind = job / 10;
        ri = (jj < 1) ? 0 : (jj < 3) ? 1 : (jj < 6) ? 2 : 3;
        si = jj - (ri * (ri + 1)) / 2;
      } else {
        kind = 2;
        si = (job == 20) ? 1 : 3;
        ri = si - 1;
      }
      if (kind == 2) {
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        Eng::store4_split(sPh + (16 * ri + ln) * L64 + 16 * si + 4 * gq,
                          sPl + (16 * ri + ln) * L64 + 16 * si + 4 * gq, z);
        continue;
      }
      // C[s][r] = sum_d K[s][d] * (K or Q)[r][d]
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const E* arow = sK + (16 * si + ln) * LDK;
      const E* brow = (kind == 0 ? sK : sQ) + (16 * ri + ln) * LDK;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) Eng::mma(acc, Eng::load(arow, kb, gq), Eng::load(brow, kb, gq));
      const int r = 16 * ri + ln;
      const float gr = sGam[r];
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * si + 4 * gq + i;
        const bool keep = (kind == 0) ? (s < r) : (s <= r);
        x[i] = keep ? expf(gr - sGam[s]) * acc[i] : 0.f;
      }
      if (kind == 0) {
        const float br = sBeta[r];
        *reinterpret_cast<float4*>(sA + r * L64 + 16 * si + 4 * gq) =
            make_float4(br * x[0], br * x[1], br * x[2], br * x[3]);
      } else {
        Eng::store4_split(sPh + r * L64 + 16 * si + 4 * gq, sPl + r * L64 + 16 * si + 4 * gq, x);
      }
    }
    __syncthreads();

    // ---------------- a4: X = (I + A)^-1, blocked, fp32 ----------------
    if (w == 0) {
      // diagonal blocks: lane = (block bi, column cc); forward substitution down the column
      const int bi = lane >> 4, cc = lane & 15;
      float xcol[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == cc) ? 1.f : 0.f;
        const float* arow = sA + (16 * bi + r) * L64 + 16 * bi;
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= arow[s] * xcol[s];
        xcol[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sX[(16 * bi + r) * L64 + 16 * bi + cc] = xcol[r];
    }
    __syncthreads();
    {
      const int r = tid >> 4, cc = tid & 15;
#pragma unroll
      for (int d = 1; d < 4; ++d) {
        // R_ij = sum_{k=j}^{i-1} A_ik X_kj  for blocks (i, j) = (d + b, b)
#pragma unroll
        for (int b = 0; b + d < 4; ++b) {
          const int i = d + b, j = b;
          float acc = 0.f;
          for (int kk = j; kk < i; ++kk) {
            const float* arow = sA + (16 * i + r) * L64 + 16 * kk;
            const float* xcol = sX + (16 * kk) * L64 + 16 * j + cc;
#pragma unroll
            for (int s = 0; s < 16; ++s) acc += arow[s] * xcol[s * L64];
          }
          sR[b * 256 + r * 16 + cc] = acc;
        }
        __syncthreads();
        // X_ij = -X_ii R_ij
#pragma unroll
        for (int b = 0; b + d < 4; ++b) {
          const int i = d + b, j = b;
          const float* xrow = sX + (16 * i + r) * L64 + 16 * i;
          float acc = 0.f;
#pragma unroll
          for (int s = 0; s < 16; ++s) acc += xrow[s] * sR[b * 256 + s * 16 + cc];
          sX[(16 * i + r) * L64 + 16 * j + cc] = -acc;
        }
        __syncthreads();
      }
    }
    // T = X diag(beta), T' = T diag(e^gamma); zero above the block diagonal.
    {
      const int r = tid >> 2, q4 = (tid & 3) * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s0 = q4 + 4 * u;
        float tv[4], tg[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = s0 + e;
          const float xv = ((s >> 4) <= (r >> 4)) ? sX[r * L64 + s] : 0.f;
          tv[e] = xv * sBeta[s];
          tg[e] = tv[e] * sEg[s];
        }
        Eng::store4_split(sTh + r * L64 + s0, sTl + r * L64 + s0, tv);
        Eng::store4_split(sTgh + r * L64 + s0, sTgl + r * L64 + s0, tg);
      }
    }
    __syncthreads();

    // ---------------- a5: W^T = K^T T'^T (-> sW row-major), U = T V ----------------
    {
      constexpr int DPW = NT / 4;  // dk tiles of W^T per wave
#pragma unroll
      for (int dd = 0; dd < DPW; ++dd) {
        const int di = DPW * w + dd;
        const E* arow = sKT + (16 * di + ln) * L64;
        Fr a0 = Eng::load(arow, 0, gq);
        Fr a1 = Eng::load(arow, 1, gq);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const E* bh = sTgh + (16 * ti + ln) * L64;
          Eng::mma(acc, a0, Eng::load(bh, 0, gq));
          if constexpr (Eng::kSplit) Eng::mma(acc, a0, Eng::load(sTgl + (16 * ti + ln) * L64, 0, gq));
          if (ti >= 2) {
            Eng::mma(acc, a1, Eng::load(bh, 1, gq));
            if constexpr (Eng::kSplit) Eng::mma(acc, a1, Eng::load(sTgl + (16 * ti + ln) * L64, 1, gq));
          }
          // acc[i] = W^T[16di + 4gq + i][16ti + ln] = W[16ti + ln][16di + 4gq + i]
          Eng::store4(sW + (16 * ti + ln) * LDK + 16 * di + 4 * gq, acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    f32x4 uacc[4];
    {
      const E* brow = sVT + (16 * w + ln) * L64;
      const Fr b0 = Eng::load(brow, 0, gq);
      const Fr b1 = Eng::load(brow, 1, gq);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        uacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
        Eng::mma(uacc[ti], Eng::load(sTh + (16 * ti + ln) * L64, 0, gq), b0);
        if constexpr (Eng::kSplit) Eng::mma(uacc[ti], Eng::load(sTl + (16 * ti + ln) * L64, 0, gq), b0);
        if (ti >= 2) {
          Eng::mma(uacc[ti], Eng::load(sTh + (16 * ti + ln) * L64, 1, gq), b1);
          if constexpr (Eng::kSplit) Eng::mma(uacc[ti], Eng::load(sTl + (16 * ti + ln) * L64, 1, gq), b1);
        }
      }
    }
    __syncthreads();  // sW complete

    // ---------------- a6 + a7 (inter-chunk part): W S^T and Q S^T ----------------
    // After a QDQ (bf16 engine) feed the codes, exact in bf16, and scale by s.
    const bool use_codes = Eng::kSplit && coded;
    f32x4 wacc[4], oacc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      wacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      oacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = st[2 * kb][i];
        sv[4 + i] = st[2 * kb + 1][i];
      }
      Fr bh, bl;
      if (use_codes) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] *= inv_s;  // the codes, exact in bf16
        bh = Eng::round(sv);
      } else {
        Eng::split(sv, bh, bl);
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const Fr aw = Eng::load(sW + (16 * ti + ln) * LDK, kb, gq);
        const Fr aq = Eng::load(sQ + (16 * ti + ln) * LDK, kb, gq);
        Eng::mma(wacc[ti], aw, bh);
        Eng::mma(oacc[ti], aq, bh);
        if constexpr (Eng::kSplit) {
          if (!use_codes) {
            Eng::mma(wacc[ti], aw, bl);
            Eng::mma(oacc[ti], aq, bl);
          }
        }
      }
    }
    const float sc = use_codes ? s_cur : 1.0f;
    // U' = U - W S^T (fp32), rows 16ti + 4gq + i, column vcol
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uacc[ti][i] = uacc[ti][i] - sc * wacc[ti][i];
        oacc[ti][i] = sEg[16 * ti + 4 * gq + i] * (sc * oacc[ti][i]);
      }

    // ---------------- a7 (intra-chunk part): O += P U' ----------------
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float uv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uv[i] = uacc[2 * kb][i];
        uv[4 + i] = uacc[2 * kb + 1][i];
      }
      Fr bh, bl;
      Eng::split(uv, bh, bl);
#pragma unroll
      for (int ti = 2 * kb; ti < 4; ++ti) {
        const Fr ah = Eng::load(sPh + (16 * ti + ln) * L64, kb, gq);
        Eng::mma(oacc[ti], ah, bh);
        if constexpr (Eng::kSplit) {
          const Fr al = Eng::load(sPl + (16 * ti + ln) * L64, kb, gq);
          Eng::mma(oacc[ti], ah, bl);
          Eng::mma(oacc[ti], al, bh);
        }
      }
    }
    // store o rows (valid tokens only)
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ti + 4 * gq + i;
        if (r < nv) io<TO>::st(go_ + (int64_t)(t0 + r) * v_row + (int64_t)h * dv + vcol0, oacc[ti][i]);
      }

    // ---------------- a8: S^T <- e^gC S^T + K^T diag(e^(gC - gamma)) U' ----------------
    {
      const float aC = sRed[4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[t][i] *= aC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float uv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uv[i] = sEgc[32 * kb + 4 * gq + i] * uacc[2 * kb][i];
          uv[4 + i] = sEgc[32 * kb + 16 + 4 * gq + i] * uacc[2 * kb + 1][i];
        }
        Fr bh, bl;
        Eng::split(uv, bh, bl);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const Fr a = Eng::load(sKT + (16 * t + ln) * L64, kb, gq);
          Eng::mma(st[t], a, bh);
          if constexpr (Eng::kSplit) Eng::mma(st[t], a, bl);
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
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[t][i] = qdq_value(st[t][i], s_new);
      coded = true;
      s_cur = s_new;
      inv_s = 1.0f / s_new;
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
    float* sq = sA;          // q_t, k_t: DK each; v_t: 64
    float* sk = sA + 256;
    float* sv = sA + 512;
    float* sg = sA + 640;    // g_t (scalar) / DK values; beta at sg[DK]
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
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[t2][i] = qdq_value(st[t2][i], s);
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
  static bool attr_set = false;  // per process; the attribute is per function
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
                            const gdn_debug_t* debug, hipStream_t stream) {
  if (s.gate_per_channel) return hipErrorNotSupported;
  ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
  a.cu_seqlens = cu_seqlens; a.seq_lens = seq_lens; a.prefix_lens = prefix_lens;
  a.init = initial_state; a.o = o; a.fin = final_state;
  a.bound_offsets = debug ? debug->bound_offsets : nullptr;
  a.bound_pre = debug ? debug->bound_pre : nullptr;
  a.bound_post = debug ? debug->bound_post : nullptr;
  a.bound_scales = debug ? debug->scales : nullptr;
  a.H = s.n_heads; a.dv = s.dv; a.flags = s.qdq_flags;
  const bool ob = s.o_dtype == GDN_BF16;
  if (s.io_dtype == GDN_BF16) {
    if (s.dk == 128)
      return ob ? launch_typed<128, EngBF16, uint16_t, uint16_t>(s, a, stream)
                : launch_typed<128, EngBF16, uint16_t, float>(s, a, stream);
    return ob ? launch_typed<64, EngBF16, uint16_t, uint16_t>(s, a, stream)
              : launch_typed<64, EngBF16, uint16_t, float>(s, a, stream);
  }
  if (s.dk == 64)
    return ob ? launch_typed<64, EngF32, float, uint16_t>(s, a, stream)
              : launch_typed<64, EngF32, float, float>(s, a, stream);
  return hipErrorNotSupported;
}

}  // namespace gdn
