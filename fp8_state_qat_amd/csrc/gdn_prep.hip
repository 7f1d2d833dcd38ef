// gdn_prep.hip -- the state-independent part of the chunked gated delta rule
// (Model-Optimizer #2497: 64-token chunks with WY/UT-transformed W and U;
// #2506: the exact triangular solve), for every (chunk, head) in parallel.
//
// Per chunk of n <= 64 tokens of sequence n, head h (rows past n are zero):
//     gamma_r = sum_{s<=r} g_s                                (in-chunk scan)
//     A[r][s] = beta_r exp(gamma_r - gamma_s) k_r . k_s       (s < r)
//     T       = (I + A)^-1 diag(beta)                         (exact solve)
//     P[t][s] = exp(gamma_t - gamma_s) q_t . k_s              (s <= t)
// T and P are written to the workspace for the sequential kernel, which forms
// U' = T (V - exp(gamma) * K S^T) and O = exp(gamma) * Q S^T + P U' from them.
//
// The solve is blocked on 16 x 16 blocks in fp32: the four diagonal blocks
// by forward substitution (one lane per column), then the off-diagonal
// blocks level by level, X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj, on the fp32
// MFMA.
//
// Workspace layout: int32 chunk offsets [N + 1] (prefix sums of
// ceil(P_n / 64)), padded to 256 bytes, then one 12 KiB T record per (chunk,
// head), then one P record per (chunk, head) of the same layout.  A record
// holds the six nonzero 16 x 32 fragments of a block lower-triangular 64 x 64
// matrix M, pair p = (ti, kb) in (0,0) (1,0) (2,0) (3,0) (2,1) (3,1): lane l
// of fragment p holds M[16 ti + l % 16][32 kb + kperm(l / 16, j)] for
// j = 0..7 (kperm as in gdn_device.hpp), fragments stored one after the
// other, lane-major.  bf16 inputs store hi = bf16(M) (six fragments) then
// lo = bf16(M - hi) (six more); fp32 inputs store M in fp32.  The sequential
// kernels copy a record into LDS unchanged and read each fragment with one
// lane-linear load (T as the A operand of T X, P as the B operand of
// U'^T P^T).
#include "gdn_chunk_common.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// chunk offsets: offs[n] = sum_{m < n} ceil(P_m / 64), one workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void chunk_offsets_kernel(const int32_t* __restrict__ cu,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 const int32_t* __restrict__ prefix_lens,
                                                                 int N, int32_t* __restrict__ offs) {
  __shared__ int32_t part[kThreads];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += kThreads) {
    const int n = base + threadIdx.x;
    int32_t cnt = 0;
    if (n < N) {
      const int32_t L = seq_lens ? seq_lens[n] : (cu[n + 1] - cu[n]);
      const int32_t P = prefix_lens ? prefix_lens[n] : L;
      cnt = (P + kChunk - 1) / kChunk;
    }
    part[threadIdx.x] = cnt;
    __syncthreads();
    // inclusive Hillis-Steele scan over the tile
    for (int off = 1; off < kThreads; off <<= 1) {
      const int32_t v = (threadIdx.x >= off) ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    if (n < N) offs[n] = carry + part[threadIdx.x] - cnt;
    __syncthreads();
    if (threadIdx.x == kThreads - 1) carry += part[kThreads - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) offs[N] = carry;
}

struct PrepArgs {
  const void* q;  // per-key-channel gate only
  const void* k;
  const float* beta;
  const float* g;
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* prefix_lens;
  const int32_t* offs;
  void* T;        // one record of kTRecBytes per (chunk, head)
  void* P;        // per-key-channel gate: one P record per (chunk, head)
  int N;
  int H;
};

// Row stride (floats) of the 64 x 64 fp32 LDS matrices of the prep kernels.
constexpr int kL64 = 64 + 4;

// X = (I + A)^-1 for the strictly lower A in sA (only the block-lower 16 x 16
// blocks are read), 256 threads.  sX receives X row-major (block-lower part;
// the diagonal blocks carry zeros above their diagonal).  Contains barriers.
//   diagonal blocks: forward substitution, wave 0, one lane per (block, column)
//   X_ij (i > j), level by level (i - j = 1, 2, 3), one wave per block:
//       X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj
//   on the fp32 MFMA (16x16x4).  Instruction q of a 16-deep product takes
//   k = 4 (l / 16) + q from lane l, so the accumulator of the sum (lane l
//   holds rows 4 (l / 16) .. + 3 of column l % 16) is the B operand of the
//   product with X_ii as it stands.
__device__ __forceinline__ void solve_unit_lower(const float* sA, float* sX) {
  constexpr int L64 = kL64;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  if (w == 0) {
    const int bi = gq, cc = ln;
    const float* Ab = sA + 16 * bi * L64 + 16 * bi;
    float xc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int q4 = 0; q4 * 4 < r; ++q4) {
        const float4 a4 = *reinterpret_cast<const float4*>(Ab + r * L64 + 4 * q4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * q4 + i < r) acc = fmaf(-av[i], xc[4 * q4 + i], acc);
      }
      xc[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[(16 * bi + r) * L64 + 16 * bi + cc] = xc[r];
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w + d < 4) {
      const int i = w + d, j = w;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = j; kb < i; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float av = sA[(16 * i + ln) * L64 + 16 * kb + 4 * gq + q];
          const float bv = sX[(16 * kb + 4 * gq + q) * L64 + 16 * j + ln];
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, y, 0, 0, 0);
        }
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(sX[(16 * i + ln) * L64 + 16 * i + 4 * gq + q], y[q], x, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sX[(16 * i + 4 * gq + r) * L64 + 16 * j + ln] = -x[r];
    }
    __syncthreads();
  }
}

// Writes the block-lower part of the 64 x 64 matrix M (row-major, stride
// kL64, zeros above the diagonal of its diagonal blocks), times diag(colscale)
// when colscale is not null, as one record in MFMA fragment order (the record
// layout described at the top of this file), 256 threads.
template <bool kBF>
__device__ __forceinline__ void store_record(const float* M, const float* colscale, char* rec) {
  constexpr int L64 = kL64;
  const int tid = threadIdx.x;
  for (int slot = tid; slot < 6 * 64; slot += kThreads) {
    const int p = slot >> 6, l = slot & 63, g4 = l >> 4;
    const int ti = p < 4 ? p : p - 2, kb = p < 4 ? 0 : 1;
    const int r = 16 * ti + (l & 15);
    float t8[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int s0 = 32 * kb + 16 * half + 4 * g4;
      float4 x4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if ((s0 >> 4) <= ti) x4 = *reinterpret_cast<const float4*>(M + r * L64 + s0);
      const float4 b4 = colscale ? *reinterpret_cast<const float4*>(colscale + s0)
                                 : make_float4(1.f, 1.f, 1.f, 1.f);
      t8[4 * half] = x4.x * b4.x;
      t8[4 * half + 1] = x4.y * b4.y;
      t8[4 * half + 2] = x4.z * b4.z;
      t8[4 * half + 3] = x4.w * b4.w;
    }
    if constexpr (kBF) {
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split_bf16x2(t8[2 * q], t8[2 * q + 1], hv[q], lv[q]);
      uint4* dst = reinterpret_cast<uint4*>(rec);
      dst[p * 64 + l] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      dst[(6 + p) * 64 + l] = make_uint4(lv[0], lv[1], lv[2], lv[3]);
    } else {
      float4* dst = reinterpret_cast<float4*>(rec) + 2 * (p * 64 + l);
      dst[0] = make_float4(t8[0], t8[1], t8[2], t8[3]);
      dst[1] = make_float4(t8[4], t8[5], t8[6], t8[7]);
    }
  }
}

// One workgroup (4 waves) per (chunk, head).  TIO: uint16_t (bf16) or float.
template <int DK, typename TIO>
__global__ __launch_bounds__(kThreads, 3) void chunk_prep_kernel(PrepArgs a) {
  constexpr bool kBF = sizeof(TIO) == 2;
  constexpr int L64 = kL64;
  constexpr int NKB = DK / 32;
  // k and q rows unpadded, 16-byte pieces XOR-swizzled by row (piece p of row r
  // at slot p ^ (r % PPR)), so that direct loads fill them 1 KiB at a time and
  // the fragment reads of 16 rows at one column hit different banks
  constexpr int RB = DK * (int)sizeof(TIO);  // bytes per row
  constexpr int PPR = RB / 16;               // pieces per row
  constexpr int KQ = 2 * 64 * RB;
  constexpr int KX = (KQ > 64 * L64 * 4) ? KQ : 64 * L64 * 4;
  __shared__ __align__(16) char sKX[KX];  // k, q, then (once A and P are formed) the solve's X
  __shared__ __align__(16) float sA[64 * L64];
  __shared__ float sG2[64], sBeta[64];
  const char* sK = sKX;
  const char* sQ = sKX + 64 * RB;
  float* sX = reinterpret_cast<float*>(sKX);
  // byte address of element c of row r in the k or q block
  auto kq_at = [](int r, int c) {
    const int p = c * (int)sizeof(TIO) / 16, within = c * (int)sizeof(TIO) % 16;
    return r * RB + ((p ^ (r & (PPR - 1))) * 16) + within;
  };

  const int H = a.H;
  const int j = blockIdx.x / H, h = blockIdx.x % H;
  const int total = a.offs[a.N];
  if (j >= total) return;  // grid is sized for the worst case
  // sequence of chunk j: last n with offs[n] <= j
  int lo = 0, hi = a.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.offs[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int n = lo, c = j - a.offs[n];
  const int seg0 = a.cu_seqlens[n];
  const int L = a.seq_lens ? a.seq_lens[n] : (a.cu_seqlens[n + 1] - seg0);
  const int P = a.prefix_lens ? a.prefix_lens[n] : L;
  const int t0 = seg0 + c * kChunk;
  const int nv = min(kChunk, P - c * kChunk);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;

  // ---- stage K and Q by direct loads (rows past nv repeat the last valid row:
  // beta is zero there, which zeroes those rows of A and columns of T, and P
  // rows past nv only reach outputs that are not stored), gates
  {
    const uint32_t lds0 = lds_base_u32(sKX);
    const TIO* gk = reinterpret_cast<const TIO*>(a.k) + ((int64_t)t0 * H + h) * DK;
    const TIO* gqv = reinterpret_cast<const TIO*>(a.q) + ((int64_t)t0 * H + h) * DK;
    constexpr int NI = 64 * RB / 1024;  // instructions per block
    static_assert(NI % 4 == 0, "staging geometry");
#pragma unroll
    for (int ii = 0; ii < NI / 4; ++ii) {
      const int i = uniform(w) + 4 * ii;
      const int u = i * 64 + lane, r = u / PPR, p = (u % PPR) ^ (r & (PPR - 1));
      const uint32_t off = (uint32_t)((min(r, nv - 1) * H * DK) * (int)sizeof(TIO) + p * 16);
      lds_load16(gk, off, lds0 + i * 1024);
      lds_load16(gqv, off, lds0 + 64 * RB + i * 1024);
    }
    if (w == 0) {
      float gv = 0.f, bv = 0.f;
      if (lane < nv) {
        gv = a.g[(int64_t)(t0 + lane) * H + h];
        bv = a.beta[(int64_t)(t0 + lane) * H + h];
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(gv, off, 64);
        if (lane >= off) gv += y;
      }
      sG2[lane] = gv * 1.4426950408889634f;
      sBeta[lane] = bv;
    }
    wait_vmem();
  }
  __syncthreads();

  // C[s][t] = x_s . y_t for one 16 x 16 tile (rows sr of x, tr of y): lane holds s = 16 si + 4 gq + i, t = 16 ti + ln
  auto tile = [&](const char* xb, int sr, const char* yb, int tr) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBF) {
      bf16x8 af[NKB], bf[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint2 a0 = *reinterpret_cast<const uint2*>(xb + kq_at(sr, 32 * kb + 4 * gq));
        const uint2 a1 = *reinterpret_cast<const uint2*>(xb + kq_at(sr, 32 * kb + 16 + 4 * gq));
        const uint2 b0 = *reinterpret_cast<const uint2*>(yb + kq_at(tr, 32 * kb + 4 * gq));
        const uint2 b1 = *reinterpret_cast<const uint2*>(yb + kq_at(tr, 32 * kb + 16 + 4 * gq));
        af[kb] = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
        bf[kb] = __builtin_bit_cast(bf16x8, make_uint4(b0.x, b0.y, b1.x, b1.y));
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) mma_bf16(acc, af[kb], bf[kb]);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float av[8], bv[8];
        const float4 a0 = *reinterpret_cast<const float4*>(xb + kq_at(sr, 32 * kb + 4 * gq));
        const float4 a1 = *reinterpret_cast<const float4*>(xb + kq_at(sr, 32 * kb + 16 + 4 * gq));
        const float4 b0 = *reinterpret_cast<const float4*>(yb + kq_at(tr, 32 * kb + 4 * gq));
        const float4 b1 = *reinterpret_cast<const float4*>(yb + kq_at(tr, 32 * kb + 16 + 4 * gq));
        av[0] = a0.x; av[1] = a0.y; av[2] = a0.z; av[3] = a0.w; av[4] = a1.x; av[5] = a1.y; av[6] = a1.z; av[7] = a1.w;
        bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w; bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
        mma_f32(acc, av, bv);
      }
    }
    return acc;
  };
  // ---- ten tile jobs (ri, si), si <= ri, at most 3 per wave: with C_A = K K^T
  // and C_P = K Q^T on the tile (one shared A operand, the k rows of block si)
  //   A[r][s] = beta_r exp(gamma_r - gamma_s) C_A[s][r]    (s < r)   -> sA
  //   P[r][s] = exp(gamma_r - gamma_s) C_P[s][r]           (s <= r)  -> the P record
  // plus the two zero P tiles (0,1) and (2,3) that complete fragment pairs.
  char* prec = reinterpret_cast<char*>(a.P) + ((int64_t)j * H + h) * kTRecBytes;
  auto put_p = [&](int ri, int si, const float (&v)[4]) {
    // record slot: pair pr = (ri, si / 2), lane l, elements 4 (si % 2) .. + 3
    const int pr = (si >= 2) ? ri + 2 : ri, jb = (si & 1) * 4;
    if constexpr (kBF) {
      uint32_t h0, l0, h1, l1;
      split_bf16x2(v[0], v[1], h0, l0);
      split_bf16x2(v[2], v[3], h1, l1);
      *reinterpret_cast<uint2*>(prec + (pr * 64 + lane) * 16 + jb * 2) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(prec + ((6 + pr) * 64 + lane) * 16 + jb * 2) = make_uint2(l0, l1);
    } else {
      *reinterpret_cast<float4*>(prec + (pr * 64 + lane) * 32 + jb * 4) = make_float4(v[0], v[1], v[2], v[3]);
    }
  };
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    const int job = w + 4 * jj;
    if (job < 10) {
      const int ri = (job < 1) ? 0 : (job < 3) ? 1 : (job < 6) ? 2 : 3;
      const int si = job - (ri * (ri + 1)) / 2;
      const int r = 16 * ri + ln;
      const f32x4 ca = tile(sK, 16 * si + ln, sK, r);
      const f32x4 cp = tile(sK, 16 * si + ln, sQ, r);
      const float g2r = sG2[r], br = sBeta[r];
      float va[4], vp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * si + 4 * gq + i;
        const float e = (s <= r) ? __builtin_amdgcn_exp2f(g2r - sG2[s]) : 0.f;
        va[i] = (s < r) ? br * e * ca[i] : 0.f;
        vp[i] = e * cp[i];
      }
      *reinterpret_cast<float4*>(sA + r * L64 + 16 * si + 4 * gq) = make_float4(va[0], va[1], va[2], va[3]);
      put_p(ri, si, vp);
    } else if (job < 12) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
      const int si = (job == 10) ? 1 : 3;
      put_p(si - 1, si, z);
    }
  }
  __syncthreads();

  solve_unit_lower(sA, sX);
  store_record<kBF>(sX, sBeta, reinterpret_cast<char*>(a.T) + ((int64_t)j * H + h) * kTRecBytes);
}


// ---------------------------------------------------------------------------
// Per-key-channel gate (#2506 "What does this PR do?": per-key-channel
// retention, pairwise exponentials from prefix differences).  g is
// [T, H, dk], gamma_r in R^dk, and per chunk
//     A[r][s] = beta_r sum_c k_rc k_sc exp(gamma_rc - gamma_sc)      (s < r)
//     P[r][s] = sum_c q_rc k_sc exp(gamma_rc - gamma_sc)             (s <= r)
//     T       = (I + A)^-1 diag(beta)
// No exp(-gamma) is formed on its own (it overflows).  Each 16 x 16 tile
// (R, S) is an fp32 MFMA product of operands scaled to a reference token m
// of block R: exp(gamma_r - gamma_s) = exp(gamma_r - gamma_m)
// exp(gamma_m - gamma_s), both factors <= 1 for non-positive gates when S < R;
// on the diagonal tiles the factors stay within a guard band or the tile is
// summed channel by channel from the differences.  T and P are written as
// two records per (chunk, head) in the layout above.
// ---------------------------------------------------------------------------
template <int DK, typename TIO>
struct KdaPrepLds {
  static constexpr int LX = DK + 16 / (int)sizeof(TIO);  // k, q row stride (elements)
  static constexpr int LG = DK + 4;                      // gamma row stride (floats)
  static constexpr size_t oK = 0;
  static constexpr size_t oQ = oK + 64 * LX * sizeof(TIO);
  static constexpr size_t oG = oQ + 64 * LX * sizeof(TIO);
  static constexpr size_t oA = oG + 64 * LG * sizeof(float);
  static constexpr size_t oP = oA + 64 * kL64 * sizeof(float);
  static constexpr size_t oTot = oP + 64 * kL64 * sizeof(float);
  static constexpr size_t oBeta = oTot + kThreads * sizeof(float);
  static constexpr size_t bytes = oBeta + 64 * sizeof(float);
  // once A and P are formed, the solve's X overlays k and q
  static constexpr size_t oX = oK;
  static_assert(64 * kL64 * sizeof(float) <= oG - oK, "X does not fit over k and q");
};

template <typename TIO>
__device__ __forceinline__ void load4f(const TIO* p, float (&x)[4]) {
  if constexpr (sizeof(TIO) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
}

template <int DK, typename TIO>
__global__ __launch_bounds__(kThreads, 1) void kda_prep_kernel(PrepArgs a) {
  using Ls = KdaPrepLds<DK, TIO>;
  constexpr bool kBF = sizeof(TIO) == 2;
  constexpr int LX = Ls::LX, LG = Ls::LG, L64 = kL64, NKB = DK / 32;
  extern __shared__ __align__(16) char smem[];
  TIO* sK = reinterpret_cast<TIO*>(smem + Ls::oK);
  TIO* sQ = reinterpret_cast<TIO*>(smem + Ls::oQ);
  float* sG = reinterpret_cast<float*>(smem + Ls::oG);    // gamma * log2(e)
  float* sA = reinterpret_cast<float*>(smem + Ls::oA);
  float* sP = reinterpret_cast<float*>(smem + Ls::oP);
  float* sTot = reinterpret_cast<float*>(smem + Ls::oTot);
  float* sBeta = reinterpret_cast<float*>(smem + Ls::oBeta);
  float* sX = reinterpret_cast<float*>(smem + Ls::oX);

  const int H = a.H;
  const int j = blockIdx.x / H, h = blockIdx.x % H;
  const int total = a.offs[a.N];
  if (j >= total) return;  // grid is sized for the worst case
  int lo = 0, hi = a.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.offs[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int n = lo, c = j - a.offs[n];
  const int seg0 = a.cu_seqlens[n];
  const int L = a.seq_lens ? a.seq_lens[n] : (a.cu_seqlens[n + 1] - seg0);
  const int P = a.prefix_lens ? a.prefix_lens[n] : L;
  const int t0 = seg0 + c * kChunk;
  const int nv = min(kChunk, P - c * kChunk);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;

  // ---- stage k and q (rows past nv are zero), beta, and the per-channel gate prefix
  {
    constexpr int EPS = 16 / (int)sizeof(TIO);
    constexpr int SPR = DK / EPS;
    const TIO* gk = reinterpret_cast<const TIO*>(a.k);
    const TIO* gqv = reinterpret_cast<const TIO*>(a.q);
    static_assert(64 * SPR % kThreads == 0, "staging geometry");
#pragma unroll
    for (int jj = 0; jj < 64 * SPR / kThreads; ++jj) {
      const int seg = tid + kThreads * jj;
      const int r = seg / SPR, c0 = (seg % SPR) * EPS;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), qv = make_uint4(0u, 0u, 0u, 0u);
      if (r < nv) {
        const int64_t off = ((int64_t)(t0 + r) * H + h) * DK + c0;
        kv = *reinterpret_cast<const uint4*>(gk + off);
        qv = *reinterpret_cast<const uint4*>(gqv + off);
      }
      *reinterpret_cast<uint4*>(sK + r * LX + c0) = kv;
      *reinterpret_cast<uint4*>(sQ + r * LX + c0) = qv;
    }
    if (tid < 64) sBeta[tid] = (tid < nv) ? a.beta[(int64_t)(t0 + tid) * H + h] : 0.f;
  }
  constexpr int NPART = kThreads / DK, TPP = 64 / NPART;  // token parts of the per-channel scan
  {
    const int d = tid % DK, part = tid / DK;
    float gv[TPP];  // all loads in flight before the scan
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      const int r = part * TPP + i;
      gv[i] = (r < nv) ? a.g[((int64_t)(t0 + r) * H + h) * DK + d] : 0.f;
    }
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      run += gv[i];
      sG[(part * TPP + i) * LG + d] = run;
    }
    sTot[tid] = run;
  }
  __syncthreads();
  {
    const int d = tid % DK, part = tid / DK;
    float off = 0.f;
    for (int pp = 0; pp < part; ++pp) off += sTot[pp * DK + d];
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      const int r = part * TPP + i;
      sG[r * LG + d] = (sG[r * LG + d] + off) * 1.4426950408889634f;
    }
  }
  __syncthreads();

  // ---- the ten 16 x 16 tiles (R, S), S <= R, one job each: C[s][r] with
  // A = k_s exp(gamma_m - gamma_s), B = x_r exp(gamma_r - gamma_m) (x = k for
  // A, q for P), m = 16 R the first token of block R.  For S < R both factors
  // are <= 1.  On the diagonal tile the first factor is >= 1: it is used only
  // when every |gamma_t - gamma_m| of the block stays under 2^kGuard in
  // magnitude (no overflow, no underflow), else that tile is summed channel
  // by channel with the exponential of each difference.
  constexpr float kGuard = 100.f;  // log2 units
  for (int job = w; job < 10; job += 4) {
    const int R = (job < 1) ? 0 : (job < 3) ? 1 : (job < 6) ? 2 : 3;
    const int S = job - (R * (R + 1)) / 2;
    const int m = 16 * R;
    const int s = 16 * S + ln, r = 16 * R + ln;  // A-operand row s, B-operand column r of this lane
    f32x4 ca = {0.f, 0.f, 0.f, 0.f}, cp = {0.f, 0.f, 0.f, 0.f};
    float span = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float av[8], bk[8], bq[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c0 = 32 * kb + 16 * hh + 4 * gq;  // channels kperm(gq, 4 hh .. 4 hh + 3)
        const float4 gs4 = *reinterpret_cast<const float4*>(sG + s * LG + c0);
        const float4 gm4 = *reinterpret_cast<const float4*>(sG + m * LG + c0);
        const float4 gr4 = *reinterpret_cast<const float4*>(sG + r * LG + c0);
        const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
        const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
        const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w};
        float ks[4], kr[4], qr[4];
        load4f(sK + s * LX + c0, ks);
        load4f(sK + r * LX + c0, kr);
        load4f(sQ + r * LX + c0, qr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          span = fmaxf(span, fmaxf(fabsf(gm[i] - gs[i]), fabsf(gr[i] - gm[i])));
          av[4 * hh + i] = ks[i] * __builtin_amdgcn_exp2f(fminf(gm[i] - gs[i], kGuard));
          const float f = __builtin_amdgcn_exp2f(fminf(gr[i] - gm[i], kGuard));
          bk[4 * hh + i] = kr[i] * f;
          bq[4 * hh + i] = qr[i] * f;
        }
      }
      mma_f32(ca, av, bk);
      mma_f32(cp, av, bq);
    }
    const bool exact = (S < R) || wave_max_dpp(span) < kGuard;
    if (exact) {
      // lane holds C[16 S + 4 gq + i][16 R + ln]; zero at and above the diagonal (A), above it (P)
      const float br = sBeta[r];
      float va[4], vp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sc = 16 * S + 4 * gq + i;
        va[i] = (sc < r) ? br * ca[i] : 0.f;
        vp[i] = (sc <= r) ? cp[i] : 0.f;
      }
      *reinterpret_cast<float4*>(sA + r * L64 + 16 * S + 4 * gq) = make_float4(va[0], va[1], va[2], va[3]);
      *reinterpret_cast<float4*>(sP + r * L64 + 16 * S + 4 * gq) = make_float4(vp[0], vp[1], vp[2], vp[3]);
    } else {
      // diagonal tile with a large in-block decay: pairs s <= r, channel by channel
      for (int pi = lane; pi < 256; pi += 64) {
        const int rl = pi >> 4, sl = pi & 15;
        const int rr = 16 * R + rl, ss = 16 * R + sl;
        float sa[4] = {0.f, 0.f, 0.f, 0.f}, sp[4] = {0.f, 0.f, 0.f, 0.f};
        if (sl <= rl) {
          for (int c0 = 0; c0 < DK; c0 += 4) {
            float kr[4], qr[4], ks[4];
            load4f(sK + rr * LX + c0, kr);
            load4f(sQ + rr * LX + c0, qr);
            load4f(sK + ss * LX + c0, ks);
            const float4 gr4 = *reinterpret_cast<const float4*>(sG + rr * LG + c0);
            const float4 gs4 = *reinterpret_cast<const float4*>(sG + ss * LG + c0);
            const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w};
            const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float ke = ks[i] * __builtin_amdgcn_exp2f(gr[i] - gs[i]);
              sa[i] = fmaf(kr[i], ke, sa[i]);
              sp[i] = fmaf(qr[i], ke, sp[i]);
            }
          }
        }
        const float av = (sa[0] + sa[1]) + (sa[2] + sa[3]);
        const float pv = (sp[0] + sp[1]) + (sp[2] + sp[3]);
        sA[rr * L64 + ss] = (sl < rl) ? sBeta[rr] * av : 0.f;
        sP[rr * L64 + ss] = (sl <= rl) ? pv : 0.f;
      }
    }
  }
  __syncthreads();

  const int64_t rec = ((int64_t)j * H + h) * kTRecBytes;
  store_record<kBF>(sP, nullptr, reinterpret_cast<char*>(a.P) + rec);
  solve_unit_lower(sA, sX);
  store_record<kBF>(sX, sBeta, reinterpret_cast<char*>(a.T) + rec);
}

size_t prep_workspace_bytes(int64_t n_seqs, int64_t n_heads, int64_t total_tokens) {
  const int64_t max_chunks = (total_tokens + kChunk - 1) / kChunk + n_seqs;
  const size_t offs = ((size_t)(n_seqs + 1) * 4 + 255) / 256 * 256;
  return offs + (size_t)max_chunks * n_heads * kTRecBytes * 2;
}

template <int DK, typename TIO>
static hipError_t launch_kda_prep(dim3 grid, const PrepArgs& a, hipStream_t stream) {
  auto kern = kda_prep_kernel<DK, TIO>;
  constexpr size_t lds = KdaPrepLds<DK, TIO>::bytes;
  static bool attr_set = false;  // the attribute is per function; setting it twice is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_prep(const gdn_shape_t& s, const void* q, const void* k, const float* beta,
                       const float* g, const int32_t* cu_seqlens, const int32_t* seq_lens,
                       const int32_t* prefix_lens, void* workspace, const int32_t** offs_out,
                       void** T_out, void** P_out, hipStream_t stream) {
  int32_t* offs = reinterpret_cast<int32_t*>(workspace);
  const size_t offs_bytes = ((size_t)(s.n_seqs + 1) * 4 + 255) / 256 * 256;
  const int64_t max_chunks = (s.total_tokens + kChunk - 1) / kChunk + s.n_seqs;
  const int64_t blocks = max_chunks * s.n_heads;
  void* T = reinterpret_cast<char*>(workspace) + offs_bytes;
  void* Prec = reinterpret_cast<char*>(T) + (size_t)blocks * kTRecBytes;
  *offs_out = offs;
  *T_out = T;
  *P_out = Prec;
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, seq_lens,
                     prefix_lens, s.n_seqs, offs);
  if (blocks == 0) return hipGetLastError();
  PrepArgs a;
  a.q = q; a.k = k; a.beta = beta; a.g = g; a.cu_seqlens = cu_seqlens; a.seq_lens = seq_lens;
  a.prefix_lens = prefix_lens; a.offs = offs; a.T = T; a.P = Prec; a.N = s.n_seqs; a.H = s.n_heads;
  const dim3 grid((unsigned)blocks);
  if (s.gate_per_channel) {
    if (s.io_dtype == GDN_BF16)
      return s.dk == 128 ? launch_kda_prep<128, uint16_t>(grid, a, stream)
                         : launch_kda_prep<64, uint16_t>(grid, a, stream);
    if (s.dk != 64) return hipErrorNotSupported;  // fp32 inputs: dk = 64 only
    return launch_kda_prep<64, float>(grid, a, stream);
  }
  if (s.io_dtype == GDN_BF16) {
    if (s.dk == 128)
      hipLaunchKernelGGL((chunk_prep_kernel<128, uint16_t>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<64, uint16_t>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (s.dk != 64) return hipErrorNotSupported;  // fp32 inputs: dk = 64 only
    hipLaunchKernelGGL((chunk_prep_kernel<64, float>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
