// gdn_prep.hip -- the state-independent part of the chunked gated delta rule
// (Model-Optimizer #2497: 64-token chunks with WY/UT-transformed W and U;
// #2506: the exact triangular solve), for every (chunk, head) in parallel:
// the in-chunk gate scan, A, T = (I + A)^-1 diag(beta) and the decayed,
// masked P = Q K^T (gdn_prep_item.hpp for the scalar gate, kda_prep_kernel
// below for a per-key-channel gate).  The sequential kernel forms
// U' = T (V - exp(gamma) * K S^T) and O = exp(gamma) * Q S^T + P U' from them.
//
// The solve is blocked on 16 x 16 blocks in fp32: the four diagonal blocks
// by forward substitution (one lane per column), then the off-diagonal
// blocks level by level, X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj, on the fp32
// MFMA.
//
// Workspace layout: int32 chunk offsets [N + 1] (prefix sums of
// ceil(P_n / 64)) and the largest chunk count of a sequence, padded to 256
// bytes; one uint32 ready flag per (chunk, head) (used by the fused launch of
// the scalar-gate kernel), padded to 256 bytes; then one 12 KiB T record per
// (chunk, head), then one P record per (chunk, head) of the same layout.  A
// record holds the six nonzero 16 x 32 fragments of a block lower-triangular
// 64 x 64 matrix M, pair p = (ti, kb) in (0,0) (1,0) (2,0) (3,0) (2,1) (3,1):
// lane l of fragment p holds M[16 ti + l % 16][32 kb + kperm(l / 16, j)] for
// j = 0..7 (kperm as in gdn_device.hpp), fragments stored one after the
// other, lane-major.  bf16 inputs store hi = bf16(M) (six fragments) then
// lo = bf16(M - hi) (six more); fp32 inputs store M in fp32.  The sequential
// kernels copy a record into LDS unchanged and read each fragment with one
// lane-linear load (T as the A operand of T X, P as the B operand of
// U'^T P^T).
#include <algorithm>

#include "gdn_prep_item.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// chunk offsets: offs[n] = sum_{m < n} ceil(P_m / 64), offs[N + 1] = the
// largest ceil(P_n / 64), in workgroup 0; every workgroup clears its share of
// the n_ready ready flags (none when ready is null).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void chunk_offsets_kernel(const int32_t* __restrict__ cu,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 const int32_t* __restrict__ prefix_lens,
                                                                 int N, int32_t* __restrict__ offs,
                                                                 unsigned* __restrict__ ready, int64_t n_ready) {
  if (ready != nullptr) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_ready; i += (int64_t)gridDim.x * kThreads)
      ready[i] = 0u;
  }
  if (blockIdx.x != 0) return;
  __shared__ int32_t part[kThreads];
  __shared__ int32_t carry, most;
  if (threadIdx.x == 0) {
    carry = 0;
    most = 0;
  }
  __syncthreads();
  int32_t my_most = 0;
  for (int base = 0; base < N; base += kThreads) {
    const int n = base + threadIdx.x;
    int32_t cnt = 0;
    if (n < N) {
      const int32_t L = seq_lens ? seq_lens[n] : (cu[n + 1] - cu[n]);
      const int32_t P = prefix_lens ? prefix_lens[n] : L;
      cnt = (P + kChunk - 1) / kChunk;
    }
    my_most = max(my_most, cnt);
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
  atomicMax(&most, my_most);
  __syncthreads();
  if (threadIdx.x == 0) {
    offs[N] = carry;
    offs[N + 1] = most;
  }
}

// One workgroup (4 waves) per (chunk, head).  TIO: uint16_t (bf16) or float.
template <int DK, typename TIO>
__global__ __launch_bounds__(kThreads, 3) void chunk_prep_kernel(PrepArgs a) {
  __shared__ __align__(16) char lds[PrepItemLds<DK, TIO>::bytes];
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
  prep_item<DK, TIO>(a, j, h, seg0 + c * kChunk, min(kChunk, P - c * kChunk), lds, threadIdx.x, true);
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
  store_record<kBF>(sP, nullptr, reinterpret_cast<char*>(a.P) + rec, threadIdx.x);
  solve_unit_lower(sA, sX, threadIdx.x);
  store_record<kBF>(sX, sBeta, reinterpret_cast<char*>(a.T) + rec, threadIdx.x);
}

PrepLayout prep_layout(const gdn_shape_t& s, void* workspace) {
  PrepLayout L;
  char* w = reinterpret_cast<char*>(workspace);
  const int64_t max_chunks = (s.total_tokens + kChunk - 1) / kChunk + s.n_seqs;
  L.items = max_chunks * s.n_heads;
  const size_t offs_bytes = ((size_t)(s.n_seqs + 2) * 4 + 255) / 256 * 256;
  const size_t ready_bytes = ((size_t)L.items * 4 + 255) / 256 * 256;
  L.offs = nullptr;
  L.ready = nullptr;
  L.T = L.P = nullptr;
  if (w != nullptr) {
    L.offs = reinterpret_cast<int32_t*>(w);
    L.ready = reinterpret_cast<unsigned*>(w + offs_bytes);
    L.T = w + offs_bytes + ready_bytes;
    L.P = w + offs_bytes + ready_bytes + (size_t)L.items * kTRecBytes;
  }
  L.bytes = offs_bytes + ready_bytes + (size_t)L.items * kTRecBytes * 2;
  return L;
}

size_t prep_workspace_bytes(int64_t n_seqs, int64_t n_heads, int64_t total_tokens) {
  gdn_shape_t s{};
  s.n_seqs = (int32_t)n_seqs;
  s.n_heads = (int32_t)n_heads;
  s.total_tokens = total_tokens;
  return prep_layout(s, nullptr).bytes;
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
                       const int32_t* prefix_lens, const PrepLayout& L, bool records, hipStream_t stream) {
  // with records false the fused launch produces them and needs cleared ready flags
  const int64_t zero_blocks = records ? 1 : std::min<int64_t>(64, std::max<int64_t>(1, (L.items + 4095) / 4096));
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3((unsigned)zero_blocks), dim3(kThreads), 0, stream, cu_seqlens,
                     seq_lens, prefix_lens, s.n_seqs, L.offs, records ? nullptr : L.ready, L.items);
  if (!records || L.items == 0) return hipGetLastError();
  PrepArgs a;
  a.q = q; a.k = k; a.beta = beta; a.g = g; a.cu_seqlens = cu_seqlens; a.seq_lens = seq_lens;
  a.prefix_lens = prefix_lens; a.offs = L.offs; a.T = L.T; a.P = L.P; a.N = s.n_seqs; a.H = s.n_heads;
  const dim3 grid((unsigned)L.items);
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
