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
// Workspace layout: the int32 status word, padded to 256 bytes; int32 chunk
// offsets [N + 1] (prefix sums of ceil(P_n / 64)) and the largest chunk count
// of a sequence, padded to 256 bytes; one uint32 ready flag per (chunk, head) (used by the fused launch of
// the scalar-gate kernel), padded to 256 bytes; then one 12 KiB T record per
// (chunk, head) (18 KiB slots), then one P record per (chunk, head) of the
// same layout (12 KiB), then with W QDQ one W record per (chunk, head)
// (layout in gdn_launch.hpp).  A record holds the six nonzero 16 x 32
// fragments of a block lower-triangular 64 x 64 matrix M, pair p = (ti, kb)
// in (0,0) (1,0) (2,0) (3,0) (2,1) (3,1): lane l of fragment p holds
// M[16 ti + l % 16][32 kb + kperm(l / 16, j)] for j = 0..7 (kperm as in
// gdn_device.hpp), fragments stored one after the other, lane-major.  bf16
// inputs store planes of six fragments each: hi = bf16(M), then mid =
// bf16(M - hi), and for T a third, lo = bf16(M - hi - mid) (24 significant
// bits in all); fp32 inputs store M in fp32.  The sequential
// kernels copy a record into LDS unchanged and read each fragment with one
// lane-linear load (T as the A operand of T X, P as the B operand of
// U'^T P^T).
#include <algorithm>

#include "gdn_prep_item.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// chunk offsets: offs[n] = sum_{m < n} ceil(P_m / 64), offs[N + 1] = the
// largest ceil(P_n / 64), in workgroup 0; every workgroup clears its share of
// the n_ready ready flags (none when ready is null).  Workgroup 0 also checks
// the index arrays against their contract (0 <= cu[n] <= cu[n + 1] <=
// total_tokens, 0 <= L_n <= cu[n + 1] - cu[n], 0 <= P_n <= L_n) and writes
// the status word: kStatusBadIndex when any of them is violated, else 0.
// The kernels that follow on the stream read it first and do nothing on a
// violation, so out-of-contract indices never become out-of-bounds accesses.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void chunk_offsets_kernel(const int32_t* __restrict__ cu,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 const int32_t* __restrict__ prefix_lens,
                                                                 int N, int64_t total_tokens,
                                                                 int32_t* __restrict__ offs,
                                                                 int32_t* __restrict__ status,
                                                                 unsigned* __restrict__ ready, int64_t n_ready) {
  if (ready != nullptr) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_ready; i += (int64_t)gridDim.x * kThreads)
      ready[i] = 0u;
  }
  if (blockIdx.x != 0) return;
  __shared__ int32_t part[kThreads];
  __shared__ int32_t carry, most, bad;
  if (threadIdx.x == 0) {
    carry = 0;
    most = 0;
    bad = (cu[0] < 0) ? 1 : 0;
  }
  __syncthreads();
  int32_t my_most = 0, my_bad = 0;
  for (int base = 0; base < N; base += kThreads) {
    const int n = base + threadIdx.x;
    int32_t cnt = 0;
    if (n < N) {
      const int32_t c0 = cu[n], c1 = cu[n + 1];
      const int32_t L = seq_lens ? seq_lens[n] : (c1 - c0);
      const int32_t P = prefix_lens ? prefix_lens[n] : L;
      if (c1 < c0 || (int64_t)c1 > total_tokens || L < 0 || L > c1 - c0 || P < 0 || P > L) my_bad = 1;
      cnt = my_bad ? 0 : (P + kChunk - 1) / kChunk;
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
  if (my_bad) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    offs[N] = carry;
    offs[N + 1] = most;
    if (status != nullptr) status[0] = bad ? kStatusBadIndex : 0;
  }
}

// One workgroup (4 waves) per (chunk, head).  TIO: uint16_t (bf16) or float.
// kW: W QDQ, the W record too (its LDS block is dynamic: over 64 KiB).
template <int DK, typename TIO, bool kW>
__global__ __launch_bounds__(kThreads, kW ? 2 : 3) void chunk_prep_kernel(PrepArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int H = a.H;
  const int j = blockIdx.x / H, h = blockIdx.x % H;
  if (index_check_failed(a.status)) return;
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
  prep_item<DK, TIO, kW>(a, j, h, seg0 + c * kChunk, min(kChunk, P - c * kChunk), lds, threadIdx.x, true);
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
template <int DK, typename TIO, bool kW>
__global__ __launch_bounds__(kThreads, 1) void kda_prep_kernel(PrepArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int H = a.H;
  const int j = blockIdx.x / H, h = blockIdx.x % H;
  if (index_check_failed(a.status)) return;
  const int total = a.offs[a.N];
  if (j >= total) return;
  int lo = 0, hi = a.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.offs[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int n = lo, c = j - a.offs[n];
  const int seg0 = a.cu_seqlens[n];
  const int L = a.seq_lens ? a.seq_lens[n] : (a.cu_seqlens[n + 1] - seg0);
  const int P = a.prefix_lens ? a.prefix_lens[n] : L;
  kda_prep_item<DK, TIO, kW>(a, j, h, seg0 + c * kChunk, min(kChunk, P - c * kChunk), smem, threadIdx.x);
}

__global__ void copy_status_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst) {
  if (threadIdx.x == 0) dst[0] = src[0];
}

hipError_t launch_copy_status(const int32_t* status, int32_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, stream, status, dst);
  return hipGetLastError();
}

PrepLayout prep_layout(const gdn_shape_t& s, void* workspace) {
  PrepLayout L;
  char* w = reinterpret_cast<char*>(workspace);
  const int64_t max_chunks = (s.total_tokens + kChunk - 1) / kChunk + s.n_seqs;
  L.items = max_chunks * s.n_heads;
  const size_t offs_bytes = ((size_t)(s.n_seqs + 2) * 4 + 255) / 256 * 256;
  const size_t ready_bytes = ((size_t)L.items * 4 + 255) / 256 * 256;
  L.status = nullptr;
  L.offs = nullptr;
  L.ready = nullptr;
  L.T = L.P = L.W = nullptr;
  const size_t w_bytes = (s.qdq_flags & GDN_QDQ_W) ? (size_t)L.items * w_rec_bytes(s.dk) : 0;
  if (w != nullptr) {
    L.status = reinterpret_cast<int32_t*>(w);
    w += kStatusBytes;
    L.offs = reinterpret_cast<int32_t*>(w);
    L.ready = reinterpret_cast<unsigned*>(w + offs_bytes);
    L.T = w + offs_bytes + ready_bytes;
    L.P = w + offs_bytes + ready_bytes + (size_t)L.items * kTRecBytes;
    if (w_bytes) L.W = w + offs_bytes + ready_bytes + (size_t)L.items * (kTRecBytes + kPRecBytes);
  }
  L.bytes = kStatusBytes + offs_bytes + ready_bytes + (size_t)L.items * (kTRecBytes + kPRecBytes) + w_bytes;
  return L;
}

size_t prep_workspace_bytes(const gdn_shape_t& s) { return prep_layout(s, nullptr).bytes; }

template <int DK, typename TIO, bool kW>
static hipError_t launch_chunk_prep(dim3 grid, const PrepArgs& a, hipStream_t stream) {
  auto kern = chunk_prep_kernel<DK, TIO, kW>;
  constexpr size_t lds = PrepItemLds<DK, TIO, kW>::bytes;
  static PerDeviceOnce lds_attr;
  if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DK, typename TIO, bool kW>
static hipError_t launch_kda_prep(dim3 grid, const PrepArgs& a, hipStream_t stream) {
  auto kern = kda_prep_kernel<DK, TIO, kW>;
  constexpr size_t lds = KdaPrepLds<DK, TIO, kW>::bytes;
  static PerDeviceOnce lds_attr;
  if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_prep(const gdn_shape_t& s, const void* q, const void* k, const float* beta,
                       const float* g, const int32_t* cu_seqlens, const int32_t* seq_lens,
                       const int32_t* prefix_lens, const PrepLayout& L, bool records, float* w_pre,
                       float* w_post, hipStream_t stream) {
  // with records false the fused launch produces them and needs cleared ready flags
  const int64_t zero_blocks = records ? 1 : std::min<int64_t>(64, std::max<int64_t>(1, (L.items + 4095) / 4096));
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3((unsigned)zero_blocks), dim3(kThreads), 0, stream, cu_seqlens,
                     seq_lens, prefix_lens, s.n_seqs, (int64_t)s.total_tokens, L.offs, L.status,
                     records ? nullptr : L.ready, L.items);
  if (!records || L.items == 0) return hipGetLastError();
  PrepArgs a;
  a.q = q; a.k = k; a.beta = beta; a.g = g; a.cu_seqlens = cu_seqlens; a.seq_lens = seq_lens;
  a.prefix_lens = prefix_lens; a.offs = L.offs; a.T = L.T; a.P = L.P; a.N = s.n_seqs; a.H = s.n_heads;
  a.W = L.W; a.w_pre = w_pre; a.w_post = w_post; a.status = L.status;
  const dim3 grid((unsigned)L.items);
  const bool wq = L.W != nullptr;
  if (s.gate_per_channel) {
    if (s.io_dtype == GDN_BF16) {
      if (s.dk == 128)
        return wq ? launch_kda_prep<128, uint16_t, true>(grid, a, stream)
                  : launch_kda_prep<128, uint16_t, false>(grid, a, stream);
      return wq ? launch_kda_prep<64, uint16_t, true>(grid, a, stream)
                : launch_kda_prep<64, uint16_t, false>(grid, a, stream);
    }
    if (s.dk != 64) return hipErrorNotSupported;  // fp32 inputs: dk = 64 only
    return wq ? launch_kda_prep<64, float, true>(grid, a, stream)
              : launch_kda_prep<64, float, false>(grid, a, stream);
  }
  if (s.io_dtype == GDN_BF16) {
    if (s.dk == 128)
      return wq ? launch_chunk_prep<128, uint16_t, true>(grid, a, stream)
                : launch_chunk_prep<128, uint16_t, false>(grid, a, stream);
    return wq ? launch_chunk_prep<64, uint16_t, true>(grid, a, stream)
              : launch_chunk_prep<64, uint16_t, false>(grid, a, stream);
  }
  if (s.dk != 64) return hipErrorNotSupported;  // fp32 inputs: dk = 64 only
  return wq ? launch_chunk_prep<64, float, true>(grid, a, stream)
            : launch_chunk_prep<64, float, false>(grid, a, stream);
}

}  // namespace gdn
