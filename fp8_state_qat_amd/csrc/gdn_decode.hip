// gdn_decode.hip -- single-token recurrent step with per-write state QDQ
// (Model-Optimizer #2519 "What does this PR do?", step 3: each token reads
// the stored state, computes its output from the updated working state, and
// quantizes the state before storing it for the next token).
//
// Per (sequence, head) and 64-row value tile of the state S (64 x dk fp32):
//     S~ = S * a                       (a = exp(g); per-key-channel: S diag(exp(g));
//                                       g on the log-retention grid when one is set)
//     y  = S~ k ;  z = S~ q ;  u = beta (v - y)
//     o  = z + (k . q) u               (= S' q with S' = S~ + u k^T)
//     S' = S~ + u k^T ;  S <- QDQ(S')  (one scale for the tile)
//
// A nullable active mask [N] skips whole sequences: their state, o and
// records are left as they are (a batch whose sequences end at different
// lengths, #2519 "What does this PR do?": prefill and full sequence lengths
// per sequence).
//
// Memory bound: the tile is read once and written once (2 * 4 * 64 * dk
// bytes); q, k, v, beta, g and o are a few hundred bytes per head.  One
// workgroup (256 threads) per tile.  Thread t owns the float4 column group
// c4 = t % (dk/4) and rows t / (dk/4) + p * (256 / (dk/4)); every load and
// store instruction of the block covers 4 KiB of contiguous state.  Row dot
// products are reduced over the dk/4 lanes of a row by DPP lane moves (a
// fixed order); the tile's 64 outputs go through LDS and leave as one
// contiguous store.
//
// kInt8: the per-write QDQ is INT8 with one scale per block of 32
// consecutive key columns of a state row (#2519: dynamic INT8 state recipes
// with 32-element blocks; scale amax / 127, round half to even): a block is
// the float4s of 8 adjacent lanes, so its amax is three DPP steps and the
// tile needs no workgroup reduction.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int DK, typename TIO, typename TO, bool PC, bool kInt8>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    const TIO* __restrict__ q, const TIO* __restrict__ k, const TIO* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ g, const int32_t* __restrict__ active,
    float* __restrict__ state, TO* __restrict__ o, float* __restrict__ state_pre,
    float* __restrict__ scales, int H, int dv, int do_qdq, int grid_log2) {
  constexpr int F = DK / 4;         // float4 per state row
  constexpr int RPP = kThreads / F; // rows covered by one pass of the block
  constexpr int NP = kTileRows / RPP;
  __shared__ float red[4];
  __shared__ float s_o[kTileRows];

  const int tiles = dv / kTileRows;
  const int vt = blockIdx.x % tiles;
  const int64_t nh = blockIdx.x / tiles;  // n * H + h
  // an inactive sequence (finished, or padding of a batch): nothing is read or written
  if (active != nullptr && __builtin_amdgcn_readfirstlane(active[nh / H]) == 0) return;
  const int t = threadIdx.x;
  const int c4 = t % F;
  const int rr = t / F;

  // this thread's four key columns
  float kc[4], qc[4], dec[4];
  const TIO* kp = k + nh * DK + 4 * c4;
  const TIO* qp = q + nh * DK + 4 * c4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kc[j] = io<TIO>::ld(kp + j);
    qc[j] = io<TIO>::ld(qp + j);
  }
  if constexpr (PC) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dec[j] = expf(grid_gate(g[nh * DK + 4 * c4 + j], grid_log2));
  } else {
    const float a = expf(grid_gate(g[nh], grid_log2));
#pragma unroll
    for (int j = 0; j < 4; ++j) dec[j] = a;
  }
  const float b = beta[nh];

  // k . q over all dk columns (same fixed tree in every row group)
  const float kq = group_sum<F>(kc[0] * qc[0] + kc[1] * qc[1] + kc[2] * qc[2] + kc[3] * qc[3]);

  const int64_t tile_base = (nh * dv + (int64_t)kTileRows * vt) * DK;  // float offset
  float4* S = reinterpret_cast<float4*>(state + tile_base);
  float4 x[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) x[p] = ld_stream(S + t + kThreads * p);

  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = rr + RPP * p;
    float sd0 = x[p].x * dec[0], sd1 = x[p].y * dec[1], sd2 = x[p].z * dec[2], sd3 = x[p].w * dec[3];
    const float y = group_sum<F>(sd0 * kc[0] + sd1 * kc[1] + sd2 * kc[2] + sd3 * kc[3]);
    const float z = group_sum<F>(sd0 * qc[0] + sd1 * qc[1] + sd2 * qc[2] + sd3 * qc[3]);
    const float vr = io<TIO>::ld(v + nh * dv + kTileRows * vt + row);
    const float u = b * (vr - y);
    const float orow = z + kq * u;
    if (c4 == 0) s_o[row] = orow;
    x[p].x = sd0 + u * kc[0];
    x[p].y = sd1 + u * kc[1];
    x[p].z = sd2 + u * kc[2];
    x[p].w = sd3 + u * kc[3];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[p].x), fabsf(x[p].y)), fmaxf(fabsf(x[p].z), fabsf(x[p].w))));
  }
  if (state_pre != nullptr) {
    float4* P = reinterpret_cast<float4*>(state_pre + tile_base);
#pragma unroll
    for (int p = 0; p < NP; ++p) P[t + kThreads * p] = x[p];
  }
  float s = 1.0f;
  if (kInt8 && do_qdq) {
    static_assert(DK % 32 == 0, "INT8 blocks of 32 key columns");
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float bm = lane8_max_dpp(fmaxf(fmaxf(fabsf(x[p].x), fabsf(x[p].y)), fmaxf(fabsf(x[p].z), fabsf(x[p].w))));
      const float sb = int8_scale_f64(bm);
      qdq_int8_4_f64(x[p], sb);
      if (scales != nullptr && (c4 & 7) == 0)
        scales[(nh * dv + kTileRows * vt + rr + RPP * p) * (DK / 32) + (c4 >> 3)] = sb;
    }
    __syncthreads();  // s_o
  } else if (do_qdq) {
    amax = block_max(amax, red);  // its barriers also publish s_o
    s = qdq_scale_f64(amax);
    const double r = rcp_f64(s);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      f32x4 v = {x[p].x, x[p].y, x[p].z, x[p].w};
      float cv[4];
      qdq4c_f64(v, cv, s, r);
      x[p] = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
    __syncthreads();  // s_o
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) st_stream(S + t + kThreads * p, x[p]);
  if (t < kTileRows) io<TO>::st(o + nh * dv + kTileRows * vt + t, s_o[t]);
  if (!kInt8 && scales != nullptr && t == 0) scales[nh * tiles + vt] = s;
}

template <int DK, typename TIO, typename TO>
static void launch_dk_io_o(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const int32_t* active, float* state,
                           void* o, float* state_pre, float* scales, hipStream_t stream) {
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows);
  const int qdq = (s.qdq_flags & GDN_QDQ_WRITE) ? 1 : 0;
  const bool i8 = (s.qdq_flags & GDN_QDQ_INT8) != 0;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), 0, stream, (const TIO*)q, (const TIO*)k,
                       (const TIO*)v, beta, g, active, state, (TO*)o, state_pre, scales, s.n_heads, s.dv, qdq,
                       s.gate_grid_log2);
  };
  if (s.gate_per_channel) {
    if (i8) go(decode_step_kernel<DK, TIO, TO, true, true>);
    else go(decode_step_kernel<DK, TIO, TO, true, false>);
  } else {
    if (i8) go(decode_step_kernel<DK, TIO, TO, false, true>);
    else go(decode_step_kernel<DK, TIO, TO, false, false>);
  }
}

template <int DK>
static void launch_dk(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                      const float* beta, const float* g, const int32_t* active, float* state, void* o,
                      float* state_pre, float* scales, hipStream_t stream) {
  const bool ib = s.io_dtype == GDN_BF16, ob = s.o_dtype == GDN_BF16;
  if (ib && ob)
    launch_dk_io_o<DK, uint16_t, uint16_t>(s, q, k, v, beta, g, active, state, o, state_pre, scales, stream);
  else if (ib)
    launch_dk_io_o<DK, uint16_t, float>(s, q, k, v, beta, g, active, state, o, state_pre, scales, stream);
  else if (ob)
    launch_dk_io_o<DK, float, uint16_t>(s, q, k, v, beta, g, active, state, o, state_pre, scales, stream);
  else
    launch_dk_io_o<DK, float, float>(s, q, k, v, beta, g, active, state, o, state_pre, scales, stream);
}

hipError_t launch_decode_step(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                              const float* beta, const float* g, const int32_t* active, float* state,
                              void* o, float* state_pre, float* scales, hipStream_t stream) {
  if (s.dk == 64)
    launch_dk<64>(s, q, k, v, beta, g, active, state, o, state_pre, scales, stream);
  else
    launch_dk<128>(s, q, k, v, beta, g, active, state, o, state_pre, scales, stream);
  return hipGetLastError();
}

}  // namespace gdn
