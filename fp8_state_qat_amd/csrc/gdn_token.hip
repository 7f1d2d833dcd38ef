// gdn_token.hip -- the chunked forward for fp32 q, k, v with dk = 128 (the
// reference-precision inputs), as the token recurrence it regroups
// (Model-Optimizer #2497 "What does this PR do?": the chunked form with the
// state QDQ at every 64-token boundary; #2519 "What does this PR do?", step
// 3: QDQ at the handoff and after every later recurrent write).  Inside a
// chunk the token steps give the chunked products' result up to rounding
// (no QDQ falls inside a chunk), so one kernel serves the prefix and the
// suffix: per token t of sequence n (decay a_t = exp(g_t), or a row of
// per-key-channel factors; on the log-retention grid for t > P only)
//     S~ = S a_t,  y = S~ k_t,  z = S~ q_t,  u = beta_t (v_t - y)
//     o_t = z + (k_t . q_t) u      (= S_t q_t),   S = S~ + u k_t^T
// then the tile QDQ where the chunked kernels take it: after the last token
// of each prefix chunk (GDN_QDQ_CHUNK; the last one also for GDN_QDQ_WRITE)
// and after every suffix token (GDN_QDQ_WRITE).  The boundary and suffix
// records are those of the chunked kernels.
//
// One workgroup (256 threads) per (sequence, head, 64-row value tile) holds
// its 64 x dk slice of the state in registers in the decode step's layout
// (thread t: float4 column group t % (dk/4) of rows t / (dk/4) + p * 256 /
// (dk/4)); row dot products by the decode step's fixed DPP tree; two
// workgroup barriers per token (three more at a QDQ).  fp32 throughout: the
// MFMA chunk kernels' fp32 engine does not fit this dk in LDS, and this path
// exists for its precision, not its speed.
#include "gdn_chunk_common.hpp"

namespace gdn {

constexpr int kTokThreads = 256;

template <int DK, typename TO, bool PC>
__global__ __launch_bounds__(kTokThreads) void chunk_token_kernel(ChunkArgs args) {
  constexpr int F = DK / 4;              // float4 per state row
  constexpr int RPP = kTokThreads / F;   // rows per pass
  constexpr int NP = kTileRows / RPP;    // passes over the tile
  static_assert(NP * RPP == kTileRows, "tile geometry");
  __shared__ float red[4];
  __shared__ float s_o[kTileRows];
  __shared__ float s_v[kTileRows];
  if (index_check_failed(args.status)) return;

  const int H = args.H, dv = args.dv, tiles = dv / kTileRows;
  const int vt = (int)blockIdx.x % tiles;
  const int nh = (int)blockIdx.x / tiles;
  const int h = nh % H, n = nh / H;
  const int seg0 = args.cu_seqlens[n], seg1 = args.cu_seqlens[n + 1];
  const int L = args.seq_lens ? args.seq_lens[n] : (seg1 - seg0);
  const int P = args.prefix_lens ? args.prefix_lens[n] : L;
  const int t = threadIdx.x, c4 = t % F, rr = t / F;
  const float* gq_ = reinterpret_cast<const float*>(args.q);
  const float* gk_ = reinterpret_cast<const float*>(args.k);
  const float* gv_ = reinterpret_cast<const float*>(args.v);
  TO* go_ = reinterpret_cast<TO*>(args.o);
  const int64_t qk_row = (int64_t)H * DK, v_row = (int64_t)H * dv;
  const int row_base = kTileRows * vt;  // first value row of the tile
  // element offset of this thread's float4 in row r of the tile, in a [.., H, dv, dk] array
  auto tile_off = [&](int64_t lead, int r) { return ((lead * H + h) * dv + row_base + r) * DK + 4 * c4; };

  float4 x[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    x[p] = args.init ? *reinterpret_cast<const float4*>(args.init + tile_off(n, rr + RPP * p))
                     : make_float4(0.f, 0.f, 0.f, 0.f);

  const unsigned flags = args.flags;
  const int bound0 = args.bound_offsets ? args.bound_offsets[n] : 0;
  const int64_t sfx0 = args.sfx_offsets ? args.sfx_offsets[n] : 0;
  auto store_rows = [&](float* base, int64_t lead) {
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<float4*>(base + tile_off(lead, rr + RPP * p)) = x[p];
  };

  for (int tok = 0; tok < L; ++tok) {
    const int64_t row = seg0 + tok;
    const bool sfx = tok >= P;
    const float4 k4 = *reinterpret_cast<const float4*>(gk_ + row * qk_row + (int64_t)h * DK + 4 * c4);
    const float4 q4 = *reinterpret_cast<const float4*>(gq_ + row * qk_row + (int64_t)h * DK + 4 * c4);
    float dec[4];
    if constexpr (PC) {
      const float4 g4 = *reinterpret_cast<const float4*>(args.g + (row * H + h) * DK + 4 * c4);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) dec[j] = expf(sfx ? grid_gate(gg[j], args.grid_log2) : gg[j]);
    } else {
      const float gs = args.g[row * H + h];
      const float a = expf(sfx ? grid_gate(gs, args.grid_log2) : gs);
#pragma unroll
      for (int j = 0; j < 4; ++j) dec[j] = a;
    }
    const float b = args.beta[row * H + h];
    if (t < kTileRows) s_v[t] = gv_[row * v_row + (int64_t)h * dv + row_base + t];
    __syncthreads();  // s_v of this token; every read of the last token's s_o is done

    const float kq = group_sum<F>(k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w);
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = rr + RPP * p;
      const float sd0 = x[p].x * dec[0], sd1 = x[p].y * dec[1], sd2 = x[p].z * dec[2], sd3 = x[p].w * dec[3];
      const float y = group_sum<F>(sd0 * k4.x + sd1 * k4.y + sd2 * k4.z + sd3 * k4.w);
      const float z = group_sum<F>(sd0 * q4.x + sd1 * q4.y + sd2 * q4.z + sd3 * q4.w);
      const float u = b * (s_v[r] - y);
      if (c4 == 0) s_o[r] = z + kq * u;
      x[p] = make_float4(sd0 + u * k4.x, sd1 + u * k4.y, sd2 + u * k4.z, sd3 + u * k4.w);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[p].x), fabsf(x[p].y)), fmaxf(fabsf(x[p].z), fabsf(x[p].w))));
    }
    __syncthreads();  // s_o complete
    if (t < kTileRows) io<TO>::st(go_ + row * v_row + (int64_t)h * dv + row_base + t, s_o[t]);

    // the QDQ and the records where the chunked kernels take them
    const bool boundary = !sfx && ((tok + 1) % kChunk == 0 || tok + 1 == P);
    bool do_qdq = false;
    if (boundary) do_qdq = (flags & GDN_QDQ_CHUNK) || ((flags & GDN_QDQ_WRITE) && tok + 1 == P);
    else if (sfx) do_qdq = (flags & GDN_QDQ_WRITE) != 0;
    const int bidx = bound0 + tok / kChunk;
    if (boundary && args.bound_pre) store_rows(args.bound_pre, bidx);
    if (sfx && args.sfx_offsets && args.sfx_pre) store_rows(args.sfx_pre, sfx0 + tok - P);
    float s = 1.0f;
    if (do_qdq) {
      s = qdq_scale_f64(block_max(amax, red));
      const double rs = rcp_f64(s);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        f32x4 v = {x[p].x, x[p].y, x[p].z, x[p].w};
        float cv[4];
        qdq4c_f64(v, cv, s, rs);
        x[p] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    if (boundary) {
      if (args.bound_post) store_rows(args.bound_post, bidx);
      if (args.bound_scales && t == 0) args.bound_scales[((int64_t)bidx * H + h) * tiles + vt] = s;
    }
    if (sfx && args.sfx_offsets && args.sfx_post) store_rows(args.sfx_post, sfx0 + tok - P);
  }

  store_rows(args.fin, n);
  // padding rows of the segment: o = 0
  for (int r = L + (t >> 6); r < seg1 - seg0; r += kTokThreads / 64)
    io<TO>::st(go_ + (int64_t)(seg0 + r) * v_row + (int64_t)h * dv + row_base + (t & 63), 0.f);
}

hipError_t launch_chunk_token(const gdn_shape_t& s, const ChunkArgs& a, hipStream_t stream) {
  if (s.io_dtype != GDN_F32 || s.dk != 128 || (s.qdq_flags & GDN_QDQ_W)) return hipErrorNotSupported;
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows);
  if (blocks == 0) return hipSuccess;
  const bool ob = s.o_dtype == GDN_BF16;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kTokThreads), 0, stream, a);
    return hipGetLastError();
  };
  if (s.gate_per_channel)
    return ob ? go(chunk_token_kernel<128, uint16_t, true>) : go(chunk_token_kernel<128, float, true>);
  return ob ? go(chunk_token_kernel<128, uint16_t, false>) : go(chunk_token_kernel<128, float, false>);
}

}  // namespace gdn
