// gdn_bwd.hip -- the backward state recurrence of the chunked gated delta
// rule with identity straight-through gradients through every QDQ
// (Model-Optimizer #2497 "What does this PR do?": QAT/QAD with identity
// straight-through gradients).  With the QDQ the identity in the backward,
// the gradient of L = sum_t o_t . do_t + <S_L, dS_L> with respect to the
// state entering chunk c, dh_c, follows from the chunk's forward algebra
// (U' = T V - W h^T, O = (Q o e^gamma) h^T + P U', h' = e^{gamma_C} h +
// U'^T (K o e^{gamma_C - gamma}), W = T (K o e^gamma)) backwards:
//     dU'  = P^T dO + diag(e^{gamma_C - gamma}) (K dh_{c+1}^T)
//     Y    = T^T dU'
//     dh_c = e^{gamma_C} dh_{c+1} + dO^T (Q o e^gamma) - Y^T (K o e^gamma)
// starting from dh = dS_L after the last chunk.  The states themselves do
// not enter (L is linear in them), so neither does the QDQ.  V enters a
// chunk only through U = T V, so Y is also the gradient of its values.
//
// chunk_bwd_prep_kernel: per (chunk, head) in parallel, T^T and P^T as full
// 64 x 64 records (prep_item_bwd).  chunk_bwd_dh_kernel: one workgroup per
// (sequence, head, 64-row value tile), the chunks in reverse order; compute
// wave w (of four) owns dh rows 16w .. 16w + 15 of the tile (dk/16 fp32
// accumulator tiles, the forward state's layout) and runs every product for
// them.  Two loader waves issue the loads of chunk c - 1 (k and q dumps, dO
// rows, both records, by direct global->LDS loads into the other of two
// buffers) while chunk c computes, and scan its gates, so that the compute
// waves never wait for the load unit to take an instruction.  Rows past a chunk's end load its last valid row; the
// P^T columns and the e^gamma entries of those rows are zero, so they reach
// no result.  bf16 inputs; fp32 operands enter the bf16 MFMA as hi + lo
// pairs.
//
// The backward of a W-QDQ forward (kW): the forward's U' = T V - Wq h^T uses
// Wq, the row-quantized W, and the quantizer's identity straight-through
// rule leaves Wq fixed in the gradient of h, so the last term becomes
//     dh_c = ... - dU'^T Wq      (in place of - Y^T (K o e^gamma) = - dU'^T W)
// with Wq = diag(w_s) codes: the forward's own producer code writes the W
// records (codes and row scales, bit for bit the forward's) into the
// workspace first, and the row scales go into the B operand (- w_s o dU').
// The codes come into LDS in place of the chunk's k dump once K dh^T has read
// it (two more barriers per chunk); the k dump's other use, the key term of
// the update, is the one they replace.
#include "gdn_prep_item.hpp"

namespace gdn {

// four compute waves own the dh rows; two loader waves issue every load
constexpr int kBwdComputeWaves = 4, kBwdLoadWaves = 2;
constexpr int kBwdThreads = 64 * (kBwdComputeWaves + kBwdLoadWaves);

// LDS of the dh kernel (bytes), two buffers by chunk parity: the k and q
// dumps of the chunk (the forward's rotated fragment layout, so K^T and Q^T
// come back by transpose reads), the tile's dO rows (padded rows), the T^T
// and P^T records, and the gates.
template <int DK>
struct BwdLds {
  static constexpr int NKB = DK / 32;
  static constexpr size_t F = 64 * 8 * 2;
  static constexpr size_t RS = 64 + 8;                 // padded dO row (elements)
  static constexpr size_t oK = 0;
  static constexpr size_t oQ = oK + 4 * NKB * F;
  static constexpr size_t oO = oQ + 4 * NKB * F;
  static constexpr size_t oTT = oO + 64 * RS * 2;
  static constexpr size_t oPT = oTT + kBRecBytes;
  static constexpr size_t oVec = oPT + kBRecBytes;     // e^gamma [64] (0 past the end), e^{gamma_C - gamma} [64], e^{gamma_C}
  static constexpr size_t oWs = oVec + (2 * 64 + 4) * sizeof(float);  // the W record's row scales [64] (kW)
  static constexpr size_t buf = oWs + 64 * sizeof(float);  // one buffer
  static constexpr size_t bytes = 2 * buf;
  static_assert(oTT % 16 == 0 && oPT % 16 == 0 && oWs % 16 == 0 && buf % 16 == 0,
                "direct loads need 16-byte aligned LDS");
  static_assert(4 * NKB * F == (size_t)w_rec_bytes(DK) - 1024, "the W codes take the k dump's place");
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

template <int DK>
__global__ __launch_bounds__(kThreads, 2) void chunk_bwd_prep_kernel(PrepArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int H = a.H;
  const int j = blockIdx.x / H, h = blockIdx.x % H;
  if (index_check_failed(a.status)) return;
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
  prep_item_bwd<DK>(a, j, h, seg0 + c * kChunk, min(kChunk, L - c * kChunk), lds, threadIdx.x);
}

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* g;
  const uint16_t* dout;
  const float* dfin;      // [N, H, dv, dk] or null
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* chunk_offs;
  const char* TT;         // one T^T record per (chunk, head)
  const char* PT;         // one P^T record per (chunk, head)
  float* dh;              // [n_bounds, H, dv, dk] or null
  float* dinit;           // [N, H, dv, dk] or null
  float* dvals;           // [T, H, dv] or null
  const char* W;          // kW: one W record per (chunk, head)
  const int32_t* status;  // the workspace's status word (index check)
  int H;
  int dv;
};

template <int DK, bool kW>
__global__ __launch_bounds__(kBwdThreads, 1) void chunk_bwd_dh_kernel(BwdArgs args) {
  using Ls = BwdLds<DK>;
  using Fr = bf16x8;
  constexpr int NT = DK / 16, NKB = DK / 32;
  constexpr int RS = (int)Ls::RS;
  extern __shared__ __align__(16) char smem[];
  if (index_check_failed(args.status)) return;
  const uint32_t lds0 = lds_base_u32(smem);

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  const int H = args.H, dv = args.dv, tiles = dv / kTileRows;
  // Workgroup b runs on XCD b % 8.  Each XCD takes a contiguous run of
  // (sequence, head, value tile) items, so that the value tiles of a head
  // share one L2 (their q, k, dO rows and records are fetched once) and the
  // value-gradient rows one XCD writes span whole lines across its channels.
  const int nb = (int)gridDim.x, xq = nb / 8, xr = nb % 8, xc = (int)blockIdx.x % 8;
  const int item = xc * xq + min(xc, xr) + (int)blockIdx.x / 8;
  const int vt = item % tiles;
  const int nh = item / tiles;
  const int h = nh % H, n = nh / H;
  const int seg0 = args.cu_seqlens[n];
  const int L = args.seq_lens ? args.seq_lens[n] : (args.cu_seqlens[n + 1] - seg0);
  const int n_chunks = (L + kChunk - 1) / kChunk;
  const int chunk0 = args.chunk_offs[n];
  const int vcol0 = kTileRows * vt + 16 * w + ln;  // this lane's dh row (value channel)
  const int64_t qk_row = (int64_t)H * DK;
  const int64_t v_row = (int64_t)H * dv;

  auto frag = [lane](const uint16_t* base, int f) { return *reinterpret_cast<const Fr*>(base + (f * 64 + lane) * 8); };
  const int qs = rot_slot(lane);
  auto qfrag = [qs](const uint16_t* base, int f) { return *reinterpret_cast<const Fr*>(base + (f * 64 + qs) * 8); };
  // element offset of x[t][d] in a k/q dump
  auto kpos = [](int t, int d) {
    return (((t >> 4) * NKB + (d >> 5)) * 64 + rot_slot(((d & 31) >> 3) * 16 + (t & 15))) * 8 + (d & 7);
  };
  // element offset of W[t][d] in a W record (the k dump's order without its rotation)
  auto wpos = [](int t, int d) {
    return (((t >> 4) * NKB + (d >> 5)) * 64 + ((d & 31) >> 3) * 16 + (t & 15)) * 8 + (d & 7);
  };

  // ---- dh of this lane: dst[t][i] = dh[vcol0][dkmap(16t + 4gq + i)]
  f32x4 dst[NT];
  const bool loader = w >= kBwdComputeWaves;
  const int lw = w - kBwdComputeWaves;  // loader wave index
  {
    const int64_t base = ((int64_t)nh * dv + vcol0) * DK;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (args.dfin && !loader) {
        const float4 x = *reinterpret_cast<const float4*>(args.dfin + base + dkmap(16 * t + 4 * gq));
        dst[t] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        dst[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // direct loads of chunk cc into buffer b: k and q dumps, dO rows (padded
  // rows, 7 per instruction), the two records, spread over the loader waves;
  // loader wave 0 fetches the log-gates
  float pg = 0.f;
  auto issue = [&](int cc, int b) {
    const int t0 = seg0 + cc * kChunk;
    const int nv = min(kChunk, L - cc * kChunk);
    const uint32_t base = lds0 + (uint32_t)(b * Ls::buf);
    const uint16_t* gk = args.k + (int64_t)t0 * qk_row + (int64_t)h * DK;
    const uint16_t* gqv = args.q + (int64_t)t0 * qk_row + (int64_t)h * DK;
#pragma unroll
    for (int i = lw; i < 4 * NKB; i += kBwdLoadWaves) {  // instruction: 64 lane slots of 16 bytes
      const int u = i * 64 + lane;
      const int f = u >> 6, l2 = rot_lane(u & 63);
      const int r = 16 * (f / NKB) + (l2 & 15);
      const int d = 32 * (f % NKB) + 8 * (l2 >> 4);
      const uint32_t off = (uint32_t)((min(r, nv - 1) * (int)qk_row + d) * 2);
      lds_load16(gk, off, base + (uint32_t)Ls::oK + i * 1024);
      lds_load16(gqv, off, base + (uint32_t)Ls::oQ + i * 1024);
    }
    const char* tt = args.TT + ((int64_t)(chunk0 + cc) * H + h) * kBRecBytes;
    const char* pt = args.PT + ((int64_t)(chunk0 + cc) * H + h) * kBRecBytes;
#pragma unroll
    for (int idx = lw; idx < (int)(kBRecBytes / 1024); idx += kBwdLoadWaves) {
      lds_load16(tt, (uint32_t)((idx * 64 + lane) * 16), base + (uint32_t)Ls::oTT + idx * 1024);
      lds_load16(pt, (uint32_t)((idx * 64 + lane) * 16), base + (uint32_t)Ls::oPT + idx * 1024);
    }
    {
      constexpr int RPI = 64 / 9, NI = (64 + RPI - 1) / RPI;  // 9 slots of 16 bytes per padded row
      const uint16_t* src = args.dout + (int64_t)t0 * v_row + (int64_t)h * dv + kTileRows * vt;
      const int rr = lane / 9, pc = lane % 9;
      const int lane_off = min(pc, 7) * 8;
#pragma unroll
      for (int i = lw; i < NI; i += kBwdLoadWaves) {
        const int r = i * RPI + rr;
        if (rr < RPI && r < 64)
          lds_load16(src, (uint32_t)((min(r, nv - 1) * (int)v_row + lane_off) * 2),
                     base + (uint32_t)Ls::oO + i * RPI * RS * 2);
      }
    }
    if (lw == 0) pg = (lane < nv) ? args.g[(int64_t)(t0 + lane) * H + h] : 0.f;
    if constexpr (kW) {  // the chunk's W row scales (16 lanes of 16 bytes)
      const char* wr = args.W + ((int64_t)(chunk0 + cc) * H + h) * w_rec_bytes(DK) + 4 * NKB * 1024;
      if (lw == 1 && lane < 16) lds_load16(wr, (uint32_t)(lane * 16), base + (uint32_t)Ls::oWs);
    }
  };
  // kW: the W codes of chunk cc into the k dump's place of buffer b (once K dh^T has read it)
  auto issue_w = [&](int cc, int b) {
    const char* wr = args.W + ((int64_t)(chunk0 + cc) * H + h) * w_rec_bytes(DK);
    const uint32_t base = lds0 + (uint32_t)(b * Ls::buf) + (uint32_t)Ls::oK;
#pragma unroll
    for (int i = lw; i < 4 * NKB; i += kBwdLoadWaves)
      lds_load16(wr, (uint32_t)((i * 64 + lane) * 16), base + i * 1024);
  };
  // loader wave 0: the gates of chunk cc from pg (e^gamma is zero past the chunk's end)
  auto scan = [&](int cc, float* vec) {
    const int nv = min(kChunk, L - cc * kChunk);
    const float x = wave_prefix_sum(pg);
    const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    vec[lane] = (lane < nv) ? __builtin_amdgcn_exp2f(x * kLog2e) : 0.f;
    vec[64 + lane] = __builtin_amdgcn_exp2f((gC - x) * kLog2e);
    if (lane == 0) vec[128] = __builtin_amdgcn_exp2f(gC * kLog2e);
  };

  // The results of chunk c + 1 (dh_{c+1}, still in dst until the update at
  // the end of chunk c, and its value gradient, kept in pend_y) are stored
  // after chunk c's prefetch is issued, so that the wait at the top of the
  // next chunk finds them long done instead of draining them.
  f32x4 pend_y[4];
  // Results are written once and not read again here: non-temporal stores.
  auto store_results = [&](int cs) {
    if (args.dh) {
      const int64_t base = (((int64_t)(chunk0 + cs) * H + h) * dv + vcol0) * DK;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        __builtin_nontemporal_store(dst[t], reinterpret_cast<f32x4*>(args.dh + base + dkmap(16 * t + 4 * gq)));
    }
    // the value gradient: lane holds Y[16ti + 4gq + i][16w + ln]
    if (args.dvals) {
      const int nv = min(kChunk, L - cs * kChunk);
      float* dvp = args.dvals + ((int64_t)(seg0 + cs * kChunk) * H + h) * dv + kTileRows * vt + 16 * w + ln;
      if (nv == kChunk) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(pend_y[ti][i], dvp + (int64_t)(16 * ti + 4 * gq + i) * v_row);
      } else {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * ti + 4 * gq + i;
            if (t < nv) __builtin_nontemporal_store(pend_y[ti][i], dvp + (int64_t)t * v_row);
          }
      }
    }
  };

  if (loader && n_chunks > 0) issue(n_chunks - 1, (n_chunks - 1) & 1);
  for (int c = n_chunks - 1; c >= 0; --c) {
    const int b = c & 1;
    char* bufp = smem + b * Ls::buf;
    uint16_t* sK = reinterpret_cast<uint16_t*>(bufp + Ls::oK);
    uint16_t* sQ = reinterpret_cast<uint16_t*>(bufp + Ls::oQ);
    uint16_t* sO = reinterpret_cast<uint16_t*>(bufp + Ls::oO);
    const uint16_t* sTT = reinterpret_cast<const uint16_t*>(bufp + Ls::oTT);
    const uint16_t* sPT = reinterpret_cast<const uint16_t*>(bufp + Ls::oPT);
    float* vec = reinterpret_cast<float*>(bufp + Ls::oVec);
    if (lw == 0) scan(c, vec);
    wait_vmem();      // this wave's loads of chunk c are in LDS
    __syncthreads();  // ... every wave's, and the gates; chunk c + 1's buffer is free
    if (loader) {
      if (c > 0) issue(c - 1, b ^ 1);
      if constexpr (kW) {
        __syncthreads();  // every compute wave has read the k dump of chunk c
        issue_w(c, b);
        wait_vmem();
        __syncthreads();  // the W codes are in LDS
      }
      continue;
    }
    if (c + 1 < n_chunks) store_results(c + 1);

    // ---- G = K dh^T (A = k rows, B = dh as hi + lo)
    Fr dhh[NKB], dhl[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float x[8] = {dst[2 * kb][0], dst[2 * kb][1], dst[2 * kb][2], dst[2 * kb][3],
                          dst[2 * kb + 1][0], dst[2 * kb + 1][1], dst[2 * kb + 1][2], dst[2 * kb + 1][3]};
      EngBF16::split(x, dhh[kb], dhl[kb]);
    }
    f32x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      Fr kf[4 * NKB];
#pragma unroll
      for (int f = 0; f < 4 * NKB; ++f) kf[f] = qfrag(sK, f);  // f = tt * NKB + kb
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          mma_bf16(acc[tt], kf[tt * NKB + kb], dhh[kb]);
          mma_bf16(acc[tt], kf[tt * NKB + kb], dhl[kb]);
        }
    }
    if constexpr (kW) __syncthreads();  // the k dump of chunk c is read: its place takes the W codes
    // ---- dO as B operands: element j of k-block kb = dO[32kb + kperm(gq, j)][16w + ln]
    Fr of[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint2 r0 = lds_read_tr16(sO + (32 * kb + 4 * gq + (ln >> 2)) * RS + 16 * w + 4 * (ln & 3));
      const uint2 r1 = lds_read_tr16(sO + (32 * kb + 16 + 4 * gq + (ln >> 2)) * RS + 16 * w + 4 * (ln & 3));
      of[kb] = __builtin_bit_cast(Fr, make_uint4(r0.x, r0.y, r1.x, r1.y));
    }
    // ---- dU' = P^T dO + D G   (lane holds dU'[16ti + 4gq + i][16w + ln])
    f32x4 uacc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) uacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (the record's fragments four pairs at a time, read before their products)
#pragma unroll
    for (int p0 = 0; p0 < 8; p0 += 4) {
      Fr ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ph[j] = frag(sPT, p0 + j);
        pl[j] = frag(sPT, 8 + p0 + j);
      }
      __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of the products
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ti = (p0 + j) >> 1, kb = (p0 + j) & 1;
        mma_bf16(uacc[ti], ph[j], of[kb]);
        mma_bf16(uacc[ti], pl[j], of[kb]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const float4 d4 = *reinterpret_cast<const float4*>(vec + 64 + 16 * tt + 4 * gq);
      uacc[tt][0] = fmaf(d4.x, acc[tt][0], uacc[tt][0]);
      uacc[tt][1] = fmaf(d4.y, acc[tt][1], uacc[tt][1]);
      uacc[tt][2] = fmaf(d4.z, acc[tt][2], uacc[tt][2]);
      uacc[tt][3] = fmaf(d4.w, acc[tt][3], uacc[tt][3]);
    }
    // ---- Y = T^T dU' (B = dU' as hi + lo: k-block kb from tiles 2kb, 2kb + 1)
    Fr uh[2], ul[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float u8[8] = {uacc[2 * kb][0], uacc[2 * kb][1], uacc[2 * kb][2], uacc[2 * kb][3],
                           uacc[2 * kb + 1][0], uacc[2 * kb + 1][1], uacc[2 * kb + 1][2], uacc[2 * kb + 1][3]};
      EngBF16::split(u8, uh[kb], ul[kb]);
    }
    f32x4 yacc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) yacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p0 = 0; p0 < 8; p0 += 4) {
      Fr th[4], tl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        th[j] = frag(sTT, p0 + j);
        tl[j] = frag(sTT, 8 + p0 + j);
      }
      __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of the products
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ti = (p0 + j) >> 1, kb = (p0 + j) & 1;
        mma_bf16(yacc[ti], th[j], uh[kb]);
        mma_bf16(yacc[ti], th[j], ul[kb]);
        mma_bf16(yacc[ti], tl[j], uh[kb]);
      }
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) pend_y[ti] = yacc[ti];
    // ---- B operands of the update: e^gamma dO, and -e^gamma Y (kW: -w_s dU'), hi + lo
    const float* ws = reinterpret_cast<const float*>(bufp + Ls::oWs);
    Fr boh[2], bol[2], byh[2], byl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4 e0 = *reinterpret_cast<const float4*>(vec + 32 * kb + 4 * gq);
      const float4 e1 = *reinterpret_cast<const float4*>(vec + 32 * kb + 16 + 4 * gq);
      const float e8[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
      const uint4 ou = __builtin_bit_cast(uint4, of[kb]);
      const uint32_t ow[4] = {ou.x, ou.y, ou.z, ou.w};
      float o8[8], y8[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o8[2 * q] = e8[2 * q] * bf16_lo(ow[q]);
        o8[2 * q + 1] = e8[2 * q + 1] * bf16_hi(ow[q]);
      }
      if constexpr (kW) {
        const float4 s0 = *reinterpret_cast<const float4*>(ws + 32 * kb + 4 * gq);
        const float4 s1 = *reinterpret_cast<const float4*>(ws + 32 * kb + 16 + 4 * gq);
        const float s8[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y8[i] = -s8[i] * uacc[2 * kb][i];
          y8[4 + i] = -s8[4 + i] * uacc[2 * kb + 1][i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y8[i] = -e8[i] * yacc[2 * kb][i];
          y8[4 + i] = -e8[4 + i] * yacc[2 * kb + 1][i];
        }
      }
      EngBF16::split(o8, boh[kb], bol[kb]);
      EngBF16::split(y8, byh[kb], byl[kb]);
    }
    // ---- dh^T <- e^{gamma_C} dh^T + Q^T (e^gamma dO) + K^T (-e^gamma Y)
    //      (kW: + codes^T (-w_s dU'), the codes in the k dump's place)
    const float eC = vec[128];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[t][i] *= eC;
    // lane (gq, l) of each 16-lane group points at x[32kb + 16h + 4gq + l/4][dkmap(16t + 4(l%4)) .. +3]
    auto tr_frags = [&](const uint16_t* base, auto pos, int t, Fr (&a)[2]) {
      const int d = dkmap(16 * t + 4 * (ln & 3));
      const int tq = 4 * gq + (ln >> 2);
      const uint2 x0 = lds_read_tr16(base + pos(tq, d)), x1 = lds_read_tr16(base + pos(tq + 16, d));
      const uint2 y0 = lds_read_tr16(base + pos(tq + 32, d)), y1 = lds_read_tr16(base + pos(tq + 48, d));
      a[0] = __builtin_bit_cast(Fr, make_uint4(x0.x, x0.y, x1.x, x1.y));
      a[1] = __builtin_bit_cast(Fr, make_uint4(y0.x, y0.y, y1.x, y1.y));
    };
    if constexpr (kW) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Fr qa[2];
        tr_frags(sQ, kpos, t, qa);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          mma_bf16(dst[t], qa[kb], boh[kb]);
          mma_bf16(dst[t], qa[kb], bol[kb]);
        }
      }
      __syncthreads();  // the W codes of chunk c are in LDS
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Fr wa[2];
        tr_frags(sK, wpos, t, wa);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          mma_bf16(dst[t], wa[kb], byh[kb]);
          mma_bf16(dst[t], wa[kb], byl[kb]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Fr qa[2], ka[2];
        tr_frags(sQ, kpos, t, qa);
        tr_frags(sK, kpos, t, ka);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          mma_bf16(dst[t], qa[kb], boh[kb]);
          mma_bf16(dst[t], qa[kb], bol[kb]);
          mma_bf16(dst[t], ka[kb], byh[kb]);
          mma_bf16(dst[t], ka[kb], byl[kb]);
        }
      }
    }
    // dst now holds dh_c, the gradient of the state entering chunk c
  }
  if (loader) return;
  if (n_chunks > 0) store_results(0);
  if (args.dvals) {  // padding rows of the segment
    const int seg_len = args.cu_seqlens[n + 1] - seg0;
    for (int r = L + w; r < seg_len; r += kBwdComputeWaves)
      args.dvals[((int64_t)(seg0 + r) * H + h) * dv + kTileRows * vt + lane] = 0.f;
  }
  if (args.dinit) {
    const int64_t base = ((int64_t)nh * dv + vcol0) * DK;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<float4*>(args.dinit + base + dkmap(16 * t + 4 * gq)) =
          make_float4(dst[t][0], dst[t][1], dst[t][2], dst[t][3]);
  }
}

// ---------------------------------------------------------------------------
// Per-key-channel gate: the reverse token recurrence itself (the oracle's
// form, written out per token; the gradient is linear in the states, so no
// forward state enters).  With G the gradient of the state after token t
// (rows: the tile's 64 value channels, columns: dk key channels), from
// G = d_final_state, for t = L .. 1:
//     G  += do_t q_t^T                      (o_t = S_t q_t)
//     y   = G k_t,   d_v[t] = beta_t y      (v_t enters through beta_t v_t k_t^T)
//     G  <- (G - beta_t y k_t^T) diag(exp(g_t))   (now the gradient of S_{t-1})
// and dh of chunk c is G once token 64c + 1 is taken back.  One workgroup
// (256 threads) per (sequence, head, 32 rows of a value tile) with G in registers,
// in the decode step's layout (thread t: float4 column group t % (dk/4) of
// rows t / (dk/4) + p * 256 / (dk/4)); row dot products by the decode step's
// fixed DPP tree.  The tokens of a chunk are staged in LDS as fp32 (q, k,
// exp(g), the tile's d_o columns, beta) and its value gradients leave from
// LDS as whole rows.  Vector ALU bound (about 4 * 64 * dk FMAs per token and
// tile); no split-bf16 products, so fp32 throughout.
// The rows of G are independent (the backward has no QDQ to couple them),
// so a workgroup takes kKdaBwdRows rows of a value tile: twice the
// workgroups of one per tile, so that a full-size call fills the GPU.
constexpr int kKdaBwdRows = 32;

template <int DK>
struct KdaBwdLds {
  static constexpr int R = kKdaBwdRows;
  static constexpr size_t oQ = 0, oK = oQ + 64 * DK, oE = oK + 64 * DK, oO = oE + 64 * DK;
  static constexpr size_t oB = oO + 64 * R, oDV = oB + 64;
  static constexpr size_t floats = oDV + 64 * R;
  static constexpr size_t bytes = floats * sizeof(float);
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

struct KdaBwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* beta;
  const float* g;         // [T, H, dk]
  const uint16_t* dout;
  const float* dfin;
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* chunk_offs;
  float* dh;
  float* dinit;
  float* dvals;
  const int32_t* status;
  int H;
  int dv;
};

template <int DK>
__global__ __launch_bounds__(kThreads) void kda_bwd_token_kernel(KdaBwdArgs a) {
  using Ls = KdaBwdLds<DK>;
  constexpr int R = kKdaBwdRows;
  constexpr int F = DK / 4;          // float4 per state row
  constexpr int RPP = kThreads / F;  // rows per pass
  constexpr int NP = R / RPP;        // passes over the workgroup's rows
  static_assert(NP >= 1 && R % RPP == 0, "row geometry");
  extern __shared__ __align__(16) float kb_smem[];
  if (index_check_failed(a.status)) return;
  float* sq = kb_smem + Ls::oQ;
  float* sk = kb_smem + Ls::oK;
  float* se = kb_smem + Ls::oE;
  float* so = kb_smem + Ls::oO;
  float* sb = kb_smem + Ls::oB;
  float* sdv = kb_smem + Ls::oDV;
  const int t = threadIdx.x, c4 = t % F, rr = t / F;
  const int H = a.H, dv = a.dv, parts = dv / R;
  // the row blocks of a (sequence, head) on one XCD (workgroup b runs on XCD
  // b % 8) when the grid comes in groups of 8 pairs, so that the chunk's q, k
  // and g reach the other blocks from that XCD's L2
  int rb, nh;
  {
    const int b = (int)blockIdx.x;
    if (parts > 1 && (int)gridDim.x % (8 * parts) == 0) {
      const int slot8 = b >> 3;
      rb = slot8 % parts;
      nh = (slot8 / parts) * 8 + (b & 7);
    } else {
      rb = b % parts;
      nh = b / parts;
    }
  }
  const int h = nh % H, n = nh / H;
  const int seg0 = a.cu_seqlens[n];
  const int L = a.seq_lens ? a.seq_lens[n] : (a.cu_seqlens[n + 1] - seg0);
  const int n_chunks = (L + kChunk - 1) / kChunk;
  const int chunk0 = a.chunk_offs[n];
  const int64_t qk_row = (int64_t)H * DK, v_row = (int64_t)H * dv;
  const int row0 = R * rb;                                     // first value row of the workgroup
  const int64_t blk = ((int64_t)nh * dv + row0) * DK;          // row row0 of (n, h) in [N, H, dv, dk]

  float4 G[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    G[p] = a.dfin ? reinterpret_cast<const float4*>(a.dfin + blk)[t + kThreads * p] : make_float4(0.f, 0.f, 0.f, 0.f);

  for (int c = n_chunks - 1; c >= 0; --c) {
    const int t0 = c * kChunk;
    const int nv = min(kChunk, L - t0);
    // every load of the chunk issued before any is used: rows past its end
    // read its last valid row (in bounds) and are replaced by 0 (by 1 for
    // exp(g)) when stored
    constexpr int NI = kChunk * DK / kThreads, NO = kChunk * R / kThreads;
    uint16_t rq[NI], rk[NI], ro[NO];
    float rg[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = t + kThreads * j, tok = i / DK, col = i % DK;
      const int64_t off = (seg0 + t0 + min(tok, nv - 1)) * qk_row + (int64_t)h * DK + col;
      rq[j] = a.q[off];
      rk[j] = a.k[off];
      rg[j] = a.g[off];
    }
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int i = t + kThreads * j, tok = i / R, r = i % R;
      ro[j] = a.dout[(seg0 + t0 + min(tok, nv - 1)) * v_row + (int64_t)h * dv + row0 + r];
    }
    const float rbeta = t < kChunk ? a.beta[(int64_t)(seg0 + t0 + min(t, nv - 1)) * H + h] : 0.f;
    __syncthreads();  // the last chunk's staged tokens and value gradients are consumed
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = t + kThreads * j;
      const bool ok = i / DK < nv;
      sq[i] = ok ? bf16_bits_to_float(rq[j]) : 0.f;
      sk[i] = ok ? bf16_bits_to_float(rk[j]) : 0.f;
      se[i] = ok ? expf(rg[j]) : 1.f;
    }
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int i = t + kThreads * j;
      so[i] = i / R < nv ? bf16_bits_to_float(ro[j]) : 0.f;
    }
    if (t < kChunk) sb[t] = t < nv ? rbeta : 0.f;
    __syncthreads();
    // the operands of token tok, read one token ahead of their use
    float4 qv, kv, ev;
    float b, dor[NP];
    auto read_token = [&](int tok) {
      qv = reinterpret_cast<const float4*>(sq + tok * DK)[c4];
      kv = reinterpret_cast<const float4*>(sk + tok * DK)[c4];
      ev = reinterpret_cast<const float4*>(se + tok * DK)[c4];
      b = sb[tok];
#pragma unroll
      for (int p = 0; p < NP; ++p) dor[p] = so[tok * R + rr + RPP * p];
    };
    read_token(nv - 1);
    for (int tok = nv - 1; tok >= 0; --tok) {
      const float4 q4 = qv, k4 = kv, e4 = ev;
      const float bt = b;
      float d4[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) d4[p] = dor[p];
      if (tok > 0) read_token(tok - 1);
      // the rows are independent: each step for all of them before the next,
      // so that their dependent chains (the reductions above all) overlap
      float dot[NP], by[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        G[p].x = fmaf(d4[p], q4.x, G[p].x);
        G[p].y = fmaf(d4[p], q4.y, G[p].y);
        G[p].z = fmaf(d4[p], q4.z, G[p].z);
        G[p].w = fmaf(d4[p], q4.w, G[p].w);
        dot[p] = G[p].x * k4.x + G[p].y * k4.y + G[p].z * k4.z + G[p].w * k4.w;
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) by[p] = bt * group_sum<F>(dot[p]);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        G[p].x = (G[p].x - by[p] * k4.x) * e4.x;
        G[p].y = (G[p].y - by[p] * k4.y) * e4.y;
        G[p].z = (G[p].z - by[p] * k4.z) * e4.z;
        G[p].w = (G[p].w - by[p] * k4.w) * e4.w;
      }
      if (c4 == 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p) sdv[tok * R + rr + RPP * p] = by[p];
      }
    }
    if (a.dh) {  // the gradient of the state entering chunk c
      float4* dst = reinterpret_cast<float4*>(a.dh + (((int64_t)(chunk0 + c) * H + h) * dv + row0) * DK);
#pragma unroll
      for (int p = 0; p < NP; ++p) dst[t + kThreads * p] = G[p];
    }
    __syncthreads();  // the chunk's value gradients are in LDS
    if (a.dvals) {
      for (int i = t; i < nv * R; i += kThreads) {
        const int tok = i / R, r = i % R;
        a.dvals[(seg0 + t0 + tok) * v_row + (int64_t)h * dv + row0 + r] = sdv[i];
      }
    }
  }
  if (a.dinit) {
#pragma unroll
    for (int p = 0; p < NP; ++p) reinterpret_cast<float4*>(a.dinit + blk)[t + kThreads * p] = G[p];
  }
  if (a.dvals) {  // padding rows of the segment
    const int seg_len = a.cu_seqlens[n + 1] - seg0;
    for (int i = L * R + t; i < seg_len * R; i += kThreads)
      a.dvals[(seg0 + i / R) * v_row + (int64_t)h * dv + row0 + i % R] = 0.f;
  }
}

size_t bwd_workspace_bytes(const gdn_shape_t& s) {
  const int64_t max_chunks = (s.total_tokens + kChunk - 1) / kChunk + s.n_seqs;
  const size_t items = (size_t)(max_chunks * s.n_heads);
  const size_t offs_bytes = ((size_t)(s.n_seqs + 2) * 4 + 255) / 256 * 256;
  if (s.gate_per_channel) return kStatusBytes + offs_bytes;  // the token recurrence needs no records
  // with W QDQ the forward's records too (its producer writes the W records)
  const size_t fwd = (s.qdq_flags & GDN_QDQ_W) ? (size_t)(kTRecBytes + kPRecBytes + w_rec_bytes(s.dk)) : 0;
  return kStatusBytes + offs_bytes + items * (kBRecBytes * 2 + fwd);
}

template <int DK, bool kW>
static hipError_t launch_bwd_dk(const gdn_shape_t& s, const PrepArgs& pa, const BwdArgs& ba, int64_t items,
                                hipStream_t stream) {
  {
    auto kern = chunk_bwd_prep_kernel<DK>;
    constexpr size_t lds = PrepBwdLds<DK>::bytes;
    static PerDeviceOnce lds_attr;
    if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
    if (items > 0) hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(kThreads), lds, stream, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto kern = chunk_bwd_dh_kernel<DK, kW>;
  constexpr size_t lds = BwdLds<DK>::bytes;
  static PerDeviceOnce lds_attr;
  if (hipError_t e = set_dyn_lds_once(lds_attr, (const void*)kern, lds); e != hipSuccess) return e;
  const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kTileRows);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBwdThreads), lds, stream, ba);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_dh(const gdn_shape_t& s, const void* q, const void* k, const float* beta,
                               const float* g, const int32_t* cu_seqlens, const int32_t* seq_lens,
                               const void* dout, const float* dfin, float* dh, float* dinit, float* dvals,
                               void* workspace, hipStream_t stream) {
  char* w = reinterpret_cast<char*>(workspace);
  const int64_t max_chunks = (s.total_tokens + kChunk - 1) / kChunk + s.n_seqs;
  const int64_t items = max_chunks * s.n_heads;
  const size_t offs_bytes = ((size_t)(s.n_seqs + 2) * 4 + 255) / 256 * 256;
  int32_t* status = reinterpret_cast<int32_t*>(w);
  int32_t* offs = reinterpret_cast<int32_t*>(w + kStatusBytes);
  char* TT = w + kStatusBytes + offs_bytes;
  char* PT = TT + (size_t)items * kBRecBytes;
  const bool wq = (s.qdq_flags & GDN_QDQ_W) != 0;
  // chunk offsets of the whole sequences (prefix = length), status word; with
  // W QDQ also the forward's records (T, P, W), by the forward's producer code
  PrepLayout L{};
  L.status = status;
  L.offs = offs;
  L.ready = nullptr;
  L.items = items;
  if (wq) {
    L.T = PT + (size_t)items * kBRecBytes;
    L.P = reinterpret_cast<char*>(L.T) + (size_t)items * kTRecBytes;
    L.W = reinterpret_cast<char*>(L.P) + (size_t)items * kPRecBytes;
  }
  hipError_t e = launch_prep(s, q, k, beta, g, cu_seqlens, seq_lens, nullptr, L, wq, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  if (s.gate_per_channel) {
    KdaBwdArgs ka{};
    ka.q = reinterpret_cast<const uint16_t*>(q);
    ka.k = reinterpret_cast<const uint16_t*>(k);
    ka.beta = beta;
    ka.g = g;
    ka.dout = reinterpret_cast<const uint16_t*>(dout);
    ka.dfin = dfin;
    ka.cu_seqlens = cu_seqlens;
    ka.seq_lens = seq_lens;
    ka.chunk_offs = offs;
    ka.dh = dh;
    ka.dinit = dinit;
    ka.dvals = dvals;
    ka.status = status;
    ka.H = s.n_heads;
    ka.dv = s.dv;
    const int64_t blocks = (int64_t)s.n_seqs * s.n_heads * (s.dv / kKdaBwdRows);
    auto go = [&](auto kern, size_t lds) {
      hipError_t e2 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e2 != hipSuccess) return e2;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), lds, stream, ka);
      return hipGetLastError();
    };
    return s.dk == 128 ? go(kda_bwd_token_kernel<128>, KdaBwdLds<128>::bytes)
                       : go(kda_bwd_token_kernel<64>, KdaBwdLds<64>::bytes);
  }
  PrepArgs pa{};
  pa.q = q; pa.k = k; pa.beta = beta; pa.g = g; pa.cu_seqlens = cu_seqlens; pa.seq_lens = seq_lens;
  pa.prefix_lens = nullptr; pa.offs = offs; pa.T = TT; pa.P = PT; pa.N = s.n_seqs; pa.H = s.n_heads;
  pa.status = status;
  BwdArgs ba{};
  ba.q = reinterpret_cast<const uint16_t*>(q);
  ba.k = reinterpret_cast<const uint16_t*>(k);
  ba.g = g;
  ba.dout = reinterpret_cast<const uint16_t*>(dout);
  ba.dfin = dfin;
  ba.cu_seqlens = cu_seqlens;
  ba.seq_lens = seq_lens;
  ba.chunk_offs = offs;
  ba.TT = TT;
  ba.PT = PT;
  ba.dh = dh;
  ba.dinit = dinit;
  ba.dvals = dvals;
  ba.status = status;
  ba.W = reinterpret_cast<const char*>(L.W);
  ba.H = s.n_heads;
  ba.dv = s.dv;
  if (wq) return s.dk == 128 ? launch_bwd_dk<128, true>(s, pa, ba, items, stream)
                             : launch_bwd_dk<64, true>(s, pa, ba, items, stream);
  return s.dk == 128 ? launch_bwd_dk<128, false>(s, pa, ba, items, stream)
                     : launch_bwd_dk<64, false>(s, pa, ba, items, stream);
}

}  // namespace gdn
