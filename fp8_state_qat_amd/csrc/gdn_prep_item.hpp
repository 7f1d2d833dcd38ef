// gdn_prep_item.hpp -- the state-independent work of one (chunk, head) of the
// chunked gated delta rule (Model-Optimizer #2497: WY/UT-transformed
// operands of a 64-token chunk; #2506: the exact triangular solve), as device
// functions shared by the standalone prep kernels (gdn_prep.hip) and the
// fused launch of the sequential kernel (gdn_chunk.hip), where some
// workgroups produce these records while the others consume them.
//
// Per chunk of n <= 64 tokens (rows past n are zero):
//     gamma_r = sum_{s<=r} g_s                                (in-chunk scan)
//     A[r][s] = beta_r exp(gamma_r - gamma_s) k_r . k_s       (s < r)
//     T       = (I + A)^-1 diag(beta)                         (exact solve)
//     P[t][s] = exp(gamma_t - gamma_s) q_t . k_s              (s <= t)
// T and P go to the workspace as records in MFMA fragment order (layout at
// the top of gdn_prep.hip).  With W QDQ (#2497: independent dynamic FP8 QDQ
// of the WY-transformed W, one scale per token and head) also
//     W       = T (K * exp(gamma)),   W <- RNE_E4M3(W / s_r) s_r per row r,
//     s_r     = max_c |W[r][c]| / 448 (1 when that is not positive)
// as a third record (codes and row scales, layout in gdn_launch.hpp).
#pragma once

#include <type_traits>

#include "gdn_chunk_common.hpp"

namespace gdn {

struct PrepArgs {
  const void* q;
  const void* k;
  const float* beta;
  const float* g;
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* prefix_lens;
  const int32_t* offs;
  void* T;        // one record of kTRecBytes per (chunk, head)
  void* P;        // one P record per (chunk, head)
  void* W;        // W QDQ: one W record (w_rec_bytes(dk)) per (chunk, head)
  float* w_pre;   // optional debug record of W before / after its QDQ,
  float* w_post;  // [chunk, head, 64, dk]
  const int32_t* status;  // the workspace's status word (index check), or null
  int N;
  int H;
};

// Row stride (floats) of the 64 x 64 fp32 LDS matrices of the prep kernels.
constexpr int kL64 = 64 + 4;

// X = (I + A)^-1 for the strictly lower A in sA (only the block-lower 16 x 16
// blocks are read), on the four waves whose item thread index is tid
// (0..255).  sX receives X row-major (block-lower part; the diagonal blocks
// carry zeros above their diagonal).  Contains workgroup barriers; with
// active false the waves only take part in them.
//   diagonal blocks: forward substitution, wave 0, one lane per (block, column)
//   X_ij (i > j), level by level (i - j = 1, 2, 3), one wave per block:
//       X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj
//   on the fp32 MFMA (16x16x4).  Instruction q of a 16-deep product takes
//   k = 4 (l / 16) + q from lane l, so the accumulator of the sum (lane l
//   holds rows 4 (l / 16) .. + 3 of column l % 16) is the B operand of the
//   product with X_ii as it stands.
__device__ __forceinline__ void solve_unit_lower(const float* sA, float* sX, int tid, bool active = true) {
  constexpr int L64 = kL64;
  const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  if (active && w == 0) {
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
    if (active && w + d < 4) {
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
// when colscale is not null, as one record in MFMA fragment order, on the
// four waves whose item thread index is tid (0..255).
template <bool kBF, int kPl = 2>
__device__ __forceinline__ void store_record(const float* M, const float* colscale, char* rec, int tid) {
  static_assert(kPl == 2 || kPl == 3, "two or three bf16 planes");
  constexpr int L64 = kL64;
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
      uint32_t hv[4], mv[4], lv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kPl == 3) {
          split3_bf16x2(t8[2 * q], t8[2 * q + 1], hv[q], mv[q], lv[q]);
        } else {
          split_bf16x2(t8[2 * q], t8[2 * q + 1], hv[q], mv[q]);
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(rec);
      dst[p * 64 + l] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      dst[(6 + p) * 64 + l] = make_uint4(mv[0], mv[1], mv[2], mv[3]);
      if constexpr (kPl == 3) dst[(12 + p) * 64 + l] = make_uint4(lv[0], lv[1], lv[2], lv[3]);
    } else {
      float4* dst = reinterpret_cast<float4*>(rec) + 2 * (p * 64 + l);
      dst[0] = make_float4(t8[0], t8[1], t8[2], t8[3]);
      dst[1] = make_float4(t8[4], t8[5], t8[6], t8[7]);
    }
  }
}

// The W record of chunk j, head h from W in accumulator layout (wave w of
// the item holds rows 16w + 4gq + i, i = 0..3, at columns 16ct + ln): a
// scale per row (amax over the row's dk columns, one 16-lane row across the
// dk/16 tiles, by DPP), the codes by the exact quotient and the hardware
// E4M3 conversion, then codes and scales staged in LDS (stage: 64 x dk bf16,
// ssc: 64 floats, both free once every wave is past the first barrier here)
// and stored as the record; the optional debug record too.  Contains two
// workgroup barriers; with active false the waves only take part in them.
template <int DK>
__device__ __forceinline__ void store_w_record(const PrepArgs& a, int j, int h, const f32x4 (&wacc)[DK / 16],
                                               uint16_t* stage, float* ssc, int tid, bool active) {
  constexpr int NT = DK / 16, NKB = DK / 32;
  const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  const int H = a.H;
  float sc[4], rc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = 0.f;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) m = fmaxf(m, fabsf(wacc[ct][i]));
    sc[i] = qdq_scale(row16_max_dpp(m));
    rc[i] = 1.0f / sc[i];
  }
  float cw[NT][4];
#pragma unroll
  for (int ct = 0; ct < NT; ct += 2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = __builtin_amdgcn_cvt_pk_fp8_f32(div_rn(wacc[ct][i], sc[i], rc[i]),
                                                    div_rn(wacc[ct + 1][i], sc[i], rc[i]), 0, false);
      cw[ct][i] = __builtin_amdgcn_cvt_f32_fp8(p, 0);
      cw[ct + 1][i] = __builtin_amdgcn_cvt_f32_fp8(p, 1);
    }
  if (active && (a.w_pre != nullptr || a.w_post != nullptr)) {
    const int64_t base = ((int64_t)j * H + h) * 64 * DK;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (16 * w + 4 * gq + i) * DK + 16 * ct + ln;
        if (a.w_pre) a.w_pre[base + e] = wacc[ct][i];
        if (a.w_post) a.w_post[base + e] = cw[ct][i] * sc[i];
      }
  }
  __syncthreads();  // every wave is done with the operands of W
  if (active) {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) stage[(16 * w + 4 * gq + i) * DK + 16 * ct + ln] = float_to_bf16_bits(cw[ct][i]);
    if (ln == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ssc[16 * w + 4 * gq + i] = sc[i];
    }
  }
  __syncthreads();
  if (active) {
    char* wrec = reinterpret_cast<char*>(a.W) + ((int64_t)j * H + h) * w_rec_bytes(DK);
    constexpr int NF = 4 * NKB;  // fragments: f = tt * NKB + kb
    for (int slot = tid; slot < NF * 64; slot += kThreads) {
      const int f = slot >> 6, l = slot & 63;
      const int r = 16 * (f / NKB) + (l & 15), c0 = 32 * (f % NKB) + 8 * (l >> 4);
      *reinterpret_cast<uint4*>(wrec + slot * 16) = *reinterpret_cast<const uint4*>(stage + r * DK + c0);
    }
    if (tid < 64) reinterpret_cast<float*>(wrec + NF * 1024)[tid] = ssc[tid];
  }
}

// LDS of one scalar-gate item (bytes): k and q rows unpadded, 16-byte pieces
// XOR-swizzled by row (piece p of row r at slot p ^ (r % PPR)), so that
// direct loads fill them 1 KiB at a time and the fragment reads of 16 rows at
// one column hit different banks; once A and P are formed the solve's X
// overlays them (with W QDQ, whose product still reads K, X has a block of
// its own at the end).  Then A, the scaled log-gates and beta.
template <int DK, typename TIO, bool kW = false>
struct PrepItemLds {
  static constexpr int RB = DK * (int)sizeof(TIO);  // bytes per k or q row
  static constexpr int PPR = RB / 16;               // pieces per row
  static constexpr int KQ = 2 * 64 * RB;
  static constexpr int KX = (KQ > 64 * kL64 * 4 || kW) ? KQ : 64 * kL64 * 4;
  static constexpr int oA = KX;
  static constexpr int oG2 = oA + 64 * kL64 * 4;
  static constexpr int oBeta = oG2 + 64 * 4;
  static constexpr int oX = kW ? oBeta + 64 * 4 : 0;
  static constexpr int bytes = oBeta + 64 * 4 + (kW ? 64 * kL64 * 4 : 0);
  static_assert(bytes % 16 == 0, "item LDS blocks stay 16-byte aligned");
  static_assert(!kW || 64 * DK * 2 <= 64 * RB, "W codes are staged over the k rows");
};

// The records of chunk j (tokens t0 .. t0 + nv - 1 of the packed inputs), head
// h, on four waves (item thread index tid = 0..255) with the LDS block lds
// (PrepItemLds bytes, 16-byte aligned).  Contains workgroup barriers; with
// active false the waves only take part in them.  On return this wave's
// record stores may still be in flight.
template <int DK, typename TIO, bool kW = false>
__device__ __forceinline__ void prep_item(const PrepArgs& a, int j, int h, int t0, int nv, char* lds,
                                          int tid, bool active) {
  using IL = PrepItemLds<DK, TIO, kW>;
  constexpr bool kBF = sizeof(TIO) == 2;
  constexpr int L64 = kL64;
  constexpr int NKB = DK / 32;
  constexpr int RB = IL::RB, PPR = IL::PPR;
  const char* sK = lds;
  const char* sQ = lds + 64 * RB;
  float* sX = reinterpret_cast<float*>(lds + IL::oX);
  float* sA = reinterpret_cast<float*>(lds + IL::oA);
  float* sG2 = reinterpret_cast<float*>(lds + IL::oG2);
  float* sBeta = reinterpret_cast<float*>(lds + IL::oBeta);
  // byte address of element c of row r in the k or q block
  auto kq_at = [](int r, int c) {
    const int p = c * (int)sizeof(TIO) / 16, within = c * (int)sizeof(TIO) % 16;
    return r * RB + ((p ^ (r & (PPR - 1))) * 16) + within;
  };
  const int H = a.H;
  const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;

  // ---- stage K and Q by direct loads (rows past nv repeat the last valid row:
  // beta is zero there, which zeroes those rows of A and columns of T, and P
  // rows past nv only reach outputs that are not stored), gates
  if (active) {
    const uint32_t lds0 = lds_base_u32(lds);
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
      sG2[lane] = gv * kLog2e;
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
  // ---- six strip jobs, one per record pair p = (ri, kb) in the record order
  // (0,0) (1,0) (2,0) (3,0) (2,1) (3,1): the tiles si = 2kb and 2kb + 1 of row
  // block ri (a tile with si > ri is zero).  With C_A = K K^T and C_P = K Q^T
  // on a tile (one shared A operand, the k rows of block si)
  //   A[r][s] = beta_r exp(gamma_r - gamma_s) C_A[s][r]    (s < r)   -> sA
  //   P[r][s] = exp(gamma_r - gamma_s) C_P[s][r]           (s <= r)  -> the P record
  // A lane holds P[r][s] for one row r and the four s of each tile that its
  // record slot takes (k-slots kperm(l / 16, 0..3) and 4..7), so it writes
  // whole 16-byte slots and every store instruction whole cache lines.
  // Waves: 0 takes pairs 0 and 5, 1 pairs 1 and 4, 2 pair 2, 3 pair 3 (three
  // nonzero tiles at most per wave).
  char* prec = reinterpret_cast<char*>(a.P) + ((int64_t)j * H + h) * kPRecBytes;
  if (active) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int pr = (jj == 0) ? w : (w == 0 ? 5 : w == 1 ? 4 : -1);
      if (pr >= 0) {
        const int ri = pr < 4 ? pr : pr - 2, kb = pr < 4 ? 0 : 1;
        const int r = 16 * ri + ln;
        const float g2r = sG2[r], br = sBeta[r];
        float vp8[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int si = 2 * kb + hh;
          if (si <= ri) {
            const f32x4 ca = tile(sK, 16 * si + ln, sK, r);
            const f32x4 cp = tile(sK, 16 * si + ln, sQ, r);
            float va[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int s = 16 * si + 4 * gq + i;
              const float e = (s <= r) ? __builtin_amdgcn_exp2f(g2r - sG2[s]) : 0.f;
              va[i] = (s < r) ? br * e * ca[i] : 0.f;
              vp8[4 * hh + i] = e * cp[i];
            }
            *reinterpret_cast<float4*>(sA + r * L64 + 16 * si + 4 * gq) = make_float4(va[0], va[1], va[2], va[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) vp8[4 * hh + i] = 0.f;
          }
        }
        if constexpr (kBF) {
          uint32_t hv[4], lv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) split_bf16x2(vp8[2 * q], vp8[2 * q + 1], hv[q], lv[q]);
          *reinterpret_cast<uint4*>(prec + (pr * 64 + lane) * 16) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
          *reinterpret_cast<uint4*>(prec + ((6 + pr) * 64 + lane) * 16) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
        } else {
          float4* dst = reinterpret_cast<float4*>(prec + (pr * 64 + lane) * 32);
          dst[0] = make_float4(vp8[0], vp8[1], vp8[2], vp8[3]);
          dst[1] = make_float4(vp8[4], vp8[5], vp8[6], vp8[7]);
        }
      }
    }
  }
  __syncthreads();

  solve_unit_lower(sA, sX, tid, active);
  if (active) store_record<kBF, 3>(sX, sBeta, reinterpret_cast<char*>(a.T) + ((int64_t)j * H + h) * kTRecBytes, tid);

  if constexpr (kW) {
    // ---- W = X diag(beta exp(gamma)) K on the MFMA: wave w forms rows
    // 16w .. 16w + 15 (lane holds W[16w + 4gq + i][16ct + ln]), so every row
    // lies in one wave.  A = X' rows (k = tokens s, only the block-lower
    // part: s / 16 <= w), B = K with k = tokens (bf16: two transpose reads
    // per fragment; fp32: one read per element).
    constexpr int NT = DK / 16;
    f32x4 wacc[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) wacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
      const int wr = 16 * w + ln;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb > w) break;  // wave-uniform: the block-upper part of X is zero
        float xa[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int s = 32 * kb + (jj < 4 ? 4 * gq + jj : 16 + 4 * gq + (jj - 4));
          xa[jj] = ((s >> 4) <= w) ? sX[wr * L64 + s] * sBeta[s] * __builtin_amdgcn_exp2f(sG2[s]) : 0.f;
        }
        if constexpr (kBF) {
          // X' as three bf16 planes (24 significant bits): W keeps fp32
          // accuracy, so its codes differ from the oracle's only at midpoints
          uint32_t hv[4], mv[4], lv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) split3_bf16x2(xa[2 * q], xa[2 * q + 1], hv[q], mv[q], lv[q]);
          const bf16x8 ah = __builtin_bit_cast(bf16x8, make_uint4(hv[0], hv[1], hv[2], hv[3]));
          const bf16x8 am = __builtin_bit_cast(bf16x8, make_uint4(mv[0], mv[1], mv[2], mv[3]));
          const bf16x8 al = __builtin_bit_cast(bf16x8, make_uint4(lv[0], lv[1], lv[2], lv[3]));
          // lane 4kk + qq of a 16-lane group points at K[s0 + kk][16ct + 4qq .. + 3], so
          // lane ln receives K[s0 + 0..3][16ct + ln]
          const int kk = ln >> 2, qq = ln & 3;
          const int s0 = 32 * kb + 4 * gq, s1 = s0 + 16;
          bf16x8 bfr[NT];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const uint2 b0 = lds_read_tr16(sK + kq_at(s0 + kk, 16 * ct + 4 * qq));
            const uint2 b1 = lds_read_tr16(sK + kq_at(s1 + kk, 16 * ct + 4 * qq));
            bfr[ct] = __builtin_bit_cast(bf16x8, make_uint4(b0.x, b0.y, b1.x, b1.y));
          }
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            mma_bf16(wacc[ct], ah, bfr[ct]);
            mma_bf16(wacc[ct], am, bfr[ct]);
            mma_bf16(wacc[ct], al, bfr[ct]);
          }
        } else {
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            float bv[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int s = 32 * kb + (jj < 4 ? 4 * gq + jj : 16 + 4 * gq + (jj - 4));
              bv[jj] = *reinterpret_cast<const float*>(sK + kq_at(s, 16 * ct + ln));
            }
            mma_f32(wacc[ct], xa, bv);
          }
        }
      }
    }
    store_w_record<DK>(a, j, h, wacc, reinterpret_cast<uint16_t*>(lds), reinterpret_cast<float*>(lds + 64 * RB),
                       tid, active);
  }
}

// ---------------------------------------------------------------------------
// Backward records.  The reverse state recurrence needs T^T and P^T as the A
// operand; both are block-upper, so they are stored as full 64 x 64 records:
// pair p = 2 ti + kb (ti = 0..3, kb = 0..1), lane l of fragment p holds
// M[16 ti + l % 16][32 kb + kperm(l / 16, j)], j = 0..7, bf16 hi plane (8
// fragments) then lo plane.
constexpr int kBRecBytes = 16384;

// M^T of the 64 x 64 matrix src (row-major, stride kL64; only its
// block-lower 16 x 16 blocks are read, the others count as zero), times
// diag(colscale) of src when colscale is not null, as a backward record, on
// four waves (item thread index tid).
__device__ __forceinline__ void store_record_t(const float* src, const float* colscale, char* rec, int tid) {
  constexpr int L64 = kL64;
  for (int slot = tid; slot < 8 * 64; slot += kThreads) {
    const int p = slot >> 6, l = slot & 63, gq = l >> 4;
    const int ti = p >> 1, kb = p & 1;
    const int m = 16 * ti + (l & 15);  // row of M = column of src
    const float cs = colscale ? colscale[m] : 1.0f;
    float t8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 32 * kb + (j < 4 ? 4 * gq + j : 16 + 4 * gq + (j - 4));  // column of M = row of src
      t8[j] = ((k >> 4) >= (m >> 4)) ? src[k * L64 + m] * cs : 0.f;
    }
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split_bf16x2(t8[2 * q], t8[2 * q + 1], hv[q], lv[q]);
    uint4* dst = reinterpret_cast<uint4*>(rec);
    dst[p * 64 + l] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    dst[(8 + p) * 64 + l] = make_uint4(lv[0], lv[1], lv[2], lv[3]);
  }
}

// LDS of one backward item: k and q rows as in PrepItemLds (the solve's X
// overlays them), A and P (64 x kL64 fp32 each), the scaled log-gates, beta.
template <int DK>
struct PrepBwdLds {
  static constexpr int RB = DK * 2;
  static constexpr int PPR = RB / 16;
  static constexpr int KQ = 2 * 64 * RB;
  static constexpr int KX = (KQ > 64 * kL64 * 4) ? KQ : 64 * kL64 * 4;
  static constexpr int oA = KX;
  static constexpr int oP = oA + 64 * kL64 * 4;
  static constexpr int oG2 = oP + 64 * kL64 * 4;
  static constexpr int oBeta = oG2 + 64 * 4;
  static constexpr int bytes = oBeta + 64 * 4;
};

// The backward records of chunk j (tokens t0 .. t0 + nv - 1), head h (bf16
// inputs): T^T with T = (I + A)^-1 diag(beta) into a.T, P^T into a.P (the
// rows of P past nv, i.e. the columns of P^T, zero).
// Four waves (item thread index tid), LDS block lds of PrepBwdLds bytes.
// Contains workgroup barriers.  On return this wave's record stores may
// still be in flight.
template <int DK>
__device__ __forceinline__ void prep_item_bwd(const PrepArgs& a, int j, int h, int t0, int nv, char* lds, int tid) {
  using IL = PrepBwdLds<DK>;
  constexpr int L64 = kL64, NKB = DK / 32, RB = IL::RB, PPR = IL::PPR;
  const char* sK = lds;
  const char* sQ = lds + 64 * RB;
  float* sX = reinterpret_cast<float*>(lds);
  float* sA = reinterpret_cast<float*>(lds + IL::oA);
  float* sP = reinterpret_cast<float*>(lds + IL::oP);
  float* sG2 = reinterpret_cast<float*>(lds + IL::oG2);
  float* sBeta = reinterpret_cast<float*>(lds + IL::oBeta);
  auto kq_at = [](int r, int c) {
    const int p = c * 2 / 16, within = c * 2 % 16;
    return r * RB + ((p ^ (r & (PPR - 1))) * 16) + within;
  };
  const int H = a.H;
  const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  {
    const uint32_t lds0 = lds_base_u32(lds);
    const uint16_t* gk = reinterpret_cast<const uint16_t*>(a.k) + ((int64_t)t0 * H + h) * DK;
    const uint16_t* gqv = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)t0 * H + h) * DK;
    constexpr int NI = 64 * RB / 1024;
#pragma unroll
    for (int ii = 0; ii < NI / 4; ++ii) {
      const int i = uniform(w) + 4 * ii;
      const int u = i * 64 + lane, r = u / PPR, p = (u % PPR) ^ (r & (PPR - 1));
      const uint32_t off = (uint32_t)((min(r, nv - 1) * H * DK) * 2 + p * 16);
      lds_load16(gk, off, lds0 + i * 1024);
      lds_load16(gqv, off, lds0 + 64 * RB + i * 1024);
    }
    if (w == 0) {
      float gv = 0.f, bv = 0.f;
      if (lane < nv) {
        gv = a.g[(int64_t)(t0 + lane) * H + h];
        bv = a.beta[(int64_t)(t0 + lane) * H + h];
      }
      sG2[lane] = wave_prefix_sum(gv) * kLog2e;
      sBeta[lane] = bv;
    }
    wait_vmem();
  }
  __syncthreads();
  // the ten tiles (R, S), S <= R: C[s][r] = x_s . y_r, lane holds s = 16S + 4gq + i, r = 16R + ln
  for (int job = w; job < 10; job += 4) {
    const int R = (job < 1) ? 0 : (job < 3) ? 1 : (job < 6) ? 2 : 3;
    const int S = job - (R * (R + 1)) / 2;
    const int r = 16 * R + ln, sr = 16 * S + ln;
    f32x4 ca = {0.f, 0.f, 0.f, 0.f}, cp = {0.f, 0.f, 0.f, 0.f};
    bf16x8 af[NKB], bk[NKB], bq[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint2 a0 = *reinterpret_cast<const uint2*>(sK + kq_at(sr, 32 * kb + 4 * gq));
      const uint2 a1 = *reinterpret_cast<const uint2*>(sK + kq_at(sr, 32 * kb + 16 + 4 * gq));
      const uint2 k0 = *reinterpret_cast<const uint2*>(sK + kq_at(r, 32 * kb + 4 * gq));
      const uint2 k1 = *reinterpret_cast<const uint2*>(sK + kq_at(r, 32 * kb + 16 + 4 * gq));
      const uint2 q0 = *reinterpret_cast<const uint2*>(sQ + kq_at(r, 32 * kb + 4 * gq));
      const uint2 q1 = *reinterpret_cast<const uint2*>(sQ + kq_at(r, 32 * kb + 16 + 4 * gq));
      af[kb] = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
      bk[kb] = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
      bq[kb] = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      mma_bf16(ca, af[kb], bk[kb]);
      mma_bf16(cp, af[kb], bq[kb]);
    }
    const float g2r = sG2[r], br = sBeta[r];
    float va[4], vp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 16 * S + 4 * gq + i;
      const float e = (s <= r) ? __builtin_amdgcn_exp2f(g2r - sG2[s]) : 0.f;
      va[i] = (s < r) ? br * e * ca[i] : 0.f;
      vp[i] = (r < nv) ? e * cp[i] : 0.f;  // rows past the chunk's end are zero
    }
    *reinterpret_cast<float4*>(sA + r * L64 + 16 * S + 4 * gq) = make_float4(va[0], va[1], va[2], va[3]);
    *reinterpret_cast<float4*>(sP + r * L64 + 16 * S + 4 * gq) = make_float4(vp[0], vp[1], vp[2], vp[3]);
  }
  __syncthreads();
  store_record_t(sP, nullptr, reinterpret_cast<char*>(a.P) + ((int64_t)j * H + h) * kBRecBytes, tid);
  solve_unit_lower(sA, sX, tid);
  store_record_t(sX, sBeta, reinterpret_cast<char*>(a.T) + ((int64_t)j * H + h) * kBRecBytes, tid);
}

template <int DK, typename TIO, bool kW = false>
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
  // once A and P are formed, the solve's X overlays k and q (with W QDQ,
  // whose product still reads k and the gates, X has a block of its own)
  static constexpr size_t oX = kW ? oBeta + 64 * sizeof(float) : oK;
  static constexpr size_t bytes = oBeta + 64 * sizeof(float) + (kW ? 64 * kL64 * sizeof(float) : 0);
  static_assert(64 * kL64 * sizeof(float) <= oG - oK, "X does not fit over k and q");
  static_assert(64 * DK * 2 <= oQ - oK && 64 * sizeof(float) <= oG - oQ, "W staging over k and q");
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

// A thread's share of one per-key-channel prep item's inputs, loaded from
// HBM into registers: 16-byte pieces of k and q rows (rows past nv zero),
// the gates of one channel over TPP consecutive tokens, one beta.
template <int DK, typename TIO>
struct KdaRaw {
  static constexpr int EPS = 16 / (int)sizeof(TIO);
  static constexpr int SPR = DK / EPS;                    // 16-byte pieces per row
  static constexpr int NJ = 64 * SPR / kThreads;          // pieces per thread
  static constexpr int NPART = kThreads / DK, TPP = 64 / NPART;  // token parts of the per-channel scan
  static_assert(64 * SPR % kThreads == 0, "staging geometry");
  uint4 kv[NJ], qv[NJ];
  float gv[TPP];
  float beta;
};
template <int DK, typename TIO>
__device__ __forceinline__ void kda_fetch(const PrepArgs& a, int h, int t0, int nv, int tid, KdaRaw<DK, TIO>& x) {
  using Raw = KdaRaw<DK, TIO>;
  const int H = a.H;
  const TIO* gk = reinterpret_cast<const TIO*>(a.k);
  const TIO* gqv = reinterpret_cast<const TIO*>(a.q);
#pragma unroll
  for (int jj = 0; jj < Raw::NJ; ++jj) {
    const int seg = tid + kThreads * jj;
    const int r = seg / Raw::SPR, c0 = (seg % Raw::SPR) * Raw::EPS;
    x.kv[jj] = make_uint4(0u, 0u, 0u, 0u);
    x.qv[jj] = make_uint4(0u, 0u, 0u, 0u);
    if (r < nv) {
      const int64_t off = ((int64_t)(t0 + r) * H + h) * DK + c0;
      x.kv[jj] = *reinterpret_cast<const uint4*>(gk + off);
      x.qv[jj] = *reinterpret_cast<const uint4*>(gqv + off);
    }
  }
  x.beta = (tid < nv) ? a.beta[(int64_t)(t0 + tid) * H + h] : 0.f;  // used by tid < 64
  const int d = tid % DK, part = tid / DK;
#pragma unroll
  for (int i = 0; i < Raw::TPP; ++i) {
    const int r = part * Raw::TPP + i;
    x.gv[i] = (r < nv) ? a.g[((int64_t)(t0 + r) * H + h) * DK + d] : 0.f;
  }
}

// The records of chunk j (tokens t0 .. t0 + nv - 1), head h, for a
// per-key-channel gate, on one workgroup of four waves (thread index tid)
// with the LDS block smem (KdaPrepLds bytes), from the inputs x that
// kda_fetch loaded.  Once x is staged in LDS, next() runs (a caller may load
// its next item into x there, so that those loads land during this item).
// Contains workgroup barriers.  On return this wave's record stores (and
// whatever next() issued) may still be in flight.
template <int DK, typename TIO, bool kW, typename Next>
__device__ __forceinline__ void kda_prep_item_from(const PrepArgs& a, int j, int h, int nv, char* smem, int tid,
                                                   KdaRaw<DK, TIO>& x, Next&& next) {
  using Ls = KdaPrepLds<DK, TIO, kW>;
  constexpr bool kBF = sizeof(TIO) == 2;
  constexpr int LX = Ls::LX, LG = Ls::LG, L64 = kL64, NKB = DK / 32;
  TIO* sK = reinterpret_cast<TIO*>(smem + Ls::oK);
  TIO* sQ = reinterpret_cast<TIO*>(smem + Ls::oQ);
  float* sG = reinterpret_cast<float*>(smem + Ls::oG);    // gamma * log2(e)
  float* sA = reinterpret_cast<float*>(smem + Ls::oA);
  float* sP = reinterpret_cast<float*>(smem + Ls::oP);
  float* sTot = reinterpret_cast<float*>(smem + Ls::oTot);
  float* sBeta = reinterpret_cast<float*>(smem + Ls::oBeta);
  float* sX = reinterpret_cast<float*>(smem + Ls::oX);

  const int H = a.H;
  const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;

  // ---- stage k and q (rows past nv are zero), beta, and the per-channel gate prefix
  using Raw = KdaRaw<DK, TIO>;
  constexpr int TPP = Raw::TPP;
  {
#pragma unroll
    for (int jj = 0; jj < Raw::NJ; ++jj) {
      const int seg = tid + kThreads * jj;
      const int r = seg / Raw::SPR, c0 = (seg % Raw::SPR) * Raw::EPS;
      *reinterpret_cast<uint4*>(sK + r * LX + c0) = x.kv[jj];
      *reinterpret_cast<uint4*>(sQ + r * LX + c0) = x.qv[jj];
    }
    if (tid < 64) sBeta[tid] = x.beta;
  }
  {
    const int d = tid % DK, part = tid / DK;
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      run += x.gv[i];
      sG[(part * TPP + i) * LG + d] = run;
    }
    sTot[tid] = run;
  }
  next();  // x is free
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
    // The LDS operands of k-block kb + 1 are read while block kb computes
    // (two buffers), so that the reads' round trip is not spent between the
    // blocks.
    using Raw4 = typename std::conditional<sizeof(TIO) == 2, uint2, float4>::type;
    struct KbIn {
      float4 gs[2], gm[2], gr[2];
      Raw4 ks[2], kr[2], qr[2];
    };
    auto load_kb = [&](const int kb, KbIn& in) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c0 = 32 * kb + 16 * hh + 4 * gq;  // channels kperm(gq, 4 hh .. 4 hh + 3)
        in.gs[hh] = *reinterpret_cast<const float4*>(sG + s * LG + c0);
        in.gm[hh] = *reinterpret_cast<const float4*>(sG + m * LG + c0);
        in.gr[hh] = *reinterpret_cast<const float4*>(sG + r * LG + c0);
        in.ks[hh] = *reinterpret_cast<const Raw4*>(sK + s * LX + c0);
        in.kr[hh] = *reinterpret_cast<const Raw4*>(sK + r * LX + c0);
        in.qr[hh] = *reinterpret_cast<const Raw4*>(sQ + r * LX + c0);
      }
    };
    auto unpack4 = [](const Raw4& u, float (&x)[4]) {
      if constexpr (sizeof(TIO) == 2) {
        x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
      } else {
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
      }
    };
    KbIn kin[2];
    load_kb(0, kin[0]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb + 1 < NKB) load_kb(kb + 1, kin[(kb + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // those reads are issued before this block's arithmetic
      const KbIn& in = kin[kb & 1];
      float av[8], bk[8], bq[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float gs[4] = {in.gs[hh].x, in.gs[hh].y, in.gs[hh].z, in.gs[hh].w};
        const float gm[4] = {in.gm[hh].x, in.gm[hh].y, in.gm[hh].z, in.gm[hh].w};
        const float gr[4] = {in.gr[hh].x, in.gr[hh].y, in.gr[hh].z, in.gr[hh].w};
        float ks[4], kr[4], qr[4];
        unpack4(in.ks[hh], ks);
        unpack4(in.kr[hh], kr);
        unpack4(in.qr[hh], qr);
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

  store_record<kBF>(sP, nullptr, reinterpret_cast<char*>(a.P) + ((int64_t)j * H + h) * kPRecBytes, tid);
  solve_unit_lower(sA, sX, tid);
  store_record<kBF, 3>(sX, sBeta, reinterpret_cast<char*>(a.T) + ((int64_t)j * H + h) * kTRecBytes, tid);

  if constexpr (kW) {
    // ---- W = X diag(beta) (K o exp(gamma)) on the fp32 MFMA (the second
    // operand is not exact in bf16): wave w forms rows 16w .. 16w + 15, A =
    // X' rows (k = tokens s, block-lower part only), B[s][c] =
    // k[s][c] exp(gamma[s][c]), read element by element.
    constexpr int NT = DK / 16;
    f32x4 wacc[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) wacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wr = 16 * w + ln;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (2 * kb > w) break;  // wave-uniform: the block-upper part of X is zero
      float xa[8];
      int sj[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        sj[jj] = 32 * kb + (jj < 4 ? 4 * gq + jj : 16 + 4 * gq + (jj - 4));
        xa[jj] = ((sj[jj] >> 4) <= w) ? sX[wr * L64 + sj[jj]] * sBeta[sj[jj]] : 0.f;
      }
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        float bv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int c = 16 * ct + ln;
          bv[jj] = io<TIO>::ld(sK + sj[jj] * LX + c) * __builtin_amdgcn_exp2f(sG[sj[jj] * LG + c]);
        }
        mma_f32(wacc[ct], xa, bv);
      }
    }
    store_w_record<DK>(a, j, h, wacc, reinterpret_cast<uint16_t*>(smem + Ls::oK),
                       reinterpret_cast<float*>(smem + Ls::oQ), tid, true);
  }
}

// One item from HBM to its records (kda_fetch, then kda_prep_item_from).
template <int DK, typename TIO, bool kW = false>
__device__ __forceinline__ void kda_prep_item(const PrepArgs& a, int j, int h, int t0, int nv, char* smem,
                                              int tid) {
  KdaRaw<DK, TIO> x;
  kda_fetch<DK, TIO>(a, h, t0, nv, tid, x);
  kda_prep_item_from<DK, TIO, kW>(a, j, h, nv, smem, tid, x, [] {});
}

// Fused launch, workgroups 0 .. n_prep - 1: the T and P records of every
// (chunk, head), two at a time (waves 0..3 and waves 4..7 each take one item).
// Producer p serves the (sequence, head) pairs nh with nh % 8 == p % 8, in
// chunk-major order: the R = n_prep / 8 producers of a class take its items
// m = r, r + R, r + 2R, ... (r = p / 8), item m being chunk m / M of the
// class's (m % M)-th pair, M the pairs in the class.  n_prep is a multiple
// of 8 and the state part maps nh to blocks on XCD nh % 8, so producer and
// consumers of a record share one L2: the record stores complete in that L2
// (every wave waits for its stores, then the workgroup barrier), then the
// flag is stored at device scope, past the L1.  A producer that finds itself
// off its XCD writes its L2 back first and says so in the flag, and a
// consumer on another XCD then invalidates its caches before reading
// (device-scope release and acquire).  Producers never wait, so the
// consumers' waits end once every producer has been dispatched; producers
// have the lower workgroup ids.
template <int DK, typename TIO, bool kW>
__device__ __forceinline__ void produce_records(const ChunkArgs& args, char* smem) {
  using IL = PrepItemLds<DK, TIO, kW>;
  const int half = uniform((int)threadIdx.x >> 8), tid = threadIdx.x & 255;  // half: wave-uniform
  char* lds = smem + half * IL::bytes;
  PrepArgs a;
  a.q = args.q; a.k = args.k; a.beta = args.beta; a.g = args.g; a.cu_seqlens = args.cu_seqlens;
  a.seq_lens = args.seq_lens; a.prefix_lens = args.prefix_lens; a.offs = args.chunk_offs;
  a.T = const_cast<void*>(args.T); a.P = const_cast<void*>(args.Prec); a.N = args.N; a.H = args.H;
  a.W = const_cast<void*>(args.Wrec); a.w_pre = args.w_pre; a.w_post = args.w_post;
  a.status = args.status;
  const int H = args.H, NH = args.N * args.H;
  const int p = blockIdx.x, x = p & 7, r = p >> 3, R = args.n_prep >> 3;
  const unsigned xcd = xcd_id();
  const bool home = xcd == (unsigned)x;
  const int M = NH > x ? (NH - x + 7) >> 3 : 0;
  const int c0 = args.prep_c0;
  const int64_t total = (int64_t)max(args.chunk_offs[args.N + 1] - c0, 0) * M;
  for (int64_t m0 = r; m0 < total; m0 += 2 * R) {
    const int64_t m = m0 + (int64_t)half * R;
    bool active = m < total;
    int j = 0, h = 0, t0 = 0, nv = 0;
    if (active) {
      const int c = c0 + (int)(m / M), nh = x + 8 * (int)(m % M);
      const int n = nh / H;
      h = nh % H;
      const int seg0 = args.cu_seqlens[n];
      const int L = args.seq_lens ? args.seq_lens[n] : (args.cu_seqlens[n + 1] - seg0);
      const int P = args.prefix_lens ? args.prefix_lens[n] : L;
      active = c * kChunk < P;
      if (active) {
        j = args.chunk_offs[n] + c;
        t0 = seg0 + c * kChunk;
        nv = min(kChunk, P - c * kChunk);
      }
    }
    // a fresh copy of the lane index per item keeps the compiler from holding
    // the item's lane-dependent LDS addresses live across the whole loop
    int tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    prep_item<DK, TIO, kW>(a, j, h, t0, nv, lds, tid_i, active);
    wait_vmem();      // this wave's record stores are complete
    __syncthreads();  // ... in every wave of the item; the LDS blocks are free again
    if (active && tid == 0) {
      unsigned flag = 1u | (xcd << 1);
      if (!home) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        flag |= kReadyReleased;
      }
      __hip_atomic_store(args.ready + ((int64_t)j * H + h), flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace gdn
