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
// the top of gdn_prep.hip).
#pragma once

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
template <bool kBF>
__device__ __forceinline__ void store_record(const float* M, const float* colscale, char* rec, int tid) {
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

// LDS of one scalar-gate item (bytes): k and q rows unpadded, 16-byte pieces
// XOR-swizzled by row (piece p of row r at slot p ^ (r % PPR)), so that
// direct loads fill them 1 KiB at a time and the fragment reads of 16 rows at
// one column hit different banks; once A and P are formed the solve's X
// overlays them.  Then A, the scaled log-gates and beta.
template <int DK, typename TIO>
struct PrepItemLds {
  static constexpr int RB = DK * (int)sizeof(TIO);  // bytes per k or q row
  static constexpr int PPR = RB / 16;               // pieces per row
  static constexpr int KQ = 2 * 64 * RB;
  static constexpr int KX = (KQ > 64 * kL64 * 4) ? KQ : 64 * kL64 * 4;
  static constexpr int oA = KX;
  static constexpr int oG2 = oA + 64 * kL64 * 4;
  static constexpr int oBeta = oG2 + 64 * 4;
  static constexpr int bytes = oBeta + 64 * 4;
  static_assert(bytes % 16 == 0, "item LDS blocks stay 16-byte aligned");
};

// The records of chunk j (tokens t0 .. t0 + nv - 1 of the packed inputs), head
// h, on four waves (item thread index tid = 0..255) with the LDS block lds
// (PrepItemLds bytes, 16-byte aligned).  Contains workgroup barriers; with
// active false the waves only take part in them.  On return this wave's
// record stores may still be in flight.
template <int DK, typename TIO>
__device__ __forceinline__ void prep_item(const PrepArgs& a, int j, int h, int t0, int nv, char* lds,
                                          int tid, bool active) {
  using IL = PrepItemLds<DK, TIO>;
  constexpr bool kBF = sizeof(TIO) == 2;
  constexpr int L64 = kL64;
  constexpr int NKB = DK / 32;
  constexpr int RB = IL::RB, PPR = IL::PPR;
  const char* sK = lds;
  const char* sQ = lds + 64 * RB;
  float* sX = reinterpret_cast<float*>(lds);
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
  char* prec = reinterpret_cast<char*>(a.P) + ((int64_t)j * H + h) * kTRecBytes;
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
  if (active) store_record<kBF>(sX, sBeta, reinterpret_cast<char*>(a.T) + ((int64_t)j * H + h) * kTRecBytes, tid);
}

}  // namespace gdn
