// gdn_qdq.hip -- standalone per-tile state QDQ (fake quantize-dequantize of
// fp32 states to FP8-E4M3 with one scalar scale per tile of 64 value rows x
// all key columns; Model-Optimizer #2497 "What does this PR do?").
//
// One workgroup of 256 threads per tile.  The tile (64 * dk fp32, 32 KiB at
// dk = 128) is read once into registers with coalesced 16-byte loads, its
// amax reduced in a fixed tree, then quantized and written back, both with
// non-temporal accesses.  Memory bound: 8 bytes of HBM traffic per state
// element.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int V4>  // float4 per thread = 64 * dk / 4 / 256 = dk / 16
__global__ __launch_bounds__(kThreads) void state_qdq_kernel(const float* in,
                                                            float* out, float* __restrict__ scales,
                                                            int dk) {
  __shared__ float red[4];
  const int64_t tile = blockIdx.x;
  const int n4 = 16 * dk;  // float4 per tile
  const float4* src = reinterpret_cast<const float4*>(in) + tile * n4;
  float4* dst = reinterpret_cast<float4*>(out) + tile * n4;
  float4 x[V4];
  // every load is issued before the first use, so they are all in flight together
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int idx = threadIdx.x + kThreads * j;
    x[j] = idx < n4 ? ld_stream(src + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < V4; ++j)
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[j].x), fabsf(x[j].y)), fmaxf(fabsf(x[j].z), fabsf(x[j].w))));
  amax = block_max(amax, red);
  const float s = qdq_scale_f64(amax);
  const double r = rcp_f64(s);
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    int idx = threadIdx.x + kThreads * j;
    if (idx < n4) {
      f32x4 v = {x[j].x, x[j].y, x[j].z, x[j].w};
      float cv[4];
      qdq4c_f64(v, cv, s, r);
      st_stream(dst + idx, make_float4(v[0], v[1], v[2], v[3]));
    }
  }
  if (scales != nullptr && threadIdx.x == 0) scales[tile] = s;
}

// INT8 block QDQ of n4 float4 (blocks of 32 consecutive values = the
// float4s of 8 adjacent lanes; #2519 dynamic INT8 state recipes with
// 32-element blocks: scale amax / 127, round half to even).  One float4 per
// thread.
__global__ __launch_bounds__(kThreads) void state_qdq_int8_kernel(const float* in, float* out,
                                                                 float* __restrict__ scales, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // n4 is a multiple of 8 and of the block
  float4 x = ld_stream(reinterpret_cast<const float4*>(in) + i);
  const float s = int8_scale_f64(lane8_max_dpp(fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)))));
  qdq_int8_4_f64(x, s);
  st_stream(reinterpret_cast<float4*>(out) + i, x);
  if (scales != nullptr && (threadIdx.x & 7) == 0) scales[i >> 3] = s;
}

hipError_t launch_state_qdq_int8(const float* in, float* out, float* scales, int64_t n_values,
                                 hipStream_t stream) {
  const int64_t n4 = n_values / 4;
  if (n4 == 0) return hipSuccess;
  // every float4 of the grid exists: n_values is a multiple of 64 * 32 (dv % 64, dk % 32)
  hipLaunchKernelGGL(state_qdq_int8_kernel, dim3((unsigned)(n4 / kThreads)), dim3(kThreads), 0, stream, in, out,
                     scales, n4);
  return hipGetLastError();
}

hipError_t launch_state_qdq(const float* in, float* out, float* scales, int64_t n_tiles, int dk,
                            hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  dim3 grid((unsigned)n_tiles), block(kThreads);
  if (dk <= 64)
    hipLaunchKernelGGL(state_qdq_kernel<4>, grid, block, 0, stream, in, out, scales, dk);
  else if (dk <= 128)
    hipLaunchKernelGGL(state_qdq_kernel<8>, grid, block, 0, stream, in, out, scales, dk);
  else
    hipLaunchKernelGGL(state_qdq_kernel<16>, grid, block, 0, stream, in, out, scales, dk);
  return hipGetLastError();
}

}  // namespace gdn
