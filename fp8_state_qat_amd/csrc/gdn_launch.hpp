// gdn_launch.hpp -- internal launch functions behind the C ABI (gdn_abi.hip).
// Arguments arrive already validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"

namespace gdn {

// A kernel's dynamic-LDS limit (hipFuncAttributeMaxDynamicSharedMemorySize)
// belongs to each device's copy of the function: set it once per device, so a
// process that drives several GPUs sets it on every one it launches on.
struct PerDeviceOnce {
  std::atomic<uint64_t> done{0};  // bit d: set on device d (devices 0..63)
};
inline hipError_t set_dyn_lds_once(PerDeviceOnce& once, const void* kern, size_t lds) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit && (once.done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess && bit) once.done.fetch_or(bit, std::memory_order_release);
  return e;  // concurrent first calls on one device both set it: harmless
}

hipError_t launch_state_qdq(const float* in, float* out, float* scales, int64_t n_tiles, int dk,
                            hipStream_t stream);

// n_values a multiple of 64 * 32 (whole 64-row tiles of 32-column blocks).
hipError_t launch_state_qdq_int8(const float* in, float* out, float* scales, int64_t n_values,
                                 hipStream_t stream);

hipError_t launch_decode_step(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                              const float* beta, const float* g, const int32_t* active, float* state,
                              void* o, float* state_pre, float* scales, hipStream_t stream);

// Status word at byte 0 of a chunk workspace (forward and backward): 0 after
// a clean call; the bits below are set by the device during the call.
constexpr int32_t kStatusWaitTimeout = 1;  // a fused consumer's bounded wait ran out
constexpr int32_t kStatusBadIndex = 2;     // index arrays out of contract: nothing ran
constexpr size_t kStatusBytes = 256;       // the status block ahead of the chunk offsets

hipError_t launch_chunk_fwd(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                            const float* beta, const float* g, const int32_t* cu_seqlens,
                            const int32_t* seq_lens, const int32_t* prefix_lens,
                            const float* initial_state, void* o, float* final_state,
                            void* workspace, const gdn_debug_t* debug, hipStream_t stream);

// Two records per (chunk, head): T = (I + A)^-1 diag(beta) and the decayed,
// masked P = Q K^T, each in MFMA fragment order (see gdn_prep.hip).  T: three
// bf16 planes (hi, mid, lo: 24 significant bits, so the state update keeps
// fp32 accuracy) or fp32, in an 18 KiB slot; P: two bf16 planes (hi, lo: it
// only reaches the outputs) or fp32, 12 KiB.
constexpr int kTRecBytes = 18432;
constexpr int kPRecBytes = 12288;

// With W QDQ, a third record per (chunk, head): the E4M3 codes of the
// row-quantized W = T (K * exp(gamma)) as bf16 values (exact), in the
// fragment order of the sequential kernel's k dump without its rotation
// (fragment f = tt * dk / 32 + kb, lane l holds W[16 tt + l % 16][32 kb +
// 8 (l / 16) .. + 7]), then one 1 KiB block whose first 64 floats are the
// row scales.
constexpr int w_rec_bytes(int dk) { return dk * 128 + 1024; }

// The chunk workspace: the status word (padded to 256 bytes), int32 chunk
// offsets [N + 1] and the largest chunk count of a sequence (padded to 256
// bytes), one uint32 ready flag per
// (chunk, head) (padded to 256 bytes; used by the fused launch), then the T
// records (kTRecBytes each), the P records (kPRecBytes each) and, with W QDQ,
// the W records, all sized for the
// worst-case chunk count ceil(total_tokens / 64) + N.
struct PrepLayout {
  int32_t* status;
  int32_t* offs;
  unsigned* ready;
  void* T;
  void* P;
  void* W;        // null without W QDQ
  int64_t items;  // (chunk, head) slots
  size_t bytes;   // total workspace bytes
};
PrepLayout prep_layout(const gdn_shape_t& s, void* workspace);
size_t prep_workspace_bytes(const gdn_shape_t& s);

// Chunk offsets (and the status word: cleared, then the index arrays are
// checked against total_tokens), then (records true) the T and P (and W)
// records of every (chunk, head); with records false the ready flags are
// cleared instead, for a fused launch that produces the records itself.  w_pre / w_post: the
// optional W record of the debug struct (null when absent).
hipError_t launch_prep(const gdn_shape_t& s, const void* q, const void* k, const float* beta,
                       const float* g, const int32_t* cu_seqlens, const int32_t* seq_lens,
                       const int32_t* prefix_lens, const PrepLayout& L, bool records, float* w_pre,
                       float* w_post, hipStream_t stream);

// Copy the status word of a workspace to a caller's device int32 (one thread).
hipError_t launch_copy_status(const int32_t* status, int32_t* dst, hipStream_t stream);

// Backward state recurrence (gdn_bwd.hip): workspace = the status word,
// chunk offsets, then one T^T and one P^T record (16 KiB each) per (chunk,
// head).
size_t bwd_workspace_bytes(const gdn_shape_t& s);
hipError_t launch_chunk_bwd_dh(const gdn_shape_t& s, const void* q, const void* k, const float* beta,
                               const float* g, const int32_t* cu_seqlens, const int32_t* seq_lens,
                               const void* dout, const float* dfin, float* dh, float* dinit, float* dvals,
                               void* workspace, hipStream_t stream);

}  // namespace gdn
