// gdn_abi.hip -- the C ABI declared in include/gdn.h: host-side argument
// checks (run before any launch, never touching device memory), a per-device
// gfx950 capability cache, and dispatch to the launch functions.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "gdn.h"
#include "gdn_launch.hpp"

// Workspace of gdn_chunk_fwd_noalloc: one array on every GPU the library runs
// on, held until the process ends.  In host code `scratch` is only a stand-in
// symbol; its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

gdn_status_t fail(gdn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

gdn_status_t check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(GDN_ERR_DEVICE, "no current HIP device");
  if (dev >= kMaxDevices) return fail(GDN_ERR_DEVICE, "device index %d out of range", dev);
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(GDN_ERR_DEVICE, "hipGetDeviceProperties failed on device %d", dev);
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(GDN_ERR_DEVICE, "device %d is not gfx950 (MI355X)", dev);
  return GDN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device address of `scratch` on the current device (dev), looked up on the
// first call on that device and kept; null when the lookup fails.
std::atomic<void*> g_scratch[kMaxDevices];

void* scratch_address(int dev) {
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

gdn_status_t check_shape(const gdn_shape_t* s, bool decode) {
  if (s == nullptr) return fail(GDN_ERR_INVALID_ARG, "shape is NULL");
  if (s->n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "n_seqs must be >= 1 (got %d)", s->n_seqs);
  if (s->n_heads < 1) return fail(GDN_ERR_INVALID_ARG, "n_heads must be >= 1 (got %d)", s->n_heads);
  if (s->dk < 1 || s->dv < 1) return fail(GDN_ERR_INVALID_ARG, "dk, dv must be positive");
  if (s->dv % 64 != 0) return fail(GDN_ERR_INVALID_ARG, "dv must be a multiple of 64 (got %d)", s->dv);
  if (s->dk != 64 && s->dk != 128) return fail(GDN_ERR_UNSUPPORTED, "dk must be 64 or 128 (got %d)", s->dk);
  if (s->dv > 256) return fail(GDN_ERR_UNSUPPORTED, "dv above 256 is not supported (got %d)", s->dv);
  if (s->total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "total_tokens must be >= 0");
  if ((s->io_dtype != GDN_F32 && s->io_dtype != GDN_BF16) ||
      (s->o_dtype != GDN_F32 && s->o_dtype != GDN_BF16))
    return fail(GDN_ERR_INVALID_ARG, "io_dtype and o_dtype must be GDN_F32 or GDN_BF16");
  if (s->gate_per_channel != 0 && s->gate_per_channel != 1)
    return fail(GDN_ERR_INVALID_ARG, "gate_per_channel must be 0 or 1");
  if (s->qdq_flags & ~(GDN_QDQ_CHUNK | GDN_QDQ_WRITE | GDN_QDQ_W | GDN_QDQ_INT8))
    return fail(GDN_ERR_INVALID_ARG, "unknown qdq_flags bits 0x%x", s->qdq_flags);
  if (s->gate_grid_log2 < 0 || s->gate_grid_log2 > 24)
    return fail(GDN_ERR_INVALID_ARG, "gate_grid_log2 must be 0 (off) or 1 .. 24 (got %d)", s->gate_grid_log2);
  const int64_t blocks = (int64_t)s->n_seqs * s->n_heads * (s->dv / 64);
  if (blocks >= (int64_t)1 << 31) return fail(GDN_ERR_UNSUPPORTED, "too many (sequence, head, tile) units");
  // the chunk kernel addresses one 64-token chunk of a head with 32-bit byte offsets
  if ((int64_t)64 * s->n_heads * (s->dk > s->dv ? s->dk : s->dv) * 4 >= (int64_t)1 << 31)
    return fail(GDN_ERR_UNSUPPORTED, "n_heads too large (64 * n_heads * max(dk, dv) * 4 bytes must be < 2^31)");
  if (decode && s->total_tokens != s->n_seqs)
    return fail(GDN_ERR_INVALID_ARG, "decode: total_tokens must equal n_seqs");
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status_t status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_DEVICE: return "GDN_ERR_DEVICE";
  }
  return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error(void) { return g_err; }

gdn_status_t gdn_state_qdq(const float* in, float* out, float* scales, int64_t n_states,
                           int32_t dv, int32_t dk, void* stream) {
  g_err[0] = 0;
  if (n_states < 0) return fail(GDN_ERR_INVALID_ARG, "n_states must be >= 0");
  if (dv < 64 || dv % 64 != 0) return fail(GDN_ERR_INVALID_ARG, "dv must be a positive multiple of 64");
  if (dk < 4 || dk % 4 != 0) return fail(GDN_ERR_INVALID_ARG, "dk must be a positive multiple of 4");
  if (dk > 256) return fail(GDN_ERR_UNSUPPORTED, "dk above 256 is not supported");
  const int64_t tiles = n_states * (dv / 64);
  if (tiles >= (int64_t)1 << 31) return fail(GDN_ERR_UNSUPPORTED, "too many tiles");
  if (n_states > 0) {
    if (in == nullptr || out == nullptr) return fail(GDN_ERR_INVALID_ARG, "in/out is NULL");
    if (!aligned(in, 16) || !aligned(out, 16)) return fail(GDN_ERR_INVALID_ARG, "in/out must be 16-byte aligned");
  }
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  hipError_t e = gdn::launch_state_qdq(in, out, scales, tiles, dk, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

gdn_status_t gdn_state_qdq_int8(const float* in, float* out, float* scales, int64_t n_states,
                                int32_t dv, int32_t dk, void* stream) {
  g_err[0] = 0;
  if (n_states < 0) return fail(GDN_ERR_INVALID_ARG, "n_states must be >= 0");
  if (dv < 64 || dv % 64 != 0) return fail(GDN_ERR_INVALID_ARG, "dv must be a positive multiple of 64");
  if (dk < 32 || dk % 32 != 0) return fail(GDN_ERR_INVALID_ARG, "dk must be a positive multiple of 32");
  if (dk > 256) return fail(GDN_ERR_UNSUPPORTED, "dk above 256 is not supported");
  const int64_t n_values = n_states * dv * dk;
  if (n_values / 4 / 256 >= (int64_t)1 << 31) return fail(GDN_ERR_UNSUPPORTED, "too many values");
  if (n_states > 0) {
    if (in == nullptr || out == nullptr) return fail(GDN_ERR_INVALID_ARG, "in/out is NULL");
    if (!aligned(in, 16) || !aligned(out, 16)) return fail(GDN_ERR_INVALID_ARG, "in/out must be 16-byte aligned");
  }
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  hipError_t e = gdn::launch_state_qdq_int8(in, out, scales, n_values, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

gdn_status_t gdn_decode_step(const gdn_shape_t* shape, const void* q, const void* k,
                             const void* v, const float* beta, const float* g, const int32_t* active,
                             float* state, void* o, float* state_pre, float* scales, void* stream) {
  g_err[0] = 0;
  gdn_status_t st = check_shape(shape, true);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !beta || !g || !state || !o)
    return fail(GDN_ERR_INVALID_ARG, "q, k, v, beta, g, state and o must be non-NULL");
  const uintptr_t ea = shape->io_dtype == GDN_BF16 ? 8 : 16;
  if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, 4) || !aligned(state, 16) ||
      (state_pre && !aligned(state_pre, 16)) || !aligned(beta, 4) || !aligned(g, 4) ||
      !aligned(active, 4) || !aligned(o, shape->o_dtype == GDN_BF16 ? 2 : 4))
    return fail(GDN_ERR_INVALID_ARG, "misaligned buffer");
  st = check_device();
  if (st != GDN_OK) return st;
  hipError_t e = gdn::launch_decode_step(*shape, q, k, v, beta, g, active, state, o, state_pre, scales,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

gdn_status_t gdn_workspace_status(const void* workspace, void* stream) {
  g_err[0] = 0;
  if (workspace == nullptr) return fail(GDN_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "reading the status word failed: %s", hipGetErrorString(e));
  if (word & gdn::kStatusBadIndex)
    return fail(GDN_ERR_INVALID_ARG, "the device found the index arrays (cu_seqlens, seq_lens, prefix_lens) "
                                     "out of contract; nothing was computed");
  if (word & gdn::kStatusWaitTimeout)
    return fail(GDN_ERR_DEVICE, "a bounded wait for a per-chunk record ran out; the affected outputs are NaN");
  if (word != 0) return fail(GDN_ERR_DEVICE, "unknown status word 0x%x", (unsigned)word);
  return GDN_OK;
}

size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape_t* shape) {
  g_err[0] = 0;
  if (check_shape(shape, false) != GDN_OK) return 0;
  return gdn::prep_workspace_bytes(*shape);
}

}  // extern "C"

namespace {

// Host checks of gdn_chunk_fwd and gdn_chunk_fwd_noalloc other than the
// workspace and the device.
gdn_status_t check_chunk_args(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                              const float* beta, const float* g, const int32_t* cu_seqlens,
                              const float* initial_state, const void* o, const float* final_state,
                              const gdn_debug_t* debug) {
  gdn_status_t st = check_shape(shape, false);
  if (st != GDN_OK) return st;
  if (shape->qdq_flags & GDN_QDQ_INT8)
    return fail(GDN_ERR_UNSUPPORTED, "GDN_QDQ_INT8 is a decode-step codec (gdn_decode_step, gdn_state_qdq_int8)");
  if (!cu_seqlens || !final_state) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens and final_state must be non-NULL");
  if (shape->total_tokens > 0 && (!q || !k || !v || !beta || !g || !o))
    return fail(GDN_ERR_INVALID_ARG, "q, k, v, beta, g and o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(final_state, 16) || (initial_state && !aligned(initial_state, 16)) ||
      !aligned(beta, 4) || !aligned(g, 4) || !aligned(cu_seqlens, 4))
    return fail(GDN_ERR_INVALID_ARG, "misaligned buffer (q, k, v, o and states need 16 bytes)");
  if (debug && (debug->bound_pre || debug->bound_post || debug->scales || debug->w_pre || debug->w_post) &&
      !debug->bound_offsets)
    return fail(GDN_ERR_INVALID_ARG, "debug record needs bound_offsets");
  if (debug && (debug->suffix_pre || debug->suffix_post) && !debug->suffix_offsets)
    return fail(GDN_ERR_INVALID_ARG, "suffix record needs suffix_offsets");
  if (debug && (!aligned(debug->bound_pre, 16) || !aligned(debug->bound_post, 16) ||
                !aligned(debug->suffix_pre, 16) || !aligned(debug->suffix_post, 16) ||
                !aligned(debug->status, 4)))
    return fail(GDN_ERR_INVALID_ARG, "misaligned debug record (states need 16 bytes)");
  if (debug && (debug->schedule < GDN_SCHEDULE_AUTO || debug->schedule > GDN_SCHEDULE_FUSED_NO_PRODUCERS))
    return fail(GDN_ERR_INVALID_ARG, "debug schedule must be GDN_SCHEDULE_AUTO, _SPLIT, _FUSED or _FUSED_NO_PRODUCERS");
  if (shape->io_dtype == GDN_F32 && shape->dk == 128 && (shape->qdq_flags & GDN_QDQ_W))
    return fail(GDN_ERR_UNSUPPORTED, "fp32 inputs with dk = 128 take no W QDQ (the token recurrence has no W)");
  return GDN_OK;
}

gdn_status_t run_chunk_fwd(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const int32_t* cu_seqlens,
                           const int32_t* seq_lens, const int32_t* prefix_lens,
                           const float* initial_state, void* o, float* final_state,
                           void* workspace, const gdn_debug_t* debug, void* stream) {
  hipError_t e = gdn::launch_chunk_fwd(*shape, q, k, v, beta, g, cu_seqlens, seq_lens, prefix_lens,
                                       initial_state, o, final_state, workspace, debug,
                                       (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(GDN_ERR_UNSUPPORTED, "configuration not supported");
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status_t gdn_chunk_fwd(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const int32_t* cu_seqlens,
                           const int32_t* seq_lens, const int32_t* prefix_lens,
                           const float* initial_state, void* o, float* final_state,
                           void* workspace, size_t workspace_bytes,
                           const gdn_debug_t* debug, void* stream) {
  g_err[0] = 0;
  gdn_status_t st = check_chunk_args(shape, q, k, v, beta, g, cu_seqlens, initial_state, o, final_state, debug);
  if (st != GDN_OK) return st;
  const size_t need = gdn::prep_workspace_bytes(*shape);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GDN_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  st = check_device();
  if (st != GDN_OK) return st;
  return run_chunk_fwd(shape, q, k, v, beta, g, cu_seqlens, seq_lens, prefix_lens, initial_state, o, final_state,
                       workspace, debug, stream);
}

gdn_status_t gdn_chunk_fwd_noalloc(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                                   const float* beta, const float* g, const int32_t* cu_seqlens,
                                   const int32_t* seq_lens, const int32_t* prefix_lens,
                                   const float* initial_state, void* o, float* final_state,
                                   const gdn_debug_t* debug, void* stream) {
  g_err[0] = 0;
  gdn_status_t st = check_chunk_args(shape, q, k, v, beta, g, cu_seqlens, initial_state, o, final_state, debug);
  if (st != GDN_OK) return st;
  const size_t need = gdn::prep_workspace_bytes(*shape);
  if (need > GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of workspace; the static scratch holds %zu "
                "(use gdn_chunk_fwd with a caller-owned workspace)",
                need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  st = check_device();
  if (st != GDN_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_DEVICE, "no current HIP device");
  void* ws = scratch_address(dev);
  if (ws == nullptr) return fail(GDN_ERR_DEVICE, "hipGetSymbolAddress of the static scratch failed on device %d", dev);
  return run_chunk_fwd(shape, q, k, v, beta, g, cu_seqlens, seq_lens, prefix_lens, initial_state, o, final_state,
                       ws, debug, stream);
}

size_t gdn_chunk_bwd_workspace_bytes(const gdn_shape_t* shape) {
  g_err[0] = 0;
  if (check_shape(shape, false) != GDN_OK) return 0;
  return gdn::bwd_workspace_bytes(*shape);
}

gdn_status_t gdn_chunk_bwd_dh(const gdn_shape_t* shape, const void* q, const void* k, const float* beta,
                              const float* g, const int32_t* cu_seqlens, const int32_t* seq_lens,
                              const void* d_o, const float* d_final_state, float* dh, float* d_initial_state,
                              float* d_v, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  gdn_status_t st = check_shape(shape, false);
  if (st != GDN_OK) return st;
  if (shape->io_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_bwd_dh takes bf16 q, k and d_o");
  if (shape->qdq_flags & GDN_QDQ_INT8)
    return fail(GDN_ERR_UNSUPPORTED, "GDN_QDQ_INT8 is a decode-step codec");
  if (shape->gate_per_channel && (shape->qdq_flags & GDN_QDQ_W))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_bwd_dh: the per-key-channel gate's backward is the token "
                "recurrence, which has no W; the backward of a per-channel W-QDQ forward is not built");
  if (shape->gate_grid_log2 != 0)
    return fail(GDN_ERR_INVALID_ARG, "gdn_chunk_bwd_dh covers fully chunked sequences, which have no "
                "recurrent writes: gate_grid_log2 must be 0");
  const size_t need = gdn::bwd_workspace_bytes(*shape);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GDN_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (!cu_seqlens) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens must be non-NULL");
  if (!dh && !d_initial_state && !d_v) return fail(GDN_ERR_INVALID_ARG, "dh, d_initial_state and d_v are all NULL");
  if (shape->total_tokens > 0 && (!q || !k || !beta || !g || !d_o))
    return fail(GDN_ERR_INVALID_ARG, "q, k, beta, g and d_o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(d_o, 16) || !aligned(dh, 16) ||
      !aligned(d_initial_state, 16) || !aligned(d_final_state, 16) || !aligned(d_v, 4) || !aligned(beta, 4) ||
      !aligned(g, 4) ||
      !aligned(cu_seqlens, 4))
    return fail(GDN_ERR_INVALID_ARG, "misaligned buffer (q, k, d_o and states need 16 bytes)");
  st = check_device();
  if (st != GDN_OK) return st;
  hipError_t e = gdn::launch_chunk_bwd_dh(*shape, q, k, beta, g, cu_seqlens, seq_lens, d_o, d_final_state, dh,
                                          d_initial_state, d_v, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

}  // extern "C"
