// mla_sparse_decode_noalloc: the decode entry point for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). It runs the
// same host checks and kernels as mla_sparse_decode; only the split partials (the one scratch
// buffer the decode uses) go to a fixed device array owned by the library instead of a caller
// workspace.
//
// The array is a file-scope __device__ object of MLA_NOALLOC_SCRATCH_BYTES, allocated by the HIP
// runtime with the code object on each device the library runs on and held until the process ends.
// Its device address is looked up once per device (hipGetSymbolAddress, with that device current)
// and kept; kernels receive that address, never the host-side name of the array. Nothing in it has
// to start at zero: every partial the merge reads is written earlier in the same call. Calls that
// overlap on one device share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla.h"
#include "mla_internal.h"

namespace {

static_assert(MLA_NOALLOC_SCRATCH_BYTES % 256 == 0, "the partial lse area stays 256-byte aligned");

__device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call per device).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int mla_sparse_decode_noalloc(const void* q, const uint8_t* k_cache, int64_t k_tokens,
                                         const int32_t* indices, int topk,
                                         const uint8_t* extra_k_cache, int64_t extra_tokens,
                                         const int32_t* extra_indices, int extra_topk, int batch,
                                         int seq_len_q, int h_q, float softmax_scale,
                                         const int32_t* sched, const int32_t* split_ptr,
                                         int num_parts_used, void* out, float* lse, void* stream) {
  const mla::DecodeCall c{q, k_cache, k_tokens, indices, topk, extra_k_cache, extra_tokens,
                          extra_indices, extra_topk, batch, seq_len_q, h_q, softmax_scale, sched,
                          split_ptr, num_parts_used, out, lse, stream};
  mla::WorkspaceSource ws;
  ws.fixed_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  ws.fixed_ptr = scratch_on_current_device;
  return mla::sparse_decode(c, ws);
}
