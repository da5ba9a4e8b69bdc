// Diagnostics that run the decode kernel's own device routines outside the attention loop:
// whole-record dequantisation (the same dequant_fp8_16 / dequant_fp4_16 the QK^T operands use) and
// an index range count.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

// One thread per (token, 16-value group): 32 groups per record.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ cache,
                                                      int record_bytes,
                                                      const int32_t* __restrict__ idx, int n,
                                                      uint16_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n * 32) return;
  const int t = (int)(gid >> 5);
  const int grp = (int)(gid & 31);                 // values 16*grp .. 16*grp+15
  const int64_t tokid = idx[t];
  bf16x8 lo, hi;
  if (record_bytes == kFp8Rec) {
    const uint8_t* rec = cache + tokid * kFp8Rec;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(rec + 16 * grp);
    const uint32_t sb = rec[kHeadDim + grp / 2];
    dequant_fp8_16(raw, sb, lo, hi);
  } else {
    const uint8_t* rec = cache + tokid * kFp4Rec;
    const u32x2 raw = *reinterpret_cast<const u32x2*>(rec + 8 * grp);
    const float sf = e4m3_to_f32(rec[kHeadDim / 2 + grp]);
    dequant_fp4_16(raw[0], raw[1], sf, lo, hi);
  }
  bf16x8* dst = reinterpret_cast<bf16x8*>(out + (int64_t)t * kHeadDim + 16 * grp);
  dst[0] = lo;
  dst[1] = hi;
}

__global__ void zero_kernel(int32_t* p) { *p = 0; }

__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                       int64_t num_tokens, int32_t* bad) {
  int cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    cnt += (int64_t)idx[i] >= num_tokens;
  if (cnt) atomicAdd(bad, cnt);
}

int launch_dequant(const uint8_t* cache, int record_bytes, const int32_t* idx, int n,
                   uint16_t* out, hipStream_t stream) {
  const int64_t threads = (int64_t)n * 32;
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), 0, stream, cache, record_bytes, idx,
                     n, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_validate(const int32_t* idx, int64_t n, int64_t num_tokens, int32_t* bad,
                    hipStream_t stream) {
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, stream, bad);
  if (n > 0) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(validate_kernel, dim3((int)blocks), dim3(256), 0, stream, idx, n, num_tokens,
                       bad);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
