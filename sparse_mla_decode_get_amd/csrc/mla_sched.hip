// Tile-scheduler metadata kernel: the partition of (row, unit) work over parts, computed once before
// the decode loop (page "flops/flashmla-decode-fp8-fp4-kv", section "Workarounds": tile-scheduler
// metadata computed once rather than per step, split decoding with num_splits). The partition rule
// is this library's own: units u = row * tiles + tile; part p covers [floor(p*U/P), floor((p+1)*U/P)).
// One workgroup computes split counts per row, their exclusive prefix sum, then the per-part records.
#include "mla_internal.h"

namespace mla {

constexpr int kSchedThreads = 1024;

// Part owning unit u: the largest p with floor(p*U/P) <= u, i.e. ceil((u+1)*P/U) - 1.
__device__ __forceinline__ int64_t part_of_unit(int64_t u, int64_t units, int64_t parts) {
  return ((u + 1) * parts + units - 1) / units - 1;
}

__global__ __launch_bounds__(kSchedThreads) void metadata_kernel(int rows, int tiles, int parts,
                                                                 int32_t* sched, int32_t* split_ptr) {
  __shared__ int32_t scan[kSchedThreads];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int64_t units = (int64_t)rows * tiles;
  if (tid == 0) carry = 0;
  __syncthreads();
  // split_ptr[r] = sum over r' < r of (parts meeting row r'), chunk by chunk
  for (int base = 0; base < rows; base += kSchedThreads) {
    const int r = base + tid;
    int ns = 0;
    if (r < rows) {
      const int64_t first = part_of_unit((int64_t)r * tiles, units, parts);
      const int64_t last = part_of_unit((int64_t)(r + 1) * tiles - 1, units, parts);
      ns = (int)(last - first + 1);
    }
    scan[tid] = ns;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {      // inclusive Hillis-Steele scan
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int c = carry;
    if (r < rows) split_ptr[r + 1] = c + scan[tid];
    if (base == 0 && tid == 0) split_ptr[0] = 0;
    __syncthreads();
    if (tid == kSchedThreads - 1) carry = c + scan[tid];
    __syncthreads();
  }
  if (rows == 0 && tid == 0) split_ptr[0] = 0;
  __syncthreads();
  for (int p = tid; p < parts; p += kSchedThreads) {
    const int64_t b = (int64_t)p * units / parts;
    const int64_t e = (int64_t)(p + 1) * units / parts;
    int32_t* s = sched + (int64_t)p * 8;
    s[0] = (int32_t)(b / tiles);
    s[1] = (int32_t)(b % tiles);
    s[2] = (int32_t)(e / tiles);
    s[3] = (int32_t)(e % tiles);
    int32_t first_slot = 0;
    if (b < e) {
      const int64_t r0 = b / tiles;
      first_slot = split_ptr[r0] + (int32_t)(p - part_of_unit(r0 * tiles, units, parts));
    } else {
      const int64_t r0 = b / tiles;
      first_slot = rows ? split_ptr[r0 < rows ? r0 : rows] : 0;
    }
    s[4] = first_slot;
    s[5] = 0;
    s[6] = 0;
    s[7] = 0;
  }
}

int launch_metadata(int rows, int tiles, int parts, int32_t* sched, int32_t* split_ptr,
                    hipStream_t stream) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kSchedThreads), 0, stream, rows, tiles, parts,
                     sched, split_ptr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
