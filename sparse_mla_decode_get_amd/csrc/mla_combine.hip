// Log-sum-exp merge of split-KV partials (page "flops/flashmla-decode-fp8-fp4-kv", section
// "Workarounds": split decoding with num_splits). For each (row, head): M = max_i lse_i,
// w_i = exp(lse_i - M), lse = M + log(sum w_i), out = sum_i w_i o_i / sum w_i, where each o_i is
// already normalised by its own softmax sum. Splits with lse = -inf carry no weight; a row with no
// live split gets out = 0 and lse = -inf.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kCombineThreads = 128;   // 4 dims per thread

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ partial, const float* __restrict__ partial_lse,
    const int32_t* __restrict__ split_ptr, int h_q, uint16_t* __restrict__ out,
    float* __restrict__ lse, int skip_single) {
  const int row = blockIdx.x;
  const int head = blockIdx.y;
  const int a = split_ptr[row];
  const int n = split_ptr[row + 1] - a;
  if (skip_single && n == 1) return;      // written directly by the decode kernel
  const float ninf = -__builtin_inff();
  float m = ninf;
  for (int i = 0; i < n; ++i) m = fmaxf(m, partial_lse[(int64_t)(a + i) * h_q + head]);
  const int dim = 4 * threadIdx.x;
  f32x4 acc = f32x4{};
  float wsum = 0.0f;
  if (m != ninf) {
    for (int i = 0; i < n; ++i) {
      const float li = partial_lse[(int64_t)(a + i) * h_q + head];
      if (li == ninf) continue;
      const float w = __expf(li - m);
      wsum += w;
      const f32x4 o = *reinterpret_cast<const f32x4*>(partial + ((int64_t)(a + i) * h_q + head) * kHeadDim + dim);
      acc += w * o;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x4*>(out + ((int64_t)row * h_q + head) * kHeadDim + dim) = r;
  if (threadIdx.x == 0) lse[(int64_t)row * h_q + head] = wsum > 0.0f ? m + __logf(wsum) : ninf;
}

int launch_combine(const float* partial, const float* partial_lse, const int32_t* split_ptr,
                   int rows, int h_q, uint16_t* out, float* lse, bool skip_single,
                   hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(rows, h_q), dim3(kCombineThreads), 0, stream, partial,
                     partial_lse, split_ptr, h_q, out, lse, skip_single ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
