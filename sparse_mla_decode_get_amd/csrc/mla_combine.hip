// Log-sum-exp merge of split-KV partials (page "flops/flashmla-decode-fp8-fp4-kv", section
// "Workarounds": split decoding with num_splits). For each (row, head): M = max_i lse_i,
// w_i = exp(lse_i - M), lse = M + log(sum w_i), out = sum_i w_i o_i / sum w_i, where each o_i is
// already normalised by its own softmax sum. Splits with lse = -inf carry no weight; a row with no
// live split gets out = 0 and lse = -inf.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kCombineThreads = 128;   // the fused merge: 4 dims per thread

// One 16-byte load of a partial row per split and thread: 4 dims of fp32 partials (mla_combine's
// input and the fused decode's workspace) or 8 dims of the bf16 partials the plain decode kernels
// write, so that each load instruction moves as many bytes for either type.
template <typename PT>
struct PartialLoad {
  static constexpr int kDims = 16 / (int)sizeof(PT);
  static constexpr int kThreads = kHeadDim / kDims;
  __device__ static float dim(const u32x4& w, int k) {
    // the element is copied out first: bit-casting the vector element itself reads element 0
    const uint32_t e = w[sizeof(PT) == 4 ? k : k >> 1];
    if constexpr (sizeof(PT) == 4) return __builtin_bit_cast(float, e);
    else return __builtin_bit_cast(float, (k & 1) ? (e & 0xFFFF0000u) : (e << 16));
  }
};

template <typename PT>
__global__ __launch_bounds__(PartialLoad<PT>::kThreads) void combine_kernel(
    const PT* __restrict__ partial, const float* __restrict__ partial_lse,
    const int32_t* __restrict__ split_ptr, int h_q, uint16_t* __restrict__ out,
    float* __restrict__ lse, int skip_single) {
  using PL = PartialLoad<PT>;
  constexpr int kDims = PL::kDims;
  const int row = blockIdx.x;
  const int head = blockIdx.y;
  const int a = split_ptr[row];
  const int n = split_ptr[row + 1] - a;
  if (skip_single && n == 1) return;      // written directly by the decode kernel
  const float ninf = -__builtin_inff();
  const float* lse_col = partial_lse + (int64_t)a * h_q + head;
  const int dim = kDims * threadIdx.x;
  const PT* o_col = partial + ((int64_t)a * h_q + head) * kHeadDim + dim;
  // One pass over the splits, kBatch at a time, with every lse and partial load of a batch issued
  // before any is used (one memory round trip per batch, none waiting on an earlier maximum). The
  // sums are kept relative to the running maximum m and rescaled when a batch raises it:
  // wsum = sum_i exp(lse_i - m), acc = sum_i exp(lse_i - m) o_i.
  constexpr int kBatch = 8;
  float m = ninf;
  float acc[kDims] = {};
  float wsum = 0.0f;
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    float li[kBatch];
    u32x4 o[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool in = i0 + u < n;
      li[u] = in ? lse_col[(int64_t)(i0 + u) * h_q] : ninf;
      o[u] = in ? *reinterpret_cast<const u32x4*>(o_col + (int64_t)(i0 + u) * h_q * kHeadDim) : u32x4{};
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mb = fmaxf(mb, li[u]);
    if (mb == ninf) continue;                // no live split so far
    const float sc = __expf(m - mb);         // 0 while m = -inf, when acc and wsum are still 0
#pragma unroll
    for (int k = 0; k < kDims; ++k) acc[k] *= sc;
    wsum *= sc;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // an empty split (lse -inf) carries no weight, whatever its partial holds
      if (li[u] == ninf) continue;
      const float w = __expf(li[u] - mb);
      wsum += w;
#pragma unroll
      for (int k = 0; k < kDims; ++k) acc[k] += w * PL::dim(o[u], k);
    }
    m = mb;
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  uint16_t* const orow = out + ((int64_t)row * h_q + head) * kHeadDim + dim;
  if constexpr (kDims == 4) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (__bf16)(acc[i] * inv);
    *reinterpret_cast<bf16x4*>(orow) = r;
  } else {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)(acc[i] * inv);
    *reinterpret_cast<bf16x8*>(orow) = r;
  }
  if (threadIdx.x == 0) lse[(int64_t)row * h_q + head] = wsum > 0.0f ? m + __logf(wsum) : ninf;
}

// The same merge for the fused decode's split rows: the merged row's rotary pairs (dims 448 + 2i,
// 449 + 2i) are rotated back by the row's angle and the row is stored as an fp8 record (512 e4m3
// values, then 16 e8m0 scales; a 32-dim block is the 8 threads 8b .. 8b+7 of one wave).
__global__ __launch_bounds__(kCombineThreads) void combine_fused_kernel(
    const float* __restrict__ partial, const float* __restrict__ partial_lse,
    const int32_t* __restrict__ split_ptr, int h_q, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, uint8_t* __restrict__ out_fp8, float* __restrict__ lse) {
  const int row = blockIdx.x;
  const int head = blockIdx.y;
  const int a = split_ptr[row];
  const int n = split_ptr[row + 1] - a;
  if (n == 1) return;                      // written directly by the decode kernel
  const float ninf = -__builtin_inff();
  const int t = threadIdx.x;
  const int dim = 4 * t;
  const float* lse_col = partial_lse + (int64_t)a * h_q + head;
  const float* o_col = partial + ((int64_t)a * h_q + head) * kHeadDim + dim;
  float m = ninf, wsum = 0.0f;
  f32x4 acc = f32x4{};
  for (int i = 0; i < n; ++i) {            // two passes are not needed: rescale as the max grows
    const float li = lse_col[(int64_t)i * h_q];
    if (li == ninf) continue;
    const f32x4 o = *reinterpret_cast<const f32x4*>(o_col + (int64_t)i * h_q * kHeadDim);
    const float mn = fmaxf(m, li);
    const float sc = __expf(m - mn);
    const float w = __expf(li - mn);
    acc = acc * sc + w * o;
    wsum = wsum * sc + w;
    m = mn;
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = acc[i] * inv;
  if (dim >= 448) {
    const int pi = (dim - 448) / 2;         // pairs pi and pi + 1
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const float c = rope_cos[(int64_t)row * 32 + pi + jj], sn = rope_sin[(int64_t)row * 32 + pi + jj];
      const float x0 = y[2 * jj], x1 = y[2 * jj + 1];
      y[2 * jj] = x0 * c + x1 * sn;
      y[2 * jj + 1] = x1 * c - x0 * sn;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = fmaxf(amax, __builtin_fabsf(y[i]));
  const int lane = t & 63;
#pragma unroll
  for (int msk = 1; msk < 8; msk <<= 1)
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                           (lane ^ msk) << 2, __builtin_bit_cast(int, amax))));
  const int k = fp8_block_exponent(amax);
  const uint32_t w = e4m3_codes4(y[0], y[1], y[2], y[3], k);
  uint8_t* rec = out_fp8 + ((int64_t)row * h_q + head) * kFp8Rec;
  *reinterpret_cast<uint32_t*>(rec + dim) = w;
  if ((t & 7) == 0) rec[kHeadDim + (t >> 3)] = (uint8_t)(k + 127);
  if (t == 0) lse[(int64_t)row * h_q + head] = wsum > 0.0f ? m + __logf(wsum) : ninf;
}

int launch_combine_fused(const float* partial, const float* partial_lse, const int32_t* split_ptr,
                         int rows, int h_q, const float* rope_cos, const float* rope_sin,
                         uint8_t* out_fp8, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(combine_fused_kernel, dim3(rows, h_q), dim3(kCombineThreads), 0, stream, partial,
                     partial_lse, split_ptr, h_q, rope_cos, rope_sin, out_fp8, lse);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_combine(const float* partial, const float* partial_lse, const int32_t* split_ptr,
                   int rows, int h_q, uint16_t* out, float* lse, bool skip_single,
                   hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel<float>, dim3(rows, h_q), dim3(PartialLoad<float>::kThreads), 0, stream,
                     partial, partial_lse, split_ptr, h_q, out, lse, skip_single ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_combine_bf16(const uint16_t* partial, const float* partial_lse, const int32_t* split_ptr,
                        int rows, int h_q, uint16_t* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(rows, h_q), dim3(PartialLoad<uint16_t>::kThreads), 0, stream,
                     partial, partial_lse, split_ptr, h_q, out, lse, 1);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
