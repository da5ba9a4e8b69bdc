// Cache writer: bf16 latents -> per-token quantized records, written into the paged cache at given
// token slots (the step before decode).
//
// Record layouts (page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity"; page
// "deepseek-ai/FlashMLA", section "Key technical details": the raw quantized values first, then
// the token's scale factors):
//   fp8, 528 B: 512 e4m3 values, then 16 e8m0 scales (scale j covers values 32j .. 32j+31);
//   fp4, 288 B: 256 B of e2m1, value 2k in the low nibble of byte k and 2k+1 in the high nibble,
//               then 32 e4m3 scales (scale j covers values 16j .. 16j+15).
// The pages leave the choice of scales open; the rule here:
//   fp8 block, a = max |x|: k = ceil(log2(a / 448)) clipped to [-127, 127] (0 for a = 0), scale
//       byte k + 127, values e4m3(x * 2^-k) rounded to nearest, ties to even (|x * 2^-k| <= 448);
//   fp4 block: scale = e4m3(a / 6) rounded to nearest, ties to even, saturating at 448 (1.0 when that
//       rounds to 0); values e2m1(x / scale) rounded to nearest, ties to even, saturating at +-6.
// Rounding keeps the sign (a negative value that rounds to zero is stored as negative zero).
//
// One wave per token row at a time: lane l loads values 8l .. 8l+7 (one 16-byte load), the block
// maximum comes from the 4 (fp8) or 2 (fp4) lanes sharing a block, each lane stores its 8 (fp8) or
// 4 (fp4) data bytes, and the scale bytes are gathered four to a dword and stored by a few lanes.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kQuantWaves = 4;
// rows per wave: fp4 (its 288 B records written whole by 8 lanes) gains from four rows in flight;
// fp8 measured fastest with one (1 GiB in: 0.40 ms per 2^20 rows against 0.43 ms with four)
template <bool FP8> constexpr int kRowsPerWave = FP8 ? 1 : 4;

// Nearest e2m1 code of x / s for a finite f32 x and an e4m3 scale value s > 0 (ties to even),
// saturating at +-6, sign kept. The magnitude code counts the midpoints 0.25, 0.75, 1.25, 1.75,
// 2.5, 3.5, 5 (times s) below |x|; at a midpoint the even code wins (0.25 -> 0, 0.75 -> 2,
// 1.25 -> 2, 1.75 -> 4, 2.5 -> 4, 3.5 -> 6, 5 -> 6). t[i] = midpoint_i * s is exact in f32 (at most
// 3 + 4 significant bits), so comparing |x| with it decides exactly as |x| / s against the midpoint
// would, without a division.
__device__ __forceinline__ uint32_t e2m1_code(float x, const float (&t)[7]) {
  const float a = __builtin_fabsf(x);
  const uint32_t c = (uint32_t)(a > t[0]) + (uint32_t)(a >= t[1]) + (uint32_t)(a > t[2]) +
                     (uint32_t)(a >= t[3]) + (uint32_t)(a > t[4]) + (uint32_t)(a >= t[5]) +
                     (uint32_t)(a > t[6]);
  return c | ((__builtin_bit_cast(uint32_t, x) >> 28) & 8u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ float shfl_xor(float v, int lane, int m) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2,
                                                                __builtin_bit_cast(int, v)));
}
__device__ __forceinline__ uint32_t shfl_from(uint32_t v, int src_lane) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

// Encodes one token row: `w` holds this lane's 8 values (8 * lane ..), `tok` its cache slot.
template <bool FP8>
__device__ __forceinline__ void quantize_row(const u32x4& w, int64_t tok, uint8_t* cache, int lane) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
  if constexpr (FP8) {
    uint8_t* rec = cache + tok * kFp8Rec;
    a = fmaxf(a, shfl_xor(a, lane, 1));
    a = fmaxf(a, shfl_xor(a, lane, 2));                       // block lane / 4: 32 values
    const int k = fp8_block_exponent(a);
    const uint32_t b0 = e4m3_codes4(v[0], v[1], v[2], v[3], k);
    const uint32_t b1 = e4m3_codes4(v[4], v[5], v[6], v[7], k);
    *reinterpret_cast<u32x2*>(rec + 8 * lane) = u32x2{b0, b1};
    // scale byte of block j is held by lane 4j; lane 16d packs blocks 4d .. 4d+3
    const uint32_t sb = (uint32_t)(k + 127);
    const uint32_t d = sb | (shfl_from(sb, lane + 4) << 8) | (shfl_from(sb, lane + 8) << 16) |
                       (shfl_from(sb, lane + 12) << 24);
    if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(rec + kHeadDim + (lane >> 2)) = d;
  } else {
    uint8_t* rec = cache + tok * kFp4Rec;
    a = fmaxf(a, shfl_xor(a, lane, 1));                       // block lane / 2: 16 values
    uint32_t sc = e4m3_code(__fdiv_rn(a, 6.0f));
    sc = (sc & 0x7Fu) == 0 ? 0x38u : sc;                      // a zero scale is stored as 1.0
    const float sv = e4m3_to_f32(sc);
    const float t[7] = {0.25f * sv, 0.75f * sv, 1.25f * sv, 1.75f * sv, 2.5f * sv, 3.5f * sv, 5.0f * sv};
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(v[i], t) << (4 * i);
    *reinterpret_cast<uint32_t*>(rec + 4 * lane) = packed;
    // scale byte of block j is held by lane 2j; lane 8d packs blocks 4d .. 4d+3
    const uint32_t d = sc | (shfl_from(sc, lane + 2) << 8) | (shfl_from(sc, lane + 4) << 16) |
                       (shfl_from(sc, lane + 6) << 24);
    if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(rec + kHeadDim / 2 + (lane >> 1)) = d;
  }
}

// Each wave encodes kRowsPerWave consecutive rows; all their loads are issued before the first is
// used, so a wave keeps several 1 KB rows in flight.
template <bool FP8>
__global__ __launch_bounds__(64 * kQuantWaves) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t n, const int32_t* __restrict__ slots,
    uint8_t* __restrict__ cache, int64_t cache_tokens) {
  const int lane = (int)(threadIdx.x & 63);
  constexpr int R = kRowsPerWave<FP8>;
  const int64_t row0 = ((int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6)) * R;
  u32x4 w[R];
  int64_t tok[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < n ? row0 + r : n - 1;      // clamped: a valid address
    w[r] = *reinterpret_cast<const u32x4*>(x + row * kHeadDim + 8 * lane);
    tok[r] = row0 + r >= n ? -1 : slots ? (int64_t)slots[row] : row;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (tok[r] >= 0 && tok[r] < cache_tokens)                 // wave-uniform
      quantize_row<FP8>(w[r], tok[r], cache, lane);
}

}  // namespace

int launch_quantize(const uint16_t* x, int64_t n, const int32_t* slots, int record_bytes,
                    uint8_t* cache, int64_t cache_tokens, hipStream_t stream) {
  const bool fp8 = record_bytes == kFp8Rec;
  const int64_t rows_per_block = (int64_t)kQuantWaves * (fp8 ? kRowsPerWave<true> : kRowsPerWave<false>);
  const int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  if (fp8)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0,
                       stream, x, n, slots, cache, cache_tokens);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0,
                       stream, x, n, slots, cache, cache_tokens);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
