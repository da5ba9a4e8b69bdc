// Sparse MLA decode kernel for gfx950 (MI355X), 64-head groups (h_q <= 64; larger head counts use
// the 128-head kernel in mla_decode_wide.hip).
//
// What it computes (page "flops/flashmla-decode-fp8-fp4-kv", sections "Arithmetic intensity" and
// "Workarounds"; page "deepseek-ai/FlashMLA", sections "How to use it" and "Key technical details"):
// for every query row and head, softmax attention over the row's selected tokens, where the key and
// the value of a token are the same 512-dim latent decoded from its quantized record, negative index
// entries are ignored, and the output comes with its natural-log log-sum-exp.
//
// Work decomposition. The grid is (parts, head groups). A workgroup takes the contiguous range of
// (row, 64-slot unit) work the tile-scheduler metadata gives its part, for HG query heads
// (HG = 64 here) with W = HG / 16 = 4 waves. Every wave has the same register
// footprint: Q of 16 heads (64 VGPRs) and an fp32 output accumulator of 8 MFMA blocks.
// Each 64-slot unit runs as two sub-tiles of 32 tokens:
//   1. gather   all lanes copy 16-byte chunks of the selected records (data and scales together,
//               one contiguous record per token) straight from HBM into LDS with
//               global_load_lds_dwordx4, one sub-tile ahead, chunk-major: slot(chunk c, token t) =
//               c * 32 + t, so one wave instruction fills a contiguous 1 KB (chunks 2q, 2q+1).
//   2. QK^T     wave w owns heads 16w..16w+15; each lane reads 16 raw bytes of one token (a
//               conflict-free ds_read_b128 thanks to the chunk-major layout), dequantizes them in
//               registers with the record's own scale, and issues v_mfma_f32_16x16x32_bf16 against
//               its register-resident Q: S^T[16 tokens x 16 heads] over all 512 dims.
//   3. V slice  while dequantizing, wave w stores the bf16 values of its own PV dim slice
//               (512 / W dims) to a private LDS area, zeroing ignored tokens.
//   4. softmax  lanes n, n+16, n+32, n+48 share head n: masked max over the sub-tile, lazy rescale of
//               the running max (only when it grows by more than 2^8), exp2, bf16 P to LDS, the
//               running sum of the fp32 probabilities (so lse carries no bf16 rounding), and a
//               per-wave "rescale needed" flag.
//   5. PV       wave w accumulates O^T[its dim slice x all HG heads] += V^T P^T with
//               v_mfma_f32_32x32x16_bf16; V^T comes from its private slice via ds_read_b64_tr_b16,
//               P^T from LDS.
//   6. epilogue one split: out = O / l in bf16 and lse = ln(2) * (m + log2 l); several splits: the
//               normalised fp32 partial and its lse go to the workspace for the merge kernel.

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

template <int W>
struct DecodeCfg {
  static constexpr int HG = 16 * W;                 // heads per workgroup
  static constexpr int kThreads = 64 * W;
  static constexpr int kSlice = kHeadDim / W;       // PV dims per wave
  static constexpr int kDB = kSlice / 32;           // 32-dim output blocks per wave
  static constexpr int kHB = HG / 32;               // 32-head output blocks
  static constexpr int kNQ = (17 + W - 1) / W;      // gather instructions per wave per sub-tile
  static constexpr int kRawBytes = kFp8Chunks * kSubTokens * 16;   // 16896 per raw buffer
  static constexpr int kVStride = kSlice * 2 + 16;  // bytes per token row of a V slice
  static constexpr int kVBytes = kSubTokens * kVStride;
  static constexpr int kPStride = 80;               // bytes per head row of P (32 bf16 + pad)
  static constexpr int kOffV = 0;
  static constexpr int kOffP = kOffV + W * kVBytes;
  static constexpr int kOffAlpha = kOffP + HG * kPStride;
  static constexpr int kOffMFin = kOffAlpha + HG * 4;
  static constexpr int kOffLFin = kOffMFin + HG * 4;
  static constexpr int kOffFlag = kOffLFin + HG * 4;
  static constexpr int kLdsBytes = kOffFlag + 4 * W;
  static_assert(kDB * kHB == 8, "every wave holds 8 output blocks");
};

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

// Index entry of token `tok` of sub-tile `s` in the unit range that starts at unit `t0` of `row`.
template <bool EXTRA>
__device__ __forceinline__ int load_index(const DecodeParams& p, int row, int t0, int s, int tok) {
  const int unit = t0 + (s >> 1);
  const int half = s & 1;
  if (!EXTRA || unit < p.tiles_k) {
    const int pos = unit * kUnitTokens + half * kSubTokens + tok;
    return pos < p.topk ? p.idx[(int64_t)row * p.topk + pos] : -1;
  }
  const int pos = (unit - p.tiles_k) * kUnitTokens + half * kSubTokens + tok;
  return pos < p.extra_topk ? p.xidx[(int64_t)row * p.extra_topk + pos] : -1;
}

// Value of lane (lane ^ 16); `lane` is the caller's (opaque) lane id.
__device__ __forceinline__ float xor16(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 16) << 2,
                                                                __builtin_bit_cast(int, v)));
}

// Lane id from the exec-mask counters (cheap to recompute anywhere).
// The empty asm makes each call's result opaque, so the compiler recomputes lane-derived offsets
// where they are used instead of hoisting dozens of them out of the loops.
__device__ __forceinline__ int lane_id() {
  int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

// Workgroup barriers written out so that the direct-to-LDS gather of the next sub-tile can stay in
// flight across the mid-tile barrier: `barrier_all` waits for this wave's outstanding global->LDS
// copies and LDS accesses, `barrier_lds` only for LDS accesses. The memory clobber keeps the
// compiler from moving memory accesses across either barrier.
__device__ __forceinline__ void barrier_all() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One lane's 16-byte global -> LDS copy (global_load_lds_dwordx4): the wave's active lanes write
// LDS bytes m0 + 16 * lane. Issued as inline asm so that the compiler does not treat every later LDS
// read as possibly aliasing it (which would make it wait for the copy right away); completion is
// awaited explicitly by barrier_all's vmcnt(0). m0 is saved and restored around the copy, and
// `lds_base` must be wave-uniform.
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gptr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int W, bool EXTRA>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_decode_kernel(DecodeParams p) {
  using C = DecodeCfg<W>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];
  __shared__ __attribute__((aligned(16))) char rawbuf[2 * C::kRawBytes];   // double-buffered records

  // The wave index is uniform: keep it (and everything derived from it) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int head_base = blockIdx.y * C::HG;

  char* vslice = smem + C::kOffV + wave * C::kVBytes;
  char* pbuf = smem + C::kOffP;
  float* alpha_s = reinterpret_cast<float*>(smem + C::kOffAlpha);
  float* mfin_s = reinterpret_cast<float*>(smem + C::kOffMFin);
  float* lfin_s = reinterpret_cast<float*>(smem + C::kOffLFin);
  int* flag_s = reinterpret_cast<int*>(smem + C::kOffFlag);

  // This part's units run from (sc[0], sc[1]) to the exclusive end (sc[2], sc[3]); they are walked
  // row segment by row segment without any division.
  const int32_t* sc = p.sched + blockIdx.x * 8;
  int row = sc[0];
  int t0 = sc[1];
  const int end_row = sc[2];
  const int end_tile = sc[3];
  const int slot_first = sc[4];
  bool first_seg = true;

  while (row < end_row || (row == end_row && t0 < end_tile)) {
    // Lane-derived indices are recomputed from an opaque copy of the lane id in each row segment
    // (and again in each sub-tile below) rather than kept live across the whole kernel.
    int lane = lane_id();
    const int tok = lane & 31;      // token of this lane in the gather
    const int hh = lane >> 5;       // which chunk of a chunk pair this lane gathers
    const int t16 = lane & 15;      // QK^T: token (A operand) / head (B operand, C column)
    const int q4 = lane >> 4;       // QK^T: 16-dim group inside a 64-dim step
    // QK^T role: lane (t16, q4) holds Q of head my_head for dims 64c + 16*q4 .. +15.
    const int my_head = head_base + 16 * wave + t16;

    const int t1 = row < end_row ? p.tiles : end_tile;
    const int nsub = 2 * (t1 - t0);
    const int split_base = p.split_ptr[row];
    const int nsplit = p.split_ptr[row + 1] - split_base;
    const int slot = first_seg ? slot_first : split_base;

    // Q (B operand): heads past h_q load a copy of the last head; their results are never stored.
    // Q (B operand): heads past h_q load a copy of the last head; their results are never stored.
    bf16x8 qreg[8][2];
    {
      const int qh = min(my_head, p.h_q - 1);
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          p.q + ((int64_t)row * p.h_q + qh) * kHeadDim + 16 * q4);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qreg[c][0] = __builtin_bit_cast(bf16x8, qp[8 * c]);
        qreg[c][1] = __builtin_bit_cast(bf16x8, qp[8 * c + 1]);
      }
    }

    f32x16 oacc[C::kDB][C::kHB];
#pragma unroll
    for (int d = 0; d < C::kDB; ++d)
#pragma unroll
      for (int b = 0; b < C::kHB; ++b) oacc[d][b] = f32x16{};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;

    // ---- gather: direct HBM -> LDS copies of sub-tile s+1 while sub-tile s is computed.
    // Wave instruction q moves chunks 2q (lanes 0..31) and 2q+1 (lanes 32..63) of the 32 tokens;
    // lanes whose token is ignored, and lanes past the record, issue nothing.
    auto issue = [&](int s, int my_idx, char* buf, bool& is_fp4) -> uint32_t {
      const int unit = t0 + (s >> 1);
      is_fp4 = EXTRA && unit >= p.tiles_k;
      const bool valid = my_idx >= 0;
      const uint32_t bal = (uint32_t)__ballot(valid);   // lanes 0..31 carry tokens 0..31
      const int nq = is_fp4 ? (kFp4Chunks / 2) : 17;
      const int nch = is_fp4 ? kFp4Chunks : kFp8Chunks;
      const uint32_t buf_lds = __builtin_amdgcn_readfirstlane(lds_addr(buf));
      // per-lane record pointer, already advanced to this lane's chunk of each chunk pair
      const uint8_t* lane_base = (is_fp4 ? p.xc + (int64_t)(valid ? my_idx : 0) * kFp4Rec
                                         : p.kc + (int64_t)(valid ? my_idx : 0) * kFp8Rec) + 16 * hh;
#pragma unroll
      for (int j = 0; j < C::kNQ; ++j) {
        const int qi = wave + W * j;                      // uniform: chunks 2qi (+0) and 2qi+1 (+16)
        if (qi < nq) {
          const uint32_t dst = __builtin_amdgcn_readfirstlane(buf_lds + 1024 * qi);
          const bool ok = valid && (2 * qi + 1 < nch || hh == 0);
          if (ok) copy16_to_lds(lane_base + 32 * qi, dst);
        }
      }
      return bal;
    };

    int idx_cur = load_index<EXTRA>(p, row, t0, 0, tok);
    bool fp4_next = false;
    uint32_t mask_next = issue(0, idx_cur, rawbuf, fp4_next);
    int idx_next = nsub > 1 ? load_index<EXTRA>(p, row, t0, 1, tok) : -1;

    for (int s = 0; s < nsub; ++s) {
      char* raw = rawbuf + (s & 1) * C::kRawBytes;
      char* raw_other = rawbuf + ((s + 1) & 1) * C::kRawBytes;
      const uint32_t mask = mask_next;
      const bool is_fp4 = EXTRA && fp4_next;
      const int lane = lane_id();
      const int tok = lane & 31;
      const int hh = lane >> 5;
      const int t16 = lane & 15;
      const int q4 = lane >> 4;
      barrier_all();
      if (s + 1 < nsub) {
        mask_next = issue(s + 1, idx_next, raw_other, fp4_next);
        idx_next = (s + 2 < nsub) ? load_index<EXTRA>(p, row, t0, s + 2, tok) : -1;
      }
      if (mask != 0) {
        // ---------------- QK^T with in-register dequant (two token blocks, two MFMA chains).
        // The LDS read of step c+1 is issued before step c is converted; the scheduling barrier
        // keeps the compiler from hoisting every read of the loop (which would exhaust registers).
        f32x4 sacc[2] = {f32x4{}, f32x4{}};
        if (!is_fp4) {
          u32x4 scl[2], rn[2];
          const uint32_t sc_shift = 8 * (q4 >> 1);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            scl[tb] = lds_read16(raw, (32 * kSubTokens + 16 * tb + t16) * 16);   // e8m0 scales
            rn[tb] = lds_read16(raw, ((0 + q4) * kSubTokens + 16 * tb + t16) * 16);
          }
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            u32x4 r[2] = {rn[0], rn[1]};
            if (c + 1 < 8) {
#pragma unroll
              for (int tb = 0; tb < 2; ++tb)
                rn[tb] = lds_read16(raw, ((4 * (c + 1) + q4) * kSubTokens + 16 * tb + t16) * 16);
            }
            // 32-dim scale block 2c + q4/2: word c/2 of the 16 scale bytes (a constant index),
            // byte 2(c&1) + q4/2 inside it (a per-lane shift)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              const uint32_t sb = __builtin_amdgcn_ubfe(scl[tb][c >> 1], 16 * (c & 1) + sc_shift, 8);
              bf16x8 a0, a1;
              dequant_fp8_16(r[tb], sb, a0, a1);
              sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[c][0], sacc[tb], 0, 0, 0);
              sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[c][1], sacc[tb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          u32x2 rn[2];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            rn[tb] = *reinterpret_cast<const u32x2*>(
                raw + ((q4 >> 1) * kSubTokens + 16 * tb + t16) * 16 + 8 * (q4 & 1));
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            // dims 64c + 16*q4 .. +15 = bytes 32c + 8*q4 .. +7 = chunk 2c + q4/2, offset 8*(q4&1);
            // their e4m3 scale is byte j % 16 of chunk 16 + j / 16, j = 4c + q4
            u32x2 r[2] = {rn[0], rn[1]};
            if (c + 1 < 8) {
#pragma unroll
              for (int tb = 0; tb < 2; ++tb)
                rn[tb] = *reinterpret_cast<const u32x2*>(
                    raw + ((2 * (c + 1) + (q4 >> 1)) * kSubTokens + 16 * tb + t16) * 16 + 8 * (q4 & 1));
            }
            const int j = 4 * c + q4;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              const uint32_t sb = *reinterpret_cast<const uint8_t*>(
                  raw + ((16 + (j >> 4)) * kSubTokens + 16 * tb + t16) * 16 + (j & 15));
              bf16x8 a0, a1;
              dequant_fp4_16(r[tb][0], r[tb][1], e4m3_to_f32(sb), a0, a1);
              sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[c][0], sacc[tb], 0, 0, 0);
              sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[c][1], sacc[tb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---------------- this wave's PV dim slice of the same tokens, dequantized for the V operand
        // (zero for ignored tokens) into the wave's private LDS slice, token-major.
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = 16 * tb + t16;
          const bool tok_valid = (mask >> t) & 1u;
#pragma unroll
          for (int cs = 0; cs < C::kSlice / 64; ++cs) {
            const int c = wave * (C::kSlice / 64) + cs;                       // uniform
            bf16x8 a0, a1;
            if (!is_fp4) {
              const u32x4 r = lds_read16(raw, ((4 * c + q4) * kSubTokens + t) * 16);
              const uint32_t sb = *reinterpret_cast<const uint8_t*>(
                  raw + (32 * kSubTokens + t) * 16 + 2 * c + (q4 >> 1));   // e8m0 of the block
              dequant_fp8_16(r, sb, a0, a1);
            } else {
              const u32x2 r = *reinterpret_cast<const u32x2*>(
                  raw + ((2 * c + (q4 >> 1)) * kSubTokens + t) * 16 + 8 * (q4 & 1));
              const int j = 4 * c + q4;
              const uint32_t sb = *reinterpret_cast<const uint8_t*>(
                  raw + ((16 + (j >> 4)) * kSubTokens + t) * 16 + (j & 15));
              dequant_fp4_16(r[0], r[1], e4m3_to_f32(sb), a0, a1);
            }
            const int off = t * C::kVStride + (64 * cs + 16 * q4) * 2;
            lds_write16(vslice, off, tok_valid ? __builtin_bit_cast(u32x4, a0) : u32x4{});
            lds_write16(vslice, off + 16, tok_valid ? __builtin_bit_cast(u32x4, a1) : u32x4{});
          }
        }

        // ---------------- online softmax for head 16*wave + t16; sacc[tb][i] is token 16tb+4q4+i
        float x[8];
        float mx = -__builtin_inff();
        const uint32_t mq = mask >> (4 * q4);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = ((mq >> (16 * tb + i)) & 1u) ? sacc[tb][i] * p.scale_log2
                                                          : -__builtin_inff();
            x[4 * tb + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, xor16(mx, lane));
        mx = max_xor32(mx);
        const float m_new = fmaxf(m_run, mx);
        const bool resc = m_new > m_run + 8.0f;    // also true for the first sub-tile with a token
        float alpha = 1.0f;
        if (resc) {
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // exp2(-inf) = 0
          m_run = m_new;
        }
        const bool live = m_run != -__builtin_inff();
        float ls = 0.0f;
        char* prow = pbuf + (16 * wave + t16) * C::kPStride;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          bf16x4 pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = live ? __builtin_amdgcn_exp2f(x[4 * tb + i] - m_run) : 0.0f;
            pk[i] = (__bf16)e;     // bf16 only as the PV operand; the running sum stays in fp32
            ls += e;
          }
          *reinterpret_cast<bf16x4*>(prow + (16 * tb + 4 * q4) * 2) = pk;
        }
        ls += xor16(ls, lane);
        ls = sum_xor32(ls);
        l_run = l_run * alpha + ls;
        const uint64_t any_resc = __ballot(resc);
        if (q4 == 0) alpha_s[16 * wave + t16] = alpha;
        if (lane == 0) flag_s[wave] = any_resc != 0;
      }
      barrier_lds();

      if (mask != 0) {
        // ---------------- PV: O^T[this wave's dims x all heads] += V^T P^T
#pragma unroll
        for (int b = 0; b < C::kHB; ++b) {
          if (flag_s[2 * b] | flag_s[2 * b + 1]) {
            const float a = alpha_s[32 * b + (lane & 31)];
#pragma unroll
            for (int d = 0; d < C::kDB; ++d) oacc[d][b] *= a;
          }
        }
        const int g = lane >> 4, j = lane & 15;
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        // V^T operand for (ks, d): two transposed reads of the private slice, lane (dim, 8 tokens)
        auto load_v = [&](int ks, int d) -> bf16x8 {
          const int row0 = 16 * ks + 8 * (g >> 1) + (j >> 2);
          const int col = 32 * d + 16 * (g & 1) + 4 * (j & 3);
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(vslice + row0 * C::kVStride + col * 2));
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(vslice + (row0 + 4) * C::kVStride + col * 2));
          return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 av_next = load_v(0, 0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 pb[C::kHB];
#pragma unroll
          for (int b = 0; b < C::kHB; ++b)
            pb[b] = *reinterpret_cast<const bf16x8*>(
                pbuf + (32 * b + (lane & 31)) * C::kPStride + (16 * ks + 8 * hh) * 2);
#pragma unroll
          for (int d = 0; d < C::kDB; ++d) {
            const bf16x8 av = av_next;
            if (d + 1 < C::kDB) av_next = load_v(ks, d + 1);
            else if (ks == 0) av_next = load_v(1, 0);
#pragma unroll
            for (int b = 0; b < C::kHB; ++b)
              oacc[d][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[b], oacc[d][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    __syncthreads();

    // ---------------- epilogue for this row segment
    lane = lane_id();
    const int t16e = lane & 15, q4e = lane >> 4, hhe = lane >> 5;
    if (q4e == 0) {
      mfin_s[16 * wave + t16e] = m_run;
      lfin_s[16 * wave + t16e] = l_run;
    }
    __syncthreads();
    const bool final_out = nsplit == 1;
#pragma unroll
    for (int b = 0; b < C::kHB; ++b) {
      const int hl = 32 * b + (lane & 31);
      const int head = head_base + hl;
      if (head < p.h_q) {
        const float l = lfin_s[hl];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
        for (int d = 0; d < C::kDB; ++d) {
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            const int dim = wave * C::kSlice + 32 * d + 8 * jb + 4 * hhe;
            if (final_out) {
              bf16x4 o;
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = (__bf16)(oacc[d][b][4 * jb + i] * inv);
              *reinterpret_cast<bf16x4*>(p.out + ((int64_t)row * p.h_q + head) * kHeadDim + dim) = o;
            } else {
              f32x4 o;
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = oacc[d][b][4 * jb + i] * inv;
              *reinterpret_cast<f32x4*>(p.part_o + ((int64_t)slot * p.h_q + head) * kHeadDim + dim) = o;
            }
          }
        }
      }
    }
    const int head_e = head_base + 16 * wave + t16e;
    if (q4e == 0 && head_e < p.h_q) {
      const float lse = l_run > 0.0f ? (m_run + __log2f(l_run)) * 0.69314718055994530942f
                                     : -__builtin_inff();
      if (final_out)
        p.lse[(int64_t)row * p.h_q + head_e] = lse;
      else
        p.part_lse[(int64_t)slot * p.h_q + head_e] = lse;
    }
    __syncthreads();
    ++row;
    t0 = 0;
    first_seg = false;
  }
}

int launch_sparse_decode(const DecodeParams& p, int parts, int groups, int waves, hipStream_t stream) {
  dim3 grid(parts, groups);
  const bool extra = p.extra_topk > 0;
  switch (waves * 2 + (extra ? 1 : 0)) {
    case 8: hipLaunchKernelGGL((sparse_decode_kernel<4, false>), grid, dim3(256), 0, stream, p); break;
    case 9: hipLaunchKernelGGL((sparse_decode_kernel<4, true>), grid, dim3(256), 0, stream, p); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
