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
// (HG = 64 here). The workgroup is two halves of W = HG / 16 = 4 waves (eight waves, two per SIMD,
// one workgroup per CU); half h takes the sub-tiles s = h (mod 2) of the part with its own LDS
// areas, and the halves' softmax states are merged by log-sum-exp at the end of each row segment.
// Every wave has the same register footprint: Q of 16 heads (64 VGPRs; each head's row is copied
// once per workgroup into LDS at a row segment's start and read from there) and an fp32 output
// accumulator of 8 MFMA blocks. Each 64-slot unit runs as two sub-tiles of 32 tokens:
//   1. indices  each wave copies the sub-tile's 32 index entries into its LDS index ring
//               (global_load_lds_dword), 2 * kDepth sub-tiles ahead of the compute.
//   2. gather   all lanes copy 16-byte chunks of the selected records (data and scales together,
//               one contiguous record per token) straight from HBM into LDS with
//               global_load_lds_dwordx4, kDepth sub-tiles ahead, chunk-major: slot(chunk c, token t)
//               = c * 32 + t, so one wave instruction fills a contiguous 1 KB (chunks 2q, 2q+1).
//               A fixed number of copies per wave and sub-tile lets one s_waitcnt wait for
//               exactly the oldest sub-tile while the newer ones stay in flight.
//   3. dequant  wave w converts its 512 / W dims of the 32 tokens to bf16 (the record's own scale,
//               in registers) into its slice of the LDS tile (an ignored token's zero record
//               decodes to zeros); the W slices form the sub-tile's bf16 tile, written once and
//               read by every wave.
//   4. QK^T     wave w owns heads 16w..16w+15: v_mfma_f32_16x16x32_bf16 of tile rows (conflict-free
//               ds_read_b128) against its register-resident Q, S^T[16 tokens x 16 heads] over all
//               512 dims.
//   5. softmax  lanes n, n+16, n+32, n+48 share head n: masked max over the sub-tile, lazy rescale of
//               the running max (only when it grows by more than 2^8), exp2, bf16 P to LDS, the
//               running sum of the fp32 probabilities (so lse carries no bf16 rounding), and a
//               per-wave "rescale needed" flag.
//   6. PV       wave w accumulates O^T[its dim slice x all HG heads] += V^T P^T with
//               v_mfma_f32_32x32x16_bf16; V^T comes from its own tile slice via ds_read_b64_tr_b16,
//               P^T from LDS.
//   7. merge    half h keeps the 32-head O block h and passes the other block, with its per-head
//               maximum and sum, to the other half through LDS; each half rescales both
//               contributions to its heads to the larger maximum, adds them and normalises.
//   8. epilogue the normalised rows are staged in bf16 in LDS and stored as whole 1 KB head rows by
//               all eight waves. One split: out = O / l in bf16 and lse = ln(2) * (m + log2 l);
//               several splits: the normalised partial (bf16) and its lse (fp32) go to the
//               workspace for the merge kernel.

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

// Gather distance in iterations of a half: the records of iteration k + kDepth are requested while
// iteration k is computed, and its index entries kDepth iterations before that.
constexpr int kDepth = 1;
// Each workgroup runs two independent halves of W waves over the even and odd sub-tiles of its
// part (two waves per SIMD), merged by log-sum-exp at the end of every row segment.
constexpr int kHalves = 2;

template <int W>
struct DecodeCfg {
  static constexpr int HG = 16 * W;                 // heads per workgroup
  static constexpr int kThreads = 64 * W;
  static constexpr int kSlice = kHeadDim / W;       // dims per wave (dequant and PV)
  static constexpr int kDB = kSlice / 32;           // 32-dim output blocks per wave
  static constexpr int kHB = HG / 32;               // 32-head output blocks
  static constexpr int kNQ = (17 + W - 1) / W;      // record copies per wave per sub-tile
  static constexpr int kRawSlots = kDepth + 1;
  // 34 chunks of 32 tokens: the copy of fp8 chunk pair 16 also writes a (zero) 34th chunk
  static constexpr int kRawSlotBytes = 34 * kSubTokens * 16;
  static constexpr int kIdxSlots = kDepth + 1;      // index rows per wave
  static constexpr int kVStride = kSlice * 2 + 16;  // bytes per token row of a tile slice
  static constexpr int kVBytes = kSubTokens * kVStride;
  static constexpr int kPStride = 80;               // bytes per head row of P (32 bf16 + pad)
  static constexpr int kOffV = 0;
  static constexpr int kOffP = kOffV + W * kVBytes;
  static constexpr int kOffAlpha = kOffP + HG * kPStride;
  static constexpr int kOffMFin = kOffAlpha + HG * 4;
  static constexpr int kOffLFin = kOffMFin + HG * 4;
  static constexpr int kOffFlag = kOffLFin + HG * 4;
  static constexpr int kOffIdx = kOffFlag + 16;
  static constexpr int kOffDummy = kOffIdx + W * kIdxSlots * kSubTokens * 4;
  static constexpr int kLdsBytes = kOffDummy + 1024;
  // the steady-state wait: everything but the copies of the kDepth - 1 newest sub-tiles
  static constexpr int kVmcntAfterOldest = (kDepth - 1) * (kNQ + 1);
  static_assert(kDB * kHB == 8, "every wave holds 8 output blocks");
  static_assert(W * kNQ * 2 >= kFp8Chunks, "the copies cover an fp8 record");
  static_assert(kOffIdx % 16 == 0 && kOffDummy % 16 == 0, "aligned LDS areas");
  static_assert(kHalves * (kLdsBytes + kRawSlots * kRawSlotBytes) <= 160 * 1024, "LDS of one workgroup");
  static_assert(kLdsBytes % 16 == 0 && (kRawSlots * kRawSlotBytes) % 16 == 0, "aligned halves");
  static_assert(kVmcntAfterOldest < 64, "vmcnt counts up to 63");
};

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
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

// One 4-byte global -> LDS copy per lane of the lower half-wave (global_load_lds_dword with EXEC =
// lanes 0..31): LDS bytes m0 + 4 * lane. Issued with that EXEC inside the assembly, so no branch can
// skip it; m0 and EXEC are restored.
__device__ __forceinline__ void copy4_to_lds_lo32(const void* gptr, uint32_t lds_base) {
  uint32_t saved_m0;
  uint64_t saved_exec;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 0xffffffff\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %3, off\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0), "=&s"(saved_exec)
      : "s"(lds_base), "v"(gptr)
      : "memory");
}

// Waits until only the copies of the kDepth - 1 newest sub-tiles are outstanding in this wave (its
// copies of the oldest sub-tile and the index row issued right after them have landed) and that all
// of its LDS accesses are done, then synchronises the workgroup.
#define MLA_NARROW_VMCNT 0
static_assert(MLA_NARROW_VMCNT == DecodeCfg<4>::kVmcntAfterOldest, "wait count of the gather pipeline");
#define MLA_STR2(x) #x
#define MLA_STR(x) MLA_STR2(x)
__device__ __forceinline__ void wait_gather_and_barrier() {
  asm volatile("s_waitcnt vmcnt(" MLA_STR(MLA_NARROW_VMCNT) ") lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Read-only zeros standing in for the records of ignored tokens and for unused copies (an fp8
// record's 34th chunk included): every gather copy has a valid source.
__device__ const uint8_t g_zero_record[34 * 16] = {};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int W, bool EXTRA>
__global__ __launch_bounds__(64 * W * kHalves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_decode_kernel(DecodeParams p) {
  using C = DecodeCfg<W>;
  constexpr int kRawHalfBytes = C::kRawSlots * C::kRawSlotBytes;
  // both halves' areas, then both halves' gathered records; at the end of a row segment the whole
  // array holds the merge's exchange (half 1's O, then every half's m and l)
  constexpr int kMergeOBytes = W * C::kDB * C::kHB * 16 * 64 * 4;
  static_assert(kMergeOBytes + kHalves * 2 * C::HG * 4 <= kHalves * (C::kLdsBytes + kRawHalfBytes),
                "the merge exchange fits in the workgroup's LDS");
  __shared__ __attribute__((aligned(16))) char lds[kHalves * (C::kLdsBytes + kRawHalfBytes)];
  // epilogue staging of the bf16 output rows (16 bytes of padding per 1 KB row)
  constexpr int kStageRow = 2 * kHeadDim + 16;
  static_assert(C::HG * kStageRow <= kMergeOBytes, "the output staging reuses the O exchange area");
  static_assert(C::kHB == kHalves, "each half keeps one 32-head O block");

  // The wave index is uniform: keep it (and everything derived from it) in scalar registers.
  // Half h (waves hW .. hW+W-1) takes the sub-tiles s = h (mod 2) of the part, with its own LDS
  // areas; `wave` is the index inside the half.
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave_all / W;
  const int wave = wave_all % W;
  char* const smem = lds + half * C::kLdsBytes;
  char* const rawbuf = lds + kHalves * C::kLdsBytes + half * kRawHalfBytes;
  const int head_base = blockIdx.y * C::HG;

  char* vslice = smem + C::kOffV + wave * C::kVBytes;
  // Q staging at a row segment's start: head row hr (bf16, 1 KB) in the tile area of half hr / 32
  // at (hr % 32) * kQRow bytes; the 16-byte padding keeps 16 rows at one offset on distinct banks.
  constexpr int kQRow = 2 * kHeadDim + 16;
  static_assert(32 * kQRow <= W * C::kVBytes && C::HG == 64, "the Q staging fits in the tile areas");
  auto q_row = [&](int hr) -> char* {
    return lds + (hr >> 5) * C::kLdsBytes + C::kOffV + (hr & 31) * kQRow;
  };
  char* pbuf = smem + C::kOffP;
  float* alpha_s = reinterpret_cast<float*>(smem + C::kOffAlpha);
  int* flag_s = reinterpret_cast<int*>(smem + C::kOffFlag);

  // This part's units run from (row, t0) to the exclusive end (end_row, end_tile); they are walked
  // row segment by row segment without any division.
  int row, t0, end_row, end_tile, slot_first;
  if (p.prefill_parts > 0) {
    // whole rows, evenly: part b takes prefill_q rows, plus one for the first prefill_r parts
    const int b = (int)blockIdx.x;
    row = b * p.prefill_q + min(b, p.prefill_r);
    end_row = row + p.prefill_q + (b < p.prefill_r ? 1 : 0);
    t0 = 0;
    end_tile = 0;
    slot_first = 0;
  } else {
    const int32_t* sc = p.sched + blockIdx.x * 8;
    row = sc[0];
    t0 = sc[1];
    end_row = sc[2];
    end_tile = sc[3];
    slot_first = sc[4];
  }
  bool first_seg = true;

  while (row < end_row || (row == end_row && t0 < end_tile)) {
    // Lane-derived indices are recomputed from an opaque copy of the lane id in each row segment
    // (and again in each sub-tile below) rather than kept live across the whole kernel.
    int lane = lane_id();
    const int t16 = lane & 15;      // QK^T: token (A operand) / head (B operand, C column)
    const int q4 = lane >> 4;       // QK^T: 16-dim group inside a 64-dim step
    // QK^T role: lane (t16, q4) holds Q of head my_head for dims 64c + 16*q4 .. +15.
    const int my_head = head_base + 16 * wave + t16;

    const int t1 = row < end_row ? p.tiles : end_tile;
    const int nsub = 2 * (t1 - t0);

    // Q (B operand): heads past h_q load a copy of the last head; their results are never stored.
    // Q (B operand): heads past h_q load a copy of the last head; their results are never stored.
    // Q rows of the workgroup's heads are copied once into LDS (8 head rows of 1 KB per wave, row
    // hr of half hr / 32's tile area at (hr % 32) * kQRow, free until the first dequantization) and
    // read into registers from there below, instead of every half loading all of Q from memory.
    auto copy_q = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int hr = 8 * wave_all + i;
        const int qh = min(head_base + hr, p.h_q - 1);
        const uint16_t* src = p.q + ((int64_t)row * p.h_q + qh) * kHeadDim + 8 * lane_id();
        copy16_to_lds(src, __builtin_amdgcn_readfirstlane(lds_addr(q_row(hr))));
      }
    };
    bf16x8 qreg[8][2];

    f32x16 oacc[C::kDB][C::kHB];
#pragma unroll
    for (int d = 0; d < C::kDB; ++d)
#pragma unroll
      for (int b = 0; b < C::kHB; ++b) oacc[d][b] = f32x16{};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;

    // ---- asynchronous stages, per half. Iteration k of half h handles sub-tile j = 2k + h. Its 32
    // index entries are copied to this wave's index ring slot k % kIdxSlots, 2 * kDepth iterations
    // ahead of its compute; its records are gathered into raw slot k % kRawSlots kDepth iterations
    // ahead. Every wave issues exactly kNQ record copies and one index copy per iteration, all with
    // a non-empty EXEC, whatever the sub-tile holds (ignored tokens, the missing 34th chunk of an
    // fp8 record, an fp4 sub-tile's unused copies and sub-tiles past the segment read a zero
    // record; unused copies land in a dummy LDS area), so that one s_waitcnt with a fixed count
    // waits for exactly the oldest iteration's copies.
    const int nk = (nsub + kHalves - 1) / kHalves;     // iterations of each half
    const uint32_t idx_ring = lds_addr(smem + C::kOffIdx + wave * C::kIdxSlots * kSubTokens * 4);
    auto sub_count = [&](int j, int& pos0, bool& fp4) -> int {   // entries of j's index array
      const int unit = t0 + (j >> 1);
      fp4 = EXTRA && unit >= p.tiles_k;
      if (!fp4) { pos0 = unit * kUnitTokens + (j & 1) * kSubTokens; return p.topk; }
      pos0 = (unit - p.tiles_k) * kUnitTokens + (j & 1) * kSubTokens;
      return p.extra_topk;
    };
    auto load_idx = [&](int k) {
      const int j = kHalves * k + half;
      const int32_t* src = p.sched;                  // a valid address when j is past the segment
      if (j < nsub) {
        int pos0;
        bool fp4;
        const int count = sub_count(j, pos0, fp4);
        if (count > 0)
          src = (fp4 ? p.xidx : p.idx) + (int64_t)row * count + min(pos0 + (lane_id() & 31), count - 1);
      }
      copy4_to_lds_lo32(src, __builtin_amdgcn_readfirstlane(idx_ring + (k % C::kIdxSlots) * kSubTokens * 4));
    };
    // Gather of iteration k's sub-tile (its index entries have landed); returns its validity mask.
    auto gather = [&](int k) -> uint32_t {
      const int j = kHalves * k + half;
      const int ln = lane_id();
      const int t = ln & 31, hw = ln >> 5;
      int pos0 = 0;
      bool fp4 = false;
      const int count = j < nsub ? sub_count(j, pos0, fp4) : 0;
      const int v = *reinterpret_cast<const int*>(smem + C::kOffIdx +
                                                  (wave * C::kIdxSlots + k % C::kIdxSlots) * kSubTokens * 4 + 4 * t);
      const bool valid = pos0 + t < count && v >= 0;
      const uint32_t bal = (uint32_t)__ballot(valid);
      const int nq = fp4 ? kFp4Chunks / 2 : (kFp8Chunks + 1) / 2;
      const int nch = fp4 ? kFp4Chunks : kFp8Chunks;
      const uint8_t* rec = !valid ? g_zero_record
                                  : fp4 ? p.xc + (int64_t)v * kFp4Rec : p.kc + (int64_t)v * kFp8Rec;
      const uint32_t raw_lds = lds_addr(rawbuf + (k % C::kRawSlots) * C::kRawSlotBytes);
#pragma unroll
      for (int i = 0; i < C::kNQ; ++i) {
        const int qi = wave + W * i;                   // uniform: chunks 2qi (+0) and 2qi+1 (+16)
        const bool used = qi < nq;
        const uint8_t* src = used && 2 * qi + hw < nch ? rec + 32 * qi + 16 * hw : g_zero_record;
        const uint32_t dst = used ? raw_lds + 1024 * qi : lds_addr(smem + C::kOffDummy);
        copy16_to_lds(src, __builtin_amdgcn_readfirstlane(dst));
      }
      return bal;
    };

    // Prologue: index entries of iterations 0 .. kDepth-1, then the Q rows; as soon as the index
    // entries have landed (at most the 8 Q copies outstanding) the gathers of those iterations are
    // issued, each followed by the index copy kDepth further on, as in the loop, so that their
    // latency overlaps the Q traffic; then Q is awaited (at most the gathers' copies outstanding).
    static_assert(kDepth * (C::kNQ + 1) == 6, "wait count of the prologue");
#pragma unroll
    for (int k = 0; k < kDepth; ++k) load_idx(k);
    copy_q();
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    uint32_t mk[kDepth + 1];                          // validity masks of iterations k .. k+kDepth
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      mk[k] = gather(k);
      load_idx(k + kDepth);
    }
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __syncthreads();                                  // every wave's Q rows are in LDS
    {
      // lane (t16, q4) takes dims 64c + 16*q4 .. +15 of head my_head
      const char* qrow = q_row(16 * wave + t16) + 32 * q4;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qreg[c][0] = __builtin_bit_cast(bf16x8, lds_read16(qrow, 128 * c));
        qreg[c][1] = __builtin_bit_cast(bf16x8, lds_read16(qrow, 128 * c + 16));
      }
      // complete before any wave can reach the first dequantization, which overwrites these rows
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // The split bookkeeping is needed only by the epilogue. It is read after the segment's first
    // copies are issued, so its memory round trip overlaps theirs instead of delaying the Q load.
    const int split_base = p.split_ptr ? p.split_ptr[row] : 0;
    const int nsplit = p.split_ptr ? p.split_ptr[row + 1] - split_base : 1;
    const int slot = first_seg ? slot_first : split_base;

    // Both halves run nk iterations with the same three workgroup barriers each (a half whose
    // sub-tile is past the segment or fully ignored only skips the work between them).
    for (int k = 0; k < nk; ++k) {
      const int s = kHalves * k + half;
      const char* raw = rawbuf + (k % C::kRawSlots) * C::kRawSlotBytes;
      const uint32_t mask = mk[0];
      int pos0_s;
      bool is_fp4;
      sub_count(s, pos0_s, is_fp4);
      // The gather of this iteration (and the index entries of iteration k + kDepth) have landed
      // for every wave; every wave is done with the previous iteration's tile, P and raw slot.
      wait_gather_and_barrier();
      mk[kDepth] = gather(k + kDepth);
      load_idx(k + 2 * kDepth);
      const int lane = lane_id();
      const int t16 = lane & 15;
      const int q4 = lane >> 4;
      const int hh = lane >> 5;
      if (mask != 0) {
        // ---------------- this wave's dim slice of the sub-tile's 32 tokens, raw -> bf16 tile slice;
        // the four slices make up the tile that QK^T and PV read. An ignored token's record is the
        // zero record (all bytes 0, scale byte 0), which decodes to exact +0.
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = 16 * tb + t16;
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
              const int jj = 4 * c + q4;
              const uint32_t sb = *reinterpret_cast<const uint8_t*>(
                  raw + ((16 + (jj >> 4)) * kSubTokens + t) * 16 + (jj & 15));
              dequant_fp4_16(r[0], r[1], e4m3_to_f32(sb), a0, a1);
            }
            const int off = t * C::kVStride + (64 * cs + 16 * q4) * 2;
            lds_write16(vslice, off, __builtin_bit_cast(u32x4, a0));
            lds_write16(vslice, off + 16, __builtin_bit_cast(u32x4, a1));
          }
        }
      }
      barrier_lds();
      if (mask != 0) {
        // ---------------- QK^T from the bf16 tile: S^T[32 tokens x 16 heads] in two token blocks.
        // Step (c, h) multiplies dims 64c + 16*q4 + 8h .. +7 of token 16tb + t16 (slice c/2 of the
        // tile) with the same dims of Q.
        // The four K operands of step c + 1 are read before the four MFMAs of step c, and the two
        // token blocks alternate, so that neither an LDS read nor the previous MFMA on the same
        // accumulator is waited for right before each MFMA.
        f32x4 sacc[2] = {f32x4{}, f32x4{}};
        auto read_k = [&](int c, bf16x8 (&kb)[4]) {
          const char* kslice = smem + C::kOffV + (c >> 1) * C::kVBytes + ((c & 1) * 64 + 16 * q4) * 2;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const char* kp = kslice + (16 * tb + t16) * C::kVStride;
            kb[2 * tb] = __builtin_bit_cast(bf16x8, lds_read16(kp, 0));
            kb[2 * tb + 1] = __builtin_bit_cast(bf16x8, lds_read16(kp, 16));
          }
        };
        bf16x8 kbuf[2][4];
        read_k(0, kbuf[0]);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (c + 1 < 8) read_k(c + 1, kbuf[(c + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);         // keep those reads ahead of these MFMAs
          const bf16x8 (&kb)[4] = kbuf[c & 1];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[2 * tb + h], qreg[c][h], sacc[tb], 0, 0, 0);
        }

        // ---------------- online softmax for head 16*wave + t16; sacc[tb][i] is token 16tb+4q4+i
        float x[8];
        float mx = -__builtin_inff();
        if (mask == 0xFFFFFFFFu) {                   // all 32 tokens valid: no masking
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[4 * tb + i] = sacc[tb][i] * p.scale_log2;
              mx = fmaxf(mx, x[4 * tb + i]);
            }
        } else {
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
        // V^T operand for (ks, d): two transposed reads of the wave's own tile slice, lane (dim,
        // 8 tokens)
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
#pragma unroll
      for (int j = 0; j < kDepth; ++j) mk[j] = mk[j + 1];
    }
    // the copies issued past the segment's end land in unused slots; drain them before the slots
    // and the index ring are reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---------------- merge of the two halves (log-sum-exp) and staging of the output. Half h keeps
    // the 32-head O block h and hands its other block to the other half through LDS, with its
    // running maximum and sum per head. Each half then rescales both contributions to its heads to
    // the larger maximum, adds them, normalises by the combined sum and stages the result in bf16
    // in LDS (head rows kStageRow bytes apart). A half that saw no valid token (m = -inf) carries
    // no weight.
    lane = lane_id();
    const int t16e = lane & 15, q4e = lane >> 4, hhe = lane >> 5;
    float* const xbuf = reinterpret_cast<float*>(lds);                 // [to half][wave][d][r][lane]
    float* const ml = reinterpret_cast<float*>(lds + kMergeOBytes);   // [half][m, l][head]
    char* const stage = lds;                                           // after xbuf is consumed
    auto xoff = [&](int to, int d, int r) { return (((to * W + wave) * C::kDB + d) * 16 + r) * 64 + lane; };
    if (q4e == 0) {
      ml[(2 * half + 0) * C::HG + 16 * wave + t16e] = m_run;
      ml[(2 * half + 1) * C::HG + 16 * wave + t16e] = l_run;
    }
    if (half == 0) {
#pragma unroll
      for (int d = 0; d < C::kDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) xbuf[xoff(1, d, r)] = oacc[d][1][r];
    } else {
#pragma unroll
      for (int d = 0; d < C::kDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) xbuf[xoff(0, d, r)] = oacc[d][0][r];
    }
    __syncthreads();
    const float ninf = -__builtin_inff();
    // combined weights of head hl: a_h = 2^(m_h - m) / l with m the larger maximum and l the
    // combined sum (0 for a half without a valid token, and for both when the head saw none)
    auto weights = [&](int hl, float& a0, float& a1, float& m, float& l) {
      const float m0 = ml[0 * C::HG + hl], m1 = ml[2 * C::HG + hl];
      m = fmaxf(m0, m1);
      a0 = m0 == ninf ? 0.0f : __builtin_amdgcn_exp2f(m0 - m);
      a1 = m1 == ninf ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
      l = a0 * ml[1 * C::HG + hl] + a1 * ml[3 * C::HG + hl];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      a0 *= inv;
      a1 *= inv;
    };
    {
      const int hl = 32 * half + (lane & 31);
      float a0, a1, m, l;
      weights(hl, a0, a1, m, l);
      const float a_own = half == 0 ? a0 : a1, a_other = half == 0 ? a1 : a0;
      f32x16 on[C::kDB];
#pragma unroll
      for (int d = 0; d < C::kDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float own = half == 0 ? oacc[d][0][r] : oacc[d][1][r];
          on[d][r] = a_own * own + a_other * xbuf[xoff(half, d, r)];
        }
      __syncthreads();                          // xbuf is read by everyone before the staging
#pragma unroll
      for (int d = 0; d < C::kDB; ++d) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const int dim = wave * C::kSlice + 32 * d + 8 * jb + 4 * hhe;
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = (__bf16)on[d][4 * jb + i];
          *reinterpret_cast<bf16x4*>(stage + hl * kStageRow + 2 * dim) = o;
        }
      }
    }
    __syncthreads();
    // the final row, or this split's normalised partial (bf16 as well: the merge takes it back to
    // fp32 and weights it)
    const bool final_out = nsplit == 1;
    for (int hr = wave_all; hr < C::HG; hr += W * kHalves) {
      const int head = head_base + hr;
      if (head < p.h_q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + hr * kStageRow + 16 * lane);
        uint16_t* const dst = final_out ? p.out + ((int64_t)row * p.h_q + head) * kHeadDim
                                        : static_cast<uint16_t*>(p.part_o) + ((int64_t)slot * p.h_q + head) * kHeadDim;
        *reinterpret_cast<u32x4*>(dst + 8 * lane) = v;
      }
    }
    const int hs = 16 * wave + t16e;
    const int head_e = head_base + hs;
    if (half == 0 && q4e == 0 && head_e < p.h_q) {
      float a0, a1, m, l;
      weights(hs, a0, a1, m, l);
      const float lse = l > 0.0f ? (m + __log2f(l)) * 0.69314718055994530942f : -__builtin_inff();
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
    case 8: hipLaunchKernelGGL((sparse_decode_kernel<4, false>), grid, dim3(256 * kHalves), 0, stream, p); break;
    case 9: hipLaunchKernelGGL((sparse_decode_kernel<4, true>), grid, dim3(256 * kHalves), 0, stream, p); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
