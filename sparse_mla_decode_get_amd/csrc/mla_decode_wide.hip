// Sparse MLA decode kernel for gfx950, 128-head groups (h_q > 64).
//
// Same computation as the kernel in mla_decode.hip (page "flops/flashmla-decode-fp8-fp4-kv",
// sections "Arithmetic intensity" and "Workarounds"; page "deepseek-ai/FlashMLA", section "Key
// technical details"): per query row and head, one softmax over the row's selected tokens, key and
// value both the 512-dim latent decoded from the token's quantized record, negative indices ignored,
// natural-log lse returned beside the output.
//
// Layout of the work. One workgroup = 4 waves = one wave per SIMD, each wave with the full 512
// registers of its SIMD. Wave w owns query heads 32w..32w+31 of the head group for QK^T and the
// softmax:
//   Q      bf16, 32 heads x 512 dims, 128 VGPRs (B operand of the QK^T product)
//   S^T    fp32, 32 tokens x 32 heads per 32-token sub-tile, 16 VGPRs
// so the softmax (max, exp, sum, P) of a head never leaves its wave: P goes from the QK^T
// accumulator layout to the PV operand layout with v_permlane32_swap. O takes all 256 AGPRs of
// a wave as 16 MFMA blocks of 32x32, in one of two splits:
//   - the fp8 pipeline splits PV by dims: wave w accumulates O^T for dims 128w..128w+127 of all
//     128 heads, so each wave reads only its quarter of the V tile (8 KB per sub-tile instead of
//     32 KB); the P^T operands of the four head groups meet in a small LDS exchange buffer;
//   - the extra-cache variant splits PV by heads: O^T of the wave's own 32 heads, all 512 dims.
//
// Each selected record is gathered once (HBM -> LDS with global_load_lds_dwordx4) and dequantized
// once, by all four waves together (each takes 128 dims), into a bf16 tile [32 tokens][512 dims]
// that both products read: QK^T as row reads (ds_read_b128), PV as transposed reads
// (ds_read_b64_tr_b16). Three tiles and three raw buffers rotate through a software pipeline in
// which iteration s
//   - loads the indices of sub-tile s+6 and gathers the records of sub-tile s+4,
//   - runs QK^T of sub-tile s+1 (the scores land in VGPRs),
//   - runs PV of sub-tile s (O stays in the accumulation registers),
//   - runs the softmax of sub-tile s+1 and dequantizes sub-tile s+2.
// The index loads and gathers are issued as inline assembly that writes LDS directly; the only
// waits on them are the explicit vmcnt waits at the iteration barrier, whose counts follow the
// issue order (loads complete in order).

#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// One all-zero fp8 record (its e8m0 scale byte 0 decodes to the scale 0.0): the gather source of
// ignored tokens and of sub-tiles outside the segment in the fp8 pipeline, so that their rows
// dequantize to exact zeros whatever the cache holds. The nonzero tag after the record gives the
// object an explicit initializer, so its zeros are stored in the code object (read-only data)
// instead of an uninitialized section.
struct alignas(16) ZeroRecord {
  uint8_t bytes[1024];
  uint32_t tag;
};
__device__ const ZeroRecord g_zero = {{}, 1u};

// Score added to ignored tokens by the extra QK^T k-step (bf16 -2^100): after scaling it is far
// below any real score, so its probability is exactly 0 and it never wins a maximum.
constexpr uint32_t kIgnoredScoreBits = 0xF180u;

constexpr int kWaves = 4;
constexpr int kGroupHeads = 32 * kWaves;
// bf16 tile: token row r at r * 1088 bytes (1 KB of data and 64 bytes of padding); its 16-byte
// chunk c (dims 8c .. 8c+7) is stored at chunk position c ^ tile_xor(r), which only permutes the
// chunks within aligned groups of four. The padding moves each row by four 4-bank groups and the
// XOR picks among the four of a group, so every access pattern of the kernel is free of LDS bank
// conflicts:
//   - reads are served 256 bytes at a time: 16 rows at one chunk (K row reads) hit 16 different
//     4-bank groups, and so do 4 rows x 4 consecutive chunks (the transposed V reads);
//   - 16-byte writes are served 8 lanes (128 bytes, 32 banks) at a time: 8 consecutive rows at one
//     chunk (the dequant writes) hit 8 different 4-bank groups of 32 banks, which needs different
//     XOR values among the even rows and among the odd rows of each group of 8.
// Since the XOR leaves the chunk index above bit 1 alone, operand addresses differ from a few
// per-lane bases by immediates.
constexpr int kTileStride = 1088;
constexpr int kTileBytes = kSubTokens * kTileStride;    // 34816
constexpr int kRawBytes = kFp8Chunks * kSubTokens * 16; // 16896, chunk-major [chunk][token][16 B]
constexpr int kIdxBytes = kSubTokens * 4;     // one index slot (lanes 0..31 write it)
// epilogue staging of the bf16 output: 32 rows of 1 KB per wave, from the start of LDS, 1032
// bytes apart (each row moves by two banks, so 32 lanes writing 8 bytes to 32 rows hit 64
// different banks, and a row is read contiguously)
constexpr int kStageRow = 1032;
constexpr int kStageBytes = 32 * kStageRow;
constexpr int kFusedRow = kFp8Rec;            // fused decode: one fp8 record per staged head row
static_assert(32 * kFusedRow <= kStageBytes, "the fp8 records fit the bf16 staging");
constexpr int kStages = 3;
constexpr int kOffRaw = kStages * kTileBytes;
constexpr int kOffIdx = kOffRaw + kStages * kRawBytes;
// P^T exchange buffer of the fp8 pipeline: the B operand of PV for the 4 head groups and 2 token
// halves of one sub-tile, 16 bytes per lane (head group g, half ks at 1024 (2 g + ks))
constexpr int kPBytes = kWaves * 2 * 64 * 16;
// The rest of the layout depends on the variant. The fp8 pipeline shares one index ring among the
// waves (each wave loads 8 of a slot's 32 entries) and holds the P^T exchange buffer; the
// extra-cache variant gives every wave its own ring and exchanges nothing.
template <bool EXTRA>
struct Lds {
  static constexpr int kIdxSlots = EXTRA ? kWaves * kStages : kStages;
  static constexpr int kOffFlags = kOffIdx + kIdxSlots * kIdxBytes;
  static constexpr int kOffScan = kOffFlags + 16;   // per-wave last live sub-tile, two segment buffers
  static constexpr int kOffP = kOffScan + 2 * kWaves * 4;
  static constexpr int kBytes = kOffP + (EXTRA ? 0 : kPBytes);
  static_assert(kBytes <= 160 * 1024, "LDS of one workgroup");
  static_assert(kOffP % 16 == 0, "16-byte P^T operands");
};
static_assert(kWaves * kStageBytes <= kOffIdx, "the epilogue staging leaves the index ring alone");
static_assert(16 * kTileStride + 3 * 256 + 8 < 65536, "PV operand offsets fit the DS immediate");
// Largest allowed excess of a score over its head's probability reference, in log2 units: P stays
// below 2^64, the sums far inside fp32 range for any cache value in the exactly decodable range.
constexpr float kRefSlack = 64.0f;

// Gather instructions per wave and sub-tile: fp8 = 4 chunk pairs + 1 scale chunk instruction,
// fp4 = 2 chunk pairs + 1 scale chunk instruction.
constexpr int kGatherFp8 = 5;
constexpr int kGatherFp4 = 3;
// fp8 pipeline: K and V operands are read kAhead MFMAs before use, through rings of kRing
// registers (an operand register is rewritten two MFMAs after the MFMA that read it)
constexpr int kAhead = 5;
constexpr int kRing = kAhead + 2;

__device__ __forceinline__ int lane_id() {
  int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte and 4-byte global -> LDS copies: the wave's active lanes write LDS bytes m0 + 16 * lane
// (resp. m0 + 4 * lane). m0 is set and not restored: no compiler-generated code of these kernels
// reads m0 (the build's assembly check rejects any that does). `lds_base` must be wave-uniform. The masked
// forms run the copy with EXEC = `lanes` (wave-uniform, never 0) and restore EXEC afterwards, so
// that a partial-wave copy needs no branch around it.
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds_base), "v"(gptr)
      : "memory");
}
// Same copy from gptr + OFF: the instruction's immediate offset applies to the LDS address as well
// (LDS address = m0 + offset + 16 * lane), so m0 is set to lds_base - OFF.
template <int OFF>
__device__ __forceinline__ void copy16_to_lds_off(const void* gptr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off offset:%2"
      :
      : "s"(lds_base - OFF), "v"(gptr), "i"(OFF)
      : "memory");
}
__device__ __forceinline__ void copy16_to_lds_masked(const void* gptr, uint32_t lds_base, uint64_t lanes) {
  uint64_t saved_exec;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, %3\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved_exec)
      : "s"(lds_base), "v"(gptr), "s"(lanes)
      : "memory");
}
__device__ __forceinline__ void copy4_to_lds_masked(const void* gptr, uint32_t lds_base, uint64_t lanes) {
  uint64_t saved_exec;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, %3\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved_exec)
      : "s"(lds_base), "v"(gptr), "s"(lanes)
      : "memory");
}

// 4-byte buffer -> LDS copy by the lanes in `lanes` (wave-uniform, never 0): lane l writes LDS
// bytes m0 + 4 * lane from byte `voff` of the buffer described by `rsrc`; offsets at or past its
// size read nothing from memory and return 0.
__device__ __forceinline__ void buffer_copy4_to_lds(u32x4 rsrc, uint32_t voff, uint32_t lds_base,
                                                    uint64_t lanes) {
  uint64_t saved_exec;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, %4\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved_exec)
      : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(lanes)
      : "memory");
}

// One MFMA step as an assembly statement: QK^T (scores in VGPRs, chained) and PV (O in the
// accumulation registers). Used where other work is interleaved between the steps.
__device__ __forceinline__ void mfma_qk_first(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma_qk(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma_pv(f32x16& o, const bf16x8& v, const bf16x8& pb) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(pb));
}

typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_w;   // read/write view
__device__ __forceinline__ bf16x8 lds_k(uint32_t a) {
  return __builtin_bit_cast(bf16x8, *(lds_u32x4*)(uintptr_t)a);
}
__device__ __forceinline__ bf16x8 lds_v(uint32_t a0, uint32_t a1) {
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)a0);
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)a1);
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Wait until at most n of this wave's vector memory operations are outstanding (and all of its
// LDS operations are done), then synchronise the workgroup. n is wave-uniform.
__device__ __forceinline__ void wait_and_barrier(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// The XOR pattern of token row r: bit 1 = bit 1 ^ bit 3 of r, bit 0 = bit 2 of r (the same for r and
// r + 16).
__device__ __forceinline__ int tile_xor(int r) { return (((r >> 1) ^ (r >> 3)) & 1) * 2 + ((r >> 2) & 1); }

__device__ __forceinline__ u32x4 lds_read16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void lds_write16(char* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void lds_write16_at(uint32_t a, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)(uintptr_t)a = v;
}

// Where sub-tile j of a row segment starting at unit t0 lives in the index arrays.
struct SubTile {
  bool fp4;
  int pos0;       // position of token 0 of the sub-tile inside its index row
  int count;      // index entries of that row (topk or extra_topk)
};

template <bool EXTRA>
__device__ __forceinline__ SubTile locate(const DecodeParams& p, int t0, int j) {
  const int unit = t0 + (j >> 1);
  SubTile st;
  st.fp4 = EXTRA && unit >= p.tiles_k;
  const int u = st.fp4 ? unit - p.tiles_k : unit;
  st.pos0 = u * kUnitTokens + (j & 1) * kSubTokens;
  st.count = st.fp4 ? p.extra_topk : p.topk;
  return st;
}


// QK^T of one sub-tile: S^T[32 tokens x 32 heads] = K[32 x 512] Q^T with 32 chained
// v_mfma_f32_32x32x16_bf16 steps. Step kk reads this lane's K fragment (token l%32, dims
// 16kk + 8(l/32) .. +7) at a[kk % 8] + 256 (kk / 8) (swizzled tile, see tile_xor). K fragments
// are read four steps ahead into eight rotating registers, so no fragment is overwritten while an
// MFMA that reads it may still be in flight.
//
// Written as one assembly block so that the scores land in VGPRs: with O occupying all 256
// accumulation registers, compiler-selected MFMAs would put the scores there as well. The block
// waits for its own LDS reads (lgkmcnt, after draining any earlier LDS/scalar operations), starts
// with 5 wait states (Q may have just been moved by VALU instructions) and ends with 20, more than
// the 12 the compiler inserts between this MFMA writing a VGPR and a VALU reading it.
__device__ __forceinline__ f32x16 qk_chain(const uint32_t (&a)[8], const bf16x8 (&q)[32]) {
  f32x16 s;
  bf16x8 k0, k1, k2, k3, k4, k5, k6, k7;
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 4\n\t"
      "ds_read_b128 %[k0], %[a0] offset:0\n\t"
      "ds_read_b128 %[k1], %[a1] offset:0\n\t"
      "ds_read_b128 %[k2], %[a2] offset:0\n\t"
      "ds_read_b128 %[k3], %[a3] offset:0\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k0], %[q0], 0\n\t"
      "ds_read_b128 %[k4], %[a4] offset:0\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k1], %[q1], %[s]\n\t"
      "ds_read_b128 %[k5], %[a5] offset:0\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k2], %[q2], %[s]\n\t"
      "ds_read_b128 %[k6], %[a6] offset:0\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k3], %[q3], %[s]\n\t"
      "ds_read_b128 %[k7], %[a7] offset:0\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k4], %[q4], %[s]\n\t"
      "ds_read_b128 %[k0], %[a0] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k5], %[q5], %[s]\n\t"
      "ds_read_b128 %[k1], %[a1] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k6], %[q6], %[s]\n\t"
      "ds_read_b128 %[k2], %[a2] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k7], %[q7], %[s]\n\t"
      "ds_read_b128 %[k3], %[a3] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k0], %[q8], %[s]\n\t"
      "ds_read_b128 %[k4], %[a4] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k1], %[q9], %[s]\n\t"
      "ds_read_b128 %[k5], %[a5] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k2], %[q10], %[s]\n\t"
      "ds_read_b128 %[k6], %[a6] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k3], %[q11], %[s]\n\t"
      "ds_read_b128 %[k7], %[a7] offset:256\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k4], %[q12], %[s]\n\t"
      "ds_read_b128 %[k0], %[a0] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k5], %[q13], %[s]\n\t"
      "ds_read_b128 %[k1], %[a1] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k6], %[q14], %[s]\n\t"
      "ds_read_b128 %[k2], %[a2] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k7], %[q15], %[s]\n\t"
      "ds_read_b128 %[k3], %[a3] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k0], %[q16], %[s]\n\t"
      "ds_read_b128 %[k4], %[a4] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k1], %[q17], %[s]\n\t"
      "ds_read_b128 %[k5], %[a5] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k2], %[q18], %[s]\n\t"
      "ds_read_b128 %[k6], %[a6] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k3], %[q19], %[s]\n\t"
      "ds_read_b128 %[k7], %[a7] offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k4], %[q20], %[s]\n\t"
      "ds_read_b128 %[k0], %[a0] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k5], %[q21], %[s]\n\t"
      "ds_read_b128 %[k1], %[a1] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k6], %[q22], %[s]\n\t"
      "ds_read_b128 %[k2], %[a2] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k7], %[q23], %[s]\n\t"
      "ds_read_b128 %[k3], %[a3] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k0], %[q24], %[s]\n\t"
      "ds_read_b128 %[k4], %[a4] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k1], %[q25], %[s]\n\t"
      "ds_read_b128 %[k5], %[a5] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k2], %[q26], %[s]\n\t"
      "ds_read_b128 %[k6], %[a6] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k3], %[q27], %[s]\n\t"
      "ds_read_b128 %[k7], %[a7] offset:768\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k4], %[q28], %[s]\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k5], %[q29], %[s]\n\t"
      "s_waitcnt lgkmcnt(1)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k6], %[q30], %[s]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[k7], %[q31], %[s]\n\t"
      "s_nop 15\n\t"
      "s_nop 3"
      : [s] "=&v"(s), [k0] "=&v"(k0), [k1] "=&v"(k1), [k2] "=&v"(k2), [k3] "=&v"(k3), [k4] "=&v"(k4), [k5] "=&v"(k5), [k6] "=&v"(k6), [k7] "=&v"(k7)
      : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [a4] "v"(a[4]), [a5] "v"(a[5]), [a6] "v"(a[6]), [a7] "v"(a[7]), [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]), [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]), [q10] "v"(q[10]), [q11] "v"(q[11]), [q12] "v"(q[12]), [q13] "v"(q[13]), [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]), [q18] "v"(q[18]), [q19] "v"(q[19]), [q20] "v"(q[20]), [q21] "v"(q[21]), [q22] "v"(q[22]), [q23] "v"(q[23]), [q24] "v"(q[24]), [q25] "v"(q[25]), [q26] "v"(q[26]), [q27] "v"(q[27]), [q28] "v"(q[28]), [q29] "v"(q[29]), [q30] "v"(q[30]), [q31] "v"(q[31])
      : "memory");
  return s;
}


// PV of one sub-tile: O^T[512 dims x 32 heads] += V^T P^T as 32 v_mfma_f32_32x32x16_bf16 steps
// (step i: token half ks = i / 16, dim block d = i % 16). The V^T operand of a step is two
// transposed LDS reads (ds_read_b64_tr_b16) at a[d % 4] and a[4 + d % 4], plus 16 kTileStride ks +
// 256 (d / 4) (swizzled tile, see tile_xor). Reads run three steps ahead through six fixed operand buffers
// (v232..v255, declared clobbered so that the compiler keeps nothing there); O stays in the
// accumulation registers. The block starts with 5 wait states (P may have just been written by
// VALU instructions) and ends with 20 (before O is read outside).
__device__ __forceinline__ void pv_chain(const uint32_t (&a)[8], f32x16 (&o)[16], const bf16x8 (&pb)[2]) {
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 4\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[v0] offset:0\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[v4] offset:0\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[v1] offset:0\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[v5] offset:0\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[v2] offset:0\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[v6] offset:0\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], v[232:235], %[p0], %[o0]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[v3] offset:0\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[v7] offset:0\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], v[236:239], %[p0], %[o1]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[v0] offset:256\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[v4] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o2], v[240:243], %[p0], %[o2]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[v1] offset:256\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[v5] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o3], v[244:247], %[p0], %[o3]\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[v2] offset:256\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[v6] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o4], v[248:251], %[p0], %[o4]\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[v3] offset:256\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[v7] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o5], v[252:255], %[p0], %[o5]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[v0] offset:512\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[v4] offset:512\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o6], v[232:235], %[p0], %[o6]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[v1] offset:512\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[v5] offset:512\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o7], v[236:239], %[p0], %[o7]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[v2] offset:512\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[v6] offset:512\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o8], v[240:243], %[p0], %[o8]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[v3] offset:512\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[v7] offset:512\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o9], v[244:247], %[p0], %[o9]\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[v0] offset:768\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[v4] offset:768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o10], v[248:251], %[p0], %[o10]\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[v1] offset:768\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[v5] offset:768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o11], v[252:255], %[p0], %[o11]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[v2] offset:768\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[v6] offset:768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o12], v[232:235], %[p0], %[o12]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[v3] offset:768\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[v7] offset:768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o13], v[236:239], %[p0], %[o13]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[v0] offset:17408\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[v4] offset:17408\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o14], v[240:243], %[p0], %[o14]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[v1] offset:17408\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[v5] offset:17408\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o15], v[244:247], %[p0], %[o15]\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[v2] offset:17408\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[v6] offset:17408\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], v[248:251], %[p1], %[o0]\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[v3] offset:17408\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[v7] offset:17408\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], v[252:255], %[p1], %[o1]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[v0] offset:17664\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[v4] offset:17664\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o2], v[232:235], %[p1], %[o2]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[v1] offset:17664\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[v5] offset:17664\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o3], v[236:239], %[p1], %[o3]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[v2] offset:17664\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[v6] offset:17664\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o4], v[240:243], %[p1], %[o4]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[v3] offset:17664\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[v7] offset:17664\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o5], v[244:247], %[p1], %[o5]\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[v0] offset:17920\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[v4] offset:17920\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o6], v[248:251], %[p1], %[o6]\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[v1] offset:17920\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[v5] offset:17920\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o7], v[252:255], %[p1], %[o7]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[v2] offset:17920\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[v6] offset:17920\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o8], v[232:235], %[p1], %[o8]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[v3] offset:17920\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[v7] offset:17920\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o9], v[236:239], %[p1], %[o9]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[v0] offset:18176\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[v4] offset:18176\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o10], v[240:243], %[p1], %[o10]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[v1] offset:18176\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[v5] offset:18176\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o11], v[244:247], %[p1], %[o11]\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[v2] offset:18176\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[v6] offset:18176\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o12], v[248:251], %[p1], %[o12]\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[v3] offset:18176\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[v7] offset:18176\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o13], v[252:255], %[p1], %[o13]\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o14], v[232:235], %[p1], %[o14]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o15], v[236:239], %[p1], %[o15]\n\t"
      "s_nop 15\n\t"
      "s_nop 3"
      : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]), [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]), [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]), [o15] "+a"(o[15])
      : [v0] "v"(a[0]), [v1] "v"(a[1]), [v2] "v"(a[2]), [v3] "v"(a[3]), [v4] "v"(a[4]), [v5] "v"(a[5]), [v6] "v"(a[6]), [v7] "v"(a[7]), [p0] "v"(pb[0]), [p1] "v"(pb[1])
      : "memory", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255");
}

template <bool EXTRA, bool FUSED>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_decode_wide_kernel(DecodeParams p) {
  using L = Lds<EXTRA>;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  char* const tiles = smem;
  char* const raws = smem + kOffRaw;
  int* const redo_flags = reinterpret_cast<int*>(smem + L::kOffFlags);
  int* const scan_slots = reinterpret_cast<int*>(smem + L::kOffScan);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int head_base = blockIdx.y * kGroupHeads + 32 * wave;   // this wave's first head
  // index ring: the wave's own (extra-cache variant) or the one all waves share (fp8 pipeline)
  char* const idx_ring = smem + kOffIdx + (EXTRA ? wave * kStages * kIdxBytes : 0);
  // lanes of the scale-chunk copies: tokens 8w .. 8w+7 (first lane half; fp4: both halves)
  const uint64_t scale_lanes_fp8 = 0xFFull << (8 * wave);
  const uint64_t scale_lanes_fp4 = scale_lanes_fp8 | (scale_lanes_fp8 << 32);

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
  int seg_parity = 0;

  while (row < end_row || (row == end_row && t0 < end_tile)) {
    const int t1 = row < end_row ? p.tiles : end_tile;
    const int nsub_all = 2 * (t1 - t0);
    int nsub = nsub_all;                       // the live length once the scan below has run

    // Index load of sub-tile j into this wave's index slot j % 3 (lanes 0..31, one entry each;
    // entries past the end of the index row are fetched from a clamped address and replaced by
    // -1 when read). It is issued for every iteration: past the last sub-tile, or for a selection
    // of size 0 (no index array), it reads from the schedule instead (a valid address).
    // In the shared ring of the fp8 pipeline, wave w loads entries 8w .. 8w+7 (lanes 0..7).
    auto load_indices = [&](int j, int slot) {
      const int e = EXTRA ? lane_id() : 8 * wave + (lane_id() & 7);   // the lane's entry
      const int32_t* src_ptr = p.sched;
      if (j < nsub) {
        const SubTile st = locate<EXTRA>(p, t0, j);
        if (st.count > 0)
          src_ptr = (st.fp4 ? p.xidx : p.idx) + (int64_t)row * st.count + min(st.pos0 + e, st.count - 1);
      }
      copy4_to_lds_masked(src_ptr,
                          __builtin_amdgcn_readfirstlane(lds_addr(idx_ring + slot * kIdxBytes) + (EXTRA ? 0 : 32 * wave)),
                          EXTRA ? 0xFFFFFFFFull : 0xFFull);
    };

    // ---- segment start: the first batch of the live-length scan, the first two index rows of
    // the pipeline and Q are all issued before anything waits, so their latencies overlap.
    // opaque, so that nothing derived from the thread index is hoisted out of the segment loop
    // and kept live through the pipeline
    int tid = 64 * wave + lane_id();       // threadIdx.x, rebuilt so that v0 need not stay live
    asm volatile("" : "+v"(tid));
    // Entry e of the segment is entry e % 32 of its sub-tile e / 32. The 8 loads of a batch are
    // unconditional (clamped addresses; an empty selection reads the schedule instead), so they
    // are all in flight together; entries outside the segment or past the index row count as -1.
    auto scan_batch = [&](int e0, int (&v)[8]) {
      bool in[8];
      const int32_t* src[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 64 * kWaves * u + tid;
        const SubTile st = locate<EXTRA>(p, t0, min(e / kSubTokens, nsub_all - 1));
        const int pos = st.pos0 + e % kSubTokens;
        in[u] = e / kSubTokens < nsub_all && pos < st.count;
        src[u] = st.count > 0
                     ? (st.fp4 ? p.xidx : p.idx) + (int64_t)row * st.count + min(pos, st.count - 1)
                     : p.sched;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *src[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = in[u] ? v[u] : -1;
    };
    // fp8 pipeline: gather of sub-tile j (j < 3, before the loop) from index slot j into raw slot
    // j; sub-tiles past `live` or entries past the index row are ignored (they copy the zero
    // record). Returns the sub-tile's validity mask.
    auto fp8_gather_first = [&](int j, int live) -> uint32_t {
      const int lane = lane_id();
      const int t = lane & 31, hh = lane >> 5;
      const int gv = *reinterpret_cast<const int*>(idx_ring + j * kIdxBytes + 4 * t);
      const bool valid = j < live && p.topk > 0 && kUnitTokens * t0 + kSubTokens * j + t < p.topk && gv >= 0;
      const uint32_t mask = (uint32_t)__ballot(valid);
      const uint8_t* grec = valid ? p.kc + (int64_t)gv * kFp8Rec : g_zero.bytes;
      const uint8_t* gdat = grec + 32 * wave + 16 * hh;
      const uint32_t graw = lds_addr(smem) + kOffRaw + j * kRawBytes;
      copy16_to_lds_off<0>(gdat, graw + 1024 * wave);
      copy16_to_lds_off<128>(gdat, graw + 1024 * (wave + 4));
      copy16_to_lds_off<256>(gdat, graw + 1024 * (wave + 8));
      copy16_to_lds_off<384>(gdat, graw + 1024 * (wave + 12));
      copy16_to_lds_masked(grec + 512, graw + 32 * 512, scale_lanes_fp8);
      return mask;
    };
    uint32_t mk_first[3] = {0u, 0u, 0u};
    int scan_v[8];
    scan_batch(0, scan_v);
    load_indices(0, 0);                          // "iteration -6" of the first pass
    load_indices(1, 1);                          // "iteration -5"
    if constexpr (!EXTRA) load_indices(2, 2);

    // ---- Q of this wave's 32 heads, B-operand layout of v_mfma_f32_32x32x16_bf16:
    // lane l holds head l%32, dims 16kk + 8(l/32) .. +7 of k-step kk. Heads past h_q load a copy
    // of the last head; their results are never stored.
    bf16x8 qreg[32];
    {
      const int lane = lane_id();
      const int qh = min(head_base + (lane & 31), p.h_q - 1);
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          p.q + ((int64_t)row * p.h_q + qh) * kHeadDim + 8 * (lane >> 5));
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) qreg[kk] = __builtin_bit_cast(bf16x8, qp[2 * kk]);
    }
    if constexpr (!EXTRA) {
      // The first three sub-tiles are gathered as soon as their index rows are in, while Q is
      // still arriving: the pipeline then starts one memory latency after the Q traffic instead
      // of two. The scan batch and idx(0 .. 2) have landed once at most the 32 Q loads issued
      // after them are outstanding; the barrier makes every wave's quarter of the shared index
      // slots visible. It also keeps a later segment's gathers until every wave is done with the
      // previous segment's epilogue staging, which overlaps the raw slots.
      asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int j = 0; j < 3; ++j) mk_first[j] = fp8_gather_first(j, nsub_all);
      // every wave has read slots 0 and 1 before any wave refills them
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_indices(3, 0);
      load_indices(4, 1);
    }
    if constexpr (FUSED) {
      // Fused decode: the query row is RMS-normalised with the weight w (q / sqrt(mean(q^2) + eps)
      // * w) and its rotary pairs (dims 448 + 2i, 449 + 2i; k-steps 28..31) are rotated by the row's
      // cos / sin, in fp32, then rounded back to bf16 (page "deepseek-ai/FlashMLA", section "What
      // it is": Q-norm and RoPE in the same kernel as the attention). Lanes l and l ^ 32 hold the
      // two halves of head l % 32's dims.
      const int lane = lane_id();
      const int g = lane >> 5;
      // the sum of squares in fp64 (each bf16 square is exact there, and 512 terms lose almost
      // nothing), so that the roundings before the bf16 query are those of the mean, the
      // reciprocal square root and the fp32 products below, each of order 2^-24
      double ss = 0.0;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double v = (double)(float)qreg[kk][j];
          ss = __builtin_fma(v, v, ss);
        }
      {
        // lanes l and l ^ 32: each swap returns this lane's word and the partner's, in an order
        // that depends on the lane half, so both are rebuilt and added (the sum is symmetric)
        const uint64_t b = __builtin_bit_cast(uint64_t, ss);
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
        ss = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]) +
             __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
      }
      // opaque: the products below convert qreg again instead of keeping 256 converted values live
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) asm volatile("" : "+v"(qreg[kk]));
      float eps = p.qn_eps;
      asm volatile("" : "+s"(eps));    // converted here, not kept live across the whole kernel
      const float inv_rms = 1.0f / __builtin_sqrtf((float)(ss * (1.0 / kHeadDim) + (double)eps));
      const u32x4* wp = reinterpret_cast<const u32x4*>(p.qn_weight + 8 * g);
      const float* cs = p.rope_cos + (int64_t)row * 32 + 4 * g;
      const float* sn = p.rope_sin + (int64_t)row * 32 + 4 * g;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) {
        const bf16x8 wv = __builtin_bit_cast(bf16x8, wp[2 * kk]);
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = (float)qreg[kk][j] * inv_rms * (float)wv[j];
        if (kk >= 28) {
          // dims 16 kk + 8 g + j: pair 8 (kk - 28) + 4 g + j / 2
          const f32x4 c = *reinterpret_cast<const f32x4*>(cs + 8 * (kk - 28));
          const f32x4 sv = *reinterpret_cast<const f32x4*>(sn + 8 * (kk - 28));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float x0 = y[2 * jj], x1 = y[2 * jj + 1];
            y[2 * jj] = x0 * c[jj] - x1 * sv[jj];
            y[2 * jj + 1] = x0 * sv[jj] + x1 * c[jj];
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) qreg[kk][j] = (__bf16)y[j];
        // one k-step at a time: the weight and angle loads are not hoisted into registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- live length of the segment. A sub-tile whose 32 entries are all ignored (negative, or
    // past the end of the index row) contributes nothing, so the segment ends after the last
    // sub-tile with a valid entry; with no valid entry at all it runs no sub-tile and its output is
    // the empty softmax (zeros, lse -inf). Sub-tiles of ignored entries before that point are
    // processed with all their tokens masked. Each thread tests entries tid, tid + 256, ... in
    // batches of 8 independent loads; the per-wave maxima meet in LDS (one buffer per segment
    // parity, so a wave already in the next segment never overwrites values still being read).
    {
      int last = -1;
      for (int e0 = 0; e0 < nsub_all * kSubTokens; e0 += 8 * 64 * kWaves) {
        int v[8];
        if (e0 == 0) {
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = scan_v[u];
        } else {
          scan_batch(e0, v);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (v[u] >= 0) last = max(last, (e0 + 64 * kWaves * u + tid) / kSubTokens);
      }
      // wave maximum, bit by bit from the top with ballots (uniform, no lane shuffles)
      int wmax = -1;
      if (__ballot(last >= 0) != 0) {
        wmax = 0;
        for (int b = 31 - __builtin_clz((unsigned)nsub_all); b >= 0; --b)
          if (__ballot(last >= (wmax | (1 << b))) != 0) wmax |= 1 << b;
      }
      int* const slots = scan_slots + kWaves * seg_parity;
      if (lane_id() == 0) slots[wave] = wmax;
      __syncthreads();
      nsub = __builtin_amdgcn_readfirstlane(max(max(slots[0], slots[1]), max(slots[2], slots[3])) + 1);
      seg_parity ^= 1;
    }
    // (the pointer is taken afresh here, so that its null test is not hoisted into a register
    // kept through the pipeline)
    typedef __attribute__((address_space(1))) const int32_t global_i32;
    global_i32* split_ptr = (global_i32*)p.split_ptr;
    asm volatile("" : "+s"(split_ptr));
    const int split_base = split_ptr ? split_ptr[row] : 0;
    const int nsplit = split_ptr ? split_ptr[row + 1] - split_base : 1;
    const int slot = first_seg ? slot_first : split_base;

    // Q and the first two index rows are resident before any further asynchronous copy of this
    // segment is issued, so the compiler's own wait for Q cannot end up waiting for the gathers.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // ---- asynchronous stages (see the file comment).
    // Gather of sub-tile j into raw slot j % 3; returns the validity mask of its 32 tokens.
    // Ignored tokens fetch record 0 (it exists whenever the selection is not empty), so every wave
    // issues a fixed number of copies per sub-tile; their values are never used. A sub-tile of an
    // empty selection issues nothing.
    auto gather = [&](int j) -> uint32_t {
      const SubTile st = locate<EXTRA>(p, t0, j);
      if (st.count == 0) return 0u;
      const int lane = lane_id();
      const int t = lane & 31;
      const int hh = lane >> 5;
      const int v = *reinterpret_cast<const int*>(idx_ring + (j % 3) * kIdxBytes + 4 * t);
      const bool valid = st.pos0 + t < st.count && v >= 0;
      const uint32_t mask = (uint32_t)__ballot(valid);
      const int tok = valid ? v : 0;
      char* raw = raws + (j % 3) * kRawBytes;
      const uint32_t raw_lds = __builtin_amdgcn_readfirstlane(lds_addr(raw));
      if (!st.fp4) {
        const uint8_t* rec = p.kc + (int64_t)tok * kFp8Rec;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = wave + 4 * i;                       // chunks 2q (hh = 0) and 2q + 1
          copy16_to_lds(rec + (2 * q + hh) * 16, __builtin_amdgcn_readfirstlane(raw_lds + 1024 * q));
        }
        copy16_to_lds_masked(rec + 512, __builtin_amdgcn_readfirstlane(raw_lds + 32 * 512), scale_lanes_fp8);
      } else {
        const uint8_t* rec = p.xc + (int64_t)tok * kFp4Rec;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int q = wave + 4 * i;
          copy16_to_lds(rec + (2 * q + hh) * 16, __builtin_amdgcn_readfirstlane(raw_lds + 1024 * q));
        }
        copy16_to_lds_masked(rec + (16 + hh) * 16, __builtin_amdgcn_readfirstlane(raw_lds + 16 * 512),
                             scale_lanes_fp4);
      }
      return mask;
    };
    // Dequantization of sub-tile j: this wave's 128 dims of all 32 tokens, raw slot -> bf16 tile
    // slot j % 3 (ignored tokens become zeros).
    auto dequant = [&](int j, uint32_t mask) {
      const SubTile st = locate<EXTRA>(p, t0, j);
      const int lane = lane_id();
      const int t = lane & 31;
      const int g = lane >> 5;
      const bool valid = (mask >> t) & 1u;
      const char* raw = raws + (j % 3) * kRawBytes;
      char* trow = tiles + (j % 3) * kTileBytes + t * kTileStride;
      const int sw = tile_xor(t);
      auto chunk = [&](int c) { return trow + 16 * (c ^ sw); };   // bf16 chunk c of this token
      if (!st.fp4) {
        const int c0 = 8 * wave + 4 * g;                     // first of this lane's 4 fp8 chunks
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(raw + (32 * kSubTokens + t) * 16 + c0 / 2);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const u32x4 r = lds_read16(raw + ((c0 + cc) * kSubTokens + t) * 16);
          bf16x8 lo, hi;
          dequant_fp8_16(r, (sc2 >> (8 * (cc >> 1))) & 0xFFu, lo, hi);
          lds_write16(chunk(2 * (c0 + cc)), valid ? __builtin_bit_cast(u32x4, lo) : u32x4{});
          lds_write16(chunk(2 * (c0 + cc) + 1), valid ? __builtin_bit_cast(u32x4, hi) : u32x4{});
        }
      } else {
        const int c0 = 4 * wave + 2 * g;                     // 2 data chunks = dims 32c0 .. 32c0+63
        const int j0 = 8 * wave + 4 * g;                     // e4m3 scales j0 .. j0+3
        const uint32_t sc4 = *reinterpret_cast<const uint32_t*>(
            raw + ((16 + (j0 >> 4)) * kSubTokens + t) * 16 + (j0 & 15));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const u32x4 r = lds_read16(raw + ((c0 + cc) * kSubTokens + t) * 16);
          bf16x8 a0, a1, a2, a3;
          dequant_fp4_16(r[0], r[1], e4m3_to_f32(sc4 >> (16 * cc)), a0, a1);
          dequant_fp4_16(r[2], r[3], e4m3_to_f32(sc4 >> (16 * cc + 8)), a2, a3);
          const int b = 4 * (c0 + cc);                       // bf16 chunks b .. b+3
          lds_write16(chunk(b), valid ? __builtin_bit_cast(u32x4, a0) : u32x4{});
          lds_write16(chunk(b + 1), valid ? __builtin_bit_cast(u32x4, a1) : u32x4{});
          lds_write16(chunk(b + 2), valid ? __builtin_bit_cast(u32x4, a2) : u32x4{});
          lds_write16(chunk(b + 3), valid ? __builtin_bit_cast(u32x4, a3) : u32x4{});
        }
      }
    };
    auto gather_count = [&](int j) -> int {
      if (j < 0 || j >= nsub) return 0;
      const SubTile st = locate<EXTRA>(p, t0, j);
      return st.count == 0 ? 0 : st.fp4 ? kGatherFp4 : kGatherFp8;
    };
    auto is_fp8 = [&](int j) -> bool { return !locate<EXTRA>(p, t0, j).fp4; };

    // Per-lane LDS addresses in tile slot 0 (add slot * kTileBytes).
    // QK^T step kk reads token row r = l%32, logical chunk 2kk + g (g = l/32), physical chunk
    // 4 (kk / 2) + ((2 (kk % 2) + g) ^ tile_xor(r)), i.e. k_addr[kk % 8] + 256 (kk / 8).
    // PV step (ks, d) reads, for h = 0, 1, token row 16ks + 8((l/16)/2) + 4h + (l%16)/4 and logical
    // chunk 4d + 2((l/16)%2) + (l%4)/2 (8-byte half l%2), i.e. v_addr[4h + d%4] + 16 kTileStride ks
    // + 256 (d / 4). The fp8 pipeline only reads its own dim blocks d = 4w .. 4w+3, and its v_addr
    // already hold the + 256 w.
    uint32_t k_addr[8], v_addr[8];
    {
      const int lane = lane_id();
      const int r = lane & 31, g = lane >> 5, x = tile_xor(r);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        k_addr[j] = lds_addr(tiles + r * kTileStride + 64 * (j >> 1) + 16 * ((2 * (j & 1) + g) ^ x));
      const int g2 = lane >> 4, jj = lane & 15;
      const int c_lo = 2 * (g2 & 1) + ((jj & 3) >> 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rw = 8 * (g2 >> 1) + 4 * h + (jj >> 2);
        const int xr = tile_xor(rw);
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
          v_addr[4 * h + dd] = lds_addr(tiles + rw * kTileStride + 16 * (4 * dd + (c_lo ^ xr)) + 8 * (jj & 1) +
                                        (EXTRA ? 0 : 256 * wave));
      }
    }
    // Operand base of tile slot `sl` (a constant in the unrolled fp8 loop). Offsets into slots 0
    // and 1 fit the 16-bit DS immediate and fold into the instructions; slot 2 starts past 64 KB,
    // so its base is formed once in a register instead of once per access.
    auto slot_base = [&](uint32_t base, int sl) -> uint32_t {
      uint32_t a = base + sl * kTileBytes;
      if (sl == 2) asm volatile("" : "+v"(a));
      return a;
    };
    // fp8 pipeline, per-lane constants (opaque, so that they are kept rather than rebuilt):
    //  dq_w[m]  tile slot 0 address of this lane's bf16 chunk 2 c0 + j, j % 4 = m (the swizzle
    //           permutes chunks within groups of four): chunk 2 c0 + j is at dq_w[j % 4] + 64 (j / 4);
    //  raw_r    raw slot 0 address of the lane's first fp8 chunk (c0, token t); chunk c0 + cc at
    //           + 512 cc;  raw_s  the lane's two scale bytes (c0 / 2, token t);
    //  idx_r    index slot 0 entry of token t;  idx_v  its byte offset in a 32-entry index block;
    //  idx_l    byte offset of the entry this lane loads into the shared ring (8 w + l, l < 8);
    //  g_base / g_zb   record byte 32 w + 16 hh (this lane's first copied chunk) of record 0 of
    //           the cache and of the zero record.
    uint32_t dq_w[4], raw_r, raw_s, idx_r, idx_v, idx_l;
    uint64_t g_base, g_zb;
    {
      const int lane = lane_id();
      const int t = lane & 31, hh = lane >> 5;
      const int sw = tile_xor(t);
      const int c0 = 8 * wave + 4 * hh;
#pragma unroll
      for (int m = 0; m < 4; ++m) dq_w[m] = lds_addr(tiles + t * kTileStride + 32 * c0 + 16 * (m ^ sw));
      raw_r = lds_addr(raws + (c0 * kSubTokens + t) * 16);
      raw_s = lds_addr(raws + (32 * kSubTokens + t) * 16 + c0 / 2);
      idx_r = lds_addr(idx_ring + 4 * t);
      idx_v = 4 * t;
      idx_l = 4 * (8 * wave + (lane & 7));
      g_base = (uint64_t)(uintptr_t)(p.kc + 32 * wave + 16 * hh);
      g_zb = (uint64_t)(uintptr_t)(g_zero.bytes + 32 * wave + 16 * hh);
      asm volatile("" : "+v"(dq_w[0]), "+v"(dq_w[1]), "+v"(dq_w[2]), "+v"(dq_w[3]), "+v"(raw_r),
                   "+v"(raw_s), "+v"(idx_r), "+v"(idx_v), "+v"(idx_l), "+v"(g_base), "+v"(g_zb));
    }
    //  p_rd     P^T exchange buffer address of this lane's 16 bytes of head group 0, token half 0
    //           (group g, half ks at + 1024 (2 g + ks)).
    uint32_t p_rd = lds_addr(smem) + L::kOffP + 16 * lane_id();
    asm volatile("" : "+v"(p_rd));
    // byte address of the segment row's index entries (the buffer base of the index loads)
    const uint64_t idx_row = (uint64_t)(uintptr_t)(p.idx + (int64_t)row * p.topk);
    auto slot_addr = [&](const uint32_t (&base)[8], int sl, uint32_t (&out)[8]) {
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = base[j] + sl * kTileBytes;
    };

    // ---- softmax state. Scores are in log2 units (x = q.k * scale * log2 e). Probabilities are
    // taken against a fixed per-head reference m_ref, the maximum of the head's first sub-tile with
    // a valid token, instead of a running maximum: O is never rescaled inside the loop. m_max
    // tracks the true maximum. If it ends more than kRefSlack above m_ref for some head (larger
    // probabilities could overflow), the segment is computed again with m_ref = m_max, which is
    // then exact; for scores of realistic range that second pass never runs.
    float m_ref_next = -__builtin_inff();     // reference for the next pass (-inf: take the first)
    f32x16 oacc[16];
    float m_ref, m_max, l_sum;
    // fp8 pipeline: per-lane running raw maximum and probability sum, the exponent offset
    // (-m_ref once the reference is set, 0 before) and whether it is set (wave-uniform)
    float m_lane, l_lane, ref_off;
    bool ref_set;
    for (int pass = 0;; ++pass) {
      m_ref = m_ref_next;
      m_max = -__builtin_inff();
      l_sum = 0.0f;
      m_lane = -__builtin_inff();
      l_lane = 0.0f;
      ref_set = pass > 0;
      ref_off = pass > 0 ? -m_ref : 0.0f;
      {
        // 0 x 0 + 0 per block, in one assembly block whose leading wait states separate the VALU
        // write of the zero operand from its first read by an MFMA (an MFMA issued right after that
        // write reads stale lanes). The O accumulators then only ever take values from assembly
        // with AGPR constraints, so the compiler never moves them through VGPRs.
        const bf16x8 zero8 = bf16x8{};
        asm volatile(
            "s_nop 4\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %1, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %2, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %3, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %4, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %5, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %6, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %7, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %8, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %9, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %10, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %11, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %12, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %13, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %14, %16, %16, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %15, %16, %16, 0"
            : "=a"(oacc[0]), "=a"(oacc[1]), "=a"(oacc[2]), "=a"(oacc[3]), "=a"(oacc[4]),
              "=a"(oacc[5]), "=a"(oacc[6]), "=a"(oacc[7]), "=a"(oacc[8]), "=a"(oacc[9]),
              "=a"(oacc[10]), "=a"(oacc[11]), "=a"(oacc[12]), "=a"(oacc[13]), "=a"(oacc[14]),
              "=a"(oacc[15])
            : "v"(zero8));
      }

      // Softmax of one sub-tile's scores sv (lane l: head l%32, tokens 8(r/4) + 4(l/32) + r%4 in
      // sv[r]; lanes l and l^32 together hold the head's 32 tokens), split into steps so that the
      // pieces can be spread over the PV MFMAs: 0-3 scale and mask 4 scores each, 4 the maximum,
      // 5-12 two exponentials each, 13-14 the P^T operand of one token half each, 15 the sum.
      struct SoftmaxTemps { float x[16], e[16], mx, ls; };    // local to one sub-tile's softmax
      auto softmax_step = [&](SoftmaxTemps& st, int step, const f32x16& sv, uint32_t mask,
                              bf16x8 (&pb)[2]) {
        float (&x)[16] = st.x;
        float (&e)[16] = st.e;
        float& mx = st.mx;
        float& ls = st.ls;
        const int lane = lane_id();
        if (step < 4) {
          if (step == 0) { mx = -__builtin_inff(); ls = 0.0f; }
#pragma unroll
          for (int r = 4 * step; r < 4 * step + 4; ++r) x[r] = sv[r] * p.scale_log2;
          if (mask != 0xFFFFFFFFu) {             // ignored tokens in this sub-tile: -inf scores
            const uint32_t mq = mask >> (4 * (lane >> 5));
#pragma unroll
            for (int r = 4 * step; r < 4 * step + 4; ++r)
              if (!((mq >> (8 * (r >> 2) + (r & 3))) & 1u)) x[r] = -__builtin_inff();
          }
          mx = fmaxf(mx, fmaxf(fmaxf(x[4 * step], x[4 * step + 1]), fmaxf(x[4 * step + 2], x[4 * step + 3])));
        } else if (step == 4) {
          mx = max_xor32(mx);             // -inf only if the sub-tile has no valid token
          m_max = fmaxf(m_max, mx);
          m_ref = m_ref == -__builtin_inff() ? mx : m_ref;
          // while no valid token has been seen (m_ref = -inf) every x is -inf: exp2(-inf - 0) = 0
          mx = m_ref == -__builtin_inff() ? 0.0f : m_ref;   // reused as the exponent offset
        } else if (step < 13) {
#pragma unroll
          for (int r = 2 * (step - 5); r < 2 * (step - 5) + 2; ++r) {
            e[r] = __builtin_amdgcn_exp2f(x[r] - mx);     // 0 for ignored tokens (x = -inf)
            ls += e[r];
          }
        } else if (step < 15) {
          // P^T operand for token block ks: lane l needs head l%32 and tokens 16ks + 8(l/32) .. +7.
          // X (r = 8ks..8ks+3) and Y (r = 8ks+4..8ks+7) hold tokens 16ks + 4g + 0..3 and
          // 16ks + 8 + 4g + 0..3 (g = l/32); one permlane32 swap of X's upper half with Y's lower
          // half leaves tokens 16ks + 8g' + 0..3 in X and + 4..7 in Y for lane group g'.
          const int ks = step - 13;
          uint32_t xw[2], yw[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            bf16x2 xa, ya;
            xa[0] = (__bf16)e[8 * ks + 2 * h];
            xa[1] = (__bf16)e[8 * ks + 2 * h + 1];
            ya[0] = (__bf16)e[8 * ks + 4 + 2 * h];
            ya[1] = (__bf16)e[8 * ks + 4 + 2 * h + 1];
            auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, xa),
                                                       __builtin_bit_cast(uint32_t, ya), false, false);
            xw[h] = (uint32_t)sw[0];
            yw[h] = (uint32_t)sw[1];
          }
          const u32x4 packed = {xw[0], xw[1], yw[0], yw[1]};
          pb[ks] = __builtin_bit_cast(bf16x8, packed);
        } else if (step == 15) {
          l_sum += sum_xor32(ls);
        }
      };
      // The same for the fp8 pipeline, whose scores of ignored tokens already hold the ignored
      // score (no masking), with the scale folded into the exponent. The maximum and the sum are
      // kept per lane over the whole segment and reduced across the lane pair once, after the
      // loop: steps 0-3 fold 4 raw scores each into the lane's running maximum; step 4 takes the
      // reference on the first live sub-tile (a wave-uniform branch, so the cross-lane reduction
      // runs once per segment); steps 5-12 two exponentials each, added to the lane's sum in
      // fp32; 13-14 the P^T operand of one token half each.
      auto softmax_step_fp8 = [&](SoftmaxTemps& st, int step, const f32x16& sv, bool live,
                                  bf16x8 (&pb)[2]) {
        float (&e)[16] = st.e;
        if (step < 4) {
          const int r = 4 * step;
          asm("v_max3_f32 %0, %0, %1, %2" : "+v"(m_lane) : "v"(sv[r]), "v"(sv[r + 1]));
          asm("v_max3_f32 %0, %0, %1, %2" : "+v"(m_lane) : "v"(sv[r + 2]), "v"(sv[r + 3]));
        } else if (step == 4) {
          // before the first live sub-tile every score is the ignored score and every lane's
          // maximum is that score: the reduction then gives this sub-tile's own maximum
          if (!ref_set && live) {
            m_ref = max_xor32(m_lane) * p.scale_log2;    // the scale is positive
            ref_off = -m_ref;
            ref_set = true;
          }
        } else if (step < 13) {
#pragma unroll
          for (int r = 2 * (step - 5); r < 2 * (step - 5) + 2; ++r) {
            e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], p.scale_log2, ref_off));
            l_lane += e[r];
          }
        } else if (step < 15) {
          const int ks = step - 13;
          uint32_t xw[2], yw[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            bf16x2 xa, ya;
            xa[0] = (__bf16)e[8 * ks + 2 * h];
            xa[1] = (__bf16)e[8 * ks + 2 * h + 1];
            ya[0] = (__bf16)e[8 * ks + 4 + 2 * h];
            ya[1] = (__bf16)e[8 * ks + 4 + 2 * h + 1];
            auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, xa),
                                                       __builtin_bit_cast(uint32_t, ya), false, false);
            xw[h] = (uint32_t)sw[0];
            yw[h] = (uint32_t)sw[1];
          }
          const u32x4 packed = {xw[0], xw[1], yw[0], yw[1]};
          pb[ks] = __builtin_bit_cast(bf16x8, packed);
        }
      };
      auto softmax = [&](const f32x16& sv, uint32_t mask, bf16x8 (&pb)[2]) {
        SoftmaxTemps st;
#pragma unroll
        for (int step = 0; step < 16; ++step) softmax_step(st, step, sv, mask, pb);
      };

      // Validity masks of sub-tiles s .. s+4 (scalar ring) and the P^T operand of sub-tile s.
      uint32_t mk0 = 0, mk1 = 0, mk2 = 0, mk3 = 0, mk4 = 0;
      bf16x8 pb_cur[2] = {bf16x8{}, bf16x8{}};
      // K operand ring of the fp8 pipeline; between iterations kb[0 .. kAhead-1] hold the first
      // operands of the next QK^T
      bf16x8 kb[kRing];
      // opaque, so that no copy of the loop is specialised for this constant
      asm volatile("" : "+v"(pb_cur[0]), "+v"(pb_cur[1]));

      // ---- one iteration of the fp8-only pipeline, the same code for every s in [-4, nsub):
      // phase A runs the 32 QK^T MFMAs of sub-tile s+1 with the index load of s+6, the gather of
      // s+4 and half the dequantization of s+2 spread between them; phase B runs the 32 PV MFMAs
      // of sub-tile s with the softmax of s+1 and the other half of the dequantization spread
      // between them. The barrier at phase B's step 27 and one at the start of phase A order the
      // tile, raw-slot and P^T exchange traffic across waves. Every step ends in a scheduling
      // barrier, so each piece stays next to its MFMA. Sub-tiles outside 0..nsub-1 take part with
      // an all-invalid mask: they gather from a valid dummy address, dequantize to zeros, get zero
      // probabilities and add nothing.
      auto fp8_iteration = [&](auto first, int s, int r0, int r1, int r2) {
        // iteration -1 (first): there is no sub-tile -1, so it skips PV and the reads of its
        // operands; tile slot 2 and the P^T buffer are then never read before they are written
        constexpr bool kFirst = decltype(first)::value;
        // operand addresses: K of sub-tile s+1 (phase A), V of sub-tile s (phase B); kb[0..2]
        // already hold the first three K operands
        // K of step kk at ka[kk % 2] + 64 (kk / 2), V of PV step n at va[h] + 16 kTileStride (n / 16)
        // + 64 (n % 16), h = 0, 1
        const uint32_t ka[2] = {slot_base(k_addr[0], r1), slot_base(k_addr[1], r1)};
        const uint32_t va[2] = {slot_base(v_addr[0], r0), slot_base(v_addr[4], r0)};
        // V^T operand n (0..7): token half n / 4, this wave's dim block n % 4
        auto read_v = [&](int n) {
          const uint32_t off = 16 * kTileStride * (n >> 2) + 64 * (n & 3);
          return lds_v(va[0] + off, va[1] + off);
        };
        // PV operands: V^T through a ring of three (operand n in vv[n % 3]), P^T of head group g
        // for the first and second token half in p0[g], p1[g]
        bf16x8 vv[3], p0[4], p1[4];
        f32x16 s_acc;
        // A operand of the extra k-step: lane l (token l%32, dims 8(l/32) ..) holds bf16 1.0 in
        // dim 1 if token l%32 of sub-tile s+1 is ignored (lanes 0..31 only)
        // and the B operand: lane l (head l%32, dims 8(l/32) ..) holds the ignored score in dim 1.
        // Both are rebuilt every iteration instead of occupying registers.
        bf16x8 kflag, qflag;
        // dequantization of s+2 (raw slot r2 -> tile slot r2): this lane's 4 chunks of 16 values,
        // two in registers at a time
        const uint32_t draw = raw_r + r2 * kRawBytes;
        uint32_t dqa[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) dqa[m] = slot_base(dq_w[m], r2);
        uint32_t sc2 = 0;
        u32x4 rr0, rr1;
        bf16x8 dlo, dhi;
        // step k (0..15) of that dequantization: raw chunk cc = k / 4 (in rr0, rr1, rr0, rr1),
        // its first and second 8 values, then both bf16 chunks to the tile
        auto dequant_step = [&](int k) {
          const int cc = k >> 2, part = k & 3;
          const uint32_t sb = (sc2 >> (8 * (cc >> 1))) & 0xFFu;
          const u32x4& r = (cc & 1) ? rr1 : rr0;
          if (part == 0) dlo = dequant_fp8_8(r[0], r[1], sb);
          else if (part == 1) dhi = dequant_fp8_8(r[2], r[3], sb);
          else if (part == 2) {
            // bf16 chunks j = 2 cc (dlo) and 2 cc + 1 (dhi)
            lds_write16_at(dqa[(2 * cc) & 3] + 64 * ((2 * cc) >> 2), __builtin_bit_cast(u32x4, dlo));
            lds_write16_at(dqa[(2 * cc + 1) & 3] + 64 * ((2 * cc + 1) >> 2), __builtin_bit_cast(u32x4, dhi));
          }
        };
        // gather of s+4 (index slot r1 -> raw slot r1): tokens t < g_lim of the sub-tile are in
        // the index row (none past the live segment)
        const int g_pos0 = kUnitTokens * t0 + kSubTokens * (s + 4);   // fp8 sub-tile s+4
        const int g_lim = (s + 4 < nsub && p.topk > g_pos0) ? p.topk - g_pos0 : 0;
        // LDS byte addresses formed from the array itself (no generic-pointer null check)
        const uint32_t graw = lds_addr(smem) + kOffRaw + r1 * kRawBytes;
        int gv = 0;
        uint64_t gdat = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          // The P^T operands written at the end of the previous iteration (its last three LDS
          // operations are the K reads that follow them) are visible to every wave after this
          // barrier; the first P^T read is at step 27.
          if (i == 0) asm volatile("s_waitcnt lgkmcnt(3)\n\ts_barrier" ::: "memory");
          // operands are read kAhead MFMAs ahead, into phase B's first operands at the end
          if (i + kAhead < 32) {
            const int kk = i + kAhead;
            kb[kk % kRing] = lds_k(ka[kk & 1] + 64 * (kk >> 1));
          } else {
            // phase B's first operands: V^T 0 (step 27), P^T of the first token half of head
            // groups 0..3 (steps 27..30), V^T 1 (step 31)
            static_assert(kAhead == 5, "the reads below cover steps 32 - kAhead .. 31");
            if (!kFirst && i == 27) vv[0] = read_v(0);
            if (!kFirst && i < 31) p0[i - 27] = lds_k(p_rd + 2048 * (i - 27));
            if (!kFirst && i == 31) vv[1] = read_v(1);
          }
          // operands are awaited in pairs: before an even step, the next step's operand too, so
          // that every other step needs no wait of its own
          if ((i & 1) == 0) asm volatile("" ::"v"(kb[(i + 1) % kRing]));
          if (i == 0) mfma_qk_first(s_acc, kb[0], qreg[0]);
          else mfma_qk(s_acc, kb[i % kRing], qreg[i]);
          // extra k-step after the last one: the ignored score for ignored tokens of s+1, +0 for
          // the others (its operands are built two steps earlier); a sub-tile whose 32 tokens are
          // all valid needs none
          if (i == 31 && mk1 != 0xFFFFFFFFu) {
            // the compiler may build the operands' constant parts right before this step: two
            // wait states separate those VALU writes from the MFMA's read
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+v"(s_acc) : "v"(kflag), "v"(qflag));
          }
          if (i == 1) {
            sc2 = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(
                (uintptr_t)(raw_s + r2 * kRawBytes));
            rr0 = *(lds_u32x4*)(uintptr_t)(draw);
            rr1 = *(lds_u32x4*)(uintptr_t)(draw + 512);
            gv = *reinterpret_cast<const __attribute__((address_space(3))) int*>(
                (uintptr_t)(idx_r + r1 * kIdxBytes));
          } else if (i == 3) {
            const bool valid = idx_v < (uint32_t)(4 * g_lim) && gv >= 0;
            mk4 = (uint32_t)__ballot(valid);
            // ignored tokens and sub-tiles outside the segment read the zero record, so every copy
            // below is always issued
            const uint64_t a = g_base + (uint64_t)(int64_t)gv * kFp8Rec;
            gdat = valid ? a : g_zb;                         // chunk 2(w + 4i) + hh at +128 i
          }
          // gather copies at steps 4, 9, 14, 19 and 24 (spread out, so that the address work of
          // one 64-address copy is done before the next is issued): 4 chunk pairs (wave w moves
          // chunks 2(w + 4c) + hh of all 32 tokens) and the scale chunks of tokens 8w .. 8w+7
          // (lanes of the first half: the record's byte 512 is 512 - 32 w past gdat there)
          if (i >= 4 && i < 24 && (i - 4) % 5 == 0) {
            const int c = (i - 4) / 5;
            const uint32_t dst = __builtin_amdgcn_readfirstlane(graw + 1024 * (wave + 4 * c));
            const void* gp = (const void*)(uintptr_t)gdat;
            if (c == 0) copy16_to_lds_off<0>(gp, dst);
            else if (c == 1) copy16_to_lds_off<128>(gp, dst);
            else if (c == 2) copy16_to_lds_off<256>(gp, dst);
            else copy16_to_lds_off<384>(gp, dst);
          } else if (i == 24) {
            copy16_to_lds_masked((const void*)(uintptr_t)(gdat + (uint64_t)(512 - 32 * wave)),
                                 __builtin_amdgcn_readfirstlane(graw + 32 * 512), scale_lanes_fp8);
          }
          if (i == 29 && mk1 != 0xFFFFFFFFu) {
            // (the B operand's dim 9 in lanes 32..63 also holds the ignored score; A is 0 there)
            uint32_t f0, g0;
            const uint64_t ign = (uint64_t)(uint32_t)~mk1;
            asm volatile("v_cndmask_b32_e64 %0, 0, 1.0, %1" : "=v"(f0) : "s"(ign));
            asm volatile("v_mov_b32 %0, %1" : "=v"(g0) : "i"(kIgnoredScoreBits << 16));
            kflag = __builtin_bit_cast(bf16x8, u32x4{f0, 0u, 0u, 0u});
            qflag = __builtin_bit_cast(bf16x8, u32x4{g0, 0u, 0u, 0u});
          }
          if (i == 26) {
            // index load of sub-tile s+6 (positions 64 t0 + 32 (s+6) + 8 w + l, lanes l < 8) into
            // this wave's quarter of the shared index slot r0, from a buffer that ends at the index
            // row's end, or is empty past the live segment
            const int pos = kUnitTokens * t0 + kSubTokens * (s + 6);
            const int n_in = (s + 6 < nsub && p.topk > pos) ? p.topk - pos : 0;
            const uint64_t base = idx_row + (uint64_t)(4 * (int64_t)pos);
            const u32x4 rsrc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, (uint32_t)(4 * n_in),
                                0x00020000u};
            buffer_copy4_to_lds(rsrc, idx_l, lds_addr(smem) + kOffIdx + r0 * kIdxBytes + 32 * wave, 0xFFull);
          }
          // the second pair of raw chunks, once the first pair's values are converted
          if (i == 10) rr0 = *(lds_u32x4*)(uintptr_t)(draw + 1024);
          if (i == 14) rr1 = *(lds_u32x4*)(uintptr_t)(draw + 1536);
          // the first two of the four raw chunks here, the other two in phase B (whose LDS traffic
          // is lighter), four steps each
          if (i >= 8 && i < 16) dequant_step(i - 8);
          __builtin_amdgcn_sched_barrier(0);
        }

        // phase B: PV of sub-tile s for this wave's 128 dims and all four head groups, with the
        // softmax of sub-tile s+1 (this wave's heads). Step i accumulates block i % 16 = 4 b + g
        // (dim block 4 w + b, head group g) over token half i / 16: V^T operand i / 4 with the
        // P^T operand of group g. The P^T operands of sub-tile s+1 are written to the exchange
        // buffer after the barrier at step 27, by which every wave has read those of sub-tile s.
        const uint32_t kb_next[2] = {slot_base(k_addr[0], r2), slot_base(k_addr[1], r2)};
        bf16x8 pb_new[2];
        SoftmaxTemps st;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (!kFirst && (i + kAhead) % 4 == 0 && i + kAhead < 32) vv[((i + kAhead) / 4) % 3] = read_v((i + kAhead) / 4);
          if (!kFirst && i >= 16 - kAhead && i < 20 - kAhead) p1[i - (16 - kAhead)] = lds_k(p_rd + 2048 * (i - (16 - kAhead)) + 1024);
          // each new operand set is awaited in one wait
          if (!kFirst) {
            if (i == 0) asm volatile("" ::"v"(p0[0]), "v"(p0[1]), "v"(p0[2]), "v"(p0[3]), "v"(vv[0]));
            if (i == 16) asm volatile("" ::"v"(p1[0]), "v"(p1[1]), "v"(p1[2]), "v"(p1[3]), "v"(vv[1]));
            mfma_pv(oacc[i & 15], vv[(i / 4) % 3], i < 16 ? p0[i & 3] : p1[i & 3]);
          }
          // the scores are read by VALU instructions next: 20 wait states after the last QK^T
          // MFMA (the PV MFMA above runs meanwhile)
          if (i == 0) asm volatile("s_nop 15\n\ts_nop 3" : "+v"(s_acc));
          if ((i & 1) == 0) softmax_step_fp8(st, i >> 1, s_acc, mk1 != 0, pb_new);   // steps 0..15
          if (i >= 1 && i < 9) dequant_step(i + 7);
          if (i == 29) {
            // this wave's P^T operands of sub-tile s+1 (built at steps 26 and 28)
            asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024"
                         :: "v"(p_rd + 2048 * wave), "v"(pb_new[0]), "v"(pb_new[1]) : "memory");
          }
          if (i == 32 - kAhead) {
            // Start of iteration s+1, while the last PV MFMAs (operands already read) still run:
            // every V read of this iteration is complete, idx(s+5) and the gather of s+3 (issued
            // in iteration s-1) have landed and all waves' dequantization of s+2 is written, so
            // the first K operands of QK^T(s+2) can be read.
            wait_and_barrier(1 + kGatherFp8);
          }
          if (i >= 32 - kAhead) {
            const int kk = i - (32 - kAhead);
            kb[kk] = lds_k(kb_next[kk & 1] + 64 * (kk >> 1));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };


      // The fp8 pipeline starts at iteration -1 with sub-tiles 0 .. 2 gathered and idx(3), idx(4)
      // loaded (at the segment start, or here for a repeated pass) and sub-tile 0 dequantized.
      if (EXTRA && pass > 0) {                   // the first pass's were issued with Q
        load_indices(0, 0);                      // "iteration -6"
        load_indices(1, 1);                      // "iteration -5"
      }
      if (!EXTRA && pass > 0) {
        load_indices(0, 0);
        load_indices(1, 1);
        load_indices(2, 2);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int j = 0; j < 3; ++j) mk_first[j] = fp8_gather_first(j, nsub);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        load_indices(3, 0);
        load_indices(4, 1);
      }

      // slots of sub-tiles s, s+1, s+2 (s % 3 ... for s >= -4), rotated every iteration
      int r0 = 2, r1 = 0, r2 = 1;
      int s_first = -4;
      if constexpr (!EXTRA) {
        // every wave's part of sub-tile 0 has landed: dequantize it into tile slot 0
        wait_and_barrier(0);
        {
          const int lane = lane_id();
          const int t = lane & 31, hh = lane >> 5;
          const char* draw = raws;
          char* trow = tiles + t * kTileStride;
          const int sw = tile_xor(t);
          const int c0 = 8 * wave + 4 * hh;
          const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(draw + (32 * kSubTokens + t) * 16 + c0 / 2);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const u32x4 r = lds_read16(draw + ((c0 + cc) * kSubTokens + t) * 16);
            const uint32_t sb = (sc2 >> (8 * (cc >> 1))) & 0xFFu;
            lds_write16(trow + 16 * ((2 * (c0 + cc)) ^ sw), __builtin_bit_cast(u32x4, dequant_fp8_8(r[0], r[1], sb)));
            lds_write16(trow + 16 * ((2 * (c0 + cc) + 1) ^ sw), __builtin_bit_cast(u32x4, dequant_fp8_8(r[2], r[3], sb)));
          }
        }
        // tile 0 is complete and raw slot 0 free for the gather of sub-tile 3
        wait_and_barrier(0);
        mk0 = 0u;
        mk1 = mk_first[0];
        mk2 = mk_first[1];
        mk3 = mk_first[2];
        mk4 = 0u;
        // the first K operands of QK^T(0) (tile slot 0)
#pragma unroll
        for (int kk = 0; kk < kAhead; ++kk)
          kb[kk] = lds_k(k_addr[kk & 1] + 64 * (kk >> 1));
        s_first = -1;
      }

      auto rotate = [&]() {
        mk0 = mk1;
        mk1 = mk2;
        mk2 = mk3;
        mk3 = mk4;
        mk4 = 0;
        const int r_old = r0;
        r0 = r1;
        r1 = r2;
        r2 = r_old;
      };
      if constexpr (!EXTRA) {
        // Iteration s works on slots s % 3, (s+1) % 3, (s+2) % 3; after iteration -1, three
        // iterations with constant slots repeat, so every slot offset is a compile-time constant.
        // Each iteration's wait and barrier are issued by the previous iteration (every iteration
        // issues one index load and kGatherFp8 gather copies) or before the loop.
        fp8_iteration(std::true_type{}, s_first, 2, 0, 1);
        rotate();
#pragma clang loop unroll(disable)
        for (int s = s_first + 1; s < nsub; s += 3) {
          fp8_iteration(std::false_type{}, s, 0, 1, 2);
          rotate();
          if (s + 1 >= nsub) break;
          fp8_iteration(std::false_type{}, s + 1, 1, 2, 0);
          rotate();
          if (s + 2 >= nsub) break;
          fp8_iteration(std::false_type{}, s + 2, 2, 0, 1);
          rotate();
        }
      }
#pragma clang loop unroll(disable)
      for (int s = s_first; EXTRA && s < nsub; ++s) {
        // Top of iteration s: idx(s+4) and the gather of sub-tile s+2 (issued in iteration s-2)
        // have landed once only iteration s-1's operations (idx(s+5), gather(s+3)) may still be
        // pending.
        {
          wait_and_barrier(1 + gather_count(s + 3));
          load_indices(s + 6, (s + 6) % 3);
          if (s + 4 >= 0 && s + 4 < nsub) mk4 = gather(s + 4);
          // QK^T of sub-tile s+1 (tile (s+1) % 3).
          const bool do_qk = s + 1 >= 0 && s + 1 < nsub && mk1 != 0;
          f32x16 s_new = f32x16{};
          if (do_qk) {
            uint32_t a[8];
            slot_addr(k_addr, (s + 1) % 3, a);
            s_new = qk_chain(a, qreg);
          }
          // PV of sub-tile s, softmax of sub-tile s+1, dequantization of sub-tile s+2.
          if (s >= 0 && mk0 != 0) {
            uint32_t a[8];
            slot_addr(v_addr, s % 3, a);
            pv_chain(a, oacc, pb_cur);
          }
          if (do_qk) softmax(s_new, mk1, pb_cur);
          if (s + 2 >= 0 && s + 2 < nsub && mk2 != 0) dequant(s + 2, mk2);
        }
        rotate();
      }
      // O is read by VALU instructions below: 20 wait states after the last PV MFMA, which writes
      // block 15 (every other block was written at least one MFMA, 32 cycles, earlier).
      // The last iterations' copies (dummy gathers and index loads past the segment) are awaited
      // here, before this workgroup's LDS is reused or released.
      asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 15\n\ts_nop 3" : "+a"(oacc[15]) :: "memory");
      if constexpr (!EXTRA) {
        // the fp8 pipeline's per-lane state, reduced over the lane pair of each head; with no live
        // sub-tile the reference was never set, every probability was 0 and no pass is repeated
        m_max = ref_set ? max_xor32(m_lane) * p.scale_log2 : -__builtin_inff();
        l_sum = sum_xor32(l_lane);
      }

      // A second pass is needed when some head's probabilities relative to m_ref could have
      // overflowed; the decision has to be the same for the whole workgroup. After the second
      // pass every wave waits here until all waves are done with the tile slots: the epilogue's
      // staging area covers them, and another wave's last PV may still be reading its tile.
      if (pass > 0) {
        wait_and_barrier(0);
        break;
      }
      const bool any_big = __ballot(m_max > m_ref + kRefSlack) != 0;   // all lanes vote
      if (lane_id() == 0) redo_flags[wave] = any_big ? 1 : 0;
      wait_and_barrier(0);
      // (the flags are written again only after this segment's next pass or the next segment's
      // first, many barriers later, so no second barrier is needed before they are reused)
      const bool redo = (redo_flags[0] | redo_flags[1] | redo_flags[2] | redo_flags[3]) != 0;
      if (!redo) break;
      m_ref_next = m_max;
    }

    // ---- epilogue of this row segment. O^T block j holds head group hg(j) and dim block d(j):
    // lane l has head 32 hg + l%32 and dims 32 d + 8(r/4) + 4(l/32) + r%4 in register r. The fp8
    // pipeline splits PV by dims (hg = j % 4, d = 4 w + j / 4), the extra-cache variant by heads
    // (hg = w, d = j). Every head group's probability sum comes from the wave that owns its heads.
    {
      const int lane = lane_id();
      const int g = lane >> 5;
      const int h = lane & 31;
      const int head = head_base + h;
      const bool final_out = nsplit == 1;
      auto blk_hg = [&](int j) { return EXTRA ? wave : (j & 3); };
      auto blk_d = [&](int j) { return EXTRA ? j : 4 * wave + (j >> 2); };
      float inv_g[4];
      if constexpr (EXTRA) {
        inv_g[0] = l_sum > 0.0f ? 1.0f / l_sum : 0.0f;
      } else {
        // every wave is past its last PV (the barrier that ended the pass), so the exchange
        // buffer is free for the four head groups' sums
        float* const lsums = reinterpret_cast<float*>(smem + L::kOffP);
        if (g == 0) lsums[32 * wave + h] = l_sum;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float l = lsums[32 * k + h];
          inv_g[k] = l > 0.0f ? 1.0f / l : 0.0f;
        }
      }
      auto inv_of = [&](int j) { return EXTRA ? inv_g[0] : inv_g[j & 3]; };
      if (FUSED && final_out) {
        // Fused decode: the rotary pairs of the output (dim blocks 14 and 15: dims 448 + 2i,
        // 449 + 2i) are rotated back by the row's angle and every head row is cast to an fp8 record
        // (512 e4m3 values, then 16 e8m0 scales, one per 32-dim block d: k = ceil(log2(amax /
        // 448)), values rounded to nearest, ties to even), staged in LDS (head group hg's rows at
        // hg * kStageBytes, kFusedRow bytes apart) and stored by the group's wave as whole 528-byte
        // records.
        const float* cs = p.rope_cos + (int64_t)row * 32 + 2 * g;
        const float* sn = p.rope_sin + (int64_t)row * 32 + 2 * g;
        // scale bytes: per 4-block word (extra-cache variant: words 0..3 of the wave's heads;
        // fp8 pipeline: word w of head group 0..3)
        uint32_t kb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int hg = blk_hg(j), d = blk_d(j);
          const float inv = inv_of(j);
          float y[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) y[r] = oacc[j][r] * inv;
          if (d >= 14) {
            // dims 32 d + 8 rb + 4 g + {0..3}: pairs 16 (d - 14) + 4 rb + 2 g + {0, 1}
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
              const f32x2 c = *reinterpret_cast<const f32x2*>(cs + 16 * (d - 14) + 4 * rb);
              const f32x2 sv = *reinterpret_cast<const f32x2*>(sn + 16 * (d - 14) + 4 * rb);
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                const float x0 = y[4 * rb + 2 * jj], x1 = y[4 * rb + 2 * jj + 1];
                y[4 * rb + 2 * jj] = x0 * c[jj] + x1 * sv[jj];
                y[4 * rb + 2 * jj + 1] = x1 * c[jj] - x0 * sv[jj];
              }
            }
          }
          float a = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) a = fmaxf(a, __builtin_fabsf(y[r]));
          a = max_xor32(a);
          const int k = fp8_block_exponent(a);
          const uint32_t rowa = lds_addr(smem + hg * kStageBytes + h * kFusedRow + 4 * g) + 32 * d;
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const uint32_t w = e4m3_codes4(y[4 * rb], y[4 * rb + 1], y[4 * rb + 2], y[4 * rb + 3], k);
            *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(rowa + 8 * rb) = w;
          }
          if (EXTRA) kb[j >> 2] |= (uint32_t)(k + 127) << (8 * (j & 3));
          else kb[j & 3] |= (uint32_t)(k + 127) << (8 * (j >> 2));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (g == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // word i: head group hg, scale bytes 4 q .. 4 q + 3
            const int hg = EXTRA ? wave : i, q = EXTRA ? i : wave;
            *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(
                lds_addr(smem + hg * kStageBytes + h * kFusedRow + kHeadDim + 4 * q)) = kb[i];
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // this wave's head group: record rr, 16-byte chunk c (33 per record) from lane (33 rr + c) % 64
        char* const stage = smem + wave * kStageBytes;
        for (int e = lane; e < 32 * (kFusedRow / 16); e += 64) {
          const int rr = e / (kFusedRow / 16), c = e % (kFusedRow / 16);
          if (head_base + rr < p.h_q) {
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                lds_addr(stage + rr * kFusedRow + 16 * c));
            *reinterpret_cast<u32x4*>(p.out_fp8 + ((int64_t)row * p.h_q + head_base + rr) * kFp8Rec + 16 * c) = v;
          }
        }
      } else if (final_out) {
        // Final rows in bf16, staged through LDS so that every store writes one head's 1 KB row:
        // head 32 hg + h at hg * kStageBytes + h * kStageRow (the tiles and the start of the raw
        // slots, free after the pass); 8-byte unit u (dims 4u .. 4u+3) at + 8u. Each wave writes
        // its blocks, then stores the 32 rows of its own head group.
        const uint32_t wbase = lds_addr(smem + h * kStageRow + 8 * g);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t jbase = wbase + blk_hg(j) * kStageBytes + 64 * blk_d(j);
          const float inv = inv_of(j);
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (__bf16)(oacc[j][4 * jb + i] * inv);
            *reinterpret_cast<lds_bf16x4_w*>(jbase + 16 * jb) = o;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // row r: lane l moves dims 8l .. 8l+7 (units 2l, 2l+1), stored from a uniform row address
        const uint32_t rbase = lds_addr(smem + wave * kStageBytes + 16 * lane);
        char* const orow = reinterpret_cast<char*>(p.out) + ((int64_t)row * p.h_q + head_base) * (2 * kHeadDim);
        for (int r = 0; r < 32 && head_base + r < p.h_q; ++r) {
          const bf16x4 lo = *reinterpret_cast<const lds_bf16x4_w*>(rbase + r * kStageRow);
          const bf16x4 hi = *reinterpret_cast<const lds_bf16x4_w*>(rbase + r * kStageRow + 8);
          *reinterpret_cast<bf16x8*>(orow + r * (2 * kHeadDim) + 16 * lane) =
              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      } else if constexpr (!FUSED) {
        // the normalised bf16 partial of this split, staged like the final rows
        const uint32_t wbase = lds_addr(smem + h * kStageRow + 8 * g);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t jbase = wbase + blk_hg(j) * kStageBytes + 64 * blk_d(j);
          const float inv = inv_of(j);
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (__bf16)(oacc[j][4 * jb + i] * inv);
            *reinterpret_cast<lds_bf16x4_w*>(jbase + 16 * jb) = o;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const uint32_t rbase = lds_addr(smem + wave * kStageBytes + 16 * lane);
        char* const prow = static_cast<char*>(p.part_o) + ((int64_t)slot * p.h_q + head_base) * (2 * kHeadDim);
        for (int r = 0; r < 32 && head_base + r < p.h_q; ++r) {
          const bf16x4 lo = *reinterpret_cast<const lds_bf16x4_w*>(rbase + r * kStageRow);
          const bf16x4 hi = *reinterpret_cast<const lds_bf16x4_w*>(rbase + r * kStageRow + 8);
          *reinterpret_cast<bf16x8*>(prow + r * (2 * kHeadDim) + 16 * lane) =
              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      } else {
        // the fused decode's fp32 partial, which its merge encodes into fp8 records
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int head_j = blockIdx.y * kGroupHeads + 32 * blk_hg(j) + h;
          const float inv = inv_of(j);
          if (head_j < p.h_q) {
            const int64_t base = ((int64_t)slot * p.h_q + head_j) * kHeadDim;
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
              const int dim = 32 * blk_d(j) + 8 * jb + 4 * g;
              f32x4 o;
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = oacc[j][4 * jb + i] * inv;
              *reinterpret_cast<f32x4*>(static_cast<float*>(p.part_o) + base + dim) = o;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (g == 0 && head < p.h_q) {
        const float lse = l_sum > 0.0f ? (m_ref + __log2f(l_sum)) * 0.69314718055994530942f
                                       : -__builtin_inff();
        if (final_out)
          p.lse[(int64_t)row * p.h_q + head] = lse;
        else
          p.part_lse[(int64_t)slot * p.h_q + head] = lse;
      }
    }
    ++row;
    t0 = 0;
    first_seg = false;
  }
}

}  // namespace

int launch_sparse_decode_wide(const DecodeParams& p, int parts, int groups, hipStream_t stream) {
  dim3 grid(parts, groups);
  const bool fused = p.out_fp8 != nullptr;
  if (p.extra_topk > 0) {
    if (fused)
      hipLaunchKernelGGL((sparse_decode_wide_kernel<true, true>), grid, dim3(64 * kWaves), 0, stream, p);
    else
      hipLaunchKernelGGL((sparse_decode_wide_kernel<true, false>), grid, dim3(64 * kWaves), 0, stream, p);
  } else {
    if (fused)
      hipLaunchKernelGGL((sparse_decode_wide_kernel<false, true>), grid, dim3(64 * kWaves), 0, stream, p);
    else
      hipLaunchKernelGGL((sparse_decode_wide_kernel<false, false>), grid, dim3(64 * kWaves), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
