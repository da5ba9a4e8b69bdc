// Sparse MLA decode kernel for gfx950, 64-head groups (h_q <= 64).
//
// Same computation as the other decode kernels (page "flops/flashmla-decode-fp8-fp4-kv", sections
// "Arithmetic intensity" and "Workarounds"; page "deepseek-ai/FlashMLA", section "Key technical
// details"): per query row and head, one softmax over the row's selected tokens, key and value both
// the 512-dim latent decoded from the token's 528-byte fp8 record (or 288-byte fp4 record of the
// extra cache), negative indices ignored, natural-log lse returned beside the output.
//
// The software pipeline is the one of the 128-head kernel (mla_decode_wide.hip), cut to 64 heads:
// one workgroup of 4 waves per CU, one wave per SIMD, one stream of 32-token sub-tiles. Wave w owns
//   Q      bf16, heads 16w..16w+15 x 512 dims, 64 VGPRs (B operand of v_mfma_f32_16x16x32_bf16)
//   S^T    fp32, 32 tokens x its 16 heads per sub-tile, two 16x16 blocks (8 VGPRs)
//   O^T    fp32, dims 128w..128w+127 x all 64 heads, 8 blocks of 32x32 (128 AGPRs)
// so QK^T reads the whole K tile per wave for a quarter of the heads, while PV reads only the
// wave's quarter of the V tile. The softmax of a head stays in its wave; the four waves' P^T
// operands meet in a 4 KB LDS exchange buffer, in the B-operand layout of the PV product.
//
// Iteration s of the pipeline, behind two workgroup barriers:
//   phase A  the 32 QK^T MFMAs of sub-tile s+1 (16x16x32, two token blocks alternating), with the
//            index load of s+6, the gather of s+4 and the dequantization of s+2 between them;
//   phase B  the 16 PV MFMAs of sub-tile s (32x32x16), with the softmax of s+1 and the K operands
//            of the next QK^T between them.
// Gathers, index loads, the raw-record and bf16 tile layouts and the dequantization are those of
// the 128-head kernel. With an extra cache (EXTRA) a segment's units past the row's fp8 units are
// fp4 units. Phase A, which holds all of the dequantization, is compiled once per format of the
// sub-tile it dequantizes, chosen by one wave-uniform branch per iteration (with one wave per SIMD a
// taken branch stalls the SIMD, so a branch per step costs; a copy of phase B per format would make
// the compiler move the 128 O accumulators where the copies join). An fp4 sub-tile issues the same five record copies as an fp8 one (two of them read the zero record into
// chunks the fp4 layout leaves unused), so the fixed s_waitcnt counts hold for any mix.

#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

struct alignas(16) ZeroRecord64 {
  uint8_t bytes[1024];
  uint32_t tag;
};
// the gather source of ignored tokens and of sub-tiles outside the segment: decodes to zeros
__device__ const ZeroRecord64 g_zero64 = {{}, 1u};

// Raw score of ignored tokens (-2^100): after scaling far below any real score, so its probability
// is exactly 0 and it never wins a maximum.
constexpr float kIgnoredScore = -1.2676506002282294e30f;

constexpr int kWaves = 4;
constexpr int kGroupHeads = 16 * kWaves;
// bf16 tile: token row r at r * 1088 bytes, 16-byte chunk c at position c ^ xor64(r) within its
// aligned group of four (the layout of the 128-head kernel, free of bank conflicts for 16 rows at
// one chunk, for 4 rows x 4 chunks of the transposing reads and for 8 rows at one chunk written)
constexpr int kTileStride = 1088;
constexpr int kTileBytes = kSubTokens * kTileStride;
constexpr int kRawBytes = kFp8Chunks * kSubTokens * 16;   // [chunk][token][16 B]
constexpr int kIdxBytes = kSubTokens * 4;
constexpr int kStages = 3;
constexpr int kOffRaw = kStages * kTileBytes;
constexpr int kOffIdx = kOffRaw + kStages * kRawBytes;     // one ring shared by the waves
constexpr int kOffFlags = kOffIdx + kStages * kIdxBytes;
constexpr int kOffScan = kOffFlags + 16;
constexpr int kOffP = kOffScan + 2 * kWaves * 4;
// P^T exchange: head block hb (32 heads), token half ks, 16 bytes per lane at 1024 (2 hb + ks)
constexpr int kPBytes = 2 * 2 * 64 * 16;
constexpr int kLdsBytes = kOffP + kPBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
static_assert(kOffP % 16 == 0, "16-byte P^T operands");
// bf16 output staging: 64 head rows of 1 KB, 1032 bytes apart, from the start of LDS
constexpr int kStageRow = 1032;
static_assert(kGroupHeads * kStageRow <= kOffIdx, "the staging leaves the index ring alone");
constexpr float kRefSlack = 64.0f;
constexpr int kGatherFp8 = 5;
// QK^T operands are read kAhead MFMAs (16 cycles each) ahead through a ring of kRing registers
constexpr int kAhead = 10;
constexpr int kRing = kAhead + 2;

__device__ __forceinline__ int lane64() {
  int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}
__device__ __forceinline__ uint32_t lds_a(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ int xor64(int r) { return (((r >> 1) ^ (r >> 3)) & 1) * 2 + ((r >> 2) & 1); }

template <int OFF>
__device__ __forceinline__ void g2l16_off(const void* gptr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off offset:%2"
      :
      : "s"(lds_base - OFF), "v"(gptr), "i"(OFF)
      : "memory");
}
__device__ __forceinline__ void g2l16_masked(const void* gptr, uint32_t lds_base, uint64_t lanes) {
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
__device__ __forceinline__ void g2l4_masked(const void* gptr, uint32_t lds_base, uint64_t lanes) {
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
// 4-byte buffer -> LDS copy by the lanes in `lanes`; offsets at or past the buffer's size read
// nothing from memory and return 0
__device__ __forceinline__ void buf2l4(u32x4 rsrc, uint32_t voff, uint32_t lds_base, uint64_t lanes) {
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

// QK^T step (16x16x32, scores in VGPRs) and PV step (32x32x16, O in the accumulation registers)
__device__ __forceinline__ void mfma_qk16_first(f32x4& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma_qk16(f32x4& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma_pv32(f32x16& o, const bf16x8& v, const bf16x8& pb) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(pb));
}

typedef __attribute__((address_space(3))) const u32x4 lds_u32x4_r;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_rw;
__device__ __forceinline__ bf16x8 lds_b128(uint32_t a) {
  return __builtin_bit_cast(bf16x8, *(lds_u32x4_r*)(uintptr_t)a);
}
__device__ __forceinline__ bf16x8 lds_vt(uint32_t a0, uint32_t a1) {
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_rw*)(uintptr_t)a0);
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_rw*)(uintptr_t)a1);
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void lds_w16(uint32_t a, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)(uintptr_t)a = v;
}

// wait until at most n of this wave's vector memory operations are outstanding and all of its LDS
// operations are done, then synchronise the workgroup (n wave-uniform)
__device__ __forceinline__ void wait_barrier(int n) {
  switch (n) {
    case 6: asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// maximum and sum over the four lanes of one head (l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Where sub-tile j of a segment that starts at unit t0 takes its entries: the extra (fp4) cache
// when its unit lies past the row's tiles_k fp8 units; pos0 is its first entry in that cache's
// index row of `count` entries.
struct SubTile {
  bool x;
  int pos0;
  int count;
};
template <bool EXTRA>
__device__ __forceinline__ SubTile locate(const DecodeParams& p, int t0, int j) {
  // unit t0 + j / 2 is an fp4 one when t0 + j / 2 >= tiles_k, i.e. when 2 t0 + j >= 2 tiles_k
  SubTile st;
  st.x = EXTRA && 2 * t0 + j >= 2 * p.tiles_k;
  st.pos0 = kUnitTokens * (st.x ? t0 - p.tiles_k : t0) + kSubTokens * j;
  st.count = st.x ? p.extra_topk : p.topk;
  return st;
}

template <bool EXTRA>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_decode_h64_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  char* const tiles = smem;
  char* const raws = smem + kOffRaw;
  char* const idx_ring = smem + kOffIdx;
  int* const redo_flags = reinterpret_cast<int*>(smem + kOffFlags);
  int* const scan_slots = reinterpret_cast<int*>(smem + kOffScan);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group_base = blockIdx.y * kGroupHeads;
  const int head_base = group_base + 16 * wave;                 // this wave's first QK^T head
  const uint64_t scale_lanes = 0xFFull << (8 * wave);           // scale chunks of tokens 8w..8w+7
  const uint64_t scale_lanes_x = scale_lanes | (scale_lanes << 32);  // fp4: both 16 B scale halves

  int row, t0, end_row, end_tile, slot_first;
  if (p.prefill_parts > 0) {
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
    int nsub = nsub_all;

    // index load of sub-tile j into the shared slot `slot`: wave w loads entries 8w .. 8w+7
    // (clamped addresses; a selection of size 0 reads the schedule instead)
    auto load_indices = [&](int j, int slot) {
      const int e = 8 * wave + (lane64() & 7);
      const SubTile st = locate<EXTRA>(p, t0, j);
      const int32_t* src_ptr = p.sched;
      if (j < nsub && st.count > 0)
        src_ptr = (st.x ? p.xidx : p.idx) + (int64_t)row * st.count + min(st.pos0 + e, st.count - 1);
      g2l4_masked(src_ptr, __builtin_amdgcn_readfirstlane(lds_a(idx_ring + slot * kIdxBytes) + 32 * wave),
                  0xFFull);
    };

    int tid = 64 * wave + lane64();
    asm volatile("" : "+v"(tid));
    // live-length scan: entry e of the segment is entry e % 32 of sub-tile e / 32
    auto scan_batch = [&](int e0, int (&v)[8]) {
      bool in[8];
      const int32_t* src[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 64 * kWaves * u + tid;
        if constexpr (EXTRA) {
          const SubTile st = locate<EXTRA>(p, t0, min(e / kSubTokens, nsub_all - 1));
          const int pos = st.pos0 + e % kSubTokens;
          in[u] = e / kSubTokens < nsub_all && pos < st.count;
          src[u] = st.count > 0 ? (st.x ? p.xidx : p.idx) + (int64_t)row * st.count + min(pos, st.count - 1)
                                : p.sched;
        } else {
          const int pos = kUnitTokens * t0 + e;
          in[u] = e / kSubTokens < nsub_all && pos < p.topk;
          src[u] = p.topk > 0 ? p.idx + (int64_t)row * p.topk + min(pos, p.topk - 1) : p.sched;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *src[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = in[u] ? v[u] : -1;
    };
    // gather of sub-tile j (< 3) from index slot j into raw slot j; returns its validity mask
    auto gather_first = [&](int j, int live) -> uint32_t {
      const int lane = lane64();
      const int t = lane & 31, hh = lane >> 5;
      const SubTile st = locate<EXTRA>(p, t0, j);
      const int gv = *reinterpret_cast<const int*>(idx_ring + j * kIdxBytes + 4 * t);
      const bool valid = j < live && st.pos0 + t < st.count && gv >= 0;
      const uint32_t mask = (uint32_t)__ballot(valid);
      const uint32_t graw = lds_a(smem) + kOffRaw + j * kRawBytes;
      if (EXTRA && st.x) {
        const uint8_t* grec = valid ? p.xc + (int64_t)gv * kFp4Rec : g_zero64.bytes;
        const uint8_t* gdat = grec + 32 * wave + 16 * hh;
        g2l16_off<0>(gdat, graw + 1024 * wave);
        g2l16_off<128>(gdat, graw + 1024 * (wave + 4));
        g2l16_masked(grec + 256 + 16 * hh, graw + 16 * 512, scale_lanes_x);
      } else {
        const uint8_t* grec = valid ? p.kc + (int64_t)gv * kFp8Rec : g_zero64.bytes;
        const uint8_t* gdat = grec + 32 * wave + 16 * hh;
        g2l16_off<0>(gdat, graw + 1024 * wave);
        g2l16_off<128>(gdat, graw + 1024 * (wave + 4));
        g2l16_off<256>(gdat, graw + 1024 * (wave + 8));
        g2l16_off<384>(gdat, graw + 1024 * (wave + 12));
        g2l16_masked(grec + 512, graw + 32 * 512, scale_lanes);
      }
      return mask;
    };
    uint32_t mk_first[3] = {0u, 0u, 0u};
    int scan_v[8];
    scan_batch(0, scan_v);
    load_indices(0, 0);
    load_indices(1, 1);
    load_indices(2, 2);

    // ---- Q of this wave's 16 heads, B-operand layout of v_mfma_f32_16x16x32_bf16: lane l holds
    // head 16w + l%16, dims 32kk + 8(l/16) .. +7 of k-step kk. Heads past h_q load a copy of the
    // last head; their results are never stored.
    bf16x8 qreg[16];
    {
      const int lane = lane64();
      const int qh = min(head_base + (lane & 15), p.h_q - 1);
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          p.q + ((int64_t)row * p.h_q + qh) * kHeadDim + 8 * (lane >> 4));
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) qreg[kk] = __builtin_bit_cast(bf16x8, qp[4 * kk]);
    }
    // The scan batch and idx(0 .. 2) have landed once at most the 16 Q loads are outstanding;
    // the barrier makes every wave's quarter of the index slots visible (and keeps a later
    // segment's gathers until every wave is done with the previous epilogue's staging).
    asm volatile("s_waitcnt vmcnt(16)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int j = 0; j < 3; ++j) mk_first[j] = gather_first(j, nsub_all);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_indices(3, 0);
    load_indices(4, 1);

    // ---- live length of the segment (the last sub-tile with a valid entry, over all waves)
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
      int wmax = -1;
      if (__ballot(last >= 0) != 0) {
        wmax = 0;
        for (int b = 31 - __builtin_clz((unsigned)nsub_all); b >= 0; --b)
          if (__ballot(last >= (wmax | (1 << b))) != 0) wmax |= 1 << b;
      }
      int* const slots = scan_slots + kWaves * seg_parity;
      if (lane64() == 0) slots[wave] = wmax;
      __syncthreads();
      nsub = __builtin_amdgcn_readfirstlane(max(max(slots[0], slots[1]), max(slots[2], slots[3])) + 1);
      seg_parity ^= 1;
    }
    typedef __attribute__((address_space(1))) const int32_t global_i32;
    global_i32* split_ptr = (global_i32*)p.split_ptr;
    asm volatile("" : "+s"(split_ptr));
    const int split_base = split_ptr ? split_ptr[row] : 0;
    const int nsplit = split_ptr ? split_ptr[row + 1] - split_base : 1;
    const int slot = first_seg ? slot_first : split_base;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): Q resident before the pipeline's copies

    // ---- per-lane LDS addresses in tile / raw / index slot 0 (add slot * bytes)
    //  k_addr[tb]  QK^T A operand, token block tb: row 16 tb + l%16, logical chunk 4 kk + l/16 at
    //              + 64 kk (the chunk XOR stays inside the aligned group of four)
    //  v_addr[h]   PV A operand (V^T of this wave's dim block 4w + b, token half ks) at
    //              + 64 b + 16 kTileStride ks: token row 16 ks + 8((l/16)/2) + 4h + (l%16)/4,
    //              logical chunk 16 w + 4 b + 2((l/16)%2) + (l%4)/2, 8-byte half l%2
    //  dq_w[m]     the lane's bf16 chunks of its dequantization (chunk 2 c0 + j at dq_w[j % 4]
    //              + 64 (j / 4)); raw_r / raw_s its fp8 chunk and scale bytes (token t);
    //              raw_r4 / raw_s4 its fp4 chunks 4w + 2hh, +1 and e4m3 scale bytes 8w + 4hh .. +3
    //  idx_r       index entry of token t; idx_v its byte offset in a 32-entry block; idx_l the
    //              byte offset of the entry this lane loads into the shared ring
    //  g_base / g_zb  record byte 32 w + 16 hh of record 0 of the cache / of the zero record
    //  p_rd        P^T exchange buffer, this lane's 16 bytes of head block 0, token half 0
    uint32_t k_addr[2], v_addr[2], dq_w[4], raw_r, raw_s, raw_r4 = 0, raw_s4 = 0, idx_r, idx_v, idx_l, p_rd;
    uint64_t g_base, g_zb;
    {
      const int lane = lane64();
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int r = 16 * tb + (lane & 15);
        k_addr[tb] = lds_a(tiles + r * kTileStride + 16 * ((lane >> 4) ^ xor64(r)));
      }
      const int g2 = lane >> 4, jj = lane & 15;
      const int c_lo = 2 * (g2 & 1) + ((jj & 3) >> 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rw = 8 * (g2 >> 1) + 4 * h + (jj >> 2);
        v_addr[h] = lds_a(tiles + rw * kTileStride + 16 * (c_lo ^ xor64(rw)) + 8 * (jj & 1)) + 256 * wave;
      }
      const int t = lane & 31, hh = lane >> 5;
      const int sw = xor64(t);
      const int c0 = 8 * wave + 4 * hh;
#pragma unroll
      for (int m = 0; m < 4; ++m) dq_w[m] = lds_a(tiles + t * kTileStride + 32 * c0 + 16 * (m ^ sw));
      raw_r = lds_a(raws + (c0 * kSubTokens + t) * 16);
      raw_s = lds_a(raws + (32 * kSubTokens + t) * 16 + c0 / 2);
      idx_r = lds_a(idx_ring + 4 * t);
      idx_v = 4 * t;
      idx_l = 4 * (8 * wave + (lane & 7));
      p_rd = lds_a(smem + kOffP) + 16 * lane;
      g_base = (uint64_t)(uintptr_t)(p.kc + 32 * wave + 16 * hh);
      g_zb = (uint64_t)(uintptr_t)(g_zero64.bytes + 32 * wave + 16 * hh);
      asm volatile("" : "+v"(k_addr[0]), "+v"(k_addr[1]), "+v"(v_addr[0]), "+v"(v_addr[1]),
                   "+v"(dq_w[0]), "+v"(dq_w[1]), "+v"(dq_w[2]), "+v"(dq_w[3]), "+v"(raw_r),
                   "+v"(raw_s), "+v"(idx_r), "+v"(idx_v), "+v"(idx_l), "+v"(p_rd), "+v"(g_base),
                   "+v"(g_zb));
      if constexpr (EXTRA) {
        raw_r4 = lds_a(raws + ((4 * wave + 2 * hh) * kSubTokens + t) * 16);
        raw_s4 = lds_a(raws + ((16 + (wave >> 1)) * kSubTokens + t) * 16 + 8 * (wave & 1) + 4 * hh);
        asm volatile("" : "+v"(raw_r4), "+v"(raw_s4));
      }
    }
    const uint64_t idx_row = (uint64_t)(uintptr_t)(p.idx + (int64_t)row * p.topk);
    const uint64_t xidx_row = EXTRA ? (uint64_t)(uintptr_t)(p.xidx + (int64_t)row * p.extra_topk) : 0;
    const uint64_t x_delta = EXTRA ? (uint64_t)(uintptr_t)p.xc - (uint64_t)(uintptr_t)p.kc : 0;
    // operand base of slot sl; slot 2 starts past 64 KB, so its base is formed in a register
    auto slot_base = [&](uint32_t base, int sl) -> uint32_t {
      uint32_t a = base + sl * kTileBytes;
      if (sl == 2) asm volatile("" : "+v"(a));
      return a;
    };

    // ---- softmax state: scores in log2 units against a fixed per-head reference m_ref (the
    // maximum of the head's first sub-tile with a valid token); if some head's true maximum ends
    // more than kRefSlack above it, the segment is computed again with m_ref = that maximum.
    float m_ref_next = -__builtin_inff();
    f32x16 oacc[8];
    float m_ref, m_max, l_sum;
    float m_lane, l_lane, ref_off;
    bool ref_set;
    for (int pass = 0;; ++pass) {
      m_ref = m_ref_next;
      m_lane = -__builtin_inff();
      l_lane = 0.0f;
      ref_set = pass > 0;
      ref_off = pass > 0 ? -m_ref : 0.0f;
      {
        const bf16x8 zero8 = bf16x8{};
        asm volatile(
            "s_nop 4\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %1, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %2, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %3, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %4, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %5, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %6, %8, %8, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %7, %8, %8, 0"
            : "=a"(oacc[0]), "=a"(oacc[1]), "=a"(oacc[2]), "=a"(oacc[3]), "=a"(oacc[4]),
              "=a"(oacc[5]), "=a"(oacc[6]), "=a"(oacc[7])
            : "v"(zero8));
      }

      // validity masks of sub-tiles s .. s+4 and the QK^T K operand ring
      uint32_t mk0 = 0, mk1 = 0, mk2 = 0, mk3 = 0, mk4 = 0;
      bf16x8 kb[kRing];

      // ---- one iteration (s in [-1, nsub)); r0, r1, r2 are the slots of sub-tiles s, s+1, s+2
      auto iteration = [&](auto first, int s, int r0, int r1, int r2) {
        // iteration -1 (first): there is no sub-tile -1, so it skips PV and the reads of its
        // operands; tile slot 2 and the P^T buffer are then never read before they are written
        constexpr bool kFirst = decltype(first)::value;
        // sub-tile s+2, dequantized in this iteration, is an fp4 one
        const bool dx = EXTRA && __builtin_amdgcn_readfirstlane(locate<EXTRA>(p, t0, s + 2).x ? 1 : 0) != 0;
        const uint32_t ka[2] = {slot_base(k_addr[0], r1), slot_base(k_addr[1], r1)};
        const uint32_t va[2] = {slot_base(v_addr[0], r0), slot_base(v_addr[1], r0)};
        // V^T operand n (0..7): token half n / 4, this wave's dim block n % 4
        auto read_v = [&](int n) {
          const uint32_t off = 16 * kTileStride * (n >> 2) + 64 * (n & 3);
          return lds_vt(va[0] + off, va[1] + off);
        };
        // PV operands: V^T through a ring of four, P^T of head block hb for the two token halves
        bf16x8 vv[4], p0[2], p1[2];
        f32x4 sacc[2];
        // dequantization of s+2 (raw slot r2 -> tile slot r2), four raw chunks in two registers
        const uint32_t draw = raw_r + r2 * kRawBytes;
        uint32_t dqa[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) dqa[m] = slot_base(dq_w[m], r2);
        uint32_t sc2 = 0;
        u32x4 rr0, rr1, fr0, fr1;
        bf16x8 dlo, dhi;
        u32x4 flo, fhi;
        float fsc = 0.0f;
        // step k of 16: quarter k % 4 of the lane's 16-value block k / 4 (fp8: two steps convert,
        // one writes; fp4: four e2m1 values times the block's e4m3 scale per step, written at the end)
        auto dequant_step = [&](auto fp4, int k) {
          const int cc = k >> 2, part = k & 3;
          if constexpr (decltype(fp4)::value) {
            const u32x4& r = (cc >> 1) ? fr1 : fr0;
            const uint32_t w = r[2 * (cc & 1) + (part >> 1)];
            if (part == 0) fsc = e4m3_to_f32(sc2 >> (8 * cc));
            uint32_t a, b;
            if (part & 1) {
              a = __builtin_bit_cast(uint32_t, fp4_byte<2>(w, fsc));
              b = __builtin_bit_cast(uint32_t, fp4_byte<3>(w, fsc));
            } else {
              a = __builtin_bit_cast(uint32_t, fp4_byte<0>(w, fsc));
              b = __builtin_bit_cast(uint32_t, fp4_byte<1>(w, fsc));
            }
            u32x4& d = (part >> 1) ? fhi : flo;
            d[2 * (part & 1)] = a;
            d[2 * (part & 1) + 1] = b;
            if (part == 3) {
              lds_w16(dqa[(2 * cc) & 3] + 64 * ((2 * cc) >> 2), flo);
              lds_w16(dqa[(2 * cc + 1) & 3] + 64 * ((2 * cc + 1) >> 2), fhi);
            }
            return;
          }
          const uint32_t sb = (sc2 >> (8 * (cc >> 1))) & 0xFFu;
          const u32x4& r = (cc & 1) ? rr1 : rr0;
          if (part == 0) dlo = dequant_fp8_8(r[0], r[1], sb);
          else if (part == 1) dhi = dequant_fp8_8(r[2], r[3], sb);
          else if (part == 2) {
            lds_w16(dqa[(2 * cc) & 3] + 64 * ((2 * cc) >> 2), __builtin_bit_cast(u32x4, dlo));
            lds_w16(dqa[(2 * cc + 1) & 3] + 64 * ((2 * cc + 1) >> 2), __builtin_bit_cast(u32x4, dhi));
          }
        };
        // gather of s+4 (index slot r1 -> raw slot r1); gdat2 is the source of copies 2 and 3, the
        // zero record for an fp4 sub-tile (its 256 data bytes are copies 0 and 1)
        const SubTile gs = locate<EXTRA>(p, t0, s + 4);
        const bool gx = EXTRA && gs.x;
        const int g_lim = (s + 4 < nsub && gs.count > gs.pos0) ? gs.count - gs.pos0 : 0;
        const uint32_t graw = lds_a(smem) + kOffRaw + r1 * kRawBytes;
        int gv = 0;
        uint64_t gdat = 0, gdat2 = 0;

        // phase A: QK^T of sub-tile s+1, step i = token block i % 2 of k-step i / 2; one copy per
        // format of s+2's dequantization
        auto phase_a = [&](auto fp4) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          // The P^T operands written at the end of the previous iteration (its last six LDS
          // operations are the K reads that follow them) are visible after this barrier.
          if (i == 0) asm volatile("s_waitcnt lgkmcnt(6)\n\ts_barrier" ::: "memory");
          if (i + kAhead < 32) {
            const int st = i + kAhead;
            kb[st % kRing] = lds_b128(ka[st & 1] + 64 * (st >> 1));
          }
          // phase B's first operands
          if (!kFirst && i == 27) vv[0] = read_v(0);
          if (!kFirst && i == 28) p0[0] = lds_b128(p_rd);
          if (!kFirst && i == 29) vv[1] = read_v(1);
          if (!kFirst && i == 30) p0[1] = lds_b128(p_rd + 2048);
          if (!kFirst && i == 31) vv[2] = read_v(2);
          if ((i & 1) == 0) asm volatile("" ::"v"(kb[(i + 1) % kRing]));
          if (i < 2) mfma_qk16_first(sacc[i], kb[i % kRing], qreg[0]);
          else mfma_qk16(sacc[i & 1], kb[i % kRing], qreg[i >> 1]);
          if (i == 1) {
            if constexpr (decltype(fp4)::value) {
              const uint32_t draw4 = raw_r4 + r2 * kRawBytes;
              sc2 = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
                  (uintptr_t)(raw_s4 + r2 * kRawBytes));
              fr0 = *(lds_u32x4_r*)(uintptr_t)(draw4);
              fr1 = *(lds_u32x4_r*)(uintptr_t)(draw4 + 512);
            } else {
              sc2 = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(
                  (uintptr_t)(raw_s + r2 * kRawBytes));
              rr0 = *(lds_u32x4_r*)(uintptr_t)(draw);
              rr1 = *(lds_u32x4_r*)(uintptr_t)(draw + 512);
            }
            gv = *reinterpret_cast<const __attribute__((address_space(3))) int*>(
                (uintptr_t)(idx_r + r1 * kIdxBytes));
          } else if (i == 3) {
            const bool valid = idx_v < (uint32_t)(4 * g_lim) && gv >= 0;
            mk4 = (uint32_t)__ballot(valid);
            const uint64_t a =
                g_base + (gx ? x_delta : 0ull) + (uint64_t)(int64_t)gv * (gx ? kFp4Rec : kFp8Rec);
            gdat = valid ? a : g_zb;
            gdat2 = gx ? g_zb : gdat;
          }
          // gather copies at steps 4, 9, 14, 19 (chunk pairs 2(w + 4c) + hh) and 24 (scale chunks of
          // tokens 8w .. 8w+7: the record's byte 512 is 512 - 32 w past gdat; fp4: both halves of
          // the 32 scale bytes at byte 256, into chunks 16 and 17)
          if (i >= 4 && i < 24 && (i - 4) % 5 == 0) {
            const int c = (i - 4) / 5;
            // an fp4 sub-tile's copy 2 lands on copy 3's chunks (unused by it), clear of chunks 16, 17
            const int cd = (gx && c == 2) ? 3 : c;
            const uint32_t dst = __builtin_amdgcn_readfirstlane(graw + 1024 * (wave + 4 * cd));
            const void* gp = (const void*)(uintptr_t)gdat;
            const void* gp2 = (const void*)(uintptr_t)gdat2;
            if (c == 0) g2l16_off<0>(gp, dst);
            else if (c == 1) g2l16_off<128>(gp, dst);
            else if (c == 2) g2l16_off<256>(gp2, dst);
            else g2l16_off<384>(gp2, dst);
          } else if (i == 24) {
            const int sofs = (gx ? 256 : 512) - 32 * wave;
            g2l16_masked((const void*)(uintptr_t)(gdat + (uint64_t)(int64_t)sofs),
                         __builtin_amdgcn_readfirstlane(graw + (gx ? 16 : 32) * 512),
                         gx ? scale_lanes_x : scale_lanes);
          }
          if (i == 26) {
            // index load of sub-tile s+6 into this wave's quarter of index slot r0, from a buffer
            // that ends at the index row's end (empty past the live segment)
            const SubTile is = locate<EXTRA>(p, t0, s + 6);
            const int n_in = (s + 6 < nsub && is.count > is.pos0) ? is.count - is.pos0 : 0;
            const uint64_t base = (EXTRA && is.x ? xidx_row : idx_row) + (uint64_t)(4 * (int64_t)is.pos0);
            const u32x4 rsrc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, (uint32_t)(4 * n_in),
                                0x00020000u};
            buf2l4(rsrc, idx_l, lds_a(smem) + kOffIdx + r0 * kIdxBytes + 32 * wave, 0xFFull);
          }
          if (i == 10) rr0 = *(lds_u32x4_r*)(uintptr_t)(draw + 1024);
          if (i == 14) rr1 = *(lds_u32x4_r*)(uintptr_t)(draw + 1536);
          // dequantization of s+2, steps 8 .. 23 (chunks 2 and 3 of fp8 were read at steps 10, 14)
          if (i >= 8 && i < 24) dequant_step(fp4, i - 8);
          __builtin_amdgcn_sched_barrier(0);
        }
        };
        if (EXTRA && dx) phase_a(std::true_type{});
        else phase_a(std::false_type{});

        // phase B: PV of sub-tile s. Step i accumulates block 2 b + hb (dim block 4w + b, head
        // block hb) over token half ks = i / 8 with V^T operand i / 2 and P^T operand (hb, ks).
        // The softmax of s+1 runs between the steps; its P^T operands are written to the exchange
        // buffer after the barrier at step 11, by which every wave has read those of sub-tile s.
        const uint32_t kb_next[2] = {slot_base(k_addr[0], r2), slot_base(k_addr[1], r2)};
        float e[8];
        float sv[8];
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // V^T operand n is read five steps before its first use (step 2n), P^T of the second
          // token half at steps 3 and 4
          if (!kFirst) {
            if (i == 1) vv[3] = read_v(3);
            if (i == 3) vv[0] = read_v(4);
            if (i == 5) vv[1] = read_v(5);
            if (i == 7) vv[2] = read_v(6);
            if (i == 9) vv[3] = read_v(7);
            if (i == 3) p1[0] = lds_b128(p_rd + 1024);
            if (i == 4) p1[1] = lds_b128(p_rd + 3072);
            if (i == 0) asm volatile("" ::"v"(p0[0]), "v"(p0[1]), "v"(vv[0]));
            if (i == 8) asm volatile("" ::"v"(p1[0]), "v"(p1[1]), "v"(vv[0]));
            mfma_pv32(oacc[i & 7], vv[(i >> 1) & 3], (i < 8 ? p0 : p1)[i & 1]);
          }
          if (i == 0) {
            // scores: 20 wait states after the last QK^T MFMA before VALU reads them; ignored
            // tokens of a partially valid sub-tile take the ignored score
            asm volatile("s_nop 15\n\ts_nop 3" : "+v"(sacc[0]), "+v"(sacc[1]));
#pragma unroll
            for (int r = 0; r < 8; ++r) sv[r] = sacc[r >> 2][r & 3];
            if (mk1 != 0xFFFFFFFFu) {
              const uint32_t mq = mk1 >> (4 * (lane64() >> 4));
#pragma unroll
              for (int r = 0; r < 8; ++r)
                sv[r] = ((mq >> (16 * (r >> 2) + (r & 3))) & 1u) ? sv[r] : kIgnoredScore;
            }
          }
          if (i == 1) {
            asm("v_max3_f32 %0, %0, %1, %2" : "+v"(m_lane) : "v"(sv[0]), "v"(sv[1]));
            asm("v_max3_f32 %0, %0, %1, %2" : "+v"(m_lane) : "v"(sv[2]), "v"(sv[3]));
          }
          if (i == 2) {
            asm("v_max3_f32 %0, %0, %1, %2" : "+v"(m_lane) : "v"(sv[4]), "v"(sv[5]));
            asm("v_max3_f32 %0, %0, %1, %2" : "+v"(m_lane) : "v"(sv[6]), "v"(sv[7]));
            // the reference is taken on the first live sub-tile (before it, every score was the
            // ignored score, so the four lanes' maximum is this sub-tile's own)
            if (!ref_set && mk1 != 0) {
              m_ref = max_xor32(max_xor16(m_lane)) * p.scale_log2;
              ref_off = -m_ref;
              ref_set = true;
            }
          }
          if (i >= 3 && i < 11) {
            const int r = i - 3;
            e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], p.scale_log2, ref_off));
            l_lane += e[r];
          }
          if (i == 11) {
            // this wave's P^T values: tokens 16 tb + 4(l/16) + 0..3 of head 16w + l%16, as bf16
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              bf16x2 v2;
              v2[0] = (__bf16)e[2 * k];
              v2[1] = (__bf16)e[2 * k + 1];
              pw[k] = __builtin_bit_cast(uint32_t, v2);
            }
          }
          if (i == 11) {
            // Start of iteration s+1: every V and P^T read of this iteration is complete,
            // idx(s+5) and the gather of s+3 have landed and the dequantization of s+2 is written.
            wait_barrier(1 + kGatherFp8);
          }
          if (i == 13) {
            // P^T of sub-tile s+1 for head block w / 2: token half tb goes to lane
            // 16(w%2) + l%16 + 32((l/16)/2), 8-byte half (l/16)%2
            const int lane = lane64();
            const uint32_t pa = lds_a(smem + kOffP) + 2048 * (wave >> 1) +
                                16 * (16 * (wave & 1) + (lane & 15) + 32 * ((lane >> 4) >> 1)) +
                                8 * ((lane >> 4) & 1);
            asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %0, %2 offset:1024"
                         :: "v"(pa), "v"(u32x2{pw[0], pw[1]}), "v"(u32x2{pw[2], pw[3]}) : "memory");
          }
          if (i >= 11) {
            // the first kAhead K operands of QK^T(s+2), two per step
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int st = 2 * (i - 11) + h;
              kb[st] = lds_b128(kb_next[st & 1] + 64 * (st >> 1));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // ---- pipeline start: sub-tiles 0 .. 2 gathered, idx(3), idx(4) loaded
      if (pass > 0) {
        load_indices(0, 0);
        load_indices(1, 1);
        load_indices(2, 2);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int j = 0; j < 3; ++j) mk_first[j] = gather_first(j, nsub);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        load_indices(3, 0);
        load_indices(4, 1);
      }
      int r0 = 2, r1 = 0, r2 = 1;
      wait_barrier(0);
      {
        // dequantize sub-tile 0 into tile slot 0
        const int lane = lane64();
        const int t = lane & 31, hh = lane >> 5;
        char* trow = tiles + t * kTileStride;
        const int sw = xor64(t);
        if (EXTRA && locate<EXTRA>(p, t0, 0).x) {
          // fp4: raw chunks c0, c0 + 1 (32 e2m1 values each) with e4m3 scale bytes j0 .. j0 + 3
          const int c0 = 4 * wave + 2 * hh, j0 = 8 * wave + 4 * hh;
          const uint32_t s4 = *reinterpret_cast<const uint32_t*>(
              raws + ((16 + (j0 >> 4)) * kSubTokens + t) * 16 + (j0 & 15));
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(raws + ((c0 + cc) * kSubTokens + t) * 16);
            bf16x8 a[4];
            dequant_fp4_16(r[0], r[1], e4m3_to_f32(s4 >> (16 * cc)), a[0], a[1]);
            dequant_fp4_16(r[2], r[3], e4m3_to_f32(s4 >> (16 * cc + 8)), a[2], a[3]);
#pragma unroll
            for (int m = 0; m < 4; ++m)
              *reinterpret_cast<u32x4*>(trow + 16 * (4 * (c0 + cc) + (m ^ sw))) =
                  __builtin_bit_cast(u32x4, a[m]);
          }
        } else {
          const int c0 = 8 * wave + 4 * hh;
          const uint32_t s2 = *reinterpret_cast<const uint16_t*>(raws + (32 * kSubTokens + t) * 16 + c0 / 2);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(raws + ((c0 + cc) * kSubTokens + t) * 16);
            const uint32_t sb = (s2 >> (8 * (cc >> 1))) & 0xFFu;
            *reinterpret_cast<u32x4*>(trow + 16 * ((2 * (c0 + cc)) ^ sw)) =
                __builtin_bit_cast(u32x4, dequant_fp8_8(r[0], r[1], sb));
            *reinterpret_cast<u32x4*>(trow + 16 * ((2 * (c0 + cc) + 1) ^ sw)) =
                __builtin_bit_cast(u32x4, dequant_fp8_8(r[2], r[3], sb));
          }
        }
      }
      wait_barrier(0);
      mk0 = 0u;
      mk1 = mk_first[0];
      mk2 = mk_first[1];
      mk3 = mk_first[2];
      mk4 = 0u;
#pragma unroll
      for (int st = 0; st < kAhead; ++st) kb[st] = lds_b128(k_addr[st & 1] + 64 * (st >> 1));

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
      // after iteration -1, three iterations with constant slots repeat, so every slot offset is
      // a constant
      iteration(std::true_type{}, -1, 2, 0, 1);
      rotate();
#pragma clang loop unroll(disable)
      for (int s = 0; s < nsub; s += 3) {
        iteration(std::false_type{}, s, 0, 1, 2);
        rotate();
        if (s + 1 >= nsub) break;
        iteration(std::false_type{}, s + 1, 1, 2, 0);
        rotate();
        if (s + 2 >= nsub) break;
        iteration(std::false_type{}, s + 2, 2, 0, 1);
        rotate();
      }
      // O is read by VALU instructions below (20 wait states after the last PV MFMA); the last
      // iterations' copies are awaited before the LDS is reused
      asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 15\n\ts_nop 3" : "+a"(oacc[7]) :: "memory");
      m_max = ref_set ? max_xor32(max_xor16(m_lane)) * p.scale_log2 : -__builtin_inff();
      l_sum = sum_xor32(sum_xor16(l_lane));

      if (pass > 0) {
        wait_barrier(0);
        break;
      }
      const bool any_big = __ballot(m_max > m_ref + kRefSlack) != 0;
      if (lane64() == 0) redo_flags[wave] = any_big ? 1 : 0;
      wait_barrier(0);
      const bool redo = (redo_flags[0] | redo_flags[1] | redo_flags[2] | redo_flags[3]) != 0;
      if (!redo) break;
      m_ref_next = m_max;
    }

    // ---- epilogue. O^T block j = 2 b + hb: lane l holds head 32 hb + l%32 and dims 32(4w + b) +
    // 8(r/4) + 4(l/32) + r%4 in register r. Head h's probability sum comes from wave h / 16.
    {
      const int lane = lane64();
      const int g = lane >> 5;
      const int h = lane & 31;
      const bool final_out = nsplit == 1;
      float* const lsums = reinterpret_cast<float*>(smem + kOffP);
      if (lane < 16) lsums[16 * wave + lane] = l_sum;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      float inv_b[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float l = lsums[32 * hb + h];
        inv_b[hb] = l > 0.0f ? 1.0f / l : 0.0f;
      }
      // head rows (the final output, or this split's normalised bf16 partial) staged in bf16 (row
      // hd at hd * kStageRow, 8-byte unit u at + 8u), then each wave stores the 1 KB rows of its
      // own 16 heads
      {
        const uint32_t wbase = lds_a(smem + h * kStageRow + 8 * g) + 256 * wave;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int hb = j & 1, b = j >> 1;
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (__bf16)(oacc[j][4 * jb + i] * inv_b[hb]);
            *reinterpret_cast<lds_bf16x4_rw*>(wbase + 32 * hb * kStageRow + 64 * b + 16 * jb) = o;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const uint32_t rbase = lds_a(smem + 16 * wave * kStageRow) + 16 * lane;
        char* const orow =
            final_out ? reinterpret_cast<char*>(p.out) + ((int64_t)row * p.h_q + head_base) * (2 * kHeadDim)
                      : static_cast<char*>(p.part_o) + ((int64_t)slot * p.h_q + head_base) * (2 * kHeadDim);
        for (int r = 0; r < 16 && head_base + r < p.h_q; ++r) {
          const bf16x4 lo = *reinterpret_cast<const lds_bf16x4_rw*>(rbase + r * kStageRow);
          const bf16x4 hi = *reinterpret_cast<const lds_bf16x4_rw*>(rbase + r * kStageRow + 8);
          *reinterpret_cast<bf16x8*>(orow + r * (2 * kHeadDim) + 16 * lane) =
              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      const int head = head_base + (lane & 15);
      if (lane < 16 && head < p.h_q) {
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

int launch_sparse_decode_h64(const DecodeParams& p, int parts, int groups, hipStream_t stream) {
  if (p.extra_topk > 0)
    hipLaunchKernelGGL(sparse_decode_h64_kernel<true>, dim3(parts, groups), dim3(64 * kWaves), 0, stream, p);
  else
    hipLaunchKernelGGL(sparse_decode_h64_kernel<false>, dim3(parts, groups), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mla
