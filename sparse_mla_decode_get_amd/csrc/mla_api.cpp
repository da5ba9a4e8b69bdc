// C-ABI entry points of libmla (declared in include/mla.h): argument checks, the host side of the
// schedule (part count, whether any row is split) and kernel launches. No allocation, no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla.h"
#include "mla_internal.h"

namespace {

constexpr int kMaxRows = 1 << 24;

int tiles_per_row(int topk, int extra_topk, int* tiles_k) {
  const int tk = (topk + MLA_TILE_TOKENS - 1) / MLA_TILE_TOKENS;
  const int tx = (extra_topk + MLA_TILE_TOKENS - 1) / MLA_TILE_TOKENS;
  if (tiles_k) *tiles_k = tk;
  return tk + tx > 0 ? tk + tx : 1;
}

// Kernel choice: head counts above 64 run in 128-head groups (mla_decode_wide.hip: four waves of
// 32 heads, one workgroup per CU); up to 64 heads run in one 64-head group of four waves of 16
// heads, with heads past h_q masked, in one of two kernels:
//  - mla_decode_h64.hip: one software-pipelined sub-tile stream, one wave per SIMD; about 1.1 us
//    per 32-token fp8 sub-tile, but a longer start than the other;
//  - mla_decode.hip: two halves of four waves with a one-deep pipeline; about 1.6 us per sub-tile.
// The first is taken when the parts average at least kStreamMinSubtiles sub-tiles (measured on
// MI355X over 32 rows of 64 heads: 3 us ahead at 8 sub-tiles per part, level at 4, behind at 2),
// or kStreamMinSubtilesExtra with an fp4 cache of a fifth of the tokens (32 and 64 such rows: 3 us
// behind at 6 sub-tiles per part, level or 3 us ahead at 8, 9% ahead at 80).
bool wide_for(int h_q) { return h_q > 64; }
constexpr int kStreamMinSubtiles = 6;
constexpr int kStreamMinSubtilesExtra = 8;
bool h64_stream_for(int rows, int tiles, int parts, int extra_topk) {
  const int64_t need = extra_topk > 0 ? kStreamMinSubtilesExtra : kStreamMinSubtiles;
  return 2 * (int64_t)rows * tiles >= need * parts;
}
int group_heads(int h_q) { return wide_for(h_q) ? 128 : 64; }
int head_groups(int h_q) { return (h_q + group_heads(h_q) - 1) / group_heads(h_q); }

constexpr int kAutoMinUnits = 4;

int default_parts(int h_q) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  // one workgroup per CU: a 128-head group uses about 150 KB of LDS and all registers of its CU,
  // a 64-head group's two halves of four waves about 150 KB of LDS and two waves per SIMD
  const int per_cu = 1;
  const int parts = cus * per_cu / head_groups(h_q);
  return parts > 0 ? parts : 1;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Largest number of (row, unit) pairs: with at most kMaxParts parts, the partition's products
// p * U and (u + 1) * P (host and metadata kernel) stay below 2^60.
constexpr int64_t kMaxUnits = int64_t(1) << 40;
constexpr int kMaxParts = 1 << 20;

int check_shape(int batch, int seq_len_q, int h_q, int topk, int extra_topk) {
  if (batch < 0 || seq_len_q < 0 || h_q <= 0 || topk < 0 || extra_topk < 0) return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * seq_len_q > kMaxRows) return MLA_ERR_UNSUPPORTED;
  if (h_q > 4096) return MLA_ERR_UNSUPPORTED;
  if (topk > (1 << 28) || extra_topk > (1 << 28)) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)batch * seq_len_q * tiles_per_row(topk, extra_topk, nullptr) > kMaxUnits)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int resolve_parts(int batch, int seq_len_q, int h_q, int topk, int extra_topk, int num_parts,
                  int min_tiles_per_part, int* out) {
  int rc = check_shape(batch, seq_len_q, h_q, topk, extra_topk);
  if (rc != MLA_OK) return rc;
  if (num_parts < 0 || min_tiles_per_part < 1 || !out) return MLA_ERR_INVALID_ARG;
  if (num_parts == 0) {
    // the default also keeps at least kAutoMinUnits units per part: a part's fixed traffic (its
    // rows' Q, and a 512-float partial per head when it splits a row) is worth several units of
    // 64 records
    num_parts = default_parts(h_q);
    if (min_tiles_per_part < kAutoMinUnits) min_tiles_per_part = kAutoMinUnits;
  }
  const int64_t units = (int64_t)batch * seq_len_q * tiles_per_row(topk, extra_topk, nullptr);
  int64_t p = units / min_tiles_per_part;
  if (p > num_parts) p = num_parts;
  if (p < 1) p = 1;
  if (p > kMaxParts) return MLA_ERR_UNSUPPORTED;
  *out = (int)p;
  return MLA_OK;
}

// True when some part boundary falls strictly inside a row (then that row has several splits).
bool any_split(int64_t rows, int tiles, int parts) {
  const int64_t units = rows * tiles;
  for (int64_t p = 1; p < parts; ++p)
    if (((p * units) / parts) % tiles != 0) return true;
  return false;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Bytes per partial output value: the 64-head kernel writes bf16 partials (the merge takes them back
// to fp32), the 128-head kernel fp32 ones (its registers leave no room for the conversion).
// partials are bf16, except the fused 128-head decode's (fp32); the workspace is sized for the
// larger, so that one workspace serves both entry points
size_t partial_elem_bytes(int h_q) { return wide_for(h_q) ? sizeof(float) : sizeof(uint16_t); }

size_t split_workspace_bytes(int batch, int seq_len_q, int h_q, int num_parts_used) {
  const size_t slots = (size_t)batch * seq_len_q + (size_t)num_parts_used - 1;
  // partial outputs, then fp32 partial lse
  return align256(slots * h_q * MLA_HEAD_DIM * partial_elem_bytes(h_q)) +
         align256(slots * h_q * sizeof(float));
}


}  // namespace

namespace mla {

int sparse_decode(const DecodeCall& c, const WorkspaceSource& ws) {
  const int batch = c.batch, seq_len_q = c.seq_len_q, h_q = c.h_q, topk = c.topk;
  const int extra_topk = c.extra_topk, num_parts_used = c.num_parts_used;
  int rc = check_shape(batch, seq_len_q, h_q, topk, extra_topk);
  if (rc != MLA_OK) return rc;
  const int rows = batch * seq_len_q;
  if (rows == 0) return MLA_OK;
  if (!c.q || !c.out || !c.lse) return MLA_ERR_INVALID_ARG;
  if (c.fused) {
    // the fused query transform and fp8 output live in the 128-head kernel only
    if (!wide_for(h_q)) return MLA_ERR_UNSUPPORTED;
    if (!c.qn_weight || !c.rope_cos || !c.rope_sin || !aligned(c.qn_weight, 16) ||
        !aligned(c.rope_cos, 16) || !aligned(c.rope_sin, 16) || !aligned(c.out, 16) ||
        !std::isfinite(c.qn_eps) || c.qn_eps < 0.0f || c.prefill)
      return MLA_ERR_INVALID_ARG;
  }
  if (!c.prefill && (!c.sched || !c.split_ptr || num_parts_used < 1)) return MLA_ERR_INVALID_ARG;
  if (topk > 0 && (!c.k_cache || !c.indices || c.k_tokens <= 0)) return MLA_ERR_INVALID_ARG;
  if (extra_topk > 0 && (!c.extra_k_cache || !c.extra_indices || c.extra_tokens <= 0))
    return MLA_ERR_INVALID_ARG;
  if (!aligned(c.q, 16) || !aligned(c.out, 8) || !aligned(c.lse, 4) || !aligned(c.k_cache, 16) ||
      !aligned(c.extra_k_cache, 16) || !aligned(c.indices, 4) || !aligned(c.extra_indices, 4))
    return MLA_ERR_INVALID_ARG;
  // The scale must be positive and finite: the 128-head kernel takes the largest scaled score as
  // the scaled largest raw score, and ignored entries carry a large negative raw score.
  if (!std::isfinite(c.softmax_scale) || !(c.softmax_scale > 0.0f)) return MLA_ERR_INVALID_ARG;
  if (num_parts_used > kMaxParts) return MLA_ERR_INVALID_ARG;
  int tiles_k = 0;
  const int tiles = tiles_per_row(topk, extra_topk, &tiles_k);
  // prefill: whole rows per part, as many parts as the device runs at once (none split)
  const int parts = c.prefill ? (rows < default_parts(h_q) ? rows : default_parts(h_q)) : num_parts_used;
  const bool split = !c.prefill && any_split(rows, tiles, num_parts_used);
  void* part_o = nullptr;
  float* part_lse = nullptr;
  if (split) {
    const size_t need = split_workspace_bytes(batch, seq_len_q, h_q, num_parts_used);
    void* base = ws.caller_ptr;
    if (ws.fixed_bytes > 0) {
      // the fixed device array: checked against its size before the device is touched
      if (need > ws.fixed_bytes) return MLA_ERR_SCRATCH_LIMIT;
      base = ws.fixed_ptr();
      if (!base) return MLA_ERR_HIP;
    } else if (!base || ws.caller_bytes < need || !aligned(base, 256)) {
      return MLA_ERR_WORKSPACE;
    }
    const size_t slots = (size_t)rows + (size_t)num_parts_used - 1;
    part_o = base;
    part_lse = reinterpret_cast<float*>(static_cast<char*>(base) +
                                        align256(slots * h_q * MLA_HEAD_DIM * partial_elem_bytes(h_q)));
  }
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(c.q);
  p.kc = c.k_cache;
  p.idx = c.indices;
  p.xc = extra_topk > 0 ? c.extra_k_cache : nullptr;
  p.xidx = extra_topk > 0 ? c.extra_indices : nullptr;
  p.topk = topk;
  p.extra_topk = extra_topk;
  p.tiles_k = tiles_k;
  p.tiles = tiles;
  p.rows = rows;
  p.h_q = h_q;
  p.scale_log2 = c.softmax_scale * 1.4426950408889634f;
  // prefill: the query itself stands in as the kernels' always-valid dummy load address
  p.sched = c.prefill ? static_cast<const int32_t*>(c.q) : c.sched;
  p.split_ptr = c.prefill ? nullptr : c.split_ptr;
  p.prefill_parts = c.prefill ? parts : 0;
  p.prefill_q = c.prefill ? rows / parts : 0;
  p.prefill_r = c.prefill ? rows % parts : 0;
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.out = c.fused ? nullptr : static_cast<uint16_t*>(c.out);
  p.lse = c.lse;
  p.qn_weight = static_cast<const uint16_t*>(c.qn_weight);
  p.qn_eps = c.qn_eps;
  p.rope_cos = c.rope_cos;
  p.rope_sin = c.rope_sin;
  p.out_fp8 = c.fused ? static_cast<uint8_t*>(c.out) : nullptr;
  hipStream_t s = (hipStream_t)c.stream;
  const int launched =
      wide_for(h_q) ? launch_sparse_decode_wide(p, parts, head_groups(h_q), s)
      : h64_stream_for(rows, tiles, parts, extra_topk) ? launch_sparse_decode_h64(p, parts, head_groups(h_q), s)
                                                       : launch_sparse_decode(p, parts, head_groups(h_q), 4, s);
  if (launched != 0) return MLA_ERR_HIP;
  if (split && c.fused) {
    if (launch_combine_fused(static_cast<const float*>(part_o), part_lse, c.split_ptr, rows, h_q,
                             c.rope_cos, c.rope_sin, p.out_fp8, c.lse, s) != 0)
      return MLA_ERR_HIP;
  } else if (split) {
    // every decode kernel writes bf16 partials for the plain decode
    if (launch_combine_bf16(static_cast<const uint16_t*>(part_o), part_lse, c.split_ptr, rows, h_q,
                            p.out, c.lse, s) != 0)
      return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // namespace mla

extern "C" {

const char* mla_error_string(int code) {
  switch (code) {
    case MLA_OK: return "success";
    case MLA_ERR_INVALID_ARG: return "invalid argument (null pointer, shape, alignment or consistency)";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_INDEX_RANGE: return "index outside the cache";
    case MLA_ERR_HIP: return "HIP runtime or kernel launch failure";
    case MLA_ERR_SCRATCH_LIMIT:
      return "split partials need more than the fixed scratch array of mla_sparse_decode_noalloc "
             "(MLA_NOALLOC_SCRATCH_BYTES); use mla_sparse_decode with a workspace";
    default: return "unknown mla status";
  }
}

int mla_metadata_parts(int batch, int seq_len_q, int h_q, int topk, int extra_topk, int num_parts,
                       int min_tiles_per_part, int* num_parts_used) {
  return resolve_parts(batch, seq_len_q, h_q, topk, extra_topk, num_parts, min_tiles_per_part,
                       num_parts_used);
}

int mla_get_metadata(int batch, int seq_len_q, int h_q, int topk, int extra_topk, int num_parts,
                     int min_tiles_per_part, int32_t* sched, int sched_capacity, int32_t* split_ptr,
                     int* num_parts_used, void* stream) {
  int parts = 0;
  int rc = resolve_parts(batch, seq_len_q, h_q, topk, extra_topk, num_parts, min_tiles_per_part,
                         &parts);
  if (rc != MLA_OK) return rc;
  if (!sched || !split_ptr || sched_capacity < parts) return MLA_ERR_INVALID_ARG;
  const int rows = batch * seq_len_q;
  const int tiles = tiles_per_row(topk, extra_topk, nullptr);
  if (mla::launch_metadata(rows, tiles, parts, sched, split_ptr, (hipStream_t)stream) != 0)
    return MLA_ERR_HIP;
  *num_parts_used = parts;
  return MLA_OK;
}

size_t mla_workspace_bytes(int batch, int seq_len_q, int h_q, int topk, int extra_topk,
                           int num_parts_used) {
  if (check_shape(batch, seq_len_q, h_q, topk, extra_topk) != MLA_OK || num_parts_used < 1) return 0;
  const int64_t rows = (int64_t)batch * seq_len_q;
  if (rows == 0 || !any_split(rows, tiles_per_row(topk, extra_topk, nullptr), num_parts_used)) return 0;
  return split_workspace_bytes(batch, seq_len_q, h_q, num_parts_used);
}

int mla_sparse_decode(const void* q, const uint8_t* k_cache, int64_t k_tokens,
                      const int32_t* indices, int topk, const uint8_t* extra_k_cache,
                      int64_t extra_tokens, const int32_t* extra_indices, int extra_topk, int batch,
                      int seq_len_q, int h_q, float softmax_scale, const int32_t* sched,
                      const int32_t* split_ptr, int num_parts_used, void* workspace,
                      size_t workspace_bytes, void* out, float* lse, void* stream) {
  const mla::DecodeCall c{q, k_cache, k_tokens, indices, topk, extra_k_cache, extra_tokens,
                          extra_indices, extra_topk, batch, seq_len_q, h_q, softmax_scale, sched,
                          split_ptr, num_parts_used, out, lse, stream};
  mla::WorkspaceSource ws;
  ws.caller_ptr = workspace;
  ws.caller_bytes = workspace_bytes;
  return mla::sparse_decode(c, ws);
}

int mla_sparse_decode_fused(const void* q, const void* q_norm_weight, float q_norm_eps,
                            const float* rope_cos, const float* rope_sin, const uint8_t* k_cache,
                            int64_t k_tokens, const int32_t* indices, int topk,
                            const uint8_t* extra_k_cache, int64_t extra_tokens,
                            const int32_t* extra_indices, int extra_topk, int batch, int seq_len_q,
                            int h_q, float softmax_scale, const int32_t* sched,
                            const int32_t* split_ptr, int num_parts_used, void* workspace,
                            size_t workspace_bytes, uint8_t* out_fp8, float* lse, void* stream) {
  mla::DecodeCall c{q, k_cache, k_tokens, indices, topk, extra_k_cache, extra_tokens, extra_indices,
                    extra_topk, batch, seq_len_q, h_q, softmax_scale, sched, split_ptr,
                    num_parts_used, out_fp8, lse, stream};
  c.fused = true;
  c.qn_weight = q_norm_weight;
  c.qn_eps = q_norm_eps;
  c.rope_cos = rope_cos;
  c.rope_sin = rope_sin;
  mla::WorkspaceSource ws;
  ws.caller_ptr = workspace;
  ws.caller_bytes = workspace_bytes;
  return mla::sparse_decode(c, ws);
}

int mla_sparse_prefill(const void* q, int s_q, int h_q, const uint8_t* k_cache, int64_t k_tokens,
                       const int32_t* indices, int topk, const uint8_t* extra_k_cache,
                       int64_t extra_tokens, const int32_t* extra_indices, int extra_topk,
                       float softmax_scale, void* out, float* lse, void* stream) {
  mla::DecodeCall c{q, k_cache, k_tokens, indices, topk, extra_k_cache, extra_tokens, extra_indices,
                    extra_topk, 1, s_q, h_q, softmax_scale, nullptr, nullptr, 1, out, lse, stream};
  c.prefill = true;
  return mla::sparse_decode(c, mla::WorkspaceSource{});
}

int mla_combine(const float* partial, const float* partial_lse, const int32_t* split_ptr, int rows,
                int h_q, void* out, float* lse, void* stream) {
  if (rows < 0 || h_q <= 0 || h_q > 65535) return MLA_ERR_INVALID_ARG;
  if (rows == 0) return MLA_OK;
  if (!partial || !partial_lse || !split_ptr || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned(partial, 16) || !aligned(out, 8)) return MLA_ERR_INVALID_ARG;
  if (rows > kMaxRows) return MLA_ERR_UNSUPPORTED;
  return mla::launch_combine(partial, partial_lse, split_ptr, rows, h_q,
                             static_cast<uint16_t*>(out), lse, false, (hipStream_t)stream) == 0
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_dequant_records(const uint8_t* cache, int record_bytes, const int32_t* idx, int n,
                        void* out_bf16, void* stream) {
  if (n < 0) return MLA_ERR_INVALID_ARG;
  if (record_bytes != MLA_FP8_RECORD_BYTES && record_bytes != MLA_FP4_RECORD_BYTES)
    return MLA_ERR_UNSUPPORTED;
  if (n == 0) return MLA_OK;
  if (!cache || !idx || !out_bf16 || !aligned(cache, 16) || !aligned(out_bf16, 16))
    return MLA_ERR_INVALID_ARG;
  return mla::launch_dequant(cache, record_bytes, idx, n, static_cast<uint16_t*>(out_bf16),
                             (hipStream_t)stream) == 0
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_validate_indices(const int32_t* idx, int64_t n, int64_t num_tokens, int32_t* bad_count,
                         void* stream) {
  if (n < 0 || num_tokens < 0 || !bad_count || (n > 0 && !idx)) return MLA_ERR_INVALID_ARG;
  return mla::launch_validate(idx, n, num_tokens, bad_count, (hipStream_t)stream) == 0 ? MLA_OK
                                                                                       : MLA_ERR_HIP;
}

int mla_quantize_records(const void* x, int64_t n, const int32_t* slots, int record_bytes,
                         uint8_t* cache, int64_t cache_tokens, void* stream) {
  if (n < 0 || cache_tokens < 0) return MLA_ERR_INVALID_ARG;
  if (record_bytes != MLA_FP8_RECORD_BYTES && record_bytes != MLA_FP4_RECORD_BYTES)
    return MLA_ERR_UNSUPPORTED;
  if (n == 0) return MLA_OK;
  if (!x || !cache || !aligned(x, 16) || !aligned(cache, 16) || !aligned(slots, 4))
    return MLA_ERR_INVALID_ARG;
  if (!slots && n > cache_tokens) return MLA_ERR_INVALID_ARG;
  if (n > (int64_t(1) << 33)) return MLA_ERR_UNSUPPORTED;     // grid of n / 4 workgroups
  return mla::launch_quantize(static_cast<const uint16_t*>(x), n, slots, record_bytes, cache,
                              cache_tokens, (hipStream_t)stream) == 0
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_check_indices(const int32_t* idx, int64_t n, int64_t num_tokens, int32_t* bad_count,
                      void* stream) {
  const int rc = mla_validate_indices(idx, n, num_tokens, bad_count, stream);
  if (rc != MLA_OK) return rc;
  int32_t bad = 0;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&bad, bad_count, sizeof(bad), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MLA_ERR_HIP;
  return bad == 0 ? MLA_OK : MLA_ERR_INDEX_RANGE;
}

}  // extern "C"
