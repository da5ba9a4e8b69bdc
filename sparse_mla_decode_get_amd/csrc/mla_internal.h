// Host/device interface between the C-ABI entry points (mla_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeParams {
  const uint16_t* q;         // bf16 [rows][h_q][512]
  const uint8_t* kc;         // fp8 records
  const int32_t* idx;        // [rows][topk]
  const uint8_t* xc;         // fp4 records (may be null when extra_topk == 0)
  const int32_t* xidx;       // [rows][extra_topk]
  int topk, extra_topk;
  int tiles_k, tiles;        // fp8 units per row, all units per row
  int rows, h_q;
  float scale_log2;          // softmax_scale * log2(e)
  const int32_t* sched;      // [parts][8]; with prefill_parts > 0 only a valid dummy address
  const int32_t* split_ptr;  // [rows + 1]; null with prefill_parts > 0 (no row is split)
  int prefill_parts;         // > 0: no metadata; part b takes whole rows, prefill_q of them plus
  int prefill_q, prefill_r;  // one for b < prefill_r (rows = prefill_q * parts + prefill_r)
  void* part_o;              // workspace partial outputs [slots][h_q][512]: bf16, except fp32 from
                             // the fused 128-head decode
  float* part_lse;           // workspace partial lse [slots][h_q]
  uint16_t* out;             // bf16 [rows][h_q][512]
  float* lse;                // [rows][h_q]
  // fused decode (mla_sparse_decode_fused, 128-head kernel only): RMSNorm weight and epsilon of the
  // query rows, the rotary cos / sin of each row's 32 pairs (dims 448 + 2i, 449 + 2i), and the fp8
  // output records [rows][h_q][528] that replace `out`
  const uint16_t* qn_weight;  // bf16 [512]
  float qn_eps;
  const float* rope_cos;      // [rows][32]
  const float* rope_sin;      // [rows][32]
  uint8_t* out_fp8;
};

// Arguments of one decode call, as the C entry points receive them (include/mla.h).
struct DecodeCall {
  const void* q;
  const uint8_t* k_cache;
  int64_t k_tokens;
  const int32_t* indices;
  int topk;
  const uint8_t* extra_k_cache;
  int64_t extra_tokens;
  const int32_t* extra_indices;
  int extra_topk;
  int batch, seq_len_q, h_q;
  float softmax_scale;
  const int32_t* sched;
  const int32_t* split_ptr;
  int num_parts_used;
  void* out;
  float* lse;
  void* stream;
  bool prefill = false;      // mla_sparse_prefill: no metadata, whole rows per part, no split
  // mla_sparse_decode_fused: query transform and fp8 output (out is then uint8 [rows][h_q][528])
  bool fused = false;
  const void* qn_weight = nullptr;
  float qn_eps = 0.0f;
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
};

// Where the split partials go: the caller's workspace (mla_sparse_decode), or, when fixed_bytes > 0,
// the library's fixed device array of that size, whose address fixed_ptr() returns (nullptr on
// failure) and which is looked up only once a call is known to need it and to fit.
struct WorkspaceSource {
  void* caller_ptr = nullptr;
  size_t caller_bytes = 0;
  size_t fixed_bytes = 0;
  void* (*fixed_ptr)() = nullptr;
};

// Host checks, then the decode kernel and (for split rows) the merge on c.stream; an mla_status.
int sparse_decode(const DecodeCall& c, const WorkspaceSource& ws);

int launch_sparse_decode(const DecodeParams& p, int parts, int groups, int nw, hipStream_t stream);
// 128-head groups, four waves of 32 heads each (mla_decode_wide.hip).
int launch_sparse_decode_wide(const DecodeParams& p, int parts, int groups, hipStream_t stream);
// 64-head groups of fp8 records only (no extra cache), four waves of 16 heads each
// (mla_decode_h64.hip); its partials are bf16, like those of launch_sparse_decode.
int launch_sparse_decode_h64(const DecodeParams& p, int parts, int groups, hipStream_t stream);
int launch_metadata(int rows, int tiles, int parts, int32_t* sched, int32_t* split_ptr,
                    hipStream_t stream);
// Merge of fp32 partials (mla_combine, and the 128-head decode's workspace) or of the 64-head
// decode's bf16 partials; after a decode, rows with a single split (written directly by the decode
// kernel) are skipped.
int launch_combine(const float* partial, const float* partial_lse, const int32_t* split_ptr,
                   int rows, int h_q, uint16_t* out, float* lse, bool skip_single,
                   hipStream_t stream);
int launch_combine_bf16(const uint16_t* partial, const float* partial_lse, const int32_t* split_ptr,
                        int rows, int h_q, uint16_t* out, float* lse, hipStream_t stream);
// Merge of the 128-head kernel's fp32 partials for the fused decode: the merged rows get the
// conjugate rotation and are stored as fp8 records [rows][h_q][528]; single-split rows are skipped.
int launch_combine_fused(const float* partial, const float* partial_lse, const int32_t* split_ptr,
                         int rows, int h_q, const float* rope_cos, const float* rope_sin,
                         uint8_t* out_fp8, float* lse, hipStream_t stream);
int launch_dequant(const uint8_t* cache, int record_bytes, const int32_t* idx, int n,
                   uint16_t* out, hipStream_t stream);
int launch_validate(const int32_t* idx, int64_t n, int64_t num_tokens, int32_t* bad,
                    hipStream_t stream);
// Cache writer (mla_quant.hip): bf16 [n][512] -> records at token slots (row i when slots is null).
int launch_quantize(const uint16_t* x, int64_t n, const int32_t* slots, int record_bytes,
                    uint8_t* cache, int64_t cache_tokens, hipStream_t stream);

}  // namespace mla
