// Internal launch parameters shared by the host layer (api.cpp) and the HIP kernels.
// Not part of the public ABI (include/fp8attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp8attn {

// Everything one attention kernel launch needs, passed by value as the kernel argument.
struct AttnParams {
  const void* q;
  int64_t q_stride_tok, q_stride_head;        // elements
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  int64_t kv_stride_page, kv_stride_tok, kv_stride_head;  // bytes
  int32_t page_size;
  int32_t batch;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  int32_t total_q;
  int32_t hq, hkv, group;                      // group = hq / hkv
  const float* q_descale;                      // NULL -> 1
  const float* k_descale;
  const float* v_descale;
  int64_t ds_stride_b, ds_stride_h;
  float scale_log2;                            // softmax_scale * log2(e)
  int32_t window;                              // -1 or >= 1
  void* out;                                   // bf16
  int64_t out_stride_tok, out_stride_head;     // elements
  float* lse;                                  // optional, [total_q, hq]
  // split-KV decode
  int32_t num_splits;                          // S >= 1
  int32_t units_per_split;                     // 16-key units per split
  int32_t row_groups;                          // row tiles per (sequence, kv head)
  int32_t tile_rows;                           // rows per tile: 16, or 32 (split grid only)
  int32_t max_seqlen_q;
  float* part_o;                               // fp32 [S, total_q, hq, d] when S > 1
  float* part_lse;                             // fp32 [S, total_q, hq]
  // balanced partition (non-NULL selects it; the grid is the partition count R):
  // part_o [R + hkv * batch * row_groups, 16, d], part_lse [same, 16],
  // seg_meta [hkv * batch * row_groups][2] = first and last block of each row tile's range
  int32_t* seg_meta;
};

// How the kernels receive Q (values of fp8attn_dtype)
constexpr int kQBf16 = 0;       // bf16 values, BF16 MFMA with K/V dequantized
constexpr int kQE4M3 = 1;       // E4M3 codes, FP8 MFMA
constexpr int kQBf16E4M3 = 2;   // bf16 values quantized to E4M3 on load, FP8 MFMA
constexpr int kQBf16Split = 3;  // bf16 values split into two E4M3 terms on load, FP8 MFMA

// KV-cache write (fp8attn_cache_write)
struct CacheWriteParams {
  const __bf16* k_new;
  const __bf16* v_new;
  int64_t k_stride_tok, k_stride_head, v_stride_tok, v_stride_head;   // elements
  const int64_t* slot_mapping;
  uint8_t* k_cache;
  uint8_t* v_cache;
  int64_t kv_stride_page, kv_stride_tok, kv_stride_head;              // bytes
  int64_t num_tokens;
  int64_t num_slots;            // num_pages * page_size
  int32_t page_size;
  int32_t num_kv_heads, head_dim;
  int32_t blocks_per_token;     // ceil(2 * num_kv_heads * head_dim / 16 / 256)
  const float* k_descale;       // NULL -> 1
  const float* v_descale;
};
hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream);

hipError_t launch_quantize_q(const void* q, int64_t ntok, int32_t nheads, int32_t d,
                             int64_t stride_tok, int64_t stride_head, const float* q_descale,
                             void* out, hipStream_t stream);

// Split-KV paged attention over 16-row query tiles.  grid = row_groups * batch * S * hkv, or
// the partition count R when p.seg_meta is set (balanced partition).
hipError_t launch_decode(const AttnParams& p, int q_mode, int head_dim, int64_t grid,
                         hipStream_t stream);

// Native-FP8 prefill: 256 query rows per block, 64-key tiles through LDS.  head_dim 64, 96 (in a
// 128-byte LDS row layout), 128, 192 or 256.
// q_bf16: Q comes in bf16 and is quantized on load (q mode kQBf16E4M3), else E4M3 codes.
hipError_t launch_prefill_fp8(const AttnParams& p, int head_dim, bool q_bf16, hipStream_t stream);

// Prefill at head dim 512 with bf16 Q (q mode kQBf16 or, split_q, kQBf16Split): 128 query rows per
// block, 32-key tiles through LDS, both contractions on the MFMA.
hipError_t launch_prefill_wide(const AttnParams& p, bool split_q, hipStream_t stream);

// Decode with bf16 Q (q mode kQBf16, or kQBf16Split with split_q) at head dim 512 over 32-row query
// tiles (p.tile_rows == 32): the split grid's work items, one block each, K/V tiles through LDS
// shared by the 32 rows.  grid = row_groups * batch * S * hkv.
hipError_t launch_verify(const AttnParams& p, bool split_q, int64_t grid, hipStream_t stream);

hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t S, int64_t total_q,
                          int32_t hq, int32_t d, void* out, int64_t out_stride_tok,
                          int64_t out_stride_head, float* lse_out, hipStream_t stream);

// Combine of the balanced partition (decode with p.seg_meta set): merges the row tiles whose
// range spans several blocks; the others were written final by the decode kernel.
hipError_t launch_combine_parts(const float* part_o, const float* part_lse, const int32_t* seg_meta,
                                const int32_t* cu_seqlens_q, int32_t batch, int32_t row_groups, int32_t hkv,
                                int32_t group, int32_t parts, int32_t d, void* out, int64_t out_stride_tok,
                                int64_t out_stride_head, float* lse_out, hipStream_t stream);

}  // namespace fp8attn
