// Paged KV-cache write: the new keys and values of a step are quantized to OCP E4M3 with their
// per-tensor descales and stored into the paged cache (vLLM PR #60372, Details, "Why FP8 is
// slower than BF16": the KV-cache write kernels reshape the new K/V and store them into the
// paged cache, with an FP8 conversion for an FP8 cache).  Token t goes to page
// slot_mapping[t] / page_size at position slot_mapping[t] % page_size; a slot outside
// [0, num_pages * page_size) writes nothing (padding tokens carry -1).
//
// HBM-bound: each thread reads 16 bf16 (32 B) and writes 16 codes (16 B) of one (token, K or V,
// kv head, 16-element chunk).  A block covers 256 chunks of one token, so the token's slot is a
// uniform scalar load and an unused slot ends the whole block.  The quantization is the one of
// fp8attn_quantize_q (quantize8_bf16_e4m3), so a cache entry and a quantized query with the
// same value and descale get the same code.
#include "device.h"
#include "params.h"

namespace fp8attn {

__global__ void __launch_bounds__(256) cache_write_kernel(const CacheWriteParams p) {
  const int64_t tok = blockIdx.x / p.blocks_per_token;
  const int32_t part = (int32_t)(blockIdx.x % p.blocks_per_token);
  const int64_t slot = ((const __attribute__((address_space(4))) int64_t*)p.slot_mapping)[tok];
  if (slot < 0 || slot >= p.num_slots) return;
  const int32_t chunks_per_head = p.head_dim / 16;
  const int32_t chunk_all = part * 256 + (int32_t)threadIdx.x;      // over K then V of the token
  if (chunk_all >= 2 * p.num_kv_heads * chunks_per_head) return;
  const int32_t which = chunk_all / (p.num_kv_heads * chunks_per_head);   // 0 = K, 1 = V
  const int32_t rest = chunk_all - which * p.num_kv_heads * chunks_per_head;
  const int32_t head = rest / chunks_per_head;
  const int32_t chunk = rest - head * chunks_per_head;

  const float* dsp = which ? p.v_descale : p.k_descale;
  const float ds = dsp ? load_uniform(dsp, 0) : 1.0f;
  const double rcp = 1.0 / (double)ds;   // correctly rounded fp64 reciprocal

  const __bf16* src = (which ? p.v_new : p.k_new) + tok * (which ? p.v_stride_tok : p.k_stride_tok) +
                      (int64_t)head * (which ? p.v_stride_head : p.k_stride_head) + 16 * chunk;
  const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(src);
  const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(src + 8);
  const u32x2_t c0 = quantize8_bf16_e4m3(w0, rcp);
  const u32x2_t c1 = quantize8_bf16_e4m3(w1, rcp);

  const int64_t page = slot / p.page_size;
  const int64_t pos = slot - page * p.page_size;
  uint8_t* dst = (which ? p.v_cache : p.k_cache) + page * p.kv_stride_page + pos * p.kv_stride_tok +
                 (int64_t)head * p.kv_stride_head + 16 * chunk;
  // (a non-temporal store: 2% faster on the sliding-window prefill's 65,536 tokens than a plain
  // one; non-temporal loads, or two chunks per thread, measured no better)
  __builtin_nontemporal_store(u32x4_t{c0[0], c0[1], c1[0], c1[1]}, reinterpret_cast<u32x4_t*>(dst));
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t grid = p.num_tokens * p.blocks_per_token;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8attn
