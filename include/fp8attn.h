/*
 * fp8attn: paged attention forward over an FP8 E4M3 KV cache for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers, sizes and strides; no framework types.  All tensor
 * pointers are DEVICE pointers unless stated; the argument structs themselves
 * live in host memory and are read during the call only.
 *
 * Sources (by page and section):
 *  [63139]  vLLM PR #63139 (FA4 native FP8 forward for all Gemma-4 layers on SM90), Overview:
 *           sliding-window layers (head dim 256) quantize Q to E4M3 and run attention on E4M3
 *           Q/K/V with FP8 matrix multiplies.
 *  [60372]  vLLM PR #60372 "[Kernel] Integrate FA4 SM90 FP8 MMA for Gemma-4 full attention",
 *           Overview / Claims / review thread: full-attention layers (head dim 512) keep BF16 Q
 *           over the FP8 KV cache; descale layouts are normalized; the split-KV count is chosen
 *           automatically with no fixed cap; pages are 64 tokens (framework blocks must be a
 *           multiple of 64); only causal and local (sliding-window) masks are supported; an
 *           unsupported combination raises an error naming the q/k/v dtypes and head sizes.
 *  [48666]  prhub digest of vLLM PR #48666, Implementation items 1-3 and Key code
 *           (flash_attn_varlen_func excerpt): paged float8_e4m3fn K/V are dequantized in the
 *           kernel with per-tensor K/V descales folded in, BF16 Q is consumed as is (no quantized
 *           Q input on that path), and the call returns the output and softmax_lse.
 *
 * What every attention call computes (fp32 accumulation; the CPU oracle does it in fp64):
 *   for sequence b with KV length L_b and q_len_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] new
 *   tokens, query token i sits at position p = L_b - q_len_b + i (the new tokens are the last
 *   positions).  Key j is visible iff j <= p and (window < 1 or j > p - window).
 *   q head hq reads kv head hq / (num_q_heads / num_kv_heads).
 *     s_j   = softmax_scale * <q_hat, k_hat_j>,   q_hat = q (bf16) or code(q) * q_descale (e4m3)
 *     k_hat = code(k) * k_descale,   v_hat = code(v) * v_descale
 *     out   = sum_j softmax(s)_j v_hat_j            (bf16)
 *     lse   = max_j s_j + ln(sum_j exp(s_j - max_j s_j))   (fp32, natural log; optional)
 *
 * Ownership and threading: the caller owns every buffer.  The library never allocates device
 * memory and never synchronizes; all work is enqueued on `stream`.  Calls are re-entrant; the
 * only global state is a per-device cache of the compute-unit count and a thread-local error
 * string.  Validation of host-visible arguments is complete before any HIP call; contents of
 * device arrays (block tables, lengths) are trusted and must be in range.
 */
#ifndef FP8ATTN_H
#define FP8ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8attn_status {
  FP8ATTN_OK = 0,
  FP8ATTN_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad stride, inconsistent shape */
  FP8ATTN_ERR_UNSUPPORTED = 2,   /* a valid request this library does not implement ([60372]) */
  FP8ATTN_ERR_WORKSPACE = 3,     /* decode workspace missing or too small */
  FP8ATTN_ERR_HIP = 4            /* a HIP runtime error (message from hipGetErrorString) */
} fp8attn_status;

typedef enum fp8attn_dtype {
  FP8ATTN_BF16 = 0,              /* bfloat16 */
  FP8ATTN_E4M3 = 1,              /* OCP float8 E4M3 (torch.float8_e4m3fn), stored as bytes */
  FP8ATTN_BF16_TO_E4M3 = 2,      /* bfloat16 Q quantized to E4M3 inside the call (q only) */
  FP8ATTN_BF16_SPLIT = 3         /* bfloat16 Q kept at full precision on the FP8 MFMA: each query
                                    row is scaled by a power of two 2^e (largest magnitude <= 448)
                                    and written as hi + lo/16 with hi, lo E4M3, which is exact for
                                    every value above about 2^-14 of the row's largest; QK^T is
                                    the two-part sum K.hi + K.lo/16, times 2^-e ([60372] review
                                    thread: the d512 FP8-MMA kernel keeps BF16 queries and builds
                                    a split QK accumulation).  PV runs on the FP8 MFMA too, with
                                    P as two E4M3 terms (8 significant bits, as bf16 P).  No
                                    q_descale.  (q only) */
} fp8attn_dtype;

/*
 * Arguments shared by fp8attn_prefill_varlen and fp8attn_decode_paged.
 * Strides are in ELEMENTS of the tensor's own dtype (bytes for E4M3 tensors).
 */
typedef struct fp8attn_attn_args {
  /* Queries [total_q, num_q_heads, head_dim], head_dim contiguous.
   * q_dtype FP8ATTN_E4M3: codes from fp8attn_quantize_q (native FP8 variant, [63139]).
   * q_dtype FP8ATTN_BF16_TO_E4M3: bf16 values that the call quantizes with q_descale exactly
   *   as fp8attn_quantize_q would (identical codes, so identical results), then the native
   *   FP8 variant; it saves the separate quantization pass.  Head dims as for E4M3.
   * q_dtype FP8ATTN_BF16: bf16 values (K/V dequantized in-kernel, [48666]).            */
  const void* q;
  int32_t q_dtype;
  int32_t reserved0;                /* must be 0 */
  int64_t q_stride_tok, q_stride_head;

  /* Paged cache: separate K and V pools of E4M3 bytes, indexed [page, slot, kv_head, d],
   * d contiguous.  Token j of sequence b lives in page block_table[b*block_table_stride +
   * j/page_size] at slot j%page_size.  page_size must be a positive multiple of 64 ([60372]). */
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  int64_t kv_stride_page, kv_stride_tok, kv_stride_head;   /* bytes; same for K and V */
  int32_t page_size;
  int32_t reserved1;                /* must be 0 */
  const int32_t* block_table;       /* [batch, >= ceil(max_seqlen_k/page_size)] */
  int64_t block_table_stride;
  const int32_t* cu_seqlens_q;      /* [batch+1], cu[0] = 0, non-decreasing */
  const int32_t* seqlens_k;         /* [batch], KV length including the new tokens, >= q_len */
  int32_t batch;                    /* number of sequences (host value) */
  int32_t total_q;                  /* cu_seqlens_q[batch] (host value) */
  int32_t max_seqlen_q;             /* host upper bound of q_len over the batch */
  int32_t max_seqlen_k;             /* host upper bound of seqlens_k over the batch */
  int32_t num_q_heads, num_kv_heads, head_dim;

  /* Descales: device fp32.  NULL means 1.0 (a unit scale needs no tensor).  K/V descales may
   * vary per (sequence, kv head): element [b*descale_stride_b + h*descale_stride_h]; strides
   * 0,0 give one per-tensor value ([60372] Claims: normalized descale layouts; [48666]).
   * q_descale is one per-tensor value (used by E4M3 and BF16_TO_E4M3); it must be NULL when
   * q_dtype is BF16, because that path takes unquantized Q ([48666] Implementation item 3).                                 */
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  int64_t descale_stride_b, descale_stride_h;

  float softmax_scale;              /* <= 0 selects 1/sqrt(head_dim) */
  int32_t causal;                   /* must be 1: causal and local masks only ([60372]) */
  int32_t window;                   /* -1: none.  W >= 1: keys p-W < j <= p.  0 (a window that
                                       shows no key) is FP8ATTN_ERR_UNSUPPORTED; < -1 INVALID_ARG */

  void* out;                        /* bf16 [total_q, num_q_heads, head_dim], d contiguous */
  int64_t out_stride_tok, out_stride_head;
  float* lse;                       /* optional fp32 [total_q, num_q_heads] contiguous, or NULL */
} fp8attn_attn_args;

/*
 * Quantize Q to E4M3 before the native FP8 forward ([63139] Overview; the pages do not spell
 * out the rounding, the reading taken is): code = E4M3_RNE_SAT(float32(q) / float32(*q_descale)),
 * i.e. one IEEE fp32 division, round to nearest even, +-448 saturation, NaN -> 0x7F|sign.
 *   q_bf16     : bf16 [num_tokens, num_heads, head_dim] with the given element strides
 *   q_descale  : device fp32 scalar, or NULL for 1.0
 *   q_e4m3_out : bytes [num_tokens, num_heads, head_dim], contiguous
 * head_dim must be a multiple of 8; strides must be multiples of 8 and the pointers 16-byte
 * aligned.  Empty inputs (num_tokens == 0) are a no-op.
 */
fp8attn_status fp8attn_quantize_q(const void* q_bf16, int64_t num_tokens, int32_t num_heads,
                                  int32_t head_dim, int64_t stride_tok, int64_t stride_head,
                                  const float* q_descale, void* q_e4m3_out, hipStream_t stream);

/*
 * Paged attention for varlen batches of new tokens (prefill / chunked prefill), any q_len.
 * Supported: (q_dtype E4M3 or BF16_TO_E4M3, head_dim 64, 96, 128, 192 or 256) and (q_dtype
 * BF16 or BF16_SPLIT, head_dim 64, 96, 128, 192, 256 or 512); K/V are E4M3 with V head dim equal
 * to head_dim ([60372] review thread; [63139] Overview lists 64/96/128/192/256 for the native FP8
 * forward).
 * Writes args->out and, if non-NULL, args->lse.
 */
fp8attn_status fp8attn_prefill_varlen(const fp8attn_attn_args* args, hipStream_t stream);

/*
 * Paged attention for few new tokens per sequence (decode, spec-decode verify), with split-KV
 * over the key range and a log-sum-exp combine ([60372] Claims: the split count is picked
 * automatically, with no fixed cap).  max_seqlen_q must be <= 16.
 *   num_splits      : 0 = automatic; N > 0 = N splits per (sequence, kv head, 16-row tile),
 *                     clamped to the key range; -R = the balanced partition into R parts
 *                     (R <= 2^20): the visible 16-key units of all tiles, laid end to end, are
 *                     cut into R equal ranges, one per thread block, so that every block streams
 *                     the same number of keys whatever the mix of sequence lengths
 *   workspace       : device scratch for partials; NULL with workspace_needed != NULL is a
 *                     size query that launches nothing.  256-byte aligned
 *   workspace_needed: out, bytes needed for the chosen plan (may be NULL)
 *   num_splits_used : out, the split count chosen, or -R for a balanced partition (may be NULL)
 * Automatic mode takes the balanced partition (R = blocks resident on the device at once) when
 * every sequence's rows fit one 16-row tile and max_seqlen_k (or the window) spans at least
 * 4096 keys; otherwise it takes just enough splits to fill the device once.  Planning reads host
 * values only (the call is capturable in a HIP graph); the partition reads the device lengths
 * inside the kernel.  With one split no workspace is needed and the output is written directly.
 */
fp8attn_status fp8attn_decode_paged(const fp8attn_attn_args* args, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes,
                                    size_t* workspace_needed, int32_t* num_splits_used,
                                    hipStream_t stream);

/*
 * fp8attn_decode_paged without a workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same validation,
 * plan, kernels and results as fp8attn_decode_paged with the same num_splits (bit for bit); the
 * split-KV partials live in a static device array of FP8ATTN_NOALLOC_SCRATCH_BYTES (32 MiB) that
 * every GPU the library runs on holds from the library's load until the process ends.  The call
 * allocates nothing.  Its first call on a device looks up that device's array address once.
 *   num_splits, num_splits_used: as for fp8attn_decode_paged
 * A plan that needs more partials than the array holds returns FP8ATTN_ERR_WORKSPACE before any
 * launch (fp8attn_decode_paged with a workspace takes any size).  Every call on one GPU shares
 * that GPU's array and it keeps the last call's contents: calls that overlap on one GPU (several
 * streams or threads) race on it, so the caller serializes them.  Nothing needs clearing between
 * calls: every partial a call reads, the same call wrote.
 */
#define FP8ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fp8attn_status fp8attn_decode_paged_noalloc(const fp8attn_attn_args* args, int32_t num_splits,
                                            int32_t* num_splits_used, hipStream_t stream);

/*
 * Log-sum-exp merge of split-KV partials ([60372] Details: the combine work of split-KV).
 * For each row n (a (token, q head) pair) and split s:
 *   M = max_s lse[s,n];  w_s = exp(lse[s,n] - M)  (a split with lse = -inf has weight 0 and its
 *   partial is not read);  out[n] = sum_s w_s o[s,n] / sum_s w_s;  lse_out[n] = M + ln sum_s w_s.
 *   partial_o   : fp32 [num_splits, total_q, num_q_heads, head_dim] contiguous
 *   partial_lse : fp32 [num_splits, total_q, num_q_heads] contiguous (natural log)
 *   out_bf16    : bf16 [total_q, num_q_heads, head_dim] with the given element strides
 *   lse_out     : optional fp32 [total_q, num_q_heads] contiguous
 * head_dim must be 64, 96, 128, 192, 256 or 512.  A row whose every split is -inf gets out = 0,
 * lse = -inf.
 */
fp8attn_status fp8attn_splitkv_combine(const float* partial_o, const float* partial_lse,
                                       int32_t num_splits, int64_t total_q, int32_t num_q_heads,
                                       int32_t head_dim, void* out_bf16, int64_t out_stride_tok,
                                       int64_t out_stride_head, float* lse_out, hipStream_t stream);

/*
 * Paged KV-cache write ([60372] Details, "Why FP8 is slower than BF16": the KV-cache write
 * kernels reshape the new keys and values and store them into the paged cache, converting them
 * for an FP8 cache).  For every token t whose slot s = slot_mapping[t] lies in
 * [0, num_pages * page_size):
 *   k_cache[s / page_size, s % page_size, h, :] = E4M3_RNE_SAT(float32(k_new[t, h, :]) / float32(*k_descale))
 *   v_cache[...same...]                         = E4M3_RNE_SAT(float32(v_new[t, h, :]) / float32(*v_descale))
 * with the rounding of fp8attn_quantize_q.  Other tokens (padding carries -1) write nothing, so a
 * slot out of range is never an out-of-bounds store.  Slots must be distinct: with a repeated
 * slot the entry ends up holding one of the tokens, which one is unspecified.
 *   k_new, v_new       : bf16 [num_tokens, num_kv_heads, head_dim], element strides per tensor
 *                        (head_dim contiguous), 16-byte aligned
 *   slot_mapping       : device int64 [num_tokens]
 *   k_cache, v_cache   : E4M3 bytes [num_pages, page_size, num_kv_heads, head_dim] with byte
 *                        strides kv_stride_page / kv_stride_tok / kv_stride_head (the layout of
 *                        fp8attn_attn_args), 16-byte aligned
 *   k_descale, v_descale: device fp32 scalars, or NULL for 1.0
 * head_dim must be a multiple of 16, page_size >= 1, and every stride a multiple of 16 bytes.
 * num_tokens == 0 is a no-op.  Nothing is allocated; the work is enqueued on the stream.
 */
fp8attn_status fp8attn_cache_write(const void* k_new, const void* v_new, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t k_stride_tok,
                                   int64_t k_stride_head, int64_t v_stride_tok, int64_t v_stride_head,
                                   const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                   int64_t num_pages, int32_t page_size, int64_t kv_stride_page,
                                   int64_t kv_stride_tok, int64_t kv_stride_head,
                                   const float* k_descale, const float* v_descale, hipStream_t stream);

/* Text of the last error on the calling thread ("" after a successful call).  Messages for
 * unsupported combinations name the q/k/v dtypes and head sizes ([60372] review thread). */
const char* fp8attn_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t fp8attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8ATTN_H */
