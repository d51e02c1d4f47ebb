// C-ABI entry points (include/fp8attn.h): argument validation, split-KV planning, dispatch.
//
// Validation runs entirely on host-visible values and finishes before the first HIP call, so
// every rejection path can be exercised without a GPU.  Rejections for unsupported
// combinations name the q/k/v dtypes and head sizes, following the gating convention in vLLM
// PR #60372 (review thread: unsupported calls raise an error naming dtypes and head sizes).
#include "../../include/fp8attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "params.h"

// ---- the allocation-free decode: split-KV partials in a static device array ------------------
// Every GPU the library runs on holds its own copy of `scratch` from the module's load until the
// process ends.  In host code the name `scratch` is a host-side stand-in, not a device address:
// each device's address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[FP8ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

fp8attn_status fail(fp8attn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

fp8attn_status ok() {
  g_err.clear();
  return FP8ATTN_OK;
}

fp8attn_status hip_fail(const char* where, hipError_t e) {
  return fail(FP8ATTN_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

const char* dtype_name(int32_t t) {
  return t == FP8ATTN_BF16 ? "bf16" : t == FP8ATTN_E4M3 ? "e4m3" : t == FP8ATTN_BF16_TO_E4M3 ? "bf16->e4m3"
         : t == FP8ATTN_BF16_SPLIT ? "bf16-split" : "unknown";
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Supported (q dtype, head dim) pairs: native FP8 at head dim 256 (vLLM PR #63139, Overview) and
// BF16 Q at head dim 512 (vLLM PR #60372, Overview), plus head dims 64, 96, 128 and 192 for both
// (vLLM PR #63139, Overview: the FA4 native FP8 forward also covers 64/96/128/192), and 256 for
// BF16 Q (same kernel).  96 is not a multiple of the 64-byte k-step: decode and FP8 prefill run
// it in a 128 layout whose last 32 bytes are zeros.
bool supported_combo(int32_t q_dtype, int32_t d) {
  const bool small = d == 64 || d == 96 || d == 128 || d == 192;
  if (q_dtype == FP8ATTN_E4M3 || q_dtype == FP8ATTN_BF16_TO_E4M3) return small || d == 256;
  if (q_dtype == FP8ATTN_BF16 || q_dtype == FP8ATTN_BF16_SPLIT) return small || d == 256 || d == 512;
  return false;
}

fp8attn_status validate_attn(const char* fn, const fp8attn_attn_args* a, bool decode) {
  if (!a) return fail(FP8ATTN_ERR_INVALID_ARG, "%s: args is NULL", fn);
  if (a->q_dtype != FP8ATTN_BF16 && a->q_dtype != FP8ATTN_E4M3 && a->q_dtype != FP8ATTN_BF16_TO_E4M3 &&
      a->q_dtype != FP8ATTN_BF16_SPLIT)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: unknown q_dtype %d", fn, a->q_dtype);
  if (a->reserved0 != 0 || a->reserved1 != 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: reserved fields must be 0", fn);
  if (a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->head_dim <= 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: head counts and head_dim must be positive (num_q_heads=%d num_kv_heads=%d head_dim=%d)",
                fn, a->num_q_heads, a->num_kv_heads, a->head_dim);
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: num_q_heads (%d) must be a multiple of num_kv_heads (%d)", fn,
                a->num_q_heads, a->num_kv_heads);
  if (!supported_combo(a->q_dtype, a->head_dim))
    return fail(FP8ATTN_ERR_UNSUPPORTED,
                "%s: unsupported combination q=%s k=e4m3 v=e4m3 head_size=%d head_size_v=%d "
                "(supported: q=e4m3 or bf16->e4m3 with head_size 64, 96, 128, 192 or 256; q=bf16 or bf16-split with "
                "head_size 64, 96, 128, 192, 256 or 512; "
                "k/v always e4m3 with head_size_v == head_size)",
                fn, dtype_name(a->q_dtype), a->head_dim, a->head_dim);
  if (a->causal != 1)
    return fail(FP8ATTN_ERR_UNSUPPORTED,
                "%s: non-causal attention is not supported (q=%s k=e4m3 v=e4m3 head_size=%d): only causal "
                "and sliding-window masks are implemented",
                fn, dtype_name(a->q_dtype), a->head_dim);
  if (a->window < -1)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: window must be -1 (none) or >= 1, got %d", fn, a->window);
  if (a->window == 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED,
                "%s: window 0 (no visible key) is not supported (q=%s k=e4m3 v=e4m3 head_size=%d): window must be "
                "-1 (none) or >= 1", fn, dtype_name(a->q_dtype), a->head_dim);
  if (a->page_size <= 0 || a->page_size % 64 != 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED,
                "%s: page_size %d is not a positive multiple of 64 (q=%s k=e4m3 v=e4m3 head_size=%d)", fn,
                a->page_size, dtype_name(a->q_dtype), a->head_dim);
  if ((a->q_dtype == FP8ATTN_BF16 || a->q_dtype == FP8ATTN_BF16_SPLIT) && a->q_descale != nullptr)
    return fail(FP8ATTN_ERR_UNSUPPORTED,
                "%s: q=%s takes unquantized queries, so q_descale must be NULL (k=e4m3 v=e4m3 head_size=%d)",
                fn, dtype_name(a->q_dtype), a->head_dim);
  if (a->batch < 0 || a->total_q < 0 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: batch, total_q, max_seqlen_q and max_seqlen_k must be >= 0", fn);
  if (a->total_q > 0 && a->max_seqlen_q == 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: total_q > 0 needs max_seqlen_q > 0", fn);
  if (a->max_seqlen_q > a->max_seqlen_k && a->total_q > 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: max_seqlen_q (%d) exceeds max_seqlen_k (%d): q_len must be <= KV length",
                fn, a->max_seqlen_q, a->max_seqlen_k);
  if (decode && a->max_seqlen_q > 16)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: max_seqlen_q %d > 16; use fp8attn_prefill_varlen", fn, a->max_seqlen_q);
  if (!(a->softmax_scale == a->softmax_scale) || std::isinf(a->softmax_scale))
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: softmax_scale must be finite", fn);
  if (a->descale_stride_b < 0 || a->descale_stride_h < 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: descale strides must be >= 0", fn);
  if (a->total_q == 0 || a->batch == 0) return ok();

  if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->cu_seqlens_q || !a->seqlens_k || !a->out)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: a required pointer (q, k_cache, v_cache, block_table, cu_seqlens_q, "
                "seqlens_k, out) is NULL", fn);
  const int64_t qelt = a->q_dtype == FP8ATTN_E4M3 ? 1 : 2;
  if (!aligned(a->q, 16) || (a->q_stride_tok * qelt) % 16 != 0 || (a->q_stride_head * qelt) % 16 != 0 ||
      a->q_stride_tok < 0 || a->q_stride_head < 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: q must be 16-byte aligned with 16-byte-multiple strides", fn);
  if (!aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) || a->kv_stride_tok % 16 != 0 ||
      a->kv_stride_page % 16 != 0 || a->kv_stride_head % 16 != 0 || a->kv_stride_tok < a->head_dim ||
      a->kv_stride_head < 0 || a->kv_stride_page < 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: k/v caches must be 16-byte aligned with 16-byte-multiple strides "
                "(kv_stride_tok >= head_dim)", fn);
  // the kernels address the keys of one 64-key tile with 32-bit byte offsets from its first key
  if (a->kv_stride_tok > (int64_t)(UINT32_MAX / 64))
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: kv_stride_tok %lld is too large: 64 token strides must stay below 2^32 "
                "bytes", fn, (long long)a->kv_stride_tok);
  if (!aligned(a->out, 16) || (a->out_stride_tok * 2) % 16 != 0 || (a->out_stride_head * 2) % 16 != 0 ||
      a->out_stride_tok < 0 || a->out_stride_head < 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: out must be 16-byte aligned with 16-byte-multiple strides", fn);
  if (a->lse && !aligned(a->lse, 4)) return fail(FP8ATTN_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
  const int64_t need_pages = (a->max_seqlen_k + a->page_size - 1) / a->page_size;
  if (a->block_table_stride < need_pages && a->batch > 1)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: block_table_stride %lld is smaller than ceil(max_seqlen_k/page_size) = %lld",
                fn, (long long)a->block_table_stride, (long long)need_pages);
  return ok();
}

fp8attn::AttnParams make_params(const fp8attn_attn_args* a) {
  fp8attn::AttnParams p{};
  p.q = a->q;
  p.q_stride_tok = a->q_stride_tok;
  p.q_stride_head = a->q_stride_head;
  p.k_cache = a->k_cache;
  p.v_cache = a->v_cache;
  p.kv_stride_page = a->kv_stride_page;
  p.kv_stride_tok = a->kv_stride_tok;
  p.kv_stride_head = a->kv_stride_head;
  p.page_size = a->page_size;
  p.batch = a->batch;
  p.block_table = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.cu_seqlens_q = a->cu_seqlens_q;
  p.seqlens_k = a->seqlens_k;
  p.total_q = a->total_q;
  p.hq = a->num_q_heads;
  p.hkv = a->num_kv_heads;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.q_descale = a->q_descale;
  p.k_descale = a->k_descale;
  p.v_descale = a->v_descale;
  p.ds_stride_b = a->descale_stride_b;
  p.ds_stride_h = a->descale_stride_h;
  const float sc = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)a->head_dim);
  p.scale_log2 = sc * 1.4426950408889634f;
  p.window = a->window;
  p.out = a->out;
  p.out_stride_tok = a->out_stride_tok;
  p.out_stride_head = a->out_stride_head;
  p.lse = a->lse;
  p.max_seqlen_q = a->max_seqlen_q;
  p.num_splits = 1;
  p.tile_rows = 16;
  return p;
}

struct DecodePlan {
  int32_t row_groups;
  int32_t tile_rows;         // 16, or 32 (split grid with more than 16 rows per sequence and kv head)
  int32_t max_units;
  int32_t splits;            // split count, or minus the partition count (balanced partition)
  int32_t units_per_split;
  bool balanced;
  size_t ws_bytes;
  int64_t grid;
};

// Automatic mode takes the balanced partition for long key ranges with one row tile per
// sequence: there a spread of lengths leaves most compute units idle behind the longest sequence
// (B64 d512, lengths U[8K, 32K]: 1.04 ms at one split against 0.87 ms for the same bytes at
// equal lengths), and more splits cost more than they balance (1.14 ms at 16).  Short ranges
// (a 1024-key window) are uniform by construction and keep the one-kernel plan; several row
// tiles per sequence (spec-decode verify) keep theirs, because the split grid runs a
// sequence's tiles side by side.
// The split grid takes 32-row tiles when a sequence has more than 16 rows per kv head and the head
// dim is at most 256: each K/V unit is then loaded once for 32 rows instead of once per 16.  At
// head dim 512 the two halves' O accumulators alone fill the 256 accumulation registers of a
// decode wave (that kernel spilled in its loop, 5x slower), so 32-row tiles at 512 run in the
// verify kernel, whose waves split the head dim of O.
constexpr int32_t kBalancedMinUnits = 256;   // 4096 keys
constexpr int32_t kMaxParts = 1 << 20;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Split-KV plan from host-known maxima only (no device reads, so the call is capturable).
// Automatic mode picks the split count with no fixed cap (vLLM PR #60372, Claims): just enough
// splits for the grid to fill the chip once (the blocks that fit at once: two per compute unit
// at head dim <= 256, one at 512, four at 64), with at least 32 units (512 keys) per split.
// Every block pays a Q load, a merge of its waves and, when split, a partial write, so fewer and
// longer blocks measured faster on every decode workload here (B64 d512 full decode: 1.15 ms at
// the former 16 splits, 1.04 ms at one; spec-verify 1.36 ms at 15, 1.11 ms at one).
DecodePlan plan_decode(const fp8attn_attn_args* a, int32_t requested) {
  DecodePlan pl{};
  const int G = a->num_q_heads / a->num_kv_heads;
  const int64_t rows = (int64_t)a->max_seqlen_q * G;
  pl.tile_rows = 16;
  pl.row_groups = (int32_t)((rows + 15) / 16);
  int64_t vis = a->max_seqlen_k;
  if (a->window >= 1) vis = std::min<int64_t>(vis, (int64_t)a->window + a->max_seqlen_q - 1);
  pl.max_units = (int32_t)((vis + 15) / 16 + 1);
  int64_t items = (int64_t)a->num_kv_heads * a->batch * pl.row_groups;
  const int64_t per_cu = a->head_dim > 256 ? 1 : a->head_dim > 64 ? 2 : 4;
  if (requested < 0 || (requested == 0 && pl.row_groups == 1 && pl.max_units >= kBalancedMinUnits)) {
    // balanced partition into R parts: one block per part, all resident at once in automatic mode
    const int64_t R = requested < 0 ? -(int64_t)requested : (int64_t)cu_count() * per_cu;
    const size_t slots = (size_t)R + (size_t)items;
    pl.balanced = true;
    pl.splits = (int32_t)-R;
    pl.units_per_split = 0;
    pl.ws_bytes = round_up(slots * 16 * a->head_dim * sizeof(float)) + round_up(slots * 16 * sizeof(float)) +
                  round_up((size_t)items * 2 * sizeof(int32_t));
    pl.grid = R;
    return pl;
  }
  if (rows > 16) {
    pl.tile_rows = 32;
    pl.row_groups = (int32_t)((rows + 31) / 32);
    items = (int64_t)a->num_kv_heads * a->batch * pl.row_groups;
  }
  int64_t S;
  if (requested > 0) {
    S = requested;
  } else {
    const int64_t resident = (int64_t)cu_count() * per_cu;
    S = (resident + items - 1) / items;
    S = std::min<int64_t>(S, std::max<int64_t>(1, pl.max_units / 32));
  }
  S = std::max<int64_t>(1, std::min<int64_t>(S, pl.max_units));
  pl.units_per_split = (int32_t)((pl.max_units + S - 1) / S);
  S = (pl.max_units + pl.units_per_split - 1) / pl.units_per_split;
  pl.splits = (int32_t)S;
  pl.ws_bytes = 0;
  if (S > 1) {
    const size_t rows = (size_t)a->total_q * a->num_q_heads;
    pl.ws_bytes = round_up(S * rows * a->head_dim * sizeof(float)) + round_up(S * rows * sizeof(float));
  }
  pl.grid = items * S;   // the caller rejects grids of 2^31 blocks or more
  return pl;
}

// Checks shared by both decode entry points once the plan is known (host values only).
fp8attn_status check_plan(const char* fn, const fp8attn_attn_args* args, const DecodePlan& pl) {
  if (pl.balanced &&
      (int64_t)args->num_kv_heads * args->batch * pl.row_groups + pl.grid >= (int64_t)1 << 31)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: %lld row tiles are too many for a balanced partition", fn,
                (long long)args->num_kv_heads * args->batch * pl.row_groups);
  if (pl.grid >= (int64_t)1 << 31)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: grid of %lld blocks is too large", fn, (long long)pl.grid);
  return FP8ATTN_OK;
}

// Launches of a decode plan: the partial kernel, then the combine when the plan leaves partials.
// workspace holds at least pl.ws_bytes (256-byte aligned) whenever pl.ws_bytes > 0.
fp8attn_status run_decode(const char* fn, const fp8attn_attn_args* args, const DecodePlan& pl, void* workspace,
                          hipStream_t stream) {
  fp8attn::AttnParams p = make_params(args);
  p.num_splits = pl.splits;
  p.units_per_split = pl.units_per_split;
  p.row_groups = pl.row_groups;
  p.tile_rows = pl.tile_rows;
  char* ws = reinterpret_cast<char*>(workspace);
  if (pl.balanced) {
    const size_t items = (size_t)args->num_kv_heads * args->batch * pl.row_groups;
    const size_t slots = (size_t)pl.grid + items;
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + round_up(slots * 16 * args->head_dim * sizeof(float)));
    p.seg_meta = reinterpret_cast<int32_t*>(ws + round_up(slots * 16 * args->head_dim * sizeof(float)) +
                                            round_up(slots * 16 * sizeof(float)));
  } else if (pl.splits > 1) {
    const size_t rows = (size_t)args->total_q * args->num_q_heads;
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + round_up((size_t)pl.splits * rows * args->head_dim * sizeof(float)));
  }
  hipError_t e = pl.tile_rows == 32 && args->head_dim == 512
                     ? fp8attn::launch_verify(p, args->q_dtype == FP8ATTN_BF16_SPLIT, pl.grid, stream)
                     : fp8attn::launch_decode(p, args->q_dtype, args->head_dim, pl.grid, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (pl.balanced) {
    e = fp8attn::launch_combine_parts(p.part_o, p.part_lse, p.seg_meta, args->cu_seqlens_q, args->batch,
                                      pl.row_groups, args->num_kv_heads, args->num_q_heads / args->num_kv_heads,
                                      (int32_t)pl.grid, args->head_dim, args->out, args->out_stride_tok, args->out_stride_head,
                                      args->lse, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  } else if (pl.splits > 1) {
    e = fp8attn::launch_combine(p.part_o, p.part_lse, pl.splits, args->total_q, args->num_q_heads, args->head_dim,
                                args->out, args->out_stride_tok, args->out_stride_head, args->lse, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return ok();
}

fp8attn_status scratch_address(const char* fn, void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= 64) return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: device index %d: at most 64 devices", fn, dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(fn, e);
    if (!a || !aligned(a, kAlign))
      return fail(FP8ATTN_ERR_HIP, "%s: the scratch array of device %d is not %zu-byte aligned", fn, dev, kAlign);
    addr[dev] = a;
  }
  *out = addr[dev];
  return FP8ATTN_OK;
}

fp8attn_status decode_checks(const char* fn, const fp8attn_attn_args* args, int32_t num_splits) {
  fp8attn_status st = validate_attn(fn, args, true);
  if (st != FP8ATTN_OK) return st;
  if (num_splits < -kMaxParts)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: num_splits %d: a balanced partition takes at most %d parts", fn,
                num_splits, kMaxParts);
  return FP8ATTN_OK;
}

}  // namespace

extern "C" {

int32_t fp8attn_version(void) { return 100; }

const char* fp8attn_last_error(void) { return g_err.c_str(); }

fp8attn_status fp8attn_quantize_q(const void* q_bf16, int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                                  int64_t stride_tok, int64_t stride_head, const float* q_descale,
                                  void* q_e4m3_out, hipStream_t stream) {
  const char* fn = "fp8attn_quantize_q";
  if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: num_tokens >= 0, num_heads > 0 and head_dim > 0 required", fn);
  if (head_dim % 8 != 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: head_dim %d is not a multiple of 8", fn, head_dim);
  if (stride_tok < 0 || stride_head < 0 || stride_tok % 8 != 0 || stride_head % 8 != 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: strides must be non-negative multiples of 8 elements", fn);
  if (num_tokens == 0) return ok();
  if (!q_bf16 || !q_e4m3_out) return fail(FP8ATTN_ERR_INVALID_ARG, "%s: q_bf16 and q_e4m3_out must be non-NULL", fn);
  if (!aligned(q_bf16, 16) || !aligned(q_e4m3_out, 8))
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: q_bf16 must be 16-byte and q_e4m3_out 8-byte aligned", fn);
  hipError_t e = fp8attn::launch_quantize_q(q_bf16, num_tokens, num_heads, head_dim, stride_tok, stride_head,
                                            q_descale, q_e4m3_out, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

fp8attn_status fp8attn_cache_write(const void* k_new, const void* v_new, int64_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int64_t k_stride_tok, int64_t k_stride_head, int64_t v_stride_tok,
                                   int64_t v_stride_head, const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                   int64_t num_pages, int32_t page_size, int64_t kv_stride_page, int64_t kv_stride_tok,
                                   int64_t kv_stride_head, const float* k_descale, const float* v_descale,
                                   hipStream_t stream) {
  const char* fn = "fp8attn_cache_write";
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_pages < 0 || page_size <= 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: num_tokens >= 0, num_pages >= 0, num_kv_heads > 0, head_dim > 0 and "
                "page_size > 0 required", fn);
  if (head_dim % 16 != 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: head_dim %d is not a multiple of 16 (k=e4m3 v=e4m3)", fn, head_dim);
  const int64_t bstr[4] = {k_stride_tok, k_stride_head, v_stride_tok, v_stride_head};
  for (int64_t x : bstr)
    if (x < 0 || (x * 2) % 16 != 0)
      return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: k_new/v_new strides must be non-negative multiples of 8 elements", fn);
  if (kv_stride_page < 0 || kv_stride_tok < 0 || kv_stride_head < 0 || kv_stride_page % 16 != 0 ||
      kv_stride_tok % 16 != 0 || kv_stride_head % 16 != 0)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: cache strides must be non-negative multiples of 16 bytes", fn);
  const int64_t chunks = 2 * (int64_t)num_kv_heads * (head_dim / 16);
  const int64_t bpt = (chunks + 255) / 256;
  if (num_tokens * bpt > INT32_MAX)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: %lld tokens exceed one launch", fn, (long long)num_tokens);
  if (num_pages > INT64_MAX / page_size)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: num_pages * page_size overflows", fn);
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: k_new, v_new, slot_mapping, k_cache and v_cache must be non-NULL", fn);
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: k_new, v_new and the caches must be 16-byte aligned, slot_mapping "
                "8-byte aligned", fn);
  fp8attn::CacheWriteParams p{};
  p.k_new = static_cast<const __bf16*>(k_new);
  p.v_new = static_cast<const __bf16*>(v_new);
  p.k_stride_tok = k_stride_tok;
  p.k_stride_head = k_stride_head;
  p.v_stride_tok = v_stride_tok;
  p.v_stride_head = v_stride_head;
  p.slot_mapping = slot_mapping;
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.kv_stride_page = kv_stride_page;
  p.kv_stride_tok = kv_stride_tok;
  p.kv_stride_head = kv_stride_head;
  p.num_tokens = num_tokens;
  p.num_slots = num_pages * page_size;
  p.page_size = page_size;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.blocks_per_token = (int32_t)bpt;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  hipError_t e = fp8attn::launch_cache_write(p, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

fp8attn_status fp8attn_decode_paged(const fp8attn_attn_args* args, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, size_t* workspace_needed, int32_t* num_splits_used,
                                    hipStream_t stream) {
  const char* fn = "fp8attn_decode_paged";
  fp8attn_status st = decode_checks(fn, args, num_splits);
  if (st != FP8ATTN_OK) return st;
  if (args->total_q == 0 || args->batch == 0) {
    if (workspace_needed) *workspace_needed = 0;
    if (num_splits_used) *num_splits_used = 1;
    return ok();
  }
  const DecodePlan pl = plan_decode(args, num_splits);
  if (workspace_needed) *workspace_needed = pl.ws_bytes;
  if (num_splits_used) *num_splits_used = pl.splits;
  if (!workspace && workspace_needed) return ok();  // size query
  st = check_plan(fn, args, pl);
  if (st != FP8ATTN_OK) return st;
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return fail(FP8ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %s %d, got %zu", fn,
                  pl.ws_bytes, pl.balanced ? "a balanced partition of parts" : "split count",
                  pl.balanced ? -pl.splits : pl.splits, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, kAlign))
      return fail(FP8ATTN_ERR_INVALID_ARG, "%s: workspace must be %zu-byte aligned", fn, kAlign);
  }
  return run_decode(fn, args, pl, workspace, stream);
}

fp8attn_status fp8attn_decode_paged_noalloc(const fp8attn_attn_args* args, int32_t num_splits,
                                            int32_t* num_splits_used, hipStream_t stream) {
  const char* fn = "fp8attn_decode_paged_noalloc";
  fp8attn_status st = decode_checks(fn, args, num_splits);
  if (st != FP8ATTN_OK) return st;
  if (args->total_q == 0 || args->batch == 0) {
    if (num_splits_used) *num_splits_used = 1;
    return ok();
  }
  const DecodePlan pl = plan_decode(args, num_splits);
  if (num_splits_used) *num_splits_used = pl.splits;
  st = check_plan(fn, args, pl);
  if (st != FP8ATTN_OK) return st;
  if (pl.ws_bytes > FP8ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(FP8ATTN_ERR_WORKSPACE, "%s: %s %d needs %zu bytes of split-KV scratch, more than the %zu of the "
                "static scratch array; call fp8attn_decode_paged with a workspace (or ask for fewer splits)", fn,
                pl.balanced ? "a balanced partition of parts" : "split count", pl.balanced ? -pl.splits : pl.splits,
                pl.ws_bytes, (size_t)FP8ATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_address(fn, &ws);
    if (st != FP8ATTN_OK) return st;
  }
  return run_decode(fn, args, pl, ws, stream);
}

fp8attn_status fp8attn_prefill_varlen(const fp8attn_attn_args* args, hipStream_t stream) {
  const char* fn = "fp8attn_prefill_varlen";
  fp8attn_status st = validate_attn(fn, args, false);
  if (st != FP8ATTN_OK) return st;
  if (args->total_q == 0 || args->batch == 0) return ok();
  fp8attn::AttnParams p = make_params(args);
  hipError_t e;
  if (args->q_dtype == FP8ATTN_E4M3 || args->q_dtype == FP8ATTN_BF16_TO_E4M3) {
    e = fp8attn::launch_prefill_fp8(p, args->head_dim, args->q_dtype == FP8ATTN_BF16_TO_E4M3, stream);
  } else if (args->head_dim == 512) {
    // the full-attention layers' head dim with bf16 Q: the d512 MFMA prefill
    e = fp8attn::launch_prefill_wide(p, args->q_dtype == FP8ATTN_BF16_SPLIT, stream);
  } else {
    // BF16 queries at head dims up to 256: the split-KV kernel over 32-row query tiles (16 when
    // no sequence has more rows per kv head), one split per tile.
    const int G = args->num_q_heads / args->num_kv_heads;
    const int64_t rows = (int64_t)args->max_seqlen_q * G;
    p.tile_rows = rows > 16 && args->head_dim <= 256 ? 32 : 16;
    p.row_groups = (int32_t)((rows + p.tile_rows - 1) / p.tile_rows);
    p.num_splits = 1;
    p.units_per_split = (int32_t)(((int64_t)args->max_seqlen_k + 15) / 16 + 1);
    const int64_t grid = (int64_t)args->num_kv_heads * args->batch * p.row_groups;
    if (grid >= (int64_t)1 << 31)
      return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: grid of %lld blocks is too large", fn, (long long)grid);
    e = fp8attn::launch_decode(p, args->q_dtype, args->head_dim, grid, stream);
  }
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

fp8attn_status fp8attn_splitkv_combine(const float* partial_o, const float* partial_lse, int32_t num_splits,
                                       int64_t total_q, int32_t num_q_heads, int32_t head_dim, void* out_bf16,
                                       int64_t out_stride_tok, int64_t out_stride_head, float* lse_out,
                                       hipStream_t stream) {
  const char* fn = "fp8attn_splitkv_combine";
  if (num_splits <= 0 || total_q < 0 || num_q_heads <= 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: num_splits > 0, total_q >= 0 and num_q_heads > 0 required", fn);
  if (head_dim != 64 && head_dim != 96 && head_dim != 128 && head_dim != 192 && head_dim != 256 && head_dim != 512)
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 96, 128, 192, 256, 512}", fn, head_dim);
  if (out_stride_tok < 0 || out_stride_head < 0)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: output strides must be >= 0", fn);
  if (total_q == 0) return ok();
  if (!partial_o || !partial_lse || !out_bf16)
    return fail(FP8ATTN_ERR_INVALID_ARG, "%s: partial_o, partial_lse and out_bf16 must be non-NULL", fn);
  if (!aligned(partial_o, 16) || !aligned(partial_lse, 4) || !aligned(out_bf16, 2) || (lse_out && !aligned(lse_out, 4)))
    return fail(FP8ATTN_ERR_UNSUPPORTED, "%s: partial_o must be 16-byte aligned", fn);
  hipError_t e = fp8attn::launch_combine(partial_o, partial_lse, num_splits, total_q, num_q_heads, head_dim, out_bf16,
                                         out_stride_tok, out_stride_head, lse_out, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

}  // extern "C"
