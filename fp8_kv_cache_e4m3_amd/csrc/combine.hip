// Log-sum-exp combine of split-KV partials (vLLM PR #60372, Details: the combine work that
// split-KV adds).  One wave per row (token, q head): M = max_s lse_s, w_s = exp(lse_s - M),
// o = sum_s w_s o_s / sum_s w_s, lse = M + ln sum_s w_s.  Splits with lse = -inf are skipped
// (their partials are never read).  Each lane owns ceil(D/64) contiguous values of the row.
#include "device.h"
#include "params.h"

namespace fp8attn {

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, int32_t S,
                                                      int64_t rows, int32_t hq, __bf16* __restrict__ out,
                                                      int64_t out_stride_tok, int64_t out_stride_head,
                                                      float* __restrict__ lse_out) {
  constexpr int PL = (D + 63) / 64;  // values per lane (head dim 96: lanes 48.. hold none)
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= rows) return;
  const bool lane_ok = lane * PL < D;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_lse[(int64_t)s * rows + n]);
  float acc[PL];
#pragma unroll
  for (int c = 0; c < PL; ++c) acc[c] = 0.f;
  float wsum = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float l = part_lse[(int64_t)s * rows + n];
      if (l == kNegInf) continue;
      const float w = __expf(l - M);
      wsum += w;
      const float* src = part_o + ((int64_t)s * rows + n) * D + lane * PL;
      if constexpr (PL == 8) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) { acc[c] += w * a[c]; acc[4 + c] += w * b[c]; }
      } else if constexpr (PL == 4) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += w * a[c];
      } else if (lane_ok) {
#pragma unroll
        for (int c = 0; c < PL; ++c) acc[c] += w * src[c];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  const int64_t tok = n / hq, hh = n % hq;
  __bf16* dst = out + tok * out_stride_tok + hh * out_stride_head + lane * PL;
  if (lane_ok) {
#pragma unroll
    for (int c = 0; c < PL; ++c) dst[c] = (__bf16)(acc[c] * inv);
  }
  if (lse_out && lane == 0) lse_out[n] = wsum > 0.f ? M + __logf(wsum) : kNegInf;
}

// The balanced partition's combine: one wave per (row tile, tile row).  A tile whose range lay
// inside one block was written final by that block (first == last) and is skipped; otherwise the
// partials of blocks first..last sit in slots (block + tile index), and are merged as above.
template <int D>
__global__ void __launch_bounds__(256) combine_parts_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_lse,
                                                            const int32_t* __restrict__ seg_meta,
                                                            const int32_t* __restrict__ cu_seqlens_q,
                                                            int32_t tiles_per_head, int32_t row_groups,
                                                            int32_t group, int32_t parts, int64_t n_rows,
                                                            __bf16* __restrict__ out,
                                                            int64_t out_stride_tok, int64_t out_stride_head,
                                                            float* __restrict__ lse_out, int32_t hq) {
  constexpr int PL = (D + 63) / 64;  // values per lane (head dim 96: lanes 48.. hold none)
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_rows) return;
  const bool lane_ok = lane * PL < D;
  const int g = (int)(n >> 4), r = (int)(n & 15);
  const int h = g / tiles_per_head, j = g - h * tiles_per_head;
  const int b = j / row_groups, rt = j - b * row_groups;
  const int t0 = cu_seqlens_q[b], t1 = cu_seqlens_q[b + 1];
  const int row = rt * 16 + r;
  if (row >= (t1 - t0) * group) return;
  const int first = seg_meta[2 * g], last = seg_meta[2 * g + 1];
  // (a tile with rows always has a unit, so its entry is from this launch; the bounds check only
  // keeps lengths below q_len, which the call does not allow, from reading outside the workspace)
  if (first == last || first < 0 || first > last || last >= parts) return;
  float M = kNegInf;
  for (int i = first; i <= last; ++i) M = fmaxf(M, part_lse[(int64_t)(i + g) * 16 + r]);
  float acc[PL];
#pragma unroll
  for (int c = 0; c < PL; ++c) acc[c] = 0.f;
  float wsum = 0.f;
  if (M != kNegInf) {
    for (int i = first; i <= last; ++i) {
      const int64_t e = (int64_t)(i + g) * 16 + r;
      const float l = part_lse[e];
      if (l == kNegInf) continue;
      const float w = __expf(l - M);
      wsum += w;
      const float* src = part_o + e * D + lane * PL;
      if (lane_ok) {
#pragma unroll
        for (int c = 0; c < PL; ++c) acc[c] += w * src[c];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  const int64_t tok = t0 + row / group, hh = (int64_t)h * group + row % group;
  __bf16* dst = out + tok * out_stride_tok + hh * out_stride_head + lane * PL;
  if (lane_ok) {
#pragma unroll
    for (int c = 0; c < PL; ++c) dst[c] = (__bf16)(acc[c] * inv);
  }
  if (lse_out && lane == 0) lse_out[tok * hq + hh] = wsum > 0.f ? M + __logf(wsum) : kNegInf;
}

hipError_t launch_combine_parts(const float* part_o, const float* part_lse, const int32_t* seg_meta,
                                const int32_t* cu_seqlens_q, int32_t batch, int32_t row_groups, int32_t hkv,
                                int32_t group, int32_t parts, int32_t d, void* out, int64_t out_stride_tok,
                                int64_t out_stride_head, float* lse_out, hipStream_t stream) {
  const int32_t tiles = batch * row_groups;
  const int64_t n_rows = (int64_t)hkv * tiles * 16;
  if (n_rows == 0) return hipSuccess;
  const dim3 g((unsigned)((n_rows + 3) / 4)), blk(256);
  __bf16* o = reinterpret_cast<__bf16*>(out);
  const int32_t hq = hkv * group;
#define FP8ATTN_COMBINE_PARTS(DIM)                                                                   \
  hipLaunchKernelGGL(combine_parts_kernel<DIM>, g, blk, 0, stream, part_o, part_lse, seg_meta, cu_seqlens_q, \
                     tiles, row_groups, group, parts, n_rows, o, out_stride_tok, out_stride_head, lse_out, hq)
  switch (d) {
    case 512: FP8ATTN_COMBINE_PARTS(512); break;
    case 256: FP8ATTN_COMBINE_PARTS(256); break;
    case 192: FP8ATTN_COMBINE_PARTS(192); break;
    case 128: FP8ATTN_COMBINE_PARTS(128); break;
    case 96: FP8ATTN_COMBINE_PARTS(96); break;
    default: FP8ATTN_COMBINE_PARTS(64); break;
  }
#undef FP8ATTN_COMBINE_PARTS
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t S, int64_t total_q,
                          int32_t hq, int32_t d, void* out, int64_t out_stride_tok,
                          int64_t out_stride_head, float* lse_out, hipStream_t stream) {
  const int64_t rows = total_q * hq;
  if (rows == 0) return hipSuccess;
  const dim3 g((unsigned)((rows + 3) / 4)), blk(256);
  __bf16* o = reinterpret_cast<__bf16*>(out);
  if (d == 512)
    hipLaunchKernelGGL(combine_kernel<512>, g, blk, 0, stream, part_o, part_lse, S, rows, hq, o,
                       out_stride_tok, out_stride_head, lse_out);
  else if (d == 256)
    hipLaunchKernelGGL(combine_kernel<256>, g, blk, 0, stream, part_o, part_lse, S, rows, hq, o,
                       out_stride_tok, out_stride_head, lse_out);
  else if (d == 192)
    hipLaunchKernelGGL(combine_kernel<192>, g, blk, 0, stream, part_o, part_lse, S, rows, hq, o,
                       out_stride_tok, out_stride_head, lse_out);
  else if (d == 128)
    hipLaunchKernelGGL(combine_kernel<128>, g, blk, 0, stream, part_o, part_lse, S, rows, hq, o,
                       out_stride_tok, out_stride_head, lse_out);
  else if (d == 96)
    hipLaunchKernelGGL(combine_kernel<96>, g, blk, 0, stream, part_o, part_lse, S, rows, hq, o,
                       out_stride_tok, out_stride_head, lse_out);
  else
    hipLaunchKernelGGL(combine_kernel<64>, g, blk, 0, stream, part_o, part_lse, S, rows, hq, o,
                       out_stride_tok, out_stride_head, lse_out);
  return hipGetLastError();
}

}  // namespace fp8attn
