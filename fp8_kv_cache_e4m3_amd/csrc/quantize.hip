// Q quantization to OCP E4M3 ahead of the native-FP8 attention (vLLM PR #63139, Overview:
// sliding-window layers quantize Q before the FP8 forward).  Rule: one IEEE fp32 division by the
// per-tensor descale, round to nearest even, saturate at +-448.  HBM-bound elementwise pass:
// each thread moves 8 bf16 in (16 B) and 8 codes out (8 B).
#include "device.h"
#include "params.h"

namespace fp8attn {

__global__ void __launch_bounds__(256) quantize_q_kernel(const __bf16* __restrict__ q, int64_t nvec,
                                                         int32_t nheads, int32_t vec_per_head,
                                                         int64_t stride_tok, int64_t stride_head,
                                                         const float* __restrict__ q_descale,
                                                         uint8_t* __restrict__ out) {
  const float ds = q_descale ? q_descale[0] : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t c = v % vec_per_head;
    const int64_t th = v / vec_per_head;
    const int64_t hd = th % nheads;
    const int64_t tok = th / nheads;
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(q + tok * stride_tok + hd * stride_head + c * 8);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = __uint_as_float(w[k] << 16);
      const float x1 = __uint_as_float(w[k] & 0xffff0000u);
      const uint32_t c0 = f32_to_e4m3_rne_sat(x0 / ds);
      const uint32_t c1 = f32_to_e4m3_rne_sat(x1 / ds);
      const uint32_t pair = c0 | (c1 << 8);
      if (k < 2) lo |= pair << (16 * k);
      else hi |= pair << (16 * (k - 2));
    }
    *reinterpret_cast<u32x2_t*>(out + v * 8) = u32x2_t{lo, hi};
  }
}

hipError_t launch_quantize_q(const void* q, int64_t ntok, int32_t nheads, int32_t d,
                             int64_t stride_tok, int64_t stride_head, const float* q_descale,
                             void* out, hipStream_t stream) {
  const int32_t vph = d / 8;
  const int64_t nvec = ntok * nheads * vph;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(quantize_q_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const __bf16*>(q), nvec, nheads, vph, stride_tok, stride_head,
                     q_descale, reinterpret_cast<uint8_t*>(out));
  return hipGetLastError();
}

}  // namespace fp8attn
