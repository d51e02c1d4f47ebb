// Q quantization to OCP E4M3 ahead of the native-FP8 attention (vLLM PR #63139, Overview:
// sliding-window layers quantize Q before the FP8 forward).  Rule: one IEEE fp32 division by the
// per-tensor descale, round to nearest even, saturate at +-448.  HBM-bound elementwise pass:
// each thread moves 8 bf16 in (16 B) and 8 codes out (8 B).
//
// The fp32 quotient without a division per element: q = RN32(RN64(x * RN64(1 / descale))).  The
// fp64 product is within about 2^-52 (relative) of x / descale.  For x with at most 24
// significant bits (bf16 here) and an fp32 descale, x / descale is never exactly halfway between
// two fp32 values.  It is also at least 2^-47 (relative) away from any halfway point: the
// difference x - m * descale, for a halfway point m, is a nonzero multiple of a power of two
// that small relative to x.  So the single rounding to fp32 lands where the correctly rounded
// division does.  The E4M3 rounding then uses the converter (round to nearest even) on the
// value clamped to +-448, which is the saturation of the rule.  The clamp turns a NaN quotient
// (a NaN input, or 0 / 0 with a zero descale) into a finite value, whereas the rule gives
// 0x7F | sign with the quotient's IEEE sign, sign(x) XOR sign(descale): a branch taken only where
// a lane's quotient is NaN writes those codes.
#include "device.h"
#include "params.h"

namespace fp8attn {

// CONTIG: Q rows (token, head) are back to back (head stride d, token stride heads * d), so the
// input vector index is the output one and no index arithmetic is needed.
//
// Each thread issues kQuantUnroll 16-byte loads (vectors v and v + T for T threads in the grid,
// so every load instruction of a wave is one contiguous 1 KiB) before the first conversion, and
// the grid has a block per 256 * kQuantUnroll vectors: one trip through the loop per thread.  A
// grid capped at 64 blocks per CU, each thread looping over several trips with one load at a
// time, reached 4.8 TB/s on the 1 GiB prefill Q; this shape reaches 6.0-6.2 TB/s, the rate of
// torch's own bf16 -> E4M3 cast over the same bytes.  Loads and stores are non-temporal: every
// byte is touched once.
constexpr int kQuantUnroll = 2;

template <bool CONTIG>
__global__ void __launch_bounds__(256) quantize_q_kernel(const __bf16* __restrict__ q, int64_t nvec,
                                                         int32_t nheads, int32_t vec_per_head,
                                                         int64_t stride_tok, int64_t stride_head,
                                                         const float* __restrict__ q_descale,
                                                         uint8_t* __restrict__ out) {
  const float ds = q_descale ? q_descale[0] : 1.0f;
  const double rcp = 1.0 / (double)ds;   // correctly rounded fp64 reciprocal
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  auto src_of = [&](int64_t v) __attribute__((always_inline)) -> int64_t {
    if constexpr (CONTIG) return v * 8;
    const int64_t c = v % vec_per_head;
    const int64_t th = v / vec_per_head;
    const int64_t hd = th % nheads;
    const int64_t tok = th / nheads;
    return tok * stride_tok + hd * stride_head + c * 8;
  };
  for (int64_t v0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v0 < nvec; v0 += kQuantUnroll * nthr) {
    u32x4_t w[kQuantUnroll];
#pragma unroll
    for (int k = 0; k < kQuantUnroll; ++k) {
      const int64_t v = v0 + k * nthr;
      w[k] = v < nvec ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q + src_of(v)))
                      : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kQuantUnroll; ++k) {
      const int64_t v = v0 + k * nthr;
      const u32x2_t codes = quantize8_bf16_e4m3(w[k], rcp);   // (all lanes: it holds a wave ballot)
      if (v < nvec) __builtin_nontemporal_store(codes, reinterpret_cast<u32x2_t*>(out + v * 8));
    }
  }
}

hipError_t launch_quantize_q(const void* q, int64_t ntok, int32_t nheads, int32_t d,
                             int64_t stride_tok, int64_t stride_head, const float* q_descale,
                             void* out, hipStream_t stream) {
  const int32_t vph = d / 8;
  const int64_t nvec = ntok * nheads * vph;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 256 * kQuantUnroll - 1) / (256 * kQuantUnroll);
  if (blocks > (1 << 30)) blocks = 1 << 30;   // beyond that, the grid-stride loop takes the rest
  const bool contig = stride_head == d && stride_tok == (int64_t)nheads * d;
  if (contig)
    hipLaunchKernelGGL(quantize_q_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const __bf16*>(q), nvec, nheads, vph, stride_tok, stride_head, q_descale,
                       reinterpret_cast<uint8_t*>(out));
  else
    hipLaunchKernelGGL(quantize_q_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const __bf16*>(q), nvec, nheads, vph, stride_tok, stride_head, q_descale,
                       reinterpret_cast<uint8_t*>(out));
  return hipGetLastError();
}

}  // namespace fp8attn
