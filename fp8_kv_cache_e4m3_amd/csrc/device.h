// Device helpers for gfx950 (CDNA4): vector types, E4M3 conversions, MFMA wrappers,
// wave-level reductions and the XCD-aware block remap.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp8attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector memory operations of
// this wave are outstanding and leaves the other counters unconstrained
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// A uniform read of read-only data through the constant address space: a scalar load, which
// waits on lgkmcnt and leaves the vector memory counter to the streaming loads.
__device__ __forceinline__ float load_uniform(const float* p, int64_t i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// ---------------------------------------------------------------------------------------------
// Direct-to-LDS loads, issued from inline assembly on purpose: the compiler then does not track
// them, and the kernel alone orders them against the LDS reads (explicit vmcnt waits before the
// barrier that publishes a tile).  When the compiler tracks them itself, it cannot prove that
// reads of one stage are independent of loads into another across loop iterations and drains
// all loads in flight before every read.
// ---------------------------------------------------------------------------------------------
// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One wave-wide direct-to-LDS load: lane i copies the 16 bytes at gbase + voff (voff per lane)
// to LDS address lds_dst + 16 i.  M0 holds the LDS address; gfx9 needs one wait state between an
// SALU write of M0 and the load that reads it.  M0 is not otherwise live in these kernels.
__device__ __forceinline__ void lds_dma16(const uint8_t* gbase, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds_dst)
               : "memory", "m0");
}
// The same copy through a buffer resource (V#): base address, no stride, num_records bytes.  A
// lane whose offset lies at or past num_records is out of range and, as for every buffer load,
// reads zeros, which land in LDS like any other data.
__device__ __forceinline__ void lds_dma16_buf(const i32x4_t rsrc, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_dst)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource for the loads above: 48-bit base, stride 0 (offsets are plain byte offsets),
// num_records bytes in range, and the gfx9 dword-3 word for untyped 32-bit accesses.
__device__ __forceinline__ i32x4_t buffer_rsrc(const uint8_t* base, uint32_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)num_records, 0x00020000};
}

// ---------------------------------------------------------------------------------------------
// E4M3 -> bf16, exact: every E4M3 value is a bf16 value.  gfx950's v_cvt_scalef32_pk_bf16_fp8
// converts two OCP E4M3 bytes (bytes 0,1 or 2,3 of the dword) with a unit scale.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bf16x2_t e4m3x2_lo_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ bf16x2_t e4m3x2_hi_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}
// 8 E4M3 bytes (two dwords) -> 8 bf16 in byte order
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  bf16x2_t a = e4m3x2_lo_to_bf16(w0), b = e4m3x2_hi_to_bf16(w0);
  bf16x2_t c = e4m3x2_lo_to_bf16(w1), d = e4m3x2_hi_to_bf16(w1);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// 4 E4M3 bytes (one dword) -> 4 bf16 in byte order
__device__ __forceinline__ bf16x4_t e4m3x4_to_bf16(uint32_t w) {
  bf16x2_t a = e4m3x2_lo_to_bf16(w), b = e4m3x2_hi_to_bf16(w);
  return bf16x4_t{a[0], a[1], b[0], b[1]};
}

// ---------------------------------------------------------------------------------------------
// 4x4 byte transpose: in row k holds bytes x[k][0..3]; out e holds x[0..3][e].  Eight
// v_perm_b32: interleave the bytes of rows (0,1) and (2,3), then pair up their 16-bit halves.
// (v_perm_b32 selector byte 0..3 picks a byte of the second source, 4..7 of the first.)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void transpose4x4_u8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                uint32_t& t0, uint32_t& t1, uint32_t& t2, uint32_t& t3) {
  const uint32_t p01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0.0 a1.0 a0.1 a1.1
  const uint32_t p01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0.2 a1.2 a0.3 a1.3
  const uint32_t p23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
  const uint32_t p23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  t0 = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
  t1 = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
  t2 = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
  t3 = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
}

// ---------------------------------------------------------------------------------------------
// Q quantization to E4M3, shared by fp8attn_quantize_q and the attention kernels that take bf16
// Q for the native-FP8 path (both give identical codes).  The rule: fp32 quotient q / descale,
// round to nearest even, saturate at +-448; a NaN quotient gives 0x7F with the quotient's sign,
// which IEEE division takes as sign(x) XOR sign(descale) also when the quotient is NaN (an input
// NaN, or 0 / 0 and inf / inf with a zero or infinite descale).  The fp32 quotient is
// RN32(RN64(x * RN64(1 / descale))), which equals the correctly rounded division for every x
// with at most 24 significant bits; the argument is given where fp8attn_quantize_q is defined.
// rcp is RN64(1 / descale) and carries the descale's sign (1 / +-0 = +-inf).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float q_quotient(float x, double rcp) { return (float)((double)x * rcp); }
__device__ __forceinline__ float clamp448(float q) {
  return __builtin_fminf(__builtin_fmaxf(q, -448.0f), 448.0f);   // a NaN is fixed afterwards
}
// the 8 bf16 of a 16-byte word -> 8 E4M3 codes (element i in byte i of the two dwords).
// The clamp maps a NaN quotient to a finite value, so NaN quotients are patched afterwards.  The
// test for them is a wave-wide ballot (one compare per element, OR-ed in scalar registers), and
// the patch is a wave-uniform branch that real data never takes.
__device__ __forceinline__ u32x2_t quantize8_bf16_e4m3(const u32x4_t w, double rcp) {
  float x[8], y[8];
  uint64_t nan_lanes = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float q = q_quotient(x[k], rcp);
    nan_lanes |= __builtin_amdgcn_ballot_w64(q != q);
    y[k] = clamp448(q);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  if (nan_lanes != 0) {
    const uint32_t ds_sign = (uint32_t)((uint64_t)__double_as_longlong(rcp) >> 56) & 0x80u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float q = q_quotient(x[k], rcp);
      if (q != q) {
        const uint32_t code = 0x7fu | (((__float_as_uint(x[k]) >> 24) & 0x80u) ^ ds_sign);
        const int sh = 8 * (k & 3);
        if (k < 4) lo = (int)(((uint32_t)lo & ~(0xffu << sh)) | (code << sh));
        else hi = (int)(((uint32_t)hi & ~(0xffu << sh)) | (code << sh));
      }
    }
  }
  return u32x2_t{(uint32_t)lo, (uint32_t)hi};
}

// ---------------------------------------------------------------------------------------------
// MFMA wrappers (operand layouts measured on gfx950):
//  16x16x32 bf16 / fp8 : lane l supplies row (A) or column (B) l%16 and 8 k-values for k-group
//                        l/16; C lane l holds rows 4*(l/16)+i, column l%16.
//  16x16x16 bf16       : same with 4 k-values per lane.
// A and B use the same (lane group, slot) -> k assignment, so any consistent mapping of the
// contraction index onto slots is valid.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x16(bf16x4_t a, bf16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_fp8_16x16x32(uint64_t a, uint64_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// Cross-lane helpers (wave64)
// ---------------------------------------------------------------------------------------------
// gfx950's lane-swap instructions exchange 16-lane rows (v_permlane16_swap: rows 0<->1 and 2<->3)
// or 32-lane halves (v_permlane32_swap) between two registers on the VALU, without the LDS round
// trip of a ds_bpermute.  Given the value twice, the two results hold, in every lane, the lane's
// own value and its partner's (lane l ^ 16, or l ^ 32), in an order that depends on the lane;
// max and sum of the pair are symmetric, so every lane gets the pair's max or sum (bit-identical
// to v + shfl(v), since fp32 addition commutes).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// reduce over the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float max_over_groups(float v) { return max_xor32(max_xor16(v)); }
__device__ __forceinline__ float sum_over_groups(float v) { return sum_xor32(sum_xor16(v)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------------
// XCD-aware remap: the dispatcher sends block i to XCD i % 8.  Give each XCD a contiguous
// range of logical ids so that neighbouring work items (which share K/V pages) share an L2.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcd_remap32(uint32_t bid, uint32_t n) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = n / kXcd, rem = n % kXcd;
  const uint32_t x = bid % kXcd, k = bid / kXcd;
  return x * per + (x < rem ? x : rem) + k;
}
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
  constexpr int64_t kXcd = 8;
  const int64_t per = n / kXcd, rem = n % kXcd;
  const int64_t x = bid % kXcd, k = bid / kXcd;
  return x * per + (x < rem ? x : rem) + k;
}

// ---------------------------------------------------------------------------------------------
// 32x32 FP8 MFMA with operand scales, P packing, LDS operand addressing (the prefill kernels)
// ---------------------------------------------------------------------------------------------
constexpr int kE8M0One = 127;        // E8M0 scale 2^0
constexpr int kE8M0Sixteenth = 123;  // E8M0 scale 2^-4

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 16x16x128 FP8 MFMA with a scale on the B operand (unit scale on A)
__device__ __forceinline__ f32x4_t mfma_fp8_16x16x128(const i32x8_t& a, const i32x8_t& b, f32x4_t c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, scale_b);
}
__device__ __forceinline__ f32x16_t mfma_fp8_32x32x64(const i32x8_t& a, const i32x8_t& b, f32x16_t c,
                                                      int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, scale_b);
}

// four fp32 -> four E4M3 bytes (round to nearest even; inputs are in [0, 448])
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// exact decode of the four E4M3 bytes of a dword (only used for the split-P residual)
__device__ __forceinline__ void unpack4_e4m3(uint32_t w, float out[4]) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// A per-lane LDS byte offset the optimiser treats as opaque, so that it is not split into a chain
// of address computations.  Every operand read is then the stage array plus this offset plus a
// constant, and the LDS lowering can still tell which array (stage) each read touches: that is
// what lets a read of one stage proceed while direct-to-LDS loads into another are in flight.
__device__ __forceinline__ int lane_offset(int x) {
  asm("" : "+v"(x));
  return x;
}

// MFMA row m of a 32-key half tile holds key kperm(m): bits 2 and 3 of m swapped.
__device__ __forceinline__ int kperm(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// ---------------------------------------------------------------------------------------------
// Split Q: bf16 values as two E4M3 terms (the decode and d512 prefill kernels)
// ---------------------------------------------------------------------------------------------
// Split Q (kQBf16Split): one query row, scaled by a power of two 2^e so that its largest
// magnitude is at most 448, is written as hi + lo / 16 with hi = E4M3(x 2^e) and
// lo = E4M3(16 (x 2^e - hi)).  A bf16 value has 8 significant bits; hi keeps the top 4 (rounded
// to nearest even) and the residual then has at most 4, so hi + lo / 16 equals x 2^e exactly
// unless hi or lo falls below E4M3's normal range (|x| under about 2^-14 of the row's largest).
// QK^T is then accumulated in two parts on the FP8 MFMA, S = K hi + (K lo) / 16, and scaled back
// by 2^-e: the BF16 product up to the order of the fp32 sums.
__device__ __forceinline__ void split8_bf16_e4m3(const u32x4_t w, const float scale, uint64_t& hi, uint64_t& lo) {
  float x[8], r[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16) * scale;           // exact: a power-of-two scale
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u) * scale;
  }
  int h[2], l[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    h[q] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q], x[4 * q + 1], 0, false);
    h[q] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q + 2], x[4 * q + 3], h[q], true);
    const f32x2_t d0 = __builtin_amdgcn_cvt_pk_f32_fp8(h[q], false);
    const f32x2_t d1 = __builtin_amdgcn_cvt_pk_f32_fp8(h[q], true);
    r[4 * q] = (x[4 * q] - d0[0]) * 16.0f;                    // exact differences
    r[4 * q + 1] = (x[4 * q + 1] - d0[1]) * 16.0f;
    r[4 * q + 2] = (x[4 * q + 2] - d1[0]) * 16.0f;
    r[4 * q + 3] = (x[4 * q + 3] - d1[1]) * 16.0f;
    l[q] = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * q], r[4 * q + 1], 0, false);
    l[q] = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * q + 2], r[4 * q + 3], l[q], true);
  }
  hi = (uint64_t)(uint32_t)h[0] | ((uint64_t)(uint32_t)h[1] << 32);
  lo = (uint64_t)(uint32_t)l[0] | ((uint64_t)(uint32_t)l[1] << 32);
}

// 2^e with e = floor(log2(448 / amax)), clamped to [-126, 126] (both 2^e and 2^-e normal); an
// all-zero row takes 2^126.
__device__ __forceinline__ int split_exponent(float amax) {
  const float m = 448.0f / amax;
  const int e = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;
  return max(-126, min(126, e));
}

}  // namespace fp8attn
