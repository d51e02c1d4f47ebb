// Split-KV paged attention for a few query tokens per sequence (decode, spec-decode verify).
//
// What it computes: masked softmax attention of one 16-row query tile (rows = (token, q head)
// pairs of one kv head, token-major) over the keys of one KV split, on a paged E4M3 cache with
// per-tensor descales (vLLM PR #60372, Overview/Claims; prhub digest of vLLM PR #48666, Key
// code), for both variants:
//   QM = kQE4M3   : E4M3 Q codes (vLLM PR #63139, Overview), QK^T on the FP8 MFMA;
//   QM = kQBf16E4M3: bf16 Q quantized to E4M3 as the kernel loads it, with the same arithmetic
//                   as fp8attn_quantize_q (identical codes), then the same FP8 path;
//   QM = kQBf16   : BF16 Q, K dequantized in registers (exact: E4M3 values are bf16 values),
//                   QK^T on the BF16 MFMA;
//   QM = kQBf16Split: BF16 Q split into two E4M3 terms per value (per-row power-of-two scale),
//                   QK^T on the FP8 MFMA as a two-part accumulation (vLLM PR #60372, review
//                   thread: the d512 FP8-MMA kernel keeps BF16 queries and builds a split QK
//                   accumulation; the split itself is not described there, see split8_bf16_e4m3).
// PV runs on the BF16 MFMA in the first three modes: V bytes are dequantized exactly to bf16 and
// P is rounded once to bf16.  Decode is HBM-bound, so the cheaper FP8 PV would not move the time,
// and plain E4M3 P would cost accuracy on short rows.  Split Q runs PV on the FP8 MFMA with P as
// two E4M3 terms, as many significant bits as bf16 P (see compute).
//
// Design (gfx950, wave64):
//  * Work item = (kv head, split, sequence, row tile), XCD-aware block order, or a range of the
//    balanced partition (decode_balanced_kernel).  4 waves per block; each wave streams its own
//    16-key units (a quarter of the range) straight from HBM into registers, with the next
//    unit's loads in flight while the current one is computed.  No barriers in the main loop;
//    K passes through a wave-private LDS tile to turn its row-order loads into MFMA operands.
//  * S^T = K * Q^T: the 16 keys are MFMA rows, the 16 query rows are MFMA columns, so every
//    query row lives on one lane column (lane % 16) and its softmax state is per lane.
//  * O^T = V^T * P^T: P^T comes straight out of the S^T accumulator layout (lane (r, g) holds
//    keys 4g..4g+3 of row r), which is the B operand of the 16x16x16 BF16 MFMA.  V^T operands
//    come from 4 keys x 16 bytes per lane via a byte transpose (v_perm) and an exact convert.
//  * The 4 waves' (max, sum, O) are merged through LDS at the end; one split writes bf16 O and
//    LSE directly, several splits write fp32 partials for the LSE combine.
#include "device.h"
#include "params.h"

namespace fp8attn {

// Timeline builds only (build.py --timeline, for bench.py --timeline): the split-grid decode kernel
// stamps the phases of each of its first kTimelineBlocks blocks with the shader clock
// (s_memtime), one 64-bit slot per stamp, written by lane 0 of the stamping wave:
//   0 entry, 1-4 first unit computed (waves 0-3), 5-8 stream done (waves 0-3), 9 merge done,
//   10 outputs stored, 11 HW_ID, 12 XCC_ID, 13/14 real-time clock at entry / end.
#ifdef FP8ATTN_TIMELINE
constexpr int kTimelineBlocks = 4096;
constexpr int kTimelineSlots = 16;
__device__ uint64_t g_decode_timeline[kTimelineBlocks * kTimelineSlots];
__device__ __forceinline__ void tl_mark(int slot, uint64_t v) {
  if ((threadIdx.x & 63) == 0 && blockIdx.x < kTimelineBlocks)
    g_decode_timeline[blockIdx.x * kTimelineSlots + slot] = v;
}
#endif

constexpr float kLazyMax = 8.0f;   // log2 units: the running max moves by more than 2^8 or not at all

template <int D>
struct DecodeShape {
  static constexpr int kKeys = 16;                    // keys per unit
  static constexpr int KCH = D / 64;                  // 16-byte K chunks per lane per unit
  static constexpr int CW = D >= 256 ? 16 : D / 16;   // V bytes per lane per key per block
  static constexpr int VBLK = D / (16 * CW);          // V column blocks
  static constexpr int NT = D / 16;                   // O^T tiles (16 d-rows each)
  static constexpr int RS = D + 4;                    // LDS row stride (floats), padded
  static constexpr bool KROW = D <= 256;              // K loaded in row order (see UnitOffsets)
  static constexpr int KTS = D + 16;                  // K tile row stride (bytes), padded
  static constexpr int KOFS = KROW && 1024 % D != 0 ? KCH : 1;   // per-lane K load offsets kept
  static_assert(D == 64 || D == 128 || D == 192 || D == 256 || D == 512, "head dim");
};

template <int D>
struct UnitRegs {
  u32x4_t k[DecodeShape<D>::KCH];
  uint32_t v[4][DecodeShape<D>::VBLK][DecodeShape<D>::CW / 4];
};

// K/V byte loads through a buffer resource whose range ends after the unit's last key below the
// sequence length: lanes addressing keys at or past it read zeros (out-of-range buffer loads).
// Those slots are never written for this sequence and may hold any bytes, E4M3 NaN codes
// included; their keys are masked (P = 0), but 0 * NaN is NaN in the MFMA.  NT marks the loads
// non-temporal (streamed once, no reuse).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t unit_rsrc(const uint8_t* base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)num_records, 0x00020000);
}
template <bool NT>
__device__ __forceinline__ u32x4_t stream_load16(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ u32x2_t stream_load8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ uint32_t stream_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, NT ? 2 : 0);
}

// Per-lane byte offsets inside a unit, the same for every unit.  A unit's loads are a uniform
// base (page plus first slot) plus these 32-bit offsets: the SGPR-base form of the global loads.
//  * K is read in row order: load c covers bytes [1024 c, 1024 c + 1024) of the unit's 16 x D
//    bytes taken row by row, lane l the 16 bytes at 16 (64 c + l), so each 16-lane quarter of a
//    load reads whole 256-byte runs of one or more key rows.  (The MFMA operand layout read
//    straight from memory, lane (col, grp) taking bytes 16 grp + 64 c of key col, has every
//    quarter touch 16 rows: a plain gather with that pattern is 7% slower on the sliding-window
//    decode's K/V stream.)  The operand layout then comes out of a wave-private LDS tile
//    (k_operands).  Load c's offset is k[0] + c kstep (1024 / D rows per load), or k[c] (head
//    dim 192, whose rows straddle the loads).  Head dim 512 keeps the operand layout in its loads
//    (k[0] + 64 c): its rows already fill two quarters each way, and the LDS round trip measured
//    0.6% slower on the full-attention decode.
//  * V rows 4 grp + i, bytes col * CW (+ 16 CW blk): each quarter reads whole rows already.
template <int D>
struct UnitOffsets {
  uint32_t k[DecodeShape<D>::KOFS];
  uint32_t kstep;
  uint32_t v[4];
};

// position of lane l's K bytes of load c in the unit's row-major 16 x D bytes
template <int D>
__device__ __forceinline__ int k_row(int c, int lane) { return (16 * (64 * c + lane)) / D; }
template <int D>
__device__ __forceinline__ int k_col(int c, int lane) { return (16 * (64 * c + lane)) % D; }

template <int D>
__device__ __forceinline__ UnitOffsets<D> unit_offsets(const int64_t sT, const int lane) {
  using S = DecodeShape<D>;
  const int col = lane & 15, grp = lane >> 4;
  UnitOffsets<D> o;
  if constexpr (S::KROW) {
#pragma unroll
    for (int c = 0; c < S::KOFS; ++c) o.k[c] = (uint32_t)(k_row<D>(c, lane) * sT) + (uint32_t)k_col<D>(c, lane);
    o.kstep = (uint32_t)((1024 / D) * sT);
  } else {
    o.k[0] = (uint32_t)(col * sT) + 16u * (uint32_t)grp;
    o.kstep = 64u;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) o.v[i] = (uint32_t)((4 * grp + i) * sT) + (uint32_t)(col * S::CW);
  return o;
}

// K of a unit from the row order of the loads to the MFMA A-operand layout (lane (col, grp):
// key col, bytes 16 grp + 64 c of chunk c) through the wave's LDS tile of 16 rows x KTS bytes.
// The padded row stride puts the 16 rows that one read quarter touches in distinct banks.  The
// tile is the wave's own: its accesses are ordered by the wave's program order, no barrier.
template <int D>
__device__ __forceinline__ void k_operands(const u32x4_t (&in)[DecodeShape<D>::KCH],
                                           u32x4_t (&out)[DecodeShape<D>::KCH], uint8_t* kt, const int lane) {
  using S = DecodeShape<D>;
  if constexpr (!S::KROW) {
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) out[c] = in[c];
    return;
  }
#pragma unroll
  for (int c = 0; c < S::KCH; ++c)
    *reinterpret_cast<u32x4_t*>(kt + k_row<D>(c, lane) * S::KTS + k_col<D>(c, lane)) = in[c];
  const uint8_t* rd = kt + (lane & 15) * S::KTS + 16 * (lane >> 4);
#pragma unroll
  for (int c = 0; c < S::KCH; ++c) out[c] = *reinterpret_cast<const u32x4_t*>(rd + 64 * c);
}

// D: the register layout's head dim; DV < D (head dim 96 in a 128 layout): the lanes whose
// bytes lie past DV (k_ok false: the K bytes, at the same columns in every load; v_ok false:
// the V columns) load nothing and hold zeros, so no byte outside the head is read and the
// padding adds nothing.  trailing: the unit is a filler load past the stream's end (see issue in
// decode_tile): every lane reads the unit's first 16 bytes.
template <int D, int DV, bool NT>
__device__ __forceinline__ void load_unit(UnitRegs<D>& ur, const rsrc_t kunit, const rsrc_t vunit,
                                          const UnitOffsets<D>& off, const bool k_ok, const bool v_ok,
                                          const bool trailing) {
  using S = DecodeShape<D>;
  static_assert(DV == D || (S::KROW && S::KOFS == 1), "a padded head dim needs the same K columns in every load");
  const uint32_t kstep = trailing ? 0u : off.kstep;
#pragma unroll
  for (int c = 0; c < S::KCH; ++c) {
    if (DV == D || k_ok) {
      if constexpr (S::KOFS == 1)
        ur.k[c] = stream_load16<NT>(kunit, trailing ? 0u : off.k[0], c * kstep);
      else
        ur.k[c] = stream_load16<NT>(kunit, trailing ? 0u : off.k[c]);
    } else {
      ur.k[c] = u32x4_t{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int blk = 0; blk < S::VBLK; ++blk) {
      if (DV != D && !v_ok) {
#pragma unroll
        for (int x = 0; x < S::CW / 4; ++x) ur.v[i][blk][x] = 0u;
        continue;
      }
      const uint32_t vo = off.v[i] + blk * 16 * S::CW;
      if constexpr (S::CW == 16) {
        const u32x4_t w = stream_load16<NT>(vunit, vo);
        ur.v[i][blk][0] = w[0];
        ur.v[i][blk][1] = w[1];
        ur.v[i][blk][2] = w[2];
        ur.v[i][blk][3] = w[3];
      } else if constexpr (S::CW == 8) {
        const u32x2_t w = stream_load8<NT>(vunit, vo);
        ur.v[i][blk][0] = w[0];
        ur.v[i][blk][1] = w[1];
      } else {   // 4 or 12 bytes: dword loads
#pragma unroll
        for (int x = 0; x < S::CW / 4; ++x) ur.v[i][blk][x] = stream_load4<NT>(vunit, vo + 4 * x);
      }
    }
  }
}

// Per-variant tuning (measured on MI355X, sliding-window decode, cold K/V).  Two units in
// flight per wave; deeper register rings (3 or 4 units, which fit at two waves per SIMD) were
// slower, as were rings staged through LDS with direct-to-LDS loads.  A plain gather of the
// same 269 MB in the same order (whole 256-byte row slices per 16-lane quarter, 4 waves x 512
// blocks) takes 41.9 us; the kernel about 45.7 us.  Non-temporal loads help the d256 stream
// (+4%) and the balanced partition at d512 (full-attention decode 908 -> 853 us); on the split
// grid at d512 they measured 11% slower (they are set per launch shape in decode_tile).
template <bool QFP8, int D>
struct DecodeTune {
  static constexpr int NBUF = 2;
  static constexpr bool NT = QFP8 && D == 256;
  // d256 runs two waves per SIMD: the register budget is 256 per wave
  static constexpr int MIN_WAVES = D == 256 ? 2 : 1;
};

template <bool QFP8, int D>
struct QRegs;
template <int D>
struct QRegs<true, D> { uint64_t q[2 * DecodeShape<D>::KCH]; };
template <int D>
struct QRegs<false, D> { bf16x8_t q[2 * DecodeShape<D>::KCH]; };

// One 16-row query tile: row tile rt of sequence b under kv head h, over units
// [u_begin + o0, u_begin + o1) of the tile's visible unit range [u_begin, u_end).  whole: the
// segment is the tile's whole range, so O and LSE are final and go to the output; otherwise the
// tile writes fp32 partials to entry pidx (a split index, or a slot of the balanced partition).
template <int QM, int D, bool BAL>
__device__ __forceinline__ void decode_tile(const AttnParams& p, const int b, const int h, const int rt,
                                            const int o0, const int o1, const int pidx, const bool whole) {
  constexpr bool QFP8 = QM != kQBf16;   // QK^T on the FP8 MFMA
  // head dim 96 runs in the 128 layout: the bytes past 96 are never loaded and count as zeros
  constexpr int DP = D == 96 ? 128 : D;
  using S = DecodeShape<DP>;
  using T = DecodeTune<QFP8, DP>;
  constexpr int NBUF = T::NBUF;
  // LDS: the 4 waves' softmax state and O tiles for the final merge
  __shared__ __attribute__((aligned(16))) float sm_o[4][16][S::RS];
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  // The balanced partition at head dim 512 keeps the Q^T operands in LDS (the 4 waves hold the
  // same rows): in registers they pushed the loop past the 512 registers of a wave (spills).
  constexpr bool QLDS = DP == 512 && BAL;
  __shared__ __attribute__((aligned(16))) uint8_t sm_q[QLDS ? 16384 : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.group;
#ifdef FP8ATTN_TIMELINE
  if (!BAL && wave == 0) {
    tl_mark(0, __builtin_amdgcn_s_memtime());
    tl_mark(11, (uint64_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4));
    tl_mark(12, (uint64_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 20));
    tl_mark(13, __builtin_amdgcn_s_memrealtime());
  }
#endif

  // Every per-item scalar of the prologue is requested here, before any branch, so that the
  // loads share one round trip.  A NULL descale reads a valid stand-in address (the sequence's
  // length) and is replaced by 1 below.
  const int64_t dsi = (int64_t)b * p.ds_stride_b + (int64_t)h * p.ds_stride_h;
  const int t0 = load_uniform(p.cu_seqlens_q, b);
  const int t1 = load_uniform(p.cu_seqlens_q, b + 1);
  const int L = load_uniform(p.seqlens_k, b);
  const float* stand_in = reinterpret_cast<const float*>(p.seqlens_k);
  const float kd_raw = load_uniform(p.k_descale ? p.k_descale : stand_in, p.k_descale ? dsi : 0);
  const float vd_raw = load_uniform(p.v_descale ? p.v_descale : stand_in, p.v_descale ? dsi : 0);
  const float qd_raw = load_uniform(p.q_descale ? p.q_descale : stand_in, 0);
  // (the compiler would otherwise sink each load to its first use, behind the branches below)
  asm volatile("" ::"s"(t0), "s"(t1), "s"(L), "s"(kd_raw), "s"(vd_raw), "s"(qd_raw));
  const int ql = t1 - t0;
  const int nrows = ql * G;
  const int row0 = rt * 16;
  if (row0 >= nrows) return;
  const int rlast = min(row0 + 16, nrows) - 1;
  const int p_first = L - ql + row0 / G;
  const int p_last = L - ql + rlast / G;
  const int W = p.window;
  const int k_lo = W >= 1 ? max(0, p_first - W + 1) : 0;
  const int u_begin = k_lo / 16;
  const int u_end = (p_last + 16) / 16;              // ceil((p_last + 1) / 16)
  const int su0 = u_begin + o0;
  const int su1 = min(u_end, u_begin + o1);
  // keys every row of this tile can see: [full_lo, p_first]
  const int full_lo = W >= 1 ? p_last - W + 1 : 0;

  // this lane's query row
  const int r = row0 + col;
  const bool rvalid = r < nrows;
  const int tok = rvalid ? r / G : rlast / G;
  const int hq = h * G + (rvalid ? r % G : rlast % G);
  const int pos = L - ql + tok;

  if (su0 >= su1) {  // nothing visible in this split: neutral partial for the combine
    // (a segment of the balanced partition is never empty)
    if (!BAL && !whole && threadIdx.x < 16 && rvalid)
      p.part_lse[((int64_t)pidx * p.total_q + t0 + tok) * p.hq + hq] = kNegInf;
    return;
  }

  const float kd = p.k_descale ? kd_raw : 1.0f;
  const float vd = p.v_descale ? vd_raw : 1.0f;
  const float qd = QFP8 && p.q_descale ? qd_raw : 1.0f;
  const float cscale = p.scale_log2 * kd * qd;

  // Page ids of the split's keys: lane i holds the id of page pg_base + i (clamped to the split's
  // last page), refreshed 64 pages at a time.  A unit's page id is then a register read
  // (v_readlane) instead of a memory load on the path to the unit's loads.  Units are issued in
  // increasing order, so the window only moves forward.  (Read before Q, so that waiting for it
  // does not wait for the Q loads.)
  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const int ps = p.page_size;
  const int pg_last = ((su1 - 1) * 16) / ps;
  int pg_base = (su0 * 16) / ps;
  int pg_vec = bt[min(pg_base + lane, pg_last)];

  // ---- Q^T operand (rows on lane columns) ---------------------------------------------------
  constexpr bool SPLIT = QM == kQBf16Split;
  QRegs<QFP8, DP> qr;                                   // (split Q: the hi terms)
  uint64_t qlo[SPLIT ? 2 * S::KCH : 1];                 // split Q: the lo terms
  u32x4_t qraw[QM == kQBf16E4M3 || SPLIT ? 2 * S::KCH : 1];
  if constexpr (QM == kQE4M3) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                        (int64_t)hq * p.q_stride_head + 16 * grp;
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      const bool ok = rvalid && (D == DP || 64 * c + 16 * grp < D);
      u32x4_t w = ok ? *reinterpret_cast<const u32x4_t*>(qp + 64 * c) : u32x4_t{0, 0, 0, 0};
      qr.q[2 * c] = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
      qr.q[2 * c + 1] = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
    }
  } else if constexpr (QM == kQBf16E4M3 || SPLIT) {
    // the same 16 d values per k-chunk as above, read as bf16 here and quantized once the first
    // units' loads are in flight (below); a row past the end reads the clamped row
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                       (int64_t)hq * p.q_stride_head + 16 * grp;
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      const bool ok = D == DP || 64 * c + 16 * grp < D;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qraw[2 * c + hf] = ok ? *reinterpret_cast<const u32x4_t*>(qp + 64 * c + 8 * hf) : u32x4_t{0, 0, 0, 0};
    }
  } else {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                       (int64_t)hq * p.q_stride_head + 16 * grp;
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      const bf16x8_t z = {};
      const bool ok = rvalid && (D == DP || 64 * c + 16 * grp < D);
      qr.q[2 * c] = ok ? *reinterpret_cast<const bf16x8_t*>(qp + 64 * c) : z;
      qr.q[2 * c + 1] = ok ? *reinterpret_cast<const bf16x8_t*>(qp + 64 * c + 8) : z;
    }
  }
  float cs = cscale;   // per lane for split Q: the row's 2^-e folds into the logit scale
  if constexpr (SPLIT) {
    // the row's largest magnitude (its 4 lane groups hold its head dim), then the split
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 2 * S::KCH; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        amax = fmaxf(amax, fabsf(__uint_as_float(qraw[i][k] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(qraw[i][k] & 0xffff0000u)));
      }
    }
    amax = max_over_groups(amax);
    const int e = split_exponent(amax);
    const float up = __uint_as_float((uint32_t)(127 + e) << 23);
    cs = cscale * __uint_as_float((uint32_t)(127 - e) << 23);
#pragma unroll
    for (int i = 0; i < 2 * S::KCH; ++i) split8_bf16_e4m3(qraw[i], up, qr.q[i], qlo[i]);
  }
  f32x4_t oacc[S::NT];
#pragma unroll
  for (int t = 0; t < S::NT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const uint8_t* kbase = p.k_cache + (int64_t)h * p.kv_stride_head;
  const uint8_t* vbase = p.v_cache + (int64_t)h * p.kv_stride_head;
  const int64_t sT = p.kv_stride_tok, sP = p.kv_stride_page;
  auto page_of = [&](int u) __attribute__((always_inline)) -> int {
    const int pi = (u * 16) / ps;
    if (pi - pg_base >= 64) {   // wave-uniform; only splits longer than 64 pages get here
      pg_base = pi;
      pg_vec = bt[min(pi + lane, pg_last)];
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    return __builtin_amdgcn_readlane(pg_vec, pi - pg_base);
  };

  // (head dim 96 in the 128 layout: this lane's K bytes, and its V columns, lie in the head)
  const bool k_ok = !S::KROW || k_col<DP>(0, lane) < D;
  const bool v_ok = col * S::CW < D;
  const UnitOffsets<DP> uoff = unit_offsets<DP>(sT, lane);
  // Loads past the split's last unit keep the number of loads per trip fixed, so that the
  // compiler waits for exactly the oldest unit.  They read the last unit's first 16 bytes in every
  // lane: one cache line, which costs next to nothing and lands quickly at the end of the stream.
  const int ulast = su1 - 1;
  auto issue = [&](UnitRegs<DP>& ur, int u) __attribute__((always_inline)) {
    const bool trailing = u > ulast;
    const int uc = trailing ? ulast : u;
    const int64_t unit = page_of(uc) * sP + (int64_t)((uc * 16) % ps) * sT;
    // the unit's keys below L (at least one: uc * 16 <= p_last < L)
    const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(16, L - uc * 16))) * (uint32_t)sT;
    UnitOffsets<DP> o = uoff;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = trailing ? 0u : o.v[i];
    load_unit<DP, D, T::NT || (BAL && DP == 512)>(ur, unit_rsrc(kbase + unit, nrec), unit_rsrc(vbase + unit, nrec), o, k_ok, v_ok,
                            trailing);
  };

  // S^T tile of a unit: rows = its 16 keys, columns = the 16 query rows
  auto qk = [&](const u32x4_t (&kk)[S::KCH]) __attribute__((always_inline)) -> f32x4_t {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
    int qoff = lane;
    if constexpr (QLDS) asm volatile("" : "+v"(qoff));   // (read Q from LDS for every unit)
    if constexpr (SPLIT) {   // the split accumulation: K hi + (K lo) / 16
      f32x4_t slo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < S::KCH; ++c) {
        const uint64_t k0 = (uint64_t)kk[c][0] | ((uint64_t)kk[c][1] << 32);
        const uint64_t k1 = (uint64_t)kk[c][2] | ((uint64_t)kk[c][3] << 32);
        uint64_t h0 = qr.q[2 * c], h1 = qr.q[2 * c + 1], l0 = qlo[2 * c], l1 = qlo[2 * c + 1];
        if constexpr (QLDS) {
          h0 = *reinterpret_cast<const uint64_t*>(sm_q + ((2 * c) * 64 + qoff) * 8);
          h1 = *reinterpret_cast<const uint64_t*>(sm_q + ((2 * c + 1) * 64 + qoff) * 8);
          l0 = *reinterpret_cast<const uint64_t*>(sm_q + 8192 + ((2 * c) * 64 + qoff) * 8);
          l1 = *reinterpret_cast<const uint64_t*>(sm_q + 8192 + ((2 * c + 1) * 64 + qoff) * 8);
        }
        sacc = mfma_fp8_16x16x32(k0, h0, sacc);
        slo = mfma_fp8_16x16x32(k0, l0, slo);
        sacc = mfma_fp8_16x16x32(k1, h1, sacc);
        slo = mfma_fp8_16x16x32(k1, l1, slo);
      }
      return sacc + slo * 0.0625f;
    }
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      if constexpr (QFP8) {
        const uint64_t k0 = (uint64_t)kk[c][0] | ((uint64_t)kk[c][1] << 32);
        const uint64_t k1 = (uint64_t)kk[c][2] | ((uint64_t)kk[c][3] << 32);
        sacc = mfma_fp8_16x16x32(k0, qr.q[2 * c], sacc);
        sacc = mfma_fp8_16x16x32(k1, qr.q[2 * c + 1], sacc);
      } else {
        bf16x8_t q0 = qr.q[2 * c], q1 = qr.q[2 * c + 1];
        if constexpr (QLDS) {
          q0 = *reinterpret_cast<const bf16x8_t*>(sm_q + ((2 * c) * 64 + qoff) * 16);
          q1 = *reinterpret_cast<const bf16x8_t*>(sm_q + ((2 * c + 1) * 64 + qoff) * 16);
        }
        sacc = mfma_bf16_16x16x32(e4m3x8_to_bf16(kk[c][0], kk[c][1]), q0, sacc);
        sacc = mfma_bf16_16x16x32(e4m3x8_to_bf16(kk[c][2], kk[c][3]), q1, sacc);
      }
    }
    return sacc;
  };

  // mask, online softmax update, P^T operand of unit u (lane (row, g) holds keys 4g..4g+3)
  // split Q also runs PV on the FP8 MFMA, with P <= 2^4 (see compute); the other modes keep
  // P <= 2^8
  constexpr float kLazy = SPLIT ? 4.0f : kLazyMax;
  auto softmax = [&](const f32x4_t sacc, int u) __attribute__((always_inline)) -> f32x4_t {
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = sacc[i] * cs;
    const int j0 = u * 16;
    if (!(j0 >= full_lo && j0 + 15 <= p_first)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * grp + i;
        const bool vis = j <= pos && (W < 1 || j > pos - W);
        sv[i] = vis ? sv[i] : kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = max_over_groups(mx);
    // Lazy running max: it moves only when a unit exceeds it by more than 2^8, so P <= 256 and
    // the O rescale (64 accumulators) is rare after the first unit.  A row whose max is still
    // -inf has O = 0 and l = 0, so its first move needs no rescale of O.
    const bool grow = mx > m_run + kLazy;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));   // 1 where not grown
      l_run *= alpha;
      if (__any(grow && m_run != kNegInf)) {
#pragma unroll
        for (int t = 0; t < S::NT; ++t) oacc[t] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[i] - m_use);
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    return f32x4_t{pv[0], pv[1], pv[2], pv[3]};
  };

  // O^T += V^T * P^T with V in registers (lane (col, g) holds bytes col*CW.. of keys 4g..4g+3):
  // a 4x4 byte transpose gives, per O^T tile t, row col <-> d = 16 col + t (d256) or the
  // analogous interleave (d64, d512)
  //
  // Split Q runs PV on the FP8 MFMA too, at the precision of bf16 P: each P (<= 2^4) is written
  // as 16 hi + lo with hi = E4M3(P) and lo = E4M3(16 (P - hi)); 16 hi is exact and at most 256.
  // One 16x16x32 MFMA per O^T tile takes the lane's 4 keys twice, 16 hi in byte slots 0-3 and
  // lo in slots 4-7, against the same 4 V bytes in both halves of the A operand, so it
  // accumulates 16 O; the 1/16 goes into the final 1/l.
  // the wave's K tile: the first bytes of its O slot in the merge buffer, which it writes only
  // after the barrier that ends every wave's stream
  uint8_t* ktile = reinterpret_cast<uint8_t*>(&sm_o[wave][0][0]);
  static_assert(sizeof(sm_o[0]) >= 16 * S::KTS, "K tile");
  auto compute = [&](const UnitRegs<DP>& ur, int u) __attribute__((always_inline)) {
    u32x4_t kk[S::KCH];
    k_operands<DP>(ur.k, kk, ktile, lane);
    const f32x4_t pf = softmax(qk(kk), u);
    uint64_t p8 = 0;
    bf16x4_t pb = {};
    if constexpr (SPLIT) {
      int hc = __builtin_amdgcn_cvt_pk_fp8_f32(pf[0], pf[1], 0, false);
      hc = __builtin_amdgcn_cvt_pk_fp8_f32(pf[2], pf[3], hc, true);
      const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hc, false);
      const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hc, true);
      int h16 = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * h01[0], 16.0f * h01[1], 0, false);
      h16 = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * h23[0], 16.0f * h23[1], h16, true);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (pf[0] - h01[0]), 16.0f * (pf[1] - h01[1]), 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (pf[2] - h23[0]), 16.0f * (pf[3] - h23[1]), lo, true);
      p8 = (uint64_t)(uint32_t)h16 | ((uint64_t)(uint32_t)lo << 32);
    } else {
      pb = bf16x4_t{(__bf16)pf[0], (__bf16)pf[1], (__bf16)pf[2], (__bf16)pf[3]};
    }
#pragma unroll
    for (int blk = 0; blk < S::VBLK; ++blk) {
#pragma unroll
      for (int w = 0; w < S::CW / 4; ++w) {
        uint32_t tr[4];
        transpose4x4_u8(ur.v[0][blk][w], ur.v[1][blk][w], ur.v[2][blk][w], ur.v[3][blk][w],
                        tr[0], tr[1], tr[2], tr[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = blk * S::CW + 4 * w + e;
          if constexpr (SPLIT)
            oacc[t] = mfma_fp8_16x16x32((uint64_t)tr[e] | ((uint64_t)tr[e] << 32), p8, oacc[t]);
          else
            oacc[t] = mfma_bf16_16x16x16(e4m3x4_to_bf16(tr[e]), pb, oacc[t]);
        }
      }
    }
  };

  // ---- main loop: this wave takes units su0+wave, su0+wave+4, ... --------------------------
  const int u0 = su0 + wave;
  {
    // A ring of NBUF register buffers: NBUF - 1 units stay in flight while one is computed.
    // Every trip issues the same loads (see issue), so the compiler can wait for exactly the
    // oldest unit instead of draining every outstanding load.
    UnitRegs<DP> buf[NBUF];
#pragma unroll
    for (int k = 0; k < NBUF; ++k) issue(buf[k], u0 + 4 * k);
    if constexpr (QLDS) {
      // wave 0 writes the Q^T operand image (the same in every wave); the previous tile of this
      // block finished reading its image before the barrier that ended that tile
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 2 * S::KCH; ++i) {
          if constexpr (SPLIT) {
            *reinterpret_cast<uint64_t*>(sm_q + (i * 64 + lane) * 8) = qr.q[i];
            *reinterpret_cast<uint64_t*>(sm_q + 8192 + (i * 64 + lane) * 8) = qlo[i];
          } else {
            *reinterpret_cast<bf16x8_t*>(sm_q + (i * 64 + lane) * 16) = qr.q[i];
          }
        }
      }
      __syncthreads();
    }
    if constexpr (QM == kQBf16E4M3) {
      // quantize bf16 Q with the arithmetic of the stand-alone quantize call (identical codes)
      const double rcp = 1.0 / (double)qd;
#pragma unroll
      for (int i = 0; i < 2 * S::KCH; ++i) {
        const u32x2_t e = quantize8_bf16_e4m3(qraw[i], rcp);
        qr.q[i] = rvalid ? ((uint64_t)e[0] | ((uint64_t)e[1] << 32)) : 0;
      }
    }
    for (int u = u0; u < su1; u += 4 * NBUF) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        const int uk = u + 4 * k;
        if (uk < su1) compute(buf[k], uk);
#ifdef FP8ATTN_TIMELINE
        if (!BAL && k == 0 && u == u0) tl_mark(1 + wave, __builtin_amdgcn_s_memtime());
#endif
        issue(buf[k], uk + 4 * NBUF);
      }
    }
  }
#ifdef FP8ATTN_TIMELINE
  if (!BAL) tl_mark(5 + wave, __builtin_amdgcn_s_memtime());
#endif
  l_run = sum_over_groups(l_run);

  // ---- merge the 4 waves through LDS --------------------------------------------------------
  if (grp == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_run;
  }
  __syncthreads();
  {
    float M = fmaxf(fmaxf(sm_m[0][col], sm_m[1][col]), fmaxf(sm_m[2][col], sm_m[3][col]));
    const float sc = M == kNegInf ? 0.f : fast_exp2(m_run - M);
    float* orow = &sm_o[wave][col][0];
#pragma unroll
    for (int blk = 0; blk < S::VBLK; ++blk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e4 = 0; e4 < S::CW / 4; ++e4) {
          const int t = blk * S::CW + 4 * e4;
          const f32x4_t v = {oacc[t][i] * sc, oacc[t + 1][i] * sc, oacc[t + 2][i] * sc, oacc[t + 3][i] * sc};
          *reinterpret_cast<f32x4_t*>(orow + blk * 16 * S::CW + (4 * grp + i) * S::CW + 4 * e4) = v;
        }
      }
    }
  }
  __syncthreads();
#ifdef FP8ATTN_TIMELINE
  if (!BAL && wave == 0) tl_mark(9, __builtin_amdgcn_s_memtime());
#endif

  // ---- final: thread -> (row, d-part) -------------------------------------------------------
  {
    const int row = threadIdx.x & 15;
    const int part = threadIdx.x >> 4;                 // 16 parts of DP/16 values
    constexpr int PW = DP / 16;
    const int rr = row0 + row;
    if (rr < nrows && part * PW < D) {                 // (parts past a padded head dim write nothing)
      float mw[4], M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) { mw[w] = sm_m[w][row]; M = fmaxf(M, mw[w]); }
      float Ls = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < 4; ++w) Ls += sm_l[w][row] * fast_exp2(mw[w] - M);
      }
      const int tk = t0 + rr / G;
      const int hh = h * G + rr % G;
      const float inv = Ls > 0.f ? vd / (SPLIT ? 16.0f * Ls : Ls) : 0.f;   // (split Q accumulates 16 O)
      const float lse2 = Ls > 0.f ? (M + fast_log2(Ls)) : kNegInf;
      if (whole) {
        __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)tk * p.out_stride_tok +
                     (int64_t)hh * p.out_stride_head + part * PW;
#pragma unroll
        for (int c = 0; c < PW; c += 4) {
          f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sm_o[0][row][part * PW + c]);
#pragma unroll
          for (int w = 1; w < 4; ++w) a += *reinterpret_cast<const f32x4_t*>(&sm_o[w][row][part * PW + c]);
          a *= inv;
          const bf16x4_t o = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
          *reinterpret_cast<bf16x4_t*>(op + c) = o;
        }
        if (p.lse && part == 0) p.lse[(int64_t)tk * p.hq + hh] = lse2 * kLn2;
      } else {
        // split: [split, token, q head]; balanced partition: [slot, tile row]
        const int64_t e = BAL ? (int64_t)pidx * 16 + row : ((int64_t)pidx * p.total_q + tk) * p.hq + hh;
        float* op = p.part_o + e * D + part * PW;
#pragma unroll
        for (int c = 0; c < PW; c += 4) {
          f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sm_o[0][row][part * PW + c]);
#pragma unroll
          for (int w = 1; w < 4; ++w) a += *reinterpret_cast<const f32x4_t*>(&sm_o[w][row][part * PW + c]);
          *reinterpret_cast<f32x4_t*>(op + c) = a * inv;
        }
        if (part == 0) p.part_lse[e] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
      }
    }
  }
#ifdef FP8ATTN_TIMELINE
  if (!BAL && wave == 0) {
    tl_mark(10, __builtin_amdgcn_s_memtime());
    tl_mark(14, __builtin_amdgcn_s_memrealtime());
  }
#endif
  // a block of the balanced partition runs several tiles in turn: the next tile's merge must not
  // overwrite the LDS this one is still reading
  if constexpr (BAL) __syncthreads();
}

// Split grid: one block per (kv head, split, sequence, row tile), XCD-aware order.
template <int QM, int D>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(DecodeTune<QM != kQBf16, D>::MIN_WAVES))) decode_kernel(const AttnParams p) {
  // (32-bit index arithmetic: the host keeps the grid below 2^31)
  uint32_t id = xcd_remap32(blockIdx.x, gridDim.x);
  const uint32_t n_rt = (uint32_t)p.row_groups, n_b = (uint32_t)p.batch, n_s = (uint32_t)p.num_splits;
  const int rt = (int)(id % n_rt); id /= n_rt;
  const int b = (int)(id % n_b); id /= n_b;
  const int s = (int)(id % n_s);
  const int h = (int)(id / n_s);
  const int o0 = s * p.units_per_split;
  decode_tile<QM, D, false>(p, b, h, rt, o0, o0 + p.units_per_split, s, p.num_splits == 1);
}

// ---- 32-row tiles ------------------------------------------------------------------------------
// A tile of 32 rows, two 16-row halves (the MFMA's column count), for decode steps with more than
// 16 rows per (sequence, kv head) such as speculative-decode verification (GQA 8 x 4 query tokens):
// every K/V unit is loaded, and for BF16 Q dequantized, once for both halves instead of once per
// 16-row tile, which halves the K/V stream of such steps.  The four waves split the key range as in
// decode_tile, with the same mask, softmax, PV and merge.  Q lives in LDS as the image of the MFMA
// B operands, written once by waves 0 and 1 before the loop; the registers it frees hold the second
// half's O accumulators.  Head dims up to 256 (at 512 the two halves' accumulators alone take a
// wave's 256 accumulation registers).
template <int QM, int D>
__device__ __forceinline__ void decode_tile32(const AttnParams& p, const int b, const int h, const int rt,
                                              const int o0, const int o1, const int pidx, const bool whole) {
  constexpr bool QFP8 = QM != kQBf16;   // QK^T on the FP8 MFMA
  constexpr bool SPLIT = QM == kQBf16Split;
  constexpr int DP = D == 96 ? 128 : D;
  using S = DecodeShape<DP>;
  using T = DecodeTune<QFP8, DP>;
  constexpr int NBUF = T::NBUF;
  constexpr int NQ = 2 * S::KCH;                      // B operands per half (16 d values each)
  constexpr int QB = QFP8 ? 8 : 16;                   // bytes of one lane's operand
  constexpr int QIMG = 2 * NQ * 64 * QB;              // image [half][operand][lane] (split Q: hi)
  constexpr int QLDS = SPLIT ? 2 * QIMG : QIMG;       // (split Q: the lo image follows)
  constexpr int MERGE = 4 * 16 * S::RS * 4;           // one half's O of the 4 waves, fp32
  constexpr int KT = QLDS + 4 * 16 * S::KTS;         // Q image, then the 4 waves' K tiles
  __shared__ __attribute__((aligned(16))) uint8_t smem[KT > MERGE ? KT : MERGE];
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  __shared__ float sm_cs[32];
  float (*sm_o)[16][S::RS] = reinterpret_cast<float (*)[16][S::RS]>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.group;

  // per-item scalars, requested together (see decode_tile)
  const int64_t dsi = (int64_t)b * p.ds_stride_b + (int64_t)h * p.ds_stride_h;
  const int t0 = load_uniform(p.cu_seqlens_q, b);
  const int t1 = load_uniform(p.cu_seqlens_q, b + 1);
  const int L = load_uniform(p.seqlens_k, b);
  const float* stand_in = reinterpret_cast<const float*>(p.seqlens_k);
  const float kd_raw = load_uniform(p.k_descale ? p.k_descale : stand_in, p.k_descale ? dsi : 0);
  const float vd_raw = load_uniform(p.v_descale ? p.v_descale : stand_in, p.v_descale ? dsi : 0);
  const float qd_raw = load_uniform(p.q_descale ? p.q_descale : stand_in, 0);
  asm volatile("" ::"s"(t0), "s"(t1), "s"(L), "s"(kd_raw), "s"(vd_raw), "s"(qd_raw));
  const int ql = t1 - t0;
  const int nrows = ql * G;
  const int row0 = rt * 32;
  if (row0 >= nrows) return;
  const int rlast = min(row0 + 32, nrows) - 1;
  const int p_first = L - ql + row0 / G;
  const int p_last = L - ql + rlast / G;
  const int W = p.window;
  const int k_lo = W >= 1 ? max(0, p_first - W + 1) : 0;
  const int u_begin = k_lo / 16;
  const int u_end = (p_last + 16) / 16;
  const int su0 = u_begin + o0;
  const int su1 = min(u_end, u_begin + o1);
  const int full_lo = W >= 1 ? p_last - W + 1 : 0;   // keys [full_lo, p_first] are seen by every row

  // this lane's row in each half
  int tok[2], hqr[2], pos[2];
  bool rvalid[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = row0 + 16 * hh + col;
    rvalid[hh] = r < nrows;
    tok[hh] = (rvalid[hh] ? r : rlast) / G;
    hqr[hh] = h * G + (rvalid[hh] ? r : rlast) % G;
    pos[hh] = L - ql + tok[hh];
  }

  if (su0 >= su1) {  // nothing visible in this split: neutral partial for the combine
    if (!whole && threadIdx.x < 32) {
      const int r = row0 + (int)threadIdx.x;
      if (r < nrows) p.part_lse[((int64_t)pidx * p.total_q + t0 + r / G) * p.hq + h * G + r % G] = kNegInf;
    }
    return;
  }

  const float kd = p.k_descale ? kd_raw : 1.0f;
  const float vd = p.v_descale ? vd_raw : 1.0f;
  const float qd = QFP8 && p.q_descale ? qd_raw : 1.0f;
  const float cscale = p.scale_log2 * kd * qd;

  // page ids of the split's keys, one per lane (see decode_tile)
  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const int ps = p.page_size;
  const int pg_last = ((su1 - 1) * 16) / ps;
  int pg_base = (su0 * 16) / ps;
  int pg_vec = bt[min(pg_base + lane, pg_last)];

  const uint8_t* kbase = p.k_cache + (int64_t)h * p.kv_stride_head;
  const uint8_t* vbase = p.v_cache + (int64_t)h * p.kv_stride_head;
  const int64_t sT = p.kv_stride_tok, sP = p.kv_stride_page;
  auto page_of = [&](int u) __attribute__((always_inline)) -> int {
    const int pi = (u * 16) / ps;
    if (pi - pg_base >= 64) {
      pg_base = pi;
      pg_vec = bt[min(pi + lane, pg_last)];
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    return __builtin_amdgcn_readlane(pg_vec, pi - pg_base);
  };
  const bool k_ok = !S::KROW || k_col<DP>(0, lane) < D;
  const bool v_ok = col * S::CW < D;
  const UnitOffsets<DP> uoff = unit_offsets<DP>(sT, lane);
  const int ulast = su1 - 1;
  auto issue = [&](UnitRegs<DP>& ur, int u) __attribute__((always_inline)) {
    const bool trailing = u > ulast;
    const int uc = trailing ? ulast : u;
    const int64_t unit = page_of(uc) * sP + (int64_t)((uc * 16) % ps) * sT;
    const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(16, L - uc * 16))) * (uint32_t)sT;
    UnitOffsets<DP> o = uoff;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = trailing ? 0u : o.v[i];
    load_unit<DP, D, T::NT>(ur, unit_rsrc(kbase + unit, nrec), unit_rsrc(vbase + unit, nrec), o, k_ok, v_ok,
                            trailing);
  };

  // the first units' loads go out before Q is staged, so their latencies overlap
  const int u0 = su0 + wave;
  UnitRegs<DP> buf[NBUF];
#pragma unroll
  for (int k = 0; k < NBUF; ++k) issue(buf[k], u0 + 4 * k);

  // ---- Q: wave hh (0 or 1) writes the B-operand image of half hh ------------------------------
  // Operand i of half hh, lane l: row 16 hh + l % 16, d values 64 (i / 2) + 16 (l / 16) + 8 (i % 2)
  // .. + 7 (the layout of decode_tile's Q registers), at byte ((hh NQ + i) 64 + l) QB.
  if (wave < 2) {
    const int hh = wave;
    const int64_t qrow = (int64_t)(t0 + tok[hh]) * p.q_stride_tok + (int64_t)hqr[hh] * p.q_stride_head + 16 * grp;
    uint8_t* img = smem + (size_t)(hh * NQ * 64 + lane) * QB;
    if constexpr (QM == kQE4M3) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + qrow;
#pragma unroll
      for (int c = 0; c < S::KCH; ++c) {
        const bool ok = rvalid[hh] && (D == DP || 64 * c + 16 * grp < D);
        const u32x4_t w = ok ? *reinterpret_cast<const u32x4_t*>(qp + 64 * c) : u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<uint64_t*>(img + (2 * c) * 64 * QB) = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
        *reinterpret_cast<uint64_t*>(img + (2 * c + 1) * 64 * QB) = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
      }
    } else if constexpr (QM == kQBf16) {
      const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + qrow;
#pragma unroll
      for (int c = 0; c < S::KCH; ++c) {
        const bool ok = rvalid[hh] && (D == DP || 64 * c + 16 * grp < D);
        const bf16x8_t z = {};
        *reinterpret_cast<bf16x8_t*>(img + (2 * c) * 64 * QB) = ok ? *reinterpret_cast<const bf16x8_t*>(qp + 64 * c) : z;
        *reinterpret_cast<bf16x8_t*>(img + (2 * c + 1) * 64 * QB) =
            ok ? *reinterpret_cast<const bf16x8_t*>(qp + 64 * c + 8) : z;
      }
    } else {
      // bf16 Q, quantized (BF16_TO_E4M3) or split into two E4M3 terms (split Q); a row past the
      // end reads the clamped row
      const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + qrow;
      u32x4_t qraw[NQ];
#pragma unroll
      for (int c = 0; c < S::KCH; ++c) {
        const bool ok = D == DP || 64 * c + 16 * grp < D;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          qraw[2 * c + hf] = ok ? *reinterpret_cast<const u32x4_t*>(qp + 64 * c + 8 * hf) : u32x4_t{0, 0, 0, 0};
      }
      if constexpr (QM == kQBf16E4M3) {
        const double rcp = 1.0 / (double)qd;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const u32x2_t e = quantize8_bf16_e4m3(qraw[i], rcp);
          *reinterpret_cast<uint64_t*>(img + i * 64 * QB) = rvalid[hh] ? ((uint64_t)e[0] | ((uint64_t)e[1] << 32)) : 0;
        }
      } else {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            amax = fmaxf(amax, fabsf(__uint_as_float(qraw[i][k] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(qraw[i][k] & 0xffff0000u)));
          }
        }
        amax = max_over_groups(amax);
        const int e = split_exponent(amax);
        const float up = __uint_as_float((uint32_t)(127 + e) << 23);
        if (grp == 0) sm_cs[16 * hh + col] = cscale * __uint_as_float((uint32_t)(127 - e) << 23);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          uint64_t hi, lo;
          split8_bf16_e4m3(qraw[i], up, hi, lo);
          *reinterpret_cast<uint64_t*>(img + i * 64 * QB) = hi;
          *reinterpret_cast<uint64_t*>(img + QIMG + i * 64 * QB) = lo;
        }
      }
    }
  }
  __syncthreads();
  float cs[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) cs[hh] = SPLIT ? sm_cs[16 * hh + col] : cscale;
  auto qop8 = [&](int hh, int i, bool lo) __attribute__((always_inline)) -> uint64_t {
    return *reinterpret_cast<const uint64_t*>(smem + (lo ? QIMG : 0) + (size_t)((hh * NQ + i) * 64 + lane) * QB);
  };
  auto qop16 = [&](int hh, int i) __attribute__((always_inline)) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(smem + (size_t)((hh * NQ + i) * 64 + lane) * QB);
  };

  f32x4_t oacc[2][S::NT];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int t = 0; t < S::NT; ++t) oacc[hh][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};

  // S^T tiles of a unit for both halves: rows = its 16 keys, columns = 16 query rows each
  auto qk = [&](const u32x4_t (&kk)[S::KCH], f32x4_t (&sacc)[2]) __attribute__((always_inline)) {
    f32x4_t slo[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) sacc[hh] = slo[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      if constexpr (QFP8) {
        const uint64_t k0 = (uint64_t)kk[c][0] | ((uint64_t)kk[c][1] << 32);
        const uint64_t k1 = (uint64_t)kk[c][2] | ((uint64_t)kk[c][3] << 32);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          sacc[hh] = mfma_fp8_16x16x32(k0, qop8(hh, 2 * c, false), sacc[hh]);
          sacc[hh] = mfma_fp8_16x16x32(k1, qop8(hh, 2 * c + 1, false), sacc[hh]);
          if constexpr (SPLIT) {   // the split accumulation: K hi + (K lo) / 16
            slo[hh] = mfma_fp8_16x16x32(k0, qop8(hh, 2 * c, true), slo[hh]);
            slo[hh] = mfma_fp8_16x16x32(k1, qop8(hh, 2 * c + 1, true), slo[hh]);
          }
        }
      } else {
        const bf16x8_t kb0 = e4m3x8_to_bf16(kk[c][0], kk[c][1]);
        const bf16x8_t kb1 = e4m3x8_to_bf16(kk[c][2], kk[c][3]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          sacc[hh] = mfma_bf16_16x16x32(kb0, qop16(hh, 2 * c), sacc[hh]);
          sacc[hh] = mfma_bf16_16x16x32(kb1, qop16(hh, 2 * c + 1), sacc[hh]);
        }
      }
    }
    if constexpr (SPLIT) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) sacc[hh] += slo[hh] * 0.0625f;
    }
  };

  // mask, online softmax update and P^T operand of half hh (as in decode_tile)
  constexpr float kLazy = SPLIT ? 4.0f : kLazyMax;
  auto softmax = [&](const f32x4_t sacc, int u, int hh) __attribute__((always_inline)) -> f32x4_t {
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = sacc[i] * cs[hh];
    const int j0 = u * 16;
    if (!(j0 >= full_lo && j0 + 15 <= p_first)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * grp + i;
        const bool vis = j <= pos[hh] && (W < 1 || j > pos[hh] - W);
        sv[i] = vis ? sv[i] : kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = max_over_groups(mx);
    const bool grow = mx > m_run[hh] + kLazy;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run[hh];
      const float alpha = fast_exp2(m_run[hh] - (m_new == kNegInf ? 0.f : m_new));
      l_run[hh] *= alpha;
      if (__any(grow && m_run[hh] != kNegInf)) {
#pragma unroll
        for (int t = 0; t < S::NT; ++t) oacc[hh][t] *= alpha;
      }
      m_run[hh] = m_new;
    }
    const float m_use = m_run[hh] == kNegInf ? 0.f : m_run[hh];
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[i] - m_use);
    l_run[hh] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    return f32x4_t{pv[0], pv[1], pv[2], pv[3]};
  };

  // O^T += V^T * P^T for both halves; the V^T operands (byte transpose, dequant) are made once
  uint8_t* ktile = smem + QLDS + wave * 16 * S::KTS;   // the wave's K tile, after the Q image
  auto compute = [&](const UnitRegs<DP>& ur, int u) __attribute__((always_inline)) {
    f32x4_t sacc[2];
    u32x4_t kk[S::KCH];
    k_operands<DP>(ur.k, kk, ktile, lane);
    qk(kk, sacc);
    uint64_t p8[2] = {0, 0};
    bf16x4_t pb[2] = {};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const f32x4_t pf = softmax(sacc[hh], u, hh);
      if constexpr (SPLIT) {
        int hc = __builtin_amdgcn_cvt_pk_fp8_f32(pf[0], pf[1], 0, false);
        hc = __builtin_amdgcn_cvt_pk_fp8_f32(pf[2], pf[3], hc, true);
        const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hc, false);
        const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hc, true);
        int h16 = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * h01[0], 16.0f * h01[1], 0, false);
        h16 = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * h23[0], 16.0f * h23[1], h16, true);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (pf[0] - h01[0]), 16.0f * (pf[1] - h01[1]), 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (pf[2] - h23[0]), 16.0f * (pf[3] - h23[1]), lo, true);
        p8[hh] = (uint64_t)(uint32_t)h16 | ((uint64_t)(uint32_t)lo << 32);
      } else {
        pb[hh] = bf16x4_t{(__bf16)pf[0], (__bf16)pf[1], (__bf16)pf[2], (__bf16)pf[3]};
      }
    }
#pragma unroll
    for (int blk = 0; blk < S::VBLK; ++blk) {
#pragma unroll
      for (int w = 0; w < S::CW / 4; ++w) {
        uint32_t tr[4];
        transpose4x4_u8(ur.v[0][blk][w], ur.v[1][blk][w], ur.v[2][blk][w], ur.v[3][blk][w],
                        tr[0], tr[1], tr[2], tr[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = blk * S::CW + 4 * w + e;
          if constexpr (SPLIT) {
            const uint64_t a = (uint64_t)tr[e] | ((uint64_t)tr[e] << 32);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) oacc[hh][t] = mfma_fp8_16x16x32(a, p8[hh], oacc[hh][t]);
          } else {
            const bf16x4_t a = e4m3x4_to_bf16(tr[e]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) oacc[hh][t] = mfma_bf16_16x16x16(a, pb[hh], oacc[hh][t]);
          }
        }
      }
    }
  };

  // ---- main loop: this wave takes units su0+wave, su0+wave+4, ... --------------------------
  for (int u = u0; u < su1; u += 4 * NBUF) {
#pragma unroll
    for (int k = 0; k < NBUF; ++k) {
      const int uk = u + 4 * k;
      if (uk < su1) compute(buf[k], uk);
      issue(buf[k], uk + 4 * NBUF);
    }
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) l_run[hh] = sum_over_groups(l_run[hh]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the trailing loads land before the block ends
  __syncthreads();                            // every wave is done with the Q image

  // ---- merge the 4 waves through LDS, one half at a time ------------------------------------
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (grp == 0) {
      sm_m[wave][col] = m_run[hh];
      sm_l[wave][col] = l_run[hh];
    }
    __syncthreads();
    {
      const float M = fmaxf(fmaxf(sm_m[0][col], sm_m[1][col]), fmaxf(sm_m[2][col], sm_m[3][col]));
      const float sc = M == kNegInf ? 0.f : fast_exp2(m_run[hh] - M);
      float* orow = &sm_o[wave][col][0];
#pragma unroll
      for (int blk = 0; blk < S::VBLK; ++blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int e4 = 0; e4 < S::CW / 4; ++e4) {
            const int t = blk * S::CW + 4 * e4;
            const f32x4_t v = {oacc[hh][t][i] * sc, oacc[hh][t + 1][i] * sc, oacc[hh][t + 2][i] * sc,
                               oacc[hh][t + 3][i] * sc};
            *reinterpret_cast<f32x4_t*>(orow + blk * 16 * S::CW + (4 * grp + i) * S::CW + 4 * e4) = v;
          }
        }
      }
    }
    __syncthreads();
    {
      const int row = threadIdx.x & 15;
      const int part = threadIdx.x >> 4;
      constexpr int PW = DP / 16;
      const int rr = row0 + 16 * hh + row;
      if (rr < nrows && part * PW < D) {
        float mw[4], M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) { mw[w] = sm_m[w][row]; M = fmaxf(M, mw[w]); }
        float Ls = 0.f;
        if (M != kNegInf) {
#pragma unroll
          for (int w = 0; w < 4; ++w) Ls += sm_l[w][row] * fast_exp2(mw[w] - M);
        }
        const int tk = t0 + rr / G;
        const int hq = h * G + rr % G;
        const float inv = Ls > 0.f ? vd / (SPLIT ? 16.0f * Ls : Ls) : 0.f;   // (split Q accumulates 16 O)
        const float lse2 = Ls > 0.f ? (M + fast_log2(Ls)) : kNegInf;
        if (whole) {
          __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)tk * p.out_stride_tok +
                       (int64_t)hq * p.out_stride_head + part * PW;
#pragma unroll
          for (int c = 0; c < PW; c += 4) {
            f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sm_o[0][row][part * PW + c]);
#pragma unroll
            for (int w = 1; w < 4; ++w) a += *reinterpret_cast<const f32x4_t*>(&sm_o[w][row][part * PW + c]);
            a *= inv;
            const bf16x4_t o = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
            *reinterpret_cast<bf16x4_t*>(op + c) = o;
          }
          if (p.lse && part == 0) p.lse[(int64_t)tk * p.hq + hq] = lse2 * kLn2;
        } else {
          const int64_t e = ((int64_t)pidx * p.total_q + tk) * p.hq + hq;   // [split, token, q head]
          float* op = p.part_o + e * D + part * PW;
#pragma unroll
          for (int c = 0; c < PW; c += 4) {
            f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sm_o[0][row][part * PW + c]);
#pragma unroll
            for (int w = 1; w < 4; ++w) a += *reinterpret_cast<const f32x4_t*>(&sm_o[w][row][part * PW + c]);
            *reinterpret_cast<f32x4_t*>(op + c) = a * inv;
          }
          if (part == 0) p.part_lse[e] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
        }
      }
    }
    __syncthreads();   // the next half reuses the merge buffers
  }
}

// Split grid over 32-row tiles (row_groups counts 32-row tiles here)
template <int QM, int D>
__global__ void __launch_bounds__(256) decode32_kernel(const AttnParams p) {
  uint32_t id = xcd_remap32(blockIdx.x, gridDim.x);
  const uint32_t n_rt = (uint32_t)p.row_groups, n_b = (uint32_t)p.batch, n_s = (uint32_t)p.num_splits;
  const int rt = (int)(id % n_rt); id /= n_rt;
  const int b = (int)(id % n_b); id /= n_b;
  const int s = (int)(id % n_s);
  const int h = (int)(id / n_s);
  const int o0 = s * p.units_per_split;
  decode_tile32<QM, D>(p, b, h, rt, o0, o0 + p.units_per_split, s, p.num_splits == 1);
}

// ---- balanced partition ----------------------------------------------------------------------
// The row tiles' visible 16-key units, laid end to end in (kv head, sequence, row tile) order,
// form one stream of T units; block i of R = min(grid, T) takes units [i T / R, (i + 1) T / R).
// Every block then streams the same number of units (within one), whatever the mix of sequence
// lengths, and each block pays one pipeline fill and drain instead of one per split.  A block's
// range cuts into tiles: a tile whose range lies inside one block is final there; a tile cut by
// block boundaries leaves one fp32 partial per block in slot (block + tile index), and records
// the first and last block of its range for the combine.  The unit counts come from the device
// lengths (every block recomputes them, a wave-wide prefix sum per 64 tiles), so the host plans
// from the grid size and the shapes alone.

// Units of row tile rt of sequence b: the range decode_tile walks for that tile.
__device__ __forceinline__ uint32_t tile_units(const AttnParams& p, int b, int rt) {
  const int t0 = p.cu_seqlens_q[b], t1 = p.cu_seqlens_q[b + 1], L = p.seqlens_k[b];
  const int ql = t1 - t0, nrows = ql * p.group, row0 = rt * 16;
  if (row0 >= nrows) return 0u;
  const int rlast = min(row0 + 16, nrows) - 1;
  const int p_first = L - ql + row0 / p.group, p_last = L - ql + rlast / p.group;
  const int k_lo = p.window >= 1 ? max(0, p_first - p.window + 1) : 0;
  return (uint32_t)max(0, (p_last + 16) / 16 - k_lo / 16);
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, (unsigned)o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// 64 consecutive row tiles (tile index j = sequence * row_groups + row tile), one per lane
struct TileChunk {
  int base;          // first tile of the chunk
  uint32_t acc;      // units of the tiles before the chunk (within one kv head)
  uint32_t n, incl;  // this lane's tile: units, inclusive prefix within the chunk
  uint32_t total;    // units of the chunk
};

__device__ __forceinline__ TileChunk load_chunk(const AttnParams& p, int base, uint32_t acc, int J) {
  TileChunk c;
  c.base = base;
  c.acc = acc;
  const int j = base + (int)(threadIdx.x & 63);
  c.n = j < J ? tile_units(p, j / p.row_groups, j % p.row_groups) : 0u;
  c.incl = wave_inclusive_sum(c.n);
  c.total = (uint32_t)__builtin_amdgcn_readlane((int)c.incl, 63);
  return c;
}

// Wave-uniform values computed on the vector ALU (64-bit division) are moved back to scalar
// registers, so that the loop state around a tile costs no vector registers.
__device__ __forceinline__ uint32_t to_sgpr(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ uint64_t to_sgpr(uint64_t x) {
  return (uint64_t)to_sgpr((uint32_t)x) | ((uint64_t)to_sgpr((uint32_t)(x >> 32)) << 32);
}

template <int QM, int D>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(DecodeTune<QM != kQBf16, D>::MIN_WAVES)))
    decode_balanced_kernel(const AttnParams p) {
  const uint32_t i = xcd_remap32(blockIdx.x, gridDim.x);
  const int J = p.batch * p.row_groups;          // row tiles per kv head
  uint32_t t_head = 0;
  for (int base = 0; base < J; base += 64) t_head += load_chunk(p, base, 0u, J).total;
  t_head = to_sgpr(t_head);
  const uint64_t T = (uint64_t)t_head * (uint32_t)p.hkv;
  // At most T parts, so that every part holds a unit and the blocks of a tile's range are
  // consecutive (the combine walks them from first to last); blocks past that have no work.
  const uint32_t R = (uint32_t)(T < gridDim.x ? T : gridDim.x);
  if (i >= R) return;
  const uint64_t start = to_sgpr((uint64_t)i * T / R), end = to_sgpr((uint64_t)(i + 1) * T / R);
  // Only the chunk's position stays live across a tile (its per-lane counts are loaded again for
  // the next segment), which keeps the tile's register budget.
  int c_base = 0;
  uint32_t c_acc = 0;
  for (uint64_t u = start; u < end;) {
    const int h = (int)to_sgpr((uint32_t)(u / t_head));
    const uint32_t rem = (uint32_t)(u - (uint64_t)h * t_head);
    if (rem < c_acc) c_base = 0, c_acc = 0;        // the next kv head starts over at tile 0
    TileChunk c = load_chunk(p, c_base, c_acc, J);
    while (rem >= c.acc + c.total && c.base + 64 < J) c = load_chunk(p, c.base + 64, c.acc + c.total, J);
    c_base = c.base;
    c_acc = c.acc;
    // the tile holding unit rem: the first lane whose inclusive prefix passes it
    const int idx = (int)__popcll(__ballot(c.acc + c.incl <= rem));
    const int j = c.base + idx;
    if (idx >= 64 || j >= J) break;   // (only if the lengths changed under the kernel)
    const uint32_t n_j = (uint32_t)__builtin_amdgcn_readlane((int)c.n, idx);
    const uint32_t u_j = c.acc + (uint32_t)__builtin_amdgcn_readlane((int)c.incl, idx) - n_j;
    const uint64_t lo = (uint64_t)h * t_head + u_j, hi = lo + n_j;
    const uint64_t seg_end = hi < end ? hi : end;
    if (seg_end <= u) break;
    const int o0 = (int)(u - lo), o1 = (int)(seg_end - lo);
    const int g = h * J + j;
    if (o0 == 0 && threadIdx.x == 0) {   // the tile's first segment: blocks of its first and last unit
      p.seg_meta[2 * g] = (int32_t)i;
      p.seg_meta[2 * g + 1] = (int32_t)((hi * R - 1) / T);
    }
    decode_tile<QM, D, true>(p, j / p.row_groups, h, j % p.row_groups, o0, o1, (int)i + g,
                             o0 == 0 && seg_end == hi);
    u = to_sgpr(seg_end);
  }
}

template <int QM, bool BAL>
static void launch_decode_dims(const AttnParams& p, int head_dim, dim3 g, hipStream_t stream) {
  const dim3 blk(256);
#define FP8ATTN_DECODE(DIM)                                                                  \
  do {                                                                                       \
    if constexpr (BAL) hipLaunchKernelGGL((decode_balanced_kernel<QM, DIM>), g, blk, 0, stream, p); \
    else if (DIM <= 256 && p.tile_rows == 32)                                                 \
      hipLaunchKernelGGL((decode32_kernel<QM, (DIM <= 256 ? DIM : 256)>), g, blk, 0, stream, p); \
    else hipLaunchKernelGGL((decode_kernel<QM, DIM>), g, blk, 0, stream, p);                 \
  } while (0)
  switch (head_dim) {
    case 64: FP8ATTN_DECODE(64); break;
    case 96: FP8ATTN_DECODE(96); break;
    case 128: FP8ATTN_DECODE(128); break;
    case 192: FP8ATTN_DECODE(192); break;
    default:
      // the last head dims: 256 (FP8 Q); 256 and 512 (BF16 and split Q)
      if constexpr (QM == kQBf16 || QM == kQBf16Split) {
        if (head_dim == 512) FP8ATTN_DECODE(512);
        else FP8ATTN_DECODE(256);
      } else FP8ATTN_DECODE(256);
  }
#undef FP8ATTN_DECODE
}

template <bool BAL>
static void launch_decode_modes(const AttnParams& p, int q_mode, int head_dim, dim3 g, hipStream_t stream) {
  if (q_mode == kQE4M3) launch_decode_dims<kQE4M3, BAL>(p, head_dim, g, stream);
  else if (q_mode == kQBf16E4M3) launch_decode_dims<kQBf16E4M3, BAL>(p, head_dim, g, stream);
  else if (q_mode == kQBf16Split) launch_decode_dims<kQBf16Split, BAL>(p, head_dim, g, stream);
  else launch_decode_dims<kQBf16, BAL>(p, head_dim, g, stream);
}

hipError_t launch_decode(const AttnParams& p, int q_mode, int head_dim, int64_t grid,
                         hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid);
  if (p.seg_meta) launch_decode_modes<true>(p, q_mode, head_dim, g, stream);
  else launch_decode_modes<false>(p, q_mode, head_dim, g, stream);
  return hipGetLastError();
}

#ifdef FP8ATTN_TIMELINE
// Copies the stamps of the last split-grid decode launch (kTimelineBlocks x kTimelineSlots
// uint64 values, blocks past the grid left as they were) to host memory; 0 on success.
extern "C" __attribute__((visibility("default"))) int fp8attn_decode_timeline(uint64_t* host_dst, int64_t max_values) {
  const int64_t n = (int64_t)kTimelineBlocks * kTimelineSlots;
  if (host_dst == nullptr || max_values < n) return -1;
  if (hipDeviceSynchronize() != hipSuccess) return -2;
  return hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(g_decode_timeline), n * sizeof(uint64_t), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : -3;
}
// Clears the stamps (zeros).
extern "C" __attribute__((visibility("default"))) int fp8attn_decode_timeline_clear(void) {
  static uint64_t zeros[kTimelineBlocks * kTimelineSlots];
  return hipMemcpyToSymbol(HIP_SYMBOL(g_decode_timeline), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) ==
                 hipSuccess ? 0 : -1;
}
#endif

}  // namespace fp8attn
