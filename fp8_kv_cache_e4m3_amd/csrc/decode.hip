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
//                   QK^T on the BF16 MFMA.
// PV runs on the BF16 MFMA in both variants: V bytes are dequantized exactly to bf16 and P is
// rounded once to bf16.  Decode is HBM-bound, so the cheaper FP8 PV would not move the time but
// would cost accuracy on short rows.
//
// Design (gfx950, wave64):
//  * Work item = (kv head, split, sequence, row tile), XCD-aware block order.  4 waves per
//    block; each wave streams its own 16-key units (a quarter of the split) straight from HBM
//    into registers, with the next unit's loads in flight while the current one is computed.
//    No LDS staging and no barriers in the main loop.
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

constexpr float kLazyMax = 8.0f;   // log2 units: the running max moves by more than 2^8 or not at all

template <int D>
struct DecodeShape {
  static constexpr int kKeys = 16;                    // keys per unit
  static constexpr int KCH = D / 64;                  // 16-byte K chunks per lane per unit
  static constexpr int CW = D >= 256 ? 16 : D / 16;   // V bytes per lane per key per block
  static constexpr int VBLK = D / (16 * CW);          // V column blocks
  static constexpr int NT = D / 16;                   // O^T tiles (16 d-rows each)
  static constexpr int RS = D + 4;                    // LDS row stride (floats), padded
  static_assert(D == 64 || D == 128 || D == 192 || D == 256 || D == 512, "head dim");
};

template <int D>
struct UnitRegs {
  u32x4_t k[DecodeShape<D>::KCH];
  uint32_t v[4][DecodeShape<D>::VBLK][DecodeShape<D>::CW / 4];
};

// K/V byte loads; NT marks them non-temporal (streamed once, no reuse).
template <bool NT, class T>
__device__ __forceinline__ T stream_load(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Per-lane byte offsets inside a unit, the same for every unit: K row col, bytes 16 grp (+ 64 c);
// V rows 4 grp + i, bytes col * CW (+ 16 CW blk).  A unit's loads are then a uniform base (page
// plus first slot) plus these 32-bit offsets: the SGPR-base form of the global loads.
struct UnitOffsets {
  uint32_t k;
  uint32_t v[4];
};

template <int D, bool NT>
__device__ __forceinline__ void load_unit(UnitRegs<D>& ur, const uint8_t* __restrict__ kunit,
                                          const uint8_t* __restrict__ vunit, const UnitOffsets& off) {
  using S = DecodeShape<D>;
#pragma unroll
  for (int c = 0; c < S::KCH; ++c)
    ur.k[c] = stream_load<NT>(reinterpret_cast<const u32x4_t*>(kunit + off.k + 64 * c));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int blk = 0; blk < S::VBLK; ++blk) {
      const uint8_t* vp = vunit + off.v[i] + blk * 16 * S::CW;
      if constexpr (S::CW == 16) {
        const u32x4_t w = stream_load<NT>(reinterpret_cast<const u32x4_t*>(vp));
        ur.v[i][blk][0] = w[0];
        ur.v[i][blk][1] = w[1];
        ur.v[i][blk][2] = w[2];
        ur.v[i][blk][3] = w[3];
      } else if constexpr (S::CW == 8) {
        const u32x2_t w = stream_load<NT>(reinterpret_cast<const u32x2_t*>(vp));
        ur.v[i][blk][0] = w[0];
        ur.v[i][blk][1] = w[1];
      } else {   // 4 or 12 bytes: dword loads
#pragma unroll
        for (int x = 0; x < S::CW / 4; ++x)
          ur.v[i][blk][x] = stream_load<NT>(reinterpret_cast<const uint32_t*>(vp + 4 * x));
      }
    }
  }
}

// Per-variant tuning (measured on MI355X, sliding-window decode, cold K/V).  Two units in
// flight per wave; deeper register rings (3 or 4 units, which fit at two waves per SIMD) were
// slower, as were rings staged through LDS with direct-to-LDS loads.  A plain gather with this
// access pattern (256-byte row slices, 16 rows per instruction) tops out near 47 us for the
// 269 MB, against about 50 us for the kernel.  Non-temporal loads help the d256 stream (+4%)
// and hurt the split d512 stream (-11%).
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

template <int QM, int D>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(DecodeTune<QM != kQBf16, D>::MIN_WAVES))) decode_kernel(const AttnParams p) {
  constexpr bool QFP8 = QM != kQBf16;   // QK^T on the FP8 MFMA
  using S = DecodeShape<D>;
  using T = DecodeTune<QFP8, D>;
  constexpr int NBUF = T::NBUF;
  // LDS: the 4 waves' softmax state and O tiles for the final merge
  __shared__ __attribute__((aligned(16))) float sm_o[4][16][S::RS];
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;

  // ---- work item (32-bit index arithmetic: the host keeps the grid below 2^31) ----------
  uint32_t id = xcd_remap32(blockIdx.x, gridDim.x);
  const uint32_t n_rt = (uint32_t)p.row_groups, n_b = (uint32_t)p.batch, n_s = (uint32_t)p.num_splits;
  const int rt = (int)(id % n_rt); id /= n_rt;
  const int b = (int)(id % n_b); id /= n_b;
  const int s = (int)(id % n_s);
  const int h = (int)(id / n_s);
  const int G = p.group;

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
  const int su0 = u_begin + s * p.units_per_split;
  const int su1 = min(u_end, su0 + p.units_per_split);
  // keys every row of this tile can see: [full_lo, p_first]
  const int full_lo = W >= 1 ? p_last - W + 1 : 0;

  // this lane's query row
  const int r = row0 + col;
  const bool rvalid = r < nrows;
  const int tok = rvalid ? r / G : rlast / G;
  const int hq = h * G + (rvalid ? r % G : rlast % G);
  const int pos = L - ql + tok;

  if (su0 >= su1) {  // nothing visible in this split: neutral partial for the combine
    if (p.num_splits > 1 && threadIdx.x < 16 && rvalid)
      p.part_lse[((int64_t)s * p.total_q + t0 + tok) * p.hq + hq] = kNegInf;
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
  QRegs<QFP8, D> qr;
  u32x4_t qraw[QM == kQBf16E4M3 ? 2 * S::KCH : 1];
  if constexpr (QM == kQE4M3) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                        (int64_t)hq * p.q_stride_head + 16 * grp;
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      u32x4_t w = rvalid ? *reinterpret_cast<const u32x4_t*>(qp + 64 * c) : u32x4_t{0, 0, 0, 0};
      qr.q[2 * c] = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
      qr.q[2 * c + 1] = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
    }
  } else if constexpr (QM == kQBf16E4M3) {
    // the same 16 d values per k-chunk as above, read as bf16 here and quantized once the first
    // units' loads are in flight (below); a row past the end reads the clamped row
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                       (int64_t)hq * p.q_stride_head + 16 * grp;
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) qraw[2 * c + hf] = *reinterpret_cast<const u32x4_t*>(qp + 64 * c + 8 * hf);
    }
  } else {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                       (int64_t)hq * p.q_stride_head + 16 * grp;
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      const bf16x8_t z = {};
      qr.q[2 * c] = rvalid ? *reinterpret_cast<const bf16x8_t*>(qp + 64 * c) : z;
      qr.q[2 * c + 1] = rvalid ? *reinterpret_cast<const bf16x8_t*>(qp + 64 * c + 8) : z;
    }
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

  UnitOffsets uoff;
  uoff.k = (uint32_t)(col * sT) + 16u * (uint32_t)grp;
#pragma unroll
  for (int i = 0; i < 4; ++i) uoff.v[i] = (uint32_t)((4 * grp + i) * sT) + (uint32_t)(col * S::CW);
  // Loads past the split's last unit keep the number of loads per trip fixed, so that the
  // compiler waits for exactly the oldest unit.  They read the last unit's first 16 bytes in every
  // lane: one cache line, which costs next to nothing and lands quickly at the end of the stream.
  const int ulast = su1 - 1;
  auto issue = [&](UnitRegs<D>& ur, int u) __attribute__((always_inline)) {
    const bool trailing = u > ulast;
    const int uc = trailing ? ulast : u;
    const int64_t unit = page_of(uc) * sP + (int64_t)((uc * 16) % ps) * sT;
    UnitOffsets o = uoff;
    o.k = trailing ? 0u : o.k;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = trailing ? 0u : o.v[i];
    load_unit<D, T::NT>(ur, kbase + unit, vbase + unit, o);
  };

  // S^T tile of a unit: rows = its 16 keys, columns = the 16 query rows
  auto qk = [&](const u32x4_t (&kk)[S::KCH]) __attribute__((always_inline)) -> f32x4_t {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S::KCH; ++c) {
      if constexpr (QFP8) {
        const uint64_t k0 = (uint64_t)kk[c][0] | ((uint64_t)kk[c][1] << 32);
        const uint64_t k1 = (uint64_t)kk[c][2] | ((uint64_t)kk[c][3] << 32);
        sacc = mfma_fp8_16x16x32(k0, qr.q[2 * c], sacc);
        sacc = mfma_fp8_16x16x32(k1, qr.q[2 * c + 1], sacc);
      } else {
        sacc = mfma_bf16_16x16x32(e4m3x8_to_bf16(kk[c][0], kk[c][1]), qr.q[2 * c], sacc);
        sacc = mfma_bf16_16x16x32(e4m3x8_to_bf16(kk[c][2], kk[c][3]), qr.q[2 * c + 1], sacc);
      }
    }
    return sacc;
  };

  // mask, online softmax update, P^T operand of unit u (lane (row, g) holds keys 4g..4g+3)
  auto softmax = [&](const f32x4_t sacc, int u) __attribute__((always_inline)) -> bf16x4_t {
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = sacc[i] * cscale;
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
    const bool grow = mx > m_run + kLazyMax;
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
    return bf16x4_t{(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
  };

  // O^T += V^T * P^T with V in registers (lane (col, g) holds bytes col*CW.. of keys 4g..4g+3):
  // a 4x4 byte transpose gives, per O^T tile t, row col <-> d = 16 col + t (d256) or the
  // analogous interleave (d64, d512)
  auto compute = [&](const UnitRegs<D>& ur, int u) __attribute__((always_inline)) {
    const bf16x4_t pb = softmax(qk(ur.k), u);
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
    UnitRegs<D> buf[NBUF];
#pragma unroll
    for (int k = 0; k < NBUF; ++k) issue(buf[k], u0 + 4 * k);
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
        issue(buf[k], uk + 4 * NBUF);
      }
    }
  }
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

  // ---- final: thread -> (row, d-part) -------------------------------------------------------
  {
    const int row = threadIdx.x & 15;
    const int part = threadIdx.x >> 4;                 // 16 parts of D/16 values
    constexpr int PW = D / 16;
    const int rr = row0 + row;
    if (rr < nrows) {
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
      const float inv = Ls > 0.f ? vd / Ls : 0.f;
      const float lse2 = Ls > 0.f ? (M + fast_log2(Ls)) : kNegInf;
      if (p.num_splits == 1) {
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
        float* op = p.part_o + (((int64_t)s * p.total_q + tk) * p.hq + hh) * D + part * PW;
#pragma unroll
        for (int c = 0; c < PW; c += 4) {
          f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sm_o[0][row][part * PW + c]);
#pragma unroll
          for (int w = 1; w < 4; ++w) a += *reinterpret_cast<const f32x4_t*>(&sm_o[w][row][part * PW + c]);
          *reinterpret_cast<f32x4_t*>(op + c) = a * inv;
        }
        if (part == 0) p.part_lse[((int64_t)s * p.total_q + tk) * p.hq + hh] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
      }
    }
  }
}

template <int QM>
static void launch_decode_dims(const AttnParams& p, int head_dim, dim3 g, hipStream_t stream) {
  const dim3 blk(256);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((decode_kernel<QM, 64>), g, blk, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((decode_kernel<QM, 128>), g, blk, 0, stream, p); break;
    case 192: hipLaunchKernelGGL((decode_kernel<QM, 192>), g, blk, 0, stream, p); break;
    default:
      // the last head dim of each variant: 256 (FP8 Q) or 512 (BF16 Q)
      if constexpr (QM == kQBf16) hipLaunchKernelGGL((decode_kernel<QM, 512>), g, blk, 0, stream, p);
      else hipLaunchKernelGGL((decode_kernel<QM, 256>), g, blk, 0, stream, p);
  }
}

hipError_t launch_decode(const AttnParams& p, int q_mode, int head_dim, int64_t grid,
                         hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid);
  if (q_mode == kQE4M3) launch_decode_dims<kQE4M3>(p, head_dim, g, stream);
  else if (q_mode == kQBf16E4M3) launch_decode_dims<kQBf16E4M3>(p, head_dim, g, stream);
  else launch_decode_dims<kQBf16>(p, head_dim, g, stream);
  return hipGetLastError();
}

}  // namespace fp8attn
