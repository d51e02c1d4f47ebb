// Native-FP8 paged attention for many query tokens per sequence (prefill, chunked prefill).
//
// What it computes: masked softmax attention of E4M3 Q against the paged E4M3 K/V cache with
// per-tensor descales, causal plus optional sliding window (vLLM PR #63139, Overview: the
// sliding-window layers run attention on E4M3 Q/K/V with FP8 matrix multiplies; vLLM PR #60372
// review thread: causal and local masks only).  Both contractions run on the gfx950 FP8 MFMA.
//
// Design (gfx950, wave64, 512 threads = 8 waves, 2 waves per SIMD):
//  * A block owns 256 query rows of one (sequence, kv head): rows are (token, q head in the GQA
//    group) pairs, token-major, so one K/V tile serves every q head of the group.  Each wave
//    owns 32 rows.
//  * K and V arrive one 64-token page at a time straight from HBM into LDS
//    (global_load_lds_dwordx4) in a ring of four stages.  Key rows are padded to D + 16 bytes
//    so that the MFMA operand reads below are free of bank conflicts.
//  * The 8 waves form two groups half a tile apart, one barrier per tile: while one wave of a
//    SIMD runs the softmax of a tile on the VALU, its partner runs MFMAs (PV of the previous tile
//    and QK^T of the next), so the matrix cores and the VALU overlap.
//  * S^T = K * Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales): keys are the MFMA rows,
//    query rows the columns, so each query row lives on one lane column (lane % 32) and its
//    softmax state is per lane, reduced across the two 32-lane halves with one exchange.
//  * P^T comes straight out of the S^T accumulator layout as the B operand of the PV MFMA
//    (O^T = V^T * P^T).  V^T operands are read with ds_read_b64_tr_b8, which transposes 8-byte
//    chunks of 8 key rows into 8 keys of one d column per lane.
//  * Softmax in the log2 domain with a lazy maximum: the running max only moves when a tile's
//    max exceeds it by more than 8, so P <= 2^8 fits E4M3 (max 448) and the O rescale is rare.
//  * P precision: E4M3 keeps 3 mantissa bits.  Rows that see few keys would feel that directly,
//    so blocks whose first row sees fewer than kSplitPKeys keys run in a second instance
//    (SPLIT = true) that also feeds the residual p - e4m3(p), scaled by 16, through a second
//    MFMA with a 2^-4 operand scale (P = hi + lo).  Keeping it a separate instance keeps the
//    common instance within 256 registers (2 waves per SIMD).
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "params.h"

namespace fp8attn {

constexpr int kSplitPKeys = 512;
constexpr float kLazyMax = 8.0f;

template <int D>
struct PrefillShape {
  static constexpr int NW = 8;            // waves per block
  static constexpr int RW = 32;           // rows per wave
  static constexpr int BM = NW * RW;      // rows per block
  static constexpr int BK = 64;           // keys per tile (one kernel page)
  // LDS row width: D, or 128 at D = 96 (the QK^T k-steps take 64 d; bytes 96-127 hold zeros)
  static constexpr int DL = D == 96 ? 128 : D;
  static constexpr int NCH = DL / 16;     // 16-byte chunks per LDS key row
  static constexpr int KSTEP = DL / 64;   // QK^T k-steps (64 d each)
  static constexpr int NDT = D / 32;      // O^T tiles of 32 d-rows
  static constexpr int RS = DL + 16;      // LDS row stride: one 16-byte pad per key row
  static constexpr int SLOTS = NCH + 1;   // 16-byte LDS slots per key row
  static constexpr int TILE = BK * RS;    // bytes of one K (or V) tile in LDS
  static constexpr int LOADS = 2 * SLOTS; // wave-wide 1 KiB load instructions per K+V tile
  static constexpr int MAXI = (LOADS + NW - 1) / NW;  // load instructions per wave per tile
  static_assert(MAXI <= NDT + 2 * KSTEP, "loads are issued one per MFMA");
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dim");
};

// Direct-to-LDS loads of one K and one V tile: DL/16 + 1 16-byte slots per key row (the pad slot
// gets a copy of the row's first chunk), 64 lanes per instruction, 2 * (DL/16 + 1) instructions
// per tile.  Wave w issues instructions w, w + 8, ...; every wave issues MAXI of them, a wave
// that has one fewer repeating its previous one (the same bytes to the same place), so that the
// issue is branch-free and every wave has the same number of loads in flight.
// The loads go through buffer resources whose range ends after the tile's last key below the
// sequence length: the rows of keys at or past it read zeros.  Those slots are never written for
// this sequence and may hold any bytes, E4M3 NaN codes included; their keys are masked (P = 0),
// but 0 * NaN is NaN in the MFMA, so their V rows must be finite, and zeros cost nothing here.
struct TileLoad {
  i32x4_t k_rsrc;         // K tile (page base plus the tile's first slot), uniform
  i32x4_t v_rsrc;         // V tile
  uint32_t lds_stage;     // LDS address of the stage's [K tile | V tile]
};
template <int D>
__device__ __forceinline__ int load_instruction(int wave, int k) {
  using S = PrefillShape<D>;
  const int ins = wave + S::NW * k;
  return ins < S::LOADS ? ins : ins - S::NW;
}
// idle: a load past the block's last tile, which only keeps the number of loads per interval
// fixed.  Its lanes all read the tile's first 16 bytes (one cache line) into the free stage.
template <int D>
__device__ __forceinline__ void tile_load_step(const TileLoad& tl, const uint32_t* loff, int wave, int k,
                                               bool idle) {
  using S = PrefillShape<D>;
  const int ins = load_instruction<D>(wave, k);
  const int which = ins / S::SLOTS;
  const int blk = ins % S::SLOTS;
  lds_dma16_buf(which ? tl.v_rsrc : tl.k_rsrc, idle ? 0u : loff[k],
                tl.lds_stage + (uint32_t)(which * S::TILE + blk * 1024));
}

// The MFMA work of one wave between two barriers: O^T += V^T * P^T for one tile (PV) and then
// S^T = K * Q^T for another (QK).  Operands are read from LDS two MFMAs ahead of their use, in a
// ring of three operand registers, so the LDS latency hides behind the MFMAs instead of
// stalling each one; the schedule barriers keep exactly that order.
//  * PV op dt (d tile of 32 rows): four transposing reads gather 32 keys per lane.  Slots
//    8q..8q+7 of lane group lg hold the 8 consecutive keys 32(q/2) + 16(q%2) + 8*lg + j, where j
//    is the source row this lane supplies; vp already holds the lane's part of the address.
//  * QK op (h2, c): key rows 32*h2 + kperm(m) (kp holds the lane's row and half), d bytes
//    64c .. 64c + 63.  The two 32-key halves alternate so consecutive MFMAs are independent.
// DO_PV / DO_QK leave out the PV or the QK^T half: a wave skips a tile none of its rows sees.
template <int D, bool SPLIT, bool DO_PV, bool DO_QK>
__device__ __forceinline__ void mfma_stream(const uint8_t* vp, const uint8_t* kp,
                                            f32x16_t (&oacc)[PrefillShape<D>::NDT], f32x16_t (&sacc)[2],
                                            const i32x8_t& pb, const i32x8_t& pbl,
                                            const i32x8_t (&qop)[PrefillShape<D>::KSTEP]) {
  using S = PrefillShape<D>;
  constexpr int NPV = DO_PV ? S::NDT : 0;
  constexpr int NOPS = NPV + (DO_QK ? 2 * S::KSTEP : 0);
  i32x8_t buf[3];
#pragma unroll
  for (int j = 0; j < NOPS + 2; ++j) {
    if (j < NOPS) {
      i32x8_t& o = buf[j % 3];
      if (j < NPV) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2_t v2 = lds_read_tr8(vp + ((32 * (q >> 1) + 16 * (q & 1)) * S::RS + 16 * j));
          o[2 * q] = v2[0];
          o[2 * q + 1] = v2[1];
        }
      } else {
        const int idx = j - NPV, h2 = idx & 1, c = idx >> 1;
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(kp + (32 * h2 * S::RS + 64 * c));
        const u32x4_t y = *reinterpret_cast<const u32x4_t*>(kp + (32 * h2 * S::RS + 64 * c + 16));
        o = i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // the reads of op j go out before the MFMA of op j - 2
    if (j >= 2) {
      const int i = j - 2;
      const i32x8_t& a = buf[i % 3];
      if (i < NPV) {
        oacc[i] = mfma_fp8_32x32x64(a, pb, oacc[i], kE8M0One);
        if constexpr (SPLIT) oacc[i] = mfma_fp8_32x32x64(a, pbl, oacc[i], kE8M0Sixteenth);
      } else {
        const int idx = i - NPV, h2 = idx & 1, c = idx >> 1;
        sacc[h2] = mfma_fp8_32x32x64(a, qop[c], c == 0 ? f32x16_t{} : sacc[h2], kE8M0One);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// QBF16: Q comes in bf16 and is quantized to E4M3 as it is loaded, with the same arithmetic as
// fp8attn_quantize_q (identical codes); otherwise Q holds E4M3 codes.
template <int D, bool SPLIT, bool QBF16>
__global__ void __launch_bounds__(512) prefill_fp8_kernel(const AttnParams p, int32_t qb_end,
                                                          const int32_t* __restrict__ block_table) {
  using S = PrefillShape<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;          // this lane's row within the wave (MFMA column)
  const int lg = lane >> 5;          // 32-lane half

  // ---- work item: (sequence, kv head) outer, q block descending (heaviest first) -----------
  // the block grid covers q blocks [0, qb_end) of every (sequence, kv head)
  // (32-bit index arithmetic: the host keeps the grid below 2^31)
  uint32_t id = xcd_remap32(blockIdx.x, gridDim.x);
  const int qb = qb_end - 1 - (int)(id % (uint32_t)qb_end); id /= (uint32_t)qb_end;
  const int h = (int)(id % (uint32_t)p.hkv);
  const int b = (int)(id / (uint32_t)p.hkv);
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
  const int r0 = qb * S::BM;
  if (r0 >= nrows) return;
  const int W = p.window;
  const int rlast = min(r0 + S::BM, nrows) - 1;
  const int pf = L - ql + r0 / G;           // first row's position
  const int pl = L - ql + rlast / G;        // last row's position
  const int k_lo = W >= 1 ? max(0, pf - W + 1) : 0;
  // inclusive tile range of the block (at least tile kt0, also when lengths break the contract)
  const int kt0 = k_lo / S::BK, kt1 = max(kt0, pl / S::BK);

  // this wave's rows and key range
  const int wr0 = r0 + wave * S::RW;
  const bool wave_active = wr0 < nrows;
  const int wrl = min(wr0 + S::RW, nrows) - 1;
  const int wpf = L - ql + (wave_active ? wr0 : rlast) / G;
  const int wpl = L - ql + (wave_active ? wrl : rlast) / G;
  const int wfull_lo = W >= 1 ? wpl - W + 1 : 0;     // keys [wfull_lo, wpf] are visible to every row
  // tiles holding a key that some row of the wave sees (wave-uniform)
  const int wt0 = __builtin_amdgcn_readfirstlane((W >= 1 ? max(0, wpf - W + 1) : 0) / S::BK);
  const int wt1 = __builtin_amdgcn_readfirstlane(wave_active ? wpl / S::BK : kt0 - 1);
  // this lane's row
  const int r = wr0 + lr;
  const bool rvalid = r < nrows;
  const int tok = (rvalid ? r : rlast) / G;
  const int hq = h * G + (rvalid ? r : rlast) % G;
  const int pos = L - ql + tok;
  // blocks whose first row sees few keys belong to the split-P instance, the rest to the other
  const int min_keys = W >= 1 ? min(pf + 1, W) : pf + 1;
  if ((min_keys < kSplitPKeys) != SPLIT) return;

  const float kd = p.k_descale ? kd_raw : 1.0f;
  const float vd = p.v_descale ? vd_raw : 1.0f;
  const float qd = p.q_descale ? qd_raw : 1.0f;
  const float cs = p.scale_log2 * kd * qd;

  // ---- Q^T operand: lane (row lr, half lg) holds Q[row][64c + 32lg .. +32] per k-step c -------
  i32x8_t qop[S::KSTEP];
  if constexpr (!QBF16) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                        (int64_t)hq * p.q_stride_head + 32 * lg;
#pragma unroll
    for (int c = 0; c < S::KSTEP; ++c) {
      u32x4_t a = {0, 0, 0, 0}, bb = {0, 0, 0, 0};
      if (rvalid && 64 * c + 32 * lg < D) {   // (d past the head dim, at D = 96: zeros)
        a = *reinterpret_cast<const u32x4_t*>(qp + 64 * c);
        bb = *reinterpret_cast<const u32x4_t*>(qp + 64 * c + 16);
      }
      qop[c] = i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bb[0], (int)bb[1], (int)bb[2], (int)bb[3]};
    }
  }
  // (bf16 Q is loaded and quantized further down, once the first tiles' loads are in flight)

  f32x16_t oacc[S::NDT];
#pragma unroll
  for (int t = 0; t < S::NDT; ++t) oacc[t] = f32x16_t{};
  float m_used = kNegInf, l_run = 0.f;
  float l_q = 0.f;   // single P: the sum of the E4M3 P values (the normalization of O)
  f32x16_t sacc[2];                 // S^T of the tile being processed (two 32-key halves)
  i32x8_t pb = {}, pbl = {};        // P^T operands (hi and, for SPLIT, lo) of that tile

  // (read through a restrict pointer: the page ids come in with scalar loads, which leaves the
  // vector memory counter to the tile loads alone)
  const int32_t* bt = block_table + (int64_t)b * p.bt_stride;
  const uint8_t* kbase = p.k_cache + (int64_t)h * p.kv_stride_head;
  const uint8_t* vbase = p.v_cache + (int64_t)h * p.kv_stride_head;
  const int64_t sT = p.kv_stride_tok, sP = p.kv_stride_page;
  const int ps = p.page_size;

  // ---- LDS stages --------------------------------------------------------------------------
  // Four stages of [K tile | V tile]; tile x lives in stage (x - kt0) mod 4.
  constexpr int SB = 2 * S::TILE;   // bytes per stage
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * SB];
  auto stage_of = [&](int x) __attribute__((always_inline)) { return ((x - kt0) & 3) * SB; };
  const uint32_t lds_base = lds_address(lds);

  // ---- tile loader: HBM -> LDS directly (global_load_lds_dwordx4, 16 bytes per lane) ---------
  // A wave-wide instruction fills 64 consecutive 16-byte LDS slots (lane i -> slot i).  Key rows
  // occupy DL/16 + 1 slots: DL bytes of data and one pad slot, which receives a duplicate of the
  // row's first chunk.  The pad makes the row stride DL + 16 bytes (see the operand reads).
  // Wave w issues instructions w, w + 8, ...; each lane's byte offset inside the 64-key tile is
  // fixed, so it is computed once and every load is a scalar tile base plus that offset.
  uint32_t loff[S::MAXI];
#pragma unroll
  for (int t = 0; t < S::MAXI; ++t) {
    const int ins = load_instruction<D>(wave, t);
    const int sl = (ins % S::SLOTS) * 64 + lane;
    const int row = sl / S::SLOTS, posn = sl % S::SLOTS;
    // chunks past the head dim (D = 96) take an offset outside every buffer's range: zeros
    loff[t] = 16 * posn >= D && posn != S::NCH
                  ? 0xFFFFFFF0u
                  : (uint32_t)(row * sT) + 16u * (uint32_t)(posn == S::NCH ? 0 : posn);
  }
  auto page_id = [&](int kt) __attribute__((always_inline)) -> int {
    return bt[ps == S::BK ? kt : (kt * S::BK) / ps];
  };
  // issue this wave's loads of tile kt (page id page) into the stage at byte offset so; the range
  // of the tile's buffers ends with its last key below L (rows past it read zeros)
  auto issue = [&](int so, int kt, int page, bool idle = false) __attribute__((always_inline)) {
    const int slot0 = ps == S::BK ? 0 : kt * S::BK - ((kt * S::BK) / ps) * ps;
    const int64_t tile_off = (int64_t)page * sP + (int64_t)slot0 * sT;
    const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(S::BK, L - kt * S::BK))) * (uint32_t)sT;
    const TileLoad tl{buffer_rsrc(kbase + tile_off, nrec), buffer_rsrc(vbase + tile_off, nrec),
                      lds_base + (uint32_t)so};
#pragma unroll
    for (int k = 0; k < S::MAXI; ++k) tile_load_step<D>(tl, loff, wave, k, idle);
  };

  // Row assignments.  MFMA row m of a 32-key half tile holds key kperm(m), which swaps bits 2
  // and 3 of m.  Then the 8 keys one transposing read gathers are 8 consecutive keys, and the
  // two 16-lane halves of the read (d rows 0..15 and 16..31 of an O^T tile, which hold d and
  // d + D/2) touch 16 distinct 16-byte LDS slots: no bank conflicts with the D + 16 row stride.
  // O^T tile dt, row m holds d = 16*dt + m for m < 16 and d = 16*dt + D/2 + (m - 16) otherwise.
  // per-lane constants for the V^T transposing reads
  const int tr_blk = (lane >> 4) & 1;        // which 16-row half of the 32 d-rows
  const int tr_j = (lane & 15) >> 1;         // source row j (0..7) supplied by this lane
  const int tr_h = lane & 1;                 // 8-byte half of the 16-byte chunk

  // S^T = K * Q^T for tile kt (K tile in stage st).  A operand row m holds key kperm(m).
  const int k_lane = lane_offset(kperm(lr) * S::RS + 32 * lg);

  // softmax of tile kt: mask (boundary tiles), lazy max, O rescale, P^T operands, running sum
  auto softmax = [&](int kt) __attribute__((always_inline)) {
    const int j0 = kt * S::BK;
    const bool need_mask = !(j0 >= wfull_lo && j0 + S::BK - 1 <= wpf);
    if (need_mask) {
      // value i of this lane is S^T row 8*(i/4) + 4*lg + i%4, i.e. key kperm(that row); the
      // visible keys of the row are (pos - W, pos]
      // (the lane's 8*lg term is folded into the bounds so that jj is a constant)
      const int jlo = (W >= 1 ? pos - W - j0 : -1 - j0) - 8 * lg, jhi = pos - j0 - 8 * lg;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int jj = 32 * h2 + ((i >> 3) << 4) + (((i >> 2) & 1) << 2) + (i & 3);
          sacc[h2][i] = (jj > jlo && jj <= jhi) ? sacc[h2][i] : kNegInf;
        }
      }
    }
    float mxr = kNegInf;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mxr = fmaxf(mxr, sacc[h2][i]);
    }
    mxr = max_xor32(mxr);
    const float mx = mxr * cs;
    // lazy maximum: move it only when the tile exceeds it by more than 2^8
    const bool grow = mx > m_used + kLazyMax;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_used;
      const float alpha = fast_exp2(m_used - (m_new == kNegInf ? 0.f : m_new));
      if (grow) {
        l_run *= alpha;
        if constexpr (!SPLIT) l_q *= alpha;
        m_used = m_new;
      }
      const float a = grow ? alpha : 1.0f;
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) oacc[t] *= a;
    }
    const float neg_m = m_used == kNegInf ? 0.f : -m_used;
    // P = exp2(s * cs - m), packed to E4M3 in the B-operand slot order (slot 16*h2 + i).  The
    // single-P instance normalizes O by the sum of the E4M3 values the PV MFMA takes, so that the
    // weights of a row sum to 1 exactly: with the unrounded sum, a row whose attention sits on a
    // few keys carried their rounding error straight into O (on the sliding-window prefill's 2M
    // rows the worst row erred by 0.036 against the exact softmax, 0.028 with this sum, for about
    // 1% more time).  The LSE keeps the unrounded sum.  The split-P instance's hi + lo / 16 is
    // within the unrounded sum's rounding.
    float lsum = 0.f, lqsum = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          e[k] = fast_exp2(__builtin_fmaf(sacc[h2][4 * q4 + k], cs, neg_m));
          lsum += e[k];
        }
        const uint32_t hi = pack4_e4m3(e[0], e[1], e[2], e[3]);
        pb[4 * h2 + q4] = (int)hi;
        if constexpr (!SPLIT) {
          float r4[4];
          unpack4_e4m3(hi, r4);
          lqsum += (r4[0] + r4[1]) + (r4[2] + r4[3]);
        }
        if constexpr (SPLIT) {
          float back[4], rsd[4];
          unpack4_e4m3(hi, back);
#pragma unroll
          for (int k = 0; k < 4; ++k) rsd[k] = (e[k] - back[k]) * 16.0f;
          pbl[4 * h2 + q4] = (int)pack4_e4m3(rsd[0], rsd[1], rsd[2], rsd[3]);
        }
      }
    }
    l_run += lsum;
    if constexpr (!SPLIT) l_q += lqsum;
    // P and the running sum are needed right here: without this the compiler sinks the whole
    // exponential block past the barrier that follows, into the MFMA half of the period.
    asm volatile("" ::"v"(pb), "v"(l_run), "v"(l_q));
    if constexpr (SPLIT) asm volatile("" ::"v"(pbl));
  };

  // O^T += V^T * P^T with the V tile in stage st: per 32-row d tile, 4 transposing reads gather
  // 32 keys per lane.  Slots 8q..8q+7 of lane group lg hold the 8 consecutive keys
  // 32(q/2) + 16(q%2) + 8*lg + j, where j is the source row this lane supplies to the read.
  const int v_lane = lane_offset((8 * lg + tr_j) * S::RS + (D / 2) * tr_blk + 8 * tr_h);
  // MFMA work between two barriers: PV of tile tv (stage so_v), then QK^T of tile tk (stage so_k).
  // A half runs only for a tile inside the wave's tile range [wt0, wt1]: a tile outside it is
  // masked for every row of the wave (P = 0), so its PV adds nothing and its S is never used.
  // (Before the first tile and after the last one the tile index is outside the range too.)
  auto run_stream = [&](int so_v, int so_k, int tv, int tk) __attribute__((always_inline)) {
    const uint8_t* vp = lds + (so_v + S::TILE + v_lane);
    const uint8_t* kp = lds + (so_k + k_lane);
    const bool pv = tv >= wt0 && tv <= wt1, qk = tk >= wt0 && tk <= wt1;
    if (pv) mfma_stream<D, SPLIT, true, false>(vp, kp, oacc, sacc, pb, pbl, qop);
    if (qk) mfma_stream<D, SPLIT, false, true>(vp, kp, oacc, sacc, pb, pbl, qop);
    // S is needed in this half period: keep the compiler from sinking the QK^T MFMAs past the
    // barrier that may follow
    asm volatile("" ::"v"(sacc[0]), "v"(sacc[1]));
  };

  // ---- main loop: two wave groups half a period apart -----------------------------------------
  // Waves 0-3 (group A) and 4-7 (group B) share the SIMDs pairwise.  Barrier t opens interval t:
  //   group A:  PV(t), QK(t+1) | loads of t+3, softmax(t+1)
  //   group B:  loads of t+3, softmax(t) | PV(t), QK(t+1)
  // so one wave of each SIMD runs MFMAs while the other runs the softmax, and each group issues
  // its loads in its softmax half, while its partner wave runs MFMAs (issued at the start of the
  // MFMA halves instead, the kernel measured 1-5% slower).  Only tiles t and t+1 are read in
  // interval t; tile t+2 is landing (it is needed after barrier t+1) and tile t+3 goes into the
  // stage tile t-1 has left, so a tile's loads have about an interval to land.  Before each barrier a wave waits for all
  // its loads but the ones of the interval that ends there.  Loads past the last tile read one
  // cache line into the free stage, which keeps the number of loads the same every interval.
  // Before a barrier: the loads older than this interval's have landed.  Also a scheduling fence:
  // the compiler may not move the softmax or MFMA work of one half period across the barrier into
  // the other half, which would take away the overlap.
  auto wait_loads = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(S::MAXI));
  };
  // The two groups run separate loops (wave-uniform branch) so that each keeps only its own
  // values live across the barrier: S^T in group B, P^T in group A.  Both loops meet the same
  // barriers: one before the first tile and one per tile.
  // page id of the tile interval I loads (tile min(I + 3, kt1)), read one interval ahead
  int page_ahead = page_id(min(kt0 + 2, kt1));
  auto interval_loads = [&](int I) __attribute__((always_inline)) {
    issue(stage_of(I + 3), min(I + 3, kt1), page_ahead, I + 3 > kt1);
    page_ahead = page_id(min(I + 4, kt1));
  };

  issue(stage_of(kt0), kt0, page_id(kt0));
  issue(stage_of(kt0 + 1), min(kt0 + 1, kt1), page_id(min(kt0 + 1, kt1)), kt0 + 1 > kt1);
  if constexpr (QBF16) {
    // The same 32 d values per k-step as the E4M3 codes, read as bf16 and quantized here, with
    // the arithmetic of the stand-alone quantize call (identical codes).  Every load is issued
    // before the first conversion so that their latencies overlap each other and the tile loads
    // above; a row past the end reads the clamped row and is zeroed.
    const double rcp = 1.0 / (double)qd;   // (qd was read before the tile loads: no wait here)
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                       (int64_t)hq * p.q_stride_head + 32 * lg;
    u32x4_t qw[S::KSTEP][4];
#pragma unroll
    for (int c = 0; c < S::KSTEP; ++c) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qw[c][k] = 64 * c + 32 * lg < D ? *reinterpret_cast<const u32x4_t*>(qp + 64 * c + 8 * k) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < S::KSTEP; ++c) {
      u32x2_t e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = quantize8_bf16_e4m3(qw[c][k], rcp);
      qop[c] = i32x8_t{(int)e[0][0], (int)e[0][1], (int)e[1][0], (int)e[1][1],
                       (int)e[2][0], (int)e[2][1], (int)e[3][0], (int)e[3][1]};
#pragma unroll
      for (int k = 0; k < 8; ++k) qop[c][k] = rvalid && 64 * c + 32 * lg < D ? qop[c][k] : 0;
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();   // tiles kt0 and kt0 + 1 are in LDS; this opens interval kt0 - 1
  interval_loads(kt0 - 1);
  // Every wave processes every tile of the block; tiles outside a wave's key range are fully
  // masked for its rows (P = 0), which keeps the loop body one straight MFMA stream.
  const bool grpB = wave >= S::NW / 2;
  if (!grpB) {
    run_stream(stage_of(kt0), stage_of(kt0), kt0 - 1, kt0);   // QK^T of the first tile
    for (int t = kt0; t <= kt1; ++t) {
      if (t > kt0) interval_loads(t - 1);        // loads of interval t - 1, in its softmax half
      if (t >= wt0 && t <= wt1) softmax(t);
      wait_loads();
      __syncthreads();
      run_stream(stage_of(t), stage_of(t + 1), t, t + 1);
    }
    interval_loads(kt1);
  } else {
    // the stream at step t belongs to interval t - 1; one step past the last tile finishes PV
    // of the last tile
    for (int t = kt0; t <= kt1 + 1; ++t) {
      run_stream(t > kt0 ? stage_of(t - 1) : stage_of(t), stage_of(t), t - 1, t);
      if (t <= kt1) {
        wait_loads();
        __syncthreads();
        interval_loads(t);                       // interval t
        if (t >= wt0 && t <= wt1) softmax(t);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));       // nothing may land after the block ends

  // ---- epilogue ------------------------------------------------------------------------------
  // O leaves through LDS.  Each wave writes its 32 normalized bf16 rows, in the accumulator
  // layout, into its own part of the freed stage ring, and reads them back along the rows.  Every
  // store instruction then writes whole row segments, 16 bytes per lane with consecutive lanes
  // on consecutive bytes.  Stored straight from the accumulators, one instruction writes 8 bytes
  // into each of 32 rows, and HBM took a third more bytes than O has.  The split-P instance
  // (the first few hundred rows of each sequence) keeps the direct stores: it has no registers
  // to spare for the staging.
  l_run = sum_xor32(l_run);
  if constexpr (!SPLIT) l_q = sum_xor32(l_q);
  const float l_norm = SPLIT ? l_run : l_q;
  const float inv = l_norm > 0.f ? vd / l_norm : 0.f;
  if constexpr (!SPLIT) {
    constexpr int ORS = 2 * D + 16;                 // LDS row stride of the staged O (bytes)
    static_assert(S::NW * S::RW * ORS <= 4 * SB, "the staged O fits the stage ring");
    __syncthreads();                                // every wave's loads have landed and its reads are done
    uint8_t* const ow = lds + wave * (S::RW * ORS);
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 16 * dt + (i4 >= 2 ? D / 2 : 0) + 8 * (i4 & 1) + 4 * lg;
        const bf16x4_t o = {(__bf16)(oacc[dt][4 * i4] * inv), (__bf16)(oacc[dt][4 * i4 + 1] * inv),
                            (__bf16)(oacc[dt][4 * i4 + 2] * inv), (__bf16)(oacc[dt][4 * i4 + 3] * inv)};
        *reinterpret_cast<bf16x4_t*>(ow + lr * ORS + 2 * d) = o;
      }
    }
    // (a wave reads back only the rows it wrote: its own LDS accesses stay in program order)
    constexpr int CPR = D / 8;                      // 16-byte chunks per row
    __bf16* const obase = reinterpret_cast<__bf16*>(p.out);
#pragma unroll
    for (int k = 0; k < S::RW * CPR / 64; ++k) {
      const int c = 64 * k + lane;
      const int row = c / CPR, col = c % CPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ow + row * ORS + 16 * col);
      const int rr = wr0 + row;
      if (rr < nrows) {
        const int tk = rr / G, hh = h * G + rr % G;
        // (non-temporal: O is written once; 0.5-1.7% faster than plain stores)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(obase + (int64_t)(t0 + tk) * p.out_stride_tok +
                                                                  (int64_t)hh * p.out_stride_head + 8 * col));
      }
    }
  } else if (rvalid) {
    __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)(t0 + tok) * p.out_stride_tok +
                 (int64_t)hq * p.out_stride_head;
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 16 * dt + (i4 >= 2 ? D / 2 : 0) + 8 * (i4 & 1) + 4 * lg;
        const bf16x4_t o = {(__bf16)(oacc[dt][4 * i4] * inv), (__bf16)(oacc[dt][4 * i4 + 1] * inv),
                            (__bf16)(oacc[dt][4 * i4 + 2] * inv), (__bf16)(oacc[dt][4 * i4 + 3] * inv)};
        *reinterpret_cast<bf16x4_t*>(op + d) = o;
      }
    }
  }
  if (p.lse && lg == 0 && rvalid)
    p.lse[(int64_t)(t0 + tok) * p.hq + hq] = l_run > 0.f ? (m_used + fast_log2(l_run)) * kLn2 : kNegInf;
}

template <int D, bool QBF16>
static void launch_prefill_pair(const AttnParams& p, int64_t grid, int64_t nqb, int64_t grid_split,
                                int64_t nqb_split, hipStream_t stream) {
  const dim3 blk(512);
  hipLaunchKernelGGL((prefill_fp8_kernel<D, false, QBF16>), dim3((unsigned)grid), blk, 0, stream, p, (int32_t)nqb,
                     p.block_table);
  hipLaunchKernelGGL((prefill_fp8_kernel<D, true, QBF16>), dim3((unsigned)grid_split), blk, 0, stream, p,
                     (int32_t)nqb_split, p.block_table);
}

hipError_t launch_prefill_fp8(const AttnParams& p, int head_dim, bool q_bf16, hipStream_t stream) {
  const int G = p.group;
  const int64_t nqb = ((int64_t)p.max_seqlen_q * G + 255) / 256;
  if (nqb <= 0 || p.hkv <= 0 || p.batch <= 0) return hipSuccess;
  // A block runs in the split-P instance iff its first row sees fewer than kSplitPKeys keys:
  // min(position + 1, window).  A window shorter than kSplitPKeys puts every block there.
  // Otherwise the first row's token index must be below kSplitPKeys, so only q blocks
  // qb < nqb_split can.
  const bool short_window = p.window >= 1 && p.window < kSplitPKeys;
  const int64_t nqb_split =
      short_window ? nqb : std::min<int64_t>(nqb, ((int64_t)(kSplitPKeys - 1) * G) / 256 + 1);
  const int64_t grid = nqb * p.hkv * p.batch, grid_split = nqb_split * p.hkv * p.batch;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
  if (head_dim == 256) {
    if (q_bf16) launch_prefill_pair<256, true>(p, grid, nqb, grid_split, nqb_split, stream);
    else launch_prefill_pair<256, false>(p, grid, nqb, grid_split, nqb_split, stream);
  } else if (head_dim == 192) {
    if (q_bf16) launch_prefill_pair<192, true>(p, grid, nqb, grid_split, nqb_split, stream);
    else launch_prefill_pair<192, false>(p, grid, nqb, grid_split, nqb_split, stream);
  } else if (head_dim == 96) {
    if (q_bf16) launch_prefill_pair<96, true>(p, grid, nqb, grid_split, nqb_split, stream);
    else launch_prefill_pair<96, false>(p, grid, nqb, grid_split, nqb_split, stream);
  } else if (head_dim == 128) {
    if (q_bf16) launch_prefill_pair<128, true>(p, grid, nqb, grid_split, nqb_split, stream);
    else launch_prefill_pair<128, false>(p, grid, nqb, grid_split, nqb_split, stream);
  } else {
    if (q_bf16) launch_prefill_pair<64, true>(p, grid, nqb, grid_split, nqb_split, stream);
    else launch_prefill_pair<64, false>(p, grid, nqb, grid_split, nqb_split, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8attn
