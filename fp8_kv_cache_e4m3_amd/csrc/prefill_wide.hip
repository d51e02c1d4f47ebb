// Paged attention prefill at head dim 512 with BF16 queries over the E4M3 KV cache: the
// full-attention layers, which keep BF16 Q and dequantize the FP8 cache inside the kernel (vLLM PR
// #60372, Overview; prhub digest of vLLM PR #48666, Implementation items 1-3).  Two MFMA variants,
// with the per-element arithmetic of the decode kernel's two bf16-Q modes:
//   SPLITQ = false (q_dtype BF16): K and V bytes are converted exactly to bf16 as they are read, P
//     is rounded once to bf16, and both contractions run on the BF16 MFMA (16x16x32);
//   SPLITQ = true (q_dtype BF16_SPLIT): each query row is scaled by a power of two and written as
//     hi + lo / 16 in E4M3 (exact for bf16 values, see split8_bf16_e4m3), and QK^T runs on the
//     scaled FP8 MFMA (16x16x128) with the lo terms at operand scale 2^-4; P (<= 2^4) is written as
//     16 hi + lo and PV runs on the FP8 MFMA (16x16x32) with both terms against the same V bytes:
//     no dequantization at all (vLLM PR #60372, review thread: the d512 FP8-MMA kernel keeps BF16
//     queries and builds a split QK accumulation).
//
// Design (gfx950, wave64, 512 threads = 8 waves, two per SIMD):
//  * A block owns 128 query rows of one (sequence, kv head), rows token-major as in the other
//    kernels; each wave owns 16 rows (the MFMA's column count), so its O^T (512 d x 16 rows, fp32)
//    takes 128 accumulation registers and its Q 64 registers.
//  * K and V arrive one 32-key tile at a time straight into LDS (buffer loads with an LDS
//    destination, range ending at the sequence length so rows past it read zeros), in a ring of
//    four stages; key rows are padded to 528 bytes (a copy of the row's first 16 bytes), which
//    spreads the 16 key rows of an operand read over distinct banks.  A tile is requested two
//    barriers before it is first read: with two stages of 64-key tiles (all the LDS holds at this
//    head dim) the wait for the next tile took a third of the time.  One barrier per tile.
//  * The two waves of a SIMD run half a tile apart (waves 0-3 against 4-7), so one's softmax runs
//    on the VALU while the other's MFMAs run.
//  * S^T = K Q^T with keys on the MFMA rows and query rows on the columns, so a row's softmax state
//    is per lane.  MFMA row m of 16-key block kb holds key 8 (m / 4) + 4 kb + m % 4: then the 8
//    keys whose P a lane group feeds to one PV MFMA are 8 consecutive keys, and one transposing LDS
//    read (ds_read_b64_tr_b8) gives the matching V^T operand.
#include <type_traits>

#include "device.h"
#include "params.h"


namespace fp8attn {

namespace {

constexpr int kD = 512;
constexpr int kNW = 8;                    // waves per block (two per SIMD)
constexpr int kRW = 16;                   // rows per wave
constexpr int kBM = kNW * kRW;            // rows per block
constexpr int kBK = 32;                   // keys per tile
constexpr int kNS = 4;                    // stages in the LDS ring
constexpr int kNCH = kD / 16;             // 16-byte chunks per key row
constexpr int kRS = kD + 16;              // LDS row stride (one pad slot)
constexpr int kSlots = kNCH + 1;          // 16-byte LDS slots per key row
constexpr int kRowSlots = kBK * kSlots;   // 1,056 slots of key rows per tile ...
constexpr int kInsPerTile = (kRowSlots + 63) / 64;   // ... written by 17 wave-wide loads
constexpr int kTile = kInsPerTile * 1024; // bytes of one K (or V) tile: rows, then 32 spare slots
constexpr int kStage = 2 * kTile;         // [K tile | V tile]
constexpr int kLoads = 2 * kInsPerTile;   // wave-wide 1 KiB loads per K+V tile
constexpr int kMaxI = (kLoads + kNW - 1) / kNW;   // loads per wave per tile
constexpr int kNT = kD / 16;              // O^T tiles of 16 d rows

// load instruction k of this wave: instructions w, w + 4, ...; a wave with one fewer repeats its
// previous one (the same bytes to the same place), so every wave issues the same count
__device__ __forceinline__ int wide_load_instruction(int wave, int k) {
  const int ins = wave + kNW * k;
  return ins < kLoads ? ins : ins - kNW;
}

// key of MFMA row m in 16-key block kb of a tile
__device__ __forceinline__ int block_key(int kb, int m) { return 8 * (m >> 2) + 4 * kb + (m & 3); }

}  // namespace

template <bool SPLITQ>
__global__ void __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(2))) prefill_wide_kernel(const AttnParams p, int32_t qb_end,
                                                           const int32_t* __restrict__ block_table) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;         // this lane's row within the wave (MFMA column)
  const int grp = lane >> 4;         // 16-lane group

  // ---- work item: (sequence, kv head) outer, q block descending (heaviest first) -------------
  uint32_t id = xcd_remap32(blockIdx.x, gridDim.x);
  const int qb = qb_end - 1 - (int)(id % (uint32_t)qb_end); id /= (uint32_t)qb_end;
  const int h = (int)(id % (uint32_t)p.hkv);
  const int b = (int)(id / (uint32_t)p.hkv);
  const int G = p.group;
  // per-item scalars, requested together before any branch (see the decode kernel)
  const int64_t dsi = (int64_t)b * p.ds_stride_b + (int64_t)h * p.ds_stride_h;
  const int t0 = load_uniform(p.cu_seqlens_q, b);
  const int t1 = load_uniform(p.cu_seqlens_q, b + 1);
  const int L = load_uniform(p.seqlens_k, b);
  const float* stand_in = reinterpret_cast<const float*>(p.seqlens_k);
  const float kd_raw = load_uniform(p.k_descale ? p.k_descale : stand_in, p.k_descale ? dsi : 0);
  const float vd_raw = load_uniform(p.v_descale ? p.v_descale : stand_in, p.v_descale ? dsi : 0);
  asm volatile("" ::"s"(t0), "s"(t1), "s"(L), "s"(kd_raw), "s"(vd_raw));
  const int ql = t1 - t0;
  const int nrows = ql * G;
  const int r0 = qb * kBM;
  if (r0 >= nrows) return;
  const int W = p.window;
  const int rlast = min(r0 + kBM, nrows) - 1;
  const int pf = L - ql + r0 / G;
  const int pl = L - ql + rlast / G;
  const int k_lo = W >= 1 ? max(0, pf - W + 1) : 0;
  const int kt0 = k_lo / kBK, kt1 = max(kt0, pl / kBK);   // (one tile at least, also for bad lengths)

  // this wave's rows and the tiles some row of it sees
  const int wr0 = r0 + wave * kRW;
  const bool wave_active = wr0 < nrows;
  const int wrl = min(wr0 + kRW, nrows) - 1;
  const int wpf = L - ql + (wave_active ? wr0 : rlast) / G;
  const int wpl = L - ql + (wave_active ? wrl : rlast) / G;
  const int wfull_lo = W >= 1 ? wpl - W + 1 : 0;     // keys [wfull_lo, wpf] are visible to every row
  const int wt0 = __builtin_amdgcn_readfirstlane((W >= 1 ? max(0, wpf - W + 1) : 0) / kBK);
  const int wt1 = __builtin_amdgcn_readfirstlane(wave_active ? wpl / kBK : kt0 - 1);
  const int r = wr0 + col;
  const bool rvalid = r < nrows;
  const int tok = (rvalid ? r : rlast) / G;
  const int hq = h * G + (rvalid ? r : rlast) % G;
  const int pos = L - ql + tok;

  const float kd = p.k_descale ? kd_raw : 1.0f;
  const float vd = p.v_descale ? vd_raw : 1.0f;
  float cs = p.scale_log2 * kd;      // (split Q: times the row's 2^-e)

  // ---- LDS ring and tile loads ---------------------------------------------------------------
  __shared__ __attribute__((aligned(16))) uint8_t lds[kNS * kStage];
  const uint32_t lds_base = lds_address(lds);
  const int32_t* bt = block_table + (int64_t)b * p.bt_stride;
  const uint8_t* kbase = p.k_cache + (int64_t)h * p.kv_stride_head;
  const uint8_t* vbase = p.v_cache + (int64_t)h * p.kv_stride_head;
  const int64_t sT = p.kv_stride_tok, sP = p.kv_stride_page;
  const int ps = p.page_size;
  // This wave's loads of tile kt into stage st: a wave-wide instruction fills 64 consecutive
  // 16-byte slots; key rows take kSlots slots, the last one a copy of the row's first chunk, and
  // the slots past the rows (the last instruction's second half) get the tile's first chunk.  The
  // buffers' range ends with the tile's last key below L: rows past it read zeros (slots never
  // written for this sequence, possibly holding NaN codes, which 0 * NaN in the MFMA would spread).
  // idle: a load past the block's last tile, which only keeps the count of loads per tile fixed;
  // all its lanes read the tile's first 16 bytes.  The lane offsets are recomputed for every tile
  // from an opaque copy of the lane id, so that they are not hoisted into 17 live registers.
  auto issue = [&](int st, int kt, bool idle) __attribute__((always_inline)) {
    const int page = bt[ps == kBK ? kt : (kt * kBK) / ps];
    const int slot0 = ps == kBK ? 0 : kt * kBK - ((kt * kBK) / ps) * ps;
    const int64_t tile_off = (int64_t)page * sP + (int64_t)slot0 * sT;
    const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(kBK, L - kt * kBK))) * (uint32_t)sT;
    const i32x4_t krs = buffer_rsrc(kbase + tile_off, nrec), vrs = buffer_rsrc(vbase + tile_off, nrec);
    const uint32_t so = lds_base + (uint32_t)(st * kStage);
    const int ln = lane_offset(lane);
#pragma unroll
    for (int k = 0; k < kMaxI; ++k) {
      const int ins = wide_load_instruction(wave, k);
      const int which = ins / kInsPerTile, blk = ins % kInsPerTile;
      const int sl = blk * 64 + ln;
      const int row = sl / kSlots, posn = sl % kSlots;
      const uint32_t voff = idle || sl >= kRowSlots ? 0u : (uint32_t)(row * sT) + 16u * (uint32_t)(posn == kNCH ? 0 : posn);
      lds_dma16_buf(which ? vrs : krs, voff, so + (uint32_t)(which * kTile + blk * 1024));
    }
  };
  issue(0, kt0, false);
  issue(1, min(kt0 + 1, kt1), kt0 + 1 > kt1);
  issue(2, min(kt0 + 2, kt1), kt0 + 2 > kt1);

  // ---- Q^T operands ---------------------------------------------------------------------------
  // BF16: per 32-d step c, lane (row col, group grp) holds Q[row][32 c + 8 grp .. + 7].
  // Split: per 128-d step c, lane (col, grp) holds the hi (and lo) codes of Q[row][128 c + 32 grp .. + 31].
  const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                     (int64_t)hq * p.q_stride_head;
  constexpr int NQ = SPLITQ ? kD / 128 : kD / 32;
  bf16x8_t qb16[SPLITQ ? 1 : NQ];
  i32x8_t qhi[SPLITQ ? NQ : 1], qlo[SPLITQ ? NQ : 1];
  if constexpr (!SPLITQ) {
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      const bf16x8_t z = {};
      qb16[c] = rvalid ? *reinterpret_cast<const bf16x8_t*>(qp + 32 * c + 8 * grp) : z;
    }
  } else {
    // the row's largest magnitude (its 4 lane groups hold the row), then the split
    u32x4_t raw[NQ][4];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        raw[c][k] = *reinterpret_cast<const u32x4_t*>(qp + 128 * c + 32 * grp + 8 * k);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          amax = fmaxf(amax, fabsf(__uint_as_float(raw[c][k][x] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(raw[c][k][x] & 0xffff0000u)));
        }
      }
    }
    amax = max_over_groups(amax);
    const int e = split_exponent(amax);
    const float up = __uint_as_float((uint32_t)(127 + e) << 23);
    cs *= __uint_as_float((uint32_t)(127 - e) << 23);
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      uint64_t hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        split8_bf16_e4m3(raw[c][k], up, hi[k], lo[k]);
        if (!rvalid) hi[k] = lo[k] = 0;
      }
      qhi[c] = i32x8_t{(int)(uint32_t)hi[0], (int)(hi[0] >> 32), (int)(uint32_t)hi[1], (int)(hi[1] >> 32),
                       (int)(uint32_t)hi[2], (int)(hi[2] >> 32), (int)(uint32_t)hi[3], (int)(hi[3] >> 32)};
      qlo[c] = i32x8_t{(int)(uint32_t)lo[0], (int)(lo[0] >> 32), (int)(uint32_t)lo[1], (int)(lo[1] >> 32),
                       (int)(uint32_t)lo[2], (int)(lo[2] >> 32), (int)(uint32_t)lo[3], (int)(lo[3] >> 32)};
    }
  }

  f32x4_t oacc[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  float o_scale = 1.f;                 // pending rescale of O (lazy max moved), per row
  bool o_rescale = false;              // ... for some row of the wave

  // per-lane LDS offsets: the K row of each 16-key block for the S^T A operand, and the V^T
  // transposing reads (this lane supplies source row j = col / 2, 8-byte half col % 2; its group
  // reads keys 8 grp .. 8 grp + 7 of the tile)
  const int k_lane0 = lane_offset(block_key(0, col) * kRS + (SPLITQ ? 32 : 8) * grp);
  const int k_lane1 = lane_offset(block_key(1, col) * kRS + (SPLITQ ? 32 : 8) * grp);
  const int v_lane = lane_offset((8 * grp + (col >> 1)) * kRS + 8 * (col & 1));

  // S^T = K Q^T of the tile in stage st, two 16-key blocks.  Operands stream in two MFMAs ahead of
  // their use through a ring of three registers (fixed by scheduling barriers).
  //   BF16: op j = (32-d step j / 2, block j % 2), K bytes converted exactly to bf16.
  //   Split: op j = (128-d step j / 2, block j % 2), the MFMA pair K hi + (K lo) 2^-4.
  typedef typename std::conditional<SPLITQ, i32x8_t, bf16x8_t>::type kop_t;
  auto qk = [&](int st, f32x4_t (&sacc)[2]) __attribute__((always_inline)) {
    const uint8_t* kst = lds + st * kStage;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int NOPS = 2 * NQ;
    kop_t buf[3];
#pragma unroll
    for (int j = 0; j < NOPS + 2; ++j) {
      if (j < NOPS) {
        const int kb = j & 1, c = j >> 1;
        const uint8_t* kp = kst + (kb ? k_lane1 : k_lane0);
        if constexpr (SPLITQ) {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(kp + 128 * c);
          const u32x4_t y = *reinterpret_cast<const u32x4_t*>(kp + 128 * c + 16);
          buf[j % 3] = i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        } else {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(kp + 32 * c);
          buf[j % 3] = e4m3x8_to_bf16(x[0], x[1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (j >= 2) {
        const int i = j - 2, kb = i & 1, c = i >> 1;
        if constexpr (SPLITQ) {
          sacc[kb] = mfma_fp8_16x16x128(buf[i % 3], qhi[c], sacc[kb], kE8M0One);
          sacc[kb] = mfma_fp8_16x16x128(buf[i % 3], qlo[c], sacc[kb], kE8M0Sixteenth);
        } else {
          sacc[kb] = mfma_bf16_16x16x32(buf[i % 3], qb16[c], sacc[kb]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // softmax of tile kt: mask (boundary tiles), lazy max, O rescale, running sum, P operands.
  // S^T value i of block kb in this lane is row 4 grp + i, i.e. key block_key(kb, 4 grp + i)
  // = 8 grp + 4 kb + i of the tile.
  // BF16: the P^T operand is P of keys 8 grp + 0..7, as bf16.
  // Split: P <= 2^4 (lazy max at 2^4) and block kb's operand is 16 hi in bytes 0-3 and lo in bytes
  // 4-7 for keys 8 grp + 4 kb + 0..3, with hi = E4M3(P), lo = E4M3(16 (P - hi)).
  constexpr float kLazy = SPLITQ ? 4.0f : 8.0f;
  bf16x8_t pb16;
  uint64_t p8[2];
  auto softmax = [&](int kt, f32x4_t (&sacc)[2]) __attribute__((always_inline)) {
    float sv[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[kb][i] = sacc[kb][i] * cs;
    }
    const int j0 = kt * kBK;
    if (!(j0 >= wfull_lo && j0 + kBK - 1 <= wpf)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 8 * grp + 4 * kb + i;
          const bool vis = j <= pos && (W < 1 || j > pos - W);
          sv[kb][i] = vis ? sv[kb][i] : kNegInf;
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mx = fmaxf(mx, fmaxf(fmaxf(sv[kb][0], sv[kb][1]), fmaxf(sv[kb][2], sv[kb][3])));
    mx = max_over_groups(mx);
    const bool grow = mx > m_run + kLazy;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));   // 1 where not grown
      l_run *= alpha;
      if (__any(grow && m_run != kNegInf)) {
        o_scale *= alpha;              // applied to O before the tile's PV
        o_rescale = true;
      }
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float pall[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[kb][i] - m_use);
      l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
      if constexpr (SPLITQ) {
        int hc = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
        hc = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], hc, true);
        const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hc, false);
        const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hc, true);
        int h16 = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * h01[0], 16.0f * h01[1], 0, false);
        h16 = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * h23[0], 16.0f * h23[1], h16, true);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (pv[0] - h01[0]), 16.0f * (pv[1] - h01[1]), 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (pv[2] - h23[0]), 16.0f * (pv[3] - h23[1]), lo, true);
        p8[kb] = (uint64_t)(uint32_t)h16 | ((uint64_t)(uint32_t)lo << 32);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pall[4 * kb + i] = pv[i];
      }
    }
    if constexpr (!SPLITQ)
      pb16 = bf16x8_t{(__bf16)pall[0], (__bf16)pall[1], (__bf16)pall[2], (__bf16)pall[3],
                      (__bf16)pall[4], (__bf16)pall[5], (__bf16)pall[6], (__bf16)pall[7]};
    // P and the running sum are needed here: the compiler would otherwise sink the exponentials
    // past the barrier that may follow, into the MFMA half of the interval
    if constexpr (SPLITQ) asm volatile("" ::"v"(p8[0]), "v"(p8[1]), "v"(l_run));
    else asm volatile("" ::"v"(pb16), "v"(l_run));
  };

  // O^T += V^T P^T with the V tile in stage st.  Transposing read t gives this lane, for d row
  // 16 t + col, the 8 keys 8 grp + 0..7.  O^T tile t, lane (col, grp) holds d = 16 t + 4 grp + i of
  // row col.  Operands stream two MFMAs ahead as in qk.
  //   BF16: op t: one MFMA with the 8 keys as bf16.
  //   Split: op t: two MFMAs, keys 0-3 and 4-7 of the 8, each with its 4 V bytes twice (against
  //   16 hi and lo of P).
  auto pv = [&](int st) __attribute__((always_inline)) {
    if (o_rescale) {
#pragma unroll
      for (int t = 0; t < kNT; ++t) oacc[t] *= o_scale;
      o_scale = 1.f;
      o_rescale = false;
    }
    const uint8_t* vp = lds + (st * kStage + kTile + v_lane);
    constexpr int NOPS = kNT;
    uint64_t buf[3];
#pragma unroll
    for (int j = 0; j < NOPS + 2; ++j) {
      if (j < NOPS) {
        const i32x2_t v2 = lds_read_tr8(vp + 16 * j);
        buf[j % 3] = (uint64_t)(uint32_t)v2[0] | ((uint64_t)(uint32_t)v2[1] << 32);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (j >= 2) {
        const int t = j - 2;
        const uint64_t v8 = buf[t % 3];
        if constexpr (SPLITQ) {
          const uint64_t lo4 = v8 & 0xffffffffull, hi4 = v8 >> 32;
          oacc[t] = mfma_fp8_16x16x32(lo4 | (lo4 << 32), p8[0], oacc[t]);
          oacc[t] = mfma_fp8_16x16x32(hi4 | (hi4 << 32), p8[1], oacc[t]);
        } else {
          oacc[t] = mfma_bf16_16x16x32(e4m3x8_to_bf16((uint32_t)v8, (uint32_t)(v8 >> 32)), pb16, oacc[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop -------------------------------------------------------------------------------
  // Tile x lives in stage (x - kt0) mod 4.  The two waves of a SIMD (wave w and w + 4) run half a
  // tile apart, so that one's softmax overlaps the other's MFMAs.  Between barriers t - 1 and t:
  //   group A (waves 0-3): PV(t), QK(t + 1) | softmax(t + 1)
  //   group B (waves 4-7): softmax(t)       | PV(t), QK(t + 1)
  // Both read tiles t and t + 1 there, so after barrier t - 1 the stage of tile t - 1 is free and
  // takes tile t + 3, which has until barrier t + 1 to land.  Each group issues its share of those
  // loads at the start of its softmax half, while its partner wave runs MFMAs (issued at the start
  // of the MFMA half instead, they cost 11% with split Q).  The O rescale of a moved lazy max is
  // applied at the next PV, so O is updated in one place (two places made the compiler spill O).
  const bool group_a = wave < kNW / 2;
  auto sees = [&](int t) __attribute__((always_inline)) { return t >= wt0 && t <= wt1; };
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();                     // tiles kt0 .. kt0 + 2 are in LDS
  f32x4_t sacc[2];
  if (sees(kt0)) {
    qk(0, sacc);
    if (group_a) softmax(kt0, sacc);
  }
  for (int t = kt0; t <= kt1; ++t) {
    const int st = (t - kt0) & (kNS - 1), st1 = (st + 1) & (kNS - 1);
    const bool next = t + 1 <= kt1 && sees(t + 1);
    if (!group_a) {
      issue((st + 3) & (kNS - 1), min(t + 3, kt1), t + 3 > kt1);
      if (sees(t)) softmax(t, sacc);
    }
    if (sees(t)) pv(st);
    if (next) qk(st1, sacc);
    asm volatile("" ::"v"(sacc[0]), "v"(sacc[1]));   // S stays in this half (not sunk past the barrier)
    if (group_a) {
      issue((st + 3) & (kNS - 1), min(t + 3, kt1), t + 3 > kt1);
      if (next) softmax(t + 1, sacc);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMaxI));   // tile t + 2 has landed (this wave's part)
    __syncthreads();                   // ... every wave's part, and every wave is done with tile t
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // nothing may land after the block ends

  // ---- epilogue: O through LDS, whole-row stores -------------------------------------------------
  l_run = sum_over_groups(l_run);
  const float inv = l_run > 0.f ? vd / (SPLITQ ? 16.0f * l_run : l_run) : 0.f;   // (split P accumulates 16 O)
  constexpr int ORS = 2 * kD + 16;                  // LDS row stride of the staged O (bytes)
  static_assert(kNW * kRW * ORS <= kNS * kStage, "the staged O fits the stage ring");
  __syncthreads();
  uint8_t* const ow = lds + wave * (kRW * ORS);
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const bf16x4_t o = {(__bf16)(oacc[t][0] * inv), (__bf16)(oacc[t][1] * inv), (__bf16)(oacc[t][2] * inv),
                        (__bf16)(oacc[t][3] * inv)};
    *reinterpret_cast<bf16x4_t*>(ow + col * ORS + 2 * (16 * t + 4 * grp)) = o;
  }
  constexpr int CPR = kD / 8;                       // 16-byte chunks per row
  __bf16* const obase = reinterpret_cast<__bf16*>(p.out);
#pragma unroll
  for (int k = 0; k < kRW * CPR / 64; ++k) {
    const int c = 64 * k + lane;
    const int row = c / CPR, cc = c % CPR;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ow + row * ORS + 16 * cc);
    const int rr = wr0 + row;
    if (rr < nrows) {
      const int tk = rr / G, hh = h * G + rr % G;
      // (non-temporal: O is written once)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(obase + (int64_t)(t0 + tk) * p.out_stride_tok +
                                                                (int64_t)hh * p.out_stride_head + 8 * cc));
    }
  }
  if (p.lse && grp == 0 && rvalid)
    p.lse[(int64_t)(t0 + tok) * p.hq + hq] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
}

hipError_t launch_prefill_wide(const AttnParams& p, bool split_q, hipStream_t stream) {
  const int64_t nqb = ((int64_t)p.max_seqlen_q * p.group + kBM - 1) / kBM;
  if (nqb <= 0 || p.hkv <= 0 || p.batch <= 0) return hipSuccess;
  const int64_t grid = nqb * p.hkv * p.batch;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
  if (split_q)
    hipLaunchKernelGGL(prefill_wide_kernel<true>, dim3((unsigned)grid), dim3(kNW * 64), 0, stream, p, (int32_t)nqb,
                       p.block_table);
  else
    hipLaunchKernelGGL(prefill_wide_kernel<false>, dim3((unsigned)grid), dim3(kNW * 64), 0, stream, p, (int32_t)nqb,
                       p.block_table);
  return hipGetLastError();
}

}  // namespace fp8attn
