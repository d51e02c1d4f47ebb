// Multi-token decode at head dim 512 with bf16 queries: steps with more than 16 query rows per
// (sequence, kv head), such as speculative-decode verification, where GQA 8 times 4 tokens (the
// target token and three drafts) meet one long cached context (vLLM PR #60372, Validation: MTP with
// three speculative tokens over a shared prefix; Overview: the full-attention layers at head dim 512
// keep BF16 queries; review thread: the d512 FP8-MMA kernel with its split QK accumulation).
//
// What it computes: the masked softmax attention of the decode kernel's two bf16-Q modes, for a
// tile of 32 query rows over one split of the key range:
//   SPLIT = true (q_dtype BF16_SPLIT): Q per row as 2^-e (hi + lo / 16) in E4M3 (exact for bf16
//     values), QK^T and PV on the FP8 MFMA, P as two E4M3 terms;
//   SPLIT = false (q_dtype BF16): K and V converted exactly to bf16, BF16 MFMAs, P rounded to bf16.
//
// Design (gfx950, wave64, 640 threads = 10 waves, one block per compute unit):
//  * Every K/V byte of the tile's key range is loaded once for all 32 rows: 32-key tiles go from
//    HBM straight into LDS (buffer loads with an LDS destination, range ending at the sequence
//    length) through a K ring of five stages and a V ring of four.  Key rows are padded to 528
//    bytes (a copy of the row's first 16 bytes), which makes the operand reads conflict-free.
//  * Three roles.  Two loader waves (8: K, 9: V) only issue the tile loads, so no computing wave
//    ever stalls on a full load queue.  Four QK waves: wave (parity, row half) computes S^T = K Q^T
//    for the 16 rows of its half and all 32 keys of every other tile (scaled 16x16x128 FP8 MFMA
//    with the lo terms of Q at operand scale 2^-4, or 16x16x32 BF16), half the head dim in each of
//    two intervals, then that tile's softmax in the next interval while the MFMAs of its next tile
//    run.  Four PV waves each own 128 of the 512 head-dim columns of O for all 32 rows and run
//    O^T += V^T P^T (scaled 32x32x64 FP8, or 32x32x16 BF16).  One barrier per tile; tile x: QK^T
//    in intervals x - 3 and x - 2, softmax in x - 1, PV in x.
//  * No running maximum is shared between waves.  A QK wave keeps, per row, an integer reference
//    m that moves lazily (when the tile exceeds it by more than 2, to the ceiling of the tile's
//    row maximum: the only cross-lane reduction, rare after the first tiles), so that
//    P = 2^(s - m + 6) <= 2^8, and it publishes m - 6 with P and its lanes' partial row sums.  The
//    PV waves bring each tile from its reference to their common one by an exact power of two.
//    With split Q that is the PV MFMA's per-lane E8M0 operand scale: on gfx950 the B scale of lane
//    n + 32 kb covers bytes 16 kb .. 16 kb + 15 of both lane groups of column n.  Lane group g
//    holds hi = E4M3(P) of keys 16 g .. 16 g + 15 in bytes 0-15 (scale block 0) and lo =
//    E4M3(P - hi) of the same keys in bytes 16-31 (scale block 1), against the same V bytes twice
//    in A; both blocks carry the tile's scale for row n.  With BF16 Q the PV waves multiply the
//    bf16 P by it.  The common reference moves lazily too (by more than 2^16), with an O rescale
//    by an exact power of two.
#include "device.h"
#include "params.h"

namespace fp8attn {

namespace {

constexpr int kD = 512;
constexpr int kRows = 32;                 // query rows per block
constexpr int kBK = 32;                   // keys per tile
constexpr int kNSK = 5;                   // stages of the K ring
constexpr int kNSV = 4;                   // stages of the V ring
constexpr int kNCH = kD / 16;             // 16-byte chunks per key row
constexpr int kRS = kD + 16;              // LDS row stride (one pad slot)
constexpr int kSlots = kNCH + 1;          // 16-byte LDS slots per key row
constexpr int kRowSlots = kBK * kSlots;   // 1,056 slots of key rows per tile ...
constexpr int kIns = (kRowSlots + 63) / 64;   // ... written by 17 wave-wide loads
constexpr int kTile = kIns * 1024;        // bytes of one stage: rows, then 32 spare slots
constexpr int kPRS = 80;                  // LDS row stride of P: lane group 0 | lane group 1 | pad
constexpr int kPBuf = kRows * kPRS;       // bytes of one P buffer
constexpr int kDT = 4;                    // 32-column O^T tiles per PV wave
constexpr float kLazyQK = 2.0f;           // a QK wave's reference moves when a tile exceeds it by this
constexpr float kSlack = 16.0f;           // the PV reference moves when a tile exceeds it by this
constexpr int kThreads = 640;

// 2^e for an integer-valued float e <= 127 (0 below the fp32 range)
__device__ __forceinline__ float pow2i(float e) { return __builtin_amdgcn_ldexpf(1.0f, (int)fmaxf(e, -200.0f)); }

}  // namespace

template <bool SPLIT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) verify_kernel(const AttnParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- work item: (kv head, split, sequence, row tile), XCD-aware order as in the decode grid ----
  // (32-bit index arithmetic: the host keeps the grid below 2^31)
  uint32_t id = xcd_remap32(blockIdx.x, gridDim.x);
  const uint32_t n_rt = (uint32_t)p.row_groups, n_b = (uint32_t)p.batch, n_s = (uint32_t)p.num_splits;
  const int rt = (int)(id % n_rt); id /= n_rt;
  const int b = (int)(id % n_b); id /= n_b;
  const int s = (int)(id % n_s);
  const int h = (int)(id / n_s);
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
  const int row0 = rt * kRows;
  if (row0 >= nrows) return;
  const int rlast = min(row0 + kRows, nrows) - 1;
  const int p_first = L - ql + row0 / G;
  const int p_last = L - ql + rlast / G;
  const int W = p.window;
  // this split's keys: 16-key units [su0, su1) of the tile's visible range, as in the decode grid
  const int k_lo = W >= 1 ? max(0, p_first - W + 1) : 0;
  const int u_begin = k_lo / 16;
  const int u_end = (p_last + 16) / 16;
  const int su0 = u_begin + s * p.units_per_split;
  const int su1 = min(u_end, su0 + p.units_per_split);
  const bool whole = p.num_splits == 1;
  if (su0 >= su1) {   // nothing visible in this split: neutral partials for the combine
    if (!whole && tid < kRows && row0 + tid < nrows) {
      const int rr = row0 + tid;
      p.part_lse[((int64_t)s * p.total_q + t0 + rr / G) * p.hq + h * G + rr % G] = kNegInf;
    }
    return;
  }
  const int ks0 = 16 * su0, ks1 = 16 * su1;          // keys [ks0, ks1) (masked to each row's range)
  const int kt0 = ks0 / kBK, kt1 = (ks1 - 1) / kBK;  // tiles of the block
  // Tile order: the last nt / 4 tiles of the range are interleaved with the others, one in every
  // four positions.  Where the range ends in keys that no other sequence shares (a shared prefix,
  // then each sequence's own tokens), those tiles miss the caches and come from HBM; in key order
  // they would form the stream's tail in every block at once.  Interleaved, their loads overlap
  // the cache-served ones (spec-verify 0.65 -> 0.63 ms split Q, 0.76 -> 0.73 ms bf16 Q; one in
  // every 2 or 8 positions measured the same or slower).  Position x in [kt0, kt1] holds tile
  // tile_at(x); stages and the softmax references follow the position, masks and page ids the tile.
  const int nt = kt1 - kt0 + 1, nu = nt / 4;
  auto tile_at = [&](int x) __attribute__((always_inline)) -> int {
    const int i = x - kt0;
    return kt0 + ((i & 3) == 3 && (i >> 2) < nu ? nt - nu + (i >> 2) : i - min(i >> 2, nu));
  };
  // keys every row of the block can see inside the split: [full_lo, full_hi]
  const int full_lo = max(W >= 1 ? p_last - W + 1 : 0, ks0);
  const int full_hi = min(p_first, ks1 - 1);

  const float kd = p.k_descale ? kd_raw : 1.0f;
  const float vd = p.v_descale ? vd_raw : 1.0f;

  __shared__ __attribute__((aligned(16))) uint8_t sm_k[kNSK * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t sm_v[kNSV * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t sm_p[2 * kPBuf];
  __shared__ __attribute__((aligned(16))) float sm_m[2][kRows];        // per row: the tile's reference
  __shared__ __attribute__((aligned(16))) float sm_l[2][kRows][4];     // ... and its four partial sums

  if (wave >= 8) {
    // ================================ loader waves =============================================
    // Wave 8 loads K, wave 9 V: 17 wave-wide 16-byte-per-lane loads per tile.  Interval t loads K of
    // tile t + 6 and V of tile t + 3, each into the stage its ring's tile five (four) before left
    // (the QK^T of tile x reads K in intervals x - 3 and x - 2, the PV reads V in interval x).  Before
    // each barrier a loader waits for the loads of two intervals back: a load has two intervals to
    // land.  Loads of tiles past the block's last read the first bytes of its last tile (they only
    // keep the count per interval fixed) into the free stage.  The buffers' range ends with the
    // tile's last key below L, so rows past it read zeros (see the prefill kernels).  Page ids come
    // in with scalar loads, requested an interval ahead.
    const bool is_v = wave == 9;
    const uint8_t* base = (is_v ? p.v_cache : p.k_cache) + (int64_t)h * p.kv_stride_head;
    const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
    const int64_t sT = p.kv_stride_tok, sP = p.kv_stride_page;
    const int ps = p.page_size;
    const int ahead = is_v ? 3 : 6;
    const int nst = is_v ? kNSV : kNSK;
    const uint32_t ring = is_v ? lds_address(sm_v) : lds_address(sm_k);
    uint32_t loff[kIns];
#pragma unroll
    for (int k = 0; k < kIns; ++k) {
      const int sl = k * 64 + lane;
      const int row = sl / kSlots, posn = sl % kSlots;
      loff[k] = sl >= kRowSlots ? 0u : (uint32_t)(row * sT) + 16u * (uint32_t)(posn == kNCH ? 0 : posn);
    }
    auto page_of = [&](int x) __attribute__((always_inline)) { return load_uniform(bt, (tile_at(min(x, kt1)) * kBK) / ps); };
    auto issue = [&](int x, int page) __attribute__((always_inline)) {
      const int kt = tile_at(min(x, kt1));
      const bool idle = x > kt1;
      const int slot0 = kt * kBK - ((kt * kBK) / ps) * ps;
      const int64_t tile_off = (int64_t)page * sP + (int64_t)slot0 * sT;
      const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(kBK, L - kt * kBK))) * (uint32_t)sT;
      const i32x4_t rs = buffer_rsrc(base + tile_off, nrec);
      const uint32_t st = ring + (uint32_t)((x % nst) * kTile);
#pragma unroll
      for (int k = 0; k < kIns; ++k) lds_dma16_buf(rs, idle ? 0u : loff[k], st + (uint32_t)(k * 1024));
    };
    int pg = 0;
    if (!is_v) {
      // K of tiles kt0 .. kt0 + 2 ahead of the loop (the first interval is kt0 - 3)
      issue(kt0, page_of(kt0));
      issue(kt0 + 1, page_of(kt0 + 1));
      issue(kt0 + 2, page_of(kt0 + 2));
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kIns));   // K of tile kt0 has landed
    }
    pg = page_of(kt0 - 3 + ahead);
    __syncthreads();
    for (int t = kt0 - 3; t <= kt1; ++t) {
      issue(t + ahead, pg);
      pg = page_of(t + 1 + ahead);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kIns));   // the loads of interval t - 2 have landed
      __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));           // nothing may land after the block ends
  } else if (wave < 4) {
    // ================================ QK waves =================================================
    const int rh = wave & 1, par = wave >> 1;         // row half; parity of the tiles it computes
    const int col = lane & 15, grp = lane >> 4;
    const int n = 16 * rh + col;                      // this lane's row within the block
    const int r = row0 + n;
    const bool rvalid = r < nrows;
    const int tok = (rvalid ? r : rlast) / G;
    const int hq = h * G + (rvalid ? r : rlast) % G;
    const int pos = L - ql + tok;

    // Q^T operands.  Split: per 128-d step c, lane (col, grp) holds hi and lo of
    // Q[row][128 c + 32 grp .. + 31].  BF16: per 32-d step c, lane (col, grp) holds Q[row][32 c + 8 grp .. + 7].
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                       (int64_t)hq * p.q_stride_head;
    i32x8_t qhi[SPLIT ? 4 : 1], qlo[SPLIT ? 4 : 1];
    bf16x8_t qb[SPLIT ? 1 : 16];
    float cs = p.scale_log2 * kd;
    if constexpr (SPLIT) {
      u32x4_t raw[4][4];
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
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
      for (int c = 0; c < 4; ++c) {
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
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const bf16x8_t z = {};
        qb[c] = rvalid ? *reinterpret_cast<const bf16x8_t*>(qp + 32 * c + 8 * grp) : z;
      }
    }
    // A operand of key block kb: MFMA row col holds key 16 kb + col; lane group grp takes d bytes
    // 128 c + 32 grp .. + 31 (split) or 32 c + 8 grp .. + 7 (BF16)
    const int k_lane = lane_offset(col * kRS + (SPLIT ? 32 : 8) * grp);
    // this lane's P bytes in row n.  Split: lane group kb's 32 bytes (keys 16 kb ..), hi at 4 grp ..
    // and lo at 16 + 4 grp ...  BF16: P of keys 16 kb + 4 grp .. + 3 as bf16, at byte 2 (16 kb + 4 grp).
    const int p_lane = lane_offset(n * kPRS + (SPLIT ? 4 : 8) * grp);

    // Half hf of S^T of tile x (the first or second half of the head dim), both 16-key blocks: every
    // operand read first, then the MFMAs (two independent chains, one per key block).  Split: k-steps
    // 2 hf, 2 hf + 1 of 128 d, K bytes as they are.  BF16: k-steps 8 hf .. 8 hf + 7 of 32 d, K bytes
    // converted exactly to bf16.
    f32x4_t acc[2], done[2];
    auto qk_half = [&](int x, int hf) __attribute__((always_inline)) {
      const uint8_t* kst = sm_k + (x % kNSK) * kTile + k_lane;
      if constexpr (SPLIT) {
        i32x8_t kop[2][2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const uint8_t* kp = kst + 16 * kb * kRS + 128 * (2 * hf + c2);
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kp);
            const u32x4_t bb = *reinterpret_cast<const u32x4_t*>(kp + 16);
            kop[c2][kb] = i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bb[0], (int)bb[1], (int)bb[2], (int)bb[3]};
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (hf == 0) {
          acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int c = 2 * hf + c2;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) acc[kb] = mfma_fp8_16x16x128(kop[c2][kb], qhi[c], acc[kb], kE8M0One);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) acc[kb] = mfma_fp8_16x16x128(kop[c2][kb], qlo[c], acc[kb], kE8M0Sixteenth);
        }
      } else {
        u32x2_t kraw[8][2];
#pragma unroll
        for (int c2 = 0; c2 < 8; ++c2) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            kraw[c2][kb] = *reinterpret_cast<const u32x2_t*>(kst + 16 * kb * kRS + 32 * (8 * hf + c2));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (hf == 0) {
          acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int c2 = 0; c2 < 8; ++c2) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            acc[kb] = mfma_bf16_16x16x32(e4m3x8_to_bf16(kraw[c2][kb][0], kraw[c2][kb][1]), qb[8 * hf + c2], acc[kb]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // softmax of tile x from its S^T (sacc).  The reference m_run (per row) is an integer that moves
    // lazily: only when the tile exceeds it by more than kLazyQK, to the ceiling of the tile's row
    // maximum.  P = 2^(s - m_blk) with m_blk = m_run - 8 + kLazyQK, so P <= 2^8 and the largest P of
    // a tile that moved the reference lies above 2^(7 - kLazyQK), where both E4M3 terms keep their
    // precision.  The lane's partial row sum goes to LDS as it is: the PV waves add the four.
    float m_run = kNegInf;
    auto softmax = [&](int x, const f32x4_t (&sacc)[2]) __attribute__((always_inline)) {
      // value i of block kb in this lane: row n, key 16 kb + 4 grp + i of the tile
      float sv[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kb][i] = sacc[kb][i] * cs;
      }
      const int j0 = tile_at(x) * kBK;
      if (!(j0 >= full_lo && j0 + kBK - 1 <= full_hi)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + 16 * kb + 4 * grp + i;
            const bool vis = j >= ks0 && j < ks1 && j <= pos && (W < 1 || j > pos - W);
            sv[kb][i] = vis ? sv[kb][i] : kNegInf;
          }
        }
      }
      float local = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) local = fmaxf(local, fmaxf(fmaxf(sv[kb][0], sv[kb][1]), fmaxf(sv[kb][2], sv[kb][3])));
      if (__any(local > m_run + kLazyQK)) {
        const float mx = max_over_groups(local);
        if (mx > m_run + kLazyQK) m_run = __builtin_ceilf(mx);
      }
      const float mb = m_run == kNegInf ? 0.f : m_run - (8.0f - kLazyQK);
      float lsum = 0.f;
      uint8_t* pb = sm_p + (x & 1) * kPBuf + p_lane;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[kb][i] - mb);
        lsum += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        if constexpr (SPLIT) {
          const uint32_t hi = pack4_e4m3(pv[0], pv[1], pv[2], pv[3]);
          float back[4];
          unpack4_e4m3(hi, back);
          const uint32_t lo = pack4_e4m3(pv[0] - back[0], pv[1] - back[1], pv[2] - back[2], pv[3] - back[3]);
          *reinterpret_cast<uint32_t*>(pb + 32 * kb) = hi;
          *reinterpret_cast<uint32_t*>(pb + 32 * kb + 16) = lo;
        } else {
          const bf16x4_t pw = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
          *reinterpret_cast<bf16x4_t*>(pb + 32 * kb) = pw;
        }
      }
      sm_l[x & 1][n][grp] = lsum;
      if (grp == 0) sm_m[x & 1][n] = m_run == kNegInf ? kNegInf : m_run - (8.0f - kLazyQK);
    };

    // The loop.  This wave computes the tiles x with x % 2 == par: in interval t it runs the first half
    // of tile t + 3 and the softmax of tile t + 1 (whose S^T the previous interval finished), or the
    // second half of tile t + 2.
    __syncthreads();                                  // K of tile kt0 is in LDS
    for (int t = kt0 - 3; t <= kt1; ++t) {
      if (((t + 3 - par) & 1) == 0) {
        done[0] = acc[0];
        done[1] = acc[1];
        if (t + 3 <= kt1) qk_half(t + 3, 0);
        if (t + 1 >= kt0 && t + 1 <= kt1) softmax(t + 1, done);
      } else {
        if (t + 2 >= kt0 && t + 2 <= kt1) qk_half(t + 2, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
  } else {
    // ================================ PV waves =================================================
    const int v = wave - 4;                           // this wave's 128 head-dim columns: below
    const int n = lane & 31, g = lane >> 5;           // this lane's row (MFMA column), lane group
    // O^T tile dt (0..3) of PV wave v: row m < 16 holds column cb + 16 dt + m and row m >= 16 column
    // cb + 128 + 16 dt + m - 16, with cb = 256 (v / 2) + 64 (v % 2).  The two 16-lane halves of a
    // transposing read then touch bytes 128 apart: with the 528-byte key rows, the read's 32 lanes
    // cover 32 distinct 8-byte slots of a 256-byte window (no bank conflicts).
    const int cb = 256 * (v >> 1) + 64 * (v & 1);
    // V^T transposing reads: this lane supplies key row 16 g + 8 o + (lane % 16) / 2 and 8-byte half
    // lane % 2 at column cb + 16 dt + 128 ((lane / 16) % 2); lane (n, g) receives O^T row n's column
    // of keys 16 g + 8 o .. + 7
    // (BF16: key rows 16 s + 8 g + (lane % 16) / 2 for k-step s)
    const int v_lane = lane_offset(((SPLIT ? 16 : 8) * g + ((lane & 15) >> 1)) * kRS + 128 * ((lane >> 4) & 1) + 8 * (lane & 1));

    f32x16_t oacc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t) oacc[t] = f32x16_t{};
    float m_ref = kNegInf, l_ref = 0.f;
    // the common reference moves lazily, when a tile exceeds it by more than 2^16: O and l are
    // rescaled by an exact power of two
    auto rescale = [&](float m_t) __attribute__((always_inline)) {
      const bool grow = m_t > m_ref + kSlack;
      if (__any(grow)) {
        const float alpha = grow && m_ref != kNegInf ? pow2i(m_ref - m_t) : 1.0f;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= alpha;
        l_ref *= alpha;
        m_ref = grow ? m_t : m_ref;
      }
    };

    __syncthreads();
    for (int t = kt0 - 3; t <= kt1; ++t) {
      if (t >= kt0) {
        // the tile's reference and partial sums for row n, then the common reference (moved lazily)
        const float m_t = sm_m[t & 1][n];
        const f32x4_t lp = *reinterpret_cast<const f32x4_t*>(&sm_l[t & 1][n][0]);
        const uint8_t* prow = sm_p + (t & 1) * kPBuf + n * kPRS;
        const uint8_t* vst = sm_v + (t % kNSV) * kTile + v_lane;
        if constexpr (SPLIT) {
          // P^T operand: lane group g's 32 bytes of row n (hi, then lo, of keys 16 g .. 16 g + 15)
          const u32x4_t p0 = *reinterpret_cast<const u32x4_t*>(prow + 32 * g);
          const u32x4_t p1 = *reinterpret_cast<const u32x4_t*>(prow + 32 * g + 16);
          const i32x8_t pop = {(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3], (int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]};
          // V^T operands: the 16 keys of lane group g, twice (against hi and lo)
          i32x8_t a[kDT];
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
            const i32x2_t v0 = lds_read_tr8(vst + cb + 16 * dt);
            const i32x2_t v1 = lds_read_tr8(vst + 8 * kRS + cb + 16 * dt);
            a[dt] = i32x8_t{v0[0], v0[1], v1[0], v1[1], v0[0], v0[1], v1[0], v1[1]};
          }
          rescale(m_t);
          // E8M0 scale of the tile for this row: 2^(m_t - m_ref) (at most 2^16; a masked tile: 0)
          const int code = m_t == kNegInf ? 0 : 127 + (int)fmaxf(m_t - m_ref, -127.0f);
          if (m_t != kNegInf) l_ref += ((lp[0] + lp[1]) + (lp[2] + lp[3])) * pow2i(m_t - m_ref);
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt)
            oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[dt], pop, oacc[dt], 0, 0, 0, kE8M0One, 0, code);
        } else {
          // P^T operands of k-steps s = 0, 1: row n's bf16 P of keys 16 s + 8 g .. + 7, brought from the
          // tile's reference to the common one (an exact power of two)
          bf16x8_t pop[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) pop[s2] = *reinterpret_cast<const bf16x8_t*>(prow + 32 * s2 + 16 * g);
          // V^T operands: keys 16 s + 8 g .. + 7 of the lane's column, converted exactly to bf16
          u32x2_t vraw[kDT][2];
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const i32x2_t v2 = lds_read_tr8(vst + 16 * s2 * kRS + cb + 16 * dt);
              vraw[dt][s2] = u32x2_t{(uint32_t)v2[0], (uint32_t)v2[1]};
            }
          }
          rescale(m_t);
          if (m_t != kNegInf) l_ref += ((lp[0] + lp[1]) + (lp[2] + lp[3])) * pow2i(m_t - m_ref);
          const float sc = m_t == kNegInf ? 0.f : pow2i(m_t - m_ref);
          if (!__all(sc == 1.0f)) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
              for (int i = 0; i < 8; ++i) pop[s2][i] = (__bf16)((float)pop[s2][i] * sc);
            }
          }
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16(vraw[dt][s2][0], vraw[dt][s2][1]),
                                                                 pop[s2], oacc[dt], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }

    // ---- epilogue: lane (n, g) holds, for O^T tile dt and a = 0..3, rows 8 a + 4 g + 0..3, i.e.
    // columns cb + 16 dt + 8 a + 4 g + 0..3 (a < 2) and cb + 128 + 16 dt + 8 (a - 2) + 4 g + 0..3 ----
    const int r = row0 + n;
    if (r < nrows) {
      const int tk = r / G, hh = h * G + r % G;
      const float inv = l_ref > 0.f ? vd / l_ref : 0.f;
      const float lse2 = l_ref > 0.f ? m_ref + fast_log2(l_ref) : kNegInf;
      if (whole) {
        __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)(t0 + tk) * p.out_stride_tok +
                     (int64_t)hh * p.out_stride_head;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const bf16x4_t o = {(__bf16)(oacc[dt][4 * a4] * inv), (__bf16)(oacc[dt][4 * a4 + 1] * inv),
                                (__bf16)(oacc[dt][4 * a4 + 2] * inv), (__bf16)(oacc[dt][4 * a4 + 3] * inv)};
            *reinterpret_cast<bf16x4_t*>(op + cb + 16 * dt + 8 * a4 + 4 * g + (a4 >= 2 ? 112 : 0)) = o;
          }
        }
        if (p.lse && v == 0 && g == 0) p.lse[(int64_t)(t0 + tk) * p.hq + hh] = lse2 * kLn2;
      } else {
        const int64_t e = ((int64_t)s * p.total_q + t0 + tk) * p.hq + hh;
        float* op = p.part_o + e * kD;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const f32x4_t o = {oacc[dt][4 * a4] * inv, oacc[dt][4 * a4 + 1] * inv, oacc[dt][4 * a4 + 2] * inv,
                               oacc[dt][4 * a4 + 3] * inv};
            *reinterpret_cast<f32x4_t*>(op + cb + 16 * dt + 8 * a4 + 4 * g + (a4 >= 2 ? 112 : 0)) = o;
          }
        }
        if (v == 0 && g == 0) p.part_lse[e] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
      }
    }
  }
}

hipError_t launch_verify(const AttnParams& p, bool split_q, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (split_q) hipLaunchKernelGGL(verify_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL(verify_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8attn
