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
//    (global_load_lds_dwordx4), double buffered, with one barrier per tile.  Key rows are padded
//    to D + 16 bytes so that the MFMA operand reads below are free of bank conflicts.
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
#include "device.h"
#include "params.h"

namespace fp8attn {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kSplitPKeys = 512;
constexpr int kE8M0One = 127;        // E8M0 scale 2^0
constexpr int kE8M0Sixteenth = 123;  // E8M0 scale 2^-4
constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ f32x16_t mfma_fp8_32x32x64(const i32x8_t& a, const i32x8_t& b, f32x16_t c,
                                                      int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, scale_b);
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
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

// MFMA row m of a 32-key half tile holds key kperm(m): bits 2 and 3 of m swapped.
__device__ __forceinline__ int kperm(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D>
struct PrefillShape {
  static constexpr int NW = 8;            // waves per block
  static constexpr int RW = 32;           // rows per wave
  static constexpr int BM = NW * RW;      // rows per block
  static constexpr int BK = 64;           // keys per tile (one kernel page)
  static constexpr int NCH = D / 16;      // 16-byte chunks per key row
  static constexpr int KSTEP = D / 64;    // QK^T k-steps (64 d each)
  static constexpr int NDT = D / 32;      // O^T tiles of 32 d-rows
  static constexpr int RS = D + 16;       // LDS row stride: one 16-byte pad per key row
  static constexpr int SLOTS = NCH + 1;   // 16-byte LDS slots per key row
  static constexpr int TILE = BK * RS;    // bytes of one K (or V) tile in LDS
  static constexpr int LOADS = 2 * SLOTS; // wave-wide 1 KiB load instructions per K+V tile
  static constexpr int MAXI = (LOADS + NW - 1) / NW;  // load instructions per wave per tile
  static_assert(D == 64 || D == 256, "head dim");
};

// Issue this wave's direct-to-LDS loads of one K and one V tile (instructions wave, wave + 8,
// ...).  lds_stage points at [K tile | V tile] of one stage.
template <int D>
__device__ __forceinline__ void load_tile_to_lds(const uint8_t* ktb, const uint8_t* vtb, const uint32_t* loff,
                                                 int wave, uint8_t* lds_stage) {
  using S = PrefillShape<D>;
#pragma unroll
  for (int t = 0; t < S::MAXI; ++t) {
    const int ins = wave + S::NW * t;
    if (ins < S::LOADS) {
      const int which = ins / S::SLOTS;
      const int blk = ins % S::SLOTS;
      __builtin_amdgcn_global_load_lds((which ? vtb : ktb) + loff[t],
                                       (__attribute__((address_space(3))) void*)(lds_stage + which * S::TILE + blk * 1024),
                                       16, 0, 0);
    }
  }
}

template <int D, bool SPLIT>
__global__ void __launch_bounds__(512) prefill_fp8_kernel(const AttnParams p, int32_t nqb) {
  using S = PrefillShape<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][S::TILE];   // [stage][K|V][key row]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;          // this lane's row within the wave (MFMA column)
  const int lg = lane >> 5;          // 32-lane half

  // ---- work item: (sequence, kv head) outer, q block descending (heaviest first) -----------
  int64_t id = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = nqb - 1 - (int)(id % nqb); id /= nqb;
  const int h = (int)(id % p.hkv); id /= p.hkv;
  const int b = (int)id;
  const int G = p.group;
  const int t0 = p.cu_seqlens_q[b];
  const int ql = p.cu_seqlens_q[b + 1] - t0;
  const int L = p.seqlens_k[b];
  const int nrows = ql * G;
  const int r0 = qb * S::BM;
  if (r0 >= nrows) return;
  const int W = p.window;
  const int rlast = min(r0 + S::BM, nrows) - 1;
  const int pf = L - ql + r0 / G;           // first row's position
  const int pl = L - ql + rlast / G;        // last row's position
  const int k_lo = W >= 1 ? max(0, pf - W + 1) : 0;
  const int kt0 = k_lo / S::BK, kt1 = pl / S::BK;   // inclusive tile range of the block

  // this wave's rows and key range
  const int wr0 = r0 + wave * S::RW;
  const bool wave_active = wr0 < nrows;
  const int wrl = min(wr0 + S::RW, nrows) - 1;
  const int wpf = L - ql + (wave_active ? wr0 : rlast) / G;
  const int wpl = L - ql + (wave_active ? wrl : rlast) / G;
  const int wk_lo = W >= 1 ? max(0, wpf - W + 1) : 0;
  const int wfull_lo = W >= 1 ? wpl - W + 1 : 0;     // keys [wfull_lo, wpf] are visible to every row
  // this lane's row
  const int r = wr0 + lr;
  const bool rvalid = r < nrows;
  const int tok = (rvalid ? r : rlast) / G;
  const int hq = h * G + (rvalid ? r : rlast) % G;
  const int pos = L - ql + tok;
  // blocks whose first row sees few keys belong to the split-P instance, the rest to the other
  const int min_keys = W >= 1 ? min(pf + 1, W) : pf + 1;
  if ((min_keys < kSplitPKeys) != SPLIT) return;

  const float kd = p.k_descale ? p.k_descale[b * p.ds_stride_b + h * p.ds_stride_h] : 1.0f;
  const float vd = p.v_descale ? p.v_descale[b * p.ds_stride_b + h * p.ds_stride_h] : 1.0f;
  const float qd = p.q_descale ? p.q_descale[0] : 1.0f;
  const float cs = p.scale_log2 * kd * qd;

  // ---- Q^T operand: lane (row lr, half lg) holds Q[row][64c + 32lg .. +32] per k-step c -------
  i32x8_t qop[S::KSTEP];
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)(t0 + tok) * p.q_stride_tok +
                        (int64_t)hq * p.q_stride_head + 32 * lg;
#pragma unroll
    for (int c = 0; c < S::KSTEP; ++c) {
      u32x4_t a = {0, 0, 0, 0}, bb = {0, 0, 0, 0};
      if (rvalid) {
        a = *reinterpret_cast<const u32x4_t*>(qp + 64 * c);
        bb = *reinterpret_cast<const u32x4_t*>(qp + 64 * c + 16);
      }
      qop[c] = i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bb[0], (int)bb[1], (int)bb[2], (int)bb[3]};
    }
  }

  f32x16_t oacc[S::NDT];
#pragma unroll
  for (int t = 0; t < S::NDT; ++t) oacc[t] = f32x16_t{};
  float m_used = kNegInf, l_run = 0.f;

  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const uint8_t* kbase = p.k_cache + (int64_t)h * p.kv_stride_head;
  const uint8_t* vbase = p.v_cache + (int64_t)h * p.kv_stride_head;
  const int64_t sT = p.kv_stride_tok, sP = p.kv_stride_page;
  const int ps = p.page_size;

  // ---- tile loader: HBM -> LDS directly (global_load_lds_dwordx4, 16 bytes per lane) ---------
  // A wave-wide instruction fills 64 consecutive 16-byte LDS slots (lane i -> slot i).  Key rows
  // occupy D/16 + 1 slots: D bytes of data and one pad slot, which receives a duplicate of the
  // row's first chunk.  The pad makes the row stride D + 16 bytes (see the operand reads).
  // Wave w issues instructions w, w + 8, ...; each lane's byte offset inside the 64-key tile is
  // fixed, so it is computed once and every load is a scalar tile base plus that offset.
  uint32_t loff[S::MAXI];
#pragma unroll
  for (int t = 0; t < S::MAXI; ++t) {
    const int ins = wave + S::NW * t;
    const int sl = (ins % S::SLOTS) * 64 + lane;
    const int row = sl / S::SLOTS, posn = sl % S::SLOTS;
    loff[t] = (uint32_t)(row * sT) + 16u * (uint32_t)(posn == S::NCH ? 0 : posn);
  }
  auto issue = [&](int kt, int stage) {
    const int j0 = kt * S::BK;
    int pidx, slot0;
    if (ps == S::BK) { pidx = kt; slot0 = 0; } else { pidx = j0 / ps; slot0 = j0 - pidx * ps; }
    const int64_t tile_off = (int64_t)bt[pidx] * sP + (int64_t)slot0 * sT;
    load_tile_to_lds<D>(kbase + tile_off, vbase + tile_off, loff, wave, &lds[stage][0][0]);
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

  auto compute = [&](int kt, int stage) {
    const uint8_t* ktile = lds[stage][0];
    const uint8_t* vtile = lds[stage][1];
    const int j0 = kt * S::BK;
    // S^T for the two 32-key halves of the tile
    f32x16_t sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = f32x16_t{};
      const int krow = 32 * st + kperm(lr);       // A operand row m holds key kperm(m)
      const uint8_t* rowp = ktile + krow * S::RS + 32 * lg;
#pragma unroll
      for (int c = 0; c < S::KSTEP; ++c) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(rowp + 64 * c);
        const u32x4_t y = *reinterpret_cast<const u32x4_t*>(rowp + 64 * c + 16);
        const i32x8_t ka = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        sacc[st] = mfma_fp8_32x32x64(ka, qop[c], sacc[st], kE8M0One);
      }
    }
    // mask (boundary tiles only) and tile max, on unscaled scores (the scale is positive)
    const bool need_mask = !(j0 >= wfull_lo && j0 + S::BK - 1 <= wpf);
    float mxr = kNegInf;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = sacc[st][i];
        if (need_mask) {
          // value i of this lane is S^T row 8*(i/4) + 4*lg + i%4, i.e. key kperm(that row)
          const int j = j0 + 32 * st + ((i >> 3) << 4) + (lg << 3) + (((i >> 2) & 1) << 2) + (i & 3);
          const bool vis = j <= pos && (W < 1 || j > pos - W);
          v = vis ? v : kNegInf;
          sacc[st][i] = v;
        }
        mxr = fmaxf(mxr, v);
      }
    }
    mxr = fmaxf(mxr, __shfl_xor(mxr, 32, 64));
    const float mx = mxr * cs;
    // lazy maximum: move it only when the tile exceeds it by more than 2^8
    const bool grow = mx > m_used + kLazyMax;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_used;
      const float alpha = fast_exp2(m_used - (m_new == kNegInf ? 0.f : m_new));
      if (grow) {
        l_run *= alpha;
        m_used = m_new;
      }
      const float a = grow ? alpha : 1.0f;
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) oacc[t] *= a;
    }
    const float neg_m = m_used == kNegInf ? 0.f : -m_used;
    // P = exp2(s * cs - m), packed to E4M3 in the B-operand slot order (slot 16*st + i)
    i32x8_t pb, pl = {};
    float lsum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          e[k] = fast_exp2(__builtin_fmaf(sacc[st][4 * q4 + k], cs, neg_m));
          lsum += e[k];
        }
        const uint32_t hi = pack4_e4m3(e[0], e[1], e[2], e[3]);
        pb[4 * st + q4] = (int)hi;
        if constexpr (SPLIT) {
          float back[4], rsd[4];
          unpack4_e4m3(hi, back);
#pragma unroll
          for (int k = 0; k < 4; ++k) rsd[k] = (e[k] - back[k]) * 16.0f;
          pl[4 * st + q4] = (int)pack4_e4m3(rsd[0], rsd[1], rsd[2], rsd[3]);
        }
      }
    }
    l_run += lsum;
    // O^T += V^T * P^T : for each 32-row d tile, gather 32 keys per lane with 4 transposing reads
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt) {
      const int col = 16 * dt + (D / 2) * tr_blk + 8 * tr_h;
      i32x8_t va;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // slots 8q..8q+7 of group lg hold the 8 consecutive keys 32(q/2) + 16(q%2) + 8*lg + j
        const int key = 32 * (q >> 1) + 16 * (q & 1) + 8 * lg + tr_j;
        const uint8_t* src = vtile + key * S::RS + col;
        const i32x2_t v2 = lds_read_tr8(src);
        va[2 * q] = v2[0];
        va[2 * q + 1] = v2[1];
      }
      oacc[dt] = mfma_fp8_32x32x64(va, pb, oacc[dt], kE8M0One);
      if constexpr (SPLIT) oacc[dt] = mfma_fp8_32x32x64(va, pl, oacc[dt], kE8M0Sixteenth);
    }
  };

  // ---- main loop over key tiles (2-stage LDS ring, one barrier per tile) ---------------------
  // Iteration kt: wait for this wave's loads of tile kt, barrier (every wave's loads of kt have
  // landed and every wave has finished tile kt-1), start loading tile kt+1 into the stage that
  // held tile kt-1, then compute tile kt.
  issue(kt0, 0);
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int stage = (kt - kt0) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt < kt1) issue(kt + 1, stage ^ 1);
    const int j0 = kt * S::BK;
    if (wave_active && j0 + S::BK > wk_lo && j0 <= wpl) compute(kt, stage);
  }

  // ---- epilogue ------------------------------------------------------------------------------
  l_run += __shfl_xor(l_run, 32, 64);
  if (!rvalid) return;
  const float inv = l_run > 0.f ? vd / l_run : 0.f;
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
  if (p.lse && lg == 0)
    p.lse[(int64_t)(t0 + tok) * p.hq + hq] = l_run > 0.f ? (m_used + fast_log2(l_run)) * kLn2 : kNegInf;
}

hipError_t launch_prefill_fp8(const AttnParams& p, int head_dim, hipStream_t stream) {
  const int G = p.group;
  const int64_t nqb = ((int64_t)p.max_seqlen_q * G + 255) / 256;
  const int64_t grid = nqb * p.hkv * p.batch;
  if (grid <= 0) return hipSuccess;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
  // Every block index is launched twice, once per instance; each block runs in exactly one of
  // them (decided by the key count its first row sees) and returns at once in the other.
  const dim3 g((unsigned)grid), blk(512);
  if (head_dim == 256) {
    hipLaunchKernelGGL((prefill_fp8_kernel<256, false>), g, blk, 0, stream, p, (int32_t)nqb);
    hipLaunchKernelGGL((prefill_fp8_kernel<256, true>), g, blk, 0, stream, p, (int32_t)nqb);
  } else {
    hipLaunchKernelGGL((prefill_fp8_kernel<64, false>), g, blk, 0, stream, p, (int32_t)nqb);
    hipLaunchKernelGGL((prefill_fp8_kernel<64, true>), g, blk, 0, stream, p, (int32_t)nqb);
  }
  return hipGetLastError();
}

}  // namespace fp8attn
