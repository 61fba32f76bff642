// fa_bwd_kernels.hpp -- kernels of the backward pass of exact attention by
// recomputation, and their launch template. Included by fa_bwd.hip (plain,
// causal and dropout instantiations) and fa_bwd_window.hip (sliding window),
// which are compiled with different register-form options.
//
// The probabilities are never stored: each kernel rebuilds P tile by tile
// from Q, K and the fp32 log-sum-exp the forward saved (aimlrounds
// "FlashAttention", follow-up on why the backward pass recomputes instead of
// storing P). The products are the ones of the standard backward
// (zerotofrontier "Efficient attention: memory-bound", section "Real code
// moves even more"): dV = P^T dO, dP = dO V^T, dS from P and dP, dQ and dK
// from dS, with the softmax Jacobian dS_ij = P_ij (dP_ij - D_i) and
// D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic.
//
// With dropout (the DROP instantiations) both kernels regenerate the
// forward's keep mask from the same Philox contract: dV = (P Z)^T dO / kappa,
// dP is replaced by (dO V^T) Z / kappa, and D_i = rowsum(dO * O) still equals
// sum_j P_ij dP_ij because O already carries the dropout.
//
// Two kernels, no atomics (the result is deterministic), dq first:
//   dq    one workgroup per 32 query rows per wave (8 waves at d = 64, 4 at
//         d = 128), laid out like the forward
//         (S^T = K Q^T, one query per lane): dQ^T = K^T dS^T with K^T from
//         transposed LDS reads. Its prologue also forms each row's
//         D_i = rowsum(dO * O) and LSE * log2(e) and stores them for dkdv
//         (two planes: LSE * log2(e) of every row, then -D).
//   dkdv  one workgroup per 16 or 32 keys per wave of a KV head (K and V
//         fragments held in registers); it walks every query tile of every
//         query head of the group. S = Q K^T puts one key per lane, so P and
//         dS feed dV^T = dO^T P and dK^T = Q^T dS straight from the
//         accumulators; dO^T and Q^T come from ds_read_b64_tr_b16.
//         bwd_dkdv16_kernel (16 keys per wave on 16x16x32 MFMAs, two or four
//         waves per SIMD) serves d = 128 and causal d = 64, with or without a
//         window; bwd_dkdv_kernel (32 keys per wave on 32x32x16 MFMAs)
//         dropout, non-causal d = 64 and the second tiling.
#pragma once
#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

// ----------------------------------------------------------------- dk dv

namespace {

// The 32-key layout (non-causal d = 64, dropout, the second tiling). Defaults:
// 64-row query tiles in two LDS stages; d = 64: 8 waves of 32 keys with the
// small-GEMM interleave hint (iglp 0) ordering the LDS reads among the MFMAs;
// d = 128: 4 waves (the dK/dV accumulators need up to 512 registers per
// wave; 8 waves spill) and no hint. The launch picks other shapes per case
// (non-causal d = 64 runs 4-wave workgroups of 32-row tiles).
template <int D, int NW_ = (D == 64 ? 8 : 4), int BQ_ = 64, int NSTAGE_ = 2, int IGLP_ = (D == 64 ? 0 : -1),
          int OCC_ = 1>
struct DkdvCfg {
  static constexpr int NW = NW_;                     // waves per workgroup
  static constexpr int OCC = OCC_;                   // workgroups per CU the register budget allows
  static constexpr int IGLP = IGLP_;                 // compiler interleave strategy for the body (-1: none)
  static constexpr int NT = 64 * NW;
  static constexpr int BK = 32 * NW;                 // keys per workgroup (32 per wave)
  static constexpr int BQ = BQ_;                     // query rows per tile
  static constexpr int QB = BQ / 32;                 // 32-row blocks per tile
  static constexpr int ROWB = 2 * D;                 // LDS bytes per row (swizzled, unpadded)
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int QTILE = BQ * ROWB;            // one Q (or dO) tile
  // row statistics: the lse2 plane, then the -D plane, each in whole 256-byte wave loads
  static constexpr int SLOT = (BQ * 4 + 255) / 256 * 256;
  static constexpr int STATS = 2 * SLOT;
  static constexpr int STAGE = 2 * QTILE + STATS;
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr int TILE_DMA = 2 * BQ * CH / 64;  // 128-bit wave loads per tile (Q and dO)
  static constexpr int DMA_PER_WAVE = TILE_DMA / NW;
  static constexpr int STAT_DMA = STATS / 256;       // 32-bit wave loads of the statistics
  static constexpr int VM_PER_TILE = DMA_PER_WAVE + STAT_DMA;
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * NW == TILE_DMA, "tile loads must split over the waves");
};

}  // namespace

// One workgroup per BK keys of one KV head; each wave owns 32 keys, with its
// K and V rows held as MFMA B operands. The workgroup walks every query tile
// (BQ rows) of every query head of the group that can see one of its keys:
//   S = Q K^T, dP = dO V^T        (A operands: Q and dO rows from LDS)
//   P = 2^(S c - lse2), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS  (A operands: transposed LDS reads)
// S puts one key per lane, so P and dS feed the second pair of products
// straight from the accumulator registers. Q, dO and the row statistics reach
// LDS through direct-to-LDS loads into a ring of C::NSTAGE tiles (the next
// tile loads while one is consumed; at d = 64 two stages measured fastest);
// tiles are stored unpadded with an XOR swizzle.
template <int D, bool CAUSAL, class C = DkdvCfg<D>, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(C::NT, C::OCC) void bwd_dkdv_kernel(BwdArgs a, int n_ktiles) {
  static_assert(CAUSAL || !WIN, "a sliding window is a causal band");
  static_assert(!(WIN && DROP), "dropout is not offered with a sliding window");
  constexpr int BQ = C::BQ, QB = C::QB, ROWB = C::ROWB, CH = C::CH, QTILE = C::QTILE, STAGE = C::STAGE;
  // dropout: a wave-private 32 x 32 byte tile turns row-major Philox bytes into key columns;
  // rows are 48 bytes apart, which keeps its 128-bit writes and byte reads free of bank conflicts
  constexpr int ZPITCH = 48, ZTILE = 32 * ZPITCH;
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[C::NSTAGE * STAGE + (DROP ? C::NW * ZTILE : 0)];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // Causal without a window, a workgroup takes key tiles p and n - 1 - p, one
  // after the other (the same number of query tiles for every workgroup);
  // otherwise one key tile.
  constexpr bool PAIRK = CAUSAL && !WIN;
  const int n_units = PAIRK ? (n_ktiles + 1) / 2 : n_ktiles;
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = (int)(t % (uint32_t)n_units);
  const int bhk = (int)(t / (uint32_t)n_units);
  const int b = bhk / a.Hkv, hk = bhk - b * a.Hkv;
  const int G = a.Hq / a.Hkv;

  // One key tile kt of this workgroup.
  auto key_tile = [&](const int kt) __attribute__((always_inline)) {
    const int k0 = kt * C::BK;
    const int kw0 = k0 + wave * 32;                 // first key of this wave
    const int key = kw0 + col;                      // this lane's key
    const int shift = a.Tk - a.Tq;
    const size_t kvoff = (size_t)bhk * a.Tk * D;

    // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T.
    bf16x8 kf[D / 16], vf[D / 16];
    {
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + kvoff, (uint32_t)a.Tk * D * 2);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + kvoff, (uint32_t)a.Tk * D * 2);
      const uint32_t base = key < a.Tk ? (uint32_t)(key * D + 8 * half) * 2 : kOutOfRange;
  #pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        kf[ks] = as_bf16x8(buf_load_b128(krs, base + ks * 32));
        vf[ks] = as_bf16x8(buf_load_b128(vrs, base + ks * 32));
      }
    }

    f32x16 dv_acc[D / 32], dk_acc[D / 32];
  #pragma unroll
    for (int db = 0; db < D / 32; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) {
        dv_acc[db][r] = 0.f;
        dk_acc[db][r] = 0.f;
      }

    // Query tiles that can see any key of this workgroup, for each query head of the group.
    int qt_begin = 0;
    if (CAUSAL) qt_begin = max(0, k0 - shift) / BQ;
    int n_qt = (a.Tq + BQ - 1) / BQ;
    if (WIN) {   // rows past the last key's window see none of these keys
      const int last_row = k0 + C::BK - 1 - shift + a.window - 1;
      n_qt = last_row < 0 ? 0 : min(n_qt, last_row / BQ + 1);
    }
    const int per_head = max(0, n_qt - qt_begin);
    const int n_iter = per_head * G;

    // This thread's share of the tile loads: physical chunk p of the tile holds
    // logical chunk p ^ swz(row) of its row.
    uint32_t dma_off[C::DMA_PER_WAVE], dma_dst[C::DMA_PER_WAVE];
    bool dma_is_do[C::DMA_PER_WAVE];
  #pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
      const int n = wave * C::DMA_PER_WAVE + i;
      const int m = n % (C::TILE_DMA / 2);
      dma_is_do[i] = n >= C::TILE_DMA / 2;
      const int p = 64 * m + lane;
      const int r = p / CH, pc = p % CH;
      dma_off[i] = (uint32_t)(r * D + (pc ^ swz<D>(r)) * 8) * 2;
      dma_dst[i] = (dma_is_do[i] ? QTILE : 0) + m * 1024;
    }
    const size_t plane = (size_t)a.B * a.Hq * a.Tq;   // -D plane of the statistics workspace

    // Iteration order. The workgroups resident on one XCD hold consecutive key
    // tiles of one KV head.
    //   * Without a window: query tiles from the last one down to the first
    //     that sees this workgroup's keys, every query head of the group per
    //     tile. The resident workgroups start on the same (tile, head) and walk
    //     in step, so each Q/dO tile they read is fetched once into the XCD's L2.
    //   * With a window each workgroup sees only a band of about W / BQ tiles
    //     that starts at its diagonal: the heads are outermost and the tiles go
    //     up from the diagonal, so a neighbour reads the same tile two steps
    //     later, while it is still in L2.
    // DOWN is the first order. Tile iterator for the loads (ahead of the compute):
    constexpr bool DOWN = !WIN;
    int ld_it = 0, ld_h = 0, ld_qi = DOWN ? n_qt - 1 : qt_begin;
    // Rows past Tq lie past the end of the buffer ranges and read as zeros, so
    // only an exhausted iterator needs an out-of-range base.
    auto issue = [&](auto stage_c) FA_INLINE {
      FA_LDS uint8_t* st = smem + decltype(stage_c)::value * STAGE;
      const bool live = ld_it < n_iter;
      const size_t rows = ((size_t)b * a.Hq + (size_t)(hk * G + (live ? ld_h : 0))) * a.Tq;
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + rows * D, (uint32_t)a.Tq * D * 2);
      const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.dout + rows * D, (uint32_t)a.Tq * D * 2);
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.stats + rows, (uint32_t)a.Tq * 4);
      const __amdgpu_buffer_rsrc_t drs = make_rsrc(a.stats + plane + rows, (uint32_t)a.Tq * 4);
      const uint32_t tbase = live ? (uint32_t)(ld_qi * BQ) * D * 2 : kOutOfRange;
      const uint32_t sbase = live ? (uint32_t)(ld_qi * BQ) * 4 : kOutOfRange;
  #pragma unroll
      for (int i = 0; i < C::DMA_PER_WAVE; ++i) dma_b128(dma_is_do[i] ? grs : qrs, st + dma_dst[i], tbase + dma_off[i]);
  #pragma unroll
      for (int i = 0; i < C::STAT_DMA; ++i) {   // every wave loads them (same bytes, same place)
        // lanes past BQ rows (BQ < 64) fill unread bytes of the slot
        constexpr int PER_PLANE = C::STAT_DMA / 2;
        const int pl = i / PER_PLANE, row = 64 * (i % PER_PLANE) + lane;
        dma_b32(pl ? drs : lrs, st + 2 * QTILE + pl * C::SLOT + 256 * (i % PER_PLANE), sbase + (uint32_t)row * 4);
      }
      ++ld_it;
      if constexpr (DOWN) {
        if (++ld_h == G) {
          ld_h = 0;
          if (ld_qi > qt_begin) --ld_qi;   // past the last tile: loads read zeros (live is false)
        }
      } else if (++ld_qi == n_qt) {
        ld_qi = qt_begin;
        if (ld_h + 1 < G) ++ld_h;          // past the last head: loads read zeros (live is false)
      }
    };

    // LDS read offsets (bytes inside a tile).
    const uint32_t fq = swz<D>(col);
    const uint32_t q_rd = col * ROWB + 16 * (half ^ (fq & 1)) + 32 * (fq >> 1);   // ^ 32 ks
    const int grp = lane >> 4, gi = lane & 15;
    const int tr_row = 4 * (grp >> 1) + (gi >> 2);
    const uint32_t low2 = 2 * (grp & 1) + ((gi >> 1) & 1);
    const uint32_t f_lo = swz<D>(tr_row), f_hi = swz<D>(tr_row + 8);
    const uint32_t tr_lo = tr_row * ROWB + 64 * (f_lo >> 2) + 16 * (low2 ^ (f_lo & 3)) + 8 * (gi & 1);        // ^ 64 db
    const uint32_t tr_hi = (tr_row + 8) * ROWB + 64 * (f_hi >> 2) + 16 * (low2 ^ (f_hi & 3)) + 8 * (gi & 1);

    FA_LDS uint8_t* ztile = smem + C::NSTAGE * STAGE + wave * ZTILE;

    auto body = [&](const FA_LDS uint8_t* st, int q0, int head, auto masked) FA_INLINE {
      const FA_LDS uint8_t* qt = st;
      const FA_LDS uint8_t* gt = st + QTILE;
      const FA_LDS uint8_t* stt = st + 2 * QTILE;
      const uint32_t bhq = (uint32_t)(b * a.Hq + hk * G + head);   // flattened query head (dropout stream)
      // S = Q K^T and dP = dO V^T for BQ queries x 32 keys (one key per lane).
      // On unmasked tiles without dropout the dP product starts from -D
      // (accumulator register r of block qb holds row 32 qb + 8 (r / 4) +
      // 4 half + r % 4, so four -D values of consecutive rows fill registers
      // 4 g4 .. 4 g4 + 3), and dP - D comes out of the matrix cores; masked
      // tiles (fewer, and short of registers) and dropout add -D afterwards.
      constexpr bool FOLD = !DROP && !decltype(masked)::value;
      f32x16 s[QB], dp[QB];
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x16 dinit{};
        if constexpr (FOLD) {
  #pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 nd = *(const FA_LDS f32x4*)(stt + C::SLOT + (qb * 32 + 8 * g4 + 4 * half) * 4);
  #pragma unroll
            for (int e = 0; e < 4; ++e) dinit[4 * g4 + e] = nd[e];
          }
        }
  #pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const uint32_t off = qb * 32 * ROWB + (q_rd ^ (32 * ks));
          // the first products start from an inline zero (no register clearing) or from -D
          s[qb] = mfma32(as_bf16x8(lds_read_b128(qt, off)), kf[ks], ks == 0 ? f32x16{} : s[qb]);
          dp[qb] = mfma32(as_bf16x8(lds_read_b128(gt, off)), vf[ks], ks == 0 ? dinit : dp[qb]);
        }
      }
      // P and dS, packed to bf16 in the accumulator order (rows 32 qb + 8 g4 + 4 half + e).
      // Masked tiles: row q0 + 32 qb + 8 g4 + 4 half + e sees this lane's key iff
      // 0 <= dist < window with dist = (that row + shift - key) = dbase + 32 qb + 8 g4 + e.
      const int dbase = q0 + 4 * half + shift - key;
      uint32_t pw[QB][8], dsw[QB][8];
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // Dropout bytes for (row 32 qb + 8 g4 + 4 half + e, this lane's key), in
        // register order 4 g4 + e. Lane (c, h) draws row 32 qb + c's bytes for
        // the 16 keys kw0 + 16 h .. +15 (the forward's Philox contract), stores
        // them row-major in the wave's tile and reads back its own key column.
        uint32_t zbyte[16];
        if constexpr (DROP) {
          const u32x4 w = philox4x32_10<false>((uint32_t)(kw0 / 16 + half), (uint32_t)(q0 + 32 * qb + col), bhq,
                                        a.drop.offset, a.drop.seed_lo, a.drop.seed_hi);
          lds_write_b128(ztile, col * ZPITCH + 16 * half, w);
  #pragma unroll
          for (int i = 0; i < 16; ++i) zbyte[i] = ztile[(8 * (i >> 2) + 4 * half + (i & 3)) * ZPITCH + col];
        }
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int rq = qb * 32 + 8 * g4 + 4 * half;
          const f32x4 l2 = *(const FA_LDS f32x4*)(stt + rq * 4);   // lse2 of rows rq .. rq + 3
          f32x4 nd{};                                               // their -D, unless folded into dP
          if constexpr (!FOLD) nd = *(const FA_LDS f32x4*)(stt + C::SLOT + rq * 4);
          float p[4], ds[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float pe = exp2_fast(fmaf(s[qb][r], a.c, -l2[e]));
            if constexpr (decltype(masked)::value) {
              const int dist = dbase + (qb * 32 + 8 * g4 + e);   // one unsigned compare for the band
              if (WIN ? (uint32_t)dist >= (uint32_t)a.window : dist < 0) pe = 0.f;
            }
            float dpe = dp[qb][r];   // dP - D when folded, else dP
            float pv = pe;
            if constexpr (DROP) {   // dV takes the kept P; dP is dropped and rescaled
              const bool keep = zbyte[r] < a.drop.t;
              pv = keep ? pe : 0.f;
              dpe = keep ? dpe * a.drop.inv_keep : 0.f;
            }
            if constexpr (!FOLD) dpe += nd[e];
            p[e] = pv;
            ds[e] = pe * dpe;
          }
          pw[qb][2 * g4] = pack_bf16x2(p[0], p[1]);
          pw[qb][2 * g4 + 1] = pack_bf16x2(p[2], p[3]);
          dsw[qb][2 * g4] = pack_bf16x2(ds[0], ds[1]);
          dsw[qb][2 * g4 + 1] = pack_bf16x2(ds[2], ds[3]);
        }
      }
      // (the hint on the unmasked body only: on the masked one it costs registers)
      if constexpr (C::IGLP >= 0 && !decltype(masked)::value) __builtin_amdgcn_iglp_opt(C::IGLP);
      // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per step.
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const bf16x8 pb = as_bf16x8(u32x4{pw[qb][4 * hs], pw[qb][4 * hs + 1], pw[qb][4 * hs + 2], pw[qb][4 * hs + 3]});
          const bf16x8 sb = as_bf16x8(u32x4{dsw[qb][4 * hs], dsw[qb][4 * hs + 1], dsw[qb][4 * hs + 2], dsw[qb][4 * hs + 3]});
          const uint32_t hb = (qb * 32 + hs * 16) * ROWB;
  #pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const u32x2 glo = lds_read_tr(gt, hb + (tr_lo ^ (64 * db)));
            const u32x2 ghi = lds_read_tr(gt, hb + (tr_hi ^ (64 * db)));
            dv_acc[db] = mfma32(as_bf16x8(u32x4{glo[0], glo[1], ghi[0], ghi[1]}), pb, dv_acc[db]);
            const u32x2 qlo = lds_read_tr(qt, hb + (tr_lo ^ (64 * db)));
            const u32x2 qhi = lds_read_tr(qt, hb + (tr_hi ^ (64 * db)));
            dk_acc[db] = mfma32(as_bf16x8(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}), sb, dk_acc[db]);
          }
        }
    };

    // Ring of NSTAGE tiles, NSTAGE - 1 loads ahead of the compute. The loop is
    // unrolled NSTAGE times, so every stage is a compile-time LDS offset.
    constexpr int AHEAD_VM = (C::NSTAGE - 2) * C::VM_PER_TILE;
    if (n_iter > 0) {
      static_for<0, C::NSTAGE - 1>([&](auto st) FA_INLINE { issue(st); });
      wait_vm_barrier<AHEAD_VM>();          // K/V rows and tile 0 have landed
    }
    int cur_qi = DOWN ? n_qt - 1 : qt_begin, cur_h = 0;
    auto step = [&](auto stage_c, auto may_mask) FA_INLINE {
      constexpr int CS = decltype(stage_c)::value;
      issue(std::integral_constant<int, (CS + C::NSTAGE - 1) % C::NSTAGE>{});   // zeros past the end
      const FA_LDS uint8_t* st = smem + CS * STAGE;
      const int q0 = cur_qi * BQ;
      // some (row, key) pair of this wave is masked (causal limit or window start)
      if (decltype(may_mask)::value &&
          ((CAUSAL && q0 + shift < kw0 + 31) || (WIN && q0 + BQ - 1 + shift - a.window + 1 > kw0)))
        body(st, q0, cur_h, std::true_type{});
      else
        body(st, q0, cur_h, std::false_type{});
      wait_vm_barrier<AHEAD_VM>();          // the next tile has landed; this stage is free
      if constexpr (DOWN) {
        if (++cur_h == G) {
          cur_h = 0;
          --cur_qi;
        }
      } else if (++cur_qi == n_qt) {
        cur_qi = qt_begin;
        ++cur_h;
      }
    };
    int it = 0;
    if constexpr (CAUSAL && !WIN) {
      // tiles whose first row sees every key of the workgroup need no mask; the
      // downward walk visits them first (whole groups of NSTAGE iterations)
      const int qi_full = (k0 + C::BK - 1 - shift + BQ - 1) / BQ;   // first tile with no masked pair
      const int it_full = max(0, n_qt - max(qi_full, qt_begin)) * G / C::NSTAGE * C::NSTAGE;
      for (; it < it_full; it += C::NSTAGE)
        static_for<0, C::NSTAGE>([&](auto s) FA_INLINE { step(s, std::false_type{}); });
    }
    for (; it < n_iter; it += C::NSTAGE)
      static_for<0, C::NSTAGE>([&](auto s) FA_INLINE {
        if (it + decltype(s)::value < n_iter) step(s, std::true_type{});
      });
    if (n_iter > 0) wait_vm_barrier<0>();   // no load is left writing LDS when the workgroup exits

    if (key < a.Tk) {
      uint16_t* dkp = a.dk + kvoff + (size_t)key * D;
      uint16_t* dvp = a.dv + kvoff + (size_t)key * D;
  #pragma unroll
      for (int db = 0; db < D / 32; ++db)
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * half;
          const f32x16& kk = dk_acc[db];
          const f32x16& vv = dv_acc[db];
          *(u32x2*)(dkp + d0) = u32x2{pack_bf16x2(kk[4 * g4] * a.scale, kk[4 * g4 + 1] * a.scale),
                                      pack_bf16x2(kk[4 * g4 + 2] * a.scale, kk[4 * g4 + 3] * a.scale)};
          const float sv = DROP ? a.drop.inv_keep : 1.f;   // dV = (P Z)^T dO * 256 / t
          *(u32x2*)(dvp + d0) = u32x2{pack_bf16x2(vv[4 * g4] * sv, vv[4 * g4 + 1] * sv),
                                      pack_bf16x2(vv[4 * g4 + 2] * sv, vv[4 * g4 + 3] * sv)};
        }
    }
  };

  if constexpr (PAIRK) {
    key_tile(unit);
    if (n_ktiles - 1 - unit != unit) {   // the middle tile of an odd count runs alone
      __syncthreads();                   // every wave is done with the first tile's LDS ring
      key_tile(n_ktiles - 1 - unit);
    }
  } else {
    key_tile(unit);
  }
}

// ------------------------------------------------- dk dv, 16 keys per wave

namespace {

// Without dropout: 8 waves of 16 keys each (128 keys per workgroup) on
// v_mfma_f32_16x16x32_bf16. Each wave holds half the state of
// the 32-key layout (K and V fragments, dK and dV accumulators, S and dP of
// one query tile), about 150 registers instead of up to 512, so two waves
// share every SIMD and hide each other's LDS and barrier waits. The price is
// twice the LDS operand reads per MFMA: every Q or dO fragment now serves 16
// keys instead of 32.
template <int D, int NSTAGE_ = (D == 64 ? 2 : 3)>
struct Dkdv16Cfg {
  static constexpr int NW = 8;                       // waves per workgroup
  static constexpr int OCC = D == 64 ? 2 : 1;        // workgroups per CU the register budget allows
  static constexpr int NT = 64 * NW;
  static constexpr int BK = 16 * NW;                 // keys per workgroup
  static constexpr int BQ = 64;                      // query rows per tile
  static constexpr int RB = BQ / 16;                 // 16-row blocks per tile
  static constexpr int ROWB = 2 * D;
  static constexpr int CH = D / 8;
  static constexpr int QTILE = BQ * ROWB;
  static constexpr int SLOT = (BQ * 4 + 255) / 256 * 256;
  static constexpr int STATS = 2 * SLOT;
  static constexpr int STAGE = 2 * QTILE + STATS;
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr int TILE_DMA = 2 * BQ * CH / 64;
  static constexpr int DMA_PER_WAVE = TILE_DMA / NW;
  static constexpr int STAT_DMA = STATS / 256;
  static constexpr int VM_PER_TILE = DMA_PER_WAVE + STAT_DMA;
  static_assert(D == 64 || D == 128, "head width");
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * NW == TILE_DMA, "tile loads must split over the waves");
};

}  // namespace

// One workgroup per 128 keys of one KV head (a key tile); wave w owns keys
// k0 + 16 w .. k0 + 16 w + 15, lane (q = lane / 16, c = lane % 16) key
// k0 + 16 w + c.
//   S = Q K^T, dP = dO V^T   per 16-row block: lane holds rows 4 q .. 4 q + 3
//   dV^T += dO^T P, dK^T += Q^T dS   per 32-row step; k-slot (q, e) of the
//       step is row 4 q + e (e < 4) or 16 + 4 q + e - 4 (e >= 4), so P and dS
//       go from the S/dP accumulators into the B operand with no lane
//       exchange, and the A operand (dO^T or Q^T) comes from two transposed
//       LDS reads of 4 consecutive rows each.
//
// Order of the work. The workgroups that run together on an XCD (its 32 CUs)
// hold key tiles of one KV head and should read each Q/dO tile at the same
// time, so that it is fetched into the XCD's L2 once.
//   * Causal without a window, a workgroup takes two key tiles, p and
//     n - 1 - p, one after the other: tile p walks the query tiles from the
//     last one down to its diagonal, then tile n - 1 - p from its diagonal up
//     to the last one, the group's heads innermost. Every workgroup then does
//     the same number of steps, and after s steps each is at query tile
//     n_qt - 1 - s / G (first walk) or at s / G - 2 (second walk, BK = 2 BQ),
//     whatever its p: the resident workgroups share two tiles at a time.
//   * Without a causal mask every workgroup walks all query tiles from the
//     last one down, the heads innermost.
//   * With a window each workgroup sees only a band of about W / BQ tiles
//     that starts at its diagonal: the heads are outermost and the tiles go
//     up from the diagonal, so a neighbour reads the same tile two steps
//     later, while it is still in L2.
enum class Walk { kDown, kUpHeadsInner, kUpHeadsOuter };

template <int D, bool CAUSAL, class C = Dkdv16Cfg<D>, bool WIN = false>
__global__ __launch_bounds__(C::NT, C::OCC) void bwd_dkdv16_kernel(BwdArgs a, int n_ktiles, int n_units) {
  static_assert(CAUSAL || !WIN, "a sliding window is a causal band");
  static_assert(C::BK == 2 * C::BQ, "the paired causal walk keeps step with BK = 2 BQ");
  constexpr int BQ = C::BQ, RB = C::RB, ROWB = C::ROWB, CH = C::CH, QTILE = C::QTILE, STAGE = C::STAGE;
  constexpr bool PAIR = CAUSAL && !WIN;
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[C::NSTAGE * STAGE];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, col = lane & 15;

  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = (int)(t % (uint32_t)n_units);
  const int bhk = (int)(t / (uint32_t)n_units);
  const int b = bhk / a.Hkv, hk = bhk - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int shift = a.Tk - a.Tq;
  const size_t kvoff = (size_t)bhk * a.Tk * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + kvoff, (uint32_t)a.Tk * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + kvoff, (uint32_t)a.Tk * D * 2);
  const size_t plane = (size_t)a.B * a.Hq * a.Tq;   // -D plane of the statistics workspace

  // This thread's share of the tile loads (physical chunk p of a row holds
  // logical chunk p ^ swz16<D>(row)).
  uint32_t dma_off[C::DMA_PER_WAVE], dma_dst[C::DMA_PER_WAVE];
  bool dma_is_do[C::DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
    const int n = wave * C::DMA_PER_WAVE + i;
    const int m = n % (C::TILE_DMA / 2);
    dma_is_do[i] = n >= C::TILE_DMA / 2;
    const int p = 64 * m + lane;
    const int r = p / CH, pc = p % CH;
    dma_off[i] = (uint32_t)(r * D + (pc ^ swz16<D>(r)) * 8) * 2;
    dma_dst[i] = (dma_is_do[i] ? QTILE : 0) + m * 1024;
  }

  // LDS read offsets inside a tile. A operand of S and dP: row 16 rb + c,
  // logical chunk 4 ks + q (^ 64 ks on the byte offset).
  const uint32_t a_rd = col * ROWB + 16 * (q ^ swz16<D>(col));
  // Transposed reads: lane c of group q names row 4 q + c / 4 of a 16-row
  // block and the 8 bytes at d = 16 db + 4 (c % 4) (^ 32 db on the offset).
  const uint32_t tr_row = 4 * q + (col >> 2);
  const uint32_t tr_rd = tr_row * ROWB + 16 * (((col & 3) >> 1) ^ swz16<D>(tr_row)) + 8 * (col & 1);

  // One key tile: dK and dV of its 128 keys over every query tile of every
  // query head of the group that sees one of them, in the given order.
  auto key_tile = [&](const int kt, auto walk_c) FA_INLINE {
    constexpr Walk W = decltype(walk_c)::value;
    constexpr bool HEADS_INNER = W != Walk::kUpHeadsOuter;
    constexpr int DIR = W == Walk::kDown ? -1 : 1;
    const int k0 = kt * C::BK;
    const int kw0 = k0 + wave * 16;                 // first key of this wave
    const int key = kw0 + col;                      // this lane's key

    // B operands: lane (q, c) holds K[key][32 ks + 8 q + e] and V[key][...], e < 8.
    bf16x8 kf[D / 32], vf[D / 32];
    {
      const uint32_t base = key < a.Tk ? (uint32_t)(key * D + 8 * q) * 2 : kOutOfRange;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        kf[ks] = as_bf16x8(buf_load_b128(krs, base + ks * 64));
        vf[ks] = as_bf16x8(buf_load_b128(vrs, base + ks * 64));
      }
    }
    // dV^T and dK^T in 16-wide d blocks: register r of block db is d = 16 db + 4 q + r.
    f32x4 dv_acc[D / 16], dk_acc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      dv_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dk_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int qt_begin = 0;
    if (CAUSAL) qt_begin = max(0, k0 - shift) / BQ;
    int n_qt = (a.Tq + BQ - 1) / BQ;
    if (WIN) {   // rows past the last key's window see none of these keys
      const int last_row = k0 + C::BK - 1 - shift + a.window - 1;
      n_qt = last_row < 0 ? 0 : min(n_qt, last_row / BQ + 1);
    }
    const int per_head = max(0, n_qt - qt_begin);
    const int n_iter = per_head * G;
    const int qi_first = W == Walk::kDown ? n_qt - 1 : qt_begin;

    // Load iterator (ahead of the compute). Rows past Tq lie past the end of
    // the buffer ranges and read as zeros.
    int ld_it = 0, ld_h = 0, ld_qi = qi_first;
    auto issue = [&](auto stage_c) FA_INLINE {
      FA_LDS uint8_t* st = smem + decltype(stage_c)::value * STAGE;
      // The buffer ranges start at the tile's first row and hold the rows left
      // in the head (none once the iterator is exhausted), so the per-lane
      // offsets are the same for every tile.
      const bool live = ld_it < n_iter;
      const int r0 = live ? ld_qi * BQ : 0;
      const size_t rows = ((size_t)b * a.Hq + (size_t)(hk * G + (live ? ld_h : 0))) * a.Tq + r0;
      const uint32_t left = live ? (uint32_t)(a.Tq - r0) : 0u;
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + rows * D, left * D * 2);
      const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.dout + rows * D, left * D * 2);
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.stats + rows, left * 4);
      const __amdgpu_buffer_rsrc_t drs = make_rsrc(a.stats + plane + rows, left * 4);
#pragma unroll
      for (int i = 0; i < C::DMA_PER_WAVE; ++i) dma_b128(dma_is_do[i] ? grs : qrs, st + dma_dst[i], dma_off[i]);
#pragma unroll
      for (int i = 0; i < C::STAT_DMA; ++i) {   // every wave loads them (same bytes, same place)
        constexpr int PER_PLANE = C::STAT_DMA / 2;
        const int pl = i / PER_PLANE, row = 64 * (i % PER_PLANE) + lane;
        dma_b32(pl ? drs : lrs, st + 2 * QTILE + pl * C::SLOT + 256 * (i % PER_PLANE), (uint32_t)row * 4);
      }
      ++ld_it;
      if constexpr (HEADS_INNER) {
        if (++ld_h == G) {
          ld_h = 0;
          ld_qi += DIR;   // past the last tile the loads are not live
        }
      } else if (++ld_qi == n_qt) {
        ld_qi = qt_begin;
        if (ld_h + 1 < G) ++ld_h;   // past the last head the loads are not live
      }
    };

    // At d = 128 the operand reads of both product pairs run two items ahead
    // of their MFMAs (chunk_pipeline; measured on MI355X: causal 32k GQA
    // backward -11%, sliding-window -6%). At d = 64 the compiler's own order
    // was faster (causal GPT-2 shape +8% with the pipeline) and is kept.
    constexpr bool AHEAD = D == 128;
    constexpr int CK = 2;
    auto body = [&](const FA_LDS uint8_t* st, int q0, auto masked) FA_INLINE {
      const FA_LDS uint8_t* qt = st;
      const FA_LDS uint8_t* gt = st + QTILE;
      const FA_LDS uint8_t* stt = st + 2 * QTILE;
      // Unmasked tiles start the dP product from -D of the lane's four rows.
      constexpr bool FOLD = !decltype(masked)::value;
      // S = Q K^T and dP = dO V^T. Item i is (rb, ks, Q or dO) =
      // (i / (2 KS), i / 2 % KS, i % 2): one 128-bit read and one MFMA.
      constexpr int KS = D / 32;
      f32x4 s[RB], dp[RB], dinit[RB];
      bf16x8 abuf[2][CK];
      auto sd_read = [&](auto i_c) FA_INLINE {
        constexpr int i = decltype(i_c)::value, rb = i / (2 * KS), ks = i / 2 % KS, w = i % 2;
        if constexpr (FOLD && ks == 0 && w == 1)
          dinit[rb] = *(const FA_LDS f32x4*)(stt + C::SLOT + (16 * rb + 4 * q) * 4);
        abuf[i / CK & 1][i % CK] = as_bf16x8(lds_read_b128(w ? gt : qt, rb * 16 * ROWB + (a_rd ^ (64 * ks))));
      };
      auto sd_mma = [&](auto i_c) FA_INLINE {
        constexpr int i = decltype(i_c)::value, rb = i / (2 * KS), ks = i / 2 % KS, w = i % 2;
        const bf16x8 x = abuf[i / CK & 1][i % CK];
        if constexpr (w == 0) s[rb] = mfma16(x, kf[ks], ks == 0 ? f32x4{} : s[rb]);
        else dp[rb] = mfma16(x, vf[ks], ks == 0 ? (FOLD ? dinit[rb] : f32x4{}) : dp[rb]);
      };
      if constexpr (AHEAD) {
        chunk_pipeline<2 * RB * KS, CK>(sd_read, sd_mma);
      } else {
        static_for<0, 2 * RB * KS>([&](auto i) FA_INLINE { sd_read(i); sd_mma(i); });
      }
      // P and dS of rows 16 rb + 4 q + e, packed in pairs; masked tiles: row
      // q0 + 16 rb + 4 q + e sees this lane's key iff 0 <= dist < window with
      // dist = dbase + 16 rb + e (no upper limit without a window).
      const int dbase = q0 + 4 * q + shift - key;
      uint32_t pw[RB][2], dsw[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f32x4 l2 = *(const FA_LDS f32x4*)(stt + (16 * rb + 4 * q) * 4);
        f32x4 nd{};
        if constexpr (!FOLD) nd = *(const FA_LDS f32x4*)(stt + C::SLOT + (16 * rb + 4 * q) * 4);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pe = exp2_fast(fmaf(s[rb][e], a.c, -l2[e]));
          if constexpr (decltype(masked)::value) {
            const int dist = dbase + 16 * rb + e;   // one unsigned compare for the band
            if (WIN ? (uint32_t)dist >= (uint32_t)a.window : dist < 0) pe = 0.f;
          }
          p[e] = pe;
          ds[e] = pe * (FOLD ? dp[rb][e] : dp[rb][e] + nd[e]);
        }
        pw[rb][0] = pack_bf16x2(p[0], p[1]);
        pw[rb][1] = pack_bf16x2(p[2], p[3]);
        dsw[rb][0] = pack_bf16x2(ds[0], ds[1]);
        dsw[rb][1] = pack_bf16x2(ds[2], ds[3]);
      }
      // The compiler's interleave strategy 1 on the unmasked body (measured on
      // MI355X: causal 32k GQA backward -4.5%; with the operand reads issued
      // ahead also the sliding-window backward -1..2% and the non-causal one
      // -0.4..2.6%, which had run 23% slower with it before).
      if constexpr (!decltype(masked)::value) __builtin_amdgcn_iglp_opt(1);
      // dV^T += dO^T P and dK^T += Q^T dS, 32 rows (blocks 2 hs and 2 hs + 1) per
      // step. Item i is (hs, db, dO^T or Q^T) = (i / (2 NDB), i / 2 % NDB, i % 2):
      // two transposed reads and one MFMA.
      constexpr int NDB = D / 16;
      u32x4 tbuf[2][CK];
      auto dkv_read = [&](auto i_c) FA_INLINE {
        constexpr int i = decltype(i_c)::value, hs = i / (2 * NDB), db = i / 2 % NDB, w = i % 2;
        const uint32_t o = tr_rd ^ (32 * db);
        const FA_LDS uint8_t* src = w ? qt : gt;
        const u32x2 lo = lds_read_tr(src, 32 * hs * ROWB + o), hi = lds_read_tr(src, (32 * hs + 16) * ROWB + o);
        tbuf[i / CK & 1][i % CK] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      auto dkv_mma = [&](auto i_c) FA_INLINE {
        constexpr int i = decltype(i_c)::value, hs = i / (2 * NDB), db = i / 2 % NDB, w = i % 2;
        const bf16x8 x = as_bf16x8(tbuf[i / CK & 1][i % CK]);
        if constexpr (w == 0)
          dv_acc[db] = mfma16(x, as_bf16x8(u32x4{pw[2 * hs][0], pw[2 * hs][1], pw[2 * hs + 1][0], pw[2 * hs + 1][1]}),
                              dv_acc[db]);
        else
          dk_acc[db] = mfma16(x, as_bf16x8(u32x4{dsw[2 * hs][0], dsw[2 * hs][1], dsw[2 * hs + 1][0], dsw[2 * hs + 1][1]}),
                              dk_acc[db]);
      };
      if constexpr (AHEAD) {
        chunk_pipeline<2 * (BQ / 32) * NDB, CK>(dkv_read, dkv_mma);
      } else {
        static_for<0, 2 * (BQ / 32) * NDB>([&](auto i) FA_INLINE { dkv_read(i); dkv_mma(i); });
      }
    };

    // Ring of NSTAGE tiles, NSTAGE - 1 loads ahead of the compute. The loop is
    // unrolled NSTAGE times, so every stage is a compile-time LDS offset.
    constexpr int AHEAD_VM = (C::NSTAGE - 2) * C::VM_PER_TILE;
    if (n_iter > 0) {
      static_for<0, C::NSTAGE - 1>([&](auto st) FA_INLINE { issue(st); });
      wait_vm_barrier<AHEAD_VM>();          // K/V rows and tile 0 have landed
    }
    int cur_qi = qi_first, cur_h = 0;
    auto step = [&](auto stage_c, auto may_mask) FA_INLINE {
      constexpr int CS = decltype(stage_c)::value;
      issue(std::integral_constant<int, (CS + C::NSTAGE - 1) % C::NSTAGE>{});   // zeros past the end
      const FA_LDS uint8_t* st = smem + CS * STAGE;
      const int q0 = cur_qi * BQ;
      // some (row, key) pair of this wave is masked (causal limit or window start)
      if (decltype(may_mask)::value &&
          ((CAUSAL && q0 + shift < kw0 + 15) || (WIN && q0 + BQ - 1 + shift - a.window + 1 > kw0)))
        body(st, q0, std::true_type{});
      else
        body(st, q0, std::false_type{});
      wait_vm_barrier<AHEAD_VM>();          // the next tile has landed; this stage is free
      if constexpr (HEADS_INNER) {
        if (++cur_h == G) {
          cur_h = 0;
          cur_qi += DIR;
        }
      } else if (++cur_qi == n_qt) {
        cur_qi = qt_begin;
        ++cur_h;
      }
    };
    // Query tiles whose first row sees every key of the tile need no mask:
    // qi >= qi_full. They run in loops of their own (whole groups of NSTAGE
    // iterations), so the masked body's registers do not weigh on them.
    const int qi_full = (k0 + C::BK - 1 - shift + BQ - 1) / BQ;
    const int n_full_it = CAUSAL && !WIN ? max(0, n_qt - max(qi_full, qt_begin)) * G : 0;
    int it = 0;
    auto masked_groups = [&](int until) FA_INLINE {
      for (; it < until; it += C::NSTAGE)
        static_for<0, C::NSTAGE>([&](auto s) FA_INLINE {
          if (it + decltype(s)::value < n_iter) step(s, std::true_type{});
        });
    };
    if constexpr (W == Walk::kDown && CAUSAL) {   // unmasked tiles first
      for (; it < n_full_it / C::NSTAGE * C::NSTAGE; it += C::NSTAGE)
        static_for<0, C::NSTAGE>([&](auto s) FA_INLINE { step(s, std::false_type{}); });
    } else if constexpr (W == Walk::kUpHeadsInner) {   // masked tiles first, then the unmasked ones
      masked_groups((n_iter - n_full_it + C::NSTAGE - 1) / C::NSTAGE * C::NSTAGE);
      for (; it + C::NSTAGE <= n_iter; it += C::NSTAGE)
        static_for<0, C::NSTAGE>([&](auto s) FA_INLINE { step(s, std::false_type{}); });
    }
    masked_groups(n_iter);
    if (n_iter > 0) wait_vm_barrier<0>();   // no load is left writing LDS (the ring is free again)

    if (key < a.Tk) {
      uint16_t* dkp = a.dk + kvoff + (size_t)key * D + 4 * q;
      uint16_t* dvp = a.dv + kvoff + (size_t)key * D + 4 * q;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 kk = dk_acc[db], vv = dv_acc[db];
        *(u32x2*)(dkp + 16 * db) = u32x2{pack_bf16x2(kk[0] * a.scale, kk[1] * a.scale),
                                         pack_bf16x2(kk[2] * a.scale, kk[3] * a.scale)};
        *(u32x2*)(dvp + 16 * db) = u32x2{pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
      }
    }
  };

  if constexpr (PAIR) {
    key_tile(unit, std::integral_constant<Walk, Walk::kDown>{});
    const int kt2 = n_ktiles - 1 - unit;
    if (kt2 != unit) key_tile(kt2, std::integral_constant<Walk, Walk::kUpHeadsInner>{});
  } else if constexpr (WIN) {
    key_tile(unit, std::integral_constant<Walk, Walk::kUpHeadsOuter>{});
  } else {
    key_tile(unit, std::integral_constant<Walk, Walk::kDown>{});
  }
}

// -------------------------------------------------------------------- dq

namespace {

// d = 64: 8 waves (two per SIMD at about 128 registers, so two workgroups per
// CU; the non-causal launch takes 4-wave workgroups, four per CU) and 32-key
// tiles; d = 128: 4 waves, 32-key tiles in a 3-stage ring and
// two workgroups per CU (256 registers per wave), with the MFMA/exp interleave
// hint. Both measured fastest on MI355X (at d = 128 the causal loop must be
// split, see bwd_dq_kernel, for the two-workgroup tiling to fit).
template <int D, int NW_ = (D == 64 ? 8 : 4), int BC_ = 32, int NSTAGE_ = (D == 64 ? 2 : 3),
          int IGLP_ = (D == 64 ? -1 : 2), int OCC_ = (D == 64 ? 1 : 2)>
struct DqCfg {
  static constexpr int NW = NW_;                      // waves per workgroup
  static constexpr int OCC = OCC_;                    // workgroups per CU the register budget allows
  static constexpr int IGLP = IGLP_;                  // compiler interleave strategy for the body (-1: none)
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;                  // query rows per workgroup
  static constexpr int BC = BC_;                      // keys per tile
  static constexpr int ROWB = 2 * D;
  static constexpr int CH = D / 8;
  static constexpr int KTILE = BC * ROWB;             // one K (or V) tile
  static constexpr int STAGE = 2 * KTILE;
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr int TILE_DMA = 2 * BC * CH / 64;   // 128-bit wave loads per tile (K and V)
  static constexpr int DMA_PER_WAVE = TILE_DMA / NW;
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * NW == TILE_DMA, "tile loads must split over the waves");
};

}  // namespace

// One workgroup per BR query rows; each wave owns 32 rows, with its Q and dO
// rows held as MFMA B operands, and walks the key tiles its rows can see:
//   S^T = K Q^T, dP^T = V dO^T        (A operands: K and V rows from LDS)
//   P = 2^(S c - lse2), dS = P (dP - D)
//   dQ^T += K^T dS^T                   (A operand: transposed reads of K)
// The layout mirrors the forward kernel: one query per lane, so dS^T feeds
// the last product from the accumulator registers. K and V arrive through
// direct-to-LDS loads into a ring of C::NSTAGE tiles, swizzled like the
// dK/dV kernel's tiles. Keys past Tk read as zero rows and contribute nothing to dQ.
template <int D, bool CAUSAL, class C = DqCfg<D>, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(C::NT, C::OCC) void bwd_dq_kernel(BwdArgs a, int n_qtiles, int n_units) {
  static_assert(CAUSAL || !WIN, "a sliding window is a causal band");
  static_assert(!(WIN && DROP), "dropout is not offered with a sliding window");
  constexpr int BC = C::BC, ROWB = C::ROWB, CH = C::CH, KTILE = C::KTILE, STAGE = C::STAGE;
  constexpr int KB = BC / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[C::NSTAGE * STAGE];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // Work order: (batch, kv head) outermost, then the unit (query tile or
  // pair of them), then the query heads that share the kv head, so the
  // workgroups that run together on an XCD read the same K/V tiles at about
  // the same time.
  //   * Causal without a window, a unit is a pair of query tiles:
  //     tile p walks its key tiles up from the first, then tile n - 1 - p
  //     walks its key tiles down from the last. Every workgroup then does the
  //     same number of steps, and after s steps each reads key tile s (first
  //     walk) or (n + 1) BR / BC - 1 - s (second walk) whatever its p (for
  //     Tq = Tk): the resident workgroups share two K/V tiles at a time.
  //   * Otherwise a unit is one query tile, causal ones longest first.
  constexpr bool PAIR = CAUSAL && !WIN;
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t G = (uint32_t)(a.Hq / a.Hkv), per_grp = (uint32_t)n_units * G;
  const uint32_t kvg = t / per_grp, r = t - kvg * per_grp;
  const int unit = (int)(r / G), g = (int)(r - (uint32_t)unit * G);
  const int b = (int)kvg / a.Hkv, hk = (int)kvg - b * a.Hkv;
  const int h = hk * (int)G + g, bh = b * a.Hq + h;
  const size_t qoff = (size_t)bh * a.Tq;
  const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const int shift = a.Tk - a.Tq;

  // One query tile, its key tiles walked up (UP) or down.
  auto query_tile = [&](const int qt, auto up_c) FA_INLINE {
    constexpr bool UP = decltype(up_c)::value;
    const int q0 = qt * C::BR;
    const int qw0 = q0 + wave * 32;                 // first row of this wave
    const int qrow = qw0 + col;                     // this lane's query row
    int kv_end = a.Tk;
    if (CAUSAL) kv_end = min(a.Tk, q0 + C::BR + shift);
    const int n_kv = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
    // tiles before j_begin are invisible to every row of the workgroup
    const int j_begin = WIN ? min(n_kv, max(0, q0 + shift - a.window + 1) / BC) : 0;
    const int n_it = n_kv - j_begin;
    auto tile_of = [&](int it) FA_INLINE { return UP ? j_begin + it : n_kv - 1 - it; };

    // Q and dO rows of this lane's query (B operands; the lane holds half of
    // the dims, lane ^ 32 the other half), its lse2 = LSE * log2(e) and
    // D = sum_c dO_c O_c, which are also stored for the dK/dV kernel. A row
    // that saw no key (LSE = -inf) gets lse2 = +inf, so every rebuilt
    // probability is 0.
    bf16x8 qf[D / 16], gf[D / 16];
    float lse2, delta;
    {
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + qoff * D, (uint32_t)a.Tq * D * 2);
      const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.dout + qoff * D, (uint32_t)a.Tq * D * 2);
      const __amdgpu_buffer_rsrc_t ors = make_rsrc(a.o + qoff * D, (uint32_t)a.Tq * D * 2);
      const bool live = qrow < a.Tq;
      const uint32_t base = live ? (uint32_t)(qrow * D + 8 * half) * 2 : kOutOfRange;
      float dsum = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 qw = buf_load_b128(qrs, base + ks * 32);
        const u32x4 gw = buf_load_b128(grs, base + ks * 32);
        const u32x4 ow = buf_load_b128(ors, base + ks * 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dsum = fmaf(bf16_lo(gw[e]), bf16_lo(ow[e]), dsum);
          dsum = fmaf(bf16_hi(gw[e]), bf16_hi(ow[e]), dsum);
        }
        qf[ks] = as_bf16x8(qw);
        gf[ks] = as_bf16x8(gw);
      }
      delta = pair_sum32(dsum);
      // rows past Tq: Q = dO = 0, so dS = 0 whatever lse2 holds
      const float lse = live ? a.lse[qoff + qrow] : 0.f;
      lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
      if (live && half == 0) {   // two planes: lse2 for every row, then -D
        a.stats[qoff + qrow] = lse2;
        a.stats[(size_t)a.B * a.Hq * a.Tq + qoff + qrow] = -delta;
      }
    }

    f32x16 dq_acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.f;

    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + kvoff, (uint32_t)a.Tk * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + kvoff, (uint32_t)a.Tk * D * 2);
    uint32_t dma_off[C::DMA_PER_WAVE], dma_dst[C::DMA_PER_WAVE];
    bool dma_is_v[C::DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
      const int n = wave * C::DMA_PER_WAVE + i;
      const int m = n % (C::TILE_DMA / 2);
      dma_is_v[i] = n >= C::TILE_DMA / 2;
      const int p = 64 * m + lane;
      const int r = p / CH, pc = p % CH;
      dma_off[i] = (uint32_t)(r * D + (pc ^ swz<D>(r)) * 8) * 2;
      dma_dst[i] = (dma_is_v[i] ? KTILE : 0) + m * 1024;
    }
    // Keys past Tk lie past the end of the buffer ranges and read as zeros, so
    // only an iteration past the walk needs an out-of-range base.
    auto issue = [&](int it, auto stage_c) FA_INLINE {
      FA_LDS uint8_t* st = smem + decltype(stage_c)::value * STAGE;
      const uint32_t tbase = it < n_it ? (uint32_t)(tile_of(it) * BC) * D * 2 : kOutOfRange;
#pragma unroll
      for (int i = 0; i < C::DMA_PER_WAVE; ++i) dma_b128(dma_is_v[i] ? vrs : krs, st + dma_dst[i], tbase + dma_off[i]);
    };

    const uint32_t fq = swz<D>(col);
    const uint32_t k_rd = col * ROWB + 16 * (half ^ (fq & 1)) + 32 * (fq >> 1);   // ^ 32 ks
    const int grp = lane >> 4, gi = lane & 15;
    const int tr_row = 4 * (grp >> 1) + (gi >> 2);
    const uint32_t low2 = 2 * (grp & 1) + ((gi >> 1) & 1);
    const uint32_t f_lo = swz<D>(tr_row), f_hi = swz<D>(tr_row + 8);
    const uint32_t tr_lo = tr_row * ROWB + 64 * (f_lo >> 2) + 16 * (low2 ^ (f_lo & 3)) + 8 * (gi & 1);        // ^ 64 db
    const uint32_t tr_hi = (tr_row + 8) * ROWB + 64 * (f_hi >> 2) + 16 * (low2 ^ (f_hi & 3)) + 8 * (gi & 1);
    const int lim = CAUSAL ? min(a.Tk - 1, qrow + shift) : a.Tk - 1;
    const int lo = WIN ? qrow + shift - a.window + 1 : 0;   // window start of this lane's row

    // Dropout: the Philox bytes of this lane's row for the 32-key blocks of the
    // current tile (the forward's layout and contract); the next tile's are
    // drawn while the matrix cores run this tile's dQ product.
    u32x4 zcur[KB];
    auto drop_bytes = [&](int j, int kb) -> u32x4 {
      // plain XORs here: the bitop3 form costs this kernel a register past the
      // two-workgroups-per-CU budget at d = 64 (and spills in dK/dV)
      return dropout_bytes_32keys<false>((uint32_t)(j * BC + kb * 32), (uint32_t)qrow, (uint32_t)bh, a.drop.offset,
                                  a.drop.seed_lo, a.drop.seed_hi, half);
    };

    // At d = 128 without dropout every dP^T chain starts from a register block
    // holding -D (one query per lane, so one value), read as the first
    // product's accumulator input: dP - D comes out of the matrix cores at no
    // per-tile cost. (d = 64 has no 16 registers to spare at two workgroups per
    // CU; dropout needs dP itself.)
    constexpr bool FOLD = D == 128 && !DROP;
    f32x16 ndelta;
#pragma unroll
    for (int r = 0; r < 16; ++r) ndelta[r] = FOLD ? -delta : 0.f;

    auto body = [&](const FA_LDS uint8_t* st, int j, auto masked) FA_INLINE {
      const FA_LDS uint8_t* kt = st;
      const FA_LDS uint8_t* vt = st + KTILE;
      f32x16 s[KB], dp[KB];
      // Both products take their LDS operands two items ahead of the MFMAs
      // (chunk_pipeline; measured on MI355X: sliding-window backward -7.5%,
      // causal 32k GQA -2%, dropout at d = 128 -9%), except the d = 64
      // dropout pass, which ran 5% slower with it and keeps the compiler's
      // order. S = K Q^T and dP - D: item i is (kb, ks, K or V) =
      // (i / (2 KS), i / 2 % KS, i % 2), one 128-bit read and one MFMA.
      constexpr bool AHEAD = !(DROP && D == 64);
      constexpr int KS = D / 16, CK = 2;
      {
        u32x4 ab[2][CK];
        auto rd = [&](auto i_c) FA_INLINE {
          constexpr int i = decltype(i_c)::value, kb = i / (2 * KS), ks = i / 2 % KS, w = i % 2;
          ab[i / CK & 1][i % CK] = lds_read_b128(w ? vt : kt, kb * 32 * ROWB + (k_rd ^ (32 * ks)));
        };
        auto mm = [&](auto i_c) FA_INLINE {
          constexpr int i = decltype(i_c)::value, kb = i / (2 * KS), ks = i / 2 % KS, w = i % 2;
          const bf16x8 x = as_bf16x8(ab[i / CK & 1][i % CK]);
          if constexpr (w == 0) s[kb] = mfma32(x, qf[ks], ks == 0 ? f32x16{} : s[kb]);
          else dp[kb] = mfma32(x, gf[ks], ks == 0 ? (FOLD ? ndelta : f32x16{}) : dp[kb]);
        };
        if constexpr (AHEAD) chunk_pipeline<2 * KB * KS, CK>(rd, mm);
        else static_for<0, 2 * KB * KS>([&](auto i) FA_INLINE { rd(i); mm(i); });
      }
      uint32_t dsw[KB][8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 zb = zcur[kb];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = exp2_fast(fmaf(s[kb][r], a.c, -lse2));
          float p1 = exp2_fast(fmaf(s[kb][r + 1], a.c, -lse2));
          if constexpr (decltype(masked)::value) {
            const int kr = j * BC + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (kr > lim || (WIN && kr < lo)) p0 = 0.f;
            if (kr + 1 > lim || (WIN && kr + 1 < lo)) p1 = 0.f;
          }
          float dp0 = dp[kb][r], dp1 = dp[kb][r + 1];
          if constexpr (DROP) {   // dP of a dropped entry is 0, of a kept one scaled by 256 / t
            dp0 = dropout_keep(zb, r, a.drop.t) ? dp0 * a.drop.inv_keep : 0.f;
            dp1 = dropout_keep(zb, r + 1, a.drop.t) ? dp1 * a.drop.inv_keep : 0.f;
          }
          const float dsub = FOLD ? 0.f : delta;   // folded: dp already holds dP - D
          dsw[kb][r >> 1] = pack_bf16x2(p0 * (dp0 - dsub), p1 * (dp1 - dsub));
        }
      }
      if constexpr (C::IGLP >= 0) __builtin_amdgcn_iglp_opt(C::IGLP);
      // dQ^T[d, query] += K^T[d, key] dS^T[key, query], 16 keys per step: item
      // i is (16-key step, db) = (i / NDB, i % NDB), two transposed reads and
      // one MFMA.
      {
        constexpr int NDB = D / 32;
        u32x4 tb[2][CK];
        auto rd = [&](auto i_c) FA_INLINE {
          constexpr int i = decltype(i_c)::value, kh = i / NDB, db = i % NDB;
          const uint32_t rb = kh * 16 * ROWB;
          const u32x2 lo = lds_read_tr(kt, rb + (tr_lo ^ (64 * db)));
          const u32x2 hi = lds_read_tr(kt, rb + (tr_hi ^ (64 * db)));
          tb[i / CK & 1][i % CK] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        auto mm = [&](auto i_c) FA_INLINE {
          constexpr int i = decltype(i_c)::value, kh = i / NDB, db = i % NDB, kb = kh / 2, hs = kh % 2;
          const bf16x8 sb = as_bf16x8(u32x4{dsw[kb][4 * hs], dsw[kb][4 * hs + 1], dsw[kb][4 * hs + 2], dsw[kb][4 * hs + 3]});
          dq_acc[db] = mfma32(as_bf16x8(tb[i / CK & 1][i % CK]), sb, dq_acc[db]);
        };
        if constexpr (AHEAD) chunk_pipeline<2 * KB * NDB, CK>(rd, mm);
        else static_for<0, 2 * KB * NDB>([&](auto i) FA_INLINE { rd(i); mm(i); });
      }
      if constexpr (DROP) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) zcur[kb] = drop_bytes(UP ? j + 1 : j - 1, kb);   // the next tile's
      }
    };

    // Ring of NSTAGE tiles, NSTAGE - 1 loads ahead of the compute. The loop is
    // unrolled NSTAGE times, so every stage is a compile-time LDS offset.
    constexpr int AHEAD_VM = (C::NSTAGE - 2) * C::DMA_PER_WAVE;
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) zcur[kb] = drop_bytes(tile_of(0), kb);
    }
    if (n_it > 0) {
      static_for<0, C::NSTAGE - 1>([&](auto st) FA_INLINE { issue(decltype(st)::value, st); });
      wait_vm_barrier<AHEAD_VM>();          // Q/dO rows, statistics and the first tile have landed
    }
    auto step = [&](int it, auto stage_c, auto may_mask) FA_INLINE {
      constexpr int CS = decltype(stage_c)::value;
      issue(it + C::NSTAGE - 1, std::integral_constant<int, (CS + C::NSTAGE - 1) % C::NSTAGE>{});
      const int j = tile_of(it);
      const FA_LDS uint8_t* st = smem + CS * STAGE;
      // some (row, key) pair of this wave is masked (causal limit or window start)
      if (decltype(may_mask)::value &&
          ((CAUSAL && j * BC + BC - 1 > qw0 + shift) || (WIN && j * BC < qw0 + 31 + shift - a.window + 1)))
        body(st, j, std::true_type{});
      else
        body(st, j, std::false_type{});
      wait_vm_barrier<AHEAD_VM>();
    };
    // Key tiles every row of the workgroup sees whole need no mask; they run in
    // a loop of their own (whole groups of NSTAGE tiles), so the masked body's
    // registers do not weigh on it. Walking up, the tiles before the last row's
    // window start (window) come first, masked, and the causal diagonal last;
    // walking down, the diagonal comes first.
    int it = 0;
    auto masked_groups = [&](int until) FA_INLINE {
      for (; it < until; it += C::NSTAGE)
        static_for<0, C::NSTAGE>([&](auto s) FA_INLINE {
          if (it + decltype(s)::value < n_it) step(it + decltype(s)::value, s, std::true_type{});
        });
    };
    auto unmasked_groups = [&](int until) FA_INLINE {
      for (; it + C::NSTAGE <= until; it += C::NSTAGE)
        static_for<0, C::NSTAGE>([&](auto s) FA_INLINE { step(it + decltype(s)::value, s, std::false_type{}); });
    };
    if constexpr (CAUSAL) {
      const int j_end_full = min(n_kv, max(0, q0 + shift + 1) / BC);   // the tiles before it have no causal mask
      if constexpr (UP) {
        if constexpr (WIN) {
          const int first_full = min(n_kv, (max(0, q0 + C::BR - 1 + shift - a.window + 1) + BC - 1) / BC);
          masked_groups((first_full - j_begin + C::NSTAGE - 1) / C::NSTAGE * C::NSTAGE);
        }
        unmasked_groups(j_end_full - j_begin);
      } else {
        masked_groups((n_kv - max(j_end_full, j_begin) + C::NSTAGE - 1) / C::NSTAGE * C::NSTAGE);
        unmasked_groups(n_it);
      }
    }
    masked_groups(n_it);
    if (n_it > 0) wait_vm_barrier<0>();   // no load is left writing LDS (the ring is free again)

    if (qrow < a.Tq) {
      uint16_t* dst = a.dq + (qoff + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * half;
          const f32x16& q = dq_acc[db];
          *(u32x2*)(dst + d0) = u32x2{pack_bf16x2(q[4 * g4] * a.scale, q[4 * g4 + 1] * a.scale),
                                      pack_bf16x2(q[4 * g4 + 2] * a.scale, q[4 * g4 + 3] * a.scale)};
        }
    }
  };

  if constexpr (PAIR) {
    query_tile(unit, std::true_type{});
    const int qt2 = n_qtiles - 1 - unit;
    if (qt2 != unit) query_tile(qt2, std::false_type{});
  } else {
    query_tile(CAUSAL ? n_qtiles - 1 - unit : unit, std::true_type{});
  }
}

// ---------------------------------------------------------------- launch

// The default tiling, or (ALT) a second one of the same kernels, offered to
// check that the result does not depend on the tile shape: dQ takes 64-key
// tiles where the default takes 32 and 32 where it takes 64, dK/dV walks
// 32-row query tiles where the default walks 64 and 64 where it walks 32.
// One workgroup per CU with 64-key tiles at d = 128, for the dQ pass whose
// registers do not fit the two-workgroup tiling: dropout (the Philox bytes of
// a tile). The sliding window takes the two-workgroup tiling: its loop is
// split like the causal one (masked head, unmasked middle, masked tail).
template <int D>
using DqOneCfg = DqCfg<D, DqCfg<D>::NW, (D == 64 ? 32 : 64), (D == 64 ? 2 : 3), DqCfg<D>::IGLP, 1>;

template <int D, bool CAUSAL, bool WIN = false, bool DROP = false, bool ALT = false>
static hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  // non-causal d = 64, with or without dropout: 4-wave workgroups, four per
  // CU (measured on MI355X: GPT-2-shaped backward -1.3% and its dropout form
  // -1.6%, on top of the dK/dV tilings below; the causal masked body spills
  // in that shape and keeps 8 waves)
  using DQ64 = DqCfg<D, 4, 32, 2, -1, 4>;
  using QD = typename std::conditional<
      D == 64 && !CAUSAL, DQ64, typename std::conditional<DROP, DqOneCfg<D>, DqCfg<D>>::type>::type;
  using QC = typename std::conditional<ALT, DqCfg<D, QD::NW, (QD::BC == 32 ? 64 : 32)>, QD>::type;
  // dq first: it also stores the per-row statistics the dK/dV kernel reads
  const int n_qtiles = (a.Tq + QC::BR - 1) / QC::BR;
  // causal without a window: one workgroup per pair of query tiles p, n - 1 - p
  const int n_qunits = CAUSAL && !WIN ? (n_qtiles + 1) / 2 : n_qtiles;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, QC, WIN, DROP>), dim3((unsigned)(n_qunits * a.B * a.Hq)), dim3(QC::NT), 0,
                     stream, a, n_qtiles, n_qunits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // masked d = 64 tiles: 32-row query tiles (the 64-row masked body spills at
  // two waves per SIMD; measured 27% faster on a causal T2048 layer)
  // causal d = 128 with dropout: 32-row tiles as well (the mask bytes push the
  // 64-row masked body past 512 registers)
  // non-causal d = 64: 4-wave workgroups of 32-row tiles, three per CU at
  // 150 registers without dropout, two per CU at 188 with it (measured on
  // MI355X against one 8-wave workgroup of 64-row tiles: GPT-2-shaped
  // backward -6%, its dropout form -3%; three per CU spilled with dropout)
  using KD = typename std::conditional<
      D == 64 && CAUSAL, DkdvCfg<D, 8, 32>,
      typename std::conditional<
          DROP && CAUSAL, DkdvCfg<D, 4, 32>,
          typename std::conditional<D == 64, DkdvCfg<D, 4, 32, 2, 0, (DROP ? 2 : 3)>, DkdvCfg<D>>::type>::type>::type;
  // 16 keys per wave at d = 128, and for causal d = 64 (measured on MI355X:
  // causal GQA 32k backward -6%, its sliding-window form -22%, causal B64 H16
  // T1024 d64 -20%; the non-causal d = 64 layer timed the same with either
  // layout and keeps the 32-key one)
  if constexpr (!DROP && !ALT && (D == 128 || CAUSAL)) {
    // the sliding window takes a two-stage ring at d = 128 too (measured on
    // MI355X: -2.3% against three stages; the causal layers are no faster so)
    using K16 = Dkdv16Cfg<D, (WIN || D == 64) ? 2 : 3>;
    const int n_ktiles = (a.Tk + K16::BK - 1) / K16::BK;
    // causal without a window: one workgroup per pair of key tiles p, n - 1 - p
    const int n_units = CAUSAL && !WIN ? (n_ktiles + 1) / 2 : n_ktiles;
    hipLaunchKernelGGL((bwd_dkdv16_kernel<D, CAUSAL, K16, WIN>), dim3((unsigned)(n_units * a.B * a.Hkv)), dim3(K16::NT), 0,
                       stream, a, n_ktiles, n_units);
    return hipGetLastError();
  } else {
    using KC = typename std::conditional<ALT, DkdvCfg<D, KD::NW, (KD::BQ == 64 ? 32 : 64)>, KD>::type;
    const int n_ktiles = (a.Tk + KC::BK - 1) / KC::BK;
    // causal without a window: one workgroup per pair of key tiles p, n - 1 - p
    const int n_kunits = CAUSAL && !WIN ? (n_ktiles + 1) / 2 : n_ktiles;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, KC, WIN, DROP>), dim3((unsigned)(n_kunits * a.B * a.Hkv)), dim3(KC::NT),
                       0, stream, a, n_ktiles);
    return hipGetLastError();
  }
}

}  // namespace fa
