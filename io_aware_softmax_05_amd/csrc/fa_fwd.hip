// fa_fwd.hip -- tiled exact attention forward, bf16 in/out, fp32 accumulation.
//
// Method (kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
// Bottleneck", sections "Flash Attention Uses Tiles" and "Softmax Looks Like
// an Obstacle"; aimlrounds "FlashAttention", "Softmax without seeing the
// whole row"): a tile of queries stays on chip while key/value tiles stream
// past it; each query row keeps a running maximum m, a running sum l of
// exponentials relative to m, and a running weighted sum u; when the maximum
// moves to m', l and u are both scaled by e^(m - m') before the tile's own
// terms are added. Scores and probabilities live only in registers.
//
// gfx950 mapping
//   * workgroup = NW waves x 32 query rows (NW = 8 at d = 128, 4 at d = 64);
//     grid = work items x heads x batch, remapped so that the tiles of one
//     kv head (all query heads that share it) run on one XCD and its L2,
//     query heads of a group side by side. A work item is one query tile,
//     but causal without a window it is query tiles n - 1 - i and i, taken
//     in turn (the same work for every workgroup); with a window the tiles
//     run longest first.
//     Causal: waves w and w + NW / 2 (one SIMD) take row blocks b and
//     NW - 1 - b, and past the diagonal (or, with a window, below the band)
//     a wave skips the tiles none of its rows sees, so the SIMDs share those
//     stretches evenly.
//   * 64-key K and V tiles stream HBM -> registers -> LDS through buffer
//     loads (out-of-range rows read as zeros, so the loop has no branches),
//     double buffered with one barrier per tile. Row pitches are chosen for
//     the 64-bank LDS: K rows are padded by 16 bytes (the 16 lanes of a
//     128-bit row read land on distinct banks), V rows by 64 bytes (the
//     transposed 64-bit reads land on distinct banks).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query
//     column and 16 keys of a 32-key block, so the row maximum is an in-lane
//     max plus one permlane32 swap and the running sum stays a per-lane
//     partial until the end.
//   * O^T = V^T P^T: the probabilities are reused straight from the S^T
//     accumulator layout as the B operand, V^T comes from ds_read_b64_tr_b16,
//     and every O^T register of a lane belongs to that lane's query.
//   * Two-stage software pipeline per key tile j: stage A issues the MFMAs
//     of S_{j+1} = K_{j+1} Q^T while the vector unit turns S_j into
//     probabilities; stage B issues O += V_j P_j while the vector unit takes
//     the row maximum of S_{j+1}. A compiler interleave strategy orders the
//     instructions of each stage (small-GEMM at d = 128, MFMA/exp at d = 64).
//   * The running maximum is only moved when some row of the wave grows by
//     more than 2^8; otherwise the stale maximum is kept, the probabilities
//     stay below 256 and l and u need no rescale (the result is the same up
//     to rounding, since l and u always share one reference).
//   * exponentials are exp2 with scale*log2(e) folded into one FMA; the row
//     sum adds the fp32 probabilities, so the saved log-sum-exp keeps fp32
//     accuracy for the backward.
//   * dropout (the DROP instantiations): probabilities are dropped after the
//     row sum and before the product with V (zerotofrontier "Efficient
//     attention: memory-bound", section "Real code moves even more", places
//     dropout there in a training forward pass). Each lane draws the Philox
//     bytes of its row for one 16-key group per 32-key block and swaps half
//     of them with its partner lane; the 256 / t rescale rides on 1 / l.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

// Default tiling: 8 waves (256 query rows) at d = 128, 4 waves at d = 64,
// 64-key tiles. FwdAltCfg is a second tiling of the same kernel (32-key tiles,
// and 128-row query tiles at d = 128), offered to check that the result does
// not depend on the tile shape.
template <int D, int NW_ = (D == 128 ? 8 : 4), int BC_ = 64>
struct FwdCfg {
  static constexpr int NW = NW_;                // waves per workgroup
  static constexpr int BR = 32 * NW;            // query rows per workgroup
  static constexpr int BC = BC_;                // keys per tile
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int KPITCH = (D + 8) * 2;    // LDS bytes per K row
  static constexpr int VPITCH = (D + 32) * 2;   // LDS bytes per V row
  static constexpr int KTILE = BC * KPITCH;
  static constexpr int VTILE = BC * VPITCH;
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int LOADS = BC * CH / NT;    // chunks per thread per tile
  static_assert(LOADS >= 1 && LOADS * NT == BC * CH, "a tile must split evenly over the workgroup");
};

template <int D>
using FwdAltCfg = FwdCfg<D, 4, 32>;

// Stale-maximum allowance (log2 units): probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.f;

}  // namespace

template <int D, bool CAUSAL, bool WIN = false, bool DROP = false, class C = FwdCfg<D>>
__global__ __launch_bounds__(C::NT, 8 / C::NW) void fwd_bf16_kernel(FwdArgs a) {
  static_assert(CAUSAL || !WIN, "a sliding window is a causal band");
  static_assert(!(WIN && DROP), "dropout is not offered with a sliding window");
  constexpr int BR = C::BR, BC = C::BC, NT = C::NT, CH = C::CH, LOADS = C::LOADS;
  constexpr int KPITCH = C::KPITCH, VPITCH = C::VPITCH, KTILE = C::KTILE, VTILE = C::VTILE;
  constexpr int KB = BC / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * KTILE + 2 * VTILE];
  FA_LDS uint8_t* kbuf = (FA_LDS uint8_t*)smem_raw;
  FA_LDS uint8_t* vbuf = kbuf + 2 * KTILE;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5;             // which 16-key half of a 32-key block
  const int col = lane & 31;              // query column owned by this lane

  // Work order: (batch, kv head) outermost, then work item, then the query
  // heads that share the kv head, so the workgroups that run together on an
  // XCD read the same K/V tiles at about the same time. A work item is one
  // query tile; causal without a window, item i is the pair of query tiles
  // n - 1 - i and i, which together see about n + 1 tiles of keys, so every
  // workgroup has the same work and pays its start (Q fragments, the first
  // K/V tiles in flight) once per two query tiles.
  constexpr bool PAIRED = CAUSAL && !WIN;
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t G = (uint32_t)(a.Hq / a.Hkv);
  const uint32_t per_grp = (uint32_t)(PAIRED ? (a.n_qtiles + 1) / 2 : a.n_qtiles) * G;
  const uint32_t kvg = t / per_grp, r = t - kvg * per_grp;
  const int item = (int)(r / G), g = (int)(r - (uint32_t)item * G);
  const int b = (int)kvg / a.Hkv, hk = (int)kvg - b * a.Hkv;
  const int h = hk * (int)G + g, bh = b * a.Hq + h;
  // One query tile qt of this workgroup.
  auto run = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * BR;
    const size_t qoff = (size_t)bh * a.Tq * D;
    const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + kvoff, (uint32_t)a.Tk * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + kvoff, (uint32_t)a.Tk * D * 2);

    // Causal: key j is visible to row i iff j <= i + shift.
    const int shift = a.Tk - a.Tq;
    int kv_end = a.Tk;
    if (CAUSAL) kv_end = min(a.Tk, q0 + BR + shift);
    const int n_kv = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
    // Tiles [0, n_full) are complete and visible to every row of the workgroup.
    int n_full = a.Tk / BC;
    if (CAUSAL) n_full = min(n_full, max(0, q0 + shift + 1) / BC);
    n_full = min(n_full, n_kv - 1);
    // Sliding window: row i sees keys (i + shift - W, i + shift]. Tiles before
    // j_begin are invisible to every row; tiles [j_begin, j_head) hold keys
    // below some row's window and need the mask.
    int j_begin = 0, j_head = 0;
    if (WIN) {
      j_begin = min(n_kv, max(0, q0 + shift - a.window + 1) / BC);
      const int lo_last = q0 + BR - 1 + shift - a.window + 1;   // window start of the last row
      j_head = min(n_kv, max(j_begin, (max(0, lo_last) + BC - 1) / BC));
    }

    // Causal: the two waves that share a SIMD (w and w + NW / 2) take row
    // blocks b and NW - 1 - b, so every SIMD has the same share of the tiles
    // past the diagonal (and below a window), which a wave skips when none of
    // its rows sees them.
    constexpr bool SKIP = CAUSAL && !DROP;
    const int rblk = SKIP && wave >= C::NW / 2 ? C::NW - 1 - (wave - C::NW / 2) : wave;
    const int qrow = q0 + rblk * 32 + col;
    // Tiles [w_head, w_full) are complete and visible to every row of this
    // wave; tiles before w_begin (below every row's window) and from w_end on
    // are visible to none of them.
    int w_begin = j_begin, w_head = j_head, w_full = n_full, w_end = n_kv;
    if (SKIP) {
      const int r_first = q0 + rblk * 32 + shift;
      w_full = __builtin_amdgcn_readfirstlane(max(n_full, min(a.Tk / BC, max(0, r_first + 1) / BC)));
      w_end = __builtin_amdgcn_readfirstlane(min(n_kv, (min(a.Tk, max(0, r_first + 32)) + BC - 1) / BC));
      if (WIN) {
        w_begin = __builtin_amdgcn_readfirstlane(max(j_begin, min(n_kv, max(0, r_first - a.window + 1) / BC)));
        w_head = __builtin_amdgcn_readfirstlane(min(j_head, max(w_begin, (max(0, r_first + 31 - a.window + 1) + BC - 1) / BC)));
      }
    }

    // Q fragments: B operand of S^T = K Q^T (lane: query column, 8 dims).
    bf16x8 qf[D / 16];
    {
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + qoff, (uint32_t)a.Tq * D * 2);
      const uint32_t base = qrow < a.Tq ? (uint32_t)(qrow * D + 8 * half) * 2 : kOutOfRange;
  #pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(buf_load_b128(qrs, base + ks * 32));
    }

    f32x16 oacc[D / 32];
  #pragma unroll
    for (int db = 0; db < D / 32; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = -INFINITY;   // running max of scaled scores, log2 units
    float l = 0.f;         // this lane's partial running sum
    float lc = 0.f;        // its compensation (l - lc is the sum)

    // This thread's share of a tile: LOADS 16-byte chunks (row, chunk).
    uint32_t g_off[LOADS], k_lds[LOADS], v_lds[LOADS];
  #pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = i * NT + tid;
      const int row = c / CH, ch = c % CH;
      g_off[i] = (uint32_t)(row * D + ch * 8) * 2;
      k_lds[i] = row * KPITCH + ch * 16;
      v_lds[i] = row * VPITCH + ch * 16;
    }
    u32x4 kst[LOADS], vst[LOADS];
    auto tile_base = [&](int j) -> uint32_t { return j < n_kv ? (uint32_t)(j * BC * D * 2) : kOutOfRange; };
    auto load_k = [&](int j) {
      const uint32_t tb = tile_base(j);
  #pragma unroll
      for (int i = 0; i < LOADS; ++i) kst[i] = buf_load_b128(krs, tb + g_off[i]);
    };
    auto load_v = [&](int j) {
      const uint32_t tb = tile_base(j);
  #pragma unroll
      for (int i = 0; i < LOADS; ++i) vst[i] = buf_load_b128(vrs, tb + g_off[i]);
    };
    auto store_k = [&](int buf) {
  #pragma unroll
      for (int i = 0; i < LOADS; ++i) lds_write_b128(kbuf + buf * KTILE, k_lds[i], kst[i]);
    };
    auto store_v = [&](int buf) {
  #pragma unroll
      for (int i = 0; i < LOADS; ++i) lds_write_b128(vbuf + buf * VTILE, v_lds[i], vst[i]);
    };

    // S^T[key, query] for the BC keys of the tile in `buf` and this wave's 32 queries.
    const uint32_t k_rd = col * KPITCH + 16 * half;
    auto scores = [&](int buf, f32x16* s) {
      const FA_LDS uint8_t* kb = kbuf + buf * KTILE + k_rd;
  #pragma unroll
      for (int kb_i = 0; kb_i < KB; ++kb_i) {
  #pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 kv = lds_read_b128(kb, kb_i * 32 * KPITCH + ks * 32);
          // the first product starts from an inline zero (no register clearing)
          s[kb_i] = mfma32(as_bf16x8(kv), qf[ks], ks == 0 ? f32x16{} : s[kb_i]);
        }
      }
    };
    // keys past the causal limit or past Tk (or before the window) get -inf
    auto mask = [&](int j, f32x16* s) {
      const int key_base = j * BC;
      const int lim = CAUSAL ? min(a.Tk - 1, qrow + shift) : a.Tk - 1;
      const int lo = WIN ? qrow + shift - a.window + 1 : 0;
  #pragma unroll
      for (int kb_i = 0; kb_i < KB; ++kb_i)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key_base + kb_i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > lim || (WIN && key < lo)) s[kb_i][r] = -INFINITY;
        }
    };
    // row maximum: in-lane over 16 keys per block, then the partner half (lane ^ 32)
    auto rowmax = [&](const f32x16* s) -> float {
      float mx = -INFINITY;
  #pragma unroll
      for (int kb_i = 0; kb_i < KB; ++kb_i)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb_i][r]);
      return pair_max32(mx);
    };

    // Transposed-read coordinates of this lane inside its 16-lane group.
    const int grp = lane >> 4, gi = lane & 15;
    const int tr_row = 4 * (grp >> 1) + (gi >> 2);
    const int tr_col = 16 * (grp & 1) + 4 * (gi & 3);
    const uint32_t v_rd = tr_row * VPITCH + tr_col * 2;

    // LDS ring: iteration j reads K_{j+1} from kbuf[(j+1)&1] and V_j from
    // vbuf[j&1]; it refills kbuf[j&1] with K_{j+2} and vbuf[(j+1)&1] with V_{j+1}.
    f32x16 s_a[KB], s_b[KB];
    // Dropout: the Philox bytes of this lane's row for the 32-key blocks of a tile.
    u32x4 z_a[KB], z_b[KB];
    auto drop_bytes = [&](int j, int kb_i) -> u32x4 {
      return dropout_bytes_32keys((uint32_t)(j * BC + kb_i * 32), (uint32_t)qrow, (uint32_t)bh, a.drop.offset,
                                  a.drop.seed_lo, a.drop.seed_hi, half);
    };
    const int j0 = j_begin;
    if (j0 < n_kv) {
      load_k(j0);
      load_v(j0);
      store_k(j0 & 1);
      store_v(j0 & 1);
      load_k(j0 + 1);
      store_k((j0 + 1) & 1);
      __syncthreads();
      scores(j0 & 1, s_a);
      if constexpr (DROP) {   // dropout bytes of the first tile; later tiles draw theirs a tile ahead
  #pragma unroll
        for (int kb_i = 0; kb_i < KB; ++kb_i) z_a[kb_i] = drop_bytes(j0, kb_i);
      }
      if (j0 >= n_full || j0 < j_head) mask(j0, s_a);
      m = rowmax(s_a) * a.c;   // l and u are still zero: nothing to rescale
      __syncthreads();         // every wave has read K_j0 before K_j0+2 replaces it
    }

    // Tile j (s_cur = S_j, masked; m covers it): P_j and O += V_j P_j, while
    // S_{j+1} goes to s_nxt, is masked if needed, and its row max moves m.
    auto body = [&](int j, auto next_masked, auto has_next, f32x16* s_cur, f32x16* s_nxt, u32x4* z_cur,
                    u32x4* z_nxt) {
      constexpr bool HN = decltype(has_next)::value;
      constexpr bool NM = decltype(next_masked)::value;
      load_k(j + 2);
      load_v(j + 1);
      // masked stretch: this wave's rows may see none of tile j or j + 1
      const bool cur_live = !(SKIP && NM) || (j < w_end && j >= w_begin);
      const bool nxt_live = !(SKIP && NM) || (j + 1 < w_end && j + 1 >= w_begin);
      const float m_ref = (m == -INFINITY) ? 0.f : m;
      // stage A: S_{j+1} on the matrix cores, P_j = 2^(S_j c - m) on the vector unit
      if constexpr (HN) {
        if (nxt_live) scores((j + 1) & 1, s_nxt);
      }
      bf16x8 pb[KB * 2];
      float lsum = 0.f;
      if (cur_live) {
  #pragma unroll
        for (int kb_i = 0; kb_i < KB; ++kb_i) {
          // dropout: the row sum takes every probability, the product with V only the kept ones
          const u32x4 zb = z_cur[kb_i];
  #pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            uint32_t pw[4];
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * hs + 2 * e;
              float p0 = exp2_fast(fmaf(s_cur[kb_i][r], a.c, -m_ref));
              float p1 = exp2_fast(fmaf(s_cur[kb_i][r + 1], a.c, -m_ref));
              lsum += p0 + p1;
              if constexpr (DROP) {
                if (!dropout_keep(zb, r, a.drop.t)) p0 = 0.f;
                if (!dropout_keep(zb, r + 1, a.drop.t)) p1 = 0.f;
              }
              pw[e] = pack_bf16x2(p0, p1);
            }
            pb[kb_i * 2 + hs] = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
          }
        }
        // the compiler's interleave strategy: the small-GEMM one (0) at d = 128,
        // the MFMA/exp one (2) at d = 64 (each measured fastest on MI355X there)
        __builtin_amdgcn_iglp_opt(D == 128 ? 0 : 2);
        // stage B: O^T[d, query] += V^T[d, key] P^T[key, query], 16 keys per step
        const FA_LDS uint8_t* vb = vbuf + (j & 1) * VTILE + v_rd;
  #pragma unroll
        for (int kb_i = 0; kb_i < KB; ++kb_i)
  #pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int row = kb_i * 32 + hs * 16;
  #pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const u32x2 lo = lds_read_tr(vb, row * VPITCH + db * 64);
              const u32x2 hi = lds_read_tr(vb, (row + 8) * VPITCH + db * 64);
              oacc[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[kb_i * 2 + hs], oacc[db]);
            }
          }
      }
      // the next tile's dropout bytes, drawn while the matrix cores run O += V_j P_j
      if constexpr (DROP && HN) {
  #pragma unroll
        for (int kb_i = 0; kb_i < KB; ++kb_i) z_nxt[kb_i] = drop_bytes(j + 1, kb_i);
      }
      kahan_add(l, lc, lsum);
      if constexpr (HN) {
        float m_new = m;
        if (nxt_live) {
          if constexpr (NM) {
            if (!SKIP || j + 1 >= w_full || (WIN && j + 1 < w_head)) mask(j + 1, s_nxt);
          }
          m_new = fmaxf(m, rowmax(s_nxt) * a.c);
        }
        const bool move = __builtin_amdgcn_ballot_w64(m_new > m + kRescaleSlack) != 0;
        store_k(j & 1);
        store_v((j + 1) & 1);
        if (move) {
          // move the reference: l and u are rescaled together (after O += V_j P_j)
          const float alpha = exp2_fast(m - (m_new == -INFINITY ? 0.f : m_new));
          l *= alpha;
          lc *= alpha;
  #pragma unroll
          for (int db = 0; db < D / 32; ++db)
  #pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          m = m_new;
        }
        __syncthreads();
      }
    };

    // Unrolled by two so that the score registers swap roles without copies;
    // after the tiles every row sees completely, each next tile is masked (a
    // complete tile passes through the mask unchanged).
    int j = j0;
    if constexpr (WIN) {   // the window's first tiles: masked, one at a time
      for (; j + 1 < j_head; ++j) {
        body(j, std::true_type{}, std::true_type{}, s_a, s_b, z_a, z_b);
  #pragma unroll
        for (int kb_i = 0; kb_i < KB; ++kb_i) s_a[kb_i] = s_b[kb_i];
      }
    }
    for (; j + 2 < n_full; j += 2) {
      body(j, std::false_type{}, std::true_type{}, s_a, s_b, z_a, z_b);
      body(j + 1, std::false_type{}, std::true_type{}, s_b, s_a, z_b, z_a);
    }
    for (; j + 2 < n_kv; j += 2) {
      body(j, std::true_type{}, std::true_type{}, s_a, s_b, z_a, z_b);
      body(j + 1, std::true_type{}, std::true_type{}, s_b, s_a, z_b, z_a);
    }
    if (j + 1 < n_kv) {
      body(j, std::true_type{}, std::true_type{}, s_a, s_b, z_a, z_b);
      body(j + 1, std::true_type{}, std::false_type{}, s_b, s_a, z_b, z_a);
    } else if (j < n_kv) {
      body(j, std::true_type{}, std::false_type{}, s_a, s_b, z_a, z_b);
    }

    const float l_tot = pair_sum32(l - lc);
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if constexpr (DROP) inv *= a.drop.inv_keep;   // kept probabilities are scaled by 256 / t
    if (qrow < a.Tq) {
      uint16_t* dst = a.o + qoff + (size_t)qrow * D;
  #pragma unroll
      for (int db = 0; db < D / 32; ++db)
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * half;
          const u32x2 w = {pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                           pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
          *(u32x2*)(dst + d0) = w;
        }
      if (a.lse != nullptr && half == 0)
        a.lse[(size_t)bh * a.Tq + qrow] = l_tot > 0.f ? (m + log2_fast(l_tot)) * kLn2 : -INFINITY;
    }
  };

  if constexpr (PAIRED) {
    run(a.n_qtiles - 1 - item);
    if (2 * item + 1 != a.n_qtiles) {   // the middle tile of an odd count runs alone
      __syncthreads();                  // every wave is done with the first tile's K/V in LDS
      run(item);
    }
  } else {
    run(CAUSAL ? a.n_qtiles - 1 - item : item);   // a window's short first tiles last
  }
}

template <int D, bool CAUSAL, bool WIN = false, bool DROP = false, class C = FwdCfg<D>>
static hipError_t launch_fwd(FwdArgs a, hipStream_t stream) {
  a.n_qtiles = (a.Tq + C::BR - 1) / C::BR;
  const uint32_t items = (CAUSAL && !WIN) ? (a.n_qtiles + 1) / 2 : a.n_qtiles;   // paired causal tiles
  const uint32_t n = items * (uint32_t)(a.B * a.Hq);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, WIN, DROP, C>), dim3(n), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

// the smallest query tile of either tiling (grid-size checks use it)
int fwd_rows_per_workgroup(int d) { return d == 128 ? FwdAltCfg<128>::BR : FwdAltCfg<64>::BR; }

hipError_t launch_fwd_bf16_alt_tiles(FwdArgs a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fwd<64, true, false, false, FwdAltCfg<64>>(a, stream)
                             : launch_fwd<64, false, false, false, FwdAltCfg<64>>(a, stream);
  return causal ? launch_fwd<128, true, false, false, FwdAltCfg<128>>(a, stream)
                : launch_fwd<128, false, false, false, FwdAltCfg<128>>(a, stream);
}

hipError_t launch_fwd_bf16(FwdArgs a, int d, bool causal, hipStream_t stream) {
  if (a.window > 0) return d == 64 ? launch_fwd<64, true, true>(a, stream) : launch_fwd<128, true, true>(a, stream);
  if (a.drop.t != 0) {
    if (d == 64) return causal ? launch_fwd<64, true, false, true>(a, stream) : launch_fwd<64, false, false, true>(a, stream);
    return causal ? launch_fwd<128, true, false, true>(a, stream) : launch_fwd<128, false, false, true>(a, stream);
  }
  if (d == 64) return causal ? launch_fwd<64, true>(a, stream) : launch_fwd<64, false>(a, stream);
  return causal ? launch_fwd<128, true>(a, stream) : launch_fwd<128, false>(a, stream);
}

}  // namespace fa
