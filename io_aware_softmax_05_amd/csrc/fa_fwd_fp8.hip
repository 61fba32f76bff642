// fa_fwd_fp8.hip -- tiled exact attention forward on fp8 inputs, both products
// on the gfx950 fp8 matrix cores, bf16 output and fp32 log-sum-exp.
//
// Method: the tile loop of the bf16 forward (kgptalkie "Flash Attention: Why
// Memory Traffic, Not Compute, Is the Bottleneck", sections "Flash Attention
// Uses Tiles" and "Softmax Looks Like an Obstacle"; aimlrounds
// "FlashAttention", "Softmax without seeing the whole row"). The aimlrounds
// page's "FlashAttention 1, 2, 3" table credits FP8 to FlashAttention-3 and
// gives no recipe; the one used here:
//   * Inputs are OCP e4m3 bytes with one fp32 factor per (batch, head): the
//     value of a byte x of Q is x * q_scale[b, hq] (K and V alike, per kv
//     head). V arrives transposed, [B, Hkv, d, Tk], so the V^T tiles the PV
//     product reads are plain row reads (the caller's quantisation pass
//     writes that layout at no extra cost).
//   * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales;
//     scale * log2(e) * q_scale * k_scale folds into the exponent's FMA.
//   * P' = 2^(S c - m + 5) is rounded to e4m3 for O^T += V^T P'^T. The running
//     maximum m moves only when a row grows by more than 2^3, so P' <= 2^8,
//     inside e4m3's range (448); the shift keeps probabilities down to 2^-11
//     of the reference in e4m3's normal range. The row sum l uses the
//     unrounded fp32 P', and O = v_scale * O' / l (the 2^5 cancels).
//
// gfx950 mapping (rows and tiles as in the bf16 forward: 32 queries per wave,
// 64-key tiles, two-stage software pipeline, one barrier per tile, causal
// query tiles n - 1 - i and i in one workgroup, and the causal row-block
// pairing with per-wave skipping past the diagonal)
//   * MFMA row m of 32-key block kb reads key row
//     32 ((m >> 2) & 1) + 16 kb + 4 (m >> 3) + (m & 3) of the tile, so the S^T
//     accumulator register r of lane half h holds key 32 h + 16 kb + r: each
//     half of the wave owns 32 consecutive keys, which is exactly the k range
//     the half supplies to the PV product, so P' goes from the accumulators to
//     the B operand with no lane exchange.
//   * K rows (d bytes) and V^T rows (64 bytes) are stored unpadded in LDS with
//     an XOR swizzle of their 16-byte chunks that makes the 128-bit operand
//     reads and the tile stores conflict free on the 64 banks.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// D = A B + C on e4m3 A and B (format code 0 for both) with unit block
// scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int D>
struct Fp8Cfg {
  static constexpr int NW = D == 128 ? 8 : 4;   // waves per workgroup
  static constexpr int BR = 32 * NW;            // query rows per workgroup
  static constexpr int BC = 64;                 // keys per tile
  static constexpr int NT = 64 * NW;
  static constexpr int KCH = D / 16;            // 16-byte chunks per K row
  static constexpr int KTILE = BC * D;          // bytes of a K tile (unpadded)
  static constexpr int VTILE = D * BC;          // bytes of a V^T tile (d rows of 64 keys)
  static_assert(BC * KCH == NT && D * (BC / 16) == NT, "one K chunk and one V^T chunk per thread");
};

// chunk swizzles (checked conflict free for the reads and the stores)
template <int D>
__device__ __forceinline__ uint32_t swk(uint32_t r) {
  return D == 128 ? (((r >> 1) & 3u) | ((r >> 3) & 4u)) : (((r >> 2) & 1u) | ((r >> 4) & 2u));
}
__device__ __forceinline__ uint32_t swv(uint32_t r) { return (r >> 2) & 3u; }

constexpr float kSlack8 = 3.f;   // the reference maximum moves when a row grows by more than 2^3
constexpr float kShift8 = 5.f;   // P' = 2^(S c - m + 5) <= 2^8

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(Fp8Cfg<D>::NT, 8 / Fp8Cfg<D>::NW) void fwd_fp8_kernel(Fp8Args a) {
  using C = Fp8Cfg<D>;
  constexpr int BR = C::BR, BC = C::BC, KTILE = C::KTILE, VTILE = C::VTILE;
  constexpr int KS = D / 64;   // 64-deep steps of S^T over d
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * KTILE + 2 * VTILE];
  FA_LDS uint8_t* kbuf = (FA_LDS uint8_t*)smem_raw;
  FA_LDS uint8_t* vbuf = kbuf + 2 * KTILE;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;

  // Work order as in the bf16 forward: (batch, kv head) outermost, then the
  // work item, then the query heads of the group; a work item is one query
  // tile, or causal, query tiles n - 1 - i and i taken in turn.
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t G = (uint32_t)(a.Hq / a.Hkv);
  const uint32_t per_grp = (uint32_t)(CAUSAL ? (a.n_qtiles + 1) / 2 : a.n_qtiles) * G;
  const uint32_t kvg = t / per_grp, rr = t - kvg * per_grp;
  const int item = (int)(rr / G), g = (int)(rr - (uint32_t)item * G);
  const int b = (int)kvg / a.Hkv, hk = (int)kvg - b * a.Hkv;
  const int bh = b * a.Hq + hk * (int)G + g, bhk = b * a.Hkv + hk;
  // One query tile qt of this workgroup.
  auto run = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * BR;
    const size_t qoff = (size_t)bh * a.Tq * D;     // bytes
    const size_t kvoff = (size_t)bhk * a.Tk * D;   // bytes (K rows and V^T rows alike)
    const float c = a.c * a.q_scale[bh] * a.k_scale[bhk];   // log2 units per raw product
    const float v_scale = a.v_scale[bhk];
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + kvoff, (uint32_t)a.Tk * D);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vt + kvoff, (uint32_t)a.Tk * D);

    // Causal: key j is visible to row i iff j <= i + shift.
    const int shift = a.Tk - a.Tq;
    int kv_end = a.Tk;
    if (CAUSAL) kv_end = min(a.Tk, q0 + BR + shift);
    const int n_kv = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
    // Tiles [0, n_full) are complete and visible to every row of the workgroup.
    int n_full = a.Tk / BC;
    if (CAUSAL) n_full = min(n_full, max(0, q0 + shift + 1) / BC);
    n_full = min(n_full, n_kv - 1);

    // Q fragments (B operand of S^T): lane half h holds dims [64 ks + 32 h, +32).
    // Causal: the two waves that share a SIMD (w and w + NW / 2) take row
    // blocks b and NW - 1 - b, so every SIMD has the same share of the tiles
    // past the diagonal, which a wave skips when none of its rows sees them.
    const int rblk = CAUSAL && wave >= C::NW / 2 ? C::NW - 1 - (wave - C::NW / 2) : wave;
    const int qrow = q0 + rblk * 32 + col;
    // Tiles [0, w_full) are complete and visible to every row of this wave,
    // tiles [w_end, n_kv) to none of them.
    int w_full = n_full, w_end = n_kv;
    if (CAUSAL) {
      const int r_first = q0 + rblk * 32 + shift;
      w_full = __builtin_amdgcn_readfirstlane(max(n_full, min(a.Tk / BC, max(0, r_first + 1) / BC)));
      w_end = __builtin_amdgcn_readfirstlane(min(n_kv, (min(a.Tk, max(0, r_first + 32)) + BC - 1) / BC));
    }
    i32x8 qf[KS];
    {
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + qoff, (uint32_t)a.Tq * D);
      const uint32_t base = qrow < a.Tq ? (uint32_t)(qrow * D + 32 * half) : kOutOfRange;
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = join8(buf_load_b128(qrs, base + 64 * ks), buf_load_b128(qrs, base + 64 * ks + 16));
    }

    f32x16 oacc[D / 32];
  #pragma unroll
    for (int db = 0; db < D / 32; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = -INFINITY;   // reference maximum of the scaled scores, log2 units
    float l = 0.f;         // this lane's partial running sum of P'
    float lc = 0.f;        // its compensation (l - lc is the sum)

    // This thread's chunk of each tile: K row kr, chunk kc; V^T row vr, chunk vc.
    const int kr = tid / C::KCH, kc = tid % C::KCH;
    const uint32_t k_goff = (uint32_t)(kr * D + kc * 16);
    const uint32_t k_lds = (uint32_t)(kr * D) + ((kc ^ swk<D>(kr)) * 16);
    const int vr = tid >> 2, vc = tid & 3;
    const uint32_t v_lds = (uint32_t)(vr * BC) + ((vc ^ swv(vr)) * 16);
    u32x4 kst, vst;
    auto load_k = [&](int j) { kst = buf_load_b128(krs, j < n_kv ? (uint32_t)(j * BC * D) + k_goff : kOutOfRange); };
    // V^T rows are Tk bytes long (Tk a multiple of 16): a chunk past the row end reads zeros
    auto load_v = [&](int j) {
      const int key = j * BC + vc * 16;
      vst = buf_load_b128(vrs, (j < n_kv && key < a.Tk) ? (uint32_t)vr * (uint32_t)a.Tk + (uint32_t)key : kOutOfRange);
    };
    auto store_k = [&](int buf) { lds_write_b128(kbuf + buf * KTILE, k_lds, kst); };
    auto store_v = [&](int buf) { lds_write_b128(vbuf + buf * VTILE, v_lds, vst); };

    // S^T[key, query] for the 64 keys of the tile in `buf` and this wave's 32 queries.
    const int krow0 = 32 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    auto scores = [&](int buf, f32x16* s) {
      const FA_LDS uint8_t* kt = kbuf + buf * KTILE;
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t row = (uint32_t)(krow0 + 16 * kb), sw = swk<D>(row);
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t c0 = 4 * ks + 2 * half;
          const u32x4 lo = lds_read_b128(kt, row * D + ((c0 ^ sw) * 16));
          const u32x4 hi = lds_read_b128(kt, row * D + (((c0 + 1) ^ sw) * 16));
          // the first product starts from an inline zero (no register clearing)
          s[kb] = mfma32_fp8(join8(lo, hi), qf[ks], ks == 0 ? f32x16{} : s[kb]);
        }
      }
    };
    // keys past the causal limit or past Tk get -inf
    auto mask = [&](int j, f32x16* s) {
      const int lim = CAUSAL ? min(a.Tk - 1, qrow + shift) : a.Tk - 1;
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j * BC + 32 * half + 16 * kb + r > lim) s[kb][r] = -INFINITY;
    };
    // row maximum: in-lane over 32 keys, then the partner half (lane ^ 32)
    auto rowmax = [&](const f32x16* s) -> float {
      float mx = -INFINITY;
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      return pair_max32(mx);
    };

    // V^T operand rows of this lane: d = 32 db + col, keys [32 half, +32).
    auto pv = [&](int buf, i32x8 pb) {
      const FA_LDS uint8_t* vt = vbuf + buf * VTILE;
  #pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint32_t row = (uint32_t)(32 * db + col), sw = swv(row);
        const u32x4 lo = lds_read_b128(vt, row * BC + (((2 * half) ^ sw) * 16));
        const u32x4 hi = lds_read_b128(vt, row * BC + (((2 * half + 1) ^ sw) * 16));
        oacc[db] = mfma32_fp8(join8(lo, hi), pb, oacc[db]);
      }
    };

    // LDS ring: iteration j reads K_{j+1} from kbuf[(j+1)&1] and V_j from
    // vbuf[j&1]; it refills kbuf[j&1] with K_{j+2} and vbuf[(j+1)&1] with V_{j+1}.
    f32x16 s_a[2], s_b[2];
    if (n_kv > 0) {
      load_k(0);
      load_v(0);
      store_k(0);
      store_v(0);
      load_k(1);
      store_k(1);
      __syncthreads();
      scores(0, s_a);
      if (0 >= n_full) mask(0, s_a);
      m = rowmax(s_a) * c;   // l and u are still zero: nothing to rescale
      __syncthreads();       // every wave has read K_0 before K_2 replaces it
    }

    // Tile j (s_cur = S_j, masked; m covers it): P'_j and O' += V_j P'_j, while
    // S_{j+1} goes to s_nxt, is masked if needed, and its row max moves m.
    auto body = [&](int j, auto next_masked, auto has_next, f32x16* s_cur, f32x16* s_nxt) {
      constexpr bool HN = decltype(has_next)::value;
      constexpr bool NM = decltype(next_masked)::value;
      load_k(j + 2);
      load_v(j + 1);
      // masked stretch: this wave's rows may see none of tile j or j + 1
      const bool cur_live = !(CAUSAL && NM) || j < w_end;
      const bool nxt_live = !(CAUSAL && NM) || j + 1 < w_end;
      const float neg_ref = kShift8 - ((m == -INFINITY) ? 0.f : m);
      // stage A: S_{j+1} on the matrix cores, P'_j on the vector unit
      if constexpr (HN) {
        if (nxt_live) scores((j + 1) & 1, s_nxt);
      }
      float lsum = 0.f;
      if (cur_live) {
        uint32_t pw[8];
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const float p0 = exp2_fast(fmaf(s_cur[kb][r], c, neg_ref));
            const float p1 = exp2_fast(fmaf(s_cur[kb][r + 1], c, neg_ref));
            const float p2 = exp2_fast(fmaf(s_cur[kb][r + 2], c, neg_ref));
            const float p3 = exp2_fast(fmaf(s_cur[kb][r + 3], c, neg_ref));
            lsum += (p0 + p1) + (p2 + p3);
            // bytes 16 kb + r .. +3 of this half: keys 32 half + 16 kb + r .. +3
            const int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
            pw[4 * kb + r / 4] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
          }
        const i32x8 pb = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
        __builtin_amdgcn_iglp_opt(0);
        // stage B: O'^T[d, query] += V^T[d, key] P'^T[key, query]
        pv(j & 1, pb);
      }
      kahan_add(l, lc, lsum);
      if constexpr (HN) {
        float m_new = m;
        if (nxt_live) {
          if constexpr (NM) {
            if (!CAUSAL || j + 1 >= w_full) mask(j + 1, s_nxt);
          }
          m_new = fmaxf(m, rowmax(s_nxt) * c);
        }
        const bool move = __builtin_amdgcn_ballot_w64(m_new > m + kSlack8) != 0;
        store_k(j & 1);
        store_v((j + 1) & 1);
        if (move) {
          // move the reference: l and u are rescaled together (after O' += V_j P'_j)
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
    // after the tiles every row sees completely, each next tile is masked.
    int j = 0;
    for (; j + 2 < n_full; j += 2) {
      body(j, std::false_type{}, std::true_type{}, s_a, s_b);
      body(j + 1, std::false_type{}, std::true_type{}, s_b, s_a);
    }
    for (; j + 2 < n_kv; j += 2) {
      body(j, std::true_type{}, std::true_type{}, s_a, s_b);
      body(j + 1, std::true_type{}, std::true_type{}, s_b, s_a);
    }
    if (j + 1 < n_kv) {
      body(j, std::true_type{}, std::true_type{}, s_a, s_b);
      body(j + 1, std::true_type{}, std::false_type{}, s_b, s_a);
    } else if (j < n_kv) {
      body(j, std::true_type{}, std::false_type{}, s_a, s_b);
    }

    const float l_tot = pair_sum32(l - lc);
    const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
    if (qrow < a.Tq) {
      uint16_t* dst = a.o + (size_t)bh * a.Tq * D + (size_t)qrow * D;
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
        a.lse[(size_t)bh * a.Tq + qrow] = l_tot > 0.f ? (m + log2_fast(l_tot) - kShift8) * kLn2 : -INFINITY;
    }
  };

  if constexpr (CAUSAL) {
    run(a.n_qtiles - 1 - item);
    if (2 * item + 1 != a.n_qtiles) {   // the middle tile of an odd count runs alone
      __syncthreads();                  // every wave is done with the first tile's K/V in LDS
      run(item);
    }
  } else {
    run(item);
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fp8(Fp8Args a, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  a.n_qtiles = (a.Tq + C::BR - 1) / C::BR;
  const uint32_t items = CAUSAL ? (a.n_qtiles + 1) / 2 : a.n_qtiles;   // paired causal tiles
  const uint32_t n = items * (uint32_t)(a.B * a.Hq);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(n), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

int fwd_fp8_rows_per_workgroup(int d) { return d == 128 ? Fp8Cfg<128>::BR : Fp8Cfg<64>::BR; }

hipError_t launch_fwd_fp8(Fp8Args a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fp8<64, true>(a, stream) : launch_fp8<64, false>(a, stream);
  return causal ? launch_fp8<128, true>(a, stream) : launch_fp8<128, false>(a, stream);
}

}  // namespace fa
