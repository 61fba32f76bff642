// fa_fwd.hip -- tiled exact attention forward, bf16 in/out, fp32 accumulation.
//
// Method (kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
// Bottleneck", sections "Flash Attention Uses Tiles" and "Softmax Looks Like
// an Obstacle"; aimlrounds "FlashAttention", "Softmax without seeing the
// whole row"): a tile of queries stays on chip while key/value tiles stream
// past it; each query row keeps a running maximum m, a running sum l of
// exponentials relative to m, and a running weighted sum u; when a tile
// raises the maximum to m', l and u are both scaled by e^(m - m') before the
// tile's own terms are added. Scores and probabilities live only in
// registers.
//
// gfx950 mapping
//   * workgroup = 4 waves = 128 query rows (32 per wave); grid = query tiles
//     x heads x batch, remapped so the tiles of one head share an XCD (and
//     its L2), causal tiles longest first.
//   * K and V tiles of 64 keys stream HBM -> registers -> LDS, double
//     buffered (one barrier per tile). Rows are padded by 32 bytes so that
//     both the row reads of K and the transposed reads of V are free of
//     bank conflicts.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query
//     column and 16 keys, so the row maximum is an in-lane max plus one
//     permlane32 swap, and the running sum stays a per-lane partial until
//     the end.
//   * O^T = V^T P^T: the probabilities are reused straight from the S^T
//     accumulator layout as the B operand (the contraction order over keys
//     is permuted identically on the A side), V^T comes from
//     ds_read_b64_tr_b16; every O^T register of a lane belongs to that
//     lane's query, so the e^(m - m') rescale is a per-lane scalar.
//   * exponentials are exp2 with scale*log2(e) folded into one FMA.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BR = 128;                 // query rows per workgroup
  constexpr int BC = 64;                  // keys per tile
  constexpr int PITCH = (D + 16) * 2;     // LDS bytes per key row
  constexpr int TILE = BC * PITCH;        // LDS bytes per K (or V) tile
  constexpr int CH = D / 8;               // 16-byte chunks per key row
  constexpr int LOADS = BC * CH / 256;    // chunks per thread per tensor
  static_assert(LOADS * 256 == BC * CH, "tile must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * 2 * TILE];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5;             // which 16-key half of a 32-key block
  const int col = lane & 31;              // query column owned by this lane

  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int qt_lin = (int)(t % (uint32_t)a.n_qtiles);
  const int bh = (int)(t / (uint32_t)a.n_qtiles);
  const int qt = CAUSAL ? (a.n_qtiles - 1 - qt_lin) : qt_lin;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int q0 = qt * BR;
  const size_t qoff = (size_t)bh * a.Tq * D;
  const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const uint16_t* __restrict__ Kp = a.k + kvoff;
  const uint16_t* __restrict__ Vp = a.v + kvoff;

  // Causal: key j is visible to row i iff j <= i + shift.
  const int shift = a.Tk - a.Tq;
  int kv_end = a.Tk;
  if (CAUSAL) kv_end = min(a.Tk, q0 + BR + shift);
  const int n_kv = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // Q fragments: B operand of S^T = K Q^T (lane: query col, 8 dims).
  const int qrow = q0 + wave * 32 + col;
  bf16x8 qf[D / 16];
  if (qrow < a.Tq) {
    const uint16_t* src = a.q + qoff + (size_t)qrow * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(global_load_b128(src + ks * 16));
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(u32x4{0, 0, 0, 0});
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -INFINITY;   // running max of scaled scores, log2 units
  float l = 0.f;         // this lane's partial running sum

  u32x4 kst[LOADS], vst[LOADS];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = i * 256 + tid;
      const int row = c / CH, ch = c % CH;
      const int key = j * BC + row;
      if (key < a.Tk) {
        kst[i] = global_load_b128(Kp + (size_t)key * D + ch * 8);
        vst[i] = global_load_b128(Vp + (size_t)key * D + ch * 8);
      } else {
        kst[i] = u32x4{0, 0, 0, 0};
        vst[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    FA_LDS uint8_t* kb = smem + buf * 2 * TILE;
    FA_LDS uint8_t* vb = kb + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = i * 256 + tid;
      const int row = c / CH, ch = c % CH;
      lds_write_b128(kb, row * PITCH + ch * 16, kst[i]);
      lds_write_b128(vb, row * PITCH + ch * 16, vst[i]);
    }
  };

  if (n_kv > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  // Transposed-read coordinates of this lane inside its 16-lane group.
  const int grp = lane >> 4, gi = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (gi >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (gi & 3);

  for (int j = 0; j < n_kv; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_kv) load_tile(j + 1);
    const FA_LDS uint8_t* kb = smem + buf * 2 * TILE;
    const FA_LDS uint8_t* vb = kb + TILE;

    // S^T[key, query] for 64 keys x 32 queries.
    f32x16 s[BC / 32];
#pragma unroll
    for (int kb_i = 0; kb_i < BC / 32; ++kb_i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb_i][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kv = lds_read_b128(kb, (kb_i * 32 + col) * PITCH + (ks * 16 + 8 * half) * 2);
        s[kb_i] = mfma32(as_bf16x8(kv), qf[ks], s[kb_i]);
      }
    }

    const int key_base = j * BC;
    const bool need_mask = (key_base + BC > a.Tk) ||
                           (CAUSAL && key_base + BC - 1 > q0 + wave * 32 + shift);
    if (need_mask) {
      const int lim = CAUSAL ? min(a.Tk - 1, qrow + shift) : a.Tk - 1;
#pragma unroll
      for (int kb_i = 0; kb_i < BC / 32; ++kb_i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key_base + kb_i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > lim) s[kb_i][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb_i = 0; kb_i < BC / 32; ++kb_i)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb_i][r]);
    mx = pair_max32(mx);
    const float m_new = fmaxf(m, mx * a.c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // P = 2^(S*c - m), packed to bf16 in the accumulator order.
    uint32_t pw[BC / 32][8];
    float lsum = 0.f;
#pragma unroll
    for (int kb_i = 0; kb_i < BC / 32; ++kb_i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_fast(fmaf(s[kb_i][r], a.c, -m_use));
        const float p1 = exp2_fast(fmaf(s[kb_i][r + 1], a.c, -m_use));
        lsum += p0 + p1;
        pw[kb_i][r >> 1] = pack_bf16x2(p0, p1);
      }
    l += lsum;

    // O^T[d, query] += V^T[d, key] P^T[key, query], 16 keys per step.
#pragma unroll
    for (int kb_i = 0; kb_i < BC / 32; ++kb_i)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const bf16x8 pb = as_bf16x8(u32x4{pw[kb_i][4 * hs], pw[kb_i][4 * hs + 1],
                                          pw[kb_i][4 * hs + 2], pw[kb_i][4 * hs + 3]});
        const int row = kb_i * 32 + hs * 16 + tr_row;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int cb = (db * 32 + tr_col) * 2;
          const u32x2 lo = lds_read_tr(vb, row * PITCH + cb);
          const u32x2 hi = lds_read_tr(vb, (row + 8) * PITCH + cb);
          oacc[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, oacc[db]);
        }
      }

    if (j + 1 < n_kv) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum32(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const uint32_t n = (uint32_t)a.n_qtiles * (uint32_t)(a.B * a.Hq);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(FwdArgs a, int d, bool causal, hipStream_t stream) {
  a.n_qtiles = (a.Tq + 127) / 128;
  if (d == 64) return causal ? launch_fwd<64, true>(a, stream) : launch_fwd<64, false>(a, stream);
  return causal ? launch_fwd<128, true>(a, stream) : launch_fwd<128, false>(a, stream);
}

}  // namespace fa
