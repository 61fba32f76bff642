// fa_decode.hip -- split-KV decoding: one query token per head against a
// long KV cache.
//
// aimlrounds "FlashAttention", note under the "FlashAttention 1, 2, 3" table:
// with a single query token the long KV cache is split across workgroups.
// zerotofrontier "Efficient attention: memory-bound", section "Every kernel
// is below the ridge": decoding does about one FLOP per cached byte, so the
// time is set by how fast the cache streams out of HBM.
//
// Kernel 1 (split): one wave per (split, KV-head, query-row group, batch).
//   The query heads that share a KV head are the rows of one 16-row MFMA
//   tile, so every cached key and value is read from HBM exactly once. The
//   wave walks its chunk of the cache in 32-key tiles (HBM -> registers ->
//   LDS, double buffered) and runs the online-softmax recurrence, then
//   stores its partial state (m, l, u).
// Kernel 2 (merge): per (batch, query head), folds the partial states with
//   the same rescale rule (m* = max m_s; l = sum 2^(m_s - m*) l_s; same for
//   u), then writes O = u / l and the log-sum-exp.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a, int n_rowgroups) {
  constexpr int BC = 32;                  // keys per tile
  constexpr int PITCH = (D + 16) * 2;
  constexpr int TILE = BC * PITCH;
  constexpr int CH = D / 8;
  constexpr int LOADS = BC * CH / 64;     // chunks per lane per tensor
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * 2 * TILE];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int lane = threadIdx.x;
  const int split = blockIdx.x;
  const int hk = blockIdx.y / n_rowgroups, rg = blockIdx.y % n_rowgroups;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int L = a.seq_lens[b];
  if (L < 1 || L > a.Tk_max) return;      // reported as NaN by the merge
  const int k_begin = split * a.chunk;
  if (k_begin >= L) return;               // the merge ignores splits past L
  const int k_end = min(L, k_begin + a.chunk);
  const int n_kv = (k_end - k_begin + BC - 1) / BC;

  const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk_max * D;
  const uint16_t* __restrict__ Kp = a.k + kvoff;
  const uint16_t* __restrict__ Vp = a.v + kvoff;

  // B operand of S^T = K q^T: lane holds query row (lane % 16), 8 dims.
  const int qcol = lane & 15, quad = lane >> 4;
  const int g = rg * 16 + qcol;           // head index inside the group
  const bool live = g < G;
  const int hq = hk * G + (live ? g : 0);
  bf16x8 qf[D / 32];
  {
    const uint16_t* src = a.q + ((size_t)b * a.Hq + hq) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = as_bf16x8(live ? global_load_b128(src + ks * 32) : u32x4{0, 0, 0, 0});
  }

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  u32x4 kst[LOADS], vst[LOADS];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = i * 64 + lane;
      const int row = c / CH, ch = c % CH;
      const int key = k_begin + j * BC + row;
      if (key < k_end) {
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
      const int c = i * 64 + lane;
      const int row = c / CH, ch = c % CH;
      lds_write_b128(kb, row * PITCH + ch * 16, kst[i]);
      lds_write_b128(vb, row * PITCH + ch * 16, vst[i]);
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int tr_row = 4 * quad + (qcol >> 2);
  const int tr_col = 4 * (qcol & 3);

  for (int j = 0; j < n_kv; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_kv) load_tile(j + 1);
    const FA_LDS uint8_t* kb = smem + buf * 2 * TILE;
    const FA_LDS uint8_t* vb = kb + TILE;

    // S^T[key, row] for two 16-key blocks.
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const u32x4 kv = lds_read_b128(kb, (blk * 16 + qcol) * PITCH + (ks * 32 + 8 * quad) * 2);
        s[blk] = mfma16(as_bf16x8(kv), qf[ks], s[blk]);
      }
    }
    const int key_base = k_begin + j * BC;
    if (key_base + BC > k_end) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key_base + blk * 16 + 4 * quad + r >= k_end) s[blk][r] = -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[blk][r]);
    {  // max over the four lanes holding this row: l, l^16, l^32, l^48
      auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      mx = pair_max32(mx);
    }
    const float m_new = fmaxf(m, mx * a.c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;

    uint32_t pw[4];
    float lsum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = exp2_fast(fmaf(s[blk][r], a.c, -m_use));
        const float p1 = exp2_fast(fmaf(s[blk][r + 1], a.c, -m_use));
        lsum += p0 + p1;
        pw[blk * 2 + (r >> 1)] = pack_bf16x2(p0, p1);
      }
    l += lsum;
    const bf16x8 pb = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});

    // O^T[d, row] += V^T[d, key] P^T[key, row]; k-slots 0..3 are keys
    // 4*quad + t of block 0, k-slots 4..7 the same keys of block 1.
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int cb = (db * 16 + tr_col) * 2;
      const u32x2 lo = lds_read_tr(vb, tr_row * PITCH + cb);
      const u32x2 hi = lds_read_tr(vb, (tr_row + 16) * PITCH + cb);
      oacc[db] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, oacc[db]);
    }

    if (j + 1 < n_kv) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Partial sum over the four lanes of the row.
  {
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    l = pair_sum32(l);
  }
  if (live) {
    const size_t pidx = ((size_t)b * a.Hq + hq) * a.n_splits + split;
    if (quad == 0) {
      a.part_m[pidx] = m;
      a.part_l[pidx] = l;
    }
    float* u = a.part_u + pidx * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) *(f32x4*)(u + db * 16 + 4 * quad) = oacc[db];
  }
}

// One wave per (batch, query head); each lane owns D/64 output columns.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq;
  const int L = a.seq_lens[b];
  uint16_t* dst = a.o + (size_t)bh * D + lane * PER;
  if (L < 1 || L > a.Tk_max) {
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = 0x7FC0;   // quiet NaN
    if (a.lse != nullptr && lane == 0) a.lse[bh] = __builtin_nanf("");
    return;
  }
  const int n_used = (L + a.chunk - 1) / a.chunk;
  const size_t base = (size_t)bh * a.n_splits;
  float mstar = -INFINITY;
  for (int s = 0; s < n_used; ++s) mstar = fmaxf(mstar, a.part_m[base + s]);
  float lsum = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s = 0; s < n_used; ++s) {
    const float w = exp2_fast(a.part_m[base + s] - mstar);
    lsum += w * a.part_l[base + s];
    const float* u = a.part_u + (base + s) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, u[e], acc[e]);
  }
  const float inv = 1.f / lsum;
  if (PER == 2) {
    *(uint32_t*)dst = pack_bf16x2(acc[0] * inv, acc[PER - 1] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const uint32_t w = pack_bf16x2(acc[e] * inv, 0.f);
      dst[e] = (uint16_t)(w & 0xffffu);
    }
  }
  if (a.lse != nullptr && lane == 0) a.lse[bh] = (mstar + log2_fast(lsum)) * kLn2;
}

template <int D>
static hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int n_rowgroups = (G + 15) / 16;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3(a.n_splits, a.Hkv * n_rowgroups, a.B), dim3(64), 0, stream,
                     a, n_rowgroups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbh = a.B * a.Hq;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((nbh + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(DecodeArgs a, int d, hipStream_t stream) {
  return d == 64 ? launch<64>(a, stream) : launch<128>(a, stream);
}

}  // namespace fa
