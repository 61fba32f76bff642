// fa_fwd_f32.hip -- tiled exact attention forward kept in fp32 end to end.
//
// The accuracy path for small problems (and for the pages' worked rows): the
// same online-softmax recurrence as the bf16 kernel (kgptalkie "Flash
// Attention: Why Memory Traffic, Not Compute, Is the Bottleneck", section
// "Carry the Actual Values Through Both Tiles": rescale the running sum and
// the running weighted sum by e^(m - m') together), but with scores,
// probabilities and accumulators all in fp32 and natural exponentials.
// One workgroup per 64 query rows, one row per lane; its NWK waves take the
// 32-key K/V tiles j = w, w + NWK, ... (staged in each wave's own LDS slot and
// read as broadcasts), each keeping a partial state (m, l, u) per row. At the
// end the partial states of the waves are folded with the same rescale rule
// (m* = max m_w, l = sum e^(m_w - m*) l_w, same for u), as the split-KV merge
// does.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

// Waves per 64-row tile, splitting its keys (at d = 128 the q and u rows
// already take most of a wave's 512 registers: one wave).
template <int D>
constexpr int f32_waves() { return D == 64 ? 4 : 1; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * f32_waves<D>()) void fwd_f32_kernel(FwdF32Args a, int n_qtiles) {
  constexpr int BR = 64, BC = 32, NWK = f32_waves<D>();
  // per wave: its K and V tiles; reused for the partial states at the end
  __shared__ __attribute__((aligned(16))) float kvs[NWK][2][BC][D];
  __shared__ float part_m[NWK][BR], part_l[NWK][BR];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qt = blockIdx.x % n_qtiles;
  const int bh = blockIdx.x / n_qtiles;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int row = qt * BR + lane;
  const float* Kp = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const float* Vp = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;
  float (*ks)[D] = kvs[wave][0];
  float (*vs)[D] = kvs[wave][1];

  const int shift = a.Tk - a.Tq;
  int kv_end = a.Tk;
  if (CAUSAL) kv_end = min(a.Tk, qt * BR + BR + shift);
  const int n_kv = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const int lim = CAUSAL ? min(a.Tk - 1, row + shift) : a.Tk - 1;

  float q[D], o[D];
  const bool live = row < a.Tq;
  const float* qsrc = a.q + ((size_t)bh * a.Tq + (live ? row : 0)) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = live ? qsrc[c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int j = wave; j < n_kv; j += NWK) {
    for (int e = lane * 4; e < BC * D; e += 64 * 4) {
      const int r = e / D, c = e % D;
      const int key = j * BC + r;
      float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < a.Tk) {
        kv = *(const float4*)(Kp + (size_t)key * D + c);
        vv = *(const float4*)(Vp + (size_t)key * D + c);
      }
      *(float4*)&ks[r][c] = kv;
      *(float4*)&vs[r][c] = vv;
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's tile is in LDS (the slot is private to the wave)
    __builtin_amdgcn_wave_barrier();

    float s[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], ks[jj][c], acc);
      s[jj] = (j * BC + jj <= lim) ? acc * a.scale : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      const float p = expf(s[jj] - m_use);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, vs[jj][c], o[c]);
    }
    __builtin_amdgcn_s_waitcnt(0);   // every lane has read the tile before it is replaced
    __builtin_amdgcn_wave_barrier();
  }

  if constexpr (NWK == 1) {
    if (live) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* dst = a.o + ((size_t)bh * a.Tq + row) * D;
#pragma unroll
      for (int c = 0; c < D; c += 4) *(float4*)(dst + c) = float4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
      if (a.lse != nullptr) a.lse[(size_t)bh * a.Tq + row] = l > 0.f ? m + logf(l) : -INFINITY;
    }
    return;
  }
  // Fold the waves' partial states: every wave publishes (m, l, u), then
  // wave w finishes the columns [w D/NWK, (w+1) D/NWK) of every row.
  __syncthreads();   // all tiles are consumed: the K/V slots become the u buffers
  float* u_all = &kvs[0][0][0][0];   // [NWK][D][BR] (lanes contiguous) fits in [NWK][2][BC][D]
  static_assert(BR * D <= 2 * BC * D, "partial sums fit in a wave's tile slots");
  part_m[wave][lane] = m;
  part_l[wave][lane] = l;
#pragma unroll
  for (int c = 0; c < D; ++c) u_all[(wave * D + c) * BR + lane] = o[c];
  __syncthreads();
  float mstar = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWK; ++w) mstar = fmaxf(mstar, part_m[w][lane]);
  const float m_ref = (mstar == -INFINITY) ? 0.f : mstar;
  float wgt[NWK], l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < NWK; ++w) {
    wgt[w] = expf(part_m[w][lane] - m_ref);
    l_tot = fmaf(wgt[w], part_l[w][lane], l_tot);
  }
  if (live) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* dst = a.o + ((size_t)bh * a.Tq + row) * D;
    constexpr int CW = D / NWK;
#pragma unroll
    for (int c = wave * CW; c < wave * CW + CW; c += 4) {
      float r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NWK; ++w) acc = fmaf(wgt[w], u_all[(w * D + c + e) * BR + lane], acc);
        r4[e] = acc * inv;
      }
      *(float4*)(dst + c) = float4{r4[0], r4[1], r4[2], r4[3]};
    }
    if (a.lse != nullptr && wave == 0) a.lse[(size_t)bh * a.Tq + row] = l_tot > 0.f ? m_ref + logf(l_tot) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdF32Args& a, hipStream_t stream) {
  const int n_qtiles = (a.Tq + 63) / 64;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(n_qtiles * a.B * a.Hq), dim3(64 * f32_waves<D>()), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(FwdF32Args a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
