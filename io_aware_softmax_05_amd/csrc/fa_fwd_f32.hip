// fa_fwd_f32.hip -- tiled exact attention forward kept in fp32 end to end.
//
// The accuracy path for small problems (and for the pages' worked rows): the
// same online-softmax recurrence as the bf16 kernel (kgptalkie "Flash
// Attention: Why Memory Traffic, Not Compute, Is the Bottleneck", section
// "Carry the Actual Values Through Both Tiles": rescale the running sum and
// the running weighted sum by e^(m - m') together), but with scores,
// probabilities and accumulators all in fp32 and natural exponentials.
// One wave per 64 query rows, one row per lane; 32-key K/V tiles are staged
// in LDS and read as broadcasts.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdF32Args a, int n_qtiles) {
  constexpr int BR = 64, BC = 32;
  __shared__ __attribute__((aligned(16))) float ks[BC][D];
  __shared__ __attribute__((aligned(16))) float vs[BC][D];

  const int lane = threadIdx.x;
  const int qt = blockIdx.x % n_qtiles;
  const int bh = blockIdx.x / n_qtiles;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int row = qt * BR + lane;
  const float* Kp = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const float* Vp = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;

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

  for (int j = 0; j < n_kv; ++j) {
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
    __syncthreads();

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
    __syncthreads();
  }

  if (live) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = a.o + ((size_t)bh * a.Tq + row) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) *(float4*)(dst + c) = float4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
    if (a.lse != nullptr) a.lse[(size_t)bh * a.Tq + row] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdF32Args& a, hipStream_t stream) {
  const int n_qtiles = (a.Tq + 63) / 64;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(n_qtiles * a.B * a.Hq), dim3(64), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(FwdF32Args a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
