// fa_fwd_f32.hip -- tiled exact attention forward kept in fp32 end to end.
//
// The accuracy path for small problems (and for the pages' worked rows): the
// same online-softmax recurrence as the bf16 kernel (kgptalkie "Flash
// Attention: Why Memory Traffic, Not Compute, Is the Bottleneck", section
// "Carry the Actual Values Through Both Tiles": rescale the running sum and
// the running weighted sum by e^(m - m') together), but with scores,
// probabilities and accumulators all in fp32 and natural exponentials.
//
// Layout: one wave per query row, four rows per workgroup, so even a single
// head of 256 rows spreads over 256 waves. The keys stream past the row in
// tiles of 64 * KPL: lane l scores keys t0 + 64 r + l (r < KPL) with the
// whole query row in its registers, the tile's maximum and sum are wave
// reductions, and for u += p V each lane owns D / 64 output columns, taking
// every key's probability from the lane that scored it (a readlane) and the
// key's value row with one coalesced load. m and l are the same in every lane
// of the wave; u is spread over the lanes.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kF32RowsPerGroup = 4;   // waves (query rows) per workgroup
constexpr int kF32KeysPerLane = 4;    // keys per lane per tile: tiles of 256 keys

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kF32RowsPerGroup) void fwd_f32_kernel(FwdF32Args a) {
  constexpr int KPL = kF32KeysPerLane, TILE = 64 * KPL, CPL = D / 64;   // output columns per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long rowid = (long long)blockIdx.x * kF32RowsPerGroup + wave;   // flattened (b, h, i)
  if (rowid >= (long long)a.B * a.Hq * a.Tq) return;   // the whole wave leaves
  const int i = (int)(rowid % a.Tq);
  const int bh = (int)(rowid / a.Tq);
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const float* Kp = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const float* Vp = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;

  // key j is visible iff j <= lim (the causal rule aligns the diagonal to the
  // bottom-right corner); the row sees keys [0, kv_end)
  const int lim = CAUSAL ? min(a.Tk - 1, i + (a.Tk - a.Tq)) : a.Tk - 1;
  const int kv_end = lim + 1;   // <= 0: no visible key

  float q[D];
  {
    const float4* qs = (const float4*)(a.q + (size_t)rowid * D);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 v = qs[c];
      q[4 * c] = v.x;
      q[4 * c + 1] = v.y;
      q[4 * c + 2] = v.z;
      q[4 * c + 3] = v.w;
    }
  }
  float u[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) u[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int t0 = 0; t0 < kv_end; t0 += TILE) {
    // S for this lane's keys of the tile (masked keys: -inf)
    float s[KPL];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int key = t0 + 64 * r + lane;
      float acc = -INFINITY;
      if (key < kv_end) {
        const float4* kr = (const float4*)(Kp + (size_t)key * D);
        acc = 0.f;
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
          const float4 kv = kr[c];
          acc = fmaf(q[4 * c], kv.x, acc);
          acc = fmaf(q[4 * c + 1], kv.y, acc);
          acc = fmaf(q[4 * c + 2], kv.z, acc);
          acc = fmaf(q[4 * c + 3], kv.w, acc);
        }
        acc *= a.scale;
      }
      s[r] = acc;
      mt = fmaxf(mt, acc);
    }
    // m' = max(m, tile max); l and u are rescaled together by e^(m - m')
    const float m_new = fmaxf(m, wave_max(mt));   // finite: the tile holds a visible key
    const float alpha = expf(m - m_new);          // 0 while m is still -inf
    l *= alpha;
#pragma unroll
    for (int e = 0; e < CPL; ++e) u[e] *= alpha;
    m = m_new;
    float p[KPL], psum = 0.f;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      p[r] = expf(s[r] - m);   // exactly 0 for a masked key
      psum += p[r];
    }
    l += wave_sum(psum);
    // u += sum_j p_j V_j over the tile's visible keys, 64 keys per block
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int k0 = t0 + 64 * r;
      if (k0 >= kv_end) break;
      const float* vr = Vp + (size_t)k0 * D + CPL * lane;
      if (k0 + 64 <= kv_end) {
#pragma unroll
        for (int src = 0; src < 64; ++src) {
          const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[r]), src));
          if constexpr (CPL == 1) {
            u[0] = fmaf(pj, vr[(size_t)src * D], u[0]);
          } else {
            const float2 v2 = *(const float2*)(vr + (size_t)src * D);
            u[0] = fmaf(pj, v2.x, u[0]);
            u[1] = fmaf(pj, v2.y, u[1]);
          }
        }
      } else {   // the last, partial block: only its visible keys are read
        for (int src = 0; src < kv_end - k0; ++src) {
          const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[r]), src));
          if constexpr (CPL == 1) {
            u[0] = fmaf(pj, vr[(size_t)src * D], u[0]);
          } else {
            const float2 v2 = *(const float2*)(vr + (size_t)src * D);
            u[0] = fmaf(pj, v2.x, u[0]);
            u[1] = fmaf(pj, v2.y, u[1]);
          }
        }
      }
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* dst = a.o + (size_t)rowid * D + CPL * lane;
  if constexpr (CPL == 1) {
    dst[0] = u[0] * inv;
  } else {
    *(float2*)dst = float2{u[0] * inv, u[1] * inv};
  }
  if (a.lse != nullptr && lane == 0) a.lse[rowid] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdF32Args& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.Tq;
  const unsigned groups = (unsigned)((rows + kF32RowsPerGroup - 1) / kF32RowsPerGroup);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(groups), dim3(64 * kF32RowsPerGroup), 0, stream, a);
  return hipGetLastError();
}

int fwd_f32_rows_per_workgroup() { return kF32RowsPerGroup; }

hipError_t launch_fwd_f32(FwdF32Args a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
