// fa_fwd_f32.hip -- tiled exact attention forward kept in fp32 end to end.
//
// The accuracy path for small problems (and for the pages' worked rows): the
// same online-softmax recurrence as the bf16 kernel (kgptalkie "Flash
// Attention: Why Memory Traffic, Not Compute, Is the Bottleneck", section
// "Carry the Actual Values Through Both Tiles": rescale the running sum and
// the running weighted sum by e^(m - m') together), but with scores,
// probabilities and accumulators all in fp32 and natural exponentials.
//
// Layout: one wave per query row, four rows of one head per workgroup, so
// even a single head of 256 rows spreads over 64 workgroups. The keys stream
// past the rows in tiles of 64 KPL: the workgroup copies a tile's K and V
// rows into LDS once (coalesced 16-byte loads, the next tile's loads issued
// before the current tile is scored), lane l scores keys t0 + 64 r + l
// (r < KPL) with the whole query row in its registers, the tile's maximum
// and sum are wave reductions, and for u += p V each lane owns D / 64 output
// columns, taking every key's probability from the lane that scored it (a
// readlane) and the value from the tile in LDS. m and l are the same in every lane of the wave; u is
// spread over the lanes. l is a compensated sum, so long rows keep fp32
// accuracy.
#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kF32RowsPerGroup = 4;   // waves (query rows of one head) per workgroup
// keys per lane per tile: 2 at d = 64 (128-key tiles), 1 at d = 128, whose
// 128-key tiles would need 132 KB of LDS and hold one workgroup per CU
template <int D>
constexpr int kF32KeysPerLane = D == 64 ? 2 : 1;

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
  constexpr int NW = kF32RowsPerGroup, KPL = kF32KeysPerLane<D>, TK = 64 * KPL;
  constexpr int CPL = D / 64;                    // output columns per lane
  constexpr int CH = D / 4;                      // 16-byte chunks per row
  constexpr int KP = D + 4;                      // K row pitch in LDS (floats): the 16 lanes of a
                                                 // 128-bit row read land on distinct banks
  constexpr int LOADS = TK * CH / (64 * NW);     // chunks of K (and of V) per thread per tile
  static_assert(LOADS * 64 * NW == TK * CH, "a tile must split evenly over the workgroup");
  __shared__ __attribute__((aligned(16))) float ks[TK * KP];
  __shared__ __attribute__((aligned(16))) float vs[TK * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_rt = (a.Tq + NW - 1) / NW;         // row tiles per head
  const int bh = (int)blockIdx.x / n_rt;         // flattened (b, h)
  const int i0 = ((int)blockIdx.x - bh * n_rt) * NW;
  const int i = i0 + wave;                       // this wave's row
  const bool live = i < a.Tq;                    // rows past Tq still load tiles and meet the barriers
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const float* Kp = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const float* Vp = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;

  // key j is visible to row i iff j < kv_end(i) (the causal rule aligns the
  // diagonal to the bottom-right corner); kv_end <= 0: no visible key
  const int shift = a.Tk - a.Tq;
  const int kv_end = CAUSAL ? min(a.Tk, i + shift + 1) : a.Tk;
  const int last = min(a.Tq, i0 + NW) - 1;      // the workgroup's last row
  const int wg_end = CAUSAL ? min(a.Tk, last + shift + 1) : a.Tk;   // keys some row sees

  float q[D];
  if (live) {
    const float4* qs = (const float4*)(a.q + ((size_t)bh * a.Tq + i) * D);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
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
  float m = -INFINITY, l = 0.f, lc = 0.f;   // l - lc is the running sum

  // this thread's chunks of a tile: (row, chunk) = (c / CH, c % CH), c = n * 64 NW + tid
  float4 kst[LOADS], vst[LOADS];
  auto load = [&](int t0) {
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int c = n * 64 * NW + tid, key = t0 + c / CH;
      const bool in = key < wg_end;
      kst[n] = in ? ((const float4*)(Kp + (size_t)key * D))[c % CH] : float4{0.f, 0.f, 0.f, 0.f};
      vst[n] = in ? ((const float4*)(Vp + (size_t)key * D))[c % CH] : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (wg_end > 0) load(0);
  for (int t0 = 0; t0 < wg_end; t0 += TK) {
    if (t0 > 0) __syncthreads();   // every wave is done with the previous tile
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int c = n * 64 * NW + tid, row = c / CH, ch = c % CH;
      *(float4*)&ks[row * KP + 4 * ch] = kst[n];
      *(float4*)&vs[row * D + 4 * ch] = vst[n];
    }
    __syncthreads();
    if (t0 + TK < wg_end) load(t0 + TK);   // in flight while this tile is used
    if (!live || t0 >= kv_end) continue;    // wave-uniform: no key of the tile is visible to the row

    // S for this lane's keys of the tile (masked keys: -inf)
    float sk[KPL];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int key = t0 + 64 * r + lane;
      float sv = -INFINITY;
      if (key < kv_end) {
        const float4* kr = (const float4*)&ks[(64 * r + lane) * KP];
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const float4 kv = kr[c];
          acc = fmaf(q[4 * c], kv.x, acc);
          acc = fmaf(q[4 * c + 1], kv.y, acc);
          acc = fmaf(q[4 * c + 2], kv.z, acc);
          acc = fmaf(q[4 * c + 3], kv.w, acc);
        }
        sv = acc * a.scale;
      }
      sk[r] = sv;
      mt = fmaxf(mt, sv);
    }
    // m' = max(m, tile max); l and u are rescaled together by e^(m - m')
    const float m_new = fmaxf(m, wave_max(mt));   // finite: key t0 is visible
    const float alpha = expf(m - m_new);         // 0 while m is still -inf
    l *= alpha;
    lc *= alpha;
#pragma unroll
    for (int e = 0; e < CPL; ++e) u[e] *= alpha;
    m = m_new;
    float pk[KPL], psum = 0.f;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      pk[r] = expf(sk[r] - m);   // exactly 0 for a masked key
      psum += pk[r];
    }
    kahan_add(l, lc, wave_sum(psum));
    // u += sum_j p_j V_j over the tile's visible keys, 64 keys per block
    const float* vr = vs + CPL * lane;
    auto add_key = [&](int r, int j) {
      const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pk[r]), j));
      const int row = 64 * r + j;
      if constexpr (CPL == 1) {
        u[0] = fmaf(pj, vr[row * D], u[0]);
      } else {
        const float2 v2 = *(const float2*)(vr + row * D);
        u[0] = fmaf(pj, v2.x, u[0]);
        u[1] = fmaf(pj, v2.y, u[1]);
      }
    };
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int n = kv_end - t0 - 64 * r;
      if (n <= 0) break;
      if (n >= 64) {
#pragma unroll
        for (int j = 0; j < 64; ++j) add_key(r, j);
      } else {   // the row's last, partial block: only its visible keys
        for (int j = 0; j < n; ++j) add_key(r, j);
      }
    }
  }

  if (!live) return;
  const float l_tot = l - lc;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* dst = a.o + ((size_t)bh * a.Tq + i) * D + CPL * lane;
  if constexpr (CPL == 1) {
    dst[0] = u[0] * inv;
  } else {
    *(float2*)dst = float2{u[0] * inv, u[1] * inv};
  }
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)bh * a.Tq + i] = l_tot > 0.f ? m + logf(l_tot) : -INFINITY;
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdF32Args& a, hipStream_t stream) {
  const long long groups_ll = (long long)a.B * a.Hq * ((a.Tq + kF32RowsPerGroup - 1) / kF32RowsPerGroup);
  const unsigned groups = (unsigned)groups_ll;   // the entry point keeps it below 2^31
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(groups), dim3(64 * kF32RowsPerGroup), 0, stream, a);
  return hipGetLastError();
}

int fwd_f32_rows_per_workgroup() { return kF32RowsPerGroup; }

hipError_t launch_fwd_f32(FwdF32Args a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
