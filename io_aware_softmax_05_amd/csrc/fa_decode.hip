// fa_decode.hip -- split-KV decoding: one query token per head against a
// long KV cache.
//
// aimlrounds "FlashAttention", note under the "FlashAttention 1, 2, 3" table:
// with a single query token the long KV cache is split across workgroups.
// zerotofrontier "Efficient attention: memory-bound", section "Every kernel
// is below the ridge": decoding does about one FLOP per cached byte, so its
// run time follows the rate at which HBM delivers the cache.
//
// Kernel 1 (split). Work items are (batch, KV head, query-row group, chunk)
// for the chunks that hold cached keys; the item list is dense (chunks past a
// sequence's length are not items) and is dealt round-robin to a grid of a
// few single-wave workgroups per compute unit. Each wave streams the tiles of
// its items back to back through a three-stage ring of direct-to-LDS loads,
// so two 32-key K/V tiles are always in flight, also across item
// boundaries. The cache is read exactly once, so its loads carry the
// non-temporal hint. The query heads that share a KV head are the rows of one
// 16-row MFMA tile, so every cached key and value is read from HBM once. Per
// item the wave runs the online-softmax recurrence and stores the partial
// state (m, l, u).
// Kernel 2 (merge): per (batch, query head), folds the partial states with
//   the same rescale rule (m* = max m_s; l = sum 2^(m_s - m*) l_s; same for
//   u), then writes O = u / l and the log-sum-exp.
#include <algorithm>
#include <atomic>

#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

template <int D, int NSTAGE_ = 3>
struct DecCfg {
  static constexpr int BC = 32;                  // keys per tile
  static constexpr int ROWB = 2 * D;             // LDS bytes per row (swizzled, unpadded)
  static constexpr int CH = D / 8;
  static constexpr int TILE = BC * ROWB;         // one K (or V) tile
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr int DMA = BC * CH / 64;       // wave loads per tensor per tile
  static constexpr int VM_PER_TILE = 2 * DMA;
  static constexpr int MAX_QDMA = 16 * CH / 64;  // wave loads of a full 16-row query group
  static_assert((NSTAGE - 1) * (VM_PER_TILE + MAX_QDMA) < 64, "vmcnt range");
  // LDS per stage: K tile, V tile, then the query rows of the item (G rows,
  // at most 16, in whole 1 KiB wave loads); the size is set at launch.
  __host__ __device__ static constexpr int stage_bytes(int rows) { return 2 * TILE + (rows * ROWB + 1023) / 1024 * 1024; }
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Position in a workgroup's stream of tiles.
struct DecCursor {
  int item;     // index in the dense item list
  int b;        // batch entry of `item` (items of earlier entries: `base`)
  int base;
  int hk, rg, c;   // c: split index (chunk index minus the first chunk in use)
  int k0, kend; // keys [k0, kend) of the item
  int klo;      // first visible key of the sequence (window start)
  int nt, t;    // tiles of the item, current tile; nt = 0 once the stream is over
};

}  // namespace

template <int D, int NSTAGE>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a, int n_rowgroups) {
  using C = DecCfg<D, NSTAGE>;
  constexpr int BC = C::BC, ROWB = C::ROWB, CH = C::CH, TILE = C::TILE;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_dyn[];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_dyn;

  const int lane = threadIdx.x;
  const int qcol = lane & 15, quad = lane >> 4;
  const int G = a.Hq / a.Hkv;
  const int groups = a.Hkv * n_rowgroups;        // items per chunk of one batch entry
  const int q_rows = min(G, 16);                 // query rows stored per stage
  const int STAGE = C::stage_bytes(q_rows);

  // chunks of batch entry b in use (0 for a length outside [1, Tk_max]: the
  // merge writes NaN); with a window only those meeting the last W keys
  auto first_key = [&](int L) -> int { return a.window > 0 ? max(0, L - a.window) : 0; };
  auto n_chunks = [&](int b) -> int {
    const int L = a.seq_lens[b];
    return (L < 1 || L > a.Tk_max) ? 0 : (L + a.chunk - 1) / a.chunk - first_key(L) / a.chunk;
  };
  auto locate = [&](DecCursor& u) {
    while (u.b < a.B) {
      const int cnt = n_chunks(u.b) * groups;
      if (u.item < u.base + cnt) break;
      u.base += cnt;
      ++u.b;
    }
    if (u.b >= a.B) {
      u.nt = 0;
      return;
    }
    const int nb = n_chunks(u.b);
    const int r = u.item - u.base;
    const int grp = r / nb;
    u.c = r - grp * nb;
    u.hk = grp / n_rowgroups;
    u.rg = grp - u.hk * n_rowgroups;
    const int L = a.seq_lens[u.b];
    u.klo = first_key(L);
    const int chunk_idx = u.klo / a.chunk + u.c;
    u.k0 = max(chunk_idx * a.chunk, u.klo / BC * BC);   // whole tiles from the window start
    u.kend = min(L, chunk_idx * a.chunk + a.chunk);
    u.nt = (u.kend - u.k0 + BC - 1) / BC;
    u.t = 0;
  };
  auto advance = [&](DecCursor& u) {
    if (u.nt == 0) return;
    if (++u.t >= u.nt) {
      u.item += gridDim.x;
      locate(u);
    }
  };

  // Loads: physical chunk p of a tile holds logical chunk p ^ swz16(row) of its row
  // (the chunk swizzle of the 16x16x32 operand reads, conflict free for both below).
  uint32_t dma_off[C::DMA];
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int p = 64 * i + lane;
    const int r = p / CH, pc = p % CH;
    dma_off[i] = (uint32_t)(r * D + (pc ^ swz16<D>(r)) * 8) * 2;
  }
  DecCursor ld{(int)blockIdx.x, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  locate(ld);
  DecCursor cp = ld;
  auto issue = [&](int stage) {
    FA_LDS uint8_t* st = smem + stage * STAGE;
    const bool live = ld.nt > 0;
    // the buffer ranges end at the item's last key, so rows past it (and
    // every row once the stream is over) read as zeros with no per-lane test
    const int kt0 = ld.k0 + ld.t * BC;
    const size_t tile0 = live ? ((size_t)(ld.b * a.Hkv + ld.hk) * a.Tk_max + kt0) * D : 0;
    const uint32_t bytes = live ? (uint32_t)(ld.kend - kt0) * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + tile0, bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + tile0, bytes);
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {   // each cached row is read once: non-temporal loads
      dma_b128_stream(krs, st + i * 1024, dma_off[i]);
      dma_b128_stream(vrs, st + TILE + i * 1024, dma_off[i]);
    }
    if (live && ld.t == 0) {
      // first tile of an item: its query rows come along (swizzled like the
      // tiles); a wait that counts only tile loads stays safe, it just waits
      // a little longer
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + ((size_t)ld.b * a.Hq + ld.hk * G) * D, (uint32_t)G * D * 2);
      // q_rows rows of CH chunks, 64 chunks (1 KiB) per wave load; lanes past
      // the last row read out of range and write zeros inside the slot
      for (int i = 0; i * 64 < q_rows * CH; ++i) {
        const int p = 64 * i + lane;
        const int r = ld.rg * 16 + p / CH;
        const bool ok = p < q_rows * CH && p / CH + ld.rg * 16 < G;
        const uint32_t chunk = (uint32_t)(p % CH) ^ swz16<D>((uint32_t)(p / CH));
        dma_b128(qrs, st + 2 * TILE + i * 1024, ok ? (uint32_t)(r * D + chunk * 8) * 2 : kOutOfRange);
      }
    }
    advance(ld);
  };

  // LDS read offsets. K rows (A operand of S^T = K q^T): row 16 blk + qcol,
  // chunk 4 ks + quad. V^T (A operand of O^T = V^T P^T): transposed reads of
  // rows tr_row (+16), chunk 2 db + ((qcol >> 1) & 1).
  const uint32_t fk = swz16<D>(qcol);
  const uint32_t q_rd = qcol * ROWB + 16 * (quad ^ fk);   // query row qcol, chunk 4 ks + quad (^ 64 ks)
  const uint32_t k_rd = qcol * ROWB + 64 * (fk >> 2) + 16 * (quad ^ (fk & 3));            // ^ 64 ks
  const int tr_row = 4 * quad + (qcol >> 2);
  const uint32_t fv = swz16<D>(tr_row);
  const uint32_t v_rd = tr_row * ROWB + 32 * (fv >> 1) + 16 * (((qcol >> 1) & 1) ^ (fv & 1)) + 8 * (qcol & 1);  // ^ 32 db

  bf16x8 qf[D / 32];
  f32x4 oacc[D / 16];
  float m = -INFINITY, l = 0.f;
  bool live_row = false;
  int hq = 0;

  for (int st = 0; st < NSTAGE - 1; ++st) issue(st);
  int cs = 0, ls = NSTAGE - 1;
  while (cp.nt > 0) {
    issue(ls);
    wait_vm<(NSTAGE - 1) * C::VM_PER_TILE>();   // the tile in stage cs has landed
    if (cp.t == 0) {
      // new item: query rows of this KV head's row group, fresh state
      const int g = cp.rg * 16 + qcol;
      live_row = g < G;
      hq = cp.hk * G + (live_row ? g : 0);
      const FA_LDS uint8_t* qs = smem + cs * STAGE + 2 * TILE;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qf[ks] = as_bf16x8(live_row ? lds_read_b128(qs, q_rd ^ (64 * ks)) : u32x4{0, 0, 0, 0});
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      m = -INFINITY;
      l = 0.f;
    }
    const FA_LDS uint8_t* kb = smem + cs * STAGE;
    const FA_LDS uint8_t* vb = kb + TILE;

    // S^T[key, row] for two 16-key blocks.
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const u32x4 kv = lds_read_b128(kb, blk * 16 * ROWB + (k_rd ^ (64 * ks)));
        s[blk] = mfma16(as_bf16x8(kv), qf[ks], ks == 0 ? f32x4{} : s[blk]);
      }
    }
    const int key_base = cp.k0 + cp.t * BC;
    if (key_base + BC > cp.kend || key_base < cp.klo) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key_base + blk * 16 + 4 * quad + r;
          if (key >= cp.kend || key < cp.klo) s[blk][r] = -INFINITY;
        }
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
    // the reference maximum only moves when some row grows by more than 2^8
    // (l and u keep a common stale reference otherwise; probabilities < 256)
    const float m_new = fmaxf(m, mx * a.c);
    if (__builtin_amdgcn_ballot_w64(m_new > m + 8.f)) {
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_ref);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
      m = m_new;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;

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
      const u32x2 lo = lds_read_tr(vb, v_rd ^ (32 * db));
      const u32x2 hi = lds_read_tr(vb, 16 * ROWB + (v_rd ^ (32 * db)));
      oacc[db] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, oacc[db]);
    }

    if (cp.t == cp.nt - 1) {
      // end of the item: its partial state
      float lt;
      {
        auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
        lt = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
        lt = pair_sum32(lt);
      }
      if (live_row) {
        const size_t pidx = ((size_t)cp.b * a.Hq + hq) * a.n_splits + cp.c;
        if (quad == 0) {
          a.part_m[pidx] = m;
          a.part_l[pidx] = lt;
        }
        float* u = a.part_u + pidx * D;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *(f32x4*)(u + db * 16 + 4 * quad) = oacc[db];
      }
    }
    advance(cp);
    cs = cs == NSTAGE - 1 ? 0 : cs + 1;
    ls = ls == NSTAGE - 1 ? 0 : ls + 1;
  }
  wait_vm<0>();   // no load of this wave is left writing LDS when it exits
}

// One workgroup (4 waves) per (batch, query head). Wave w folds the splits
// s = w, w + 4, ... (the split's m and l are uniform, so they come through
// scalar loads); each lane owns D/64 output columns. The four partial sums,
// all relative to the same maximum, are then added through LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  static_assert(PER == 1 || PER == 2, "head width");
  __shared__ float red_m[4];
  // one row per wave: its D partial sums (written and read as PER-float
  // vectors, so the lanes' accesses fall on distinct banks) and its l
  __shared__ __attribute__((aligned(16))) float red_u[4][D + 4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int L = a.seq_lens[b];
  uint16_t* dst = a.o + (size_t)bh * D + lane * PER;
  if (L < 1 || L > a.Tk_max) {
    if (wave == 0) {
#pragma unroll
      for (int e = 0; e < PER; ++e) dst[e] = 0x7FC0;   // quiet NaN
      if (a.lse != nullptr && lane == 0) a.lse[bh] = __builtin_nanf("");
    }
    return;
  }
  const int n_used = (L + a.chunk - 1) / a.chunk - (a.window > 0 ? max(0, L - a.window) : 0) / a.chunk;
  const size_t base = (size_t)bh * a.n_splits;

  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < n_used; s += 256) mloc = fmaxf(mloc, a.part_m[base + s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if (lane == 0) red_m[wave] = mloc;
  __syncthreads();
  const float mstar = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float lsum = 0.f, lcomp = 0.f, acc[PER];   // lsum - lcomp: compensated sum over thousands of splits
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int s = wave; s < n_used; s += 4) {
    const float w = exp2_fast(a.part_m[base + s] - mstar);
    kahan_add(lsum, lcomp, w * a.part_l[base + s]);
    const float* u = a.part_u + (base + s) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, u[e], acc[e]);
  }
  if constexpr (PER == 2) {
    *(float2*)&red_u[wave][lane * 2] = float2{acc[0], acc[PER - 1]};
  } else {
    red_u[wave][lane] = acc[0];
  }
  if (lane == 0) red_u[wave][D] = lsum - lcomp;
  __syncthreads();
  if (wave != 0) return;
  const float l_tot = red_u[0][D] + red_u[1][D] + red_u[2][D] + red_u[3][D];
  const float inv = 1.f / l_tot;
  float o[PER];
  if constexpr (PER == 2) {
    float2 t = *(const float2*)&red_u[0][lane * 2];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float2 x = *(const float2*)&red_u[w][lane * 2];
      t.x += x.x;
      t.y += x.y;
    }
    o[0] = t.x * inv;
    o[PER - 1] = t.y * inv;
  } else {
    o[0] = (red_u[0][lane] + red_u[1][lane] + red_u[2][lane] + red_u[3][lane]) * inv;
  }
  if (PER == 2) {
    *(uint32_t*)dst = pack_bf16x2(o[0], o[PER - 1]);
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = (uint16_t)(pack_bf16x2(o[e], 0.f) & 0xffffu);
  }
  if (a.lse != nullptr && lane == 0) a.lse[bh] = (mstar + log2_fast(l_tot)) * kLn2;
}

// Devices whose per-device facts are cached (compute-unit count, address of
// the fixed scratch); a device index at or beyond it is looked up every call
// (compute units) or refused (scratch).
constexpr int kMaxDevices = 64;

// Compute units of the current device, looked up once per device: the
// persistent split grid is sized from it.
static hipError_t current_cu_count(int* n_cu) {
  static std::atomic<int> cached[kMaxDevices];   // 0: not looked up yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *n_cu = c;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && cacheable && *n_cu > 0) cached[dev].store(*n_cu, std::memory_order_relaxed);
  return e;
}

// Split plus merge with an NSTAGE ring and WG_PER_CU resident workgroups per
// compute unit (the grid never exceeds the item count's upper bound).
template <int D, int NSTAGE, int WG_PER_CU>
hipError_t launch_decode_cfg(const DecodeArgs& a, hipStream_t stream) {
  using C = DecCfg<D, NSTAGE>;
  const int G = a.Hq / a.Hkv;
  const int n_rowgroups = (G + 15) / 16;
  int n_cu = 0;
  hipError_t e = current_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const long long slots = (long long)a.B * a.Hkv * n_rowgroups * a.n_splits;
  const long long grid = std::min<long long>(slots, (long long)std::max(1, n_cu) * WG_PER_CU);
  const int q_rows = std::min(G, 16);
  const size_t lds = (size_t)NSTAGE * C::stage_bytes(q_rows);
  hipLaunchKernelGGL((decode_split_kernel<D, NSTAGE>), dim3((unsigned)grid), dim3(64), lds, stream, a, n_rowgroups);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(a.B * a.Hq)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(DecodeArgs a, int d, hipStream_t stream) {
  return d == 64 ? launch_decode_cfg<64, 3, 4>(a, stream) : launch_decode_cfg<128, 3, 3>(a, stream);
}

// ------------------------------------------------------------ fixed scratch
//
// The partial states of fa_decode_splitkv_noalloc live in this file-scope
// device array, so that entry point allocates nothing. Every GPU the library
// runs on holds its own copy, at its own address, until the process ends. In
// host code the array's name is only a stand-in: its device address is
// looked up with hipGetSymbolAddress once per device, with that device
// current, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];   // null: not looked up yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fa
