// fa_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// Matrix-core conventions (measured on gfx950, 64-lane waves):
//   v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32]
//     lane l holds A[l%32][8*(l/32) + e] and B[8*(l/32) + e][l%32], e = 0..7,
//     and D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator register r = 0..15.
//   v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16]
//     lane l holds A[l%16][8*(l/16) + e], B[8*(l/16) + e][l%16], and
//     D[4*(l/16) + r][l%16] in register r = 0..3.
//   ds_read_b64_tr_b16: inside each 16-lane group, lane i names a row R_i of
//     four 16-bit values; lane j receives R_{4t + j/4}[j%4] as element t.
//   v_permlane32_swap (x, x): returns {x[l%32], x[32 + l%32]} in every lane l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))
// Lambdas of a kernel's main loop are always inlined (a call would move
// their captures to scratch memory and make uniform values per-lane).
#define FA_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (exact 0 for -inf).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit.
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// max / sum of x over lanes l and l^32 (the two lanes that share a column of
// a 32x32 accumulator), returned in both.
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposed 4 x 16-bit read (see header comment), from an LDS byte offset.
__device__ __forceinline__ u32x2 lds_read_tr(const FA_LDS uint8_t* base, uint32_t byte_off) {
  auto p = (FA_LDS s16x4*)(base + byte_off);
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read_b128(const FA_LDS uint8_t* base, uint32_t byte_off) {
  return *(const FA_LDS u32x4*)(base + byte_off);
}

__device__ __forceinline__ void lds_write_b128(FA_LDS uint8_t* base, uint32_t byte_off, u32x4 v) {
  *(FA_LDS u32x4*)(base + byte_off) = v;
}

__device__ __forceinline__ u32x4 global_load_b128(const void* p) {
  return *(const u32x4*)p;
}

// Raw buffer resource over [p, p + bytes): loads at byte offsets >= bytes
// return zeros without touching memory, which keeps tile loads branch free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset that is always out of range

// Direct global -> LDS loads (no registers): lane l of the wave writes its
// 16 (or 4) bytes to lds_wave_base + 16 l (or 4 l); the global offset is per lane.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t r, FA_LDS void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma_b32(__amdgpu_buffer_rsrc_t r, FA_LDS void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 4, off, 0, 0, 0);
}
// dma_b128 with the non-temporal cache-policy bit (nt, bit 1 of the gfx950
// buffer-load cache policy): for data read exactly once, such as the KV cache
// a decoding step streams. Measured on MI355X: split-KV decode 203 -> 186 us.
constexpr int kCpolNonTemporal = 2;
__device__ __forceinline__ void dma_b128_stream(__amdgpu_buffer_rsrc_t r, FA_LDS void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, off, 0, 0, kCpolNonTemporal);
}

// Wait until at most N vector-memory operations of this wave are in flight and
// its LDS operations are done, then meet the workgroup barrier. The asm has a
// memory clobber, so the compiler keeps LDS accesses on their side of it; the
// wait is what makes earlier direct-to-LDS loads visible to the other waves.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// f(std::integral_constant<int, I>{}) for I = B .. E - 1: loops over ring
// stages whose index must be a compile-time constant (LDS offsets then become
// instruction immediates instead of per-iteration address arithmetic).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Items 0 .. NI - 1, each an operand read followed by the MFMA that uses it,
// run with the reads one chunk of CK items ahead: the reads of chunk c + 1 are
// issued before the MFMAs of chunk c. Left to itself the compiler issues each
// LDS operand read right before its MFMA, which then waits out the whole LDS
// latency; the scheduling fences between chunks keep the reads where they are
// written (vector and scalar ALU work may still move across them). read(i)
// and mma(i) get i as a std::integral_constant and keep the operands of chunk
// c in buffer c & 1.
constexpr int kFenceLetAluCross = 0x2 | 0x4;   // sched_barrier mask: VALU, SALU
template <int NI, int CK, class Read, class Mma>
__device__ __forceinline__ void chunk_pipeline(Read&& read, Mma&& mma) {
  static_assert(NI % CK == 0, "whole chunks");
  static_for<0, CK>([&](auto j) { read(j); });
  static_for<0, NI / CK>([&](auto c_c) {
    constexpr int c = decltype(c_c)::value;
    if constexpr (c + 1 < NI / CK)
      static_for<0, CK>([&](auto j) { read(std::integral_constant<int, CK * (c + 1) + decltype(j)::value>{}); });
    __builtin_amdgcn_sched_barrier(kFenceLetAluCross);
    static_for<0, CK>([&](auto j) { mma(std::integral_constant<int, CK * c + decltype(j)::value>{}); });
    __builtin_amdgcn_sched_barrier(kFenceLetAluCross);
  });
}

// XOR swizzle of the 16-byte chunks of a row of D bf16 values, for LDS tiles
// stored without padding. Chunk c of row r lives at chunk c ^ swz<D>(r).
// With 64 four-byte banks it makes both access patterns conflict free:
//   * 128-bit reads of one chunk from 16 consecutive rows (MFMA A operand);
//   * 64-bit transposed reads of 4 consecutive rows x 64 bytes (two 16-lane
//     groups of ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ uint32_t swz(uint32_t r) {
  static_assert(D == 64 || D == 128, "head width");
  if constexpr (D == 128) {
    return ((r & 3u) << 2) | ((r >> 2) & 3u);
  } else {
    const uint32_t k = (r >> 1) & 7u;   // two 128-byte rows share a bank row
    return ((k & 1u) << 2) | ((k >> 1) & 3u);
  }
}

// Chunk swizzle for the 16x16x32 layouts (the 16-key dK/dV kernel's Q and dO
// tiles, the 16-query forward's K and V tiles): chunk c of row r lives at
// chunk c ^ swz16<D>(r). Measured on gfx950 with the LDS bank-conflict
// counter, ds_read_b128 serves a wave in four passes of 16 lanes, told apart
// by lane bit 5 and by the parity of lane bits 2, 3 and 4, and
// ds_read_b64_tr_b16 in two passes (lanes 0-31, 32-63). These tables give
// every lane of a pass its own banks in both read patterns of those kernels:
// the A-operand reads (16 rows at chunks 4 ks + q) and the transposed reads
// (8 consecutive rows at two neighbouring chunks). At d = 128 a row is one bank
// row; at d = 64 two rows share one, so the table ignores row bit 0. The
// 32x32 kernels' swizzles leave 2-way conflicts on both patterns here.
template <int D>
__device__ __forceinline__ uint32_t swz16(uint32_t r) {
  if constexpr (D == 128) {
    return (((r & 7u) << 1) | ((r >> 3) & 1u)) ^ (r & 8u);
  } else {
    return (((r >> 1) & 3u) << 1) ^ (((r >> 3) & 1u) * 5u);
  }
}

// Philox-4x32-10 counter-based generator (Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section 3.2 and
// Table 2): ten rounds, each multiplying words 0 and 2 of the counter by the
// two round multipliers, taking each 64-bit product's halves and mixing the
// high halves with words 1 and 3 and the key; the key is bumped by the two
// Weyl constants between rounds. The key is the same in every lane, so its
// schedule stays in scalar registers.
// a ^ b ^ c in one v_bitop3_b32 (truth table 0x96; gfx950 has no v_xor3).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// BITOP3 picks the XOR form: v_bitop3_b32 (fewer instructions) or two
// v_xor_b32 (fewer live registers in some kernels); the result is the same.
template <bool BITOP3 = true>
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = BITOP3 ? xor3((uint32_t)(p1 >> 32), c1, k0) : (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = BITOP3 ? xor3((uint32_t)(p0 >> 32), c3, k1) : (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

// Dropout bytes of one query row for the 32 keys k0 .. k0 + 31 (k0 a
// multiple of 32) in the 32x32 accumulator layout where lane l owns query
// column l % 32 and the keys 8 q + 4 (l / 32) + e, q, e = 0..3. The contract:
// the 16 keys 16 g .. 16 g + 15 of row i use the four words of one Philox
// call with counter (g, i, head, offset), key j taking byte j mod 16 (byte n
// = bits 8 (n mod 4) .. +7 of word n / 4). Lane l computes the call for
// group k0 / 16 + l / 32 and swaps the words its partner lane l ^ 32 needs:
// word q of the result holds the bytes of keys 8 q + 4 (l / 32) + 0..3.
template <bool BITOP3 = true>
__device__ __forceinline__ u32x4 dropout_bytes_32keys(uint32_t key0, uint32_t row, uint32_t head, uint32_t offset,
                                                      uint32_t seed_lo, uint32_t seed_hi, int half) {
  const u32x4 w = philox4x32_10<BITOP3>(key0 / 16 + (uint32_t)half, row, head, offset, seed_lo, seed_hi);
  // v_permlane32_swap(x, y): lanes 0-31 get {x[l], x[l + 32]}, lanes 32-63 {y[l - 32], y[l]}
  const auto s01 = __builtin_amdgcn_permlane32_swap(w[0], w[1], false, false);
  const auto s23 = __builtin_amdgcn_permlane32_swap(w[2], w[3], false, false);
  return u32x4{s01[0], s23[0], s01[1], s23[1]};
}

// Is the byte for accumulator register r (key 8 (r / 4) + 4 half + r % 4) below t?
__device__ __forceinline__ bool dropout_keep(const u32x4& bytes, int r, uint32_t t) {
  return ((bytes[r >> 2] >> (8 * (r & 3))) & 0xFFu) < t;
}

// Compensated (Kahan) summation: s accumulates, c carries the rounding error
// of each addition with its sign flipped, and s - c is the sum. A row of
// millions of keys adds one tile partial at a time to a running sum that can
// be far larger than each partial (after a dominant early key, for instance);
// plain fp32 addition would lose up to 2^-24 of the sum per tile.
__device__ __forceinline__ void kahan_add(float& s, float& c, float x) {
  const float y = x - c;
  const float t = s + y;
  c = (t - s) - y;
  s = t;
}

// Workgroup index remap so that consecutive logical tiles share one XCD.
// Hardware deals workgroups round-robin over the 8 XCDs (id % 8); logical
// tile t is placed on XCD t / ceil-share, which keeps the tiles of one head
// (and their K/V stream) inside one XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = n / kXcd, rem = n % kXcd;
  const uint32_t x = bid % kXcd, k = bid / kXcd;
  return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

}  // namespace fa
