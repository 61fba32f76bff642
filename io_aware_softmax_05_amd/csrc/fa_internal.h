// fa_internal.h -- launch interfaces between the C ABI layer and the kernels.
// Every launcher assumes its arguments were validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Dropout of the attention probabilities: P_ij is kept iff its Philox byte is
// below t (keep probability t / 256) and kept entries are scaled by 256 / t.
struct DropArgs {
  uint32_t t;               // keep threshold in [1, 256]; 0: no dropout
  uint32_t seed_lo, seed_hi;
  uint32_t offset;
  float inv_keep;           // 256 / t
};

struct FwdArgs {
  const uint16_t* q;  // [B,Hq,Tq,d] bf16
  const uint16_t* k;  // [B,Hkv,Tk,d] bf16
  const uint16_t* v;  // [B,Hkv,Tk,d] bf16
  uint16_t* o;        // [B,Hq,Tq,d] bf16
  float* lse;         // [B,Hq,Tq] or null
  int B, Hq, Hkv, Tq, Tk;
  float c;            // scale * log2(e)
  int n_qtiles;       // filled in by the launcher
  int window;         // causal band of this many keys (0: plain mask)
  DropArgs drop;
};

struct Fp8Args {
  const uint8_t* q;         // [B,Hq,Tq,d] e4m3
  const uint8_t* k;         // [B,Hkv,Tk,d] e4m3
  const uint8_t* vt;        // [B,Hkv,d,Tk] e4m3 (V transposed)
  const float* q_scale;     // [B,Hq]  value = byte * scale
  const float* k_scale;     // [B,Hkv]
  const float* v_scale;     // [B,Hkv]
  uint16_t* o;              // [B,Hq,Tq,d] bf16
  float* lse;               // [B,Hq,Tq] or null
  int B, Hq, Hkv, Tq, Tk;
  float c;                  // scale * log2(e)
  int n_qtiles;             // filled in by the launcher
};

struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Tq, Tk;
  float scale;
};

struct DecodeArgs {
  const uint16_t* q;        // [B,Hq,d]
  const uint16_t* k;        // [B,Hkv,Tk_max,d]
  const uint16_t* v;        // [B,Hkv,Tk_max,d]
  const int* seq_lens;      // [B]
  uint16_t* o;              // [B,Hq,d]
  float* lse;               // [B,Hq] or null
  float* part_m;            // [B,Hq,S]   running max, log2 units
  float* part_l;            // [B,Hq,S]   running sum
  float* part_u;            // [B,Hq,S,d] weighted sum
  int B, Hq, Hkv, Tk_max;
  int chunk;                // keys per split (multiple of 64)
  int n_splits;             // ceil(Tk_max / chunk)
  float c;                  // scale * log2(e)
  int window;               // only the last `window` keys are seen (0: all)
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;         // natural log
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* stats;             // workspace: [B,Hq,Tq] LSE * log2 e, then [B,Hq,Tq] -rowsum(dO * O)
  int B, Hq, Hkv, Tq, Tk;
  float scale;
  float c;                  // scale * log2(e)
  int window;               // causal band of this many keys (0: plain mask)
  DropArgs drop;
};

hipError_t launch_fwd_bf16(FwdArgs a, int d, bool causal, hipStream_t stream);
int fwd_rows_per_workgroup(int d);
hipError_t launch_fwd_f32(FwdF32Args a, int d, bool causal, hipStream_t stream);
int fwd_f32_rows_per_workgroup();
hipError_t launch_fwd_fp8(Fp8Args a, int d, bool causal, hipStream_t stream);
int fwd_fp8_rows_per_workgroup(int d);
hipError_t launch_decode(DecodeArgs a, int d, hipStream_t stream);
hipError_t launch_bwd(BwdArgs a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_window(BwdArgs a, int d, hipStream_t stream);   // a.window >= 1
// The same passes with the second tiling of their kernels (plain and causal masks).
hipError_t launch_fwd_bf16_alt_tiles(FwdArgs a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_alt_tiles(BwdArgs a, int d, bool causal, hipStream_t stream);

// Kernels address one head's rows through 32-bit buffer offsets below 2^31.
constexpr long long kMaxHeadBytes = 1ll << 31;

constexpr float kLog2eHost = 1.44269504088896340736f;
constexpr int kDecodeMinChunk = 64;
constexpr int kDecodeAutoChunk = 1024;

// Size of the fixed device scratch fa_decode_splitkv_noalloc keeps its
// partial states in, and the lookup of its address on the current device.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fa
