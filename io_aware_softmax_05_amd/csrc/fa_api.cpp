// fa_api.cpp -- the C ABI: argument checks on the host, then kernel launches.
// Every check happens before anything is enqueued, so an error return means
// no kernel ran and no output was touched.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_SCRATCH_BYTES, "one scratch size");

namespace {

constexpr int kMaxGrid = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // element offsets are formed in size_t, row indices in int
  if ((int64_t)B * Hq > INT32_MAX / 2 || (int64_t)B * Hkv > INT32_MAX / 2) return FA_ERR_INVALID_ARG;
  // one head's rows are addressed with 32-bit buffer offsets
  if ((int64_t)Tq * d * 2 >= fa::kMaxHeadBytes || (int64_t)Tk * d * 2 >= fa::kMaxHeadBytes) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Dropout arguments for a usable p_drop (t in [1, 255]); t = 256 keeps
// everything and is returned as "no dropout" (t = 0).
int make_drop(float p_drop, uint64_t seed, uint32_t offset, fa::DropArgs* out) {
  const int t = fa_dropout_keep_threshold(p_drop);
  if (t < 0) return t;
  *out = fa::DropArgs{};
  if (t == 256) return FA_OK;
  out->t = (uint32_t)t;
  out->seed_lo = (uint32_t)seed;
  out->seed_hi = (uint32_t)(seed >> 32);
  out->offset = offset;
  out->inv_keep = 256.f / (float)t;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

int fa_dropout_keep_threshold(float p_drop) {
  if (!isfinite(p_drop) || p_drop < 0.f || p_drop >= 1.f) return FA_ERR_INVALID_ARG;
  const double t = nearbyint((1.0 - (double)p_drop) * 256.0);   // default rounding: ties to even
  if (t < 1.0 || t > 256.0) return FA_ERR_INVALID_ARG;
  return (int)t;
}

static int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal, int window,
                    hipStream_t stream, const fa::DropArgs& drop = fa::DropArgs{}, bool alt_tiles = false) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  const int st = check_common(B, Hq, Hkv, Tq, Tk, d, scale);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  const int br = fa::fwd_rows_per_workgroup(d);
  if ((int64_t)((Tq + br - 1) / br) * B * Hq > INT32_MAX) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.c = scale * fa::kLog2eHost;
  a.window = window;
  a.drop = drop;
  if (alt_tiles) return to_status(fa::launch_fwd_bf16_alt_tiles(a, d, causal != 0, stream));
  return to_status(fa::launch_fwd_bf16(a, d, causal != 0, stream));
}

int fa_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal, int tile_shape,
                 hipStream_t stream) {
  if (tile_shape != 0 && tile_shape != 1) return FA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, 0, stream, fa::DropArgs{}, tile_shape == 1);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
                   float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream) {
  fa::DropArgs drop;
  const int st = make_drop(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, 0, stream, drop);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
           hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, 0, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* vt,
               const float* q_scale, const float* k_scale, const float* v_scale,
               void* o, float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int d,
               float scale, int causal, hipStream_t stream) {
  if (!q || !k || !vt || !q_scale || !k_scale || !v_scale || !o) return FA_ERR_INVALID_ARG;
  const int st = check_common(B, Hq, Hkv, Tq, Tk, d, scale);
  if (st != FA_OK) return st;
  if (Tk % 16 != 0) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
       reinterpret_cast<uintptr_t>(v_scale)) & 3u)
    return FA_ERR_INVALID_ARG;
  const int br = fa::fwd_fp8_rows_per_workgroup(d);
  if ((int64_t)((Tq + br - 1) / br) * B * Hq > INT32_MAX) return FA_ERR_INVALID_ARG;
  fa::Fp8Args a{};
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.vt = static_cast<const uint8_t*>(vt);
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.c = scale * fa::kLog2eHost;
  return to_status(fa::launch_fwd_fp8(a, d, causal != 0, stream));
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int window,
                  hipStream_t stream) {
  if (window < 1) return FA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, 1, window, stream);
}

int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
               hipStream_t stream) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  const int st = check_common(B, Hq, Hkv, Tq, Tk, d, scale);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  // one wave per query row, a few rows of one head per workgroup
  const int rows_per_group = fa::fwd_f32_rows_per_workgroup();
  if ((int64_t)B * Hq * ((Tq + rows_per_group - 1) / rows_per_group) > INT32_MAX) return FA_ERR_INVALID_ARG;
  fa::FwdF32Args a{};
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.o = static_cast<float*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.scale = scale;
  return to_status(fa::launch_fwd_f32(a, d, causal != 0, stream));
}

size_t fa_bwd_workspace_size(int B, int Hq, int Tq, int d) {
  if (B <= 0 || Hq <= 0 || Tq <= 0 || d <= 0) return 0;
  return round256((size_t)B * Hq * Tq * 2 * sizeof(float));
}

static int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                    int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal, int window,
                    hipStream_t stream, const fa::DropArgs& drop = fa::DropArgs{}, bool alt_tiles = false) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  const int st = check_common(B, Hq, Hkv, Tq, Tk, d, scale);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  // grids of 32-row (32-key) granularity must fit the launch limits
  if ((int64_t)((Tq + 31) / 32) * B * Hq > INT32_MAX || (int64_t)((Tk + 31) / 32) * B * Hkv > INT32_MAX)
    return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) || ws_bytes < fa_bwd_workspace_size(B, Hq, Tq, d))
    return FA_ERR_WORKSPACE;
  fa::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.stats = static_cast<float*>(workspace);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.scale = scale;
  a.c = scale * fa::kLog2eHost;
  a.window = window;
  a.drop = drop;
  if (alt_tiles) return to_status(fa::launch_bwd_alt_tiles(a, d, causal != 0, stream));
  return to_status(window > 0 ? fa::launch_bwd_window(a, d, stream) : fa::launch_bwd(a, d, causal != 0, stream));
}

int fa_bwd_tiles(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                 int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal, int tile_shape,
                 hipStream_t stream) {
  if (tile_shape != 0 && tile_shape != 1) return FA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal, 0,
                  stream, fa::DropArgs{}, tile_shape == 1);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                   int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
                   float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream) {
  fa::DropArgs drop;
  const int st = make_drop(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale,
                  causal, 0, stream, drop);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
           hipStream_t stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale,
                  causal, 0, stream);
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int window,
                  hipStream_t stream) {
  if (window < 1) return FA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale,
                  1, window, stream);
}


// Bytes of the partial states for `per` (batch, query head, split) entries:
// planes m and l, then u[d], each plane starting on a 256-byte boundary.
static size_t decode_partials_bytes(size_t per, int d) {
  return round256(per * sizeof(float)) * 2 + round256(per * d * sizeof(float));
}

size_t fa_decode_workspace_size(int B, int Hq, int Tk_max, int d) {
  if (B <= 0 || Hq <= 0 || Tk_max <= 0 || d <= 0) return 0;
  const size_t splits = ((size_t)Tk_max + fa::kDecodeMinChunk - 1) / fa::kDecodeMinChunk;
  return decode_partials_bytes((size_t)B * Hq * splits, d);
}

// The caller's workspace (sized for the largest split count the library may
// choose) or, with workspace == nullptr and fixed_scratch set, the library's
// fixed device scratch laid out for this call's split count.
static int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                       const int* seq_lens, void* o, float* lse,
                       void* workspace, size_t ws_bytes,
                       int B, int Hq, int Hkv, int Tk_max, int d, float scale, int window, int chunk,
                       hipStream_t stream, bool fixed_scratch = false) {
  if (!q || !k_cache || !v_cache || !seq_lens || !o) return FA_ERR_INVALID_ARG;
  const int st = check_common(B, Hq, Hkv, 1, Tk_max, d, scale);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (chunk == 0) chunk = fa::kDecodeAutoChunk;
  if (chunk < fa::kDecodeMinChunk || chunk % 64 != 0) return FA_ERR_INVALID_ARG;
  const int max_chunk = (Tk_max + 63) / 64 * 64;
  if (chunk > max_chunk) chunk = max_chunk;
  const int n_splits = (Tk_max + chunk - 1) / chunk;
  const int G = Hq / Hkv;
  if (B > kMaxGrid || (int64_t)Hkv * ((G + 15) / 16) > kMaxGrid) return FA_ERR_INVALID_ARG;
  size_t per = 0;   // partial-state entries between the planes
  char* ws = nullptr;
  if (fixed_scratch) {
    per = (size_t)B * Hq * n_splits;
    if (decode_partials_bytes(per, d) > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
    // the scratch address is per device: the stream must run on the current one
    if (stream != nullptr) {
      int cur = 0, sdev = 0;
      if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
      if (cur != sdev) return FA_ERR_INVALID_ARG;
    }
    void* p = nullptr;
    if (fa::decode_scratch(&p) != hipSuccess) return FA_ERR_HIP;
    ws = static_cast<char*>(p);
  } else {
    if (!workspace || !aligned16(workspace) || ws_bytes < fa_decode_workspace_size(B, Hq, Tk_max, d))
      return FA_ERR_WORKSPACE;
    per = (size_t)B * Hq * (((size_t)Tk_max + fa::kDecodeMinChunk - 1) / fa::kDecodeMinChunk);
    ws = static_cast<char*>(workspace);
  }
  fa::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.seq_lens = seq_lens;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.part_m = reinterpret_cast<float*>(ws);
  a.part_l = reinterpret_cast<float*>(ws + round256(per * sizeof(float)));
  a.part_u = reinterpret_cast<float*>(ws + 2 * round256(per * sizeof(float)));
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tk_max = Tk_max;
  a.chunk = chunk;
  a.n_splits = n_splits;
  a.c = scale * fa::kLog2eHost;
  a.window = window;
  return to_status(fa::launch_decode(a, d, stream));
}

int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int* seq_lens, void* o, float* lse,
                      void* workspace, size_t ws_bytes,
                      int B, int Hq, int Hkv, int Tk_max, int d, float scale, int chunk,
                      hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, o, lse, workspace, ws_bytes, B, Hq, Hkv, Tk_max, d, scale,
                     0, chunk, stream);
}

int fa_decode_splitkv_window(const void* q, const void* k_cache, const void* v_cache,
                             const int* seq_lens, void* o, float* lse,
                             void* workspace, size_t ws_bytes,
                             int B, int Hq, int Hkv, int Tk_max, int d, float scale, int window, int chunk,
                             hipStream_t stream) {
  if (window < 1) return FA_ERR_INVALID_ARG;
  return decode_impl(q, k_cache, v_cache, seq_lens, o, lse, workspace, ws_bytes, B, Hq, Hkv, Tk_max, d, scale,
                     window, chunk, stream);
}

int fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seq_lens, void* o, float* lse,
                              int B, int Hq, int Hkv, int Tk_max, int d, float scale, int chunk,
                              hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, o, lse, nullptr, 0, B, Hq, Hkv, Tk_max, d, scale, 0, chunk,
                     stream, true);
}

}  // extern "C"
