/*
 * fa.h -- C ABI of the exact tiled-attention library for AMD MI355X (gfx950).
 *
 * The library computes exact softmax attention
 *     O = softmax(scale * Q K^T [+ causal mask]) V
 * tile by tile with the online-softmax recurrence: per query row a running
 * maximum m, a running sum l of exponentials taken relative to m, and a
 * running value-weighted sum u, with l and u rescaled together by e^(m - m')
 * whenever the maximum grows to m'. The T x T score and probability matrices
 * never reach device memory.
 *   kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
 *   Bottleneck", sections "Flash Attention Uses Tiles", "Softmax Looks Like an
 *   Obstacle" and "Causal Masks Still Apply";
 *   aimlrounds "FlashAttention", section "Softmax without seeing the whole
 *   row" and the "FlashAttention 1, 2, 3" table (recomputation in the backward
 *   pass, split-KV decoding).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major ("contiguous") device buffers owned by the
 *     caller. bf16 tensors hold raw bfloat16 bit patterns (2 bytes each).
 *       q, o, dout, dq : [B, Hq,  Tq, d]
 *       k, v, dk, dv   : [B, Hkv, Tk, d]
 *       lse            : [B, Hq,  Tq]  fp32, natural-log log-sum-exp of the
 *                        scaled, masked scores of each query row.
 *   - Grouped KV heads: query head h reads KV head h / (Hq / Hkv); Hq must be
 *     a multiple of Hkv (Hq == Hkv is ordinary multi-head attention).
 *   - causal != 0 masks key j for query i unless j <= i + (Tk - Tq): the
 *     diagonal is aligned to the bottom-right corner, which is the ordinary
 *     "query i sees keys 0..i" rule when Tq == Tk. A query that sees no key
 *     (only possible when causal and Tq > Tk) gets O = 0 and LSE = -inf.
 *   - scale multiplies Q K^T and must be finite and > 0 (typically 1/sqrt(d)).
 *   - d must be 64 or 128. Every pointer must be 16-byte aligned. One head's
 *     rows must span less than 2^31 bytes (T * d * 2 < 2^31, i.e. T below 8M at
 *     d = 128): kernels address them with 32-bit offsets.
 *   - Every call is asynchronous on `stream` (0 = the null stream); results
 *     are valid once the stream has completed. The library never allocates,
 *     frees or synchronises, and keeps no global mutable state: concurrent
 *     calls on different streams are safe when their outputs do not overlap.
 *   - Argument checks run on the host before anything is enqueued: when a
 *     call returns an error, nothing was launched and no output was touched.
 *     FA_ERR_HIP reports a launch failure seen by hipGetLastError afterwards.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misalignment, bad scale */
  FA_ERR_UNSUPPORTED = -2,   /* head width other than 64 or 128 */
  FA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  FA_ERR_HIP = -4            /* a kernel launch failed */
} fa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

/*
 * Forward pass, bf16 inputs and outputs, fp32 accumulation.
 *   q [B,Hq,Tq,d], k and v [B,Hkv,Tk,d]  (bf16, read only)
 *   o [B,Hq,Tq,d]                        (bf16, written)
 *   lse [B,Hq,Tq] fp32, written when non-NULL; it is what fa_bwd needs to
 *   recompute the probabilities (aimlrounds "FlashAttention": the forward
 *   keeps a single fp32 log-sum-exp for each row of each head, for the
 *   backward pass).
 * QK^T and PV run on bf16 matrix cores; the probabilities are rounded to bf16
 * before the PV product, the running sum uses them unrounded.
 * Errors: FA_ERR_INVALID_ARG (q/k/v/o NULL, any size <= 0, Hq % Hkv != 0,
 * scale not finite or <= 0, misaligned pointer), FA_ERR_UNSUPPORTED (d).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
           hipStream_t stream);

/*
 * Causal sliding-window forward: as fa_fwd with causal set, except that query
 * row i sees only the window of `window` keys ending at its own position,
 * i.e. key j is visible iff i + (Tk - Tq) - window < j <= i + (Tk - Tq).
 * The pages list sliding windows among the masks the method works with
 * (aimlrounds "FlashAttention", section "In practice") without defining
 * them; this band is the reading taken. Key tiles wholly outside every row's
 * window are skipped. Errors: as fa_fwd, plus FA_ERR_INVALID_ARG for
 * window < 1.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int window,
                  hipStream_t stream);

/*
 * Forward pass with fp32 inputs and outputs (same parameter list and layout
 * as fa_fwd, every tensor fp32). It computes the same tiled recurrence as
 * fa_fwd (kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
 * Bottleneck", section "Carry the Actual Values Through Both Tiles"; aimlrounds
 * "FlashAttention", section "Softmax without seeing the whole row", whose
 * worked rows are fp32-exact), but scores, probabilities and accumulators stay
 * in fp32 throughout: this is the accuracy path for small problems and those
 * worked rows, not a throughput path. Same errors as fa_fwd.
 */
int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
               hipStream_t stream);

/*
 * Forward pass on fp8 inputs (OCP e4m3 bytes), bf16 output, fp32 log-sum-exp.
 * The aimlrounds "FlashAttention" page (table "FlashAttention 1, 2, 3") lists
 * FP8 among the FlashAttention-3 changes without a recipe; this is the one
 * taken:
 *   q [B,Hq,Tq,d] and k [B,Hkv,Tk,d]  e4m3 bytes, row-major (read only)
 *   vt [B,Hkv,d,Tk]                   e4m3 bytes of V, TRANSPOSED (read only)
 *   q_scale [B*Hq], k_scale [B*Hkv], v_scale [B*Hkv]  fp32 device arrays:
 *                                     the value of a byte x of head (b, h) is
 *                                     x * scale[b*H + h]
 *   o [B,Hq,Tq,d] bf16 and lse [B,Hq,Tq] fp32 (written; lse may be NULL)
 * Computes softmax(scale * Q K^T (+ causal mask)) V on the dequantised values.
 * QK^T and PV run on fp8 matrix cores with fp32 accumulation; the
 * probabilities (times 2^5, at most 2^8) are rounded to e4m3 before the PV
 * product, the running sum uses them unrounded, so O carries a relative error
 * of up to 2^-4 per probability, LSE only the score rounding.
 * Every q_scale, k_scale and v_scale entry must be finite and > 0: the kernel
 * takes the row maximum of the raw byte products and multiplies it by the
 * positive factor scale * log2(e) * q_scale * k_scale, which is the maximum of
 * the scaled scores only for a positive factor. The factors sit in device
 * memory, so the host cannot check them: a zero, negative or NaN factor gives
 * unspecified (possibly non-finite) o and lse, and no error is reported.
 * Errors: as fa_fwd, plus FA_ERR_INVALID_ARG for NULL vt/q_scale/k_scale/
 * v_scale and for Tk not a multiple of 16 (the V^T rows are read in 16-byte
 * chunks); every pointer must be 16-byte aligned except the scale arrays
 * (4-byte).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* vt,
               const float* q_scale, const float* k_scale, const float* v_scale,
               void* o, float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int d,
               float scale, int causal, hipStream_t stream);

/*
 * Workspace bytes fa_bwd needs: two fp32 per query row, the row's LSE in
 * base-2 units and D_i = sum_c dO_ic O_ic, rounded up to 256 bytes. Linear in
 * Tq, never quadratic (aimlrounds "FlashAttention": the N x N matrix is not
 * stored).
 * Returns 0 for non-positive sizes.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Tq, int d);

/*
 * Backward pass by recomputation (bf16 tensors, fp32 accumulation).
 *   q, k, v        forward inputs                        (bf16, read only)
 *   o              forward output from fa_fwd            (bf16, read only)
 *   dout           gradient of the loss w.r.t. o          (bf16, read only)
 *   lse            log-sum-exp written by fa_fwd          (fp32, read only)
 *   dq [B,Hq,Tq,d], dk and dv [B,Hkv,Tk,d]                (bf16, written;
 *                  dk and dv sum over the query heads of each KV group)
 *   workspace      device scratch of at least fa_bwd_workspace_size() bytes
 * The probabilities are rebuilt tile by tile from Q, K and lse instead of
 * being read back (aimlrounds "FlashAttention", follow-up on why the backward
 * pass recomputes; zerotofrontier "Efficient attention: memory-bound",
 * section "Real code moves even more", for the products dV = P^T dO,
 * dP = dO V^T, dS from P and dP, dQ and dK from dS). With
 * dS_ij = P_ij (dP_ij - D_i): dQ = scale dS K, dK = scale dS^T Q.
 * The result is deterministic (no atomics). Errors: as fa_fwd, plus
 * FA_ERR_INVALID_ARG for NULL o/dout/lse/dq/dk/dv and FA_ERR_WORKSPACE.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
           hipStream_t stream);

/*
 * Backward of fa_fwd_window (same band; the parameters of fa_bwd with causal
 * replaced by window >= 1). Errors: as fa_bwd, plus FA_ERR_INVALID_ARG for
 * window < 1.
 */
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int window,
                  hipStream_t stream);

/*
 * fa_fwd and fa_bwd computed with a chosen compiled tiling, for checking that
 * the result does not depend on the tile shape (aimlrounds "FlashAttention",
 * section "Softmax without seeing the whole row": the tiled recurrence gives
 * the same answer for every tile size, up to floating-point rounding).
 *   tile_shape 0: the tiling fa_fwd and fa_bwd use (the same kernels);
 *   tile_shape 1: a second tiling of the same kernels --
 *     forward: 32-key tiles instead of 64, and 128-row query tiles instead
 *              of 256 at d = 128 (d = 64 keeps its 128-row tiles);
 *     backward: dQ takes 32-key tiles at d = 128 and 64-key tiles at d = 64
 *              (the default is the other way round); dK/dV walks 32-row
 *              query tiles where the default walks 64, and 64 where it
 *              walks 32 (causal d = 64).
 * The two tilings round differently (the probabilities are rounded to bf16
 * relative to a running maximum that moves at tile boundaries), so their
 * outputs agree to the bf16 tolerance, not bitwise. Parameters, layouts,
 * workspace and errors are those of fa_fwd and fa_bwd, plus
 * FA_ERR_INVALID_ARG for a tile_shape other than 0 or 1.
 */
int fa_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal, int tile_shape,
                 hipStream_t stream);
int fa_bwd_tiles(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                 int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal, int tile_shape,
                 hipStream_t stream);

/*
 * Dropout of the attention probabilities in the fused forward and backward.
 * The zerotofrontier page "Efficient attention: memory-bound" (section "Real
 * code moves even more") lists dropout among the elementwise steps a training
 * forward pass applies to the probabilities before the product with V; the
 * pages give no random-number contract. The one fixed here:
 *   - keep threshold t = round((1 - p_drop) * 256) (ties to even), which must
 *     lie in [1, 256]; an entry is kept with probability t / 256 and kept
 *     entries are scaled by 256 / t, so O = (P * Z) V * 256 / t;
 *   - for query row i of flattened head bh = b * Hq + h and the 16 keys
 *     16 g .. 16 g + 15, one Philox-4x32-10 call (Salmon, Moraes, Dror and
 *     Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) with counter
 *     (g, i, bh, offset) and key (seed mod 2^32, seed >> 32) yields four
 *     32-bit words; key j takes byte j mod 16 (byte n = bits 8 (n mod 4) ..
 *     8 (n mod 4) + 7 of word n / 4) and is kept iff that byte is below t;
 *   - the log-sum-exp is that of the softmax before dropout, so the forward's
 *     lse feeds fa_bwd_dropout unchanged.
 * The same (p_drop, seed, offset) must be passed to the forward and the
 * backward of one layer; distinct offsets (or seeds) give independent masks.
 */

/* Keep threshold t in [1, 256] for a dropout probability p_drop in [0, 1), or
 * FA_ERR_INVALID_ARG when p_drop is not finite, outside [0, 1), or so close
 * to 1 that t would be 0. */
int fa_dropout_keep_threshold(float p_drop);

/*
 * Forward with dropout: the parameters of fa_fwd plus p_drop, seed and
 * offset (see above); d, layout, ownership and errors as fa_fwd, plus
 * FA_ERR_INVALID_ARG for an unusable p_drop. p_drop = 0 (t = 256) keeps
 * every entry and runs the plain forward.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
                   float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream);

/*
 * Backward of fa_fwd_dropout with the same (p_drop, seed, offset): the mask
 * is regenerated, never stored. o and lse are the dropout forward's outputs.
 * dV = (P * Z)^T dO * 256 / t, the softmax gradient takes
 * dP = (dO V^T) * Z * 256 / t, and rowsum(dO * O) still equals
 * sum_j P_ij dP_ij. Parameters, workspace and errors as fa_bwd, plus
 * FA_ERR_INVALID_ARG for an unusable p_drop.
 */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                   int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
                   float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream);

/*
 * Workspace bytes fa_decode_splitkv needs for KV caches of up to Tk_max
 * positions: per (batch, query head, split) one partial state (m, l, u[d])
 * in fp32, for the largest split count the library may choose (64-key
 * splits). Each split is one tile-sized piece of the row whose running
 * maximum, sum and weighted sum are later merged with the rescale rule
 * (kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
 * Bottleneck", section "Softmax Looks Like an Obstacle"; aimlrounds
 * "FlashAttention", note under the "FlashAttention 1, 2, 3" table on
 * splitting the cache). Linear in Tk_max, never quadratic. Returns 0 for
 * non-positive sizes.
 */
size_t fa_decode_workspace_size(int B, int Hq, int Tk_max, int d);

/*
 * One query token per (batch, query head) against a KV cache (split-KV
 * decoding, aimlrounds "FlashAttention", note under the "FlashAttention 1,
 * 2, 3" table: the long cache is split across workgroups).
 *   q [B,Hq,d]                 (bf16, read only)
 *   k_cache, v_cache [B,Hkv,Tk_max,d]  (bf16, read only; positions at or
 *                              beyond seq_lens[b] are never read)
 *   seq_lens [B]               (int32, device memory) valid cache lengths
 *   o [B,Hq,d]                 (bf16, written)
 *   lse [B,Hq]                 (fp32, written when non-NULL)
 *   workspace                  fp32 partial states, >= fa_decode_workspace_size
 *   chunk                      keys per split: 0 lets the library choose,
 *                              otherwise a multiple of 64 in [64, Tk_max
 *                              rounded up to 64]
 * Each split runs the online recurrence over its keys and stores its partial
 * (m, l, u); a second kernel merges the splits with the same rescale rule.
 * Device-side range errors: a seq_lens[b] outside [1, Tk_max] cannot be
 * reported without a synchronisation; that batch entry's o (and lse) are
 * written as NaN instead. Errors: FA_ERR_INVALID_ARG (NULL q/k_cache/v_cache/
 * seq_lens/o, sizes, Hq % Hkv, scale, chunk), FA_ERR_UNSUPPORTED (d),
 * FA_ERR_WORKSPACE.
 */
int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int* seq_lens, void* o, float* lse,
                      void* workspace, size_t ws_bytes,
                      int B, int Hq, int Hkv, int Tk_max, int d, float scale, int chunk,
                      hipStream_t stream);

/*
 * Split-KV decoding with a sliding window: as fa_decode_splitkv, but the
 * query of batch entry b sees only the last `window` cached keys
 * (positions max(0, seq_lens[b] - window) .. seq_lens[b] - 1; the band of
 * fa_fwd_window for the query at position seq_lens[b] - 1). Chunks wholly
 * before the window are not read. Same workspace size. Errors: as
 * fa_decode_splitkv, plus FA_ERR_INVALID_ARG for window < 1.
 */
int fa_decode_splitkv_window(const void* q, const void* k_cache, const void* v_cache,
                             const int* seq_lens, void* o, float* lse,
                             void* workspace, size_t ws_bytes,
                             int B, int Hq, int Hkv, int Tk_max, int d, float scale, int window, int chunk,
                             hipStream_t stream);

/* Bytes of the fixed device scratch behind fa_decode_splitkv_noalloc (16 MiB). */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * Split-KV decoding that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Parameters, layouts,
 * results and errors are those of fa_decode_splitkv without the workspace
 * arguments, and for the same chunk the output is bitwise identical to
 * fa_decode_splitkv's (the same kernels run).
 *   - The partial states live in a fixed device scratch of
 *     FA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 *     runs on until the process ends. A call uses
 *     2 * r(4 n) + r(4 d n) bytes of it, with n = B * Hq * ceil(Tk_max / chunk)
 *     (chunk 0 means 1024) and r() rounding up to a multiple of 256; a call
 *     that needs more returns FA_ERR_WORKSPACE and launches nothing. (B = 16,
 *     Hq = 32, Tk_max = 32768, d = 128 needs 8.5 MB at the automatic chunk.)
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's partial states (no part of it has to start at zero). Calls that
 *     overlap in time on one GPU (on different streams, or from different
 *     host threads) race on it and give wrong results: serialise them, e.g.
 *     on one stream.
 *   - stream must belong to the current device (FA_ERR_INVALID_ARG
 *     otherwise). FA_ERR_HIP if the scratch's address cannot be looked up.
 */
int fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seq_lens, void* o, float* lse,
                              int B, int Hq, int Hkv, int Tk_max, int d, float scale, int chunk,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
