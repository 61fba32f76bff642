"""Plain fp64 CPU oracle for exact (softmax) attention: forward, backward, decode.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
tests, the package smoke check and the benchmark's CPU-baseline leg import it.
It shares no code with the HIP library and imports nothing from the package.

What it computes is the plain three-step definition (scores, probabilities,
weighted values), never the tiled online recurrence:
  * zerotofrontier "Efficient attention: memory-bound", section "Standard
    attention, kernel by kernel": S from Q and K, P as the row softmax of S,
    O = P V, with the scores scaled by 1/sqrt(d_k) (section "Real code moves
    even more" names the scale step);
  * same page, section "The obstacle, a normalizer that needs the whole row":
    P_ij uses the row maximum m_i only for safety and the normaliser l_i;
  * kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
    Bottleneck", section "Causal Masks Still Apply": a query sees keys up to
    and including its own position;
  * aimlrounds "FlashAttention", section "Softmax without seeing the whole
    row": the per-row log-sum-exp kept for the backward pass;
  * zerotofrontier page, section "Real code moves even more": the backward
    products dV = P^T dO, dP = dO V^T, dS from P and dP, dQ and dK from dS.

Readings taken where the pages are silent (each is pinned by a test):
  * causal with Tq != Tk aligns the diagonal bottom-right: key j is visible to
    query i iff j <= i + (Tk - Tq);
  * a query with no visible key (only causal with Tq > Tk) has O = 0 and
    LSE = -inf, and contributes nothing to any gradient;
  * LSE is the natural log of sum_j exp(S_ij), S already scaled;
  * the softmax backward is the textbook Jacobian:
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik);
  * grouped KV heads are contiguous groups: query head h uses KV head
    h // (Hq // Hkv); dK and dV sum over the group;
  * a sliding window (aimlrounds "FlashAttention", section "In practice",
    lists sliding windows among the masks the method works with, without a
    definition) of W >= 1 keys is read as a causal band: key j is visible to query
    i iff i + (Tk - Tq) - W < j <= i + (Tk - Tq), i.e. each query sees its
    own position and the W - 1 keys before it; in decoding the one query
    sees the last W cached keys. W = 0 means no window;
  * dropout (zerotofrontier page, section "Real code moves even more": a
    training forward pass applies it to the probabilities before the final
    product) keeps P_ij with probability kappa = t / 256 and scales kept
    entries by 1 / kappa, so O = (P * Z / kappa) V with the keep mask Z of
    `dropout_keep`; the log-sum-exp is that of the softmax before dropout.

Rows are independent, so every function may work on any subset of query rows
(the full-size checks evaluate sampled rows one block at a time). Keys are
never split: each row always sees its whole score row at once.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import philox4x32_10

_ROW_BLOCK = 512


@dataclass(frozen=True)
class Dropout:
    """Dropout of the attention probabilities.

    t in [1, 256] is the keep threshold (keep probability kappa = t / 256);
    seed (64 bits) and offset (32 bits) choose the random stream."""
    t: int
    seed: int
    offset: int = 0

    @property
    def kappa(self) -> float:
        return self.t / 256.0


def keep_threshold(p_drop: float) -> int:
    """Keep threshold for a dropout probability: t = (1 - p) * 256 rounded to
    the nearest integer (ties to even), valid when 1 <= t <= 256."""
    t = round((1.0 - float(p_drop)) * 256.0)
    if not (0.0 <= float(p_drop) < 1.0) or not 1 <= t <= 256:
        raise ValueError(f"dropout probability {p_drop} gives no usable keep threshold")
    return int(t)


def dropout_keep(drop: Dropout, bh: int, rows, Tk: int) -> np.ndarray:
    """Boolean [len(rows), Tk]: is P[i, j] of flattened head bh = b * Hq + h kept?

    Random-number contract: for query row i and the 16 keys 16 g .. 16 g + 15,
    one Philox-4x32-10 call with counter (g, i, bh, offset) and key
    (seed mod 2^32, seed div 2^32) gives four words; key j uses byte j mod 16
    of them, byte n being bits 8 (n mod 4) .. 8 (n mod 4) + 7 of word n div 4.
    The entry is kept iff that byte is below t."""
    rows = np.asarray(rows, dtype=np.int64)
    n_groups = (Tk + 15) // 16
    g = np.arange(n_groups, dtype=np.int64)
    words = philox4x32_10(g[None, :], rows[:, None], bh, drop.offset,
                          drop.seed & 0xFFFFFFFF, (drop.seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=-1).astype(np.uint32)            # [n, groups, word]
    b = w[..., None] >> (np.arange(4, dtype=np.uint32) * 8)   # [n, groups, word, byte]
    bytes_ = (b & 0xFF).reshape(rows.shape[0], n_groups * 16)[:, :Tk]
    return bytes_ < drop.t


def _dropped(p: np.ndarray, drop, bh: int, rows, Tk: int):
    """(P * Z / kappa, Z / kappa) for the rows of one head; (P, 1) without dropout."""
    if drop is None:
        return p, 1.0
    z = dropout_keep(drop, bh, rows, Tk) / drop.kappa
    return p * z, z


def visible(rows: np.ndarray, Tq: int, Tk: int, causal: bool, window: int = 0) -> np.ndarray:
    """Boolean [len(rows), Tk]: may query row i look at key j (a window needs causal)."""
    rows = np.asarray(rows, dtype=np.int64)
    if not causal:
        assert window == 0, "a sliding window is a causal band"
        return np.ones((rows.shape[0], Tk), dtype=bool)
    j = np.arange(Tk, dtype=np.int64)
    last = rows[:, None] + (Tk - Tq)
    vis = j[None, :] <= last
    if window > 0:
        vis &= j[None, :] > last - window
    return vis


def row_probs(q_rows: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray,
              Tq: int, causal: bool, window: int = 0):
    """Scores, probabilities and log-sum-exp for some query rows of one head.

    q_rows [n,d], k [Tk,d] (fp64). Returns P [n,Tk] (zero where masked and for
    empty rows) and lse [n] (-inf for empty rows)."""
    Tk = k.shape[0]
    s = scale * (q_rows @ k.T)
    vis = visible(rows, Tq, Tk, causal, window)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return p, lse


def _kv_head(hq: int, Hq: int, Hkv: int) -> int:
    return hq // (Hq // Hkv)


def attention_fwd(q, k, v, scale: float, causal: bool, rows=None, window: int = 0, dropout=None):
    """Forward: O [B,Hq,n,d] and LSE [B,Hq,n] for query rows `rows` (all if None).

    q [B,Hq,Tq,d]; k, v [B,Hkv,Tk,d]; any float dtype, computed in fp64.
    `dropout` (a Dropout or None) drops probabilities before the product with V."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0 and k.shape[0] == B and v.shape == k.shape
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, Hq, rows.shape[0], v.shape[3]))
    lse = np.zeros((B, Hq, rows.shape[0]))
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            for s in range(0, rows.shape[0], _ROW_BLOCK):
                r = rows[s:s + _ROW_BLOCK]
                p, l = row_probs(q[b, h, r], k[b, hk], scale, r, Tq, causal, window)
                pd, _ = _dropped(p, dropout, b * Hq + h, r, k.shape[2])
                o[b, h, s:s + _ROW_BLOCK] = pd @ v[b, hk]
                lse[b, h, s:s + _ROW_BLOCK] = l
    return o, lse


def attention_fwd_head_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows, dropout=None):
    """O [n,d] and LSE [n] of some query rows of one (batch, query head), from
    the full tensors, so that the dropout stream sees the head's own index
    b * Hq + h. Same computation as attention_fwd."""
    Hq, Hkv = np.shape(q)[1], np.shape(k)[1]
    hk = _kv_head(h, Hq, Hkv)
    kk = np.asarray(k[b, hk], dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    # the sampled rows are taken before widening (a head may hold millions of rows)
    p, lse = row_probs(np.asarray(np.asarray(q[b, h])[rows], dtype=np.float64), kk, scale, rows, np.shape(q)[2],
                       causal)
    pd, _ = _dropped(p, dropout, b * Hq + h, rows, kk.shape[0])
    return pd @ np.asarray(v[b, hk], dtype=np.float64), lse


def e4m3_to_f64(bits) -> np.ndarray:
    """Values of OCP 8-bit floats in the E4M3 format, exactly, as fp64.

    E4M3 (the variant without infinities): 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits. Exponent field 0 holds the subnormals
    (mantissa / 8) * 2^-6; the codes S.1111.111 are NaN; every other code is
    (1 + mantissa / 8) * 2^(exponent - 7), the largest being 448."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where((b >> 7) != 0, -1.0, 1.0)
    e = (b >> 3) & 15
    f = (b & 7).astype(np.float64)
    mag = np.where(e == 0, (f / 8.0) * 2.0 ** -6, (1.0 + f / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


def attention_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, scale: float, causal: bool, rows=None):
    """Forward on fp8 inputs: exact attention over the values the bytes stand for.

    aimlrounds "FlashAttention", table "FlashAttention 1, 2, 3", lists FP8
    among the FlashAttention-3 changes and gives no recipe; the reading taken
    is per-(batch, head) dequantisation factors:
      q8 [B,Hq,Tq,d], k8 [B,Hkv,Tk,d] e4m3 bytes; vt8 [B,Hkv,d,Tk] e4m3 bytes
      of V transposed; q_scale [B,Hq], k_scale and v_scale [B,Hkv];
      Q = e4m3(q8) * q_scale[b, h] (likewise K and V per kv head).
    Returns O and LSE of softmax(scale Q K^T [+causal]) V, as attention_fwd."""
    q = e4m3_to_f64(q8) * np.asarray(q_scale, dtype=np.float64)[:, :, None, None]
    k = e4m3_to_f64(k8) * np.asarray(k_scale, dtype=np.float64)[:, :, None, None]
    v = np.swapaxes(e4m3_to_f64(vt8), 2, 3) * np.asarray(v_scale, dtype=np.float64)[:, :, None, None]
    return attention_fwd(q, k, v, scale, causal, rows)


def attention_bwd(q, k, v, do, scale: float, causal: bool, window: int = 0, dropout=None):
    """Backward of O = softmax(scale Q K^T [+mask]) V given dO.

    Returns dQ [B,Hq,Tq,d], dK and dV [B,Hkv,Tk,d] in fp64. P is recomputed
    here from Q and K (this oracle never sees the GPU's O or LSE). With
    dropout, O = Pd V with Pd = P Z / kappa, so dV = Pd^T dO and the softmax
    sees dP = (dO V^T) Z / kappa."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            for s in range(0, Tq, _ROW_BLOCK):
                r = np.arange(s, min(Tq, s + _ROW_BLOCK))
                p, _ = row_probs(q[b, h, r], k[b, hk], scale, r, Tq, causal, window)
                pd, z = _dropped(p, dropout, b * Hq + h, r, k.shape[2])
                g = do[b, h, r]
                dv[b, hk] += pd.T @ g
                dp = (g @ v[b, hk].T) * z
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, r] = scale * (ds @ k[b, hk])
                dk[b, hk] += scale * (ds.T @ q[b, h, r])
    return dq, dk, dv


def attention_bwd_dq_rows(q, k, v, do, scale: float, causal: bool, b: int, h: int, rows, window: int = 0,
                          dropout=None):
    """dQ for some query rows of one (batch, query head): each row's gradient
    needs only that row's own scores, so it can be evaluated at any size."""
    Hq, Hkv = np.shape(do)[1], np.shape(k)[1]
    hk = _kv_head(h, Hq, Hkv)
    kk = np.asarray(k[b, hk], dtype=np.float64)
    vv = np.asarray(v[b, hk], dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    Tq = np.shape(q)[2]
    # the sampled rows are taken before widening (a head may hold millions of rows)
    p, _ = row_probs(np.asarray(np.asarray(q[b, h])[rows], dtype=np.float64), kk, scale, rows, Tq, causal, window)
    _, z = _dropped(p, dropout, b * Hq + h, rows, kk.shape[0])
    g = np.asarray(np.asarray(do[b, h])[rows], dtype=np.float64)
    dp = (g @ vv.T) * z
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ kk)


def attention_bwd_dkdv_keys(q, k, v, do, scale: float, causal: bool, b: int, hk: int, keys, window: int = 0,
                            dropout=None):
    """dK and dV for some keys of one (batch, KV head).

    A key's gradient sums contributions of every query row of the group that
    sees it; each row's probabilities still come from that row's whole score
    row. Keys near the end of a causal sequence are seen by few rows, so they
    can be evaluated at any length. Returns (dK [n,d], dV [n,d]) in fp64."""
    Hq, Hkv = np.shape(q)[1], np.shape(k)[1]
    g = Hq // Hkv
    Tq = np.shape(q)[2]
    kk = np.asarray(k[b, hk], dtype=np.float64)
    vv = np.asarray(v[b, hk], dtype=np.float64)
    keys = np.asarray(keys, dtype=np.int64)
    Tk = kk.shape[0]
    first, stop = 0, Tq
    if causal:
        first = max(0, int(keys.min()) - (Tk - Tq))
    if window > 0:   # rows past the last key's window see none of these keys
        stop = max(first, min(Tq, int(keys.max()) - (Tk - Tq) + window))
    dk = np.zeros((keys.shape[0], kk.shape[1]))
    dv = np.zeros((keys.shape[0], vv.shape[1]))
    for h in range(hk * g, (hk + 1) * g):
        qq = np.asarray(q[b, h], dtype=np.float64)
        gg = np.asarray(do[b, h], dtype=np.float64)
        for s in range(first, stop, _ROW_BLOCK):
            r = np.arange(s, min(stop, s + _ROW_BLOCK))
            p, _ = row_probs(qq[r], kk, scale, r, Tq, causal, window)
            pd, z = _dropped(p, dropout, b * Hq + h, r, Tk)
            dp = (gg[r] @ vv.T) * z
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dv += pd[:, keys].T @ gg[r]
            dk += scale * (ds[:, keys].T @ qq[r])
    return dk, dv


def decode(q, k_cache, v_cache, seq_lens, scale: float, heads=None, window: int = 0):
    """One query token per (batch, head) against the first seq_lens[b] cached keys
    (only the last `window` of them when window > 0).

    q [B,Hq,d]; caches [B,Hkv,Tk_max,d]. Returns O [B,Hq,d] and LSE [B,Hq];
    `heads` optionally limits the work to a list of (b, hq) pairs (others 0)."""
    B, Hq, d = np.shape(q)
    Hkv = np.shape(k_cache)[1]
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    for b, h in pairs:
        L = int(seq_lens[b])
        lo = max(0, L - window) if window > 0 else 0
        hk = _kv_head(h, Hq, Hkv)
        kk = np.asarray(k_cache[b, hk, lo:L], dtype=np.float64)
        vv = np.asarray(v_cache[b, hk, lo:L], dtype=np.float64)
        qq = np.asarray(q[b, h], dtype=np.float64)[None, :]
        p, l = row_probs(qq, kk, scale, np.zeros(1, dtype=np.int64), 1, False)
        o[b, h] = (p @ vv)[0]
        lse[b, h] = l[0]
    return o, lse
