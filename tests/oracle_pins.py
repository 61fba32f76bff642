"""Checks that pin the CPU oracle's forward to facts outside itself.

Each check takes a forward function with the oracle's signature
fwd(q, k, v, scale, causal) -> (O, LSE) and raises AssertionError on a
mismatch, so the same checks can be run against deliberately broken copies
of the forward (see test_oracle_mutants.py).

Sources of truth:
  * numbers the pages print for their worked rows (tests/golden/worked_rows.json);
  * brute force: the softmax definition evaluated with pure-Python loops and
    math.fsum, with no max shift, on tiny inputs;
  * closed forms: zero queries average the visible values, constant values
    pass through, causal row 0 returns V_0 with LSE = scale q_0 . k_0,
    jointly permuting keys and values changes nothing (non-causal).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_rows.json")


def load_worked_rows() -> dict:
    with open(GOLDEN) as f:
        return json.load(f)


def embed_row(scores, values, d: int = 64):
    """One query whose scaled scores against the keys are `scores` and whose
    value rows are constant `values` (scale 1): q = e0, k_j = s_j e0,
    v_j = val_j * ones. Every number here is exact in bf16 and fp32."""
    T = len(scores)
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, T, d))
    k[0, 0, :, 0] = scores
    v = np.repeat(np.asarray(values, dtype=np.float64)[:, None], d, axis=1)[None, None]
    return q, k, v


def closed_form_four_key():
    """The tiled normaliser and numerator the kgptalkie page writes out after
    the second tile of the 4-key row (its section 'Carry the Actual Values
    Through Both Tiles'), relative to the new maximum 3."""
    l2 = math.exp(-1) * (1 + math.exp(-1)) + 1 + math.exp(-3)
    u2 = math.exp(-1) * (10 + 20 * math.exp(-1)) + 30 + 40 * math.exp(-3)
    return l2, u2


def brute_attention(q, k, v, scale, causal):
    """Pure-Python softmax attention for one head (lists of lists), no max shift."""
    Tq, Tk, d = len(q), len(k), len(q[0])
    out, lse = [], []
    for i in range(Tq):
        terms = []
        for j in range(Tk):
            if causal and j > i + (Tk - Tq):
                continue
            s = scale * math.fsum(q[i][c] * k[j][c] for c in range(d))
            terms.append((math.exp(s), j))
        if not terms:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        z = math.fsum(w for w, _ in terms)
        out.append([math.fsum(w * v[j][c] for w, j in terms) / z for c in range(len(v[0]))])
        lse.append(math.log(z))
    return out, lse


def pin_worked_rows(fwd):
    g = load_worked_rows()
    r4 = g["four_key_row"]
    l2, u2 = closed_form_four_key()
    q, k, v = embed_row(r4["scores"], r4["values"])
    o, lse = fwd(q, k, v, 1.0, False)
    assert np.allclose(o[0, 0, 0], u2 / l2, rtol=r4["check_rel_tol"], atol=0), (o[0, 0, 0, 0], u2 / l2)
    assert math.isclose(lse[0, 0, 0], 3.0 + math.log(l2), rel_tol=1e-12)
    # after the first tile (keys 0, 1) the row's output is u/l of the printed state
    a = r4["after_tile_1"]
    q1, k1, v1 = embed_row(r4["scores"][:2], r4["values"][:2])
    o1, lse1 = fwd(q1, k1, v1, 1.0, False)
    half_ulp = 0.5 * 10 ** -a["printed_decimals"]
    l_first = math.exp(lse1[0, 0, 0] - a["m"])      # sum of e^(s - m) over the tile
    assert abs(l_first - a["l"]) <= half_ulp + 1e-15, l_first
    assert abs(o1[0, 0, 0, 0] * l_first - a["u"]) <= half_ulp + 1e-13, o1[0, 0, 0, 0] * l_first

    r8 = g["eight_key_row"]
    tol = 0.5 * 10 ** -r8["printed_decimals"]
    q, k, v = embed_row(r8["scores"], r8["values"])
    o, lse = fwd(q, k, v, 1.0, False)
    assert abs(o[0, 0, 0, 0] - r8["final_output"]) <= tol, o[0, 0, 0, 0]
    t = r8["tile"]
    q, k, v = embed_row(r8["scores"][:t], r8["values"][:t])
    o, _ = fwd(q, k, v, 1.0, False)
    assert abs(o[0, 0, 0, 0] - r8["output_after_tile_1"]) <= tol, o[0, 0, 0, 0]


def pin_brute_force(fwd, seed: int = 0):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    cases = [(1, 1, 1, 5, 5, 3, False), (1, 1, 1, 6, 6, 4, True), (2, 2, 1, 3, 7, 2, True),
             (1, 4, 2, 7, 4, 3, True), (1, 2, 2, 8, 3, 4, False), (1, 1, 1, 1, 8, 4, True)]
    for (B, Hq, Hkv, Tq, Tk, d, causal) in cases:
        q = rng.standard_normal((B, Hq, Tq, d))
        k = rng.standard_normal((B, Hkv, Tk, d))
        v = rng.standard_normal((B, Hkv, Tk, d))
        scale = 0.7
        o, lse = fwd(q, k, v, scale, causal)
        g = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                bo, bl = brute_attention(q[b, h].tolist(), k[b, h // g].tolist(),
                                         v[b, h // g].tolist(), scale, causal)
                assert np.allclose(o[b, h], np.array(bo), rtol=1e-13, atol=1e-14), (B, Hq, Hkv, Tq, Tk, d, causal)
                bl = np.array(bl)
                fin = np.isfinite(bl)
                assert np.array_equal(np.isfinite(lse[b, h]), fin)
                assert np.allclose(lse[b, h][fin], bl[fin], rtol=1e-13, atol=1e-14)


def pin_closed_forms(fwd):
    rng = np.random.Generator(np.random.PCG64(77))
    B, H, T, d = 2, 3, 37, 8
    v = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H, T, d))
    q0 = np.zeros((B, H, T, d))
    # zero queries: every visible key has weight 1/count
    o, lse = fwd(q0, k, v, 0.3, False)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-13)
    assert np.allclose(lse, math.log(T), atol=1e-13)
    o, lse = fwd(q0, k, v, 0.3, True)
    counts = np.arange(1, T + 1)
    assert np.allclose(o, np.cumsum(v, axis=2) / counts[:, None], atol=1e-13)
    assert np.allclose(lse, np.log(counts), atol=1e-13)
    # Tq < Tk with causal: query i sees keys 0 .. i + Tk - Tq
    Tq = 5
    o, lse = fwd(q0[:, :, :Tq], k, v, 0.3, True)
    vis = np.arange(Tq) + (T - Tq) + 1
    assert np.allclose(o, np.cumsum(v, axis=2)[:, :, T - Tq:] / vis[:, None], atol=1e-13)
    assert np.allclose(lse, np.log(vis), atol=1e-13)
    # constant values pass through unchanged
    q = rng.standard_normal((B, H, T, d))
    c = np.full_like(v, -2.5)
    for causal in (False, True):
        o, _ = fwd(q, k, c, 0.3, causal)
        assert np.allclose(o, -2.5, atol=1e-13)
    # causal row 0 sees only key 0
    o, lse = fwd(q, k, v, 0.3, True)
    assert np.allclose(o[:, :, 0], v[:, :, 0], atol=1e-14)
    assert np.allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-13)
    # a joint permutation of keys and values changes nothing (non-causal)
    perm = rng.permutation(T)
    o1, l1 = fwd(q, k, v, 0.3, False)
    o2, l2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)
    # empty rows: causal with Tq > Tk leaves the first Tq - Tk queries with no key
    o, lse = fwd(q[:, :, :4], k[:, :, :2], v[:, :, :2], 0.3, True)
    assert np.all(o[:, :, :2] == 0) and np.all(np.isneginf(lse[:, :, :2]))
    assert np.allclose(o[:, :, 2], v[:, :, 0], atol=1e-14)


ALL_FWD_PINS = (pin_worked_rows, pin_brute_force, pin_closed_forms)
