"""CPU pins for the fp64 oracle and the online-softmax model (no GPU).

Every check here compares the oracle with something other than itself: the
pages' printed worked rows, brute force, closed forms, finite differences, or
the independent tiled recurrence model.
"""
import math

import numpy as np
import pytest

from oracle import attention_ref as ref
from oracle import online_model as om
from tests import oracle_pins as pins


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("pin", pins.ALL_FWD_PINS, ids=lambda f: f.__name__)
def test_forward_pins(pin):
    pin(ref.attention_fwd)


def test_probabilities_sum_to_one():
    rng = np.random.Generator(np.random.PCG64(3))
    q = rng.standard_normal((9, 5))
    k = rng.standard_normal((12, 5))
    for causal in (False, True):
        p, _ = ref.row_probs(q, k, 0.5, np.arange(9), 9, causal)
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
        if causal:
            # bottom-right aligned: row i sees keys 0 .. i + 3
            assert np.all(np.triu(p, k=4) == 0)
            assert np.all(p[np.tril(np.ones_like(p, dtype=bool), k=3)] > 0)


def test_causal_rule_position_three():
    """A query at position 3 (Tq = Tk) uses keys 0..3 and ignores 4 and later
    (kgptalkie page, section 'Causal Masks Still Apply')."""
    vis = ref.visible(np.array([3]), 8, 8, True)[0]
    assert vis.tolist() == [True] * 4 + [False] * 4


def test_sampled_rows_equal_full():
    rng = np.random.Generator(np.random.PCG64(4))
    q = rng.standard_normal((1, 2, 40, 6))
    k = rng.standard_normal((1, 1, 40, 6))
    v = rng.standard_normal((1, 1, 40, 6))
    o, lse = ref.attention_fwd(q, k, v, 0.4, True)
    rows = np.array([0, 7, 39, 13])
    o2, lse2 = ref.attention_fwd(q, k, v, 0.4, True, rows=rows)
    assert np.array_equal(o2, o[:, :, rows]) and np.array_equal(lse2, lse[:, :, rows])


# ------------------------------------------------------- online recurrence pins

def test_online_four_key_row_printed_state():
    g = pins.load_worked_rows()["four_key_row"]
    hist = om.row_tiles(g["scores"], g["values"], g["tile"])
    a = g["after_tile_1"]
    half = 0.5 * 10 ** -a["printed_decimals"]
    assert hist[0].m == a["m"]
    assert abs(hist[0].l - a["l"]) <= half
    assert abs(hist[0].u[0] - a["u"]) <= half
    l2, u2 = pins.closed_form_four_key()
    assert hist[1].m == g["after_tile_2"]["m"]
    assert math.isclose(hist[1].l, l2, rel_tol=1e-15)
    assert math.isclose(hist[1].u[0], u2, rel_tol=1e-15)
    # the page's equality check between the tiled and whole-row results
    s = np.array(g["scores"])
    w = np.exp(s - s.max())
    whole = float(w @ np.array(g["values"]) / w.sum())
    assert math.isclose(hist[1].u[0] / hist[1].l, whole, rel_tol=g["check_rel_tol"])


def test_online_eight_key_row_printed_outputs():
    g = pins.load_worked_rows()["eight_key_row"]
    tol = 0.5 * 10 ** -g["printed_decimals"]
    hist = om.row_tiles(g["scores"], g["values"], g["tile"])
    assert hist[0].m == g["tile_1_max"] and hist[1].m == g["final_max"]
    assert abs(hist[0].u[0] / hist[0].l - g["output_after_tile_1"]) <= tol
    assert abs(hist[1].u[0] / hist[1].l - g["final_output"]) <= tol
    finals = [om.row_tiles(g["scores"], g["values"], t)[-1] for t in range(1, 9)]
    for f in finals:
        assert math.isclose(f.u[0] / f.l, finals[-1].u[0] / finals[-1].l, rel_tol=1e-13)
    # merging the two tile partials (split-KV style) gives the same final row
    parts = [om.row_tiles(g["scores"][:4], g["values"][:4], 4)[-1],
             om.row_tiles(g["scores"][4:], g["values"][4:], 4)[-1]]
    merged = om.merge(parts)
    assert abs(merged.output()[0] - g["final_output"]) <= tol
    assert math.isclose(merged.output()[0], finals[-1].u[0] / finals[-1].l, rel_tol=1e-13)


def test_online_rescale_applies_to_both_sums():
    """Rescaling only the normaliser (and not the numerator) must change the
    answer: the check that makes the recurrence test meaningful."""
    g = pins.load_worked_rows()["eight_key_row"]
    s, v = np.array(g["scores"]), np.array(g["values"])
    m1 = s[:4].max()
    l1, u1 = np.exp(s[:4] - m1).sum(), np.exp(s[:4] - m1) @ v[:4]
    m2 = max(m1, s[4:].max())
    l_ok = math.exp(m1 - m2) * l1 + np.exp(s[4:] - m2).sum()
    u_ok = math.exp(m1 - m2) * u1 + np.exp(s[4:] - m2) @ v[4:]
    u_bad = u1 + np.exp(s[4:] - m2) @ v[4:]
    assert abs(u_ok / l_ok - g["final_output"]) <= 0.005
    assert abs(u_bad / l_ok - g["final_output"]) > 1.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(17, 17), (9, 23), (23, 9), (1, 30)])
def test_tile_size_invariance(causal, shape):
    """The recurrence at any tile size equals the three-step oracle
    (aimlrounds page: the result does not depend on the tile size, up to rounding)."""
    Tq, Tk = shape
    rng = np.random.Generator(np.random.PCG64(Tq * 100 + Tk))
    q = rng.standard_normal((Tq, 5)) * 2.0
    k = rng.standard_normal((Tk, 5))
    v = rng.standard_normal((Tk, 5))
    o_ref, lse_ref = ref.attention_fwd(q[None, None], k[None, None], v[None, None], 0.8, causal)
    for tile in (1, 2, 3, 5, 7, 16, 64, Tk):
        o, lse = om.attention_online(q, k, v, 0.8, causal, tile)
        assert np.allclose(o, o_ref[0, 0], rtol=1e-12, atol=1e-13), tile
        fin = np.isfinite(lse_ref[0, 0])
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.allclose(lse[fin], lse_ref[0, 0][fin], rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------------- backward

def _loss(q, k, v, do, scale, causal):
    o, _ = ref.attention_fwd(q, k, v, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(1, 1, 1, 5, 5, 3), (1, 2, 1, 4, 6, 2), (2, 2, 2, 6, 3, 3), (1, 4, 2, 3, 3, 2)])
def test_backward_finite_differences(causal, dims):
    B, Hq, Hkv, Tq, Tk, d = dims
    rng = np.random.Generator(np.random.PCG64(sum(dims) * 7 + causal))
    q = rng.standard_normal((B, Hq, Tq, d))
    k = rng.standard_normal((B, Hkv, Tk, d))
    v = rng.standard_normal((B, Hkv, Tk, d))
    do = rng.standard_normal((B, Hq, Tq, d))
    scale = 0.9
    dq, dk, dv = ref.attention_bwd(q, k, v, do, scale, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(g, num, rtol=1e-7, atol=1e-8), np.max(np.abs(g - num))


def test_backward_dq_rows_match_full():
    rng = np.random.Generator(np.random.PCG64(11))
    q = rng.standard_normal((1, 4, 30, 5))
    k = rng.standard_normal((1, 2, 30, 5))
    v = rng.standard_normal((1, 2, 30, 5))
    do = rng.standard_normal((1, 4, 30, 5))
    dq, _, _ = ref.attention_bwd(q, k, v, do, 0.6, True)
    rows = np.array([29, 0, 5])
    dq_r = ref.attention_bwd_dq_rows(q, k, v, do, 0.6, True, 0, 3, rows)
    assert np.allclose(dq_r, dq[0, 3, rows], atol=1e-14)


def test_backward_sampled_keys_match_full():
    rng = np.random.Generator(np.random.PCG64(15))
    q = rng.standard_normal((2, 4, 37, 5))
    k = rng.standard_normal((2, 2, 41, 5))
    v = rng.standard_normal((2, 2, 41, 5))
    do = rng.standard_normal((2, 4, 37, 5))
    for causal in (False, True):
        _, dk, dv = ref.attention_bwd(q, k, v, do, 0.6, causal)
        keys = np.array([40, 3, 22])
        dk_s, dv_s = ref.attention_bwd_dkdv_keys(q, k, v, do, 0.6, causal, 1, 1, keys)
        assert np.allclose(dk_s, dk[1, 1, keys], atol=1e-13)
        assert np.allclose(dv_s, dv[1, 1, keys], atol=1e-13)


def test_backward_sum_identities():
    """sum_j dV_j equals the summed dO of the group (rows of P sum to one) and
    sum_j dK_j is zero (each row of dS sums to zero)."""
    rng = np.random.Generator(np.random.PCG64(12))
    q = rng.standard_normal((2, 4, 20, 6))
    k = rng.standard_normal((2, 2, 20, 6))
    v = rng.standard_normal((2, 2, 20, 6))
    do = rng.standard_normal((2, 4, 20, 6))
    for causal in (False, True):
        _, dk, dv = ref.attention_bwd(q, k, v, do, 0.6, causal)
        grp = do.reshape(2, 2, 2, 20, 6).sum(axis=(2, 3))
        assert np.allclose(dv.sum(axis=2), grp, atol=1e-12)
        assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)


# ------------------------------------------------------------------------ GQA

def test_gqa_equals_expanded_mha():
    rng = np.random.Generator(np.random.PCG64(13))
    B, Hq, Hkv, T, d = 2, 8, 2, 11, 4
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    do = rng.standard_normal((B, Hq, T, d))
    ke, ve = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    for causal in (False, True):
        o1, l1 = ref.attention_fwd(q, k, v, 0.5, causal)
        o2, l2 = ref.attention_fwd(q, ke, ve, 0.5, causal)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        dq1, dk1, dv1 = ref.attention_bwd(q, k, v, do, 0.5, causal)
        dq2, dk2, dv2 = ref.attention_bwd(q, ke, ve, do, 0.5, causal)
        assert np.allclose(dq1, dq2, atol=1e-14)
        assert np.allclose(dk1, dk2.reshape(B, Hkv, Hq // Hkv, T, d).sum(axis=2), atol=1e-13)
        assert np.allclose(dv1, dv2.reshape(B, Hkv, Hq // Hkv, T, d).sum(axis=2), atol=1e-13)


# --------------------------------------------------------------------- decode

def test_decode_matches_forward_and_split_merge():
    rng = np.random.Generator(np.random.PCG64(14))
    B, Hq, Hkv, Tmax, d = 3, 4, 2, 50, 8
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, Hkv, Tmax, d))
    vc = rng.standard_normal((B, Hkv, Tmax, d))
    lens = np.array([50, 1, 23])
    o, lse = ref.decode(q, kc, vc, lens, 0.35)
    for b in range(B):
        L = lens[b]
        of, lf = ref.attention_fwd(q[b][None, :, None, :], kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], 0.35, False)
        assert np.allclose(o[b], of[0, :, 0], atol=1e-14) and np.allclose(lse[b], lf[0, :, 0], atol=1e-14)
        # any split of the keys into chunks, merged with the rescale rule, agrees
        for chunk in (1, 7, 16, 64):
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                s = 0.35 * (kc[b, hk, :L] @ q[b, h])
                parts = [om.row_tiles(s[c:c + chunk], vc[b, hk, c:min(L, c + chunk)], chunk)[-1]
                         for c in range(0, L, chunk)]
                m = om.merge(parts)
                assert np.allclose(m.output(), o[b, h], atol=1e-13)
                assert math.isclose(m.lse(), lse[b, h], rel_tol=1e-13, abs_tol=1e-13)
    # a poisoned cache tail beyond the length is never used
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[2, :, 23:] = np.nan
    vc2[2, :, 23:] = np.nan
    o2, _ = ref.decode(q, kc2, vc2, lens, 0.35)
    assert np.array_equal(o2[2], o[2])
