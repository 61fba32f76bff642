"""Pins of the oracle's dropout: the Philox generator and the dropped forward and backward.

Sources of truth outside the oracle:
  * numpy's own Philox bit generator (Philox-4x64-10) for the round structure
    and key schedule of the scalar generator;
  * the published Philox-4x32-10 known-answer vectors (tests/golden/);
  * the random-number contract evaluated element by element in pure Python;
  * closed forms and invariants: t = 256 is no dropout; the mean over seeds
    is the undropped output (inverted dropout is unbiased); the keep fraction
    is t / 256 within binomial bounds;
  * central finite differences of L = sum(O * dO) with the mask held fixed.

Mutants at the end plant plausible mistakes in copies of the oracle and show
that these pins reject each one.
"""
from __future__ import annotations

import inspect
import json
import math
import os
import sys
import types

import numpy as np
import pytest

from oracle import attention_ref as ref
from oracle.philox import philox4x32_10, philox_ref
from tests import oracle_pins as pins

KAT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.json")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------ Philox


@pytest.mark.parametrize("key,counter", [((5, 7), (0, 0, 0, 0)), ((0, 0), (41, 3, 0, 9)),
                                          ((2**64 - 1, 12345), (2**64 - 3, 2**63, 1, 0))])
def test_philox64_matches_numpy_bit_generator(key, counter):
    # numpy's generator adds one to the counter before each block of four outputs
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(8)]
    c = list(counter)
    for blk in range(2):
        c[0] = (c[0] + 1) % 2**64
        carry = c[0] == 0
        for w in range(1, 4):   # carry into the higher words
            if not carry:
                break
            c[w] = (c[w] + 1) % 2**64
            carry = c[w] == 0
        assert list(philox_ref(c, key, width=64, rounds=10)) == raw[4 * blk:4 * blk + 4]


def test_philox32_known_answer_vectors():
    with open(KAT) as f:
        vecs = json.load(f)["vectors"]
    for v in vecs:
        ctr = [int(x, 16) for x in v["counter"]]
        key = [int(x, 16) for x in v["key"]]
        want = [int(x, 16) for x in v["out"]]
        assert list(philox_ref(ctr, key, width=32, rounds=10)) == want
        got = philox4x32_10(*ctr, *key)
        assert [int(x) for x in got] == want


def test_philox32_vectorised_matches_scalar():
    rng = np.random.default_rng(11)
    ctr = rng.integers(0, 2**32, size=(4, 300), dtype=np.uint64)
    ctr[:, :3] = 2**32 - 1
    for key in ((0, 0), (0xDEADBEEF, 0x01234567), (2**32 - 1, 1)):
        got = philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], *key)
        for n in range(ctr.shape[1]):
            assert tuple(int(g[n]) for g in got) == philox_ref(ctr[:, n], key, 32, 10)


# ---------------------------------------------------------------- the mask


def _brute_keep(drop, bh: int, i: int, j: int) -> bool:
    """The contract, one element at a time in Python integers."""
    w = philox_ref((j // 16, i, bh, drop.offset), (drop.seed % 2**32, drop.seed // 2**32), 32, 10)
    byte = (w[(j % 16) // 4] >> (8 * (j % 4))) & 0xFF
    return byte < drop.t


@pytest.mark.parametrize("Tk", [5, 16, 37])
def test_keep_mask_matches_the_contract_element_by_element(Tk, m=ref):
    drop = m.Dropout(t=128, seed=0x0123456789ABCDEF, offset=7)
    rows = np.array([0, 1, 5, 33])
    for bh in (0, 3):
        z = m.dropout_keep(drop, bh, rows, Tk)
        for a, i in enumerate(rows):
            for j in range(Tk):
                assert z[a, j] == _brute_keep(drop, bh, int(i), j), (bh, i, j)


def test_keep_fraction_is_t_over_256(m=ref):
    for t in (230, 128, 13):
        drop = m.Dropout(t=t, seed=99, offset=0)
        z = m.dropout_keep(drop, 2, np.arange(200), 512)
        n, frac = z.size, z.mean()
        kappa = t / 256
        assert abs(frac - kappa) <= 5 * math.sqrt(kappa * (1 - kappa) / n), (t, frac)


def test_streams_differ_by_seed_offset_and_head():
    base = ref.dropout_keep(ref.Dropout(128, 1, 0), 0, np.arange(8), 64)
    for other in (ref.dropout_keep(ref.Dropout(128, 2, 0), 0, np.arange(8), 64),
                  ref.dropout_keep(ref.Dropout(128, 1, 1), 0, np.arange(8), 64),
                  ref.dropout_keep(ref.Dropout(128, 1, 0), 1, np.arange(8), 64)):
        assert (base != other).mean() > 0.3


@pytest.mark.parametrize("p,t", [(0.0, 256), (0.1, 230), (0.5, 128), (0.25, 192), (0.998, 1)])
def test_keep_threshold(p, t):
    assert ref.keep_threshold(p) == t


@pytest.mark.parametrize("p", [1.0, -0.1, 0.999, float("nan")])
def test_keep_threshold_rejects(p):
    with pytest.raises(ValueError):
        ref.keep_threshold(p)


# ------------------------------------------------------- forward / backward


def test_threshold_256_is_no_dropout():
    q, k, v, do = _rand(1, 2, 4, 24, 8), _rand(2, 2, 2, 24, 8), _rand(3, 2, 2, 24, 8), _rand(4, 2, 4, 24, 8)
    drop = ref.Dropout(t=256, seed=5)
    for causal in (False, True):
        o0, l0 = ref.attention_fwd(q, k, v, 0.3, causal)
        o1, l1 = ref.attention_fwd(q, k, v, 0.3, causal, dropout=drop)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
        for a, b in zip(ref.attention_bwd(q, k, v, do, 0.3, causal), ref.attention_bwd(q, k, v, do, 0.3, causal, dropout=drop)):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_dropped_forward_matches_brute_force(causal, m=ref):
    Tq, Tk, d, scale = 5, 7, 3, 0.7
    q, k, v = _rand(5, 1, 2, Tq, d), _rand(6, 1, 1, Tk, d), _rand(7, 1, 1, Tk, d)
    drop = m.Dropout(t=128, seed=77, offset=3)
    o, lse = m.attention_fwd(q, k, v, scale, causal, dropout=drop)
    n_dropped = 0
    for h in range(2):
        bo, blse = pins.brute_attention(q[0, h].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, causal)
        # brute-force probabilities: O without dropout is sum_j P_ij V_j; rebuild P from the definition
        for i in range(Tq):
            terms = [math.exp(scale * sum(q[0, h, i, c] * k[0, 0, j, c] for c in range(d)))
                     if (not causal or j <= i + Tk - Tq) else 0.0 for j in range(Tk)]
            tot = math.fsum(terms)
            for c in range(d):
                acc = []
                for j in range(Tk):
                    if _brute_keep(drop, h, i, j):
                        acc.append(terms[j] / tot * v[0, 0, j, c] / drop.kappa)
                    else:
                        n_dropped += terms[j] > 0
                assert o[0, h, i, c] == pytest.approx(math.fsum(acc), rel=1e-12, abs=1e-12)
            assert lse[0, h, i] == pytest.approx(blse[i], rel=1e-13)
    assert n_dropped > 0


def test_dropout_is_unbiased_over_seeds(m=ref):
    q, k, v = _rand(8, 1, 1, 16, 4), _rand(9, 1, 1, 16, 4), _rand(10, 1, 1, 16, 4)
    o_plain, _ = m.attention_fwd(q, k, v, 0.5, False)
    outs = np.stack([m.attention_fwd(q, k, v, 0.5, False, dropout=m.Dropout(128, s))[0] for s in range(400)])
    mean, se = outs.mean(axis=0), outs.std(axis=0, ddof=1) / math.sqrt(outs.shape[0])
    assert np.all(np.abs(mean - o_plain) <= 6 * se + 1e-12)
    # an unscaled mask would average to kappa * O: make sure the check can tell
    assert np.max(np.abs(0.5 * o_plain - o_plain) / (se + 1e-30)) > 6


def _loss(q, k, v, do, causal, drop, m):
    o, _ = m.attention_fwd(q, k, v, 0.8, causal, dropout=drop)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1)])
def test_dropped_backward_finite_differences(causal, Hq, Hkv, m=ref):
    T, d, h = 6, 3, 1e-6
    q, k, v, do = _rand(11, 1, Hq, T, d), _rand(12, 1, Hkv, T, d), _rand(13, 1, Hkv, T, d), _rand(14, 1, Hq, T, d)
    drop = m.Dropout(t=128, seed=2024, offset=1)
    assert not m.dropout_keep(drop, 0, np.arange(T), T).all()
    grads = m.attention_bwd(q, k, v, do, 0.8, causal, dropout=drop)
    for x, gx in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (_loss(*args_p, do, causal, drop, m) - _loss(*args_m, do, causal, drop, m)) / (2 * h)
        np.testing.assert_allclose(gx, num, rtol=1e-6, atol=1e-8)


def test_dropped_sampled_rows_and_gradients_match_full():
    Hq, Hkv, T, d = 4, 2, 40, 8
    q, k, v, do = _rand(15, 2, Hq, T, d), _rand(16, 2, Hkv, T, d), _rand(17, 2, Hkv, T, d), _rand(18, 2, Hq, T, d)
    drop = ref.Dropout(t=230, seed=31337, offset=5)
    for causal in (False, True):
        dq, dk, dv = ref.attention_bwd(q, k, v, do, 0.4, causal, dropout=drop)
        rows = np.array([0, 17, 39])
        np.testing.assert_allclose(ref.attention_bwd_dq_rows(q, k, v, do, 0.4, causal, 1, 3, rows, dropout=drop),
                                   dq[1, 3, rows], rtol=1e-12, atol=1e-12)
        o, lse = ref.attention_fwd(q, k, v, 0.4, causal, dropout=drop)
        ho, hl = ref.attention_fwd_head_rows(q, k, v, 0.4, causal, 1, 3, rows, dropout=drop)
        np.testing.assert_allclose(ho, o[1, 3, rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hl, lse[1, 3, rows], rtol=1e-12, atol=1e-12)
        keys = np.array([2, 20, 39])
        sk, sv = ref.attention_bwd_dkdv_keys(q, k, v, do, 0.4, causal, 1, 1, keys, dropout=drop)
        np.testing.assert_allclose(sk, dk[1, 1, keys], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sv, dv[1, 1, keys], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- mutants


def _mutant(old: str, new: str) -> types.ModuleType:
    src = inspect.getsource(ref)
    assert old in src, old
    name = "oracle._dropout_mutant"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    sys.modules[name] = mod   # dataclasses look their module up by name
    try:
        exec(compile(src.replace(old, new, 1), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


MUTANTS = {
    "no 1/kappa rescale": ("z = dropout_keep(drop, bh, rows, Tk) / drop.kappa",
                           "z = dropout_keep(drop, bh, rows, Tk) * 1.0"),
    "bytes taken high to low": (">> (np.arange(4, dtype=np.uint32) * 8)",
                                ">> ((3 - np.arange(4, dtype=np.uint32)) * 8)"),
    "keep iff byte <= t": ("return bytes_ < drop.t", "return bytes_ <= drop.t"),
    "row and key group swapped in the counter": ("philox4x32_10(g[None, :], rows[:, None], bh,",
                                                 "philox4x32_10(rows[:, None], g[None, :], bh,"),
    "seed halves swapped": ("drop.seed & 0xFFFFFFFF, (drop.seed >> 32) & 0xFFFFFFFF",
                            "(drop.seed >> 32) & 0xFFFFFFFF, drop.seed & 0xFFFFFFFF"),
    "dP not dropped": ("dp = (g @ v[b, hk].T) * z", "dp = g @ v[b, hk].T"),
    "dV from undropped P": ("dv[b, hk] += pd.T @ g", "dv[b, hk] += p.T @ g"),
    "head index not in the stream": ("pd, _ = _dropped(p, dropout, b * Hq + h, r, k.shape[2])",
                                     "pd, _ = _dropped(p, dropout, b, r, k.shape[2])"),
}


def _fails_some_pin(mod) -> bool:
    checks = [lambda: test_keep_mask_matches_the_contract_element_by_element(37, m=mod),
              lambda: test_keep_fraction_is_t_over_256(m=mod),
              lambda: test_dropout_is_unbiased_over_seeds(m=mod),
              lambda: test_dropped_forward_matches_brute_force(False, m=mod),
              lambda: test_dropped_backward_finite_differences(True, 2, 1, m=mod)]
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_dropout_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert _fails_some_pin(_mutant(old, new)), name


def test_unmodified_oracle_passes_the_mutant_harness():
    assert not _fails_some_pin(_mutant("_ROW_BLOCK = 512", "_ROW_BLOCK = 512"))
