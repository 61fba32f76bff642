"""Pins for the oracle's sliding-window reading (a causal band of W keys ending
at each query's own position, bottom-right aligned; in decoding the last W
cached keys). The pages name sliding windows without defining them
(aimlrounds "FlashAttention", section "In practice"), so the band is pinned
to facts that do not restate it: a window as long as the sequence is the
already-pinned causal mask, a window of one key returns that key's value,
zero queries average the values inside the band, the gradients match finite
differences, and decode equals the forward on the last W keys."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import attention_ref as ref


def _rand(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("Tq,Tk", [(9, 9), (5, 9), (9, 6)])
def test_window_covering_everything_is_causal(Tq, Tk):
    q, k, v = _rand(1, 2, 4, Tq, 5), _rand(2, 2, 2, Tk, 5), _rand(3, 2, 2, Tk, 5)
    o0, l0 = ref.attention_fwd(q, k, v, 0.7, True)
    for w in (Tk + max(0, Tq - Tk), Tk + Tq, 10 ** 6):
        o1, l1 = ref.attention_fwd(q, k, v, 0.7, True, window=w)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("Tq,Tk", [(7, 7), (4, 7), (7, 4)])
def test_window_of_one_returns_the_diagonal_value(Tq, Tk):
    q, k, v = _rand(4, 1, 2, Tq, 3), _rand(5, 1, 1, Tk, 3), _rand(6, 1, 1, Tk, 3)
    o, lse = ref.attention_fwd(q, k, v, 0.5, True, window=1)
    for i in range(Tq):
        j = i + (Tk - Tq)
        for h in range(2):
            if j < 0:   # no key at all: the empty-row reading
                assert np.all(o[0, h, i] == 0) and lse[0, h, i] == -np.inf
            else:
                assert np.allclose(o[0, h, i], v[0, 0, j], atol=1e-15)
                assert math.isclose(lse[0, h, i], 0.5 * float(q[0, h, i] @ k[0, 0, j]), rel_tol=1e-14, abs_tol=1e-15)


@pytest.mark.parametrize("w", [1, 2, 3, 5])
def test_zero_queries_average_the_band(w):
    Tq, Tk = 6, 8
    q = np.zeros((1, 1, Tq, 4))
    k, v = _rand(7, 1, 1, Tk, 4), _rand(8, 1, 1, Tk, 4)
    o, lse = ref.attention_fwd(q, k, v, 1.0, True, window=w)
    for i in range(Tq):
        hi = i + (Tk - Tq)
        lo = max(0, hi - w + 1)
        n = hi - lo + 1
        assert np.allclose(o[0, 0, i], v[0, 0, lo:hi + 1].mean(axis=0), atol=1e-15)
        assert math.isclose(lse[0, 0, i], math.log(n), rel_tol=1e-14, abs_tol=1e-15)


def _loss(q, k, v, do, w):
    o, _ = ref.attention_fwd(q, k, v, 0.8, True, window=w)
    return float(np.sum(o * do))


@pytest.mark.parametrize("w", [1, 2, 4])
@pytest.mark.parametrize("dims", [(1, 2, 1, 6, 6, 2), (1, 2, 2, 4, 7, 2)])
def test_window_backward_finite_differences(w, dims):
    B, Hq, Hkv, Tq, Tk, d = dims
    q, k, v = _rand(9 + w, B, Hq, Tq, d), _rand(10 + w, B, Hkv, Tk, d), _rand(11 + w, B, Hkv, Tk, d)
    do = _rand(12 + w, B, Hq, Tq, d)
    dq, dk, dv = ref.attention_bwd(q, k, v, do, 0.8, True, window=w)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, w)
            x[idx] = old - h
            lm = _loss(q, k, v, do, w)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(g, num, rtol=1e-7, atol=1e-8), np.max(np.abs(g - num))


def test_window_sampled_backward_matches_full():
    q, k, v, do = _rand(20, 1, 4, 33, 5), _rand(21, 1, 2, 40, 5), _rand(22, 1, 2, 40, 5), _rand(23, 1, 4, 33, 5)
    for w in (1, 6, 17):
        dq, dk, dv = ref.attention_bwd(q, k, v, do, 0.6, True, window=w)
        rows = np.array([32, 0, 9])
        assert np.allclose(ref.attention_bwd_dq_rows(q, k, v, do, 0.6, True, 0, 3, rows, window=w), dq[0, 3, rows], atol=1e-14)
        keys = np.array([39, 2, 20, 7])
        dk_s, dv_s = ref.attention_bwd_dkdv_keys(q, k, v, do, 0.6, True, 0, 1, keys, window=w)
        assert np.allclose(dk_s, dk[0, 1, keys], atol=1e-13) and np.allclose(dv_s, dv[0, 1, keys], atol=1e-13)


def test_window_decode_is_the_forward_over_the_last_keys():
    B, Hq, Hkv, Tmax, d = 3, 4, 2, 30, 6
    q, kc, vc = _rand(30, B, Hq, d), _rand(31, B, Hkv, Tmax, d), _rand(32, B, Hkv, Tmax, d)
    lens = np.array([30, 1, 17])
    for w in (1, 5, 17, 40):
        o, lse = ref.decode(q, kc, vc, lens, 0.4, window=w)
        for b in range(B):
            L = int(lens[b])
            lo = max(0, L - w)
            of, lf = ref.attention_fwd(q[b][None, :, None, :], kc[b:b + 1, :, lo:L], vc[b:b + 1, :, lo:L], 0.4, False)
            assert np.allclose(o[b], of[0, :, 0], atol=1e-14) and np.allclose(lse[b], lf[0, :, 0], atol=1e-14)
            # the same as the causal forward of the query at position L - 1 with the window
            qq = np.zeros((1, Hq, L, d))
            qq[0, :, L - 1] = q[b]
            oc, lc = ref.attention_fwd(qq, kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], 0.4, True, rows=[L - 1], window=w)
            assert np.allclose(o[b], oc[0, :, 0], atol=1e-14) and np.allclose(lse[b], lc[0, :, 0], atol=1e-14)
