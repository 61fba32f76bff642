"""Plant plausible mistakes in copies of the oracle (on the CPU) and show that
the pins reject every one of them.

Each mutant is the oracle's own source with one textual edit, executed as a
separate module; the real oracle is never modified.
"""
import inspect
import sys
import types

import numpy as np
import pytest

from oracle import attention_ref as ref
from tests import oracle_pins as pins


def _mutant(old: str, new: str) -> types.ModuleType:
    src = inspect.getsource(ref)
    assert old in src, old
    name = "oracle._mutant"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"   # the oracle imports its Philox module relatively
    sys.modules[name] = mod      # dataclasses look their module up by name
    try:
        exec(compile(src.replace(old, new, 1), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _fails_some_forward_pin(mod) -> bool:
    for pin in pins.ALL_FWD_PINS:
        try:
            pin(mod.attention_fwd)
        except (AssertionError, ValueError, IndexError):
            return True
    return False


FWD_MUTANTS = {
    "scale dropped": ("s = scale * (q_rows @ k.T)", "s = q_rows @ k.T"),
    "keys reversed": ("s = scale * (q_rows @ k.T)", "s = scale * (q_rows @ k[::-1].T)"),
    "diagonal excluded": ("vis = j[None, :] <= last", "vis = j[None, :] < last"),
    "top-left causal alignment": ("last = rows[:, None] + (Tk - Tq)", "last = rows[:, None]"),
    "max missing from lse": ("lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))", "lse = np.where(empty, -np.inf, np.log(l_safe))"),
    "not normalised": ("p = e / l_safe[:, None]", "p = e"),
    "wrong kv head map": ("return hq // (Hq // Hkv)", "return hq % Hkv"),
    "values swapped for keys": ("o[b, h, s:s + _ROW_BLOCK] = pd @ v[b, hk]", "o[b, h, s:s + _ROW_BLOCK] = pd @ k[b, hk]"),
}


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name):
    assert _fails_some_forward_pin(_mutant(*FWD_MUTANTS[name])), name


def _fd_check(mod) -> bool:
    """True when the mutant's backward agrees with central differences of the
    (unmodified) forward on a small GQA causal case and a non-causal one."""
    for causal, dims in ((True, (1, 4, 2, 4, 5, 3)), (False, (1, 2, 2, 3, 4, 2))):
        B, Hq, Hkv, Tq, Tk, d = dims
        rng = np.random.Generator(np.random.PCG64(99))
        q = rng.standard_normal((B, Hq, Tq, d))
        k = rng.standard_normal((B, Hkv, Tk, d))
        v = rng.standard_normal((B, Hkv, Tk, d))
        do = rng.standard_normal((B, Hq, Tq, d))
        try:
            grads = mod.attention_bwd(q, k, v, do, 0.9, causal)
        except (ValueError, IndexError):
            return False
        for x, g in zip((q, k, v), grads):
            if g.shape != x.shape:
                return False
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + 1e-6
                lp = np.sum(ref.attention_fwd(q, k, v, 0.9, causal)[0] * do)
                x[idx] = old - 1e-6
                lm = np.sum(ref.attention_fwd(q, k, v, 0.9, causal)[0] * do)
                x[idx] = old
                if abs((lp - lm) / 2e-6 - g[idx]) > 1e-6 + 1e-6 * abs(g[idx]):
                    return False
    return True


BWD_MUTANTS = {
    "row term dropped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "row term sign": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    "dq scale dropped": ("dq[b, h, r] = scale * (ds @ k[b, hk])", "dq[b, h, r] = ds @ k[b, hk]"),
    "dk uses dO": ("dk[b, hk] += scale * (ds.T @ q[b, h, r])", "dk[b, hk] += scale * (ds.T @ g)"),
    "dv overwritten per group": ("dv[b, hk] += pd.T @ g", "dv[b, hk] = pd.T @ g"),
    "dp not transposed": ("dp = (g @ v[b, hk].T) * z", "dp = (g @ v[b, hk][::-1].T) * z"),
}


def test_unmutated_backward_passes_fd():
    assert _fd_check(ref)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    assert not _fd_check(_mutant(*BWD_MUTANTS[name])), name


# A sliding-window mistake must fail the window pins (tests/test_oracle_window.py).
WINDOW_MUTANTS = {
    "window one key too wide": ("vis &= j[None, :] > last - window", "vis &= j[None, :] >= last - window"),
    "window one key too narrow": ("vis &= j[None, :] > last - window", "vis &= j[None, :] > last - window + 1"),
    "window ignored": ("vis &= j[None, :] > last - window", "pass"),
    "decode window from the front": ("lo = max(0, L - window) if window > 0 else 0", "lo = 0"),
}


@pytest.mark.parametrize("name", sorted(WINDOW_MUTANTS))
def test_window_mutant_is_caught(name, monkeypatch):
    from tests import test_oracle_window as tw
    mod = _mutant(*WINDOW_MUTANTS[name])
    monkeypatch.setattr(tw, "ref", mod)
    checks = [lambda: tw.test_window_of_one_returns_the_diagonal_value(7, 7),
              lambda: tw.test_window_of_one_returns_the_diagonal_value(4, 7),
              lambda: tw.test_zero_queries_average_the_band(3),
              lambda: tw.test_window_decode_is_the_forward_over_the_last_keys()]
    failed = False
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed = True
            break
    assert failed, name


FP8_MUTANTS = {
    "exponent bias 8": ("np.exp2((e - 7).astype(np.float64))", "np.exp2((e - 8).astype(np.float64))"),
    "subnormals as normals": ("np.where(e == 0, (f / 8.0) * 2.0 ** -6,", "np.where(e < 0, (f / 8.0) * 2.0 ** -6,"),
    "subnormal step 2^-7": ("(f / 8.0) * 2.0 ** -6", "(f / 8.0) * 2.0 ** -7"),
    "S.1111.111 not NaN": ("mag = np.where((e == 15) & (f == 7), np.nan, mag)", "pass"),
    "V not transposed back": ("v = np.swapaxes(e4m3_to_f64(vt8), 2, 3)", "v = e4m3_to_f64(vt8).reshape(np.swapaxes(vt8, 2, 3).shape)"),
    "q factor ignored": ("q = e4m3_to_f64(q8) * np.asarray(q_scale", "q = e4m3_to_f64(q8) * 0 + e4m3_to_f64(q8) * np.ones_like(q_scale"),
    "v factor ignored": ("np.swapaxes(e4m3_to_f64(vt8), 2, 3) * np.asarray(v_scale", "np.swapaxes(e4m3_to_f64(vt8), 2, 3) * np.ones_like(v_scale"),
    "k factor from the query heads": ("k = e4m3_to_f64(k8) * np.asarray(k_scale, dtype=np.float64)[:, :, None, None]",
                                       "k = e4m3_to_f64(k8) * np.asarray(k_scale, dtype=np.float64)[:, ::-1, None, None]"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    from tests import test_oracle_fp8 as tf
    mod = _mutant(*FP8_MUTANTS[name])
    monkeypatch.setattr(tf, "ref", mod)
    checks = [tf.test_e4m3_fixed_points, tf.test_e4m3_nan_codes_and_ordering,
              tf.test_zero_queries_average_the_values_and_v_is_transposed,
              tf.test_two_keys_closed_form_with_factors, tf.test_factors_stay_with_their_heads]
    failed = False
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed = True
            break
    assert failed, name
