"""Helpers for the GPU parity tests: moving seeded inputs to the device and
the tolerance rules the HIP path must meet against the fp64 oracle.

Tolerances (written here, used by every GPU test):
  * fp32 path: max |x - ref| <= 1e-5, taken relative to max(1, |ref|) so that
    the pages' worked rows (|O| ~ 62) get the same ~2-3 fp32 ulps;
  * bf16 path: max |x - ref| / max(1, |ref|) <= 2e-2 and
    ||x - ref||_2 / ||ref||_2 <= 1e-2 for every output tensor. The relative
    L2 term keeps the check meaningful when |O| ~ sqrt(e/T) is small; the
    max(1, |ref|) divisor only matters for outputs above 1 in magnitude, where
    storing the exact answer in bf16 alone can miss by more than 2e-2;
  * LSE: max |x - ref| <= 1e-4 (bf16 inputs), <= 1e-5 (fp32 inputs).
"""
from __future__ import annotations

import numpy as np
import torch

from io_aware_softmax_05_amd import inputs
from oracle import attention_ref as ref


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def report(name: str, got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: non-finite pattern differs"
    diff = np.where(fin, got - np.where(fin, ref, 0), 0.0)
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(np.where(fin, ref, 0)))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else max_abs
    refv = np.where(fin, ref, 0.0)
    floor = float(np.max(np.abs(inputs.bf16_bits_to_f32(inputs.bf16_bits_from_f32(refv.astype(np.float32)))
                                - refv))) if refv.size else 0.0
    print(f"  {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} max|ref|={float(np.max(np.abs(refv), initial=0)):.3e} "
          f"bf16_floor={floor:.3e}", flush=True)
    return max_abs, rel


def check_bf16(name: str, got, ref) -> None:
    got = host(got) if isinstance(got, torch.Tensor) else got
    max_abs, rel = report(name, got, ref)
    fin = np.isfinite(ref)
    refv = np.where(fin, ref, 0.0)
    scaled = float(np.max(np.abs(np.where(fin, got, 0.0) - refv) / np.maximum(1.0, np.abs(refv)), initial=0.0))
    assert scaled <= 2e-2 and rel <= 1e-2, f"{name}: max_abs={max_abs:.3e} (scaled {scaled:.3e}) rel={rel:.3e}"


def storage_allowance(hv, scale, causal, dropout=None):
    """First-order error that bf16 storage of O, P and dS can cause, per
    output element (unit roundoff u = 2^-8).

    D_i = sum_c dO_ic O_ic is formed from the stored bf16 O, so it may be off
    by dD_i = u sum_c |dO_ic O_ic|; dS_ij = P_ij (dP_ij - D_i) inherits
    P_ij dD_i, which matters when a row is dominated by one key (dP_ij and D_i
    then nearly cancel). P and dS are also rounded to bf16 before their
    matrix products. With dropout, O and dP carry the keep mask scaled by
    1 / kappa (the oracle's mask), and O is no longer a copy of a stored V
    row even where one key holds all the weight, so the cancellation shows
    up in ordinary causal rows (row 0 sees one key)."""
    u = 2.0 ** -8
    q, k, v, do = hv["q"], hv["k"], hv["v"], hv["do"]
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    o, _ = ref.attention_fwd(q, k, v, scale, causal, dropout=dropout)
    dD = u * np.sum(np.abs(do * o), axis=-1)
    a_dq, a_dk, a_dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            p, _ = ref.row_probs(q[b, h], k[b, hk], scale, np.arange(Tq), Tq, causal)
            z = 1.0 if dropout is None else ref.dropout_keep(dropout, b * Hq + h, np.arange(Tq), Tk) / dropout.kappa
            dp = (do[b, h] @ v[b, hk].T) * z
            ds = np.abs(p * (dp - (p * dp).sum(axis=1, keepdims=True)))
            a_dq[b, h] = scale * (dD[b, h][:, None] * (p @ np.abs(k[b, hk])) + u * ds @ np.abs(k[b, hk]))
            a_dk[b, hk] += scale * (p.T @ (dD[b, h][:, None] * np.abs(q[b, h])) + u * ds.T @ np.abs(q[b, h]))
            a_dv[b, hk] += u * (p * z).T @ np.abs(do[b, h])
    return a_dq, a_dk, a_dv


def check_with_allowance(name, got, want, allow):
    """The bf16 rule of check_bf16 with a per-element allowance added to its max-abs term."""
    got = host(got) if isinstance(got, torch.Tensor) else got
    _, rel = report(name, got, want)
    excess = np.abs(got - want) - (2e-2 * np.maximum(1.0, np.abs(want)) + allow)
    print(f"    worst excess over allowance {float(excess.max()):.3e}", flush=True)
    assert float(excess.max()) <= 0.0 and rel <= 1e-2, name


def check_f32(name: str, got, ref) -> None:
    got = host(got) if isinstance(got, torch.Tensor) else got
    report(name, got, ref)
    fin = np.isfinite(ref)
    err = np.abs(np.where(fin, got - np.where(fin, ref, 0), 0.0)) / np.maximum(1.0, np.abs(np.where(fin, ref, 0)))
    assert float(err.max(initial=0.0)) <= 1e-5, f"{name}: scaled max err {float(err.max()):.3e}"


def check_lse(name: str, got, ref, tol: float) -> None:
    got = host(got) if isinstance(got, torch.Tensor) else got
    max_abs, _ = report(name, got, ref)
    assert max_abs <= tol, f"{name}: max_abs={max_abs:.3e} > {tol}"


def attention_case(seed, B, Hq, Hkv, Tq, Tk, d, dtype="bf16", with_dout=False, q_gain=1.0):
    """Seeded inputs (numpy, exact values) and their device copies."""
    x = inputs.draw_attention_inputs(seed, B, Hq, Hkv, Tq, Tk, d, dtype, with_dout)
    if q_gain != 1.0:
        qv = inputs.widen(x["q"]) * q_gain     # exact: a power-of-two gain keeps bf16 values exact
        x["q"] = inputs.bf16_bits_from_f32(qv.astype(np.float32)) if dtype == "bf16" else qv.astype(np.float32)
    host_vals = {n: inputs.widen(a) for n, a in x.items()}
    to_dev = dev_bf16 if dtype == "bf16" else dev_f32
    dev = {n: to_dev(a) for n, a in x.items()}
    return host_vals, dev


def causal_dkdv_keys_by_row_ranges(raw, scale, hk, keys, row_range=4096, workers=None):
    """Oracle dK, dV of `keys` for KV head hk of a causal problem with
    Tq == Tk, as a sum over the query heads of the group and over ranges of
    query rows (raw: bf16 bit arrays q, k, v, do with batch 1).

    A row range [r0, r1) only sees keys below r1, so its share of a key's
    gradient is the oracle's dK/dV of that key for the sub-problem of those
    rows against keys [0, r1): Tq = r1 - r0 and Tk = r1 put the causal
    diagonal at key r0 + i for local row i, which is the full problem's rule.
    The shares are independent and run in a thread pool (numpy releases the
    interpreter lock inside its array operations)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention_ref as ref

    Hq, Tq = raw["q"].shape[1], raw["q"].shape[2]
    Hkv, d = raw["k"].shape[1], raw["k"].shape[3]
    assert raw["k"].shape[2] == Tq and raw["q"].shape[0] == 1
    g = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    k = inputs.widen(raw["k"][:, hk:hk + 1])
    v = inputs.widen(raw["v"][:, hk:hk + 1])

    def share(h, r0, r1):
        q = inputs.widen(raw["q"][:, h:h + 1, r0:r1])
        do = inputs.widen(raw["do"][:, h:h + 1, r0:r1])
        sel = keys < r1
        if not sel.any():
            return sel, 0.0, 0.0
        dk, dv = ref.attention_bwd_dkdv_keys(q, k[:, :, :r1], v[:, :, :r1], do, scale, True, 0, 0, keys[sel])
        return sel, dk, dv

    jobs = [(h, r0, min(Tq, r0 + row_range)) for h in range(hk * g, (hk + 1) * g) for r0 in range(0, Tq, row_range)]
    jobs.sort(key=lambda j: -j[2])   # longest first
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    n = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), ThreadPoolExecutor(n) as ex:
        for sel, a, b in ex.map(lambda j: share(*j), jobs):
            dk[sel] += a
            dv[sel] += b
    return dk, dv
