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
