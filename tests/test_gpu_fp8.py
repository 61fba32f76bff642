"""GPU parity of fa_fwd_fp8 (e4m3 inputs, both products on fp8 matrix cores)
against the fp64 oracle on the dequantised inputs.

The fp8 path makes two approximations the bf16 path does not, so its bound is
derived here, per element, from the exact quantities the oracle provides:
  * the probabilities (times 2^5) are rounded to e4m3 before the PV product:
    relative error <= 2^-4 for normal values, absolute <= 2^-10 (i.e. 2^-15
    of a unit probability) for subnormal ones;
  * the fp8 matrix cores sum the products of a step in a window aligned to
    the largest product, so a dot product can miss the exact sum; 2^-11 of
    sum |products| is allowed, on S (each score, in log2 units eps_S = 2^-11 *
    scale * log2(e) * max_j sum_k |q_k k_jk|, moves p by a factor up to
    2^eps_S, and l with it) and on PV. test_fp8_score_accumulation_error_is_
    within_the_bound below pins that allowance on the hardware through this
    entry point (random rows miss by about 2^-17 of sum |products|; rows where
    one product dwarfs the others by 2^-12).
So with A_ic = sum_j P_ij |V_jc| (exact P):
  |O - O_ref| <= (2^-4 + 2^-11 + 1.5 eps_S) A + 2^-15 sum_j visible |V_jc|
                 + 2^-8 |O_ref| + 1e-6            (the last two: bf16 output, fp32)
  |LSE - LSE_ref| <= ln 2 * eps_S + 1e-5 max(1, |LSE_ref|).
The relative L2 error of O is reported; rounding errors of independent
probabilities average out to about 2^-4 / sqrt(3) ~ 3.6 %, and 5 % is checked.
"""
import math

import numpy as np
import pytest
import torch

from io_aware_softmax_05_amd import fa, inputs
from oracle import attention_ref as ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def _run(x, scale, causal):
    B, Hq, Tq, d = x["q8"].shape
    Hkv, Tk = x["k8"].shape[1], x["k8"].shape[2]
    dev = {n: _dev_u8(x[n]) for n in ("q8", "k8", "vt8")}
    sc = {n: gu.dev_f32(x[n].reshape(-1)) for n in ("q_scale", "k_scale", "v_scale")}
    o = torch.empty((B, Hq, Tq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_fp8(dev["q8"], dev["k8"], dev["vt8"], sc["q_scale"], sc["k_scale"], sc["v_scale"], o, lse,
                  B, Hq, Hkv, Tq, Tk, d, scale, causal)
    torch.cuda.synchronize()
    return o, lse


def _check(x, o, lse, scale, causal, rows=None, heads=None):
    """Per-element bound of the module docstring, on query rows `rows` (all if None)."""
    B, Hq, Tq, d = x["q8"].shape
    Hkv, Tk = x["k8"].shape[1], x["k8"].shape[2]
    g = Hq // Hkv
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    og, lg = gu.host(o), gu.host(lse)
    worst_o = worst_l = 0.0
    diffs, refs = [], []
    for b, h in heads:
        hk = h // g
        qv = ref.e4m3_to_f64(x["q8"][b, h, rows]) * float(x["q_scale"][b, h])
        kv = ref.e4m3_to_f64(x["k8"][b, hk]) * float(x["k_scale"][b, hk])
        vv = ref.e4m3_to_f64(x["vt8"][b, hk]).T * float(x["v_scale"][b, hk])
        p, l_ref = ref.row_probs(qv, kv, scale, rows, Tq, causal)
        o_ref = p @ vv
        vis = ref.visible(rows, Tq, Tk, causal)
        mag = np.abs(qv) @ np.abs(kv).T
        eps_s = 2.0 ** -11 * scale * LOG2E * np.max(np.where(vis, mag, 0.0), axis=1)
        a = p @ np.abs(vv)
        sub = vis.astype(np.float64) @ np.abs(vv)
        bound = ((2.0 ** -4 + 2.0 ** -11 + 1.5 * eps_s)[:, None] * a + 2.0 ** -15 * sub
                 + 2.0 ** -8 * np.abs(o_ref) + 1e-6)
        err = np.abs(og[b, h, rows] - o_ref)
        assert np.all(np.isfinite(og[b, h, rows])), (b, h)
        worst_o = max(worst_o, float(np.max(err / bound)))
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lg[b, h, rows]), fin), (b, h)
        lb = math.log(2) * eps_s + 1e-5 * np.maximum(1.0, np.abs(np.where(fin, l_ref, 0.0)))
        le = np.abs(np.where(fin, lg[b, h, rows] - np.where(fin, l_ref, 0.0), 0.0))
        worst_l = max(worst_l, float(np.max(le / lb)))
        diffs.append((og[b, h, rows] - o_ref).ravel())
        refs.append(o_ref.ravel())
    dd, rr = np.concatenate(diffs), np.concatenate(refs)
    rel = float(np.linalg.norm(dd) / np.linalg.norm(rr)) if np.linalg.norm(rr) > 0 else float(np.linalg.norm(dd))
    print(f"  O: worst err/bound {worst_o:.3f}, rel_l2 {rel:.4f}; LSE: worst err/bound {worst_l:.3f}", flush=True)
    assert worst_o <= 1.0, f"O exceeds its bound by {worst_o:.3f}x"
    assert worst_l <= 1.0, f"LSE exceeds its bound by {worst_l:.3f}x"
    assert rel <= 5e-2, f"O rel_l2 {rel:.4f}"


FP8_SHAPES = [
    # B, Hq, Hkv, Tq, Tk, d, causal
    (1, 8, 8, 64, 64, 128, False),      # one tile
    (1, 2, 1, 200, 256, 128, False),    # ragged query tail, several key tiles
    (1, 2, 1, 200, 256, 128, True),     # Tq < Tk: bottom-right diagonal
    (2, 2, 2, 130, 192, 64, False),
    (1, 4, 2, 384, 384, 64, True),      # GQA, several diagonal tiles
    (1, 6, 2, 333, 336, 128, True),     # 3 query heads per kv head, ragged
    (1, 2, 2, 300, 128, 128, True),     # Tq > Tk: the first 172 rows see no key
    (1, 2, 2, 700, 320, 128, True),     # Tq > Tk over several 256-row tiles: whole waves see no key
    (1, 4, 2, 600, 1024, 128, True),    # Tq < Tk: every wave's diagonal past the first key tile
    (1, 2, 1, 100, 16, 64, False),      # a single 16-key chunk
]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_forward_parity(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[fp8 fwd {shape}]", flush=True)
    x = inputs.draw_fp8_attention_inputs(800 + Tq + Tk, B, Hq, Hkv, Tq, Tk, d)
    scale = d ** -0.5
    o, lse = _run(x, scale, causal)
    _check(x, o, lse, scale, causal)
    if causal and Tq > Tk:
        og, lg = gu.host(o), gu.host(lse)
        assert np.all(og[:, :, :Tq - Tk] == 0) and np.all(lg[:, :, :Tq - Tk] == -np.inf)


def _random_fp8_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.integers(1, 3))
        out.append((1, hkv * int(rng.integers(1, 4)), hkv, int(rng.integers(1, 700)), 16 * int(rng.integers(1, 45)),
                    int(rng.choice([64, 128])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _random_fp8_shapes(8, 11), ids=lambda s: "x".join(map(str, s)))
def test_fp8_forward_random_shapes(shape):
    """Seeded random draws (Tk a multiple of 16, as the entry point requires)."""
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[fp8 fwd random {shape}]", flush=True)
    x = inputs.draw_fp8_attention_inputs(1300 + Tq + Tk, B, Hq, Hkv, Tq, Tk, d)
    scale = d ** -0.5
    o, lse = _run(x, scale, causal)
    _check(x, o, lse, scale, causal)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_peaky_scores_move_the_reference(d):
    # scale x8: scores spread over many powers of two, so the reference max
    # moves (slack 2^3) often and the e4m3 probabilities span their range
    print(f"[fp8 peaky d{d}]", flush=True)
    x = inputs.draw_fp8_attention_inputs(77 + d, 1, 4, 2, 256, 256, d)
    scale = 8 * d ** -0.5
    for causal in (False, True):
        o, lse = _run(x, scale, causal)
        _check(x, o, lse, scale, causal)


def test_fp8_forward_is_deterministic():
    x = inputs.draw_fp8_attention_inputs(5, 1, 4, 2, 320, 320, 128)
    o1, l1 = _run(x, 128 ** -0.5, True)
    o2, l2 = _run(x, 128 ** -0.5, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.slow
def test_fp8_forward_full_size_sampled_rows():
    # the benchmarked shape, B1 H32 T8192 d128 causal, checked on sampled rows of sampled heads
    B, H, T, d = 1, 32, 8192, 128
    print("[fp8 fwd B1 H32 T8192 d128 causal, sampled rows]", flush=True)
    x = inputs.draw_fp8_attention_inputs(3, B, H, H, T, T, d)
    o, lse = _run(x, d ** -0.5, True)
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(T - 64, T),
                                     np.random.Generator(np.random.PCG64(9)).integers(0, T, 128)]))
    _check(x, o, lse, d ** -0.5, True, rows=rows, heads=[(0, 0), (0, 13), (0, 31)])


def test_fp8_tiny_positive_factors():
    # the factors must be finite and > 0; a tiny one is inside that range:
    # q factor 2^-60 on head 0 and k factor 2^-60 on KV head 1 leave every
    # score of those heads at about 0, so their rows average V (the oracle's
    # closed form); v factor 2^-100 on KV head 0 scales its heads' outputs
    # down by that much, still finite in bf16
    print("[fp8 tiny factors]", flush=True)
    x = inputs.draw_fp8_attention_inputs(321, 1, 4, 2, 192, 192, 128)
    x["q_scale"] = x["q_scale"].copy()
    x["k_scale"] = x["k_scale"].copy()
    x["v_scale"] = x["v_scale"].copy()
    x["q_scale"][0, 0] *= np.float32(2.0 ** -60)
    x["k_scale"][0, 1] *= np.float32(2.0 ** -60)
    for causal in (False, True):
        o, lse = _run(x, 128 ** -0.5, causal)
        _check(x, o, lse, 128 ** -0.5, causal)
    x["v_scale"][0, 0] *= np.float32(2.0 ** -100)
    o, lse = _run(x, 128 ** -0.5, True)
    og = gu.host(o)
    assert np.all(np.isfinite(og)) and np.any(og[0, :2] != 0)
    assert float(np.max(np.abs(og[0, :2]))) < 2.0 ** -90


def _single_key_scores(q8, k8):
    """LSE of row 0 with causal Tq = Tk = 16 and unit factors at scale 1: the
    fp8 matrix cores' value of q_0 . k_0 (row 0 sees only key 0, so P' = 2^5
    and l' = 2^5 exactly)."""
    H, T, d = q8.shape[1], q8.shape[2], q8.shape[3]
    v8 = inputs.e4m3_bits_from_f64(np.ones((1, H, T, d)))
    one = np.ones((1, H), dtype=np.float32)
    x = {"q8": q8, "k8": k8, "vt8": np.ascontiguousarray(np.swapaxes(v8, 2, 3)),
         "q_scale": one, "k_scale": one, "v_scale": one}
    _, lse = _run(x, 1.0, True)
    qd, kd = ref.e4m3_to_f64(q8[0, :, 0]), ref.e4m3_to_f64(k8[0, :, 0])
    return gu.host(lse)[0, :, 0], np.sum(qd * kd, axis=1), qd * kd


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_accumulation_error_is_within_the_bound(d):
    """Pins the eps_S term of the bound above through the entry point itself:
    the fp8 matrix cores' q . k misses the exact sum by at most 2^-11 of
    sum |q_i k_i|, the allowance the per-element bound uses, over many random
    e4m3 rows (N(0,1) with per-row gains spanning 2^-6 .. 2^5) and over rows
    built so that one product dwarfs the others."""
    print(f"[fp8 score accumulation d{d}]", flush=True)
    rng = np.random.Generator(np.random.PCG64(4242 + d))
    H, T = 256, 16
    qv = rng.standard_normal((1, H, T, d)) * np.exp2(rng.integers(-6, 6, (1, H, T, 1)))
    kv = rng.standard_normal((1, H, T, d)) * np.exp2(rng.integers(-6, 6, (1, H, T, 1)))
    q8 = inputs.e4m3_bits_from_f64(np.clip(qv, -448, 448))
    k8 = inputs.e4m3_bits_from_f64(np.clip(kv, -448, 448))
    got, exact, prods = _single_key_scores(q8, k8)
    ratio = np.abs(got - exact) / np.sum(np.abs(prods), axis=1)
    print(f"  random rows: worst |error| / sum|products| = 2^{np.log2(max(float(ratio.max()), 2.0 ** -60)):.2f}",
          flush=True)
    assert float(ratio.max()) <= 2.0 ** -11
    # one product dwarfing the rest (448 beside d - 1 terms of +-2^-6): the
    # matrix cores keep the small terms only to about 12 bits below the large
    # one, the worst case for the allowance
    qv = rng.choice([-1.0, 1.0], (1, 64, T, d)) * 2.0 ** -6
    qv[0, :, 0, 0] = 448.0
    kv = rng.choice([-1.0, 1.0], (1, 64, T, d))
    got, exact, prods = _single_key_scores(inputs.e4m3_bits_from_f64(qv), inputs.e4m3_bits_from_f64(kv))
    err = np.abs(got - exact)
    small = np.abs(exact - prods[:, 0])            # |sum of the small terms|
    print(f"  dominant product: worst |error| = {float(err.max()):.4g}, worst |error| / sum|products| = "
          f"2^{np.log2(max(float((err / np.sum(np.abs(prods), axis=1)).max()), 2.0 ** -60)):.2f}, "
          f"|sum of small terms| up to {float(small.max()):.4g}, error / that = "
          f"{float(np.max(err / np.maximum(small, 1e-30))):.3f}", flush=True)
    assert float(np.max(err / np.sum(np.abs(prods), axis=1))) <= 2.0 ** -11
