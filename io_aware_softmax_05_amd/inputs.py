"""Seeded synthetic inputs for exact attention, shared by the HIP path's tests
and benchmark and by the CPU oracle's tests.

This module only draws random numbers and rounds them to the storage types the
kernels consume (fp32, bf16, and e4m3 bytes with per-head factors). It holds
none of the attention arithmetic.

Recipe (one PCG64 stream per workload, seeded with the workload's number):
  * draw order: [seq_lens], Q, K, V, dO -- each tensor is drawn in full, in
    row-major order, before the next one starts;
  * values: standard normal in fp64, rounded to fp32 (round to nearest even),
    then, for bf16 workloads, rounded to bf16 (round to nearest even, done on
    the fp32 bit pattern);
  * decode lengths: integers uniform on [4096, 32768], both ends included;
  * fp8 workloads: Q, K, V drawn as fp32, then each (batch, head) divided by
    max|x| / 448 and rounded to e4m3 (nearest, ties to even); V is handed
    over transposed, [B, Hkv, d, Tk].
Both sides consume the rounded values: the GPU gets the bit patterns, the
oracle gets the same numbers widened to fp64.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

# Draw tensors in chunks so that multi-GiB caches never need a full fp64 copy.
# PCG64 standard_normal draws are sequence-consistent, so chunking does not
# change the values.
_CHUNK = 1 << 24


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even, returning uint16 bit patterns.

    NaN maps to a quiet NaN of the same sign; overflow rounds to +-inf, and
    fp32 subnormals round to bf16 subnormals (same exponent field width)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    rounded = ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    is_nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if is_nan.any():
        sign = ((b >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
        rounded = np.where(is_nan, sign | np.uint16(0x7FC0), rounded)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws in fp64, rounded to fp32."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s).astype(np.float32)
    return out.reshape(shape)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws rounded fp64 -> fp32 -> bf16; returns uint16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = bf16_bits_from_f32(rng.standard_normal(e - s).astype(np.float32))
    return out.reshape(shape)


def _e4m3_positive_grid() -> np.ndarray:
    """The 127 non-negative finite OCP E4M3 values, indexed by their code 0x00..0x7E."""
    codes = np.arange(127)
    e, f = codes >> 3, codes & 7
    return np.where(e == 0, f * 2.0 ** -9, (8 + f) * np.exp2(e - 10.0))


_E4M3_GRID = _e4m3_positive_grid()


def e4m3_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round values with |x| <= 448 to OCP E4M3 bytes, nearest, ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if not np.all(a <= 448.0):
        raise ValueError("e4m3 input out of range (|x| <= 448)")
    hi = np.clip(np.searchsorted(_E4M3_GRID, a, side="left"), 1, 126)
    lo = hi - 1
    d_lo, d_hi = a - _E4M3_GRID[lo], _E4M3_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    return (code | np.where(np.signbit(x) & (code != 0), 0x80, 0)).astype(np.uint8)


def quantize_e4m3_per_head(x: np.ndarray):
    """x [B,H,T,d] -> (e4m3 bytes [B,H,T,d], fp32 factors [B,H]): each (batch, head)
    is divided by max|x| / 448 (its largest magnitude lands on 448) and rounded."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=(2, 3))
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    y = x / scale.astype(np.float64)[:, :, None, None]
    return e4m3_bits_from_f64(np.clip(y, -448.0, 448.0)), scale


def draw_fp8_attention_inputs(seed: int, B: int, Hq: int, Hkv: int, Tq: int, Tk: int, d: int) -> dict:
    """fp8 forward inputs: Q, K, V drawn as for fp32 (N(0,1) -> fp32), then
    quantised per (batch, head) to e4m3; V is handed over transposed.

    Returns q8 [B,Hq,Tq,d], k8 [B,Hkv,Tk,d], vt8 [B,Hkv,d,Tk] (uint8) and
    q_scale [B,Hq], k_scale, v_scale [B,Hkv] (fp32)."""
    rng = make_rng(seed)
    q = normal_f32(rng, (B, Hq, Tq, d))
    k = normal_f32(rng, (B, Hkv, Tk, d))
    v = normal_f32(rng, (B, Hkv, Tk, d))
    q8, qs = quantize_e4m3_per_head(q)
    k8, ks = quantize_e4m3_per_head(k)
    v8, vs = quantize_e4m3_per_head(v)
    return {"q8": q8, "k8": k8, "vt8": np.ascontiguousarray(np.swapaxes(v8, 2, 3)),
            "q_scale": qs, "k_scale": ks, "v_scale": vs}


def decode_lengths(rng: np.random.Generator, batch: int, lo: int = 4096, hi: int = 32768) -> np.ndarray:
    return rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, dtype and mode."""
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    d: int
    dtype: str           # "f32" or "bf16"
    causal: bool
    backward: bool
    decode: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads the method is measured on.
WORKLOADS = {
    1: Workload("single-head fp32 fwd B1 H1 T256 d64", 1, 1, 1, 1, 256, 256, 64, "f32", False, False),
    2: Workload("GPT-2-medium attention fwd+bwd B64 H16 T1024 d64", 2, 64, 16, 16, 1024, 1024, 64, "bf16", False, True),
    3: Workload("causal long-context fwd B1 H32 T8192 d128", 3, 1, 32, 32, 8192, 8192, 128, "bf16", True, False),
    4: Workload("causal 32k GQA fwd+bwd B1 Hq32 Hkv8 T32768 d128", 4, 1, 32, 8, 32768, 32768, 128, "bf16", True, True),
    5: Workload("split-KV decode B16 Hq32 Hkv8 Tk<=32768 d128", 5, 16, 32, 8, 1, 32768, 128, "bf16", False, False, True),
}


def draw_attention_inputs(seed: int, B: int, Hq: int, Hkv: int, Tq: int, Tk: int, d: int,
                          dtype: str = "bf16", with_dout: bool = False) -> dict:
    """Q [B,Hq,Tq,d], K and V [B,Hkv,Tk,d], optional dO [B,Hq,Tq,d].

    bf16 tensors come back as uint16 bit patterns, fp32 tensors as float32."""
    rng = make_rng(seed)
    draw = normal_bf16 if dtype == "bf16" else normal_f32
    out = {"q": draw(rng, (B, Hq, Tq, d)),
           "k": draw(rng, (B, Hkv, Tk, d)),
           "v": draw(rng, (B, Hkv, Tk, d))}
    if with_dout:
        out["do"] = draw(rng, (B, Hq, Tq, d))
    return out


def draw_decode_inputs(seed: int, B: int, Hq: int, Hkv: int, Tk_max: int, d: int,
                       lo: int = 4096, hi: int = 32768) -> dict:
    """seq_lens int32 [B], q [B,Hq,d], K and V caches [B,Hkv,Tk_max,d], bf16 bits."""
    rng = make_rng(seed)
    seq_lens = decode_lengths(rng, B, lo, min(hi, Tk_max))
    q = normal_bf16(rng, (B, Hq, d))
    k = normal_bf16(rng, (B, Hkv, Tk_max, d))
    v = normal_bf16(rng, (B, Hkv, Tk_max, d))
    return {"seq_lens": seq_lens, "q": q, "k": k, "v": v}


def workload_inputs(w: Workload) -> dict:
    if w.decode:
        return draw_decode_inputs(w.seed, w.B, w.Hq, w.Hkv, w.Tk, w.d)
    return draw_attention_inputs(w.seed, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, w.dtype, w.backward)


def widen(x: np.ndarray) -> np.ndarray:
    """The exact numeric values of a drawn tensor, as fp64."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)
