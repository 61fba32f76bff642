"""GPU parity of attention dropout (fa_fwd_dropout, fa_bwd_dropout) against the fp64 oracle.

The keep mask is integer work, so it is checked bit for bit: with zero
queries every probability of a row is equal, and values V_j = 2^-(j div d) e_(j mod d)
make each output element an exact binary number whose bits are the kept
flags of keys c, c + d, ..., c + 7 d. The dropped outputs and gradients are
checked to the bf16 tolerances of tests/gpu_util.py, at small shapes that
span several tiles with ragged tails and at the full GPT-2-medium layer
(sampled heads, rows and keys, in the launch configuration the benchmark
times)."""
import numpy as np
import pytest
import torch

from io_aware_softmax_05_amd import fa, inputs
from oracle import attention_ref as ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED, OFFSET = 0x5EED0123456789AB, 7


def _fwd(dev, causal, scale, p_drop, seed=SEED, offset=OFFSET):
    q, k, v = dev["q"], dev["k"], dev["v"]
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, p_drop, seed, offset)
    return o, lse


def _bwd(dev, o, lse, causal, scale, p_drop, seed=SEED, offset=OFFSET):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, Tq, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal,
                      p_drop, seed, offset)
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,Tq", [(1, 2, 2, 96), (2, 3, 1, 301)])
def test_keep_mask_bit_exact(d, B, Hq, Hkv, Tq):
    """Zero queries: P = 1 / Tk in every row, so O_ic = (2 / Tk) sum_m Z_i,c+md 2^-m
    (t = 128) is exact in bf16 and its 8 bits are the kept flags."""
    Tk = 8 * d
    print(f"[dropout mask d={d} B={B} Hq={Hq} Hkv={Hkv} Tq={Tq}]", flush=True)
    t = fa.fa_dropout_keep_threshold(0.5)
    assert t == 128
    j = np.arange(Tk)
    v1 = np.zeros((Tk, d), dtype=np.float32)
    v1[j, j % d] = 2.0 ** -(j // d)
    v = np.broadcast_to(v1, (B, Hkv, Tk, d))
    q = np.zeros((B, Hq, Tq, d), dtype=np.float32)
    k = np.random.Generator(np.random.PCG64(3)).standard_normal((B, Hkv, Tk, d)).astype(np.float32)
    dev = {n: gu.dev_bf16(inputs.bf16_bits_from_f32(x)) for n, x in (("q", q), ("k", k), ("v", v))}
    o, _ = _fwd(dev, False, d ** -0.5, 0.5)
    torch.cuda.synchronize()
    code = np.rint(gu.host(o) * Tk / 2 * 128).astype(np.int64)          # [B,Hq,Tq,d], 8 bits each
    assert code.min() >= 0 and code.max() <= 255
    bits = (code[..., None] >> (7 - np.arange(8))) & 1                 # [..., c, m] -> key c + m d
    got = np.swapaxes(bits, -1, -2).reshape(B, Hq, Tq, Tk).astype(bool)
    drop = ref.Dropout(t=t, seed=SEED, offset=OFFSET)
    for b in range(B):
        for h in range(Hq):
            want = ref.dropout_keep(drop, b * Hq + h, np.arange(Tq), Tk)
            bad = int((got[b, h] != want).sum())
            assert bad == 0, f"head ({b},{h}): {bad} mask bits differ"
    print(f"  kept fraction {got.mean():.4f}", flush=True)


FWD_SHAPES = [
    (1, 2, 2, 130, 130, 64, False),
    (1, 2, 2, 130, 130, 64, True),
    (1, 4, 2, 257, 257, 128, True),
    (1, 4, 4, 256, 300, 128, False),
    (2, 4, 1, 100, 200, 128, True),     # Tq < Tk, 4 query heads per KV head
    (1, 2, 2, 150, 90, 64, True),       # Tq > Tk: the first 60 rows see no key
    (1, 6, 2, 190, 190, 64, True),
    (1, 4, 2, 333, 517, 64, False),     # ragged 32-row query tiles of the 4-wave dK/dV, Tq < Tk
    (1, 4, 2, 700, 700, 64, True),      # causal pairs: 3 query tiles and 3 key tiles, the middle ones alone
    (1, 2, 1, 450, 450, 128, True),     # causal pairs: 4 query tiles of 128 rows, 4 key tiles of 128 keys
]


@pytest.mark.parametrize("p_drop", [0.1, 0.5])
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dropout_fwd_bwd_parity(shape, p_drop):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[dropout fwd+bwd {shape} p={p_drop}]", flush=True)
    hv, dev = gu.attention_case(300 + Tq, B, Hq, Hkv, Tq, Tk, d, with_dout=True)
    scale = d ** -0.5
    drop = ref.Dropout(t=fa.fa_dropout_keep_threshold(p_drop), seed=SEED, offset=OFFSET)
    o, lse = _fwd(dev, causal, scale, p_drop)
    dq, dk, dv = _bwd(dev, o, lse, causal, scale, p_drop)
    torch.cuda.synchronize()
    o_r, lse_r = ref.attention_fwd(hv["q"], hv["k"], hv["v"], scale, causal, dropout=drop)
    gu.check_bf16("O", o, o_r)
    gu.check_lse("LSE", lse, lse_r, 1e-4)
    dq_r, dk_r, dv_r = ref.attention_bwd(hv["q"], hv["k"], hv["v"], hv["do"], scale, causal, dropout=drop)
    a_dq, a_dk, a_dv = gu.storage_allowance(hv, scale, causal, dropout=drop)
    gu.check_with_allowance("dQ", dq, dq_r, a_dq)
    gu.check_with_allowance("dK", dk, dk_r, a_dk)
    gu.check_with_allowance("dV", dv, dv_r, a_dv)


def _random_dropout_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.integers(1, 3))
        out.append((1, hkv * int(rng.integers(1, 4)), hkv, int(rng.integers(1, 500)), int(rng.integers(1, 500)),
                    int(rng.choice([64, 128])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _random_dropout_shapes(6, 13), ids=lambda s: "x".join(map(str, s)))
def test_dropout_random_shapes(shape):
    """Seeded random draws over Tq, Tk, d, the group size and the mask, p = 0.2."""
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[dropout random {shape}]", flush=True)
    hv, dev = gu.attention_case(1700 + Tq + Tk, B, Hq, Hkv, Tq, Tk, d, with_dout=True)
    scale = d ** -0.5
    drop = ref.Dropout(t=fa.fa_dropout_keep_threshold(0.2), seed=SEED, offset=OFFSET)
    o, lse = _fwd(dev, causal, scale, 0.2)
    dq, dk, dv = _bwd(dev, o, lse, causal, scale, 0.2)
    torch.cuda.synchronize()
    o_r, lse_r = ref.attention_fwd(hv["q"], hv["k"], hv["v"], scale, causal, dropout=drop)
    gu.check_bf16("O", o, o_r)
    gu.check_lse("LSE", lse, lse_r, 1e-4)
    dq_r, dk_r, dv_r = ref.attention_bwd(hv["q"], hv["k"], hv["v"], hv["do"], scale, causal, dropout=drop)
    a_dq, a_dk, a_dv = gu.storage_allowance(hv, scale, causal, dropout=drop)
    gu.check_with_allowance("dQ", dq, dq_r, a_dq)
    gu.check_with_allowance("dK", dk, dk_r, a_dk)
    gu.check_with_allowance("dV", dv, dv_r, a_dv)


def test_dropout_zero_is_the_plain_pass():
    hv, dev = gu.attention_case(41, 1, 2, 2, 200, 200, 64, with_dout=True)
    o0 = torch.empty_like(dev["q"])
    lse0 = torch.empty((1, 2, 200), dtype=torch.float32, device="cuda")
    fa.fa_fwd(dev["q"], dev["k"], dev["v"], o0, lse0, 1, 2, 2, 200, 200, 64, 0.125, True)
    o1, lse1 = _fwd(dev, True, 0.125, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(lse0, lse1)


def test_dropout_deterministic_and_stream_dependent():
    hv, dev = gu.attention_case(42, 1, 4, 2, 257, 257, 128, with_dout=True)
    runs = []
    for offset in (OFFSET, OFFSET, OFFSET + 1):
        o, lse = _fwd(dev, True, 128 ** -0.5, 0.2, offset=offset)
        dq, dk, dv = _bwd(dev, o, lse, True, 128 ** -0.5, 0.2, offset=offset)
        torch.cuda.synchronize()
        runs.append([x.clone() for x in (o, dq, dk, dv)])
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b)
    assert not torch.equal(runs[0][0], runs[2][0])


@pytest.mark.slow
def test_full_size_gpt2_medium_dropout():
    """B64 H16 T1024 d64 non-causal, p = 0.1: the whole forward and backward
    run on the GPU; the oracle checks sampled rows of three heads, their dQ
    rows and the dK/dV of sampled keys of their KV heads."""
    w = inputs.WORKLOADS[2]
    print(f"[full size dropout: {w.name}, p=0.1]", flush=True)
    raw = inputs.workload_inputs(w)
    dev = {n: gu.dev_bf16(a) for n, a in raw.items()}
    o, lse = _fwd(dev, w.causal, w.scale, 0.1)
    dq, dk, dv = _bwd(dev, o, lse, w.causal, w.scale, 0.1)
    torch.cuda.synchronize()
    drop = ref.Dropout(t=fa.fa_dropout_keep_threshold(0.1), seed=SEED, offset=OFFSET)
    hv = {n: inputs.widen(a) for n, a in raw.items()}
    rng = np.random.Generator(np.random.PCG64(45))
    for (b, h) in [(0, 0), (17, 5), (63, 15)]:
        rows = np.array(sorted(set([0, 1, 63, 64, w.Tq - 1] + rng.integers(0, w.Tq, 20).tolist())))
        o_r, lse_r = ref.attention_fwd_head_rows(hv["q"], hv["k"], hv["v"], w.scale, w.causal, b, h, rows,
                                                 dropout=drop)
        gu.check_bf16(f"O[{b},{h}] rows", gu.host(o[b, h, rows]), o_r)
        gu.check_lse(f"LSE[{b},{h}] rows", gu.host(lse[b, h, rows]), lse_r, 1e-4)
        dq_r = ref.attention_bwd_dq_rows(hv["q"], hv["k"], hv["v"], hv["do"], w.scale, w.causal, b, h, rows,
                                         dropout=drop)
        gu.check_bf16(f"dQ[{b},{h}] rows", gu.host(dq[b, h, rows]), dq_r)
        keys = np.array(sorted(set([0, 31, 32, w.Tk - 1] + rng.integers(0, w.Tk, 12).tolist())))
        dk_r, dv_r = ref.attention_bwd_dkdv_keys(hv["q"], hv["k"], hv["v"], hv["do"], w.scale, w.causal, b, h,
                                                 keys, dropout=drop)
        gu.check_bf16(f"dK[{b},{h}] keys", gu.host(dk[b, h, keys]), dk_r)
        gu.check_bf16(f"dV[{b},{h}] keys", gu.host(dv[b, h, keys]), dv_r)
