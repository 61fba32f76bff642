"""GPU parity of split-KV decoding (fa_decode_splitkv) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from io_aware_softmax_05_amd import fa, inputs
from oracle import attention_ref as ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _decode(dev, lens_dev, scale, chunk=0, ws=None):
    q, kc, vc = dev["q"], dev["k"], dev["v"]
    B, Hq, d = q.shape
    Hkv, Tk_max = kc.shape[1], kc.shape[2]
    ws_bytes = fa.fa_decode_workspace_size(B, Hq, Tk_max, d)
    if ws is None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    fa.fa_decode_splitkv(q, kc, vc, lens_dev, o, lse, ws, ws.numel(), B, Hq, Hkv, Tk_max, d, scale, chunk)
    torch.cuda.synchronize()
    return o, lse


def _case(seed, B, Hq, Hkv, Tk_max, d, lo, hi):
    raw = inputs.draw_decode_inputs(seed, B, Hq, Hkv, Tk_max, d, lo=lo, hi=hi)
    dev = {n: gu.dev_bf16(raw[n]) for n in ("q", "k", "v")}
    lens = torch.from_numpy(raw["seq_lens"]).cuda()
    return raw, dev, lens


@pytest.mark.parametrize("shape", [(3, 8, 2, 300, 128, 1, 300), (2, 4, 4, 1000, 64, 1, 1000),
                                   (4, 32, 8, 700, 128, 60, 700), (2, 32, 1, 129, 128, 1, 129),
                                   (1, 16, 16, 64, 64, 64, 64),
                                   (2, 24, 4, 500, 128, 1, 500),     # 6 query heads per KV head
                                   (2, 48, 2, 400, 128, 1, 400),     # 24: a full and a partial row group
                                   (3, 12, 4, 333, 64, 1, 333)],     # 3 query heads per KV head, d = 64
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("chunk", [0, 64, 192])
def test_decode_parity(shape, chunk):
    B, Hq, Hkv, Tk_max, d, lo, hi = shape
    print(f"[decode {shape} chunk={chunk}]", flush=True)
    raw, dev, lens = _case(50 + Tk_max, B, Hq, Hkv, Tk_max, d, lo, hi)
    scale = d ** -0.5
    o, lse = _decode(dev, lens, scale, chunk)
    o_ref, lse_ref = ref.decode(inputs.widen(raw["q"]), inputs.widen(raw["k"]), inputs.widen(raw["v"]),
                                raw["seq_lens"], scale)
    gu.check_bf16("O", o, o_ref)
    gu.check_lse("LSE", lse, lse_ref, 1e-4)


def _random_decode_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.integers(1, 5))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        t_max = int(rng.integers(1, 3000))
        lo = int(rng.integers(1, t_max + 1))
        out.append((int(rng.integers(1, 5)), hkv * g, hkv, t_max, int(rng.choice([64, 128])), lo, t_max,
                    int(rng.choice([0, 64, 256, 1024]))))
    return out


@pytest.mark.parametrize("shape", _random_decode_shapes(10, 17), ids=lambda s: "x".join(map(str, s)))
def test_decode_random_shapes(shape):
    """Seeded random draws over batch, group size (up to a full 16-row MFMA),
    cache length, length spread, d and the chunk size."""
    B, Hq, Hkv, Tk_max, d, lo, hi, chunk = shape
    print(f"[decode random {shape}]", flush=True)
    raw, dev, lens = _case(2100 + Tk_max, B, Hq, Hkv, Tk_max, d, lo, hi)
    scale = d ** -0.5
    o, lse = _decode(dev, lens, scale, chunk)
    o_ref, lse_ref = ref.decode(inputs.widen(raw["q"]), inputs.widen(raw["k"]), inputs.widen(raw["v"]),
                                raw["seq_lens"], scale)
    gu.check_bf16("O", o, o_ref)
    gu.check_lse("LSE", lse, lse_ref, 1e-4)


def test_decode_matches_fwd_one_query():
    """Decoding equals the forward pass with one query row over the first L keys."""
    raw, dev, lens = _case(3, 2, 8, 2, 500, 128, 200, 500)
    o, lse = _decode(dev, lens, 0.1)
    for b in range(2):
        L = int(raw["seq_lens"][b])
        q = dev["q"][b].reshape(1, 8, 1, 128).contiguous()
        k = dev["k"][b:b + 1, :, :L].contiguous()
        v = dev["v"][b:b + 1, :, :L].contiguous()
        of = torch.empty_like(q)
        lf = torch.empty((1, 8, 1), dtype=torch.float32, device="cuda")
        fa.fa_fwd(q, k, v, of, lf, 1, 8, 2, 1, L, 128, 0.1, False)
        torch.cuda.synchronize()
        gu.check_bf16("O vs fwd", o[b], gu.host(of[0, :, 0]))
        gu.check_lse("LSE vs fwd", lse[b], lf[0, :, 0].cpu().numpy().astype(np.float64), 1e-4)


def test_decode_deterministic_and_chunk_invariant():
    raw, dev, lens = _case(4, 4, 16, 4, 2000, 128, 1, 2000)
    o1, l1 = _decode(dev, lens, 0.09)
    o2, l2 = _decode(dev, lens, 0.09)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for chunk in (64, 128, 1024, 2048):
        o3, l3 = _decode(dev, lens, 0.09, chunk)
        gu.check_bf16(f"O chunk {chunk} vs auto", o3, gu.host(o1))
        gu.check_lse(f"LSE chunk {chunk} vs auto", l3, l1.cpu().numpy().astype(np.float64), 1e-4)


def test_decode_never_reads_past_length():
    """Cache positions at and beyond seq_lens[b] are NaN: the result is finite
    and equal to the oracle's."""
    raw, dev, lens = _case(6, 3, 8, 2, 600, 128, 1, 600)
    for n in ("k", "v"):
        for b in range(3):
            dev[n][b, :, int(raw["seq_lens"][b]):] = float("nan")
    o, lse = _decode(dev, lens, 0.1)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, lse_ref = ref.decode(inputs.widen(raw["q"]), inputs.widen(raw["k"]), inputs.widen(raw["v"]),
                                raw["seq_lens"], 0.1)
    gu.check_bf16("O", o, o_ref)


def test_decode_bad_lengths_give_nan():
    raw, dev, lens = _case(8, 4, 8, 2, 256, 64, 1, 256)
    bad = torch.tensor([0, 100, 257, -5], dtype=torch.int32, device="cuda")
    o, lse = _decode(dev, bad, 0.125)
    of, lf = gu.host(o), lse.cpu().numpy()
    for b in (0, 2, 3):
        assert np.all(np.isnan(of[b])) and np.all(np.isnan(lf[b]))
    assert np.all(np.isfinite(of[1]))
    o_ref, _ = ref.decode(inputs.widen(raw["q"]), inputs.widen(raw["k"]), inputs.widen(raw["v"]),
                          np.array([1, 100, 1, 1]), 0.125)
    gu.check_bf16("O (valid entry)", of[1], o_ref[1])


@pytest.mark.slow
def test_decode_full_size_sampled():
    """B16 Hq32 Hkv8 Tk<=32768 d128 with lengths U[4096, 32768], seed 5, in the
    launch configuration the benchmark times; every (b, head) is checked."""
    w = inputs.WORKLOADS[5]
    print(f"[full size decode: {w.name}]", flush=True)
    raw = inputs.workload_inputs(w)
    dev = {n: gu.dev_bf16(raw[n]) for n in ("q", "k", "v")}
    lens = torch.from_numpy(raw["seq_lens"]).cuda()
    o, lse = _decode(dev, lens, w.scale)
    qh = inputs.widen(raw["q"])
    o_ref = np.zeros((w.B, w.Hq, w.d))
    lse_ref = np.zeros((w.B, w.Hq))
    g = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(raw["seq_lens"][b])
        for hk in range(w.Hkv):
            k = inputs.widen(raw["k"][b, hk, :L])
            v = inputs.widen(raw["v"][b, hk, :L])
            p, l = ref.row_probs(qh[b, hk * g:(hk + 1) * g], k, w.scale, np.zeros(g, dtype=np.int64), 1, False)
            o_ref[b, hk * g:(hk + 1) * g] = p @ v
            lse_ref[b, hk * g:(hk + 1) * g] = l
    gu.check_bf16("O", o, o_ref)
    gu.check_lse("LSE", lse, lse_ref, 1e-4)
