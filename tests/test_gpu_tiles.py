"""Tile-size invariance on the GPU: the forward and the backward computed with
two compiled tilings of the same kernels (fa_fwd_tiles / fa_bwd_tiles with
tile_shape 0 and 1) on the same seeded inputs.

aimlrounds "FlashAttention", section "Softmax without seeing the whole row":
the tiled recurrence gives the same answer for every tile size, up to
floating-point rounding. Both tilings must meet the bf16 parity bar against
the fp64 oracle, and they must agree with each other to that bar (they are
not bitwise equal: probabilities are rounded to bf16 relative to a running
maximum that moves at tile boundaries). Tiling 0 must also be bitwise the
plain entry points' result. The CPU half of this pin (the recurrence at tile
sizes 1..T equals the three-step oracle) is in tests/test_oracle.py."""
import numpy as np
import pytest
import torch

from io_aware_softmax_05_amd import fa
from oracle import attention_ref as ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, Hq, Hkv, Tq, Tk, d, causal: ragged tails, Tq != Tk, GQA, both widths
    (1, 4, 2, 300, 300, 128, True),
    (1, 4, 4, 333, 333, 128, False),
    (2, 6, 2, 200, 259, 128, True),
    (1, 4, 2, 300, 300, 64, True),
    (2, 4, 4, 270, 270, 64, False),
    (1, 2, 1, 150, 90, 64, True),       # Tq > Tk: the first 60 rows see no key
]


def _run(dev, causal, shape_id):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_tiles(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, shape_id)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    n = fa.fa_bwd_workspace_size(B, Hq, Tq, d)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    fa.fa_bwd_tiles(q, k, v, o, do, lse, dq, dk, dv, ws, n, B, Hq, Hkv, Tq, Tk, d, scale, causal, shape_id)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_two_tilings_agree_with_the_oracle_and_each_other(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[tilings {shape}]", flush=True)
    hv, dev = gu.attention_case(600 + Tq + d, B, Hq, Hkv, Tq, Tk, d, with_dout=True)
    scale = d ** -0.5
    o_r, lse_r = ref.attention_fwd(hv["q"], hv["k"], hv["v"], scale, causal)
    dq_r, dk_r, dv_r = ref.attention_bwd(hv["q"], hv["k"], hv["v"], hv["do"], scale, causal)
    want = {"O": o_r, "dQ": dq_r, "dK": dk_r, "dV": dv_r}
    runs = [_run(dev, causal, t) for t in (0, 1)]
    for t, r in enumerate(runs):
        for name, w in want.items():
            gu.check_bf16(f"{name} tiling {t}", r[name], w)
        gu.check_lse(f"LSE tiling {t}", r["LSE"], lse_r, 1e-4)
    for name in want:
        gu.check_bf16(f"{name} tiling 1 vs 0", runs[1][name], gu.host(runs[0][name]))
    gu.check_lse("LSE tiling 1 vs 0", runs[1]["LSE"], gu.host(runs[0]["LSE"]), 1e-4)


def test_tiling_zero_is_the_plain_entry_points():
    hv, dev = gu.attention_case(77, 1, 4, 2, 260, 260, 128, with_dout=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    B, Hq, Tq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, Hq, 2, Tq, Tq, d, 0.09, True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    n = fa.fa_bwd_workspace_size(B, Hq, Tq, d)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, n, B, Hq, 2, Tq, Tq, d, 0.09, True)
    torch.cuda.synchronize()
    o0 = torch.empty_like(q)
    lse0 = torch.empty_like(lse)
    fa.fa_fwd_tiles(q, k, v, o0, lse0, B, Hq, 2, Tq, Tq, d, 0.09, True, 0)
    dq0, dk0, dv0 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.fa_bwd_tiles(q, k, v, o, do, lse, dq0, dk0, dv0, ws, n, B, Hq, 2, Tq, Tq, d, 0.09, True, 0)
    torch.cuda.synchronize()
    for a, b in ((o, o0), (lse, lse0), (dq, dq0), (dk, dk0), (dv, dv0)):
        assert torch.equal(a, b)
