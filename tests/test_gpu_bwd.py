"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle.

The GPU pipeline is the real one: fa_fwd produces O and the LSE, fa_bwd
consumes them. The oracle recomputes everything from the exact inputs."""
import numpy as np
import pytest
import torch

from io_aware_softmax_05_amd import fa, inputs
from oracle import attention_ref as ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _fwd_bwd(dev, causal, scale):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, Tq, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal)
    torch.cuda.synchronize()
    return dq, dk, dv


BWD_SHAPES = [
    (1, 2, 2, 130, 130, 64, False),
    (1, 2, 2, 130, 130, 64, True),
    (1, 4, 2, 257, 257, 128, True),
    (1, 4, 4, 256, 256, 128, False),
    (2, 4, 1, 100, 200, 128, True),     # Tq < Tk, 4 query heads per KV head
    (1, 2, 2, 150, 90, 64, True),       # Tq > Tk: the first 60 rows see no key
    (1, 2, 2, 64, 300, 128, False),
    (1, 8, 8, 17, 17, 128, True),
    (2, 2, 1, 200, 129, 64, False),
    (1, 6, 2, 190, 190, 64, True),      # 3 query heads per KV head, ragged 64-row tiles
    (1, 6, 2, 300, 300, 128, False),
    (1, 2, 2, 600, 600, 64, False),     # several 128-key workgroups and a ragged one
    (1, 4, 2, 333, 517, 64, False),     # ragged 32-row query tiles and key tiles, Tq < Tk, GQA
    # causal walks that pair tile p with tile n - 1 - p (dK/dV over 128-key
    # tiles, dQ over query tiles): many pairs, an odd middle tile, Tq != Tk
    (1, 4, 2, 1152, 1152, 128, True),   # 9 key tiles, 9 query tiles: four pairs and a middle one
    (1, 2, 1, 700, 1000, 128, True),    # Tq < Tk across several pairs
    (1, 4, 2, 900, 900, 64, True),      # the 16-key kernel at d = 64, ragged last tile
    (1, 2, 2, 1000, 700, 64, True),     # Tq > Tk: the first 300 rows see no key
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_parity(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[bwd {shape}]", flush=True)
    hv, dev = gu.attention_case(200 + Tq, B, Hq, Hkv, Tq, Tk, d, with_dout=True)
    scale = d ** -0.5
    dq, dk, dv = _fwd_bwd(dev, causal, scale)
    dq_r, dk_r, dv_r = ref.attention_bwd(hv["q"], hv["k"], hv["v"], hv["do"], scale, causal)
    gu.check_bf16("dQ", dq, dq_r)
    gu.check_bf16("dK", dk, dk_r)
    gu.check_bf16("dV", dv, dv_r)


def _random_bwd_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.integers(1, 3))
        out.append((1, hkv * int(rng.integers(1, 4)), hkv, int(rng.integers(1, 800)), int(rng.integers(1, 800)),
                    int(rng.choice([64, 128])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _random_bwd_shapes(10, 5), ids=lambda s: "x".join(map(str, s)))
def test_bwd_random_shapes(shape):
    """Seeded random draws over Tq, Tk, d, the group size and the mask: the
    paired causal walks, the diagonal and the ragged tiles land anywhere."""
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    print(f"[bwd random {shape}]", flush=True)
    hv, dev = gu.attention_case(5000 + Tq + Tk, B, Hq, Hkv, Tq, Tk, d, with_dout=True)
    scale = d ** -0.5
    dq, dk, dv = _fwd_bwd(dev, causal, scale)
    dq_r, dk_r, dv_r = ref.attention_bwd(hv["q"], hv["k"], hv["v"], hv["do"], scale, causal)
    gu.check_bf16("dQ", dq, dq_r)
    gu.check_bf16("dK", dk, dk_r)
    gu.check_bf16("dV", dv, dv_r)


@pytest.mark.parametrize("gain", [4.0, 8.0])
def test_bwd_peaky_scores(gain):
    """Queries scaled up so scores have sigma ~ gain: rows are dominated by a
    few keys. Checked against the oracle with the bf16 storage allowance."""
    print(f"[bwd peaky gain {gain}]", flush=True)
    scale = 128 ** -0.5
    hv, dev = gu.attention_case(17, 1, 4, 2, 200, 200, 128, with_dout=True, q_gain=gain)
    dq, dk, dv = _fwd_bwd(dev, True, scale)
    dq_r, dk_r, dv_r = ref.attention_bwd(hv["q"], hv["k"], hv["v"], hv["do"], scale, True)
    a_dq, a_dk, a_dv = gu.storage_allowance(hv, scale, True)
    gu.check_with_allowance("dQ", dq, dq_r, a_dq)
    gu.check_with_allowance("dK", dk, dk_r, a_dk)
    gu.check_with_allowance("dV", dv, dv_r, a_dv)


def test_bwd_deterministic():
    hv, dev = gu.attention_case(19, 1, 4, 2, 300, 300, 128, with_dout=True)
    a = _fwd_bwd(dev, True, 0.09)
    b = _fwd_bwd(dev, True, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# --------------------------------------------------- full workload sizes

@pytest.mark.slow
def test_full_size_gpt2_medium_backward():
    """B64 H16 T1024 d64 non-causal: the whole pass runs on the GPU; the oracle
    checks complete heads (dQ, dK, dV of a head depend only on that head)."""
    w = inputs.WORKLOADS[2]
    print(f"[full size bwd: {w.name}]", flush=True)
    raw = inputs.workload_inputs(w)
    dev = {n: gu.dev_bf16(a) for n, a in raw.items()}
    dq, dk, dv = _fwd_bwd(dev, w.causal, w.scale)
    for (b, h) in [(0, 0), (17, 5), (63, 15)]:
        sl = lambda n: inputs.widen(raw[n][b:b + 1, h:h + 1])  # noqa: E731
        dq_r, dk_r, dv_r = ref.attention_bwd(sl("q"), sl("k"), sl("v"), sl("do"), w.scale, w.causal)
        gu.check_bf16(f"dQ[{b},{h}]", gu.host(dq[b:b + 1, h:h + 1]), dq_r)
        gu.check_bf16(f"dK[{b},{h}]", gu.host(dk[b:b + 1, h:h + 1]), dk_r)
        gu.check_bf16(f"dV[{b},{h}]", gu.host(dv[b:b + 1, h:h + 1]), dv_r)


# Early keys of a causal 32k KV head: each sums contributions of the 4 query
# heads of its group times up to 32768 rows, the longest accumulations of the
# dK/dV kernel's query-tile walk.
EARLY_KEYS = np.array([0, 1, 31, 32, 63, 64, 127, 128, 4095, 16384])


@pytest.mark.slow
def test_full_size_causal_gqa_32k_backward():
    """B1 Hq32 Hkv8 T32768 d128 causal: sampled dQ rows; dK/dV element by
    element for the early keys of KV heads 0 and 7 (the longest sums: 4 heads
    times up to 32768 rows) and for the last 200 keys of both; and two
    identities over every key: sum_j dV_j = sum of the group's dO rows, and
    sum_j dK_j = 0."""
    w = inputs.WORKLOADS[4]
    print(f"[full size bwd: {w.name}]", flush=True)
    raw = inputs.workload_inputs(w)
    dev = {n: gu.dev_bf16(a) for n, a in raw.items()}
    dq, dk, dv = _fwd_bwd(dev, w.causal, w.scale)
    g = w.Hq // w.Hkv
    rng = np.random.Generator(np.random.PCG64(44))
    for hk in (0, w.Hkv - 1):
        grp = slice(hk * g, (hk + 1) * g)
        q = inputs.widen(raw["q"][:, grp])
        do = inputs.widen(raw["do"][:, grp])
        k = inputs.widen(raw["k"][:, hk:hk + 1])
        v = inputs.widen(raw["v"][:, hk:hk + 1])
        rows = np.array(sorted(set([0, 1, 127, 128, w.Tq - 1] + rng.integers(0, w.Tq, 12).tolist())))
        for hl in (0, g - 1):
            dq_r = ref.attention_bwd_dq_rows(q, k, v, do, w.scale, True, 0, hl, rows)
            gu.check_bf16(f"dQ rows head {hk * g + hl}", gu.host(dq[0, hk * g + hl, rows]), dq_r)
        keys = np.arange(w.Tk - 200, w.Tk)
        dk_r, dv_r = ref.attention_bwd_dkdv_keys(q, k, v, do, w.scale, True, 0, 0, keys)
        gu.check_bf16(f"dK last keys kv {hk}", gu.host(dk[0, hk, keys]), dk_r)
        gu.check_bf16(f"dV last keys kv {hk}", gu.host(dv[0, hk, keys]), dv_r)
        dk_r, dv_r = gu.causal_dkdv_keys_by_row_ranges(raw, w.scale, hk, EARLY_KEYS)
        gu.check_bf16(f"dK early keys kv {hk}", gu.host(dk[0, hk, EARLY_KEYS]), dk_r)
        gu.check_bf16(f"dV early keys kv {hk}", gu.host(dv[0, hk, EARLY_KEYS]), dv_r)
    # identities over all keys, every KV head
    dvs = gu.host(dv).sum(axis=2)                       # [1, Hkv, d]
    want = inputs.widen(raw["do"]).reshape(1, w.Hkv, g, w.Tq, w.d).sum(axis=(2, 3))
    rel = np.linalg.norm(dvs - want) / np.linalg.norm(want)
    print(f"  sum dV vs sum dO: rel_l2={rel:.3e}", flush=True)
    assert rel <= 1e-2
    dkh = gu.host(dk)
    dks = dkh.sum(axis=2)
    spread = np.sqrt((dkh ** 2).sum(axis=2))
    ratio = float(np.max(np.abs(dks) / spread))
    print(f"  |sum dK| / sqrt(sum dK^2): max={ratio:.3e}", flush=True)
    assert ratio <= 0.05
