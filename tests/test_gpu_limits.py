"""GPU parity at the largest sizes the C ABI accepts.

The kernels address one head's rows through 32-bit buffer offsets, and the
host accepts T * d * 2 < 2^31 bytes per head: at d = 128 the largest key or
query count is 2^23 - 1 (a ragged count, not a multiple of any tile). These
cases run the forward, the backward and decoding right at that boundary and
compare sampled outputs with the fp64 oracle (the oracle sees the whole
8M-key rows: each checked row's scores are complete).

Host memory: up to about 25 GiB per case for the fp64 copies the oracle
works on."""
import numpy as np
import pytest
import torch

from io_aware_softmax_05_amd import fa, inputs
from oracle import attention_ref as ref
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

D = 128
TMAX = (1 << 23) - 1          # largest T with T * D * 2 < 2^31


def _bf16(x: float) -> np.uint16:
    return inputs.bf16_bits_from_f32(np.array([x], dtype=np.float32))[0]


def test_largest_key_count_fwd_bwd():
    """Three query rows against 2^23 - 1 keys. Row i's query is e_i and only
    key hit_i (first, middle, last) has K = 16 e_i, so each row puts about half
    of its weight on one far-apart key and half on the other 8M."""
    Tq, Tk = 3, TMAX
    print(f"[limits: fwd+bwd Tq={Tq} Tk={Tk} d={D}]", flush=True)
    rng = inputs.make_rng(61)
    v = inputs.normal_bf16(rng, (1, 1, Tk, D))
    do = inputs.normal_bf16(rng, (1, 1, Tq, D))
    q = np.zeros((1, 1, Tq, D), dtype=np.uint16)
    k = np.zeros((1, 1, Tk, D), dtype=np.uint16)
    hits = [0, Tk // 2, Tk - 1]
    for i, j in enumerate(hits):
        q[0, 0, i, i] = _bf16(1.0)
        k[0, 0, j, i] = _bf16(16.0)
    scale = 1.0
    dev = {n: gu.dev_bf16(a) for n, a in (("q", q), ("k", k), ("v", v), ("do", do))}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((1, 1, Tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, 1, 1, 1, Tq, Tk, D, scale, False)
    dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    ws_bytes = fa.fa_bwd_workspace_size(1, 1, Tq, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, ws, ws_bytes, 1, 1, 1, Tq, Tk, D,
              scale, False)
    torch.cuda.synchronize()
    # every key's dV is written: sum_j dV_j = sum_i dO_i (each row of P sums to one)
    dv_sum = dv[0, 0].float().sum(dim=0).double().cpu().numpy()
    do_sum = inputs.widen(do)[0, 0].sum(axis=0)
    rel = np.linalg.norm(dv_sum - do_sum) / np.linalg.norm(do_sum)
    print(f"  sum dV vs sum dO: rel_l2={rel:.3e}", flush=True)
    assert rel <= 1e-2

    qf, kf, vf, dof = (inputs.widen(a) for a in (q, k, v, do))
    del k, v
    o_r, lse_r = ref.attention_fwd(qf, kf, vf, scale, False)
    gu.check_bf16("O", o, o_r)
    gu.check_lse("LSE", lse, lse_r, 1e-4)
    dq_r = ref.attention_bwd_dq_rows(qf, kf, vf, dof, scale, False, 0, 0, np.arange(Tq))
    gu.check_bf16("dQ", dq[0, 0], dq_r)
    rng_k = np.random.Generator(np.random.PCG64(62))
    keys = np.array(sorted(set([0, 1, 63, 64, Tk // 2 - 1, Tk // 2, Tk // 2 + 1, Tk - 65, Tk - 64, Tk - 2, Tk - 1]
                               + rng_k.integers(0, Tk, 20).tolist())))
    dk_r, dv_r = ref.attention_bwd_dkdv_keys(qf, kf, vf, dof, scale, False, 0, 0, keys)
    gu.check_bf16("dK sampled keys", gu.host(dk[0, 0, keys]), dk_r)
    gu.check_bf16("dV sampled keys", gu.host(dv[0, 0, keys]), dv_r)


@pytest.mark.parametrize("causal", [False, True])
def test_largest_query_count_fwd(causal):
    """2^23 - 1 query rows against 77 keys. Causal aligns the diagonal
    bottom-right, so every row but the last 77 sees no key (O = 0, LSE = -inf)."""
    Tq, Tk = TMAX, 77
    print(f"[limits: fwd Tq={Tq} Tk={Tk} d={D} causal={causal}]", flush=True)
    rng = inputs.make_rng(63)
    q = inputs.normal_bf16(rng, (1, 1, Tq, D))
    k = inputs.normal_bf16(rng, (1, 1, Tk, D))
    v = inputs.normal_bf16(rng, (1, 1, Tk, D))
    dev = {n: gu.dev_bf16(a) for n, a in (("q", q), ("k", k), ("v", v))}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((1, 1, Tq), dtype=torch.float32, device="cuda")
    scale = D ** -0.5
    fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, 1, 1, 1, Tq, Tk, D, scale, causal)
    torch.cuda.synchronize()
    rng_r = np.random.Generator(np.random.PCG64(64))
    rows = np.array(sorted(set([0, 1, 255, 256, Tq // 2, Tq - 79, Tq - 78, Tq - 77, Tq - 76, Tq - 2, Tq - 1]
                               + rng_r.integers(0, Tq, 10).tolist())))
    q32 = inputs.bf16_bits_to_f32(q)   # exact values; the oracle widens only the sampled rows
    o_r, lse_r = ref.attention_fwd_head_rows(q32, inputs.widen(k), inputs.widen(v), scale, causal, 0, 0, rows)
    gu.check_bf16("O sampled rows", gu.host(o[0, 0, rows]), o_r)
    gu.check_lse("LSE sampled rows", gu.host(lse[0, 0, rows]), lse_r, 1e-4)
    if causal:   # rows that see no key: exactly zero output and -inf everywhere before the last 77
        head = o[0, 0, :Tq - Tk]
        assert int(torch.count_nonzero(head)) == 0
        assert bool(torch.all(torch.isneginf(lse[0, 0, :Tq - Tk])))


def test_largest_decode_cache():
    """One sequence filling a cache of 2^23 - 1 positions, four query heads on one KV head."""
    Hq, Tk_max = 4, TMAX
    print(f"[limits: decode Tk_max={Tk_max} d={D}]", flush=True)
    rng = inputs.make_rng(65)
    qd = inputs.normal_bf16(rng, (1, Hq, D))
    vc = inputs.normal_bf16(rng, (1, 1, Tk_max, D))
    kc = np.ascontiguousarray(vc[..., ::-1])    # distinct keys, exact values, no second draw
    lens = np.array([Tk_max], dtype=np.int32)
    dq_, dk_, dv_ = gu.dev_bf16(qd), gu.dev_bf16(kc), gu.dev_bf16(vc)
    ws_bytes = fa.fa_decode_workspace_size(1, Hq, Tk_max, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dq_)
    lse = torch.empty((1, Hq), dtype=torch.float32, device="cuda")
    scale = D ** -0.5
    fa.fa_decode_splitkv(dq_, dk_, dv_, torch.from_numpy(lens).cuda(), o, lse, ws, ws_bytes, 1, Hq, 1, Tk_max, D,
                         scale, 0)
    torch.cuda.synchronize()
    o_r, lse_r = ref.decode(inputs.widen(qd), inputs.widen(kc), inputs.widen(vc), lens, scale)
    gu.check_bf16("O", o, o_r)
    gu.check_lse("LSE", lse, lse_r, 1e-4)
