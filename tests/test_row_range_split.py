"""The GPU tests evaluate the oracle's dK/dV of early causal keys as a sum of
row-range shares (tests/gpu_util.causal_dkdv_keys_by_row_ranges). On the CPU:
that sum equals one direct oracle call, and it is not the trivial zero."""
import numpy as np

from io_aware_softmax_05_amd import inputs
from oracle import attention_ref as ref
from tests import gpu_util as gu


def test_row_range_shares_sum_to_the_direct_gradient():
    raw = inputs.draw_attention_inputs(31, 1, 6, 2, 300, 300, 64, "bf16", with_dout=True)
    keys = np.array([0, 1, 63, 64, 130, 299])
    scale = 0.125
    for hk in (0, 1):
        grp = slice(hk * 3, hk * 3 + 3)
        want_k, want_v = ref.attention_bwd_dkdv_keys(inputs.widen(raw["q"][:, grp]), inputs.widen(raw["k"][:, hk:hk + 1]),
                                                     inputs.widen(raw["v"][:, hk:hk + 1]), inputs.widen(raw["do"][:, grp]),
                                                     scale, True, 0, 0, keys)
        for rr in (64, 100, 300):
            got_k, got_v = gu.causal_dkdv_keys_by_row_ranges(raw, scale, hk, keys, row_range=rr, workers=3)
            assert np.allclose(got_k, want_k, rtol=1e-12, atol=1e-13)
            assert np.allclose(got_v, want_v, rtol=1e-12, atol=1e-13)
        assert np.all(np.abs(want_v).sum(axis=1) > 0)
