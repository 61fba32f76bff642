"""The tensor helpers of the binding (forward, backward, decode) reject
tensors whose shape, dtype or device does not match q before anything reaches
the library: the kernels index every tensor by q's sizes, so a mismatched one
would be read or written past its end.

Runs on the CPU: the library loader is replaced by one that fails the test,
so a check that let a bad argument through would show up as that failure.
"""
import pytest
import torch

from io_aware_softmax_05_amd import fa

B, HQ, HKV, T, D = 2, 4, 2, 16, 64


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def fail(*a, **k):
        raise AssertionError("a bad argument reached the library")
    monkeypatch.setattr(fa, "load_library", fail)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def good_bwd():
    return dict(q=bf(B, HQ, T, D), k=bf(B, HKV, T + 3, D), v=bf(B, HKV, T + 3, D), o=bf(B, HQ, T, D),
                dout=bf(B, HQ, T, D), lse=torch.zeros((B, HQ, T), dtype=torch.float32))


BWD_BAD = {
    "o rows": ("o", bf(B, HQ, T + 1, D)),
    "o heads": ("o", bf(B, HQ - 1, T, D)),
    "dout width": ("dout", bf(B, HQ, T, 128)),
    "dout batch": ("dout", bf(B + 1, HQ, T, D)),
    "v length": ("v", bf(B, HKV, T + 2, D)),
    "v heads": ("v", bf(B, HKV + 1, T + 3, D)),
    "k batch": ("k", bf(B - 1, HKV, T + 3, D)),
    "k width": ("k", bf(B, HKV, T + 3, 128)),
    "lse rows": ("lse", torch.zeros((B, HQ, T - 1), dtype=torch.float32)),
    "lse heads": ("lse", torch.zeros((B, HKV, T), dtype=torch.float32)),
    "lse dtype": ("lse", torch.zeros((B, HQ, T), dtype=torch.bfloat16)),
    "o dtype": ("o", torch.zeros((B, HQ, T, D), dtype=torch.float32)),
    "dout not contiguous": ("dout", bf(B, HQ, D, T).transpose(2, 3)),
}


@pytest.mark.parametrize("case", sorted(BWD_BAD))
def test_backward_rejects_mismatch(case):
    name, bad = BWD_BAD[case]
    args = good_bwd()
    args[name] = bad
    with pytest.raises(ValueError):
        fa.backward(**args)


def test_backward_rejects_head_ratio():
    args = good_bwd()
    args["k"], args["v"] = bf(B, 3, T + 3, D), bf(B, 3, T + 3, D)
    with pytest.raises(ValueError, match="multiple"):
        fa.backward(**args)


def test_backward_rejects_cpu_tensors():
    # shapes all agree: the last check (one GPU) refuses host memory
    with pytest.raises(ValueError, match="GPU"):
        fa.backward(**good_bwd())


FWD_BAD = {
    "k width": dict(k=bf(B, HKV, T, 128)),
    "v length": dict(v=bf(B, HKV, T + 1, D)),
    "k batch": dict(k=bf(B + 1, HKV, T, D), v=bf(B + 1, HKV, T, D)),
    "k dtype": dict(k=torch.zeros((B, HKV, T, D), dtype=torch.float32)),
    "q dtype": dict(q=torch.zeros((B, HQ, T, D), dtype=torch.float16)),
    "head ratio": dict(k=bf(B, 3, T, D), v=bf(B, 3, T, D)),
}


@pytest.mark.parametrize("case", sorted(FWD_BAD))
def test_forward_rejects_mismatch(case):
    args = dict(q=bf(B, HQ, T, D), k=bf(B, HKV, T, D), v=bf(B, HKV, T, D))
    args.update(FWD_BAD[case])
    with pytest.raises(ValueError):
        fa.forward(**args)


def good_dec():
    return dict(q=bf(B, HQ, D), k_cache=bf(B, HKV, 100, D), v_cache=bf(B, HKV, 100, D),
                seq_lens=torch.full((B,), 50, dtype=torch.int32))


DEC_BAD = {
    "v_cache length": dict(v_cache=bf(B, HKV, 99, D)),
    "v_cache heads": dict(v_cache=bf(B, HKV * 2, 100, D)),
    "k_cache width": dict(k_cache=bf(B, HKV, 100, 128), v_cache=bf(B, HKV, 100, 128)),
    "k_cache batch": dict(k_cache=bf(B + 1, HKV, 100, D), v_cache=bf(B + 1, HKV, 100, D)),
    "seq_lens short": dict(seq_lens=torch.full((B - 1,), 50, dtype=torch.int32)),
    "seq_lens dtype": dict(seq_lens=torch.full((B,), 50, dtype=torch.int64)),
    "head ratio": dict(k_cache=bf(B, 3, 100, D), v_cache=bf(B, 3, 100, D)),
}


@pytest.mark.parametrize("case", sorted(DEC_BAD))
def test_decode_rejects_mismatch(case):
    args = good_dec()
    args.update(DEC_BAD[case])
    with pytest.raises(ValueError):
        fa.decode(**args)


def test_one_gpu_rejects_mixed_devices():
    with pytest.raises(ValueError, match="one device"):
        fa._one_gpu(a=torch.zeros(1), b=torch.zeros(1, device="meta"))
