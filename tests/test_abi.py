"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before launching anything.

Only argument combinations that the host checks reject are passed; the tests
are skipped on a machine with a GPU so that a checking bug can never turn a
fake pointer into a launch there.
"""
import ctypes

import pytest
import torch

from io_aware_softmax_05_amd import fa

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks; fake pointers")

A = 0x10000          # fake, 16-byte aligned "device" address (never dereferenced)
MIS = 0x10008        # misaligned by 8 bytes


def lib():
    return fa.load_library()


def test_every_declared_function_is_exported():
    names = fa.header_functions()
    assert set(names) == set(fa._SIGNATURES), names
    handle = lib()
    for n in names:
        assert hasattr(handle, n), n
        assert ctypes.cast(getattr(handle, n), ctypes.c_void_p).value


def test_status_strings():
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(-1) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(-2) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(-3) == "FA_ERR_WORKSPACE"
    assert fa.fa_status_string(-4) == "FA_ERR_HIP"
    assert fa.fa_status_string(7) == "FA_UNKNOWN_STATUS"


def _fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=None, B=1, Hq=2, Hkv=1, Tq=8, Tk=8, d=64, scale=0.125, causal=0)
    args.update(kw)
    return lib().fa_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["Hq"],
                        args["Hkv"], args["Tq"], args["Tk"], args["d"], args["scale"], args["causal"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(Tq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Tk=-3), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(q=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(o=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(lse=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(Tk=1 << 23, d=128), fa.FA_ERR_INVALID_ARG),   # one head's keys span 2^31 bytes
    (dict(Tq=1 << 23, Tk=8, d=128), fa.FA_ERR_INVALID_ARG),
])
def test_fwd_rejects(kw, want):
    assert _fwd(**kw) == want
    kw32 = dict(kw)
    args = dict(q=A, k=A, v=A, o=A, lse=None, B=1, Hq=2, Hkv=1, Tq=8, Tk=8, d=64, scale=0.125, causal=0)
    args.update(kw32)
    got = lib().fa_fwd_f32(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["Hq"],
                           args["Hkv"], args["Tq"], args["Tk"], args["d"], args["scale"], args["causal"], None)
    assert got == want


def test_workspace_sizes_are_linear():
    assert fa.fa_bwd_workspace_size(1, 32, 32768, 128) == 32 * 32768 * 8          # 8 MiB, two fp32 per row
    assert fa.fa_bwd_workspace_size(0, 1, 1, 64) == 0
    w1 = fa.fa_decode_workspace_size(16, 32, 32768, 128)
    w2 = fa.fa_decode_workspace_size(16, 32, 65536, 128)
    assert 1.9 * w1 < w2 < 2.1 * w1
    assert w1 < 2 * 16 * 8 * 32768 * 128 * 2 / 8    # far below the cache it serves
    assert fa.fa_decode_workspace_size(1, 1, 0, 64) == 0


def _bwd(ws=A, ws_bytes=1 << 20, **kw):
    args = dict(B=1, Hq=2, Hkv=1, Tq=8, Tk=8, d=64, scale=0.125, causal=0)
    args.update(kw)
    ptr = {n: kw.get(n, A) for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv")}
    return lib().fa_bwd(ptr["q"], ptr["k"], ptr["v"], ptr["o"], ptr["dout"], ptr["lse"], ptr["dq"], ptr["dk"],
                        ptr["dv"], ws, ws_bytes, args["B"], args["Hq"], args["Hkv"], args["Tq"], args["Tk"],
                        args["d"], args["scale"], args["causal"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(dout=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=None), fa.FA_ERR_INVALID_ARG),
    (dict(dk=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=4, Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=8), fa.FA_ERR_WORKSPACE),
    (dict(ws=MIS), fa.FA_ERR_WORKSPACE),
])
def test_bwd_rejects(kw, want):
    assert _bwd(**kw) == want


def _dec(ws=A, ws_bytes=1 << 30, **kw):
    args = dict(q=A, k=A, v=A, lens=A, o=A, lse=None, B=2, Hq=8, Hkv=2, Tk_max=256, d=128, scale=0.1, chunk=0)
    args.update(kw)
    return lib().fa_decode_splitkv(args["q"], args["k"], args["v"], args["lens"], args["o"], args["lse"], ws,
                                   ws_bytes, args["B"], args["Hq"], args["Hkv"], args["Tk_max"], args["d"],
                                   args["scale"], args["chunk"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lens=None), fa.FA_ERR_INVALID_ARG),
    (dict(lens=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=32), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=100), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=-64), fa.FA_ERR_INVALID_ARG),
    (dict(Tk_max=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(B=70000), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), fa.FA_ERR_WORKSPACE),
])
def test_decode_rejects(kw, want):
    assert _dec(**kw) == want


def test_binding_raises_on_error():
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(A, A, A, A, None, 1, 1, 1, 4, 4, 48, 0.1, False, stream=0)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------ sliding window

@pytest.mark.parametrize("window", [0, -1, -4096])
def test_window_entry_points_reject_empty_windows(window):
    L = lib()
    assert L.fa_fwd_window(A, A, A, A, None, 1, 2, 1, 8, 8, 64, 0.125, window, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_window(A, A, A, A, A, A, A, A, A, A, 1 << 20, 1, 2, 1, 8, 8, 64, 0.125, window,
                           None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_decode_splitkv_window(A, A, A, A, A, None, A, 1 << 30, 2, 8, 2, 256, 128, 0.1, window, 0,
                                      None) == fa.FA_ERR_INVALID_ARG


def test_window_entry_points_check_like_the_plain_ones():
    L = lib()
    # the same argument checks run first: d, Hq % Hkv, NULL outputs, workspace
    assert L.fa_fwd_window(A, A, A, A, None, 1, 2, 1, 8, 8, 48, 0.125, 4, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_fwd_window(A, A, A, None, None, 1, 2, 1, 8, 8, 64, 0.125, 4, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_window(A, A, A, A, A, A, A, A, A, None, 1 << 20, 1, 2, 1, 8, 8, 64, 0.125, 4,
                           None) == fa.FA_ERR_WORKSPACE
    assert L.fa_decode_splitkv_window(A, A, A, A, A, None, A, 1 << 30, 2, 6, 4, 256, 128, 0.1, 4, 0,
                                      None) == fa.FA_ERR_INVALID_ARG


# ------------------------------------------------------------------ fp8 forward

def test_fp8_forward_rejects_bad_arguments():
    L = lib()
    S = 0x10004   # a 4-byte aligned (not 16-byte aligned) address for the scale arrays
    ok = (A, A, A, S, S, S, A, None, 1, 2, 1, 8, 32, 64, 0.125, 1, None)
    bad = {
        "Tk not a multiple of 16": (A, A, A, S, S, S, A, None, 1, 2, 1, 8, 40, 64, 0.125, 1, None),
        "NULL vt": (A, A, None, S, S, S, A, None, 1, 2, 1, 8, 32, 64, 0.125, 1, None),
        "NULL q_scale": (A, A, A, None, S, S, A, None, 1, 2, 1, 8, 32, 64, 0.125, 1, None),
        "NULL v_scale": (A, A, A, S, S, None, A, None, 1, 2, 1, 8, 32, 64, 0.125, 1, None),
        "misaligned scale": (A, A, A, S + 2, S, S, A, None, 1, 2, 1, 8, 32, 64, 0.125, 1, None),
        "misaligned vt": (A, A, A + 8, S, S, S, A, None, 1, 2, 1, 8, 32, 64, 0.125, 1, None),
        "Hq % Hkv": (A, A, A, S, S, S, A, None, 1, 3, 2, 8, 32, 64, 0.125, 1, None),
        "zero scale": (A, A, A, S, S, S, A, None, 1, 2, 1, 8, 32, 64, 0.0, 1, None),
    }
    for name, args in bad.items():
        assert L.fa_fwd_fp8(*args) == fa.FA_ERR_INVALID_ARG, name
    assert L.fa_fwd_fp8(*ok[:13], 48, *ok[14:]) == fa.FA_ERR_UNSUPPORTED   # d


@pytest.mark.parametrize("p", [0.0, 0.1, 0.25, 0.5, 0.9, 1.0 / 512, 3.0 / 512, 0.998, 0.3333])
def test_dropout_keep_threshold_matches_the_oracle(p):
    from oracle import attention_ref as ref
    # the library takes p as fp32; the oracle's rule is applied to that same value
    p32 = float(ctypes.c_float(p).value)
    assert fa.fa_dropout_keep_threshold(p) == ref.keep_threshold(p32)


@pytest.mark.parametrize("p", [1.0, -0.01, 0.999, float("nan"), float("inf")])
def test_dropout_keep_threshold_rejects(p):
    assert lib().fa_dropout_keep_threshold(p) == fa.FA_ERR_INVALID_ARG
    with pytest.raises(fa.FaError):
        fa.fa_dropout_keep_threshold(p)


def test_dropout_entry_points_check_like_the_plain_ones():
    common = (1, 2, 1, 8, 8, 64, 0.125, 1)
    # an unusable dropout probability is refused before anything else is looked at
    for p in (1.0, -0.5, float("nan")):
        assert lib().fa_fwd_dropout(A, A, A, A, None, *common, p, 1, 0, None) == fa.FA_ERR_INVALID_ARG
        assert lib().fa_bwd_dropout(A, A, A, A, A, A, A, A, A, A, 1 << 20, *common, p, 1, 0, None) \
            == fa.FA_ERR_INVALID_ARG
    # with a usable one, the plain entry points' checks apply
    assert lib().fa_fwd_dropout(None, A, A, A, None, *common, 0.1, 1, 0, None) == fa.FA_ERR_INVALID_ARG
    assert lib().fa_fwd_dropout(A, A, A, A, None, 1, 2, 1, 8, 8, 96, 0.125, 1, 0.1, 1, 0, None) \
        == fa.FA_ERR_UNSUPPORTED
    assert lib().fa_fwd_dropout(A, A, A, MIS, None, *common, 0.1, 1, 0, None) == fa.FA_ERR_INVALID_ARG
    assert lib().fa_bwd_dropout(A, A, A, A, A, A, A, A, A, A, 0, *common, 0.1, 1, 0, None) == fa.FA_ERR_WORKSPACE
    assert lib().fa_bwd_dropout(A, A, A, A, A, None, A, A, A, A, 1 << 20, *common, 0.1, 1, 0, None) \
        == fa.FA_ERR_INVALID_ARG
    assert lib().fa_bwd_dropout(A, A, A, A, A, A, A, A, A, A, 1 << 20, 1, 3, 2, 8, 8, 64, 0.125, 1, 0.1, 1, 0,
                                None) == fa.FA_ERR_INVALID_ARG


# ------------------------------------------------------------ tile shapes

@pytest.mark.parametrize("shape", [-1, 2, 7])
def test_tile_shape_entry_points_reject_unknown_shapes(shape):
    L = lib()
    assert L.fa_fwd_tiles(A, A, A, A, None, 1, 2, 1, 8, 8, 64, 0.125, 1, shape, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_tiles(A, A, A, A, A, A, A, A, A, A, 1 << 20, 1, 2, 1, 8, 8, 64, 0.125, 1, shape,
                          None) == fa.FA_ERR_INVALID_ARG


def test_tile_shape_entry_points_check_like_the_plain_ones():
    L = lib()
    for shape in (0, 1):
        assert L.fa_fwd_tiles(A, A, A, A, None, 1, 2, 1, 8, 8, 48, 0.125, 1, shape, None) == fa.FA_ERR_UNSUPPORTED
        assert L.fa_fwd_tiles(A, A, A, A, None, 1, 3, 2, 8, 8, 64, 0.125, 1, shape, None) == fa.FA_ERR_INVALID_ARG
        assert L.fa_bwd_tiles(A, A, A, A, A, A, A, A, A, None, 1 << 20, 1, 2, 1, 8, 8, 64, 0.125, 1, shape,
                              None) == fa.FA_ERR_WORKSPACE
        assert L.fa_bwd_tiles(A, A, A, A, A, A, A, A, A, A, 16, 1, 2, 1, 8, 8, 64, 0.125, 1, shape,
                              None) == fa.FA_ERR_WORKSPACE
