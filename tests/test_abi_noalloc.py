"""Host-side checks of fa_decode_splitkv_noalloc on the CPU: the argument
checks of fa_decode_splitkv apply, and a call whose partial states would not
fit the fixed scratch is refused before anything is looked up or launched.
Fake, never dereferenced pointers; skipped where a GPU is visible."""
import pytest
import torch

from io_aware_softmax_05_amd import fa

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks; fake pointers")

A = 0x10000
MIS = 0x10008


def _call(q=A, k=A, v=A, lens=A, o=A, lse=None, B=16, Hq=32, Hkv=8, Tk=4096, d=128, scale=0.1, chunk=64):
    return fa.load_library().fa_decode_splitkv_noalloc(q, k, v, lens, o, lse, B, Hq, Hkv, Tk, d, scale, chunk, None)


@pytest.mark.parametrize("kw, want", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lens=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(lens=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Hkv=5), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=96), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=32), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    # 16 * 32 * 64 partial states of 130 fp32 need 17039360 bytes > 16 MiB
    (dict(), fa.FA_ERR_WORKSPACE),
    (dict(B=1 << 12, Tk=1 << 20, chunk=0), fa.FA_ERR_WORKSPACE),
])
def test_noalloc_rejects(kw, want):
    assert _call(**kw) == want


def test_scratch_size_constant():
    assert fa.FA_DECODE_NOALLOC_SCRATCH_BYTES == 16 * 1024 * 1024
    with open(fa.HEADER_PATH) as f:
        assert "#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in f.read()
