"""The seeded generators and the bf16 rounding they use (no GPU)."""
import numpy as np

from io_aware_softmax_05_amd import inputs


def _bits(u32):
    return np.array([u32], dtype=np.uint32).view(np.float32)


def test_bf16_round_nearest_even_bit_patterns():
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0x3F808000: 0x3F80,  # exactly half way, even below -> stays
        0x3F818000: 0x3F82,  # exactly half way, odd below -> rounds up to even
        0x3F808001: 0x3F81,  # just above half way
        0x3F807FFF: 0x3F80,  # just below half way
        0xBF818000: 0xBF82,  # sign carried
        0x00008000: 0x0000,  # subnormal tie to even (zero)
        0x00018000: 0x0002,  # subnormal tie rounds up to even
        0x00000001: 0x0000,  # tiny subnormal
        0x7F7FFFFF: 0x7F80,  # largest float rounds to +inf
        0xFF7FFFFF: 0xFF80,  # and its negative to -inf
        0x7F800000: 0x7F80,  # +inf
        0x80000000: 0x8000,  # -0
        0x7FC00001: 0x7FC0,  # NaN stays a quiet NaN
        0xFF800001: 0xFFC0,  # signalling negative NaN -> quiet negative NaN
        0x3F7FFFFF: 0x3F80,  # rounding carries into the exponent
    }
    for src, want in cases.items():
        got = int(inputs.bf16_bits_from_f32(_bits(src))[0])
        assert got == want, (hex(src), hex(got), hex(want))


def test_bf16_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = inputs.bf16_bits_to_f32(bits)
    back = inputs.bf16_bits_from_f32(f)
    finite = np.isfinite(f)
    assert np.array_equal(back[finite], bits[finite])


def test_generators_are_seeded_and_chunk_invariant():
    a = inputs.draw_attention_inputs(2, 1, 2, 1, 33, 40, 8, "bf16", with_dout=True)
    b = inputs.draw_attention_inputs(2, 1, 2, 1, 33, 40, 8, "bf16", with_dout=True)
    for key in ("q", "k", "v", "do"):
        assert np.array_equal(a[key], b[key])
    # draw order Q, K, V, dO from one PCG64 stream, fp64 -> fp32 -> bf16
    rng = np.random.Generator(np.random.PCG64(2))
    z = rng.standard_normal(2 * 33 * 8 + 2 * 40 * 8)
    q = inputs.bf16_bits_from_f32(z[:2 * 33 * 8].astype(np.float32)).reshape(1, 2, 33, 8)
    assert np.array_equal(q, a["q"])
    old = inputs._CHUNK
    try:
        inputs._CHUNK = 37
        c = inputs.draw_attention_inputs(2, 1, 2, 1, 33, 40, 8, "bf16", with_dout=True)
    finally:
        inputs._CHUNK = old
    for key in ("q", "k", "v", "do"):
        assert np.array_equal(a[key], c[key])


def test_decode_lengths_in_range():
    d = inputs.draw_decode_inputs(5, 16, 4, 1, 64, 8, lo=4, hi=64)
    assert d["seq_lens"].dtype == np.int32
    assert np.all((d["seq_lens"] >= 4) & (d["seq_lens"] <= 64))
    lens = inputs.decode_lengths(inputs.make_rng(5), 16)
    assert np.all((lens >= 4096) & (lens <= 32768))


def test_workloads_table():
    w = inputs.WORKLOADS
    assert (w[3].B, w[3].Hq, w[3].Tq, w[3].d, w[3].causal) == (1, 32, 8192, 128, True)
    assert (w[4].Hq, w[4].Hkv, w[4].Tq, w[4].backward) == (32, 8, 32768, True)
    assert w[2].scale == 0.125 and w[1].dtype == "f32"
