"""Host-side checks of bench.py's bookkeeping (no GPU): kernel-name keys, the
launch units whose HBM traffic is recorded, and the per-unit source hashes
that decide whether a recorded figure still describes the current kernels."""
import json
import os
import shutil

import pytest

import bench


def test_kernel_key_keeps_variant_arguments_and_drops_config_structs():
    assert bench.kernel_key("void fa::fwd_bf16_kernel<128, true, false, true>(fa::FwdArgs)") == \
        "fwd_bf16_kernel<128, true, false, true>"
    name = ("void fa::bwd_dkdv_kernel<64, false, fa::(anonymous namespace)::DkdvCfg<64, 8, 64, 2, 0, 1>, "
            "false, true>(fa::BwdArgs, int)")
    assert bench.kernel_key(name) == "bwd_dkdv_kernel<64, false, false, true>"
    assert bench.kernel_key("void fa::decode_merge_kernel<128>(fa::DecodeArgs)") == "decode_merge_kernel<128>"


def test_every_traffic_unit_maps_to_existing_sources():
    for unit, kernels in bench.TRAFFIC_UNITS.items():
        assert kernels, unit
        for spec in kernels:
            family = spec.split("<")[0]
            assert family in bench.KERNEL_SOURCES, (unit, spec)
            for f in bench.KERNEL_SOURCES[family]:
                assert os.path.exists(os.path.join(bench.CSRC, f)), f
        assert len(bench.unit_source_hash(unit)) == 64


def test_unit_hash_follows_only_its_own_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, csrc, ignore=shutil.ignore_patterns("*.o", "*.so"))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    fwd, dec = "fa_fwd causal B1 H32 T8192 d128", "fa_decode_splitkv B16 Hq32 Hkv8 d128"
    h_fwd, h_dec = bench.unit_source_hash(fwd), bench.unit_source_hash(dec)
    with open(csrc / "fa_decode.hip", "a") as f:
        f.write("\n// edit\n")
    assert bench.unit_source_hash(fwd) == h_fwd
    assert bench.unit_source_hash(dec) != h_dec
    with open(csrc / "fa_common.hpp", "a") as f:   # shared header: every unit changes
        f.write("\n// edit\n")
    assert bench.unit_source_hash(fwd) != h_fwd


def test_recorded_traffic_is_null_for_stale_or_unknown_units(tmp_path, monkeypatch):
    unit = "fa_fwd B64 H16 T1024 d64"
    rec = {"units": {unit: {"bytes": 123, "source_sha256": bench.unit_source_hash(unit), "kernels": {}},
                     "not a unit": {"bytes": 1, "source_sha256": "x", "kernels": {}}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.recorded_traffic(unit) == 123.0
    assert bench.recorded_traffic("not a unit") is None
    rec["units"][unit]["source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.recorded_traffic(unit) is None


@pytest.mark.parametrize("B,Hq,T,d,causal,want", [(1, 1, 4, 2, False, 4 * 2 * 16), (1, 1, 4, 2, True, 4 * 2 * 10),
                                                    (2, 3, 8192, 128, True, 4 * 128 * 8192 * 8193 // 2 * 6)])
def test_flop_convention(B, Hq, T, d, causal, want):
    assert bench.fwd_flops(B, Hq, T, T, d, causal) == want


def test_fraction_at_the_measured_clock():
    # the matrix peak scales with the engine clock: at 2000 MHz of 2400 it is 5/6 of the spec figure
    assert bench.frac_at_clock(1000.0, 2500.0, [2000.0, 2000.0]) == round(1000.0 / (2500.0 * 2000 / 2400), 4)
    assert bench.frac_at_clock(1000.0, 2500.0, [2400.0]) == 0.4
    assert bench.frac_at_clock(1000.0, 2500.0, None) is None
    assert bench.frac_at_clock(1000.0, 2500.0, []) is None
    assert bench.frac_at_clock(1000.0, 2500.0, 2000) == round(1000.0 / (2500.0 * 2000 / 2400), 4)


def test_gfx_clocks_reads_only_the_engine_clocks():
    # amd-smi metric --clock --json: one "clk" per clock domain; only the gfx ones are the engine's
    out = {"gpu_data": [{"gpu": 0, "clock": {
        "gfx_0": {"clk": {"value": 1400, "unit": "MHz"}, "min_clk": {"value": 500}},
        "gfx_1": {"clk": {"value": 2200, "unit": "MHz"}},
        "mem_0": {"clk": {"value": 1900, "unit": "MHz"}},
        "vclk_0": {"clk": {"value": 29, "unit": "MHz"}}}}]}
    assert bench.gfx_clocks(out) == [1400.0, 2200.0]
    assert bench.gfx_clocks({"gfx_0": {"clk": "N/A"}}) == []
