#!/usr/bin/env python3
"""Benchmark of the exact tiled-attention library on one MI355X.

    python bench.py [--steps K] [--warmup W]

The headline step is one pass of the forward hot path (grid plan, Q-tile
load, K/V streaming, S = scale QK^T on the matrix cores, causal mask, online
softmax, u += PV, epilogue) over the causal long-context layer: fa_fwd on
B1 H32 T8192 d128 bf16 (the Llama-3-8B attention shape of zerotofrontier
"Efficient attention: memory-bound"), scale 1/sqrt(128), inputs drawn with the
seeded recipe of io_aware_softmax_05_amd/inputs.py (the same values the parity
tests check) and resident in HBM before timing starts. W untimed steps, then
exactly K steps timed between two device synchronisations; HIP events
recorded around every launch, on the stream the kernel runs on, give the
launch duration behind `roofline`.

Before the headline, in the same run, under "targets" (each the median of
timed launches after untimed ones, seeded inputs unless stated):
  * the GPT-2-medium layer fwd+bwd (B64 H16 T1024 d64, non-causal);
  * the causal 32k GQA layer fwd and bwd (B1 Hq32 Hkv8 T32768 d128);
  * split-KV decoding (B16 Hq32 Hkv8 Tk<=32768 d128, lengths U[4096, 32768]);
    the seeded cache and a device copy of it are used in turn, so no call
    finds the previous call's rows in the 256 MiB MALL;
  * outside the five workloads, with torch-drawn N(0,1) inputs: the
    sliding-window layer (B1 Hq32 Hkv8 T32768 W4096 d128) fwd and bwd, the
    fp8 causal forward (B1 H32 T8192 d128) and the GPT-2-medium layer with
    dropout p = 0.1;
  * the fp32 single-head forward (B1 H1 T256 d64) as a latency.
After the headline: the fp64 CPU oracle timed on the host cores
(`cpu_baseline`), and the GPU clock read while the headline kernel runs.

FLOP convention: 4*d per visible (query, key) pair for the forward (two
contractions), 2.5x that for the backward (five contractions); a causal
square problem has T(T+1)/2 visible pairs. Decode bytes: every cached key and
value row read once (sum_b L_b * Hkv * 2 * d * 2 bytes) plus q and o.

Measured HBM traffic. `roofline.traffic` comes from profiles/hbm_traffic.json,
written by `--record-traffic DIR` from four rocprofv3 counter runs:
    DIR/fetch_all   rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline
    DIR/write_all   rocprofv3 --pmc WRITE_SIZE -- (same)
    DIR/fetch_copy  rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --only copy --steps 2
    DIR/write_copy  rocprofv3 --pmc WRITE_SIZE -- (same)
(each with --output-format csv -d DIR/<name> -o run). Each counter is scaled
by the ratio of the known copy size to what that counter reads for the plain
1 GiB device copy. Each unit records a hash of the sources its kernels are
built from (plus the shared headers); when those change, that unit's traffic is
reported as null until the counters are taken again. `--record-counters DIR`
does the same for the instruction and cycle counters of profiles/counters.json.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak (AMD spec)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak (AMD spec)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak (AMD spec)
SPEC_SCLK_MHZ = 2400          # MI355X peak engine clock the matrix peak assumes

COPY_BYTES = 1 << 30          # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "io_aware_softmax_05_amd", "csrc")

METRIC = "attention fwd/bwd TFLOPS and % of MI355X bf16 MFMA peak; decode HBM GB/s"
HEADLINE_UNIT = "fa_fwd causal B1 H32 T8192 d128"

# Launch units whose HBM traffic (and counters) are recorded: unit -> kernel
# names (prefix of the demangled name, up to the argument list).
TRAFFIC_UNITS = {
    "fa_fwd B64 H16 T1024 d64": ["fwd_bf16_kernel<64, false, false, false>"],
    "fa_bwd B64 H16 T1024 d64": ["bwd_dq_kernel<64, false, false, false>", "bwd_dkdv_kernel<64, false, false, false>"],
    # the causal 8k and 32k forwards run the same kernel: told apart by grid size (threads)
    "fa_fwd causal B1 H32 T8192 d128": ["fwd_bf16_kernel<128, true, false, false>@262144"],
    "fa_decode_splitkv B16 Hq32 Hkv8 d128": ["decode_split_kernel<128, 3>", "decode_merge_kernel<128>"],
    "fa_fwd causal GQA B1 Hq32 Hkv8 T32768 d128": ["fwd_bf16_kernel<128, true, false, false>@1048576"],
    "fa_bwd causal GQA B1 Hq32 Hkv8 T32768 d128": ["bwd_dq_kernel<128, true, false, false>",
                                                   "bwd_dkdv16_kernel<128, true, false>"],
    "fa_fwd_window B1 Hq32 Hkv8 T32768 W4096 d128": ["fwd_bf16_kernel<128, true, true, false>"],
    "fa_bwd_window B1 Hq32 Hkv8 T32768 W4096 d128": ["bwd_dq_kernel<128, true, true, false>",
                                                     "bwd_dkdv16_kernel<128, true, true>"],
    "fa_fwd_fp8 causal B1 H32 T8192 d128": ["fwd_fp8_kernel<128, true>"],
    "fa_fwd_dropout B64 H16 T1024 d64 p0.1": ["fwd_bf16_kernel<64, false, false, true>"],
    "fa_bwd_dropout B64 H16 T1024 d64 p0.1": ["bwd_dq_kernel<64, false, false, true>",
                                              "bwd_dkdv_kernel<64, false, false, true>"],
}


def fwd_flops(B, Hq, Tq, Tk, d, causal):
    pairs = Tq * (Tq + 1) // 2 if causal else Tq * Tk
    return 4.0 * d * pairs * B * Hq


# Source file of each kernel family; every kernel also depends on the shared headers.
_BWD = ("fa_bwd_kernels.hpp", "fa_bwd.hip", "fa_bwd_window.hip")
KERNEL_SOURCES = {"fwd_bf16_kernel": ("fa_fwd.hip",), "fwd_fp8_kernel": ("fa_fwd_fp8.hip",),
                  "bwd_dq_kernel": _BWD, "bwd_dkdv_kernel": _BWD, "bwd_dkdv16_kernel": _BWD,
                  "decode_split_kernel": ("fa_decode.hip",), "decode_merge_kernel": ("fa_decode.hip",)}
SHARED_SOURCES = ("fa_common.hpp", "fa_internal.h")


def source_hash(files=None) -> str:
    """sha256 over the named kernel sources (all of them when None)."""
    if files is None:
        paths = [p for p in glob.glob(os.path.join(CSRC, "*")) if p.endswith((".hip", ".hpp", ".h", ".cpp"))]
    else:
        paths = [os.path.join(CSRC, f) for f in files]
    h = hashlib.sha256()
    for p in sorted(paths):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def unit_source_hash(unit: str) -> str:
    """Hash of the sources the kernels of a traffic unit are built from."""
    files = set(SHARED_SOURCES)
    for spec in TRAFFIC_UNITS[unit]:
        files.update(KERNEL_SOURCES[spec.split("<")[0]])
    return source_hash(sorted(files))


def _fresh_record(path: str, unit: str):
    """The record of `unit` in a profiles/ JSON file, or None when it is
    missing or the unit's kernels changed since the counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    u = rec.get("units", {}).get(unit)
    if u is None or unit not in TRAFFIC_UNITS or u.get("source_sha256") != unit_source_hash(unit):
        return None
    return u


def recorded_traffic(unit: str):
    """Measured HBM bytes per launch of `unit`, or None (not recorded, or the
    kernels changed since the counters were taken)."""
    u = _fresh_record(TRAFFIC_FILE, unit)
    return None if u is None else float(u["bytes"])


def recorded_counters(unit: str):
    """Derived counter figures of `unit` (matrix-core busy fraction, VALU
    co-execution, clock, ...) from profiles/counters.json, or None."""
    u = _fresh_record(COUNTERS_FILE, unit)
    return None if u is None else u.get("derived")


# ------------------------------------------------------------------ GPU timing

class Timer:
    """HIP events around launches on one stream; durations in ms."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = []

    def record(self, fn):
        import torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(self.stream)
        fn()
        e.record(self.stream)
        self.pairs.append((s, e))

    def times(self):
        return [s.elapsed_time(e) for s, e in self.pairs]

    def mean_ms(self):
        return float(np.mean(self.times())) if self.pairs else float("nan")

    def median_ms(self):
        return float(np.median(self.times())) if self.pairs else float("nan")


def timed(calls, steps, warmup, stream):
    """Run `calls` (list of (name, fn)) warmup times untimed, then `steps`
    times between two device synchronisations, with events around each call.
    Returns (wall seconds, {name: Timer})."""
    import torch
    timers = {n: Timer(stream) for n, _ in calls}
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for n, fn in calls:
            timers[n].record(fn)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, timers


def to_device(raw):
    """Seeded host arrays (bf16 bit patterns as uint16, or fp32) -> device tensors."""
    import torch
    out = {}
    for n, a in raw.items():
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return out


def roofline(bound, work, ms, unit_name, algorithmic_bytes=None, peak_tflops=PEAK_BF16_TFLOPS):
    """Roofline entry for one launch unit: `work` is FLOP (bound "mfma", against
    the matrix peak of the unit's dtype) or bytes (bound "hbm") per launch, `ms`
    the launch duration."""
    if bound == "mfma":
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, peak_tflops, "TFLOP/s"
    else:
        achieved, peak, unit = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    out = {"kernel": unit_name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": recorded_traffic(unit_name), "ms": round(ms, 4)}
    if algorithmic_bytes is not None:
        out["algorithmic_bytes"] = algorithmic_bytes
    cnt = recorded_counters(unit_name)
    if cnt is not None:
        out["counters"] = cnt
    return out


def fwd_algorithmic_bytes(B, Hq, Hkv, T, d):
    """HBM bytes the forward cannot avoid: read Q, K, V once, write O and the LSE."""
    return 2 * B * Hq * T * d * 2 + 2 * B * Hkv * T * d * 2 + 4 * B * Hq * T


def bwd_algorithmic_bytes(B, Hq, Hkv, T, d):
    """HBM bytes the backward cannot avoid: read Q, O, dO, LSE and K, V once,
    write dQ, dK, dV, plus the per-row statistics (written once by the dQ
    kernel, read once by the dK/dV kernel)."""
    q_like = B * Hq * T * d * 2
    kv_like = B * Hkv * T * d * 2
    rows = B * Hq * T
    return 3 * q_like + 2 * kv_like + 4 * rows + q_like + 2 * kv_like + 2 * 8 * rows


def _attention_buffers(dev, backward):
    import torch
    from io_aware_softmax_05_amd import fa
    q, k = dev["q"], dev["k"]
    B, Hq, T, d = q.shape
    bufs = {"o": torch.empty_like(q), "lse": torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")}
    if backward:
        bufs.update(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(k))
        n = fa.fa_bwd_workspace_size(B, Hq, T, d)
        bufs["ws"] = torch.empty(n, dtype=torch.uint8, device="cuda")
        bufs["ws_bytes"] = n
    return bufs


def attention_calls(dev, causal, backward, p_drop=0.0, seed=0, offset=0):
    """[(name, fn)] for the forward (and backward) of one layer on device inputs."""
    from io_aware_softmax_05_amd import fa
    q, k, v = dev["q"], dev["k"], dev["v"]
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    scale = d ** -0.5
    b = _attention_buffers(dev, backward)

    def f():
        if p_drop > 0:
            fa.fa_fwd_dropout(q, k, v, b["o"], b["lse"], B, Hq, Hkv, T, T, d, scale, causal, p_drop, seed, offset)
        else:
            fa.fa_fwd(q, k, v, b["o"], b["lse"], B, Hq, Hkv, T, T, d, scale, causal)

    calls = [("fwd", f)]
    if backward:
        do = dev["do"]

        def g():
            args = (q, k, v, b["o"], do, b["lse"], b["dq"], b["dk"], b["dv"], b["ws"], b["ws_bytes"],
                    B, Hq, Hkv, T, T, d, scale, causal)
            if p_drop > 0:
                fa.fa_bwd_dropout(*args, p_drop, seed, offset)
            else:
                fa.fa_bwd(*args)
        calls.append(("bwd", g))
    return calls


DROPOUT_P = 0.1                # attention dropout of the GPT-2-medium layer with dropout
DROPOUT_SEED, DROPOUT_OFFSET = 0x5EED, 0


def _randn_bf16(shape, gen):
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def run_decode(raw, steps, warmup):
    """Split-KV decode on the seeded cache; a device copy of it is used on
    alternate calls so that no call finds the previous call's rows in the MALL."""
    import torch
    from io_aware_softmax_05_amd import fa
    dev = to_device({n: raw[n] for n in ("q", "k", "v")})
    lens = torch.from_numpy(raw["seq_lens"]).cuda()
    q = dev["q"]
    B, Hq, d = q.shape
    Hkv, Tk_max = dev["k"].shape[1], dev["k"].shape[2]
    caches = [(dev["k"], dev["v"]), (dev["k"].clone(), dev["v"].clone())]
    ws_bytes = fa.fa_decode_workspace_size(B, Hq, Tk_max, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    turn = [0]

    def call():
        kc, vc = caches[turn[0] & 1]
        turn[0] += 1
        fa.fa_decode_splitkv(q, kc, vc, lens, o, lse, ws, ws_bytes, B, Hq, Hkv, Tk_max, d, d ** -0.5, 0)

    _, t = timed([("dec", call)], steps, warmup, torch.cuda.current_stream())
    kv_bytes = float(raw["seq_lens"].astype(np.int64).sum()) * Hkv * 2 * d * 2
    io_bytes = 2.0 * B * Hq * d * 2
    return {"median_ms": t["dec"].median_ms(), "bytes": kv_bytes + io_bytes, "sum_lengths": int(raw["seq_lens"].sum())}


def window_pairs(T, W):
    """Visible (query, key) pairs of a square causal band of W keys."""
    W = min(W, T)
    return W * T - W * (W - 1) // 2


def run_window(steps, warmup):
    """Causal sliding-window layer fwd + bwd: B1 Hq32 Hkv8 T32768 d128, W = 4096."""
    import torch
    from io_aware_softmax_05_amd import fa
    B, Hq, Hkv, T, d, W = 1, 32, 8, 32768, 128, 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    q, k, v, do = (_randn_bf16(s, gen) for s in ((B, Hq, T, d), (B, Hkv, T, d), (B, Hkv, T, d), (B, Hq, T, d)))
    b = _attention_buffers({"q": q, "k": k}, True)

    def f():
        fa.fa_fwd_window(q, k, v, b["o"], b["lse"], B, Hq, Hkv, T, T, d, d ** -0.5, W)

    def g():
        fa.fa_bwd_window(q, k, v, b["o"], do, b["lse"], b["dq"], b["dk"], b["dv"], b["ws"], b["ws_bytes"],
                         B, Hq, Hkv, T, T, d, d ** -0.5, W)

    _, t = timed([("fwd", f), ("bwd", g)], steps, warmup, torch.cuda.current_stream())
    ff = 4.0 * d * window_pairs(T, W) * B * Hq
    return {"fwd_ms": t["fwd"].median_ms(), "bwd_ms": t["bwd"].median_ms(), "fwd_flop": ff, "bwd_flop": 2.5 * ff}


def run_fp8(steps, warmup):
    """fp8 forward on the causal long-context shape (B1 H32 T8192 d128): Q, K, V
    drawn N(0,1), quantised per (batch, head) to e4m3 (largest magnitude on 448),
    V handed over transposed."""
    import torch
    from io_aware_softmax_05_amd import fa
    B, H, T, d = 1, 32, 8192, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)

    def quant(x):
        s = (x.abs().amax(dim=(2, 3)) / 448.0).clamp_min(1e-30)
        return (x / s[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8), s.float().contiguous()

    q8, qs = quant(torch.randn((B, H, T, d), generator=gen, device="cuda"))
    k8, ks = quant(torch.randn((B, H, T, d), generator=gen, device="cuda"))
    v8, vs = quant(torch.randn((B, H, T, d), generator=gen, device="cuda"))
    vt8 = v8.transpose(2, 3).contiguous()
    o = torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")

    def call():
        fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, o, lse, B, H, H, T, T, d, d ** -0.5, True)

    _, t = timed([("fp8", call)], steps, warmup, torch.cuda.current_stream())
    return {"median_ms": t["fp8"].median_ms(), "flop": fwd_flops(B, H, T, T, d, True)}


def run_small_f32(raw, steps, warmup):
    """The single-head fp32 workload (B1 H1 T256 d64): latency only."""
    import torch
    from io_aware_softmax_05_amd import fa
    dev = to_device(raw)
    q, k, v = dev["q"], dev["k"], dev["v"]
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 256), dtype=torch.float32, device="cuda")

    def call():
        fa.fa_fwd_f32(q, k, v, o, lse, 1, 1, 1, 256, 256, 64, 0.125, False)

    _, t = timed([("f32", call)], steps, warmup, torch.cuda.current_stream())
    return {"median_ms": t["f32"].median_ms(), "flop": fwd_flops(1, 1, 256, 256, 64, False)}


# ------------------------------------------------------------ clock reading

def frac_at_clock(achieved, peak, mhz):
    """achieved / (peak scaled from the spec clock to `mhz`: one clock, or the
    mean of a list of them); None without a clock."""
    if isinstance(mhz, (int, float)):
        mhz = [mhz]
    if not mhz:
        return None
    mean = sum(mhz) / len(mhz)
    if mean <= 0:
        return None
    return round(achieved / (peak * mean / SPEC_SCLK_MHZ), 4)


def gfx_clocks(amd_smi_json):
    """The gfx engine clocks (MHz, one per XCD) in the JSON of `amd-smi metric --clock`."""
    mhz = []

    def walk(x, key=""):
        if isinstance(x, dict):
            for kk, vv in x.items():
                if kk == "clk" and key.lower().startswith("gfx"):
                    val = vv.get("value") if isinstance(vv, dict) else vv
                    try:
                        mhz.append(float(val))
                    except (TypeError, ValueError):
                        pass
                else:
                    walk(vv, kk if isinstance(vv, dict) else key)
        elif isinstance(x, list):
            for vv in x:
                walk(vv, key)
    walk(amd_smi_json)
    return mhz


def read_sclk_under_load(launch, samples=6, gap=0.3):
    """Engine clock reported by amd-smi while `launch` (the headline kernel) is
    issued back to back: the matrix peak assumes the 2400 MHz top clock, and
    sustained matrix work runs below it. amd-smi reads an instantaneous value,
    so it is sampled `samples` times; "mhz" is the median of the samples' means
    over the XCDs. Returns {"mhz": ..., "samples": [...], ...} or an error."""
    import torch
    box = {"out": []}

    def reader():
        time.sleep(0.5)   # let the clock settle under the load
        try:
            for _ in range(samples):
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                                   text=True, timeout=20)
                if r.returncode != 0:
                    box["rc"] = r.returncode
                    return
                box["out"].append(r.stdout)
                time.sleep(gap)
        except Exception as e:  # noqa: BLE001 - reported, never fatal
            box["err"] = repr(e)

    th = threading.Thread(target=reader)
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() and time.perf_counter() - t0 < 60:
        for _ in range(50):
            launch()
        torch.cuda.synchronize()
    th.join()
    if "err" in box or "rc" in box or not box["out"]:
        return {"mhz": None, "error": box.get("err") or f"amd-smi rc {box.get('rc')}"}
    per_sample = []
    for out in box["out"]:
        try:
            clk = gfx_clocks(json.loads(out))
        except ValueError:
            return {"mhz": None, "error": "amd-smi output is not JSON"}
        if clk:
            per_sample.append(round(sum(clk) / len(clk), 1))
    if not per_sample:
        return {"mhz": None, "error": "no gfx clock in the amd-smi output"}
    return {"mhz": statistics.median(per_sample), "samples": per_sample,
            "source": "amd-smi metric --clock, sampled while the headline kernel runs (mean over XCDs per sample)"}


# ------------------------------------------------------------- CPU baseline

def _pool_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)   # one BLAS thread per worker process: the pool supplies the parallelism


def _oracle_job(job):
    """One unit of oracle work in a worker process (imports no GPU code)."""
    from io_aware_softmax_05_amd import inputs
    from oracle import attention_ref as ref
    kind = job[0]
    if kind == "fwd":          # one head: q [Tq,d], k, v [Tk,d] bit patterns or fp32
        _, q, k, v, scale, causal = job
        ref.attention_fwd(inputs.widen(q)[None, None], inputs.widen(k)[None, None], inputs.widen(v)[None, None],
                          scale, causal)
    elif kind == "fwdbwd":     # one head, forward then backward
        _, q, k, v, do, scale, causal = job
        qq, kk, vv, dd = (inputs.widen(x)[None, None] for x in (q, k, v, do))
        ref.attention_fwd(qq, kk, vv, scale, causal)
        ref.attention_bwd(qq, kk, vv, dd, scale, causal)
    elif kind == "fwd_rows":   # some rows of one head
        _, q, k, v, rows, scale, causal = job
        ref.attention_fwd(inputs.widen(q)[None, None], inputs.widen(k)[None, None], inputs.widen(v)[None, None],
                          scale, causal, rows=rows)
    elif kind == "decode":     # one batch entry: q [Hq,d], caches [Hkv,L,d]
        _, q, k, v, L, scale = job
        ref.decode(inputs.widen(q)[None], inputs.widen(k)[None], inputs.widen(v)[None], np.array([L]), scale)
    else:
        raise ValueError(kind)
    return 0


def _pool_wall(pool, jobs):
    t0 = time.perf_counter()
    list(pool.imap_unordered(_oracle_job, jobs, chunksize=1))
    return time.perf_counter() - t0


def host_info():
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: i.get(k) for k in ("internal_api", "version", "architecture", "num_threads")}
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # noqa: BLE001 - informational
        pass
    return {"cpu_model": cpu, "blas": blas, "affinity_cores": len(os.sched_getaffinity(0)),
            "numpy": np.__version__}


def cpu_baseline(raw, full=False):
    """The fp64 oracle, untouched, timed on the host cores: one job per head
    (or batch entry), spread over a pool of worker processes with one BLAS
    thread each. The headline (`value`) is the whole causal B1 H32 T8192 d128
    forward, median of 3 passes; the other workloads are reported beside it."""
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")          # workers never touch the GPU
    out = {"unit": "TFLOP/s", "cores": cores, "kind": "oracle"}
    out.update(host_info())
    cfg = {}
    with ctx.Pool(cores, initializer=_pool_init) as pool:
        pool.map(_oracle_job, [("fwd", np.zeros((2, 64), np.float32), np.zeros((2, 64), np.float32),
                                np.zeros((2, 64), np.float32), 0.1, False)] * cores)   # start the workers
        # headline: the whole causal 8k forward, every head
        r3 = raw[3]
        w3 = INPUT_WORKLOADS[3]
        jobs = [("fwd", r3["q"][0, h], r3["k"][0, h], r3["v"][0, h], w3.scale, True) for h in range(w3.Hq)]
        walls = [_pool_wall(pool, jobs) for _ in range(3)]
        flop3 = fwd_flops(1, w3.Hq, w3.Tq, w3.Tk, w3.d, True)
        out["value"] = round(flop3 / float(np.median(walls)) / 1e12, 5)
        out["sample"] = (f"the whole {w3.name} (all {w3.Hq} heads, seeded inputs), fp64 numpy three-step oracle, "
                         f"one head per job on {cores} worker processes with one BLAS thread each; median of 3 "
                         f"passes: {', '.join(f'{x:.2f}' for x in walls)} s")
        # single-head fp32 workload: whole, median of 3
        r1, w1 = raw[1], INPUT_WORKLOADS[1]
        walls = [_pool_wall(pool, [("fwd", r1["q"][0, 0], r1["k"][0, 0], r1["v"][0, 0], w1.scale, False)])
                 for _ in range(3)]
        cfg[w1.name] = {"median_s": round(float(np.median(walls)), 5), "passes": 3, "whole_workload": True}
        # GPT-2-medium layer fwd+bwd: whole (1024 heads)
        r2, w2 = raw[2], INPUT_WORKLOADS[2]
        jobs = [("fwdbwd", r2["q"][b, h], r2["k"][b, h], r2["v"][b, h], r2["do"][b, h], w2.scale, False)
                for b in range(w2.B) for h in range(w2.Hq)]
        walls = [_pool_wall(pool, jobs) for _ in range(3)]
        flop2 = 3.5 * fwd_flops(w2.B, w2.Hq, w2.Tq, w2.Tk, w2.d, False)
        cfg[w2.name] = {"median_s": round(float(np.median(walls)), 3), "passes": len(walls),
                        "TFLOP/s": round(flop2 / float(np.median(walls)) / 1e12, 5), "whole_workload": True}
        # split-KV decode: whole (16 batch entries, their cached prefixes)
        r5, w5 = raw[5], INPUT_WORKLOADS[5]
        lens = r5["seq_lens"]
        jobs = [("decode", r5["q"][b], r5["k"][b, :, :int(lens[b])], r5["v"][b, :, :int(lens[b])], int(lens[b]),
                 w5.scale) for b in range(w5.B)]
        walls = [_pool_wall(pool, jobs) for _ in range(3)]
        dec_bytes = float(lens.astype(np.int64).sum()) * w5.Hkv * 2 * w5.d * 2 + 2.0 * w5.B * w5.Hq * w5.d * 2
        cfg[w5.name] = {"median_s": round(float(np.median(walls)), 4), "passes": 3,
                        "GB/s": round(dec_bytes / float(np.median(walls)) / 1e9, 4), "whole_workload": True}
        # causal 32k GQA layer
        r4, w4 = raw[4], INPUT_WORKLOADS[4]
        g = w4.Hq // w4.Hkv
        heads = [(hk * g + i, hk) for hk in (0, w4.Hkv - 1) for i in range(g)]   # KV groups 0 and 7
        flop4 = fwd_flops(1, w4.Hq, w4.Tq, w4.Tk, w4.d, True)
        if full:
            jobs = [("fwdbwd", r4["q"][0, h], r4["k"][0, hk], r4["v"][0, hk], r4["do"][0, h], w4.scale, True)
                    for h, hk in heads]
            wall = _pool_wall(pool, jobs)
            cfg[w4.name] = {"s_for_kv_groups_0_and_7": round(wall, 2), "extrapolated_s": round(wall * w4.Hkv / 2, 1),
                            "TFLOP/s": round(3.5 * flop4 / (wall * w4.Hkv / 2) / 1e12, 5),
                            "extrapolation": f"fwd+bwd of the {len(heads)} query heads of KV groups 0 and 7 timed in "
                                             f"full, scaled x{w4.Hkv // 2} to all {w4.Hkv} groups (heads are "
                                             "independent)"}
        else:
            rows = np.arange(0, w4.Tq, w4.Tq // 256)   # 256 evenly spaced rows per head
            jobs = [("fwd_rows", r4["q"][0, h], r4["k"][0, hk], r4["v"][0, hk], rows, w4.scale, True)
                    for h, hk in heads]
            wall = _pool_wall(pool, jobs)
            scale_up = (w4.Tq / len(rows)) * (w4.Hq / len(heads))
            cfg[w4.name] = {"fwd_rows_s": round(wall, 2), "fwd_extrapolated_s": round(wall * scale_up, 1),
                            "fwd_TFLOP/s": round(flop4 / (wall * scale_up) / 1e12, 5),
                            "extrapolation": f"forward of 256 evenly spaced full-length rows of each of the "
                                             f"{len(heads)} query heads of KV groups 0 and 7 (the oracle computes "
                                             f"every key of a row, masked or not), scaled x{scale_up:g} to the whole "
                                             "forward; the backward is timed only with --cpu-full"}
    out["configs"] = cfg
    return out


# ----------------------------------------------------------- counter records

def kernel_key(name: str) -> str:
    """'void fa::k<128, true, fa::Cfg<128, 4>, true>(fa::Args)' -> 'k<128, true, true>':
    the template arguments that pick the variant, without tuning-config structs."""
    base = name[len("void fa::"):] if name.startswith("void fa::") else name
    head, lt, rest = base.partition("<")
    if not lt:
        return base.split("(")[0]
    args, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "<":
            depth += 1
        elif ch == ">":
            if depth == 0:
                break
            depth -= 1
        if ch == "," and depth == 0:
            args.append(cur.strip()); cur = ""
        else:
            cur += ch
    args.append(cur.strip())
    return head + "<" + ", ".join(a for a in args if not a.startswith("fa::")) + ">"


def _counter_means(path, counter):
    """Mean per-dispatch value of `counter` for each fa:: kernel (and the
    runtime's copy kernel) in one rocprofv3 counter_collection.csv."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if name.startswith("void fa::"):
                key = kernel_key(name)
            elif "copyBuffer" in name:
                key = "copy"
            else:
                continue
            per[(key, int(r["Grid_Size"]))][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def _match_unit_kernels(table, unit):
    """(kernel key, grid) entries of a counter table that make up `unit`."""
    found = []
    for spec in TRAFFIC_UNITS[unit]:
        k, _, grid = spec.partition("@")
        hits = [nk for nk in table if nk[0] == k and (not grid or nk[1] == int(grid))]
        if len(hits) != 1:
            return None
        found.append(hits[0])
    return found


def record_traffic(d):
    def one(name, counter):
        paths = glob.glob(os.path.join(d, name, "*counter_collection.csv"))
        if not paths:
            raise SystemExit(f"missing {name}/*counter_collection.csv under {d}")
        return _counter_means(paths[0], counter)
    fetch, write = one("fetch_all", "FETCH_SIZE"), one("write_all", "WRITE_SIZE")

    def copy_value(m):
        vals = [v for (n, _), v in m.items() if n == "copy"]
        if len(vals) != 1:
            raise SystemExit(f"expected one copy kernel record, found {len(vals)}")
        return vals[0]
    cf, cw = copy_value(one("fetch_copy", "FETCH_SIZE")), copy_value(one("write_copy", "WRITE_SIZE"))
    f_fac, w_fac = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    units = {}
    for unit in TRAFFIC_UNITS:
        hits = _match_unit_kernels(fetch, unit)
        if hits is None:
            raise SystemExit(f"the counter records do not match the kernels of {unit}")
        ks, total = {}, 0.0
        for nk in hits:
            ks[f"{nk[0]} grid {nk[1]}"] = {"fetch_kib": round(fetch[nk], 1), "write_kib": round(write.get(nk, 0.0), 1)}
            total += fetch[nk] * 1024 * f_fac + write.get(nk, 0.0) * 1024 * w_fac
        units[unit] = {"bytes": round(total), "source_sha256": unit_source_hash(unit), "kernels": ks}
    rec = {"source_sha256": source_hash(),   # all kernel sources; each unit also records its own
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
           "units": units}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


# Instruction and cycle counters (rocprofv3 --pmc passes of at most 8 SQ
# counters each). Per-dispatch values are sums over the 8 XCDs and their SIMDs;
# GRBM_GUI_ACTIVE counts each XCD's busy clocks, so GRBM_GUI_ACTIVE / 8 over
# the dispatch's duration is the engine clock it ran at.
COUNTER_PASSES = [
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_MFMA",
     "SQ_INSTS_VALU", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
     "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_INSTS_VALU_TRANS_F32", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_VALU_MFMA_MOPS_F8",
     "SQ_WAVES", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_ACTIVE_INST_MISC", "GRBM_GUI_ACTIVE"],
]
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def _counter_table(paths):
    """{(kernel key, grid): {counter: mean per dispatch, "_duration_s": mean}} over counter CSVs."""
    vals = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    durs = collections.defaultdict(dict)
    for path in paths:
        tag = os.path.dirname(path)
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if not name.startswith("void fa::"):
                    continue
                key = (kernel_key(name), int(r["Grid_Size"]))
                did = (tag, r["Dispatch_Id"])
                vals[key][r["Counter_Name"]][did] += float(r["Counter_Value"])
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    durs[key][did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = {}
    for key, cs in vals.items():
        out[key] = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        if durs[key]:
            out[key]["_duration_s"] = sum(durs[key].values()) / len(durs[key])
    return out


def derived_counters(c):
    """Fractions of the kernel's time (per SIMD or CU) from one kernel's counter means."""
    g = c.get("GRBM_GUI_ACTIVE")
    d = {}
    if not g:
        return d
    cyc = g / N_XCD                                   # busy clocks of one XCD
    if c.get("_duration_s"):
        d["duration_us_under_counters"] = round(c["_duration_s"] * 1e6, 1)
        if c["_duration_s"] >= 50e-6:   # shorter dispatches: launch overhead dominates the ratio
            d["clock_mhz"] = round(cyc / c["_duration_s"] / 1e6)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        d["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD), 4)
        if c["SQ_VALU_MFMA_BUSY_CYCLES"] > 0 and "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
            d["valu_coexec_of_mfma_busy"] = round(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
    if "SQ_ACTIVE_INST_VALU" in c:                   # quad-cycles summed over a CU's 4 SIMDs
        d["valu_busy"] = round(c["SQ_ACTIVE_INST_VALU"] / (cyc * N_CU), 4)
    if "SQ_LDS_IDX_ACTIVE" in c:
        d["lds_busy"] = round(c["SQ_LDS_IDX_ACTIVE"] / (cyc * N_CU), 4)
    if c.get("SQ_WAVE_CYCLES"):
        for k, name in (("SQ_WAIT_ANY", "wave_waiting"), ("SQ_WAIT_INST_ANY", "wave_waiting_for_issue"),
                        ("SQ_WAIT_INST_LDS", "wave_waiting_for_lds_issue")):
            if k in c:
                d[name] = round(c[k] / c["SQ_WAVE_CYCLES"], 4)
    m = c.get("SQ_INSTS_MFMA")
    if m:
        if "SQ_INSTS_VALU" in c:
            d["valu_insts_per_mfma"] = round((c["SQ_INSTS_VALU"] - m) / m, 3)
        for k, name in (("SQ_INSTS_VALU_TRANS_F32", "exp_log_insts_per_mfma"), ("SQ_INSTS_LDS", "lds_insts_per_mfma"),
                        ("SQ_INSTS_SALU", "salu_insts_per_mfma")):
            if k in c:
                d[name] = round(c[k] / m, 3)
    for k, name in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", "mfma_bf16_flop"), ("SQ_INSTS_VALU_MFMA_MOPS_F8", "mfma_fp8_flop")):
        if c.get(k):
            d[name] = c[k] * 512
    if "SQ_LDS_BANK_CONFLICT" in c:
        d["lds_bank_conflict_cycles"] = c["SQ_LDS_BANK_CONFLICT"]
    return d


def record_counters(d):
    paths = sorted(glob.glob(os.path.join(d, "*", "*counter_collection.csv")))
    if not paths:
        raise SystemExit(f"no */*counter_collection.csv under {d}")
    table = _counter_table(paths)
    units = {}
    for unit in TRAFFIC_UNITS:
        hits = _match_unit_kernels(table, unit)
        if hits is None:
            continue
        ks = {f"{k} grid {g}": {"derived": derived_counters(table[(k, g)]),
                                "counters": {c: round(v, 1) for c, v in sorted(table[(k, g)].items())}}
              for k, g in hits}
        units[unit] = {"source_sha256": unit_source_hash(unit), "kernels": ks,
                       "derived": {kk: vv["derived"] for kk, vv in ks.items()}}
    rec = {"note": "rocprofv3 --pmc passes (see profiles/counters.md); fractions are of the kernel's busy clocks",
           "passes": COUNTER_PASSES, "units": units}
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({u: v["derived"] for u, v in units.items()}, indent=1))
    return 0


def summarize_trace(d):
    """Markdown table of the fa:: kernels in a rocprofv3 --kernel-trace run:
    per (kernel, grid size) calls and durations, registers and LDS."""
    paths = glob.glob(os.path.join(d, "*kernel_trace.csv"))
    if not paths:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    rows = collections.defaultdict(list)
    info = {}
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not name.startswith("void fa::"):
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            key = (kernel_key(name), grid)
            rows[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
            info[key] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"], r["Scratch_Size"],
                         int(r["Workgroup_Size_X"]))
    out = ["| kernel | grid (threads) | calls | avg us | min us | max us | VGPR | AGPR | LDS B | scratch B | block |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(rows, key=lambda k: -sum(rows[k])):
        t = rows[key]
        v, a, lds, scr, blk = info[key]
        out.append(f"| `{key[0]}` | {key[1]} | {len(t)} | {np.mean(t):.1f} | {min(t):.1f} | {max(t):.1f} | {v} | {a} | "
                   f"{lds} | {scr} | {blk} |")
    print("\n".join(out))
    return 0


# ---------------------------------------------------------------------- main

INPUT_WORKLOADS = None   # inputs.WORKLOADS, bound in main() (workers import it themselves)


def main():
    global INPUT_WORKLOADS
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="oracle baseline with the 32k GQA layer's fwd+bwd for KV groups 0 and 7 in full "
                         "(minutes of CPU time)")
    ap.add_argument("--no-extras", action="store_true", help="headline only")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the amd-smi clock reading (profiled runs: a profiler loaded into every child "
                         "process makes starting amd-smi unsafe)")
    ap.add_argument("--only", choices=["headline", "step", "gqa32k", "decode", "dropout", "fp8", "window", "f32",
                                       "copy"],
                    help="run one measurement alone (profiling runs); 'copy' runs a plain device copy "
                         "of 1 GiB, the calibration for HBM byte counters")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/hbm_traffic.json from rocprofv3 counter runs under DIR (no GPU needed)")
    ap.add_argument("--record-counters", metavar="DIR",
                    help="write profiles/counters.json from rocprofv3 --pmc passes in DIR/<pass>/ (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown table of the fa:: kernels of a rocprofv3 --kernel-trace run in DIR")
    ap.add_argument("--print-counter-passes", action="store_true",
                    help="print the counter passes, one comma-separated line each (for the profiling commands)")
    args = ap.parse_args()
    if args.print_counter_passes:
        for p in COUNTER_PASSES:
            print(",".join(p))
        return 0
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.record_traffic:
        return record_traffic(args.record_traffic)
    if args.record_counters:
        return record_counters(args.record_counters)
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (there is no multi-GPU path); --gpus must be 1"}))
        return 2

    import torch
    from io_aware_softmax_05_amd import fa, inputs
    INPUT_WORKLOADS = inputs.WORKLOADS
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    fa.load_library()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    W = inputs.WORKLOADS

    if args.only == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": max(1, args.steps)}), flush=True)
        return 0

    want = (lambda name: args.only is None or args.only == name)
    extras = not args.no_extras and args.only is None
    raw = {}
    if want("headline") or not args.no_cpu_baseline:
        raw[3] = inputs.workload_inputs(W[3])
    out = {"targets": {}}

    # ---- targets (before the headline; their inputs are freed afterwards)
    if extras or want("step"):
        raw[2] = inputs.workload_inputs(W[2])
        w = W[2]
        dev = to_device(raw[2])
        wall, t = timed(attention_calls(dev, w.causal, True), 20, 5, stream)
        ff = fwd_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal)
        out["targets"]["GPT-2-medium fwd+bwd B64 H16 T1024 d64 step"] = {
            "ms_per_step": round(wall * 1e3 / 20, 4), "TFLOP/s": round(3.5 * ff / (wall / 20) / 1e12, 2)}
        out["targets"]["fa_fwd B64 H16 T1024 d64"] = roofline(
            "mfma", ff, t["fwd"].median_ms(), "fa_fwd B64 H16 T1024 d64",
            fwd_algorithmic_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.d))
        out["targets"]["fa_bwd B64 H16 T1024 d64"] = roofline(
            "mfma", 2.5 * ff, t["bwd"].median_ms(), "fa_bwd B64 H16 T1024 d64",
            bwd_algorithmic_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.d))
        del dev
        torch.cuda.empty_cache()
    if extras or want("gqa32k"):
        raw[4] = inputs.workload_inputs(W[4])
        w = W[4]
        dev = to_device(raw[4])
        _, t = timed(attention_calls(dev, w.causal, True), 3, 1, stream)
        ff = fwd_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal)
        out["targets"]["fa_fwd causal GQA B1 Hq32 Hkv8 T32768 d128"] = roofline(
            "mfma", ff, t["fwd"].median_ms(), "fa_fwd causal GQA B1 Hq32 Hkv8 T32768 d128",
            fwd_algorithmic_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.d))
        out["targets"]["fa_bwd causal GQA B1 Hq32 Hkv8 T32768 d128"] = roofline(
            "mfma", 2.5 * ff, t["bwd"].median_ms(), "fa_bwd causal GQA B1 Hq32 Hkv8 T32768 d128",
            bwd_algorithmic_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.d))
        del dev
        torch.cuda.empty_cache()
    if extras or want("decode"):
        raw[5] = inputs.workload_inputs(W[5])
        dec = run_decode(raw[5], 50, 10)
        u = "fa_decode_splitkv B16 Hq32 Hkv8 d128"
        out["targets"][u] = roofline("hbm", dec["bytes"], dec["median_ms"], u, dec["bytes"])
        out["targets"][u]["sum_lengths"] = dec["sum_lengths"]
        torch.cuda.empty_cache()
    if extras or want("window"):
        sw = run_window(5, 2)
        for ph in ("fwd", "bwd"):
            u = f"fa_{ph}_window B1 Hq32 Hkv8 T32768 W4096 d128"
            out["targets"][u] = roofline("mfma", sw[f"{ph}_flop"], sw[f"{ph}_ms"], u)
        torch.cuda.empty_cache()
    if extras or want("fp8"):
        f8 = run_fp8(50, 10)
        u = "fa_fwd_fp8 causal B1 H32 T8192 d128"
        out["targets"][u] = roofline("mfma", f8["flop"], f8["median_ms"], u, peak_tflops=PEAK_FP8_TFLOPS)
        torch.cuda.empty_cache()
    if extras or want("dropout"):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(2)
        w = W[2]
        dev = {n: _randn_bf16((w.B, w.Hq, w.Tq, w.d), gen) for n in ("q", "k", "v", "do")}
        _, t = timed(attention_calls(dev, False, True, DROPOUT_P, DROPOUT_SEED, DROPOUT_OFFSET), 20, 5, stream)
        ff = fwd_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, False)
        out["targets"]["fa_fwd_dropout B64 H16 T1024 d64 p0.1"] = roofline(
            "mfma", ff, t["fwd"].median_ms(), "fa_fwd_dropout B64 H16 T1024 d64 p0.1")
        out["targets"]["fa_bwd_dropout B64 H16 T1024 d64 p0.1"] = roofline(
            "mfma", 2.5 * ff, t["bwd"].median_ms(), "fa_bwd_dropout B64 H16 T1024 d64 p0.1",
            bwd_algorithmic_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.d))
        del dev
        torch.cuda.empty_cache()
    if extras or want("f32"):
        raw[1] = inputs.workload_inputs(W[1])
        f32 = run_small_f32(raw[1], 50, 10)
        out["latency"] = {"fa_fwd_f32 B1 H1 T256 d64": {"median_us": round(f32["median_ms"] * 1e3, 2),
                                                        "flop": f32["flop"], "bound": "latency"}}
    if args.only is not None and args.only != "headline":
        print(json.dumps(out), flush=True)
        return 0

    # ---- headline: fa_fwd over the causal long-context layer
    w = W[3]
    dev = to_device(raw[3])
    calls = attention_calls(dev, w.causal, False)
    wall, t = timed(calls, args.steps, args.warmup, stream)
    flop = fwd_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal)
    ms_step = wall * 1e3 / args.steps
    res = {
        "metric": METRIC, "value": round(flop / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), the parity tests' inputs)",
        "config": {"workload": "causal long-context attention forward (Llama-3-8B layer shape)", "B": w.B,
                   "Hq": w.Hq, "Hkv": w.Hkv, "seq_len": w.Tq, "head_dim": w.d, "causal": True,
                   "scale": w.scale, "step": "fa_fwd", "flop_per_step": flop,
                   "flop_convention": "4*d per visible (query, key) pair; T(T+1)/2 causal pairs per head"},
        # the step's only launch, fwd_bf16_kernel<128, true>
        "roofline": roofline("mfma", flop, t["fwd"].mean_ms(), HEADLINE_UNIT,
                             fwd_algorithmic_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.d)),
    }
    res["roofline"]["median_ms"] = round(t["fwd"].median_ms(), 4)
    if extras and not args.no_clock:
        sclk = read_sclk_under_load(calls[0][1])
        res["roofline"]["sclk_under_load"] = sclk
        res["roofline"]["sclk_spec_mhz"] = SPEC_SCLK_MHZ
        at = frac_at_clock(res["roofline"]["achieved"], res["roofline"]["peak"], sclk.get("mhz"))
        if at is not None:   # the same peak scaled to the clock amd-smi read under the load
            res["roofline"]["frac_at_sclk_under_load"] = at
    # the same peak scaled to the clock the counter run measured for this kernel
    # (GRBM_GUI_ACTIVE over the dispatch's duration)
    for c in (res["roofline"].get("counters") or {}).values():
        at = frac_at_clock(res["roofline"]["achieved"], res["roofline"]["peak"], c.get("clock_mhz"))
        if at is not None:
            res["roofline"]["frac_at_counter_clock"] = at
            break
    del dev
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        for n in (1, 2, 4, 5):
            if n not in raw:
                raw[n] = inputs.workload_inputs(W[n])
        res["cpu_baseline"] = cpu_baseline(raw, full=args.cpu_full)
    res.update({k: v for k, v in out.items() if v})
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
