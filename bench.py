#!/usr/bin/env python3
"""Benchmark of the exact tiled-attention library on one MI355X.

    python bench.py [--steps K] [--warmup W]

One step is one pass of the hot path over one batch: fa_fwd then fa_bwd
(recomputation from the saved LSE) on the GPT-2-medium attention layer
(B64 H16 T1024 d64, bf16, non-causal, scale 1/8), with Q, K, V, dO already
resident in HBM. W untimed steps, then K steps timed between two device
synchronisations; HIP events recorded around every launch, on the stream the
kernels run on, give per-launch durations.

After the timed region, in the same run (not part of `value`), under "targets":
  * the causal long-context forward (B1 H32 T8192 d128) and split-KV decoding
    (B16 Hq32 Hkv8, lengths U[4096, 32768] from seed 5, d128), each the median
    of 50 launches after 10 untimed;
  * the causal 32k GQA layer (B1 Hq32 Hkv8 T32768 d128) fwd and bwd, the
    sliding-window layer (same, W4096) fwd and bwd, the fp8 causal forward
    (B1 H32 T8192 d128) and the GPT-2-medium layer with dropout p = 0.1 fwd and
    bwd; the fp32 single-head forward (B1 H1 T256 d64) as a latency;
  * the fp64 CPU oracle is timed on a bounded sample of the step's workload.
Prints one JSON line.

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
reported as null until the counters are taken again.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak (AMD spec)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak (AMD spec)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak (AMD spec)

COPY_BYTES = 1 << 30          # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "io_aware_softmax_05_amd", "csrc")

METRIC = "attention fwd/bwd TFLOPS and % of MI355X bf16 MFMA peak; decode HBM GB/s"

WORKLOADS = {
    # name: (B, Hq, Hkv, T, d, causal, seed)
    "gpt2-medium-fwd-bwd": (64, 16, 16, 1024, 64, False, 2),
    "causal-8k-fwd": (1, 32, 32, 8192, 128, True, 3),
    "causal-32k-gqa-fwd-bwd": (1, 32, 8, 32768, 128, True, 4),
}
DECODE = dict(B=16, Hq=32, Hkv=8, Tk_max=32768, d=128, seed=5)

# Launch units whose HBM traffic is recorded: unit -> kernel names (prefix of
# the demangled name, up to the argument list).
TRAFFIC_UNITS = {
    "fa_fwd B64 H16 T1024 d64": ["fwd_bf16_kernel<64, false, false, false>"],
    "fa_bwd B64 H16 T1024 d64": ["bwd_dq_kernel<64, false, false, false>", "bwd_dkdv_kernel<64, false, false, false>"],
    # the causal 8k and 32k forwards run the same kernel: told apart by grid size (threads)
    "fa_fwd causal B1 H32 T8192 d128": ["fwd_bf16_kernel<128, true, false, false>@524288"],
    "fa_decode_splitkv B16 Hq32 Hkv8 d128": ["decode_split_kernel<128, 3>", "decode_merge_kernel<128>"],
    "fa_fwd causal GQA B1 Hq32 Hkv8 T32768 d128": ["fwd_bf16_kernel<128, true, false, false>@2097152"],
    "fa_bwd causal GQA B1 Hq32 Hkv8 T32768 d128": ["bwd_dq_kernel<128, true, false, false>",
                                                   "bwd_dkdv_kernel<128, true, false, false>"],
    "fa_fwd_window B1 Hq32 Hkv8 T32768 W4096 d128": ["fwd_bf16_kernel<128, true, true, false>"],
    "fa_bwd_window B1 Hq32 Hkv8 T32768 W4096 d128": ["bwd_dq_kernel<128, true, true, false>",
                                                     "bwd_dkdv_kernel<128, true, true, false>"],
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
                  "bwd_dq_kernel": _BWD, "bwd_dkdv_kernel": _BWD,
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


def recorded_traffic(unit: str):
    """Measured HBM bytes per launch of `unit`, or None (not recorded, or the
    kernels changed since the counters were taken)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    u = rec.get("units", {}).get(unit)
    if u is None or unit not in TRAFFIC_UNITS or u.get("source_sha256") != unit_source_hash(unit):
        return None
    return float(u["bytes"])


# ------------------------------------------------------------------ GPU timing

def _randn_bf16(shape, gen):
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


class Timer:
    """HIP events around launches on one stream; averages in ms."""

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

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs])) if self.pairs else float("nan")

    def median_ms(self):
        return float(np.median([s.elapsed_time(e) for s, e in self.pairs])) if self.pairs else float("nan")


DROPOUT_P = 0.1                # attention dropout of the GPT-2-medium layer with dropout
DROPOUT_SEED, DROPOUT_OFFSET = 0x5EED, 0


def run_attention(name, steps, warmup, backward=True, p_drop=0.0):
    import torch
    from io_aware_softmax_05_amd import fa
    B, Hq, Hkv, T, d, causal, seed = WORKLOADS[name]
    scale = d ** -0.5
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = _randn_bf16((B, Hq, T, d), gen)
    k = _randn_bf16((B, Hkv, T, d), gen)
    v = _randn_bf16((B, Hkv, T, d), gen)
    do = _randn_bf16((B, Hq, T, d), gen)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, T, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    t_fwd, t_bwd = Timer(stream), Timer(stream)

    def f():
        if p_drop > 0:
            fa.fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, T, T, d, scale, causal, p_drop, DROPOUT_SEED,
                              DROPOUT_OFFSET, stream)
        else:
            fa.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, T, T, d, scale, causal, stream)

    def b():
        if p_drop > 0:
            fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, T, T, d, scale, causal,
                              p_drop, DROPOUT_SEED, DROPOUT_OFFSET, stream)
        else:
            fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, T, T, d, scale, causal, stream)

    for _ in range(warmup):
        f()
        if backward:
            b()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        t_fwd.record(f)
        if backward:
            t_bwd.record(b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ff = fwd_flops(B, Hq, T, T, d, causal)
    res = {"workload": name, "B": B, "Hq": Hq, "Hkv": Hkv, "T": T, "d": d, "causal": causal,
           "wall_s": wall, "ms_per_step": wall * 1e3 / steps,
           "fwd_ms": t_fwd.mean_ms(), "fwd_median_ms": t_fwd.median_ms(), "fwd_flop": ff,
           "step_flop": ff * (3.5 if backward else 1.0)}
    if backward:
        res["bwd_ms"] = t_bwd.mean_ms()
        res["bwd_median_ms"] = t_bwd.median_ms()
        res["bwd_flop"] = 2.5 * ff
    res["host"] = {"q": q, "k": k, "v": v, "do": do}
    return res


def run_decode(steps, warmup):
    import torch
    from io_aware_softmax_05_amd import fa, inputs
    B, Hq, Hkv, Tk_max, d = (DECODE[k] for k in ("B", "Hq", "Hkv", "Tk_max", "d"))
    lens_np = inputs.decode_lengths(inputs.make_rng(DECODE["seed"]), B)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(DECODE["seed"])
    q = _randn_bf16((B, Hq, d), gen)
    # two cache copies (1 GiB per tensor each), used in turn, so that no call
    # finds the previous call's rows in the 256 MiB MALL
    caches = [(_randn_bf16((B, Hkv, Tk_max, d), gen), _randn_bf16((B, Hkv, Tk_max, d), gen)) for _ in range(2)]
    lens = torch.from_numpy(lens_np).cuda()
    ws_bytes = fa.fa_decode_workspace_size(B, Hq, Tk_max, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    t = Timer(stream)

    turn = [0]

    def call():
        kc, vc = caches[turn[0] & 1]
        turn[0] += 1
        fa.fa_decode_splitkv(q, kc, vc, lens, o, lse, ws, ws_bytes, B, Hq, Hkv, Tk_max, d, d ** -0.5, 0, stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    for _ in range(steps):
        t.record(call)
    torch.cuda.synchronize()
    kv_bytes = float(lens_np.astype(np.int64).sum()) * Hkv * 2 * d * 2
    io_bytes = 2.0 * B * Hq * d * 2
    return {"ms": t.mean_ms(), "median_ms": t.median_ms(), "bytes": kv_bytes + io_bytes,
            "sum_lengths": int(lens_np.sum())}


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
    q = _randn_bf16((B, Hq, T, d), gen)
    k = _randn_bf16((B, Hkv, T, d), gen)
    v = _randn_bf16((B, Hkv, T, d), gen)
    do = _randn_bf16((B, Hq, T, d), gen)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, T, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    t_f, t_b = Timer(stream), Timer(stream)

    def f():
        fa.fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, T, T, d, d ** -0.5, W, stream)

    def b():
        fa.fa_bwd_window(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, T, T, d, d ** -0.5, W, stream)

    for _ in range(warmup):
        f()
        b()
    torch.cuda.synchronize()
    for _ in range(steps):
        t_f.record(f)
        t_b.record(b)
    torch.cuda.synchronize()
    ff = 4.0 * d * window_pairs(T, W) * B * Hq
    return {"fwd_ms": t_f.median_ms(), "bwd_ms": t_b.median_ms(), "fwd_flop": ff, "bwd_flop": 2.5 * ff}


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
    stream = torch.cuda.current_stream()
    t = Timer(stream)

    def call():
        fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, o, lse, B, H, H, T, T, d, d ** -0.5, True, stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    for _ in range(steps):
        t.record(call)
    torch.cuda.synchronize()
    return {"median_ms": t.median_ms(), "flop": fwd_flops(B, H, T, T, d, True)}


def run_small_f32(steps, warmup):
    """The single-head fp32 workload (B1 H1 T256 d64): latency only."""
    import torch
    from io_aware_softmax_05_amd import fa
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    q, k, v = (torch.randn((1, 1, 256, 64), generator=gen, device="cuda", dtype=torch.float32) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 256), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    t = Timer(stream)

    def call():
        fa.fa_fwd_f32(q, k, v, o, lse, 1, 1, 1, 256, 256, 64, 0.125, False, stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    for _ in range(steps):
        t.record(call)
    torch.cuda.synchronize()
    return {"median_ms": t.median_ms(), "flop": fwd_flops(1, 1, 256, 256, 64, False)}


def roofline(bound, work, ms, unit_name, algorithmic_bytes=None, peak_tflops=PEAK_BF16_TFLOPS):
    """Roofline entry for one launch unit: `work` is FLOP (bound "mfma", against
    the matrix peak of the unit's dtype) or bytes (bound "hbm") per launch, `ms`
    the mean launch duration."""
    if bound == "mfma":
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, peak_tflops, "TFLOP/s"
    else:
        achieved, peak, unit = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    out = {"kernel": unit_name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": recorded_traffic(unit_name), "ms": round(ms, 4)}
    if algorithmic_bytes is not None:
        out["algorithmic_bytes"] = algorithmic_bytes
    return out


def bwd_algorithmic_bytes(B, Hq, Hkv, T, d):
    """HBM bytes the backward cannot avoid: read Q, O, dO, LSE and K, V once,
    write dQ, dK, dV, plus the per-row statistics (written once by the dQ
    kernel, read once by the dK/dV kernel)."""
    q_like = B * Hq * T * d * 2
    kv_like = B * Hkv * T * d * 2
    rows = B * Hq * T
    return 3 * q_like + 2 * kv_like + 4 * rows + q_like + 2 * kv_like + 2 * 8 * rows


# ------------------------------------------------------------- CPU baseline

def cpu_baseline(res, seconds):
    """The fp64 oracle, untouched, on whole (batch, head) slices of the same
    workload until about `seconds` of CPU work; reported in the step's unit."""
    from oracle import attention_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))
    B, Hq, Hkv, T, d, causal = (res[k] for k in ("B", "Hq", "Hkv", "T", "d", "causal"))
    h = res["host"]
    g = Hq // Hkv
    scale = d ** -0.5
    done, t0 = 0, time.perf_counter()
    while True:
        b, hq = divmod(done, Hq)
        hk = hq // g
        sl = lambda t, hh: t[b:b + 1, hh:hh + 1].float().cpu().numpy().astype(np.float64)  # noqa: E731
        qh, kh, vh, doh = sl(h["q"], hq), sl(h["k"], hk), sl(h["v"], hk), sl(h["do"], hq)
        ref.attention_fwd(qh, kh, vh, scale, causal)
        ref.attention_bwd(qh, kh, vh, doh, scale, causal)
        done += 1
        if time.perf_counter() - t0 >= seconds or done >= B * Hq:
            break
    elapsed = time.perf_counter() - t0
    per_head_flop = res["step_flop"] / (B * Hq)
    return {"value": per_head_flop * done / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {B * Hq} (batch, head) slices of the step's workload, fp64 numpy fwd+bwd, "
                      f"{elapsed:.1f} s wall"}


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
    for unit, kernels in TRAFFIC_UNITS.items():
        ks = {}
        total = 0.0
        for spec in kernels:
            k, _, grid = spec.partition("@")
            hits = [nk for nk in fetch if nk[0] == k and (not grid or nk[1] == int(grid))]
            if len(hits) != 1:
                raise SystemExit(f"{len(hits)} counter records match kernel {spec}: {hits}")
            nk = hits[0]
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


# ---------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the causal 8k and decode measurements")
    ap.add_argument("--only", choices=["step", "causal-8k-fwd", "causal-8k-fp8", "decode", "dropout", "copy"],
                    help="run one measurement alone (profiling runs); 'copy' runs a plain device copy "
                         "of 1 GiB, the calibration for HBM byte counters")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/hbm_traffic.json from rocprofv3 counter runs under DIR (no GPU needed)")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(args.record_traffic)
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (there is no multi-GPU path); --gpus must be 1"}))
        return 2

    import torch
    from io_aware_softmax_05_amd import fa
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    fa.load_library()
    torch.cuda.set_device(0)

    if args.only == "causal-8k-fwd":
        r = run_attention("causal-8k-fwd", args.steps, args.warmup, backward=False)
        r.pop("host")
        print(json.dumps(r), flush=True)
        return 0
    if args.only == "causal-8k-fp8":
        print(json.dumps(run_fp8(args.steps, args.warmup)), flush=True)
        return 0
    if args.only == "decode":
        print(json.dumps(run_decode(args.steps, args.warmup)), flush=True)
        return 0
    if args.only == "dropout":
        r = run_attention("gpt2-medium-fwd-bwd", args.steps, args.warmup, backward=True, p_drop=DROPOUT_P)
        r.pop("host")
        print(json.dumps(r), flush=True)
        return 0
    if args.only == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": max(1, args.steps)}), flush=True)
        return 0
    if args.only == "step":
        args.no_extras = True
        args.no_cpu_baseline = True

    res = run_attention("gpt2-medium-fwd-bwd", args.steps, args.warmup, backward=True)
    B, Hq, Hkv, T, d = (res[k] for k in ("B", "Hq", "Hkv", "T", "d"))
    value = res["step_flop"] / (res["ms_per_step"] * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GPT-2-medium attention layer fwd+bwd", "B": B, "Hq": Hq, "Hkv": Hkv,
                   "seq_len": T, "head_dim": d, "causal": res["causal"], "step": "fa_fwd + fa_bwd",
                   "flop_per_step": res["step_flop"]},
        # the dominant launch of the step: fa_bwd (its two kernels)
        "roofline": roofline("mfma", res["bwd_flop"], res["bwd_ms"], "fa_bwd B64 H16 T1024 d64",
                             bwd_algorithmic_bytes(B, Hq, Hkv, T, d)),
        "phases": {"fa_fwd": roofline("mfma", res["fwd_flop"], res["fwd_ms"], "fa_fwd B64 H16 T1024 d64")},
    }
    if not args.no_extras:
        torch.cuda.empty_cache()
        # the targets: 10 untimed launches, then the median of 50 timed ones
        tgt = run_attention("causal-8k-fwd", 50, 10, backward=False)
        tgt.pop("host")
        out["targets"] = {"fa_fwd causal B1 H32 T8192 d128":
                          roofline("mfma", tgt["fwd_flop"], tgt["fwd_median_ms"], "fa_fwd causal B1 H32 T8192 d128")}
        torch.cuda.empty_cache()
        dec = run_decode(50, 10)
        out["targets"]["fa_decode_splitkv B16 Hq32 Hkv8 d128"] = roofline(
            "hbm", dec["bytes"], dec["median_ms"], "fa_decode_splitkv B16 Hq32 Hkv8 d128", dec["bytes"])
        out["targets"]["fa_decode_splitkv B16 Hq32 Hkv8 d128"]["sum_lengths"] = dec["sum_lengths"]
        torch.cuda.empty_cache()
        g32 = run_attention("causal-32k-gqa-fwd-bwd", 3, 1, backward=True)
        g32.pop("host")
        out["targets"]["fa_fwd causal GQA B1 Hq32 Hkv8 T32768 d128"] = roofline(
            "mfma", g32["fwd_flop"], g32["fwd_ms"], "fa_fwd causal GQA B1 Hq32 Hkv8 T32768 d128")
        out["targets"]["fa_bwd causal GQA B1 Hq32 Hkv8 T32768 d128"] = roofline(
            "mfma", g32["bwd_flop"], g32["bwd_ms"], "fa_bwd causal GQA B1 Hq32 Hkv8 T32768 d128")
        torch.cuda.empty_cache()
        sw = run_window(5, 2)
        out["targets"]["fa_fwd_window B1 Hq32 Hkv8 T32768 W4096 d128"] = roofline(
            "mfma", sw["fwd_flop"], sw["fwd_ms"], "fa_fwd_window B1 Hq32 Hkv8 T32768 W4096 d128")
        out["targets"]["fa_bwd_window B1 Hq32 Hkv8 T32768 W4096 d128"] = roofline(
            "mfma", sw["bwd_flop"], sw["bwd_ms"], "fa_bwd_window B1 Hq32 Hkv8 T32768 W4096 d128")
        torch.cuda.empty_cache()
        f8 = run_fp8(50, 10)
        out["targets"]["fa_fwd_fp8 causal B1 H32 T8192 d128"] = roofline(
            "mfma", f8["flop"], f8["median_ms"], "fa_fwd_fp8 causal B1 H32 T8192 d128", peak_tflops=PEAK_FP8_TFLOPS)
        torch.cuda.empty_cache()
        dr = run_attention("gpt2-medium-fwd-bwd", 20, 5, backward=True, p_drop=DROPOUT_P)
        dr.pop("host")
        out["targets"]["fa_fwd_dropout B64 H16 T1024 d64 p0.1"] = roofline(
            "mfma", dr["fwd_flop"], dr["fwd_median_ms"], "fa_fwd_dropout B64 H16 T1024 d64 p0.1")
        out["targets"]["fa_bwd_dropout B64 H16 T1024 d64 p0.1"] = roofline(
            "mfma", dr["bwd_flop"], dr["bwd_median_ms"], "fa_bwd_dropout B64 H16 T1024 d64 p0.1",
            bwd_algorithmic_bytes(B, Hq, Hkv, T, d))
        f32 = run_small_f32(50, 10)
        out["latency"] = {"fa_fwd_f32 B1 H1 T256 d64": {"median_us": round(f32["median_ms"] * 1e3, 2),
                                                        "flop": f32["flop"], "bound": "latency"}}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
