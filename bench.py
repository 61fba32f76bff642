#!/usr/bin/env python3
"""Benchmark of the exact tiled-attention library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one batch: fa_fwd then fa_bwd
(recomputation from the saved LSE) at the GPT-2-medium attention shape
(B64 H16 T1024 d64, bf16, non-causal, scale 1/8). W untimed steps, then K
steps timed between two device synchronisations; HIP events around every
launch, recorded on the stream the kernels run on, give per-launch durations.

After the timed region, in the same run (not part of `value`):
  * the causal long-context forward (B1 H32 T8192 d128) and split-KV decoding
    (B16 Hq32 Hkv8, lengths U[4096, 32768], d128) are timed the same way;
  * the fp64 CPU oracle is timed on a bounded sample of the step's workload.
Prints one JSON line.

FLOP convention: 4*d per visible (query, key) pair for the forward (two
contractions), 2.5x that for the backward (five contractions); a causal
square problem has T(T+1)/2 visible pairs. Decode bytes: every cached key and
value row read once (sum_b L_b * Hkv * 2 * d * 2 bytes) plus q and o.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak

COPY_BYTES = 1 << 30          # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE

METRIC = "attention fwd/bwd TFLOPS and % of MI355X bf16 MFMA peak; decode HBM GB/s"

WORKLOADS = {
    # name: (B, Hq, Hkv, T, d, causal, seed)
    "gpt2-medium-fwd-bwd": (64, 16, 16, 1024, 64, False, 2),
    "causal-8k-fwd": (1, 32, 32, 8192, 128, True, 3),
    "causal-32k-gqa-fwd-bwd": (1, 32, 8, 32768, 128, True, 4),
}


def fwd_flops(B, Hq, Tq, Tk, d, causal):
    pairs = Tq * (Tq + 1) // 2 if causal else Tq * Tk
    return 4.0 * d * pairs * B * Hq


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


def attention_step_buffers(B, Hq, Hkv, T, d, seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = _randn_bf16((B, Hq, T, d), gen)
    k = _randn_bf16((B, Hkv, T, d), gen)
    v = _randn_bf16((B, Hkv, T, d), gen)
    do = _randn_bf16((B, Hq, T, d), gen)
    return q, k, v, do


def run_attention(name, steps, warmup, backward=True):
    import torch
    from io_aware_softmax_05_amd import fa
    B, Hq, Hkv, T, d, causal, seed = WORKLOADS[name]
    scale = d ** -0.5
    q, k, v, do = attention_step_buffers(B, Hq, Hkv, T, d, seed)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, T, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    t_fwd, t_bwd = Timer(stream), Timer(stream)

    def step(timed):
        f = lambda: fa.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, T, T, d, scale, causal, stream)  # noqa: E731
        b = lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, T, T, d,  # noqa: E731
                              scale, causal, stream)
        if timed:
            t_fwd.record(f)
            if backward:
                t_bwd.record(b)
        else:
            f()
            if backward:
                b()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ff = fwd_flops(B, Hq, T, T, d, causal)
    res = {
        "workload": name, "B": B, "Hq": Hq, "Hkv": Hkv, "T": T, "d": d, "causal": causal,
        "wall_s": wall, "ms_per_step": wall * 1e3 / steps,
        "fwd_ms": t_fwd.mean_ms(), "fwd_flop": ff,
        "fwd_tflops": ff / (t_fwd.mean_ms() * 1e-3) / 1e12,
    }
    res["step_flop"] = ff * (3.5 if backward else 1.0)
    if backward:
        res["bwd_ms"] = t_bwd.mean_ms()
        res["bwd_flop"] = 2.5 * ff
        res["bwd_tflops"] = 2.5 * ff / (t_bwd.mean_ms() * 1e-3) / 1e12
    res["host"] = {"q": q, "k": k, "v": v, "do": do}
    return res


def run_decode(steps, warmup):
    import torch
    from io_aware_softmax_05_amd import fa, inputs
    B, Hq, Hkv, Tk_max, d = 16, 32, 8, 32768, 128
    rng = inputs.make_rng(5)
    lens_np = inputs.decode_lengths(rng, B)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    q = _randn_bf16((B, Hq, d), gen)
    kc = _randn_bf16((B, Hkv, Tk_max, d), gen)
    vc = _randn_bf16((B, Hkv, Tk_max, d), gen)
    lens = torch.from_numpy(lens_np).cuda()
    ws_bytes = fa.fa_decode_workspace_size(B, Hq, Tk_max, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    t = Timer(stream)
    call = lambda: fa.fa_decode_splitkv(q, kc, vc, lens, o, lse, ws, ws_bytes, B, Hq, Hkv, Tk_max, d,  # noqa: E731
                                        d ** -0.5, 0, stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    for _ in range(steps):
        t.record(call)
    torch.cuda.synchronize()
    kv_bytes = float(lens_np.astype(np.int64).sum()) * Hkv * 2 * d * 2
    io_bytes = 2.0 * B * Hq * d * 2
    ms = t.mean_ms()
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    return {"workload": "split-KV decode B16 Hq32 Hkv8 Tk<=32768 d128", "ms": ms, "bytes": kv_bytes + io_bytes,
            "sum_lengths": int(lens_np.sum()), "GB_per_s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}


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
        t_start = time.perf_counter()
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2-medium-fwd-bwd", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the side measurements")
    ap.add_argument("--only", choices=["step", "causal-8k-fwd", "decode", "copy"],
                    help="run one measurement alone (profiling runs); 'copy' runs a plain device copy "
                         "of 1 GiB, the calibration for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
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
    if args.only == "decode":
        print(json.dumps(run_decode(args.steps, args.warmup)), flush=True)
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

    backward = not args.workload.endswith("-fwd")
    res = run_attention(args.workload, args.steps, args.warmup, backward=backward)
    value = res["step_flop"] / (res["ms_per_step"] * 1e-3) / 1e12
    dom_ms = res["bwd_ms"] if backward else res["fwd_ms"]
    dom_flop = res["bwd_flop"] if backward else res["fwd_flop"]
    achieved = dom_flop / (dom_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": res["workload"], "B": res["B"], "Hq": res["Hq"], "Hkv": res["Hkv"],
                   "seq_len": res["T"], "head_dim": res["d"], "causal": res["causal"],
                   "step": "fa_fwd + fa_bwd" if backward else "fa_fwd",
                   "flop_per_step": res["step_flop"]},
        "roofline": {"kernel": ("fa_bwd launch (bwd_pre + bwd_dkdv + bwd_dq)" if backward else "fa_fwd launch"),
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "phases": {"fwd_ms": round(res["fwd_ms"], 4), "fwd_tflops": round(res["fwd_tflops"], 2)},
    }
    if backward:
        out["phases"].update({"bwd_ms": round(res["bwd_ms"], 4), "bwd_tflops": round(res["bwd_tflops"], 2)})
    if not args.no_extras:
        torch.cuda.empty_cache()
        tgt = run_attention("causal-8k-fwd", max(10, args.steps), 3, backward=False)
        tgt.pop("host")
        dec = run_decode(max(10, args.steps), 3)
        out["targets"] = {
            "causal_fwd_B1_H32_T8192_d128": {"ms": round(tgt["fwd_ms"], 4), "tflops": round(tgt["fwd_tflops"], 2),
                                             "frac_of_bf16_peak": round(tgt["fwd_tflops"] / PEAK_BF16_TFLOPS, 4)},
            "decode_B16_Hq32_Hkv8_Tk32768_d128": {"us": round(dec["ms"] * 1e3, 2), "GB_per_s": round(dec["GB_per_s"], 1),
                                                  "frac_of_hbm_peak": round(dec["frac_of_hbm_peak"], 4),
                                                  "bytes": dec["bytes"]},
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
