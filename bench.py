"""Benchmark: one step = the whole per-rank hot path on one batch of synthetic input:
mlp_shard_fwd + mlp_shard_bwd + vocab_ce_shard_fwd + ce_combine.

    python bench.py [--gpus 1] [--steps K] [--warmup W (default 50)] [--workload NAME] [--no-cpu-baseline]
                    [--rows ce_bwd,attn|none] [--shards NAME,...|none]

Default workload: the GPT-2 1.5B-like full layer (t=1): T = 8*1024 tokens, h = 1600,
FFN 6400, vocab 50304 (padded).  Inputs are seeded synthetic bf16 tensors, resident
in HBM before the timed region.  Prints one JSON line.

value = algorithmic TFLOP/s of the whole step: (12*T*h*f_i + 2*T*h*v_i) / step time.
The MLP fwd+bwd TFLOP/s, the CE tokens/s and their fractions of the bf16 MFMA peak
are reported alongside.  ``ms_per_step`` is host wall time over the K timed steps;
``step_ms_events`` gives the median, minimum and 90th percentile of K further steps
timed one by one with HIP events (the MLP and CE phase times come from those too).  ``roofline`` covers the dominant kernel, the logits GEMM
with the fused CE epilogue: the library records a pair of HIP events on its launch
stream around that one launch in every timed step (ms_arm_kernel_events), and
``achieved`` = 2*T*h*v_i / the mean of those durations.  ``traffic`` is the HBM
bytes per launch that the committed counter summary for this workload gives
(FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or null when the
kernel sources have changed since the counters were taken.  ``kernels_us`` is a
per-GEMM breakdown from a separate pass after the timed region.  The
``cpu_baseline`` leg times the fp64 oracle on a bounded token sample of the same
workload on the host cores.

After the headline workload, the same step is timed on the three rank-shard
workloads (8.3B-GPT-like t=8, 3.9B-BERT-like t=4, 176B-scale t=4) and reported
under ``shard_configs``; the CE backward and the attention shard of the headline
workload are timed under ``ce_bwd`` and ``attn``, and each shard workload's
attention shard under its own ``attn``.  ``peak_box`` restates the
bf16 peak from the compute-unit count and peak clock the HIP runtime reports
(compute units x 4096 flop/clock x clock).

    python bench.py --copy-calibration   # only a plain 1 GiB device copy, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0
# sources that define the GEMM kernels; counter-derived traffic is trusted only for these exact bytes
KERNEL_SOURCES = ("gemm_core.hpp", "epilogues.hpp", "kernels.hip", "launch.hpp")
TRAFFIC_MARK = "TRAFFIC_JSON "
# the GEMM launches of one step, in launch order (ids of the library's measurement hook)
STEP_KERNELS = ("fwd_h", "fwd_z", "bwd_dh", "bwd_db", "bwd_da", "bwd_dx", "ce_gemm")
# rank-shard workloads timed after the headline one
SHARD_WORKLOADS = ("gpt_8p3b_t8", "bert_3p9b_t4", "bloom_176b_t4")
FLOP_PER_CU_CLOCK = 4096  # gfx950 dense bf16 MFMA: 4 matrix cores x 1024 flop per clock


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="gpt2_1p5b")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle CPU time")
    p.add_argument("--no-breakdown", action="store_true", help="skip the per-GEMM breakdown pass")
    p.add_argument("--rows", default="ce_bwd,attn",
                   help="comma list of further rows timed after the step: ce_bwd, attn (or none)")
    p.add_argument("--shards", default=",".join(SHARD_WORKLOADS),
                   help="comma list of further workloads whose step is timed (or none)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of 1 GiB (5 launches) and exit")
    a = p.parse_args()
    a.rows = "" if a.rows == "none" else a.rows
    a.shards = "" if a.shards == "none" else a.shards
    unknown = sorted(set(r for r in a.rows.split(",") if r) - {"ce_bwd", "attn"})
    if unknown:
        p.error(f"unknown --rows entries {unknown} (known: ce_bwd, attn)")
    unknown = sorted(set(r for r in a.shards.split(",") if r) - set(SHARD_WORKLOADS))
    if unknown:
        p.error(f"unknown --shards entries {unknown} (known: {', '.join(SHARD_WORKLOADS)})")
    return a


def kernel_sources_sha256() -> str:
    """SHA-256 over the GEMM sources with comments and blank lines removed, so that
    only a change to the code itself invalidates counters taken on it."""
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "megatron_tensor_transformer_mlp_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def committed_traffic(workload: str):
    """HBM bytes per launch of the CE GEMM from profiles/, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", f"ce_gemm_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith(TRAFFIC_MARK):
                rec = json.loads(line[len(TRAFFIC_MARK):])
    if rec is None:
        return None, "counter summary has no traffic record"
    if rec.get("source_sha256") != kernel_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    return int(rec["hbm_bytes_per_launch"]), os.path.relpath(path, ROOT)


def copy_calibration():
    """A plain streaming copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 28  # fp32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)  # elementwise: reads n*4 bytes, writes n*4 bytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": n * 4, "write_bytes": n * 4, "launches": 5,
                                           "kernel": "torch.neg elementwise (fp32, 1 GiB)"}}), flush=True)


def cpu_baseline(cfg, d, target_s: float):
    """Time the fp64 oracle (as it stands) on the first Ts tokens of the same inputs:
    MLP fwd + bwd on Ts tokens and the CE shard + combine on Ts tokens."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def run(Ts):
        X, dZ, tg = d["X"][:Ts], d["dZ"][:Ts], d["targets"][:Ts]
        t0 = time.perf_counter()
        oracle.mlp_shard_fwd(X, d["A"], d["B"])
        oracle.mlp_shard_bwd(X, d["A"], d["B"], dZ)
        p = oracle.vocab_ce_shard(X, d["E"], tg, 0)
        oracle.ce_combine(p["m"], p["s"], p["z"])
        return time.perf_counter() - t0

    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        # the weight conversions are a fixed cost per call, so grow the sample by doubling
        # until one run takes target_s (or the sample is the whole batch)
        Ts = min(cfg.T, 256)
        dt = run(Ts)
        while dt < target_s and Ts < cfg.T:
            Ts = min(cfg.T, 2 * Ts)
            dt = run(Ts)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    flop = 12 * Ts * cfg.h * cfg.f_i + 2 * Ts * cfg.h * cfg.v_i
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": model, "kind": "oracle",
            "sample": f"numpy fp64 oracle, MLP fwd+bwd + CE shard + combine on the first {Ts} of {cfg.T} "
                      f"tokens ({flop / 1e9:.1f} GFLOP in {dt:.2f} s, weight conversions included)",
            "seconds": dt}


class StepRunner:
    """Device-resident inputs, outputs and workspaces of one workload's step."""

    def __init__(self, torch, mshard, cfg, d, dev):
        self.torch, self.ms, self.cfg, self.dev = torch, mshard, cfg, dev
        T, h, f, v = cfg.T, cfg.h, cfg.f_i, cfg.v_i
        up = self.up
        self.X, self.A, self.B, self.E, self.dZ = up(d["X"]), up(d["A"]), up(d["B"]), up(d["E"]), up(d["dZ"])
        self.tg = torch.from_numpy(d["targets"]).to(dev)
        bf = torch.bfloat16
        self.H = torch.empty((T, f), dtype=bf, device=dev)
        self.Y = torch.empty((T, f), dtype=bf, device=dev)
        self.Z = torch.empty((T, h), dtype=torch.float32, device=dev)
        self.dX = torch.empty((T, h), dtype=torch.float32, device=dev)
        self.dA = torch.empty((h, f), dtype=bf, device=dev)
        self.dB = torch.empty((f, h), dtype=bf, device=dev)
        self.mlp_ws = torch.empty(max(mshard.mlp_shard_workspace_bytes(T, h, f), 1), dtype=torch.uint8, device=dev)
        self.ce_ws = torch.empty(max(mshard.vocab_ce_workspace_bytes(T, h, v), 1), dtype=torch.uint8, device=dev)
        self.m, self.s, self.z = (torch.empty((1, T), dtype=torch.float32, device=dev) for _ in range(3))
        self.loss = torch.empty((T,), dtype=torch.float32, device=dev)
        self.mean = torch.empty((1,), dtype=torch.float32, device=dev)
        self.vstart = int(d["vocab_start"])
        self.stream = torch.cuda.current_stream(dev)

    def up(self, u):
        return self.torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(self.torch.bfloat16).to(self.dev)

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)  # creates the device event so its handle can be handed to the library
        return e

    def step(self, phase=None, arm=()):
        ms = self.ms
        for name, (e0, e1) in arm:
            ms.arm_kernel_events(name, e0, e1)
        if phase is not None:
            phase[0].record(self.stream)
        ms.mlp_shard_fwd(self.X, self.A, self.B, None, out=(self.H, self.Y, self.Z), workspace=self.mlp_ws)
        ms.mlp_shard_bwd(self.X, self.A, self.B, self.H, self.Y, self.dZ, workspace=self.mlp_ws,
                         out=(self.dX, self.dA, self.dB, None))
        if phase is not None:
            phase[1].record(self.stream)
        ms.vocab_ce_shard_fwd(self.X, self.E, self.tg, self.vstart, workspace=self.ce_ws,
                              out=(self.m[0], self.s[0], self.z[0]))
        ms.ce_combine(self.m, self.s, self.z, out=(self.loss, self.mean))
        if phase is not None:
            phase[2].record(self.stream)

    def timed_steps(self, steps, warmup):
        """Wall time per step over `steps` steps (after `warmup`), with the CE GEMM's
        own launch time from the library's hook on each of them; then the same number
        of steps again with events at the phase boundaries, for the MLP and CE phase
        times and the per-step spread (kept out of the timed steps, whose only events
        are the CE GEMM's)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        phases = [[self.ev() for _ in range(3)] for _ in range(steps)]
        gemm_ev = [(self.ev(), self.ev()) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.step(arm=[("ce_gemm", gemm_ev[k])])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for k in range(steps):
            self.step(phases[k])
        torch.cuda.synchronize()
        per_step = np.array([e[0].elapsed_time(e[2]) for e in phases])
        return {"ms_step": wall * 1e3 / steps,
                "step_stats": {"median": round(float(np.median(per_step)), 4),
                               "min": round(float(per_step.min()), 4),
                               "p90": round(float(np.percentile(per_step, 90)), 4)},
                "mlp_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in phases])),
                "ce_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in phases])),
                "gemm_ms": float(np.mean([e0.elapsed_time(e1) for e0, e1 in gemm_ev]))}

    def breakdown(self, reps=5):
        torch = self.torch
        names = list(STEP_KERNELS)
        kev = [[(self.ev(), self.ev()) for _ in names] for _ in range(reps)]
        torch.cuda.synchronize()
        for r in range(reps):
            self.step(arm=list(zip(names, kev[r])))
        torch.cuda.synchronize()
        return {n: round(1e3 * float(np.mean([kev[r][i][0].elapsed_time(kev[r][i][1]) for r in range(reps)])), 1)
                for i, n in enumerate(names)}

    def timed(self, fn, reps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        evs = [(self.ev(), self.ev()) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))


def step_summary(cfg, t):
    mlp_tflops = cfg.mlp_flop / (t["mlp_ms"] * 1e-3) / 1e12
    ce_tflops = cfg.ce_flop / (t["ce_ms"] * 1e-3) / 1e12
    gemm_tflops = cfg.ce_flop / (t["gemm_ms"] * 1e-3) / 1e12
    value = (cfg.mlp_flop + cfg.ce_flop) / (t["ms_step"] * 1e-3) / 1e12
    return {"value": value, "mlp_tflops": mlp_tflops, "ce_tflops": ce_tflops, "gemm_tflops": gemm_tflops}


def attn_row(torch, mshard, run, cfg, dev, steps, warmup):
    """Times this workload's attention shard (forward, then backward) on the runner's stream."""
    from megatron_tensor_transformer_mlp_amd import inputs
    bf = torch.bfloat16
    T, h = cfg.T, cfg.h
    ac = inputs.ATTN_CONFIGS[cfg.name]
    assert ac.b * ac.s == T and ac.h == h, (ac, cfg)
    ad = inputs.make_attn_config_inputs(ac)
    up = run.up
    Xa, Wqkv, Wo, dZa = up(ad["X"]), up(ad["Wqkv"]), up(ad["Wo"]), up(ad["dZ"])
    nd = ac.n * ac.d
    QKV = torch.empty((T, 3 * nd), dtype=bf, device=dev)
    Oa = torch.empty((T, nd), dtype=bf, device=dev)
    lse = torch.empty((ac.n, T), dtype=torch.float32, device=dev)
    Za = torch.empty((T, h), dtype=torch.float32, device=dev)
    dXa = torch.empty((T, h), dtype=torch.float32, device=dev)
    dWqkv = torch.empty((h, 3 * nd), dtype=bf, device=dev)
    dWo = torch.empty((nd, h), dtype=bf, device=dev)
    attn_ws = torch.empty(max(mshard.attn_shard_workspace_bytes(ac.b, ac.s, h, ac.n, ac.d), 1), dtype=torch.uint8,
                          device=dev)
    fwd = lambda: mshard.attn_shard_fwd(Xa, Wqkv, Wo, ac.b, ac.s, ac.n, ac.d, ac.causal, out=(QKV, Oa, lse, Za))
    bwd = lambda: mshard.attn_shard_bwd(Xa, Wqkv, Wo, QKV, Oa, lse, dZa, ac.b, ac.s, ac.n, ac.d, ac.causal,
                                        workspace=attn_ws, out=(dXa, dWqkv, dWo))
    ms_f = run.timed(fwd, steps, warmup)
    ms_b = run.timed(bwd, steps, warmup)
    pairs = ac.b * ac.n * (ac.s * (ac.s + 1) // 2 if ac.causal else ac.s * ac.s)  # visible (query, key) pairs
    proj = 2 * T * h * 3 * nd + 2 * T * nd * h
    f_flop = proj + 4 * pairs * ac.d            # projections; S and P V
    b_flop = 2 * proj + 8 * pairs * ac.d        # their gradients; dV, dP, dQ, dK (recompute not counted)
    return {"config": f"b={ac.b} s={ac.s} h={h} n={ac.n} d={ac.d} causal={ac.causal}",
            "fwd_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
            "fwd_tflops": round(f_flop / (ms_f * 1e-3) / 1e12, 2),
            "bwd_tflops": round(b_flop / (ms_b * 1e-3) / 1e12, 2),
            "algorithmic_flop": {"fwd": f_flop, "bwd": b_flop}}


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (the multi-GPU exchange "
              "is not part of this library)", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return

    import torch

    from megatron_tensor_transformer_mlp_amd import build as _b, inputs
    if not os.path.exists(os.path.join(ROOT, "megatron_tensor_transformer_mlp_amd", "libmshard.so")):
        _b.build_library(verbose=False)
    from megatron_tensor_transformer_mlp_amd import mshard

    cfg = inputs.CONFIGS[a.workload]
    T, h, f, v = cfg.T, cfg.h, cfg.f_i, cfg.v_i
    d = inputs.make_config_inputs(cfg)
    dev = torch.device("cuda:0")
    run = StepRunner(torch, mshard, cfg, d, dev)
    bf = torch.bfloat16

    t = run.timed_steps(a.steps, a.warmup)
    sm = step_summary(cfg, t)
    ms_step, mlp_ms, ce_ms, gemm_ms = t["ms_step"], t["mlp_ms"], t["ce_ms"], t["gemm_ms"]
    value, mlp_tflops, ce_tflops, gemm_tflops = sm["value"], sm["mlp_tflops"], sm["ce_tflops"], sm["gemm_tflops"]
    kernels_us = None if a.no_breakdown else run.breakdown()

    rows = [r for r in a.rows.split(",") if r]
    extra = {}
    X, E, tg, m, s, vstart = run.X, run.E, run.tg, run.m, run.s, run.vstart

    if "ce_bwd" in rows:
        ce_bwd_ws = torch.empty(max(mshard.vocab_ce_bwd_workspace_bytes(T, h, v), 1), dtype=torch.uint8, device=dev)
        dXc = torch.empty((T, h), dtype=torch.float32, device=dev)
        dEc = torch.empty((h, v), dtype=bf, device=dev)
        ms_ce = run.timed(lambda: mshard.vocab_ce_shard_bwd(X, E, tg, m, s, vstart, workspace=ce_bwd_ws,
                                                             out=(dXc, dEc)), a.steps, a.warmup)
        flop = 3 * 2 * T * h * v  # logits recompute, dX = dL E^T, dE = X^T dL
        extra["ce_bwd"] = {"ms": round(ms_ce, 4), "tflops": round(flop / (ms_ce * 1e-3) / 1e12, 2),
                           "pct_of_peak": round(100 * flop / (ms_ce * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                           "tokens_per_s": round(T / (ms_ce * 1e-3), 1), "algorithmic_flop": flop}
        del ce_bwd_ws, dXc, dEc
    if "attn" in rows:
        extra["attn"] = attn_row(torch, mshard, run, cfg, dev, a.steps, a.warmup)

    info = mshard.device_info(0)
    box_peak = info["compute_units"] * FLOP_PER_CU_CLOCK * info["clock_khz"] * 1e3 / 1e12
    traffic, traffic_src = committed_traffic(cfg.name)
    out = {
        "metric": "MLP-shard fwd+bwd TFLOP/s + fused vocab-CE tokens/s, % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms_events": t["step_stats"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one rank's MLP shard fwd+bwd + vocab-parallel fused CE + combine, "
                               f"t={cfg.t}, T={T} tokens, h={h}, f_i={f}, v_i={v}",
                   "tokens": T, "h": h, "f_i": f, "v_i": v, "t": cfg.t},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "peak_box": {"compute_units": info["compute_units"], "clock_mhz": round(info["clock_khz"] / 1e3, 1),
                     "flop_per_cu_clock": FLOP_PER_CU_CLOCK, "tflops": round(box_peak, 1),
                     "pct_of_box_peak": round(100 * value / box_peak, 2) if box_peak > 0 else None},
        "mlp_fwd_bwd_tflops": round(mlp_tflops, 2),
        "mlp_pct_of_peak": round(100 * mlp_tflops / PEAK_BF16_TFLOPS, 2),
        "mlp_ms": round(mlp_ms, 4),
        "ce_tokens_per_s": round(T / (ce_ms * 1e-3), 1),
        "ce_tflops": round(ce_tflops, 2),
        "ce_pct_of_peak": round(100 * ce_tflops / PEAK_BF16_TFLOPS, 2),
        "ce_ms": round(ce_ms, 4),
        "roofline": {"bound": "mfma", "kernel": "logits GEMM X E_i with fused CE epilogue (gemm_kernel<EpiCE>)",
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src, "launch_us": round(gemm_ms * 1e3, 1),
                     "algorithmic_flop_per_launch": cfg.ce_flop},
        "kernels_us": kernels_us,
    }
    out.update(extra)
    del run
    torch.cuda.empty_cache()

    shards = {}
    for name in [w for w in a.shards.split(",") if w]:
        c2 = inputs.CONFIGS[name]
        r2 = StepRunner(torch, mshard, c2, inputs.make_config_inputs(c2), dev)
        t2 = r2.timed_steps(a.steps, a.warmup)
        s2 = step_summary(c2, t2)
        shards[name] = {
            "workload": f"T={c2.T}, h={c2.h}, f_i={c2.f_i}, v_i={c2.v_i}, t={c2.t}",
            "ms_per_step": round(t2["ms_step"], 4), "step_ms_events": t2["step_stats"],
            "tflops": round(s2["value"], 2),
            "pct_of_bf16_peak": round(100 * s2["value"] / PEAK_BF16_TFLOPS, 2),
            "mlp_fwd_bwd_tflops": round(s2["mlp_tflops"], 2),
            "mlp_pct_of_peak": round(100 * s2["mlp_tflops"] / PEAK_BF16_TFLOPS, 2),
            "ce_tokens_per_s": round(c2.T / (t2["ce_ms"] * 1e-3), 1), "ce_tflops": round(s2["ce_tflops"], 2),
            "ce_pct_of_peak": round(100 * s2["ce_tflops"] / PEAK_BF16_TFLOPS, 2),
            "ce_gemm_tflops": round(s2["gemm_tflops"], 2),
            "kernels_us": None if a.no_breakdown else r2.breakdown()}
        if "attn" in rows:
            shards[name]["attn"] = attn_row(torch, mshard, r2, c2, dev, a.steps, a.warmup)
        del r2
        torch.cuda.empty_cache()
    if shards:
        out["shard_configs"] = shards
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, d, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
