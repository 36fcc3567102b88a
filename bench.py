"""Benchmark: fused attention forward TFLOP/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]
                    [--no-cpu-baseline] [--no-configs] [--no-backward] [--no-fp8]
                    [--no-dropout] [--no-general] [--no-sweep]
    python bench.py --counter-pass            # dispatches for rocprofv3 --pmc runs
    python bench.py --summarize-counters DIR  # rocprofv3 CSVs -> profiles/*_traffic.json

A step is one attention forward over the whole workload (B=2, H=32, N=8192,
d=128, causal, Q and K scaled by 4 -- the headline case) with inputs already
resident in HBM.  W untimed warm-up steps, then K timed steps bracketed by
device synchronisation; the kernel's own average duration is taken with HIP
events recorded on the launch stream around the same K launches.  Flops are
the algorithmic count 4*B*H*N^2*d, halved when causal (page "GPU Programming &
Kernel Development", Self-check: fusion does not change the flop count).

Before the headline's own warm-up and timed steps, the other workloads are
measured one by one (``configs``: tiny, ragged, N=2048 causal and N=32768
causal, each with per-launch median/p10/p90 from HIP events and the float64
oracle timed on the host cores).  That also brings the GPU to the clock it
holds under this load, so a short warm-up does not decide the headline number.

Prints ONE JSON line.  Beside the headline: ``backward`` (attn_bwd on the same
workload), ``fp8_scores`` (the FP8-score forward alone and with its quantiser
end to end), ``dropout`` (forward and backward), ``general_shapes``
(attn_fwd_ex / attn_fwd_split / attn_bwd_ex), ``seq_sweep`` (forward and
backward latency and memory as the sequence grows, page "22. GPU Engineering:
Correctness, Throughput, and Attention", sec. 22.5 lab), ``device`` (GPU,
driver, ROCm, compiler and the clock observed during the headline kernel) and
``cpu_baseline`` (the float64 oracle on a bounded sample of the headline).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of bf16 MFMA peak (N=8192, d=128, causal)"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0         # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 256 << 20           # calibration copy of --counter-pass (bytes read = bytes written)
PROFILES = os.path.join(ROOT, "profiles")

FWD_SOURCES = ("attn_common.hpp", "attn_fwd.hip", "attn_fwd_kernel.hpp")
BWD_SOURCES = ("attn_bwd.hip", "attn_bwd_kernel.hpp", "attn_common.hpp")
FP8_SOURCES = ("attn_common.hpp", "attn_fp8.hip", "attn_fp8_quant.hpp", "attn_fwd_kernel.hpp")
TRAFFIC_FILE = os.path.join(PROFILES, "attn_fwd_headline_traffic.json")
BWD_TRAFFIC_FILE = os.path.join(PROFILES, "attn_bwd_headline_traffic.json")
PATH_TRAFFIC_FILE = os.path.join(PROFILES, "attn_paths_headline_traffic.json")

DROP_T = 26            # drop probability 26/256 (about 0.1)
DROP_SEED = 2024

# General-shape forward workloads (attn_fwd_ex): name, B, H, Nq, Nk, d, dv, offset, causal.
GENERAL = [
    ("chunked prefill: 1024 queries at positions 7168.. of 8192 keys", 2, 32, 1024, 8192, 128, 128,
     7168, True),
    ("value width 64: B=2,H=32,N=8192,d=128,dv=64", 2, 32, 8192, 8192, 128, 64, 0, True),
    ("decode step: 1 query at position 8191 of 8192 keys, B=16,H=32", 16, 32, 1, 8192, 128, 128,
     8191, True),
    ("decode step, few sequences: 16 queries at positions 32752.. of 32768 keys, B=2,H=8", 2, 8,
     16, 32768, 128, 128, 32752, True),
]

# The configurations besides the headline (configs 1, 2, 3, 5 of the workload list).
CONFIG_WORKLOADS = (("tiny", 1), ("ragged", 2), ("mid_causal", 3), ("long", 5))
SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768)


# ---------------------------------------------------------------- helpers

def kernel_source_hash(names=FWD_SOURCES) -> str:
    """sha256 over the HIP sources a kernel is built from, without their //
    comments, trailing blanks and empty lines (traffic figures are only valid
    for the kernel they were measured on; a comment edit does not change it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_attention_09_amd", "csrc")
    for name in sorted(names):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in f.read().splitlines())
            code = "\n".join(ln for ln in lines if ln)
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def measured_traffic(workload_name: str, path: str = TRAFFIC_FILE, names=FWD_SOURCES, key=None):
    """HBM bytes per launch from a committed counter summary, or None when it
    is missing, for another workload, or older than the current kernel.  With
    ``key`` the file holds several paths: entry ``key`` of ``paths``."""
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("workload") != workload_name:
        return None
    if key is not None:
        t = t.get("paths", {}).get(key)
        if t is None:
            return None
    if t.get("kernel_source_sha256") != kernel_source_hash(names):
        return None
    return t.get("bytes_per_launch")


def roofline_mfma(tflops: float, peak: float = PEAK_BF16_TFLOPS, traffic=None) -> dict:
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4), "traffic": traffic}


def roofline_hbm(gbs: float, traffic=None) -> dict:
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}


def event_ms(fn, stream, calls: int, warmup: int) -> float:
    """Average ms of ``fn`` over ``calls`` calls after about 0.25 s of untimed
    back-to-back calls (the clock this load holds) and ``warmup`` more, from
    HIP events recorded on the launch stream."""
    import torch
    warm_for(fn, 0.25)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def per_launch_ms(fn, stream, samples: int, batch: int = 1):
    """Sorted per-launch ms from ``samples`` event pairs, each around ``batch`` calls."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(samples)]
    for a, b in evs:
        a.record(stream)
        for _ in range(batch):
            fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / batch for a, b in evs)


def warm_for(fn, seconds: float) -> None:
    """Run ``fn`` back to back for about ``seconds`` (the GPU reaches the clock it
    holds under this load; an idle GPU starts slower)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def spread(per) -> dict:
    return {"median": round(per[len(per) // 2], 5), "p10": round(per[len(per) // 10], 5),
            "p90": round(per[(9 * len(per)) // 10], 5)}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return 0


# ---------------------------------------------------------------- device metadata

def _run(cmd, timeout=20):
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
        return r.stdout if r.returncode == 0 else None
    except Exception:
        return None


def profiler_present() -> bool:
    """True under rocprofv3, whose preloaded library initialises the GPU before
    main(): no child process may be started then."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "")


def host_metadata() -> dict:
    """ROCm, driver and compiler versions.  Runs helper programs, so it must be
    called before anything touches the GPU."""
    info = {"host_cores": len(os.sched_getaffinity(0))}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    drv = None
    try:
        drv = open("/sys/module/amdgpu/version").read().strip() or None
    except OSError:
        pass
    if drv is None:
        out = _run(["rocm-smi", "--showdriverversion"])
        m = re.search(r"Driver version:\s*(\S+)", out or "")
        drv = m.group(1) if m else None
    info["driver"] = drv
    cc = _run(["/opt/rocm/llvm/bin/clang", "--version"])
    info["compiler"] = cc.splitlines()[0].strip() if cc else None
    return info


_SAMPLER = r"""
import json, re, subprocess, sys, time
def mhz():
    # amd-smi: {"gpu_data": [{"gpu": 0, "clock": {"gfx_0": {"clk": {"value": ..}}, ..}}]}
    # -- the mean over the XCDs' graphics clocks; else rocm-smi's sclk line.
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True, timeout=10)
        d = json.loads(r.stdout)
        if isinstance(d, dict) and "gpu_data" in d:
            d = d["gpu_data"]
        d = d[0] if isinstance(d, list) else d
        c = d.get("clock", {})
        vals = [float(v["clk"]["value"]) for k, v in c.items()
                if k.lower().startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        if vals:
            return sum(vals) / len(vals)
    except Exception:
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10)
        m = re.findall(r"sclk[^\n]*?\((\d+)Mhz\)", r.stdout)
        return float(m[0]) if m else None
    except Exception:
        return None
while True:
    t = time.time()
    v = mhz()
    if v is None:
        break
    print("%.3f %.3f %.1f" % (t, time.time(), v), flush=True)
"""


def start_clock_sampler():
    """A child process that prints (time, graphics clock MHz) lines from amd-smi
    (else rocm-smi) until stopped.  Started before anything touches the GPU."""
    try:
        return subprocess.Popen([sys.executable, "-c", _SAMPLER], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except Exception:
        return None


def stop_clock_sampler(proc, t0: float, t1: float):
    """Stop the sampler; the clock readings taken between t0 and t1 (time.time())."""
    if proc is None:
        return None
    proc.terminate()
    try:
        out, _ = proc.communicate(timeout=15)
    except Exception:
        proc.kill()
        return None
    vals = []
    for line in (out or "").splitlines():
        try:
            ta_, tb_, v = (float(x) for x in line.split())
        except ValueError:
            continue
        if t0 <= ta_ and tb_ <= t1:          # the reading started and ended inside the window
            vals.append(v)
    if not vals:
        return None
    return {"samples": vals, "median": statistics.median(vals),
            "source": "amd-smi (mean over the XCDs; else rocm-smi) gfx clock read while the "
                      "headline kernel runs back to back for 3 s, outside the timed region"}


def device_info(dev, meta: dict) -> dict:
    """GPU name, arch, CU count and HIP version, with the host metadata."""
    import torch
    props = torch.cuda.get_device_properties(dev)
    return dict({"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                 "cus": props.multi_processor_count, "hip": torch.version.hip}, **meta)


# ---------------------------------------------------------------- oracle timings

def oracle_timing(w, rows_per_head=None) -> dict:
    """Time the float64 oracle as it is on workload ``w``: every row of every
    head, or ``rows_per_head`` seeded sampled rows per head."""
    import numpy as np

    from oracle import attention_ref, bf16_bits_to_f64, f32_scale
    from tiled_attention_09_amd.synth import bf16_bits, make_workload, sample_rows
    q, k, v = make_workload(w)
    s = f32_scale(w.scale)
    flops, nrows = 0.0, 0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            rows = (np.arange(w.N) if rows_per_head is None
                    else sample_rows(w.N, rows_per_head, w.seed + 100 + b * w.H + h))
            attention_ref(bf16_bits_to_f64(bf16_bits(q[b, h])), bf16_bits_to_f64(bf16_bits(k[b, h])),
                          bf16_bits_to_f64(bf16_bits(v[b, h])), s, w.causal, rows=rows)
            visible = (rows + 1) if w.causal else np.full(rows.size, w.N)
            flops += float(4 * w.d * visible.sum())
            nrows += rows.size
    dt = time.perf_counter() - t0
    return {"seconds": round(dt, 3), "tflops": flops / dt / 1e12, "rows": nrows,
            "rows_per_head": "all" if rows_per_head is None else rows_per_head,
            "cores": blas_threads(), "kind": "oracle (float64 two-pass, NumPy)"}


def cpu_baseline(w, budget_s: float = 15.0, rows_per_head: int = 4096):
    """Time the float64 oracle on a seeded row sample of every head, head by
    head, until the time budget is spent.  Returns the JSON object."""
    import numpy as np

    from oracle import attention_ref, bf16_bits_to_f64, f32_scale
    from tiled_attention_09_amd.synth import bf16_bits, make_workload, sample_rows

    q, k, v = make_workload(w)
    s = f32_scale(w.scale)
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            rows = sample_rows(w.N, rows_per_head, w.seed + 100 + b * w.H + h)
            qd = bf16_bits_to_f64(bf16_bits(q[b, h]))
            kd = bf16_bits_to_f64(bf16_bits(k[b, h]))
            vd = bf16_bits_to_f64(bf16_bits(v[b, h]))
            attention_ref(qd, kd, vd, s, w.causal, rows=rows)
            visible = (rows + 1) if w.causal else np.full(rows.size, w.N)
            flops += float(4 * w.d * visible.sum())
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": "float64 two-pass oracle on %d heads x %d seeded query rows "
                      "(all N keys, causal mask), %.1f s; value = algorithmic flops of "
                      "those rows / wall time; host cores visible %d" % (
                          heads, min(rows_per_head, w.N), dt, len(os.sched_getaffinity(0)))}


# ---------------------------------------------------------------- measurement legs

def time_configs(stream):
    """The workloads besides the headline: after 0.25 s of back-to-back launches,
    per-launch median/p10/p90 over 50 event pairs (batches of 100 launches for
    the two launch-bound ones) and the algorithmic TFLOP/s at the median.  The
    oracle timings are added later (add_config_oracle), after all GPU work, so
    that the host-side computation leaves no idle spell between GPU legs."""
    import torch

    import tiled_attention_09_amd as ta
    from tiled_attention_09_amd.synth import WORKLOADS, make_workload
    dev = torch.device("cuda:0")
    out = []
    for name, num in CONFIG_WORKLOADS:
        w = WORKLOADS[name]
        q, k, v = (x.to(dev) for x in make_workload(w))
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def fwd():
            ta.attn_fwd(q, k, v, w.scale, w.causal, out=o, lse=lse, stream=stream.cuda_stream)

        batch = 100 if w.flops < 1e11 else 1
        warm_for(fwd, 0.25)
        per = per_launch_ms(fwd, stream, 50, batch)
        sp = spread(per)
        tflops = w.flops / (sp["median"] * 1e-3) / 1e12
        gbs = w.alg_bytes / (sp["median"] * 1e-3) / 1e9
        entry = {"config": num, "workload": "attention fwd " + w.describe(), "B": w.B, "H": w.H,
                 "N": w.N, "d": w.d, "causal": w.causal, "seed": w.seed,
                 "launches": 50 * batch, "launches_per_event_pair": batch,
                 "kernel_ms": sp, "tflops": round(tflops, 2),
                 "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
                 "gbs": round(gbs, 1), "flops": w.flops, "alg_bytes": w.alg_bytes,
                 "roofline": roofline_mfma(tflops)}
        if w.flops < 1e11:
            entry["note"] = "launch-bound: one kernel of a few microseconds"
        del q, k, v, o, lse
        out.append(entry)
        print("bench: config %d %s median %.4f ms" % (num, name, sp["median"]), file=sys.stderr,
              flush=True)
    torch.cuda.empty_cache()
    return out


def add_config_oracle(configs) -> None:
    """The float64 oracle timed on each config: every row for configs 1-3,
    256 sampled rows per head for the N = 32768 one."""
    from tiled_attention_09_amd.synth import WORKLOADS
    names = dict((num, name) for name, num in CONFIG_WORKLOADS)
    for entry in configs:
        w = WORKLOADS[names[entry["config"]]]
        entry["oracle"] = oracle_timing(w, None if w.full_oracle else 256)


def time_backward(w, q, k, v, o, lse, stream, steps: int, warmup: int):
    """attn_bwd on the forward's O and LSE: HIP events around ``steps`` calls."""
    import torch

    import tiled_attention_09_amd as ta
    from tiled_attention_09_amd.synth import make_dout
    dev = q.device
    g = make_dout(w.B, w.H, w.N, w.d, w.seed).to(dev)
    ws = torch.empty(ta.attn_bwd_workspace_size(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
    grads = tuple(torch.empty_like(o) for _ in range(3))

    def bstep():
        ta.attn_bwd(q, k, v, o, lse, g, w.scale, w.causal, workspace=ws, grads=grads,
                    stream=stream.cuda_stream)

    warm_for(bstep, 0.25)   # the gradient's host-side set-up left the GPU idle
    for _ in range(warmup):
        bstep()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        bstep()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = ev0.elapsed_time(ev1) / steps
    achieved = w.bwd_flops / (ms * 1e-3) / 1e12
    return {"metric": "attention bwd TFLOP/s (dQ, dK, dV; 2.5x forward flops)",
            "value": round(w.bwd_flops / (wall_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(wall_ms, 5), "kernel_ms": round(ms, 5),
            "flops_per_step": w.bwd_flops,
            "roofline": roofline_mfma(achieved, traffic=measured_traffic(
                w.name, BWD_TRAFFIC_FILE, BWD_SOURCES)),
            "steps": steps, "warmup": warmup, "grad_dtype": "fp32", "dout_dtype": "bf16"}


def time_fp8(w, q, k, v, stream, steps: int, warmup: int, bf16_ms: float):
    """The FP8-score forward (attn_fwd_fp8) with Q and K quantised beforehand,
    the quantiser alone, and both together (quantise Q, quantise K, forward)
    as one end-to-end step.  Half of the algorithmic flops (the scores) run at
    the fp8 rate and half (P V) at the bf16 rate, so the roofline peak is the
    time-weighted combination 2 / (1/5000 + 1/2500) = 3333 TFLOP/s."""
    import torch

    import tiled_attention_09_amd as ta
    dev = q.device
    if w.d != 128:
        return None
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    qd = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    kd = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    sc = stream.cuda_stream

    def quant():
        ta.attn_quantize_fp8(q, out=q8, descale=qd, stream=sc)
        ta.attn_quantize_fp8(k, out=k8, descale=kd, stream=sc)

    def fwd():
        ta.attn_fwd_fp8(q8, k8, v, qd, kd, w.scale, w.causal, out=o, lse=lse, stream=sc)

    def both():
        quant()
        fwd()

    quant_ms = event_ms(quant, stream, steps, warmup)
    ms = event_ms(fwd, stream, steps, warmup)
    e2e_ms = event_ms(both, stream, steps, warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    peak = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    qbytes = 2 * (w.B * w.H * w.N * w.d * 3 + w.B * w.H * 4)   # Q and K: read bf16, write codes
    return {"metric": "attention fwd TFLOP/s with FP8 scores (Q, K as E4M3 codes, per-head descale)",
            "value": round(tflops, 2), "unit": "TFLOP/s", "kernel_ms": round(ms, 5),
            "roofline": roofline_mfma(tflops, round(peak, 1), measured_traffic(
                w.name, PATH_TRAFFIC_FILE, FP8_SOURCES, "fp8_forward")),
            "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "quantize_q_and_k_ms": round(quant_ms, 5),
            "quantize_gbs": round(qbytes / (quant_ms * 1e-3) / 1e9, 1),
            "end_to_end": {"what": "quantise Q, quantise K, FP8-score forward",
                           "ms": round(e2e_ms, 5),
                           "tflops": round(w.flops / (e2e_ms * 1e-3) / 1e12, 2),
                           "bf16_forward_ms": round(bf16_ms, 5),
                           "speedup_vs_bf16_forward": round(bf16_ms / e2e_ms, 4)},
            "steps": steps, "warmup": warmup}


def time_dropout(w, q, k, v, stream, steps: int, warmup: int):
    """attn_fwd_dropout and attn_bwd_dropout (drop probability DROP_T/256) on
    the workload; the flop counts are those of the plain forward and backward
    (the mask adds no products)."""
    import torch

    import tiled_attention_09_amd as ta
    from tiled_attention_09_amd.synth import make_dout
    dev = q.device
    sc = stream.cuda_stream
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    g = make_dout(w.B, w.H, w.N, w.d, w.seed).to(dev)
    ws = torch.empty(ta.attn_bwd_workspace_size(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
    grads = tuple(torch.empty_like(o) for _ in range(3))

    def fwd():
        ta.attn_fwd_dropout(q, k, v, DROP_SEED, DROP_T, w.scale, w.causal, out=o, lse=lse,
                            stream=sc)

    def bwd():
        ta.attn_bwd_dropout(q, k, v, o, lse, g, DROP_SEED, DROP_T, w.scale, w.causal,
                            workspace=ws, grads=grads, stream=sc)

    out = {"metric": "attention TFLOP/s with dropout (Philox-4x32-10 masks regenerated in "
                     "the kernels)", "drop_t": DROP_T, "drop_probability": DROP_T / 256.0,
           "steps": steps, "warmup": warmup}
    for name, fn, flops, key in (("forward", fwd, w.flops, "dropout_forward"),
                                 ("backward", bwd, w.bwd_flops, "dropout_backward")):
        ms = event_ms(fn, stream, steps, warmup)
        tf = flops / (ms * 1e-3) / 1e12
        srcs = FWD_SOURCES if name == "forward" else BWD_SOURCES
        out[name] = {"kernel_ms": round(ms, 5), "tflops": round(tf, 2),
                     "roofline": roofline_mfma(tf, traffic=measured_traffic(
                         w.name, PATH_TRAFFIC_FILE, srcs, key))}
    return out


def _general_inputs(B, H, Nq, Nk, d, dv, dev):
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(900 + Nq)
    q = torch.randn((B, H, Nq, d), generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn((B, H, Nk, d), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((B, H, Nk, dv), generator=g).to(torch.bfloat16).to(dev)
    return q, k, v, g


def time_general(stream, steps: int, warmup: int):
    """attn_fwd_ex on the GENERAL workloads (seeded bf16 normal inputs),
    attn_fwd_split where it plans a split of the keys, and attn_bwd_ex on the
    shapes with more than one query.  Flops count the visible (query, key)
    pairs: 2 (d + dv) per pair forward, 2 (3 d + 2 dv) backward (S recomputed,
    dP, dV, dK, dQ); forward bytes are Q, K, V read once and O, LSE written once."""
    import torch

    import tiled_attention_09_amd as ta
    dev = torch.device("cuda:0")
    res = []
    for i, (name, B, H, Nq, Nk, d, dv, off, causal) in enumerate(GENERAL):
        q, k, v, g = _general_inputs(B, H, Nq, Nk, d, dv, dev)
        o = torch.empty((B, H, Nq, dv), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)

        def run():
            ta.attn_fwd_ex(q, k, v, 1.0 / d ** 0.5, causal, off, out=o, lse=lse,
                           stream=stream.cuda_stream)

        ms = event_ms(run, stream, steps, warmup)
        pairs = sum(min(Nk, off + i + 1) for i in range(Nq)) if causal else Nq * Nk
        flops = 2.0 * (d + dv) * B * H * pairs
        nbytes = B * H * (Nq * d * 2 + Nk * (d + dv) * 2 + Nq * dv * 4 + Nq * 4)
        tflops = flops / (ms * 1e-3) / 1e12
        gbs = nbytes / (ms * 1e-3) / 1e9
        hbm_bound = flops / nbytes < (PEAK_BF16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
        traffic = measured_traffic("headline", PATH_TRAFFIC_FILE, FWD_SOURCES, "general_%d" % i)
        roof = roofline_hbm(gbs, traffic) if hbm_bound else roofline_mfma(tflops, traffic=traffic)
        entry = {"workload": name, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "dv": dv,
                 "query_offset": off, "causal": causal, "kernel_ms": round(ms, 5),
                 "tflops": round(tflops, 2), "gbs": round(gbs, 1), "flops": flops,
                 "alg_bytes": nbytes, "roofline": roof, "steps": steps}
        if Nq > 1:
            g_out = torch.randn((B, H, Nq, dv), generator=g).to(torch.bfloat16).to(dev)
            ws = torch.empty(max(ta.attn_bwd_workspace_size(B, H, Nq), 16), dtype=torch.uint8,
                             device=dev)
            grads = (torch.empty((B, H, Nq, d), dtype=torch.float32, device=dev),
                     torch.empty((B, H, Nk, d), dtype=torch.float32, device=dev),
                     torch.empty((B, H, Nk, dv), dtype=torch.float32, device=dev))

            def bwd():
                ta.attn_bwd_ex(q, k, v, o, lse, g_out, 1.0 / d ** 0.5, causal, off, workspace=ws,
                               grads=grads, stream=stream.cuda_stream)

            bms = event_ms(bwd, stream, steps, warmup)
            bflops = 2.0 * (3 * d + 2 * dv) * B * H * pairs
            btf = bflops / (bms * 1e-3) / 1e12
            entry["backward"] = {"kernel_ms": round(bms, 5), "tflops": round(btf, 2),
                                 "flops": bflops, "roofline": roofline_mfma(btf)}
            del g_out, ws, grads
        ws_bytes = ta.attn_fwd_split_workspace_size(B, H, Nq, Nk, dv)
        if ws_bytes > 0:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

            def split():
                ta.attn_fwd_split(q, k, v, 1.0 / d ** 0.5, causal, off, out=o, lse=lse,
                                  workspace=ws, stream=stream.cuda_stream)

            sms = event_ms(split, stream, steps, warmup)
            sgbs = nbytes / (sms * 1e-3) / 1e9
            stf = flops / (sms * 1e-3) / 1e12
            st = measured_traffic("headline", PATH_TRAFFIC_FILE, FWD_SOURCES, "split_%d" % i)
            entry["split_keys"] = {
                "kernel_ms": round(sms, 5), "tflops": round(stf, 2), "gbs": round(sgbs, 1),
                "workspace_bytes": ws_bytes,
                "roofline": roofline_hbm(sgbs, st) if hbm_bound else roofline_mfma(stf, traffic=st)}
            del ws
        res.append(entry)
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return res


def time_sweep(stream, steps: int, warmup: int):
    """Forward and backward latency and device memory as the sequence grows
    (B=1, H=16, d=128, causal, seeded bf16 normal inputs).  ``peak_bytes`` is
    torch's peak allocation while the step's buffers (Q, K, V, dO, O, LSE,
    dQ, dK, dV, workspace) exist; the N x N score matrix of one head, which the
    method never stores, is listed beside it."""
    import torch

    import tiled_attention_09_amd as ta
    from tiled_attention_09_amd.synth import make_dout, make_qkv
    dev = torch.device("cuda:0")
    B, H, d = 1, 16, 128
    points = []
    for N in SWEEP_N:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        q, k, v = (x.to(dev) for x in make_qkv(B, H, N, d, 600 + N))
        g = make_dout(B, H, N, d, 600 + N).to(dev)
        o, lse = ta.attn_fwd(q, k, v, causal=True)
        grads = ta.attn_bwd(q, k, v, o, lse, g, causal=True)
        ws = torch.empty(ta.attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=dev)

        def fwd():
            ta.attn_fwd(q, k, v, causal=True, out=o, lse=lse, stream=stream.cuda_stream)

        def bwd():
            ta.attn_bwd(q, k, v, o, lse, g, causal=True, workspace=ws, grads=grads,
                        stream=stream.cuda_stream)

        fl = 2.0 * B * H * N * N * d
        event_ms(fwd, stream, 1, warmup)
        f_per = per_launch_ms(fwd, stream, max(steps, 10))
        event_ms(bwd, stream, 1, warmup)
        b_per = per_launch_ms(bwd, stream, max(steps, 10))
        f_ms, b_ms = spread(f_per)["median"], spread(b_per)["median"]
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        points.append({"N": N, "fwd_ms": f_ms, "bwd_ms": b_ms,
                       "fwd_tflops": round(fl / (f_ms * 1e-3) / 1e12, 2),
                       "bwd_tflops": round(2.5 * fl / (b_ms * 1e-3) / 1e12, 2),
                       "peak_bytes": int(peak),
                       "score_matrix_bytes_not_stored": int(B * H * N * N * 4)})
        del q, k, v, g, o, lse, grads, ws
    torch.cuda.empty_cache()
    return {"what": "latency (median per launch) and device memory vs sequence length",
            "B": B, "H": H, "d": d, "causal": True, "points": points}


# ---------------------------------------------------------------- counter passes

def time_library_gemm(stream, n: int = 8192) -> dict:
    """The vendor BLAS library's bf16 GEMM (torch.matmul, n x n x n) timed the
    same way in the same process: the matrix rate a plain library contraction
    reaches on this chip at the clock it sustains, beside the attention
    kernels' fractions of the published peak.  Context only: no attention
    arithmetic runs here."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)

    def mm():
        torch.matmul(a, b, out=c)

    warm_for(mm, 1.0)
    per = per_launch_ms(mm, stream, 5, batch=20)
    ms = statistics.median(per)
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    out = {"what": "torch.matmul bf16 %d x %d x %d (ROCm BLAS library), context for the "
                   "attention kernels' fractions of peak" % (n, n, n),
           "ms": round(ms, 5), "tflops": round(tf, 1),
           "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del a, b, c
    torch.cuda.empty_cache()
    return out


def counter_pass(w, launches: int = 3):
    """For rocprofv3 --pmc runs: one plain device copy of COPY_BYTES (the
    calibration dispatch), then ``launches`` dispatches of each measured path
    in this order -- forward, backward (row statistics, dK/dV, dQ), the two
    quantiser passes' kernels and the FP8-score forward, the dropout forward
    and backward, and each general-shape forward (and its split form)."""
    import torch

    import tiled_attention_09_amd as ta
    from tiled_attention_09_amd.synth import make_dout, make_workload
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in make_workload(w))
    g = make_dout(w.B, w.H, w.N, w.d, w.seed).to(dev)
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    qd = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    kd = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    gen = []
    for (name, B, H, Nq, Nk, d, dv, off, causal) in GENERAL:
        gq, gk, gv, _ = _general_inputs(B, H, Nq, Nk, d, dv, dev)
        ws_bytes = ta.attn_fwd_split_workspace_size(B, H, Nq, Nk, dv)
        gws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        gen.append((gq, gk, gv, off, causal, d, ws_bytes, gws))
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        o, lse = ta.attn_fwd(q, k, v, w.scale, w.causal)
    torch.cuda.synchronize()
    for _ in range(launches):
        ta.attn_bwd(q, k, v, o, lse, g, w.scale, w.causal)
    torch.cuda.synchronize()
    for _ in range(launches):
        ta.attn_quantize_fp8(q, out=q8, descale=qd)
        ta.attn_quantize_fp8(k, out=k8, descale=kd)
    torch.cuda.synchronize()
    for _ in range(launches):
        ta.attn_fwd_fp8(q8, k8, v, qd, kd, w.scale, w.causal)
    torch.cuda.synchronize()
    for _ in range(launches):
        od, ld = ta.attn_fwd_dropout(q, k, v, DROP_SEED, DROP_T, w.scale, w.causal)
    torch.cuda.synchronize()
    for _ in range(launches):
        ta.attn_bwd_dropout(q, k, v, od, ld, g, DROP_SEED, DROP_T, w.scale, w.causal)
    torch.cuda.synchronize()
    for (gq, gk, gv, off, causal, d, ws_bytes, gws) in gen:
        for _ in range(launches):
            ta.attn_fwd_ex(gq, gk, gv, 1.0 / d ** 0.5, causal, off)
        torch.cuda.synchronize()
        if ws_bytes:
            for _ in range(launches):
                ta.attn_fwd_split(gq, gk, gv, 1.0 / d ** 0.5, causal, off, workspace=gws)
            torch.cuda.synchronize()
    print("counter pass: 1 copy of %d bytes, then %d launches of each path (%s)" % (
        COPY_BYTES, launches, w.describe()), flush=True)


def _pmc_rows(directory: str, counter: str):
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit("no *counter_collection.csv under %s" % directory)
    rows = []
    for p in paths:
        rows += [r for r in csv.DictReader(open(p)) if r.get("Counter_Name", counter) == counter]
    rows.sort(key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0))))
    return rows


def summarize_counters(fetch_dir: str, write_dir: str, launches: int = 3):
    """Turn the FETCH_SIZE and WRITE_SIZE runs of ``--counter-pass`` into the
    traffic summaries bench.py reads: each counter is scaled by what it reads
    for the calibration copy of COPY_BYTES, per launch, keyed by the sha256 of
    the kernel's sources."""
    from tiled_attention_09_amd.synth import WORKLOADS
    w = WORKLOADS["headline"]
    fr, wr = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")

    def copy_kib(rows):
        vals = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        return max(vals)

    cf, cw = copy_kib(fr), copy_kib(wr)
    ff, wf = (COPY_BYTES / 1024.0) / cf, (COPY_BYTES / 1024.0) / cw
    calib = {"bytes": COPY_BYTES, "fetch_size_kib": round(cf, 1), "write_size_kib": round(cw, 1),
             "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
    def attention_dispatches(rows):
        """The library's dispatches after the calibration copy, in order."""
        first = max(i for i, r in enumerate(rows) if "copyBuffer" in r["Kernel_Name"]) + 1
        return [r for r in rows[first:] if "tiledattn" in r["Kernel_Name"]]

    # The FETCH and WRITE runs dispatch the same sequence.
    f_att, w_att = attention_dispatches(fr), attention_dispatches(wr)
    if [r["Kernel_Name"] for r in f_att] != [r["Kernel_Name"] for r in w_att]:
        raise SystemExit("the two counter runs dispatched different kernels")
    seq = [(r["Kernel_Name"], float(r["Counter_Value"]), float(s["Counter_Value"]))
           for r, s in zip(f_att, w_att)]
    pos = [0]

    def take(kernels_per_launch: int):
        """The next ``launches`` groups of ``kernels_per_launch`` dispatches."""
        groups = []
        for _ in range(launches):
            groups.append(seq[pos[0]:pos[0] + kernels_per_launch])
            pos[0] += kernels_per_launch
        return groups

    def summary(groups, alg, sources, label):
        per = [sum(f for _, f, _ in g) * 1024 * ff + sum(x for _, _, x in g) * 1024 * wf
               for g in groups]
        fb = sum(sum(f for _, f, _ in g) for g in groups) / len(groups) * 1024 * ff
        wb = sum(sum(x for _, _, x in g) for g in groups) / len(groups) * 1024 * wf
        kern = sorted({re.sub(r"\(.*", "", n).replace("void ", "") for g in groups for n, _, _ in g})
        return {"what": label, "kernels": kern, "kernel_source_sha256": kernel_source_hash(sources),
                "bytes_per_launch_each": [int(x) for x in per],
                "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
                "bytes_per_launch": int(fb + wb), "algorithmic_bytes_per_launch": alg,
                "ratio_to_algorithmic": round((fb + wb) / alg, 3) if alg else None}

    n = w.B * w.H * w.N
    fwd = summary(take(1), w.alg_bytes, FWD_SOURCES, "forward, headline workload")
    bwd_alg = 4 * n * w.d * 2 + n * w.d * 4 + n * 4 + 3 * n * w.d * 4   # q,k,v,dO + O + LSE + dq,dk,dv
    bwd = summary(take(3), bwd_alg, BWD_SOURCES, "backward (row statistics, dK/dV, dQ)")
    quant = summary(take(8), 2 * (n * w.d * 3 + w.B * w.H * 8), FP8_SOURCES,
                    "FP8 quantiser of Q and K (4 kernels each)")
    f8 = summary(take(1), n * w.d * (1 + 1 + 2) + n * w.d * 4 + n * 4 + w.B * w.H * 8, FP8_SOURCES,
                 "FP8-score forward")
    dfw = summary(take(1), w.alg_bytes, FWD_SOURCES, "dropout forward (t = %d)" % DROP_T)
    dbw = summary(take(3), bwd_alg, BWD_SOURCES, "dropout backward (t = %d)" % DROP_T)
    paths = {"fp8_quantize": quant, "fp8_forward": f8, "dropout_forward": dfw,
             "dropout_backward": dbw}
    import tiled_attention_09_amd as ta
    ta.load_library()
    for i, (name, B, H, Nq, Nk, d, dv, off, causal) in enumerate(GENERAL):
        nbytes = B * H * (Nq * d * 2 + Nk * (d + dv) * 2 + Nq * dv * 4 + Nq * 4)
        paths["general_%d" % i] = summary(take(1), nbytes, FWD_SOURCES, name)
        if ta.attn_fwd_split_workspace_size(B, H, Nq, Nk, dv):
            paths["split_%d" % i] = summary(take(2), nbytes, FWD_SOURCES, name + " (split keys)")
    if pos[0] != len(seq):
        raise SystemExit("dispatch count mismatch: used %d of %d" % (pos[0], len(seq)))
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc {C} "
           "--output-format csv -d <out>/meas_{C} -o tr -- python3 <repo>/bench.py --counter-pass")
    common = {"workload": "headline", "copy_calibration": calib,
              "commands": [cmd.format(C="FETCH_SIZE"), cmd.format(C="WRITE_SIZE")]}
    fwd_doc = dict(common, **fwd)
    fwd_doc["kernel"] = "attn_fwd_kernel<128, 128, causal, scale>0>"
    json.dump(fwd_doc, open(TRAFFIC_FILE, "w"), indent=1)
    bwd_doc = dict(common, **bwd)
    json.dump(bwd_doc, open(BWD_TRAFFIC_FILE, "w"), indent=1)
    json.dump(dict(common, paths=paths), open(PATH_TRAFFIC_FILE, "w"), indent=1)
    for k_, v_ in [("forward", fwd), ("backward", bwd)] + sorted(paths.items()):
        print("%-18s %8.1f MB  alg %8.1f MB  ratio %s" % (
            k_, v_["bytes_per_launch"] / 1e6, v_["algorithmic_bytes_per_launch"] / 1e6,
            v_["ratio_to_algorithmic"]))


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip every oracle timing (cpu_baseline and the per-config oracle)")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-general", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-dropout", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-gemm", action="store_true",
                    help="skip the library GEMM context figure")
    ap.add_argument("--no-device-probe", action="store_true",
                    help="no helper programs (driver/compiler versions, clock sampler)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="the calibration copy and a few launches of every path, for rocprofv3 --pmc")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_traffic.json from the two counter runs' CSVs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: heads shard across GPUs with no exchange, "
              "so there is no multi-GPU path to time (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return

    probes = not (args.counter_pass or args.no_device_probe or profiler_present())
    # Helper programs run only here, before anything touches the GPU.
    meta = host_metadata() if probes else {}
    sampler = start_clock_sampler() if probes else None

    import torch

    import tiled_attention_09_amd as ta
    from tiled_attention_09_amd.synth import WORKLOADS, make_workload

    w = WORKLOADS[args.workload]
    ta.load_library()
    if args.counter_pass:
        counter_pass(w)
        return
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    q, k, v = (x.to(dev) for x in make_workload(w))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step():
        ta.attn_fwd(q, k, v, w.scale, w.causal, out=o, lse=lse, stream=stream.cuda_stream)

    # The first call of the process (code-object load), timed on its own.
    torch.cuda.synchronize()
    t_cold = time.perf_counter()
    step()
    torch.cuda.synchronize()
    cold_ms = (time.perf_counter() - t_cold) * 1e3

    configs = None if args.no_configs else time_configs(stream)

    # The other legs' host-side set-up leaves the GPU idle for a while and its
    # clock drops; run the headline back to back for about 0.5 s (untimed)
    # before the W warm-up steps, so the timed steps see the clock this load
    # holds whatever W is.
    warm_for(step, 0.5)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    per = per_launch_ms(step, stream, min(max(args.steps, 10), 50))
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (kernel_ms * 1e-3) / 1e12
    device = device_info(dev, meta)
    # The clock under this load: the headline kernel back to back for ~3 s
    # while the sampler started above reads the graphics clock.
    if sampler is not None:
        t_a = time.time()
        while time.time() - t_a < 3.0:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        device["sclk_mhz_observed"] = stop_clock_sampler(sampler, t_a + 0.1, time.time())
    else:
        device["sclk_mhz_observed"] = None

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention fwd " + w.describe(), "B": w.B, "H": w.H, "N": w.N,
                   "d": w.d, "causal": w.causal, "seed": w.seed, "out_dtype": "fp32"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline_mfma(achieved, traffic=measured_traffic(w.name)),
        "kernel_ms": dict(mean=round(kernel_ms, 5), **spread(per), cold_first_call_ms=round(cold_ms, 3)),
        "device": device,
        "flops_per_step": w.flops,
        "alg_bytes_per_step": w.alg_bytes,
    }
    if configs is not None:
        out["configs"] = configs
    if not args.no_backward:
        out["backward"] = time_backward(w, q, k, v, o, lse, stream, args.steps, args.warmup)
    if not args.no_fp8:
        out["fp8_scores"] = time_fp8(w, q, k, v, stream, args.steps, args.warmup,
                                     out["kernel_ms"]["median"])
    if not args.no_dropout:
        out["dropout"] = time_dropout(w, q, k, v, stream, args.steps, args.warmup)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    if not args.no_general:
        out["general_shapes"] = time_general(stream, max(5, args.steps // 2), max(2, args.warmup // 2))
    if not args.no_sweep:
        out["seq_sweep"] = time_sweep(stream, min(args.steps, 20), max(2, args.warmup // 10))
    if not args.no_gemm:
        out["library_gemm"] = time_library_gemm(stream)
        out["library_gemm"]["forward_over_gemm"] = round(achieved / out["library_gemm"]["tflops"], 4)
    if not args.no_cpu_baseline:
        if configs is not None:
            add_config_oracle(configs)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
