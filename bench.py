#!/usr/bin/env python3
"""Benchmark of the fused single-token decode attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one decode-block call (RMSNorm, QKV projection, RoPE, KV append,
split-KV attention, output projection + residual) on one batch.  Inputs are
synthetic (seeded on the GPU with the shapes and distributions of the
configuration) and already resident in HBM when timing starts.  The step
cycles over R distinct layer-sets (weights, caches, hidden, out) whose total
size exceeds twice the 256 MiB Infinity Cache, so no step is served from it.

Prints one JSON line: microseconds per step (the metric), achieved HBM GB/s
and % of the 8 TB/s peak over the algorithmic bytes, a roofline entry for
the dominant kernel (the one with the longest average launch; its duration
from HIP events recorded at its own start and end on the stream it runs on), and the fp64 CPU oracle timed on the host as a
baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

from attention_block_amd.inputs import (CONFIGS, FFN_CONFIGS, HEADLINE, MLA_CONFIGS, BlockConfig,  # noqa: E402
                                        FfnConfig, MlaConfig, algorithmic_bytes, algorithmic_flops,
                                        ffn_algorithmic_bytes, ffn_algorithmic_flops, layer_ffn,
                                        mla_algorithmic_bytes, mla_algorithmic_flops, positions)

METRIC = "µs per decode block step and achieved HBM GB/s (% of peak), 7B layer bs1 4K"
FFN_METRIC = "µs per FFN half-layer decode step and achieved HBM GB/s (% of peak)"
MLA_METRIC = "µs per latent-attention (MLA) decode step and achieved HBM GB/s (% of peak)"
CHAIN_METRIC = "µs per token through a chain of synthetic decoder layers (attention block + FFN each)"
PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 1024 * 1024
PROFILES = os.path.join(HERE, "profiles")


def source_digest() -> str:
    """Digest of the library's kernel sources; a counter summary is only used for the sources it was taken on."""
    csrc = os.path.join(HERE, "attention_block_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE summary, or None when
    there is none or it was taken on other kernel sources."""
    path = os.path.join(PROFILES, f"pmc_traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^- (\w+): `?([^`\s]+)`?$", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("source_digest") != source_digest():
        return None
    return int(fields["hbm_bytes_per_launch"])


def phase_bytes(cfg: BlockConfig, pos) -> dict:
    """Algorithmic bytes of each kernel; they add up to algorithmic_bytes()."""
    s = 2 if cfg.dtype == "bf16" else 4
    B, H, nq, nkv, D = cfg.batch, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    tot = int(np.sum(pos))
    qkv = s * H * cfg.n_qkv + s * H + s * B * H + s * 2 * nkv * D * B + 4 * B
    attn = s * 2 * nkv * D * tot
    # the hidden row is counted once, with the QKV kernel; the O-projection writes out
    oproj = s * nq * D * H + s * B * H
    # the separate merge kernel reads and writes workspace only (the chunk partials, the attention output)
    return {"qkv_rmsnorm_rope_append": qkv, "attention_split_kv": attn, "oproj_residual": oproj,
            "attention_oproj_residual": attn + oproj, "qkv_attention_split_kv": qkv + attn, "attention_merge": 0,
            "decode_block_fused": qkv + attn + oproj}


def make_layer_set(cfg: BlockConfig, pos, cap: int, gen, device):
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, H, nq, nkv, D = cfg.batch, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    std = 1.0 / math.sqrt(H)

    def randn(*shape, scale=1.0, shift=0.0):
        return (torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * scale + shift).to(dt)

    ls = {
        "hidden": randn(B, H),
        "norm_w": randn(H, scale=0.1, shift=1.0),
        "w_qkv": randn(cfg.n_qkv, H, scale=std),     # one output feature per row
        "w_o": randn(H, nq * D, scale=std),
        "k_cache": torch.zeros(B, cap, nkv, D, dtype=dt, device=device),
        "v_cache": torch.zeros(B, cap, nkv, D, dtype=dt, device=device),
        "pos": torch.tensor(np.asarray(pos, dtype=np.int32), device=device),
    }
    for b in range(B):
        p = int(pos[b])
        ls["k_cache"][b, :p] = randn(p, nkv, D)
        ls["v_cache"][b, :p] = randn(p, nkv, D)
    ls["out"] = torch.empty_like(ls["hidden"])
    return ls



def host_cpu() -> dict:
    """The host cores this process may run on (its affinity mask) and the CPU model."""
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
    return {"cores": cores, "model": model}


class blas_threads:
    """Limit the BLAS thread pools numpy uses to `n` threads inside the block."""

    def __init__(self, n: int):
        self.n = n
        self._ctl = None

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
            self._ctl = threadpool_limits(limits=self.n)
        except Exception:
            self._ctl = None
        return self

    def __exit__(self, *exc):
        if self._ctl is not None:
            self._ctl.unregister()
        return False


def cpu_baseline(cfg: BlockConfig, seed: int, budget_s: float) -> dict:
    """The fp64 oracle on the host, on the full step of this workload."""
    import oracle
    from attention_block_amd.inputs import make_inputs
    inp = make_inputs(cfg, seed)
    st = cfg.dtype
    pos = inp["pos"]
    B, nkv, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    # exact upcast of the stored bits, outside the timed region
    kc = np.zeros((B, int(pos.max()) + 1, nkv, D))
    vc = np.zeros_like(kc)
    for b in range(B):
        kc[b, :pos[b]] = oracle.to_f64(inp["k_cache"][b, :pos[b]], st)
        vc[b, :pos[b]] = oracle.to_f64(inp["v_cache"][b, :pos[b]], st)
    args = (oracle.to_f64(inp["hidden"], st), oracle.to_f64(inp["norm_w"], st), oracle.to_f64(inp["w_qkv"], st),
            oracle.to_f64(inp["w_o"], st), kc, vc, pos)
    kw = dict(n_q_heads=cfg.n_q_heads, n_kv_heads=nkv, head_dim=D, rope_theta=cfg.rope_theta, eps=cfg.eps,
              storage=st)
    host = host_cpu()
    with blas_threads(host["cores"]):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.decode_step_fp64(*args, **kw)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s or len(times) >= 200:
                break
    med = float(np.median(times))
    return {"value": med * 1e6, "unit": "us/step", "cores": host["cores"], "cpu_model": host["model"],
            "kind": "oracle",
            "sample": f"{len(times)} full {cfg.name} steps (seed {seed}) of the fp64 numpy oracle, median; "
                      f"bf16->fp64 upcast outside the timing; BLAS threads = cores"}


# kernel function names (as rocprofv3 reports them) -> phase names of the C ABI
KERNEL_PHASES = [("fused_kernel", "decode_block_fused"),
                 ("qkv_attn_kernel", "qkv_attention_split_kv"), ("attn_oproj_kernel", "attention_oproj_residual"),
                 ("qkv_kernel", "qkv_rmsnorm_rope_append"), ("attn_kernel", "attention_split_kv"),
                 ("oproj_kernel", "oproj_residual"), ("merge_kernel", "attention_merge"),
                 ("ffn_gate_up_kernel", "ffn_rmsnorm_gate_up_silu"),
                 ("ffn_down_kernel", "ffn_down_residual"),
                 ("ffn_str_kernel", "ffn_rmsnorm_gate_up_silu"), ("ffn_str_down_kernel", "ffn_down_residual"),
                 ("mfma_str_qkv24_kernel", "qkv_rmsnorm_rope_append"),
                 ("mla_chunk_kernel", "mla_chunk"), ("mla_merge_kernel", "mla_merge")]


def ffn_phase_bytes(cfg: FfnConfig) -> dict:
    """Algorithmic bytes of the two FFN kernels; they add up to ffn_algorithmic_bytes()."""
    s = 2 if cfg.dtype == "bf16" else 4
    B, H, F = cfg.batch, cfg.hidden, cfg.intermediate
    # hidden is counted with the first kernel, out with the second
    return {"ffn_rmsnorm_gate_up_silu": s * 2 * H * F + s * H + s * B * H,
            "ffn_down_residual": s * H * F + s * B * H}


def mla_phase_bytes(cfg: MlaConfig, pos) -> dict:
    """Algorithmic bytes of the two latent-attention kernels: the chunk kernel moves all of them (cache rows,
    q, the new rows read and appended, the output), the merge kernel only workspace partials."""
    return {"mla_chunk": mla_algorithmic_bytes(cfg, pos), "mla_merge": 0}


def phase_of(kernel_name: str):
    fn = kernel_name.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0].split("::")[-1]
    if fn in ("mfma_panel_kernel", "mfma_res_kernel", "mfma_str_kernel"):   # template argument QKV: true or false
        return "qkv_rmsnorm_rope_append" if "<true" in kernel_name else "oproj_residual"
    if fn == "ffn_mfma_kernel":                               # template argument GATE_UP: true or false
        return "ffn_rmsnorm_gate_up_silu" if "<true" in kernel_name else "ffn_down_residual"
    for k, ph in KERNEL_PHASES:
        if fn == k:
            return ph
    return None


def summarize_profiles(kt_dir: str, fetch_dir: str, write_dir: str, workload: str, copy_mib: int,
                       commands: list, bench_json: str = "") -> list:
    """Write the rocprofv3 summaries under profiles/: the kernel-trace statistics of the library's kernels,
    and per kernel the HBM bytes of one launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by what the counter reads for the copy probe (copy_mib MiB read and written)."""
    import csv
    if workload in FFN_CONFIGS:
        pb = ffn_phase_bytes(FFN_CONFIGS[workload])
    elif workload in MLA_CONFIGS:
        mc = MLA_CONFIGS[workload]
        pb = mla_phase_bytes(mc, np.full(mc.batch, mc.pos))
    else:
        pb = phase_bytes(CONFIGS[workload], positions(CONFIGS[workload], 0))
    digest = source_digest()
    written = []

    stats = [r for r in csv.DictReader(open(os.path.join(kt_dir, "run_kernel_stats.csv"))) if phase_of(r["Name"])]
    lines = [f"# rocprofv3 kernel trace: {workload}", "",
             "Commands (from /tmp with TMPDIR=/tmp; R = the repository root):", ""]
    lines += [f"    {c}" for c in commands if "--pmc" not in c]
    lines += ["", "| phase | kernel | calls | average us | min us | max us | algorithmic bytes | GB/s at average |",
              "|---|---|---|---|---|---|---|---|"]
    for r in stats:
        ph = phase_of(r["Name"])
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| {ph} | `{r['Name'].split('(')[0]}` | {r['Calls']} | {avg:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {pb[ph]} | "
                     f"{pb[ph] / (avg * 1e-6) / 1e9:.1f} |")
    lines += ["", "bench.py times each kernel with HIP events that the kernel's own dispatch records at its start "
              "and end (hipExtLaunchKernel); under the profiler those events are perturbed, so its figures "
              "are taken from an unprofiled run of the same sources."]
    if bench_json:
        with open(bench_json) as f:
            line = json.loads([ln for ln in f if ln.startswith("{")][-1])
        lines += ["", f"Unprofiled `bench.py --config {workload}` on the same sources: {line['value']} us per step; "
                      "per-kernel averages from the dispatch events:", "",
                  "| phase | event average us | kernel-trace average us |", "|---|---|---|"]
        kt_avg = {phase_of(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}
        for ph, v in (line.get("phases") or {}).items():
            kt = kt_avg.get(ph)
            lines.append(f"| {ph} | {v['us']:.3f} | {kt:.3f} |" if kt is not None else f"| {ph} | {v['us']:.3f} | - |")
    lines += ["", f"- source_digest: `{digest}`"]
    path = os.path.join(PROFILES, f"kernel_trace_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    written.append(path)

    def counters(d, counter):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        rows = [r for r in rows if r["Counter_Name"] == counter]
        probe = [r for r in rows if "neg_kernel" in r["Kernel_Name"]]
        assert len(probe) == 1, f"expected one copy probe dispatch in {d}"
        per = {}
        for r in rows:
            ph = phase_of(r["Kernel_Name"])
            if ph:
                per.setdefault(ph, []).append(float(r["Counter_Value"]))
        return per, float(probe[0]["Counter_Value"])

    if fetch_dir == "-" or write_dir == "-":
        return written
    fetch, fetch_probe = counters(fetch_dir, "FETCH_SIZE")
    write, write_probe = counters(write_dir, "WRITE_SIZE")
    probe_kib = copy_mib * 1024.0
    f_scale, w_scale = probe_kib / fetch_probe, probe_kib / write_probe
    for ph in fetch:
        if not pb.get(ph):
            continue                     # workspace-only kernels have no algorithmic bytes to compare with
        fk, wk = float(np.mean(fetch[ph])), float(np.mean(write[ph]))
        fb, wb = fk * f_scale * 1024, wk * w_scale * 1024
        total = int(round(fb + wb))
        lines = [f"# HBM traffic of {ph}: {workload}", "",
                 "Counter runs (each its own rocprofv3 pass; from /tmp with TMPDIR=/tmp; R = the repository root):",
                 ""]
        lines += [f"    {c}" for c in commands if "--pmc" in c or "--summarize-profiles" in c]
        lines += ["",
                  f"Copy probe: one elementwise copy of {copy_mib} MiB ({probe_kib:.0f} KiB read, {probe_kib:.0f} KiB "
                  f"written) reads FETCH_SIZE {fetch_probe:.1f} KiB and WRITE_SIZE {write_probe:.1f} KiB, so the "
                  f"counters are scaled by {f_scale:.5f} (fetch) and {w_scale:.5f} (write).", "",
                  "| counter | dispatches | KiB per dispatch (mean) | scale | bytes per launch |", "|---|---|---|---|---|",
                  f"| FETCH_SIZE | {len(fetch[ph])} | {fk:.2f} | {f_scale:.5f} | {fb:.0f} |",
                  f"| WRITE_SIZE | {len(write[ph])} | {wk:.2f} | {w_scale:.5f} | {wb:.0f} |", "",
                  f"Measured HBM traffic per launch is {total / pb[ph]:.4f} x the algorithmic bytes.", "",
                  f"- hbm_bytes_per_launch: `{total}`",
                  f"- algorithmic_bytes_per_launch: `{pb[ph]}`",
                  f"- source_digest: `{digest}`"]
        path = os.path.join(PROFILES, f"pmc_traffic_{ph}_{workload}.md")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    return written


def read_probe(nbytes: int, device, stream_gib: float = 2.0, reps: int = 20) -> dict:
    """The library's read probe (one plain stream with the step's 16-byte non-temporal loads) as a
    bandwidth reference: over `stream_gib` GiB, and over exactly `nbytes` (the step's algorithmic bytes),
    cycling through enough distinct buffers that no launch is served from the Infinity Cache."""
    import torch
    import attention_block_amd as ab
    out = torch.empty(ab.READ_PROBE_BLOCKS, dtype=torch.int32, device=device)

    def timed(bufs, n):
        for b in bufs[:2]:
            ab.read_probe(b, out)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            ab.read_probe(bufs[i % len(bufs)], out)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) * 1e3 / n          # us per launch

    big = int(stream_gib * (1 << 30)) // 16 * 16
    buf = torch.ones(big // 4, dtype=torch.int32, device=device)
    us_big = timed([buf], reps)
    del buf
    step = max(16, nbytes // 16 * 16)
    nbuf = max(3, math.ceil(2 * MALL_BYTES / step) + 1)
    bufs = [torch.ones(step // 4, dtype=torch.int32, device=device) for _ in range(nbuf)]
    us_step = timed(bufs, max(reps, 4 * nbuf))
    del bufs
    return {"stream_gib": stream_gib, "stream_gbps": round(big / (us_big * 1e-6) / 1e9, 1),
            "step_bytes": step, "step_bytes_us": round(us_step, 3),
            "step_bytes_gbps": round(step / (us_step * 1e-6) / 1e9, 1)}


def graph_time(step, steps: int, R: int) -> float:
    """Microseconds per step over exactly `steps` steps replayed from HIP graphs.

    One captured launch sequence per step, over all layer-sets, so host-side
    marshalling never starves the GPU: a graph of L steps replayed steps // L
    times plus a remainder graph."""
    import torch
    import attention_block_amd as ab
    L = min(steps, R * max(1, math.ceil(64 / R)))

    def capture(nsteps, first):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(first)                     # warm call on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(nsteps):
                step(first + i)
        torch.cuda.synchronize()
        return g

    g_main = capture(L, 0)
    n_main, rem = divmod(steps, L)
    g_rem = capture(rem, 0) if rem else None
    g_main.replay()
    torch.cuda.synchronize()

    start, end = ab.HipEvent(), ab.HipEvent()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    # one more untimed replay right ahead of the start event: the GPU keeps streaming (clocks up, caches
    # and TLBs in their steady state) while the host submits the timed graphs, so the interval between
    # the events is the GPU time of the K steps, not the host's submission or a cold start
    g_main.replay()
    start.record(stream.cuda_stream)
    for _ in range(n_main):
        g_main.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record(stream.cuda_stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_ms(end) * 1e3 / steps


def event_phase_times(step, nphases: int, steps: int) -> list:
    """Average duration of each kernel over `steps` eager steps, from the events its own dispatch records
    (step(i, events) records events[2k] / events[2k + 1] at the start / end of kernel k); the steps are
    enqueued behind a spin kernel so that they run back to back on the GPU."""
    import torch
    import attention_block_amd as ab
    ev = [[ab.HipEvent() for _ in range(2 * nphases)] for _ in range(steps)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2.4e9 * 1e-4 * steps))   # ~100 us of spinning per queued step
    for i in range(steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    return [float(np.mean([ev[i][2 * k].elapsed_ms(ev[i][2 * k + 1]) * 1e3 for i in range(steps)]))
            for k in range(nphases)]


def make_ffn_set(cfg: FfnConfig, gen, device):
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, H, F = cfg.batch, cfg.hidden, cfg.intermediate

    def randn(*shape, scale=1.0, shift=0.0):
        return (torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * scale + shift).to(dt)

    ls = {"hidden": randn(B, H), "norm_w": randn(H, scale=0.1, shift=1.0),
          "w_gate": randn(F, H, scale=1 / math.sqrt(H)), "w_up": randn(F, H, scale=1 / math.sqrt(H)),
          "w_down": randn(H, F, scale=1 / math.sqrt(F))}      # one output feature per row
    ls["out"] = torch.empty_like(ls["hidden"])
    return ls


def ffn_cpu_baseline(cfg: FfnConfig, seed: int, budget_s: float) -> dict:
    """The fp64 FFN oracle on the host, on the full step of this workload."""
    import oracle
    from attention_block_amd.inputs import make_ffn_inputs
    inp = make_ffn_inputs(cfg, seed)
    st = cfg.dtype
    args = [oracle.to_f64(inp[k], st) for k in ("hidden", "norm_w", "w_gate", "w_up", "w_down")]
    host = host_cpu()
    with blas_threads(host["cores"]):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.ffn_step_fp64(*args, eps=cfg.eps, storage=st)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s or len(times) >= 200:
                break
    med = float(np.median(times))
    return {"value": med * 1e6, "unit": "us/step", "cores": host["cores"], "cpu_model": host["model"],
            "kind": "oracle",
            "sample": f"{len(times)} full {cfg.name} steps (seed {seed}) of the fp64 numpy FFN oracle, median; "
                      f"bf16->fp64 upcast outside the timing; BLAS threads = cores"}


def bench_ffn(args, dev) -> int:
    """The FFN half of the layer: RMSNorm + gate/up + silu, then down + residual, one JSON line."""
    import torch
    import attention_block_amd as ab
    cfg = FFN_CONFIGS[args.config]
    nbytes = ffn_algorithmic_bytes(cfg)
    R = max(3, math.ceil(2 * MALL_BYTES / nbytes) + 1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321 + args.seed)
    sets = [make_ffn_set(cfg, gen, dev) for _ in range(R)]
    c = ab.DabFfnConfig(cfg.batch, cfg.hidden, cfg.intermediate, ab.DAB_BF16 if cfg.dtype == "bf16" else ab.DAB_F32,
                        cfg.eps)
    ws = ab.Workspace(ab.ffn_workspace_size(c), dev)
    phases = list(ab.FFN_PHASES)

    def step(i, events=None):
        s = sets[i % R]
        w = (s["hidden"], s["norm_w"], s["w_gate"], s["w_up"], s["w_down"], cfg.eps)
        if events is None:
            ab.decode_ffn_block(*w, out=s["out"], workspace=ws, weight_layout="out_in")
        else:
            ab.decode_ffn_block_timed(events, *w, out=s["out"], workspace=ws, weight_layout="out_in")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    us = graph_time(step, args.steps, R)
    phase_us = None if args.no_phase_timing else event_phase_times(step, len(phases), args.steps)
    pb = ffn_phase_bytes(cfg)
    roofline = phase_report = None
    if phase_us is not None:
        # the dominant kernel: the one with the longest average launch
        k = max(range(len(phases)), key=lambda i: phase_us[i])
        dom = phases[k]
        ach = pb[dom] / (phase_us[k] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_GBPS, 4), "traffic": measured_traffic(dom, cfg.name), "kernel": dom,
                    "bytes_per_launch": pb[dom], "avg_launch_us": round(phase_us[k], 3)}
        phase_report = {n: {"us": round(phase_us[i], 3), "bytes": pb[n],
                            "gbps": round(pb[n] / (phase_us[i] * 1e-6) / 1e9, 1)} for i, n in enumerate(phases)}
    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
    cpu = None if args.no_cpu_baseline else ffn_cpu_baseline(cfg, args.seed, args.cpu_budget)
    gbps = nbytes / (us * 1e-6) / 1e9
    line = {
        "metric": FFN_METRIC, "value": round(us, 3), "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "hidden": cfg.hidden,
                   "intermediate": cfg.intermediate, "layer_sets": R, "parallelism": "single GPU",
                   "schedule": "+".join(phases)},
        "hbm_gbps": round(gbps, 1), "hbm_pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "algorithmic_bytes": nbytes, "algorithmic_flops": ffn_algorithmic_flops(cfg),
        "roofline": roofline, "phases": phase_report, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def make_mla_set(cfg: MlaConfig, cap: int, gen, device):
    import torch
    B, nh, R, P = cfg.batch, cfg.n_heads, cfg.kv_lora_rank, cfg.rope_dim

    def randn(*shape, scale=1.0, dt=torch.bfloat16):
        return (torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * scale).to(dt)

    ls = {"q_lat": randn(B, nh, R, scale=0.5, dt=torch.float32), "q_rope": randn(B, nh, P, dt=torch.float32),
          "c_new": randn(B, R), "kr_new": randn(B, P),
          "c_cache": torch.zeros(B, cap, R, dtype=torch.bfloat16, device=device),
          "kr_cache": torch.zeros(B, cap, P, dtype=torch.bfloat16, device=device),
          "pos": torch.full((B,), cfg.pos, dtype=torch.int32, device=device)}
    ls["c_cache"][:, :cfg.pos] = randn(B, cfg.pos, R)
    ls["kr_cache"][:, :cfg.pos] = randn(B, cfg.pos, P)
    ls["out"] = torch.empty(B, nh, R, dtype=torch.float32, device=device)
    return ls


def mla_cpu_baseline(cfg: MlaConfig, seed: int, budget_s: float) -> dict:
    """The fp64 latent-attention oracle on the host, on whole sequences of this workload."""
    import oracle
    from attention_block_amd.inputs import make_mla_inputs
    one = MlaConfig(cfg.name, 1, cfg.n_heads, cfg.pos, cfg.kv_lora_rank, cfg.rope_dim, cfg.softmax_scale, cfg.dtype)
    inp = make_mla_inputs(one, seed)
    host = host_cpu()
    with blas_threads(host["cores"]):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.mla_decode_from_inputs(inp)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s or len(times) >= 200:
                break
    med = float(np.median(times)) * cfg.batch
    return {"value": med * 1e6, "unit": "us/step", "cores": host["cores"], "cpu_model": host["model"],
            "kind": "oracle",
            "sample": f"{len(times)} single-sequence {cfg.name} steps (seed {seed}) of the fp64 numpy MLA "
                      f"oracle (bf16 upcast included), median x batch {cfg.batch}; BLAS threads = cores"}


def bench_mla(args, dev) -> int:
    """Latent attention decode (chunk kernel + merge kernel), one JSON line."""
    import torch
    import attention_block_amd as ab
    cfg = MLA_CONFIGS[args.config]
    pos = np.full(cfg.batch, cfg.pos)
    cap = max(args.cap, cfg.pos + 1)
    nbytes = mla_algorithmic_bytes(cfg, pos)
    flops = mla_algorithmic_flops(cfg, pos)
    R = max(3, math.ceil(2 * MALL_BYTES / nbytes) + 1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2468 + args.seed)
    sets = [make_mla_set(cfg, cap, gen, dev) for _ in range(R)]
    c = ab.DabMlaConfig(cfg.batch, cfg.n_heads, cfg.kv_lora_rank, cfg.rope_dim, cap, cfg.softmax_scale, args.kv_chunk)
    ws = ab.Workspace(ab.mla_workspace_size(c), dev)
    phases = list(ab.MLA_PHASES)

    def step(i, events=None):
        s = sets[i % R]
        a = (s["q_lat"], s["q_rope"], s["c_new"], s["kr_new"], s["c_cache"], s["kr_cache"], s["pos"],
             cfg.softmax_scale)
        if events is None:
            ab.mla_decode_attn(*a, kv_chunk=args.kv_chunk, out=s["out"], workspace=ws)
        else:
            ab.mla_decode_attn_timed(events, *a, kv_chunk=args.kv_chunk, out=s["out"], workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if ab.read_device_error(ws) != 0:
        print("device error flag raised during warm-up", file=sys.stderr)
        return 1
    us = graph_time(step, args.steps, R)
    phase_us = None if args.no_phase_timing else event_phase_times(step, len(phases), args.steps)
    pb = mla_phase_bytes(cfg, pos)
    roofline = phase_report = None
    if phase_us is not None:
        k = max(range(len(phases)), key=lambda i: phase_us[i])
        dom = phases[k]
        ach = pb[dom] / (phase_us[k] * 1e-6) / 1e9
        # 240 flops per byte at 128 heads: below the bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312), so HBM bounds it
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_GBPS, 4), "traffic": measured_traffic(dom, cfg.name), "kernel": dom,
                    "bytes_per_launch": pb[dom], "avg_launch_us": round(phase_us[k], 3),
                    "mfma_tflops": round(flops / (phase_us[k] * 1e-6) / 1e12, 1)}
        phase_report = {n: {"us": round(phase_us[i], 3), "bytes": pb[n],
                            "gbps": round(pb[n] / (phase_us[i] * 1e-6) / 1e9, 1)} for i, n in enumerate(phases)}
    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
    cpu = None if args.no_cpu_baseline else mla_cpu_baseline(cfg, args.seed, args.cpu_budget)
    gbps = nbytes / (us * 1e-6) / 1e9
    line = {
        "metric": MLA_METRIC, "value": round(us, 3), "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "heads": cfg.n_heads, "kv_lora_rank": cfg.kv_lora_rank,
                   "rope_dim": cfg.rope_dim, "kv_tokens": cfg.pos, "cache_capacity": cap, "layer_sets": R,
                   "kv_chunk": args.kv_chunk, "parallelism": "single GPU", "schedule": "+".join(phases)},
        "hbm_gbps": round(gbps, 1), "hbm_pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
        "roofline": roofline, "phases": phase_report, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_chain(args, dev) -> int:
    """--layers N: one token through N decoder layers, each the attention block of --config followed by
    its FFN (distinct weights and caches per layer; layer l's output is layer l + 1's input), all N
    layers captured as one HIP graph; reports µs per token (a synthetic time per output token, without
    embedding, final norm and LM head)."""
    import torch
    import attention_block_amd as ab
    cfg = CONFIGS[args.config]
    fcfg = layer_ffn(cfg)
    N = args.layers
    pos = positions(cfg, args.seed)
    cap = int(pos.max()) + 1
    gen = torch.Generator(device=dev)
    gen.manual_seed(777 + args.seed)
    layers = []
    for _ in range(N):
        attn = make_layer_set(cfg, pos, cap, gen, dev)
        ffn = make_ffn_set(fcfg, gen, dev)
        layers.append((attn, ffn))
    x0 = layers[0][0]["hidden"]
    acfg = ab.make_config(batch=cfg.batch, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                          head_dim=cfg.head_dim, cache_capacity=cap, dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                          eps=cfg.eps, kv_chunk=args.kv_chunk, schedule=args.schedule)
    ws = ab.Workspace(ab.workspace_size(acfg), dev)
    ffn_c = ab.DabFfnConfig(fcfg.batch, fcfg.hidden, fcfg.intermediate,
                            ab.DAB_BF16 if fcfg.dtype == "bf16" else ab.DAB_F32, fcfg.eps)
    fws = ab.Workspace(ab.ffn_workspace_size(ffn_c), dev)
    # one dab_decode_layer call per layer in --layer-schedule, or with --two-calls the attention block and
    # the FFN as calls of their own
    overlapped = not args.two_calls and args.layer_schedule == "overlap"
    if overlapped and not ab.layer_overlapped(acfg, ffn_c):
        print(f"--layer-schedule overlap is not built for {args.config}", file=sys.stderr)
        return 2
    if overlapped:
        schedule = ab.phase_names(acfg)[0] + "+attention_oproj_ffn_gate_up+" + ab.FFN_PHASES[1]
    else:
        schedule = "+".join(ab.phase_names(acfg)) + " | " + "+".join(ab.FFN_PHASES)

    def token(_i=0):
        x = x0
        for attn, ffn in layers:
            if args.two_calls:
                h = ab.decode_attn_block(x, attn["norm_w"], attn["w_qkv"], attn["w_o"], attn["k_cache"],
                                         attn["v_cache"], attn["pos"], cfg.rope_theta, cfg.eps, out=attn["out"],
                                         workspace=ws, kv_chunk=args.kv_chunk, schedule=args.schedule,
                                         weight_layout="out_in")
                x = ab.decode_ffn_block(h, ffn["norm_w"], ffn["w_gate"], ffn["w_up"], ffn["w_down"], fcfg.eps,
                                        out=ffn["out"], workspace=fws, weight_layout="out_in")
            else:
                _, x = ab.decode_layer(x, attn["norm_w"], attn["w_qkv"], attn["w_o"], attn["k_cache"],
                                       attn["v_cache"], attn["pos"], ffn["norm_w"], ffn["w_gate"], ffn["w_up"],
                                       ffn["w_down"], cfg.rope_theta, cfg.eps, fcfg.eps, h=attn["out"],
                                       out=ffn["out"], workspace=ws, ffn_workspace=fws, kv_chunk=args.kv_chunk,
                                       schedule=args.schedule, layer_schedule=args.layer_schedule,
                                       weight_layout="out_in")

    for i in range(max(1, args.warmup // 10)):
        token(i)
    torch.cuda.synchronize()
    if ab.read_device_error(ws) != 0:
        print("device error flag raised during warm-up", file=sys.stderr)
        return 1
    steps = max(1, args.steps // 10)
    us = graph_time(token, steps, 1)
    if ab.read_device_error(ws) != 0:
        print("device error flag raised during timing", file=sys.stderr)
        return 1
    per_layer = algorithmic_bytes(cfg, pos) + ffn_algorithmic_bytes(fcfg)
    nbytes = N * per_layer
    gbps = nbytes / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        a = cpu_baseline(cfg, args.seed, args.cpu_budget / 2)
        f = ffn_cpu_baseline(fcfg, args.seed, args.cpu_budget / 2)
        cpu = {"value": N * (a["value"] + f["value"]), "unit": "us/token", "cores": max(a["cores"], f["cores"]),
               "kind": "oracle", "sample": f"one layer: {a['sample']}; {f['sample']}; times {N} layers"}
    line = {
        "metric": CHAIN_METRIC, "value": round(us, 3), "unit": "us/token", "n_gpus": 1, "steps": steps,
        "warmup": max(1, args.warmup // 10), "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name} x {N} layers", "layers": N, "batch": cfg.batch, "hidden": cfg.hidden,
                   "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}",
                   "intermediate": fcfg.intermediate, "kv_tokens": int(pos[0]) if cfg.ragged is None else
                   f"ragged sum {int(np.sum(pos))}", "parallelism": "single GPU",
                   "schedule": schedule, "layer_call": "two calls" if args.two_calls else
                   f"dab_decode_layer ({args.layer_schedule})", "overlapped": bool(overlapped)},
        "hbm_gbps": round(gbps, 1), "hbm_pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "algorithmic_bytes": nbytes, "us_per_layer": round(us / N, 3),
        "algorithmic_flops": N * (algorithmic_flops(cfg, pos) + ffn_algorithmic_flops(fcfg)),
        # per-kernel events are not taken through the chain's graph: the entry covers the whole token
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_GBPS, 4), "traffic": None,
                     "kernel": f"whole token: {N} layers x ({schedule})", "bytes_per_launch": nbytes,
                     "avg_launch_us": round(us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=HEADLINE,
                    choices=sorted(CONFIGS) + sorted(FFN_CONFIGS) + sorted(MLA_CONFIGS),
                    help="a decode attention block workload, an FFN half-layer workload (*_ffn_*), or a "
                         "latent-attention (MLA) workload (*_mla_*)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layer-schedule", default="auto", choices=["auto", "sequential", "overlap"],
                    help="with --layers: dab_decode_layer's schedule (auto: sequential, measured faster)")
    ap.add_argument("--two-calls", action="store_true",
                    help="with --layers: run each layer as dab_decode_attn_block + dab_decode_ffn_block instead "
                         "of one dab_decode_layer call")
    ap.add_argument("--layers", type=int, default=0,
                    help="time one token through this many decoder layers (attention block of --config + its "
                         "FFN), one HIP graph; 0: the single attention block step")
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--cap", type=int, default=0,
                    help="cache capacity per sequence (token rows); 0: the largest position + 1")
    ap.add_argument("--pos-hint", action="store_true",
                    help="give the library the batch's largest position (dab_config.max_position), so that a "
                         "--cap far above the positions provisions no idle work")
    ap.add_argument("--schedule", default="auto", choices=["auto", "phased", "attn_oproj", "qkv_attn", "fused"])
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phase-timing", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the plain-stream bandwidth reference (the library's read probe)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("KERNEL_TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="turn rocprofv3 csv output (kernel trace, FETCH_SIZE pass, WRITE_SIZE pass of a "
                         "--copy-probe-mb run; '-' for no counter passes) into the summaries under profiles/ "
                         "for --config; no GPU needed")
    ap.add_argument("--commands", default="", help="with --summarize-profiles: the commands that made the "
                                                     "output, separated by ';', recorded in the summaries")
    ap.add_argument("--bench-json", default="", help="with --summarize-profiles: output of an unprofiled bench.py "
                                                      "run of the same sources, whose event timings are quoted")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one elementwise copy of this many MiB (fp32 in, fp32 out): the "
                         "reference kernel of known size for the FETCH_SIZE / WRITE_SIZE counter runs")
    args = ap.parse_args()

    if args.summarize_profiles:
        kt, fd, wd = args.summarize_profiles
        cmds = [c.strip() for c in args.commands.split(";") if c.strip()]
        for p in summarize_profiles(kt, fd, wd, args.config, args.copy_probe_mb or 256, cmds, args.bench_json):
            print("wrote", os.path.relpath(p, HERE))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode block runs on a single MI355X here "
              "(sharding across GPUs is described in the design notes but not built). Use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import attention_block_amd as ab

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.config in FFN_CONFIGS:
        return bench_ffn(args, dev)
    if args.config in MLA_CONFIGS:
        return bench_mla(args, dev)
    if args.layers > 0:
        return bench_chain(args, dev)
    cfg = CONFIGS[args.config]
    pos = positions(cfg, args.seed)
    cap = int(pos.max()) + 1
    if args.cap:
        if args.cap < cap:
            print(f"--cap {args.cap} is below the largest position + 1 ({cap})", file=sys.stderr)
            return 2
        cap = args.cap
    # --pos-hint: the configuration carries the batch's largest position (dab_config.max_position)
    max_position = int(pos.max()) if args.pos_hint and int(pos.max()) > 0 else 0
    nbytes = algorithmic_bytes(cfg, pos)
    flops = algorithmic_flops(cfg, pos)
    R = max(3, math.ceil(2 * MALL_BYTES / nbytes) + 1)

    gen = torch.Generator(device=dev)
    gen.manual_seed(1234 + args.seed)
    sets = [make_layer_set(cfg, pos, cap, gen, dev) for _ in range(R)]
    c = ab.make_config(batch=cfg.batch, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, cache_capacity=cap, dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                       eps=cfg.eps, kv_chunk=args.kv_chunk, schedule=args.schedule, max_position=max_position)
    ws = ab.Workspace(ab.workspace_size(c), dev)
    phases = ab.phase_names(c)

    def step(i, events=None):
        s = sets[i % R]
        if events is None:
            ab.decode_attn_block(s["hidden"], s["norm_w"], s["w_qkv"], s["w_o"], s["k_cache"], s["v_cache"],
                                 s["pos"], cfg.rope_theta, cfg.eps, out=s["out"], workspace=ws,
                                 kv_chunk=args.kv_chunk, schedule=args.schedule, weight_layout="out_in",
                                 max_position=max_position)
        else:
            ab.decode_attn_block_timed(events, s["hidden"], s["norm_w"], s["w_qkv"], s["w_o"], s["k_cache"],
                                       s["v_cache"], s["pos"], cfg.rope_theta, cfg.eps, out=s["out"],
                                       workspace=ws, kv_chunk=args.kv_chunk, schedule=args.schedule,
                                       weight_layout="out_in", max_position=max_position)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if ab.read_device_error(ws) != 0:
        print("device error flag raised during warm-up", file=sys.stderr)
        return 1

    us = graph_time(step, args.steps, R)
    if ab.read_device_error(ws) != 0:
        print("device error flag raised during timing", file=sys.stderr)
        return 1

    phase_us = None if args.no_phase_timing else event_phase_times(step, len(phases), args.steps)

    gbps = nbytes / (us * 1e-6) / 1e9
    pb = phase_bytes(cfg, pos)
    roofline = None
    phase_report = None
    if phase_us is not None:
        # the dominant kernel: the one with the longest average launch
        k = max(range(len(phases)), key=lambda i: phase_us[i])
        dom = phases[k]
        ach = pb[dom] / (phase_us[k] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_GBPS, 4), "traffic": measured_traffic(dom, cfg.name), "kernel": dom,
                    "bytes_per_launch": pb[dom], "avg_launch_us": round(phase_us[k], 3)}
        phase_report = {n: {"us": round(phase_us[i], 3), "bytes": pb[n],
                            "gbps": round(pb[n] / (phase_us[i] * 1e-6) / 1e9, 1)} for i, n in enumerate(phases)}

    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"copy probe: {n * 4} bytes read, {n * 4} bytes written", file=sys.stderr)

    probe = None if args.no_read_probe else read_probe(nbytes, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.seed, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "hidden": cfg.hidden,
                   "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}",
                   "kv_tokens": int(pos[0]) if cfg.ragged is None else f"ragged sum {int(np.sum(pos))}",
                   "cache_capacity": cap, "max_position": max_position, "layer_sets": R, "parallelism": "single GPU",
                   "schedule": "+".join(phases)},
        "hbm_gbps": round(gbps, 1),
        "hbm_pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": flops,
        "roofline": roofline,
        "phases": phase_report,
        "hbm_read_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
