#!/usr/bin/env python3
"""Benchmark of the alternating-attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
(Q, K, V resident in HBM): the layer schedule (host), one frame-attention
layer, one exact global-attention layer and one Subsampled Global Attention
layer (key selection, gather + mean, attention).  The default workload is
100 frames x 1374 tokens (37x37 patches + 5 specials), 16 heads x 64, bf16.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload n100|n300|n800|n800reg|shard8|sweep]

Prints ONE JSON line.  `value` is tokens/s through one step (T / step time).
With the default workload the line also carries, measured after the timed
steps, the 300- and 800-frame comparisons ("n300", "n800"): one exact global
layer against one SGA layer (2x2 at 300 frames, 3x3 at 800), with the frame
layer and the 24-slot AVGGT schedule at 800 frames (--no-extras skips them).
Other workloads:
  n300    -- one exact global layer vs one SGA 2x2 layer at 300 frames
             (speedup, output deviation);
  n800    -- the 24-slot AVGGT schedule (8 frame + 16 SGA 3x3) at 800 frames
             vs one exact global layer timed once (x24);
  n800reg -- register attention vs SGA 3x3 at 800 frames, each against one
             exact global layer (speed and output deviation), and the 24-slot
             schedules that use them;
  shard8  -- one device's share of an 8-way query-row split at 800 frames
             (rows [3T/8, 4T/8) against all keys), exact global and SGA 3x3,
             against the full layers;
  sweep   -- SGA at 300 frames over strides 2x2, 3x3, 4x4 and the ablations
             (unit-weight mean column, no diagonal, no mean column).
--copy-probe runs a plain 1 GiB device copy (for scaling HBM counters).
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

METRIC = ("attention tokens/s + TFLOP/s (% MFMA peak), exact vs SGA, "
          "N=100/300/800 frames")
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
HEAD_DIM = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work model
def flops_global(T, H, d=HEAD_DIM):
    """QK^T and PV: 2 * 2 * T * T * d per head."""
    return 4.0 * T * T * d * H


def flops_frame(N, L, H, d=HEAD_DIM):
    return 4.0 * N * L * L * d * H


def flops_sga(T, num_kept, H, d=HEAD_DIM):
    return 4.0 * T * num_kept * d * H


def flops_linear(T, c_in, c_out):
    """y = x W^T + b for T tokens: 2*T*c_in*c_out (the bias is negligible)."""
    return 2.0 * T * c_in * c_out


def bytes_gather(T, num_kept, H, d=HEAD_DIM, esize=2):
    """Read K and V once, write the kept rows of both."""
    return 2.0 * T * H * d * esize + 2.0 * num_kept * H * d * esize


def attention_matrix(tokens, bytes_per_entry):
    """(entries, bytes) of one dense tokens x tokens attention matrix."""
    n = float(tokens) * tokens
    return n, n * bytes_per_entry


# ---------------------------------------------------------------- helpers
class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.a = self.torch.cuda.Event(enable_timing=True)
        self.b = self.torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def cpu_baseline(workload, frames, sga_list, modes, qkv_host, rows_count, seed=7,
                 row_range=None, proj=None, counts=None):
    """The fp64 oracle on a bounded sample: `rows_count` seeded query rows
    (all heads) of each kind of layer of the step, each timed once, weighted
    by how often the step runs it (`counts`, aligned with modes + sga_list;
    default once each) and extrapolated x (rows of the step) / rows_count.
    row_range: the step's query rows (default all T).  proj: (x, w_qkv, b_qkv,
    w_o, b_o) host bits when every attention layer of the step sits between a
    QKV and an output projection (their rows are timed too)."""
    import oracle
    q, k, v = qkv_host
    T = frames.tokens
    r0, r1 = row_range if row_range is not None else (0, T)
    rows = r0 + np.sort(np.random.default_rng(seed).choice(r1 - r0, size=rows_count,
                                                            replace=False))
    args = (frames.num_frames, frames.tokens_per_frame, frames.grid_h, frames.grid_w, 0.125)
    counts = counts or [1] * (len(modes) + len(sga_list))
    assert len(counts) == len(modes) + len(sga_list)
    layer_s = []
    for mode in modes:
        code = {"frame": oracle.MODE_FRAME, "global": oracle.MODE_GLOBAL,
                "register": oracle.MODE_REGISTER}[mode]
        t0 = time.perf_counter()
        oracle.attention(code, q, k, v, *args, rows=rows)
        layer_s.append(time.perf_counter() - t0)
    for p in sga_list:
        t0 = time.perf_counter()
        oracle.attention(oracle.MODE_SGA, q, k, v, *args,
                         dict(stride_h=p.stride_h, stride_w=p.stride_w, phase_h=p.phase_h,
                              phase_w=p.phase_w, diagonal=int(p.diagonal),
                              mean_fill=int(p.mean_fill)), rows=rows)
        layer_s.append(time.perf_counter() - t0)
    if proj is not None:
        x, wqkv, bqkv, wo, bo = proj
        xr = np.ascontiguousarray(x[rows])
        for i in range(len(layer_s)):
            t0 = time.perf_counter()
            oracle.qkv_proj(xr, wqkv, bqkv, frames.num_heads)
            oracle.linear(xr, wo, bo)
            layer_s[i] += time.perf_counter() - t0
    dt = sum(layer_s)
    step_s = sum(c * t for c, t in zip(counts, layer_s)) * (r1 - r0) / rows_count
    return {"value": (r1 - r0) / step_s, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "host": host_cpu(),
            "sample": "%d seeded query rows x %d heads of each kind of layer of the step "
                      "(%s), timed %.1f s, weighted by its count in the step and "
                      "extrapolated x %d/%d" % (
                          rows_count, frames.num_heads,
                          "+".join("%dx%s" % (c, n) for c, n in
                                   zip(counts, list(modes) + ["sga"] * len(sga_list)))
                          + (", each with its QKV and output projections" if proj else ""),
                          dt, r1 - r0,
                          rows_count),
            "seconds_per_step": step_s}


def code_digest(path):
    """sha256 of a source file's code: comments and all whitespace removed,
    so that edits to comments or layout keep the digest."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    tok = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/', re.S)
    text = tok.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return hashlib.sha256(re.sub(r"\s+", "", text).encode()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE/WRITE_SIZE scaled by a plain copy), or None when the
    kernel code changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_n100.json")
    src = os.path.join(ROOT, "alternating_attention_amd", "csrc", "flash_attn.hip")
    try:
        rec = json.load(open(path))
        digest = code_digest(src)
    except (OSError, ValueError):
        return None
    if rec.get("sources_code_digest", {}).get("flash_attn.hip") != digest:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return k["hbm_bytes"] if k else None


def smi_sample():
    """Socket power (W) and the engine clock of each XCD (MHz) as amd-smi
    reports them (best effort: None when the tool is missing or fails)."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock"],
                           capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    pw = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", r.stdout)
    clk = [float(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([\d.]+)\s*MHz", r.stdout)]
    if pw is None and not clk:
        return None
    return {"socket_power_w": float(pw.group(1)) if pw else None, "gfx_clk_mhz": clk}


class SmiWatch:
    """Samples smi_sample() in a background thread while the timed region
    runs, so that the report shows the power and clock the work ran at."""

    def __init__(self, enabled):
        import threading
        self.enabled, self.samples = enabled, []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    def _loop(self):
        while not self._stop.is_set():
            rec = smi_sample()
            if rec is None:
                return
            self.samples.append(rec)
            self._stop.wait(0.25)

    def __enter__(self):
        if self.enabled:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.enabled:
            self._stop.set()
            self._thread.join()

    def summary(self):
        pw = sorted(x["socket_power_w"] for x in self.samples if x["socket_power_w"] is not None)
        clk = sorted(float(np.mean(x["gfx_clk_mhz"])) for x in self.samples if x["gfx_clk_mhz"])
        if not pw and not clk:
            return None
        return {"samples": len(self.samples),
                "socket_power_w_median": pw[len(pw) // 2] if pw else None,
                "socket_power_w_max": pw[-1] if pw else None,
                "gfx_clk_mhz_median": clk[len(clk) // 2] if clk else None}


def host_cpu():
    """Model, logical CPUs and sockets of the host (from /proc/cpuinfo; best
    effort: None where the file is missing)."""
    try:
        text = open("/proc/cpuinfo").read()
    except OSError:
        return None
    models = [l.split(":", 1)[1].strip() for l in text.splitlines() if l.startswith("model name")]
    sockets = {l.split(":", 1)[1].strip() for l in text.splitlines() if l.startswith("physical id")}
    return {"model": models[0] if models else None, "logical_cpus": len(models),
            "sockets": len(sockets) or None, "affinity_cpus": len(os.sched_getaffinity(0))}


def host_bits(t, torch):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def deviation(a, b):
    """max-abs, mean-abs and relative L2 of a - b (b the exact reference)."""
    d = a.float() - b.float()
    return {"max_abs": float(d.abs().max()), "mean_abs": float(d.abs().mean()),
            "rel_l2": float(d.norm() / b.float().norm())}


def flops_register(N, L, S, H, d=HEAD_DIM):
    """Frame attention for every row plus special rows over all N*S specials
    (the special rows' frame-attention work is included: the kernel does it)."""
    return flops_frame(N, L, H, d) + 4.0 * (N * S) ** 2 * d * H


# ---------------------------------------------------------------- workloads
def run(args):
    import torch
    import alternating_attention_amd as vga
    import vga_inputs

    base = {"n800reg": "n800", "n800ramp": "n800", "shard8": "n800", "sweep": "n300",
            "block": "n100"}
    w = vga_inputs.WORKLOADS[base.get(args.workload, args.workload)]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    frames = vga.Frames(w.num_frames, w.grid_h, w.grid_w, w.num_special, w.num_heads)
    T, H, N, L = frames.tokens, frames.num_heads, frames.num_frames, frames.tokens_per_frame
    log("generating %s (T=%d)" % (w.name, T))
    q, k, v = vga_inputs.feature_field_qkv(N, w.grid_h, w.grid_w, w.num_special, H, HEAD_DIM,
                                           seed=w.seed, device=dev)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    out_b = torch.empty_like(q)
    # the layer that precedes the SGA layer in the step, if any (the SGA
    # selection row is timed behind it)
    sel_prev = None
    timers = {}
    step_counts = None   # per kind of layer (modes, then SGA list) when the step repeats them

    def timed(name, fn):
        t = timers.setdefault(name, Timer(torch))
        with t:
            fn()

    if args.workload == "block":
        C = H * HEAD_DIM
        log("generating block inputs (token features and projection weights)")
        x, wqkv, bqkv, wo, bo = vga_inputs.feature_field_block(
            N, w.grid_h, w.grid_w, w.num_special, H, seed=w.seed + 10, device=dev)
        qkv = tuple(torch.empty_like(q) for _ in range(3))
        y = torch.empty((T, C), dtype=torch.bfloat16, device=dev)
        desc = ("N=100 frames x 1374 tokens = 137,400 tokens, 16 heads x 64 (C = 1024), bf16; "
                "step = a frame block and a global block, each the QKV projection "
                "(y = x W^T + b, 1024 -> 3072), the attention layer and the output "
                "projection (1024 -> 1024)")

        def step():
            for kind, fn in (("frame", vga.frame_attn), ("global", vga.global_attn)):
                timed("qkv_" + kind, lambda: vga.qkv_proj(x, wqkv, bqkv, frames, qkv))
                timed(kind, lambda fn=fn: fn(qkv[0], qkv[1], qkv[2], frames, out))
                timed("out_" + kind, lambda: vga.out_proj(out, wo, bo, frames, y))
        work = {"frame": flops_frame(N, L, H), "global": flops_global(T, H),
                "qkv_frame": flops_linear(T, C, 3 * C), "qkv_global": flops_linear(T, C, 3 * C),
                "out_frame": flops_linear(T, C, C), "out_global": flops_linear(T, C, C)}
        dominant, modes, sgas = "global", ["frame", "global"], []
    elif args.workload == "n100":
        sga = vga.Sga(2, 2, 0, 0, True, True)
        lay = vga.sga_workspace_layout(frames, sga)
        ws = torch.empty(int(lay.total), dtype=torch.uint8, device=dev)
        nk = int(lay.num_kept)
        desc = ("N=100 frames x 1374 tokens (37x37 patches + 5 specials) = 137,400 tokens, "
                "16 heads x 64, bf16; step = frame layer + exact global layer + SGA 2x2 layer "
                "(phase 0, diagonal, count-weighted mean-fill)")

        def step():
            vga.layer_schedule(3, 1, sga)
            timed("frame", lambda: vga.frame_attn(q, k, v, frames, out))
            timed("global", lambda: vga.global_attn(q, k, v, frames, out))
            timed("sga", lambda: vga.sga_attn(q, k, v, frames, sga, out_b, ws))
        sel_prev = ("the exact global layer", lambda: vga.global_attn(q, k, v, frames, out))
        work = {"frame": flops_frame(N, L, H), "global": flops_global(T, H),
                "sga": flops_sga(T, nk, H)}
        dominant, modes, sgas = "global", ["frame", "global"], [sga]
    elif args.workload == "n300":
        sga = vga.Sga(2, 2, 0, 0, True, True)
        lay = vga.sga_workspace_layout(frames, sga)
        ws = torch.empty(int(lay.total), dtype=torch.uint8, device=dev)
        nk = int(lay.num_kept)
        desc = ("N=300 frames x 1374 tokens = 412,200 tokens, 16 heads x 64, bf16; "
                "step = exact global layer + SGA 2x2 layer (phase 0, diagonal, mean-fill)")

        def step():
            timed("global", lambda: vga.global_attn(q, k, v, frames, out))
            timed("sga", lambda: vga.sga_attn(q, k, v, frames, sga, out_b, ws))
        sel_prev = ("the exact global layer", lambda: vga.global_attn(q, k, v, frames, out))
        work = {"global": flops_global(T, H), "sga": flops_sga(T, nk, H)}
        dominant, modes, sgas = "global", ["global"], [sga]
    elif args.workload == "n800":
        sga = vga.Sga(3, 3, 1, 1, True, True)
        lay = vga.sga_workspace_layout(frames, sga)
        ws = torch.empty(int(lay.total), dtype=torch.uint8, device=dev)
        nk = int(lay.num_kept)
        plan = vga.layer_schedule(24, 8, sga)
        desc = ("N=800 frames x 1374 tokens = 1,099,200 tokens, 16 heads x 64, bf16; "
                "step = the 24-slot AVGGT schedule: 8 frame layers + 16 SGA 3x3 layers "
                "(phase 1, diagonal, mean-fill); exact global layer timed once beside it")

        def step():
            # each slot through the schedule dispatch, as a trunk would run it
            for mode, p in vga.layer_schedule(24, 8, sga):
                name = "frame" if mode == vga.MODE_FRAME else "sga"
                dst = out if mode == vga.MODE_FRAME else out_b
                timed(name, lambda mode=mode, p=p, dst=dst:
                      vga.attention(mode, q, k, v, frames, p, dst, ws))
        work = {"frame": 8 * flops_frame(N, L, H), "sga": 16 * flops_sga(T, nk, H)}
        dominant, modes, sgas = "sga", ["frame"], [sga]
        step_counts = [8, 16]
        assert len(plan) == 24
    elif args.workload == "n800ramp":
        # per-layer strides: the SGA slots sample finely first, coarsely after
        ramp = [vga.Sga(2, 2, 0, 0, True, True)] * 8 + [vga.Sga(3, 3, 1, 1, True, True)] * 8
        plan = vga.layer_schedule_sga(24, 8, ramp)
        lays = {(p.stride_h, p.stride_w): vga.sga_workspace_layout(frames, p) for p in ramp}
        ws = torch.empty(int(max(l.total for l in lays.values())), dtype=torch.uint8, device=dev)
        desc = ("N=800 frames x 1374 tokens = 1,099,200 tokens, 16 heads x 64, bf16; "
                "step = a 24-slot schedule with per-layer strides: 8 frame layers, 8 SGA 2x2 "
                "layers (phase 0), 8 SGA 3x3 layers (phase 1), all with diagonal and "
                "mean-fill; exact global layer timed once beside it")

        def step():
            for mode, p in vga.layer_schedule_sga(24, 8, ramp):
                if mode == vga.MODE_FRAME:
                    timed("frame", lambda: vga.attention(mode, q, k, v, frames, None, out))
                else:
                    timed("sga_%dx%d" % (p.stride_h, p.stride_w),
                          lambda p=p: vga.attention(vga.MODE_SGA, q, k, v, frames, p, out_b, ws))
        work = {"frame": 8 * flops_frame(N, L, H),
                "sga_2x2": 8 * flops_sga(T, int(lays[(2, 2)].num_kept), H),
                "sga_3x3": 8 * flops_sga(T, int(lays[(3, 3)].num_kept), H)}
        dominant, modes, sgas = "sga_2x2", ["frame"], [ramp[0], ramp[8]]
        step_counts = [8, 8, 8]
        assert [m for m, _ in plan] == [vga.MODE_FRAME] * 8 + [vga.MODE_SGA] * 16
    elif args.workload == "n800reg":
        sga = vga.Sga(3, 3, 1, 1, True, True)
        lay = vga.sga_workspace_layout(frames, sga)
        ws = torch.empty(int(lay.total), dtype=torch.uint8, device=dev)
        rlay = vga.register_workspace_layout(frames)
        rws = torch.empty(int(rlay.total), dtype=torch.uint8, device=dev)
        nk = int(lay.num_kept)
        out_c = torch.empty_like(q)
        desc = ("N=800 frames x 1374 tokens = 1,099,200 tokens, 16 heads x 64, bf16; "
                "step = one register-attention layer (specials of all frames exchange, "
                "patches in frame) + one SGA 3x3 layer (phase 1, diagonal, mean-fill); "
                "exact global layer timed once beside it")

        def step():
            timed("register", lambda: vga.register_attn(q, k, v, frames, out_c, rws))
            timed("sga", lambda: vga.sga_attn(q, k, v, frames, sga, out_b, ws))
        work = {"register": flops_register(N, L, w.num_special, H),
                "sga": flops_sga(T, nk, H)}
        dominant, modes, sgas = "sga", ["register"], [sga]
    elif args.workload == "shard8":
        sga = vga.Sga(3, 3, 1, 1, True, True)
        lay = vga.sga_workspace_layout(frames, sga)
        ws = torch.empty(int(lay.total), dtype=torch.uint8, device=dev)
        nk = int(lay.num_kept)
        r0, r1 = 3 * T // 8, 4 * T // 8
        qr = q[r0:r1].contiguous()
        o_r = torch.empty_like(qr)
        desc = ("N=800 frames x 1374 tokens = 1,099,200 tokens, 16 heads x 64, bf16; "
                "step = one device's share of an 8-way query-row split: rows [%d, %d) "
                "against all keys, exact global layer + SGA 3x3 layer (selection and mean "
                "over all tokens); the full layers timed once beside it" % (r0, r1))

        def step():
            timed("global", lambda: vga.global_attn_rows(qr, k, v, frames, r0, o_r))
            timed("sga", lambda: vga.sga_attn_rows(qr, k, v, frames, sga, r0, o_r, ws))
        sel_prev = ("the row-range global layer",
                    lambda: vga.global_attn_rows(qr, k, v, frames, r0, o_r))
        work = {"global": 4.0 * (r1 - r0) * T * HEAD_DIM * H,
                "sga": 4.0 * (r1 - r0) * nk * HEAD_DIM * H}
        dominant, modes, sgas = "global", ["global"], [sga]
    elif args.workload == "sweep":
        variants = [("sga_2x2", vga.Sga(2, 2, 0, 0, True, 1)),
                    ("sga_3x3", vga.Sga(3, 3, 1, 1, True, 1)),
                    ("sga_4x4", vga.Sga(4, 4, 1, 1, True, 1)),
                    ("sga_2x2_unit_mean", vga.Sga(2, 2, 0, 0, True, 2)),
                    ("sga_2x2_no_diag", vga.Sga(2, 2, 0, 0, False, 1)),
                    ("sga_2x2_no_mean", vga.Sga(2, 2, 0, 0, True, 0))]
        lays = {n: vga.sga_workspace_layout(frames, p) for n, p in variants}
        ws = torch.empty(int(max(l.total for l in lays.values())), dtype=torch.uint8,
                         device=dev)
        outs = {n: torch.empty_like(q) for n, _ in variants}
        desc = ("N=300 frames x 1374 tokens = 412,200 tokens, 16 heads x 64, bf16; "
                "step = SGA at strides 2x2 (phase 0), 3x3 and 4x4 (phase 1), and at 2x2 "
                "with a unit-weight mean column, without the diagonal, without the mean "
                "column; exact global layer timed once beside it")

        def step():
            for n, p in variants:
                timed(n, lambda p=p, n=n: vga.sga_attn(q, k, v, frames, p, outs[n], ws))
        work = {n: flops_sga(T, int(lays[n].num_kept), H) for n, _ in variants}
        dominant, modes, sgas = "sga_2x2", [], [variants[0][1]]
        sga, nk, lay = variants[0][1], int(lays["sga_2x2"].num_kept), lays["sga_2x2"]
    else:
        raise SystemExit("unknown workload")

    state_before = None if args.no_gpu_state else smi_sample()
    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers.clear()
    log("timing %d steps" % args.steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with SmiWatch(not args.no_gpu_state) as watch:
        wall0 = time.perf_counter()
        t_start.record()
        for i in range(args.steps):
            step()
            log("  step %d enqueued" % i)
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    state_after = None if args.no_gpu_state else smi_sample()

    per = {}
    for name, t in timers.items():
        ms = t.ms()
        calls_per_step = len(ms) / args.steps
        avg = float(np.mean(ms))
        flop = work[name] / calls_per_step
        per[name] = {"ms_per_call": avg, "ms_median": float(np.median(ms)), "ms_min": float(min(ms)),
                     "calls_per_step": calls_per_step,
                     "tflops": flop / (avg * 1e-3) / 1e12,
                     "frac_mfma_peak": flop / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "tokens_per_s": T / (avg * 1e-3)}
    rows = {}
    if "sga" in per:
        gb = bytes_gather(T, nk, H)
        per["sga"]["gather_bytes"] = gb
        per["sga"]["kept_per_frame"] = int(lay.kept_per_frame)
        # the selection, gather and mean alone (the HBM-bound part of the SGA
        # call), timed after the steps on the same inputs and workspace, in
        # the step's own order: each call is queued right behind the layer
        # that precedes the SGA layer in the step (the exact global layer when
        # the step has one), so the GPU is still busy when its events are
        # enqueued (the host's launch latency does not count) and the caches
        # hold what that layer left, as in the step.  Reported beside it: 20
        # calls queued back to back (each behind the previous call's writes)
        # and one call on an idle stream (which also counts the launch
        # latency).
        if sel_prev is not None:
            prev_name, prev = sel_prev
        else:
            prev_name = "an SGA layer"
            prev = lambda: vga.sga_attn(q, k, v, frames, sga, out_b, ws)
        n_ctx = 5 if T <= 500_000 else 2
        ctx = Timer(torch)
        for _ in range(n_ctx):
            prev()
            with ctx:
                vga.sga_select(k, v, frames, sga, ws)
        torch.cuda.synchronize()
        n_sel = 20
        sel = Timer(torch)
        with sel:
            for _ in range(n_sel):
                vga.sga_select(k, v, frames, sga, ws)
        one = Timer(torch)
        for _ in range(10):
            torch.cuda.synchronize()
            with one:
                vga.sga_select(k, v, frames, sga, ws)
        torch.cuda.synchronize()
        sms = float(np.median(ctx.ms()))
        bms = float(sel.ms()[0]) / n_sel
        per["sga_select"] = {"ms_per_call": sms, "calls_per_step": 0.0,
                             "timing": "median of %d calls, each queued behind %s"
                                       % (n_ctx, prev_name),
                             "ms_all": [float(x) for x in ctx.ms()],
                             "ms_back_to_back": bms,
                             "ms_single_call_median": float(np.median(one.ms())),
                             "gb_per_s": gb / (sms * 1e-3) / 1e9,
                             "frac_hbm_peak": gb / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "frac_hbm_peak_back_to_back": gb / (bms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        att = per["sga"]["ms_per_call"] - sms
        fl_sga = work["sga"] / per["sga"]["calls_per_step"]
        rows["a3_a4_sga_select"] = {"bound": "hbm", "achieved": gb / (sms * 1e-3) / 1e9,
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": gb / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                    "algorithmic_bytes": gb, "ms": sms,
                                    "timing": per["sga_select"]["timing"]}
        rows["a5_sga_attention"] = {"bound": "mfma", "achieved": fl_sga / (att * 1e-3) / 1e12,
                                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                    "frac": fl_sga / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                    "ms": att, "note": "SGA call minus the selection call (in the step's order)"}
    for name, row in (("frame", "a1_frame"), ("global", "a2_global")):
        if name in per:
            rows[row] = {"bound": "mfma", "achieved": per[name]["tflops"],
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": per[name]["frac_mfma_peak"], "ms": per[name]["ms_per_call"]}

    extra = {}
    if args.workload == "n800reg":
        log("exact global layer, timed once")
        g = Timer(torch)
        with g:
            vga.global_attn(q, k, v, frames, out)
        torch.cuda.synchronize()
        gms = g.ms()[0]
        rms, sms = per["register"]["ms_per_call"], per["sga"]["ms_per_call"]
        fr = Timer(torch)
        with fr:
            vga.frame_attn(q, k, v, frames, out_b)
        torch.cuda.synchronize()
        fms = fr.ms()[0]
        per["global_once"] = {"ms_per_call": gms,
                              "tflops": flops_global(T, H) / (gms * 1e-3) / 1e12}
        per["frame_once"] = {"ms_per_call": fms}
        extra["register_vs_exact_layer_speedup"] = gms / rms
        extra["sga_vs_exact_layer_speedup"] = gms / sms
        vga.register_attn(q, k, v, frames, out_c, rws)
        vga.sga_attn(q, k, v, frames, sga, out_b, ws)
        torch.cuda.synchronize()
        extra["register_deviation"] = deviation(out_c, out)
        extra["sga_deviation"] = deviation(out_b, out)
        # 24 global slots, from the per-layer times above
        sched = {"exact_24_global": 24 * gms,
                 "avggt_8frame_16sga": 8 * fms + 16 * sms,
                 "omega_quarter_register_18global_6register": 18 * gms + 6 * rms,
                 "avggt_plus_register_8frame_4register_12sga": 8 * fms + 4 * rms + 12 * sms}
        extra["schedules_ms_from_layer_times"] = sched
        plan = [m for m, _ in vga.layer_schedule_register(24, 8, 4, sga)]
        assert plan.count(vga.MODE_REGISTER) == 4 and plan.count(vga.MODE_SGA) == 12
    if args.workload == "shard8":
        log("full layers, timed once")
        g = Timer(torch)
        with g:
            vga.global_attn(q, k, v, frames, out)
        with g:
            vga.sga_attn(q, k, v, frames, sga, out_b, ws)
        torch.cuda.synchronize()
        gms, sfull = g.ms()
        per["global_full_once"] = {"ms_per_call": gms}
        per["sga_full_once"] = {"ms_per_call": sfull}
        extra["row_split_efficiency_global"] = (gms / 8) / per["global"]["ms_per_call"]
        extra["row_split_efficiency_sga"] = (sfull / 8) / per["sga"]["ms_per_call"]
        vga.global_attn_rows(qr, k, v, frames, r0, o_r)
        torch.cuda.synchronize()
        extra["shard_vs_full_rows"] = deviation(o_r, out[r0:r1])
    if args.workload == "sweep":
        log("exact global layer, timed once")
        g = Timer(torch)
        with g:
            vga.global_attn(q, k, v, frames, out)
        torch.cuda.synchronize()
        gms = g.ms()[0]
        per["global_once"] = {"ms_per_call": gms}
        for n, p in variants:
            vga.sga_attn(q, k, v, frames, p, outs[n], ws)
            torch.cuda.synchronize()
            per[n]["kept_per_frame"] = int(lays[n].kept_per_frame)
            per[n]["speedup_vs_exact"] = gms / per[n]["ms_per_call"]
            per[n]["deviation_vs_exact"] = deviation(outs[n], out)
    if args.workload == "n800ramp":
        log("exact global layer, timed once")
        g = Timer(torch)
        with g:
            vga.global_attn(q, k, v, frames, out)
        torch.cuda.synchronize()
        gms = g.ms()[0]
        per["global_once"] = {"ms_per_call": gms,
                              "tflops": flops_global(T, H) / (gms * 1e-3) / 1e12}
        extra["schedule_vs_24_exact_speedup"] = 24 * gms / ms_step
        for p in (ramp[0], ramp[8]):
            name = "sga_%dx%d" % (p.stride_h, p.stride_w)
            vga.sga_attn(q, k, v, frames, p, out_b, ws)
            torch.cuda.synchronize()
            per[name]["speedup_vs_exact"] = gms / per[name]["ms_per_call"]
            per[name]["deviation_vs_exact"] = deviation(out_b, out)
            per[name]["kept_per_frame"] = int(lays[(p.stride_h, p.stride_w)].kept_per_frame)
    if args.workload in ("n300", "n800"):
        if args.workload == "n800":
            log("exact global layer, timed once")
            g = Timer(torch)
            with g:
                vga.global_attn(q, k, v, frames, out)
            torch.cuda.synchronize()
            gms = g.ms()[0]
            per["global_once"] = {"ms_per_call": gms,
                                  "tflops": flops_global(T, H) / (gms * 1e-3) / 1e12,
                                  "frac_mfma_peak": flops_global(T, H) / (gms * 1e-3) / 1e12
                                  / PEAK_BF16_TFLOPS}
            extra["schedule_vs_24_exact_speedup"] = 24 * gms / ms_step
            extra["sga_vs_exact_layer_speedup"] = gms / per["sga"]["ms_per_call"]
        else:
            extra["sga_vs_exact_layer_speedup"] = (per["global"]["ms_per_call"]
                                                   / per["sga"]["ms_per_call"])
        # deviation of SGA from exact attention (both from the GPU)
        vga.global_attn(q, k, v, frames, out)
        vga.sga_attn(q, k, v, frames, sga, out_b, ws)
        torch.cuda.synchronize()
        dev_ = (out_b.float() - out.float())
        extra["sga_deviation"] = {"max_abs": float(dev_.abs().max()),
                                  "mean_abs": float(dev_.abs().mean()),
                                  "rel_l2": float(dev_.norm() / out.float().norm())}

    flop_dom = work[dominant] / per[dominant]["calls_per_step"]
    ach = flop_dom / (per[dominant]["ms_per_call"] * 1e-3) / 1e12
    kernel = {"global": "flash_bf16_kernel<kGlobal>", "sga": "flash_bf16_kernel<kSga>",
              "sga_2x2": "flash_bf16_kernel<kSga>"}[dominant]
    if args.workload == "block":
        bl = {}
        for kind in ("frame", "global"):
            parts = [per[n]["ms_per_call"] for n in ("qkv_" + kind, kind, "out_" + kind)]
            bl[kind + "_block_ms"] = sum(parts)
            bl[kind + "_projection_share"] = (parts[0] + parts[2]) / sum(parts)
        extra_block = bl
    else:
        extra_block = None
    roofline = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": (measured_traffic(kernel) if args.workload in ("n100", "block")
                            else None),
                "kernel": kernel, "algorithmic_flops_per_launch": flop_dom}

    result = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded shifted-feature-field tokens projected by seeded random "
                "weights (no dataset, no trained weights)",
        "config": {"workload": desc, "frames": N, "tokens_per_frame": L, "tokens": T,
                   "heads": H, "head_dim": HEAD_DIM},
        "roofline": roofline, "rows": rows, "modes": per, "wall_s_timed": wall,
        "gpu_state": {"before": state_before, "during": watch.summary(), "after": state_after},
    }
    result.update(extra)
    if extra_block:
        result["blocks"] = extra_block
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, %d rows per layer)" % args.cpu_rows)
        qkv = (host_bits(q, torch), host_bits(k, torch), host_bits(v, torch))
        proj = None
        if args.workload == "block":
            proj = tuple(host_bits(t, torch) for t in (x, wqkv, bqkv, wo, bo))
        result["cpu_baseline"] = cpu_baseline(
            w, frames, sgas, modes, qkv, args.cpu_rows,
            row_range=(3 * T // 8, 4 * T // 8) if args.workload == "shard8" else None,
            proj=proj, counts=step_counts)
    if args.workload == "n100" and not args.no_extras:
        # the 300- and 800-frame comparisons of exact global attention with
        # SGA, after the timed step (not part of it)
        del q, k, v, out, out_b, ws
        torch.cuda.empty_cache()
        result["n300"] = speedup_record(vga, torch, "n300", vga.Sga(2, 2, 0, 0, True, True),
                                        with_frame=False)
        result["n800"] = speedup_record(vga, torch, "n800", vga.Sga(3, 3, 1, 1, True, True),
                                        with_frame=True)
    return result


def speedup_record(vga, torch, wname, sga, with_frame, reps=3):
    """One exact global layer (timed once, on the kernels already warm from
    the main workload) against the SGA layer (median of `reps` calls) on the
    seeded shifted-feature-field inputs of `wname`; with_frame: the frame
    layer too and the 24-slot AVGGT schedule (8 frame + 16 SGA) from the
    layer times.  Output deviation of SGA from exact attention, both from
    the GPU."""
    import vga_inputs
    w = vga_inputs.WORKLOADS[wname]
    dev = torch.device("cuda", 0)
    frames = vga.Frames(w.num_frames, w.grid_h, w.grid_w, w.num_special, w.num_heads)
    T, H, N, L = frames.tokens, frames.num_heads, frames.num_frames, frames.tokens_per_frame
    log("extra %s: generating inputs (T=%d)" % (wname, T))
    q, k, v = vga_inputs.feature_field_qkv(N, w.grid_h, w.grid_w, w.num_special, H, HEAD_DIM,
                                           seed=w.seed, device=dev)
    out, out_b = torch.empty_like(q), torch.empty_like(q)
    lay = vga.sga_workspace_layout(frames, sga)
    ws = torch.empty(int(lay.total), dtype=torch.uint8, device=dev)
    nk = int(lay.num_kept)
    torch.cuda.synchronize()

    def timed_calls(fn, n):
        t = Timer(torch)
        for _ in range(n):
            with t:
                fn()
        torch.cuda.synchronize()
        return t.ms()

    log("extra %s: SGA %dx%d layer x%d" % (wname, sga.stride_h, sga.stride_w, reps + 1))
    sga_ms = timed_calls(lambda: vga.sga_attn(q, k, v, frames, sga, out_b, ws), reps + 1)[1:]
    log("extra %s: exact global layer, once" % wname)
    g_ms = timed_calls(lambda: vga.global_attn(q, k, v, frames, out), 1)[0]
    t_sga = float(np.median(sga_ms))
    fg, fs = flops_global(T, H), flops_sga(T, nk, H)
    d = (out_b.float() - out.float())
    rec = {
        "workload": "N=%d frames x %d tokens = %d tokens, %d heads x 64, bf16; exact global "
                    "layer vs SGA %dx%d (phase %d, diagonal, count-weighted mean-fill)" % (
                        N, L, T, H, sga.stride_h, sga.stride_w, sga.phase_h),
        "global": {"ms": g_ms, "tflops": fg / (g_ms * 1e-3) / 1e12,
                   "frac_mfma_peak": fg / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                   "tokens_per_s": T / (g_ms * 1e-3), "calls": 1},
        "sga": {"ms": t_sga, "ms_all": sga_ms, "tflops": fs / (t_sga * 1e-3) / 1e12,
                "frac_mfma_peak": fs / (t_sga * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "tokens_per_s": T / (t_sga * 1e-3), "kept_per_frame": int(lay.kept_per_frame),
                "note": "whole call: selection, gather, mean and attention"},
        "sga_vs_exact_layer_speedup": g_ms / t_sga,
        "ideal_speedup_from_work": fg / fs,
        "sga_deviation": {"max_abs": float(d.abs().max()), "mean_abs": float(d.abs().mean()),
                          "rel_l2": float(d.norm() / out.float().norm())},
    }
    del d
    if with_frame:
        log("extra %s: frame layer x%d" % (wname, reps + 1))
        f_ms = float(np.median(timed_calls(lambda: vga.frame_attn(q, k, v, frames, out),
                                           reps + 1)[1:]))
        ff = flops_frame(N, L, H)
        rec["frame"] = {"ms": f_ms, "tflops": ff / (f_ms * 1e-3) / 1e12,
                        "frac_mfma_peak": ff / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        sched = 8 * f_ms + 16 * t_sga
        rec["schedule_24_slots"] = {
            "avggt_8frame_16sga_ms": sched, "exact_24_global_ms": 24 * g_ms,
            "speedup": 24 * g_ms / sched,
            "ideal_speedup_from_work": 24 * fg / (8 * ff + 16 * fs),
            "plan": [m for m, _ in vga.layer_schedule(24, 8, sga)] == [vga.MODE_FRAME] * 8
            + [vga.MODE_SGA] * 16}
    del q, k, v, out, out_b, ws
    torch.cuda.empty_cache()
    return rec


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="n100",
                    choices=["n100", "n300", "n800", "n800reg", "n800ramp", "shard8", "sweep",
                             "block"])
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="oracle rows per kind of layer (default 256; 128 for n800ramp, "
                         "whose 2x2 rows span 292,800 keys)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gpu-state", action="store_true",
                    help="skip the amd-smi power and clock samples (for runs under a profiler)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="n100 only: skip the 300- and 800-frame exact-vs-SGA records")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the multi-GPU sharding of this path is a "
              "design, not a build (see the design notes); use --gpus 1", file=sys.stderr)
        raise SystemExit(2)
    if args.copy_probe:
        copy_probe()
        return
    defaults = {"n100": (30, 20), "n300": (3, 1), "n800": (1, 1), "n800reg": (2, 1),
                "n800ramp": (1, 0), "shard8": (2, 1), "sweep": (2, 1),
                "block": (10, 5)}[args.workload]
    if args.cpu_rows is None:
        args.cpu_rows = 128 if args.workload == "n800ramp" else 256
    args.steps = args.steps if args.steps is not None else defaults[0]
    args.warmup = args.warmup if args.warmup is not None else defaults[1]
    res = run(args)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
