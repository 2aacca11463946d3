"""Benchmark of the packed variable-length attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

A step is one pass of the whole forward through the C ABI over one packed batch that is
already resident in HBM: for batches that pre-rotate keys (the default for long sequences) the
key-tile kernel (vlf_rotate_keys) and then the forward over the tiles (vlf_attend_rotated),
otherwise the one forward kernel (vlf_attend without a workspace). The default workload is
sixteen 8192-token sequences, 16 heads, bf16, full window. It prints one JSON line:

* value: effective attention TFLOP/s, counting 4 * 64 FLOPs per visible (query, key) pair per
  head, over the wall-clock of exactly K steps (synchronised on both sides);
* roofline: for the dominant kernel (the forward), the same algorithmic FLOPs over that
  kernel's average duration from HIP events recorded around it on its launch stream, against
  MI355X's dense bf16/fp16 matrix peak (2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096 FLOP/clock);
  traffic: HBM bytes per launch from rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each scaled
  by the reading of a plain copy of known size), recorded in profiles/ with the hash of the
  kernel source they were taken on (null when the source has changed since); step_traffic:
  the same for every kernel of the step (the key-tile pass and the forward), against the
  step's algorithmic bytes;
* cpu_baseline: the float64 oracle (test infrastructure) on the host cores over a bounded
  sample of rows of the same workload, in the same unit (mode B, the parity gate; mode A on a
  quarter of the rows beside it), and its wall seconds over every row of the other workloads;
* secondary: the other four workloads (tiny, encoder, sliding, many_short), each on its own
  schedule, against HBM (algorithmic bytes over the step's time, and that over 8 TB/s);
* roofline.measured_peak: the sustained rate and clock of the matrix probe (libvlf_probe.so),
  beside the 2516.6 TFLOP/s spec.

Beside wall-clock means, the line carries HIP-event means and medians per step and per kernel,
and the host time of the tile table.

Other modes:
  --profile-run        short run for rocprofv3 (no CPU baseline) plus one plain 1 GiB copy that
                       calibrates the byte counters;
  --summarize DIR      read a rocprofv3 counter-collection directory and print the traffic
                       summary for profiles/;
  --counters DIR ...   read rocprofv3 --pmc directories (any counters) and print, for one
                       kernel, each counter's average per dispatch with the derived matrix,
                       vector and LDS figures;
  --trace DIR          read a rocprofv3 --kernel-trace --stats directory and print the kernel
                       summary for profiles/ (per kernel: calls, total, average, min, max, and
                       the average over the last --steps dispatches, the timed ones);
  --mfma-peak          the matrix probe alone;
  --overlap            the overlap probe alone (matrix, vector and LDS work sharing a SIMD);
  --schedules          the phase-schedule probe (one product wave per SIMD) and the matrix
                       unit's toll on vector work.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0         # HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "variable_length_flash_amd", "csrc", "vlf_attend.hip")
KERNEL_NAMES = ("attend_pre_ph", "attend_pre", "attend_fwd", "attend_one", "attend_slide",
                "prep_tiles", "back_prep", "back_kv", "back_q")


COPY_BYTES = 1 << 30


def kernel_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_file(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if absent or taken on
    a different kernel source."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(workload: str):
    import torch
    from variable_length_flash_amd import workloads
    w = workloads.WORKLOADS[workload]()
    qkv = workloads.draw_qkv(w)
    cos, sin = workloads.rope_tables(w)
    return w, qkv, cos, sin


def cpu_baseline(w, qkv, cos, sin, target_s: float, pairs_per_head_total: int):
    """The oracle as it stands, on a bounded sample of rows of the workload (rows of the first
    sequences, all heads), scaled to effective TFLOP/s."""
    import numpy as np

    import oracle
    from variable_length_flash_amd import binding
    q32 = qkv.float().numpy()
    c32, s32 = cos.float().numpy(), sin.float().numpy()
    cores = oracle.threads(len(os.sched_getaffinity(0)))

    def visible(rows):
        # pairs the sampled rows compute, all heads
        total = 0
        cu = w.cu
        for t in rows:
            s = int(np.searchsorted(cu, t, side="right") - 1)
            L = int(cu[s + 1] - cu[s])
            i = int(t - cu[s])
            wv, causal = w.window & ~oracle.CAUSAL, w.window & oracle.CAUSAL
            lo = max(0, i - wv + 1) if wv else 0
            hi = i + 1 if causal else (min(L, i + wv) if wv else L)
            total += hi - lo
        return total * w.heads

    # calibrate on a few rows, then size the sample to the target time
    probe = np.arange(0, min(w.tokens, 32), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attend(q32, c32, s32, w.cu, w.heads, w.window, w.scale, mode="B", dtype=w.dtype,
                  rows=probe)
    dt = time.perf_counter() - t0
    n = int(min(w.tokens, max(64, len(probe) * target_s / max(dt, 1e-6))))
    rows = np.linspace(0, w.tokens - 1, n).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attend(q32, c32, s32, w.cu, w.heads, w.window, w.scale, mode="B", dtype=w.dtype,
                  rows=rows)
    dt = time.perf_counter() - t0
    # mode A (the unrounded definition) on a quarter of the same rows
    rows_a = rows[::4]
    t0 = time.perf_counter()
    oracle.attend(q32, c32, s32, w.cu, w.heads, w.window, w.scale, mode="A", dtype=w.dtype,
                  rows=rows_a)
    dt_a = time.perf_counter() - t0
    pairs = visible(rows)
    pairs_a = visible(rows_a)
    flops = 4 * 64 * pairs
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n} of {w.tokens} rows spread evenly over the workload, all {w.heads} heads "
                  f"({pairs} visible pairs, {flops / 1e9:.1f} GFLOP effective), oracle mode B "
                  f"(float64), {dt:.1f} s on {cores} threads",
        "wall_s": round(dt, 2),
        "cpu_model": cpu,
        "mode_a": {"value": 4 * 64 * pairs_a / dt_a / 1e12, "rows": len(rows_a),
                   "wall_s": round(dt_a, 2)},
    }


def algorithmic_bytes(w) -> int:
    """qkv read once, out and lse written once."""
    return (3 * w.tokens * w.heads * 64 * 2 + w.tokens * w.heads * 64 * 2
            + 4 * w.heads * w.tokens)


class Forward:
    """One workload's forward on the device, its inputs resident in HBM, as the binding
    schedules it (or a fixed tile height and path): a step is the key-tile kernel then the
    forward over the tiles (workspace path) or the one forward kernel (direct path)."""

    def __init__(self, w, qkv, cos, sin, dev, br=None, prerotate=None):
        import torch

        import variable_length_flash_amd as vlf
        self.vlf, self.w, self.dev = vlf, w, dev
        self.batch = vlf.prepare(w.cu, dev, br, prerotate, w.window)
        self.kernel = vlf.forward_kernel(self.batch.br, self.batch.prerotate, w.window,
                                         self.batch.max_len)
        self.q, self.c, self.s = qkv.to(dev), cos.to(dev), sin.to(dev)
        self.out = torch.empty((w.tokens, w.heads * 64), dtype=self.q.dtype, device=dev)
        self.lse = torch.empty((w.heads, w.tokens), dtype=torch.float32, device=dev)
        self.ws = vlf.new_workspace(self.batch, w.heads, dev)
        self.stream = torch.cuda.current_stream(dev)

    def step(self, ev=None):
        # ev: three events recorded before, between and after the step's kernels
        vlf, w, b = self.vlf, self.w, self.batch
        if ev is not None:
            ev[0].record(self.stream)
        if b.prerotate:
            vlf.rotate_keys(b, self.q, self.c, self.s, w.heads, self.ws)
            if ev is not None:
                ev[1].record(self.stream)
            vlf.attend_rotated_into(b, self.q, self.c, self.s, w.heads, w.window, w.scale,
                                    self.out, self.lse, self.ws)
        else:
            if ev is not None:
                ev[1].record(self.stream)
            vlf.attend_into(b, self.q, self.c, self.s, w.heads, w.window, w.scale, self.out,
                            self.lse)
        if ev is not None:
            ev[2].record(self.stream)

    def time(self, steps: int, warmup: int):
        """Wall-clock mean over exactly ``steps`` steps (synchronised on both sides), and the
        per-step HIP-event durations of the whole step, the forward kernel and the key-tile
        kernel (mean and median)."""
        import statistics

        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                  for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.step(events[k])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        whole = [e[0].elapsed_time(e[2]) for e in events]
        fwd = [e[1].elapsed_time(e[2]) for e in events]
        rot = [e[0].elapsed_time(e[1]) for e in events]
        return {"wall_ms": wall,
                "step_ms": statistics.mean(whole), "step_ms_median": statistics.median(whole),
                "kernel_ms": statistics.mean(fwd), "kernel_ms_median": statistics.median(fwd),
                "rotate_ms": statistics.mean(rot), "rotate_ms_median": statistics.median(rot)}


def tile_table_host_us(cu, br: int, prerotate: bool = False, window: int = 0,
                       reps: int = 50) -> float:
    """Median host time of building the launch's tile table through the library
    (vlf_tile_count, then vlf_launch_table), microseconds."""
    import statistics

    import variable_length_flash_amd as vlf
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        vlf.launch_table(cu, br, prerotate, window)
        times.append((time.perf_counter() - t0) * 1e6)
    return statistics.median(times)


SECONDARY = ("tiny", "encoder", "sliding", "many_short")


def secondary(args, dev):
    """The other workloads, each timed as the default line times long (its own schedule, HIP
    events on the launch stream), against HBM: algorithmic bytes over the forward's time."""
    import torch

    import variable_length_flash_amd as vlf
    res = {}
    for name in SECONDARY:
        w, qkv, cos, sin = make_inputs(name)
        f = Forward(w, qkv, cos, sin, dev)
        t = f.time(args.steps, args.warmup)
        pairs = vlf.visible_pairs(w.cu, w.window)
        flops = 4 * 64 * pairs * w.heads
        nbytes = algorithmic_bytes(w)
        gbs = nbytes / (t["step_ms"] / 1e3) / 1e9
        res[name] = {
            "workload": w.note, "dtype": w.dtype, "br": f.batch.br,
            "path": "prerotate" if f.batch.prerotate else "direct", "kernel": f.kernel,
            "ms_per_step": round(t["wall_ms"], 4), "step_ms_mean": round(t["step_ms"], 4),
            "step_ms_median": round(t["step_ms_median"], 4),
            "tflops": round(flops / (t["step_ms"] / 1e3) / 1e12, 2),
            "hbm_gbs_algorithmic": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
            # the forward kernel alone (HIP events around its launch), as the main line's
            # roofline takes it: the step's figures above include the key-tile pass if any and
            # the launch gaps
            "kernel_ms": round(t["kernel_ms"], 4),
            "kernel_frac_of_hbm": round(nbytes / (t["kernel_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes, "effective_flop": flops,
            "tile_table_host_us": round(tile_table_host_us(w.cu, f.batch.br, f.batch.prerotate,
                                                           w.window), 1),
        }
        del f
        torch.cuda.empty_cache()
    return res


def oracle_per_config(names):
    """Wall seconds of the oracle (mode B, the gate, and mode A) over every row of each named
    workload, on the host cores."""
    import oracle
    res = {}
    for name in names:
        w, qkv, cos, sin = make_inputs(name)
        q32 = qkv.float().numpy()
        c32, s32 = cos.float().numpy(), sin.float().numpy()
        row = {"rows": w.tokens}
        for mode in ("B", "A"):
            t0 = time.perf_counter()
            oracle.attend(q32, c32, s32, w.cu, w.heads, w.window, w.scale, mode=mode,
                          dtype=w.dtype)
            row[f"mode_{mode.lower()}_s"] = round(time.perf_counter() - t0, 2)
        res[name] = row
    return res


def run(args):
    import torch

    import variable_length_flash_amd as vlf

    if args.gpus != 1:
        print(f"bench.py measures one GPU; the library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    w, qkv, cos, sin = make_inputs(args.workload)
    if args.causal:  # the same batch under the causal window (keys i - W < j <= i)
        w.window |= vlf.CAUSAL
        w.note += ", causal"
    prerotate = None if args.path == "auto" else args.path == "prerotate"
    f = Forward(w, qkv, cos, sin, dev, args.br, prerotate)
    batch, kernel = f.batch, f.kernel
    path = "prerotate" if batch.prerotate else "direct"
    pairs = vlf.visible_pairs(w.cu, w.window)
    flops = 4 * 64 * pairs * w.heads
    alg_bytes = algorithmic_bytes(w)

    if args.backward:
        return run_backward(args, w, f.q, f.c, f.s, f.out, f.lse, f.stream)
    if args.unfused:
        return run_unfused(args, w, f.q, f.c, f.s, f.out, f.lse, f.stream, batch, f.ws)

    t = f.time(args.steps, args.warmup)
    wall_ms, kernel_ms, rotate_ms = t["wall_ms"], t["kernel_ms"], t["rotate_ms"]

    if args.profile_run:
        # a plain copy of known size on the same stream: the counter runs scale by it
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    value = flops / (wall_ms / 1e3) / 1e12
    # the committed counters are for the workloads' own windows
    traffic = None if args.causal else read_traffic(kernel, args.workload)
    # the key-tile kernel reads every key and value row once and writes each used block once
    key_tiles = sum(-(-int(L) // 64) for L in w.lens)
    rotate_bytes = (2 * w.tokens * w.heads * 64 * 2 + 2 * sum(w.lens) * 32 * 2
                    + key_tiles * w.heads * 16384)
    line = {
        "metric": "effective attention TFLOP/s (visible pairs) + % of bf16 MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {w.note}",
            "tokens": w.tokens, "sequences": w.sequences, "heads": w.heads, "head_dim": 64,
            "window": w.window, "rope_base": w.base, "scale": w.scale, "br": batch.br,
            "path": path,
            "step_ms_events": {"mean": round(t["step_ms"], 4),
                               "median": round(t["step_ms_median"], 4)},
            "kernel_ms": {kernel: round(kernel_ms, 4),
                          **({"prep_tiles": round(rotate_ms, 4)} if batch.prerotate else {})},
            "kernel_ms_median": {kernel: round(t["kernel_ms_median"], 4),
                                 **({"prep_tiles": round(t["rotate_ms_median"], 4)}
                                    if batch.prerotate else {})},
            **({"rotate_hbm_gbs_algorithmic": round(rotate_bytes / (rotate_ms / 1e3) / 1e9, 1)}
               if batch.prerotate else {}),
            "tile_table_host_us": round(tile_table_host_us(w.cu, batch.br, batch.prerotate,
                                                           w.window), 1),
            "visible_pairs_per_head": pairs, "effective_flop": flops,
            "pct_of_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "achieved_hbm_gbs_algorithmic": round(alg_bytes / (kernel_ms / 1e3) / 1e9, 1),
        },
        "roofline": roofline(kernel, flops, alg_bytes, kernel_ms, traffic),
        "cpu_baseline": None,
    }
    # the whole step's counted HBM bytes (the key-tile pass and the forward), beside the
    # dominant kernel's own in roofline.traffic
    step_kernels = ([("prep_tiles", rotate_ms)] if batch.prerotate else []) + [(kernel, kernel_ms)]
    counted = [read_traffic(k, args.workload) for k, _ in step_kernels]
    line["roofline"]["step_traffic"] = (
        {"bytes": round(sum(counted)), "kernels": [k for k, _ in step_kernels],
         "ratio_to_algorithmic": round(sum(counted) / alg_bytes, 3),
         "gbs": round(sum(counted) / (sum(ms for _, ms in step_kernels) / 1e3) / 1e9, 1)}
        if all(c is not None for c in counted) else None)
    del f
    torch.cuda.empty_cache()
    if not args.profile_run and not args.no_mfma_peak:
        from variable_length_flash_amd import probe
        peak = probe.mfma_peak(dev)
        line["roofline"]["measured_peak"] = peak
        if line["roofline"]["unit"] == "TFLOP/s":
            line["roofline"]["frac_of_measured_peak"] = round(
                line["roofline"]["achieved"] / peak["tflops"], 4)
    if not args.profile_run and not args.no_secondary and args.workload == "long" \
            and not args.causal and args.br is None and args.path == "auto":
        line["secondary"] = secondary(args, dev)
    if not args.profile_run and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, qkv, cos, sin, args.cpu_seconds, pairs)
        if "secondary" in line:
            line["cpu_baseline"]["per_config"] = oracle_per_config(SECONDARY)
    print(json.dumps(line), flush=True)


def run_mfma_peak(args):
    """``--mfma-peak``: the matrix probe alone, one JSON line."""
    import torch

    from variable_length_flash_amd import probe
    dev = torch.device("cuda:0")
    peak = probe.mfma_peak(dev)
    print(json.dumps({"metric": "sustained bf16 MFMA TFLOP/s (v_mfma_f32_32x32x16_bf16, two "
                                "waves per SIMD, independent accumulators)",
                      "value": peak["tflops"], "unit": "TFLOP/s", "spec": PEAK_BF16_TFLOPS,
                      "frac_of_spec": round(peak["tflops"] / PEAK_BF16_TFLOPS, 4), **peak}),
          flush=True)


def run_overlap(args):
    """``--overlap``: the overlap probe's loop time per role pair, one JSON line."""
    import torch

    from variable_length_flash_amd import probe
    rows = probe.overlap(torch.device("cuda:0"))
    print(json.dumps({"metric": "overlap probe: shader clocks per iteration of role pairs that "
                                "share a SIMD (one eight-wave workgroup per CU)",
                      "unit": "clocks", "pairs": rows}), flush=True)


def run_schedules(args):
    """``--schedules``: the phase-schedule and matrix-toll probes, one JSON line."""
    import torch

    from variable_length_flash_amd import probe
    res = probe.schedules(torch.device("cuda:0"))
    print(json.dumps({"metric": "schedule probe: shader clocks per 32-row wave step with one "
                                "product wave per SIMD, and the matrix unit's toll on vector work",
                      "unit": "clocks", **res}), flush=True)


def run_backward(args, w, q, c, s, out, lse, stream):
    """``--backward``: the library's forward once (out, lse), then K timed backward calls
    (include/vlf.h, vlf_attend_backward: delta, back_kv, back_q) on a seeded dout.
    Effective FLOP = 640 per visible pair and head: the five 64-deep products S, dP, dV, dK and
    dQ, against the forward's two."""
    import numpy as np
    import torch

    import variable_length_flash_amd as vlf
    dev = q.device
    vlf.attend_into(vlf.prepare(w.cu, dev, None, None, w.window), q, c, s, w.heads, w.window,
                    w.scale, out, lse)
    rng = np.random.default_rng(17)
    dout = torch.from_numpy(rng.standard_normal((w.tokens, w.heads * 64), dtype=np.float32)).to(
        dev, q.dtype)
    br = args.br or vlf.choose_backward(w.cu, w.heads, w.window)[0]
    batch = vlf.prepare(w.cu, dev, br, False, w.window)
    dqkv = torch.empty_like(q)
    ws = torch.empty(vlf.backward_workspace_bytes(w.tokens, w.sequences, w.heads, br),
                     dtype=torch.uint8, device=dev)

    def step():
        vlf.attend_backward_into(batch, q, c, s, w.heads, w.window, w.scale, out, lse, dout,
                                 dqkv, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        step()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    pairs = vlf.visible_pairs(w.cu, w.window)
    flops = 640 * pairs * w.heads
    # qkv, out and dout read once, dqkv written once, lse read once
    alg_bytes = (3 + 1 + 1 + 3) * w.tokens * w.heads * 64 * 2 + 4 * w.heads * w.tokens
    value = flops / (wall_ms / 1e3) / 1e12
    line = {
        "metric": "effective backward TFLOP/s (visible pairs, 5 products) + % of bf16 MFMA peak, "
                  "1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {w.note}", "tokens": w.tokens,
            "sequences": w.sequences, "heads": w.heads, "head_dim": 64, "window": w.window,
            "br": br, "path": "backward",
            "kernel_ms": {"backward (3 kernels)": round(kernel_ms, 4)},
            "visible_pairs_per_head": pairs, "effective_flop": flops,
            "pct_of_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        },
        "roofline": roofline("back_kv + back_q", flops, alg_bytes, kernel_ms, None),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_unfused(args, w, q, c, s, out, lse, stream, batch, ws):
    """``--unfused``: what fusing the rotation into the forward saves. Times, on the launch
    stream, the fused forward (the default schedule), the rotation pass alone (vlf_rotate_qkv)
    and the forward over its output with identity tables and scale 1 on the same schedule; both
    forwards multiply the same rounded operands."""
    import torch

    import variable_length_flash_amd as vlf
    dst = torch.empty_like(q)
    one, zero = torch.ones_like(c), torch.zeros_like(s)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    fused = timed(lambda: vlf.attend_into(batch, q, c, s, w.heads, w.window, w.scale, out, lse,
                                          workspace=ws))
    rot = timed(lambda: vlf.rotate_qkv_into(batch, q, c, s, w.heads, w.scale, dst))
    plain = timed(lambda: vlf.attend_into(batch, dst, one, zero, w.heads, w.window, 1.0, out,
                                          lse, workspace=ws))
    line = {
        "metric": "fused forward time against rotation pass + forward (unfused baseline)",
        "value": round(fused, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}: {w.note}", "br": batch.br,
                   "path": "prerotate" if batch.prerotate else "direct"},
        "fused_ms": round(fused, 4), "rotation_pass_ms": round(rot, 4),
        "forward_on_rotated_ms": round(plain, 4), "unfused_ms": round(rot + plain, 4),
        "fusion_saving_pct": round(100 * (rot + plain - fused) / (rot + plain), 2),
    }
    print(json.dumps(line), flush=True)


def roofline(kernel: str, flops: float, alg_bytes: int, kernel_ms: float, traffic):
    """The forward kernel against its bound: the matrix unit when the workload's arithmetic
    intensity (effective FLOP per algorithmic byte) is above the ridge of the bf16 peak and HBM,
    else HBM, with algorithmic bytes per launch over the kernel's average duration."""
    seconds = kernel_ms / 1e3
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    common = {"kernel": kernel, "traffic": traffic, "kernel_ms": round(kernel_ms, 4),
              "algorithmic_bytes": alg_bytes, "algorithmic_flop": flops,
              "intensity_flop_per_byte": round(flops / alg_bytes, 1)}
    if flops / alg_bytes >= ridge:
        achieved = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), **common}
    achieved = alg_bytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), **common}


def summarize(directories, workload: str, kernel: str):
    """Traffic per launch from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE), each
    scaled by the same counter's reading for the 1 GiB copy of the profile run."""
    rows = []
    for directory in directories:
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                              recursive=True):
            with open(path) as f:
                rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directories}")
    per = {}  # (counter, kind) -> list of per-dispatch values (KiB)
    for r in rows:
        name = r.get("Kernel_Name", "")
        kind = "attend" if f"::{kernel}<" in name else ("copy" if "copybuffer" in name.lower()
                                                        else None)
        if kind is None:
            continue
        per.setdefault((r["Counter_Name"], kind, r.get("Dispatch_Id", "")), 0.0)
        per[(r["Counter_Name"], kind, r.get("Dispatch_Id", ""))] += float(r["Counter_Value"])
    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        att = [v for (c, k, _), v in per.items() if c == counter and k == "attend"]
        cpy = [v for (c, k, _), v in per.items() if c == counter and k == "copy"]
        if not att or not cpy:
            raise SystemExit(f"{counter}: attend {len(att)} dispatches, copy {len(cpy)}")
        # the copy reads and writes COPY_BYTES each; its reading (KiB) calibrates the counter
        copy_kib = max(cpy)
        factor = COPY_BYTES / (copy_kib * 1024.0)
        res[counter] = (sum(att) / len(att), copy_kib, factor)
    fetch = res["FETCH_SIZE"][0] * 1024 * res["FETCH_SIZE"][2]
    write = res["WRITE_SIZE"][0] * 1024 * res["WRITE_SIZE"][2]
    print(f"kernel: {kernel}")
    print(f"workload: {workload}")
    print(f"kernel_source_sha256_16: {kernel_hash()}")
    for counter, (att, cpy, factor) in res.items():
        print(f"{counter}_kib_per_dispatch: {att:.1f}")
        print(f"{counter}_copy_kib_for_{COPY_BYTES}_bytes: {cpy:.1f}")
        print(f"{counter}_scale_factor: {factor:.4f}")
    print(f"hbm_fetch_bytes_per_launch: {fetch:.0f}")
    print(f"hbm_write_bytes_per_launch: {write:.0f}")
    print(f"hbm_bytes_per_launch: {fetch + write:.0f}")


def _short_kernel_name(name: str) -> str:
    """'void ns::(anonymous namespace)::back_kv<ns::(anonymous namespace)::BF16, 4, 2, false>(...)'
    -> 'back_kv<BF16, 4, 2, false>'."""
    import re
    name = re.sub(r"^void ", "", name)
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # drop the argument list: the first '(' outside <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not name.startswith("(anonymous", i):
            cut = i
            break
    name = name[:cut]
    return re.sub(r"[A-Za-z_0-9]+::\(anonymous namespace\)::", "", name)


def trace_summary(directories, timed: int):
    """Per-kernel summary of rocprofv3 --kernel-trace --stats directories: the stats table and
    each kernel's average over its last ``timed`` dispatches (the timed steps)."""
    stats, per = [], {}
    for directory in directories:
        for path in glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True):
            with open(path) as f:
                stats.extend(csv.DictReader(f))
        for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    per.setdefault(_short_kernel_name(r["Kernel_Name"]), []).append(
                        (int(r["Dispatch_Id"]),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {directories}")
    print(f"kernel_source_sha256_16: {kernel_hash()}")
    print("kernel | calls | total_ms | average_us | min_us | max_us | percent")
    for r in stats:
        print(f"{_short_kernel_name(r['Name'])} | {r['Calls']} | "
              f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.2f}")
    print(f"# average over the last {timed} dispatches of each kernel (the timed steps)")
    for name, rows in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        rows.sort()
        last = [d for _, d in rows[-timed:]]
        print(f"{name} | timed_average_us {sum(last) / len(last):.2f} | over {len(last)}")


def _kernel_rows(directories, kernel: str):
    """Per-dispatch sums of every counter of ``kernel`` in rocprofv3 --pmc directories."""
    import re
    pattern = re.compile(r"::" + re.escape(kernel) + r"<")
    per = {}
    for directory in directories:
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                              recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if not pattern.search(r.get("Kernel_Name", "")):
                        continue
                    key = (path, r.get("Dispatch_Id", ""))
                    d = per.setdefault(key, {})
                    d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(
                        r["Counter_Value"])
    return list(per.values())


def counters(directories, workload: str, kernel: str):
    """Averages per dispatch of every counter taken for ``kernel``, over all passes, and the
    figures derived from them. GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's active
    cycles are a eighth of it; the SQ counters are totals over the chip (the *_CYCLES ones of
    the matrix unit in clocks, SQ_ACTIVE_INST_VALU and SQ_WAVE_CYCLES in quad-cycles)."""
    rows = _kernel_rows(directories, kernel)
    if not rows:
        raise SystemExit(f"no dispatch of {kernel} under {directories}")
    names = sorted({n for r in rows for n in r})
    avg = {}
    for n in names:
        vals = [r[n] for r in rows if n in r]
        avg[n] = sum(vals) / len(vals)
    cus, simds = 256, 1024
    print(f"kernel: {kernel}")
    print(f"workload: {workload}")
    print(f"kernel_source_sha256_16: {kernel_hash()}")
    print(f"dispatches: {len(rows)}")
    for n in names:
        print(f"{n}_per_dispatch: {avg[n]:.6e}")
    grbm = avg.get("GRBM_GUI_ACTIVE")
    if not grbm:
        return
    xcd_cycles = grbm / 8
    simd_cycles = xcd_cycles * simds
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        derived.append(("mfma_busy_pct_of_simd_cycles",
                        100 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles))
    if "SQ_INSTS_MFMA" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        derived.append(("mfma_busy_cycles_per_mfma",
                        avg["SQ_VALU_MFMA_BUSY_CYCLES"] / avg["SQ_INSTS_MFMA"]))
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        derived.append(("valu_coexec_pct_of_mfma_busy",
                        100 * avg["SQ_VALU_MFMA_COEXEC_CYCLES"] /
                        avg["SQ_VALU_MFMA_BUSY_CYCLES"]))
    if "SQ_ACTIVE_INST_VALU" in avg:
        derived.append(("VALUBusy_pct (100 SQ_ACTIVE_INST_VALU / CUs / XCD cycles)",
                        100 * avg["SQ_ACTIVE_INST_VALU"] / cus / xcd_cycles))
    if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg:
        derived.append(("non_mfma_valu_insts_per_mfma",
                        (avg["SQ_INSTS_VALU"] - avg["SQ_INSTS_MFMA"]) / avg["SQ_INSTS_MFMA"]))
    if "SQ_INSTS_VALU_TRANS_F32" in avg and "SQ_INSTS_MFMA" in avg:
        derived.append(("trans_f32_insts_per_mfma",
                        avg["SQ_INSTS_VALU_TRANS_F32"] / avg["SQ_INSTS_MFMA"]))
    if "SQ_LDS_BANK_CONFLICT" in avg:
        derived.append(("LDSBankConflict_pct (100 SQ_LDS_BANK_CONFLICT / CUs / XCD cycles)",
                        100 * avg["SQ_LDS_BANK_CONFLICT"] / cus / xcd_cycles))
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            derived.append(("lds_bank_conflict_pct_of_lds_active",
                            100 * avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]))
    if "SQ_WAVE_CYCLES" in avg:
        derived.append(("waves_resident_per_cu", 4 * avg["SQ_WAVE_CYCLES"] / cus / xcd_cycles))
        for n in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY"):
            if n in avg:
                derived.append((f"{n}_pct_of_wave_cycles", 100 * avg[n] / avg["SQ_WAVE_CYCLES"]))
    if "SQ_INST_LEVEL_VMEM" in avg and avg.get("SQ_INSTS_VMEM_RD"):
        derived.append(("vmem_instructions_in_flight_per_cu",
                        avg["SQ_INST_LEVEL_VMEM"] / cus / xcd_cycles))
    for name, v in derived:
        print(f"{name}: {v:.3f}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long",
                    choices=["tiny", "encoder", "sliding", "many_short", "long"])
    ap.add_argument("--br", type=int, default=None, choices=[64, 128, 256],
                    help="query rows per workgroup (default: chosen from the longest sequence)")
    ap.add_argument("--path", default="auto", choices=["auto", "direct", "prerotate"],
                    help="direct: every workgroup rotates its key tiles; prerotate: key-tile "
                         "workspace (default: chosen from the longest sequence)")
    ap.add_argument("--kernel", default="attend_pre_ph", choices=KERNEL_NAMES,
                    help="kernel whose counters --summarize and --counters read")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other four workloads in the default line")
    ap.add_argument("--no-mfma-peak", action="store_true",
                    help="skip the matrix probe in the default line")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="run only the matrix probe (sustained bf16 MFMA rate and clock)")
    ap.add_argument("--overlap", action="store_true",
                    help="run only the overlap probe (matrix, vector and LDS work on one SIMD)")
    ap.add_argument("--schedules", action="store_true",
                    help="run only the phase-schedule and matrix-toll probes")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (vlf_attend_backward) instead of the forward")
    ap.add_argument("--causal", action="store_true",
                    help="run the workload under the causal window (window | CAUSAL)")
    ap.add_argument("--unfused", action="store_true",
                    help="time the fused forward against the rotation pass plus the forward")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--summarize", metavar="DIR", nargs="+")
    ap.add_argument("--counters", metavar="DIR", nargs="+")
    ap.add_argument("--trace", metavar="DIR", nargs="+",
                    help="summarize rocprofv3 --kernel-trace --stats output (last --steps "
                         "dispatches of each kernel are the timed ones)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload, args.kernel)
        return
    if args.counters:
        counters(args.counters, args.workload, args.kernel)
        return
    if args.trace:
        trace_summary(args.trace, args.steps)
        return
    if args.mfma_peak:
        run_mfma_peak(args)
        return
    if args.schedules:
        run_schedules(args)
        return
    if args.overlap:
        run_overlap(args)
        return
    run(args)


if __name__ == "__main__":
    main()
