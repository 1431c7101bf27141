#!/usr/bin/env python3
"""Throughput of one MoE layer forward on one MI355X.

A step is one pass of the whole hot path over one batch: route (top-k
gating), send counts, permute, grouped SwiGLU experts (routed, then the
shared expert), unpermute + gate-weighted combine.  Inputs and weights are
resident in HBM before the timed region.  The default workload is the
DeepSeek-V3-shaped prefill layer: T = 8192 tokens, d = 7168, 256 routed
experts (ffn 2048) + 1 shared, group-limited sigmoid routing (8 groups of 32,
top-4 groups, top-8), send counts for a simulated 64-way EP group.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "MoE-layer fwd tokens/s at DSV3 shape, 1 GPU; % MFMA peak; permute % HBM BW"
PEAK_MFMA = {"bf16": 2.5e15, "f32": 157.3e12}     # dense, MI355X published
PEAK_HBM = 8.0e12


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def stage_bytes(cfg, gather=False):
    """Algorithmic HBM bytes of the permute and combine stages (per layer).
    With gather the permute computes indices only (ids in, order and inv out)."""
    s = cfg.elem_bytes
    T, k, d = cfg.T, cfg.k, cfg.d
    permute = T * 12 * k if gather else T * (d * s + k * d * s + 12 * k)   # x once, k copies
    combine = T * (k * d * s + d * s + 8 * k + (d * s if cfg.shared else 0))
    return permute, combine


def expert_flops(cfg):
    """Algorithmic FLOPs: routed gate/up product, routed down product, shared expert."""
    M = cfg.T * cfg.k
    gate_up = 4 * M * cfg.d * cfg.ffn
    down = 2 * M * cfg.d * cfg.ffn
    shared = 6 * cfg.T * cfg.d * cfg.ffn if cfg.shared else 0
    return gate_up, down, shared


def gate_up_bytes(cfg, counts, gather=False):
    """Algorithmic HBM bytes of the routed gate/up launch: the gate and up
    weights of every expert that has rows, each packed row once (with gather
    read from x through order), h written."""
    s = cfg.elem_bytes
    touched = int((counts > 0).sum())
    M = cfg.T * cfg.k
    return (touched * 2 * cfg.ffn * cfg.d * s + M * cfg.d * s + M * cfg.ffn * s
            + (4 * M if gather else 0))


def packed_permute_rate(layer, cfg, nbytes, reps=10):
    """Mean duration of moe_permute with the row copy, HIP events around each
    call on the launch stream, and its algorithmic HBM rate."""
    import torch

    from token_routing_expert_amd import moe_permute
    x_perm = torch.empty((cfg.T * cfg.k, cfg.d), dtype=layer.x.dtype, device=layer.x.device)
    bufs = [torch.empty_like(layer.counts), torch.empty_like(layer.offsets),
            torch.empty_like(layer.order), torch.empty_like(layer.inv)]
    stream = torch.cuda.current_stream()

    def run():
        moe_permute(layer.x, layer.topk_ids, cfg.E, *bufs, x_perm, layer.workspace)

    for _ in range(3):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for i in range(reps):
        ev[2 * i].record(stream)
        run()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) / reps
    del x_perm
    return {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(nbytes / ms / 1e6, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / PEAK_HBM, 4)}


def forward_tile_rows(cfg, M, cus=256):
    """Rows per tile of the forward products (the library's tile choice): 32
    for few rows per expert or a problem that the larger tiles would spread
    over fewer tiles than compute units, else 320 up to 320 rows per expert
    and 256 beyond."""
    per_expert = -(-M // cfg.E) if cfg.E else 0
    if per_expert < 96 or cfg.d % 256:
        return 32
    bm = 320 if per_expert <= 320 else 256
    tiles = cfg.E * -(-per_expert // bm) * (cfg.d // 256)
    return 32 if tiles < cus else bm


def combine_rate(layer, cfg, nbytes, reps=10):
    """Mean duration of the combine launch alone (HIP events around each call
    on the launch stream, after the step's buffers exist) and its algorithmic
    HBM rate.  The in-step stage time also holds the gap between launches."""
    import torch
    from token_routing_expert_amd import moe_unpermute_combine
    y = torch.empty_like(layer.y)
    stream = torch.cuda.current_stream()

    def run():
        moe_unpermute_combine(layer.y_perm, layer.inv, layer.topk_w, layer.y_sh, y,
                              rows=layer.rows if layer.cap is not None else None)

    for _ in range(3):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for i in range(reps):
        ev[2 * i].record(stream)
        run()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) / reps
    return {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(nbytes / ms / 1e6, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / PEAK_HBM, 4)}


def load_accounting(cfg, counts, send_counts):
    """Load and padding statistics of the batch: rows per expert, the rows the
    GEMM tiles compute beyond the real ones (tile padding), and the imbalance
    of the simulated EP ranks (most-loaded receiving rank over the mean, from
    the send-count matrix's column sums)."""
    import numpy as np
    counts = np.asarray(counts, np.int64)
    M = int(counts.sum())
    bm = forward_tile_rows(cfg, M)
    tiled = int((-(-counts // bm) * bm).sum())
    blocks = int((-(-counts // 32) * 32).sum())   # MFMAs run on 32-row blocks with a live row
    out = {"rows": M, "rows_per_expert_min": int(counts.min()), "rows_per_expert_max": int(counts.max()),
           "empty_experts": int((counts == 0).sum()), "tile_rows": bm,
           "tile_padding_frac": round((tiled - M) / max(M, 1), 4),
           "mfma_padding_frac": round((blocks - M) / max(M, 1), 4), "dropped_rows": 0}
    if send_counts is not None:
        recv = np.asarray(send_counts, np.int64).sum(axis=0)
        out["ep_recv_imbalance"] = round(float(recv.max() / max(recv.mean(), 1e-9)), 4)
    return out


def time_steps(layer, stages, stream, reps, warmup=2):
    """Median step time (HIP events around each step on the launch stream)
    and mean per-stage times of `reps` steps of layer, after `warmup`."""
    import torch
    for _ in range(warmup):
        for name in stages:
            getattr(layer, name)()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record(stream)
        for j, name in enumerate(stages):
            getattr(layer, name)()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    steps = sorted(e[0].elapsed_time(e[-1]) for e in evs)
    stage_ms = {name: round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) / reps, 4)
                for j, name in enumerate(stages)}
    return steps[len(steps) // 2], stage_ms


def alternatives(cfg, layer, stages, stream, grouped_ms, grouped_load, reps=10, loop_reps=3):
    """The two other ways to run the expert products ("Expert parallelism",
    "Token permutation and grouped GEMMs"), timed on the same batch and
    weights as the grouped step: padded to capacity and batched at CF = 1 and
    1.25 (dropped and padding rows from the batch's counts), and a loop of one
    product pair per expert (its step includes the copy of the segment sizes
    to the host that the loop needs)."""
    import numpy as np
    import torch

    from token_routing_expert_amd.layer import MoeLayer, to_host
    given = cfg.gating == "given"
    common = dict(logits=layer.logits, sh_w13=getattr(layer, "sh_w13", None),
                  sh_w2=getattr(layer, "sh_w2", None),
                  topk_ids=layer.topk_ids if given else None, topk_w=layer.topk_w if given else None)
    M = cfg.T * cfg.k
    out = {"grouped": {"ms_per_step": round(grouped_ms, 4), "dropped_frac": 0.0,
                       "tile_padding_frac": grouped_load["tile_padding_frac"],
                       "mfma_padding_frac": grouped_load["mfma_padding_frac"]}}
    for cf in (1.0, 1.25):
        alt = MoeLayer(cfg, layer.x, layer.w13, layer.w2, fused_gather=True, capacity_factor=cf,
                       **common)
        ms, st = time_steps(alt, stages, stream, reps)
        counts = to_host(alt.counts).astype(np.int64)
        cap = alt.cap
        kept = np.minimum(counts, cap)
        out[f"capacity_cf{cf:g}"] = {
            "cap": cap, "ms_per_step": round(ms, 4), "tokens_per_s": cfg.T / (ms * 1e-3),
            "dropped_frac": round(float((counts - kept).sum()) / M, 4),
            "padding_slots_frac": round(float(cfg.E * cap - kept.sum()) / (cfg.E * cap), 4),
            "computed_rows_over_needed": round(cfg.E * cap / M, 4),
            "gate_up_ms": st["gate_up"], "down_ms": st["down"]}
        del alt
        torch.cuda.empty_cache()
    alt = MoeLayer(cfg, layer.x, layer.w13, layer.w2, fused_gather=False, expert_loop=True, **common)
    ms, st = time_steps(alt, stages, stream, loop_reps, warmup=1)
    out["expert_loop"] = {"ms_per_step": round(ms, 4), "tokens_per_s": cfg.T / (ms * 1e-3),
                          "experts_ms": round(st["gate_up"] + st["down"], 4),
                          "launches": 2 * int((to_host(alt.counts) > 0).sum())}
    del alt
    torch.cuda.empty_cache()
    return out


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "token_routing_expert_amd",
                           "csrc", "grouped_gemm.hip")
WGRAD_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "token_routing_expert_amd",
                            "csrc", "grouped_wgrad.hip")


# The routed gate/up launch at the DeepSeek-V3 prefill shape (320-row tiles,
# SwiGLU epilogue); other workloads' gate/up launches are found by family.
GATE_UP_KERNELS = ("k_grouped_gemm_pp<true, 320, 256, 4, 5, 4, 2, true, true, false, 0>",
                   "k_grouped_gemm_pp<true, 256, 256, 2, 3, 8, 1, true, true, false, 0>",
                   "k_grouped_gemm<true, 32, 128, 1, 4, true, 2, 4, false>",
                   "k_grouped_gemm<false, 32, 128, 1, 4, true, 2, 2, false>")


def _source_sha(path=GEMM_SOURCE):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _rocprof_rows(directory, suffix):
    """Rows (dicts) of every rocprofv3 CSV file under directory whose name
    ends with suffix."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def copy_calibration(fetch_dir, write_dir):
    """KiB of HBM traffic per KiB of FETCH_SIZE and of WRITE_SIZE, from the
    plain 1 GiB device copy of the counter runs (--copy-calibration 1024):
    the largest dispatch of the runtime's copy kernel (smaller device copies
    of the same kernel and grid, such as a clone of the layer output, are
    not it).  (None, None) when there is no such dispatch."""
    def largest(directory, counter):
        best = 0.0
        for r in _rocprof_rows(directory, "counter_collection.csv") if directory else []:
            if r.get("Counter_Name") == counter and r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer"):
                best = max(best, float(r["Counter_Value"]))
        return best
    f, w = largest(fetch_dir, "FETCH_SIZE"), largest(write_dir, "WRITE_SIZE")
    if f < 1e5 or w < 1e5:
        return None, None
    return 1024 * 1024 / f, 1024 * 1024 / w   # 1 GiB in KiB


def summarize_profile(workload, trace_dir, fetch_dir, write_dir, bench_line, warmup, commands, out_dir):
    """Summarise rocprofv3 runs of bench.py for one workload into
    out_dir/<workload>_kernels.md and out_dir/<workload>_gate_up_traffic.json.

    Durations per kernel come from the kernel trace (end - start of each
    dispatch), both over all dispatches and over the timed ones (each
    kernel's first `warmup` dispatches dropped, and only the bench line's
    `steps` after them kept: later ones -- cold-cache steps, graph replays --
    are not in the bench line's launch time); HBM bytes from one-counter
    passes FETCH_SIZE and WRITE_SIZE, scaled by what the counters read for
    the plain 1 GiB device copy of the same runs (--copy-calibration)."""
    from collections import defaultdict
    trace = _rocprof_rows(trace_dir, "kernel_trace.csv")
    if not trace:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    steps = None
    if bench_line and os.path.exists(bench_line):
        with open(bench_line) as f:
            found = [json.loads(l) for l in f if l.startswith("{")]
        steps = found[-1]["steps"] if found else None
    durs = defaultdict(list)
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        gx = r.get("Grid_Size_X")
        gsize = (int(gx) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)) if gx \
            else int(r.get("Grid_Size") or 0)
        key = (r["Kernel_Name"], gsize)
        durs[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counters(directory, counter):
        vals = defaultdict(list)
        for r in _rocprof_rows(directory, "counter_collection.csv") if directory else []:
            if r.get("Counter_Name") != counter:
                continue
            vals[(r["Kernel_Name"], int(r.get("Grid_Size") or 0))].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}

    fetch, write = counters(fetch_dir, "FETCH_SIZE"), counters(write_dir, "WRITE_SIZE")
    fs, ws = copy_calibration(fetch_dir, write_dir)
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Commands (the profiled bench runs, then this summary):", "", "```", *commands, "```", ""]
    if fs:
        lines += [f"Calibration: the plain 1 GiB device copy reads FETCH_SIZE = {1024 * 1024 / fs:.0f} KiB "
                  f"and WRITE_SIZE = {1024 * 1024 / ws:.0f} KiB, so HBM bytes = FETCH_SIZE x {fs:.3f} KiB "
                  f"+ WRITE_SIZE x {ws:.3f} KiB.", ""]
    lines += [f"Durations from the kernel trace; 'timed' drops each kernel's first {warmup} dispatches "
              "(the bench's warm-up steps), so it covers the launches the bench line times.", "",
              "| kernel | grid (threads) | dispatches | avg us (all) | avg us (timed) | FETCH KiB | WRITE KiB "
              "| HBM GB (scaled) | GB/s (timed) |", "|---|---|---|---|---|---|---|---|---|"]
    gate_up = None
    for key in sorted(durs, key=lambda k: -sum(durs[k])):
        d = durs[key]
        timed = d[warmup:] if len(d) > warmup else d
        if steps:
            timed = timed[:steps]
        avg_all, avg_t = sum(d) / len(d), sum(timed) / len(timed)
        fk, wk = fetch.get(key), write.get(key)
        gb = ((fk or 0) * fs + (wk or 0) * ws) * 1024 / 1e9 if fs and (fk or wk) else None
        name = key[0].replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {name} | {key[1]} | {len(d)} | {avg_all:.1f} | {avg_t:.1f} | "
                     f"{'' if fk is None else f'{fk:.0f}'} | {'' if wk is None else f'{wk:.0f}'} | "
                     f"{'' if gb is None else f'{gb:.3f}'} | {'' if gb is None else f'{gb / avg_t * 1e6:.0f}'} |")
        if any(k in key[0] for k in GATE_UP_KERNELS) and (gate_up is None or avg_t * len(d) > gate_up[4]):
            gate_up = (key, avg_t, len(timed), gb, avg_t * len(d))
    lines.append("")
    rec = None
    if gate_up:
        key, avg_t, n, gb, _ = gate_up
        short = key[0].replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
        lines += [f"Routed gate/up launch (`{short}`): {avg_t:.1f} us mean over its {n} timed "
                  f"dispatches" + (f"; {gb:.3f} GB of HBM traffic per launch." if gb else "."), ""]
        rec = {"workload": workload, "kernel": key[0], "grid_threads": key[1],
               "avg_us_timed": round(avg_t, 1), "timed_dispatches": n,
               "fetch_kib": fetch.get(key), "write_kib": write.get(key), "fetch_scale": fs,
               "write_scale": ws, "bytes_per_launch": int(gb * 1e9) if gb else None,
               "source": os.path.relpath(GEMM_SOURCE, os.path.dirname(PROFILES)),
               "source_sha256": _source_sha()}
    if bench_line and os.path.exists(bench_line):
        with open(bench_line) as f:
            found = [l for l in f if l.startswith("{")]
        if found:
            r = json.loads(found[-1])
            lines += ["bench.py line of the traced run (stage times from HIP events on the launch stream):",
                      "", "```", json.dumps(r.get("stages")), json.dumps(r.get("roofline")), "```", ""]
            if rec:
                rec["bench_launch_ms_events"] = r["roofline"].get("launch_ms")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{workload}_kernels.md"), "w") as f:
        f.write("\n".join(lines))
    if rec:
        with open(os.path.join(out_dir, f"{workload}_gate_up_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
    print("\n".join(lines))


# The weight-gradient launches of one training step, in the order the
# backward runs them (MoeLayer.BACKWARD_STAGES): the routed down and gate/up
# products', then the shared expert's, then the router product's.
TRAIN_WGRAD_LAUNCHES = ("routed dW_down", "routed dW13", "shared dW_down", "shared dW13", "router dW_r")


def summarize_train_profile(workload, trace_dir, fetch_dir, write_dir, bench_line, warmup, commands,
                            out_dir):
    """Summarise rocprofv3 runs of `bench.py --train` into
    out_dir/<workload>_train_kernels.md and <workload>_train_wgrad_traffic.json.
    Kernels are listed as summarize_profile lists them.  The weight-gradient
    kernel runs several times per step on one grid size, so its dispatches
    are told apart by their position within the step (TRAIN_WGRAD_LAUNCHES),
    in the trace and in the counter passes alike; the record is the routed
    dW13 launch's."""
    from collections import defaultdict
    trace = sorted(_rocprof_rows(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    if not trace:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    steps = None
    if bench_line and os.path.exists(bench_line):
        with open(bench_line) as f:
            found = [json.loads(l) for l in f if l.startswith("{")]
        line = found[-1] if found else None
        steps = line["steps"] if line else None
    else:
        line = None
    durs = defaultdict(list)
    for r in trace:
        durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def by_position(values, runs):
        """Split one kernel's per-dispatch values into per-launch-position lists."""
        per = len(values) // runs if runs else 0
        if not per or per * runs != len(values):
            raise SystemExit(f"{len(values)} weight-gradient dispatches do not split into {runs} steps")
        out = defaultdict(list)
        for i, v in enumerate(values):
            out[i % per].append(v)
        return out, per

    wg_name = next((k for k in durs if "k_weight_grad" in k), None)
    if wg_name is None or steps is None:
        raise SystemExit("no weight-gradient kernel in the trace, or no bench line")
    pos_durs, per = by_position(durs[wg_name], warmup + steps)

    def counter_positions(directory, counter):
        rows = sorted((r for r in _rocprof_rows(directory, "counter_collection.csv")
                       if r.get("Counter_Name") == counter),
                      key=lambda r: int(r.get("Dispatch_Id") or 0))
        copy = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        vals = [float(r["Counter_Value"]) for r in rows if "k_weight_grad" in r["Kernel_Name"]]
        runs = len(vals) // per if per else 0
        pos, _ = by_position(vals, runs)
        return {k: sum(v) / len(v) for k, v in pos.items()}, (max(copy) if copy else None)

    fetch, fcopy = counter_positions(fetch_dir, "FETCH_SIZE")
    write, wcopy = counter_positions(write_dir, "WRITE_SIZE")
    fs = 1024 * 1024 / fcopy if fcopy else None
    ws = 1024 * 1024 / wcopy if wcopy else None
    lines = [f"# rocprofv3 summary: {workload} training step (forward keeping pre-activations + backward)",
             "", "Commands (the profiled bench runs, then this summary):", "", "```", *commands, "```", ""]
    if fs and ws:
        lines += [f"Calibration: the plain 1 GiB device copy reads FETCH_SIZE = {fcopy:.0f} KiB and "
                  f"WRITE_SIZE = {wcopy:.0f} KiB, so HBM bytes = FETCH_SIZE x {fs:.3f} KiB + WRITE_SIZE "
                  f"x {ws:.3f} KiB.", ""]
    lines += [f"Kernel durations from the trace ({warmup} warm-up + {steps} timed steps traced); "
              "'timed' drops the warm-up steps' dispatches.", "",
              "| kernel | dispatches | avg us (timed) | total us per step |", "|---|---|---|---|"]
    runs = warmup + steps
    for name in sorted(durs, key=lambda k: -sum(durs[k])):
        d = durs[name]
        n_timed = len(d) * steps // runs
        timed = d[len(d) - n_timed:] if n_timed else d
        short = name.replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {short} | {len(d)} | {sum(timed) / len(timed):.1f} | {sum(timed) / steps:.1f} |")
    lines += ["", f"The weight-gradient kernel, by launch position within a step ({per} per step):", "",
              "| launch | avg us (timed) | FETCH KiB | WRITE KiB | HBM GB (scaled) |", "|---|---|---|---|---|"]
    rec = None
    for i in range(per):
        d = pos_durs[i]
        t = d[warmup:] if len(d) > warmup else d
        avg = sum(t) / len(t)
        fk, wk = fetch.get(i), write.get(i)
        gb = (fk * fs + wk * ws) * 1024 / 1e9 if fs and ws and fk is not None and wk is not None else None
        label = TRAIN_WGRAD_LAUNCHES[i] if i < len(TRAIN_WGRAD_LAUNCHES) else f"launch {i}"
        lines.append(f"| {label} | {avg:.1f} | {'' if fk is None else f'{fk:.0f}'} | "
                     f"{'' if wk is None else f'{wk:.0f}'} | {'' if gb is None else f'{gb:.3f}'} |")
        if i == 1:
            rec = {"workload": workload, "kernel": wg_name, "launch": label, "avg_us_timed": round(avg, 1),
                   "timed_dispatches": len(t), "fetch_kib": fk, "write_kib": wk, "fetch_scale": fs,
                   "write_scale": ws, "bytes_per_launch": int(gb * 1e9) if gb else None,
                   "source": os.path.relpath(WGRAD_SOURCE, os.path.dirname(PROFILES)),
                   "source_sha256": _source_sha(WGRAD_SOURCE)}
    lines.append("")
    if line:
        lines += ["bench.py line of the traced run (stage times from HIP events):", "", "```",
                  json.dumps(line.get("stages")), json.dumps(line.get("roofline")), "```", ""]
        if rec:
            rec["bench_launch_ms_events"] = line["roofline"].get("launch_ms")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{workload}_train_kernels.md"), "w") as f:
        f.write("\n".join(lines))
    if rec:
        with open(os.path.join(out_dir, f"{workload}_train_wgrad_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
    print("\n".join(lines))


ACTIVITY_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS",
                     "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES")


def summarize_activity(workload, pmc_dir, commands, out_dir, xcds=8, simds=1024):
    """profiles/<workload>_activity.md from one rocprofv3 --pmc pass with
    ACTIVITY_COUNTERS: per kernel, the mean dispatch duration and counter
    values, the shader clock (GRBM_GUI_ACTIVE / XCDs / duration) and the
    matrix cores' busy fraction (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs /
    (GRBM_GUI_ACTIVE / XCDs)); the derived two only for dispatches longer
    than 100 us, shorter than the counters' sampling window."""
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    for r in _rocprof_rows(pmc_dir, "counter_collection.csv"):
        name = r["Kernel_Name"].replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
        vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        durs[name][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    lines = [f"# rocprofv3 activity counters: {workload}", "",
             "One counter pass over a short bench run (means per dispatch):", "", "```", *commands, "```", "",
             "Derived: shader clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration; matrix-core busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8). Both only for dispatches "
             "longer than 100 us (for shorter ones the counters' window exceeds the dispatch).", "",
             "| kernel | dispatches | duration us | GRBM_GUI_ACTIVE | SQ_VALU_MFMA_BUSY_CYCLES | SQ_INSTS_LDS "
             "| SQ_LDS_BANK_CONFLICT | clock GHz | MFMA busy |", "|---|---|---|---|---|---|---|---|---|"]
    def mean(x):
        return sum(x) / len(x) if x else 0.0
    for name in sorted(durs, key=lambda k: -sum(durs[k].values())):
        v = vals[name]
        dur = mean(list(durs[name].values()))
        gui, mfma = mean(v["GRBM_GUI_ACTIVE"]), mean(v["SQ_VALU_MFMA_BUSY_CYCLES"])
        clock = busy = "–"
        if dur > 100 and gui > 0:
            clock = f"{gui / xcds / (dur * 1e3):.2f}"
            busy = f"{100 * mfma / simds / (gui / xcds):.1f}%"
        lines.append(f"| {name} | {len(durs[name])} | {dur:.1f} | {gui:.4g} | {mfma:.4g} | "
                     f"{mean(v['SQ_INSTS_LDS']):.4g} | {mean(v['SQ_LDS_BANK_CONFLICT']):.4g} | {clock} | {busy} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{workload}_activity.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_trace(workload):
    """The routed gate/up launch's mean duration (us) over the timed
    dispatches of the committed kernel trace of this workload, or None when
    there is none or it was taken on another kernel source."""
    try:
        with open(os.path.join(PROFILES, f"{workload}_gate_up_traffic.json")) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("workload") != workload or t.get("source_sha256") != _source_sha():
        return None
    return t.get("avg_us_timed")


def measured_traffic(workload, path="gather"):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter passes
    of this workload (taken on the default fused-gather path), or None when
    there are none, they were taken on another kernel source, or the run
    uses the packed path."""
    import hashlib
    if path != "gather":
        return None
    try:
        with open(os.path.join(PROFILES, f"{workload}_gate_up_traffic.json")) as f:
            t = json.load(f)
        with open(GEMM_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if t.get("workload") != workload or t.get("source_sha256") != sha or not t.get("bytes_per_launch"):
        return None
    return int(t["bytes_per_launch"])


def host_info():
    """The host the oracle runs on: CPU model, sockets, physical cores and
    hardware threads (from /proc/cpuinfo), and the threads this process may use."""
    model, sockets, cores = None, set(), set()
    try:
        phys = core = None
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                    sockets.add(val)
                elif key == "core id":
                    core = val
                    cores.add((phys, core))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "sockets": len(sockets) or None, "physical_cores": len(cores) or None,
            "hardware_threads": os.cpu_count(), "threads_usable_here": usable}


def oracle_small_layer_single_thread():
    """The oracle's whole forward (route, send counts, permute with the row
    copy, experts, combine) on the small fp32 layer (1,024 tokens, 8 experts,
    top-2, d 256, ffn 512), on one thread: seconds and tokens/s."""
    import oracle
    from token_routing_expert_amd import inputs
    cfg = inputs.CONFIGS["small_fp32"]
    logits, x = inputs.gen_logits(cfg), inputs.gen_x(cfg)
    w13, w2 = inputs.gen_expert_weights(cfg)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        ids, w = oracle.route(logits, cfg.k, cfg.gating, cfg.renormalize)
        oracle.send_counts(ids, cfg.E, cfg.n_ep)
        _, offsets, order, inv = oracle.permute_index(ids, cfg.E)
        rows = oracle.gather_rows(x, order, cfg.k)
        e_of = np.repeat(np.arange(cfg.E, dtype=np.int32), np.diff(offsets))
        y_perm = oracle.expert_swiglu_rows(rows, e_of, w13, w2)
        oracle.combine(y_perm, inv, w)
        sec = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    return {"workload": "small_fp32", "threads": 1, "seconds": round(sec, 4),
            "tokens_per_s": round(cfg.T / sec, 1)}


def cpu_baseline(cfg, data, budget_s=15.0, max_tokens=2048):
    """The oracle, untuned, on the host cores: route, send counts and permute on
    every token, then experts and combine on seeded tokens until about budget_s
    has passed; per-token costs extrapolated to the full batch."""
    import numpy as np

    import oracle
    from token_routing_expert_amd import inputs

    x, w13, w2, logits, sh, ids_in, w_in = data
    t0 = time.perf_counter()
    if cfg.gating == "given":
        ids, w = ids_in, w_in
    else:
        ids, w = oracle.route(logits, cfg.k, cfg.gating, cfg.renormalize, cfg.n_groups,
                              cfg.topk_groups)
    if cfg.n_ep:
        oracle.send_counts(ids, cfg.E, cfg.n_ep)
    _, _, order, _ = oracle.permute_index(ids, cfg.E)
    oracle.gather_rows(x, order, cfg.k)
    t_index = time.perf_counter() - t0
    sample = inputs.sample_tokens(cfg, max_tokens)
    done, t_exp = 0, 0.0
    while done < len(sample) and t_exp < budget_s:
        batch = sample[done:done + 16]
        t1 = time.perf_counter()
        oracle.layer_tokens(x, ids, w, w13, w2, batch, *sh)
        t_exp += time.perf_counter() - t1
        done += len(batch)
    per_token = t_index / cfg.T + t_exp / done
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "host": host_info(),
        "small_layer_single_thread": oracle_small_layer_single_thread(),
        "kind": "oracle",
        "sample": (f"route, send counts, permute and row gather on all {cfg.T} tokens "
                   f"({t_index:.2f} s) + experts and combine on {done} seeded tokens "
                   f"({t_exp:.2f} s); per-token costs extrapolated to {cfg.T} tokens"),
    }


TRAIN_TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                  "dsv3_prefill_train_wgrad_traffic.json")


def measured_train_traffic(workload):
    """HBM bytes per launch of the first product's weight gradient (dW13) from
    the committed counter passes of a training step, or None when they were
    taken on another workload or another kernel source."""
    import hashlib
    try:
        with open(TRAIN_TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(WGRAD_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if t.get("workload") != workload or t.get("source_sha256") != sha:
        return None
    return int(t["bytes_per_launch"])


TRAIN_METRIC = ("MoE-layer fwd+bwd tokens/s at DSV3 shape, 1 GPU (training step: forward keeping "
                "pre-activations, backward to dx, dW and dlogits)")


def cpu_baseline_train(cfg, data, dy, budget_s=20.0):
    """The oracle's forward and backward, untuned, on the host cores: the
    per-token part (expert outputs, the combine's and the experts' input
    gradients, the gate gradients) on seeded tokens, and the weight gradients
    on rows of one expert; per-token costs extrapolated to the full batch."""
    import numpy as np

    import oracle
    from token_routing_expert_amd import inputs

    x, w13, w2, logits, sh, ids_in, w_in = data
    t0 = time.perf_counter()
    if cfg.gating == "given":
        ids, w = ids_in, w_in
    else:
        ids, w = oracle.route(logits, cfg.k, cfg.gating, cfg.renormalize, cfg.n_groups,
                              cfg.topk_groups)
    _, offsets, order, _ = oracle.permute_index(ids, cfg.E)
    t_index = time.perf_counter() - t0
    k, d = cfg.k, cfg.d
    sample = inputs.sample_tokens(cfg, 256)
    done, t_tok = 0, 0.0
    while done < len(sample) and t_tok < budget_s / 2:
        t = sample[done:done + 4]
        t1 = time.perf_counter()
        rows = np.repeat(np.ascontiguousarray(x[t]), k, axis=0)
        e = ids[t].reshape(-1)
        y_rows = oracle.expert_swiglu_rows(rows, e, w13, w2)
        ident = np.arange(len(t) * k, dtype=np.int32)
        dy_rows, dgate = oracle.combine_backward(dy[t], ident, w[t], y_rows)
        oracle.expert_swiglu_backward_rows(rows, e, w13, w2, dy_rows, want_dw=False)
        if logits is not None:
            oracle.gate_backward(logits[t], ids[t], dgate, cfg.gating, cfg.renormalize)
        t_tok += time.perf_counter() - t1
        done += len(t)
    # Weight gradients: rows of the first non-empty expert, that expert alone.
    e0 = int(np.flatnonzero(np.diff(offsets))[0])
    seg = order[offsets[e0]:offsets[e0 + 1]][:64]
    rows = np.ascontiguousarray(x[seg // k])
    dy_rows = oracle.bf16_bits_to_f64(dy[seg // k]) if dy.dtype == np.uint16 else dy[seg // k]
    t1 = time.perf_counter()
    oracle.expert_swiglu_backward_rows(rows, np.zeros(len(seg), np.int32), w13[e0:e0 + 1],
                                       w2[e0:e0 + 1], dy_rows, want_dx=False)
    t_w = time.perf_counter() - t1
    per_token = t_index / cfg.T + t_tok / done + k * t_w / len(seg)
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"route and permute on all {cfg.T} tokens ({t_index:.2f} s); forward, combine, "
                   f"input and gate gradients on {done} seeded tokens ({t_tok:.2f} s); weight "
                   f"gradients of expert {e0} over {len(seg)} of its rows ({t_w:.2f} s); per-token "
                   f"costs extrapolated to {cfg.T} tokens (shared expert not included)"),
    }


def run_train(args, cfg, layer, data, stream):
    """--train: time forward + backward steps; one JSON line."""
    import numpy as np
    import torch

    from token_routing_expert_amd import inputs
    from token_routing_expert_amd.layer import to_device, to_host

    dy_host = inputs.f32_to_bf16_bits(
        np.random.default_rng(2000 + cfg.index).standard_normal((cfg.T, cfg.d)).astype(np.float32))
    dy = to_device(dy_host)
    fwd = ["route", "permute", "gate_up", "down", "experts_shared", "combine"]
    stages = [("fwd", n) for n in fwd] + [("bwd", n) for n in layer.BACKWARD_STAGES]

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        for i, (kind, name) in enumerate(stages):
            if kind == "fwd":
                getattr(layer, name)()
            else:
                getattr(layer, name)(dy)
            if evs is not None:
                evs[i + 1].record(stream)

    log(f"train warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    log(f"timing {K} training steps")
    t_start = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / K
    stage_ms = {name: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
                for j, (_, name) in enumerate(stages)}
    M = cfg.T * cfg.k
    d, ffn, s = cfg.d, cfg.ffn, cfg.elem_bytes
    f_gu, f_dn, _ = expert_flops(cfg)
    flops = {"gate_up": f_gu, "down": f_dn, "bwd_down": f_dn, "bwd_gate_up": f_gu,
             "bwd_wgrad_down": f_dn, "bwd_wgrad_gate_up": f_gu}
    peak = PEAK_MFMA[cfg.dtype]
    stage_info = {}
    for _, name in stages:
        info = {"ms": round(stage_ms[name], 4)}
        if name in flops:
            rate = flops[name] / (stage_ms[name] * 1e-3)
            info.update(flops=flops[name], TFLOPs=round(rate / 1e12, 1),
                        mfma_frac=round(rate / peak, 4))
        stage_info[name] = info
    # Dominant backward kernel: the first product's weight gradient (one
    # launch, 4 M d ffn FLOPs): dgu and the rows read once, every expert's
    # dW13 written once.
    gather = layer.x_perm is None
    wg_ms = stage_ms["bwd_wgrad_gate_up"]
    wg_bytes = (M * 2 * ffn * s + (cfg.T * d * s + 4 * M if gather else M * d * s)
                + cfg.E * 2 * ffn * d * s)
    intensity = f_gu / wg_bytes
    ridge = peak / PEAK_HBM
    flop_rate, byte_rate = f_gu / (wg_ms * 1e-3), wg_bytes / (wg_ms * 1e-3)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": round(byte_rate / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(byte_rate / PEAK_HBM, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(flop_rate / 1e12, 2), "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": round(flop_rate / peak, 4)}
    fwd_ms = sum(stage_ms[n] for n in fwd)
    bwd_ms = sum(stage_ms[n] for n in layer.BACKWARD_STAGES)
    result = {
        "metric": TRAIN_METRIC,
        "value": cfg.T / (ms_step * 1e-3),
        "unit": "tokens/s" if cfg.gating != "given" else "rows/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded numpy draws; random-init weights of the stated shapes)",
        "config": {"workload": cfg.name, "T": cfg.T, "E": cfg.E, "k": cfg.k, "d": d, "ffn": ffn,
                   "gating": cfg.gating, "shared_experts": int(cfg.shared), "path": args.path,
                   "train": True},
        "roofline": {"kernel": "moe_grouped_weight_grad: dW13 = dgu^T x rows (one launch)", **roof,
                     "traffic": measured_train_traffic(cfg.name), "algorithmic_bytes": wg_bytes, "algorithmic_flops": f_gu,
                     "intensity_flop_per_byte": round(intensity, 1),
                     "ridge_flop_per_byte": round(ridge, 1),
                     "mfma_frac": round(flop_rate / peak, 4),
                     "hbm_frac": round(byte_rate / PEAK_HBM, 4), "launch_ms": round(wg_ms, 4)},
        "forward_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
        "backward_TFLOPs": round(2 * (f_gu + f_dn + (6 * cfg.T * d * ffn if cfg.shared else 0))
                                 / (bwd_ms * 1e-3) / 1e12, 1),
        "stages": stage_info,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle forward + backward)")
        result["cpu_baseline"] = cpu_baseline_train(cfg, data, dy_host)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--router", action="store_true",
                    help="put the router product (x . w_router^T) and the auxiliary-loss-free "
                         "bias (selection on logits + bias, bias update after each step, rate "
                         "--bias-lr) in the step; the default step takes the logits as input")
    ap.add_argument("--bias-lr", type=float, default=1e-3)
    ap.add_argument("--path", choices=("gather", "packed"), default="gather",
                    help="gather: the first expert product reads token rows through the "
                         "permutation; packed: the permute writes the packed copy X[order] "
                         "(with --train the packed rows are kept either way, for the weight "
                         "gradient)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step instead: the forward keeping the pre-activations, "
                         "then the backward to dx, the weight gradients and dlogits (bf16 only)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="after the timed steps, time this many more from cold caches")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a HIP graph")
    ap.add_argument("--no-alternatives", action="store_true",
                    help="skip timing the capacity-padded (CF 1, 1.25) and per-expert-loop forms")
    ap.add_argument("--summarize-profile", metavar="WORKLOAD",
                    help="write profiles/WORKLOAD_kernels.md and WORKLOAD_gate_up_traffic.json from "
                         "rocprofv3 output (--trace-dir, --fetch-dir, --write-dir, --bench-line); "
                         "runs no GPU work")
    ap.add_argument("--summarize-activity", metavar="WORKLOAD",
                    help="write profiles/WORKLOAD_activity.md from a rocprofv3 --pmc pass of the "
                         "activity counters (--pmc-dir); runs no GPU work")
    ap.add_argument("--pmc-dir")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--bench-line")
    ap.add_argument("--command", action="append", default=[],
                    help="a command line that produced the profile (repeatable; recorded verbatim)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.summarize_activity:
        summarize_activity(args.summarize_activity, args.pmc_dir, args.command, PROFILES)
        return
    if args.summarize_profile:
        summarize = summarize_train_profile if args.train else summarize_profile
        summarize(args.summarize_profile, args.trace_dir, args.fetch_dir, args.write_dir,
                  args.bench_line, args.warmup, args.command, PROFILES)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path is one GPU's share of the EP layer and "
              "libmoe355 has no cross-GPU exchange. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from token_routing_expert_amd import inputs, load_library
    from token_routing_expert_amd.layer import MoeLayer

    load_library()
    cfg = inputs.CONFIGS[args.workload]
    log(f"workload {cfg.name}: generating inputs")
    t0 = time.perf_counter()
    x = inputs.gen_x(cfg)
    w13, w2 = inputs.gen_expert_weights(cfg, verbose=True)
    sh = inputs.gen_expert_weights(cfg, shared=True) if cfg.shared else (None, None)
    if cfg.gating == "given":
        logits = None
        ids_in, w_in = inputs.gen_ep_share_routing(cfg)
    else:
        logits = inputs.gen_logits(cfg)
        ids_in = w_in = None
    log(f"generated in {time.perf_counter() - t0:.1f} s; uploading")
    router = args.router and cfg.gating != "given"
    wr_kw = {}
    if router:
        wr_kw = dict(w_router=inputs.gen_router_weights(cfg),
                     bias=np.zeros(cfg.E, np.float32), bias_lr=args.bias_lr)
    layer = MoeLayer(cfg, x, w13, w2, logits=logits, sh_w13=sh[0], sh_w2=sh[1], **wr_kw,
                     topk_ids=ids_in, topk_w=w_in, fused_gather=args.path == "gather",
                     train=args.train)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        # A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE counter
        # readings calibrate the counters of the path's kernels.
        n = args.copy_calibration << 20
        src = torch.ones(n // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    if args.train:
        run_train(args, cfg, layer, (x, w13, w2, logits, sh, ids_in, w_in), stream)
        return

    stages = ["route", "permute", "gate_up", "down", "experts_shared", "combine"]
    if router:
        stages = ["router"] + stages + ["bias_update"]

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        for i, name in enumerate(stages):
            getattr(layer, name)()
            if evs is not None:
                evs[i + 1].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / K
    stage_ms = {name: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
                for j, name in enumerate(stages)}
    step_ev = sorted(evs[i][0].elapsed_time(evs[i][-1]) for i in range(K))

    def pct(q):
        return round(step_ev[min(K - 1, int(q * (K - 1) + 0.5))], 4)

    # The same step from cold caches: a 1 GiB fill before each step (outside
    # its events) evicts the L2s and the 256 MB MALL, so nothing the step
    # reads is left over from the previous one.
    n_cold = min(args.cold_steps, K)
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if n_cold else None
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(n_cold)]
    for i in range(n_cold):
        scrub.fill_(float(i))
        step(cold[i])
    torch.cuda.synchronize()
    del scrub
    cold_step = sorted(c[0].elapsed_time(c[-1]) for c in cold)
    cold_info = None
    if n_cold:
        cold_info = {"steps": n_cold, "step_ms_p50": round(cold_step[n_cold // 2], 4),
                     "tokens_per_s_p50": round(cfg.T / (cold_step[n_cold // 2] * 1e-3), 1),
                     "step_ms_p10": round(cold_step[int(0.1 * (n_cold - 1) + 0.5)], 4),
                     "step_ms_p90": round(cold_step[int(0.9 * (n_cold - 1) + 0.5)], 4),
                     "stages_ms": {name: round(sum(c[j].elapsed_time(c[j + 1]) for c in cold) / n_cold, 4)
                                   for j, name in enumerate(stages)}}

    # The same step replayed from a HIP graph of its launches: what the eager
    # step spends on launch overhead (the layer allocates nothing and sets no
    # memory with memset, so it captures as is).  The replayed step's output
    # is checked against the eager one's bits.
    graph_info = None
    if not args.no_graph:
        y_eager = layer.y.clone()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(layer.y, y_eager)) if not router else None
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ge[0].record(stream)
        for _ in range(K):
            g.replay()
        ge[1].record(stream)
        torch.cuda.synchronize()
        gms = ge[0].elapsed_time(ge[1]) / K
        graph_info = {"steps": K, "step_ms": round(gms, 4), "tokens_per_s": round(cfg.T / (gms * 1e-3), 1),
                      "output_equals_eager": same}
        del g

    from token_routing_expert_amd.layer import to_host
    counts = to_host(layer.counts)
    f_gate_up, f_down, f_shared = expert_flops(cfg)
    peak = PEAK_MFMA[cfg.dtype]
    gather = args.path == "gather"
    b_perm, b_comb = stage_bytes(cfg, gather)
    b_gate_up = gate_up_bytes(cfg, counts, gather)
    # Route: logits read once, ids and gates written; the send counts read
    # the ids again and write the n_ep x n_ep matrix.
    b_route = None
    if cfg.gating != "given":
        b_route = cfg.T * (cfg.E * 4 + cfg.k * 8)
        if cfg.n_ep:
            b_route += cfg.T * cfg.k * 4 + cfg.n_ep * cfg.n_ep * 4
    if layer.merge_shared:
        # The shared expert runs as one more group of the routed launches.
        f_gate_up += 2 * f_shared // 3
        f_down += f_shared // 3
        f_shared = 0
        s_el = cfg.elem_bytes
        b_gate_up += 2 * cfg.ffn * cfg.d * s_el + cfg.T * (cfg.d + cfg.ffn) * s_el + 4 * cfg.T
    stage_info = {}
    for name in stages:
        ms = stage_ms[name]
        info = {"ms": round(ms, 4)}
        nbytes = {"permute": b_perm, "combine": b_comb, "gate_up": b_gate_up,
                  "route": b_route}.get(name)
        flops = {"gate_up": f_gate_up, "down": f_down, "experts_shared": f_shared}.get(name)
        if flops:
            rate = flops / (ms * 1e-3)
            info.update(flops=flops, TFLOPs=round(rate / 1e12, 1), mfma_frac=round(rate / peak, 4))
        if nbytes:
            info.update(bytes=nbytes, GBps=round(nbytes / ms / 1e6, 1),
                        hbm_frac=round(nbytes / (ms * 1e-3) / PEAK_HBM, 4))
        stage_info[name] = info

    # Dominant kernel: the routed gate/up launch (about 2/3 of the FLOPs).  Its
    # bound is the roofline's: HBM when its arithmetic intensity (algorithmic
    # FLOPs per algorithmic byte) lies below the ridge peak FLOP/s / peak B/s.
    gu_ms = stage_ms["gate_up"]
    flop_rate = f_gate_up / (gu_ms * 1e-3)
    byte_rate = b_gate_up / (gu_ms * 1e-3)
    intensity = f_gate_up / b_gate_up
    ridge = peak / PEAK_HBM
    hbm_bound = intensity < ridge
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(byte_rate / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(byte_rate / PEAK_HBM, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(flop_rate / 1e12, 2), "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": round(flop_rate / peak, 4)}
    result = {
        "metric": METRIC,
        "value": cfg.T / (ms_step * 1e-3),
        "unit": "tokens/s" if cfg.gating != "given" else "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded numpy draws; random-init weights of the stated shapes)",
        "config": {
            "workload": cfg.name, "T": cfg.T, "E": cfg.E, "k": cfg.k, "d": cfg.d, "ffn": cfg.ffn,
            "gating": cfg.gating, "n_groups": cfg.n_groups, "topk_groups": cfg.topk_groups,
            "shared_experts": int(cfg.shared), "n_ep_simulated": cfg.n_ep, "path": args.path,
            "shared_in_routed_launches": bool(layer.merge_shared),
            "router": bool(router), "bias_lr": args.bias_lr if router else None,
        },
        "roofline": {
            "kernel": ("moe_grouped_gate_up_gather" if gather else "moe_grouped_gate_up")
                      + ": routed gate/up products + SwiGLU (one launch)",
            **roof,
            "traffic": measured_traffic(cfg.name, args.path),
            "algorithmic_bytes": b_gate_up,
            "algorithmic_flops": f_gate_up,
            "intensity_flop_per_byte": round(intensity, 1),
            "ridge_flop_per_byte": round(ridge, 1),
            "mfma_frac": round(flop_rate / peak, 4),
            "hbm_frac": round(byte_rate / PEAK_HBM, 4),
            "launch_ms": round(gu_ms, 4),
            "trace_launch_ms": (lambda us: None if us is None else round(us / 1e3, 4))(
                measured_trace(cfg.name) if gather else None),
        },
        "stages": stage_info,
        "step_ms_events": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
        "headline": ("value: the K timed steps back to back (wall clock around them; a step may "
                     "find the previous step's data in the L2s and the 256 MB MALL); "
                     "cold_cache.tokens_per_s_p50: the median of steps each run after a 1 GiB fill "
                     "that evicts both (HIP events, the fill outside them); graph_replay: the same "
                     "step's launches captured once in a HIP graph and replayed K times"),
        "cold_cache": cold_info,
        "graph_replay": graph_info,
        "load": load_accounting(cfg, counts,
                                to_host(layer.send_counts) if cfg.n_ep else None),
        "device": torch.cuda.get_device_name(0),
    }
    tl = result["roofline"]["trace_launch_ms"]
    if tl:
        # The same fraction from the committed kernel trace's mean duration of
        # the timed launches (a profile taken on the same kernel source).
        result["roofline"]["trace_frac"] = round(
            (b_gate_up if hbm_bound else f_gate_up) / (tl * 1e-3) / (PEAK_HBM if hbm_bound else peak), 4)
    if gather:
        # The timed path never copies rows; the row-copying permute (the
        # stable scatter into the packed buffer X[order]) is measured here
        # on the same batch, outside the timed step, for its HBM figure.
        result["permute_packed"] = packed_permute_rate(layer, cfg, stage_bytes(cfg)[0])
    result["combine_alone"] = combine_rate(layer, cfg, b_comb)
    if not args.no_alternatives and not router:
        log("alternatives: capacity CF 1 and 1.25, one product pair per expert")
        result["alternatives"] = alternatives(cfg, layer, stages, stream, step_ev[K // 2],
                                              result["load"])
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(cfg, (x, w13, w2, logits, sh, ids_in, w_in))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
