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


def load_accounting(cfg, counts, send_counts):
    """Load and padding statistics of the batch: rows per expert, the rows the
    GEMM tiles compute beyond the real ones (tile padding), and the imbalance
    of the simulated EP ranks (most-loaded receiving rank over the mean, from
    the send-count matrix's column sums)."""
    import numpy as np
    counts = np.asarray(counts, np.int64)
    M = int(counts.sum())
    per_expert = -(-M // cfg.E) if cfg.E else 0
    bm = 32 if per_expert < 96 or cfg.d % 256 else (320 if per_expert <= 288 else 256)
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


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "token_routing_expert_amd",
                           "csrc", "grouped_gemm.hip")


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
    if t.get("workload") != workload or t.get("source_sha256") != sha:
        return None
    return int(t["bytes_per_launch"])


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
        with open(GEMM_SOURCE, "rb") as f:
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
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="after the timed steps, time this many more from cold caches")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
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
                     "stages_ms": {name: round(sum(c[j].elapsed_time(c[j + 1]) for c in cold) / n_cold, 4)
                                   for j, name in enumerate(stages)}}

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
        },
        "stages": stage_info,
        "step_ms_events": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
        "cold_cache": cold_info,
        "load": load_accounting(cfg, counts,
                                to_host(layer.send_counts) if cfg.n_ep else None),
        "device": torch.cuda.get_device_name(0),
    }
    if gather:
        # The timed path never copies rows; the row-copying permute (the
        # stable scatter into the packed buffer X[order]) is measured here
        # on the same batch, outside the timed step, for its HBM figure.
        result["permute_packed"] = packed_permute_rate(layer, cfg, stage_bytes(cfg)[0])
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(cfg, (x, w13, w2, logits, sh, ids_in, w_in))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
