"""Host-side logic of bench.py (no GPU): the one-GPU rule of its command line,
and the algorithmic work its roofline figures divide by, pinned to values
derived independently from the layer's shapes.

FLOPs per routed assignment are 6 d ffn (two products of the gate/up
projection and one down projection, 2 FLOPs per multiply-add): "Expert
parallelism", section "A worked example at DeepSeek-V3's shape".  The byte
counts follow the same page's section "Token permutation and grouped GEMMs":
the row copy reads each token row once and writes its k copies, the combine
reads the k expert rows (and the shared expert's row) and writes one row.
"""
import dataclasses
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from token_routing_expert_amd import inputs  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_deepseek_prefill_work():
    cfg = inputs.CONFIGS["dsv3_prefill"]
    T, k, d, ffn = 8192, 8, 7168, 2048
    assert (cfg.T, cfg.k, cfg.d, cfg.ffn, cfg.E) == (T, k, d, ffn, 256)
    gate_up, down, shared = bench.expert_flops(cfg)
    # 6 d ffn = 88,080,384 FLOPs per assignment, two thirds in the first product
    assert 6 * d * ffn == 88_080_384
    assert gate_up + down == T * k * 88_080_384
    assert gate_up == 2 * down
    assert shared == T * 88_080_384
    # bf16 rows of 14,336 bytes
    perm, comb = bench.stage_bytes(cfg)
    assert perm == T * (14_336 * (1 + k) + 12 * k) == 1_057_751_040
    assert comb == T * (14_336 * (k + 2) + 8 * k) == 1_174_929_408
    perm_idx, _ = bench.stage_bytes(cfg, gather=True)
    assert perm_idx == T * k * 12
    # every expert touched: 256 gate/up matrices of 2 ffn x d, rows once, h once
    counts = np.full(256, T * k // 256)
    assert bench.gate_up_bytes(cfg, counts) == (256 * 2 * ffn * d * 2 + T * k * (d + ffn) * 2)
    assert bench.gate_up_bytes(cfg, counts, gather=True) == 16_240_607_232
    # experts without rows bring no weights (the rows are the batch's T k either way)
    counts[:6] = 0
    assert (bench.gate_up_bytes(cfg, np.full(256, 1)) - bench.gate_up_bytes(cfg, counts)
            == 6 * 2 * ffn * d * 2)


def test_load_accounting_by_hand():
    cfg = dataclasses.replace(inputs.CONFIGS["dsv3_prefill"], E=4)
    counts = np.array([300, 0, 10, 290])
    acc = bench.load_accounting(cfg, counts, np.array([[1, 2], [3, 4]]))
    # 600 rows, 150 per expert on average: the 320-row tiles would give only
    # 4 x 28 down tiles for 256 compute units, so the forward uses 32-row
    # tiles, which are also the MFMA blocks
    assert acc["rows"] == 600 and acc["tile_rows"] == 32
    assert acc["rows_per_expert_min"] == 0 and acc["rows_per_expert_max"] == 300
    assert acc["empty_experts"] == 1 and acc["dropped_rows"] == 0
    assert acc["tile_padding_frac"] == pytest.approx((320 + 32 + 320 - 600) / 600)
    assert acc["mfma_padding_frac"] == pytest.approx((320 + 32 + 320 - 600) / 600)
    # receiving ranks get column sums 4 and 6: 6 / mean 5
    assert acc["ep_recv_imbalance"] == pytest.approx(1.2)


def test_forward_tile_rows_at_the_workloads():
    """The tile rows the library picks at the five workloads: the prefill
    layer's ~256 rows per expert fit one 320-row tile; Mixtral and the EP64
    share have 256-row tiles; decode's few rows per expert and the small fp32
    layer (8 down tiles with 320 rows) take 32-row tiles."""
    want = {"small_fp32": 32, "mixtral_bf16": 256, "dsv3_decode": 32, "dsv3_prefill": 320,
            "ep64_share": 256}
    for name, bm in want.items():
        cfg = inputs.CONFIGS[name]
        assert bench.forward_tile_rows(cfg, cfg.T * cfg.k) == bm, name


def test_measured_traffic_is_per_workload_and_path():
    assert bench.measured_traffic("dsv3_prefill", "packed") is None
    assert bench.measured_traffic("no_such_workload") is None
    for w in inputs.CONFIG_ORDER:
        path = os.path.join(ROOT, "profiles", f"{w}_gate_up_traffic.json")
        got = bench.measured_traffic(w)
        if not os.path.exists(path):
            assert got is None
            continue
        with open(path) as f:
            rec = json.load(f)
        assert rec["workload"] == w
        # None only once the kernel source has changed since the counters
        assert got is None or got == rec["bytes_per_launch"]
