"""Host logic of bench.py (CPU only): the byte / FLOP accounting behind the roofline
object, the HBM-traffic reduction of rocprofv3 counter files, the kernel labels and
the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from workloads import FULL_CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_stage_bytes_bf16_and_mxfp8():
    """The Qwen3-shaped layer gathers its token rows (metadata-only permutation); the
    gate/up GEMM's bytes count one input row per routed assignment, and the gathered
    figure the T token rows; a layer whose rows are only 2 K-steps wide keeps the
    permuted copy (the library's plan says which)."""
    from routing_dispatch_expert_logits_amd import binding as B
    cfg = FULL_CONFIGS["qwen3_30b_a3b_shaped"]
    T, H, E, k, I, D, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.D, cfg.R
    counts = np.full(E, R // E)
    assert bench.layer_plan(B, cfg)["rows_gathered"] == 1
    st, touched = bench.stage_bytes_flops(cfg, counts, True)
    assert touched == E
    assert st["permute"] == (12 * R, 0)
    assert st["gemm_gate_up"] == (E * 2 * D * I * 2 + R * D * 2 + R * I * 2, 4 * R * D * I)
    assert st["gemm_gate_up_gathered"] == (E * 2 * D * I * 2 + T * D * 2 + R * I * 2, 4 * R * D * I)
    assert st["gemm_down"][1] == 2 * R * D * I
    mx = cfg.with_(dispatch="mxfp8")
    st8, _ = bench.stage_bytes_flops(mx, counts, True)
    q = D * 33 // 32                       # one code byte per element + one scale byte per 32
    assert st8["permute"] == (T * D * 2 + T * q + 12 * R, 0)
    assert st8["gemm_gate_up"] == (E * 2 * q * I + R * q + R * I * 2, 4 * R * D * I)
    assert st8["gemm_down"] == st["gemm_down"] and st8["combine"] == st["combine"]
    narrow = cfg.with_(H=128)
    assert bench.layer_plan(B, narrow)["rows_gathered"] == 0
    stn, _ = bench.stage_bytes_flops(narrow, counts, False)
    assert stn["permute"] == (T * 128 * 2 + R * 128 * 2 + 12 * R, 0)
    assert bench.layer_plan(B, FULL_CONFIGS["k3_shaped_decode"])["rows_gathered"] == 1  # decode tiles
    assert bench.layer_plan(B, FULL_CONFIGS["tiny_f32"])["rows_gathered"] == 0


def test_stage_bytes_follow_kept_rows():
    """With an expert capacity the rows kept (sum of counts) drive the accounting."""
    cfg = FULL_CONFIGS["qwen3_30b_a3b_shaped"]
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[:10] = 100                      # 1000 kept rows on 10 experts
    st, touched = bench.stage_bytes_flops(cfg, counts, True)
    assert touched == 10
    assert st["gemm_gate_up"][1] == 4 * 1000 * cfg.D * cfg.I


def test_sampled_steps():
    """A fixed handful of timed steps carry the gate/up events, spread over the region."""
    assert bench.sampled_steps(20) == [2, 7, 12, 17]
    assert bench.sampled_steps(50) == [6, 18, 31, 43]
    assert bench.sampled_steps(3) == [0, 1, 2]
    assert bench.sampled_steps(1) == [0]
    for n in (4, 5, 7, 100, 1000):
        s = bench.sampled_steps(n)
        assert len(s) == 4 and all(0 <= i < n for i in s)


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_from_pmc(tmp_path, monkeypatch):
    """Each counter is scaled by what it reads for the 1 GiB calibration copy, the
    GEMM's launches are averaged, and the MXFP8 kernel is told apart by its name."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic_{config}.json"))
    # the kernel the library's plan names for the Qwen3-shaped layer's gate/up GEMM
    bf = "void moe::k_gemm_wsp<128, 128, 2, 1, 3, 8, false>(unsigned short const*)"
    f8 = "void moe::k_gemm_wsp<128, 128, 2, 1, 3, 8, true>(unsigned short const*)"
    other = "void moe::k_gemm_wsp<128, 256, 1, 0, 3, 8, false>(unsigned short const*)"
    cp = "__amd_rocclr_copyBuffer"
    kib = 1 << 20                           # the copy's 1 GiB in KiB
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    # FETCH_SIZE reads half the copy's bytes (x2 scale), WRITE_SIZE all of them (x1)
    _pmc_csv(fetch, "FETCH_SIZE", [(cp, kib / 2), (cp, 10.0), (bf, 1000.0), (bf, 1200.0), (f8, 400.0),
                                   (other, 7.0)])
    _pmc_csv(write, "WRITE_SIZE", [(cp, kib), (bf, 100.0), (bf, 100.0), (f8, 50.0), (other, 7.0)])
    name = "qwen3_30b_a3b_shaped"
    bench.traffic_from_pmc(str(fetch), str(write), name, 1024, "fetch cmd", "write cmd")
    d = json.load(open(tmp_path / f"traffic_{name}.json"))
    assert d["fetch"]["launches"] == 2 and d["fetch"]["kib_per_launch"] == 1100.0
    assert d["fetch"]["scale"] == pytest.approx(2.0) and d["write"]["scale"] == pytest.approx(1.0)
    assert d["hbm_bytes_per_launch"] == int(1100 * 1024 * 2 + 100 * 1024)
    assert "false>" in d["kernel"]
    bench.traffic_from_pmc(str(fetch), str(write), name + "_mxfp8", 1024, "fetch cmd", "write cmd")
    d8 = json.load(open(tmp_path / f"traffic_{name}_mxfp8.json"))
    assert d8["fetch"]["launches"] == 1 and d8["hbm_bytes_per_launch"] == int(400 * 1024 * 2 + 50 * 1024)
    assert "true>" in d8["kernel"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
