"""Host logic of bench.py (no GPU): the algorithmic FLOP and byte counts the roofline divides
by, the stored-traffic lookup, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from mixture_experts_layer_26_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_v3_prefill_flops():
    # 3 matrices, 2 FLOP per multiply-add: 6 d d_ff per routed row and per shared row
    w = I.WORKLOADS["v3_prefill_bf16"]
    assert w.ffn_flops() == 6 * 7168 * 2048 * (8192 * 8 + 8192)


def test_v3_prefill_algorithmic_bytes():
    # weights of every active routed expert and the shared one, plus u read once; H and the
    # outputs y_routed, y_shared are not algorithmic bytes
    w = I.WORKLOADS["v3_prefill_bf16"]
    counts = np.full(256, 8192 * 8 // 256)
    got, active = bench.ffn_algorithmic_bytes(w, counts)
    weights = (256 + 1) * 3 * 7168 * 2048 * 2
    assert active == 256 and got == weights + 8192 * 7168 * 2


def test_algorithmic_bytes_count_active_experts_only():
    w = I.WORKLOADS["v3_decode_skewed"]
    counts = np.zeros(256, dtype=np.int64)
    counts[:10] = 128 * 8 // 10
    counts[10] = 128 * 8 - counts[:10].sum()
    got, active = bench.ffn_algorithmic_bytes(w, counts)
    assert active == 11
    assert got == (11 + 1) * 3 * 7168 * 2048 * 2 + 128 * 7168 * 2


def test_fp8_bytes_include_block_scales():
    w = I.WORKLOADS["v3_prefill_fp8"]
    got, _ = bench.ffn_algorithmic_bytes(w, np.full(256, 256))
    per_expert = 3 * 7168 * 2048 + 3 * 56 * 16 * 4
    assert got == 257 * per_expert + 8192 * 7168 * 2


def test_roofline_kind_per_workload():
    kinds = {n: bench.roofline_kind(w) for n, w in I.WORKLOADS.items()}
    assert kinds == {"tiny_f32": "latency", "mid_bf16": "mfma", "v3_prefill_bf16": "mfma",
                     "v3_prefill_fp8": "mfma", "v3_decode_skewed": "hbm", "v3_ep8_share_bf16": "mfma",
                     "v3_ep8_share_fp8": "mfma"}


def test_sub_workloads_cover_every_other_workload():
    assert set(bench.SUB_WORKLOADS) | {"v3_prefill_bf16"} == set(I.WORKLOADS)
    assert set(bench.CPU_TOKENS) == set(I.WORKLOADS)


def test_stored_traffic_needs_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("v3_prefill_bf16", "bf16", "tiled") is None  # no file
    h = "a" * 16
    monkeypatch.setattr(bench, "kernel_source_hash", lambda ffn: h if ffn == "bf16" else "b" * 16)
    rec = {"workload": "v3_prefill_bf16", "weights": "tiled", "kernel_source_hash": h, "hbm_bytes_per_call": 123}
    (prof / "traffic_v3_prefill_bf16.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("v3_prefill_bf16", "bf16", "tiled")["hbm_bytes_per_call"] == 123
    assert bench.stored_traffic("v3_prefill_bf16", "bf16", "rows") is None   # another weight layout
    assert bench.stored_traffic("v3_prefill_bf16", "fp8", "tiled") is None   # other kernel sources
    rec["kernel_source_hash"] = "0" * 16
    (prof / "traffic_v3_prefill_bf16.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("v3_prefill_bf16", "bf16", "tiled") is None


def test_source_hash_depends_on_the_dtype_kernel():
    assert bench.kernel_source_hash("bf16") != bench.kernel_source_hash("fp8")
    assert len(bench.kernel_source_hash("bf16")) == 16


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus must be 1" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("name", ["v3_prefill_bf16", "v3_prefill_fp8", "v3_decode_skewed"])
def test_committed_traffic_matches_its_workload(name):
    with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json")) as f:
        t = json.load(f)
    assert t["workload"] == name and t["weights"] == "tiled"
    assert abs(t["hbm_bytes_per_call"] - (t["phase1_bytes"] + t["phase2_bytes"])) <= 1  # each rounded down


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    csrc = tmp_path / "mixture_experts_layer_26_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("gemm_common.h", "ffn_bf16.hip", "device.h", "pack.hip"):
        (csrc / f).write_text("int a = 1;  // one\n/* block\n comment */ int b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash("bf16")
    (csrc / "ffn_bf16.hip").write_text("int a = 1;  // another comment\n\nint b = 2;\n")
    assert bench.kernel_source_hash("bf16") == h
    (csrc / "ffn_bf16.hip").write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash("bf16") != h
