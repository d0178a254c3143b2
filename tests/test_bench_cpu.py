"""CPU checks of bench.py's contract and bookkeeping (no GPU needed).

The algorithmic work per launch is pinned to the totals stated for the 16k
workload (gate 68.2 MB, compaction 58.6 MB, attention 23.29 GFLOP at 2384
kept rows); the traffic summary's scaling by the copy kernel is checked on a
synthetic counter file."""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import Prompt  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["gpus_requested"] == 2


def test_algorithmic_work_of_the_16k_layer():
    class _T:  # shape-only stand-ins for the tensors
        def __init__(self, *shape):
            self.shape = shape

    w = types.SimpleNamespace(x=_T(16384, 2048), w1=_T(256, 2048), hq=16, hkv=8, head_dim=128,
                              prompts=[Prompt(0, 16384, 0, 16000, 2000)])
    m = 2384
    work = bench.algorithmic_work(w, m)
    # X read once (64 MiB), W1 once (1 MiB), w2, one fp32 score per row
    assert work["gate"]["bytes"] == 16384 * 2048 * 2 + 256 * 2048 * 2 + 256 * 2 + 16384 * 4
    assert round(work["gate"]["bytes"] / 1e6, 1) == 68.2
    assert work["gate"]["flops"] == 16384 * (2 * 2048 * 256 + 4 * 256)
    # compaction: hidden 4096 B + Q 4096 + K 2048 + V 2048 per row, read and written
    assert round(work["compact"]["bytes"] / 1e6, 1) == 58.6
    # attention: 4 * D * Hq per visible pair, M (M + 1) / 2 pairs
    assert work["attention"]["flops"] == 4 * 128 * 16 * (m * (m + 1) // 2)
    assert round(work["attention"]["flops"] / 1e9, 2) == 23.29
    assert work["select"]["bytes"] == 16000 * 4 + m * 4


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    rows = ["Kernel_Name,Counter_Name,Counter_Value"]
    copy = bench.COPY_BYTES
    # the copy's counters read 2x (fetch) and 1x (write) its true bytes; kernels scale alike
    rows += [f"__amd_rocclr_copyBuffer,FETCH_SIZE,{2 * copy / 1024}", f"__amd_rocclr_copyBuffer,WRITE_SIZE,{copy / 1024}"]
    rows += [f"void tg::attn_bf16_kernel<128>(x),FETCH_SIZE,{2 * 3e6 / 1024}",
             f"void tg::attn_bf16_kernel<128>(x),FETCH_SIZE,{2 * 5e6 / 1024}",
             f"void tg::attn_bf16_kernel<128>(x),WRITE_SIZE,{1e6 / 1024}"]
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    fetch.write_text("\n".join(r for r in rows if "WRITE" not in r) + "\n")
    write.write_text("\n".join(r for r in rows if "FETCH" not in r) + "\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda rel: "h")
    bench.traffic_summary(str(fetch), str(write))
    out = json.loads((tmp_path / "profiles" / "traffic_qwen16k.json").read_text())
    a = out["attention"]
    assert a["fetch_size_bytes"] == pytest.approx(4e6)       # mean of 3 and 5 MB
    assert a["write_size_bytes"] == pytest.approx(1e6)
    assert a["hbm_bytes_per_launch"] == pytest.approx(5e6)
    assert a["fetch_size_scale"] == pytest.approx(0.5) and a["write_size_scale"] == pytest.approx(1.0)
    assert a["source_sha256_16"] == "h"
