"""Host logic of bench.py, checked without a GPU: the algorithmic work its
rates divide by, counted here position by position from the workload's
segments and the oracle's maps; the code digest that gates the measured
HBM-traffic figures; and the one-GPU contract."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import acache_oracle as O
from synth.configs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("idx", sorted(WORKLOADS))
def test_work_model_counts(idx):
    """Probe (Section 3.2: every non-affix row over the affix, q.k and p.v,
    2d FLOPs each per key, head and layer; the masked rows' q.k again for the
    column mass), read-slot attention of the decode blocks and of the
    recompute set (Section 4.3, over every logical position), the admission
    scatter (read and write every recomputed row), and the unique bytes each
    moves (the shared affix once, each request's private slots once, Q and O)."""
    w = WORKLOADS[idx]
    K = O.anchor_count(w.L, w.rate)
    m = bench.work_model(w, K)
    d, N, Hq, Hkv = w.head_dim, w.n_layers, w.n_q_heads, w.n_kv_heads
    e = {"bf16": 2, "f32": 4}[w.dtype]
    # one request's sets (every request has the same layout)
    affix = set(range(w.affix_l, w.affix_l + w.L))
    non_affix = [p for p in range(w.T) if p not in affix]
    masked = w.positions("gen")
    anchors = np.arange(K) + w.affix_l
    read, rc_pos, _ = O.build_maps(anchors, w.T, w.affix_l, w.L, np.arange(w.L), np.arange(w.T), w.page_size)
    T_b, R_b = len(read), len(rc_pos)
    assert R_b == K + len(non_affix)
    kv_pos = N * Hkv * d * e * 2                      # K and V of one position, all layers and KV heads
    rows = w.batch * len(non_affix)
    assert m["probe_flops"] == rows * w.L * (2 * d + 2 * d) * N * Hq
    assert m["cm_flops"] == w.batch * len(masked) * w.L * 2 * d * N * Hq
    assert m["probe_bytes"] == w.L * kv_pos + rows * N * Hq * (2 * d * e + 4)   # affix K/V, Q in, O out, LSE
    nb = w.batch * w.block_len
    assert m["mapped_flops"] == nb * T_b * 4 * d * N * Hq
    assert m["recompute_flops"] == w.batch * R_b * T_b * 4 * d * N * Hq
    assert m["scatter_bytes"] == 2 * w.batch * R_b * kv_pos
    assert m["mapped_bytes"] == w.L * kv_pos + w.batch * R_b * kv_pos + 2 * nb * N * Hq * d * e
    assert m["block_bytes"] == 2 * nb * kv_pos


def test_code_digest_ignores_comments_and_spacing(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// header\n__global__ void f(int* x) {\n  x[0] = 1;  /* one */\n}\n")
    d0 = bench.code_digest(str(src))
    src.write_text("// a different header\n\n__global__ void f(int* x)\n{\n    x[0] = 1;\n}\n")
    assert bench.code_digest(str(src)) == d0
    src.write_text("__global__ void f(int* x) {\n  x[0] = 2;\n}\n")
    assert bench.code_digest(str(src)) != d0


def test_measured_traffic_needs_the_measured_code(tmp_path, monkeypatch):
    """The traffic figures are reported only while the counted kernels' code
    is the code the counters were taken on."""
    csrc = tmp_path / "attention_anchor_probe_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.TRAFFIC_SOURCES:
        (csrc / f).write_text(f"// {f}\nint g() {{ return 1; }}\n")
    (tmp_path / "profiles").mkdir()
    rec = {"code_sha256": {f: bench.code_digest(str(csrc / f)) for f in bench.TRAFFIC_SOURCES},
           "kernels": {"attn_rows_mfma": {"hbm_bytes": 123.0}}}
    (tmp_path / "profiles" / "pmc_traffic_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl") == {"attn_rows_mfma": 123.0}
    (csrc / bench.TRAFFIC_SOURCES[0]).write_text("// edited comment only\nint g() { return 1; }\n")
    assert bench.measured_traffic("wl") == {"attn_rows_mfma": 123.0}
    (csrc / bench.TRAFFIC_SOURCES[0]).write_text("int g() { return 2; }\n")
    assert bench.measured_traffic("wl") == {}
    assert bench.measured_traffic("other") == {}


def test_committed_traffic_record_matches_the_sources():
    """The committed counter record was taken on the current kernel code, so
    bench.py reports its traffic figures."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic_llada-prefix-L4096-b16.json")))
    for f in bench.TRAFFIC_SOURCES:
        assert rec["code_sha256"][f] == bench.code_digest(os.path.join(ROOT, "attention_anchor_probe_amd", "csrc", f))
    assert bench.measured_traffic("llada-prefix-L4096-b16")["attn_rows48_mfma"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""
