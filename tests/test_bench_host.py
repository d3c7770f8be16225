"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the byte formulas the roofline and
the attention-stage fractions divide by, the counter calibration, and the code hash that keys the
recorded traffic."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_stage_bytes_of_the_32k_sweep():
    # Q, K, V, O once (8 heads x 32768 tokens x 64 dims x 2 bytes each) plus the selection (R = 2 int32)
    w = synth.workload("sweep")
    assert bench.stage_bytes(w) == 4 * 8 * 32768 * 64 * 2 + 8 * 32768 * 2 * 4 == 136314880


def test_selected_set_bytes_formula():
    w = synth.workload("sweep")
    pairs = 1000
    per_token = 2 * 64 * 2 + 2 * 64 * 2 * 2  # q and o, plus L = 2 local blocks of K and V rows amortised
    assert bench.selected_set_bytes(w, pairs) == 8 * 32768 * per_token + pairs * 64 * 64 * 2 * 2


def test_design_bytes_of_the_attention_kernels():
    w = synth.workload("sweep")
    st = {"pairs": 436000, "blocks_used": 4046}
    ab = bench.design_bytes(w, st)
    qkv = 8 * 32768 * 64 * 2
    # the local kernel: Q, its K/V window and O once, the selection, and one partial per pair
    assert ab["attn_local"] == 4 * qkv + 8 * 32768 * 2 * 4 + st["pairs"] * (64 * 2 + 4)
    # the binning: the selection, the per-range counts (16 ranges of 2048 tokens x 510 blocks), the lists
    assert ab["attn_bin"] == 8 * 32768 * 2 * 4 + 8 * 16 * 510 * 4 + st["pairs"] * 4 + 8 * 511 * 4
    assert all(v > 0 for v in ab.values())


def test_stage_span_brackets_the_attention_kernels():
    names = ["address", "post", "probe_rerank", "attn_bin", "attn_remote", "attn_local"]
    assert bench.stage_span(names) == (4, 6)
    assert bench.stage_span(["address", "probe_rerank", "attn_local"]) == (2, 3)


def test_cpu_baseline_uses_every_usable_core():
    """The oracle timed over a process pool: the shares cover every token of every sampled head once, and
    the record states the cores used, the CPU model and the one-thread rate beside the pool's."""
    w = synth.workload("tiny")
    inp = synth.make_core_inputs(w, 0)
    cores, avail, model = bench.host_cpu()
    assert 1 <= cores <= 16 and cores <= avail and model
    r = bench.cpu_baseline(w, inp, 8)
    assert r["cores"] == cores and r["kind"] == "oracle" and r["cpu_model"] == model
    assert r["value"] > 0 and r["one_thread_tokens_per_s"] > 0
    assert str(cores) in r["sample"] and "packed C oracle" in r["sample"]
    assert r["numpy_oracle"]["tokens_per_s"] > 0


def test_strip_comments():
    src = b"int a; // x\n/* multi\nline */ int b;\n\n  // only a comment\nint c;\n"
    assert bench.strip_comments(src) == b"int a;\n int b;\nint c;"


def test_code_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "learned_product_hash_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    for f in os.listdir(os.path.join(ROOT, "learned_product_hash_amd", "csrc")):
        if f.endswith((".hip", ".h")):
            (csrc / f).write_bytes(open(os.path.join(ROOT, "learned_product_hash_amd", "csrc", f), "rb").read())
    (tmp_path / "include" / "mdr.h").write_bytes(open(os.path.join(ROOT, "include", "mdr.h"), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_digest("attn_remote")
    f = csrc / "mdr_attn.hip"
    f.write_bytes(f.read_bytes() + b"\n// a new comment\n")
    assert bench.source_digest("attn_remote") == h0
    tiles = csrc / "mdr_tiles.h"  # an included header: its code counts
    tiles.write_bytes(tiles.read_bytes() + b"\nstatic int extra_symbol;\n")
    assert bench.source_digest("attn_remote") != h0


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            wr.writerow([r[0], r[1], counter, r[2]])


def test_ingest_scales_each_counter_by_the_calibration_copy(tmp_path, monkeypatch):
    w = synth.workload("sweep")
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda _w: str(out))
    kib = bench.CALIB_BYTES / 1024.0
    # the copy reads half its bytes by FETCH_SIZE (factor 2) and all by WRITE_SIZE (factor 1); the remote
    # kernel is dispatched twice, with its counters split over two rows (channels) per dispatch
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, "at::native::neg_kernel", kib / 2), (2, "mdr::k_attn_remote<bf16>", 600.0),
        (2, "mdr::k_attn_remote<bf16>", 400.0), (3, "mdr::k_attn_remote<bf16>", 1000.0)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, "at::native::neg_kernel", kib), (2, "mdr::k_attn_remote<bf16>", 250.0),
        (3, "mdr::k_attn_remote<bf16>", 250.0)])
    bench.ingest_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), w)
    t = json.load(open(out))
    assert t["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["calibration"]["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]["attn_remote"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == pytest.approx(1000.0 * 2 * 1024)
    assert k["write_bytes"] == pytest.approx(250.0 * 1024)
    assert k["source_sha"] == bench.source_digest("attn_remote")
