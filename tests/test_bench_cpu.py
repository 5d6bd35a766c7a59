"""Host logic of bench.py (no GPU): the kernel-source hash that keys stored
counter results, the conversion of counter runs into HBM bytes per step, and
the one-GPU guard."""

from __future__ import annotations

import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_only_strips_comments_and_layout():
    src = "int a;  /* block\n comment */\n// line comment\n   int   b; // tail\n"
    assert bench.code_only(src) == "int a; int b;"


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    d.mkdir()
    f = d / "k.h"
    f.write_text("int f(int x) { return x + 1; }\n")
    monkeypatch.setattr(bench, "KERNEL_SRC_DIR", str(d))
    h0 = bench.source_hash()
    f.write_text("// a new comment\nint f(int x) {\n  return x + 1;   /* same code */\n}\n")
    assert bench.source_hash() == h0
    f.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash() != h0


def _counter_run(path, counter, rows):
    path.mkdir()
    with open(path / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    sk = "void pa::pa_decode_sk_kernel<pa::ElemBF16, pa::Kv16, 128, 4, true, false, 1>(...)"
    mg = "void pa::pa_sk_merge_kernel<pa::ElemBF16, 128, 4, 4>(...)"
    cp = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half of a 1 GiB copy (scale 2); WRITE_SIZE all of it (scale 1).
    _counter_run(tmp_path / "f", "FETCH_SIZE", [(sk, 100), (mg, 4), (sk, 102), (mg, 4), (cp, 524288)])
    _counter_run(tmp_path / "w", "WRITE_SIZE", [(sk, 10), (mg, 2), (sk, 10), (mg, 2), (cp, 1048576)])
    tj = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tj))
    args = types.SimpleNamespace(traffic_from=f"{tmp_path / 'f'},{tmp_path / 'w'}", config=3, partition=-1,
                                 flags=-1, copy_calibration=1024)
    bench.write_traffic(args)
    rec = json.load(open(tj))["pa_decode_sk_kernel+pa_sk_merge_kernel|cfg3"]
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == (101 + 4) * 1024 * 2
    assert rec["write_bytes"] == (10 + 2) * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["per_kernel_fetch_bytes"] == {"pa_decode_sk_kernel": 101 * 2048, "pa_sk_merge_kernel": 4 * 2048}
    assert rec["source_hash"] == bench.source_hash()
    # a stored record is used only while the kernel sources are unchanged
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.traffic_for("pa_decode_sk_kernel+pa_sk_merge_kernel", "cfg3") is None


def test_traffic_keys_strip_template_arguments_and_parameters(tmp_path, monkeypatch):
    va = "void pa::pa_decode_valu_kernel<pa::ElemF16, pa::Kv16, 128, 1, true>(void*, int*)"
    order = "pa::(anonymous namespace)::pa_order_by_length_kernel(int const*, int, int, int*)"
    cp = "__amd_rocclr_copyBuffer"
    _counter_run(tmp_path / "f", "FETCH_SIZE", [(va, 1000), (order, 2), (cp, 524288)])
    _counter_run(tmp_path / "w", "WRITE_SIZE", [(va, 10), (order, 1), (cp, 1048576)])
    tj = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tj))
    args = types.SimpleNamespace(traffic_from=f"{tmp_path / 'f'},{tmp_path / 'w'}", config=2, partition=-1,
                                 flags=-1, copy_calibration=1024)
    bench.write_traffic(args)
    assert list(json.load(open(tj))) == ["pa_decode_valu_kernel+pa_order_by_length_kernel|cfg2"]


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
