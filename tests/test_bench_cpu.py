"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
and read counts behind the roofline, and the folding of rocprofv3 counter runs
into HBM bytes per decode call."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from head_latent_attention_05_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kv_reads_decode_and_causal():
    inp = synth.make_inputs("batch64", kv_lens=[5, 70], q_len=1)
    assert bench.kv_reads(inp) == 5 + 70
    pre = synth.make_inputs("prefill", kv_lens=[10, 4], q_len=3)
    # causal: query j of a sequence with L rows and q new tokens sees L - q + j + 1 rows
    assert bench.kv_reads(pre) == (8 + 9 + 10) + (2 + 3 + 4)


def test_decode_bytes_bf16_and_e4m3():
    inp = synth.make_inputs("batch64", kv_lens=[100, 37], q_len=1)
    reads, b16, flops = bench.decode_bytes_flops(inp)
    _, b8, flops8 = bench.decode_bytes_flops(inp, fp8=True)
    io = inp.T * 128 * (576 + 512) * 2       # q_lat in, o_lat out (bf16)
    assert b16 == reads * 576 * 2 + io
    assert b8 == reads * 576 + io            # one byte per cached value
    assert flops == flops8 == reads * 2 * 128 * (576 + 512)


def _write_run(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_folding(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE in KiB per dispatch are scaled by what the 1 GiB
    copy reads for the same counters, summed over the decode call's kernels and
    stamped with the source hash (which traffic_from_counters checks)."""
    copy = "__amd_rocclr_copyBuffer"
    dec = "mla::(anonymous namespace)::decode_v4_kernel(int const*)"
    mrg = "mla::(anonymous namespace)::merge_v3_kernel(mla::PlanArgs)"
    gib_kib = (1 << 30) // 1024
    _write_run(str(tmp_path / "fetch"), [(copy, "FETCH_SIZE", gib_kib / 2),
                                         (dec, "FETCH_SIZE", 1000), (dec, "FETCH_SIZE", 1200),
                                         (mrg, "FETCH_SIZE", 100)])
    _write_run(str(tmp_path / "write"), [(copy, "WRITE_SIZE", gib_kib),
                                         (dec, "WRITE_SIZE", 40), (mrg, "WRITE_SIZE", 8)])
    out = tmp_path / "counters.json"
    assert bench.counters_json("single", [str(tmp_path / "fetch"), str(tmp_path / "write")],
                               str(out)) == 0
    rec = json.load(open(out))["single"]
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    want = (1100 * 2 + 100 * 2 + 40 + 8) * 1024
    assert rec["traffic_bytes"] == pytest.approx(want)
    assert rec["source_sha"] == bench.source_hash()
    monkeypatch.setattr(bench, "COUNTERS", str(out))
    assert bench.traffic_from_counters("single") == pytest.approx(want)
    # a stale stamp is ignored
    rec["source_sha"] = "0" * 16
    json.dump({"single": rec}, open(out, "w"))
    assert bench.traffic_from_counters("single") is None
