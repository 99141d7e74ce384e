"""Host-side logic of bench.py (no GPU): the algorithmic FLOP counts, the
HBM-traffic summary built from rocprofv3 counter CSVs and its source-hash
guard, and the one-GPU guard of the command line."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_flops_match_the_shape_formulas():
    # 0.6B shape, B=2, T=2048: projections 2*M*N*K, causal attention
    # 2*B*n_q*128*T*(T+1) (QK^T and PV over the lower triangle incl. the diagonal)
    f = bench.prefill_flops(2, 2048, 1024, 16, 8)
    assert f["qkv_norm_rope_gemm"] == 2.0 * 4096 * 4096 * 1024
    assert f["o_proj_gemm"] == 2.0 * 4096 * 1024 * 2048
    assert f["attention"] == 2.0 * 2 * 16 * 128 * 2048 * 2049
    assert abs(sum(f.values()) / 1e9 - 85.92) < 0.01


def test_chunk_flops_reduce_to_prefill_without_past():
    a = bench.chunk_flops(2, 512, 0, 1024, 16, 8)
    b = bench.prefill_flops(2, 512, 1024, 16, 8)
    assert a == pytest.approx(b)


def write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_and_guards_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    copy_kib = bench.COPY_BYTES / 1024
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    qkv, oproj = bench.PMC_KERNELS["prefill_qkv"], bench.PMC_KERNELS["prefill_oproj"]
    # the copy reads COPY_BYTES and FETCH_SIZE reports half of it: scale 2
    write_counter_csv(fetch, "FETCH_SIZE", [
        ("at::native::neg_kernel", copy_kib / 2), ("q3::flash_prefill_kernel<...>", 1000),
        ("q3::flash_prefill_kernel<...>", 1200), ("q3::decode_attn_kernel<...>", 300),
        ("q3::decode_combine_kernel<...>", 20)] + [(f"void q3::{s}(...)", 700)
                                                   for s in qkv + oproj])
    write_counter_csv(write, "WRITE_SIZE", [
        ("at::native::neg_kernel", copy_kib), ("q3::flash_prefill_kernel<...>", 500),
        ("q3::decode_attn_kernel<...>", 40), ("q3::decode_combine_kernel<...>", 4)]
        + [(f"void q3::{s}(...)", 300) for s in qkv + oproj])
    bench.summarize_pmc(str(fetch), str(write), ["cmd one", "cmd two"])
    got = bench.load_traffic()
    assert got["prefill_attention"] == pytest.approx((1100 * 2 + 500) * 1024)
    assert got["decode_attention"] == pytest.approx(((300 + 20) * 2 + 40 + 4) * 1024)
    assert got["prefill_qkv"] == pytest.approx((700 * 2 + 300) * 1024)
    text = open(bench.TRAFFIC_FILE).read()
    assert "cmd one" in text and "cmd two" in text
    # a record taken from other kernel sources is not used
    rec = json.loads(text.splitlines()[-1][len("TRAFFIC_JSON "):])
    rec["source_hash"]["prefill_attention"] = "0" * 16
    with open(bench.TRAFFIC_FILE, "w") as f:
        f.write("TRAFFIC_JSON " + json.dumps(rec) + "\n")
    assert set(bench.load_traffic()) == {"decode_attention", "prefill_qkv", "prefill_oproj"}


def test_traffic_summary_needs_the_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    write_counter_csv(fetch, "FETCH_SIZE", [("q3::flash_prefill_kernel<...>", 1)])
    write_counter_csv(write, "WRITE_SIZE", [("q3::flash_prefill_kernel<...>", 1)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(fetch), str(write), [])


def test_missing_traffic_file_gives_no_figures(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.load_traffic() == {}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_duration_timed_entries_run_long_enough():
    # the 4B, wide-GQA and chunked prefills are timed over at least
    # MIN_TIMED_STEPS steps and MIN_TIMED_S seconds, whatever --steps says
    assert bench.steps_for_duration(2e-3) == max(bench.MIN_TIMED_STEPS, 100)
    assert bench.steps_for_duration(6.4e-5) * 6.4e-5 >= bench.MIN_TIMED_S
    assert bench.steps_for_duration(10.0) == bench.MIN_TIMED_STEPS


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    # the traffic figures stay valid across comment edits, not across code edits
    names = bench.KERNEL_SOURCES["prefill_attention"]
    for n in names:
        (tmp_path / n).write_text(open(os.path.join(bench.CSRC, n)).read())
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    base = bench.kernel_source_hash("prefill_attention")
    f = tmp_path / names[0]
    src = f.read_text()
    f.write_text("// a new comment line\n" + src.replace("\n", "  // note\n", 3) + "\n/* block\n comment */\n")
    assert bench.kernel_source_hash("prefill_attention") == base
    f.write_text(src.replace("kHeadDim", "kHeadDim + 0", 1))
    assert bench.kernel_source_hash("prefill_attention") != base
