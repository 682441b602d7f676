"""Host-side logic of bench.py, on the CPU: the algorithmic byte counts, the
rule that counter traffic is reported only for the kernel source it was
taken on, the scaling of rocprofv3 counters by the copy probe, and the
refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes():
    # 2 N_d gradient bytes, fp32 master/m/v read and written, one 16-bit parameter written
    assert bench.algorithmic_bytes_per_param(64) == 154
    assert bench.algorithmic_bytes_per_param(16) == 58
    assert bench.algorithmic_bytes_per_param(8) == 42


def test_traffic_only_for_its_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha": bench.kernel_source_sha(), "hbm_bytes_per_launch": 123.0}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(154.0) == 123.0
    rec["kernel_source_sha"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic(154.0) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic(154.0) is None


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    srcs = []
    for i, p in enumerate(bench.KERNEL_SOURCES):
        q = tmp_path / f"src{i}"
        q.write_text(open(p).read())
        srcs.append(q)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", tuple(str(q) for q in srcs))
    base = bench.kernel_source_sha()
    assert base == bench.kernel_source_sha()
    text = srcs[0].read_text()
    srcs[0].write_text("// a new comment\n" + text.replace("\n", "  /* a block\n comment */\n", 1) + "\n\n")
    assert bench.kernel_source_sha() == base
    srcs[0].write_text(text.replace("kTile = 512", "kTile = 256", 1))
    assert "kTile = 512" in text and bench.kernel_source_sha() != base
    srcs[0].write_text(text)
    srcs[1].write_text(srcs[1].read_text() + "\nconstexpr int kExtra = 1;\n")
    assert bench.kernel_source_sha() != base


def test_kernel_sources_hold_no_comment_marker_in_a_string():
    # code_text strips comments with two regular expressions, which would
    # misread a string literal holding "//" or "/*".
    import re
    for p in bench.KERNEL_SOURCES:
        for lit in re.findall(r'"(?:[^"\\\n]|\\.)*"', open(p).read()):
            assert "//" not in lit and "/*" not in lit, (p, lit)


def _counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_write_traffic_scales_by_the_copy_probe(tmp_path, monkeypatch):
    """FETCH_SIZE reads half the bytes of a plain copy on MI355X: the copy of
    4 GiB each way gives the scale, which turns the step's KiB into bytes."""
    k = bench.HEADLINE_KERNEL
    S = 117_187_520
    copy_kib_f, copy_kib_w = 2 * 1024 * 1024, 4 * 1024 * 1024   # 0.5 and 1.0 of 4 GiB
    step_read, step_write = 140 * S, 14 * S                     # bytes per launch
    _counters(tmp_path / "f.csv", [(f"void x::{k}(y)", "FETCH_SIZE", step_read / 1024 * 0.5)] * 2)
    _counters(tmp_path / "w.csv", [(f"void x::{k}(y)", "WRITE_SIZE", step_write / 1024)] * 2)
    _counters(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib_f)])
    _counters(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_kib_w)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                        str(tmp_path / "cw.csv"))
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(0.5) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes_per_element"] == pytest.approx(140.0)
    assert rec["write_bytes_per_element"] == pytest.approx(14.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(154 * S)
    assert rec["kernel_source_sha"] == bench.kernel_source_sha()


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env=dict(os.environ, CUDA_VISIBLE_DEVICES=""))
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr


def test_release_waits_in_proportion_to_the_bytes_freed(monkeypatch):
    class Cuda:
        def __init__(self, before, after):
            self.reserved = [before, after]
            self.emptied = 0

        def synchronize(self):
            pass

        def memory_reserved(self):
            return self.reserved[self.emptied]

        def empty_cache(self):
            self.emptied = 1

    class Torch:
        def __init__(self, before, after):
            self.cuda = Cuda(before, after)

    slept = []
    monkeypatch.setattr(bench.time, "sleep", slept.append)
    bench.release(Torch(40e9, 8e9))          # 32 GB given back
    assert slept == [pytest.approx(0.2 + 32e9 / bench.SETTLE_BYTES_PER_S)]
    bench.release(Torch(8e9, 8e9))           # nothing given back: no wait
    assert len(slept) == 1
    bench.release(Torch(500e9, 0))           # capped
    assert slept[-1] == bench.SETTLE_MAX_S
