"""Host-side logic of bench.py (no GPU): the algorithmic flop counts, the
code-only hash that keys the committed counter record, the counter CSV
reader, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("shape", [(1600, 6400), (6400, 1600), (768, 768)])
def test_ns_flops_per_iteration(shape):
    m, n = min(shape), max(shape)
    assert bench.ns_flops([shape], "gram") == m * m * n
    assert bench.ns_flops([shape], "poly") == m ** 3
    assert bench.ns_flops([shape], "bx") == 2 * m * m * n
    # the three stages together: 3 m^2 n + m^3 per matrix and iteration
    tot = sum(bench.ns_flops([shape], k) for k in ("gram", "poly", "bx"))
    assert tot == 3 * m * m * n + m ** 3


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {\n  // add one\n  return x + 1;  /* plain */\n}\n"
    b = "/* header\n   text */\nint f(int x) {\n\n    return x + 1;\n}   // tail\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_traffic_record_ignored_for_other_code(tmp_path, monkeypatch):
    rec = tmp_path / "profiles"
    rec.mkdir()
    (rec / "traffic_w.json").write_text('{"source_hash": "0000000000000000", "bytes_per_launch": 5.0}\n')
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "matrix_muon_step_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("int k;\n")
    assert bench.load_traffic(("k.hip",), "w") is None
    h = bench.source_hash(("k.hip",))
    (rec / "traffic_w.json").write_text('{"source_hash": "%s", "bytes_per_launch": 5.0}\n' % h)
    assert bench.load_traffic(("k.hip",), "w") == 5
    (csrc / "k.hip").write_text("// a comment\nint k;\n")
    assert bench.load_traffic(("k.hip",), "w") == 5
    (csrc / "k.hip").write_text("int k2;\n")
    assert bench.load_traffic(("k.hip",), "w") is None


def test_read_counter_csv_sums_per_dispatch(tmp_path):
    p = tmp_path / "c.csv"
    p.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
                 "1,kern_a,FETCH_SIZE,10\n"
                 "1,kern_a,FETCH_SIZE,5\n"
                 "2,kern_a,FETCH_SIZE,7\n"
                 "3,kern_b,FETCH_SIZE,1\n"
                 "3,kern_b,WRITE_SIZE,9\n")
    per = bench.read_counter_csv(str(p), "FETCH_SIZE")
    assert sorted(per["kern_a"]) == [7.0, 15.0]
    assert per["kern_b"] == [1.0]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_info_fields():
    info = bench.cpu_info()
    assert set(info) == {"cpu_model", "host_cpus", "blas", "blas_threads"}
    assert info["host_cpus"] == os.cpu_count()
