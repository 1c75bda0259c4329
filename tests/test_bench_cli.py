"""bench.py's command line on the CPU: more than one GPU is refused with a message
(the verify path runs on one GPU), and the summary of a rocprofv3 kernel-stats file
is a markdown table."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_stats_summary(tmp_path):
    csv = tmp_path / "stats.csv"
    csv.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                   '"verify_attn_partial_kernel(PartialArgs)",10,800000,80000.0,90.0,79000,81000,10.0\n')
    r = subprocess.run([sys.executable, "bench.py", "--summarize", "--kernel-stats", str(csv)], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[0].startswith("| kernel | calls | average us")
    assert "| 10 | 80.00 | 79.00 | 81.00 | 90.0% |" in lines[2]


def test_kernel_source_digest_follows_code_not_comments(tmp_path, monkeypatch):
    """The hash that ties counter files to the kernel source ignores comments and
    whitespace but changes with any code token, string literals included."""
    sys.path.insert(0, ROOT)
    import bench
    def digest(text):
        f = tmp_path / "k.hip"
        f.write_text(text)
        monkeypatch.setattr(bench, "KERNEL_SRC", str(f))
        return bench.kernel_source_digest()
    base = 'int f(int x) {  // scale\n  return x * 2; /* twice */\n}\nconst char* s = "a // b";\n'
    same = '// header\nint f(int x) {\n    return x * 2;\n}\n/* block\n comment */ const char* s = "a // b";\n'
    assert digest(base) == digest(same)
    assert digest(base) != digest(base.replace("x * 2", "x * 3"))
    assert digest(base) != digest(base.replace('"a // b"', '"a / b"'))
