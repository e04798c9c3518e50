"""bench.py's command line on the CPU: it measures one GPU only and says so for
any other count before touching a device; its modes are listed in --help."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--all-configs", "--calibrate-copy", "--only",
                 "--full-check", "--trace-summary", "--ceilings", "--sustain-s"):
        assert flag in r.stdout


def test_trace_summary_counts_only_timed_launches(tmp_path):
    """--trace-summary skips each kernel's warm-up launches and averages the
    timed ones, by launch order (a synthetic kernel trace, no GPU)."""
    import json
    rows = ['"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"']
    t = 0
    # 2 warm-up and 3 timed forward launches, then one more (the bwd leg's)
    for dur in (9000, 9000, 1000, 2000, 3000, 50000):
        rows.append(f'"KERNEL_DISPATCH","void fa::fa_fwd_kernel<fa::FP16, 128, false, false>(x)",'
                    f'{t},{t + dur * 1000}')
        t += dur * 1000 + 10
    path = tmp_path / "kernel_trace.csv"
    path.write_text("\n".join(rows) + "\n")
    r = run("--trace-summary", str(path), "--steps", "3", "--warmup", "2")
    assert r.returncode == 0, r.stderr
    rec = [json.loads(x) for x in r.stdout.splitlines()]
    assert len(rec) == 1 and rec[0]["leg"] == "fwd"
    assert rec[0]["timed"] == 3 and rec[0]["skipped"] == 2 and rec[0]["launches_in_trace"] == 6
    assert rec[0]["avg_us"] == 2000.0 and rec[0]["median_us"] == 2000.0
