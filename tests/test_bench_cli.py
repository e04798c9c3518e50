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
                 "--full-check", "--full-tensor", "--trace-summary", "--ceilings", "--sustain-s",
                 "--counter-summary", "--counter-table"):
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


def _counter_csv(d, rows):
    """rocprofv3 --pmc output layout: one counter_collection.csv under d."""
    d.mkdir(parents=True)
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"']
    for disp, name, ctr, val, t0, t1 in rows:
        lines.append(f'"{disp}","{name}","{ctr}","{val}","{t0}","{t1}"')
    (d / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_counter_summary_scales_by_the_copy(tmp_path):
    """--counter-summary sums a counter over its instances per dispatch, takes
    the median over dispatches and scales KiB by what the same counter read
    for the 1 GiB calibration copy (synthetic counter files, no GPU)."""
    import json
    fwd = "void fa::fa_fwd_kernel<fa::FP16, 128, false, false>(x)"
    copy = "copy_kernel"
    # fetch: 2 instances per dispatch; dispatch sums 300, 500, 400 KiB -> median 400
    _counter_csv(tmp_path / "f", [(1, fwd, "FETCH_SIZE", 100, 0, 1), (1, fwd, "FETCH_SIZE", 200, 0, 1),
                                  (2, fwd, "FETCH_SIZE", 250, 0, 1), (2, fwd, "FETCH_SIZE", 250, 0, 1),
                                  (3, fwd, "FETCH_SIZE", 400, 0, 1)])
    _counter_csv(tmp_path / "w", [(1, fwd, "WRITE_SIZE", 64, 0, 1), (2, fwd, "WRITE_SIZE", 64, 0, 1)])
    # the copy's fetch counter reads half the bytes it moves (factor 2), write reads all (factor 1)
    _counter_csv(tmp_path / "cf", [(1, copy, "FETCH_SIZE", 1 << 19, 0, 1), (2, "small", "FETCH_SIZE", 5, 0, 1)])
    _counter_csv(tmp_path / "cw", [(1, copy, "WRITE_SIZE", 1 << 20, 0, 1)])
    out = tmp_path / "traffic.json"
    r = run("--counter-summary", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
            str(tmp_path / "cw"), "--write-traffic", str(out))
    assert r.returncode == 0, r.stderr
    rec = [json.loads(x) for x in r.stdout.splitlines()]
    assert [x["name"] for x in rec] == ["fa_fwd_kernel"]
    assert rec[0]["fetch_bytes_per_launch"] == 400 * 1024 * 2
    assert rec[0]["write_bytes_per_launch"] == 64 * 1024
    assert rec[0]["dispatches"] == [3, 2]
    assert json.loads(out.read_text())["fa_fwd_kernel"]["hbm_bytes_per_launch"] == (800 + 64) * 1024


def test_counter_table_medians_per_dispatch(tmp_path):
    """--counter-table reports each counter's median per dispatch and the
    median duration of its dispatches over all passes (synthetic files)."""
    import json
    dq = "void fa::fa_bwd_dq_kernel<fa::FP16, 128, false, false>(x)"
    _counter_csv(tmp_path / "a", [(1, dq, "SQ_INSTS_MFMA", 10, 0, 2000), (2, dq, "SQ_INSTS_MFMA", 30, 0, 4000),
                                  (3, dq, "SQ_INSTS_MFMA", 20, 0, 3000)])
    _counter_csv(tmp_path / "b", [(1, dq, "SQ_WAVES", 7, 0, 1000), (1, dq, "SQ_WAVES", 1, 0, 1000)])
    r = run("--counter-table", str(tmp_path / "a"), str(tmp_path / "b"))
    assert r.returncode == 0, r.stderr
    rec = [json.loads(x) for x in r.stdout.splitlines()]
    assert len(rec) == 1 and rec[0]["name"] == "fa_bwd_dq_kernel"
    assert rec[0]["SQ_INSTS_MFMA"] == 20 and rec[0]["SQ_WAVES"] == 8
    assert rec[0]["dispatches"] == 3
    # durations of every dispatch of both passes: 2, 4, 3 and 1 us
    assert rec[0]["time_us"] == 2.5


def test_check_heads_measures_every_row():
    """bench.check_heads (the full-tensor check of --full-check and
    --all-configs --full-tensor) against a result whose errors are planted
    on the host: one element of O and one lse of the second head."""
    import importlib.util
    import numpy as np
    sys.path.insert(0, ROOT)
    from flashattention_attention_fa_amd import synth
    from oracle import oracle as oracle_mod
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    orc = oracle_mod.get()
    B, H, N, d = 1, 2, 40, 16
    q, k, v = synth.fwd_inputs(B, H, N, d, "bf16", seed=5)
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    ro, rl = orc.attention(qb, kb, vb, "bf16", True, 0.25)
    og, lg = ro.astype(np.float32), rl.astype(np.float32)
    og[0, 1, 17, 3] += 0.01
    lg[0, 1, 30] -= 0.002
    res = bench.check_heads(orc, qb, kb, vb, og, lg, "bf16", True, 0.25, [(0, 0), (0, 1)])
    assert res["heads_checked"] == 2 and res["rows_checked"] == 2 * N
    assert abs(res["max_abs"] - 0.01) < 1e-5
    assert abs(res["lse_max_abs"] - 0.002) < 1e-5
    assert res["worst_row"] == (0, 1, 17)


def test_source_digest_ignores_comments_and_layout():
    """The traffic record of a kernel stays valid across comment edits: the
    digest covers the code only, string literals included."""
    import bench
    a = bench.code_text('int f(int x) {  // first\n  return x + 1; /* two\nlines */ }\n')
    b = bench.code_text('/* header */ int f(int x)\n{\n  return x + 1;\n}  // tail\n')
    assert a == b == "int f(int x) { return x + 1; }"
    assert bench.code_text('s = "a//b /* c */"; // x') == 's = "a//b /* c */";'
    assert bench.code_text('int x = 1;') != bench.code_text('int x = 2;')
    d = bench.source_digest("fa_fwd.hip", "fa_device.hpp")
    assert len(d) == 16 and d == bench.source_digest("fa_fwd.hip", "fa_device.hpp")
