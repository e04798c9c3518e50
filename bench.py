#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

One step = one fa_fwd over the forward benchmark shape (B=8, H=32, N=8192,
d=128, fp16, non-causal: the shape of the benchmark listing on the
dailyaiworld page "FlashAttention-3 vs Triton Kernels", section
"Benchmarking Triton vs FlashAttention-3 Kernels") followed by one fa_decode
over the split-KV decode shape (B=8, Hq=32, Hkv=8, L=32768, d=128, bf16,
nsplit=16).  Inputs are seeded synthetic tensors already resident in HBM.

FLOPs follow the listing's convention, 4*B*H*N^2*d (halved when causal).
Algorithmic bytes: forward reads Q, K, V once and writes O (fp32) and lse
once; decode reads the K and V caches once (GQA: each kv head once), q once,
and writes O once.  Timing: W warm-up steps, then K timed steps between a
synchronize on both sides; HIP events recorded on the launch stream between
the two calls of every step give each call's average duration.

After the timed steps, the FP8 forward (fa_fwd_fp8) is timed on the same
forward shape with E4M3 inputs and reported in its own "fp8_fwd" object
against the dense fp8 MFMA peak, and the attention backward (fa_bwd: the dQ
kernel, then the dK/dV kernel) on the same shape in its own "bwd" object
(algorithmic FLOPs 2.5x the forward's: five N x N x d products).  Two more
objects time the variable-length paths: "varlen_fwd" (fa_fwd_varlen on a
packed batch of eight sequences of mixed lengths, 65536 tokens in all, the
forward shape's token count, H=32, d=128, fp16, non-causal) and
"paged_decode" (fa_decode_paged on the decode shape with the caches in
16-token pages reached through shuffled block tables).  None of these is
part of the step or of "value".

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOPS + % MFMA peak (B8 H32 N8192 d128); decode HBM GB/s"
PEAK_MFMA_TFLOPS = 2516.6     # MI355X dense fp16/bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA (256 CU x 8192 flop/clk x 2.4 GHz)
FWD = dict(B=8, H=32, N=8192, d=128, dtype="fp16", causal=False, seed=1002)
DEC = dict(B=8, Hq=32, Hkv=8, L=32768, d=128, dtype="bf16", nsplit=16, seed=1005)
KV_COPIES = 4                 # decode rotates among this many caches (4 GiB > 256 MB MALL)
# Untimed warm-up calls of the legs after the step (the FP8 leg uses
# max(FP8_MIN_WARMUP, --warmup // 2)); --trace-summary skips the same calls.
FP8_MIN_WARMUP, BWD_WARMUP, VARLEN_WARMUP, PAGED_WARMUP = 5, 3, 3, 5


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def fwd_bytes(B, H, N, d, esize=2):
    return 3 * B * H * N * d * esize + B * H * N * d * 4 + B * H * N * 4


def decode_bytes(B, Hq, Hkv, L, d, esize=2):
    return 2 * B * Hkv * L * d * esize + B * Hq * d * esize + B * Hq * d * 4


def code_text(src):
    """A source with its comments removed and its whitespace collapsed: what
    the compiler sees, so that editing a comment keeps the digest."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] == '"':
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def source_digest(*names):
    """Digest of the code (comments and layout excluded) of kernel sources."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "flashattention_attention_fa_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


# roofline.traffic is not measured by the run that prints it: it is read
# from the committed counter record of the same kernel source.
TRAFFIC_SOURCE = ("profiles/traffic.json: rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel source "
                  "(matched by source digest, null otherwise), not measured by this run")


def load_traffic(kernel_key, digest, launches_per_unit=1):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


class ClockPowerSampler:
    """Samples the GPU's graphics clock and socket power during a timed
    region, on a background thread, through AMD SMI's library (GPU metrics
    table: the current clock of every XCD, current socket power, hotspot
    temperature).  The table is refreshed about once a second, so a
    window needs a few seconds to hold several readings; readings are told
    apart by the table's own system clock counter.  The handle is matched
    to the torch device by PCI address.  If the library or the metrics are
    unavailable the summary says why."""

    def __init__(self, device, period_s=0.005):
        self.period, self.samples, self.error, self._h = period_s, [], None, None
        try:
            import threading
            import torch
            sys.path.append("/opt/rocm/share/amd_smi")
            import amdsmi
            self._smi = amdsmi
            amdsmi.amdsmi_init()
            props = torch.cuda.get_device_properties(device)
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            for h in amdsmi.amdsmi_get_processor_handles():
                dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._h = h
            if self._h is None:
                raise RuntimeError(f"no AMD SMI handle at PCI {want}")
            self._stop = threading.Event()
            self._t = threading.Thread(target=self._run, daemon=True)
        except Exception as e:       # sampling is a diagnostic; timing goes on without it
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 65535]
        return {"t": time.perf_counter(), "stamp": m.get("system_clock_counter"), "sclk_mhz": clks,
                "power_w": m.get("current_socket_power"), "hotspot_c": m.get("temperature_hotspot")}

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self._h is not None:
            self.t0 = time.perf_counter()
            self._t.start()
        return self

    def __exit__(self, *exc):
        if self._h is not None:
            self._stop.set()
            self._t.join()
            self.t1 = time.perf_counter()
        return False

    def summary(self):
        import statistics as st
        # one reading per refresh of the metrics table; the first one was
        # taken before the window began
        seen, reads = set(), []
        for x in self.samples:
            if x["stamp"] not in seen:
                seen.add(x["stamp"])
                reads.append(x)
        reads = reads[1:]
        if not reads:
            return {"source": None if not self.samples else "amdsmi gpu_metrics",
                    "readings": 0, "samples": len(self.samples),
                    "error": self.error or "no refresh of the metrics table inside the window"}

        def stats(xs):
            xs = [x for x in xs if isinstance(x, (int, float))]
            return {"median": st.median(xs), "min": min(xs), "max": max(xs)} if xs else None
        out = {"source": "amdsmi gpu_metrics (current_gfxclks mean over XCDs, "
                         "current_socket_power), refreshed about once a second",
               "window_s": round(self.t1 - self.t0, 2), "readings": len(reads),
               "sclk_mhz": stats([st.mean(x["sclk_mhz"]) for x in reads if x["sclk_mhz"]]),
               "sclk_mhz_per_xcd_last": reads[-1]["sclk_mhz"],
               "power_w": stats([x["power_w"] for x in reads]),
               "hotspot_c": stats([x["hotspot_c"] for x in reads])}
        if self.error:
            out["error"] = self.error
        return out


def trace_summary(paths, warmup, steps, fp8_steps, bwd_steps, varlen_steps, paged_steps):
    """Kernel times from rocprofv3 kernel-trace CSVs of one run of this
    script with the same step counts: each kernel's launches in start order,
    the untimed warm-up launches skipped, averaged over the timed ones only
    (the forward's kernel is also launched once more by the bwd leg, after
    the step's launches; those and later launches are not counted)."""
    import csv
    import statistics as st
    csv.field_size_limit(1 << 30)
    launches = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                launches.setdefault(name, []).append((int(r["Start_Timestamp"]),
                                                      int(r["End_Timestamp"])))
    fwd = FWD
    flops = fwd_flops(fwd["B"], fwd["H"], fwd["N"], fwd["d"], fwd["causal"])
    fp8_warm = max(FP8_MIN_WARMUP, warmup // 2)
    # (leg, demangled name prefix, launches skipped, launches timed, algorithmic work, peak)
    legs = [("fwd", "fa::fa_fwd_kernel<fa::FP16, 128, false, false>(", warmup, steps,
             ("TFLOP/s", flops, PEAK_MFMA_TFLOPS)),
            ("decode", "fa::fa_decode_split_kernel<fa::BF16x16, 128, false, 1, 4>(", warmup, steps,
             ("GB/s", decode_bytes(DEC["B"], DEC["Hq"], DEC["Hkv"], DEC["L"], DEC["d"]),
              PEAK_HBM_GBS)),
            ("decode", "fa::fa_decode_combine_few_kernel<16>(", warmup, steps, None),
            ("fp8_fwd", "fa::fa_fwd_fp8_kernel<128, false>(", fp8_warm, fp8_steps,
             ("TFLOP/s", flops, PEAK_FP8_TFLOPS)),
            ("bwd", "fa::fa_bwd_dq_kernel<fa::FP16, 128, false, false>(", BWD_WARMUP, bwd_steps,
             None),
            ("bwd", "fa::fa_bwd_dkdv_kernel<fa::FP16, 128, false, false>(", BWD_WARMUP, bwd_steps,
             None),
            ("varlen_fwd", "fa::fa_fwd_kernel<fa::FP16, 128, false, true>(", VARLEN_WARMUP,
             varlen_steps, None),
            ("paged_decode", "fa::fa_decode_split_kernel<fa::BF16x16, 128, true, 4, 2>(", PAGED_WARMUP,
             paged_steps, ("GB/s", decode_bytes(DEC["B"], DEC["Hq"], DEC["Hkv"], DEC["L"],
                                                  DEC["d"]), PEAK_HBM_GBS))]
    out = []
    for leg, prefix, skip, take, work in legs:
        hits = sorted(t for name, ts in launches.items()
                      if name.startswith(prefix) or name.startswith("void " + prefix) for t in ts)
        timed = [(e - b) / 1e3 for b, e in hits[skip:skip + take]]
        if not timed:
            continue
        rec = {"leg": leg, "kernel": prefix[:-1], "launches_in_trace": len(hits),
               "skipped": skip, "timed": len(timed), "avg_us": round(st.mean(timed), 2),
               "median_us": round(st.median(timed), 2), "min_us": round(min(timed), 2),
               "max_us": round(max(timed), 2)}
        if work is not None:
            unit, amount, peak = work
            rate = amount / (rec["avg_us"] * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
            rec.update({"achieved": round(rate, 2), "unit": unit, "peak": peak,
                        "frac": round(rate / peak, 4)})
            if unit == "TFLOP/s" and peak == PEAK_MFMA_TFLOPS:
                rec["frac_of_2500"] = round(rate / 2500.0, 4)
        out.append(rec)
    return out


def ceilings(mfma_ms=10.0, launches=10):
    """What the chip sustains on each bound resource doing nothing else
    (libfa_ceiling.so): 32x32x16 16-bit MFMAs in four independent chains on
    two waves per SIMD, with N(0,1) operands (the attention inputs' values)
    and with zero operands, the 16x16x32 16-bit and the FP8 products on
    N(0,1)-like operands; and a 4 GiB stream of 16-byte loads, one
    contiguous chunk per workgroup, with the decode kernel's non-temporal
    policy and with the default one.  HIP events on the launch stream; the
    GPU's clock and power sampled during each timed loop.  One JSON line."""
    import ctypes
    import torch
    from flashattention_attention_fa_amd import synth

    path = os.path.join(ROOT, "flashattention_attention_fa_amd", "libfa_ceiling.so")
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.fa_ceiling_mfma.argtypes = [P, P, I, I, I, P]
    lib.fa_ceiling_read.argtypes = [P, ctypes.c_size_t, P, I, I, P]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(call, n, window_s=3.0):
        """Average time of n calls; the calls then go on, untimed, until the
        clock/power window has lasted window_s seconds."""
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sampler = ClockPowerSampler(dev)
        with sampler:
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(n):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            while time.perf_counter() - t0 < window_s:
                for _ in range(8):
                    call()
                torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, sampler.summary()

    out = {"ceilings": "MI355X achievable throughput, one resource at a time", "mfma": [],
           "hbm_read": []}
    wg = 512                                   # two 4-wave workgroups per CU
    res = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    for dtype, shape, data in (("fp16", "32x32x16", "N(0,1)"), ("bf16", "32x32x16", "N(0,1)"),
                               ("fp16", "32x32x16", "zeros"), ("fp16", "16x16x32", "N(0,1)"),
                               ("bf16", "16x16x32", "N(0,1)"), ("fp8", "32x32x64", "8 N(0,1) in E4M3")):
        if dtype == "fp8":     # the FP8 leg's inputs: amp 8, i.e. 8 * N(0,1) rounded to E4M3
            ops = synth.fp8_inputs(1, 1, wg * 256, 64, seed=9000, device=dev)[0]
        else:
            ops = synth.normal((wg * 256 * 16,), 9000, dtype, dev)
        if data == "zeros":
            ops.zero_()
        small = shape == "16x16x32"
        code = {"bf16": 3 if small else 0, "fp16": 4 if small else 1, "fp8": 2}[dtype]
        flops_per_iter = wg * 4 * 4 * (131072.0 if dtype == "fp8" else 16384.0 if small else 32768.0)
        peak = PEAK_FP8_TFLOPS if dtype == "fp8" else PEAK_MFMA_TFLOPS
        probe = 2000
        ms, _ = timed(lambda: lib.fa_ceiling_mfma(ctypes.c_void_p(ops.data_ptr()),
                                                  ctypes.c_void_p(res.data_ptr()), wg, probe,
                                                  code, sp), 2, window_s=0.0)
        iters = max(100, int(probe * mfma_ms / max(ms, 1e-3)))
        ms, smi = timed(lambda: lib.fa_ceiling_mfma(ctypes.c_void_p(ops.data_ptr()),
                                                    ctypes.c_void_p(res.data_ptr()), wg, iters,
                                                    code, sp), launches)
        tf = flops_per_iter * iters / (ms * 1e-3) / 1e12
        kname = "fa_ceiling_mfma_fp8_kernel" if dtype == "fp8" else \
            f"fa_ceiling_mfma{'16' if small else ''}_kernel<{dtype.upper()}>"
        out["mfma"].append({"kernel": kname, "dtype": dtype, "shape": shape,
                            "operands": data, "iters": iters, "avg_launch_ms": round(ms, 4),
                            "achieved": round(tf, 1), "unit": "TFLOP/s",
                            "peak": peak, "frac": round(tf / peak, 4),
                            "clock_power": smi})
        print(f"ceiling mfma {dtype} {shape} {data}: {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    # LDS: two 4-wave workgroups per CU, 8 reads per lane per iteration.
    lib.fa_ceiling_lds.argtypes = [P, I, I, I, P]
    out["lds_read"] = []
    lds_res = torch.empty(wg * 256, dtype=torch.int32, device=dev)
    for mode, what, per_lane in ((0, "ds_read_b128, 256 contiguous bytes per 16 lanes", 128),
                                 (1, "ds_read_b64_tr_b16 (transposing)", 64)):
        probe = 2000
        ms, _ = timed(lambda: lib.fa_ceiling_lds(ctypes.c_void_p(lds_res.data_ptr()), wg, probe,
                                                 mode, sp), 2, window_s=0.0)
        iters = max(100, int(probe * mfma_ms / max(ms, 1e-3)))
        ms, smi = timed(lambda: lib.fa_ceiling_lds(ctypes.c_void_p(lds_res.data_ptr()), wg, iters,
                                                   mode, sp), launches)
        nb = wg * 256 * per_lane * iters
        bps = nb / (ms * 1e-3)
        clk = smi.get("sclk_mhz", {}).get("median") if isinstance(smi, dict) else None
        out["lds_read"].append({"kernel": f"fa_ceiling_lds_kernel<{mode}>", "read": what,
                                "iters": iters, "avg_launch_ms": round(ms, 4),
                                "achieved": round(bps / 1e12, 2), "unit": "TB/s",
                                "bytes_per_clock_per_cu": round(bps / (256 * clk * 1e6), 1) if clk else None,
                                "clock_power": smi})
        print(f"ceiling lds mode {mode}: {bps / 1e12:.2f} TB/s", file=sys.stderr, flush=True)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.view(torch.int32).fill_(0x3c003c00)
    for wgs in (1024, 4096):
        chk = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        for nt in (1, 0):
            ms, smi = timed(lambda: lib.fa_ceiling_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                                        ctypes.c_void_p(chk.data_ptr()), wgs, nt,
                                                        sp), 20)
            gbs = nbytes / (ms * 1e-3) / 1e9
            out["hbm_read"].append({"kernel": f"fa_ceiling_read_kernel<{'true' if nt else 'false'}>",
                                    "policy": "non-temporal (sc0 nt)" if nt else "default",
                                    "workgroups": wgs, "bytes": nbytes,
                                    "avg_launch_us": round(ms * 1e3, 2), "achieved": round(gbs, 1),
                                    "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                    "frac": round(gbs / PEAK_HBM_GBS, 4), "clock_power": smi})
            print(f"ceiling read wg={wgs} nt={nt}: {gbs:.1f} GB/s", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


# Kernels whose HBM traffic profiles/traffic.json records: key, demangled
# name prefix, and the sources whose digest the record carries.
TRAFFIC_KERNELS = {
    "fa_fwd_kernel": ("fa::fa_fwd_kernel<fa::FP16, 128, false, false>(", ("fa_fwd.hip", "fa_device.hpp")),
    "fa_fwd_fp8_kernel": ("fa::fa_fwd_fp8_kernel<128, false>(", ("fa_fwd_fp8.hip", "fa_device.hpp")),
    "fa_bwd_dq_kernel": ("fa::fa_bwd_dq_kernel<fa::FP16, 128, false, false>(", ("fa_bwd.hip", "fa_device.hpp")),
    "fa_bwd_dkdv_kernel": ("fa::fa_bwd_dkdv_kernel<fa::FP16, 128, false, false>(", ("fa_bwd.hip", "fa_device.hpp")),
    "fa_decode_split_kernel": ("fa::fa_decode_split_kernel<fa::BF16x16, 128, false, 1, 4>(",
                               ("fa_decode.hip", "fa_device.hpp")),
    "fa_fwd_varlen_kernel": ("fa::fa_fwd_kernel<fa::FP16, 128, false, true>(", ("fa_fwd.hip", "fa_device.hpp")),
    "fa_decode_paged_split_kernel": ("fa::fa_decode_split_kernel<fa::BF16x16, 128, true, 4, 2>(",
                                     ("fa_decode.hip", "fa_device.hpp")),
}


def counter_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_path=None):
    """HBM bytes per launch of each kernel of TRAFFIC_KERNELS from rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch, summed over the
    counter's instances), each scaled by what the same counter reads for the
    --calibrate-copy run's 1 GiB device copy.  Prints one JSON line per
    kernel; with out_path, also writes them as the traffic record bench.py
    reads (keyed by kernel, with the digest of its sources)."""
    import csv
    import glob
    import statistics as st
    csv.field_size_limit(1 << 30)

    def per_dispatch(d):
        tot = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (r["Kernel_Name"], r["Dispatch_Id"])
                    tot[key] = tot.get(key, 0.0) + float(r["Counter_Value"])
        return tot

    def copy_kib(d):
        # the device copy is the only dispatch reading or writing a full GiB
        return max(per_dispatch(d).values())

    scale_f = (1 << 20) / copy_kib(copy_fetch_dir)     # bytes of the copy / KiB read
    scale_w = (1 << 20) / copy_kib(copy_write_dir)
    fetch, write = per_dispatch(fetch_dir), per_dispatch(write_dir)
    record = {}
    for key, (prefix, sources) in TRAFFIC_KERNELS.items():
        match = lambda name: name.startswith(prefix) or name.startswith("void " + prefix)
        fk = [v for (n, _), v in fetch.items() if match(n)]
        wk = [v for (n, _), v in write.items() if match(n)]
        if not fk or not wk:
            continue
        fb = st.median(fk) * 1024 * scale_f
        wb = st.median(wk) * 1024 * scale_w
        record[key] = {"kernel": prefix[:-1], "source_digest": source_digest(*sources),
                       "hbm_bytes_per_launch": int(round(fb + wb)),
                       "fetch_bytes_per_launch": int(round(fb)),
                       "write_bytes_per_launch": int(round(wb)),
                       "fetch_kib_raw_median": st.median(fk), "write_kib_raw_median": st.median(wk),
                       "dispatches": [len(fk), len(wk)],
                       "fetch_scale": scale_f, "write_scale": scale_w}
        print(json.dumps(dict(record[key], name=key)))
    if out_path:
        with open(out_path, "w") as f:
            json.dump(record, f, indent=1)
            f.write("\n")


def counter_table(dirs):
    """Median per dispatch of every counter that rocprofv3 --pmc runs of this
    script recorded (output directories `dirs`), for each kernel of
    TRAFFIC_KERNELS; one JSON line per kernel."""
    import csv
    import glob
    import statistics as st
    csv.field_size_limit(1 << 30)
    vals, dur = {}, {}
    for n, d in enumerate(dirs):
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (r["Kernel_Name"], r["Dispatch_Id"], r["Counter_Name"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
                    dur[(r["Kernel_Name"], n, r["Dispatch_Id"])] = \
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    for name, (prefix, _) in TRAFFIC_KERNELS.items():
        match = lambda k: k.startswith(prefix) or k.startswith("void " + prefix)
        per = {}
        for (kname, _, ctr), v in vals.items():
            if match(kname):
                per.setdefault(ctr, []).append(v)
        times = [t for (kname, _, _), t in dur.items() if match(kname)]
        if times:
            per["time_us"] = times
        if per:
            print(json.dumps({"name": name, "kernel": prefix[:-1],
                              "dispatches": max(len(v) for c, v in per.items() if c != "time_us"),
                              **{c: st.median(v) for c, v in sorted(per.items())}}))


def cpu_baseline(seconds_target=15.0):
    """The fp64 oracle on a bounded sample of forward rows of the benchmark
    shape, on this host's cores."""
    import numpy as np
    from flashattention_attention_fa_amd import synth
    from oracle import oracle as oracle_mod

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    threads = int(os.environ["OMP_NUM_THREADS"])
    B, H, N, d = FWD["B"], FWD["H"], FWD["N"], FWD["d"]
    # the oracle only reads the heads the sampled rows touch: 4 heads of batch 0
    q, k, v = synth.fwd_inputs(1, 4, N, d, FWD["dtype"], seed=FWD["seed"], device="cpu")
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    orc = oracle_mod.get()
    scale = 1 / math.sqrt(d)
    per_row = 4.0 * N * d
    n = max(threads * 4, 32)
    rows = synth.sample_rows(1, 4, N, n, seed=7)
    t0 = time.perf_counter()
    orc.attention_rows(qb, kb, vb, FWD["dtype"], rows, False, scale)
    dt = time.perf_counter() - t0
    n2 = int(min(1 * N * 4, max(n, n * seconds_target / max(dt, 1e-3))))
    rows = synth.sample_rows(1, 4, N, n2, seed=8)
    t0 = time.perf_counter()
    orc.attention_rows(qb, kb, vb, FWD["dtype"], rows, False, scale)
    dt = time.perf_counter() - t0
    rate = n2 * per_row / dt
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n2} random query rows of the forward benchmark shape (each against all "
                      f"{N} keys, d={d}, fp64), {dt:.1f} s; full problem extrapolated "
                      f"{fwd_flops(B, H, N, d, False) / rate:.0f} s",
            "cpu": platform.processor() or platform.machine()}


def time_fp8(fa, synth, stream, steps, warmup):
    """fa_fwd_fp8 on the forward shape with E4M3 inputs (amp 8, descale 1/8):
    average launch time from HIP events on the launch stream."""
    import torch
    c = FWD
    q, k, v, ds = synth.fp8_inputs(c["B"], c["H"], c["N"], c["d"], seed=c["seed"],
                                   device=stream.device)
    o = torch.empty((c["B"], c["H"], c["N"], c["d"]), dtype=torch.float32, device=stream.device)
    lse = torch.empty((c["B"], c["H"], c["N"]), dtype=torch.float32, device=stream.device)
    kw = dict(q_descale=ds, k_descale=ds, v_descale=ds, causal=c["causal"],
              scale=1 / math.sqrt(c["d"]), out=o, lse=lse, stream=stream)
    for _ in range(warmup):
        fa.fwd_fp8(q, k, v, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fa.fwd_fp8(q, k, v, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = fwd_flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
    tf = flops / (ms * 1e-3) / 1e12
    digest = source_digest("fa_fwd_fp8.hip", "fa_device.hpp")
    return {"kernel": "fa_fwd_fp8_kernel", "bound": "mfma", "dtype": "fp8 e4m3",
            "workload": f"attention forward B{c['B']} H{c['H']} N{c['N']} d{c['d']} fp8 e4m3 "
                        f"non-causal, per-tensor descale",
            "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_FP8_TFLOPS, 4), "avg_launch_ms": round(ms, 4),
            "steps": steps, "traffic": load_traffic("fa_fwd_fp8_kernel", digest),
            "source_digest": digest}


def time_bwd(fa, synth, stream, steps, warmup):
    """fa_bwd on the forward shape (o and lse from one fa_fwd): average call
    time from HIP events on the launch stream."""
    import torch
    c = FWD
    q, k, v, do = synth.bwd_inputs(c["B"], c["H"], c["N"], c["d"], c["dtype"], seed=c["seed"],
                                   device=stream.device)
    scale = 1 / math.sqrt(c["d"])
    o, lse = fa.fwd(q, k, v, causal=c["causal"], scale=scale, stream=stream)
    grads = [torch.empty_like(o) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_bytes(c["B"], c["H"], c["N"]), dtype=torch.uint8,
                     device=stream.device)
    kw = dict(causal=c["causal"], scale=scale, dq=grads[0], dk=grads[1], dv=grads[2],
              workspace=ws, stream=stream)
    for _ in range(warmup):
        fa.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fa.bwd(q, k, v, o, lse, do, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.5 * fwd_flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
    tf = flops / (ms * 1e-3) / 1e12
    digest = source_digest("fa_bwd.hip", "fa_device.hpp")
    return {"kernels": "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel", "bound": "mfma",
            "dtype": c["dtype"],
            "workload": f"attention backward B{c['B']} H{c['H']} N{c['N']} d{c['d']} "
                        f"{c['dtype']} non-causal",
            "achieved": round(tf, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_MFMA_TFLOPS, 4), "avg_call_ms": round(ms, 4),
            "algorithmic_flops_per_call": flops, "steps": steps,
            "traffic": {kern: load_traffic(kern, digest)
                        for kern in ("fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel")},
            "source_digest": digest}


def time_varlen(fa, synth, stream, steps, warmup):
    """fa_fwd_varlen on a packed [T, H, d] batch of mixed lengths: average
    launch time from HIP events on the launch stream.  FLOPs are the sum of
    each sequence's own 4*H*L^2*d."""
    import torch
    c = synth.VARLEN_BENCH
    T = sum(c["lens"])
    q, k, v, cu = synth.varlen_inputs(c["lens"], c["H"], c["d"], c["dtype"], seed=c["seed"],
                                      device=stream.device)
    o = torch.empty((T, c["H"], c["d"]), dtype=torch.float32, device=stream.device)
    lse = torch.empty((c["H"], T), dtype=torch.float32, device=stream.device)
    kw = dict(causal=c["causal"], scale=1 / math.sqrt(c["d"]), out=o, lse=lse, stream=stream)
    for _ in range(warmup):
        fa.fwd_varlen(q, k, v, cu, max(c["lens"]), **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fa.fwd_varlen(q, k, v, cu, max(c["lens"]), **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = sum(fwd_flops(1, c["H"], L, c["d"], c["causal"]) for L in c["lens"])
    tf = flops / (ms * 1e-3) / 1e12
    digest = source_digest("fa_fwd.hip", "fa_device.hpp")
    return {"kernel": "fa_fwd_kernel (VARLEN)", "bound": "mfma", "dtype": c["dtype"],
            "workload": f"attention forward, packed batch of {len(c['lens'])} sequences "
                        f"(lengths {'/'.join(str(L) for L in c['lens'])}, {T} tokens) "
                        f"H{c['H']} d{c['d']} {c['dtype']} "
                        f"{'causal' if c['causal'] else 'non-causal'}",
            "achieved": round(tf, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_MFMA_TFLOPS, 4), "avg_launch_ms": round(ms, 4),
            "algorithmic_flops_per_launch": flops, "steps": steps,
            "traffic": load_traffic("fa_fwd_varlen_kernel", digest), "source_digest": digest}


def time_paged(fa, synth, stream, steps, warmup):
    """fa_decode_paged on the decode shape, caches in pages of c["page"]
    tokens ([num_pages, page, Hkv, d] pools) in shuffled order: average call
    time from HIP events on the launch stream, rotating among KV_COPIES
    input sets (seeds seed + i) as the dense decode does."""
    import torch
    c = synth.PAGED_BENCH
    B, P = c["B"], c["page"]
    pools = [synth.paged_decode_inputs(B, c["Hq"], c["Hkv"], c["L"], c["d"], P, c["dtype"],
                                       seed=c["seed"] + i, device=stream.device)
             for i in range(KV_COPIES)]
    o = torch.empty((B, c["Hq"], c["d"]), dtype=torch.float32, device=stream.device)
    lse = torch.empty((B, c["Hq"]), dtype=torch.float32, device=stream.device)
    ws = torch.empty(fa.decode_workspace_bytes(B, c["Hq"], c["d"], c["nsplit"]), dtype=torch.uint8,
                     device=stream.device)

    def call(i):
        q, kp, vp, table, seq = pools[i % KV_COPIES]
        fa.decode_paged(q, kp, vp, table, seq, nsplit=c["nsplit"], out=o, lse=lse, workspace=ws,
                        stream=stream)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = decode_bytes(B, c["Hq"], c["Hkv"], c["L"], c["d"])
    gbs = nbytes / (ms * 1e-3) / 1e9
    digest = source_digest("fa_decode.hip", "fa_device.hpp")
    return {"kernels": "fa_decode_split_kernel (PAGED) + fa_decode_combine_few_kernel<16>", "bound": "hbm",
            "dtype": c["dtype"],
            "workload": f"paged split-KV decode B{B} Hq{c['Hq']} Hkv{c['Hkv']} L{c['L']} "
                        f"d{c['d']} {c['dtype']} nsplit{c['nsplit']}, {P}-token pages, "
                        f"shuffled block tables",
            "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_call_us": round(ms * 1e3, 2),
            "algorithmic_bytes_per_call": nbytes, "steps": steps,
            "kv_cache_copies_rotated": KV_COPIES,
            "traffic": load_traffic("fa_decode_paged_split_kernel", digest),
            "source_digest": digest}


def cpu_baseline_all_configs(oracle_seconds=3.0, full_tensor=False):
    """The CPU-baseline leg for every workload of synth.CONFIGS (the tiny
    case, the forward benchmark shape, the key-scaled causal shape, the 128k
    causal prefill and the split-KV decode) and of the two variable-length
    bench legs (synth.VARLEN_BENCH, synth.PAGED_BENCH): GPU time from HIP events on the
    launch stream beside the oracle timed on the host, on the whole problem
    (tiny, decode) or on a bounded sample of rows (the three large forwards,
    extrapolated to the whole problem by its flop rate), and the error of
    the GPU result on the oracle's rows.  One JSON line per workload.  With
    full_tensor, FULL_TENSOR_CONFIG is also checked on every row of the same
    GPU result (its line gains "parity_full_tensor").  As in
    cpu_baseline(), the oracle only serves as the baseline and the checker
    here; the GPU results come from the library alone."""
    import numpy as np
    import torch
    import flashattention_attention_fa_amd as fa
    from flashattention_attention_fa_amd import synth
    from oracle import oracle as oracle_mod

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    threads = int(os.environ["OMP_NUM_THREADS"])
    orc = oracle_mod.get()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def gpu_ms(fn, warmup, steps):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def err(o, ro, lse, rl):
        o, ro = np.asarray(o, np.float64), np.asarray(ro, np.float64)
        return {"max_abs": float(np.abs(o - ro).max()),
                "rel_l2": float(np.linalg.norm(o - ro) / np.linalg.norm(ro)),
                "lse_max_abs": float(np.abs(np.asarray(lse, np.float64) - rl).max())}

    for name, c in synth.CONFIGS.items():
        print(f"config {name}", file=sys.stderr, flush=True)
        if c["kind"] == "decode":
            B, Hq, Hkv, L, d = c["B"], c["Hq"], c["Hkv"], c["L"], c["d"]
            ins = [synth.decode_inputs(B, Hq, Hkv, L, d, c["dtype"], seed=c["seed"] + i, device=dev)
                   for i in range(KV_COPIES)]
            o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
            lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
            ws = torch.empty(fa.decode_workspace_bytes(B, Hq, d, c["nsplit"]), dtype=torch.uint8,
                             device=dev)
            call = lambda i: fa.decode(*ins[i % KV_COPIES], nsplit=c["nsplit"], out=o, lse=lse,
                                       workspace=ws, stream=stream)
            ms = gpu_ms(call, 5, 40)
            call(0)
            torch.cuda.synchronize()
            q, kc, vc = ins[0]
            t0 = time.perf_counter()
            ro, rl = orc.decode(synth.to_bits(q), synth.to_bits(kc), synth.to_bits(vc), c["dtype"])
            odt = time.perf_counter() - t0
            flops = 4.0 * B * Hq * L * d
            nbytes = decode_bytes(B, Hq, Hkv, L, d)
            rec = {"config": name, "shape": f"decode B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} {c['dtype']} "
                                              f"nsplit{c['nsplit']}",
                   "gpu_us": round(ms * 1e3, 2), "value": round(nbytes / ms / 1e6, 1), "unit": "GB/s",
                   "roofline_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                   "oracle": {"what": "whole problem", "seconds": round(odt, 2),
                              "gflops_fp64": round(flops / odt / 1e9, 2), "cores": threads},
                   "speedup_vs_oracle": round(odt / (ms / 1e3)),
                   "parity": err(o.cpu().numpy(), ro, lse.cpu().numpy(), rl)}
            del ins
        else:
            B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
            q, k, v = synth.fwd_inputs(B, H, N, d, c["dtype"], seed=c["seed"], device=dev,
                                       krow_scale=c.get("krow_scale"))
            o = torch.empty(q.shape, dtype=torch.float32, device=dev)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            scale = 1 / math.sqrt(d)
            call = lambda i: fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse,
                                    stream=stream)
            flops = fwd_flops(B, H, N, d, causal)
            steps = max(3, min(50, int(2e3 / max(flops / 1e12, 1e-3))))
            ms = gpu_ms(call, 3, steps)
            qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
            if B * H * N <= 4096:
                rows = synth.sample_rows(B, H, N, B * H * N, seed=1)
                what = "whole problem"
            else:
                # rows visible keys: N (non-causal) or i + 1; size the sample to the time budget
                per_row = 4.0 * d * (N if not causal else N / 2)
                n = int(max(64, min(20000, oracle_seconds * 5e9 / per_row)))
                rows = synth.sample_rows(B, H, N, n, seed=c["seed"])
                what = f"{len(rows)} random rows (whole problem extrapolated by flop rate)"
            row_flops = float(np.sum(4.0 * d * (rows[:, 2] + 1 if causal else np.full(len(rows), N))))
            t0 = time.perf_counter()
            ro, rl = orc.attention_rows(qb, kb, vb, c["dtype"], rows, causal, scale)
            odt = time.perf_counter() - t0
            r = torch.as_tensor(rows, device=dev)
            og = o[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy()
            lg = lse[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy()
            rate = row_flops / odt
            full_s = flops / rate
            rec = {"config": name, "shape": f"fwd B{B} H{H} N{N} d{d} {c['dtype']} "
                                              f"{'causal' if causal else 'non-causal'}"
                                              + (" K rows x U[0.5,4]" if c.get("krow_scale") else ""),
                   "gpu_ms": round(ms, 4), "value": round(flops / ms / 1e9, 1), "unit": "TFLOP/s",
                   "roofline_frac": round(flops / ms / 1e9 / PEAK_MFMA_TFLOPS, 4),
                   "oracle": {"what": what, "rows": int(len(rows)), "seconds": round(odt, 2),
                              "gflops_fp64": round(rate / 1e9, 2), "cores": threads,
                              "whole_problem_seconds": round(full_s, 1)},
                   "speedup_vs_oracle": round(full_s / (ms / 1e3)),
                   "parity": err(og, ro, lg, rl)}
            if full_tensor and name == FULL_TENSOR_CONFIG:
                pairs = [(b, h) for b in range(B) for h in range(H)]
                rec["parity_full_tensor"] = check_heads(orc, qb, kb, vb, o.cpu().numpy(),
                                                        lse.cpu().numpy(), c["dtype"], causal,
                                                        scale, pairs)
            del q, k, v, o, lse
        torch.cuda.empty_cache()
        print(json.dumps(rec), flush=True)

    # The variable-length bench legs: the packed batch (sampled rows of every
    # sequence, oracle run on that sequence alone) and the paged decode
    # (whole problem, keys gathered through the block table on the host).
    c = synth.VARLEN_BENCH
    print("config varlen_bench", file=sys.stderr, flush=True)
    lens, H, d = c["lens"], c["H"], c["d"]
    q, k, v, cu = synth.varlen_inputs(lens, H, d, c["dtype"], seed=c["seed"], device=dev)
    T = sum(lens)
    o = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(d)
    call = lambda i: fa.fwd_varlen(q, k, v, cu, max(lens), causal=c["causal"], scale=scale, out=o,
                                   lse=lse, stream=stream)
    flops = sum(fwd_flops(1, H, L, d, c["causal"]) for L in lens)
    ms = gpu_ms(call, 3, 20)
    call(0)
    torch.cuda.synchronize()
    og_all, lg_all = o.cpu().numpy(), lse.cpu().numpy()
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    del q, k, v, o, lse
    got_o, got_l, ref_o, ref_l = [], [], [], []
    row_flops, odt, start = 0.0, 0.0, 0
    for n, L in enumerate(lens):
        nrow = int(max(16, oracle_seconds * 5e9 / len(lens) / (4.0 * d * L)))
        rows = synth.sample_rows(1, H, L, nrow, seed=c["seed"] + n)
        sl = slice(start, start + L)
        per = [np.ascontiguousarray(x[sl].transpose(1, 0, 2)[None]) for x in (qb, kb, vb)]
        t0 = time.perf_counter()
        ro, rl = orc.attention_rows(*per, c["dtype"], rows, c["causal"], scale)
        odt += time.perf_counter() - t0
        row_flops += 4.0 * d * L * len(rows)
        got_o.append(og_all[start + rows[:, 2], rows[:, 1]])
        got_l.append(lg_all[rows[:, 1], start + rows[:, 2]])
        ref_o.append(ro)
        ref_l.append(rl)
        start += L
    rate = row_flops / odt
    nrows = sum(len(x) for x in got_o)
    rec = {"config": "varlen_bench", "shape": f"fwd varlen {len(lens)} packed sequences "
                                             f"{'/'.join(map(str, lens))} ({T} tokens) H{H} d{d} "
                                             f"{c['dtype']} {'causal' if c['causal'] else 'non-causal'}",
           "gpu_ms": round(ms, 4), "value": round(flops / ms / 1e9, 1), "unit": "TFLOP/s",
           "roofline_frac": round(flops / ms / 1e9 / PEAK_MFMA_TFLOPS, 4),
           "oracle": {"what": f"{nrows} random rows (whole problem extrapolated by flop rate)",
                      "rows": nrows, "seconds": round(odt, 2), "gflops_fp64": round(rate / 1e9, 2),
                      "cores": threads, "whole_problem_seconds": round(flops / rate, 1)},
           "speedup_vs_oracle": round(flops / rate / (ms / 1e3)),
           "parity": err(np.concatenate(got_o), np.concatenate(ref_o), np.concatenate(got_l),
                         np.concatenate(ref_l))}
    del qb, kb, vb
    torch.cuda.empty_cache()
    print(json.dumps(rec), flush=True)

    c = synth.PAGED_BENCH
    print("config paged_bench", file=sys.stderr, flush=True)
    B, Hq, Hkv, L, d, P = c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["page"]
    ins = [synth.paged_decode_inputs(B, Hq, Hkv, L, d, P, c["dtype"], seed=c["seed"] + i, device=dev)
           for i in range(KV_COPIES)]
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(B, Hq, d, c["nsplit"]), dtype=torch.uint8, device=dev)
    call = lambda i: fa.decode_paged(*ins[i % KV_COPIES], nsplit=c["nsplit"], out=o, lse=lse,
                                     workspace=ws, stream=stream)
    ms = gpu_ms(call, 5, 40)
    call(0)
    torch.cuda.synchronize()
    q, kp, vp, table, _ = ins[0]
    qb, kpb, vpb, tb = synth.to_bits(q), synth.to_bits(kp), synth.to_bits(vp), table.cpu().numpy()
    del ins
    idx = np.arange(L)
    odt = 0.0
    ro, rl = np.zeros((B, Hq, d)), np.zeros((B, Hq))
    for b in range(B):
        kc, vc = (np.ascontiguousarray(x[tb[b, idx // P], idx % P].transpose(1, 0, 2)[None])
                  for x in (kpb, vpb))
        t0 = time.perf_counter()
        rob, rlb = orc.decode(qb[b:b + 1], kc, vc, c["dtype"])
        odt += time.perf_counter() - t0
        ro[b], rl[b] = rob[0], rlb[0]
    nbytes = decode_bytes(B, Hq, Hkv, L, d)
    rec = {"config": "paged_bench", "shape": f"paged decode B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} "
                                            f"{c['dtype']} nsplit{c['nsplit']} page{P}",
           "gpu_us": round(ms * 1e3, 2), "value": round(nbytes / ms / 1e6, 1), "unit": "GB/s",
           "roofline_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
           "oracle": {"what": "whole problem (keys gathered through the block table first, "
                              "not timed)", "seconds": round(odt, 2),
                      "gflops_fp64": round(4.0 * B * Hq * L * d / odt / 1e9, 2), "cores": threads},
           "speedup_vs_oracle": round(odt / (ms / 1e3)),
           "parity": err(o.cpu().numpy(), ro, lse.cpu().numpy(), rl)}
    print(json.dumps(rec), flush=True)


# The workload whose rows are the most peaked (a few key rows scaled up to
# 4x dominate them): the one --all-configs --full-tensor checks on every row.
FULL_TENSOR_CONFIG = "causal_b4h32n16k_kscaled"


def check_heads(orc, qb, kb, vb, og, lg, dtype, causal, scale, pairs):
    """Errors of a forward result (og [B,H,N,d], lg [B,H,N], on the host)
    against the oracle on every row of the (b, h) heads in `pairs`, one
    oracle call per head, with a progress line per head on stderr."""
    import numpy as np
    N = og.shape[2]
    sq_err = sq_ref = 0.0
    max_abs = lse_abs = worst_row = 0.0
    worst_at = None
    odt = 0.0
    for n, (b, h) in enumerate(pairs):
        rows = np.stack([np.full(N, b), np.full(N, h), np.arange(N)], 1).astype(np.int64)
        t0 = time.perf_counter()
        ro, rl = orc.attention_rows(qb, kb, vb, dtype, rows, causal, scale)
        odt += time.perf_counter() - t0
        diff = og[b, h].astype(np.float64) - ro
        sq_err += float(np.sum(diff * diff))
        sq_ref += float(np.sum(ro * ro))
        head_abs = float(np.abs(diff).max())
        row_rel = np.linalg.norm(diff, axis=1) / np.maximum(np.linalg.norm(ro, axis=1), 1e-300)
        i = int(np.argmax(row_rel))
        if row_rel[i] > worst_row:
            worst_row, worst_at = float(row_rel[i]), (int(b), int(h), i)
        max_abs = max(max_abs, head_abs)
        lse_abs = max(lse_abs, float(np.abs(lg[b, h].astype(np.float64) - rl).max()))
        print(f"head {n + 1}/{len(pairs)} (b={b}, h={h}): max-abs {head_abs:.3e}, so far "
              f"{max_abs:.3e}, lse {lse_abs:.3e}, oracle {odt:.0f} s", file=sys.stderr, flush=True)
    return {"heads_checked": len(pairs), "rows_checked": len(pairs) * N,
            "max_abs": max_abs, "rel_l2": math.sqrt(sq_err / sq_ref), "lse_max_abs": lse_abs,
            "worst_row_rel_l2": worst_row, "worst_row": worst_at, "oracle_seconds": round(odt, 1)}


def full_check(name, heads=None):
    """Check one forward workload of synth.CONFIGS against the oracle on
    every row of every head (or of the first `heads` heads): one fa_fwd
    call on the GPU, O and lse copied to the host, then the oracle head by
    head (one progress line per head on stderr).  Prints one JSON line with
    the errors over all checked rows and the worst single row."""
    import numpy as np
    import torch
    import flashattention_attention_fa_amd as fa
    from flashattention_attention_fa_amd import synth
    from oracle import oracle as oracle_mod

    c = synth.CONFIGS[name]
    if c["kind"] != "fwd":
        raise SystemExit(f"--full-check takes a forward workload, not {name}")
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    threads = int(os.environ["OMP_NUM_THREADS"])
    orc = oracle_mod.get()
    dev = torch.device("cuda:0")
    B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
    print(f"full check {name}: fa_fwd B{B} H{H} N{N} d{d} {c['dtype']} causal={causal}",
          file=sys.stderr, flush=True)
    q, k, v = synth.fwd_inputs(B, H, N, d, c["dtype"], seed=c["seed"], device=dev,
                               krow_scale=c.get("krow_scale"))
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    pairs = [(b, h) for b in range(B) for h in range(H)][:heads]
    res = check_heads(orc, qb, kb, vb, og, lg, c["dtype"], causal, scale, pairs)
    rec = {"full_check": name,
           "shape": f"fwd B{B} H{H} N{N} d{d} {c['dtype']} "
                    f"{'causal' if causal else 'non-causal'}"
                    + (" K rows x U[0.5,4]" if c.get("krow_scale") else ""),
           **{k: v for k, v in res.items() if k != "oracle_seconds"},
           "bars": {"max_abs": 2e-2, "rel_l2": 5e-3, "lse_max_abs": 1e-3},
           "oracle": {"seconds": res["oracle_seconds"], "cores": threads}}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8-steps", type=int, default=50,
                    help="timed calls of the FP8 forward on the forward shape (0 skips it)")
    ap.add_argument("--bwd-steps", type=int, default=20,
                    help="timed fa_bwd calls for the bwd object (0: skip)")
    ap.add_argument("--varlen-steps", type=int, default=20,
                    help="timed fa_fwd_varlen calls for the varlen_fwd object (0: skip)")
    ap.add_argument("--paged-steps", type=int, default=50,
                    help="timed fa_decode_paged calls for the paged_decode object (0: skip)")
    ap.add_argument("--only", choices=["fwd", "decode", "fp8", "bwd", "varlen", "paged"],
                    default=None,
                    help="run one kernel's leg only, with its --steps/--warmup or leg-step counts "
                         "(for counter passes); prints that leg's object")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, 3 times (the reference "
                         "kernel that scales the HBM byte counters)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the step: every workload (tiny, forward benchmark shape, "
                         "key-scaled causal, 128k causal, decode, varlen batch, paged decode) "
                         "with its oracle time and parity on the oracle's rows, one JSON line "
                         "each")
    ap.add_argument("--full-tensor", action="store_true",
                    help=f"with --all-configs: also check {FULL_TENSOR_CONFIG} on every row "
                         "(about 12 minutes of oracle time on 16 host threads)")
    ap.add_argument("--full-check", metavar="WORKLOAD", default=None,
                    help="instead of the step: check one forward workload (e.g. "
                         "causal_b4h32n16k_kscaled) against the oracle on every row")
    ap.add_argument("--heads", type=int, default=None,
                    help="with --full-check: check only the first HEADS heads")
    ap.add_argument("--trace-summary", nargs="+", metavar="CSV", default=None,
                    help="instead of running: per-kernel times over the timed launches only, from "
                         "rocprofv3 kernel-trace CSVs of a run of this script with the same "
                         "--steps/--warmup/leg-step options (one JSON line per kernel)")
    ap.add_argument("--counter-summary", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="instead of running: HBM bytes per launch per kernel from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE output directories of this script and of "
                         "its --calibrate-copy run")
    ap.add_argument("--counter-table", nargs="+", default=None, metavar="DIR",
                    help="instead of running: median per dispatch of every counter of rocprofv3 "
                         "--pmc output directories, per kernel")
    ap.add_argument("--write-traffic", default=None, metavar="JSON",
                    help="with --counter-summary: also write the per-kernel record to JSON")
    ap.add_argument("--sustain-s", type=float, default=3.0,
                    help="keep running the step (untimed) until this many seconds after the "
                         "timed steps began, so the clock/power readings cover several refreshes")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the step: the achievable MFMA and HBM-read ceilings "
                         "(libfa_ceiling.so), with clock and power")
    args = ap.parse_args()
    if args.counter_table:
        counter_table(args.counter_table)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary, out_path=args.write_traffic)
        return
    if args.trace_summary:
        for rec in trace_summary(args.trace_summary, args.warmup, args.steps, args.fp8_steps,
                                 args.bwd_steps, args.varlen_steps, args.paged_steps):
            print(json.dumps(rec))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.all_configs:
        cpu_baseline_all_configs(full_tensor=args.full_tensor)
        return
    if args.full_check:
        full_check(args.full_check, args.heads)
        return
    if args.ceilings:
        ceilings()
        return

    import torch
    import flashattention_attention_fa_amd as fa
    from flashattention_attention_fa_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.calibrate_copy:
        n = 1 << 28                        # 2^28 fp32 = 1 GiB
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 3}))
        return

    legs = {"fp8": lambda: time_fp8(fa, synth, stream, args.fp8_steps,
                                    max(FP8_MIN_WARMUP, args.warmup // 2)),
            "bwd": lambda: time_bwd(fa, synth, stream, args.bwd_steps, BWD_WARMUP),
            "varlen": lambda: time_varlen(fa, synth, stream, args.varlen_steps, VARLEN_WARMUP),
            "paged": lambda: time_paged(fa, synth, stream, args.paged_steps, PAGED_WARMUP)}
    if args.only in legs:
        print(json.dumps({args.only: legs[args.only]()}), flush=True)
        return

    c = FWD
    q, k, v = synth.fwd_inputs(c["B"], c["H"], c["N"], c["d"], c["dtype"], seed=c["seed"], device=dev)
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(c["d"])

    dcfg = DEC
    caches = []
    for i in range(KV_COPIES):
        dq, dk, dv = synth.decode_inputs(dcfg["B"], dcfg["Hq"], dcfg["Hkv"], dcfg["L"], dcfg["d"],
                                         dcfg["dtype"], seed=dcfg["seed"] + i, device=dev)
        caches.append((dq, dk, dv))
    do = torch.empty(caches[0][0].shape, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(dcfg["B"], dcfg["Hq"], dcfg["d"], dcfg["nsplit"]),
                     dtype=torch.uint8, device=dev)
    dlse = torch.empty(caches[0][0].shape[:2], dtype=torch.float32, device=dev)

    run_fwd = args.only in (None, "fwd")
    run_dec = args.only in (None, "decode")

    def step(i, mid=None):
        if run_fwd:
            fa.fwd(q, k, v, causal=c["causal"], scale=scale, out=o, lse=lse, stream=stream)
        if mid is not None:
            mid.record(stream)
        if run_dec:
            dq, dk, dv = caches[i % KV_COPIES]
            fa.decode(dq, dk, dv, nsplit=dcfg["nsplit"], out=do, lse=dlse, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    sampler = ClockPowerSampler(dev)
    with sampler:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(i, ev[i][1])
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # The clock and power readings refresh about once a second: keep the
        # same step running (untimed) until the window holds a few of them.
        n_extra = 0
        while time.perf_counter() - t0 < args.sustain_s:
            for _ in range(4):
                step(n_extra)
                n_extra += 1
            torch.cuda.synchronize()
    fwd_calls = [a.elapsed_time(b) for a, b, _ in ev]
    dec_calls = [b.elapsed_time(e) for _, b, e in ev]
    fwd_ms = sum(fwd_calls) / args.steps
    dec_ms = sum(dec_calls) / args.steps
    step_ms = sum(a.elapsed_time(e) for a, _, e in ev) / args.steps
    median = lambda xs: sorted(xs)[len(xs) // 2] if len(xs) % 2 else \
        0.5 * (sorted(xs)[len(xs) // 2 - 1] + sorted(xs)[len(xs) // 2])

    flops = fwd_flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
    tflops = flops / (fwd_ms * 1e-3) / 1e12 if run_fwd else 0.0
    dbytes = decode_bytes(dcfg["B"], dcfg["Hq"], dcfg["Hkv"], dcfg["L"], dcfg["d"])
    gbs = dbytes / (dec_ms * 1e-3) / 1e9 if run_dec else 0.0
    fwd_digest = source_digest("fa_fwd.hip", "fa_device.hpp")
    dec_digest = source_digest("fa_decode.hip", "fa_device.hpp")
    fwd_traffic = load_traffic("fa_fwd_kernel", fwd_digest)
    dec_traffic = load_traffic("fa_decode_split_kernel", dec_digest)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["dtype"],
        "data": "synthetic (seeded N(0,1) tensors, inputs resident in HBM)",
        "config": {
            "workload": f"attention forward B{c['B']} H{c['H']} N{c['N']} d{c['d']} {c['dtype']} "
                        f"non-causal, plus split-KV decode B{dcfg['B']} Hq{dcfg['Hq']} "
                        f"Hkv{dcfg['Hkv']} L{dcfg['L']} d{dcfg['d']} {dcfg['dtype']} "
                        f"nsplit{dcfg['nsplit']}",
            "fwd": {k_: c[k_] for k_ in ("B", "H", "N", "d", "dtype", "causal")},
            "decode": {k_: dcfg[k_] for k_ in ("B", "Hq", "Hkv", "L", "d", "dtype", "nsplit")},
        },
        "roofline": {
            "kernel": "fa_fwd_kernel",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
            "traffic": fwd_traffic,
            "traffic_source": TRAFFIC_SOURCE,
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": fwd_bytes(c["B"], c["H"], c["N"], c["d"]),
            "avg_launch_ms": round(fwd_ms, 4),
            "median_launch_ms": round(median(fwd_calls), 4),
            "source_digest": fwd_digest,
        },
        "decode": {
            "kernels": "fa_decode_split_kernel + fa_decode_combine_few_kernel<16>",
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": dec_traffic, "traffic_source": TRAFFIC_SOURCE,
            "algorithmic_bytes_per_call": dbytes,
            "avg_call_us": round(dec_ms * 1e3, 2),
            "median_call_us": round(median(dec_calls) * 1e3, 2),
            "kv_cache_copies_rotated": KV_COPIES,
            "source_digest": dec_digest,
        },
        "wall_s_timed": round(wall, 3),
        "clock_power": dict(sampler.summary(),
                            window=f"the {args.steps} timed steps, then {n_extra} more untimed "
                                   f"steps up to {args.sustain_s:g} s"),
        "device": torch.cuda.get_device_name(dev),
    }
    for key, leg, n in (("fp8_fwd", "fp8", args.fp8_steps), ("bwd", "bwd", args.bwd_steps),
                        ("varlen_fwd", "varlen", args.varlen_steps),
                        ("paged_decode", "paged", args.paged_steps)):
        if n > 0 and args.only is None:
            out[key] = legs[leg]()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
