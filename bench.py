"""Benchmark of MLA tree-verify attention on one MI355X.

A step is one verify_attn call (partial kernel + combine kernel) over one
batch of synthetic input resident in HBM. The headline workload is the
long-context H=8 configuration at 65k context (one sequence, prefix 65,536,
64-node draft tree, page_size=1 scattered slots in a 131,072-slot pool). The
H=64 point at 65k (the ragged 4-sequence batch whose sequences run 4k..200k)
and the other 65k points are reported beside it.

Timing: every step reads its own replica of (pool, q) from a rotation whose
total KV bytes exceed twice the 256 MB Infinity Cache, so repeats are served
from HBM; the K timed steps are recorded in one HIP graph, which is replayed
untimed until its time has settled and then replayed 10 times (3 for the
extras), each replay bracketed by synchronisation and timed with HIP events on
the launch stream; the reported time per call is the median replay over K.
The partial kernel is also timed on its own the same way: that duration gives
the roofline figure. A library bf16 GEMM is timed in the same run on operands
drawn like the workload's and on zeros (`mfma_reference`): the matrix cores
sustain a lower rate on toggling data than the published peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 << 20
KV_ROW_BYTES = 576 * 2
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
FLOPS_PER_KEY_ROW = 2 * 576 + 2 * 512  # QK^T + PV per (KV row, query row)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_partial_c4a.json")
KERNEL_SRC = os.path.join(ROOT, "mla_tree_verify_latent_amd", "csrc", "verify_attn.hip")

WORKLOAD_TEXT = {
    "c4a_long_scattered": "long-context verify: H=8, 1 sequence, prefix 65536, T=64, page_size=1 "
                          "scattered in a 131072-slot bf16 [slots, 576] pool",
    "c4b_long_contiguous": "long-context verify, defragmented: same values, page_size=64 contiguous",
    "c5_ragged": "ragged batched long-context: H=64, 4 sequences, prefixes 4096/23552/65536/200704, "
                 "T=64 each, shared 300000-slot pool, scattered",
    "e1_h64_65k": "full-head 65k: H=64, 1 sequence, prefix 65536, T=64, scattered",
    "e2_h8_t9_65k": "production shape: H=8, 1 sequence, prefix 65536, T=9, scattered",
    "e2_h8_t9_65k_contiguous": "production shape, defragmented: same rows at slots 0, 1, 2, ...",
    "e2_h8_t9_65k_paged64": "production shape in 64-row pages: same rows, 64 consecutive slots per page, "
                            "pages in random order",
    "c2_tp_share": "TP-share decode verify: H=8, prefix 4096, T=32, 65536-slot pool",
    "c3_full_head": "full-head verify: H=64, prefix 16384, T=32, 131072-slot pool",
    "f4_long_f32": "fp32 inputs: H=8, 1 sequence, prefix 65536, T=64, scattered, binary32 q and "
                   "[131072, 576] KV pool, fp32 output",
}


def algorithmic_bytes(wl) -> int:
    """Bytes one call must move at least: each referenced KV row and its slot index once,
    q and out once, the tree and the sequence lengths once."""
    rows = wl.total_kv
    elt = wl.kv_pool.itemsize  # 2 (bf16) or 4 (fp32)
    return (rows * (576 * elt + 4) + wl.B * wl.T * wl.H * (576 + 512) * elt
            + wl.B * wl.T * 4 + wl.B * 4)


def algorithmic_flops(wl) -> int:
    """2*(576 + 512) flops per (KV row, query row) pair of the same sequence."""
    return int(wl.seq_lens.astype(np.int64).sum()) * wl.H * wl.T * FLOPS_PER_KEY_ROW


def kernel_source_digest() -> str:
    """Hash of the kernel source's code: comments removed and whitespace runs
    collapsed (string and character literals kept as written), so that counter
    files stay matched to the code they were taken on across comment edits."""
    text = open(KERNEL_SRC, encoding="utf-8").read()
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    code = " ".join("".join(out).split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


class Bench:
    """Device copies of one workload, R replicas, and graph-timed runs."""

    def __init__(self, wl, replicas: int, nsplit: int = 0):
        import torch
        import mla_tree_verify_latent_amd as mtv
        from synthetic.device import to_device, params_of
        self.torch, self.mtv, self.wl = torch, mtv, wl
        base = to_device(wl)
        self.params = params_of(wl, nsplit)
        wsize = (mtv.verify_attn_f32_workspace_size if wl.f32 else mtv.verify_attn_workspace_size)(self.params)
        self.ws = torch.empty(wsize, dtype=torch.uint8, device="cuda")
        self.reps = []
        for r in range(replicas):
            d = dict(base)
            if r:
                d["kv_pool"] = base["kv_pool"].clone()
                d["q"] = base["q"].clone()
            self.reps.append(d)
        self.out = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.float32 if wl.f32 else torch.bfloat16,
                               device="cuda")
        self.kv_new = torch.zeros((wl.B, wl.T, 576), dtype=torch.bfloat16, device="cuda")
        self.kv_dst = None
        torch.cuda.synchronize()

    def call(self, r, stage="full"):
        d = self.reps[r % len(self.reps)]
        if self.wl.f32:  # the fp32-input path has one entry point (partial + combine)
            assert stage == "full", stage
            self.mtv.verify_attn_f32(d["q"], d["kv_pool"], d["slot_idx"], d["seq_lens"],
                                     d["tree_parent"], self.out, self.ws, self.params)
        elif stage == "full":
            self.mtv.verify_attn(d["q"], d["kv_pool"], d["slot_idx"], d["seq_lens"],
                                 d["tree_parent"], self.out, self.ws, self.params)
        elif stage == "partial":
            self.mtv.verify_attn_partial(d["q"], d["kv_pool"], d["slot_idx"], d["seq_lens"],
                                         d["tree_parent"], self.ws, self.params)
        elif stage == "combine":
            self.mtv.verify_attn_combine(d["seq_lens"], self.out, self.ws, self.params)
        elif stage == "append":  # draft-row KV append (writes the tree rows of the pool)
            self.mtv.verify_attn_append_kv(self.kv_new, d["slot_idx"], d["seq_lens"], d["kv_pool"],
                                           self.params)
        elif stage == "compact":  # KV defragmentation: every referenced row into one contiguous run
            if self.kv_dst is None:
                self.kv_dst = self.torch.empty((self.wl.total_kv, 576), dtype=self.torch.bfloat16,
                                               device="cuda")
            self.mtv.verify_attn_compact_kv(d["kv_pool"], d["slot_idx"], self.kv_dst, self.params)

    def graph(self, n, stage):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.call(0, stage)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                self.call(i, stage)
        torch.cuda.synchronize()
        return g

    def _replay_ms(self, g):
        torch = self.torch
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    def time_graph(self, steps, warmup, stage="full", repeats=3):
        """Median over `repeats` replays of a graph of `steps` calls; ms per call.
        Before the timed replays the same graph is replayed untimed until its time
        has settled (the clocks ramp up under sustained load): at least 5 replays
        and 0.2 s, until the last three agree within 3% (at most 2 s)."""
        torch = self.torch
        if warmup:
            gw = self.graph(warmup, stage)
            gw.replay()
            torch.cuda.synchronize()
        g = self.graph(steps, stage)
        settle = []
        while sum(settle) < 2000.0:
            settle.append(self._replay_ms(g))
            last = settle[-3:]
            if len(settle) >= 5 and sum(settle) >= 200.0 and max(last) <= 1.03 * min(last):
                break
        self.settle_replays = len(settle)
        times = [self._replay_ms(g) / steps for _ in range(repeats)]
        return statistics.median(times), times


def replicas_for(wl) -> int:
    return max(1, math.ceil(2 * MALL_BYTES / max(1, wl.kv_bytes())))


# Workloads timed on one replica only (the whole working set stays in the
# Infinity Cache): the 0.3 MB tiny configuration, reported as MALL-warm.
WARM_ONLY = ("c1_tiny",)


def measure(name, steps, warmup, nsplit=0, stages=("full", "partial"), repeats=3):
    from synthetic import inputs
    wl = inputs.config(name)
    R = 1 if name in WARM_ONLY else replicas_for(wl)
    b = Bench(wl, R, nsplit)
    res = {"workload": name, "replicas": R,
           "plan": None if wl.f32 else b.mtv.verify_attn_plan(b.params)}
    for st in stages:
        ms, all_ms = b.time_graph(steps, warmup, st, repeats=repeats)
        res[f"{st}_ms"] = ms
        res[f"{st}_ms_repeats"] = all_ms
        res[f"{st}_settle_replays"] = b.settle_replays
    if R == 1:
        res["full_ms_mall_warm"] = res["full_ms"]
    else:
        warm = Bench(wl, 1, nsplit)
        res["full_ms_mall_warm"], _ = warm.time_graph(steps, warmup, "full")
        del warm
    res["bytes"] = algorithmic_bytes(wl)
    res["flops"] = algorithmic_flops(wl)
    res["wl"] = wl
    del b
    return res


def binding_time_s(r) -> float:
    """Time of a call at its binding roof: its bytes at peak HBM or its flops at
    peak bf16 MFMA, whichever is longer."""
    return max(r["bytes"] / (HBM_PEAK_GBS * 1e9), r["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))


def cpu_baseline_1thread(names=("c1_tiny", "c2_tp_share")):
    """The oracle on one host thread, whole calls of the two small configurations
    (seconds per call, median of 3)."""
    import oracle
    from synthetic import inputs
    orc = oracle.load()
    res = {}
    for name in names:
        wl = inputs.config(name)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            orc.run(wl, nthreads=1)
            times.append(time.perf_counter() - t0)
        res[name] = {"s_per_call": round(statistics.median(times), 4),
                     "gbs": round(algorithmic_bytes(wl) / statistics.median(times) / 1e9, 4)}
    return res


def gemm_reference(n=8192, reps=20):
    """Sustained bf16 matrix rate of the library GEMM (torch.matmul, n x n x n, fp32
    accumulate) on operands drawn like the workload's (one factor N(0,1), the other
    N(0,1)*0.1) and on all-zero operands, and the fp32 GEMM's rate on the former. The matrix cores draw more power on toggling
    data, so the rate they sustain depends on the values; this is the reference for how
    far the partial kernel is from what the chip sustains on such data."""
    import torch
    torch.backends.cuda.matmul.allow_tf32 = False  # the fp32 GEMM stays in binary32
    g = torch.Generator(device="cuda").manual_seed(7)
    res = {"kind": f"torch.matmul bf16 {n}x{n}x{n}, fp32 accumulate (and the same in fp32)", "reps": reps}
    for label in ("normal", "zeros", "f32_normal"):
        dt = torch.float32 if label == "f32_normal" else torch.bfloat16
        if label == "zeros":
            a = torch.zeros((n, n), device="cuda", dtype=dt)
            b = torch.zeros((n, n), device="cuda", dtype=dt)
        else:
            a = torch.randn((n, n), generator=g, device="cuda", dtype=torch.float32).mul_(0.1).to(dt)
            b = torch.randn((n, n), generator=g, device="cuda", dtype=torch.float32).to(dt)
        c = torch.empty((n, n), device="cuda", dtype=dt)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        res[f"tflops_{label}_operands"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, repeats=5):
    """The oracle (fp64 C, OpenMP) on whole calls of the same workload."""
    import oracle
    from synthetic import inputs
    wl = inputs.config(name)
    orc = oracle.load()
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        orc.run(wl)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": algorithmic_bytes(wl) / t / 1e9, "unit": "GB/s", "cores": orc.num_threads(),
        "kind": "oracle", "cpu_model": model, "nproc": os.cpu_count(),
        "sample": f"{name}: whole call ({wl.B * wl.T * wl.H} output rows), median of {repeats} "
                  f"calls, {t:.2f} s per call ({sum(times):.1f} s of oracle time in all)",
        "s_per_call": t,
    }


def traffic_from_counters(partial_ms):
    """HBM bytes per partial launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters (scaled by a copy-kernel calibration), if they were taken on this source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    c = json.load(open(COUNTERS_FILE))
    if c.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    return c["hbm_bytes_per_launch"]


def counter_value(key):
    """One figure of the committed counter summary, if taken on this source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    c = json.load(open(COUNTERS_FILE))
    if c.get("kernel_source_sha256_16") != kernel_source_digest() or key not in c:
        return None
    return round(c[key], 4)


def _read_counter_csv(path, kernel_substr):
    import csv
    vals = {}
    for r in csv.DictReader(open(path)):
        if kernel_substr in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def summarize(args):
    """Write committed summaries from rocprofv3 CSV output (see --summarize)."""
    out = {}
    if args.kernel_stats:
        import csv
        rows = list(csv.DictReader(open(args.kernel_stats)))
        lines = ["| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                         f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.1f}% |")
        print("\n".join(lines))
        return
    # FETCH_SIZE / WRITE_SIZE of the partial kernel, scaled by a 1 GiB copy's counters.
    fetch, nf = _read_counter_csv(args.fetch, "verify_attn_partial")
    write, nw = _read_counter_csv(args.write, "verify_attn_partial")
    cfetch, _ = _read_counter_csv(args.copy_fetch, "copyBuffer")
    cwrite, _ = _read_counter_csv(args.copy_write, "copyBuffer")
    copy_bytes = float(1 << 30)
    f_scale = copy_bytes / (cfetch["FETCH_SIZE"] * 1024)
    w_scale = copy_bytes / (cwrite["WRITE_SIZE"] * 1024)
    fb = fetch["FETCH_SIZE"] * 1024 * f_scale
    wb = write["WRITE_SIZE"] * 1024 * w_scale
    out = {
        "kernel": "verify_attn_partial_kernel", "workload": args.workload,
        "kernel_source_sha256_16": kernel_source_digest(),
        "fetch_kib_per_dispatch": fetch["FETCH_SIZE"], "write_kib_per_dispatch": write["WRITE_SIZE"],
        "dispatches": [nf.get("FETCH_SIZE"), nw.get("WRITE_SIZE")],
        "copy_calibration": {"bytes_read_and_written": copy_bytes,
                             "fetch_kib": cfetch["FETCH_SIZE"], "write_kib": cwrite["WRITE_SIZE"],
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "hbm_read_bytes_per_launch": fb, "hbm_write_bytes_per_launch": wb,
        "hbm_bytes_per_launch": fb + wb,
    }
    if args.sq:
        # SQ counters of the same kernel: MFMA busy cycles (summed over the 1,024
        # SIMDs) over GRBM_GUI_ACTIVE (summed over the 8 XCDs) -> busy fraction.
        # GRBM_GUI_ACTIVE counts the profiled dispatch's window, not shader cycles of
        # the traced kernel time, so this share is approximate.
        sq, _ = _read_counter_csv(args.sq, "verify_attn_partial")
        out["mfma_busy_frac"] = sq["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (sq["GRBM_GUI_ACTIVE"] / 8)
        out["lds_bank_conflict_cycles"] = sq["SQ_LDS_BANK_CONFLICT"]
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4a_long_scattered")
    ap.add_argument("--extras", default="c4b_long_contiguous,e2_h8_t9_65k,e2_h8_t9_65k_contiguous,"
                                        "e2_h8_t9_65k_paged64,e1_h64_65k,c5_ragged,c1_tiny,c2_tp_share,"
                                        "c3_full_head",
                    help="comma-separated extra workloads reported beside the headline ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-f32", action="store_true", help="skip the fp32-input variant line")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the library bf16 GEMM timed as the sustained-matrix-rate reference")
    ap.add_argument("--stage", default=None, choices=[None, "full", "partial", "combine", "append", "compact", "copy"],
                    help="profiling aid: only run K calls of one stage of the headline workload; "
                         "'copy' runs K device-to-device copies of 1 GiB (counter calibration)")
    ap.add_argument("--summarize", action="store_true",
                    help="no GPU: print a summary of rocprofv3 CSV output (--kernel-stats, or "
                         "--fetch/--write/--copy-fetch/--copy-write counter files)")
    ap.add_argument("--kernel-stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--sq", help="SQ/GRBM counter file of the same kernel (MFMA busy)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verify path has no multi-GPU mode "
              "(heads, sequences or KV positions would shard across GPUs, with one exchange of the "
              "split partials before the combine for sharded KV positions).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import mla_tree_verify_latent_amd as mtv
    mtv.load_library()

    if args.stage == "copy":
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"stage": "copy", "bytes_read_per_copy": src.numel() * 4,
                          "bytes_written_per_copy": dst.numel() * 4, "copies": args.steps}))
        return
    if args.stage:
        from synthetic import inputs
        wl = inputs.config(args.workload)
        b = Bench(wl, replicas_for(wl))
        for i in range(args.warmup + args.steps):
            b.call(i, args.stage)
        torch.cuda.synchronize()
        print(json.dumps({"stage": args.stage, "workload": args.workload, "calls": args.warmup + args.steps}))
        return

    head = measure(args.workload, args.steps, args.warmup, stages=("full", "partial", "append", "compact"),
                   repeats=10)
    ms = head["full_ms"]
    gbs = head["bytes"] / (ms * 1e-3) / 1e9
    part_ms = head["partial_ms"]
    part_tflops = head["flops"] / (part_ms * 1e-3) / 1e12
    extras = {}
    for name in [e for e in args.extras.split(",") if e]:
        r = measure(name, args.steps, args.warmup)
        extras[name] = {
            "workload": WORKLOAD_TEXT.get(name, name),
            "ms_per_call": round(r["full_ms"], 5),
            "calls_per_s": round(1e3 / r["full_ms"], 1),
            "hbm_gbs": round(r["bytes"] / (r["full_ms"] * 1e-3) / 1e9, 1),
            "hbm_frac": round(r["bytes"] / (r["full_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "partial_ms": round(r["partial_ms"], 5),
            "partial_mfma_tflops": round(r["flops"] / (r["partial_ms"] * 1e-3) / 1e12, 1),
            "mfma_frac": round(r["flops"] / (r["partial_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "ms_per_call_mall_warm": round(r["full_ms_mall_warm"], 5),
            # whole call against its binding roof: max(bytes at 8 TB/s, flops at 2.5 PFLOP/s) / time
            "binding_roof_frac": round(binding_time_s(r) / (r["full_ms"] * 1e-3), 4),
            "replicas": r["replicas"],
            "timing": "MALL-warm (one replica)" if r["replicas"] == 1 else "HBM (replica rotation > 2x MALL)",
        }
        torch.cuda.empty_cache()

    f32 = None
    if not args.no_f32:
        r = measure("f4_long_f32", args.steps, args.warmup, stages=("full",))
        f32 = {
            "workload": WORKLOAD_TEXT["f4_long_f32"],
            "ms_per_call": round(r["full_ms"], 5),
            "calls_per_s": round(1e3 / r["full_ms"], 1),
            "hbm_gbs": round(r["bytes"] / (r["full_ms"] * 1e-3) / 1e9, 1),
            "mfma_f32_tflops": round(r["flops"] / (r["full_ms"] * 1e-3) / 1e12, 1),
            "mfma_f32_frac": round(r["flops"] / (r["full_ms"] * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS, 4),
            "replicas": r["replicas"],
        }
        torch.cuda.empty_cache()

    line = {
        "metric": "achieved HBM GB/s (% of peak) + verify calls/sec at 65k ctx, H=8 and H=64",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT[args.workload],
            "name": args.workload,
            "num_seqs": head["wl"].B, "heads": head["wl"].H, "tree_nodes": head["wl"].T,
            "prefix": head["wl"].prefixes, "pool_slots": head["wl"].pool_slots,
            "plan": head["plan"], "replicas": head["replicas"],
        },
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        # whole call against the binding roof: max(bytes at 8 TB/s, flops at 2.5 PFLOP/s) / time
        "binding_roof_frac": round(binding_time_s(head) / (ms * 1e-3), 4),
        "settle_replays": head["full_settle_replays"],
        "ms_per_step_repeats": [round(x, 5) for x in head["full_ms_repeats"]],
        # spread of the per-call time over the 10 timed graph replays of K calls each
        "ms_per_step_p10_p90": [round(float(np.percentile(head["full_ms_repeats"], q)), 5) for q in (10, 90)],
        "partial_kernel_ms_p10_p90": [round(float(np.percentile(head["partial_ms_repeats"], q)), 5)
                                      for q in (10, 90)],
        "calls_per_s": round(1e3 / ms, 1),
        "ms_per_call_mall_warm": round(head["full_ms_mall_warm"], 5),
        "partial_kernel_ms": round(part_ms, 5),
        "combine_share": round(1.0 - part_ms / ms, 4),
        # measured HBM bytes of the partial kernel (rocprofv3 counters) over its live time
        "partial_hbm_gbs": (round(traffic_from_counters(part_ms) / (part_ms * 1e-3) / 1e9, 1)
                            if traffic_from_counters(part_ms) else None),
        "partial_mfma_busy": counter_value("mfma_busy_frac"),
        "roofline": {
            "bound": "mfma",
            "achieved": round(part_tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(part_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_from_counters(part_ms),
        },
        "extras": extras,
        # draft-row KV append on the same workload: B*T rows of 1,152 B read and written
        "append_kv": {
            "rows": head["wl"].B * head["wl"].T,
            "us_per_call": round(head["append_ms"] * 1e3, 2),
            "gbs": round(2 * KV_ROW_BYTES * head["wl"].B * head["wl"].T / (head["append_ms"] * 1e-3) / 1e9, 1),
        },
        # fp32-input variant (whole call, partial + combine) on the same shape in binary32
        "f32_variant": f32,
        # KV defragmentation on the same workload: total_kv rows of 1,152 B gathered and written
        "compact_kv": {
            "rows": head["wl"].total_kv,
            "us_per_call": round(head["compact_ms"] * 1e3, 2),
            "gbs": round(2 * KV_ROW_BYTES * head["wl"].total_kv / (head["compact_ms"] * 1e-3) / 1e9, 1),
        },
    }
    # the pages' own figures, on their hardware: orientation only, never a target
    line["pages_context"] = {
        "hardware": "RTX PRO 6000 Blackwell (sm_120), 1.8 TB/s HBM peak",
        "triton_verify_effective_gbs": 14,
        "own_flash_kernel_vs_naive": "1.7-4.2x (all 64 heads, up to 65k context)",
        "vectorized_bf16_gather": "1.3-1.8x",
        "end_to_end_decode_vs_triton_graph": "3.0x @4k, 4.3x @16k, 6.1x @65k (8 GPUs, whole model)",
    }
    if not args.no_gemm_reference:
        ref = gemm_reference()
        ref["partial_kernel_frac_of_normal"] = round(part_tflops / ref["tflops_normal_operands"], 4)
        if f32 is not None:
            f32["mfma_f32_frac_of_library_f32"] = round(f32["mfma_f32_tflops"] / ref["tflops_f32_normal_operands"], 4)
        line["mfma_reference"] = ref
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args.workload)
        line["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                for k, v in cb.items() if k != "s_per_call"}
        line["cpu_baseline_1thread"] = cpu_baseline_1thread()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
