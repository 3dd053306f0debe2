"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step = one full pass of the layer (router, top-K, dispatch, grouped
gate/up + SwiGLU, grouped down + weights, combine) over one batch of seeded
synthetic inputs already resident in HBM.  The default workload is the
Step-3.5-Flash decode batch (T=16 tokens: 4 sequences x (1 + 3 MTP drafts)),
the configuration the headline metric is quoted on; a prefill pass at
T=4096 is reported beside it (`prefill` object) because the metric names
both.  Prints ONE JSON line.

roofline: the dominant kernel (gate/up + SwiGLU) timed with HIP events that
the library records around it on its own stream, against its algorithmic
bytes (decode, HBM bound) or FLOPs (prefill).
cpu_baseline: the float64 CPU oracle timed on the host cores on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def _hip():
    """The HIP runtime already loaded in this process (the one torch and the
    library share)."""
    maps = open("/proc/self/maps").read()
    paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", maps)))
    lib = ctypes.CDLL(paths[0] if paths else "libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class StageTimer:
    """Per-step arrays of begin/end events for every library stage."""

    def __init__(self, hip, n_steps: int, n_stages: int):
        self.hip = hip
        self.n_stages = n_stages
        self.arrays = []
        for _ in range(n_steps):
            arr = (ctypes.c_void_p * (2 * n_stages))()
            for i in range(2 * n_stages):
                ev = ctypes.c_void_p()
                assert hip.hipEventCreate(ctypes.byref(ev)) == 0
                arr[i] = ev
            self.arrays.append(arr)

    def stage_ms(self):
        """Mean duration (ms) of each stage over the recorded steps; 0 for a
        stage the call does not run (its events were never recorded)."""
        out = []
        for s in range(self.n_stages):
            tot = 0.0
            for arr in self.arrays:
                ms = ctypes.c_float()
                if self.hip.hipEventElapsedTime(ctypes.byref(ms), arr[2 * s], arr[2 * s + 1]) != 0:
                    self.hip.hipGetLastError()   # leave no error for the next runtime call
                    tot = 0.0
                    break
                tot += ms.value
            out.append(tot / len(self.arrays))
        return out

    def close(self):
        for arr in self.arrays:
            for ev in arr:
                self.hip.hipEventDestroy(ev)


def _src_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CSRC = "sparse_moe_transformer_fp32_amd/csrc/"
# sources that define each measured kernel and its launch configuration
KERNEL_SOURCES = {
    "decode": [_CSRC + "expert_gemm.hip", _CSRC + "api.cpp", _CSRC + "smoe_internal.h"],
    "prefill": [_CSRC + "expert_gemm_lds.hip", _CSRC + "api.cpp", _CSRC + "smoe_internal.h"],
}
KERNEL_SOURCES["dense_decode"] = KERNEL_SOURCES["decode"]
KERNEL_SOURCES["long"] = KERNEL_SOURCES["skew"] = KERNEL_SOURCES["prefill"]
KERNEL_SOURCES["skew_mild"] = KERNEL_SOURCES["prefill"]


def _traffic(kernel_key: str):
    """HBM bytes per launch (fetch + write, calibrated) from the committed
    rocprofv3 counter record, or None when the kernel's sources changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    wl = kernel_key.split(":")[1]
    if not rec or rec.get("source_sha") != _src_sha(KERNEL_SOURCES[wl]):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- offline helpers
def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_stats(csv_path, out_path, command, trace_csv=None, regex="smoe"):
    """Short text summary of a rocprofv3 --stats kernel table; with the
    run's kernel trace, also per launch shape (kernel, grid), since one
    kernel serves several workloads of one run (e.g. the T=16 MoE layer and
    the dense FFN side measurement launch the same register-streaming GEMM)."""
    rows = [r for r in _read_csv(csv_path) if re.search(regex, r["Name"])]
    lines = [f"# rocprofv3 kernel statistics ({os.path.basename(csv_path)})",
             f"# command: {command}",
             f"# kernels matching /{regex}/; durations in microseconds",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}  {r['Name']}")
    if trace_csv:
        import collections
        groups = collections.defaultdict(list)
        for r in _read_csv(trace_csv):
            name = r.get("Kernel_Name", "")
            if not re.search(regex, name):
                continue
            try:   # grid sizes are in work-items per dimension
                n_wg = 1
                for ax in "XYZ":
                    n_wg *= int(r.get(f"Grid_Size_{ax}") or 1) // max(1, int(r.get(f"Workgroup_Size_{ax}") or 1))
            except ValueError:
                n_wg = "?"
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            groups[(name, n_wg)].append((t0, t1))
        lines += ["", f"# per launch shape, from the kernel trace ({os.path.basename(trace_csv)})",
                  f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'wgs':>7}  kernel"]
        seg_lines = []
        for (name, n_wg), ts in sorted(groups.items(),
                                       key=lambda kv: -sum(b - a for a, b in kv[1])):
            d = [(b - a) / 1e3 for a, b in ts]
            lines.append(f"{len(d):6d} {sum(d) / len(d):10.2f} {min(d):10.2f} {max(d):10.2f} "
                         f"{n_wg!s:>7}  {name}")
            # runs of dispatches separated by more than 1 ms without one
            # (phases of the run, e.g. the sizes of a probe sweep), listed
            # for kernels with at most 8 runs
            ts = sorted(ts)
            segs, cur = [], [ts[0]]
            for a, b in ts[1:]:
                if a - cur[-1][1] > 1_000_000:
                    segs.append(cur)
                    cur = []
                cur.append((a, b))
            segs.append(cur)
            if 1 < len(segs) <= 8:
                for i, sg in enumerate(segs):
                    dd = sorted((b - a) / 1e3 for a, b in sg)
                    seg_lines.append(f"{i:4d} {len(dd):6d} {dd[len(dd) // 2]:10.2f} {dd[0]:10.2f} "
                                     f"{dd[-1]:10.2f} {n_wg!s:>7}  {name}")
        if seg_lines:
            lines += ["", "# per run of dispatches (runs separated by more than 1 ms idle), in order",
                      f"{'run':>4} {'calls':>6} {'med_us':>10} {'min_us':>10} {'max_us':>10} {'wgs':>7}  kernel"]
            lines += seg_lines
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# the gate/up kernel each counter workload launches (decode: register-streaming;
# prefill: LDS-pipelined)
GATE_UP_KERNEL = {"decode": "void smoe::expert_gemm_kernel<0,",
                  "dense_decode": "smoe::dense_gate_up_x_kernel",
                  "prefill": "void smoe::expert_gemm_lds_kernel<0>",
                  "long": "void smoe::expert_gemm_lds_kernel<0>",
                  "skew": "void smoe::expert_gemm_lds_kernel<0>",
                  "skew_mild": "void smoe::expert_gemm_lds_kernel<0>"}


# the down kernel of each counter workload
DOWN_KERNEL = {"decode": "void smoe::expert_gemm_kernel<1,",
               "dense_decode": "void smoe::dense_down_kernel",
               "prefill": "void smoe::expert_gemm_lds_kernel<1>",
               "long": "void smoe::expert_gemm_lds_kernel<1>",
               "skew": "void smoe::expert_gemm_lds_kernel<1>",
               "skew_mild": "void smoe::expert_gemm_lds_kernel<1>"}


def write_traffic(pmc_root, commands):
    """From rocprofv3 --pmc runs laid out as <pmc_root>/<name>_<COUNTER>/
    run_counter_collection.csv (name = copy, and any of decode / prefill /
    long / skew present), compute the per-dispatch HBM bytes of every smoe
    kernel, scaled by what the same counters read for a plain 1 GiB device
    copy; write one summary per workload (profiles/hbm_bytes_<workload>.txt)
    and record the gate/up kernel's bytes in profiles/traffic.json (entries
    of workloads not in this run are kept)."""
    import collections
    def per_kernel(name, counter):
        agg = collections.defaultdict(list)
        for r in _read_csv(os.path.join(pmc_root, f"{name}_{counter}", "run_counter_collection.csv")):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}
    copy_bytes = 1 << 30
    cf = max(v for k, v in per_kernel("copy", "FETCH_SIZE").items() if "copy" in k.lower())
    cw = max(v for k, v in per_kernel("copy", "WRITE_SIZE").items() if "copy" in k.lower())
    f_fetch, f_write = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    out = json.load(open(tpath)) if os.path.exists(tpath) else {}
    head = [f"# HBM bytes per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB), scaled by",
            f"# a plain 1 GiB device copy: FETCH_SIZE read {cf:.0f} KiB -> factor {f_fetch:.4f};",
            f"# WRITE_SIZE read {cw:.0f} KiB -> factor {f_write:.4f}.", "# commands:"]
    head += [f"#   {c}" for c in commands]
    for wl in ("decode", "prefill", "long", "skew", "skew_mild", "dense_decode"):
        if not os.path.isdir(os.path.join(pmc_root, f"{wl}_FETCH_SIZE")):
            continue
        fe, wr = per_kernel(wl, "FETCH_SIZE"), per_kernel(wl, "WRITE_SIZE")
        text = list(head)
        for k in sorted(fe):
            if "smoe" not in k:
                continue
            b = fe[k] * 1024 * f_fetch + wr.get(k, 0.0) * 1024 * f_write
            text.append(f"{wl:8s} fetch {fe[k] * 1024 * f_fetch / 1e9:9.4f} GB  write "
                        f"{wr.get(k, 0.0) * 1024 * f_write / 1e9:9.4f} GB  {k}")
            for role, prefix in (("gate_up", GATE_UP_KERNEL[wl]), ("down", DOWN_KERNEL[wl])):
                if k.startswith(prefix):   # the workload's gate/up + SwiGLU, or its down
                    out[f"{role}:{wl}"] = {"kernel": k, "bytes_per_launch": int(b),
                                           "fetch_kib": fe[k], "write_kib": wr.get(k, 0.0),
                                           "fetch_factor": f_fetch, "write_factor": f_write,
                                           "source_sha": _src_sha(KERNEL_SOURCES[wl])}
        with open(os.path.join(ROOT, "profiles", f"hbm_bytes_gate_up_down_{wl}.txt"), "w") as f:
            f.write("\n".join(text) + "\n")
        print("\n".join(text))
    with open(tpath, "w") as f:
        json.dump(out, f, indent=1)


def summarize_lds(root, command):
    """From rocprofv3 --pmc runs <root>/<workload>/run_counter_collection.csv
    (workload = prefill, long) with the LDS and wait counters: the share of
    cycles the LDS is active and the waves wait on LDS or on any counter."""
    import collections
    lines = ["", "# Second pass (rocprofv3 --pmc, its own run per workload): LDS activity and wait cycles",
             f"#   {command}",
             "#   LDS_active = SQ_LDS_IDX_ACTIVE / (256 CUs x cycles); LDS_wait and any_wait = "
             "SQ_WAIT_INST_LDS and SQ_WAIT_ANY over SQ_WAVE_CYCLES",
             f"{'workload':9s} {'kernel':8s} {'LDS_active':>10s} {'LDS_wait':>9s} {'any_wait':>9s}"]
    for wl_name in ("prefill", "long"):
        disp = collections.defaultdict(dict)
        for r in _read_csv(os.path.join(root, wl_name, "run_counter_collection.csv")):
            disp[(r["Kernel_Name"], r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
        for tag, key in (("gate_up", "expert_gemm_lds_kernel<0>"), ("down", "expert_gemm_lds_kernel<1>")):
            ds = [d for (k, _), d in disp.items() if key in k]
            if not ds:
                continue
            m = {c: sum(d[c] for d in ds) / len(ds) for c in ds[0]}
            cycles = m["GRBM_GUI_ACTIVE"] / 8
            lines.append(f"{wl_name:9s} {tag:8s} {100 * m['SQ_LDS_IDX_ACTIVE'] / (256 * cycles):9.1f}% "
                         f"{100 * m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:8.1f}% "
                         f"{100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:8.1f}%")
    print("\n".join(lines))
    return lines


def summarize_mfma(root, command):
    """From rocprofv3 --pmc runs <root>/<workload>/run_counter_collection.csv
    (workload = prefill, long) over the LDS-pipelined GEMMs, the per-dispatch
    MFMA work, MFMA busy fraction, shader clock and LDS bank conflicts."""
    import collections
    from sparse_moe_transformer_fp32_amd.inputs import WORKLOADS
    lines = ["# MFMA and LDS counters of the LDS-pipelined grouped GEMMs (rocprofv3 --pmc, one pass per workload)",
             "# command (workload = prefill | long):", f"#   {command}",
             "# mean per dispatch. Derived columns:",
             "#   MFMA FLOP  = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (executed, including padded token rows);",
             "#   cycles     = GRBM_GUI_ACTIVE / 8 (the 8 XCDs each count); clock = cycles / kernel time;",
             "#   MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles).",
             "# The kernel times are the same run's dispatch timestamps.",
             f"{'workload':9s} {'kernel':8s} {'time_us':>8s} {'clock_GHz':>9s} {'MFMA_TFLOP':>10s} "
             f"{'alg_TFLOP':>9s} {'pad':>5s} {'MFMA_busy':>9s} {'LDS_bank_conf':>13s} {'waves':>7s}"]
    for wl_name in ("prefill", "long"):
        wl = WORKLOADS[wl_name]
        gu_alg = 2 * (wl.K * wl.T * 2 * wl.I * wl.H + wl.T * 2 * wl.Is * wl.H)
        disp = collections.defaultdict(dict)
        for r in _read_csv(os.path.join(root, wl_name, "run_counter_collection.csv")):
            d = disp[(r["Kernel_Name"], r["Dispatch_Id"])]
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for tag, key, alg in (("gate_up", "expert_gemm_lds_kernel<0>", gu_alg),
                              ("down", "expert_gemm_lds_kernel<1>", gu_alg / 2)):
            ds = [d for (k, _), d in disp.items() if key in k]
            if not ds:
                continue
            m = {c: sum(d[c] for d in ds) / len(ds) for c in ds[0]}
            cycles = m["GRBM_GUI_ACTIVE"] / 8
            t_us = m["_ns"] / 1e3
            flop = m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            lines.append(f"{wl_name:9s} {tag:8s} {t_us:8.1f} {cycles / (t_us * 1e3):9.2f} {flop / 1e12:10.3f} "
                         f"{alg / 1e12:9.3f} {flop / alg:5.2f} "
                         f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cycles):8.1f}% "
                         f"{m['SQ_LDS_BANK_CONFLICT']:13.0f} {m['SQ_WAVES']:7.0f}")
    print("\n".join(lines))
    return lines


def read_ceiling(gib: int = 4, reps: int = 10):
    """HBM read rate of one plain read of a `gib` GiB buffer (moe_read_probe,
    two workgroups per CU, 16-byte loads), ordinary and non-temporal: the best
    of three groups of `reps` reads timed with HIP events, after two untimed
    reads.  The practical ceiling of a weight stream, next to the nominal
    8 TB/s."""
    import torch
    from sparse_moe_transformer_fp32_amd import binding as B
    buf = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = {"bytes": gib << 30}
    for name, nt in (("ordinary", False), ("nontemporal", True)):
        for _ in range(2):
            B.read_probe(buf, sink, nt)
        best = None
        for _ in range(3):   # the best of three timed groups
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                B.read_probe(buf, sink, nt)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            best = ms if best is None else min(best, ms)
        out[name] = {"us_per_read": round(best * 1e3, 1),
                     "gbs": round((gib << 30) / (best * 1e-3) / 1e9, 1)}
    out["frac_of_8tbs"] = {k: round(out[k]["gbs"] / 8000.0, 3) for k in ("ordinary", "nontemporal")}
    return out


def mfma_ceiling(iters: int = 65536, reps: int = 5):
    """The bf16 matrix-core rate the chip sustains with no memory traffic
    (moe_mfma_probe: one 8-wave workgroup per CU, four independent
    32x32x16 MFMA chains per wave), the best of `reps` timed launches after
    two untimed ones, and the shader clock it ran at (the probe's s_memtime
    and 100 MHz s_memrealtime counts over its loop).  The practical ceiling
    of the grouped GEMMs' MFMA figures, next to the nominal 2.5 PF."""
    import torch
    from sparse_moe_transformer_fp32_amd import binding as B
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clocks = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    for _ in range(2):
        B.mfma_probe(iters, clocks, sink)
    best, clk = None, None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.mfma_probe(iters, clocks, sink)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        if best is None or ms < best:
            c = clocks.view(cus, 2).double().sum(0).tolist()
            best, clk = ms, c[0] / c[1] * 0.1   # GHz: shader ticks per 100 MHz tick
    flops = cus * 8 * iters * 4 * 32768
    tf = flops / (best * 1e-3) / 1e12
    return {"iters": iters, "ms": round(best, 4), "tflops": round(tf, 1),
            "frac_of_2500": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "clock_ghz": round(clk, 3),
            "frac_of_clock_peak": round(tf / (cus * 4 * 1024 * clk * 1e9 / 1e12), 4)}


def short_read_ceiling(mibs=(88, 176, 264), reps=40):
    """HBM read rate of short non-temporal reads (moe_read_probe), the sizes
    of the dense decode FFN's down weights, gate/up weights and whole layer,
    each read of a different buffer of a rotation of over 1 GiB, so that no
    read finds its data in the 256 MB last-level cache: the median of `reps`
    single reads timed with HIP events (the launch latency included), and
    the mean of `reps` reads issued back to back between one pair of events
    (as the dense FFN's two kernels run: each launch prepared while the
    previous read runs).  The floor of a kernel that streams that many bytes
    once."""
    import torch
    from sparse_moe_transformer_fp32_amd import binding as B
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = {}
    for mib in mibs:
        nb = mib << 20
        bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(1100 // mib + 2)]
        for i in range(3):
            B.read_probe(bufs[i], sink, True)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record()
            B.read_probe(bufs[i % len(bufs)], sink, True)
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            B.read_probe(bufs[i % len(bufs)], sink, True)
        b.record()
        torch.cuda.synchronize()
        ms_b2b = a.elapsed_time(b) / reps
        out[f"{mib}MiB"] = {"us_per_read": round(ms * 1e3, 1),
                            "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                            "frac_of_8tbs": round(nb / (ms * 1e-3) / 8e12, 3),
                            "us_per_read_back_to_back": round(ms_b2b * 1e3, 1),
                            "gbs_back_to_back": round(nb / (ms_b2b * 1e-3) / 1e9, 1),
                            "frac_of_8tbs_back_to_back": round(nb / (ms_b2b * 1e-3) / 8e12, 3)}
        del bufs
        torch.cuda.empty_cache()
    return out


def layer_work(wl, counts):
    """Algorithmic bytes and FLOPs of one layer call, and of its gate/up
    kernel, from the measured expert counts."""
    T, H, E, K, I, Is = wl.T, wl.H, wl.E, wl.K, wl.I, wl.Is
    n_act = int((counts > 0).sum())
    rows = T * K + (T if Is else 0)
    w_gu = (n_act * 2 * I * H + (2 * Is * H if Is else 0)) * 2
    w_dn = (n_act * H * I + (H * Is if Is else 0)) * 2
    gu_bytes = w_gu + T * H * 2 + (T * K * I + T * Is) * 2          # weights, x, h
    layer_bytes = w_gu + w_dn + E * H * 4 + E * 4 + 2 * T * H * 2    # weights, router, x, y
    gu_flops = 2 * (T * K * 2 * I * H + (T * 2 * Is * H if Is else 0))
    layer_flops = 2 * (T * K * 3 * I * H + (T * 3 * Is * H if Is else 0))
    router_flops = 2 * T * E * H
    return dict(n_active=n_act, rows=rows, gu_bytes=gu_bytes, layer_bytes=layer_bytes,
                gu_flops=gu_flops, layer_flops=layer_flops, router_flops=router_flops)


def run_layer_bench(wl_name, steps, warmup, device="cuda"):
    import torch
    from sparse_moe_transformer_fp32_amd import binding as B
    from sparse_moe_transformer_fp32_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[wl_name]
    inp = make_inputs(wl, device=device)
    layers = []
    for li, L in enumerate(inp.layers):
        layers.append(B.MoELayer(inp.router_ws[li], inp.router_bs[li], L.w_gate, L.w_up, L.w_down,
                                 L.ws_gate, L.ws_up, L.ws_down, K=wl.K, T_max=wl.T,
                                 route_scale=wl.route_scale, norm_topk=wl.norm_topk))
    T = wl.T
    x = inp.x
    routing = B.alloc_routing(T, wl.E, wl.K, device)
    nl = len(layers)
    y = torch.empty_like(x)
    chain = B.MoEChain(layers, eps=1e-6) if nl > 1 else None

    def step():
        if chain is None:
            layers[0].forward(x, y, routing)
        else:  # pre-norm residual stream through the chained layers
            chain.forward(x, routing_last=routing)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: the K steps exactly as a caller runs them -> value
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    gpu_ms = start.elapsed_time(stop) / steps
    # timed region 2: the same K steps with the library's per-stage HIP
    # events (recorded on the stream the kernels run on) -> kernel durations
    hip = _hip()
    timer = StageTimer(hip, steps, len(B.STAGES))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(steps):
        B.set_stage_events(timer.arrays[k])
        step()
    B.set_stage_events(None)
    torch.cuda.synchronize()
    inst_ms = (time.perf_counter() - t1) * 1e3 / steps
    stage_ms = timer.stage_ms()
    timer.close()
    # timed region 3: the same step captured once in a HIP graph and
    # replayed K times (the library allocates, clears and syncs nothing)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t2 = time.perf_counter()
    g0.record()
    for _ in range(steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_wall_ms = (time.perf_counter() - t2) * 1e3 / steps
    graph_ms = g0.elapsed_time(g1) / steps
    del graph
    counts = routing["counts"].cpu().numpy()
    return dict(wl=wl, inp=inp, layers=layers, routing=routing, counts=counts, wall_ms=wall_ms,
                gpu_ms=gpu_ms, inst_ms=inst_ms, stage_ms=dict(zip(B.STAGES, stage_ms)),
                n_layers=nl, graph_ms=graph_ms, graph_wall_ms=graph_wall_ms)


def run_dense_bench(name, steps, warmup, device="cuda"):
    """The model's dense FFN (moe_dense_ffn) on its synthetic workload:
    tokens/s, bf16 TFLOP/s and algorithmic GB/s of one call.  At decode the
    calls go to the model's three dense layers in turn (distinct weights,
    830 MB), so no call finds its weights in the 256 MB last-level cache
    left there by the call before, as in a forward pass."""
    import torch
    from sparse_moe_transformer_fp32_amd import binding as B
    from sparse_moe_transformer_fp32_amd.inputs import DENSE_WORKLOADS, make_dense_inputs

    wl = DENSE_WORKLOADS[name]
    n_layers = 3 if wl.T <= 16 else 1
    ffns = []
    for i in range(n_layers):
        x_i, wg, wu, wd = make_dense_inputs(wl, device, seed=wl.seed + 1000 * i)
        if i == 0:
            x = x_i
        ffns.append(B.DenseFFN(wg, wu, wd, S=wl.slices, T_max=wl.T))
        del wg, wu, wd
    y = torch.empty_like(x)
    for k in range(warmup):
        ffns[k % n_layers](x, y)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(steps):
        ffns[k % n_layers](x, y)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    hip = _hip()
    timer = StageTimer(hip, steps, len(B.STAGES))
    for k in range(steps):
        B.set_stage_events(timer.arrays[k])
        ffns[k % n_layers](x, y)
    B.set_stage_events(None)
    torch.cuda.synchronize()
    st = dict(zip(B.STAGES, timer.stage_ms()))
    timer.close()
    T, H, I = wl.T, wl.H, wl.I
    flops = 2 * T * 3 * H * I
    nbytes = 3 * H * I * 2 + 2 * T * H * 2
    gu_ms, dn_ms = st["gate_up"], st["down"]
    layers = f", {n_layers} layers in turn" if n_layers > 1 else ""
    return {"workload": f"{wl.name}: dense gated FFN, T={T}, H={H}, I={I}, {wl.slices} slices{layers}",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "bf16_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "gate_up_tflops": round(2 * T * 2 * H * I / (gu_ms * 1e-3) / 1e12, 2),
            # HBM bytes of the gate/up kernel per launch (rocprofv3 counters,
            # committed; null once its sources changed) against 2*H*I*2 B
            "gate_up_bytes": {"algorithmic": 2 * H * I * 2,
                              "traffic": _traffic("gate_up:dense_decode") if T <= 16 else None},
            "down_tflops": round(2 * T * H * I / (dn_ms * 1e-3) / 1e12, 2),
            "stage_ms": {k: round(v, 4) for k, v in st.items() if v > 0}}


def cpu_baseline(res, max_tokens=16, budget_s=10.0):
    """Time the float64 oracle on the host on up to `max_tokens` tokens of the
    workload (weights copied to host memory first; the timed region is the
    oracle call alone, including its bf16 -> float64 widening)."""
    import numpy as np
    import oracle
    from sparse_moe_transformer_fp32_amd.inputs import bf16_bits

    wl, inp = res["wl"], res["inp"]
    L = inp.layers[0]
    rows = np.arange(min(max_tokens, wl.T))
    xs = oracle.bf16_bits_to_f64(bf16_bits(inp.x[: len(rows)])).reshape(len(rows), wl.H)
    Wr = inp.router_ws[0].double().cpu().numpy()
    b = inp.router_bs[0].double().cpu().numpy()
    sel = oracle.select_topk(oracle.selection_keys(oracle.router_scores(oracle.router_logits(xs, Wr)), b), wl.K)
    need = np.unique(sel)

    class HostStack:
        def __init__(self, t):
            self.bits = {int(e): bf16_bits(t[int(e)]) for e in need}

        def __getitem__(self, e):
            return oracle.bf16_bits_to_f64(self.bits[int(e)])

    wg, wu, wd = HostStack(L.w_gate), HostStack(L.w_up), HostStack(L.w_down)
    sh = [oracle.bf16_bits_to_f64(bf16_bits(t)).reshape(tuple(t.shape)) for t in
          (L.ws_gate, L.ws_up, L.ws_down)]
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):  # pragma: no cover
        pass
    # repeat the call until about budget_s of CPU work (at most 10 calls;
    # a call longer than the budget is timed once)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(xs, Wr, b, wg, wu, wd, *sh, K=wl.K)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= 10:
            break
    return {"value": round(reps * len(rows) / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{len(rows)} of {wl.T} tokens of the {wl.name} batch, one layer, float64 "
                      f"NumPy oracle, {reps} calls in {dt:.2f} s, weights pre-staged in host "
                      f"memory; {cpu_model}, os.cpu_count() = {os.cpu_count()}, "
                      f"BLAS threads = {cores}"}


def library_reference(reps=10):
    """The vendor library on the same math, for context: torch.bmm (hipBLASLt)
    of bf16 [E, M, K] x [E, K, N], contiguous operands, with M the mean rows
    per expert of the prefill (114), 8192-token (228) and long (910)
    workloads, for the gate/up (K=4096, N=2560) and down (K=1280, N=4096)
    shapes; no gather, no activation, no routing.  Plus one dense GEMM
    32768 x 4096 x 2560."""
    import torch
    out = []
    shapes = []
    for m in (114, 228, 910):
        shapes += [(288, m, 4096, 2560, "gate_up"), (288, m, 1280, 4096, "down")]
    shapes.append((1, 32768, 4096, 2560, "dense"))
    for E, M, K, N, what in shapes:
        a = torch.randn(E, M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(E, K, N, device="cuda", dtype=torch.bfloat16).contiguous()
        c = torch.empty(E, M, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.bmm(a, b, out=c)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            torch.bmm(a, b, out=c)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tf = 2.0 * E * M * K * N / ms / 1e9
        out.append({"shape": what, "E": E, "M": M, "K": K, "N": N, "ms": round(ms, 4),
                    "tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        del a, b, c
        torch.cuda.empty_cache()
    return out


def side_layer_obj(wl_name, steps, warmup, cpu=False, cpu_tokens=None):
    """One side workload of the default run (prefill, long, skew): whole-step
    throughput, per-layer MFMA and HBM figures, both grouped GEMMs against
    their MFMA roofline (HIP events on the launch stream; for the chained
    long workload, the last layer's kernels), the attainable fraction
    min(peak, intensity x 8 TB/s) / achieved, and for skewed routing the
    per-expert load (count max/mean, share on the boosted experts)."""
    import numpy as np
    import torch
    from sparse_moe_transformer_fp32_amd.inputs import boosted_experts
    r = run_layer_bench(wl_name, steps, warmup)
    wl, nl = r["wl"], r["n_layers"]
    w = layer_work(wl, r["counts"])
    ms = r["wall_ms"]
    lay_ms = ms / nl
    st = r["stage_ms"]
    gu_ms, dn_ms = st["gate_up"], st["down"]
    dn_flops = w["layer_flops"] - w["gu_flops"]
    # the layer's floor: its FLOPs at the MFMA peak or its bytes at 8 TB/s
    floor_ms = max(w["layer_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                   w["layer_bytes"] / (HBM_PEAK_GBS * 1e9)) * 1e3
    tkey = f"gate_up:{wl.name}"
    out = {
        "workload": f"{wl.name}: T={wl.T} tokens, Flash shape, {nl} layer(s)"
                    + (f", router bias +{wl.bias_boost} on {wl.n_boost} seeded experts"
                       if wl.n_boost else ", near-uniform routing"),
        "tokens_per_s": round(wl.T / (ms / 1e3), 1),
        "ms_per_step": round(ms, 4),
        "ms_per_layer": round(lay_ms, 4),
        "bf16_tflops": round(w["layer_flops"] / (lay_ms * 1e-3) / 1e12, 2),
        "mfma_frac": round(w["layer_flops"] / (lay_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "hbm_gbs": round(w["layer_bytes"] / (lay_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(w["layer_bytes"] / (lay_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "attainable_ms": round(floor_ms, 4),
        "attainable_frac": round(floor_ms / lay_ms, 4),
        "active_experts": w["n_active"],
        "roofline_gate_up": roofline_obj("mfma", w["gu_flops"] / (gu_ms * 1e-3) / 1e12,
                                         MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", _traffic(tkey)),
        "roofline_down": roofline_obj("mfma", dn_flops / (dn_ms * 1e-3) / 1e12,
                                      MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", _traffic(f"down:{wl.name}")),
        "gate_up_hbm_gbs": round(w["gu_bytes"] / (gu_ms * 1e-3) / 1e9, 1),
        "stage_ms": {k: round(v, 4) for k, v in st.items()},
    }
    c = r["counts"].astype(np.int64)
    if wl.n_boost:
        boost = boosted_experts(wl)
        out["expert_load"] = {"count_max": int(c.max()), "count_mean": round(float(c.mean()), 2),
                              "max_over_mean": round(float(c.max() / c.mean()), 3),
                              "boosted": int(wl.n_boost),
                              "share_on_boosted": round(float(c[boost].sum() / c.sum()), 4)}
    if cpu:
        # the oracle on the whole batch (prefill) or on a bounded sample of
        # its first tokens (skew, long: cpu_tokens), one layer
        out["cpu_baseline"] = cpu_baseline(r, max_tokens=cpu_tokens or wl.T, budget_s=15.0)
    del r
    torch.cuda.empty_cache()
    return out


def roofline_obj(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skew", "skew_mild", "long", "tiny",
                             "dense_decode", "dense_prefill"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=4096 side measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "known-size reference for HBM byte counters) and exit")
    ap.add_argument("--library-reference", action="store_true",
                    help="only time torch.bmm (the vendor GEMM library) on the grouped "
                         "GEMM shapes, for context, and exit")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the HBM read rate of a plain 4 GiB read (moe_read_probe) "
                         "with ordinary and with non-temporal loads, and exit")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the bf16 matrix-core rate with no memory traffic "
                         "(moe_mfma_probe) and the clock it runs at")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the matrix-core ceiling side measurement of the default run")
    ap.add_argument("--short-read-ceiling", action="store_true",
                    help="only measure short non-temporal reads of 88, 176 and 264 MiB "
                         "(the dense decode FFN's weight streams) on rotating buffers")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the HBM read-ceiling side measurement of the default run")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-FFN side measurements of the default run")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long (T=32768 x 4 layers) side measurement of the default run")
    ap.add_argument("--no-skew", action="store_true",
                    help="skip the skewed-routing (T=8192) side measurement of the default run")
    ap.add_argument("--summarize-stats", nargs="+", metavar="ARG",
                    help="offline: STATS_CSV OUT COMMAND [TRACE_CSV] -> a short summary of "
                         "a rocprofv3 kernel_stats.csv (and of its kernel trace per launch shape)")
    ap.add_argument("--write-traffic", nargs="+", metavar="ARG",
                    help="offline: PMC_ROOT COMMAND... -> profiles/traffic.json")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="ARG",
                    help="offline: PMC_ROOT OUT COMMAND [LDS_PMC_ROOT LDS_COMMAND]: MFMA (and "
                         "LDS/wait) counter runs over prefill and long -> a short summary")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1:])
        return
    if args.summarize_mfma:
        root, out, command = args.summarize_mfma[:3]
        lines = summarize_mfma(root, command)
        if len(args.summarize_mfma) == 5:
            lines += summarize_lds(*args.summarize_mfma[3:])
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path; --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "copies": 3}))
        return
    if args.library_reference:
        print(json.dumps({"library_reference": library_reference()}), flush=True)
        return
    if args.mfma_ceiling:
        print(json.dumps({"mfma_ceiling": mfma_ceiling()}), flush=True)
        return
    if args.short_read_ceiling:
        print(json.dumps({"short_read_ceiling": short_read_ceiling()}), flush=True)
        return
    if args.read_ceiling:
        print(json.dumps({"read_ceiling": read_ceiling()}), flush=True)
        return
    if args.workload.startswith("dense"):
        d = run_dense_bench(args.workload, args.steps, args.warmup)
        print(json.dumps({
            "metric": "dense-FFN tokens/s", "value": d["tokens_per_s"], "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": d["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": d["workload"]}, "dense": d}), flush=True)
        return
    res = run_layer_bench(args.workload, args.steps, args.warmup)
    wl = res["wl"]
    work = layer_work(wl, res["counts"])
    ms = res["wall_ms"]
    tok_s = wl.T / (ms / 1e3)
    gu_ms = res["stage_ms"]["gate_up"]
    nl = res["n_layers"]
    tkey = f"gate_up:{wl.name}" if wl.name in ("decode", "prefill") else None
    if wl.T <= 64:   # weight streaming: HBM bound
        rf = roofline_obj("hbm", work["gu_bytes"] / (gu_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                          _traffic(tkey) if tkey else None)
    else:
        rf = roofline_obj("mfma", work["gu_flops"] / (gu_ms * 1e-3) / 1e12,
                          MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", _traffic(tkey) if tkey else None)
    layer_ms = ms / nl
    line = {
        "metric": "MoE-layer tokens/s + % roofline (HBM GB/s @T=16, MFMA TFLOP/s @T=4096)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: T={wl.T} tokens, H={wl.H}, E={wl.E} routed top-{wl.K} + "
                        f"{'1 shared' if wl.Is else 'no shared'} expert, I={wl.I}, Is={wl.Is}, "
                        f"{nl} layer(s), bf16 experts, fp32 sigmoid router",
            "T": wl.T, "H": wl.H, "E": wl.E, "K": wl.K, "I": wl.I, "Is": wl.Is, "layers": nl,
            "seed": wl.seed,
        },
        "roofline": rf,
        "layer": {
            "gpu_ms_per_step": round(res["gpu_ms"], 4),
            "graph_replay_ms_per_step": round(res["graph_ms"], 4),
            "ms_per_step_with_stage_events": round(res["inst_ms"], 4),
            "active_experts": work["n_active"],
            "algorithmic_bytes": work["layer_bytes"],
            "hbm_gbs": round(work["layer_bytes"] / (layer_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(work["layer_bytes"] / (layer_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bf16_tflops": round(work["layer_flops"] / (layer_ms * 1e-3) / 1e12, 2),
            "stage_ms": {k: round(v, 4) for k, v in res["stage_ms"].items()},
        },
    }
    if args.workload == "decode" and not args.no_read_ceiling:
        # the practical HBM read ceiling, measured right after the decode
        # steps, next to the decode roofline's nominal 8 TB/s
        rc = read_ceiling(gib=4, reps=10)
        rc["roofline_achieved_over_nontemporal"] = round(rf["achieved"] / rc["nontemporal"]["gbs"], 4)
        line["read_ceiling"] = rc
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res)
    if args.workload == "decode":
        del res
        torch.cuda.empty_cache()
        # a prefill step takes ~2 ms: 25 steps after 5 warm-up steps keep
        # the figure steady at a fraction of a second of GPU time
        side_steps = max(10, args.steps // 2)
        if not args.no_prefill:
            # the metric's MFMA figure is quoted at T=4096; the oracle is
            # timed on the whole batch in the same run
            line["prefill"] = side_layer_obj("prefill", side_steps, 5,
                                             cpu=not args.no_cpu_baseline)
            torch.cuda.empty_cache()
        if not args.no_dense:
            # a decode call takes ~50 us: time 60 of them
            line["dense"] = {"dense_decode": run_dense_bench("dense_decode", max(side_steps, 60), 6),
                             "dense_prefill": run_dense_bench("dense_prefill", side_steps, 3)}
            torch.cuda.empty_cache()
        if not args.no_long:
            # the compute-bound regime: 4 chained layers at T=32768
            line["long"] = side_layer_obj("long", 3, 1, cpu=not args.no_cpu_baseline,
                                          cpu_tokens=1024)
            torch.cuda.empty_cache()
        if not args.no_skew:
            line["skew"] = side_layer_obj("skew", side_steps, 5, cpu=not args.no_cpu_baseline,
                                          cpu_tokens=2048)
            torch.cuda.empty_cache()
        if not args.no_mfma_ceiling:
            # the sustained matrix-core rate, next to the nominal 2.5 PF the
            # GEMM rooflines use
            mc = mfma_ceiling()
            line["mfma_ceiling"] = mc
            for name in ("prefill", "long", "skew"):
                if name in line:
                    for g in ("roofline_gate_up", "roofline_down"):
                        line[name][g + "_over_mfma_ceiling"] = round(
                            line[name][g]["achieved"] / mc["tflops"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
