#!/usr/bin/env python3
"""Throughput of the int4 routed-expert MoE layer on one MI355X.

A step is one whole layer forward (route -> permute -> shared expert ->
grouped gate/up + SwiGLU -> grouped down -> combine, plus the latent
wrapper / exact quantiser where the workload has them) over one batch of
seeded synthetic tokens already resident in HBM.  Default workload: the
Kimi-K2.5-shaped decode layer (T=64, hidden 7168, 384 experts, top-8,
intermediate 2048, one bf16 shared expert).

Prints ONE JSON line: tokens/s over exactly --steps timed steps (after
--warmup untimed ones), the dominant kernel's roofline fraction measured with
HIP events on the launch stream, and the CPU oracle timed on a bounded token
sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0  # dense fp16/bf16 matrix cores
INT8_PEAK_TOPS = 5000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="1 tiny, 2 K2.5 decode (default), 3 K2.5 prefill, 4 exact-mode Zipf, 5 K3 latent")
    ap.add_argument("--kernel-steps", type=int, default=10, help="forwards timed per kernel with events")
    ap.add_argument("--act-bits", type=int, default=None, choices=[8, 16],
                    help="exact workload: activation code width (16: the act_bits = 16 variant)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device-to-device copy of this many MiB (3 times), the reference "
                         "kernel for scaling HBM byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--calibrate-copy into profiles/<call>_<workload>_traffic.json")
    ap.add_argument("--prefill-leg", dest="prefill_leg", action="store_true", default=None,
                    help="after the headline workload, also time the same layer at prefill size (T=8192) and "
                         "report it under 'prefill' (default: on for the default decode workload)")
    ap.add_argument("--no-prefill-leg", dest="prefill_leg", action="store_false")
    ap.add_argument("--no-hbm-probe", action="store_true", help="skip the streaming read and copy probes")
    ap.add_argument("--no-mfma-probe", action="store_true", help="skip the matrix-core rate probe")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the forward recorded as a HIP graph (MoELayer.capture) instead of "
                         "eager forwards; the per-call times still come from eager forwards")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="also time torch's dense bf16 GEMM (hipBLASLt) at the prefill gate/up and down shapes, "
                         "a practical matrix-core reference under this part's clock behaviour")
    ap.add_argument("--json-out", metavar="PATH", help="also write the JSON line to PATH")
    ap.add_argument("--stats-from", metavar="DIR",
                    help="no run: summarise a rocprofv3 --kernel-trace --stats folder of a bench run (whose line "
                         "--bench-json names) into profiles/moe_layer_<workload>_kernel_stats.md")
    ap.add_argument("--bench-json", metavar="PATH", help="the --json-out file of the profiled run (for --stats-from)")
    ap.add_argument("--profile-cmd", metavar="CMD", action="append",
                    help="a profiled command, quoted in the summary (--stats-from, --counters-from; repeatable)")
    ap.add_argument("--counters-from", metavar="DIR", nargs="+",
                    help="no run: summarise rocprofv3 --pmc folders (one per counter pass) of one workload into "
                         "profiles/moe_layer_<workload>_counters.md (per-dispatch means and derived rates)")
    ap.add_argument("--kernel-regex", default="k_grouped", help="kernels kept by --counters-from")
    ap.add_argument("--counters-name", default="grouped",
                    help="which kernels --counters-from summarises, for the title and the file name "
                         "(other than 'grouped': profiles/moe_layer_<workload>_<name>_counters.md)")
    return ap.parse_args()


def algorithmic_work(cfg, counts, shared_I):
    """Bytes each call must move and flops it must do (weights of routed experts only)."""
    T, E, k, H, I = cfg["T"], cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    K = cfg["L"] or H
    S = T * k
    active = int((counts > 0).sum())
    exact = cfg["mode"] == "exact"
    gu_w = 2 * (I * K // 2 + I * (K // 32) * 2)   # gate+up packed + scales, per expert
    d_w = K * I // 2 + K * (I // 32) * 2           # down
    act_in = T * K * (1 if exact else 2) + (T * (K // 32) * 4 if exact else 0)
    h_bytes = S * I * (1 if exact else 2) + (S * (I // 32) * 4 if exact else 0)
    y_bytes = S * K * (4 if exact else 2)
    work = {
        "moe_route": (E * H * 2 + T * H * 2 + T * k * 8, 2 * T * E * H),
        "moe_permute": (T * k * 4 * 3 + E * 8, 0),
        "moe_int4_grouped_swiglu": (active * gu_w + act_in + h_bytes, 2 * S * 2 * K * I),
        "moe_int4_grouped_down": (active * d_w + h_bytes + y_bytes, 2 * S * I * K),
        "moe_combine": (y_bytes + T * K * (4 if exact else 2) + (T * H * 2 if shared_I and not cfg["L"] else 0),
                        2 * S * K),
    }
    if exact:
        work["moe_quant_act_int8"] = (T * K * 2 + act_in, 0)
    if shared_I:
        work["shared_gate_up"] = (2 * shared_I * H * 2 + T * H * 2 + T * shared_I * 2, 2 * T * 2 * H * shared_I)
        work["shared_down"] = (H * shared_I * 2 + T * shared_I * 2 + T * H * 2, 2 * T * shared_I * H)
    if cfg["L"]:
        L = cfg["L"]
        work["latent_down"] = (L * H * 2 + T * H * 2 + T * L * 2, 2 * T * L * H)
        work["moe_rmsnorm_bf16"] = (2 * T * L * 2 + L * 2, 0)
        work["latent_up"] = (H * L * 2 + T * L * 2 + 2 * T * H * 2, 2 * T * L * H)
    layer_bytes = (active * (gu_w + d_w) + E * H * 2 + E * 4 + T * H * 2 + T * H * (4 if exact else 2)
                   + (3 * shared_I * H * 2 if shared_I else 0)
                   + (2 * cfg["L"] * H * 2 + cfg["L"] * 2 if cfg["L"] else 0))
    layer_flops = sum(f for n, (b, f) in work.items() if n != "moe_route")
    return work, layer_bytes, layer_flops, active


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_SOURCES = ["int4_routed_expert_moe_amd/csrc/grouped_gemm.hip", "int4_routed_expert_moe_amd/csrc/moe_common.h"]


def _counter_means(folder, counter):
    """Mean value per dispatch of one counter, per kernel, from rocprofv3 csv output."""
    import csv
    import glob
    import re
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            m = re.search(r"k_grouped(?:_skinny|_exact)?<(\d+), (\d+)", name)   # <mode, op, ...>
            m32 = re.search(r"k_grouped32(?:_dma)?<(\d+),", name)          # <op, m32>
            if m or m32:
                op = m.group(2) if m else m32.group(1)
                key = "moe_int4_grouped_swiglu" if op == "0" else "moe_int4_grouped_down"
            elif "opy" in name:
                key = ("copy", int(r["Grid_Size"]))
            else:
                continue
            d = vals.setdefault(key, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    out = {k: float(np.mean(list(v.values()))) for k, v in vals.items() if not isinstance(k, tuple)}
    copies = [k for k in vals if isinstance(k, tuple)]
    if copies:  # the calibration copy is the copy launch with the largest grid (small staging copies also run)
        out["copy"] = float(np.mean(list(vals[max(copies, key=lambda k: k[1])].values())))
    return out


def write_traffic(args, cfg):
    """HBM bytes per launch of the grouped kernels from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled so that the plain copy of --calibrate-copy MiB reads and
    writes exactly its size."""
    fetch = _counter_means(args.traffic_from[0], "FETCH_SIZE")
    write = _counter_means(args.traffic_from[1], "WRITE_SIZE")
    copy_kib = args.calibrate_copy * 1024.0
    ff, fw = copy_kib / fetch["copy"], copy_kib / write["copy"]
    for call in ("moe_int4_grouped_swiglu", "moe_int4_grouped_down"):
        if call not in fetch or call not in write:
            continue
        rec = {
            "call": call, "workload": cfg["name"],
            "fetch_bytes": fetch[call] * ff * 1024, "write_bytes": write[call] * fw * 1024,
            "raw_fetch_kib": fetch[call], "raw_write_kib": write[call],
            "copy_calibration": {"mib": args.calibrate_copy, "fetch_factor": ff, "write_factor": fw},
            "sources": TRAFFIC_SOURCES, "source_sha": source_digest(TRAFFIC_SOURCES),
        }
        rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
        path = os.path.join(ROOT, "profiles", f"{call}_{cfg['name']}_traffic.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"{path}: {rec['bytes_per_launch'] / 1e9:.3f} GB per launch (copy factors {ff:.3f}, {fw:.3f})")


def traffic_record(kernel, workload_name):
    """HBM traffic measured with rocprofv3 counters for this kernel and workload, if
    the record was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_digest(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def roofline(cfg, counts, kernel_ms):
    """The dominant call (largest event-timed duration among the layer's calls) against
    its roofline, and the whole step against both peaks."""
    work, layer_bytes, layer_flops, active = algorithmic_work(cfg, counts, cfg["shared_I"])
    dom = max((n for n in kernel_ms if n in work), key=lambda n: kernel_ms[n])
    b, f = work[dom]
    dur_s = kernel_ms[dom] / 1e3
    exact = cfg["mode"] == "exact"
    if f / max(b, 1) < MFMA_F16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": b / dur_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    elif exact:
        # exact mode is rated against the int8 matrix-core peak (its integer MACs), although
        # the kernels run them as exact fp16 products
        roof = {"bound": "mfma", "achieved": f / dur_s / 1e12, "peak": INT8_PEAK_TOPS, "unit": "TOP/s"}
    else:
        roof = {"bound": "mfma", "achieved": f / dur_s / 1e12, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_record(dom, cfg["name"])
    roof["kernel"] = dom
    roof["kernel_ms"] = kernel_ms[dom]
    roof["algorithmic_bytes"] = b
    roof["algorithmic_flops"] = f
    return roof, layer_bytes, layer_flops, active


def time_layer(layer, x, steps, warmup, kernel_steps, graph=False):
    """ms per step over exactly `steps` timed forwards (after `warmup`), between two
    synchronisations, and the per-call event durations of `kernel_steps` more forwards
    (every call on the launch stream).  graph: the timed forwards are replays of the
    forward recorded as a HIP graph on x."""
    import torch
    run = layer.forward
    if graph:
        g = layer.capture(x)
        run = lambda _x: g.replay()  # noqa: E731  (x is the graph's input buffer)
    for _ in range(warmup):
        run(x)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        run(x)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / steps
    per = {}
    for _ in range(kernel_steps):
        marks = []
        layer.forward(x, marks=marks)
        torch.cuda.synchronize()
        for (_, a), (name, b) in zip(marks[:-1], marks[1:]):
            per.setdefault(name, []).append(a.elapsed_time(b))
    return ms_per_step, {n: float(np.mean(v)) for n, v in per.items()}, wall


def hbm_probe():
    """Context figures for the nominal 8 TB/s: a plain streaming read of 4 GiB
    (libmoe_probe.so) and torch's device copy of 2 GiB (read + write bytes),
    best of 5 each, timed with events."""
    import ctypes

    import torch
    from int4_routed_expert_moe_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_OUT)
    lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.moe_probe_read.restype = ctypes.c_int
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)  # every 16-byte fold is 0, never 0xFFFFFFFF
    blocks = 256 * 16
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best_read = 0.0
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        if lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr()), n, 0xFFFFFFFF, ctypes.c_void_p(out.data_ptr()), blocks,
                              st) != 0:
            raise RuntimeError("read probe launch failed")
        b.record()
        torch.cuda.synchronize()
        best_read = max(best_read, n / (a.elapsed_time(b) / 1e3) / 1e9)
    del buf
    m = 2 << 30
    src = torch.empty(m, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    best_copy = 0.0
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best_copy = max(best_copy, 2 * m / (a.elapsed_time(b) / 1e3) / 1e9)
    del src, dst
    return {"read_GBs": best_read, "copy_rw_GBs": best_copy, "read_bytes": n, "copy_bytes": m,
            "read_frac_of_peak": best_read / HBM_PEAK_GBS,
            "method": "best of 5: 16-byte grid-strided loads over 4 GiB (4096 workgroups); torch copy of 2 GiB"}


def mfma_probe():
    """Context figure for the nominal matrix-core peak: independent accumulation
    chains on register operands of the 32x32x16 bf16 shape (the dense and prefill
    kernels', 8 chains per wave) and of the 16x16x32 f16 shape (the 16x16 tile and
    decode kernels', 16 chains per wave), two waves per SIMD (512 workgroups of 4
    waves), best of 3."""
    import ctypes

    import torch
    from int4_routed_expert_moe_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_OUT)
    lib.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.moe_probe_mfma.restype = ctypes.c_int
    blocks, iters = 512, 10000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for shape, key, flops_per, chains in ((0, "bf16_32x32x16_TFs", 32768, 8), (1, "f16_16x16x32_TFs", 16384, 16)):
        best = 0.0
        for _ in range(4):  # the first run warms up
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if lib.moe_probe_mfma(shape, ctypes.c_void_p(out.data_ptr()), blocks, iters, st) != 0:
                raise RuntimeError("matrix-core probe launch failed")
            b.record()
            torch.cuda.synchronize()
            best = max(best, blocks * 4 * chains * iters * flops_per / (a.elapsed_time(b) / 1e3) / 1e12)
        res[key] = best
    res["frac_of_peak"] = max(res["bf16_32x32x16_TFs"], res["f16_16x16x32_TFs"]) / MFMA_F16_PEAK_TFS
    res["method"] = ("best of 3: independent chains on register operands (8 per wave for 32x32x16, 16 for "
                     "16x16x32), 512 workgroups of 4 waves (two waves per SIMD), 10000 rounds")
    return res


def gemm_reference():
    """torch's dense bf16 GEMM (hipBLASLt) at the total shapes of the prefill grouped
    calls without grouping or int4 (65536 x 4096 x 7168 and 65536 x 7168 x 2048):
    a practical reference for the matrix-core fraction this part sustains."""
    import torch
    out = {}
    for name, (M, N, K) in (("gate_up_shape", (65536, 4096, 7168)), ("down_shape", (65536, 7168, 2048))):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b.t()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            c = a @ b.t()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        tf = 2.0 * M * N * K / (ms / 1e3) / 1e12
        out[name] = {"M": M, "N": N, "K": K, "ms": ms, "TFLOPs": tf, "frac_of_peak": tf / MFMA_F16_PEAK_TFS}
        del a, b, c
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def stats_summary(args):
    """profiles/moe_layer_<workload>_kernel_stats.md from a rocprofv3 --kernel-trace --stats
    folder of one bench run (without the prefill leg) and that run's --json-out line."""
    import csv
    import glob
    import re
    line = json.loads(open(args.bench_json).read().strip().splitlines()[-1])
    run = line["run"]
    n_fwd = run["warmup"] + run["steps"] + run["kernel_steps"]
    stats_f = glob.glob(os.path.join(args.stats_from, "**", "*kernel_stats.csv"), recursive=True)
    trace_f = glob.glob(os.path.join(args.stats_from, "**", "*kernel_trace.csv"), recursive=True)
    if len(stats_f) != 1 or len(trace_f) != 1:
        sys.exit(f"--stats-from: expected one kernel_stats.csv and one kernel_trace.csv under {args.stats_from}")
    rows = list(csv.DictReader(open(stats_f[0])))
    trace = sorted(csv.DictReader(open(trace_f[0])), key=lambda r: int(r["Start_Timestamp"]))
    durs = {}
    for r in trace:
        durs.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def short(n):
        n = n.replace("(anonymous namespace)::", "")
        n = re.sub(r"^void ", "", n)
        return re.sub(r"\(.*\)$", "", n)

    def single_stream(name):
        """Average of the kernel's dispatches in the last kernel_steps forwards (the
        per-call event steps, every call alone on the launch stream)."""
        d = durs.get(name, [])
        if not d or len(d) % n_fwd:
            return None
        tail = d[-run["kernel_steps"] * (len(d) // n_fwd):]
        return sum(tail) / len(tail)

    cfg_name = line["config"]["workload"].split(":")[0]
    ks = run["kernel_steps"]
    out = [f"# Layer kernels, workload {cfg_name}", "",
           "Command (on the MI355X, from the repository root), then the summary:", "", "```",
           *(args.profile_cmd or ["(not given)"]),
           f"python3 bench.py --stats-from {args.stats_from} --bench-json {args.bench_json}", "```", "",
           f"The run made {n_fwd} forwards: {run['warmup']} warmup, {run['steps']} timed (the shared expert on its "
           f"own stream from {run['side_stream_min_t']} tokens), then {ks} per-call event steps with every call alone "
           "on the launch stream. The last column averages each kernel's dispatches in those last "
           f"{ks} forwards; it is what the bench line's per-call times (HIP events between the calls) measure, "
           "launch gaps included.", "",
           "| kernel | calls | per forward | avg µs | min µs | max µs | % of GPU time | avg µs, last "
           f"{ks} forwards (one stream) |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        c = int(r["Calls"])
        ss = single_stream(r["Name"])
        pf = f"{c // n_fwd}" if c % n_fwd == 0 else "–"
        out.append(f"| `{short(r['Name'])}` | {c} | {pf} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} | "
                   f"{'–' if ss is None else f'{ss:.1f}'} |")
    rf = line["roofline"]
    out += ["", "bench.py line of the same run (HIP events on the launch stream):", "",
            f"- value {line['value']:.0f} tokens/s, {line['ms_per_step']:.3f} ms per layer step",
            f"- dominant call `{rf['kernel']}`: {rf['kernel_ms'] * 1e3:.1f} µs per launch, {rf['achieved']:.1f} "
            f"{rf['unit']} algorithmic of {rf['peak']:.1f} ({100 * rf['frac']:.1f}% of peak, bound {rf['bound']})",
            "- per-call ms: " + ", ".join(f"{k} {v:.3f}" for k, v in line["kernel_ms"].items()), ""]
    path = os.path.join(ROOT, "profiles", f"moe_layer_{cfg_name}_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print(f"wrote {path}")


SIMDS = 1024          # 256 CUs x 4 SIMDs
SQ_INSTANCES = 32     # SQ_BUSY_CYCLES is summed over the shader engines (8 XCDs x 4)


def counters_summary(args, cfg):
    """profiles/moe_layer_<workload>_counters.md: per-kernel means per dispatch of every
    counter in the given rocprofv3 --pmc folders, and the rates derived from them."""
    import csv
    import glob
    import re
    vals = {}
    for d in args.counters_from:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name = re.sub(r"\(.*$", "", r["Kernel_Name"].replace("(anonymous namespace)::", ""))
                name = re.sub(r"^void ", "", name)
                if not re.search(args.kernel_regex, name):
                    continue
                key = (d, r["Dispatch_Id"])
                v = vals.setdefault(name, {}).setdefault(r["Counter_Name"], {})
                v[key] = v.get(key, 0.0) + float(r["Counter_Value"])
    # kernel durations of the counted runs: the bench lines in each folder's log, if kept beside it
    out = [f"# Counters of the {args.counters_name} kernels, workload {cfg['name']}", "",
           "Commands (on the MI355X, from the repository root; one counter pass each), then the summary:", "", "```"]
    out += list(args.profile_cmd or ["(not given)"])
    out += [f"python3 bench.py --workload {cfg['id']} --counters-from {' '.join(args.counters_from)}"
            f" --kernel-regex '{args.kernel_regex}'"
            + (f" --counters-name {args.counters_name}" if args.counters_name != "grouped" else ""), "```", "",
            "Per-dispatch means over every dispatch of the kernel in the run. Derived rates, with the "
            f"normalisations used: per-SIMD busy cycles = SQ_BUSY_CYCLES / {SQ_INSTANCES} (the counter sums its "
            f"{SQ_INSTANCES} shader-engine instances); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / {SIMDS} SIMDs / "
            "per-SIMD busy cycles (SQ_VALU_MFMA_BUSY_CYCLES adds 32 per 32x32x16 and 16 per 16x16x32 operation); "
            f"VALU busy = 4 SQ_ACTIVE_INST_VALU / {SIMDS} / per-SIMD busy cycles (quad-cycle units); co-issue = "
            f"SQ_VALU_MFMA_COEXEC_CYCLES / {SIMDS} / per-SIMD busy cycles.", ""]
    kms = {}
    if args.bench_json:  # per-call event times of a bench run (the clock estimate below)
        kms = json.loads(open(args.bench_json).read().strip().splitlines()[-1]).get("kernel_ms", {})
    for name, cs in sorted(vals.items()):
        m = {c: float(np.mean(list(v.values()))) for c, v in cs.items()}
        mo = re.search(r"k_grouped(?:_skinny|_exact)?<(\d+), (\d+)", name) or re.search(r"k_grouped32(?:_dma)?<()(\d+),", name)
        call = None if not mo else ("moe_int4_grouped_swiglu" if mo.group(2) == "0" else "moe_int4_grouped_down")
        out += [f"## `{name}`", "", "| counter | mean per dispatch |", "|---|---|"]
        out += [f"| {c} | {m[c]:.4g} |" for c in sorted(m)]
        busy = m.get("SQ_BUSY_CYCLES", 0) / SQ_INSTANCES
        if busy > 0:
            rates = []
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                rates.append(f"MFMA busy {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / SIMDS / busy:.1f}%")
            if "SQ_ACTIVE_INST_VALU" in m:
                rates.append(f"VALU busy {100 * 4 * m['SQ_ACTIVE_INST_VALU'] / SIMDS / busy:.1f}%")
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
                rates.append(f"VALU and MFMA together {100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / SIMDS / busy:.1f}%")
            if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m and m["SQ_INSTS_MFMA"] > 0:
                rates.append(f"non-MFMA VALU instructions per MFMA "
                             f"{(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_INSTS_MFMA']:.2f}")
            if call in kms:
                rates.append(f"clock about {busy / (kms[call] * 1e-3) / 1e9:.2f} GHz (per-SIMD busy cycles over "
                             f"{kms[call]:.3f} ms, the {call} event time of the --bench-json run)")
            out += ["", f"Per-SIMD busy cycles per dispatch: {busy:.4g}. " + "; ".join(rates) + "."]
        out.append("")
    tag = "" if args.counters_name == "grouped" else f"_{args.counters_name}"
    path = os.path.join(ROOT, "profiles", f"moe_layer_{cfg['name']}{tag}_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print(f"wrote {path}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    from int4_routed_expert_moe_amd import synthetic
    cfg0 = synthetic.WORKLOADS[args.workload]
    if args.traffic_from:
        if not args.calibrate_copy:
            sys.exit("--traffic-from needs --calibrate-copy MIB, the copy size of the counted run")
        write_traffic(args, cfg0)
        return
    if args.counters_from:
        counters_summary(args, cfg0)
        return
    if args.stats_from:
        if not args.bench_json:
            sys.exit("--stats-from needs --bench-json, the --json-out file of the profiled run")
        stats_summary(args)
        return
    import torch
    from int4_routed_expert_moe_amd.layer import MoELayer

    bias = None
    if cfg0.get("zipf"):
        bias = synthetic.load_bias_file(os.path.join(ROOT, "tests", "golden", "zipf_bias_k25.txt"))
    t_gen = time.perf_counter()
    inp = synthetic.make_inputs(args.workload, router_bias=bias)
    if args.act_bits is not None:
        if inp["cfg"]["mode"] != "exact":
            sys.exit("--act-bits applies to the exact workload only")
        inp["cfg"] = dict(inp["cfg"], act_bits=args.act_bits)
        if args.act_bits == 16:
            inp["cfg"]["name"] = inp["cfg"]["name"] + "_act16"
    cfg = inp["cfg"]
    layer = MoELayer.from_numpy(inp, "cuda")
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda().view(torch.bfloat16)
    t_gen = time.perf_counter() - t_gen
    T = cfg["T"]

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_per_step, kernel_ms, wall = time_layer(layer, x, args.steps, args.warmup, args.kernel_steps, args.graph)
    counts = layer.workspace(T)["counts"].cpu().numpy()
    roof, layer_bytes, layer_flops, active = roofline(cfg, counts, kernel_ms)

    step_s = ms_per_step / 1e3
    line = {
        "metric": "MoE-layer tokens/s at 1 GPU + % of HBM (decode) / MFMA (prefill) roofline",
        "value": T / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4xf16-mfma" if cfg["mode"] != "exact"
                  else "int4xint16-exact" if int(cfg.get("act_bits", 8)) == 16 else "int4xint8-exact"),
        "data": "synthetic (seeded; random-init weights of the layer's shapes)",
        "config": {
            "workload": (f"{cfg['name']}: T={T} hidden={cfg['H']} experts={cfg['E']} top-{cfg['k']} "
                         f"intermediate={cfg['I']}" + (f" latent={cfg['L']}" if cfg["L"] else "")
                         + (f" shared={cfg['shared_I']}" if cfg["shared_I"] else "") + f" mode={cfg['mode']}"),
            "tokens": T,
            "active_experts": active,
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "layer_roofline": {
            "bytes": layer_bytes, "flops": layer_flops,
            "hbm_frac": layer_bytes / step_s / (HBM_PEAK_GBS * 1e9),
            "mfma_frac": layer_flops / step_s / (MFMA_F16_PEAK_TFS * 1e12),
        },
        "kernel_ms": kernel_ms,
        "wall_s_timed": wall,
        "setup_s": t_gen,
        "run": {"warmup": args.warmup, "steps": args.steps, "kernel_steps": args.kernel_steps,
                "side_stream_min_t": MoELayer.SIDE_STREAM_MIN_T, "graph": args.graph},
    }
    if cfg["mode"] == "exact":
        line["layer_roofline"]["int8_frac"] = layer_flops / step_s / (INT8_PEAK_TOPS * 1e12)

    prefill_leg = args.prefill_leg if args.prefill_leg is not None else (args.workload == 2 and args.act_bits is None)
    if prefill_leg:
        # the same layer (workloads 2 and 3 share their weights) at prefill size
        cfg3 = dict(synthetic.WORKLOADS[3])
        if cfg3["layer_seed"] != cfg["layer_seed"] or cfg3["H"] != cfg["H"]:
            sys.exit("--prefill-leg needs a workload that shares the prefill workload's layer")
        x3 = torch.from_numpy(synthetic.gen_x(cfg3).view(np.int16)).cuda().view(torch.bfloat16)
        ms3, kms3, wall3 = time_layer(layer, x3, args.steps, args.warmup, max(3, args.kernel_steps // 2),
                                      args.graph)
        counts3 = layer.workspace(cfg3["T"])["counts"].cpu().numpy()
        roof3, lb3, lf3, active3 = roofline(cfg3, counts3, kms3)
        line["prefill"] = {
            "workload": f"{cfg3['name']}: T={cfg3['T']} (the same layer, weights shared with the headline workload)",
            "value": cfg3["T"] / (ms3 / 1e3), "unit": "tokens/s", "ms_per_step": ms3, "steps": args.steps,
            "warmup": args.warmup, "wall_s_timed": wall3, "active_experts": active3, "roofline": roof3,
            "layer_roofline": {"bytes": lb3, "flops": lf3, "mfma_frac": lf3 / (ms3 / 1e3) / (MFMA_F16_PEAK_TFS * 1e12),
                               "hbm_frac": lb3 / (ms3 / 1e3) / (HBM_PEAK_GBS * 1e9)},
            "kernel_ms": kms3,
        }
        del x3
        layer._ws.pop(cfg3["T"], None)
        torch.cuda.empty_cache()

    if not args.no_hbm_probe:
        line["hbm_probe"] = hbm_probe()
    if not args.no_mfma_probe:
        line["mfma_probe"] = mfma_probe()
    if args.gemm_reference:
        line["gemm_reference"] = gemm_reference()

    if not args.no_cpu_baseline:
        import oracle
        toks_probe = synthetic.token_sample(cfg, min(4, T), salt=1)
        t0 = time.perf_counter()
        oracle.layer_tokens(inp, toks_probe)
        per_tok = (time.perf_counter() - t0) / len(toks_probe)
        n = int(max(len(toks_probe), min(T, args.cpu_seconds / max(per_tok, 1e-9))))
        toks = synthetic.token_sample(cfg, n, salt=2)
        t0 = time.perf_counter()
        oracle.layer_tokens(inp, toks)
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": len(toks) / el, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{len(toks)} of {T} tokens of the same workload (routing of the sampled tokens "
                      f"included), {el:.1f} s",
        }
    text = json.dumps(line)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")
    print(text)


if __name__ == "__main__":
    main()
