#!/usr/bin/env python3
"""Throughput benchmark of the scan library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAMES] [--no-cpu]

A step is one call of the library on one batch of synthetic input resident in
HBM; the K timed steps are captured once into a HIP graph and replayed (pass
--eager to issue them one by one).  The headline step is the largest
single-GPU workload: the device-wide exclusive add scan of a flat i32 array of
2^28 elements, values uniform in {0..15} (seed 2).  Consecutive steps rotate
over several input/output buffer pairs, so that no step finds its data in the
256 MB Infinity Cache left there by the previous one.  The other workloads
(row scans of fp32 [1024, 4096], bf16 [8192, 8192] and [8192, 8191], the bf16
product scan, the device-wide scans of 2^28 - 37 i32 and of f32/i64 min/max,
the inclusive scan, the reductions, reduce-by-key, the radix sort and select)
are timed the same way and reported inside the same JSON line under
"workloads".

Prints ONE JSON line.  "value" is elements/s of the headline workload (wall
clock over the K timed steps); "roofline" rates the headline call by its
algorithmic bytes (read n + write n) over its average duration from HIP
events on the launch stream (the call is the scan kernel plus the small kernel
that resets its tile descriptors); "cpu_baseline" times the CPU oracle on the
same workload on one host core.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0            # MI355X HBM3E peak, GB/s
METRIC = "scan elements/s and achieved HBM GB/s (% of peak), 1 MI355X"
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
HEAD_BYTES = (1 << 28) * 4 * 2   # the headline's read + write bytes (also what copy16 moves)
KERNEL_SOURCES = {           # sources whose change invalidates stored counter readings
    "scan_rows": ["device.hpp", "scan_rows.hip"],
    "scan_device": ["device.hpp", "scan_device.hip"],
    "select": ["device.hpp", "select.hip"],
    "reduce": ["device.hpp", "reduce.hip"],
    "reduce_by_key": ["device.hpp", "reduce_by_key.hip"],
    "radix_sort": ["device.hpp", "radix_sort.hip"],
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="merge into profiles/pmc_traffic.json the counter_collection.csv files "
                         "of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--pmc-select-key", default="select_p0.5",
                    help="workload the select kernel's counters are filed under in this summary "
                         "(the profiled command ran only that select workload)")
    ap.add_argument("--pmc-command", default="", help="the profiled command, recorded with --pmc-summary")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sub-steps", type=int, default=20, help="timed calls per other workload")
    ap.add_argument("--sets", type=int, default=4, help="buffer sets rotated between steps")
    ap.add_argument("--only", default="", help="comma-separated workload names to run (profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true",
                    help="issue the timed calls one by one instead of replaying a HIP graph")
    return ap.parse_args()


def sources_sha(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "stream_compaction_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_KEYS = {                 # kernel-name prefix in the profiler output -> (workload, sources)
    "void sca::scan_rows_kernel<sca::FmtBF16, (sca::Op)0, true, 8, 4, 4>(": ("rows_bf16_excl",
                                                                           "scan_rows"),
    "void sca::scan_device_kernel<sca::FmtI32, (sca::Op)0, false, 4, 8, 16>(": ("dev_i32_add",
                                                                              "scan_device"),
    "void sca::reduce_partials_kernel<sca::FmtI32, (sca::Op)0, 4, 16>(": ("reduce_i32_add", "reduce"),
    "void sca::reduce_by_key_kernel<sca::FmtU32, sca::FmtF32, 4, 11, 6, 3, 6>(": ("reduce_by_key",
                                                                         "reduce_by_key"),
    "void sca::select_kernel<4, true, 8, 8>(": ("select_p0.5", "select"),
    "void sca::radix_scatter_kernel<unsigned int, (sca::KeyKind)0, 0, 8, 16, true>(": ("sort_u32",
                                                                                     "radix_sort"),
    "(anonymous namespace)::copy16_kernel": ("copy16", None),
}


def pmc_summary(fetch_csv, write_csv, command, select_key="select_p0.5"):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, merged into
    profiles/pmc_traffic.json (kernels absent from these CSVs keep their entries)."""
    import csv

    def read(path, counter):
        acc = {}
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                for prefix, (key, _) in KERNEL_KEYS.items():
                    if name.startswith(prefix):
                        key = select_key if key == "select_p0.5" else key
                        acc.setdefault(key, []).append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    out = {"note": "KiB per dispatch, averaged over dispatches; copy16 moved bytes/2 each way",
           "copy16": {}, "kernels": {}}
    if os.path.exists(PMC_FILE):
        with open(PMC_FILE) as fh:
            out.update(json.load(fh))
    out["copy16"] = {"bytes": HEAD_BYTES, "fetch_kib": fetch["copy16"],
                     "write_kib": write["copy16"], "command": command}
    for prefix, (key, kind) in KERNEL_KEYS.items():
        key = select_key if key == "select_p0.5" else key
        if kind and key in fetch and key in write:
            out["kernels"][key] = {"fetch_kib": fetch[key], "write_kib": write[key],
                                   "source_sha": sources_sha(kind), "command": command,
                                   "copy16": dict(out["copy16"])}
    out.pop("command", None)
    with open(PMC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


class CallTimes(list):
    """Per-call times (ms) of the eager pass, plus the graph region's average
    per call in `window_ms`."""
    window_ms = None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def gpu_facts():
    """Engine clock, GFX target and cache sizes of the first GPU node in the KFD
    topology (sysfs), and the ROCm version; each field is None where unreadable."""
    out = {"max_engine_clock_MHz": None, "gfx_target_version": None, "caches_KiB": None,
           "rocm": None}
    try:
        with open("/opt/rocm/.info/version") as fh:
            out["rocm"] = fh.read().strip()
    except OSError:
        pass
    base = "/sys/class/kfd/kfd/topology/nodes"
    try:
        for node in sorted(os.listdir(base), key=lambda x: int(x) if x.isdigit() else 1 << 30):
            props = {}
            with open(os.path.join(base, node, "properties")) as fh:
                for ln in fh:
                    k, _, v = ln.partition(" ")
                    props[k] = v.strip()
            if int(props.get("gfx_target_version", "0") or 0) == 0:
                continue                                  # a CPU node
            out["max_engine_clock_MHz"] = int(props.get("max_engine_clk_fcompute", 0)) or None
            out["gfx_target_version"] = int(props["gfx_target_version"])
            levels = {}
            cdir = os.path.join(base, node, "caches")
            for c in os.listdir(cdir):
                cp = {}
                with open(os.path.join(cdir, c, "properties")) as fh:
                    for ln in fh:
                        k, _, v = ln.partition(" ")
                        cp[k] = v.strip()
                lvl = f"L{cp.get('level', '?')}"
                levels[lvl] = max(levels.get(lvl, 0), int(cp.get("size", 0)))
            out["caches_KiB"] = dict(sorted(levels.items())) or None
            break
    except (OSError, ValueError, KeyError):
        pass
    return out


def traffic_bytes(key, kind):
    """HBM bytes per launch from the stored counter readings, scaled by what the
    same counters read for copy16; None if absent or the kernel changed since."""
    if not os.path.exists(PMC_FILE):
        return None
    try:
        with open(PMC_FILE) as fh:
            pm = json.load(fh)
        k = pm["kernels"].get(key)
        if not k or k.get("source_sha") != sources_sha(kind):
            return None
        c = k.get("copy16", pm["copy16"])
        fr = c["bytes"] / 2 / (c["fetch_kib"] * 1024)     # bytes per counted byte
        fw = c["bytes"] / 2 / (c["write_kib"] * 1024)
        return k["fetch_kib"] * 1024 * fr + k["write_kib"] * 1024 * fw
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def main():
    args = parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary[:2], command=args.pmc_command,
                    select_key=args.pmc_select_key)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: the library has no multi-GPU "
                                   "path, so --gpus must be 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import stream_compaction_amd as sc
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sc.lib()
    only = set(filter(None, args.only.split(",")))

    def want(name):
        return not only or name in only

    def timed(launch, steps, warmup):
        """Time `steps` calls of launch(i) after `warmup` untimed ones.

        Returns (wall seconds, CallTimes).  The timed region is bracketed by
        synchronizations and holds the `steps` calls back to back: captured
        once into a HIP graph and replayed (so host-side launch cost does not
        stretch short kernels), or issued one by one with --eager.  One pair
        of HIP events on the launch stream brackets the region (its average
        per call is `window_ms`); a second, eager pass brackets each call with
        its own pair of events (the list itself).  The per-call figure the
        results use is the smaller of the region average and the mean of the
        per-call pairs (both include some dispatch overhead).
        """
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        graph = None
        if not args.eager:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(steps):
                    launch(i)
            graph.replay()
            torch.cuda.synchronize()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        t0 = time.perf_counter()
        w0.record(cur)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                launch(i)
        w1.record(cur)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        window_ms = w0.elapsed_time(w1) / steps
        del graph
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            ev0[i].record(cur)
            launch(i)
            ev1[i].record(cur)
        torch.cuda.synchronize()
        per = CallTimes(a.elapsed_time(b) for a, b in zip(ev0, ev1))
        per.window_ms = window_ms
        return wall, per

    def bf16_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    results = {}

    def record(name, elems, algo_bytes, wall, per_ms, steps, note=""):
        avg_ms = float(np.mean(per_ms))
        window_ms = getattr(per_ms, "window_ms", None)
        if window_ms is not None and window_ms < avg_ms:
            avg_ms = window_ms
        r = {"elements": int(elems), "algorithmic_bytes": int(algo_bytes),
             "kernel_ms_avg": round(avg_ms, 5),
             # each call between its own pair of events (dispatch included)
             "call_ms_median": round(float(np.median(per_ms)), 5),
             "call_ms_min": round(float(np.min(per_ms)), 5),
             "elements_per_s": elems / (avg_ms * 1e-3),
             "GBps": algo_bytes / (avg_ms * 1e-3) / 1e9,
             "frac_of_peak": algo_bytes / (avg_ms * 1e-3) / 1e9 / PEAK_GBS,
             "wall_ms_per_step": wall / steps * 1e3}
        if note:
            r["note"] = note
        results[name] = r
        return r

    # ---------------- headline: i32 device-wide exclusive add scan, n = 2^28 ----------------
    head = None
    n_head = wl.FULL["dev_i32"]
    head_bytes = n_head * 4 * 2
    assert head_bytes == HEAD_BYTES
    x_head = wl.dev_i32()
    if want("dev_i32_add"):
        xs = [torch.from_numpy(x_head).to(dev) for _ in range(args.sets)]
        ys = [torch.empty_like(xs[0]) for _ in range(args.sets)]
        s_head = torch.empty(sc.scan_device_scratch_bytes(n_head, "i32"), dtype=torch.uint8,
                             device=dev)
        wall, per = timed(lambda i: sc.scan_device(xs[i % args.sets], "add", ys[i % args.sets],
                                                   s_head), args.steps, args.warmup)
        head = record("dev_i32_add", n_head, head_bytes, wall, per, args.steps,
                      "includes the descriptor-reset fill kernel")
        head["wall_s"] = wall
        del xs, ys

    # ---------------- the other workloads ----------------
    K, W = args.sub_steps, 3
    rows, n = wl.FULL["rows_bf16"]
    if want("rows_bf16_excl"):
        xb = wl.rows_bf16(rows, n)
        xs = [bf16_dev(xb) for _ in range(args.sets)]
        ys = [torch.empty_like(xs[0]) for _ in range(args.sets)]
        wall, per = timed(lambda i: sc.scan_rows(xs[i % args.sets], "add", True, ys[i % args.sets]),
                          K, W)
        record("rows_bf16_excl", rows * n, rows * n * 4, wall, per, K)
        del xs, ys
    if want("rows_bf16_ragged_excl"):
        r2, n2 = wl.FULL["rows_bf16_ragged"]
        xb2 = wl.rows_bf16(r2, n2)
        xs = [bf16_dev(xb2) for _ in range(args.sets)]
        ys = [torch.empty_like(xs[0]) for _ in range(args.sets)]
        wall, per = timed(lambda i: sc.scan_rows(xs[i % args.sets], "add", True, ys[i % args.sets]),
                          K, W)
        record("rows_bf16_ragged_excl", r2 * n2, r2 * n2 * 4, wall, per, K)
        del xs, ys
    r1, n1 = wl.FULL["rows_f32"]
    for excl in (False, True):
        name = "rows_f32_" + ("excl" if excl else "incl")
        if not want(name):
            continue
        x1 = torch.from_numpy(wl.rows_f32(r1, n1)).to(dev)
        sets = max(args.sets, 32)          # 32 MiB per set: rotate over >= 1 GiB
        xs = [x1.clone() for _ in range(sets)]
        ys = [torch.empty_like(x1) for _ in range(sets)]
        wall, per = timed(lambda i: sc.scan_rows(xs[i % sets], "add", excl, ys[i % sets]), K, W)
        record(name, r1 * n1, r1 * n1 * 8, wall, per, K)
        del xs, ys
    for name, n3 in (("dev_i32_add_odd", wl.FULL["dev_i32_odd"]),):
        if not want(name):
            continue
        x3 = torch.from_numpy(x_head[:n3]).to(dev)
        y3 = torch.empty_like(x3)
        s3 = torch.empty(sc.scan_device_scratch_bytes(n3, "i32"), dtype=torch.uint8, device=dev)
        wall, per = timed(lambda i: sc.scan_device(x3, "add", y3, s3), K, W)
        record(name, n3, n3 * 8, wall, per, K, "includes the descriptor-reset fill kernel")
        del x3, y3
    for which in ("f32", "i64"):
        if not any(want(f"dev_{which}_{op}") for op in ("min", "max")):
            continue
        x4 = torch.from_numpy(wl.dev_f32() if which == "f32" else wl.dev_i64()).to(dev)
        y4 = torch.empty_like(x4)
        s4 = torch.empty(sc.scan_device_scratch_bytes(x4.numel(), which), dtype=torch.uint8,
                         device=dev)
        for op in ("min", "max"):
            name = f"dev_{which}_{op}"
            if want(name):
                wall, per = timed(lambda i: sc.scan_device(x4, op, y4, s4), K, W)
                record(name, x4.numel(), x4.numel() * x4.element_size() * 2, wall, per, K,
                       "includes the descriptor-reset fill kernel")
        del x4, y4
    if want("rows_bf16_prod_excl"):
        xp2 = wl.prod_rows_bf16(rows, n)
        xs = [bf16_dev(xp2) for _ in range(args.sets)]
        ys = [torch.empty_like(xs[0]) for _ in range(args.sets)]
        wall, per = timed(lambda i: sc.scan_rows(xs[i % args.sets], "mul", True, ys[i % args.sets]),
                          K, W)
        record("rows_bf16_prod_excl", rows * n, rows * n * 4, wall, per, K,
               "product scan, factors +-(1 + U[-1/64, 1/64)) in bf16, seed 12")
        del xs, ys
    if want("dev_i32_add_incl"):
        n3 = wl.FULL["dev_i32"]
        x3 = torch.from_numpy(x_head).to(dev)
        y3 = torch.empty_like(x3)
        s3 = torch.empty(sc.scan_device_scratch_bytes(n3, "i32"), dtype=torch.uint8, device=dev)
        wall, per = timed(lambda i: sc.scan_device_inclusive(x3, "add", y3, s3), K, W)
        record("dev_i32_add_incl", n3, n3 * 8, wall, per, K,
               "inclusive form; includes the descriptor-reset fill kernel")
        del x3, y3
    red_cases = (("reduce_i32_add", "i32", "add"), ("reduce_f32_add", "f32", "add"),
                 ("reduce_f32_min", "f32", "min"), ("reduce_i64_max", "i64", "max"))
    for name, which, op in red_cases:
        if not want(name):
            continue
        src = {"i32": wl.dev_i32, "f32": wl.dev_f32, "i64": wl.dev_i64}[which]()
        x5 = torch.from_numpy(src).to(dev)
        y5 = torch.empty(1, dtype=x5.dtype, device=dev)
        s5 = torch.empty(max(16, sc.reduce_device_scratch_bytes(x5.numel(), which)),
                         dtype=torch.uint8, device=dev)
        wall, per = timed(lambda i: sc.reduce_device(x5, op, y5, s5), K, W)
        record(name, x5.numel(), x5.numel() * x5.element_size(), wall, per, K,
               "algorithmic bytes = n elements read; includes the one-wave final kernel")
        del x5, y5
    if want("reduce_by_key"):
        nk = wl.FULL["rbk"]
        kk, vv = wl.rbk_inputs(nk)
        kd, vd = torch.from_numpy(kk).to(dev), torch.from_numpy(vv).to(dev)
        ko, vo = torch.empty_like(kd), torch.empty_like(vd)
        nr = torch.empty(1, dtype=torch.int32, device=dev)
        sk = torch.empty(sc.reduce_by_key_scratch_bytes(nk), dtype=torch.uint8, device=dev)
        wall, per = timed(lambda i: sc.reduce_by_key(kd, vd, ko, vo, nr, sk), K, W)
        runs = int(nr.item())
        r = record("reduce_by_key", nk, nk * 8 + runs * 8 + 4, wall, per, K,
                   "i32 keys in runs of mean length 8, f32 values; algorithmic bytes = 8n read "
                   "+ 8 per run written + 4; includes the descriptor-reset fill kernel")
        r["runs"] = runs
        del kd, vd, ko, vo
    for name, with_vals in (("sort_u32", False), ("sort_u32_kv", True)):
        if not want(name):
            continue
        # the sort works in place, so every call starts from a fresh copy of the
        # unsorted keys, made before the call's own pair of HIP events
        ns = wl.FULL["sort"]
        k0 = torch.from_numpy(wl.sort_keys_u32(ns).view(np.int32)).to(dev)
        kk, tk = torch.empty_like(k0), torch.empty_like(k0)
        v0 = torch.arange(ns, dtype=torch.int32, device=dev) if with_vals else None
        vv = torch.empty_like(k0) if with_vals else None
        tv = torch.empty_like(k0) if with_vals else None
        scr = torch.empty(sc.radix_sort_scratch_bytes(ns, "u32"), dtype=torch.uint8, device=dev)
        per = []
        cur = torch.cuda.current_stream()
        t_all = 0.0
        for i in range(W + K):
            kk.copy_(k0)
            if with_vals:
                vv.copy_(v0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            sc.radix_sort(kk, vv, tk, tv, 32, scr, key_dtype="u32", value_dtype="i32")
            e1.record(cur)
            torch.cuda.synchronize()
            if i >= W:
                per.append(e0.elapsed_time(e1))
                t_all += per[-1] * 1e-3
        eb = 8 if with_vals else 4                      # bytes moved per element per pass, each way
        record(name, ns, 4 * 2 * eb * ns + 4 * ns, t_all, per, K,
               "2^28 uniform u32 keys" + (" with i32 values" if with_vals else ", keys only") +
               "; algorithmic bytes = 4 passes x (read + write of keys" +
               (" and values" if with_vals else "") + ") + one read of the keys for the "
               "digit histograms; eager calls, each after an untimed copy of the unsorted input")
        results[name]["keys_per_s"] = ns / float(np.mean(per) * 1e-3)
        del k0, kk, tk, v0, vv, tv
    nsel = wl.FULL["sel"]
    for p in wl.SELECT_P:
        name = f"select_p{p}"
        if not want(name):
            continue
        pay, fl = wl.sel_inputs(nsel, p)
        xp = torch.from_numpy(pay).to(dev)
        xf = torch.from_numpy(fl).to(dev)
        yo = torch.empty_like(xp)
        num = torch.empty(1, dtype=torch.int32, device=dev)
        ss = torch.empty(sc.select_compact_scratch_bytes(nsel), dtype=torch.uint8, device=dev)
        wall, per = timed(lambda i: sc.select_compact(xp, xf, yo, num, ss), K, W)
        k = int(num.item())
        r = record(name, nsel, nsel * 5 + 4 * k + 4, wall, per, K,
                   "algorithmic bytes = 4n payload + n flags read, 4k written, 4 count (what a "
                   "kernel that reads every payload element moves).  The kernel loads a payload "
                   "vector only if one of its elements is selected, so at low p it moves fewer "
                   "bytes and this figure can exceed the HBM peak; min_bytes counts the flags, "
                   "the 128-byte payload lines (the L2 line, the unit HBM reads are counted in) "
                   "that hold a selected element, and the output")
        r["kept"] = k
        r["read_n_plus_write_n_GBps"] = nsel * 8 / (r["kernel_ms_avg"] * 1e-3) / 1e9
        lines = int(fl[: nsel // 32 * 32].reshape(-1, 32).any(axis=1).sum())
        if nsel % 32:
            lines += int(fl[nsel // 32 * 32:].any())
        r["min_bytes"] = nsel + 128 * lines + 4 * k + 4
        r["min_bytes_GBps"] = r["min_bytes"] / (r["kernel_ms_avg"] * 1e-3) / 1e9
        r["min_bytes_frac_of_peak"] = r["min_bytes_GBps"] / PEAK_GBS
        del xp, xf, yo

    # ---------------- copy ceiling over the headline's bytes ----------------
    copy = None
    if want("copy16"):
        import ctypes
        from stream_compaction_amd import build as _b
        cl = ctypes.CDLL(_b.COPY_LIB_PATH)
        cl.copy_ceiling_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_void_p]
        half = head_bytes // 2
        srcs = [torch.empty(half, dtype=torch.uint8, device=dev).fill_(1) for _ in range(args.sets)]
        dsts = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(args.sets)]

        def cp(i):
            rc = cl.copy_ceiling_copy16(ctypes.c_void_p(srcs[i % args.sets].data_ptr()),
                                        ctypes.c_void_p(dsts[i % args.sets].data_ptr()), half,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert rc == 0, rc
        wall, per = timed(cp, args.steps, args.warmup)
        copy = record("copy16", half // 4, head_bytes, wall, per, args.steps,
                      "16-byte copy kernel moving the headline's read+write bytes")
        del srcs, dsts

    # ---------------- CPU oracle baseline on the headline workload ----------------
    # The oracle is a sequential left fold, so it runs on one core; the whole
    # 2^28-element workload takes well under a second per run.
    cpu = None
    if not args.no_cpu and head is not None:
        import oracle
        times = []
        for _ in range(5):
            t0 = time.perf_counter()
            oracle.scan(x_head, "i32", "add", exclusive=True)
            times.append(time.perf_counter() - t0)
        t = float(np.median(times))
        cpu = {"value": n_head / t, "unit": "elements/s", "cores": 1, "kind": "oracle",
               "sample": f"the full workload: exclusive add scan of the same 2^28 i32 values "
                         f"(seed 2) on one core, median of 5 runs ({t:.3f} s each)",
               "cpu": cpu_model()}

    # ---------------- stored counter readings -> HBM traffic per launch ----------------
    traffic = traffic_bytes("dev_i32_add", "scan_device")
    for key, kind in (("rows_bf16_excl", "scan_rows"), ("select_p0.5", "select"),
                      ("select_p0.01", "select"),
                      ("reduce_i32_add", "reduce"), ("reduce_by_key", "reduce_by_key")):
        t = traffic_bytes(key, kind)
        if key in results and t is not None:
            results[key]["traffic_bytes"] = t
            results[key]["traffic_over_algorithmic"] = t / results[key]["algorithmic_bytes"]
    t = traffic_bytes("sort_u32", "radix_sort")
    if "sort_u32" in results and t is not None:
        # one digit pass's scatter kernel, against its read + write of the keys
        per_pass = 8 * results["sort_u32"]["elements"]
        results["sort_u32"]["scatter_traffic_bytes"] = t
        results["sort_u32"]["scatter_traffic_over_8n"] = t / per_pass

    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": METRIC,
        "value": (n_head * args.steps / head["wall_s"]) if head else None,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (head["wall_s"] / args.steps * 1e3) if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32",
        "data": "synthetic",
        "config": {"workload": "device-wide exclusive add scan of a flat i32 array, n = 2^28, "
                               "values uniform integers in [0, 15] (seed 2)",
                   "n": n_head, "io_dtype": "i32", "op": "add", "exclusive": True,
                   "buffer_sets": args.sets},
    }
    if head:
        achieved = head_bytes / (head["kernel_ms_avg"] * 1e-3) / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                            "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                            "traffic": traffic,
                            "kernel": "scan_device_kernel<i32, add, exclusive> with its "
                                      "descriptor-reset fill kernel (the whole call)",
                            "bytes_per_launch": head_bytes}
        if copy:
            line["roofline"]["copy16_GBps"] = round(copy["GBps"], 1)
            line["roofline"]["frac_of_copy16"] = round(achieved / copy["GBps"], 4)
    line["cpu_baseline"] = cpu
    line["workloads"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                             for kk, vv in v.items() if kk != "wall_s"}
                         for k, v in results.items()}
    line["device"] = {"name": props.name, "cus": props.multi_processor_count,
                      "hbm_GiB": round(props.total_memory / 2**30, 1),
                      "l2_bytes": getattr(props, "L2_cache_size", None),
                      "arch": getattr(props, "gcnArchName", None),
                      "torch": torch.__version__, "hip": torch.version.hip, **gpu_facts()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
