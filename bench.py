"""Benchmark of the fused dequant-GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--m M]

One step is one fused dequant + GEMV (or GEMM) launch over one activation
batch, with the packed weights already resident in HBM.  Weight copies are
rotated so every step streams its weights from HBM rather than from the
256 MB Infinity Cache.  The K timed launches are replayed from a HIP graph on
one stream and bracketed by HIP events on that stream.  Prints one JSON line.

Extra reports: ``--all`` times every workload and activation count and
writes a markdown table (stderr, and ``--report PATH``).
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

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, published
METRIC = "dequant-GEMV weight GB/s & % HBM peak, INT4 g64 K=4096 N=11008 M=1"
_CSRC = "gemm_group_wise_amd/csrc/"
KERNEL_SOURCES = {  # what the timed kernel of each path is built from
    "gemv": [_CSRC + f for f in ("gemv_impl.hpp", "gemv_mfma.hpp", "device_common.hpp", "gemv.hip", "gemv_int2.hip",
                                 "gemv_int4.hip", "gemv_int8.hip", "gemv_nf4.hip")],
    "gemm": [_CSRC + f for f in ("gemm.hip", "device_common.hpp")],
}
CALIBRATION_MIB = 512          # plain copy used to scale the HBM byte counters


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def weight_bytes(wl: workloads.Workload) -> int:
    bits = {"int2": 2, "int4": 4, "int8": 8, "nf4": 4}[wl.scheme]
    per_group = 2 if wl.scheme == "nf4" else 4
    return wl.n * wl.k * bits // 8 + wl.n * (wl.k // wl.group) * per_group


def kernel_source_hash(path: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def graph_of(launch, count: int, start: int = 0):
    """A HIP graph of `count` calls launch(i, stream) on a side stream (one
    call made first, outside the capture, to warm the launch path)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch(start, s.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                launch(start + i, s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_graph(launch, rotate: int, steps: int, warmup: int) -> float:
    """ms per call over exactly `steps` calls replayed from graphs of `rotate`
    calls, between HIP events recorded on the stream the replays run on."""
    import torch
    full = graph_of(launch, rotate)
    rem = graph_of(launch, steps % rotate) if steps % rotate else None
    stream = torch.cuda.current_stream()
    for _ in range(max(1, math.ceil(warmup / rotate))):
        full.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps // rotate):
        full.replay()
    if rem is not None:
        rem.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def per_launch_stats(launch, count: int) -> dict:
    """Eager launches, each between its own pair of HIP events on the launch
    stream: median / min / p90 of the per-launch durations in us."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(count)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        launch(i, stream.cuda_stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return {"median_us": round(statistics.median(us), 3), "min_us": round(us[0], 3),
            "p90_us": round(us[min(len(us) - 1, int(0.9 * len(us)))], 3), "launches": count}


class Setup:
    """Packed weights (rotated device copies), activations and output for one workload."""

    def __init__(self, uq, wl: workloads.Workload, m: int, rotate: int | None, a8: bool = False):
        import torch
        self.uq, self.wl, self.m, self.a8 = uq, wl, m, a8
        if wl.gguf:   # GGUF blocks, re-laid on the host into the INT layout
            blob, x = workloads.make_gguf_workload(wl)
            self.w_host, self.x_host = blob.reshape(wl.n, -1), x[:m]
            self.lay, codes, params = uq.uq_import_gguf(wl.gguf, blob, wl.n, wl.k)
        else:
            w, x = workloads.make_workload(wl)
            self.w_host, self.x_host = w, x[:m]
            self.lay = uq.layout(wl.scheme, wl.group, wl.n, wl.k)
            codes, params = uq.uq_pack_weights(self.lay, w)
        self.codes_host, self.params_host = codes, params
        self.bytes = codes.nbytes + params.nbytes
        if rotate is None:  # > 256 MB Infinity Cache + 32 MB L2
            rotate = max(16, math.ceil(320e6 / self.bytes))
        self.rotate = rotate
        dc, dp = torch.from_numpy(codes).cuda(), torch.from_numpy(params.view(np.int16)).cuda()
        self.codes = [dc] + [dc.clone() for _ in range(rotate - 1)]
        self.params = [dp] + [dp.clone() for _ in range(rotate - 1)]
        if self.x_host.shape[0] != m:
            raise ValueError(f"{wl.name}: M = {m} but the workload's x has {self.x_host.shape[0]} rows")
        self.x = torch.from_numpy(np.ascontiguousarray(self.x_host)).cuda()
        self.y = torch.empty(m * wl.n, dtype=torch.float32, device="cuda")
        self.fn = uq.uq_gemv_a8 if a8 else (uq.uq_gemv if wl.path == "gemv" else uq.uq_gemm)
        # the GEMM's workspace: allocated zero-filled once, reused by every launch on the one stream
        self.ws = uq.gemm_workspace(self.lay, m) if self.fn is uq.uq_gemm else None
        torch.cuda.synchronize()

    def launch(self, i: int, stream: int) -> None:
        j = i % self.rotate
        if self.ws is not None:
            self.fn(self.lay, self.codes[j], self.params[j], self.x, self.y, self.m, self.ws, stream=stream)
        else:
            self.fn(self.lay, self.codes[j], self.params[j], self.x, self.y, self.m, stream=stream)

    def time(self, steps: int, warmup: int):
        """(ms per step, eager ms per step) over exactly `steps` launches."""
        import torch
        ms = time_graph(self.launch, self.rotate, steps, warmup)
        # eager cross-check (host launch overhead included)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_eager = min(steps, 4 * self.rotate)
        sp = stream.cuda_stream
        e0.record(stream)
        for i in range(n_eager):
            self.launch(i, sp)
        e1.record(stream)
        torch.cuda.synchronize()
        return ms, e0.elapsed_time(e1) / n_eager

    def check_sample(self, rows: int = 96, seed: int = 1) -> float:
        """Sampled parity of the timed output: oracle on `rows` random weight rows."""
        import oracle as o
        torch_y = self.y.cpu().numpy().reshape(self.m, self.wl.n)
        idx = np.sort(np.random.default_rng(seed).choice(self.wl.n, min(rows, self.wl.n), replace=False))
        if self.wl.gguf:
            blob = self.w_host[idx].reshape(-1)
            wdq = o.decode_gguf(blob, self.wl.gguf, idx.size, self.wl.k).astype(np.float32)
        else:
            codes, params = o.quantize_pack(self.w_host[idx], self.wl.scheme, self.wl.group)
            wdq = o.dequant_packed(codes, params, self.wl.scheme, self.wl.group, self.wl.k)
        if self.a8:
            if self.wl.gguf:
                q_w, s16, z16 = o.gguf_as_int(blob, self.wl.gguf, idx.size, self.wl.k)
            else:
                q_w, s16, z16 = o.quantize_int(self.w_host[idx], o.BITS[self.wl.scheme], self.wl.group)
            q_x, s_x = o.quantize_activations(self.x_host, self.wl.group)
            ref = o.gemv_a8_ref(q_x, s_x, q_w, s16, z16, self.wl.group)
            xs, ws = o.dequant_activations(q_x, s_x, self.wl.group), wdq
        elif self.wl.path == "gemv":
            ref, xs, ws = o.gemv_ref(self.x_host, wdq), self.x_host, wdq
        else:
            ref = o.gemm_ref(self.x_host, wdq)
            xs, ws = o.bf16_rne(self.x_host.astype(np.float32)), o.bf16_rne(wdq)
        got = torch_y[:, idx].astype(np.float64)
        err = got - ref
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
        bound = 2e-3 * math.sqrt(self.wl.k) * float(np.abs(xs).max()) * float(np.abs(ws).max())
        if not (rel <= 1e-3 and float(np.abs(err).max()) <= bound):
            raise SystemExit(f"bench output fails parity on sampled rows: rel-L2 {rel:.3e}")
        return rel


def cpu_baseline(wl: workloads.Workload, m: int, nbytes: int) -> dict:
    """The oracle (unpack + dequant + fp64 product) on the same matrix, on host cores."""
    import oracle as o
    ref = o.gemv_ref if wl.path == "gemv" else o.gemm_ref
    if wl.gguf:
        blob, x = workloads.make_gguf_workload(wl)
        xs = x[:m]

        def run():
            return ref(xs, o.decode_gguf(blob, wl.gguf, wl.n, wl.k))
    else:
        w, x = workloads.make_workload(wl)
        codes, params = o.quantize_pack(w, wl.scheme, wl.group)   # offline for both sides
        xs = x[:m]

        def run():
            return ref(xs, o.dequant_packed(codes, params, wl.scheme, wl.group, wl.k))

    run()
    times = []
    budget = time.perf_counter() + 30.0
    for _ in range(5):
        t = time.perf_counter()
        run()
        times.append(time.perf_counter() - t)
        if time.perf_counter() > budget:
            break
    med = statistics.median(times)
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the pool size numpy was built with
        blas = os.cpu_count() or 1
    return {"value": round(nbytes / med / 1e9, 4), "unit": "GB/s", "cores": int(blas),
            "host_cores": os.cpu_count(), "blas_threads": int(blas), "kind": "oracle",
            "sample": (f"whole {wl.name} matrix, M={m}: NumPy unpack + dequant + fp64 product, "
                       f"median of {len(times)} runs after 1 warm-up ({med * 1e3:.0f} ms each); "
                       f"elementwise steps single-threaded, product on {blas} BLAS threads")}


def traffic_path(name: str, m: int, ext: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{name}_m{m}.{ext}")


def traffic_for(wl: workloads.Workload, m: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = traffic_path(wl.name, m, "json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(wl.path):
        return None
    return t.get("hbm_bytes_per_launch")


def traffic_run(uq, wl: workloads.Workload, m: int, launches: int) -> None:
    """The workload's kernel `launches` times (eager, rotated weights), then a plain
    copy of CALIBRATION_MIB MiB five times; run under rocprofv3 --pmc."""
    import torch
    st = Setup(uq, wl, m, None)
    sp = torch.cuda.current_stream().cuda_stream
    for i in range(launches):
        st.launch(i, sp)
    torch.cuda.synchronize()
    n = CALIBRATION_MIB * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)   # reads and writes CALIBRATION_MIB MiB
    torch.cuda.synchronize()
    log(f"traffic run: {launches} launches of {wl.name} m={m}, 5 calibration copies")


def _counter_rows(directory: str, counter: str):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_parse(wl: workloads.Workload, m: int, fetch_dir: str, write_dir: str, cmds: list[str]) -> dict:
    """Scale the kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the
    same counters read for the calibration copy, and store the result."""
    kernel = "gemv_" if wl.path == "gemv" else "gemm_"  # the dot-product, matrix-core or streaming kernel
    known = CALIBRATION_MIB * 2**20
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        kv = [v for name, v in rows if kernel in name]
        cv = [v for name, v in rows if "elementwise" in name and "MulFunctor" in name]
        if not kv or not cv:
            raise SystemExit(f"{counter}: kernel or calibration dispatches missing in {d}")
        kib, cal = statistics.median(kv), statistics.median(cv)
        factor = known / (cal * 1024.0)
        out[counter] = {"kernel_kib_per_dispatch": kib, "dispatches": len(kv),
                        "calibration_kib": cal, "calibration_bytes": known, "scale": round(factor, 4),
                        "bytes_per_launch": round(kib * 1024.0 * factor)}
    alg = weight_bytes(wl)
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    t = {"workload": wl.name, "m": m, "kernel": kernel, "kernel_source_hash": kernel_source_hash(wl.path),
         "hbm_bytes_per_launch": total, "algorithmic_weight_bytes": alg,
         "traffic_over_algorithmic": round(total / alg, 4), "counters": out, "commands": cmds}
    with open(traffic_path(wl.name, m, "json"), "w") as f:
        json.dump(t, f, indent=1)
    f_, w_ = out["FETCH_SIZE"], out["WRITE_SIZE"]
    md = [f"# HBM traffic of the {wl.path} kernel: {wl.name}, M={m}", "",
          "Commands (MI355X host, repository root), one counter per run:", ""] + [f"    {c}" for c in cmds] + [
          "", "| counter | kernel KiB/dispatch (median) | dispatches | calibration copy KiB | scale | bytes/launch |",
          "|---|---|---|---|---|---|",
          f"| FETCH_SIZE | {f_['kernel_kib_per_dispatch']:.1f} | {f_['dispatches']} | {f_['calibration_kib']:.0f} | "
          f"{f_['scale']} | {f_['bytes_per_launch']:,} |",
          f"| WRITE_SIZE | {w_['kernel_kib_per_dispatch']:.1f} | {w_['dispatches']} | {w_['calibration_kib']:.0f} | "
          f"{w_['scale']} | {w_['bytes_per_launch']:,} |", "",
          f"The calibration copy is torch.mul(src, 1.0, out=dst) over {CALIBRATION_MIB} MiB (reads and writes "
          f"{known:,} bytes); scale = known bytes / counter bytes for that copy.  HBM traffic per launch "
          f"{total:,} bytes against {alg:,} algorithmic weight bytes ({total / alg:.3f}x).", ""]
    with open(traffic_path(wl.name, m, "md"), "w") as f:
        f.write("\n".join(md))
    log("\n".join(md))
    return t


class ReadProbe:
    """The streaming-read ceiling: uq_probe_read over rotated device buffers of a given size."""

    def __init__(self, uq, nbytes: int, rotate: int):
        import torch
        self.uq, self.nbytes, self.rotate = uq, nbytes, rotate
        g = torch.Generator(device="cuda").manual_seed(0)
        self.bufs = [torch.randint(0, 256, (max(nbytes, 1024),), dtype=torch.uint8, device="cuda", generator=g)
                     for _ in range(rotate)]
        self.sink = torch.zeros(4 << 20, dtype=torch.int32, device="cuda")
        self.wg, self.un = 1024, 8

    def launch(self, i: int, stream: int) -> None:
        self.uq.uq_probe_read(self.bufs[i % self.rotate], self.nbytes, self.wg, self.un, self.sink, stream=stream)

    def time(self, wg: int, un: int, steps: int, warmup: int) -> float:
        self.wg, self.un = wg, un
        return time_graph(self.launch, self.rotate, steps, warmup)


def probe_grids(nbytes: int) -> list:
    """Workgroup counts to try for a read of nbytes: whole multiples of the 256
    CUs, and the GEMV's own grid shape (one workgroup per 16 weight rows of 2304 B)."""
    grids = [256, 512, 768, 1024, 2048, 4096]
    gemv_like = math.ceil(nbytes / (16 * 2304))
    return sorted(set(g for g in grids + [gemv_like] if 4 * g <= nbytes // 1024 or g == 256))


def ceiling_line(uq, nbytes: int, steps: int, warmup: int) -> dict:
    """The best plain read of nbytes (rotated copies, graph-timed like the GEMV)
    over a few grid shapes, plus an empty launch; for the JSON line."""
    rotate = max(16, math.ceil(320e6 / nbytes))
    pr = ReadProbe(uq, nbytes, rotate)
    best = None
    for wg in (256, 512, 688, 1024):
        for un in (8, 16):
            ms = pr.time(wg, un, steps, warmup)
            if best is None or ms < best[0]:
                best = (ms, wg, un)
    empty = ReadProbe(uq, 0, 16)  # graphs of 16 launches, like the reads: per-launch cost, not replay overhead
    ms_empty = empty.time(256, 8, steps, warmup)
    del pr, empty
    ms, wg, un = best
    return {"plain_read_us": round(ms * 1e3, 3), "plain_read_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "workgroups": wg, "loads_in_flight": un, "empty_launch_us": round(ms_empty * 1e3, 3),
            "bytes": nbytes, "rotated_copies": rotate}


def report_ceiling(uq, steps: int, warmup: int, path: str | None) -> dict:
    """Plain reads of the headline's weight bytes and of 1 GiB, an empty launch,
    and the headline GEMV, all timed the same way in one run (markdown)."""
    cmd = "python bench.py " + " ".join(sys.argv[1:])
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    nbytes = weight_bytes(wl)
    rows = ["# Streaming-read ceiling of one launch", "",
            "uq_probe_read reads every byte once with the GEMV's load pattern (wave-wide 128-bit non-temporal "
            "loads, 1 KB per wave instruction, equal contiguous runs per wave).  Buffers are rotated so every "
            "launch streams from HBM; each time is HIP events around graph-replayed launches, like the bench line.",
            "", "Command (MI355X host, repository root):", "", f"    {cmd}", "",
            "| read | bytes | workgroups | loads in flight per lane | us/launch | GB/s | % of 8 TB/s |",
            "|---|---|---|---|---|---|---|"]
    out = {}
    for label, size in (("headline weight bytes", nbytes), ("1 GiB", 1 << 30)):
        rotate = max(2, math.ceil(320e6 / size)) if size < (1 << 30) else 2
        rotate = max(rotate, 16) if size < (1 << 30) else rotate
        pr = ReadProbe(uq, size, rotate)
        st = steps if size < (1 << 30) else max(20, steps // 100)
        best = None
        for wg in probe_grids(size):
            for un in (4, 8, 16, 32):
                ms = pr.time(wg, un, st, min(warmup, st))
                gbs = size / (ms * 1e-3) / 1e9
                rows.append(f"| {label} | {size:,} | {wg} | {un} | {ms * 1e3:.3f} | {gbs:.0f} | "
                            f"{100 * gbs / HBM_PEAK_GBS:.1f} |")
                log(rows[-1])
                if best is None or ms < best[0]:
                    best = (ms, wg, un)
        out[label] = {"us": round(best[0] * 1e3, 3), "gbs": round(size / (best[0] * 1e-3) / 1e9, 1),
                      "workgroups": best[1], "loads_in_flight": best[2]}
        del pr
    pr = ReadProbe(uq, 0, 16)  # graphs of 16 launches, like the reads
    ms = pr.time(256, 8, steps, warmup)
    rows.append(f"| empty launch (reads nothing) | 0 | 256 | - | {ms * 1e3:.3f} | - | - |")
    out["empty launch us"] = round(ms * 1e3, 3)
    del pr
    st = Setup(uq, wl, 1, None)
    ms_gemv, _ = st.time(steps, warmup)
    gbs = nbytes / (ms_gemv * 1e-3) / 1e9
    best = out["headline weight bytes"]
    rows += ["", f"Headline GEMV ({wl.name}, M=1) in the same run: {ms_gemv * 1e3:.3f} us/launch, {gbs:.0f} GB/s = "
             f"{100 * gbs / HBM_PEAK_GBS:.1f} % of 8 TB/s = {100 * best['us'] / (ms_gemv * 1e3):.1f} % of the best "
             f"plain read of the same bytes ({best['us']:.3f} us, {best['workgroups']} workgroups, "
             f"{best['loads_in_flight']} loads in flight per lane)."]
    out["gemv_us"] = round(ms_gemv * 1e3, 3)
    text = "\n".join(rows) + "\n"
    log(text)
    if path:
        with open(path, "w") as f:
            f.write(text)
    return out


def trace_summary(directory: str, name: str, cmds: list[str], kernel_hint: str, path_key: str | None) -> None:
    """Per-kernel duration statistics (count, median, min, p90, mean) and
    resources (VGPR, AGPR, SGPR, LDS, scratch, grid) from a rocprofv3
    --kernel-trace CSV, written to profiles/NAME.md and .json.  With path_key
    (gemv / gemm) the kernel-source hash is stored, so the bench line can tell
    whether the trace still describes the built kernel."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {directory}")
    by = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                k = r["Kernel_Name"]
                d = by.setdefault(k, {"ns": [], "res": r})
                d["ns"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    kernels = {}
    for k, d in by.items():
        ns = sorted(d["ns"])
        r = d["res"]
        kernels[k] = {"dispatches": len(ns), "median_us": round(statistics.median(ns) / 1e3, 3),
                      "min_us": round(ns[0] / 1e3, 3), "p90_us": round(ns[min(len(ns) - 1, int(0.9 * len(ns)))] / 1e3, 3),
                      "mean_us": round(statistics.fmean(ns) / 1e3, 3),
                      "vgpr": int(r.get("VGPR_Count", 0) or 0), "agpr": int(r.get("Accum_VGPR_Count", 0) or 0),
                      "sgpr": int(r.get("SGPR_Count", 0) or 0), "lds_bytes": int(r.get("LDS_Block_Size", 0) or 0),
                      "scratch_bytes": int(r.get("Scratch_Size", 0) or 0),
                      "workgroup": int(r.get("Workgroup_Size_X", 0) or 0), "grid": int(r.get("Grid_Size_X", 0) or 0)}
    order = sorted(kernels, key=lambda k: -kernels[k]["dispatches"] * kernels[k]["median_us"])
    t = {"name": name, "commands": cmds, "kernels": kernels}
    if path_key:
        t["kernel_source_hash"] = kernel_source_hash(path_key)
        hits = [k for k in order if kernel_hint in k]
        t["main_kernel"] = hits[0] if hits else None
    with open(os.path.join(ROOT, "profiles", f"{name}.json"), "w") as f:
        json.dump(t, f, indent=1)
    md = [f"# Kernel trace: {name}", "", "Commands (MI355X host, repository root):", ""] + \
         [f"    {c}" for c in cmds] + ["",
         "Durations from rocprofv3 --kernel-trace (End - Start per dispatch, warm-up and capture launches "
         "included); resources as the trace records them per kernel (VGPR counts in registers per lane, "
         "LDS in bytes per workgroup; grid in threads).", "",
         "| kernel | dispatches | median us | min us | p90 us | mean us | VGPR | AGPR | SGPR | LDS B | scratch B | "
         "wg | grid |", "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in order:
        v = kernels[k]
        md.append(f"| `{k[:110]}` | {v['dispatches']} | {v['median_us']} | {v['min_us']} | {v['p90_us']} | "
                  f"{v['mean_us']} | {v['vgpr']} | {v['agpr']} | {v['sgpr']} | {v['lds_bytes']} | "
                  f"{v['scratch_bytes']} | {v['workgroup']} | {v['grid']} |")
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    log("\n".join(md))


def counter_summary(dirs: list[str], name: str, cmds: list[str], kernel_hint: str, title: str) -> None:
    """Median per-dispatch value of every counter collected for the kernels whose
    name contains kernel_hint, over one or more rocprofv3 --pmc output folders
    (one per pass); written to profiles/NAME.md and .json."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for fn in files:
            with open(fn) as f:
                for r in csv.DictReader(f):
                    if kernel_hint in r["Kernel_Name"]:
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {kernel_hint!r}")
    med = {c: statistics.median(v) for c, v in vals.items()}
    with open(os.path.join(ROOT, "profiles", f"{name}.json"), "w") as f:
        json.dump({"name": name, "kernel_hint": kernel_hint, "commands": cmds,
                   "median_per_dispatch": med, "dispatches": {c: len(v) for c, v in vals.items()}}, f, indent=1)
    md = [f"# Counters: {title}", "", "Commands (MI355X host, repository root), one pass each:", ""] + \
         [f"    {c}" for c in cmds] + ["", f"Median per dispatch of kernels matching `{kernel_hint}`:", "",
                                      "| counter | median per dispatch | dispatches |", "|---|---|---|"]
    for c in sorted(med):
        md.append(f"| {c} | {med[c]:,.0f} | {len(vals[c])} |")
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    log("\n".join(md))


def committed_trace(wl, m: int):
    """Median / min / p90 of the timed kernel from the committed trace summary,
    if it was taken from the kernel sources as they are now."""
    path = os.path.join(ROOT, "profiles", f"trace_{wl.name}_m{m}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(wl.path) or not t.get("main_kernel"):
        return None
    k = t["kernels"][t["main_kernel"]]
    return {"median_us": k["median_us"], "min_us": k["min_us"], "p90_us": k["p90_us"],
            "dispatches": k["dispatches"], "vgpr": k["vgpr"], "lds_bytes": k["lds_bytes"],
            "source": f"profiles/trace_{wl.name}_m{m}.md"}


class NormRopeSetup:
    """Fused RMSNorm + RoPE inputs (rotated device copies of x and y) for one workload."""

    def __init__(self, uq, wl: workloads.NormRopeWorkload):
        import torch
        self.uq, self.wl = uq, wl
        x, gamma, pos = workloads.make_norm_rope(wl)
        self.x_host, self.gamma_host, self.pos_host = x, gamma, pos
        cos, sin = uq.uq_rope_table(wl.theta, wl.head_dim, wl.max_pos)
        vec_bytes = x.nbytes
        # x read + y written + the table rows and positions of every token + gamma
        self.bytes = 2 * vec_bytes + wl.tokens * (wl.head_dim // 2) * 8 + wl.tokens * 4 + wl.head_dim * 4
        self.rotate = min(256, max(4, math.ceil(320e6 / (2 * vec_bytes))))
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        self.x = [xd] + [xd.clone() for _ in range(self.rotate - 1)]
        self.y = [torch.empty_like(xd) for _ in range(self.rotate)]
        self.gamma = torch.from_numpy(gamma).cuda()
        self.pos = torch.from_numpy(pos).cuda()
        self.cos, self.sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
        torch.cuda.synchronize()

    def launch(self, i: int, stream: int) -> None:
        j = i % self.rotate
        wl = self.wl
        self.uq.uq_rmsnorm_rope(self.x[j], self.y[j], self.gamma, self.pos, self.cos, self.sin, wl.tokens,
                                wl.heads, wl.head_dim, wl.max_pos, wl.eps, stream=stream)

    time = Setup.time

    def check_sample(self) -> float:
        """The whole output of the first copy against the oracle, within one fp16 spacing."""
        import oracle as o
        y = self.y[0].cpu().numpy().view(np.float16).astype(np.float64)
        cos, sin = o.rope_table(self.wl.theta, self.wl.head_dim, self.wl.max_pos)
        ref = o.rmsnorm_rope(self.x_host, self.gamma_host, self.pos_host, cos, sin, self.wl.eps)
        if not o.within_gate(y.reshape(ref.shape), ref).all():
            raise SystemExit(f"bench output of {self.wl.name} fails parity")
        return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def report_all(uq, steps: int, warmup: int, path: str | None) -> None:
    cmd = "python bench.py " + " ".join(sys.argv[1:])
    rows = ["# Every workload and activation count: time per launch", "",
            "Launches replayed from a HIP graph, weights rotated out of the caches, inputs resident in HBM.", "",
            "Command (MI355X host, repository root):", "", f"    {cmd}", "",
            "| workload | path | M | weight MB | us/launch | weight GB/s | % HBM | TFLOP/s | % bf16 MFMA |",
            "|---|---|---|---|---|---|---|---|---|"]
    for name, wl in workloads.WORKLOADS.items():
        for m in wl.ms:
            st = Setup(uq, wl, m, None)
            ms, _ = st.time(steps, warmup)
            st.check_sample()
            gbs = st.bytes / (ms * 1e-3) / 1e9
            tfl = 2.0 * m * wl.k * wl.n / (ms * 1e-3) / 1e12
            mfma = f"{100 * tfl / BF16_PEAK_TFLOPS:.1f}" if wl.path == "gemm" else "-"
            rows.append(f"| {name} | {wl.path} | {m} | {st.bytes / 1e6:.2f} | {ms * 1e3:.2f} | "
                        f"{gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f} | {tfl:.2f} | {mfma} |")
            log(rows[-1])
            del st
            if wl.path == "gemv" and wl.scheme != "nf4":
                st = Setup(uq, wl, m, None, a8=True)
                ms, _ = st.time(steps, warmup)
                st.check_sample()
                gbs = st.bytes / (ms * 1e-3) / 1e9
                tfl = 2.0 * m * wl.k * wl.n / (ms * 1e-3) / 1e12
                rows.append(f"| {name} | gemv_a8 | {m} | {st.bytes / 1e6:.2f} | {ms * 1e3:.2f} | "
                            f"{gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f} | {tfl:.2f} | - |")
                log(rows[-1])
                del st
    rows += ["", "| fused RMSNorm + RoPE | tokens | heads | head_dim | MB moved | us/launch | GB/s | % HBM |",
             "|---|---|---|---|---|---|---|---|"]
    for name, wl in workloads.NORM_ROPE.items():
        st = NormRopeSetup(uq, wl)
        ms, _ = st.time(steps, warmup)
        st.check_sample()
        gbs = st.bytes / (ms * 1e-3) / 1e9
        rows.append(f"| {name} | {wl.tokens} | {wl.heads} | {wl.head_dim} | {st.bytes / 1e6:.2f} | "
                    f"{ms * 1e3:.2f} | {gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f} |")
        log(rows[-1])
        del st
    text = "\n".join(rows) + "\n"
    log(text)
    if path:
        with open(path, "w") as f:
            f.write(text)


def norm_rope_line(args) -> None:
    """One JSON line for a fused RMSNorm + RoPE workload (not the headline metric)."""
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    import gemm_group_wise_amd as uq
    wl = workloads.NORM_ROPE[args.workload]
    st = NormRopeSetup(uq, wl)
    ms, eager_ms = st.time(args.steps, args.warmup)
    rel = st.check_sample()
    gbs = st.bytes / (ms * 1e-3) / 1e9
    log(f"{wl.name}: {ms * 1e3:.3f} us/launch (graph), {eager_ms * 1e3:.3f} us (eager), {gbs:.1f} GB/s, "
        f"rel-L2 {rel:.2e}")
    print(json.dumps({
        "metric": "fused RMSNorm + RoPE GB/s (x read + y written + table rows)", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.tokens, "heads": wl.heads, "head_dim": wl.head_dim,
                   "bytes": st.bytes, "rotated_copies": st.rotate},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}), flush=True)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=workloads.HEADLINE,
                    choices=list(workloads.WORKLOADS) + list(workloads.NORM_ROPE))
    ap.add_argument("--m", type=int, default=None)
    ap.add_argument("--a8", action="store_true",
                    help="time the activation-quantized GEMV (uq_gemv_a8) on an INT GEMV workload instead")
    ap.add_argument("--rotate", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="also time every workload (markdown)")
    ap.add_argument("--report", default=None)
    ap.add_argument("--traffic-run", type=int, default=0, metavar="LAUNCHES",
                    help="only launch the kernel LAUNCHES times plus a calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--traffic-parse", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic_*")
    ap.add_argument("--traffic-cmd", action="append", default=[], help="command lines recorded with the result")
    ap.add_argument("--ceiling", action="store_true",
                    help="plain reads of the headline's bytes and of 1 GiB, an empty launch and the headline GEMV "
                         "(markdown to stderr and --report)")
    ap.add_argument("--trace-summary", nargs=2, default=None, metavar=("TRACE_DIR", "NAME"),
                    help="turn a rocprofv3 --kernel-trace output into profiles/NAME.md|json")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the live plain-read ceiling in the JSON line")
    ap.add_argument("--counter-summary", nargs="+", default=None, metavar="ARG",
                    help="NAME KERNEL_HINT TITLE DIR [DIR ...]: median counters per dispatch into profiles/NAME.md")
    args = ap.parse_args()

    if args.gpus != 1:
        raise SystemExit("bench.py measures one GPU: the library has no multi-GPU path "
                         "(the sharding plan is documented, not built); run with --gpus 1")
    if args.counter_summary:
        name, hint, title, *dirs = args.counter_summary
        counter_summary(dirs, name, args.traffic_cmd, hint, title)
        return
    if args.trace_summary:
        wl_ = workloads.WORKLOADS.get(args.workload)
        hint = "gemv_" if wl_ is not None and wl_.path == "gemv" else "gemm_"  # dot-product or matrix-core kernels
        if args.a8:
            hint = "gemv_a8_kernel"
        trace_summary(args.trace_summary[0], args.trace_summary[1], args.traffic_cmd, hint,
                      None if wl_ is None or args.a8 else wl_.path)
        return
    if args.workload in workloads.NORM_ROPE:
        norm_rope_line(args)
        return
    wl = workloads.WORKLOADS[args.workload]
    m = args.m if args.m is not None else wl.ms[0]
    if not 1 <= m <= wl.mmax:
        # x is generated with wl.mmax rows; the kernels read M rows of it.
        raise SystemExit(f"{wl.name}: --m must be between 1 and {wl.mmax} (the rows of its activations)")
    if args.traffic_parse:
        traffic_parse(wl, m, args.traffic_parse[0], args.traffic_parse[1], args.traffic_cmd)
        return
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    import gemm_group_wise_amd as uq

    if args.traffic_run:
        traffic_run(uq, wl, m, args.traffic_run)
        return
    if args.ceiling:
        print(json.dumps({"ceiling": report_ceiling(uq, args.steps, args.warmup, args.report)}), flush=True)
        return
    if args.a8 and (wl.path != "gemv" or wl.scheme == "nf4"):
        raise SystemExit("--a8 applies to the INT GEMV workloads")
    st = Setup(uq, wl, m, args.rotate, a8=args.a8)
    torch.cuda.synchronize()
    ms, eager_ms = st.time(args.steps, args.warmup)
    rel = st.check_sample()
    gbs = st.bytes / (ms * 1e-3) / 1e9
    log(f"{wl.name} m={m}: {ms * 1e3:.3f} us/launch (graph), {eager_ms * 1e3:.3f} us/launch (eager), "
        f"{gbs:.1f} GB/s, rotate={st.rotate}, sampled rel-L2 {rel:.2e}")

    out = {
        "metric": METRIC if not args.a8 else
        "activation-quantized (int8 per group) GEMV weight GB/s & % HBM peak (not the headline metric)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if args.a8 else ("f16" if wl.path == "gemv" else "bf16"),
        "data": "synthetic",
        "config": {"workload": f"{wl.name} {'gemv_a8' if args.a8 else wl.path} m={m}", "scheme": wl.scheme,
                   "group": wl.group,
                   "m": m, "k": wl.k, "n": wl.n, "weight_bytes": st.bytes, "rotated_copies": st.rotate,
                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "tflops": round(2.0 * m * wl.k * wl.n / (ms * 1e-3) / 1e12, 3),
                   "tokens_per_s_one_layer": round(m / (ms * 1e-3), 1)},
    }
    if wl.path == "gemv":
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None if args.a8 else traffic_for(wl, m)}
    else:
        tfl = 2.0 * m * wl.k * wl.n / (ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": round(tfl, 3), "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tfl / BF16_PEAK_TFLOPS, 4),
                           "traffic": traffic_for(wl, m)}
    out["launch_stats"] = dict(per_launch_stats(st.launch, min(args.steps, 200)),
                               note="eager launches, each between its own pair of HIP events")
    trace = committed_trace(wl, m) if not args.a8 else None
    if trace is not None:
        out["kernel_trace"] = trace
    if wl.path == "gemv" and not args.no_ceiling:
        c = ceiling_line(uq, st.bytes // 1024 * 1024, min(args.steps, 400), min(args.warmup, 40))
        c["gemv_frac_of_plain_read"] = round(c["plain_read_us"] / (ms * 1e3), 4)
        out["ceiling"] = c
    if not args.no_cpu_baseline and not args.a8:
        log("timing the oracle on the host (cpu_baseline) ...")
        out["cpu_baseline"] = cpu_baseline(wl, m, st.bytes)
    del st
    if args.all:
        report_all(uq, args.steps, args.warmup, args.report)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
