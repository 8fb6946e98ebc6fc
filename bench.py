"""Benchmark: achieved HBM bandwidth of the fused skip-add + normalize ops.

One step is one pass of the whole hot path over one batch of the large
workloads (inputs resident in HBM before timing starts):

  skip_rms_norm   ssln_f16_16x2048x4096        (Y and S outputs)
  gated_rms_norm  gated_f16_8x4096x4096_c128
  skip_group_norm sgn_f16_nhwc_2x64x64x320     (Y and S, bias, SiLU)
  skip_group_norm sgn_f32_nchw_4x1280x32x32    (broadcast skip, Y)

Bytes are algorithmic: every input read once plus every requested output
written once.  ``value`` = bytes of K steps / wall time of the K steps
(synchronized on both sides, no instrumentation inside).  Per-op times come
from a second pass of K steps with HIP events (device-scope release)
recorded around every op on the stream the kernels run on; the roofline entry
uses the dominant kernel's average from that pass.  The two 0.8-1 GB workloads exceed the 256 MB
last-level cache, and between two visits of any workload at least 1.8 GB of
other traffic passes, so every op starts from a cold cache.

Prints one JSON line on stdout (progress goes to stderr).

``--configs`` instead times each of the five reference workloads on its own:
every invocation is preceded by a 1 GiB copy (so it starts from a cold
cache) and bracketed by HIP events; the oracle is timed on one thread on the
same inputs (median of 3 runs for the small workloads, one run for the two
large ones).  It prints one JSON object and a markdown table (stderr).

``--phases`` prints per-workgroup phase timings of the single-launch
group-norm kernels from the library's phase-trace measurement build.
``--contention`` times the group-norm ops alone and beside a copy kernel
running on a second stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))  # workloads: the seeded input generator

METRIC = "achieved HBM GB/s (and % of MI355X peak) per norm op, fp16 large shapes"
PEAK_GBPS = 8000.0  # MI355X HBM3E
STEP_WORKLOADS = ["ssln_f16_16x2048x4096", "gated_f16_8x4096x4096_c128",
                  "sgn_f16_nhwc_2x64x64x320", "sgn_f32_nchw_4x1280x32x32"]
DOMINANT = "ssln_f16_16x2048x4096"
DOMINANT_KERNEL = "ssln_wave_kernel<half, 8 per vector, 4 vectors per lane, 2 waves per row>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ssln_f16_16x2048x4096.json")
KERNEL_SOURCES = ["group_normalization_amd/csrc/ssln.hip", "group_normalization_amd/csrc/device_common.h"]
COPY_BYTES = 1 << 30


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is absent or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except FileNotFoundError:
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


class HipEvents:
    """Timing events from the HIP runtime the process already uses (torch's),
    created with hipEventReleaseToDevice: a device-scope release instead of
    the default system-scope one, so recording an event does not write back
    the caches between the kernels being timed."""

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self):
        import ctypes
        import re

        maps = open("/proc/self/maps").read()
        paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", maps)))
        if not paths:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(paths[0])
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_int, ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.RELEASE_TO_DEVICE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def record(self, ev, stream_handle):
        if self.hip.hipEventRecord(ev, self.ct.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)

    def memcpy_dtod(self, dst_ptr, src_ptr, nbytes, stream_handle):
        """hipMemcpyAsync(..., hipMemcpyDeviceToDevice) on the given stream."""
        if self.hip.hipMemcpyAsync(self.ct.c_void_p(dst_ptr), self.ct.c_void_p(src_ptr), nbytes, 3,
                                   self.ct.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipMemcpyAsync failed")


def copy_ceilings(torch, gn, hev, stream, reps=10):
    """Practical bandwidth ceilings over COPY_BYTES (read + written bytes per
    second): the library's 16-byte copy kernel, and hipMemcpyDtoD (the
    runtime's device-to-device copy) as a second reference."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    out = {}
    for name, run in (("copy_kernel", lambda: gn.copy_(dst, src)),
                      ("hipMemcpyDtoD", lambda: hev.memcpy_dtod(dst.data_ptr(), src.data_ptr(),
                                                                COPY_BYTES, stream))):
        for _ in range(3):
            run()
        e0, e1 = hev.create(), hev.create()
        hev.record(e0, stream)
        for _ in range(reps):
            run()
        hev.record(e1, stream)
        torch.cuda.synchronize()
        out[name] = 2 * COPY_BYTES * reps / (hev.elapsed_ms(e0, e1) * 1e-3) / 1e9
        hev.destroy(e0)
        hev.destroy(e1)
    del src, dst
    return out


class Op:
    """One workload's device tensors and a closure that enqueues the op."""

    def __init__(self, name, torch, gn, workloads):
        w = workloads.WORKLOADS.get(name) or workloads.EXTRA_WORKLOADS[name]
        self.name = name
        self.bytes = workloads.io_bytes(w)
        host = workloads.generate(w)
        d = {k: torch.from_numpy(v).cuda() for k, v in host.items()}
        del host
        a = w.attrs
        if w.op == "skip_rms_norm":
            want_sum = "input_skip_bias_sum" in w.outputs
            want_inv = "inv_std_var" in w.outputs
            self.run = lambda: gn.skip_rms_norm(d["input"], d["skip"], d["gamma"], d.get("bias"),
                                                a["epsilon"], want_sum=want_sum,
                                                want_inv_std_var=want_inv)
        elif w.op == "skip_layer_norm":
            want_sum = "input_skip_bias_sum" in w.outputs
            self.run = lambda: gn.skip_layer_norm(d["input"], d["skip"], d["gamma"], d.get("beta"),
                                                  d.get("bias"), a["epsilon"], want_sum=want_sum)
        elif w.op == "gated_rms_norm":
            self.run = lambda: gn.gated_rms_norm(d["X"], d["scale"], d["gate"], a["epsilon"])
        else:
            ws = torch.empty(gn.skip_group_norm_workspace_size(d["X"], a["groups"], a["channels_last"]),
                             dtype=torch.uint8, device="cuda")
            want_sum = "S" in w.outputs
            self.run = lambda: gn.skip_group_norm(d["X"], d["gamma"], d["beta"], d["skip"], d.get("bias"),
                                                  groups=a["groups"], activation=a["activation"],
                                                  epsilon=a["epsilon"],
                                                  channels_last=a["channels_last"],
                                                  want_sum=want_sum, workspace=ws)
            self.workspace = ws
        self.tensors = d


def cpu_baseline(budget_s=14.0):
    """The oracle (single thread) on a bounded sample of each step workload:
    the two small group-norm workloads whole, then whole rows of the two
    large workloads, as many as fit an equal share of what remains of the
    budget."""
    import oracle
    import workloads

    total_bytes, total_s, parts, per_op = 0, 0.0, [], {}
    order = sorted(STEP_WORKLOADS, key=lambda n: workloads.WORKLOADS[n].op != "skip_group_norm")
    n_large = sum(workloads.WORKLOADS[n].op != "skip_group_norm" for n in order)
    for name in order:
        w = workloads.WORKLOADS[name]
        x = workloads.generate(w)
        a = w.attrs
        if w.op == "skip_rms_norm":
            inp, skp = x["input"].reshape(-1, x["input"].shape[-1]), x["skip"].reshape(-1, x["input"].shape[-1])
            unit_rows, per_row = inp.shape[0], workloads.io_bytes(w) / inp.shape[0]
            call = lambda lo, hi: oracle.skip_rms_norm(inp[lo:hi], skp[lo:hi], x["gamma"], x.get("bias"),
                                                       a["epsilon"], want_sum=True)
        elif w.op == "gated_rms_norm":
            C = x["scale"].size
            X, G = x["X"].reshape(-1, C), x["gate"].reshape(-1, C)
            unit_rows, per_row = X.shape[0], workloads.io_bytes(w) / X.shape[0]
            call = lambda lo, hi: oracle.gated_rms_norm(X[lo:hi], x["scale"], G[lo:hi], a["epsilon"])
        else:
            N = x["X"].shape[0]
            unit_rows, per_row = N, workloads.io_bytes(w) / N
            call = lambda lo, hi: oracle.skip_group_norm(
                x["X"][lo:hi], x["gamma"], x["beta"], x["skip"][lo:hi], x.get("bias"),
                groups=a["groups"], activation=a["activation"], epsilon=a["epsilon"],
                channels_last=a["channels_last"], want_sum="S" in w.outputs)
        share = float("inf") if w.op == "skip_group_norm" else (budget_s - total_s) / n_large
        if w.op != "skip_group_norm":
            n_large -= 1
        done, t_op, chunk = 0, 0.0, 1
        while done < unit_rows and t_op < share:
            hi = min(unit_rows, done + chunk)
            t0 = time.perf_counter()
            call(done, hi)
            t_op += time.perf_counter() - t0
            done = hi
            chunk = min(chunk * 2, 4096)
        total_bytes += per_row * done
        total_s += t_op
        unit = "rows" if w.op != "skip_group_norm" else "images"
        parts.append(f"{name}: {done}/{unit_rows} {unit}")
        per_op[name] = {"seconds": round(t_op, 3), unit: done, "of": unit_rows,
                        "gbps": round(per_row * done / t_op / 1e9, 4)}
        log(f"cpu oracle {name}: {done} {unit} in {t_op:.2f} s")
    return {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": "; ".join(parts) + f" ({total_s:.1f} s single-thread)",
            "per_op": per_op, "host": host_cpu()}


def oracle_runner(w, x):
    """A call of the oracle over the whole workload, with its outputs."""
    import oracle

    a = w.attrs
    if w.op in ("skip_rms_norm", "skip_layer_norm"):
        hidden = x["input"].shape[-1]
        inp, skp = x["input"].reshape(-1, hidden), x["skip"].reshape(-1, hidden)
        return lambda: oracle.skip_rms_norm(inp, skp, x["gamma"], x.get("bias"), a["epsilon"],
                                            want_inv_std_var="inv_std_var" in w.outputs,
                                            want_sum="input_skip_bias_sum" in w.outputs)
    if w.op == "gated_rms_norm":
        return lambda: oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], a["epsilon"])
    return lambda: oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], x.get("bias"),
                                          groups=a["groups"], activation=a["activation"],
                                          epsilon=a["epsilon"], channels_last=a["channels_last"],
                                          want_sum="S" in w.outputs)


def config_table(args):
    """Each reference workload alone, cold, K timed invocations (see the
    module docstring)."""
    import torch
    import group_normalization_amd as gn
    import workloads

    torch.cuda.set_device(0)
    hev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    ceilings = copy_ceilings(torch, gn, hev, stream)
    copy_gbps = ceilings["copy_kernel"]
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)

    def cold_times(run):
        """Event-timed invocations of run(), each after a 1 GiB copy that
        evicts the last-level cache."""
        for _ in range(args.warmup):
            gn.copy_(dst, src)
            run()
        pairs = [(hev.create(), hev.create()) for _ in range(args.steps)]
        for a, b in pairs:
            gn.copy_(dst, src)
            hev.record(a, stream)
            run()
            hev.record(b, stream)
        torch.cuda.synchronize()
        us = np.array([hev.elapsed_ms(a, b) * 1e3 for a, b in pairs])
        for a, b in pairs:
            hev.destroy(a)
            hev.destroy(b)
        return us

    rows = []
    for name in workloads.ORDER:
        w = workloads.WORKLOADS[name]
        o = Op(name, torch, gn, workloads)
        us = cold_times(o.run)
        # The same byte volume moved by the copy kernel (half read, half
        # written), cold: what streaming those bytes costs at this size,
        # launch included.
        half = (o.bytes // 2 + 15) // 16 * 16
        csrc = torch.empty(half, dtype=torch.uint8, device="cuda").fill_(1)
        cdst = torch.empty_like(csrc)
        cus = cold_times(lambda: gn.copy_(cdst, csrc))
        del csrc, cdst
        med, cmed = float(np.median(us)), float(np.median(cus))
        row = {"workload": name, "bytes": o.bytes, "invocations": args.steps,
               "median_us": round(med, 3), "min_us": round(float(us.min()), 3),
               "p90_us": round(float(np.percentile(us, 90)), 3),
               "gbps": round(o.bytes / med / 1e3, 1), "frac_of_peak": round(o.bytes / med / 1e3 / PEAK_GBPS, 4),
               "frac_of_copy": round(o.bytes / med / 1e3 / copy_gbps, 4),
               "same_bytes_copy_us": round(cmed, 3), "frac_of_same_bytes_copy": round(cmed / med, 4)}
        del o
        if not args.no_cpu_baseline:
            x = workloads.generate(w)
            run = oracle_runner(w, x)
            reps = 3 if workloads.io_bytes(w) < 100e6 else 1
            secs = []
            for _ in range(reps):
                t0 = time.perf_counter_ns()
                run()
                secs.append((time.perf_counter_ns() - t0) * 1e-9)
            row["oracle_s"] = round(float(np.median(secs)), 4)
            row["oracle_runs"] = reps
            row["oracle_gbps"] = round(workloads.io_bytes(w) / float(np.median(secs)) / 1e9, 4)
            del x
        rows.append(row)
        log(f"{name}: median {med:.2f} us ({row['gbps']} GB/s)")
    out = {"configs": rows, "copy_ceiling_gbps": round(copy_gbps, 1),
           "memcpy_dtod_ceiling_gbps": round(ceilings["hipMemcpyDtoD"], 1), "oracle_threads": 1,
           "host": host_cpu()}
    lines = ["| workload | median us | min us | p90 us | GB/s | % of 8 TB/s | % of copy | same-bytes copy us | "
             "% of same-bytes copy | oracle s | oracle GB/s |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['workload']} | {r['median_us']} | {r['min_us']} | {r['p90_us']} | {r['gbps']} | "
                     f"{100 * r['frac_of_peak']:.1f} | {100 * r['frac_of_copy']:.1f} | "
                     f"{r['same_bytes_copy_us']} | {100 * r['frac_of_same_bytes_copy']:.1f} | "
                     f"{r.get('oracle_s', '')} | {r.get('oracle_gbps', '')} |")
    print("\n".join(lines), file=sys.stderr)
    print(json.dumps(out), flush=True)


def contention_table(args):
    """SkipGroupNorm's single-launch routes exchange moments among
    workgroups that must be resident together; this times each group-norm
    workload alone and while a 1 GiB copy kernel (2 GiB of traffic, every
    CU busy) runs on a second stream of the same (default) priority, for
    the automatic route and the three-launch split route (which waits on
    nothing), events on the op's own stream."""
    import torch
    import group_normalization_amd as gn
    import workloads

    torch.cuda.set_device(0)
    hev = HipEvents()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    flush_a = torch.empty_like(src)
    rows, lines = {}, ["| workload | route | alone median us | alone p90 us | beside a copy median us | "
                       "beside a copy p90 us | beside a copy max us |", "|---|---|---|---|---|---|---|"]
    for name in ("sgn_f16_nhwc_2x64x64x320", "sgn_f32_nchw_4x1280x32x32"):
        o = Op(name, torch, gn, workloads)
        for route in ("auto", "split"):
            res = {}
            for mode in ("alone", "contended"):
                with gn.force_route(route):
                    us = []
                    for i in range(args.warmup + args.steps):
                        gn.copy_(flush_a, src)  # cold cache
                        torch.cuda.synchronize()
                        a, b = hev.create(), hev.create()
                        if mode == "contended":
                            with torch.cuda.stream(side):
                                gn.copy_(dst, src)
                            # Let the copy occupy the CUs before the op is enqueued.
                            time.sleep(20e-6)
                        hev.record(a, main.cuda_stream)
                        o.run()
                        used = gn.last_route()
                        hev.record(b, main.cuda_stream)
                        torch.cuda.synchronize()
                        if i >= args.warmup:
                            us.append(hev.elapsed_ms(a, b) * 1e3)
                        hev.destroy(a)
                        hev.destroy(b)
                us = np.array(us)
                res[mode] = {"median_us": round(float(np.median(us)), 2),
                             "p90_us": round(float(np.percentile(us, 90)), 2),
                             "max_us": round(float(us.max()), 2)}
            rows[f"{name} {used}"] = res
            lines.append(f"| {name} | {used} | {res['alone']['median_us']} | {res['alone']['p90_us']} | "
                         f"{res['contended']['median_us']} | {res['contended']['p90_us']} | "
                         f"{res['contended']['max_us']} |")
            log(f"{name} {used}: alone {res['alone']['median_us']} us, beside a copy "
                f"{res['contended']['median_us']} us (p90 {res['contended']['p90_us']}, max {res['contended']['max_us']})")
        del o
    print("\n".join(lines), file=sys.stderr)
    print(json.dumps({"contention": rows, "invocations": args.steps}), flush=True)


PHASES = ["loads", "reduce", "publish + S", "exchange + combine", "normalize + Y"]


def phase_table(args):
    """Per-workgroup phase timings of the single-launch SkipGroupNorm routes
    on the two group-norm workloads, each invocation cold (after a 1 GiB
    copy), from the measurement build of the library (SN_PHASE_TRACE: each
    workgroup's leader records the 100 MHz wall clock at six phase
    boundaries in a tail of the workspace).  Build it first with
    `python -m group_normalization_amd.build --phase-trace`."""
    from group_normalization_amd import _lib
    from group_normalization_amd import build as libbuild

    if not os.path.exists(libbuild.TRACE_LIB_PATH):
        sys.exit(f"{libbuild.TRACE_LIB_PATH} is missing: run "
                 "`python -m group_normalization_amd.build --phase-trace` first")
    _lib.LIB_PATH = libbuild.TRACE_LIB_PATH  # before the first call loads a library
    import torch
    import group_normalization_amd as gn
    import workloads

    trace_bytes = 65536 * 8 * 8  # kTraceBlocks x kTraceStamps x 8 bytes
    torch.cuda.set_device(0)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    out, lines = {}, ["| workload | route | workgroups | " + " | ".join(f"{p} us" for p in PHASES) +
                      " | start spread us | first start to last stamp us |",
                      "|---|---|---|" + "---|" * (len(PHASES) + 2)]
    for name in ("sgn_f16_nhwc_2x64x64x320", "sgn_f32_nchw_4x1280x32x32"):
        o = Op(name, torch, gn, workloads)
        tail = o.workspace[-trace_bytes:]
        per_call = []
        for i in range(args.warmup + args.steps):
            tail.zero_()
            gn.copy_(dst, src)
            o.run()
            route = gn.last_route()
            torch.cuda.synchronize()
            if i < args.warmup:
                continue
            st = tail.cpu().numpy().view(np.uint64).reshape(-1, 8)[:, :6].astype(np.int64)
            st = st[st[:, 0] != 0]
            if st.size == 0 or np.any(st == 0):
                sys.exit(f"{name}: incomplete phase stamps (route {route})")
            d = np.diff(st, axis=1) * 0.01  # ticks of 10 ns -> us
            per_call.append({"wg": len(st), "phases": np.median(d, axis=0),
                             "spread": (st[:, 0].max() - st[:, 0].min()) * 0.01,
                             "span": (st[:, 5].max() - st[:, 0].min()) * 0.01})
        ph = np.median([c["phases"] for c in per_call], axis=0)
        spread = float(np.median([c["spread"] for c in per_call]))
        span = float(np.median([c["span"] for c in per_call]))
        out[name] = {"route": route, "workgroups": per_call[0]["wg"], "invocations": len(per_call),
                     "median_phase_us": {p: round(float(v), 3) for p, v in zip(PHASES, ph)},
                     "start_spread_us": round(spread, 3), "first_start_to_last_stamp_us": round(span, 3)}
        lines.append(f"| {name} | {route} | {per_call[0]['wg']} | " + " | ".join(f"{v:.2f}" for v in ph) +
                     f" | {spread:.2f} | {span:.2f} |")
        log(f"{name}: {route}, phases " + ", ".join(f"{p} {v:.2f}" for p, v in zip(PHASES, ph)))
        del o
    print("\n".join(lines), file=sys.stderr)
    print(json.dumps({"phases": out, "clock": "wall clock, 100 MHz", "statistic":
                      "median over workgroups of each invocation, then median over invocations"}),
          flush=True)


def host_cpu():
    """Logical CPU count and model name of the machine the oracle ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "model": model}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="time each reference workload alone (cold), and the oracle on it")
    ap.add_argument("--contention", action="store_true",
                    help="group-norm ops alone and beside a copy kernel on another stream")
    ap.add_argument("--phases", action="store_true",
                    help="per-phase timings of the single-launch group-norm kernels (needs the "
                         "phase-trace build of the library)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the operators need no communication and this "
              "build runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.configs:
        config_table(args)
        return
    if args.phases:
        phase_table(args)
        return
    if args.contention:
        contention_table(args)
        return

    import torch
    import group_normalization_amd as gn
    import workloads

    torch.cuda.set_device(0)
    log("generating inputs")
    ops = [Op(n, torch, gn, workloads) for n in STEP_WORKLOADS]
    torch.cuda.synchronize()
    step_bytes = sum(o.bytes for o in ops)

    hev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream  # the stream every op launches on

    def step(events=None):
        for i, o in enumerate(ops):
            if events is not None:
                hev.record(events[i][0], stream)
            o.run()
            if events is not None:
                hev.record(events[i][1], stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps, nothing but the ops between the synchronizations.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms")

    # Per-op pass: the same K steps again with an event pair around every op
    # (each recorded event costs the stream a short drain, so this pass is
    # kept out of the throughput figure above).
    evs = [[[hev.create() for _ in range(2)] for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()

    per_op = {}
    for i, o in enumerate(ops):
        ms = [hev.elapsed_ms(evs[k][i][0], evs[k][i][1]) for k in range(args.steps)]
        avg = float(np.mean(ms))
        per_op[o.name] = {"bytes": o.bytes, "avg_us": round(avg * 1e3, 3),
                          "median_us": round(float(np.median(ms)) * 1e3, 3),
                          "min_us": round(float(np.min(ms)) * 1e3, 3),
                          "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 3),
                          "gbps": round(o.bytes / (avg * 1e-3) / 1e9, 1),
                          "frac_of_peak": round(o.bytes / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)}

    # Copy ceilings over 1 GiB, outside the timed region: the library's
    # 16-byte copy kernel (also the calibration kernel for the byte counters)
    # and hipMemcpyDtoD.
    for ev in [e for per_step in evs for pair in per_step for e in pair]:
        hev.destroy(ev)
    ceilings = copy_ceilings(torch, gn, hev, stream)
    copy_gbps = ceilings["copy_kernel"]

    for v in per_op.values():
        v["frac_of_copy"] = round(v["gbps"] / copy_gbps, 4)

    # Beyond the step: the non-simplified skip layer normalization at the
    # large SSLN shape, timed alone (its 1 GB per call keeps it cold).
    next_ops = {}
    for name in workloads.EXTRA_WORKLOADS:
        o = Op(name, torch, gn, workloads)
        for _ in range(args.warmup):
            o.run()
        pairs = [(hev.create(), hev.create()) for _ in range(args.steps)]
        for e0, e1 in pairs:
            hev.record(e0, stream)
            o.run()
            hev.record(e1, stream)
        torch.cuda.synchronize()
        ms = [hev.elapsed_ms(e0, e1) for e0, e1 in pairs]
        for e0, e1 in pairs:
            hev.destroy(e0)
            hev.destroy(e1)
        avg = float(np.mean(ms))
        gbps = o.bytes / (avg * 1e-3) / 1e9
        next_ops[name] = {"bytes": o.bytes, "avg_us": round(avg * 1e3, 3),
                          "median_us": round(float(np.median(ms)) * 1e3, 3),
                          "min_us": round(float(np.min(ms)) * 1e3, 3),
                          "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 3),
                          "gbps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4),
                          "frac_of_copy": round(gbps / copy_gbps, 4)}
        del o

    dom = per_op[DOMINANT]
    achieved = dom["bytes"] / (dom["avg_us"] * 1e-6) / 1e9
    traffic = load_traffic()
    result = {
        "metric": METRIC,
        "value": round(step_bytes * args.steps / elapsed / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64, seed 0; N(0,1), U(0.5,1.5), N(0,0.1) per tensor)",
        "config": {"workload": " + ".join(STEP_WORKLOADS), "io_dtype": "f16 (f32 for the NCHW group norm)",
                   "bytes_per_step": step_bytes, "cache": "cold (working set > last-level cache)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": DOMINANT_KERNEL, "workload": DOMINANT},
        "ops": per_op,
        "next_ops": next_ops,
        "copy_ceiling_gbps": round(copy_gbps, 1),
        "memcpy_dtod_ceiling_gbps": round(ceilings["hipMemcpyDtoD"], 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
