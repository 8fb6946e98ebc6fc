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
running on a second stream.  ``--shapes`` times general shapes (rows wider
than the registers hold, ...) on the automatic and on forced routes.  ``--summarize DIR`` writes the summaries under
profiles/ from rocprofv3 output (no GPU needed).
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
DOMINANT_KERNEL = "ssln_wave_kernel<T=f16, E=8, NV=4, FULL=1, WPR=2, CENTER=0, WPB=4>"
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

    def __init__(self, name, torch, gn, workloads, w=None, d=None):
        """The named workload with its seeded host inputs, or workload ``w``
        with the device tensors ``d`` already drawn."""
        if w is None:
            w = workloads.WORKLOADS.get(name) or workloads.EXTRA_WORKLOADS[name]
        self.name = name
        self.bytes = workloads.io_bytes(w)
        if d is None:
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


def shape_cases(workloads):
    """General shapes beyond the five workloads, each with the forced
    routes it is compared against: (label, workload, alternative routes).
    Tensors of about 2^27 elements (256 MB in float16), so every call
    starts from a cold last-level cache."""
    F16, F32 = workloads.F16, workloads.F32
    out = []

    def add(label, w, alts):
        out.append((label, w, alts))

    # Rows beyond one workgroup's registers (the wide routes).
    for h, dt in ((131072, F16), (100000, F16), (139264, F16), (65536, F32), (50004, F32)):
        rows = (1 << 27) // h
        n = np.dtype(dt).name
        add(f"ssln_{n}_{rows}x{h}", workloads.ssln("w", (rows, h), dt, bias=True, epsilon=1e-6,
                                                   outputs=("output", "input_skip_bias_sum")), ())
    rows = (1 << 27) // 131072
    add(f"sln_float16_{rows}x131072", workloads.sln("w", (rows, 131072), F16, beta=True, bias=False,
                                                    epsilon=1e-5, outputs=("output", "input_skip_bias_sum")),
        ())
    for c, dt in ((65536, F16), (131072, F16), (139264, F16), (65536, F32)):
        rows = (1 << 27) // c
        add(f"gated_{np.dtype(dt).name}_{rows}x{c}_c{c}", workloads.gated("w", (rows, c), c, dt, epsilon=1e-5),
            ())
    # Rows that are not a whole number of 16-byte vectors, and short rows:
    # phased, flat, segment and narrow-access routes.
    for h, dt in ((127, F16), (247, F16), (1000, F16), (2046, F16), (4097, F16), (4100, F16), (8193, F16),
                  (123, F32), (1021, F32), (3001, F32)):
        rows = (1 << 27) // h
        add(f"ssln_{np.dtype(dt).name}_{rows}x{h}", workloads.ssln("w", (rows, h), dt, bias=True, epsilon=1e-6,
                                                                   outputs=("output", "input_skip_bias_sum")), ())
    for c, dt in ((25, F16), (130, F16), (301, F16), (1025, F16), (2049, F16), (4097, F16), (16385, F16),
                  (129, F32), (1021, F32), (2049, F32)):
        rows = (1 << 27) // c
        add(f"gated_{np.dtype(dt).name}_{rows}x{c}_c{c}", workloads.gated("w", (rows, c), c, dt, epsilon=1e-5),
            ())
    # SkipGroupNorm beyond the two workloads: pixels that are not a whole
    # number of 16-byte vectors, NCHW planes off the grid, large images.
    for N, C, H, W, dt, cl, g in ((8, 60, 128, 128, F16, 1, 15), (8, 36, 128, 128, F16, 1, 12),
                                  (8, 15, 128, 128, F16, 1, 5), (16, 3, 256, 256, F16, 1, 1),
                                  (8, 320, 31, 31, F16, 0, 32), (4, 256, 33, 33, F32, 0, 32),
                                  (8, 320, 128, 128, F16, 1, 32), (4, 512, 64, 64, F16, 0, 32)):
        layout = "nhwc" if cl else "nchw"
        add(f"sgn_{np.dtype(dt).name}_{layout}_{N}x{C}x{H}x{W}_g{g}",
            workloads.sgn("w", N, C, H, W, dt, F32, channels_last=bool(cl), broadcast_skip=False, bias=True,
                          groups=g, activation=1, epsilon=1e-5, outputs=("Y", "S")), ())
    # A batch of small images, one workgroup per image's channel block (NHWC)
    # or group (NCHW) whatever the batch size, beside the split route.
    for cl in (1, 0):
        layout = "nhwc" if cl else "nchw"
        add(f"sgn_float16_{layout}_256x320x16x16_g32",
            workloads.sgn("w", 256, 320, 16, 16, F16, F32, channels_last=bool(cl), broadcast_skip=False, bias=True,
                          groups=32, activation=1, epsilon=1e-5, outputs=("Y", "S")), ("split",))
    return out


def shapes_table(args):
    """Each general shape alone, cold, on the automatic route and on each
    forced alternative (see shape_cases)."""
    import torch
    import group_normalization_amd as gn
    import workloads

    torch.cuda.set_device(0)
    hev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    rows, lines = [], ["| shape | route | median us | GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
    for label, w, alts in shape_cases(workloads):
        o = Op(label, torch, gn, workloads, w=w, d=workloads.generate_on_device(w, 0, torch))
        for route in ("auto",) + tuple(alts):
            with gn.force_route(route):
                for _ in range(args.warmup):
                    gn.copy_(dst, src)
                    o.run()
                used = gn.last_route()
                pairs = [(hev.create(), hev.create()) for _ in range(args.steps)]
                for a, b in pairs:
                    gn.copy_(dst, src)
                    hev.record(a, stream)
                    o.run()
                    hev.record(b, stream)
                torch.cuda.synchronize()
            us = float(np.median([hev.elapsed_ms(a, b) * 1e3 for a, b in pairs]))
            for a, b in pairs:
                hev.destroy(a)
                hev.destroy(b)
            gbps = o.bytes / us / 1e3
            rows.append({"shape": label, "forced": route, "route": used, "bytes": o.bytes,
                         "median_us": round(us, 2), "gbps": round(gbps, 1)})
            lines.append(f"| {label} | {used}{'' if route == 'auto' else ' (forced)'} | {us:.2f} | "
                         f"{gbps:.1f} | {100 * gbps / PEAK_GBPS:.1f} |")
            log(f"{label} {used}: {us:.2f} us, {gbps:.1f} GB/s")
        del o
    print("\n".join(lines), file=sys.stderr)
    print(json.dumps({"shapes": rows, "invocations": args.steps}), flush=True)


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


# ---------------------------------------------------------------------------
# Profile summaries: rocprofv3 CSV output -> the text files under profiles/.

PROF_COMMANDS = {
    "kt": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/kt -o bench -- "
          "python3 $REPO/bench.py --steps 20 --warmup 3 --no-cpu-baseline",
    "ktc": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/ktc -o configs -- "
           "python3 $REPO/bench.py --configs --steps 60 --warmup 5 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/fetch -o bench -- "
             "python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/write -o bench -- "
             "python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline",
    "configs": "python3 $REPO/bench.py --configs --steps 60 --warmup 5",
    "bench": "python3 $REPO/bench.py",
    "shapes": "python3 $REPO/bench.py --shapes --steps 10 --warmup 2",
}

# Template parameters of each kernel family, as declared in the sources.
KERNEL_PARAMS = {
    "ssln_wave_kernel": "T E NV FULL WPR CENTER WPB",
    "ssln_phase_kernel": "T E NV WPR CENTER WPB",
    "ssln_block_kernel": "T E CENTER",
    "ssln_segment_kernel": "T E L RPT CENTER",
    "ssln_flat_kernel": "T VPT NARROW CENTER",
    "gated_segment_kernel": "T E L VPL RPT LINES",
    "gated_tile_kernel": "T E VPT",
    "gated_flat_kernel": "T VPT NARROW",
    "gated_row_kernel": "T E NV TPB",
    "gated_block_kernel": "T E",
    "sgn_cluster_kernel": "T M E R BCAST",
    "sgn_cluster_phase_kernel": "T M E R BCAST",
    "sgn_nhwc_cluster_kernel": "T M E R BCAST",
    "sgn_stats_nhwc_kernel": "T E",
    "sgn_norm_nhwc_kernel": "T M E",
    "sgn_stats_group_kernel": "T E NCHW",
    "sgn_norm_group_kernel": "T M E NCHW",
}
_TYPE_CODES = {"DF16_": "f16", "f": "f32", "d": "f64"}
_TYPE_NAMES = {"_Float16": "f16", "__half": "f16", "half": "f16", "float": "f32", "double": "f64"}


def _mangled_template_args(rest):
    """Arguments of an Itanium-mangled template argument list (`I...E`) made
    of the forms these kernels use: builtin types, int and bool literals."""
    out, i = [], 1
    while i < len(rest) and rest[i] != "E":
        for code, t in _TYPE_CODES.items():
            if rest.startswith(code, i):
                out.append(t)
                i += len(code)
                break
        else:
            if rest[i] != "L":
                return None
            j = rest.index("E", i)
            lit = rest[i + 1:j]  # e.g. "i8", "b1", "in3", "j4"
            num = lit[1:].replace("n", "-")
            out.append(("1" if num == "1" else "0") if lit[0] == "b" else num)
            i = j + 1
    return out


def kernel_family(name):
    """(family, template arguments or None) of a kernel name as rocprofv3
    reports it (mangled or demangled)."""
    import re

    m = re.search(r"(\w+_kernel)<([^()]*)>\(", name)
    if m:
        args = [a.strip() for a in m.group(2).split(",")]
        return m.group(1), [_TYPE_NAMES.get(a, {"true": "1", "false": "0"}.get(a, a)) for a in args]
    if name.startswith("_ZN"):
        # Walk the nested-name components by their length prefixes.
        pos, fam = 3, None
        while pos < len(name) and name[pos].isdigit():
            k = pos
            while name[k].isdigit():
                k += 1
            ln = int(name[pos:k])
            fam, pos = name[k:k + ln], k + ln
        rest = name[pos:]
        if fam and fam.endswith("_kernel"):
            return fam, (_mangled_template_args(rest) if rest.startswith("I") else None)
    m = re.search(r"(\w+_kernel)\(", name)
    if m:
        return m.group(1), None
    return name, None


def kernel_label(name):
    fam, args = kernel_family(name)
    if name.startswith("__amd_rocclr_copyBuffer"):
        return "runtime copyBuffer (host to device set-up)"
    if "FillFunctor" in name:
        return "torch fill (set-up)"
    if args is None:
        return fam
    names = KERNEL_PARAMS.get(fam, "").split()
    if len(names) == len(args):
        return f"{fam}<" + ", ".join(f"{k}={v}" for k, v in zip(names, args)) + ">"
    return f"{fam}<" + ", ".join(args) + ">"


def step_workload(name):
    """Workload of a benchmark-step (or next_ops) kernel, from its family:
    each family serves exactly one workload of that run."""
    fam, args = kernel_family(name)
    if fam.startswith("ssln_"):
        center = args[KERNEL_PARAMS[fam].split().index("CENTER")] if args else "0"
        return EXTRA_STEP_WORKLOAD if center == "1" else "ssln_f16_16x2048x4096"
    if fam.startswith("gated_"):
        return "gated_f16_8x4096x4096_c128"
    if fam.startswith("sgn_") and ("nhwc" in fam):
        return "sgn_f16_nhwc_2x64x64x320"
    if fam.startswith("sgn_"):
        return "sgn_f32_nchw_4x1280x32x32"
    return None


EXTRA_STEP_WORKLOAD = "sln_f16_16x2048x4096"


def _find_csv(d, suffix):
    import glob

    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits[0]


def _read_csv(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _read_json_line(path):
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)
    sys.exit(f"no JSON line in {path}")


def _pmc_per_kernel(d, counter):
    """{kernel name: (dispatches, average counter value per dispatch)} from a
    rocprofv3 --pmc run (values summed over the rows of one dispatch)."""
    per_dispatch = {}
    for r in _read_csv(_find_csv(d, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per_dispatch.items():
        n, tot = out.get(name, (0, 0.0))
        out[name] = (n + 1, tot + v)
    return {k: (n, tot / n) for k, (n, tot) in out.items()}


def summarize(args):
    """Write profiles/*.md and the dominant kernel's traffic file from the
    rocprofv3 output of the commands in PROF_COMMANDS (run on the GPU with
    this same source tree), collected under one directory."""
    import workloads

    d = args.summarize
    io = {n: workloads.io_bytes(w) for n, w in {**workloads.WORKLOADS, **workloads.EXTRA_WORKLOADS}.items()}
    prof = os.path.join(ROOT, "profiles")
    cmd = lambda k: f"cd /tmp && export TMPDIR=/tmp && {PROF_COMMANDS[k]}"

    # --- Kernel trace of the benchmark step.
    stats = _read_csv(_find_csv(os.path.join(d, "kt"), "kernel_stats.csv"))
    kt_bench = _read_json_line(os.path.join(d, "kt", "bench.json"))
    lines = ["# Kernel trace of the benchmark step (all hot-path kernels)", "",
             "Workloads: " + ", ".join(STEP_WORKLOADS) + "; the next_ops leg adds "
             f"{EXTRA_STEP_WORKLOAD}. One MI355X (gfx950).", "",
             "Command (`$REPO` = repository root, `$OUT` = the directory of rocprofv3 output, the one "
             "given to `bench.py --summarize`):", "",
             "```", cmd("kt") + " > $OUT/kt/bench.json", "```", "",
             "`rocprofv3 --stats` kernel summary (`bench_kernel_stats.csv`). The GB/s column is the "
             "workload's algorithmic bytes over the kernel's average duration:", "",
             "| kernel | workload | calls | avg us | min us | max us | GB/s (avg) |",
             "|---|---|---|---|---|---|---|"]
    dom_avg_us = None
    for r in stats:
        w = step_workload(r["Name"])
        avg = float(r["AverageNs"]) / 1e3
        gbps = f"{io[w] / avg / 1e3:.1f}" if w else ""
        if w == DOMINANT:
            dom_avg_us = avg
        lines.append(f"| {kernel_label(r['Name'])} | {w or ''} | {r['Calls']} | {avg:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {gbps} |")
    lines += ["", "Same run, bench.py's HIP-event timing (per-op pass, device-scope release events, "
              "which also span each launch):", "",
              "| op | avg us (events) | GB/s | fraction of 8 TB/s |", "|---|---|---|---|"]
    for name, v in {**kt_bench["ops"], **kt_bench["next_ops"]}.items():
        lines.append(f"| {name} | {v['avg_us']} | {v['gbps']} | {v['frac_of_peak']} |")
    ev = kt_bench["ops"][DOMINANT]["avg_us"]
    lines += ["", f"Dominant kernel ({DOMINANT}): rocprofv3 average {dom_avg_us:.2f} us, event "
              f"average {ev} us. Under the profiler, bench value {kt_bench['value']} GB/s and copy "
              f"ceiling {kt_bench['copy_ceiling_gbps']} GB/s."]
    bench_path = os.path.join(d, "bench.json")
    if os.path.exists(bench_path):
        b = _read_json_line(bench_path)
        rf = b["roofline"]
        lines += ["", "Without the profiler (`" + PROF_COMMANDS["bench"] + "`), the same tree: value "
                  f"{b['value']} GB/s ({b['ms_per_step']} ms per step); dominant kernel "
                  f"{rf['achieved']} GB/s by events (frac {rf['frac']}); copy kernel "
                  f"{b['copy_ceiling_gbps']} GB/s; hipMemcpyDtoD {b['memcpy_dtod_ceiling_gbps']} GB/s."]
    with open(os.path.join(prof, "kernel_trace_bench_step.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # --- HBM traffic from the two counter passes.
    fetch = _pmc_per_kernel(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _pmc_per_kernel(os.path.join(d, "write"), "WRITE_SIZE")
    copy_name = next(k for k in fetch if kernel_family(k)[0] == "copy16_kernel")
    fu, wu = COPY_BYTES / fetch[copy_name][1], COPY_BYTES / write[copy_name][1]
    lines = ["# HBM traffic from hardware counters (FETCH_SIZE, WRITE_SIZE)", "",
             "Two counter passes over the benchmark command, one counter each:", "", "```",
             cmd("fetch"), cmd("write"), "```", "",
             f"Calibration: the library's copy kernel moves exactly 1 GiB in and 1 GiB out per "
             f"launch ({fetch[copy_name][0]} launches). It reads FETCH_SIZE = {fetch[copy_name][1]:.1f} "
             f"and WRITE_SIZE = {write[copy_name][1]:.1f} per dispatch, so one FETCH_SIZE unit is "
             f"{fu:.2f} bytes and one WRITE_SIZE unit {wu:.2f} bytes on this part.", "",
             "| kernel | workload | dispatches | FETCH_SIZE | WRITE_SIZE | fetched bytes | written bytes | "
             "total bytes | algorithmic bytes | total / algorithmic |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    dom = None
    for name in fetch:
        w = step_workload(name)
        fv, wv = fetch[name][1], write.get(name, (0, 0.0))[1]
        fb, wb = fv * fu, wv * wu
        alg = io.get(w) if w else (2 * COPY_BYTES if name == copy_name else None)
        ratio = f"{(fb + wb) / alg:.4f}" if alg else ""
        lines.append(f"| {kernel_label(name)} | {w or ''} | {fetch[name][0]} | {fv:.1f} | {wv:.1f} | "
                     f"{fb:,.0f} | {wb:,.0f} | {fb + wb:,.0f} | {f'{alg:,}' if alg else ''} | {ratio} |")
        if w == DOMINANT:
            dom = {"kernel": kernel_label(name), "workload": DOMINANT,
                   "hbm_bytes_per_launch": round(fb + wb), "fetch_bytes_per_launch": round(fb),
                   "write_bytes_per_launch": round(wb), "algorithmic_bytes_per_launch": io[w],
                   "fetch_unit_bytes": round(fu, 4), "write_unit_bytes": round(wu, 4),
                   "source": "profiles/hbm_traffic_pmc_bench_step.md",
                   "kernel_source_sha256": kernel_source_hash()}
    lines += ["", "Every input is read once and every output written once when total / algorithmic "
              "is 1; the remainder is parameter, workspace and counter-granularity traffic."]
    with open(os.path.join(prof, "hbm_traffic_pmc_bench_step.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if dom is None:
        sys.exit(f"no {DOMINANT} kernel in the counter runs")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(dom, f, indent=1)
        f.write("\n")

    # --- The five workloads alone: per-dispatch durations, attributed in order.
    trace = _read_csv(_find_csv(os.path.join(d, "ktc"), "kernel_trace.csv"))
    runs = []  # [(kernel name, [durations])] of consecutive non-copy dispatches
    for r in trace:
        fam = kernel_family(r["Kernel_Name"])[0]
        if fam == "copy16_kernel" or "FillFunctor" in r["Kernel_Name"] or "rocclr" in r["Kernel_Name"]:
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == r["Kernel_Name"]:
            runs[-1][1].append(dur)
        else:
            runs.append((r["Kernel_Name"], [dur]))
    if len(runs) != len(workloads.ORDER):
        sys.exit(f"expected {len(workloads.ORDER)} runs of op kernels in the configs trace, found {len(runs)}")
    lines = ["# The five reference workloads, each alone and cold: rocprofv3 kernel trace", "",
             "Command (`$REPO` = repository root, `$OUT` = the output directory given to "
             "`bench.py --summarize`):", "", "```",
             cmd("ktc"), "```", "",
             "Every invocation follows a 1 GiB copy (the copy kernel), so each starts from a cold cache. "
             "Durations per dispatch come from `configs_kernel_trace.csv` (5 warm-up and 60 timed "
             "dispatches per workload, all counted).", "",
             "| workload | kernel | dispatches | median us | min us | p90 us | GB/s (median) | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|"]
    for wname, (kname, durs) in zip(workloads.ORDER, runs):
        a = np.array(durs)
        med = float(np.median(a))
        gbps = io[wname] / med / 1e3
        lines.append(f"| {wname} | {kernel_label(kname)} | {len(a)} | {med:.2f} | {a.min():.2f} | "
                     f"{np.percentile(a, 90):.2f} | {gbps:.1f} | {100 * gbps / PEAK_GBPS:.1f} |")
    cfg_path = os.path.join(d, "configs.json")
    if os.path.exists(cfg_path):
        c = _read_json_line(cfg_path)
        h = c.get("host", {})
        lines += ["", "Same workloads in a separate run without the profiler (`" + PROF_COMMANDS["configs"] +
                  "`). Times are HIP events per invocation: device-scope release events around the op, "
                  "spanning the launch. The same-bytes copy is the copy kernel moving the workload's "
                  "byte count, also cold. The oracle runs on one thread. Copy ceiling "
                  f"{c['copy_ceiling_gbps']} GB/s, hipMemcpyDtoD {c['memcpy_dtod_ceiling_gbps']} GB/s; host: "
                  f"{h.get('model', '?')}, {h.get('cpu_count', '?')} logical CPUs, oracle on 1.", "",
                  "| workload | median us (events) | GB/s | % of 8 TB/s | % of copy | same-bytes copy us | "
                  "% of same-bytes copy | oracle s | oracle GB/s |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for r in c["configs"]:
            lines.append(f"| {r['workload']} | {r['median_us']} | {r['gbps']} | {100 * r['frac_of_peak']:.1f} | "
                         f"{100 * r['frac_of_copy']:.1f} | {r['same_bytes_copy_us']} | "
                         f"{100 * r['frac_of_same_bytes_copy']:.1f} | {r.get('oracle_s', '')} | "
                         f"{r.get('oracle_gbps', '')} |")
    with open(os.path.join(prof, "configs_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    shapes_path = os.path.join(d, "shapes.json")
    if os.path.exists(shapes_path):
        sh = _read_json_line(shapes_path)
        lines = ["# General shapes: every route family beyond the five workloads", "",
                 "Command (`$REPO` = repository root, `$OUT` = the output directory given to "
                 "`bench.py --summarize`):", "", "```",
                 PROF_COMMANDS["shapes"] + " > $OUT/shapes.json", "```", "",
                 "Each shape alone, cold (a 1 GiB copy before every call), HIP events around the op on its "
                 f"stream, median of {sh['invocations']} calls; inputs drawn on the device "
                 "(`workloads.generate_on_device`, seed 0). GB/s counts algorithmic bytes: every input read "
                 "once, every output (Y and S for the skip ops) written once. One MI355X.", "",
                 "| shape | route | median us | GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
        for r in sh["shapes"]:
            forced = "" if r["forced"] == "auto" else " (forced)"
            lines.append(f"| {r['shape']} | {r['route']}{forced} | {r['median_us']} | {r['gbps']} | "
                         f"{100 * r['gbps'] / PEAK_GBPS:.1f} |")
        with open(os.path.join(prof, "general_shapes.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    log(f"wrote profiles/kernel_trace_bench_step.md, hbm_traffic_pmc_bench_step.md, configs_kernel_trace.md, "
        f"{os.path.basename(TRAFFIC_FILE)} (dominant kernel {dom['hbm_bytes_per_launch']:,} bytes per launch)")


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
    ap.add_argument("--shapes", action="store_true",
                    help="general shapes (wide rows, ...) on the automatic and forced routes")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 output collected under DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
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
    if args.shapes:
        shapes_table(args)
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
