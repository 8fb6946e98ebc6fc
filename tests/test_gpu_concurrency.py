"""Concurrent use: calls on two streams at once (each with its own workspace
and inputs) and from two host threads at once must give, bit for bit, the
results the same calls give one after the other.  SkipGroupNorm's
single-launch routes exchange partial moments between the workgroups of one
launch, identified by a per-call tag; two such launches in flight together
must not take each other's moments.  (Calls that share a workspace must be
ordered; these do not share one.)"""
import threading

import numpy as np
import pytest
import torch

import group_normalization_amd as gn
from parity import assert_bitwise, to_host

pytestmark = pytest.mark.gpu


def make_inputs(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)

    def rn(*shape, dtype=torch.float16):
        return torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).to(dtype)

    t = {"x": rn(64, 4096), "k": rn(64, 4096), "gamma": rn(4096), "beta": rn(4096),
         "X": rn(256, 512), "gate": rn(256, 512), "scale": rn(128),
         "Xh": rn(2, 32, 32, 320), "kh": rn(2, 32, 32, 320), "bh": rn(320),
         "gh": rn(320, dtype=torch.float32), "eh": rn(320, dtype=torch.float32),
         # NCHW groups spread over several workgroups (moments exchanged):
         # 16-byte vectors, and 31 x 31 planes off the 16-byte grid (phased).
         "Xc": rn(2, 640, 32, 32, dtype=torch.float32), "kc": rn(2, 640, dtype=torch.float32),
         "gc": rn(640), "ec": rn(640),
         "Xp": rn(2, 320, 31, 31), "kp": rn(2, 320, 31, 31), "bp": rn(320),
         "gp": rn(320, dtype=torch.float32), "ep": rn(320, dtype=torch.float32)}
    t["ws_h"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xh"], 32, 1), dtype=torch.uint8,
                            device="cuda")
    t["ws_c"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xc"], 32, 0), dtype=torch.uint8,
                            device="cuda")
    t["ws_p"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xp"], 32, 0), dtype=torch.uint8,
                            device="cuda")
    return t


def run(t):
    a = gn.skip_rms_norm(t["x"], t["k"], t["gamma"], None, 1e-6, want_sum=True)
    b = gn.skip_layer_norm(t["x"], t["k"], t["gamma"], t["beta"], None, 1e-5, want_mean=True)
    c = gn.gated_rms_norm(t["X"], t["scale"], t["gate"], 1e-5)
    d = gn.skip_group_norm(t["Xh"], t["gh"], t["eh"], t["kh"], t["bh"], groups=32, activation=1,
                           channels_last=1, want_sum=True, workspace=t["ws_h"])
    e = gn.skip_group_norm(t["Xc"], t["gc"], t["ec"], t["kc"], None, groups=32, activation=0,
                           channels_last=0, workspace=t["ws_c"])
    f = gn.skip_group_norm(t["Xp"], t["gp"], t["ep"], t["kp"], t["bp"], groups=32, activation=1,
                           channels_last=0, want_sum=True, workspace=t["ws_p"])
    return [a.output, a.input_skip_bias_sum, b.output, b.mean, c, d.Y, d.S, e.Y, f.Y, f.S]


def host(outs):
    return [to_host(o).copy() for o in outs]


def test_two_streams_in_flight():
    ins = [make_inputs(1), make_inputs(2)]
    ref = [host(run(t)) for t in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [[], []]
    for _ in range(8):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                got[i].append(run(ins[i]))
    torch.cuda.synchronize()
    for i in range(2):
        for rep, outs in enumerate(got[i]):
            for j, (gv, rv) in enumerate(zip(host(outs), ref[i])):
                assert_bitwise(gv, rv, f"stream {i} call {rep} output {j}")


def test_two_host_threads():
    ins = [make_inputs(3), make_inputs(4)]
    ref = [host(run(t)) for t in ins]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(10):
                    outs = run(ins[i])
                    s.synchronize()
                    for j, (gv, rv) in enumerate(zip(host(outs), ref[i])):
                        assert_bitwise(gv, rv, f"thread {i} call {rep} output {j}")
        except Exception as exc:  # reported on the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[0]
