"""HIP graph capture and replay (torch.cuda.CUDAGraph): every operator is
captured once and replayed with new inputs written in place; each replay's
outputs must equal, bit for bit, the same calls made eagerly on the same
inputs, with eager work between the replays.  SkipGroupNorm's single-launch
routes tell a call's exchanged moments from earlier ones by a per-call value
that a replay repeats; under capture they record a kernel that clears those
values ahead of the launch, which these replays (with changed inputs)
exercise."""
import pytest
import torch

import group_normalization_amd as gn
from parity import assert_bitwise, to_host

pytestmark = pytest.mark.gpu


def make_inputs():
    g = torch.Generator(device="cuda").manual_seed(7)

    def rn(*shape, dtype=torch.float16):
        return torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).to(dtype)

    t = {
        "x": rn(24, 4096), "k": rn(24, 4096), "gamma": rn(4096), "beta": rn(4096),
        "X": rn(64, 4 * 128), "gate": rn(64, 4 * 128), "scale": rn(128),
        "Xh": rn(2, 16, 16, 320), "kh": rn(2, 16, 16, 320), "bh": rn(320),
        "gh": rn(320, dtype=torch.float32), "eh": rn(320, dtype=torch.float32),
        "Xc": rn(2, 640, 8, 8, dtype=torch.float32), "kc": rn(2, 640, dtype=torch.float32),
        "gc": rn(640), "ec": rn(640),
    }
    t["ws_h"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xh"], 32, 1), dtype=torch.uint8,
                            device="cuda")
    t["ws_c"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xc"], 32, 0), dtype=torch.uint8,
                            device="cuda")
    return t


def run(t):
    a = gn.skip_rms_norm(t["x"], t["k"], t["gamma"], None, 1e-6, want_inv_std_var=True, want_sum=True)
    b = gn.skip_layer_norm(t["x"], t["k"], t["gamma"], t["beta"], None, 1e-5, want_mean=True,
                           want_inv_std_var=True)
    c = gn.gated_rms_norm(t["X"], t["scale"], t["gate"], 1e-5)
    d = gn.skip_group_norm(t["Xh"], t["gh"], t["eh"], t["kh"], t["bh"], groups=32, activation=1,
                           channels_last=1, want_sum=True, workspace=t["ws_h"])
    route_h = gn.last_route()
    e = gn.skip_group_norm(t["Xc"], t["gc"], t["ec"], t["kc"], None, groups=32, activation=0,
                           channels_last=0, workspace=t["ws_c"])
    route_c = gn.last_route()
    outs = [a.output, a.inv_std_var, a.input_skip_bias_sum, b.output, b.mean, b.inv_std_var, c,
            d.Y, d.S, e.Y]
    return outs, (route_h, route_c)


def refill(t, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    for name in ("x", "k", "X", "gate", "Xh", "kh", "Xc", "kc"):
        v = t[name]
        v.copy_(torch.randn(v.shape, generator=g, device="cuda", dtype=torch.float32).to(v.dtype))


def test_graph_replays_match_eager():
    t = make_inputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured, routes = run(t)
    assert routes[0].startswith("sgn.cluster.nhwc") and routes[1].startswith("sgn.cluster.nchw"), routes
    torch.cuda.synchronize()

    names = ["ssln output", "ssln inv_std_var", "ssln S", "sln output", "sln mean", "sln inv_std_var",
             "gated Y", "sgn nhwc Y", "sgn nhwc S", "sgn nchw Y"]
    for rep in range(4):
        refill(t, seed=100 + rep)
        graph.replay()
        torch.cuda.synchronize()
        got = [to_host(o).copy() for o in captured]
        ref, _ = run(t)
        torch.cuda.synchronize()
        for n, gv, rv in zip(names, got, ref):
            assert_bitwise(gv, to_host(rv), f"replay {rep}: {n}")
