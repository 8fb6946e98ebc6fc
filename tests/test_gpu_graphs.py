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
        # Rows off the 16-byte vector grid: SSLN rows of 4095 (the phased
        # route) and GatedRMSNorm rows of 25 (the flat route).
        "xo": rn(24, 4095), "ko": rn(24, 4095), "go": rn(4095),
        "Xf": rn(300, 25), "gf": rn(300, 25), "sf": rn(25),
        # SSLN rows of 127 (the flat route).
        "xq": rn(300, 127), "kq": rn(300, 127), "gq": rn(127), "bq": rn(127),
        # SkipGroupNorm shapes whose groups span several workgroups, so that
        # every replay exchanges moments: NHWC 32 slices per channel block,
        # NCHW 16-byte vectors, and NCHW groups off the 16-byte grid (31 x 31
        # planes, the phased route).
        "Xh": rn(2, 64, 64, 320), "kh": rn(2, 64, 64, 320), "bh": rn(320),
        "gh": rn(320, dtype=torch.float32), "eh": rn(320, dtype=torch.float32),
        "Xc": rn(2, 640, 32, 32, dtype=torch.float32), "kc": rn(2, 640, dtype=torch.float32),
        "gc": rn(640), "ec": rn(640),
        "Xp": rn(2, 640, 31, 31), "kp": rn(2, 640, 31, 31), "bp": rn(640),
        "gp": rn(640, dtype=torch.float32), "ep": rn(640, dtype=torch.float32),
        # Rows of 100000 float16 (the wide route: VGPRs plus LDS), GatedRMSNorm
        # spans of 2049 (the phased route), and NHWC pixels of 15 channels
        # (the channel-block cluster with element accesses, exchanging moments).
        "xw": rn(3, 100000), "kw": rn(3, 100000), "gw": rn(100000),
        "Xg": rn(24, 2049), "gg": rn(24, 2049), "sg": rn(2049),
        "Xn": rn(2, 16, 16, 15), "kn": rn(2, 16, 16, 15), "gn": rn(15, dtype=torch.float32),
        "en": rn(15, dtype=torch.float32),
        # Larger NHWC images of 15 channels: the cluster over packed runs of
        # 8 pixels (16-byte accesses), 32 slices exchanging moments.
        "Xr": rn(8, 64, 128, 15), "kr": rn(8, 64, 128, 15), "gr": rn(15, dtype=torch.float32),
        "er": rn(15, dtype=torch.float32),
    }
    t["ws_h"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xh"], 32, 1), dtype=torch.uint8,
                            device="cuda")
    t["ws_c"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xc"], 32, 0), dtype=torch.uint8,
                            device="cuda")
    t["ws_p"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xp"], 32, 0), dtype=torch.uint8,
                            device="cuda")
    t["ws_n"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xn"], 5, 1), dtype=torch.uint8,
                            device="cuda")
    t["ws_r"] = torch.empty(gn.skip_group_norm_workspace_size(t["Xr"], 5, 1), dtype=torch.uint8,
                            device="cuda")
    return t


def run(t):
    a = gn.skip_rms_norm(t["x"], t["k"], t["gamma"], None, 1e-6, want_inv_std_var=True, want_sum=True)
    b = gn.skip_layer_norm(t["x"], t["k"], t["gamma"], t["beta"], None, 1e-5, want_mean=True,
                           want_inv_std_var=True)
    c = gn.gated_rms_norm(t["X"], t["scale"], t["gate"], 1e-5)
    o = gn.skip_rms_norm(t["xo"], t["ko"], t["go"], None, 1e-6, want_sum=True)
    route_o = gn.last_route()
    fl = gn.gated_rms_norm(t["Xf"], t["sf"], t["gf"], 1e-5)
    route_f = gn.last_route()
    q = gn.skip_rms_norm(t["xq"], t["kq"], t["gq"], t["bq"], 1e-6, want_inv_std_var=True, want_sum=True)
    route_q = gn.last_route()
    d = gn.skip_group_norm(t["Xh"], t["gh"], t["eh"], t["kh"], t["bh"], groups=32, activation=1,
                           channels_last=1, want_sum=True, workspace=t["ws_h"])
    route_h = gn.last_route()
    e = gn.skip_group_norm(t["Xc"], t["gc"], t["ec"], t["kc"], None, groups=32, activation=0,
                           channels_last=0, workspace=t["ws_c"])
    route_c = gn.last_route()
    f = gn.skip_group_norm(t["Xp"], t["gp"], t["ep"], t["kp"], t["bp"], groups=32, activation=1,
                           channels_last=0, want_sum=True, workspace=t["ws_p"])
    route_p = gn.last_route()
    wd = gn.skip_rms_norm(t["xw"], t["kw"], t["gw"], None, 1e-6, want_sum=True)
    route_w = gn.last_route()
    gp = gn.gated_rms_norm(t["Xg"], t["sg"], t["gg"], 1e-5)
    route_g = gn.last_route()
    pk = gn.skip_group_norm(t["Xn"], t["gn"], t["en"], t["kn"], None, groups=5, activation=1,
                            channels_last=1, want_sum=True, workspace=t["ws_n"])
    route_n = gn.last_route()
    pr = gn.skip_group_norm(t["Xr"], t["gr"], t["er"], t["kr"], None, groups=5, activation=1,
                            channels_last=1, want_sum=True, workspace=t["ws_r"])
    route_r = gn.last_route()
    outs = [a.output, a.inv_std_var, a.input_skip_bias_sum, b.output, b.mean, b.inv_std_var, c,
            d.Y, d.S, e.Y, f.Y, f.S, o.output, o.input_skip_bias_sum, fl, q.output, q.inv_std_var,
            q.input_skip_bias_sum, wd.output, wd.input_skip_bias_sum, gp, pk.Y, pk.S, pr.Y, pr.S]
    return outs, (route_h, route_c, route_p, route_o, route_f, route_q, route_w, route_g, route_n, route_r)


def refill(t, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    for name in ("x", "k", "X", "gate", "xo", "ko", "Xf", "gf", "xq", "kq", "Xh", "kh", "Xc", "kc", "Xp", "kp",
                 "xw", "kw", "Xg", "gg", "Xn", "kn", "Xr", "kr"):
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
    assert routes == ("sgn.cluster.nhwc.vec16", "sgn.cluster.nchw.vec16", "sgn.cluster.nchw.phase",
                      "ssln.phase.vec16", "gated.flat.vec16", "ssln.flat.vec16", "ssln.wide.vec16",
                      "gated.phase.vec16", "sgn.cluster.nhwc.scalar", "sgn.cluster.nhwc.packed.vec16"), routes
    torch.cuda.synchronize()

    names = ["ssln output", "ssln inv_std_var", "ssln S", "sln output", "sln mean", "sln inv_std_var",
             "gated Y", "sgn nhwc Y", "sgn nhwc S", "sgn nchw Y", "sgn nchw phased Y", "sgn nchw phased S",
             "ssln phased output", "ssln phased S", "gated flat Y", "ssln flat output", "ssln flat inv_std_var",
             "ssln flat S", "ssln wide output", "ssln wide S", "gated phased Y", "sgn odd-C Y", "sgn odd-C S",
             "sgn packed Y", "sgn packed S"]
    for rep in range(4):
        refill(t, seed=100 + rep)
        graph.replay()
        torch.cuda.synchronize()
        got = [to_host(o).copy() for o in captured]
        ref, _ = run(t)
        torch.cuda.synchronize()
        for n, gv, rv in zip(names, got, ref):
            assert_bitwise(gv, to_host(rv), f"replay {rep}: {n}")
