"""SkipGroupNorm: HIP path (through the C ABI) against the oracle."""
import math

import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
import workloads
from plans import nhwc_cluster_fits, nhwc_packed_cluster_fits, packed_applies, packed_blocks
from parity import assert_bitwise, assert_close, desc, to_dev, to_host

pytestmark = pytest.mark.gpu

F32, F16 = np.float32, np.float16


def run(x, w, route="auto", want_sum=True, skip_override=None):
    a = w.attrs
    skip = x["skip"] if skip_override is None else skip_override
    ref_y, ref_s = oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], skip, x.get("bias"),
                                          groups=a["groups"], activation=a["activation"],
                                          epsilon=a["epsilon"], channels_last=a["channels_last"],
                                          want_sum=True)
    with gn.force_route(route):
        out = gn.skip_group_norm(to_dev(x["X"]), to_dev(x["gamma"]), to_dev(x["beta"]), to_dev(skip),
                                 to_dev(x.get("bias")), groups=a["groups"],
                                 activation=a["activation"], epsilon=a["epsilon"],
                                 channels_last=a["channels_last"], want_sum=want_sum)
        used = gn.last_route()
    torch.cuda.synchronize()
    return (ref_y, ref_s), out, used


def check(ref, out, want_sum=True):
    assert_close(to_host(out.Y), ref[0], "Y")
    if want_sum:
        assert_bitwise(to_host(out.S), ref[1], "S")


# (N, C, H, W, T, M, channels_last, broadcast skip, bias, groups, activation)
CASES = [
    (2, 320, 16, 16, F16, F32, 1, False, True, 32, 1),    # the NHWC workload's channel layout
    (2, 1280, 8, 8, F32, F16, 0, True, False, 32, 0),     # the NCHW workload's channel layout
    (3, 64, 7, 9, F16, F16, 1, True, True, 8, 0),
    (2, 96, 5, 5, F32, F32, 0, False, True, 4, 1),        # H*W = 25: not a whole vector
    (1, 40, 13, 11, F16, F32, 1, False, False, 5, 1),
    (2, 12, 6, 6, F16, F16, 1, False, True, 3, 0),        # 24-byte pixels, 4-channel groups: 8-byte accesses
    (2, 16, 4, 4, F32, F32, 0, True, True, 16, 1),        # groups == C (instance norm)
    (2, 24, 3, 5, F16, F32, 0, False, False, 1, 0),       # one group (layer norm)
    (1, 4096, 2, 2, F16, F16, 1, False, True, 32, 0),     # 512 vectors per pixel: 2 channel blocks
    (3, 8, 1, 1, F32, F16, 1, True, False, 2, 1),         # H = W = 1
    (2, 2560, 8, 8, F32, F32, 1, False, True, 32, 1),     # 640 vectors per pixel: 8 channel blocks
    # Pixels that are not a whole number of 16-byte vectors: runs of pixels that are.
    (2, 15, 8, 8, F16, F32, 1, False, True, 5, 1),        # 8 pixels = 15 vectors per run
    (3, 3, 16, 16, F16, F16, 1, True, True, 1, 0),        # 8 pixels = 3 vectors, broadcast skip
    (2, 75, 8, 8, F16, F32, 1, False, False, 5, 1),       # 8 pixels = 75 vectors
    (2, 15, 4, 6, F32, F16, 1, False, True, 3, 1),        # float32: 4 pixels = 15 vectors
    (1, 5, 40, 40, F32, F32, 1, True, False, 5, 0),       # float32 instance norm, 4 pixels = 5 vectors
    (4, 15, 64, 64, F16, F32, 1, False, True, 5, 1),      # many pixel runs per image
    (1, 257, 4, 4, F16, F32, 1, False, True, 1, 0),       # 8 pixels = 257 vectors: scalars
    (2, 15, 5, 5, F16, F32, 1, False, True, 5, 1),        # 25 pixels, not whole runs of 8: scalars
    (1, 15, 512, 512, F16, F32, 1, False, True, 5, 1),    # 5 x 964 partials: a finalize launch
    # Packed runs in the cluster (256 workgroups): float16 parameters and a
    # broadcast skip; float32 data without bias.
    (8, 15, 64, 128, F16, F16, 1, True, True, 5, 0),
    (8, 15, 64, 64, F32, F16, 1, False, False, 5, 1),
]


def split_channel_blocks(C, cpg, e):
    """Channel blocks of the split route's NHWC tiling for vectors of e
    channels: the fewest equal blocks of whole groups and vectors, at most
    256 vectors each, that keep 90 % of a block's 256 threads busy, else the
    busiest; 0 when there is none (the library's rule, restated)."""
    if C % e or C % cpg:
        return 0
    unit = cpg // math.gcd(cpg, e) * e
    nb0 = C // unit
    best, best_busy = 0, -1
    for ncb in range(1, nb0 + 1):
        if nb0 % ncb:
            continue
        cbv = C // e // ncb
        if cbv > 256:
            continue
        busy = 256 // cbv * cbv
        if busy > best_busy:
            best, best_busy = ncb, busy
        if busy * 10 >= 256 * 9:
            break
    return best


def nhwc_route(C, groups, T, HW, N=1):
    """The NHWC route the library picks for aligned tensors of these
    channels: the cluster over packed runs of pixels where a pixel is not a
    whole number of 16-byte vectors and the runs fit; else the channel-block
    cluster with the widest of 16-, 8- and
    4-byte accesses that divides a pixel and is no wider than a group;
    otherwise the split route with the widest access, or over runs of
    pixels that make whole 16-byte vectors (at most 256 of them, H*W a
    whole number of runs), or scalars."""
    size = np.dtype(T).itemsize
    width = next((b for b in (16, 8, 4) if b > size and C * size % b == 0), size)
    names = {16: "vec16", 8: "vec8", 4: "vec4"}
    w = width
    while w > size and C // groups < w // size:
        w //= 2
    block = nhwc_cluster_fits(C, groups, w // size, HW)
    if nhwc_packed_cluster_fits(N, C, groups, size, HW, block):
        return "sgn.cluster.nhwc.packed.vec16"
    if block:
        return f"sgn.cluster.nhwc.{names[w]}" if w > size else "sgn.cluster.nhwc.scalar"
    if width > size and split_channel_blocks(C, C // groups, width // size):
        return f"sgn.split.nhwc.{names[width]}"
    if packed_applies(C, HW, size):
        # Normalize blocks combine their groups' partials themselves when
        # there are at most 64 groups and 1024 partials.
        if groups <= 64 and groups * packed_blocks(N, C, HW, size) <= 1024:
            return "sgn.split.nhwc.packed.fold.vec16"
        return "sgn.split.nhwc.packed.vec16"
    return "sgn.split.nhwc.scalar"


def make(case, seed=0):
    N, C, H, W, T, M, cl, bc, bias, groups, act = case
    w = workloads.sgn("t", N, C, H, W, T, M, channels_last=bool(cl), broadcast_skip=bc, bias=bias,
                      groups=groups, activation=act, epsilon=1e-5)
    return w, workloads.generate(w, seed=seed + N * C + H)


@pytest.mark.parametrize("route", ["auto", "split", "scalar", "block"])
@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}C{c[1]}H{c[2]}W{c[3]}-{np.dtype(c[4]).name}/"
                                             f"{np.dtype(c[5]).name}-{'nhwc' if c[6] else 'nchw'}"
                                             f"{'-bc' if c[7] else ''}{'-b' if c[8] else ''}-g{c[9]}"
                                             f"-a{c[10]}" for c in CASES])
def test_matches_oracle(case, route):
    w, x = make(case)
    ref, out, used = run(x, w, route)
    check(ref, out)
    N, C, H, W, T, M, cl, bc, bias, groups, act = case
    if route == "scalar":
        assert used.endswith(".scalar")
    if route == "split":
        assert used.startswith("sgn.split")
    if route == "block":
        assert used.startswith("sgn.split") and used.endswith(".scalar")
    if route == "auto" and not cl:
        assert used.startswith("sgn.cluster")  # every NCHW case here fits the cluster route
    if route == "auto" and cl:
        assert used == nhwc_route(C, groups, T, H * W, N)


# The split route's NHWC tiling over channel blocks: pixels wider than 256
# vectors, or whose 256-thread blocks would leave over a tenth of the
# threads idle, are cut into equal blocks of whole groups and vectors.
SPLIT_BLOCK_CASES = [
    # (case, channel blocks, route)
    ((2, 1280, 9, 7, F16, F32, 1, False, True, 32, 1), 2, "sgn.split.nhwc.vec16"),   # 160 vectors: 2 x 80
    ((2, 1280, 40, 40, F16, F32, 1, True, True, 32, 1), 2, "sgn.split.nhwc.vec16"),  # 267 pixel runs
    ((1, 2560, 5, 6, F32, F16, 1, True, False, 32, 0), 8, "sgn.split.nhwc.vec16"),   # 640 vectors: 8 x 80
    ((2, 4096, 3, 3, F16, F16, 1, False, True, 32, 1), 2, "sgn.split.nhwc.vec16"),   # 512 vectors: 2 x 256
    ((1, 1200, 4, 5, F16, F32, 1, False, True, 30, 1), 3, "sgn.split.nhwc.vec16"),   # 150 vectors: 3 x 50
    # 10-channel groups straddle 16-byte vectors: blocks of 5 vectors (4 groups) each.
    ((2, 1040, 4, 4, F16, F32, 1, True, True, 104, 1), 13, "sgn.split.nhwc.vec16"),
    ((2, 40, 8, 8, F32, F32, 1, False, True, 4, 0), 1, "sgn.split.nhwc.vec16"),      # one block
    # One group of 257 sixteen-byte vectors: no channel blocks, scalar accesses.
    ((1, 2056, 3, 3, F16, F32, 1, False, True, 1, 1), 0, "sgn.split.nhwc.scalar"),
]


@pytest.mark.parametrize("case,ncb,want_route", SPLIT_BLOCK_CASES,
                         ids=[f"N{c[0][0]}C{c[0][1]}H{c[0][2]}W{c[0][3]}-{np.dtype(c[0][4]).name}-g{c[0][9]}"
                              for c in SPLIT_BLOCK_CASES])
def test_split_channel_blocks(case, ncb, want_route):
    N, C, H, W, T, M, cl, bc, bias, groups, act = case
    size = np.dtype(T).itemsize
    assert split_channel_blocks(C, C // groups, 16 // size) == ncb
    w, x = make(case, seed=9)
    ref, out, used = run(x, w, "split")
    assert used == want_route
    check(ref, out)
    _, no_s, _ = run(x, w, "split", want_sum=False)  # pass 3 re-forms S from X and skip
    assert_bitwise(to_host(no_s.Y), to_host(out.Y), "Y without S")


# NCHW groups around the cluster route's limits (per (n, group), at most 8
# workgroups of 256 threads): 16 sixteen-byte vectors or 32 scalars per thread.
LIMIT_CASES = [
    # (N, C, H, W, T, groups, broadcast skip, expected auto route)
    (1, 32, 64, 64, F32, 1, False, "sgn.cluster.nchw.vec16"),  # 32768 vectors: 8 full workgroups
    (1, 33, 64, 64, F32, 1, False, "sgn.split.nchw.vec16"),    # 33792 vectors
    (1, 64, 64, 64, F16, 2, True, "sgn.cluster.nchw.vec16"),   # 16384 vectors of halves
    (2, 16, 32, 32, F16, 1, True, "sgn.cluster.nchw.vec16"),   # 2048 vectors, 8 small slices
    (1, 64, 31, 33, F32, 1, False, "sgn.cluster.nchw.phase"),  # odd H*W: 16370 phased vectors, 8 slices
    (1, 65, 31, 33, F32, 1, False, "sgn.split.nchw.scalar"),   # 66495 elements
    (3, 6, 7, 7, F16, 3, True, "sgn.cluster.nchw.phase"),      # 7 x 7: phased, one slice
    (1, 600, 1, 3, F32, 1, False, "sgn.cluster.nchw.scalar"),  # H*W = 3 < one vector: scalars, 8 slices
    (1, 2, 1, 3, F32, 2, False, "sgn.cluster.nchw.scalar"),    # 3 elements: 3 slices of 1
]


@pytest.mark.parametrize("case", LIMIT_CASES, ids=[f"N{c[0]}C{c[1]}H{c[2]}W{c[3]}-{np.dtype(c[4]).name}"
                                                   f"-g{c[5]}{'-bc' if c[6] else ''}" for c in LIMIT_CASES])
def test_group_block_limits(case):
    N, C, H, W, T, groups, bc, want_route = case
    w = workloads.sgn("t", N, C, H, W, T, np.float32, channels_last=False, broadcast_skip=bc,
                      bias=True, groups=groups, activation=1, epsilon=1e-5)
    x = workloads.generate(w, seed=C + H)
    ref, out, used = run(x, w)
    assert used == want_route
    check(ref, out)


# NHWC channel-block cluster around its limits: at most 64 slices per
# (image, channel block), 16 pixels per thread, 16 groups per block, and
# groups at least one 16-byte vector wide.
NHWC_LIMIT_CASES = [
    # (N, C, H, W, T, groups, broadcast skip, expected auto route)
    (2, 320, 64, 64, F16, 32, False, "sgn.cluster.nhwc.vec16"),   # 51 pixel lanes (odd), 32 slices
    (1, 320, 204, 256, F16, 32, False, "sgn.cluster.nhwc.vec16"), # 52224 pixels: 64 slices, 16 pixels/thread
    (1, 320, 205, 256, F16, 32, True, "sgn.split.nhwc.vec16"),    # 52480 pixels: too many
    (8, 40, 32, 32, F16, 5, False, "sgn.cluster.nhwc.vec16"),     # one vector per block
    (2, 72, 16, 16, F16, 8, True, "sgn.cluster.nhwc.vec16"),      # 9 channels/group: 2 groups per wave
    (16, 144, 8, 8, F16, 16, False, "sgn.cluster.nhwc.vec16"),    # 16 groups per block: 4 per wave
    (2, 96, 9, 11, F16, 8, False, "sgn.cluster.nhwc.vec16"),      # 12 channels/group, ragged last slice
    (2, 64, 8, 8, F16, 16, False, "sgn.cluster.nhwc.vec8"),       # 4 channels/group: 8-byte vectors
    (2, 64, 8, 8, F16, 32, True, "sgn.cluster.nhwc.vec4"),        # 2 channels/group: 4-byte vectors
    (2, 64, 8, 8, F16, 64, False, "sgn.cluster.nhwc.scalar"),     # 1 channel/group: element accesses
    (2, 324, 16, 16, F16, 36, False, "sgn.cluster.nhwc.vec8"),    # 648-byte pixels: 8-byte vectors
    (2, 162, 8, 8, F16, 18, True, "sgn.cluster.nhwc.vec4"),       # 324-byte pixels: 4-byte vectors
    (2, 90, 8, 8, F32, 9, False, "sgn.cluster.nhwc.vec8"),        # float32 360-byte pixels
    (1, 16, 9, 7, F32, 4, True, "sgn.cluster.nhwc.vec16"),        # float32, 4 channels/group, 1 slice
    (2, 2560, 8, 8, F32, 32, False, "sgn.cluster.nhwc.vec16"),    # 640 vectors per pixel, 3 pixel lanes
    (600, 16, 2, 2, F32, 2, True, "sgn.cluster.nhwc.vec16"),      # one slice per image: no exchange
    # Element accesses: odd C (five blocks of one 3-channel group, 85 pixel
    # lanes) up to 64 slices of 16 pixels per thread; beyond, the cluster over
    # packed runs of 8 pixels (17 run lanes) up to 64 slices of 16 runs per
    # thread, then the split route over the same runs (5 x 513 partials: a
    # finalize launch).
    (1, 15, 340, 256, F16, 5, False, "sgn.cluster.nhwc.scalar"),
    (1, 15, 341, 256, F16, 5, True, "sgn.cluster.nhwc.packed.vec16"),
    (1, 15, 544, 256, F16, 5, False, "sgn.cluster.nhwc.packed.vec16"),
    (1, 15, 545, 256, F16, 5, True, "sgn.split.nhwc.packed.vec16"),
    (2, 15, 64, 64, F32, 5, True, "sgn.cluster.nhwc.scalar"),     # float32 odd C, broadcast skip
    # Packed runs of pixels (whole 16-byte vectors) where their grid has at
    # least 256 workgroups, or 96 with 12 runs per thread; else element or
    # narrow accesses.
    (8, 15, 128, 128, F16, 5, False, "sgn.cluster.nhwc.packed.vec16"),  # runs of 8 pixels, 15 vectors
    (8, 15, 64, 128, F32, 5, True, "sgn.cluster.nhwc.packed.vec16"),    # float32 runs of 4, broadcast skip
    (16, 3, 128, 128, F16, 1, False, "sgn.cluster.nhwc.packed.vec16"),  # 3-vector runs, one group
    (8, 60, 64, 64, F16, 15, False, "sgn.cluster.nhwc.packed.vec16"),   # 15 groups of 4 channels
    (8, 36, 128, 128, F16, 12, False, "sgn.cluster.nhwc.packed.vec16"), # groups of 3 channels
    (8, 15, 256, 256, F16, 5, False, "sgn.cluster.nhwc.packed.vec16"),  # 16 runs per thread
    # 16 images of 40 slices: 640 workgroups of 16 runs per thread, more than
    # are resident at once (two a CU), each cluster's 40 ids within reach:
    # slice-major.
    (16, 15, 340, 256, F16, 5, False, "sgn.cluster.nhwc.smajor.packed.vec16"),
    (4, 12, 128, 128, F16, 3, True, "sgn.cluster.nhwc.vec8"),           # 128 workgroups: 8-byte accesses
    (4, 15, 256, 256, F16, 5, False, "sgn.cluster.nhwc.packed.vec16"),  # 128 workgroups of 16 runs per thread
    (2, 15, 256, 256, F16, 5, False, "sgn.cluster.nhwc.scalar"),        # 64 of 16: element accesses
    (2, 1, 17, 19, F16, 1, False, "sgn.cluster.nhwc.scalar"),     # one channel
    (2, 2, 5, 7, F16, 2, True, "sgn.cluster.nhwc.scalar"),        # two one-channel groups
    (3, 3, 1, 1, F32, 3, False, "sgn.cluster.nhwc.scalar"),       # one pixel: every group one value
    (2, 2, 3, 3, F16, 1, False, "sgn.cluster.nhwc.vec4"),         # 4-byte pixels, one group
    # Residency (MI355X: 256 CUs, two workgroups each at 16 pixels per
    # thread): 704 workgroups, more than are resident at once, but each
    # image's 88 within reach of one another: one launch in two rounds,
    # slice-major block order.
    (8, 640, 64, 64, F16, 32, False, "sgn.cluster.nhwc.smajor.vec16"),
    # Instance norm (one channel a group): 20 blocks of 16 channels x 16
    # slices of 16 pixels per thread, 2560 workgroups, more than are resident
    # at once: slice-major.
    (8, 320, 64, 64, F16, 320, False, "sgn.cluster.nhwc.smajor.scalar"),
    # One image of 1024 workgroups whose clusters would spread over 904
    # block ids slice-major, more than the device holds at once: the
    # cluster-major order (64 consecutive ids per cluster), two rounds.
    (1, 512, 256, 256, F16, 32, False, "sgn.cluster.nhwc.vec16"),
    # 36 slices of 1024 pixels (16 per thread) x 16 channel blocks: slice-
    # major spans 576 ids > 512 resident; cluster-major pads K to 40.
    (1, 512, 192, 192, F16, 32, True, "sgn.cluster.nhwc.vec16"),
    # 1344 workgroups, more than two rounds of the 512 resident: split.
    (8, 320, 128, 128, F16, 32, False, "sgn.split.nhwc.vec16"),
    # One slice per (image, channel block), nothing exchanged: 4096
    # workgroups of 2 pixels per thread stay in the cluster beyond two rounds;
    # float16 with 1088 of 9 pixels per thread (the 16-pixel form) takes the
    # split route, float32 with 2048 of 11 stays.
    (512, 320, 8, 8, F16, 32, False, "sgn.cluster.nhwc.vec16"),
    (136, 320, 21, 21, F16, 32, True, "sgn.split.nhwc.vec16"),
    (256, 320, 16, 16, F32, 32, False, "sgn.cluster.nhwc.vec16"),
]


@pytest.mark.parametrize("case", NHWC_LIMIT_CASES, ids=[f"N{c[0]}C{c[1]}H{c[2]}W{c[3]}-"
                                                        f"{np.dtype(c[4]).name}-g{c[5]}"
                                                        f"{'-bc' if c[6] else ''}"
                                                        for c in NHWC_LIMIT_CASES])
def test_nhwc_cluster_limits(case):
    N, C, H, W, T, groups, bc, want_route = case
    w = workloads.sgn("t", N, C, H, W, T, np.float32, channels_last=True, broadcast_skip=bc,
                      bias=True, groups=groups, activation=1, epsilon=1e-5)
    x = workloads.generate(w, seed=C + H + N)
    ref, out, used = run(x, w)
    assert used == want_route
    check(ref, out)


@pytest.mark.parametrize("route", ["auto", "split", "scalar", "block"])
@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3]])
def test_S_request_does_not_change_Y(case, route):
    w, x = make(case, seed=1)
    _, with_s, used = run(x, w, route, want_sum=True)
    _, without, used2 = run(x, w, route, want_sum=False)
    assert without.S is None and used == used2
    assert_bitwise(to_host(with_s.Y), to_host(without.Y), "Y with/without S")


@pytest.mark.parametrize("cl", [0, 1])
def test_broadcast_equals_expanded(cl):
    N, C, H, W = 2, 64, 6, 6
    w, x = make((N, C, H, W, F16, F32, cl, True, True, 8, 1), seed=2)
    _, bc, _ = run(x, w)
    full = np.broadcast_to(x["skip"].reshape((N, 1, 1, C) if cl else (N, C, 1, 1)),
                           x["X"].shape).copy()
    ref, ex, _ = run(x, w, skip_override=full)
    assert_bitwise(to_host(bc.S), to_host(ex.S), "S broadcast vs expanded")
    assert_close(to_host(bc.Y), ref[0], "Y broadcast")
    # The (N, 1, 1, C) spelling is the same broadcast.
    ref2, sp, _ = run(x, w, skip_override=x["skip"].reshape(N, 1, 1, C))
    assert_bitwise(to_host(sp.Y), to_host(bc.Y), "(N,1,1,C) spelling")


# Groups (NCHW) and channel blocks (NHWC) larger than one workgroup holds at
# six accesses per thread, so that every case exchanges moments.
FALLBACK_CASES = [
    (2, 64, 32, 32, F32, F16, 0, True, False, 8, 0),
    (1, 32, 48, 48, F16, F32, 0, False, True, 4, 1),
    (2, 12, 45, 45, F32, F32, 0, True, True, 3, 1),   # odd H*W: phased vectors, 8 slices
    (1, 64, 31, 31, F16, F32, 0, False, True, 2, 1),  # float16 phased, 8 slices
    (1, 1024, 1, 3, F32, F16, 0, False, True, 1, 0),  # H*W = 3: scalar accesses, 8 slices
    (2, 320, 24, 24, F16, F32, 1, False, True, 32, 1),  # NHWC, 11 slices of 51 pixel lanes
    (2, 72, 16, 16, F16, F16, 1, True, False, 8, 0),    # NHWC, 2 groups per wave, 9 slices
    (1, 48, 33, 31, F32, F32, 1, False, True, 4, 1),    # NHWC float32, 32 slices, ragged last
    (2, 15, 24, 24, F16, F32, 1, False, True, 5, 1),    # NHWC odd C: element accesses, 11 slices
    (8, 15, 64, 128, F16, F32, 1, False, True, 5, 1),   # NHWC odd C: packed runs, 32 slices
    (1, 32, 20, 20, F32, F16, 1, True, False, 32, 0),   # NHWC instance norm: element accesses
]


@pytest.mark.parametrize("case", FALLBACK_CASES, ids=lambda c: f"N{c[0]}C{c[1]}H{c[2]}W{c[3]}")
def test_cluster_recompute_path_matches(case):
    """With a zero wait every workgroup recomputes the other slices' moments
    itself; the results must equal those of the published-moments path bit
    for bit (and the oracle's within tolerance)."""
    w, x = make(case, seed=6)
    ref, normal, used = run(x, w)
    assert used.startswith("sgn.cluster")
    with gn.exchange_timeout_us(0):
        _, forced, used2 = run(x, w)
    assert used2 == used
    assert_bitwise(to_host(forced.Y), to_host(normal.Y), "Y recomputed vs published")
    assert_bitwise(to_host(forced.S), to_host(normal.S), "S")
    check(ref, forced)


@pytest.mark.parametrize("cl", [0, 1])
def test_cluster_tags_ignore_stale_workspace(cl):
    """A workspace left over from earlier calls (stale tags and moments from
    a different tensor) must not leak into the next call."""
    N, C, H, W = 2, 64, 32, 32  # groups spread over several workgroups in both layouts
    w, x = make((N, C, H, W, F32, F32, cl, False, True, 8, 1), seed=7)
    w2, x2 = make((N, C, H, W, F32, F32, cl, False, True, 8, 1), seed=8)
    ws = torch.empty(gn.skip_group_norm_workspace_size(to_dev(x["X"]), 8, cl), dtype=torch.uint8,
                     device="cuda")
    kw = dict(groups=8, activation=1, channels_last=cl, want_sum=True, workspace=ws)
    gn.skip_group_norm(to_dev(x2["X"]), to_dev(x2["gamma"]), to_dev(x2["beta"]), to_dev(x2["skip"]),
                       to_dev(x2["bias"]), **kw)
    out = gn.skip_group_norm(to_dev(x["X"]), to_dev(x["gamma"]), to_dev(x["beta"]), to_dev(x["skip"]),
                             to_dev(x["bias"]), **kw)
    assert gn.last_route() == ("sgn.cluster.nhwc.vec16" if cl else "sgn.cluster.nchw.vec16")
    ref_y, ref_s = oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], x["bias"],
                                          groups=8, activation=1, channels_last=cl, want_sum=True)
    assert_close(to_host(out.Y), ref_y, "Y after a call with other data")
    assert_bitwise(to_host(out.S), ref_s, "S")


def test_layouts_agree():
    N, C, H, W = 2, 64, 8, 8
    w, x = make((N, C, H, W, F32, F32, 0, False, True, 8, 0), seed=3)
    _, nchw, _ = run(x, w)
    xh = {k: (np.ascontiguousarray(v.transpose(0, 2, 3, 1)) if v.ndim == 4 else v) for k, v in x.items()}
    wh = workloads.sgn("t", N, C, H, W, F32, F32, channels_last=True, broadcast_skip=False, bias=True,
                       groups=8, activation=0, epsilon=1e-5)
    ref, nhwc, _ = run(xh, wh)
    check(ref, nhwc)
    assert_close(to_host(nhwc.Y), np.ascontiguousarray(to_host(nchw.Y).transpose(0, 2, 3, 1)), "layouts")


@pytest.mark.parametrize("cl", [0, 1])
def test_constant_group_gives_beta(cl):
    N, C, H, W = 1, 32, 8, 8
    shape = (N, H, W, C) if cl else (N, C, H, W)
    X = np.full(shape, 0.75, F32)
    skip = np.full(shape, 0.25, F32)
    gamma = np.linspace(-2, 3, C).astype(F32)
    beta = np.linspace(0.5, -1.5, C).astype(F32)
    out = gn.skip_group_norm(to_dev(X), to_dev(gamma), to_dev(beta), to_dev(skip), groups=4,
                             activation=0, channels_last=cl)
    y = to_host(out.Y)
    expect = np.broadcast_to(beta.reshape((1, 1, 1, C) if cl else (1, C, 1, 1)), shape)
    assert np.array_equal(y, expect)


def test_deterministic_and_in_bounds():
    from group_normalization_amd._lib import lib, check as ck
    N, C, H, W, pad = 2, 320, 16, 16, 2048
    w, x = make((N, C, H, W, F16, F32, 1, False, True, 32, 1), seed=4)
    d = {k: to_dev(v) for k, v in x.items()}
    n = N * C * H * W
    arena = torch.full((2 * (n + 2 * pad),), 5.0, dtype=torch.float16, device="cuda")
    Y = arena[pad: pad + n]
    S = arena[n + 3 * pad: 2 * n + 3 * pad]
    need = gn.skip_group_norm_workspace_size(d["X"], 32, 1)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    results = []
    for _ in range(2):
        ck(lib().skip_group_norm(desc(d["X"]), desc(d["gamma"]), desc(d["beta"]), desc(d["skip"]),
                                 desc(d["bias"]), 1e-5, 32, 1, 1, desc(Y, (N, H, W, C)),
                                 desc(S, (N, H, W, C)), ws.data_ptr(), need,
                                 torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        results.append((to_host(Y).copy(), to_host(S).copy()))
    assert_bitwise(results[0][0], results[1][0], "Y second run")
    a = to_host(arena)
    assert np.all(a[:pad] == 5.0) and np.all(a[pad + n: n + 3 * pad] == 5.0)
    assert np.all(a[2 * n + 3 * pad:] == 5.0)
    assert torch.all(ws[need:] == 0x5A)
    ref_y, ref_s = oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], x["bias"],
                                          groups=32, activation=1, epsilon=1e-5, channels_last=1,
                                          want_sum=True)
    assert_close(results[0][0].reshape(ref_y.shape), ref_y, "Y")
    assert_bitwise(results[0][1].reshape(ref_s.shape), ref_s, "S")


def test_empty():
    X = torch.empty(0, 4, 4, 8, dtype=torch.float16, device="cuda")
    g = torch.ones(8, dtype=torch.float32, device="cuda")
    out = gn.skip_group_norm(X, g, g, X, groups=2, activation=0)
    assert out.Y.shape == X.shape


@pytest.mark.parametrize("route", ["auto", "split", "scalar", "block"])
@pytest.mark.parametrize("cl", [0, 1])
def test_non_finite_values_stay_in_their_group(cl, route):
    """A residual sum that overflows binary16 (S = +inf) or a NaN input makes
    its own group's Y NaN, as in the oracle, and leaves every other group
    untouched; S keeps the infinity bit for bit."""
    N, C, H, W, groups = 2, 64, 6, 6, 8
    w, x = make((N, C, H, W, F16, F32, cl, False, True, groups, 1), seed=11)
    X, skip = x["X"].copy(), x["skip"].copy()
    def put(a, n, c, h, wv, v):
        if cl:
            a[n, h, wv, c] = v
        else:
            a[n, c, h, wv] = v
    put(X, 0, 17, 2, 3, 65504.0)    # group 2 of image 0: 65504 + 65504 rounds to +inf
    put(skip, 0, 17, 2, 3, 65504.0)
    put(X, 1, 45, 5, 0, np.nan)     # group 5 of image 1
    x = dict(x, X=X, skip=skip)
    ref, out, used = run(x, w, route)
    check(ref, out, want_sum=False)
    # S: the same NaN positions (NaN payloads are not compared), the rest bit for bit.
    s_got, s_ref = to_host(out.S), ref[1]
    assert np.array_equal(np.isnan(s_got), np.isnan(s_ref))
    fin = ~np.isnan(s_ref)
    assert_bitwise(s_got[fin], s_ref[fin], "S")
    assert np.isinf(s_ref).sum() == 1
    y = to_host(out.Y).astype(np.float32)
    y = y if not cl else y.transpose(0, 3, 1, 2)
    nan_groups = {(n, g) for n in range(N) for g in range(groups)
                  if np.isnan(y[n, g * 8:(g + 1) * 8]).all()}
    assert nan_groups == {(0, 2), (1, 5)}, nan_groups


LONE_INF_SHAPES = [
    # (N, C, H, W, groups): one 16-byte float16 vector per NCHW group (one
    # thread holds the whole group), small groups, and the NHWC channel layout.
    (2, 8, 2, 4, 8),
    (2, 16, 4, 4, 4),
    (2, 64, 6, 6, 8),
    (1, 15, 8, 8, 5),
    (8, 15, 64, 128, 5),  # NHWC: the cluster over packed runs of pixels (vectors holding several groups)
]


@pytest.mark.parametrize("route", ["auto", "split", "scalar", "block"])
@pytest.mark.parametrize("cl", [0, 1])
@pytest.mark.parametrize("dt", [F16, F32])
@pytest.mark.parametrize("shape", LONE_INF_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_lone_infinity_makes_its_group_nan(shape, dt, cl, route):
    """A single residual sum that overflows to +inf, without SiLU (which would
    turn -inf into NaN and hide the difference): the group's mean is +inf and
    its variance NaN, so IEEE arithmetic on the definition makes every output
    of the group NaN, as in the oracle, wherever the infinity sits in the
    group (its first, a middle or its last element) and whichever thread's
    sums hold it; the other groups match the oracle as usual."""
    N, C, H, W, groups = shape
    big = 65504.0 if dt == F16 else 3e38
    cpg, hw = C // groups, H * W
    for pos in (0, (cpg * hw) // 2, cpg * hw - 1):  # element of group 1 of image N - 1, in NCHW order
        w, x = make((N, C, H, W, dt, F32, cl, False, True, groups, 0), seed=17 + pos)
        X, skip = x["X"].copy(), x["skip"].copy()
        c, p = cpg * 1 + pos // hw, pos % hw
        h, wv = divmod(p, W)
        idx = (N - 1, h, wv, c) if cl else (N - 1, c, h, wv)
        X[idx] = big
        skip[idx] = big
        x = dict(x, X=X, skip=skip)
        ref, out, used = run(x, w, route)
        assert np.isinf(ref[1]).sum() == 1
        check(ref, out)
        y = to_host(out.Y)
        y = (y.transpose(0, 3, 1, 2) if cl else y).reshape(N, groups, cpg * hw)
        nan_groups = {(n, g) for n in range(N) for g in range(groups) if np.isnan(y[n, g]).all()}
        assert nan_groups == {(N - 1, 1)}, (pos, used, nan_groups)


@pytest.mark.parametrize("dt,N,C,H,W,groups,offset,bc", [
    (F16, 2, 64, 8, 8, 8, 1, False),     # whole vectors per plane, bases off the grid
    (F16, 2, 40, 7, 7, 4, 0, True),      # 7 x 7 planes
    (F16, 1, 64, 31, 31, 2, 5, False),   # several slices
    (F32, 2, 48, 5, 5, 6, 3, True),
    (F32, 1, 32, 33, 31, 4, 2, False),
])
def test_nchw_phased_groups(dt, N, C, H, W, groups, offset, bc):
    """NCHW groups off the 16-byte grid, through the C ABI: X, skip, Y and S
    all `offset` elements past a 16-byte boundary (or planes that are not a
    whole number of 16-byte vectors) take the phased cluster route, which
    reads aligned vectors across group boundaries.  Results match the oracle
    and nothing outside Y and S is written."""
    from group_normalization_amd._lib import lib, check as ck
    w = workloads.sgn("t", N, C, H, W, dt, F32, channels_last=False, broadcast_skip=bc, bias=True,
                      groups=groups, activation=1, epsilon=1e-5)
    x = workloads.generate(w, seed=C + H + offset)
    tdt = torch.float16 if dt == F16 else torch.float32
    n, pad = N * C * H * W, 64

    def arena():
        return torch.full((n + 2 * pad,), -7.0, dtype=tdt, device="cuda")

    bufs = {k: arena() for k in ("X", "skip", "Y", "S")}
    views = {k: b[pad + offset: pad + offset + n] for k, b in bufs.items()}
    views["X"].copy_(to_dev(x["X"]).ravel())
    skip = to_dev(x["skip"]) if bc else views["skip"]
    if not bc:
        views["skip"].copy_(to_dev(x["skip"]).ravel())
    d = {k: to_dev(x[k]) for k in ("gamma", "beta", "bias")}
    ws = torch.empty(gn.skip_group_norm_workspace_size(views["X"].view(N, C, H, W), groups, 0),
                     dtype=torch.uint8, device="cuda")
    for _ in range(2):
        xs = (N, C, H, W)
        ck(lib().skip_group_norm(desc(views["X"], xs), desc(d["gamma"]), desc(d["beta"]),
                                 desc(skip) if bc else desc(skip, xs), desc(d["bias"]), 1e-5, groups, 0, 1,
                                 desc(views["Y"], xs), desc(views["S"], xs), ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream().cuda_stream))
        assert gn.last_route() == "sgn.cluster.nchw.phase"
        torch.cuda.synchronize()
        ref_y, ref_s = oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], x["bias"],
                                              groups=groups, activation=1, epsilon=1e-5, channels_last=0,
                                              want_sum=True)
        assert_close(to_host(views["Y"]).reshape(ref_y.shape), ref_y, "Y")
        assert_bitwise(to_host(views["S"]).reshape(ref_s.shape), ref_s, "S")
        for k in ("Y", "S"):
            b = to_host(bufs[k])
            assert np.all(b[:pad + offset] == -7.0) and np.all(b[pad + offset + n:] == -7.0), k
