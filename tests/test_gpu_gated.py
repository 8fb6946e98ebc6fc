"""GatedRMSNorm: HIP path (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
from group_normalization_amd import workloads
from parity import assert_bitwise, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

F32, F16 = np.float32, np.float16

CASES = [
    # (X shape, span C, dtype): spans around 16-byte vectors, segment widths and rows per wave
    ((3, 4), 1, F32),           # the page's example shape, C = 1
    ((5, 12), 2, F16),
    ((7, 21), 3, F32),
    ((9, 8), 8, F16),            # one vector per row
    ((11, 48), 16, F16),
    ((13, 64), 64, F32),
    ((3, 7, 100), 100, F16),     # not a whole number of vectors
    ((4, 33, 128), 128, F16),    # C = 128: 16 lanes x 8 halves; ragged last block
    ((2, 4096), 128, F32),
    ((6, 1024), 1024, F16),      # 128 vectors: 64 lanes x 2
    ((3, 8192), 8192, F16),      # 1024 vectors: 64 lanes x 16
    ((2, 5000), 5000, F32),      # 1250 sixteen-byte vectors: one 512-thread workgroup per row in registers
    ((2, 2, 9000), 9000, F16),   # 1125 vectors: 8 waves, ragged
    ((1000,), 10, F16),          # rank 1
    ((4, 396), 132, F16),        # 8-byte vectors: 33 per row
    ((3, 650), 130, F16),        # 4-byte vectors: 65 per row, two per lane
    ((5, 129), 129, F16),        # odd span: scalars
    ((4, 6), 6, F32),            # float32 8-byte vectors: 3 per row
    ((2, 8200), 4100, F16),      # 1025 eight-byte vectors: row route
    ((3, 24576), 24576, F16),    # 3072 vectors: 16 waves, ragged
    ((2, 32768), 32768, F16),    # 4096 vectors: 16 waves of 4 per thread
    ((3, 32776), 32776, F16),    # 4097 vectors: two-pass block route, vectorized
    ((2, 12000), 12000, F16),    # 1500 vectors: 8 waves, ragged
    ((2, 16386), 16386, F32),    # 8193 eight-byte vectors: block route
    ((2, 16382), 16382, F32),    # 8191 eight-byte vectors: 16 waves of 8 per thread
    ((3, 4099), 4099, F16),      # 4099 scalars: 16 waves of 8 per thread
    ((2, 8195), 8195, F16),      # 8195 scalars: scalar block route
    ((3, 4095), 4095, F16),      # 4095 scalars: 16 waves of 4 per thread
    ((4, 2049), 2049, F32),      # 2049 scalars: 16 waves, ragged
    ((2, 5003), 5003, F32),      # 5003 scalars: 16 waves of 8 per thread
    # tile route (float16 rows of 33-128 vectors of 8 or 4 bytes that fill
    # < 60 % of the segment route's lanes, packed back to back): several
    # tiles, a ragged last tile and waves past the last row
    ((1000, 132), 132, F16),     # 33 eight-byte vectors: 15 rows per wave of 8 per lane
    ((257, 3, 130), 130, F16),   # 65 four-byte vectors: 15 rows per wave of 16 per lane
    ((211, 130), 130, F32),      # 65 eight-byte float32 vectors: segment (float32 never tiles)
    ((77, 2, 148), 148, F16),    # 37 eight-byte vectors: 13 rows per wave
    ((93, 150), 150, F16),       # 75 four-byte vectors: 13 rows per wave of 16 per lane
    ((1, 132), 132, F16),        # one row: one tile, one row in it
    ((3, 2, 130), 130, F16),     # six rows: fewer than one tile
    ((1, 16384), 16384, F16),    # one row through the row route
    ((1, 40000), 40000, F32),    # one row through the two-pass route
    # around the tile route's bounds: segment
    ((99, 264), 264, F16),       # 33 sixteen-byte vectors
    ((41, 124), 124, F16),       # 31 eight-byte vectors
    ((43, 156), 156, F16),       # 39 eight-byte vectors: 61 % of the lanes busy
    ((37, 516), 516, F16),       # 129 eight-byte vectors
    ((301, 254), 254, F16),      # 127 four-byte vectors: 2 x 64 lanes nearly full
    ((53, 129), 129, F32),       # scalars
]


def tile_plan(nvec, vec_bytes):
    """The host's choice between the two lane layouts, restated: (vectors per
    lane, rows per wave) of the tile route, or None for the segment route."""
    if vec_bytes not in (8, 4) or nvec <= 32 or nvec > 128 or nvec & (nvec - 1) == 0:
        return None
    lanes = 1
    while lanes < nvec and lanes < 64:
        lanes *= 2
    vpl = 1
    while lanes * vpl < nvec:
        vpl *= 2
    if nvec / (lanes * vpl) >= 0.6:
        return None
    best, plan = 0.0, None
    for vpt in (4, 8, 16):
        if vpt > 4 and vpt * vec_bytes > 64:
            continue
        rt = 64 * vpt // nvec
        if 1 <= rt <= 64 and rt * nvec / (64 * vpt) > best + 1e-9:
            best, plan = rt * nvec / (64 * vpt), (vpt, rt)
    return plan if best > nvec / (lanes * vpl) else None


def expected_route(C, dt, route="auto"):
    size = np.dtype(dt).itemsize
    width = next((b for b in (16, 8, 4) if b > size and C * size % b == 0), size)
    if route == "scalar":
        width = size
    E = width // size
    name = {16: "vec16", 8: "vec8", 4: "vec4"}.get(width) if E > 1 else "scalar"
    if route == "block":
        return "gated.block"
    if C // E > (4096 if width == 16 else 8192):  # the row route's widest rows
        return "gated.block" if E == 1 else f"gated.block.{name}"
    if C // E > 1024:
        return f"gated.row.{name}"
    if route == "auto" and size == 2 and E > 1 and tile_plan(C // E, width):
        return f"gated.tile.{name}"
    return f"gated.segment.{name}"


@pytest.mark.parametrize("route", ["auto", "scalar", "vector", "block"])
@pytest.mark.parametrize("shape,C,dt", CASES, ids=[f"{s}-C{c}-{np.dtype(d).name}" for s, c, d in CASES])
def test_matches_oracle(shape, C, dt, route):
    w = workloads.gated("t", shape, C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C + len(shape))
    ref = oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5)
    with gn.force_route(route):
        y = gn.gated_rms_norm(to_dev(x["X"]), to_dev(x["scale"]), to_dev(x["gate"]), 1e-5)
        used = gn.last_route()
    assert_close(to_host(y), ref, f"Y via {used}")
    assert used == expected_route(C, dt, route)


def test_tile_plan_examples():
    """Spot values of the restated plan (vectors per lane, rows per wave)."""
    assert tile_plan(33, 8) == (8, 15)
    assert tile_plan(65, 4) == (16, 15)
    assert tile_plan(37, 8) == (8, 13) and tile_plan(38, 8) == (8, 13)
    assert tile_plan(39, 8) is None and tile_plan(50, 8) is None
    assert tile_plan(127, 4) is None and tile_plan(33, 16) is None and tile_plan(31, 8) is None and tile_plan(129, 8) is None
    assert tile_plan(64, 8) is None and tile_plan(65, 2) is None


@pytest.mark.parametrize("C,dt", [(132, F16), (130, F16), (148, F16), (150, F16), (68 * 2 + 2, F16)])
def test_tile_route_stays_in_bounds(C, dt):
    """Tile route through raw pointers: guard elements on both sides of Y are
    untouched, two runs agree bit for bit, and the rows match the oracle."""
    from group_normalization_amd._lib import lib, check as ck
    rows, pad = 211, 4096
    w = workloads.gated("t", (rows, C), C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C)
    d = {k: to_dev(v) for k, v in x.items()}
    tdt = torch.float16 if dt == F16 else torch.float32
    arena = torch.full((rows * C + 2 * pad,), 3.0, dtype=tdt, device="cuda")
    Y = arena[pad: pad + rows * C]
    code = 1 if dt == F16 else 0
    for i in range(2):
        ck(lib().gated_rms_norm(code, rows * C, C, d["X"].data_ptr(), d["scale"].data_ptr(),
                                d["gate"].data_ptr(), 1e-5, Y.data_ptr(),
                                torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert gn.last_route().startswith("gated.tile")
        if i == 0:
            first = to_host(Y).copy()
    assert_bitwise(to_host(Y), first, "second run")
    a = to_host(arena)
    assert np.all(a[:pad] == 3.0) and np.all(a[pad + rows * C:] == 3.0)
    assert_close(first.reshape(rows, C), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


@pytest.mark.parametrize("dt", [F32, F16])
def test_zero_gate_gives_zero(dt):
    w = workloads.gated("t", (64, 256), 128, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=1)
    y = gn.gated_rms_norm(to_dev(x["X"]), to_dev(x["scale"]), torch.zeros(64, 256, dtype=to_dev(x["X"]).dtype,
                                                                           device="cuda"))
    assert torch.all(y == 0)


def test_scale_spellings_and_packing_agree():
    w = workloads.gated("t", (8, 4 * 128), 128, F16, epsilon=1e-5)
    x = workloads.generate(w, seed=2)
    X, g, s = to_dev(x["X"]), to_dev(x["gate"]), to_dev(x["scale"])
    base = to_host(gn.gated_rms_norm(X, s, g))
    for Xs, gs, ss in [(X.view(32, 128), g.view(32, 128), s.view(1, 128)),
                       (X.view(8, 4, 128), g.view(8, 4, 128), s.view(128, 1)),
                       (X.view(-1), g.view(-1), s)]:
        assert_bitwise(to_host(gn.gated_rms_norm(Xs, ss, gs)).reshape(base.shape), base, "repacked")


def test_deterministic_and_in_bounds():
    from group_normalization_amd._lib import lib, check as ck
    rows, C, pad = 1000, 128, 1024
    w = workloads.gated("t", (rows, C), C, F16, epsilon=1e-5)
    x = workloads.generate(w, seed=6)
    d = {k: to_dev(v) for k, v in x.items()}
    arena = torch.full((rows * C + 2 * pad,), 3.0, dtype=torch.float16, device="cuda")
    Y = arena[pad: pad + rows * C]
    for _ in range(2):
        ck(lib().gated_rms_norm(1, rows * C, C, d["X"].data_ptr(), d["scale"].data_ptr(),
                                d["gate"].data_ptr(), 1e-5, Y.data_ptr(),
                                torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        if _ == 0:
            first = to_host(Y).copy()
    assert_bitwise(to_host(Y), first, "second run")
    a = to_host(arena)
    assert np.all(a[:pad] == 3.0) and np.all(a[pad + rows * C:] == 3.0)
    assert_close(first.reshape(rows, C), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


def test_empty():
    e = torch.empty(0, 128, dtype=torch.float16, device="cuda")
    s = torch.ones(128, dtype=torch.float16, device="cuda")
    assert gn.gated_rms_norm(e, s, e).shape == (0, 128)
