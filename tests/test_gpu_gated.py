"""GatedRMSNorm: HIP path (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
import workloads
from parity import assert_bitwise, assert_close, desc, to_dev, to_host

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
    ((2, 8200), 4100, F16),      # 1025 eight-byte vectors: phased route
    ((3, 1012), 1012, F16),      # 253 eight-byte vectors: segment route
    ((3, 1028), 1028, F16),      # 257 eight-byte vectors: phased route
    ((3, 602), 602, F16),        # 301 four-byte vectors: phased route
    ((3, 514), 514, F16),        # 257 four-byte vectors: segment route
    ((3, 2050), 2050, F32),      # float32 8-byte vectors: phased route
    ((3, 24576), 24576, F16),    # 3072 vectors: 16 waves, ragged
    ((2, 32768), 32768, F16),    # 4096 vectors: 16 waves of 4 per thread
    ((3, 32776), 32776, F16),    # 4097 vectors: wide route, X in VGPRs, gate read after the sum
    ((2, 65536), 65536, F16),    # 8192 vectors: wide route, VGPRs only
    ((2, 100000), 100000, F16),  # 12500 vectors: wide route, ragged 5-vector LDS tail
    ((3, 139264), 139264, F16),  # 17408 vectors: wide route at its widest (9 in LDS)
    ((2, 139272), 139272, F16),  # one vector more: block route, vectorized
    ((2, 40000), 40000, F32),    # float32 wide route, 2 LDS vectors per lane
    ((2, 69632), 69632, F32),    # float32 wide route at its widest
    ((2, 12000), 12000, F16),    # 1500 vectors: 8 waves, ragged
    ((2, 16386), 16386, F32),    # 8193 eight-byte vectors: block route
    ((2, 16382), 16382, F32),    # 8191 eight-byte vectors: 16 waves of 8 per thread
    ((3, 4099), 4099, F16),      # odd span: phased route, four waves
    ((2, 8195), 8195, F16),      # odd span: phased route, eight waves
    ((2, 32759), 32759, F16),    # the phased route's longest span (4096 vectors touched)
    ((2, 32761), 32761, F16),    # one vector more: scalar block route
    ((2, 32777), 32777, F16),    # longer odd span: scalar block route
    ((3, 4095), 4095, F16),      # odd span: phased route
    ((5, 1017), 1017, F16),      # just past the flat route: phased, one wave
    ((4, 2049), 2049, F32),      # float32 odd span: phased route
    ((2, 5003), 5003, F32),      # float32 odd span: phased route
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
    # flat route (rows as one stream of 16-byte vectors): chosen automatically
    ((5000, 3), 3, F16),         # rows narrower than a vector: 339 rows per wave
    ((4000, 25), 25, F16),       # 40 rows per wave, lanes take rows in turns
    ((700, 301), 301, F32),      # 3 rows per wave, 16 lanes per row
    ((123, 602), 602, F32),      # the 2048-slot tile: 3 rows per wave
    ((77, 9), 9, F32),           # odd float32 rows from 9 elements on
    ((6, 1, 150), 150, F32),     # 8-byte float32 vectors filling 59 % of the segment lanes
    # segment rows of more than 64 vectors off the 128-byte grid: the lines
    # shared between rows are stored through L2
    ((50, 1000), 1000, F16),     # 125 sixteen-byte vectors, rows of 2000 bytes
    ((41, 264), 264, F32),       # 66 sixteen-byte vectors, rows of 1056 bytes
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


def flat_plan(C, vec_elems, large):
    """The flat route's tile, restated: (vectors per lane, rows per wave,
    share of the element slots filled), or None."""
    if not 1 <= C <= 1024 - vec_elems:  # the scale table's 1024 slots, E of them ahead
        return None
    small, best = 16 // vec_elems, None
    for vpt in (small, 2 * small):
        if vpt != small and not large:
            break
        te = 64 * vpt * vec_elems
        rt = (te - vec_elems + 1) // C
        if rt < 1:
            continue
        fill = rt * C / te
        if best is not None and (best[2] >= 0.75 or fill <= best[2]):
            continue
        best = (vpt, rt, fill)
    return best


def flat_preferred(C, size, E):
    """Whether the automatic choice takes the flat route (rows read with
    E-element accesses narrower than 16 bytes), restated."""
    plan = flat_plan(C, 16 // size, size == 4)
    if plan is None or plan[2] < 0.75:
        return False
    nvec = C // E
    if E == 1:
        return C >= (2 if size == 2 else 8)
    if E * size == 4:
        return nvec >= 2
    lanes = 1
    while lanes < nvec and lanes < 64:
        lanes *= 2
    vpl = 1
    while lanes * vpl < nvec:
        vpl *= 2
    return nvec / (lanes * vpl) < (0.75 if size == 2 else 0.6)


def expected_route(C, dt, route="auto"):
    """Route for tensors from to_dev (every base 16-byte aligned)."""
    size = np.dtype(dt).itemsize
    width = next((b for b in (16, 8, 4) if b > size and C * size % b == 0), size)
    if route == "scalar":
        width = size
    E = width // size
    name = {16: "vec16", 8: "vec8", 4: "vec4"}.get(width) if E > 1 else "scalar"
    if route == "block":
        return "gated.block"
    if route == "flat" and C <= 1024 - 16 // size:
        return "gated.flat.vec16"
    if route == "auto" and width < 16 and flat_preferred(C, size, E):
        return "gated.flat.vec16"
    # Aligned 16-byte vectors across span boundaries while a span touches 33
    # to 4096 of them: spans read element by element otherwise, and spans of
    # more than 300 four-byte or 256 eight-byte vectors.
    if route != "scalar" and 32 < C // (16 // size) + 2 <= 4096:
        if E == 1 or (width == 4 and C // E > 300) or (width == 8 and C // E > 256):
            return "gated.phase.vec16"
    if C // E > (4096 if width == 16 else 8192):  # the row route's widest rows
        if width == 16 and C // E <= 1024 * 17:  # X in 8 VGPR and up to 9 LDS vectors per lane
            return "gated.wide.vec16"
        return "gated.block" if E == 1 else f"gated.block.{name}"
    if C // E > 1024:
        return f"gated.row.{name}"
    if route in ("auto", "flat") and size == 2 and E > 1 and tile_plan(C // E, width):
        return f"gated.tile.{name}"
    return f"gated.segment.{name}"


@pytest.mark.parametrize("route", ["auto", "scalar", "vector", "block", "flat"])
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
    """Tile route through raw pointers (gate off X's 16-byte grid, so the flat
    route does not apply): guard elements on both sides of Y are
    untouched, two runs agree bit for bit, and the rows match the oracle."""
    from group_normalization_amd._lib import lib, check as ck
    rows, pad = 211, 4096
    w = workloads.gated("t", (rows, C), C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C)
    d = {k: to_dev(v) for k, v in x.items()}
    tdt = torch.float16 if dt == F16 else torch.float32
    gbuf = torch.empty(rows * C + 4, dtype=tdt, device="cuda")
    d["gate"] = gbuf[4:].view(rows, C)  # 8 bytes off the grid X lies on: no flat route
    d["gate"].copy_(torch.from_numpy(x["gate"]))
    arena = torch.full((rows * C + 2 * pad,), 3.0, dtype=tdt, device="cuda")
    Y = arena[pad: pad + rows * C]
    for i in range(2):
        ck(lib().gated_rms_norm(desc(d["X"]), desc(d["scale"]), desc(d["gate"]), 1e-5,
                                desc(Y, (rows, C)), torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert gn.last_route().startswith("gated.tile")
        if i == 0:
            first = to_host(Y).copy()
    assert_bitwise(to_host(Y), first, "second run")
    a = to_host(arena)
    assert np.all(a[:pad] == 3.0) and np.all(a[pad + rows * C:] == 3.0)
    assert_close(first.reshape(rows, C), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


FLAT_CASES = [(c, F16) for c in (1, 2, 3, 5, 7, 10, 20, 25, 50, 100, 129, 130, 301, 602, 1002, 1015, 1016)] + \
    [(c, F32) for c in (1, 3, 5, 10, 25, 129, 130, 301, 683, 1019, 1020)]


@pytest.mark.parametrize("off", [0, 1, 3])
@pytest.mark.parametrize("C,dt", FLAT_CASES, ids=[f"C{c}-{np.dtype(d).name}" for c, d in FLAT_CASES])
def test_flat_route(C, dt, off):
    """Flat route (forced): X, gate and Y start `off` elements past a 16-byte
    boundary, so tiles begin and end inside vectors; guard elements on both
    sides of Y stay untouched, two runs agree bit for bit, and the rows
    (several tiles, a ragged last one, waves past the last row) match the
    oracle."""
    from group_normalization_amd._lib import lib, check as ck
    rows, pad = 4000 // C + 7, 64
    w = workloads.gated("t", (rows, C), C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C + off)
    tdt = torch.float16 if dt == F16 else torch.float32

    def placed(a, fill=None):
        buf = torch.full((a.size + 2 * pad,), 3.0, dtype=tdt, device="cuda")
        view = buf[pad + off: pad + off + a.size]  # buf is 256-byte aligned
        if fill is None:
            view.copy_(torch.from_numpy(np.ascontiguousarray(a).ravel()))
        return buf, view

    _, X = placed(x["X"])
    _, G = placed(x["gate"])
    arena, Y = placed(x["X"], fill=3.0)
    S = to_dev(x["scale"])
    for i in range(2):
        with gn.force_route("flat"):
            ck(lib().gated_rms_norm(desc(X), desc(S), desc(G), 1e-5, desc(Y),
                                    torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert gn.last_route() == "gated.flat.vec16"
        if i == 0:
            first = to_host(Y).copy()
    assert_bitwise(to_host(Y), first, "second run")
    a = to_host(arena)
    assert np.all(a[:pad + off] == 3.0) and np.all(a[pad + off + rows * C:] == 3.0)
    assert_close(first.reshape(rows, C), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


PHASE_CASES = [(1017, F16, 1), (2049, F16, 3), (4097, F16, 5), (8195, F16, 7), (32759, F16, 2),
               (1021, F32, 1), (2049, F32, 3), (16379, F32, 2)]


@pytest.mark.parametrize("C,dt,off", PHASE_CASES, ids=[f"C{c}-{np.dtype(d).name}-off{o}" for c, d, o in PHASE_CASES])
def test_phased_spans(C, dt, off):
    """Phased route: X, gate and Y start `off` elements past a 16-byte
    boundary, spans of odd length, so every span starts and ends inside a
    vector whose other elements belong to its neighbours (or lie outside the
    tensors, at the ends).  Guard elements on both sides of Y stay
    untouched, two runs agree bit for bit, and the spans match the
    oracle."""
    from group_normalization_amd._lib import lib, check as ck
    rows, pad = max(3, 60000 // C), 64
    w = workloads.gated("t", (rows, C), C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C + off)
    tdt = torch.float16 if dt == F16 else torch.float32

    def placed(a, fill=None):
        buf = torch.full((a.size + 2 * pad,), 3.0, dtype=tdt, device="cuda")
        view = buf[pad + off: pad + off + a.size]  # buf is 256-byte aligned
        if fill is None:
            view.copy_(torch.from_numpy(np.ascontiguousarray(a).ravel()))
        return buf, view

    _, X = placed(x["X"])
    _, G = placed(x["gate"])
    arena, Y = placed(x["X"], fill=3.0)
    S = to_dev(x["scale"])
    for i in range(2):
        ck(lib().gated_rms_norm(desc(X, (rows, C)), desc(S), desc(G, (rows, C)), 1e-5, desc(Y, (rows, C)),
                                torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert gn.last_route() == "gated.phase.vec16"
        if i == 0:
            first = to_host(Y).copy()
    assert_bitwise(to_host(Y), first, "second run")
    a = to_host(arena)
    assert np.all(a[:pad + off] == 3.0) and np.all(a[pad + off + rows * C:] == 3.0)
    assert_close(first.reshape(rows, C), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


@pytest.mark.parametrize("C,dt", [(1017, F16), (1021, F32)])
def test_flat_longest_rows(C, dt):
    """One element past the flat route's longest rows: forced flat, the
    route falls back to the phased route with the same values."""
    w = workloads.gated("t", (40, C), C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C)
    with gn.force_route("flat"):
        y = gn.gated_rms_norm(to_dev(x["X"]), to_dev(x["scale"]), to_dev(x["gate"]), 1e-5)
    assert gn.last_route() == "gated.phase.vec16"
    assert_close(to_host(y), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


def test_flat_needs_a_shared_offset():
    """X and gate at different offsets from the 16-byte grid: not the flat
    route, even forced, and the same values."""
    w = workloads.gated("t", (300, 10), 10, F16, epsilon=1e-5)
    x = workloads.generate(w, seed=5)
    buf = torch.empty(3000 + 8, dtype=torch.float16, device="cuda")
    X = buf[1:3001].view(300, 10)
    X.copy_(torch.from_numpy(x["X"]))
    for route in ("auto", "flat"):
        with gn.force_route(route):
            y = gn.gated_rms_norm(X, to_dev(x["scale"]), to_dev(x["gate"]), 1e-5)
        assert gn.last_route() == "gated.segment.scalar"
        assert_close(to_host(y), oracle.gated_rms_norm(x["X"], x["scale"], x["gate"], 1e-5), "Y")


NON_FINITE_CASES = [
    # (X shape, span C, dtype): one shape for each route family
    ((9, 8), 8, F16),            # one vector per span
    ((13, 64), 64, F32),         # segment route
    ((4, 33, 128), 128, F16),    # C = 128, ragged last block
    ((1000, 25), 25, F16),       # flat route
    ((1000, 132), 132, F16),     # tile route
    ((6, 1017), 1017, F16),      # phased route
    ((6, 2048), 2048, F32),      # row route
    ((6, 100000), 100000, F16),  # wide route
    ((6, 139272), 139272, F16),  # block route
]


@pytest.mark.parametrize("route", ["auto", "block"])
@pytest.mark.parametrize("shape,C,dt", NON_FINITE_CASES, ids=[f"{s}-C{c}-{np.dtype(d).name}"
                                                                for s, c, d in NON_FINITE_CASES])
def test_non_finite_spans(shape, C, dt, route):
    """+inf, NaN and -inf in X (the span's mean square is +inf or NaN: its
    finite elements give signed zeros, the others NaN) and +inf, -inf and NaN
    gates (SiLU: +inf, -inf * 0 = NaN, NaN), each in its own span; every
    output equals the oracle's, NaN positions and infinities included, and
    the untouched spans are finite."""
    w = workloads.gated("t", shape, C, dt, epsilon=1e-5)
    x = workloads.generate(w, seed=C + 5)
    X, gate = x["X"].copy(), x["gate"].copy()
    xs, gs = X.reshape(-1, C), gate.reshape(-1, C)
    e = C // 2
    xs[0, e] = np.inf
    xs[1, 0] = np.nan
    xs[2, C - 1] = -np.inf
    gs[3, e] = np.inf
    gs[4, 0] = -np.inf
    gs[5, C - 1] = np.nan
    ref = oracle.gated_rms_norm(X, x["scale"], gate, 1e-5)
    with gn.force_route(route):
        y = gn.gated_rms_norm(to_dev(X), to_dev(x["scale"]), to_dev(gate), 1e-5)
        used = gn.last_route()
    yh = to_host(y)
    assert_close(yh, ref, f"Y via {used}")
    ys = yh.reshape(-1, C)
    assert np.isnan(ys[1]).all() and np.isnan(ys[0, e]) and np.isnan(ys[2, C - 1]), used
    assert np.isnan(ys[4, 0]) and np.isnan(ys[5, C - 1]), used
    assert np.isfinite(ys[6:]).all(), used


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
        ck(lib().gated_rms_norm(desc(d["X"]), desc(d["scale"]), desc(d["gate"]), 1e-5,
                                desc(Y, (rows, C)), torch.cuda.current_stream().cuda_stream))
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
