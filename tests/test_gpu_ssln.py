"""SkipSimplifiedLayerNormalization: HIP path (through the C ABI) against the
oracle, element by element.  Every route, both dtypes, every optional
input/output combination, ragged and unaligned shapes, edge values."""
import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
import workloads
from parity import assert_bitwise, assert_close, desc, to_dev, to_host

pytestmark = pytest.mark.gpu

F32, F16 = np.float32, np.float16


def run_both(inp, skip, gamma, bias, eps, route="auto", want=("mean", "inv", "sum")):
    ref = oracle.skip_rms_norm(inp, skip, gamma, bias, eps, want_mean=True,
                               want_inv_std_var=True, want_sum=True)
    with gn.force_route(route):
        out = gn.skip_rms_norm(to_dev(inp), to_dev(skip), to_dev(gamma), to_dev(bias), eps,
                               want_mean="mean" in want, want_inv_std_var="inv" in want,
                               want_sum="sum" in want)
        used = gn.last_route()
    torch.cuda.synchronize()
    return ref, out, used


def check(ref, out, want=("mean", "inv", "sum")):
    y_ref, mean_ref, inv_ref, s_ref = ref
    assert_close(to_host(out.output), y_ref, "output")
    if "sum" in want:
        assert_bitwise(to_host(out.input_skip_bias_sum), s_ref, "input_skip_bias_sum")
    if "inv" in want:
        assert_close(to_host(out.inv_std_var), inv_ref, "inv_std_var")
    if "mean" in want:
        assert np.all(to_host(out.mean) == 0)


SHAPES = [
    # (shape, dtype, bias): ragged row counts, widths around vector and wave sizes
    ((64, 768), F32, True),
    ((13, 768), F16, False),
    ((3, 5, 4096), F16, True),
    ((7, 8192), F16, False),
    ((5, 8192), F32, True),      # float32, eight waves per row
    ((9, 1000), F16, True),      # 125 vectors: ragged second pass over the wave
    ((6, 33), F32, False),       # not a whole number of vectors
    ((4, 1), F16, True),
    ((2, 3, 10000), F16, False), # eight waves per row, ragged
    ((257, 256), F32, False),
    ((3, 12288), F16, True),     # eight waves per row, 3 vectors per lane
    ((2, 32768), F16, False),    # sixteen waves per row, 4 vectors per lane (widest)
    ((3, 20480), F16, True),     # sixteen waves per row, ragged
    ((2, 16384), F32, True),     # float32 sixteen waves per row
    ((2, 10000), F32, False),    # float32 sixteen waves per row, ragged
    ((2, 40000), F16, True),     # sixteen waves, 5 vectors per lane
    ((2, 65544), F16, True),     # one vector past the register routes: wide route, one LDS vector
    ((2, 40000), F32, False),    # float32 wide route, 2 LDS vectors per lane
    ((2, 30000), F32, True),     # float32 sixteen waves, 8 vectors per lane, ragged
    ((2, 20004), F16, False),    # 8-byte rows of 5001 vectors: phased route
    ((3, 65536), F16, False),    # sixteen waves, 8 vectors per lane (widest register row)
    ((2, 131072), F16, False),   # wide route, 8 LDS vectors per lane
    ((3, 139264), F16, True),    # wide route at its widest: 17 vectors per lane, odd LDS tail
    ((2, 100000), F16, True),    # wide route, ragged 5-vector LDS tail
    ((2, 69632), F32, True),     # float32 wide route at its widest
    ((2, 50004), F32, False),    # float32 wide route, ragged
    ((2, 139272), F16, False),   # one vector past the wide route: block route, 16-byte vectors
    ((2, 20002), F32, True),     # float32 block route, 8-byte vectors, ragged step
    ((2, 32770), F16, True),     # block route, 4-byte vectors
    ((7, 4100), F16, True),      # 8-byte rows of 1025 vectors: phased route
    ((5, 4092), F16, True),      # 8-byte rows of 1023 vectors: phased route (odd row count)
    ((5, 4098), F16, False),     # 4-byte rows: phased route
    ((3, 2046), F16, True),      # 4-byte rows: phased route
    ((4, 4097), F16, False),     # odd width: phased route (aligned 16-byte vectors across rows)
    ((3, 6000), F16, True),      # 750 sixteen-byte vectors: four waves per row, ragged
    ((3, 6002), F32, True),      # float32 8-byte rows: phased route
    ((2, 8193), F16, True),      # odd: phased route, eight waves
    ((2, 16385), F16, True),     # odd: phased route, sixteen waves
    ((2, 32769), F16, True),     # odd and wider than the phased route: scalar block route
    # rows of at most 32 accesses: lane groups, several rows per wave
    ((1000, 128), F16, True),    # 16 sixteen-byte vectors: 16 lanes per row, 4 rows per thread
    ((777, 256), F16, False),    # 32 vectors: 32 lanes per row
    ((333, 40), F16, True),      # 5 vectors in 8 lanes
    ((64, 6), F32, False),       # 3 eight-byte vectors in 4 lanes
    ((129, 100), F16, True),     # 25 eight-byte vectors in 32 lanes
    ((50, 30), F16, False),      # 15 four-byte vectors in 16 lanes, 16 rows per thread
    ((31, 7), F16, True),        # 7 scalars in 8 lanes
    ((5, 32), F32, True),        # 8 vectors
    ((3, 5, 24), F32, False),    # rank 3, 6 sixteen-byte vectors
    ((200, 320), F16, True),     # 40 vectors: 64-lane groups, 4 rows per thread
    ((97, 384), F16, False),     # 48 vectors: the last lane-group width
    ((33, 392), F16, True),      # 49 vectors: one wave per row
    # odd rows around the phased route's shortest: 33 vectors phased, 32 not
    ((41, 255), F16, False),     # 33 sixteen-byte vectors touched: phased
    ((41, 247), F16, True),      # 32: one wave of scalars per row
    ((37, 127), F32, True),      # 33: phased
    ((37, 123), F32, False),     # 32: one wave of scalars per row
    ((300, 63), F16, True),      # 63 scalars: 64-lane groups
    ((90, 65), F32, False),      # 65 scalars: one wave per row
    ((120, 49), F32, True),      # 49 scalars: 64-lane groups
    ((200, 126), F16, False),    # 63 four-byte pairs: 64-lane groups
    ((70, 252), F16, True),      # 63 eight-byte vectors: 64-lane groups
    ((60, 130), F16, False),     # 65 four-byte pairs: one wave per row
    ((80, 102), F32, True),      # 51 eight-byte vectors: 64-lane groups
    ((40, 252), F16, False),     # 63 eight-byte vectors fill a 64-lane group: segment route
    ((40, 260), F16, True),      # 65 eight-byte vectors, half a wave's slots idle: phased route
    ((30, 508), F16, False),     # 127 eight-byte vectors fill a wave of two: wave route
    ((30, 302), F16, True),      # 151 four-byte vectors: phased route
]


def flat_expected(dt, hidden, center=False, width=None):
    """Whether the automatic choice takes the flat route, for a row whose
    other routes would use `width`-byte accesses (element rows by default):
    the measured rule of the library, restated."""
    size = np.dtype(dt).itemsize
    width = size if width is None else width
    if width == size:
        return hidden <= ((191 if center else 247) if size == 2 else (1020 if center else 255))
    if width == 4 and size == 2:
        if not 10 <= hidden <= 300:
            return False
        if not center:
            return True
        nvec = hidden // 2
        slots = 1 << (nvec - 1).bit_length() if nvec <= 64 else 64 * ((nvec + 63) // 64)
        return nvec / slots < 0.7
    if width == 8 and size == 4:
        return 42 <= hidden <= 1020
    return False


def phase_expected(dt, hidden, width, center=False):
    """Whether the automatic choice takes the phased route for a row whose
    other routes would use `width`-byte accesses (the flat route not taking
    it): the measured rule of the library, restated."""
    size = np.dtype(dt).itemsize
    if not 32 < hidden // (16 // size) + 2 <= 1024 * 4:
        return False
    if width == size or width == 4 and size == 2 or width == 8 and size == 4:
        return True
    if width != 8 or center:
        return False
    nvec = hidden // (width // size)
    if nvec > 256:
        return True
    if nvec <= 64:
        slots = 1 << (nvec - 1).bit_length()
    else:
        need = -(-nvec // 64)
        slots = 64 * (need if need <= 4 else 6 if need <= 6 else 8)
    return nvec / slots < 0.8


def expected_route(shape, dt):
    size = np.dtype(dt).itemsize
    hidden = shape[-1]
    width = next((b for b in (16, 8, 4) if b > size and hidden * size % b == 0), size)
    E = width // size
    name = {16: "vec16", 8: "vec8", 4: "vec4"}.get(width) if E > 1 else "scalar"
    nvec = hidden // E
    # All bases here are 16-byte aligned.  The flat route where it measured
    # faster; rows that would be read element by element beyond it take the
    # phased route, which reads whole aligned 16-byte vectors when a row
    # needs more than 32 and at most 1024 x 4 of them.
    if flat_expected(dt, hidden, width=width):
        return "ssln.flat.vec16"
    if phase_expected(dt, hidden, width):
        return "ssln.phase.vec16"
    if nvec <= (64 if width < 16 else 48):
        return f"ssln.segment.{name}"
    per_lane = 4 if E > 1 and width == 16 else 8 if E > 1 and width == 8 else 16
    if nvec <= 64 * per_lane:
        return f"ssln.wave.{name}"
    if nvec <= 128 * per_lane:
        return f"ssln.wave2.{name}"
    widest = 2 * per_lane if width == 16 else per_lane  # accesses per lane of 16-wave rows
    if nvec > 1024 * widest:
        if width == 16 and nvec <= 1024 * 17:  # 8 vectors per lane in VGPRs, up to 9 in LDS
            return "ssln.wide.vec16"
        return "ssln.block" if E == 1 else f"ssln.block.{name}"
    if nvec <= 256 * per_lane:
        return f"ssln.rowblock.{name}"
    if nvec <= 512 * per_lane:
        return f"ssln.row8.{name}"
    return f"ssln.row16.{name}"


@pytest.mark.parametrize("route", ["auto", "scalar", "block"])
@pytest.mark.parametrize("shape,dt,with_bias", SHAPES, ids=[f"{s}-{np.dtype(d).name}-{'b' if b else 'nb'}"
                                                            for s, d, b in SHAPES])
def test_matches_oracle(shape, dt, with_bias, route):
    w = workloads.ssln("t", shape, dt, bias=with_bias, epsilon=1e-6)
    x = workloads.generate(w, seed=sum(shape))
    ref, out, used = run_both(x["input"], x["skip"], x["gamma"], x.get("bias"), 1e-6, route)
    check(ref, out)
    if route == "auto":
        assert used == expected_route(shape, dt)


@pytest.mark.parametrize("want", [(), ("sum",), ("inv",), ("mean",), ("sum", "inv"),
                                  ("mean", "inv", "sum")])
@pytest.mark.parametrize("dt,hidden", [(F32, 2048), (F16, 2048), (F16, 16384), (F16, 131072)])
def test_optional_outputs_do_not_change_output(dt, hidden, want):
    w = workloads.ssln("t", (37, hidden), dt, bias=True, epsilon=1e-6)
    x = workloads.generate(w, seed=5)
    ref, out, _ = run_both(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6, want=want)
    check(ref, out, want)
    _, base, _ = run_both(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6, want=())
    assert_bitwise(to_host(out.output), to_host(base.output), "output with/without optional outputs")


@pytest.mark.parametrize("offset,route", [(1, "ssln.rowblock.scalar"), (2, "ssln.wave2.vec4"),
                                          (4, "ssln.wave2.vec8")])
def test_base_alignment_picks_the_vector_width(offset, route):
    """Views `offset` halves into their buffers: 2-, 4- and 8-byte aligned
    bases take scalar, 4-byte and 8-byte accesses, with the same results."""
    rows, hidden = 6, 4096
    w = workloads.ssln("t", (rows, hidden), F16, bias=True, epsilon=1e-6)
    x = workloads.generate(w, seed=12)
    def view(a):
        buf = torch.empty(rows * hidden + 8, dtype=torch.float16, device="cuda")
        v = buf[offset: offset + rows * hidden].view(rows, hidden)
        v.copy_(to_dev(a))
        return v
    out = gn.skip_rms_norm(view(x["input"]), view(x["skip"]), to_dev(x["gamma"]), to_dev(x["bias"]),
                           1e-6, want_sum=True, want_inv_std_var=True)
    assert gn.last_route() == route
    ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6,
                               want_inv_std_var=True, want_sum=True)
    assert_close(to_host(out.output), ref[0], "output")
    assert_close(to_host(out.inv_std_var), ref[2], "inv_std_var")
    assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], "S")


def test_unaligned_tensors_take_scalar_route():
    w = workloads.ssln("t", (8, 513), F16, bias=True, epsilon=1e-6)
    x = workloads.generate(w, seed=3)
    dev = {k: to_dev(v) for k, v in x.items()}
    # A view one element into a larger buffer is not 16-byte aligned.
    big = torch.empty(8 * 513 + 1, dtype=torch.float16, device="cuda")
    big[1:].copy_(dev["input"].ravel())
    inp = big[1:].view(8, 513)
    out = gn.skip_rms_norm(inp, dev["skip"], dev["gamma"], dev["bias"], 1e-6, want_sum=True)
    assert gn.last_route() == "ssln.wave.scalar"
    ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6, want_sum=True)
    assert_close(to_host(out.output), ref[0], "output")
    assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], "S")


def test_edge_values_f16():
    # Residual sums that tie, overflow to inf, become subnormal or -0.
    inp = np.array([[1, 1.0009765625, 65504, 65504, 2 ** -24, 2 ** -14, -0.0, 3]], F16)
    skip = np.array([[2 ** -11, 2 ** -11, 16, 8, 2 ** -24, -(2 ** -24), -0.0, -3]], F16)
    gamma = np.ones(8, F16)
    for route in ("auto", "scalar", "block"):
        ref, out, _ = run_both(inp, skip, gamma, None, 1e-6, route)
        assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], f"S ({route})")
        # The row holds +inf: output is NaN/0 as in the oracle.
        assert_close(to_host(out.output), ref[0], f"output ({route})")


@pytest.mark.parametrize("dt,hidden", [(F16, 139264), (F32, 50004)])
def test_wide_route_edge_values(dt, hidden):
    """Residual sums that tie, overflow, go subnormal or come out -0, planted
    in the register part and in the LDS part of wide rows (and in the last
    vector of the LDS part), against the oracle bit for bit in S."""
    rng = np.random.default_rng(3)
    rows = 3
    inp = rng.standard_normal((rows, hidden)).astype(dt)
    skip = rng.standard_normal((rows, hidden)).astype(dt)
    gamma = rng.uniform(0.5, 1.5, hidden).astype(dt)
    if dt == F16:
        vals = [(1, 2 ** -11), (1.0009765625, 2 ** -11), (2 ** -24, 2 ** -24), (2 ** -14, -(2 ** -24)),
                (-0.0, -0.0), (3, -3)]
    else:
        vals = [(1, 2 ** -24), (2 ** -149, 2 ** -149), (-0.0, -0.0), (3, -3), (2 ** -126, -(2 ** -149))]
    E = 16 // np.dtype(dt).itemsize
    for r in range(rows):
        for k, (a, b) in enumerate(vals):
            for vec in (r, 8192 + 1024 * r + 7, hidden // E - 1):  # VGPR part, LDS part, last vector
                pos = vec * E + (k % E)
                inp[r, pos], skip[r, pos] = a, b
    ref, out, used = run_both(inp, skip, gamma, None, 1e-6, "auto")
    assert used == "ssln.wide.vec16"
    check(ref, out)


def test_zero_rows_and_zero_row():
    g = np.ones(16, F32)
    z = np.zeros((0, 16), F32)
    out = gn.skip_rms_norm(to_dev(z), to_dev(z), to_dev(g))
    assert out.output.shape == (0, 16)
    zr = np.zeros((3, 16), F32)
    ref, out, _ = run_both(zr, zr, g, None, 9.999999960041972e-13)
    check(ref, out)
    assert np.all(to_host(out.inv_std_var) == np.float32(1e6))


def test_deterministic():
    w = workloads.ssln("t", (64, 4096), F16, bias=True, epsilon=1e-6)
    x = workloads.generate(w, seed=9)
    a = run_both(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6)[1]
    b = run_both(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6)[1]
    for f in ("output", "inv_std_var", "input_skip_bias_sum"):
        assert_bitwise(to_host(getattr(a, f)), to_host(getattr(b, f)), f)


def test_outputs_leave_neighbouring_memory_untouched():
    """Writes stay inside each output: canary regions around the outputs
    (passed as raw pointers through the C ABI) keep their pattern."""
    from group_normalization_amd._lib import lib, check as ck
    rows, hidden, pad = 11, 768, 4096
    w = workloads.ssln("t", (rows, hidden), F16, bias=True, epsilon=1e-6)
    x = workloads.generate(w, seed=4)
    d = {k: to_dev(v) for k, v in x.items()}
    n = rows * hidden
    arena = torch.full((3 * (n + 2 * pad),), -7.0, dtype=torch.float16, device="cuda")
    slots = [arena[i * (n + 2 * pad) + pad: i * (n + 2 * pad) + pad + n] for i in range(3)]
    stats = torch.full((2 * (rows + 2 * pad),), -7.0, dtype=torch.float32, device="cuda")
    mean = stats[pad: pad + rows]
    inv = stats[rows + 3 * pad: rows + 3 * pad + rows]
    ck(lib().skip_rms_norm(desc(d["input"]), desc(d["skip"]), desc(d["gamma"]), desc(d["bias"]), 1e-6,
                           desc(slots[0], (rows, hidden)), desc(mean, (rows, 1)), desc(inv, (rows, 1)),
                           desc(slots[1], (rows, hidden)), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x["bias"], 1e-6,
                               want_mean=True, want_inv_std_var=True, want_sum=True)
    assert_close(to_host(slots[0]).reshape(rows, hidden), ref[0], "output")
    assert_bitwise(to_host(slots[1]).reshape(rows, hidden), ref[3], "S")
    assert torch.all(slots[2] == -7.0)
    a = to_host(arena).reshape(3, -1)
    assert np.all(a[:, :pad] == -7.0) and np.all(a[:, pad + n:] == -7.0)
    s = to_host(stats)
    assert np.all(s[:pad] == -7.0) and np.all(s[pad + rows: rows + 3 * pad] == -7.0)
    assert np.all(s[2 * rows + 3 * pad:] == -7.0)


@pytest.mark.parametrize("dt,hidden,offset,center", [
    (F16, 4096, 1, False), (F16, 4096, 3, True), (F16, 4095, 0, False), (F16, 4097, 5, True),
    (F16, 1000, 7, False), (F16, 20003, 2, True), (F16, 32753, 6, False), (F16, 391, 4, True),
    (F32, 4097, 1, False), (F32, 6002, 1, True), (F32, 8191, 3, False), (F32, 4096, 3, True),
    (F16, 255, 0, True), (F16, 301, 3, False), (F32, 127, 2, False), (F32, 187, 0, True),
])
def test_phased_rows(dt, hidden, offset, center):
    """Rows that would be read element by element, through the C ABI:
    input, skip, output and S all `offset` elements past a 16-byte boundary
    (2-byte aligned for float16, 4-byte for float32), or rows of an odd
    length, take the phased route, which reads whole aligned 16-byte vectors
    across row boundaries.  Results match
    the oracle, and nothing outside the outputs is written (canaries around
    them keep their pattern)."""
    from group_normalization_amd._lib import lib, check as ck
    rows, pad = 7, 64
    if center:
        w = workloads.sln("t", (rows, hidden), dt, beta=True, bias=True, epsilon=1e-5)
    else:
        w = workloads.ssln("t", (rows, hidden), dt, bias=True, epsilon=1e-5)
    x = workloads.generate(w, seed=hidden + offset)
    tdt = torch.float16 if dt == F16 else torch.float32
    n = rows * hidden

    def arena(fill):
        return torch.full((n + 2 * pad,), fill, dtype=tdt, device="cuda")

    bufs = {k: arena(-7.0) for k in ("input", "skip", "output", "sum")}
    views = {k: b[pad + offset: pad + offset + n] for k, b in bufs.items()}
    views["input"].copy_(to_dev(x["input"]).ravel())
    views["skip"].copy_(to_dev(x["skip"]).ravel())
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    inv = torch.empty(rows, dtype=torch.float32, device="cuda")
    d = {k: to_dev(x[k]) for k in ("gamma", "bias", "beta") if x.get(k) is not None}
    shp = (rows, hidden)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        if center:
            ck(lib().skip_layer_norm(desc(views["input"], shp), desc(views["skip"], shp), desc(d["gamma"]),
                                     desc(d["beta"]), desc(d["bias"]), 1e-5, desc(views["output"], shp),
                                     desc(mean, (rows, 1)), desc(inv, (rows, 1)), desc(views["sum"], shp),
                                     stream))
            ref = oracle.skip_layer_norm(x["input"], x["skip"], x["gamma"], x["beta"], x["bias"], 1e-5,
                                         want_mean=True, want_inv_std_var=True, want_sum=True)
        else:
            ck(lib().skip_rms_norm(desc(views["input"], shp), desc(views["skip"], shp), desc(d["gamma"]),
                                   desc(d["bias"]), 1e-5, desc(views["output"], shp), desc(mean, (rows, 1)),
                                   desc(inv, (rows, 1)), desc(views["sum"], shp), stream))
            ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x["bias"], 1e-5,
                                       want_mean=True, want_inv_std_var=True, want_sum=True)
        assert gn.last_route() == ("ssln.flat.vec16" if flat_expected(dt, hidden, center)
                                   else "ssln.phase.vec16")
        torch.cuda.synchronize()
        assert_close(to_host(views["output"]).reshape(rows, hidden), ref[0], "output")
        assert_close(to_host(mean), ref[1].reshape(-1), "mean")
        assert_close(to_host(inv), ref[2].reshape(-1), "inv_std_var")
        assert_bitwise(to_host(views["sum"]).reshape(rows, hidden), ref[3], "S")
        for k in ("output", "sum"):
            b = to_host(bufs[k])
            assert np.all(b[:pad + offset] == -7.0) and np.all(b[pad + offset + n:] == -7.0), k


# ---------------------------------------------------------------- flat route
def run_rows(x, eps, center, route="auto"):
    """skip_rms_norm / skip_layer_norm with every output, and the oracle."""
    with gn.force_route(route):
        if center:
            out = gn.skip_layer_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]),
                                     to_dev(x.get("beta")), to_dev(x.get("bias")), eps, want_mean=True,
                                     want_inv_std_var=True, want_sum=True)
        else:
            out = gn.skip_rms_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]),
                                   to_dev(x.get("bias")), eps, want_mean=True, want_inv_std_var=True,
                                   want_sum=True)
        used = gn.last_route()
    if center:
        ref = oracle.skip_layer_norm(x["input"], x["skip"], x["gamma"], x.get("beta"), x.get("bias"), eps,
                                     want_mean=True, want_inv_std_var=True, want_sum=True)
    else:
        ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x.get("bias"), eps, want_mean=True,
                                   want_inv_std_var=True, want_sum=True)
    torch.cuda.synchronize()
    assert_close(to_host(out.output), ref[0], "output")
    assert_close(to_host(out.mean), ref[1], "mean")
    assert_close(to_host(out.inv_std_var), ref[2], "inv_std_var")
    assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], "S")
    return used


FLAT_ROWS = [
    # (rows, hidden, dtype): odd widths through the table's limit, rows that
    # share vectors (narrow), ragged row counts, several lane-group sizes.
    (1001, 1, F16), (777, 3, F16), (513, 5, F16), (301, 7, F16), (900, 9, F16), (333, 17, F16),
    (129, 57, F16), (100, 63, F16), (97, 127, F16), (61, 129, F16), (40, 247, F16), (37, 255, F16),
    (13, 511, F16), (9, 777, F16), (5, 1015, F16),
    (1000, 1, F32), (555, 3, F32), (301, 5, F32), (250, 33, F32), (99, 123, F32), (31, 127, F32),
    (17, 509, F32), (7, 1019, F32),
]


@pytest.mark.parametrize("center", [False, True], ids=["rms", "layer"])
@pytest.mark.parametrize("rows,hidden,dt", FLAT_ROWS,
                         ids=[f"{r}x{h}-{np.dtype(d).name}" for r, h, d in FLAT_ROWS])
def test_flat_rows(rows, hidden, dt, center):
    """Odd rows read as one stream of aligned 16-byte vectors: the automatic
    route for the lengths where it measured faster than reading them element
    by element, and forced (the mean-removed form from 3 elements on); every
    output against the oracle."""
    if center:
        w = workloads.sln("t", (rows, hidden), dt, beta=True, bias=True, epsilon=1e-5)
    else:
        w = workloads.ssln("t", (rows, hidden), dt, bias=rows % 2 == 1, epsilon=1e-5)
    x = workloads.generate(w, seed=rows + hidden)
    used = run_rows(x, 1e-5, center)
    if center and hidden < 3:
        assert used != "ssln.flat.vec16"
    else:
        assert (used == "ssln.flat.vec16") == flat_expected(dt, hidden, center)
    # The same rows forced onto the flat route wherever it applies.
    used = run_rows(x, 1e-5, center, route="flat")
    assert (used == "ssln.flat.vec16") == (not center or hidden >= 3)


@pytest.mark.parametrize("center", [False, True], ids=["rms", "layer"])
@pytest.mark.parametrize("rows,hidden,dt", [(500, 4, F16), (300, 30, F16), (200, 100, F16), (64, 1000, F16),
                                            (400, 6, F32), (100, 250, F32), (30, 1020, F32), (21, 1016, F16),
                                            (333, 34, F16), (111, 130, F16), (222, 126, F16), (77, 186, F16),
                                            (90, 42, F32), (60, 750, F32)])
def test_flat_forced_on_vector_rows(rows, hidden, dt, center):
    """Forced (route "flat"), rows that otherwise take 4-, 8- or 16-byte
    vectors on other routes give the same results."""
    w = (workloads.sln("t", (rows, hidden), dt, beta=False, bias=True, epsilon=1e-5) if center else
         workloads.ssln("t", (rows, hidden), dt, bias=True, epsilon=1e-5))
    x = workloads.generate(w, seed=hidden)
    assert run_rows(x, 1e-5, center, route="flat") == "ssln.flat.vec16"
    size = np.dtype(dt).itemsize
    width = next(b for b in (16, 8, 4) if b > size and hidden * size % b == 0)
    assert (run_rows(x, 1e-5, center) == "ssln.flat.vec16") == flat_expected(dt, hidden, center, width)


@pytest.mark.parametrize("dt,hidden,offset,center", [
    (F16, 7, 1, False), (F16, 127, 3, True), (F16, 1015, 5, False), (F16, 3, 7, True), (F16, 1, 2, False),
    (F32, 5, 1, True), (F32, 123, 2, False), (F32, 1019, 3, True), (F32, 1, 1, False),
])
def test_flat_rows_off_the_grid(dt, hidden, offset, center):
    """Through the C ABI: input, skip, output and S all `offset` elements
    past a 16-byte boundary; results match the oracle and nothing outside
    the outputs is written (canaries around them keep their pattern)."""
    from group_normalization_amd._lib import lib, check as ck
    rows, pad = 301, 64
    if center:
        w = workloads.sln("t", (rows, hidden), dt, beta=True, bias=True, epsilon=1e-5)
    else:
        w = workloads.ssln("t", (rows, hidden), dt, bias=True, epsilon=1e-5)
    x = workloads.generate(w, seed=hidden + offset)
    tdt = torch.float16 if dt == F16 else torch.float32
    n = rows * hidden
    bufs = {k: torch.full((n + 2 * pad,), -7.0, dtype=tdt, device="cuda") for k in ("input", "skip", "output", "sum")}
    views = {k: b[pad + offset: pad + offset + n] for k, b in bufs.items()}
    views["input"].copy_(to_dev(x["input"]).ravel())
    views["skip"].copy_(to_dev(x["skip"]).ravel())
    stats = torch.full((4 * pad + 2 * rows,), -7.0, dtype=torch.float32, device="cuda")
    mean, inv = stats[pad: pad + rows], stats[3 * pad + rows: 3 * pad + 2 * rows]
    d = {k: to_dev(x[k]) for k in ("gamma", "bias", "beta") if x.get(k) is not None}
    shp, st = (rows, hidden), (rows, 1)
    stream = torch.cuda.current_stream().cuda_stream
    with gn.force_route("flat"):
        if center:
            ck(lib().skip_layer_norm(desc(views["input"], shp), desc(views["skip"], shp), desc(d["gamma"]),
                                     desc(d["beta"]), desc(d["bias"]), 1e-5, desc(views["output"], shp),
                                     desc(mean, st), desc(inv, st), desc(views["sum"], shp), stream))
        else:
            ck(lib().skip_rms_norm(desc(views["input"], shp), desc(views["skip"], shp), desc(d["gamma"]),
                                   desc(d["bias"]), 1e-5, desc(views["output"], shp), desc(mean, st),
                                   desc(inv, st), desc(views["sum"], shp), stream))
    if center:
        ref = oracle.skip_layer_norm(x["input"], x["skip"], x["gamma"], x["beta"], x["bias"], 1e-5,
                                     want_mean=True, want_inv_std_var=True, want_sum=True)
    else:
        ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x["bias"], 1e-5,
                                   want_mean=True, want_inv_std_var=True, want_sum=True)
    assert gn.last_route() == "ssln.flat.vec16"
    torch.cuda.synchronize()
    assert_close(to_host(views["output"]).reshape(shp), ref[0], "output")
    assert_close(to_host(mean), ref[1].reshape(-1), "mean")
    assert_close(to_host(inv), ref[2].reshape(-1), "inv_std_var")
    assert_bitwise(to_host(views["sum"]).reshape(shp), ref[3], "S")
    for k in ("output", "sum"):
        b = to_host(bufs[k])
        assert np.all(b[:pad + offset] == -7.0) and np.all(b[pad + offset + n:] == -7.0), k
    s_ = to_host(stats)
    assert np.all(s_[:pad] == -7.0) and np.all(s_[pad + rows: 3 * pad + rows] == -7.0)
    assert np.all(s_[3 * pad + 2 * rows:] == -7.0)


def test_flat_edge_values_f16():
    # Ties, overflow to inf, subnormals and -0 in odd rows on the flat route.
    inp = np.array([[1, 1.0009765625, 65504, 65504, 2 ** -24, 2 ** -14, -0.0],
                    [3, -0.0, 2 ** -24, 1, 0.5, 0.25, 2.0]], F16)
    skip = np.array([[2 ** -11, 2 ** -11, 16, 8, 2 ** -24, -(2 ** -24), -0.0],
                     [-3, -0.0, 2 ** -24, 2 ** -11, 0.5, 0.25, -2.0]], F16)
    gamma = np.ones(7, F16)
    ref, out, used = run_both(inp, skip, gamma, None, 1e-6)
    assert used == "ssln.flat.vec16"
    assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], "S")
    assert_close(to_host(out.output), ref[0], "output")
